"""fm_op_attention_noalloc (the attention of vla.cpp Eq. (2) on the library's fixed scratch,
for callers that cannot allocate) against fm_op_attention on the same inputs, through the C ABI.
Same kernels and split plan, so the outputs are compared bit for bit; two calls in a row, the
second smaller, so that the scratch left by the first cannot leak into the second; and a call
whose scratch would exceed the fixed size is refused before any launch."""
import numpy as np
import pytest
import torch

from flow_matching_vla_amd import fm
from gpu_util import say

pytestmark = pytest.mark.gpu


def _inputs(B, Tq, nh, nkv, nk, dh, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Tq, nh, dh, generator=g).to(dtype).cuda()
    k = torch.randn(B, nkv, nk, dh, generator=g).to(dtype).cuda()
    v = torch.randn(B, nkv, nk, dh, generator=g).to(dtype).cuda()
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_attention_equals_allocating_entry_point(dtype):
    dh_big = 256 if dtype == torch.bfloat16 else 128
    cases = [(2, 50, 8, 1, 900, dh_big), (1, 16, 4, 4, 130, 64)]   # the second call is the smaller
    for i, (B, Tq, nh, nkv, nk, dh) in enumerate(cases):
        say(f"  noalloc attention {dtype}: B {B} Tq {Tq} heads {nh}/{nkv} keys {nk} dh {dh}")
        q, k, v = _inputs(B, Tq, nh, nkv, nk, dh, dtype, seed=11 + i)
        ref = fm.op_attention(q, k, v)
        o = torch.full_like(q, float("nan"))
        fm.op_attention_noalloc(q, k, v, o)
        torch.cuda.synchronize()
        a, r = o.float().cpu().numpy(), ref.float().cpu().numpy()
        assert np.isfinite(a).all()
        np.testing.assert_array_equal(a, r)


def test_noalloc_attention_refuses_oversize_scratch():
    # the V plane alone: 1 x 1 x 256 x 40000 bf16 = 20 MB > the fixed 16 MiB
    say("  noalloc attention: oversize request")
    q, k, v = _inputs(1, 4, 1, 1, 40000, 256, torch.bfloat16, seed=3)
    o = torch.zeros_like(q)
    with pytest.raises(fm.FMError, match="scratch"):
        fm.op_attention_noalloc(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0   # refused before any launch

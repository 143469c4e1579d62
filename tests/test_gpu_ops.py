"""Kernel-level parity through the C ABI: the library GEMM (tiles, ragged tails, split-K,
the weight-streaming kernel at the row counts where it computes three or four 16-row blocks,
fused bias/activation) and the attention kernel (head fold onto one K/V head, MHA,
split over keys, ragged key counts) against the CPU oracle's float64 routines."""
import numpy as np
import pytest

import oracle
from flow_matching_vla_amd import workloads as wl
from gpu_util import say

pytestmark = pytest.mark.gpu


def _dev(a, bf16):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("M,N,K", [(50, 2560, 1024), (50, 1024, 4096), (1, 64, 64), (7, 37, 96), (130, 200, 320),
                                   (400, 1024, 2048), (3200, 2560, 1024), (16, 7, 1024), (41, 4608, 1536),
                                   (48, 512, 256), (49, 512, 256), (33, 96, 64), (64, 160, 4096)])
def test_linear_matches_oracle(bf16, M, N, K):
    from flow_matching_vla_amd import fm
    import torch
    if not bf16 and K % 16:
        pytest.skip("fp32 path needs K % 16 == 0")
    say("linear", M, N, K, "bf16" if bf16 else "f32")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    if bf16:
        A, W = wl.round_bf16(A), wl.round_bf16(W)
    out = fm.op_linear(_dev(A, bf16), _dev(W, bf16), torch.from_numpy(b).cuda(), act=0, out_f32=True)
    ref = oracle.linear(A.astype(np.float64), W.astype(np.float64), b.astype(np.float64))
    err = oracle.e_rel(out.cpu().numpy(), ref)
    assert err < 1e-5, err
    # fused activation epilogues and a stored (rounded) output
    for act, f in ((1, oracle.silu), (2, oracle.gelu_tanh)):
        o2 = fm.op_linear(_dev(A, bf16), _dev(W, bf16), torch.from_numpy(b).cuda(), act=act, out_f32=False)
        e2 = oracle.e_rel(o2.float().cpu().numpy(), f(ref))
        assert e2 < (5e-3 if bf16 else 2e-6), (act, e2)


@pytest.mark.parametrize("bf16,B,Tq,nh,nkv,nk,dh", [
    (True, 1, 50, 8, 1, 866, 256),     # pi0.5 expert: prefix 816 + 50 suffix keys, head fold
    (True, 2, 50, 8, 1, 1074, 256),    # P = 1024
    (True, 1, 41, 24, 24, 600, 64),    # DiT cross-attention
    (True, 1, 41, 24, 24, 41, 64),     # DiT self-attention
    (True, 2, 20, 4, 1, 300, 128),     # 128-dim heads folded onto one K/V head: five key splits (bf16 partials)
    (True, 1, 3, 8, 1, 1, 256),        # a single key
    (True, 1, 5, 4, 1, 65, 64),        # one key past a tile
    (False, 1, 16, 4, 1, 80, 64),      # fp32 tiny expert
    (False, 2, 9, 4, 4, 7, 64),
])
def test_attention_matches_oracle(bf16, B, Tq, nh, nkv, nk, dh):
    from flow_matching_vla_amd import fm
    say("attention", B, Tq, nh, nkv, nk, dh, "bf16" if bf16 else "f32")
    rng = np.random.default_rng(nk * 13 + Tq)
    q = rng.standard_normal((B, Tq, nh, dh)).astype(np.float32) * 0.5
    k = rng.standard_normal((B, nkv, nk, dh)).astype(np.float32)
    v = rng.standard_normal((B, nkv, nk, dh)).astype(np.float32)
    if bf16:
        q, k, v = wl.round_bf16(q), wl.round_bf16(k), wl.round_bf16(v)
    o = fm.op_attention(_dev(q, bf16), _dev(k, bf16), _dev(v, bf16)).float().cpu().numpy()
    ref = oracle.attention(q.transpose(0, 2, 1, 3).astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    ref = ref.transpose(0, 2, 1, 3)
    err = oracle.e_rel(o, ref)
    assert err < (1e-2 if bf16 else 1e-5), err
    # sharp attention (large logits) stays finite and correct
    o = fm.op_attention(_dev(q * 8, bf16), _dev(k, bf16), _dev(v, bf16)).float().cpu().numpy()
    ref = oracle.attention((8 * q).transpose(0, 2, 1, 3).astype(np.float64), k.astype(np.float64), v.astype(np.float64)).transpose(0, 2, 1, 3)
    assert np.all(np.isfinite(o))
    assert oracle.e_rel(o, ref) < (2e-2 if bf16 else 1e-5)

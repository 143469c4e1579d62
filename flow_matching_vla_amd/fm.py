"""Python binding of the C ABI in include/fm.h (ctypes). Argument marshalling only: every
step of the loop runs in the HIP library; torch supplies device memory and the stream.
The binding refuses to run when the library has not been built."""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfmvla.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fm.h")

FM_OK = 0
STATUS = {0: "FM_OK", 1: "FM_ERR_INVALID_ARG", 2: "FM_ERR_SHAPE", 3: "FM_ERR_STATE", 4: "FM_ERR_SCHEDULE",
          5: "FM_ERR_UNSUPPORTED", 6: "FM_ERR_OOM", 7: "FM_ERR_DEVICE"}
F32, BF16 = 0, 1


class FMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class fm_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "arch", "dtype", "n_layers", "hidden", "n_heads", "head_dim", "n_kv_heads", "mlp_dim", "mlp_gated",
        "action_horizon", "action_dim", "state_tokens", "state_dim", "ctx_len_max", "ctx_dim",
        "max_prefix_len", "max_batch", "max_steps")] + [("rope_base", C.c_float), ("norm_eps", C.c_float)]


class fm_tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dtype", C.c_int32), ("ndim", C.c_int32), ("shape", C.c_int64 * 4),
                ("data", C.c_void_p)]


class fm_plan_info(C.Structure):
    _fields_ = [("n_sites", C.c_int32), ("pool_capacity", C.c_int32), ("n_weights", C.c_int32),
                ("weight_bytes", C.c_int64), ("pool_bytes", C.c_int64)]


_lib = None


def lib():
    """Load libfmvla.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with flow_matching_vla_amd.build.build()")
    try:  # load torch's HIP runtime first so the library binds to the same one (same SONAME)
        import torch  # noqa: F401
    except ImportError:
        pass
    L = C.CDLL(LIB_PATH)
    P, I32, VP = C.POINTER, C.c_int32, C.c_void_p
    sig = {
        "fm_query": ([P(fm_config), P(fm_plan_info), C.c_char_p, I32], I32),
        "fm_device_supported": ([C.c_char_p, I32, I32, C.c_char_p, I32], I32),
        "fm_weight_spec": ([P(fm_config), I32, P(C.c_char_p), P(I32), P(C.c_int64)], I32),
        "fm_create": ([P(fm_config), VP, P(VP)], I32),
        "fm_destroy": ([VP], I32),
        "fm_last_error": ([VP], C.c_char_p),
        "fm_load_weights": ([VP, P(fm_tensor), I32], I32),
        "fm_set_schedule": ([VP, I32, I32, P(C.c_float)], I32),
        "fm_bind_prefix_kv": ([VP, I32, I32, P(VP), P(VP), VP, VP], I32),
        "fm_bind_prefix_lengths": ([VP, P(I32)], I32),
        "fm_prefix_kv_slot": ([VP, I32, P(VP), P(VP)], I32),
        "fm_bind_prefix_inplace": ([VP, I32, I32], I32),
        "fm_bind_context_masks": ([VP, P(C.c_uint8), P(C.c_uint8)], I32),
        "fm_denoise": ([VP, VP, I32, VP], I32),
        "fm_step_velocity": ([VP, VP, I32, VP], I32),
        "fm_step_trace": ([VP, VP, I32, VP, VP], I32),
        "fm_profile_loop": ([VP, VP, I32, VP, I32, P(C.c_float), P(I32)], I32),
        "fm_set_loop_mode": ([VP, I32], I32),
        "fm_loop_status": ([VP, P(I32), P(C.c_uint32)], I32),
        "fm_set_action_stats": ([VP, I32, I32, I32, P(C.c_float), P(C.c_float)], I32),
        "fm_unnormalize": ([VP, VP, VP], I32),
        "fm_op_linear": ([I32, I32, I32, I32, VP, VP, VP, I32, VP, I32, VP], I32),
        "fm_op_attention": ([I32, I32, I32, I32, I32, I32, I32, VP, VP, VP, VP, VP], I32),
        "fm_op_attention_noalloc": ([I32, I32, I32, I32, I32, I32, I32, VP, VP, VP, VP, VP], I32),
        "fm_op_quantize_fp8": ([I32, I32, VP, VP, VP, VP, VP], I32),
        "fm_set_weight_format": ([VP, I32], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes, f.restype = args, res
    _lib = L
    return L


WEIGHTS_AS_GIVEN, WEIGHTS_FP8_E4M3 = 0, 1


def quantize_fp8(w):
    """The library's FP8 weight quantizer on a device bf16 [N, K] tensor: (codes uint8 [N, K],
    per-row scales fp32 [N], dequantized bf16 [N, K]), all device tensors."""
    torch = _torch()
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("quantize_fp8: w must be a 2-D tensor")
    N, K = w.shape
    check_tensor(w, "w", torch.bfloat16, (N, K))
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scale = torch.empty((N,), dtype=torch.float32, device=w.device)
    deq = torch.empty_like(w)
    st = torch.cuda.current_stream()
    _check(lib().fm_op_quantize_fp8(N, K, _ptr(w), _ptr(codes), _ptr(scale), _ptr(deq), C.c_void_p(st.cuda_stream)))
    return codes, scale, deq


def pool_k_col(d, head_dim: int, rope: bool):
    """Pool column of head-dim index d of a prefix key (the header's fm_pool_k_col)."""
    d = np.asarray(d)
    if not rope:
        return d
    return np.where(d < head_dim // 2, 2 * d, 2 * (d - head_dim // 2) + 1)


def pool_v_slot(j, dtype: int):
    """Slot of key j in a transposed V row (the header's fm_pool_v_slot)."""
    j = np.asarray(j)
    if dtype != BF16:
        return j
    return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3)


def header_symbols():
    """Names of the functions include/fm.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fm_status|const char\*)\s+(fm_\w+)\s*\(", txt, re.M)))


def make_config(cfg: dict) -> fm_config:
    c = fm_config()
    c.arch, c.dtype, c.n_layers, c.hidden = cfg["arch"], cfg["dtype"], cfg["n_layers"], cfg["hidden"]
    c.n_heads, c.head_dim, c.n_kv_heads = cfg["n_heads"], cfg["head_dim"], cfg["n_kv_heads"]
    c.mlp_dim, c.mlp_gated = cfg["mlp_dim"], cfg["mlp_gated"]
    c.action_horizon, c.action_dim = cfg["action_horizon"], cfg["action_dim"]
    c.state_tokens, c.state_dim = cfg.get("state_tokens", 0), cfg.get("state_dim", 0)
    c.ctx_len_max, c.ctx_dim = cfg.get("ctx_len_max", cfg.get("ctx_len", 0)), cfg.get("ctx_dim", 0)
    c.max_prefix_len = cfg.get("max_prefix_len", cfg.get("prefix_len", 0))
    c.max_batch = cfg.get("max_batch", cfg.get("batch", 1))
    c.max_steps = cfg.get("max_steps", max(cfg.get("steps", 1), 1))
    c.rope_base, c.norm_eps = cfg.get("rope_base", 0.0), cfg.get("norm_eps", 1e-6)
    return c


def _check(st: int, ctx=None):
    if st != FM_OK:
        msg = lib().fm_last_error(ctx)
        raise FMError(st, msg.decode() if msg else "")


def device_supported(gcn_arch: str, num_xcc: int, num_cus: int):
    """(True, "") when the library can run on a device with these properties, else (False,
    reason). Host only: no GPU is touched."""
    buf = C.create_string_buffer(512)
    st = lib().fm_device_supported(gcn_arch.encode() if gcn_arch is not None else None, num_xcc, num_cus, buf, 512)
    return st == FM_OK, buf.value.decode()


def check_tensor(t, name: str, dtype, shape, device_index=None, on_device: bool = True):
    """Raise ValueError unless `t` is a contiguous torch tensor of `dtype` and exactly `shape`,
    on the GPU (the context's device when device_index is given) when on_device. The C ABI
    receives bare pointers and cannot check what they point at: a host tensor, a short buffer
    or a strided view would make the library read or write past an allocation on the GPU."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if on_device:
        if not t.is_cuda:
            raise ValueError(f"{name}: must be a device tensor, got one on {t.device}")
        if device_index is not None and t.device.index != device_index:
            raise ValueError(f"{name}: on {t.device}, the context runs on cuda:{device_index}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(d) for d in shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def torch_dtype(code: int):
    """The torch dtype of a config dtype code (F32 / BF16)."""
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def query(cfg: dict) -> dict:
    info = fm_plan_info()
    buf = C.create_string_buffer(512)
    st = lib().fm_query(C.byref(make_config(cfg)), C.byref(info), buf, 512)
    if st != FM_OK:
        raise FMError(st, buf.value.decode())
    return {f: getattr(info, f) for f, _ in fm_plan_info._fields_}


def weight_spec(cfg: dict) -> list:
    c = make_config(cfg)
    n = query(cfg)["n_weights"]
    out = []
    for i in range(n):
        name, nd, shp = C.c_char_p(), C.c_int32(), (C.c_int64 * 4)()
        _check(lib().fm_weight_spec(C.byref(c), i, C.byref(name), C.byref(nd), shp))
        out.append((name.value.decode(), tuple(shp[:nd.value])))
    return out


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, dtype: int, device="cuda"):
    """Host array (float32 values) -> contiguous device tensor of the config dtype."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if dtype == BF16:
        t = t.to(torch.bfloat16)
    return t.to(device).contiguous()


class Context:
    """One fm_ctx on the current torch stream (or `stream`)."""

    def __init__(self, cfg: dict, stream=None):
        torch = _torch()
        self.cfg = dict(cfg)
        self.dtype = cfg["dtype"]
        if stream is None:
            stream = torch.cuda.current_stream()
        self.stream = stream
        self._c = make_config(cfg)
        h = C.c_void_p()
        _check(lib().fm_create(C.byref(self._c), C.c_void_p(stream.cuda_stream), C.byref(h)))
        self.h = h
        self._keep = []
        self._bound = (0, 0)   # (batch, prefix or context length) of the binding
        self._robot = None     # (robot_horizon, robot_dim) of the action statistics
        self.device_index = torch.cuda.current_device()
        self._tdtype = torch_dtype(self.dtype)

    def close(self):
        if self.h:
            lib().fm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def last_error(self) -> str:
        return lib().fm_last_error(self.h).decode()

    def load_weights(self, weights: dict):
        """weights: name -> device tensor (config dtype, contiguous)."""
        arr = (fm_tensor * len(weights))()
        names = []
        for n, t in weights.items():
            # names and shapes are the library's to check (it reports expected vs got); where
            # the data lives and how it is laid out are not visible through the pointer
            check_tensor(t, f"weight '{n}'", self._tdtype, tuple(t.shape), self.device_index)
        for i, (n, t) in enumerate(weights.items()):
            nb = n.encode()
            names.append(nb)
            arr[i].name = nb
            arr[i].dtype = BF16 if str(t.dtype) == "torch.bfloat16" else F32
            arr[i].ndim = t.dim()
            for d in range(t.dim()):
                arr[i].shape[d] = t.shape[d]
            arr[i].data = t.data_ptr()
        _check(lib().fm_load_weights(self.h, arr, len(weights)), self.h)

    def set_schedule(self, steps: int, batch: int, tau=None):
        tp = None
        if tau is not None:
            ta = np.ascontiguousarray(tau, dtype=np.float32)
            tp = ta.ctypes.data_as(C.POINTER(C.c_float))
        _check(lib().fm_set_schedule(self.h, steps, batch, tp), self.h)

    def bind_prefix_kv(self, batch: int, prefix_len: int, k=None, v=None, context=None, state=None):
        c, di = self._c, self.device_index
        if k is not None or v is not None:
            if k is None or v is None or len(k) != c.n_layers or len(v) != c.n_layers:
                raise ValueError(f"k and v need one tensor per layer ({c.n_layers})")
            for l in range(c.n_layers):
                check_tensor(k[l], f"prefix k[{l}]", self._tdtype, (batch, prefix_len, 1, c.head_dim), di)
                check_tensor(v[l], f"prefix v[{l}]", self._tdtype, (batch, prefix_len, 1, c.head_dim), di)
        if context is not None:
            check_tensor(context, "context", self._tdtype, (batch, prefix_len, c.ctx_dim), di)
        if state is not None:
            check_tensor(state, "state", _torch().float32, (batch, c.state_tokens, c.state_dim), di)
        kp = vp = None
        if k is not None:
            kp = (C.c_void_p * len(k))(*[t.data_ptr() for t in k])
            vp = (C.c_void_p * len(v))(*[t.data_ptr() for t in v])
        _check(lib().fm_bind_prefix_kv(self.h, batch, prefix_len, kp, vp, _ptr(context), _ptr(state)), self.h)
        self._bound = (batch, prefix_len)

    def prefix_kv_slot(self, layer: int):
        """Device addresses of layer `layer`'s K and V pool planes (see pool_k_col / pool_v_slot
        for where a prefix key goes)."""
        k, v = C.c_void_p(), C.c_void_p()
        _check(lib().fm_prefix_kv_slot(self.h, layer, C.byref(k), C.byref(v)), self.h)
        return k.value, v.value

    def prefix_pool_views(self, layer: int):
        """The K plane [max_batch, cap, dh] and transposed V plane [max_batch, dh, cap] of layer
        `layer` as torch tensors over the pool's own memory (no copy), for a producer that
        writes the prefix in place."""
        torch = _torch()
        cap = query(self.cfg)["pool_capacity"]
        B, dh = self._c.max_batch, self._c.head_dim
        bf16 = self.dtype == BF16
        k, v = self.prefix_kv_slot(layer)

        class _Dev:
            def __init__(self, ptr, shape):
                self.__cuda_array_interface__ = {"shape": shape, "typestr": "<i2" if bf16 else "<f4",
                                                 "data": (ptr, False), "version": 2}
        kt = torch.as_tensor(_Dev(k, (B, cap, dh)), device="cuda")
        vt = torch.as_tensor(_Dev(v, (B, dh, cap)), device="cuda")
        if bf16:
            kt, vt = kt.view(torch.bfloat16), vt.view(torch.bfloat16)
        return kt, vt

    def bind_prefix_inplace(self, batch: int, prefix_len: int):
        """Bind what the pool holds (written through prefix_kv_slot / prefix_pool_views)."""
        _check(lib().fm_bind_prefix_inplace(self.h, batch, prefix_len), self.h)
        self._bound = (batch, prefix_len)

    def set_weight_format(self, fmt: int):
        """WEIGHTS_AS_GIVEN or WEIGHTS_FP8_E4M3; applied by the next load_weights."""
        _check(lib().fm_set_weight_format(self.h, fmt), self.h)

    def bind_prefix_lengths(self, lens=None):
        """Compact prefix length P_b of each bound request (host ints [batch]); None: the whole
        bound prefix for every request."""
        import numpy as np
        arr = p = None
        if lens is not None:
            arr = np.ascontiguousarray(lens, dtype=np.int32).ravel()
            if arr.size != self._bound[0]:
                raise ValueError(f"{arr.size} lengths for a bound batch of {self._bound[0]}")
            p = arr.ctypes.data_as(C.POINTER(C.c_int32))
        _check(lib().fm_bind_prefix_lengths(self.h, p), self.h)

    def bind_context_masks(self, text=None, image=None):
        """DiT text / image masks over the bound context (host booleans [batch, ctx_len],
        true = visible); None: every token visible."""
        import numpy as np
        keep, ptrs = [], []
        for m in (text, image):
            if m is None:
                ptrs.append(None)
                continue
            a = np.ascontiguousarray(m, dtype=np.uint8)
            if a.shape != self._bound:
                raise ValueError(f"mask shape {a.shape}, bound (batch, context length) {self._bound}")
            keep.append(a)
            ptrs.append(a.ctypes.data_as(C.POINTER(C.c_uint8)))
        _check(lib().fm_bind_context_masks(self.h, ptrs[0], ptrs[1]), self.h)

    def chunk_shape(self):
        """[bound batch, H, d_a]: the shape of x0, out, x and v of the bound batch."""
        return (self._bound[0], self._c.action_horizon, self._c.action_dim)

    def _check_chunk(self, t, name):
        check_tensor(t, name, _torch().float32, self.chunk_shape(), self.device_index)

    def denoise(self, x0, steps: int, out=None):
        torch = _torch()
        self._check_chunk(x0, "x0")
        if out is None:
            out = torch.empty_like(x0)
        self._check_chunk(out, "out")
        _check(lib().fm_denoise(self.h, _ptr(x0), steps, _ptr(out)), self.h)
        return out

    def step_velocity(self, x, k: int, v=None):
        torch = _torch()
        self._check_chunk(x, "x")
        if v is None:
            v = torch.empty_like(x)
        self._check_chunk(v, "v")
        _check(lib().fm_step_velocity(self.h, _ptr(x), k, _ptr(v)), self.h)
        return v

    def set_loop_mode(self, mode: int):
        """LOOP_AUTO: the persistent loop kernel where it applies; LOOP_GRAPH: per-op graph."""
        _check(lib().fm_set_loop_mode(self.h, mode), self.h)

    def set_action_stats(self, kind: int, robot_horizon: int, robot_dim: int, q01, q99):
        """Action statistics of the step after the path (kind UNNORM_QUANTILE_EPS / _CLIP)."""
        import numpy as np
        lo = np.ascontiguousarray(q01, np.float32).ravel()
        hi = np.ascontiguousarray(q99, np.float32).ravel()
        if lo.size != robot_dim or hi.size != robot_dim:
            raise ValueError(f"q01 / q99 need {robot_dim} values each")
        fp = C.POINTER(C.c_float)
        _check(lib().fm_set_action_stats(self.h, kind, robot_horizon, robot_dim, lo.ctypes.data_as(fp),
                                         hi.ctypes.data_as(fp)), self.h)
        self._robot = (robot_horizon, robot_dim)

    def unnormalize(self, x, robot_horizon: int, robot_dim: int, out=None):
        """Model-space chunk (device fp32 [B, H, d_a]) -> robot units [B, robot_horizon, robot_dim]."""
        torch = _torch()
        if self._robot is not None and (robot_horizon, robot_dim) != self._robot:
            raise ValueError(f"robot horizon / dim {(robot_horizon, robot_dim)}, the action statistics hold {self._robot}")
        self._check_chunk(x, "x")
        if out is None:
            out = torch.empty((x.shape[0], robot_horizon, robot_dim), dtype=torch.float32, device=x.device)
        check_tensor(out, "out", torch.float32, (self._bound[0], robot_horizon, robot_dim), self.device_index)
        _check(lib().fm_unnormalize(self.h, _ptr(x), _ptr(out)), self.h)
        return out

    def loop_status(self):
        """(persistent kernel serves the loop, fault word); raises FMError on a fault."""
        p, f = C.c_int32(), C.c_uint32()
        _check(lib().fm_loop_status(self.h, C.byref(p), C.byref(f)), self.h)
        return bool(p.value), f.value

    def step_trace(self, x, k: int):
        torch = _torch()
        c = self.cfg
        self._check_chunk(x, "x")
        rows = x.shape[0] * (c.get("state_tokens", 0) + c["action_horizon"])
        tr = torch.empty((c["n_layers"] + 1, rows, c["hidden"]), dtype=torch.float32, device=x.device)
        v = torch.empty_like(x)
        _check(lib().fm_step_trace(self.h, _ptr(x), k, _ptr(v), _ptr(tr)), self.h)
        return v, tr


OP_ROLES = {"inproj": 0, "qkv": 1, "attn": 2, "oproj": 3, "mlp_up": 4, "mlp_down": 5, "out": 6, "loop": 7}
LOOP_AUTO, LOOP_GRAPH = 0, 1
UNNORM_QUANTILE_EPS, UNNORM_QUANTILE_CLIP = 0, 1


def profile_loop(ctx: "Context", x0, steps: int, role: str, out=None):
    """Eager run of the loop with events around every launch of `role`; (total ms, launches)."""
    torch = _torch()
    ctx._check_chunk(x0, "x0")
    if out is None:
        out = torch.empty_like(x0)
    ctx._check_chunk(out, "out")
    ms, n = C.c_float(), C.c_int32()
    _check(lib().fm_profile_loop(ctx.h, _ptr(x0), steps, _ptr(out), OP_ROLES[role], C.byref(ms), C.byref(n)), ctx.h)
    return ms.value, n.value


def op_linear(A, W, bias=None, act: int = 0, out_f32: bool = False):
    torch = _torch()
    if not isinstance(A, torch.Tensor) or not isinstance(W, torch.Tensor) or A.dim() != 2 or W.dim() != 2:
        raise ValueError("op_linear: A and W must be 2-D tensors")
    dt = BF16 if A.dtype == torch.bfloat16 else F32
    M, K = A.shape
    N = W.shape[0]
    check_tensor(A, "A", torch_dtype(dt), (M, K))
    check_tensor(W, "W", torch_dtype(dt), (N, K), A.device.index)
    if bias is not None:
        check_tensor(bias, "bias", torch.float32, (N,), A.device.index)
    out = torch.empty((M, N), dtype=torch.float32 if out_f32 else A.dtype, device=A.device)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().fm_op_linear(dt, M, N, K, _ptr(A), _ptr(W), _ptr(bias), act, _ptr(out), int(out_f32), C.c_void_p(s)))
    return out


def op_attention(q, k, v):
    """q [B, Tq, nh, dh]; k, v [B, nkv, nk, dh]."""
    torch = _torch()
    if not all(isinstance(t, torch.Tensor) and t.dim() == 4 for t in (q, k, v)):
        raise ValueError("op_attention: q, k and v must be 4-D tensors")
    dt = BF16 if q.dtype == torch.bfloat16 else F32
    B, Tq, nh, dh = q.shape
    nkv, nk = k.shape[1], k.shape[2]
    check_tensor(q, "q", torch_dtype(dt), (B, Tq, nh, dh))
    check_tensor(k, "k", torch_dtype(dt), (B, nkv, nk, dh), q.device.index)
    check_tensor(v, "v", torch_dtype(dt), (B, nkv, nk, dh), q.device.index)
    o = torch.empty_like(q)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().fm_op_attention(dt, B, Tq, nh, nkv, nk, dh, _ptr(q), _ptr(k), _ptr(v), _ptr(o), C.c_void_p(s)))
    return o


def op_attention_noalloc(q, k, v, o):
    """op_attention into the caller's o, with the library's fixed scratch: no allocation and no
    synchronization (the work is enqueued on torch's current stream)."""
    torch = _torch()
    if not all(isinstance(t, torch.Tensor) and t.dim() == 4 for t in (q, k, v, o)):
        raise ValueError("op_attention_noalloc: q, k, v and o must be 4-D tensors")
    dt = BF16 if q.dtype == torch.bfloat16 else F32
    B, Tq, nh, dh = q.shape
    nkv, nk = k.shape[1], k.shape[2]
    check_tensor(q, "q", torch_dtype(dt), (B, Tq, nh, dh))
    check_tensor(k, "k", torch_dtype(dt), (B, nkv, nk, dh), q.device.index)
    check_tensor(v, "v", torch_dtype(dt), (B, nkv, nk, dh), q.device.index)
    check_tensor(o, "o", torch_dtype(dt), (B, Tq, nh, dh), q.device.index)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().fm_op_attention_noalloc(dt, B, Tq, nh, nkv, nk, dh, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                         C.c_void_p(s)))
    return o

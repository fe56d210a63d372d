"""ctypes binding of liblla.so (include/lla.h). Argument marshalling only.

Each function has the name of the C entry point it calls and takes torch tensors (or None) in
place of pointers. Before calling, it checks every tensor's device, dtype, contiguity and shape
against the descriptor, because the C ABI receives bare pointers and cannot. All computation runs
in the library's HIP kernels on the current torch stream (or the stream passed in). If liblla.so
is missing this module raises at load time; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblla.so")

(LLA_OK, LLA_ERR_INVALID_ARG, LLA_ERR_UNSUPPORTED, LLA_ERR_WORKSPACE, LLA_ERR_HIP,
 LLA_ERR_SCRATCH_LIMIT) = range(6)
LLA_NOALLOC_SCRATCH_BYTES = 16 << 20
LLA_F32, LLA_BF16, LLA_BF16_Q8, LLA_BF16_I8 = 0, 1, 2, 3
_LOW_BIT = (LLA_BF16_Q8, LLA_BF16_I8)
LLA_PER_HEAD, LLA_2D = 0, 1

# dtype of the arithmetic arrays (q, W, E, mu, x, self K/V, out); low-bit latent caches are
# uint8 rows of lla_latent_row_bytes bytes
_TORCH_DTYPE = {LLA_F32: torch.float32, LLA_BF16: torch.bfloat16, LLA_BF16_Q8: torch.bfloat16,
                LLA_BF16_I8: torch.bfloat16}


class lla_desc(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("d_head", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("r_k", ctypes.c_int32),
        ("r_v", ctypes.c_int32),
        ("n_max", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]

    def __repr__(self):
        return ("lla_desc(variant=%d, dtype=%d, H=%d, d_head=%d, T=%d, r_k=%d, r_v=%d, n_max=%d, "
                "scale=%g)" % (self.variant, self.dtype, self.H, self.d_head, self.T, self.r_k,
                               self.r_v, self.n_max, self.scale))


class LLAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lla_status_string(status)} (status {status})")


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_D = ctypes.POINTER(lla_desc)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run decode_attention_lla_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    lib.lla_abi_version.restype = _I
    lib.lla_abi_version.argtypes = []
    lib.lla_status_string.restype = ctypes.c_char_p
    lib.lla_status_string.argtypes = [_I]
    lib.lla_latent_row_bytes.restype = ctypes.c_size_t
    lib.lla_latent_row_bytes.argtypes = [_I, _I]
    lib.lla_quantize_latents.restype = _I
    lib.lla_quantize_latents.argtypes = [_D, _I, _I, _P, _P, _P, _P, _P, _P]
    lib.lla_workspace_bytes.restype = ctypes.c_size_t
    lib.lla_workspace_bytes.argtypes = [_D, _I, _I]
    lib.lla_encode.restype = _I
    lib.lla_encode.argtypes = [_D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.lla_attend_decode.restype = _I
    lib.lla_attend_decode.argtypes = [_D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, ctypes.c_size_t, _P]
    lib.lla_attend_decode_noalloc.restype = _I
    lib.lla_attend_decode_noalloc.argtypes = [_D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P]
    lib.lla_rope_write.restype = _I
    lib.lla_rope_write.argtypes = [_D, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P]
    lib.lla_rope_workspace_bytes.restype = ctypes.c_size_t
    lib.lla_rope_workspace_bytes.argtypes = [_D, _I]
    lib.lla_attend_decode_rope.restype = _I
    lib.lla_attend_decode_rope.argtypes = [_D, _I, _I, _P, _P, _P, _P, _P, _I, ctypes.c_float,
                                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]
    lib.lla_attend_prefill_rope.restype = _I
    lib.lla_attend_prefill_rope.argtypes = [_D, _I, _I, _I, _P, _P, _P, _P, _P, _I, ctypes.c_float,
                                            _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.lla_reconstruct_workspace_bytes.restype = ctypes.c_size_t
    lib.lla_reconstruct_workspace_bytes.argtypes = [_D, _I]
    lib.lla_attend_decode_reconstruct.restype = _I
    lib.lla_attend_decode_reconstruct.argtypes = lib.lla_attend_decode.argtypes
    lib.lla_gather_workspace_bytes.restype = ctypes.c_size_t
    lib.lla_gather_workspace_bytes.argtypes = [_D, _I, _I]
    lib.lla_attend_decode_gather.restype = _I
    lib.lla_attend_decode_gather.argtypes = [_D, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.lla_attend_prefill.restype = _I
    lib.lla_attend_prefill.argtypes = [_D, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


def make_desc(variant, dtype, H, d_head, T, r_k, r_v, n_max, scale=0.0):
    return lla_desc(int(variant), int(dtype), int(H), int(d_head), int(T), int(r_k), int(r_v),
                    int(n_max), float(scale))


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------

def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, name, shape, dtype, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} is not 16-byte aligned")
    return t.data_ptr()


def _q8_row(r):
    return (r + 4 + 15) // 16 * 16


def _shapes(desc, B):
    """Shapes of the descriptor's arrays; for low-bit latents the cache rows are bytes."""
    H, d, T, rk, rv, n = desc.H, desc.d_head, desc.T, desc.r_k, desc.r_v, desc.n_max
    lk, lv = (_q8_row(rk), _q8_row(rv)) if desc.dtype in _LOW_BIT else (rk, rv)
    if desc.variant == LLA_PER_HEAD:
        return dict(zk=(B, H, n, lk), zv=(B, H, n, lv), Wk=(T, H, d, rk), Wv=(T, H, d, rv),
                    Ek=(H, rk, T * d), Ev=(H, rv, T * d), mu=(H, T * d))
    return dict(zk=(B, n, lk), zv=(B, n, lv), Wk=(T, H * d, rk), Wv=(T, H * d, rv),
                Ek=(rk, T * H * d), Ev=(rv, T * H * d), mu=(T * H * d,))


def _zdt(desc):
    """dtype of the latent cache tensors."""
    return torch.uint8 if desc.dtype in _LOW_BIT else _TORCH_DTYPE[desc.dtype]


def _check(status, where):
    if status != LLA_OK:
        raise LLAError(status, where)


# ---------------------------------------------------------------------------------------------
# entry points (same names as include/lla.h)
# ---------------------------------------------------------------------------------------------

def lla_abi_version():
    return _load().lla_abi_version()


def lla_status_string(status):
    return _load().lla_status_string(int(status)).decode()


def lla_latent_row_bytes(dtype, r):
    return int(_load().lla_latent_row_bytes(int(dtype), int(r)))


def lla_quantize_latents(desc, B, C, zk_src, zv_src, pos, zk, zv, stream=None):
    s = _shapes(desc, B)
    if desc.variant == LLA_PER_HEAD:
        sk, sv = (B, desc.H, C, desc.r_k), (B, desc.H, C, desc.r_v)
    else:
        sk, sv = (B, C, desc.r_k), (B, C, desc.r_v)
    args = [
        _ptr(zk_src, "zk_src", sk, torch.bfloat16), _ptr(zv_src, "zv_src", sv, torch.bfloat16),
        _ptr(pos, "pos", (B,), torch.int32),
        _ptr(zk, "zk", s["zk"], torch.uint8), _ptr(zv, "zv", s["zv"], torch.uint8),
    ]
    st = _load().lla_quantize_latents(ctypes.byref(desc), int(B), int(C), *args,
                                      _stream_ptr(stream))
    _check(st, "lla_quantize_latents")


def lla_workspace_bytes(desc, B, C=1):
    return int(_load().lla_workspace_bytes(ctypes.byref(desc), int(B), int(C)))


def lla_encode(desc, B, C, xk, xv, Ek, Ev, mu_k, mu_v, pos, zk, zv, stream=None):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    xs = (B, C, desc.T, desc.H, desc.d_head)
    args = [
        _ptr(xk, "xk", xs, dt), _ptr(xv, "xv", xs, dt),
        _ptr(Ek, "Ek", s["Ek"], dt), _ptr(Ev, "Ev", s["Ev"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(pos, "pos", (B,), torch.int32),
        _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
    ]
    st = _load().lla_encode(ctypes.byref(desc), int(B), int(C), *args, _stream_ptr(stream))
    _check(st, "lla_encode")


def lla_attend_decode(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self, v_self, out,
                      lse=None, ws=None, stream=None, _entry="lla_attend_decode"):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    qs = (B, desc.H, desc.d_head)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if ws is not None and (ws.device.type != "cuda" or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous device tensor")
    args = [
        _ptr(q, "q", qs, dt), _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
        _ptr(seq_lens, "seq_lens", (B,), torch.int32, True),
        _ptr(Wk, "Wk", s["Wk"], dt), _ptr(Wv, "Wv", s["Wv"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(k_self, "k_self", qs, dt, True), _ptr(v_self, "v_self", qs, dt, True),
        _ptr(out, "out", qs, dt), _ptr(lse, "lse", (B, desc.H), torch.float32, True),
        None if ws is None else ws.data_ptr(),
    ]
    st = getattr(_load(), _entry)(ctypes.byref(desc), int(B), int(t), *args,
                                  ctypes.c_size_t(ws_bytes), _stream_ptr(stream))
    _check(st, _entry)


def lla_attend_decode_noalloc(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self, v_self,
                              out, lse=None, stream=None):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    qs = (B, desc.H, desc.d_head)
    args = [
        _ptr(q, "q", qs, dt), _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
        _ptr(seq_lens, "seq_lens", (B,), torch.int32, True),
        _ptr(Wk, "Wk", s["Wk"], dt), _ptr(Wv, "Wv", s["Wv"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(k_self, "k_self", qs, dt, True), _ptr(v_self, "v_self", qs, dt, True),
        _ptr(out, "out", qs, dt), _ptr(lse, "lse", (B, desc.H), torch.float32, True),
    ]
    st = _load().lla_attend_decode_noalloc(ctypes.byref(desc), int(B), int(t), *args,
                                           _stream_ptr(stream))
    _check(st, "lla_attend_decode_noalloc")


def lla_rope_write(desc, B, C, d_rope, base, k_in, pos, k_rope, stream=None):
    args = [_ptr(k_in, "k_in", (B, C, d_rope), torch.bfloat16), _ptr(pos, "pos", (B,), torch.int32),
            _ptr(k_rope, "k_rope", (B, desc.n_max, d_rope), torch.bfloat16)]
    st = _load().lla_rope_write(ctypes.byref(desc), int(B), int(C), int(d_rope),
                                ctypes.c_float(base), *args, _stream_ptr(stream))
    _check(st, "lla_rope_write")


def lla_rope_workspace_bytes(desc, B):
    return int(_load().lla_rope_workspace_bytes(ctypes.byref(desc), int(B)))


def rope_workspace(desc, B, device="cuda"):
    """A device workspace tensor of lla_rope_workspace_bytes(desc, B) bytes."""
    n = lla_rope_workspace_bytes(desc, B)
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device) if n else None


def lla_attend_decode_rope(desc, B, t, q, q_rope, zk, zv, k_rope, d_rope, base, seq_lens, Wk, Wv,
                           mu_k, mu_v, k_self, v_self, k_rope_self, out, lse=None, ws=None,
                           stream=None):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    qs = (B, desc.H, desc.d_head)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if ws is not None and (ws.device.type != "cuda" or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous device tensor")
    args = [
        _ptr(q, "q", qs, dt), _ptr(q_rope, "q_rope", (B, desc.H, d_rope), torch.bfloat16),
        _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
        _ptr(k_rope, "k_rope", (B, desc.n_max, d_rope), torch.bfloat16),
        ctypes.c_int32(int(d_rope)), ctypes.c_float(base),
        _ptr(seq_lens, "seq_lens", (B,), torch.int32, True),
        _ptr(Wk, "Wk", s["Wk"], dt), _ptr(Wv, "Wv", s["Wv"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(k_self, "k_self", qs, dt, True), _ptr(v_self, "v_self", qs, dt, True),
        _ptr(k_rope_self, "k_rope_self", (B, d_rope), torch.bfloat16, True),
        _ptr(out, "out", qs, dt), _ptr(lse, "lse", (B, desc.H), torch.float32, True),
        None if ws is None else ws.data_ptr(),
    ]
    st = _load().lla_attend_decode_rope(ctypes.byref(desc), int(B), int(t), *args,
                                        ctypes.c_size_t(ws_bytes), _stream_ptr(stream))
    _check(st, "lla_attend_decode_rope")


def lla_attend_prefill_rope(desc, B, C, t, q, q_rope, zk, zv, k_rope, d_rope, base, ctx_lens,
                            Wk, Wv, mu_k, mu_v, out, ws=None, stream=None):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    qs = (B, C, desc.H, desc.d_head)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if ws is not None and (ws.device.type != "cuda" or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous device tensor")
    args = [
        _ptr(q, "q", qs, dt), _ptr(q_rope, "q_rope", (B, C, desc.H, d_rope), torch.bfloat16),
        _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
        _ptr(k_rope, "k_rope", (B, desc.n_max, d_rope), torch.bfloat16),
        ctypes.c_int32(int(d_rope)), ctypes.c_float(base),
        _ptr(ctx_lens, "ctx_lens", (B,), torch.int32),
        _ptr(Wk, "Wk", s["Wk"], dt), _ptr(Wv, "Wv", s["Wv"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(out, "out", qs, dt), None if ws is None else ws.data_ptr(),
    ]
    st = _load().lla_attend_prefill_rope(ctypes.byref(desc), int(B), int(C), int(t), *args,
                                         ctypes.c_size_t(ws_bytes), _stream_ptr(stream))
    _check(st, "lla_attend_prefill_rope")


def lla_reconstruct_workspace_bytes(desc, B):
    return int(_load().lla_reconstruct_workspace_bytes(ctypes.byref(desc), int(B)))


def lla_attend_decode_reconstruct(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self,
                                  v_self, out, lse=None, ws=None, stream=None):
    """The reconstruct-then-attend comparator; arguments as lla_attend_decode, workspace from
    lla_reconstruct_workspace_bytes."""
    lla_attend_decode(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self, v_self, out, lse,
                      ws, stream, _entry="lla_attend_decode_reconstruct")


def reconstruct_workspace(desc, B, device="cuda"):
    """A device workspace tensor of lla_reconstruct_workspace_bytes(desc, B) bytes."""
    n = lla_reconstruct_workspace_bytes(desc, B)
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device) if n else None


def lla_gather_workspace_bytes(desc, B, budget):
    return int(_load().lla_gather_workspace_bytes(ctypes.byref(desc), int(B), int(budget)))


def lla_attend_decode_gather(desc, B, t, q, zk, zv, slots, counts, Wk, Wv, mu_k, mu_v, k_self,
                             v_self, out, lse=None, ws=None, stream=None):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    qs = (B, desc.H, desc.d_head)
    if not isinstance(slots, torch.Tensor) or slots.dim() != 2:
        raise ValueError("slots must be a [B, budget] int32 device tensor")
    budget = int(slots.shape[1])
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if ws is not None and (ws.device.type != "cuda" or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous device tensor")
    args = [
        _ptr(q, "q", qs, dt), _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
        _ptr(slots, "slots", (B, budget), torch.int32), ctypes.c_int32(budget),
        _ptr(counts, "counts", (B,), torch.int32, True),
        _ptr(Wk, "Wk", s["Wk"], dt), _ptr(Wv, "Wv", s["Wv"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(k_self, "k_self", qs, dt, True), _ptr(v_self, "v_self", qs, dt, True),
        _ptr(out, "out", qs, dt), _ptr(lse, "lse", (B, desc.H), torch.float32, True),
        None if ws is None else ws.data_ptr(),
    ]
    st = _load().lla_attend_decode_gather(ctypes.byref(desc), int(B), int(t), *args,
                                          ctypes.c_size_t(ws_bytes), _stream_ptr(stream))
    _check(st, "lla_attend_decode_gather")


def gather_workspace(desc, B, budget, device="cuda"):
    """A device workspace tensor of lla_gather_workspace_bytes(desc, B, budget) bytes (None if 0)."""
    n = lla_gather_workspace_bytes(desc, B, budget)
    if n == 0:
        return None
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)


def lla_attend_prefill(desc, B, C, t, q, zk, zv, ctx_lens, Wk, Wv, mu_k, mu_v, out, ws=None,
                       stream=None):
    dt = _TORCH_DTYPE[desc.dtype]
    s = _shapes(desc, B)
    qs = (B, C, desc.H, desc.d_head)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if ws is not None and (ws.device.type != "cuda" or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous device tensor")
    args = [
        _ptr(q, "q", qs, dt), _ptr(zk, "zk", s["zk"], _zdt(desc)), _ptr(zv, "zv", s["zv"], _zdt(desc)),
        _ptr(ctx_lens, "ctx_lens", (B,), torch.int32),
        _ptr(Wk, "Wk", s["Wk"], dt), _ptr(Wv, "Wv", s["Wv"], dt),
        _ptr(mu_k, "mu_k", s["mu"], dt, True), _ptr(mu_v, "mu_v", s["mu"], dt, True),
        _ptr(out, "out", qs, dt),
        None if ws is None else ws.data_ptr(),
    ]
    st = _load().lla_attend_prefill(ctypes.byref(desc), int(B), int(C), int(t), *args,
                                    ctypes.c_size_t(ws_bytes), _stream_ptr(stream))
    _check(st, "lla_attend_prefill")


def workspace(desc, B, C=1, device="cuda"):
    """A device workspace tensor of lla_workspace_bytes(desc, B, C) bytes (None if 0)."""
    n = lla_workspace_bytes(desc, B, C)
    if n == 0:
        return None
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)

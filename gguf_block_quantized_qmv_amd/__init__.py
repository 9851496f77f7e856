"""Python binding of the gfx950 block-quantized matrix-vector library (libqmv.so).

Argument marshalling only: every function below checks tensor dtypes/devices,
takes device pointers and torch's current stream, and calls the C entry point of
the same name declared in include/qmv.h. All computation happens in the HIP
kernels of the library; there is no fallback path. Importing this package
without a built library raises ImportError.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "QmvError", "lib", "LIB_PATH", "version",
    "qmv_q8_0", "qmv_q4_k", "qmv_q4_k_pair", "qmv_iq4_xs", "qmv_q4_k_moe", "qmv_q4_k_moe_workspace", "qmv_q4_k_moe_prefill",
    "qmv_q4_k_moe_noalloc",
    "qmv_q4_k_moe_prefill_workspace", "qmv_iq4_xs_moe",
    "qmv_iq4_xs_moe_workspace", "qmm_q4_k_prefill_workspace",
    "qmm_q4_k_prefill", "qmv_dequant_q4_k_f32", "qmv_dequant_q4_k_bf16", "qmv_dequant_q8_0_f32",
    "qmv_dequant_iq4_xs_f32", "qmv_q5_k", "qmv_dequant_q5_k_f32", "qmv_q6_k", "qmv_dequant_q6_k_f32", "qmv_q4_0",
    "qmv_dequant_q4_0_f32", "qmv_stream_read", "q4_0_bytes",
    "q4_k_bytes", "q5_k_bytes", "q6_k_bytes", "q8_0_bytes",
    "iq4_xs_bytes", "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmv.so")

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/qmv.h
EXPORTS = {
    "qmv_version": (_c_int, []),
    "qmv_strerror": (ctypes.c_char_p, [_c_int]),
    "qmv_last_error": (ctypes.c_char_p, []),
    "qmv_q8_0": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_q4_k": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_q4_k_pair": (_c_int, [_vp, _vp, _c_size, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_iq4_xs": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_q5_k": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_q6_k": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_q4_0": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "qmv_q4_k_moe_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "qmv_q4_k_moe": (_c_int, [_vp, _vp, _vp, _c_size, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size,
                              _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "qmv_q4_k_moe_noalloc": (_c_int, [_vp, _vp, _vp, _c_size, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "qmv_q4_k_moe_prefill_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "qmv_q4_k_moe_prefill": (_c_int, [_vp, _vp, _vp, _c_size, _vp, _vp, _vp, _vp, _vp, _vp, _c_size,
                                      _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "qmv_iq4_xs_moe_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "qmv_iq4_xs_moe": (_c_int, [_vp, _vp, _vp, _c_size, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size,
                                _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "qmm_q4_k_prefill_workspace": (_c_size, [_c_int, _c_int, _c_int]),
    "qmm_q4_k_prefill": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_size, _vp]),
    "qmv_dequant_q4_k_f32": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_dequant_q4_k_bf16": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_dequant_q8_0_f32": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_dequant_iq4_xs_f32": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_dequant_q5_k_f32": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_dequant_q6_k_f32": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_dequant_q4_0_f32": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _vp]),
    "qmv_stream_read": (_c_int, [_vp, _c_size, _vp, _c_int, _c_int, _c_int, _vp]),
}


def _load():
    # torch's HIP build ships its own libamdhip64 (same soname as the system one).
    # Loading torch first makes libqmv.so bind to that already-loaded runtime, so
    # the process holds exactly one HIP runtime; two runtimes in one process do
    # not share a device (the second reports that no device is present).
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python gguf_block_quantized_qmv_amd/build.py` "
            "(or __graft_entry__.build()) first")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class QmvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = lib.qmv_last_error().decode() if code == -8 else ""
        super().__init__(f"{where}: {lib.qmv_strerror(code).decode()} (code {code})" + (f" [{detail}]" if detail else ""))


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise QmvError(rc, where)


def version() -> int:
    return lib.qmv_version()


def q4_k_bytes(n: int, k: int) -> int:
    return n * (k // 256) * 144


def q5_k_bytes(n: int, k: int) -> int:
    return n * (k // 256) * 176


def q6_k_bytes(n: int, k: int) -> int:
    return n * (k // 256) * 210


def q4_0_bytes(n: int, k: int) -> int:
    return n * (k // 32) * 18


def q8_0_bytes(n: int, k: int) -> int:
    return n * (k // 32) * 34


# ---------------------------------------------------------------- marshalling helpers

def _torch():
    import torch
    return torch


def _dev(t, name, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory (got {t.device})")
    if dtypes and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


# ---------------------------------------------------------------- entry points

def qmv_q8_0(w, x, n: int, k: int, y=None, stream=None):
    """y[m, n] = x[m, k] @ dequant(w)^T for a Q8_0 matrix w (uint8 bytes) and fp32 x."""
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", (torch.float32,))
    m = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    _check(lib.qmv_q8_0(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)), "qmv_q8_0")
    return y


def qmv_q4_k(w, x, n: int, k: int, y=None, stream=None):
    """y[m, n] = x[m, k] @ dequant(w)^T for a Q4_K matrix w (uint8 bytes) and bf16 x (1 <= m <= 4)."""
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    m = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    _check(lib.qmv_q4_k(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)), "qmv_q4_k")
    return y


def qmv_q4_k_pair(w0, w1, x, n: int, k: int, y0=None, y1=None, stream=None):
    """(x @ dequant(w0)^T, x @ dequant(w1)^T) for two Q4_K matrices of one shape, in one launch."""
    torch = _torch()
    _dev(w0, "w0", (torch.uint8,))
    _dev(w1, "w1", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    if _nbytes(w0) != _nbytes(w1):
        raise ValueError("qmv_q4_k_pair: w0 and w1 must have the same size")
    m = x.shape[0] if x.dim() == 2 else 1
    if y0 is None:
        y0 = torch.empty((m, n), dtype=torch.float32, device=x.device)
    if y1 is None:
        y1 = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y0, "y0", (torch.float32,))
    _dev(y1, "y1", (torch.float32,))
    _check(lib.qmv_q4_k_pair(_ptr(w0), _ptr(w1), _nbytes(w0), _ptr(x), _ptr(y0), _ptr(y1), m, n, k, _stream(stream)),
           "qmv_q4_k_pair")
    return y0, y1


def qmv_q4_k_moe_workspace(t: int, hidden: int, ffn: int, n_experts: int, top_k: int) -> int:
    return lib.qmv_q4_k_moe_workspace(t, hidden, ffn, n_experts, top_k)


def _moe(fn, ws_fn, name, w_gate, w_up, w_down, logits, x, hidden, ffn, n_experts, top_k, y, ws, routing, stream):
    torch = _torch()
    for wname, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _dev(t, wname, (torch.uint8,))
    _dev(logits, "logits", (torch.float32,))
    _dev(x, "x", _bf16_types())
    tc = x.shape[0] if x.dim() == 2 else 1
    dev = x.device
    if y is None:
        y = torch.empty((tc, hidden), dtype=torch.float32, device=dev)
    _dev(y, "y", (torch.float32,))
    need = ws_fn(tc, hidden, ffn, n_experts, top_k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(ws, "ws", (torch.uint8,))
    ids = wts = pairs = None
    if routing:
        ids = torch.empty((tc, top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((tc, top_k), dtype=torch.float32, device=dev)
        pairs = torch.empty((tc * top_k, 2), dtype=torch.int32, device=dev)
    rc = fn(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _nbytes(w_gate), _ptr(logits), _ptr(x),
            _ptr(y), _ptr(ids), _ptr(wts), _ptr(pairs), _ptr(ws), _nbytes(ws),
            tc, hidden, ffn, n_experts, top_k, _stream(stream))
    _check(rc, name)
    return y, ids, wts, pairs


def qmv_q4_k_moe(w_gate, w_up, w_down, logits, x, hidden: int, ffn: int, n_experts: int, top_k: int,
                 y=None, ws=None, routing: bool = True, stream=None):
    """Routed-expert MoE FFN; returns (y, topk_ids, topk_w, pairs) (the last three None if not routing)."""
    return _moe(lib.qmv_q4_k_moe, qmv_q4_k_moe_workspace, "qmv_q4_k_moe", w_gate, w_up, w_down, logits, x,
                hidden, ffn, n_experts, top_k, y, ws, routing, stream)


def qmv_q4_k_moe_prefill_workspace(t: int, hidden: int, ffn: int, n_experts: int, top_k: int) -> int:
    return lib.qmv_q4_k_moe_prefill_workspace(t, hidden, ffn, n_experts, top_k)


def qmv_q4_k_moe_prefill(w_gate, w_up, w_down, logits, x, hidden: int, ffn: int, n_experts: int, top_k: int,
                         y=None, ws=None, routing: bool = True, stream=None):
    """Routed-expert MoE FFN over a prompt's tokens; returns (y, topk_ids, topk_w) (the last two None if not routing)."""
    torch = _torch()
    for wname, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _dev(t, wname, (torch.uint8,))
    _dev(logits, "logits", (torch.float32,))
    _dev(x, "x", _bf16_types())
    tc = x.shape[0] if x.dim() == 2 else 1
    dev = x.device
    if y is None:
        y = torch.empty((tc, hidden), dtype=torch.float32, device=dev)
    _dev(y, "y", (torch.float32,))
    need = qmv_q4_k_moe_prefill_workspace(tc, hidden, ffn, n_experts, top_k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(ws, "ws", (torch.uint8,))
    ids = wts = None
    if routing:
        ids = torch.empty((tc, top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((tc, top_k), dtype=torch.float32, device=dev)
    _check(lib.qmv_q4_k_moe_prefill(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _nbytes(w_gate), _ptr(logits), _ptr(x),
                                    _ptr(y), _ptr(ids), _ptr(wts), _ptr(ws), _nbytes(ws), tc, hidden, ffn, n_experts,
                                    top_k, _stream(stream)), "qmv_q4_k_moe_prefill")
    return y, ids, wts


def qmv_iq4_xs_moe_workspace(t: int, hidden: int, ffn: int, n_experts: int, top_k: int) -> int:
    return lib.qmv_iq4_xs_moe_workspace(t, hidden, ffn, n_experts, top_k)


def qmv_iq4_xs_moe(w_gate, w_up, w_down, logits, x, hidden: int, ffn: int, n_experts: int, top_k: int,
                   y=None, ws=None, routing: bool = True, stream=None):
    """Routed-expert MoE FFN on IQ4_XS expert banks; returns (y, topk_ids, topk_w, pairs)."""
    return _moe(lib.qmv_iq4_xs_moe, qmv_iq4_xs_moe_workspace, "qmv_iq4_xs_moe", w_gate, w_up, w_down, logits, x,
                hidden, ffn, n_experts, top_k, y, ws, routing, stream)


def qmm_q4_k_prefill_workspace(m: int, n: int, k: int) -> int:
    return lib.qmm_q4_k_prefill_workspace(m, n, k)


def qmm_q4_k_prefill(w, x, n: int, k: int, y=None, ws=None, stream=None):
    """Y[m, n] = X[m, k] @ bf16(dequant(w))^T on bf16 matrix cores, fp32 accumulation.

    ws: None allocates the workspace the shape's K split needs (if any), or a
    uint8 device tensor of at least qmm_q4_k_prefill_workspace(m, n, k) bytes to reuse.
    """
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    if ws is None:
        need = qmm_q4_k_prefill_workspace(m, n, k)
        ws = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    if ws is not None:
        _dev(ws, "ws", (torch.uint8,))
    _check(lib.qmm_q4_k_prefill(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _ptr(ws), _nbytes(ws),
                                _stream(stream)), "qmm_q4_k_prefill")
    return y


def qmv_q5_k(w, x, n: int, k: int, y=None, stream=None):
    """y[m, n] = x[m, k] @ dequant(w)^T for a Q5_K matrix w (uint8 bytes) and bf16 x (1 <= m <= 4)."""
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    m = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    _check(lib.qmv_q5_k(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)), "qmv_q5_k")
    return y


def qmv_dequant_q5_k_f32(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.qmv_dequant_q5_k_f32(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)), "qmv_dequant_q5_k_f32")
    return out


def qmv_dequant_q4_k_f32(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.qmv_dequant_q4_k_f32(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)), "qmv_dequant_q4_k_f32")
    return out


def qmv_dequant_q4_k_bf16(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.int16, device=w.device)
    _dev(out, "out", _bf16_types())
    _check(lib.qmv_dequant_q4_k_bf16(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)),
           "qmv_dequant_q4_k_bf16")
    return out


def qmv_dequant_q8_0_f32(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.qmv_dequant_q8_0_f32(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)), "qmv_dequant_q8_0_f32")
    return out


def qmv_iq4_xs(w, x, n: int, k: int, y=None, stream=None):
    """y[m, n] = x[m, k] @ dequant_iq4_xs(w)^T for m = 1..4 bf16 rows (fp32 out)."""
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    m = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    _check(lib.qmv_iq4_xs(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)), "qmv_iq4_xs")
    return y


def qmv_dequant_iq4_xs_f32(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.qmv_dequant_iq4_xs_f32(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)),
           "qmv_dequant_iq4_xs_f32")
    return out


def iq4_xs_bytes(n: int, k: int) -> int:
    """Byte size of an n x k IQ4_XS matrix (136-byte blocks of 256 weights along k)."""
    return n * (k // 256) * 136


def qmv_q6_k(w, x, n: int, k: int, y=None, stream=None):
    """y[m, n] = x[m, k] @ dequant(w)^T for a Q6_K matrix w (uint8 bytes) and bf16 x (1 <= m <= 4)."""
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    m = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    _check(lib.qmv_q6_k(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)), "qmv_q6_k")
    return y


def qmv_dequant_q6_k_f32(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.qmv_dequant_q6_k_f32(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)), "qmv_dequant_q6_k_f32")
    return out


def qmv_q4_0(w, x, n: int, k: int, y=None, stream=None):
    """y[m, n] = x[m, k] @ dequant(w)^T for a Q4_0 matrix w (uint8 bytes) and bf16 x (1 <= m <= 4)."""
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    _dev(x, "x", _bf16_types())
    m = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, "y", (torch.float32,))
    _check(lib.qmv_q4_0(_ptr(w), _nbytes(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)), "qmv_q4_0")
    return y


def qmv_dequant_q4_0_f32(w, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _dev(w, "w", (torch.uint8,))
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.qmv_dequant_q4_0_f32(_ptr(w), _nbytes(w), _ptr(out), n, k, _stream(stream)), "qmv_dequant_q4_0_f32")
    return out


def qmv_stream_read(buf, grid: int = 1024, depth: int = 4, nontemporal: bool = False, sink=None, stream=None):
    """Plain streaming read of a device buffer (a measurement aid); returns the
    per-workgroup XOR words (uint32 as int32, [grid])."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(grid, dtype=torch.int32, device=buf.device)
    _check(lib.qmv_stream_read(_ptr(buf), _nbytes(buf), _ptr(sink), grid, depth, int(nontemporal), _stream(stream)),
           "qmv_stream_read")
    return sink

"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Functions carry the C entry points' names and argument order. Tensor arguments
are torch tensors on the current HIP device (or None for an optional pointer);
only their data pointers cross the boundary, and every step of the layer runs
in the library's kernels. A non-zero status raises MoeError. If libmoe.so has
not been built, every call raises MoeLibraryMissing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_GELU_MLP, MOE_SWIGLU = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
(MOE_STAGE_ROUTE, MOE_STAGE_PERMUTE, MOE_STAGE_FFN, MOE_STAGE_SHARED, MOE_STAGE_FORWARD, MOE_STAGE_EXPERT,
 MOE_STAGE_ROUTE_NOISY, MOE_STAGE_BACKWARD) = range(8)


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({status_name(status)})")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("score", ctypes.c_int32), ("renorm", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("capacity", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGS = {
    "moe_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_permute": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_permute_noalloc": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_ffn": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P,
                                       _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_up": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P,
                                     _P, ctypes.c_size_t, _P]),
    "moe_expert_down": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P,
                                       _P, ctypes.c_size_t, _P]),
    "moe_shared_ffn": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, ctypes.c_size_t, _P]),
    "moe_update_bias": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, ctypes.c_float, _P, _P]),
    "moe_route_noisy": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "moe_backward": (ctypes.c_int, [ctypes.POINTER(moe_shape)] + [_P] * 17 + [ctypes.c_float] + [_P] * 10
                     + [ctypes.c_size_t, _P]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}
EXPORTED = tuple(_SIGS)
# measurement probes (include/moe_probe.h), not part of the layer
_PROBE_SIGS = {
    "moe_probe_copy": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int, _P]),
    "moe_probe_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P]),
    "moe_probe_mfma_flops": (ctypes.c_double, [ctypes.c_int, ctypes.c_int]),
}
PROBES = tuple(_PROBE_SIGS)

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once); raises MoeLibraryMissing if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeLibraryMissing(f"{LIB_PATH} not found: build it with `python -m sparse_routing_expert_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in {**_SIGS, **_PROBE_SIGS}.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_name(status: int) -> str:
    try:
        return lib().moe_status_str(status).decode()
    except MoeLibraryMissing:
        return str(status)


def make_shape(T, d_model, d_ff, E, k, dtype="bf16", act="swiglu", score="softmax", renorm=True,
               d_ff_shared=0, capacity=0) -> moe_shape:
    return moe_shape(int(T), int(d_model), int(d_ff), int(E), int(k),
                     MOE_BF16 if dtype == "bf16" else MOE_F32,
                     MOE_SWIGLU if act == "swiglu" else MOE_GELU_MLP,
                     MOE_SIGMOID if score == "sigmoid" else MOE_SOFTMAX, int(bool(renorm)), int(d_ff_shared),
                     int(capacity))


def shape_of(cfg, T: Optional[int] = None, capacity: int = 0) -> moe_shape:
    """moe_shape of an inputs.LayerConfig (optionally with another token count or an expert capacity)."""
    return make_shape(cfg.T if T is None else T, cfg.d, cfg.F, cfg.E, cfg.k, cfg.dtype, cfg.act, cfg.score,
                      cfg.renorm, cfg.Fs, capacity)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws) -> int:
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def _check(name: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(name, status)


def moe_workspace_bytes(shape: moe_shape, stage: int) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(shape), int(stage), ctypes.byref(out)))
    return out.value


def moe_route(shape, x, w_router, sel_bias, logits, topk_idx, topk_w, counts, stats, ws, stream=None) -> None:
    _check("moe_route", lib().moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(logits),
                                        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(stats), _ptr(ws),
                                        _nbytes(ws), _stream(stream)))


def moe_permute(shape, topk_idx, x, offsets, sorted_token, inv_pos, x_perm, ws, stream=None) -> None:
    _check("moe_permute", lib().moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(x), _ptr(offsets),
                                            _ptr(sorted_token), _ptr(inv_pos), _ptr(x_perm), _ptr(ws), _nbytes(ws),
                                            _stream(stream)))


def moe_permute_noalloc(shape, topk_idx, x, offsets, sorted_token, inv_pos, x_perm, stream=None) -> None:
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(ctypes.byref(shape), _ptr(topk_idx), _ptr(x),
                                                            _ptr(offsets), _ptr(sorted_token), _ptr(inv_pos),
                                                            _ptr(x_perm), _stream(stream)))


def moe_grouped_ffn(shape, e_begin, e_end, x_perm, offsets, w_in, b_in, w_out, b_out, y_perm, ws, stream=None) -> None:
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(ctypes.byref(shape), int(e_begin), int(e_end), _ptr(x_perm),
                                                    _ptr(offsets), _ptr(w_in), _ptr(b_in), _ptr(w_out), _ptr(b_out),
                                                    _ptr(y_perm), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_expert_up(shape, e_begin, e_end, x_perm, offsets, w_in, b_in, h, ws, stream=None) -> None:
    _check("moe_expert_up", lib().moe_expert_up(ctypes.byref(shape), int(e_begin), int(e_end), _ptr(x_perm),
                                                _ptr(offsets), _ptr(w_in), _ptr(b_in), _ptr(h), _ptr(ws), _nbytes(ws),
                                                _stream(stream)))


def moe_expert_down(shape, e_begin, e_end, h, offsets, w_out, b_out, y_perm, ws, stream=None) -> None:
    _check("moe_expert_down", lib().moe_expert_down(ctypes.byref(shape), int(e_begin), int(e_end), _ptr(h),
                                                    _ptr(offsets), _ptr(w_out), _ptr(b_out), _ptr(y_perm), _ptr(ws),
                                                    _nbytes(ws), _stream(stream)))


def moe_shared_ffn(shape, x, ws_in, ws_out, y_shared, ws, stream=None) -> None:
    _check("moe_shared_ffn", lib().moe_shared_ffn(ctypes.byref(shape), _ptr(x), _ptr(ws_in), _ptr(ws_out),
                                                  _ptr(y_shared), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_combine(shape, y_perm, inv_pos, topk_w, y_shared, y, stream=None) -> None:
    _check("moe_combine", lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(inv_pos), _ptr(topk_w),
                                            _ptr(y_shared), _ptr(y), _stream(stream)))


def moe_forward(shape, x, w_router, sel_bias, w_in, b_in, w_out, b_out, ws_in, ws_out, y, topk_idx_out, topk_w_out,
                counts_out, stats_out, ws, stream=None) -> None:
    _check("moe_forward", lib().moe_forward(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(w_in),
                                            _ptr(b_in), _ptr(w_out), _ptr(b_out), _ptr(ws_in), _ptr(ws_out), _ptr(y),
                                            _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(counts_out), _ptr(stats_out),
                                            _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_update_bias(shape, counts, gamma: float, sel_bias, stream=None) -> None:
    _check("moe_update_bias", lib().moe_update_bias(ctypes.byref(shape), _ptr(counts), float(gamma), _ptr(sel_bias),
                                                    _stream(stream)))


def moe_route_noisy(shape, x, w_router, w_noise, noise, sel_bias, logits, topk_idx, topk_w, counts, stats, ws,
                    stream=None) -> None:
    _check("moe_route_noisy", lib().moe_route_noisy(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(w_noise),
                                                    _ptr(noise), _ptr(sel_bias), _ptr(logits), _ptr(topk_idx),
                                                    _ptr(topk_w), _ptr(counts), _ptr(stats), _ptr(ws), _nbytes(ws),
                                                    _stream(stream)))



def moe_backward(shape, x, w_router, w_in, b_in, w_out, b_out, ws_in, ws_out, logits, topk_idx, topk_w, counts,
                 offsets, inv_pos, x_perm, y_perm, dy, aux_coef: float, dx, dw_router, dw_in, db_in, dw_out, db_out,
                 dws_in, dws_out, dlogits, ws, stream=None) -> None:
    _check("moe_backward", lib().moe_backward(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(w_in), _ptr(b_in), _ptr(w_out), _ptr(b_out), _ptr(ws_in),
        _ptr(ws_out), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(inv_pos),
        _ptr(x_perm), _ptr(y_perm), _ptr(dy), float(aux_coef), _ptr(dx), _ptr(dw_router), _ptr(dw_in), _ptr(db_in),
        _ptr(dw_out), _ptr(db_out), _ptr(dws_in), _ptr(dws_out), _ptr(dlogits), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_probe_copy(src, dst, nbytes: int, blocks: int, stream=None) -> None:
    _check("moe_probe_copy", lib().moe_probe_copy(_ptr(src), _ptr(dst), int(nbytes), int(blocks), _stream(stream)))


def moe_probe_mfma(blocks: int, iters: int, out, stream=None) -> float:
    """Enqueues the MFMA-only loop; returns its floating-point work."""
    _check("moe_probe_mfma", lib().moe_probe_mfma(int(blocks), int(iters), _ptr(out), _stream(stream)))
    return float(lib().moe_probe_mfma_flops(int(blocks), int(iters)))

"""Python binding of libquads.so, the QUADS rollout hot path on MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (outputs and workspace are torch
tensors) and the current stream.  The functions carry the C ABI's names; see
include/quads.h for the exact contract of each call.

bf16 tensors may be passed as torch.bfloat16, torch.int16 or torch.uint16
(bit patterns).  Results are returned as torch tensors on the input's device.
"""

import ctypes
import os

import torch

__all__ = [
    "QuadsError", "lib", "library_path",
    "quads_nvfp4_quantize", "quads_nvfp4_quantize_partials", "quads_nvfp4_quantize_rows",
    "quads_rac_quantize", "quads_rac_quantize_partials", "quads_moe_w4a4_gemm_amax",
    "quads_moe_w4a4_gemm_amax_groups",
    "quads_rac_quantize_experts", "quads_moe_w4a4_gemm_sel_experts",
    "quads_nvfp4_weight_qdq", "quads_moe_pack", "quads_moe_w4a4_gemm",
    "quads_moe_w4a4_gemm_rowscale", "quads_moe_combine",
    "quads_mx_quantize", "quads_moe_mx_gemm",
    "EPI_NONE", "EPI_SWIGLU", "OUT_F32", "OUT_BF16", "MX_FP8", "MX_FP4",
]

EPI_NONE, EPI_SWIGLU = 0, 1
OUT_F32, OUT_BF16 = 0, 1
MX_FP8, MX_FP4 = 0, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libquads.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SIGNATURES = {
    "quads_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "quads_version": (ctypes.c_char_p, []),
    "quads_nvfp4_quantize_ws": (_SZ, [_I64, _I64]),
    "quads_nvfp4_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "quads_nvfp4_quantize_partials": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P]),
    "quads_nvfp4_quantize_rows": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "quads_rac_quantize_ws": (_SZ, [_I64, _I64, _I32]),
    "quads_rac_quantize": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _SZ, _P]),
    "quads_rac_quantize_partials": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _I64, _P, _P, _P,
                                                   _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "quads_rac_quantize_noalloc": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P,
                                                  _P, _P, _P]),
    "quads_rac_quantize_experts_ws": (_SZ, [_I64, _I64, _I32, _I32]),
    "quads_rac_quantize_experts": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _I32, _P, _P, _P, _P,
                                                  _P, _P, _P, _P, _P, _SZ, _P]),
    "quads_moe_w4a4_gemm_sel_experts": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _P, _P,
                                                       _I32, _P, _P, _P, _P, _I32, _I64,
                                                       ctypes.c_int, ctypes.c_int, _P, _P, _SZ,
                                                       _P]),
    "quads_nvfp4_weight_qdq_ws": (_SZ, [_I64, _I64, _I64]),
    "quads_nvfp4_weight_qdq": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ,
                                              _P]),
    "quads_moe_pack_ws": (_SZ, [_I64, _I32, _I32]),
    "quads_moe_pack": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "quads_moe_w4a4_gemm_ws": (_SZ, [_I64, _I64, _I32, _I32, _I64]),
    "quads_moe_w4a4_gemm": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _I32,
                                           _P, _P, _P, _P, _I32, _I64, ctypes.c_int,
                                           ctypes.c_int, _P, _P, _SZ, _P]),
    "quads_moe_w4a4_gemm_amax_groups": (_I64, [_I64, _I64, _I32, _I32, _I64]),
    "quads_moe_w4a4_gemm_amax": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _I32,
                                                _P, _P, _P, _P, _I32, _I64, _P, _P, _I64, _P,
                                                _SZ, _P]),
    "quads_moe_w4a4_gemm_rowscale": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P,
                                                    _I32, _I64, ctypes.c_int, ctypes.c_int, _P,
                                                    _P, _SZ, _P]),
    "quads_moe_combine": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _I64, _I32, _I64, _P, _P]),
    "quads_mx_quantize": (ctypes.c_int, [_P, _I64, _I64, ctypes.c_int, _P, _P, _P]),
    "quads_mx_rac_quantize_ws": (_SZ, [_I64, _I64, _I32]),
    "quads_mx_rac_quantize": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P,
                                             _SZ, _P]),
    "quads_moe_mx_rac_gemm_ws": (_SZ, [_I32, _I64, _I32]),
    "quads_moe_mx_rac_gemm": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _P, _I32, _P, _P,
                                             _P, _I32, _I64, ctypes.c_int, ctypes.c_int, _P, _P,
                                             _SZ, _P]),
    "quads_moe_mx_gemm": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _P, _I32, _I64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P]),
}


class QuadsError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().quads_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")


def lib():
    """The loaded libquads.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with "
                "`python -m nvfp4_w4a4_quantized_act_amd.build` (there is no fallback)")
        handle = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name, None)
            if fn is not None:
                fn.restype = res
                fn.argtypes = args
        _lib = handle
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ws(nbytes, device):
    nbytes = max(int(nbytes), 16)
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _check(fn, status):
    if status != 0:
        raise QuadsError(fn, status)


def _bits16(x):
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return x.contiguous()
    raise TypeError("bf16 tensors must be torch.bfloat16, int16 or uint16 bit patterns")


def quads_nvfp4_quantize(x, ts_in=None):
    """NVFP4 of bf16 x [M, K] -> (nib uint8 [M, K/2], scale uint8 [M, K/16], ts fp32 [1])."""
    x = _bits16(x)
    m, k = x.shape
    dev = x.device
    nib = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    ws, nws = _ws(lib().quads_nvfp4_quantize_ws(m, k), dev)
    _check("quads_nvfp4_quantize", lib().quads_nvfp4_quantize(
        _ptr(x), m, k, _ptr(ts_in), _ptr(nib), _ptr(scale), _ptr(ts), _ptr(ws), nws,
        _stream(dev)))
    return nib, scale, ts


def quads_nvfp4_quantize_partials(x, amax_part):
    """NVFP4 of bf16 x [M, K] with max|x| from partial maxima (uint32 bf16 magnitude bits
    [groups], e.g. from quads_moe_w4a4_gemm_amax) -> (nib, scale, ts)."""
    x = _bits16(x)
    m, k = x.shape
    dev = x.device
    nib = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    _check("quads_nvfp4_quantize_partials", lib().quads_nvfp4_quantize_partials(
        _ptr(x), m, k, _ptr(amax_part), int(amax_part.numel()), _ptr(nib), _ptr(scale), _ptr(ts),
        _stream(dev)))
    return nib, scale, ts


def quads_nvfp4_quantize_rows(x):
    """NVFP4 of bf16 x [M, K] with one tensor scale per row -> (nib uint8 [M, K/2],
    scale uint8 [M, K/16], ts fp32 [M])."""
    x = _bits16(x)
    m, k = x.shape
    dev = x.device
    nib = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(max(m, 1), dtype=torch.float32, device=dev)[:m]
    _check("quads_nvfp4_quantize_rows", lib().quads_nvfp4_quantize_rows(
        _ptr(x), m, k, _ptr(nib), _ptr(scale), _ptr(ts), _stream(dev)))
    return nib, scale, ts


def quads_rac_quantize(x, k, want_score=False):
    """RAC of bf16 x [M, K] with k channels -> dict of device tensors
    (nib, scale, ts, sel, r_nib, r_scale, r_ts[, score])."""
    x = _bits16(x)
    m, kd = x.shape
    dev = x.device
    out = dict(
        nib=torch.empty((m, kd // 2), dtype=torch.uint8, device=dev),
        scale=torch.empty((m, kd // 16), dtype=torch.uint8, device=dev),
        ts=torch.empty(4, dtype=torch.float32, device=dev)[:1],
        sel=torch.empty(max(k, 4), dtype=torch.int32, device=dev)[:k],
        r_nib=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
        r_scale=torch.empty((m, k // 16), dtype=torch.uint8, device=dev),
        r_ts=torch.empty(4, dtype=torch.float32, device=dev)[:1],
    )
    if want_score:
        out["score"] = torch.empty(kd, dtype=torch.float64, device=dev)
    ws, nws = _ws(lib().quads_rac_quantize_ws(m, kd, k), dev)
    _check("quads_rac_quantize", lib().quads_rac_quantize(
        _ptr(x), m, kd, k, _ptr(out["nib"]), _ptr(out["scale"]), _ptr(out["ts"]),
        _ptr(out["sel"]) if k else None, _ptr(out["r_nib"]) if k and m else None,
        _ptr(out["r_scale"]) if k and m else None, _ptr(out["r_ts"]), _ptr(out.get("score")),
        _ptr(ws), nws, _stream(dev)))
    return out


def quads_rac_quantize_partials(x, k, amax_part, want_score=False):
    """quads_rac_quantize with max|x| from partial maxima (uint32 [groups])."""
    x = _bits16(x)
    m, kd = x.shape
    dev = x.device
    out = dict(
        nib=torch.empty((m, kd // 2), dtype=torch.uint8, device=dev),
        scale=torch.empty((m, kd // 16), dtype=torch.uint8, device=dev),
        ts=torch.empty(4, dtype=torch.float32, device=dev)[:1],
        sel=torch.empty(max(k, 4), dtype=torch.int32, device=dev)[:k],
        r_nib=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
        r_scale=torch.empty((m, k // 16), dtype=torch.uint8, device=dev),
        r_ts=torch.empty(4, dtype=torch.float32, device=dev)[:1],
    )
    if want_score:
        out["score"] = torch.empty(kd, dtype=torch.float64, device=dev)
    ws, nws = _ws(lib().quads_rac_quantize_ws(m, kd, k), dev)
    _check("quads_rac_quantize_partials", lib().quads_rac_quantize_partials(
        _ptr(x), m, kd, k, _ptr(amax_part), int(amax_part.numel()), _ptr(out["nib"]),
        _ptr(out["scale"]), _ptr(out["ts"]),
        _ptr(out["sel"]) if k else None, _ptr(out["r_nib"]) if k and m else None,
        _ptr(out["r_scale"]) if k and m else None, _ptr(out["r_ts"]), _ptr(out.get("score")),
        _ptr(ws), nws, _stream(dev)))
    return out


RAC_NOALLOC_SCRATCH_BYTES = 64 << 20


def quads_rac_quantize_noalloc(x, k, want_score=False, out=None):
    """quads_rac_quantize through the entry point that allocates no device
    memory (the library's static per-GPU scratch).  `out` may hold the output
    tensors (a dict as returned); else they are allocated here, by torch."""
    x = _bits16(x)
    m, kd = x.shape
    dev = x.device
    if out is None:
        out = dict(
            nib=torch.empty((m, kd // 2), dtype=torch.uint8, device=dev),
            scale=torch.empty((m, kd // 16), dtype=torch.uint8, device=dev),
            ts=torch.empty(4, dtype=torch.float32, device=dev)[:1],
            sel=torch.empty(max(k, 4), dtype=torch.int32, device=dev)[:k],
            r_nib=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
            r_scale=torch.empty((m, k // 16), dtype=torch.uint8, device=dev),
            r_ts=torch.empty(4, dtype=torch.float32, device=dev)[:1],
        )
        if want_score:
            out["score"] = torch.empty(kd, dtype=torch.float64, device=dev)
    _check("quads_rac_quantize_noalloc", lib().quads_rac_quantize_noalloc(
        _ptr(x), m, kd, k, _ptr(out["nib"]), _ptr(out["scale"]), _ptr(out["ts"]),
        _ptr(out["sel"]) if k else None, _ptr(out["r_nib"]) if k and m else None,
        _ptr(out["r_scale"]) if k and m else None, _ptr(out["r_ts"]), _ptr(out.get("score")),
        _stream(dev)))
    return out


def quads_rac_quantize_experts(x, k, offsets, want_score=False):
    """RAC with one selection per expert on packed bf16 x [M, K] (offsets int32
    [E+1] on the device).  Returns a dict like quads_rac_quantize, with sel
    [E, k], r_ts [E] and score [E, K]."""
    x = _bits16(x)
    m, kd = x.shape
    e = offsets.shape[0] - 1
    dev = x.device
    out = {
        "nib": torch.empty((m, kd // 2), dtype=torch.uint8, device=dev),
        "scale": torch.empty((m, kd // 16), dtype=torch.uint8, device=dev),
        "ts": torch.empty(4, dtype=torch.float32, device=dev)[:1],
        "sel": torch.empty((e, k), dtype=torch.int32, device=dev),
        "r_nib": torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
        "r_scale": torch.empty((m, k // 16), dtype=torch.uint8, device=dev),
        "r_ts": torch.empty(e, dtype=torch.float32, device=dev),
    }
    if want_score:
        out["score"] = torch.empty((e, kd), dtype=torch.float64, device=dev)
    ws, nws = _ws(lib().quads_rac_quantize_experts_ws(m, kd, k, e), dev)
    _check("quads_rac_quantize_experts", lib().quads_rac_quantize_experts(
        _ptr(x), m, kd, k, _ptr(offsets), e, _ptr(out["nib"]), _ptr(out["scale"]),
        _ptr(out["ts"]), _ptr(out["sel"]) if k else None, _ptr(out["r_nib"]) if k else None,
        _ptr(out["r_scale"]) if k else None, _ptr(out["r_ts"]), _ptr(out.get("score")),
        _ptr(ws), nws, _stream(dev)))
    return out


def quads_nvfp4_weight_qdq(w, want_dq=False):
    """Weight QDQ of bf16 w [E, N, K] -> (nib, scale, ts [E], dq bf16 bits or None)."""
    w = _bits16(w)
    e, n, k = w.shape
    dev = w.device
    nib = torch.empty((e, n, k // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((e, n, k // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(max(e, 4), dtype=torch.float32, device=dev)[:e]
    dq = torch.empty((e, n, k), dtype=torch.int16, device=dev) if want_dq else None
    ws, nws = _ws(lib().quads_nvfp4_weight_qdq_ws(e, n, k), dev)
    _check("quads_nvfp4_weight_qdq", lib().quads_nvfp4_weight_qdq(
        _ptr(w), e, n, k, _ptr(nib), _ptr(scale), _ptr(ts), _ptr(dq), _ptr(ws), nws,
        _stream(dev)))
    return nib, scale, ts, dq


def quads_moe_pack(topk_ids, num_experts):
    """Pack int32 [T, topk] routes -> (offsets [E+1], row_token [T*topk], pos [T*topk])."""
    ids = topk_ids.contiguous()
    if ids.dtype != torch.int32:
        raise TypeError("topk_ids must be int32")
    t, topk = ids.shape
    dev = ids.device
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(max(t * topk, 4), dtype=torch.int32, device=dev)[:t * topk]
    pos = torch.empty(max(t * topk, 4), dtype=torch.int32, device=dev)[:t * topk]
    ws, nws = _ws(lib().quads_moe_pack_ws(t, topk, num_experts), dev)
    _check("quads_moe_pack", lib().quads_moe_pack(
        _ptr(ids), t, topk, num_experts, _ptr(offsets), _ptr(row_token), _ptr(pos), _ptr(ws),
        nws, _stream(dev)))
    return offsets, row_token, pos


def quads_moe_w4a4_gemm(a, w, n, rows=None, r=None, sel=None, offsets=None, row_token=None,
                        epilogue=EPI_NONE, out_dtype=OUT_F32, out=None):
    """Grouped W4A4 GEMM.  a = (nib, scale, ts); r = (nib, scale, ts) or None;
    w = (nib [E,N,K/2], scale, ts [E]).  Returns out [rows, N] (or [rows, N/2]
    for SwiGLU), fp32 or bf16 bits (int16)."""
    a_nib, a_scale, a_ts = a
    w_nib, w_scale, w_ts = w
    e = w_nib.shape[0]
    kd = a_nib.shape[1] * 2
    if rows is None:
        rows = row_token.shape[0] if row_token is not None else a_nib.shape[0]
    k = 0 if r is None else int(sel.shape[0])
    dev = a_nib.device
    ncols = n // 2 if epilogue == EPI_SWIGLU else n
    if out is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.int16
        out = torch.empty((rows, ncols), dtype=dt, device=dev)
    ws, nws = _ws(lib().quads_moe_w4a4_gemm_ws(rows, kd, k, e, n), dev)
    rn, rs, rt = r if r is not None else (None, None, None)
    _check("quads_moe_w4a4_gemm", lib().quads_moe_w4a4_gemm(
        _ptr(a_nib), _ptr(a_scale), _ptr(a_ts), _ptr(row_token), rows, kd,
        _ptr(rn) if k else None, _ptr(rs) if k else None, _ptr(rt) if k else None,
        _ptr(sel) if k else None, k, _ptr(w_nib), _ptr(w_scale), _ptr(w_ts), _ptr(offsets), e,
        n, epilogue, out_dtype, _ptr(out), _ptr(ws), nws, _stream(dev)))
    return out


def quads_moe_w4a4_gemm_amax_groups(rows, kd, k, e, n):
    """Partial-maximum slots of a SwiGLU GEMM call of these sizes (0: sizes rejected)."""
    return int(lib().quads_moe_w4a4_gemm_amax_groups(rows, kd, k, e, n))


def quads_moe_w4a4_gemm_amax(a, w, n, rows=None, r=None, sel=None, offsets=None,
                             row_token=None, out=None, amax_part=None):
    """SwiGLU W4A4 GEMM (bf16 h [rows, N/2]) that also writes the partial maxima of |h|.
    Returns (h, amax_part uint32 [groups])."""
    a_nib, a_scale, a_ts = a
    w_nib, w_scale, w_ts = w
    e = w_nib.shape[0]
    kd = a_nib.shape[1] * 2
    if rows is None:
        rows = row_token.shape[0] if row_token is not None else a_nib.shape[0]
    k = 0 if r is None else int(sel.shape[0])
    dev = a_nib.device
    if out is None:
        out = torch.empty((rows, n // 2), dtype=torch.int16, device=dev)
    if amax_part is None:
        groups = max(quads_moe_w4a4_gemm_amax_groups(rows, kd, k, e, n), 1)
        amax_part = torch.empty(groups, dtype=torch.int32, device=dev)
    ws, nws = _ws(lib().quads_moe_w4a4_gemm_ws(rows, kd, k, e, n), dev)
    rn, rs, rt = r if r is not None else (None, None, None)
    _check("quads_moe_w4a4_gemm_amax", lib().quads_moe_w4a4_gemm_amax(
        _ptr(a_nib), _ptr(a_scale), _ptr(a_ts), _ptr(row_token), rows, kd,
        _ptr(rn) if k else None, _ptr(rs) if k else None, _ptr(rt) if k else None,
        _ptr(sel) if k else None, k, _ptr(w_nib), _ptr(w_scale), _ptr(w_ts), _ptr(offsets), e,
        n, _ptr(out), _ptr(amax_part), int(amax_part.numel()), _ptr(ws), nws, _stream(dev)))
    return out, amax_part


def quads_moe_w4a4_gemm_rowscale(a, w, n, rows=None, offsets=None, row_token=None,
                                 epilogue=EPI_NONE, out_dtype=OUT_F32, out=None):
    """Grouped W4A4 GEMM with one activation tensor scale per A row:
    a = (nib, scale, ts [Ta]) as from quads_nvfp4_quantize_rows; no RAC."""
    a_nib, a_scale, a_ts = a
    w_nib, w_scale, w_ts = w
    e = w_nib.shape[0]
    kd = a_nib.shape[1] * 2
    if rows is None:
        rows = row_token.shape[0] if row_token is not None else a_nib.shape[0]
    dev = a_nib.device
    ncols = n // 2 if epilogue == EPI_SWIGLU else n
    if out is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.int16
        out = torch.empty((rows, ncols), dtype=dt, device=dev)
    ws, nws = _ws(lib().quads_moe_w4a4_gemm_ws(rows, kd, 0, e, n), dev)
    _check("quads_moe_w4a4_gemm_rowscale", lib().quads_moe_w4a4_gemm_rowscale(
        _ptr(a_nib), _ptr(a_scale), _ptr(a_ts), _ptr(row_token), rows, kd, _ptr(w_nib),
        _ptr(w_scale), _ptr(w_ts), _ptr(offsets), e, n, epilogue, out_dtype, _ptr(out),
        _ptr(ws), nws, _stream(dev)))
    return out


def quads_moe_w4a4_gemm_sel_experts(a, w, n, r, sel, offsets, epilogue=EPI_NONE,
                                    out_dtype=OUT_F32, out=None):
    """Grouped W4A4 GEMM with per-expert compensation: a = (nib, scale, ts) in
    packed order, r = (nib, scale, ts [E]), sel [E, k] (quads_rac_quantize_experts)."""
    a_nib, a_scale, a_ts = a
    w_nib, w_scale, w_ts = w
    e = w_nib.shape[0]
    kd = a_nib.shape[1] * 2
    rows = a_nib.shape[0]
    k = int(sel.shape[1])
    dev = a_nib.device
    ncols = n // 2 if epilogue == EPI_SWIGLU else n
    if out is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.int16
        out = torch.empty((rows, ncols), dtype=dt, device=dev)
    ws, nws = _ws(lib().quads_moe_w4a4_gemm_ws(rows, kd, k, e, n), dev)
    rn, rs, rt = r
    _check("quads_moe_w4a4_gemm_sel_experts", lib().quads_moe_w4a4_gemm_sel_experts(
        _ptr(a_nib), _ptr(a_scale), _ptr(a_ts), rows, kd, _ptr(rn) if k else None,
        _ptr(rs) if k else None, _ptr(rt), _ptr(sel) if k else None, k, _ptr(w_nib),
        _ptr(w_scale), _ptr(w_ts), _ptr(offsets), e, n, epilogue, out_dtype, _ptr(out),
        _ptr(ws), nws, _stream(dev)))
    return out


def quads_moe_combine(y, pos, topk_w, y_dtype=OUT_F32):
    """out fp32 [T, N] = sum_slot topk_w[t, slot] * y[pos[t*topk+slot]]."""
    t, topk = topk_w.shape
    n = y.shape[1]
    dev = y.device
    out = torch.empty((t, n), dtype=torch.float32, device=dev)
    _check("quads_moe_combine", lib().quads_moe_combine(
        _ptr(y), y_dtype, _ptr(pos), _ptr(topk_w.contiguous()), t, topk, n, _ptr(out),
        _stream(dev)))
    return out


def quads_mx_quantize(x, fmt=MX_FP8):
    """MX quantization of bf16 x [..., K] (rows = the leading dims) ->
    (codes uint8 [..., K] (FP8) or [..., K/2] (FP4), scales uint8 [..., K/32])."""
    x = _bits16(x)
    k = x.shape[-1]
    m = x.numel() // k if k else 0
    dev = x.device
    cw = k if fmt == MX_FP8 else k // 2
    codes = torch.empty(tuple(x.shape[:-1]) + (cw,), dtype=torch.uint8, device=dev)
    scales = torch.empty(tuple(x.shape[:-1]) + (k // 32,), dtype=torch.uint8, device=dev)
    _check("quads_mx_quantize", lib().quads_mx_quantize(
        _ptr(x), m, k, fmt, _ptr(codes), _ptr(scales), _stream(dev)))
    return codes, scales


def quads_moe_mx_gemm(a, w, n, rows=None, offsets=None, row_token=None, fmt=MX_FP8,
                      epilogue=EPI_NONE, out_dtype=OUT_F32, out=None):
    """Grouped MX GEMM.  a = (codes, scales) [Ta, ...]; w = (codes [E, N, ...],
    scales [E, N, K/32]).  Returns out [rows, N] (or [rows, N/2] for SwiGLU)."""
    a_codes, a_scale = a
    w_codes, w_scale = w
    e = w_codes.shape[0]
    kd = a_scale.shape[-1] * 32
    if rows is None:
        rows = row_token.shape[0] if row_token is not None else a_codes.shape[0]
    dev = a_codes.device
    ncols = n // 2 if epilogue == EPI_SWIGLU else n
    if out is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.int16
        out = torch.empty((rows, ncols), dtype=dt, device=dev)
    _check("quads_moe_mx_gemm", lib().quads_moe_mx_gemm(
        _ptr(a_codes), _ptr(a_scale), _ptr(row_token), rows, kd, _ptr(w_codes), _ptr(w_scale),
        _ptr(offsets), e, n, fmt, epilogue, out_dtype, _ptr(out), _stream(dev)))
    return out


def quads_mx_rac_quantize(x, k, want_score=False):
    """RAC on the MX FP4 mode of bf16 x [M, K] with k channels -> dict of
    device tensors (codes, scales, sel, r_codes, r_scales[, score])."""
    x = _bits16(x)
    m, kd = x.shape
    dev = x.device
    out = dict(
        codes=torch.empty((m, kd // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((m, kd // 32), dtype=torch.uint8, device=dev),
        sel=torch.empty(max(k, 4), dtype=torch.int32, device=dev)[:k],
        r_codes=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
        r_scales=torch.empty((m, k // 32), dtype=torch.uint8, device=dev),
    )
    if want_score:
        out["score"] = torch.empty(kd, dtype=torch.float64, device=dev)
    ws, nws = _ws(lib().quads_mx_rac_quantize_ws(m, kd, k), dev)
    _check("quads_mx_rac_quantize", lib().quads_mx_rac_quantize(
        _ptr(x), m, kd, k, _ptr(out["codes"]), _ptr(out["scales"]),
        _ptr(out["sel"]) if k else None, _ptr(out["r_codes"]) if k and m else None,
        _ptr(out["r_scales"]) if k and m else None, _ptr(out.get("score")), _ptr(ws), nws,
        _stream(dev)))
    return out


def quads_moe_mx_rac_gemm(a, r, sel, w, n, rows=None, offsets=None, row_token=None,
                          epilogue=EPI_NONE, out_dtype=OUT_F32):
    """MX FP4 grouped GEMM with the RAC compensation.  a = (codes, scales),
    r = (r_codes, r_scales) or None, w = (codes [E, N, K/2], scales [E, N, K/32])."""
    a_codes, a_scale = a
    w_codes, w_scale = w
    e = w_codes.shape[0]
    kd = a_codes.shape[1] * 2
    if rows is None:
        rows = row_token.shape[0] if row_token is not None else a_codes.shape[0]
    k = 0 if r is None else int(sel.shape[0])
    dev = a_codes.device
    ncols = n // 2 if epilogue == EPI_SWIGLU else n
    dt = torch.float32 if out_dtype == OUT_F32 else torch.int16
    out = torch.empty((rows, ncols), dtype=dt, device=dev)
    ws, nws = _ws(lib().quads_moe_mx_rac_gemm_ws(e, n, k), dev)
    rc, rs = r if r is not None else (None, None)
    _check("quads_moe_mx_rac_gemm", lib().quads_moe_mx_rac_gemm(
        _ptr(a_codes), _ptr(a_scale), _ptr(row_token), rows, kd, _ptr(rc) if k else None,
        _ptr(rs) if k else None, _ptr(sel) if k else None, k, _ptr(w_codes), _ptr(w_scale),
        _ptr(offsets), e, n, epilogue, out_dtype, _ptr(out), _ptr(ws), nws, _stream(dev)))
    return out

"""NVFP4 weight quantization with GPTQ + Schur Replay on AMD Instinct MI355X.

Thin ctypes binding over libnvq.so (C ABI in include/nvq.h).  Every step of
the quantization runs in the library's HIP kernels; this module only checks
tensor metadata, allocates outputs and workspaces with torch, and passes raw
device pointers plus torch's current HIP stream.  There is no CPU fallback:
importing fails if the library is missing.

Method: "Replay the Curvature: Accurate and Scalable NVFP4 Quantization for
Large Language Model Inference" (arXiv 2609.36654), Abstract.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvq.so")

NVQ_DTYPE_F32 = 0
NVQ_DTYPE_BF16 = 1
FLAG_RTN = 1
FLAG_NO_ERR = 2
FLAG_FP64 = 4
FLAG_INDEP = 8
FLAG_CHECK_FINITE = 16
FLAG_CHOL_FACTOR = 32

EXPORTS = [
    "hessian_workspace_size", "hessian_accumulate",
    "hessian_grouped_workspace_size", "hessian_accumulate_grouped",
    "hessian_host_workspace_size", "hessian_host_staging_size", "hessian_accumulate_host",
    "factor_hinv_workspace_size", "factor_hinv", "factor_hinv_batched",
    "factor_chol_workspace_size", "factor_chol", "factor_chol_batched",
    "nvfp4_global_scale_workspace_size", "nvfp4_global_scale",
    "gptq_nvfp4_workspace_size", "gptq_nvfp4_quantize", "gptq_nvfp4_quantize_batched",
    "nvfp4_dequantize", "nvfp4_gemm_workspace_size", "nvfp4_gemm", "nvfp4_gemm_noalloc", "nvq_check_finite",
    "nvq_status_string", "nvq_last_error",
]


class NvqError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m post_nvfp4_weight_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I32, F32, U32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_uint)
    sig = {
        "hessian_workspace_size": (SZ, [I64, I64, I32]),
        "hessian_accumulate": (I32, [P, I32, I64, I64, I64, P, P, SZ, P]),
        "hessian_grouped_workspace_size": (SZ, [P, I64, I64, I32]),
        "hessian_host_workspace_size": (SZ, [I64, I64, I32]),
        "hessian_host_staging_size": (SZ, [I64, I64, I32]),
        "hessian_accumulate_host": (I32, [P, I32, I64, I64, I64, P, I64, P, SZ, P, SZ, P, P]),
        "hessian_accumulate_grouped": (I32, [P, I32, I64, I64, I64, P, P, I64, P, P, SZ, P]),
        "factor_hinv_batched": (I32, [P, I64, I64, I64, F32, P, I64, P, P, P, SZ, P]),
        "gptq_nvfp4_quantize_batched": (I32, [P, I32, I64, I64, I64, I64, I64, P, I64, P, I64, P, I32, U32, P, P,
                                               P, P, P, SZ, P]),
        "factor_hinv_workspace_size": (SZ, [I64]),
        "factor_hinv": (I32, [P, I64, F32, P, P, P, P, SZ, P]),
        "factor_chol_workspace_size": (SZ, [I64]),
        "factor_chol": (I32, [P, I64, F32, P, P, P, P, SZ, P]),
        "factor_chol_batched": (I32, [P, I64, I64, I64, F32, P, I64, P, P, P, SZ, P]),
        "nvfp4_global_scale_workspace_size": (SZ, [I64, I64]),
        "nvfp4_global_scale": (I32, [P, I32, I64, I64, I64, P, P, SZ, P]),
        "gptq_nvfp4_workspace_size": (SZ, [I64, I64, U32]),
        "gptq_nvfp4_quantize": (I32, [P, I32, I64, I64, I64, P, P, P, I32, U32, P, P, P, P, P, SZ, P]),
        "nvfp4_dequantize": (I32, [P, P, P, I64, I64, P, I32, P]),
        "nvfp4_gemm_workspace_size": (SZ, [I64, I64, I64]),
        "nvfp4_gemm": (I32, [P, I32, I64, I64, I64, P, P, P, I64, P, I32, I64, P, SZ, P]),
        "nvfp4_gemm_noalloc": (I32, [P, I32, I64, I64, I64, P, P, P, I64, P, I32, I64, P]),
        "nvq_check_finite": (I32, [P, I32, I64, I64, I64, P, P]),
        "nvq_status_string": (ctypes.c_char_p, [I32]),
        "nvq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(fn, status):
    if status != 0:
        raise NvqError(fn, status, lib.nvq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return NVQ_DTYPE_BF16
    if t.dtype == torch.float32:
        return NVQ_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    # torch's caching allocator returns 256-byte aligned blocks (checked by the library).
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _rows(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    return t.shape[0], t.shape[1], t.stride(0)


def hessian_accumulate(X, H=None, ws=None):
    """H += X^T X (fp32 [k, k], full symmetric on return).  X: [n, k] bf16 or fp32."""
    n, k, ldx = _rows(X, "X")
    if H is None:
        H = torch.zeros(k, k, dtype=torch.float32, device=X.device)
    need = lib.hessian_workspace_size(n, k, _dtype_code(X))
    if ws is None or ws.numel() < need:
        ws = _workspace(need, X.device)
    _check("hessian_accumulate", lib.hessian_accumulate(_ptr(X), _dtype_code(X), n, k, ldx, _ptr(H), _ptr(ws),
                                                        need, _stream()))
    return H


def nvfp4_gemm(X, codes, scales, g, out_dtype=torch.float32, Y=None):
    """Y = X dequant(W)^T for bf16 activations X [T, k] and NVFP4 weights (codes [m, k/2], scales [m, k/16], g)."""
    T, k, ldx = _rows(X, "X")
    m = codes.shape[0]
    if Y is None:
        Y = torch.empty(T, m, dtype=out_dtype, device=X.device)
    need = lib.nvfp4_gemm_workspace_size(T, k, m)
    ws = _workspace(need, X.device) if need else None
    _check("nvfp4_gemm", lib.nvfp4_gemm(_ptr(X), _dtype_code(X), T, k, ldx, _ptr(codes), _ptr(scales), _ptr(g), m,
                                        _ptr(Y), _dtype_code(Y), Y.stride(0), _ptr(ws), need, _stream()))
    return Y


def nvfp4_gemm_noalloc(X, codes, scales, g, Y):
    """Y = X dequant(W)^T into a preallocated Y [T, m] (fp32 or bf16); the library allocates nothing."""
    T, k, ldx = _rows(X, "X")
    m = codes.shape[0]
    _check("nvfp4_gemm_noalloc", lib.nvfp4_gemm_noalloc(_ptr(X), _dtype_code(X), T, k, ldx, _ptr(codes),
                                                        _ptr(scales), _ptr(g), m, _ptr(Y), _dtype_code(Y),
                                                        Y.stride(0), _stream()))
    return Y


_copy_streams = {}


def hessian_accumulate_host(X, H=None, chunk=32768, staging=True, device="cuda:0"):
    """H += X^T X with X in host memory, streamed to the device in chunks.

    X: a CPU torch tensor (bf16 or fp32, pinned or not) or a NumPy array whose
    rows are contiguous: uint16 holding bf16 bits, or float32 (a np.memmap of
    a file on disk works).  Pageable X goes through pinned staging buffers
    (staging=True); the copies run on a library copy stream of default
    priority, overlapped with the accumulation on the current stream.
    """
    if isinstance(X, torch.Tensor):
        if X.device.type != "cpu" or X.dim() != 2 or X.stride(1) != 1:
            raise ValueError("X must be a 2-D CPU tensor with contiguous rows")
        code = _dtype_code(X)
        ptr, ldx, pinned = X.data_ptr(), X.stride(0), X.is_pinned()
    else:
        import numpy as np
        X = np.asarray(X) if not isinstance(X, np.ndarray) else X
        if X.ndim != 2 or X.strides[1] != X.itemsize:
            raise ValueError("X must be 2-D with contiguous rows")
        if X.dtype == np.uint16:
            code = NVQ_DTYPE_BF16
        elif X.dtype == np.float32:
            code = NVQ_DTYPE_F32
        else:
            raise ValueError("NumPy X must be uint16 (bf16 bits) or float32")
        ptr, ldx, pinned = X.ctypes.data, X.strides[0] // X.itemsize, False
    n, k = X.shape
    dev = torch.device(device)
    if H is None:
        H = torch.zeros(k, k, dtype=torch.float32, device=dev)
    need = lib.hessian_host_workspace_size(chunk, k, code)
    ws = _workspace(need, dev)
    stg, stg_n = None, 0
    if staging and not pinned:
        stg_n = lib.hessian_host_staging_size(chunk, k, code)
        stg = torch.empty(max(1, stg_n), dtype=torch.uint8, pin_memory=True)
    if dev not in _copy_streams:
        _copy_streams[dev] = torch.cuda.Stream(device=dev)
    cs = _copy_streams[dev]
    cur = torch.cuda.current_stream(dev)
    cs.wait_stream(cur)   # H and the workspace are ready before the first copy
    _check("hessian_accumulate_host",
           lib.hessian_accumulate_host(ctypes.c_void_p(ptr), code, n, k, ldx, _ptr(H), chunk, _ptr(ws), need,
                                       _ptr(stg), stg_n, ctypes.c_void_p(cur.cuda_stream),
                                       ctypes.c_void_p(cs.cuda_stream)))
    ws.record_stream(cs)
    return H


def factor_hinv(H, damp_rel=0.01, U=None, ws=None):
    """Returns (U, lam, info) as device tensors: (H + lam I)^-1 = U^T U, lam = damp_rel * mean(diag H)."""
    k = H.shape[0]
    U = torch.empty_like(H) if U is None else U
    lam = torch.empty(1, dtype=torch.float32, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    need = lib.factor_hinv_workspace_size(k)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, H.device)
    _check("factor_hinv", lib.factor_hinv(_ptr(H), k, float(damp_rel), _ptr(U), _ptr(lam), _ptr(info), _ptr(ws),
                                          need, _stream()))
    return U, lam, info


def nvfp4_global_scale(W):
    """Device fp32 scalar tensor g = fl32(max|W| / 2688) (1 for an all-zero W)."""
    m, k, ldw = _rows(W, "W")
    g = torch.empty(1, dtype=torch.float32, device=W.device)
    need = lib.nvfp4_global_scale_workspace_size(m, k)
    ws = _workspace(need, W.device)
    _check("nvfp4_global_scale", lib.nvfp4_global_scale(_ptr(W), _dtype_code(W), m, k, ldw, _ptr(g), _ptr(ws),
                                                        need, _stream()))
    return g


def gptq_nvfp4_quantize(W, U, H, g, n_cand=16, flags=0, ws=None, out=None):
    """NVFP4 quantization of W [m, k]; returns dict(codes [m, k/2] u8, scales [m, k/16] u8,
    row_err [m] f32 or None, row_loss [m] f32)."""
    m, k, ldw = _rows(W, "W")
    dev = W.device
    if out is None:
        out = {
            "codes": torch.empty(m, k // 2, dtype=torch.uint8, device=dev),
            "scales": torch.empty(m, k // 16, dtype=torch.uint8, device=dev),
            "row_err": None if (flags & FLAG_NO_ERR) else torch.empty(m, dtype=torch.float32, device=dev),
            "row_loss": torch.empty(m, dtype=torch.float32, device=dev),
        }
    need = lib.gptq_nvfp4_workspace_size(m, k, flags)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    _check("gptq_nvfp4_quantize", lib.gptq_nvfp4_quantize(
        _ptr(W), _dtype_code(W), m, k, ldw, _ptr(U), _ptr(H), _ptr(g), int(n_cand), int(flags),
        _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["row_err"]), _ptr(out["row_loss"]), _ptr(ws), need,
        _stream()))
    return out


def nvfp4_dequantize(codes, scales, g, out_dtype=torch.float32):
    m, kh = codes.shape
    k = kh * 2
    out = torch.empty(m, k, dtype=out_dtype, device=codes.device)
    _check("nvfp4_dequantize", lib.nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(g), m, k, _ptr(out),
                                                    _dtype_code(out), _stream()))
    return out


def hessian_accumulate_grouped(X, tok_idx, grp_off, H=None):
    """Per-group H[e] += X[idx_e]^T X[idx_e]; tok_idx: device int32 [total], grp_off: host sequence [G+1]."""
    import numpy as np
    n, k, ldx = _rows(X, "X")
    off = np.ascontiguousarray(np.asarray(grp_off, dtype=np.int64))
    G = len(off) - 1
    if H is None:
        H = torch.zeros(G, k, k, dtype=torch.float32, device=X.device)
    offp = off.ctypes.data_as(ctypes.c_void_p)
    need = lib.hessian_grouped_workspace_size(offp, G, k, _dtype_code(X))
    ws = _workspace(need, X.device)
    idx = tok_idx if tok_idx.dtype == torch.int32 else tok_idx.to(torch.int32)
    _check("hessian_accumulate_grouped", lib.hessian_accumulate_grouped(
        _ptr(X), _dtype_code(X), n, k, ldx, _ptr(idx), offp, G, _ptr(H), _ptr(ws), need, _stream()))
    return H


def factor_hinv_batched(H, damp_rel=0.01, max_ws_bytes=8 << 30):
    """H: [B, k, k] -> (U [B, k, k], lam [B], info [B]) as device tensors.

    The workspace holds as many matrices' buffers as fit in max_ws_bytes (at
    least one, at most B): the library factors that many matrices per pass,
    every launch covering all of them."""
    B, k = H.shape[0], H.shape[1]
    U = torch.empty_like(H)
    lam = torch.empty(B, dtype=torch.float32, device=H.device)
    info = torch.empty(B, dtype=torch.int32, device=H.device)
    one = lib.factor_hinv_workspace_size(k)
    need = one * max(1, min(B, max_ws_bytes // one))
    ws = _workspace(need, H.device)
    _check("factor_hinv_batched", lib.factor_hinv_batched(_ptr(H), k, B, H.stride(0), float(damp_rel), _ptr(U),
                                                          U.stride(0), _ptr(lam), _ptr(info), _ptr(ws), need,
                                                          _stream()))
    return U, lam, info


def factor_chol_batched(H, damp_rel=0.01, max_ws_bytes=8 << 30):
    """H: [B, k, k] -> (V [B, k, k], lam [B], info [B]) as device tensors, each V as
    factor_chol gives it (for FLAG_CHOL_FACTOR); passes of as many matrices as
    fit in max_ws_bytes of workspace."""
    B, k = H.shape[0], H.shape[1]
    V = torch.empty_like(H)
    lam = torch.empty(B, dtype=torch.float32, device=H.device)
    info = torch.empty(B, dtype=torch.int32, device=H.device)
    one = lib.factor_chol_workspace_size(k)
    need = one * max(1, min(B, max_ws_bytes // one))
    ws = _workspace(need, H.device)
    _check("factor_chol_batched", lib.factor_chol_batched(_ptr(H), k, B, H.stride(0), float(damp_rel), _ptr(V),
                                                          V.stride(0), _ptr(lam), _ptr(info), _ptr(ws), need,
                                                          _stream()))
    return V, lam, info


def gptq_nvfp4_quantize_batched(W, U, H, g, n_cand=16, flags=0, max_ws_bytes=8 << 30):
    """W: [B, m, k]; U, H: [B, k, k] (or None as the flags allow); g: device fp32 [B].

    The workspace holds as many matrices' working buffers as fit in
    max_ws_bytes (at least one): that many are quantized per pass."""
    B, m, k = W.shape
    dev = W.device
    if W.stride(2) != 1:
        raise ValueError("W must have unit column stride")
    out = {
        "codes": torch.empty(B, m, k // 2, dtype=torch.uint8, device=dev),
        "scales": torch.empty(B, m, k // 16, dtype=torch.uint8, device=dev),
        "row_err": None if (flags & FLAG_NO_ERR) else torch.empty(B, m, dtype=torch.float32, device=dev),
        "row_loss": torch.empty(B, m, dtype=torch.float32, device=dev),
    }
    one = lib.gptq_nvfp4_workspace_size(m, k, flags)
    need = one * max(1, min(B, max_ws_bytes // one))
    ws = _workspace(need, dev)
    _check("gptq_nvfp4_quantize_batched", lib.gptq_nvfp4_quantize_batched(
        _ptr(W), _dtype_code(W), B, m, k, W.stride(1), W.stride(0), _ptr(U), 0 if U is None else U.stride(0),
        _ptr(H), 0 if H is None else H.stride(0), _ptr(g), int(n_cand), int(flags), _ptr(out["codes"]),
        _ptr(out["scales"]), _ptr(out["row_err"]), _ptr(out["row_loss"]), _ptr(ws), need, _stream()))
    return out


def check_finite(A):
    """Device int32 tensor [1]: 0 if every value of A [rows, cols] is finite, else 1 + the first bad row."""
    rows, cols, ld = _rows(A, "A")
    status = torch.empty(1, dtype=torch.int32, device=A.device)
    _check("nvq_check_finite", lib.nvq_check_finite(_ptr(A), _dtype_code(A), rows, cols, ld, _ptr(status), _stream()))
    return status


def factor_chol(H, damp_rel=0.01, V=None, ws=None):
    """Returns (V, lam, info) as device tensors: H + lam I = R R^T with R upper triangular,
    V = -R_ij / R_jj above the diagonal, R_ii on it, 0 below (for FLAG_CHOL_FACTOR)."""
    k = H.shape[0]
    V = torch.empty_like(H) if V is None else V
    lam = torch.empty(1, dtype=torch.float32, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    need = lib.factor_chol_workspace_size(k)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, H.device)
    _check("factor_chol", lib.factor_chol(_ptr(H), k, float(damp_rel), _ptr(V), _ptr(lam), _ptr(info), _ptr(ws),
                                          need, _stream()))
    return V, lam, info


def quantize_layer(W, X, n_cand=16, damp_rel=0.01, flags=0, chol=False):
    """Whole layer: H = X^T X, the factor (U from factor_hinv, or with chol V from factor_chol and
    FLAG_CHOL_FACTOR), g, the sweep and the weighted error (all on the GPU)."""
    H = hessian_accumulate(X)
    if chol:
        U, lam, info = factor_chol(H, damp_rel)
        flags |= FLAG_CHOL_FACTOR
    else:
        U, lam, info = factor_hinv(H, damp_rel)
    g = nvfp4_global_scale(W)
    res = gptq_nvfp4_quantize(W, U, H, g, n_cand, flags)
    res.update(H=H, U=U, lam=lam, info=info, g=g)
    return res

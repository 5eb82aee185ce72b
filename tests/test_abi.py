"""The C-ABI library loads, exports every function declared in include/nvq.h, and
rejects bad arguments on the host (no GPU work is enqueued by these calls)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["hessian_accumulate", "factor_hinv", "gptq_nvfp4_quantize", "nvfp4_dequantize",
              "nvfp4_global_scale", "nvq_status_string", "nvq_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    import post_nvfp4_weight_amd as nvq
    lib = ctypes.CDLL(nvq.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(nvq.EXPORTS) == _declared()


def test_host_validation_rejects_bad_arguments():
    import post_nvfp4_weight_amd as nvq
    lib = nvq.lib
    P = ctypes.c_void_p
    fake = P(4096)   # never dereferenced: validation fails first
    # k not a multiple of 16
    assert lib.hessian_accumulate(fake, 1, 10, 24, 24, fake, None, 0, None) == -2
    # H missing
    assert lib.hessian_accumulate(fake, 1, 10, 32, 32, None, None, 0, None) == -1
    # unknown dtype
    assert lib.hessian_accumulate(fake, 7, 10, 32, 32, fake, None, 0, None) == -3
    assert b"x_dtype" in lib.nvq_last_error()
    # n = 0 is a no-op
    assert lib.hessian_accumulate(None, 1, 0, 32, 32, fake, None, 0, None) == 0
    # candidate count out of range
    rc = lib.gptq_nvfp4_quantize(fake, 1, 16, 32, 32, fake, fake, fake, 17, 0, fake, fake, fake, None,
                                 fake, 1 << 30, None)
    assert rc == -4
    # workspace too small
    rc = lib.gptq_nvfp4_quantize(fake, 1, 16, 32, 32, fake, fake, fake, 16, 0, fake, fake, fake, None,
                                 P(1 << 20), 16, None)
    assert rc == -5
    # U required without the RTN flag
    rc = lib.gptq_nvfp4_quantize(fake, 1, 16, 32, 32, None, fake, fake, 16, 0, fake, fake, fake, None,
                                 fake, 1 << 30, None)
    assert rc == -1
    # factor: negative damping, overlapping U
    assert lib.factor_hinv(fake, 32, ctypes.c_float(-1.0), P(8192), fake, fake, fake, 1 << 30, None) == -6
    assert lib.factor_hinv(fake, 32, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None) == -6
    # the Cholesky-factor form: the same checks, and a workspace too small
    assert lib.factor_chol(fake, 32, ctypes.c_float(-1.0), P(8192), fake, fake, fake, 1 << 30, None) == -6
    assert lib.factor_chol(fake, 32, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None) == -6
    assert lib.factor_chol(fake, 24, ctypes.c_float(0.01), P(8192), fake, fake, fake, 1 << 30, None) == -2
    assert lib.factor_chol(fake, 32, ctypes.c_float(0.01), P(8192), fake, fake, P(1 << 20), 16, None) == -5
    # with FLAG_CHOL_FACTOR the quantizer needs one more working copy of W
    need = lib.gptq_nvfp4_workspace_size(16, 32, nvq.FLAG_CHOL_FACTOR)
    assert need > lib.gptq_nvfp4_workspace_size(16, 32, 0)
    rc = lib.gptq_nvfp4_quantize(fake, 1, 16, 32, 32, fake, fake, fake, 16, nvq.FLAG_CHOL_FACTOR, fake, fake, fake,
                                 None, P(1 << 20), need - 256, None)
    assert rc == -5
    # dequantize: bad k, bad dtype, empty is fine
    assert lib.nvfp4_dequantize(fake, fake, fake, 4, 8, fake, 0, None) == -2
    assert lib.nvfp4_dequantize(fake, fake, fake, 4, 32, fake, 5, None) == -3
    assert lib.nvfp4_dequantize(None, None, None, 0, 32, None, 0, None) == 0
    # grouped Hessian: offsets must start at 0 and not decrease; G > 0
    off = (ctypes.c_int64 * 4)(0, 5, 3, 9)
    assert lib.hessian_accumulate_grouped(fake, 1, 10, 32, 32, fake, off, 3, fake, fake, 1 << 30, None) == -6
    off = (ctypes.c_int64 * 3)(1, 5, 9)
    assert lib.hessian_accumulate_grouped(fake, 1, 10, 32, 32, fake, off, 2, fake, fake, 1 << 30, None) == -6
    assert lib.hessian_accumulate_grouped(fake, 1, 10, 32, 32, fake, off, 0, fake, fake, 1 << 30, None) == -2
    off = (ctypes.c_int64 * 3)(0, 0, 0)   # no assignments: a no-op
    assert lib.hessian_accumulate_grouped(None, 1, 0, 32, 32, None, off, 2, fake, None, 0, None) == 0
    # batched factor / quantize: empty batch is a no-op, strides must cover an element
    assert lib.factor_hinv_batched(None, 32, 0, 1024, ctypes.c_float(0.01), None, 1024, None, None, None, 0,
                                   None) == 0
    assert lib.factor_hinv_batched(fake, 32, 2, 100, ctypes.c_float(0.01), P(1 << 24), 1024, fake, fake, fake,
                                   1 << 30, None) == -2
    assert lib.factor_chol_batched(None, 32, 0, 1024, ctypes.c_float(0.01), None, 1024, None, None, None, 0,
                                   None) == 0
    assert lib.factor_chol_batched(fake, 32, 2, 100, ctypes.c_float(0.01), P(1 << 24), 1024, fake, fake, fake,
                                   1 << 30, None) == -2
    assert lib.factor_chol_batched(fake, 24, 2, 1024, ctypes.c_float(0.01), P(1 << 24), 1024, fake, fake, fake,
                                   1 << 30, None) == -2
    assert lib.factor_chol_batched(fake, 32, 2, 1024, ctypes.c_float(-1.0), P(1 << 24), 1024, fake, fake, fake,
                                   1 << 30, None) == -6
    assert lib.factor_chol_batched(fake, 32, 2, 1024, ctypes.c_float(0.01), P(1 << 24), 1024, fake, fake, fake,
                                   16, None) == -5
    rc = lib.gptq_nvfp4_quantize_batched(fake, 1, 2, 16, 32, 32, 100, fake, 1024, fake, 1024, fake, 16, 0,
                                         fake, fake, fake, None, fake, 1 << 30, None)
    assert rc == -2
    # Hessian over host memory: chunk, shape, H, workspace and staging checks; n = 0 is a no-op
    assert lib.hessian_accumulate_host(fake, 1, 10, 32, 32, fake, 0, fake, 1 << 30, None, 0, None, None) == -2
    assert lib.hessian_accumulate_host(fake, 1, 10, 24, 24, fake, 8, fake, 1 << 30, None, 0, None, None) == -2
    assert lib.hessian_accumulate_host(fake, 1, 10, 32, 32, None, 8, fake, 1 << 30, None, 0, None, None) == -1
    assert lib.hessian_accumulate_host(None, 1, 0, 32, 32, fake, 8, None, 0, None, 0, None, None) == 0
    assert lib.hessian_accumulate_host(fake, 1, 10, 32, 32, fake, 8, P(1 << 20), 16, None, 0, None, None) == -5
    assert lib.hessian_accumulate_host(fake, 1, 10, 32, 32, fake, 8, P(1 << 20), 1 << 30, fake, 16, None,
                                       None) == -5
    # finite check: status required, dtype, shape (rows, cols, ld); unknown quantize flag
    assert lib.nvq_check_finite(fake, 1, 4, 32, 32, None, None) == -1
    assert lib.nvq_check_finite(fake, 2, 4, 32, 32, fake, None) == -3
    assert lib.nvq_check_finite(fake, 1, 4, 0, 32, fake, None) == -2
    assert lib.nvq_check_finite(fake, 1, 4, 32, 16, fake, None) == -2
    assert lib.nvq_check_finite(fake, 1, -1, 32, 32, fake, None) == -2
    assert lib.nvq_check_finite(None, 1, 4, 32, 32, fake, None) == -1
    rc = lib.gptq_nvfp4_quantize(fake, 1, 16, 32, 32, fake, fake, fake, 16, 64, fake, fake, fake, None,
                                 fake, 1 << 30, None)
    assert rc == -6 and b"flags" in lib.nvq_last_error()
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, 99):
        assert lib.nvq_status_string(s)


def test_workspace_queries_are_consistent():
    import post_nvfp4_weight_amd as nvq
    lib = nvq.lib
    assert lib.gptq_nvfp4_workspace_size(4096, 4096, 0) >= 4096 * 4096 * 4
    assert lib.factor_hinv_workspace_size(4096) >= 2 * 4096 * 4096 * 4
    assert lib.gptq_nvfp4_workspace_size(0, 16, 0) == 0
    assert lib.nvfp4_global_scale_workspace_size(16, 16) > 0
    off = (ctypes.c_int64 * 4)(0, 100, 100, 350)
    need = lib.hessian_grouped_workspace_size(off, 3, 256, 1)
    assert need >= 250 * 256 * 2 + lib.hessian_workspace_size(250, 256, 1)
    # host streaming: two chunk buffers plus the Hessian workspace of one chunk; two pinned chunks
    ws = lib.hessian_host_workspace_size(1000, 256, 1)
    assert ws >= 2 * 1000 * 256 * 2 + lib.hessian_workspace_size(1000, 256, 1)
    assert lib.hessian_host_staging_size(1000, 256, 1) >= 2 * 1000 * 256 * 2
    assert lib.hessian_host_staging_size(1000, 256, 0) >= 2 * 1000 * 256 * 4


def test_hessian_workspace_never_shrinks_as_tokens_grow():
    """One workspace serves every smaller token count (groups of a grouped call,
    the last chunk of a streamed one), so the bf16 Hessian's workspace size
    must not decrease with n: checked over channel counts whose tile plans
    switch strip-pair tail pieces on at different token counts."""
    import post_nvfp4_weight_amd as nvq
    lib = nvq.lib
    for k in (128, 400, 1024, 2320, 2560, 3072, 4096, 4608, 6144):
        prev = 0
        for n in list(range(1, 2400, 13)) + [4096, 8191, 65536, 262144]:
            ws = lib.hessian_workspace_size(n, k, 1)
            assert ws >= prev, (k, n, ws, prev)
            prev = ws

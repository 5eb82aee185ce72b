"""The no-allocation weight-only GEMM (nvfp4_gemm_noalloc) through the C ABI.

Two calls in a row -- the first with partial sums filling the whole 32 MiB
device array, the second smaller -- must give what nvfp4_gemm (with a caller
workspace) gives, bit for bit, and both lie within the fp32 accumulation bound
of the fp64 consumer oracle.  A decode-sized call (no partial sums) too.  A
shape whose partial sums exceed the array is rejected before anything is
enqueued (its output is left untouched).
"""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import codec, consumer, gptq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NVQ_ERR_WORKSPACE = -5


@pytest.fixture(scope="module")
def nvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_nvfp4_weight_amd as m
    return m


def _layer(m, k, T, seed):
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.01)
    g = codec.global_scale(W)
    r = gptq.rtn(W, g, 1)
    packed, scales = codec.pack_codes(r["codes"]), r["scales"]
    X = synth.to_bf16_values(np.random.default_rng(seed).standard_normal((T, k)).astype(np.float32))
    return X, packed, scales, g


def _noalloc(nvq, Xd, codes, scales, g, Y):
    T, k = Xd.shape
    P = ctypes.c_void_p
    return nvq.lib.nvfp4_gemm_noalloc(P(Xd.data_ptr()), nvq.NVQ_DTYPE_BF16, T, k, Xd.stride(0),
                                      P(codes.data_ptr()), P(scales.data_ptr()), P(g.data_ptr()), codes.shape[0],
                                      P(Y.data_ptr()), nvq._dtype_code(Y), Y.stride(0), nvq._stream())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_call_twice(nvq, dtype):
    # (256, 4096, 4096): 8 k splits of 256 x 4096 fp32 partial sums = exactly 32 MiB;
    # (100, 2048, 1024): 16 splits, 6.5 MB, left over from the first call's contents;
    # (8, 1024, 4096): the decode-sized kernel, no partial sums.
    for T, k, m in ((256, 4096, 4096), (100, 2048, 1024), (8, 1024, 4096)):
        X, packed, scales, g = _layer(m, k, T, seed=T)
        Xd = synth.to_bf16_tensor(X).to(DEV)
        codes = torch.from_numpy(packed).to(DEV)
        sc = torch.from_numpy(scales).to(DEV)
        gd = torch.tensor([g], dtype=torch.float32, device=DEV)
        ref = nvq.nvfp4_gemm(Xd, codes, sc, gd, out_dtype=dtype)
        Y = torch.full((T, m), float("nan"), dtype=dtype, device=DEV)
        assert _noalloc(nvq, Xd, codes, sc, gd, Y) == 0, nvq.lib.nvq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16) if dtype == torch.bfloat16 else Y.view(torch.int32),
                           ref.view(torch.int16) if dtype == torch.bfloat16 else ref.view(torch.int32)), (T, k, m)
        if dtype == torch.float32:
            Yo = consumer.weight_only_matmul(X, packed, scales, g)
            deq = np.abs(codec.dequantize(packed, scales, g).astype(np.float64))
            bnd = (np.abs(X.astype(np.float64)) @ deq.T) * ((k / 16 + 16) * 2.0 ** -23)
            assert np.all(np.abs(Y.cpu().numpy().astype(np.float64) - Yo) <= bnd + 1e-30), (T, k, m)


def test_noalloc_rejects_partial_sums_beyond_the_array(nvq):
    # 520 tokens x 4096 outputs over k = 4096 take 4 splits: 34,078,720 bytes > 32 MiB
    T, k, m = 520, 4096, 4096
    assert nvq.lib.nvfp4_gemm_workspace_size(T, k, m) > (32 << 20)
    Xd = torch.zeros(T, k, dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros(m, k // 2, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(m, k // 16, dtype=torch.uint8, device=DEV)
    gd = torch.ones(1, dtype=torch.float32, device=DEV)
    Y = torch.full((T, m), 7.0, dtype=torch.float32, device=DEV)
    assert _noalloc(nvq, Xd, codes, sc, gd, Y) == NVQ_ERR_WORKSPACE
    assert b"33554432" in nvq.lib.nvq_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))

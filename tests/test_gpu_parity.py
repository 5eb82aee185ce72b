"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars:
  * codec work (dequantization, global scale, round-to-nearest with one
    candidate) is bit-exact against the oracle;
  * round-to-nearest with several candidates is bit-exact against the oracle's
    fp32 mode (scores summed in fp32 in column order on both sides);
  * H = X^T X is exactly symmetric and within the fp32 summation bound
    (n/16 + 64) * 2^-23 * (|X|^T |X|) of the fp64 oracle;
  * U agrees with the fp64 oracle to 1e-4 of max|U| (fp32 factorization of
    well-conditioned damped matrices);
  * through the GPTQ sweep at most 0.1% of element codes and of block scales
    differ from the oracle, and the weighted error tr(dW H dW^T) agrees within
    1e-3 relative.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import codec, gptq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_nvfp4_weight_amd as m
    return m


def _to_dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def _mismatch(a, b):
    return float(np.mean(np.asarray(a) != np.asarray(b)))


# ------------------------------------------------------------------ codec
def test_dequantize_bit_exact(nvq):
    r = np.random.default_rng(100)
    m, k = 37, 272
    codes = r.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    scales = r.integers(0, 127, size=(m, k // 16), dtype=np.uint8)
    g = np.float32(0.000731)
    ref = codec.dequantize(codes, scales, g)
    out = nvq.nvfp4_dequantize(_to_dev(codes, torch.uint8), _to_dev(scales, torch.uint8),
                               _to_dev(np.array([g])), torch.float32).cpu().numpy()
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    outb = nvq.nvfp4_dequantize(_to_dev(codes, torch.uint8), _to_dev(scales, torch.uint8),
                                _to_dev(np.array([g])), torch.bfloat16).cpu()
    refb = torch.from_numpy(ref).to(torch.bfloat16)
    assert torch.equal(outb.view(torch.int16), refb.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_global_scale_bit_exact(nvq, dtype):
    W = synth.weights("attn_proj", 300, 512, 0.02, outlier_frac=0.001, bf16=(dtype == torch.bfloat16))
    g = nvq.nvfp4_global_scale(_to_dev(W, dtype)).item()
    assert np.float32(g) == codec.global_scale(W)
    z = nvq.nvfp4_global_scale(torch.zeros(4, 32, device=DEV, dtype=dtype)).item()
    assert z == 1.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("m,k,pad", [(3000, 4096, 0), (7, 13, 3), (33, 40, 1), (2, 24, 8)])
def test_global_scale_shapes_and_strides(nvq, dtype, m, k, pad):
    # More rows than workgroups, k not a multiple of 8, and rows padded by
    # pad values (odd strides take the element-wise path).  The maximum is
    # planted in the last row's last column.
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.001, bf16=(dtype == torch.bfloat16))
    W[m - 1, k - 1] = -4.0 * np.abs(W).max()
    full = np.zeros((m, k + pad), dtype=np.float32)
    full[:, :k] = W
    Wd = _to_dev(full, dtype)[:, :k]
    g = nvq.nvfp4_global_scale(Wd).item()
    assert np.float32(g) == codec.global_scale(W)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rtn_one_candidate_bit_exact(nvq, dtype):
    W = synth.weights("attn_proj", 96, 512, 0.02, outlier_frac=0.01, bf16=(dtype == torch.bfloat16))
    W[5, 32:48] = 0.0
    g = codec.global_scale(W)
    ref = gptq.rtn(W, g, 1)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, dtype), None, None, _to_dev(np.array([g])), 1,
                                  nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    assert np.array_equal(out["codes"].cpu().numpy(), codec.pack_codes(ref["codes"]))
    assert np.array_equal(out["scales"].cpu().numpy(), ref["scales"])


@pytest.mark.parametrize("K", [1, 4])
@pytest.mark.parametrize("gexp", [-9, -6, 0])
def test_rtn_exact_ties_bit_exact(nvq, K, gexp):
    # Weights on a 1/8 grid and a power-of-two global scale: many weights sit
    # exactly on an E2M1 midpoint t * s * g (and block maxima on E4M3
    # midpoints), where the rounding rule decides (ties to the even index).
    rng = np.random.default_rng(11 + gexp)
    W = (rng.integers(-64, 65, size=(64, 512)) * 0.125).astype(np.float32)
    W[3, :16] = 0.0
    g = np.float32(2.0 ** gexp)
    ref = gptq.sweep(W, np.eye(512, dtype=np.float32), g, K, dtype=np.float32)
    s = np.repeat(codec.e4m3_decode(ref["scales"]).astype(np.float64), 16, axis=1) * float(g)
    ratio = np.divide(np.abs(W), s, out=np.zeros(W.shape), where=s > 0)
    assert np.any(np.isin(ratio, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))
    out = nvq.gptq_nvfp4_quantize(_to_dev(W), None, None, _to_dev(np.array([g])), K,
                                  nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    assert np.array_equal(out["scales"].cpu().numpy(), ref["scales"])
    assert np.array_equal(out["codes"].cpu().numpy(), codec.pack_codes(ref["codes"]))


@pytest.mark.parametrize("K", [4, 8, 16])
def test_rtn_candidates_bit_exact_fp32_scores(nvq, K):
    W = synth.weights("attn_proj", 64, 256, 0.02, outlier_frac=0.01, bf16=False)
    g = codec.global_scale(W)
    ref = gptq.sweep(W, np.eye(256), g, K, dtype=np.float32)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W), None, None, _to_dev(np.array([g])), K,
                                  nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    assert np.array_equal(out["scales"].cpu().numpy(), ref["scales"])
    assert np.array_equal(out["codes"].cpu().numpy(), codec.pack_codes(ref["codes"]))


# ------------------------------------------------------------------ Hessian
def _hessian_check(H_gpu, X, n):
    Xd = X.astype(np.float64)
    ref = Xd.T @ Xd
    bound = np.abs(Xd).T @ np.abs(Xd) * ((n / 16 + 64) * 2.0 ** -23)
    assert np.array_equal(H_gpu, H_gpu.T)
    assert np.all(np.abs(H_gpu - ref) <= bound + 1e-30)


# (1500, 2320), (777, 4096), (4127, 3072) and (2000, 2048) split the strip
# pairs' token ranges into tail pieces (with ragged and empty pieces).  Layers
# of 16 256-channel segments (k in (3840, 4096]) take the four-group and
# diagonal tiles: (777, 4096), (20, 4096) and (100, 3968) add into H directly
# (the last with channels past k in the last group), (3000, 4096) splits the
# tokens in 3 and 2 ranges with one tail piece per diagonal tile, (7000, 4096)
# with two ragged tail pieces.
@pytest.mark.parametrize("n,k", [(3000, 400), (700, 256), (64, 128), (5000, 1024), (1500, 2320), (777, 4096),
                                 (4127, 3072), (2000, 2048), (3000, 4096), (20, 4096), (100, 3968), (7000, 4096)])
def test_hessian_bf16(nvq, n, k):
    X = synth.activations("attn_proj", n, k, massive=4)
    Xt = synth.to_bf16_tensor(X).to(DEV)
    H = nvq.hessian_accumulate(Xt).cpu().numpy()
    _hessian_check(H, X, n)


def test_hessian_accumulates_over_chunks(nvq):
    n, k = 2500, 384
    X = synth.activations("attn_proj", n, k)
    Xt = synth.to_bf16_tensor(X).to(DEV)
    H = nvq.hessian_accumulate(Xt[:1200])
    H = nvq.hessian_accumulate(Xt[1200:], H).cpu().numpy()
    _hessian_check(H, X, n)


def test_hessian_accumulates_over_chunks_four_group_tiles(nvq):
    # The first chunk (one stage) adds into H directly, the second through
    # token splits and the reduction.
    n, k = 1600, 4096
    X = synth.activations("attn_proj", n, k)
    Xt = synth.to_bf16_tensor(X).to(DEV)
    H = nvq.hessian_accumulate(Xt[:30])
    H = nvq.hessian_accumulate(Xt[30:], H).cpu().numpy()
    _hessian_check(H, X, n)


def test_hessian_fp32_small_layer(nvq):
    W, X = synth.small_layer()
    H = nvq.hessian_accumulate(_to_dev(X)).cpu().numpy()
    Xd = X.astype(np.float64)
    ref = Xd.T @ Xd
    bound = np.abs(Xd).T @ np.abs(Xd) * (X.shape[0] * 2.0 ** -23)
    assert np.array_equal(H, H.T)
    assert np.all(np.abs(H - ref) <= bound)


# ------------------------------------------------------------------ factor
# k = 2048 reaches the inverse level whose products split their k ranges;
# k = 4608 (nine super-panels of 512) runs the trailing updates split over two
# streams.
@pytest.mark.parametrize("k,n", [(256, 2048), (448, 4000), (1024, 8192), (2048, 6144), (4608, 9216)])
def test_factor_matches_oracle(nvq, k, n):
    X = synth.activations("attn_proj", n, k, massive=4)
    H = gptq.hessian(X)
    Uref, lam = gptq.hinv_factor(H)
    U, lam_g, info = nvq.factor_hinv(_to_dev(H.astype(np.float32)))
    assert int(info.item()) == 0
    assert lam_g.item() == pytest.approx(lam, rel=1e-5)
    U = U.cpu().numpy().astype(np.float64)
    assert np.all(np.tril(U, -1) == 0)
    assert np.max(np.abs(U - Uref)) <= 1e-4 * np.max(np.abs(Uref))


def test_factor_reports_non_pd(nvq):
    H = -np.eye(64, dtype=np.float32)
    _, _, info = nvq.factor_hinv(_to_dev(H), damp_rel=0.0)
    assert int(info.item()) > 0


# ------------------------------------------------------------------ sweep
def _sweep_case(nvq, W, X, K, w_dtype):
    H = gptq.hessian(X)
    Uref, lam = gptq.hinv_factor(H)
    g = codec.global_scale(W)
    U32 = Uref.astype(np.float32)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, w_dtype), _to_dev(U32), _to_dev(H.astype(np.float32)),
                                  _to_dev(np.array([g])), K)
    codes = codec.unpack_codes(out["codes"].cpu().numpy())
    scales = out["scales"].cpu().numpy()
    ref32 = gptq.sweep(W, U32, g, K, dtype=np.float32)
    ref64 = gptq.sweep(W, Uref, g, K)
    return H, g, codes, scales, out, ref32, ref64


@pytest.mark.parametrize("m,k,n,K", [(256, 256, 2048, 8), (200, 384, 3000, 16), (64, 1040, 4096, 16)])
def test_sweep_matches_oracle(nvq, m, k, n, K):
    if (m, k) == (256, 256):
        W, X = synth.small_layer(m, k, n)
        dt = torch.float32
    else:
        W, X = synth.attn_proj_layer(m, k, n)
        dt = torch.bfloat16
    H, g, codes, scales, out, ref32, ref64 = _sweep_case(nvq, W, X, K, dt)
    assert _mismatch(codes, ref32["codes"]) <= 1e-3
    assert _mismatch(scales, ref32["scales"]) <= 1e-3
    assert _mismatch(codes, ref64["codes"]) <= 1e-3
    assert _mismatch(scales, ref64["scales"]) <= 1e-3
    # weighted error of the GPU's own codes, and against the oracle's choice
    deq_gpu = codec.dequantize(codec.pack_codes(codes), scales, g)
    E_own = gptq.weighted_error(W, deq_gpu, H)
    E_gpu = out["row_err"].cpu().numpy().astype(np.float64)
    assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max())
    deq_ref = codec.dequantize(codec.pack_codes(ref64["codes"]), ref64["scales"], g)
    E_ref = gptq.weighted_error(W, deq_ref, H)
    assert abs(E_gpu.sum() - E_ref.sum()) <= 1e-3 * E_ref.sum()
    loss = out["row_loss"].cpu().numpy()
    assert np.allclose(loss, ref64["score"], rtol=1e-3)


@pytest.mark.parametrize("m,k,n", [(200, 384, 3000), (64, 1040, 4096)])
def test_sweep_fp64_working_precision_matches_fp64_oracle(nvq, m, k, n):
    W, X = synth.attn_proj_layer(m, k, n)
    H = gptq.hessian(X)
    Uref, _ = gptq.hinv_factor(H)
    g = codec.global_scale(W)
    U32 = Uref.astype(np.float32)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), _to_dev(U32), _to_dev(H.astype(np.float32)),
                                  _to_dev(np.array([g])), 16, nvq.FLAG_FP64)
    codes = codec.unpack_codes(out["codes"].cpu().numpy())
    scales = out["scales"].cpu().numpy()
    ref = gptq.sweep(W, U32, g, 16)   # fp64 arithmetic on the same fp32 U
    assert _mismatch(codes, ref["codes"]) <= 1e-4
    assert _mismatch(scales, ref["scales"]) <= 1e-4
    assert np.allclose(out["row_loss"].cpu().numpy(), ref["score"], rtol=1e-5)
    deq = codec.dequantize(codec.pack_codes(codes), scales, g)
    E_own = gptq.weighted_error(W, deq, H)
    assert np.allclose(out["row_err"].cpu().numpy().astype(np.float64), E_own, rtol=1e-4, atol=1e-6 * E_own.max())


def test_identity_hessian_one_candidate_is_rtn(nvq):
    W = synth.weights("attn_proj", 48, 384, 0.02, outlier_frac=0.01)
    g = codec.global_scale(W)
    ref = gptq.rtn(W, g, 1)
    I = np.eye(384, dtype=np.float32)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), _to_dev(I), _to_dev(I), _to_dev(np.array([g])), 1)
    assert np.array_equal(out["codes"].cpu().numpy(), codec.pack_codes(ref["codes"]))
    assert np.array_equal(out["scales"].cpu().numpy(), ref["scales"])


def test_end_to_end_layer(nvq):
    m, k, n, K = 256, 512, 6000, 16
    W, X = synth.attn_proj_layer(m, k, n)
    res = nvq.quantize_layer(_to_dev(W, torch.bfloat16), synth.to_bf16_tensor(X).to(DEV), n_cand=K)
    ref = gptq.quantize_layer(W, X, n_cand=K)
    codes = codec.unpack_codes(res["codes"].cpu().numpy())
    assert _mismatch(codes, ref["codes"]) <= 1e-3
    assert _mismatch(res["scales"].cpu().numpy(), ref["scales"]) <= 1e-3
    E = res["row_err"].cpu().numpy().astype(np.float64).sum()
    assert abs(E - ref["row_err"].sum()) <= 1e-3 * ref["row_err"].sum()

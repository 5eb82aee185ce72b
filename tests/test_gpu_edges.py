"""GPU edge cases against the CPU oracle: empty and ragged inputs, degenerate
weights, extreme dynamic range, one block, one candidate."""

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


def test_hessian_zero_tokens_leaves_h_unchanged(nvq):
    H0 = np.random.default_rng(1).standard_normal((64, 64)).astype(np.float32)
    H = _to_dev(H0)
    X = torch.zeros(8, 64, dtype=torch.bfloat16, device=DEV)
    rc = nvq.lib.hessian_accumulate(nvq._ptr(X), nvq.NVQ_DTYPE_BF16, 0, 64, 64, nvq._ptr(H), None, 0, nvq._stream())
    assert rc == 0
    assert np.array_equal(H.cpu().numpy(), H0)


def test_hessian_one_token_is_outer_product(nvq):
    x = synth.to_bf16_values(np.random.default_rng(2).standard_normal((1, 48)).astype(np.float32))
    H = nvq.hessian_accumulate(_to_dev(x, torch.bfloat16)).cpu().numpy()
    # bf16 x bf16 products are exact in fp32, and one token means one product per entry
    assert np.array_equal(H, (x.astype(np.float64).T @ x.astype(np.float64)).astype(np.float32))


def test_all_zero_weights(nvq):
    m, k = 20, 96
    W = np.zeros((m, k), dtype=np.float32)
    X = synth.activations("small", 500, k, bf16=False)
    res = nvq.quantize_layer(_to_dev(W), _to_dev(X), n_cand=8)
    assert float(res["g"].item()) == 1.0
    assert not res["codes"].cpu().numpy().any()
    assert not res["scales"].cpu().numpy().any()
    assert not res["row_err"].cpu().numpy().any()


def test_zero_blocks_mixed_with_nonzero(nvq):
    m, k = 33, 256
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.01)
    W[:, 0:16] = 0.0             # a zero first block in every row (nothing updates it)
    W[:, 32:64] = 0.0            # zero inputs that earlier errors make nonzero (absmax of updated weights)
    W[5, :] = 0.0                # a zero row stays zero: no errors to propagate
    W[7, 100:116] = 0.0          # the same inside a lazy batch
    X = synth.activations("attn_proj", 2000, k, massive=2)
    H = gptq.hessian(X)
    U, _ = gptq.hinv_factor(H)
    g = codec.global_scale(W)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), _to_dev(U.astype(np.float32)),
                                  _to_dev(H.astype(np.float32)), _to_dev(np.array([g])), 16)
    scales = out["scales"].cpu().numpy()
    codes = codec.unpack_codes(out["codes"].cpu().numpy())
    assert not scales[:, 0].any() and not codes[:, 0:16].any()
    assert scales[:, 2:4].any()
    assert not scales[5].any() and not codes[5].any()
    ref = gptq.sweep(W, U.astype(np.float32), g, 16, dtype=np.float32)
    assert _mismatch(codes, ref["codes"]) <= 1e-3
    assert _mismatch(scales, ref["scales"]) <= 1e-3
    assert float(out["row_err"][5].item()) == 0.0


def test_extreme_dynamic_range_rtn_bit_exact(nvq):
    # Blocks spanning 2^-40 .. 2^3 relative magnitudes: windows shifted at
    # both ends of the E4M3 range, subnormal scales and saturated ones.
    rng = np.random.default_rng(3)
    m, k = 64, 512
    mag = 2.0 ** rng.uniform(-40, 3, size=(m, k // 16, 1)) * rng.standard_normal((m, k // 16, 16))
    W = mag.reshape(m, k).astype(np.float32)
    g = codec.global_scale(W)
    for K in (1, 4, 16):
        out = nvq.gptq_nvfp4_quantize(_to_dev(W), None, None, _to_dev(np.array([g])), K,
                                      nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
        ref = gptq.sweep(W, np.eye(k, dtype=np.float32), g, K, dtype=np.float32)
        assert np.array_equal(out["scales"].cpu().numpy(), ref["scales"]), K
        assert np.array_equal(out["codes"].cpu().numpy(), codec.pack_codes(ref["codes"])), K
    deq = nvq.nvfp4_dequantize(out["codes"], out["scales"], _to_dev(np.array([g])))
    assert np.array_equal(deq.cpu().numpy().view(np.uint32),
                          codec.dequantize(codec.pack_codes(ref["codes"]), ref["scales"], g).view(np.uint32))


@pytest.mark.parametrize("m,k,K", [(1, 16, 16), (37, 592, 16), (9, 144, 1), (5, 528, 3)])
def test_ragged_shapes_sweep(nvq, m, k, K):
    # k not a multiple of the 128-column batch or the 512-column block; one
    # block; one row; odd candidate counts.
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.01)
    X = synth.activations("attn_proj", 3 * k + 7, k, massive=min(8, k // 16))
    H = gptq.hessian(X)
    U, _ = gptq.hinv_factor(H)
    g = codec.global_scale(W)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), _to_dev(U.astype(np.float32)),
                                  _to_dev(H.astype(np.float32)), _to_dev(np.array([g])), K)
    codes = codec.unpack_codes(out["codes"].cpu().numpy())
    scales = out["scales"].cpu().numpy()
    ref = gptq.sweep(W, U.astype(np.float32), g, K, dtype=np.float32)
    assert _mismatch(codes, ref["codes"]) <= 1e-3
    assert _mismatch(scales, ref["scales"]) <= 1e-3
    deq = codec.dequantize(codec.pack_codes(codes), scales, g)
    E_own = gptq.weighted_error(W, deq, H)
    E_gpu = out["row_err"].cpu().numpy().astype(np.float64)
    assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * max(E_own.max(), 1e-30))


@pytest.mark.parametrize("k", [208, 592, 1104])
def test_factor_ragged_last_panel(nvq, k):
    # The last 64-column panel holds 16 columns; 592 and 1104 also end in a
    # partial 512-column super-panel after one or two full ones (each full
    # one's columns to the right are updated once, by all its panels).
    X = synth.activations("small", max(1500, 2 * k), k, bf16=False)
    H = gptq.hessian(X)
    U, lam, info = nvq.factor_hinv(_to_dev(H.astype(np.float32)))
    assert int(info.item()) == 0
    Uref, _ = gptq.hinv_factor(H.astype(np.float32).astype(np.float64))
    assert np.max(np.abs(U.cpu().numpy() - Uref)) <= 1e-4 * np.max(np.abs(Uref))


def test_factor_singular_without_damping_reports_order(nvq):
    # Rank-deficient H with no damping: the failing trailing minor is reported.
    k = 128
    X = synth.activations("small", 40, k, bf16=False)   # rank <= 40 < k
    H = gptq.hessian(X).astype(np.float32)
    _, _, info = nvq.factor_hinv(_to_dev(H), damp_rel=0.0)
    assert 0 < int(info.item()) <= k


@pytest.mark.parametrize("scale", [1e-36, 1e12])
def test_extreme_magnitudes_rtn_bit_exact(nvq, scale):
    # Weights near 1e-36 give a subnormal global scale g (the candidate window
    # is then found by the exact search rather than from 1 / (6 g), which
    # overflows); weights near 1e12 give a large one.  Scales and codes must
    # still match the oracle bit for bit.
    W = synth.weights("attn_proj", 48, 256, 0.02, outlier_frac=0.01, bf16=False)
    W = (W.astype(np.float64) * scale).astype(np.float32)
    g = codec.global_scale(W)
    ref = gptq.sweep(W, np.eye(256), g, 8, dtype=np.float32)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W), None, None, _to_dev(np.array([g], dtype=np.float32)), 8,
                                  nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    assert np.array_equal(out["scales"].cpu().numpy(), ref["scales"])
    assert np.array_equal(out["codes"].cpu().numpy(), codec.pack_codes(ref["codes"]))


def test_tiny_magnitudes_sweep(nvq):
    # The GPTQ sweep with a subnormal global scale (weights near 1e-36).
    m, k = 32, 256
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.01, bf16=False)
    W = (W.astype(np.float64) * 1e-36).astype(np.float32)
    X = synth.activations("attn_proj", 2048, k, massive=4)
    H = gptq.hessian(X)
    U, _ = gptq.hinv_factor(H)
    g = codec.global_scale(W)
    assert g < 2.0 ** -120
    out = nvq.gptq_nvfp4_quantize(_to_dev(W), _to_dev(U.astype(np.float32)), _to_dev(H.astype(np.float32)),
                                  _to_dev(np.array([g], dtype=np.float32)), 16, nvq.FLAG_NO_ERR)
    ref = gptq.sweep(W, U.astype(np.float32), g, 16, dtype=np.float32)
    assert _mismatch(codec.unpack_codes(out["codes"].cpu().numpy()), ref["codes"]) <= 1e-3
    assert _mismatch(out["scales"].cpu().numpy(), ref["scales"]) <= 1e-3

"""GPU parity of the Cholesky-factor form (factor_chol and NVQ_FLAG_CHOL_FACTOR) against the CPU oracle.

The oracle defines the sweep with U, the upper Cholesky factor of (H + lam I)^-1.  factor_chol returns V
built from R = U^-1 (H + lam I = R R^T, R upper): V_ij = -R_ij / R_jj above the diagonal, V_ii = R_ii,
0 below.  Its reference here is the oracle's own fp64 U inverted in fp64, and the GPU's R is also held
to the fp32 Cholesky backward-error bound |R R^T - (H + lam I)| <= gamma_{k+1} |R| |R|^T elementwise.
With exact arithmetic the sweep in this form takes the inverse form's updates and scores term by term,
so the bars are those of the inverse form against the fp64 oracle: at most 0.1% of element codes and of
block scales differ, the weighted error tr(dW H dW^T) agrees within 1e-3 relative and row_loss within
1e-3.
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


def _v_from_u(U):
    """V of the oracle's U: R = U^-1 (fp64), V = -R_ij / R_jj above the diagonal, R_ii on it."""
    R = np.triu(np.linalg.inv(U))
    d = np.diag(R)
    V = -R / d[None, :]
    V = np.triu(V, 1) + np.diag(d)
    return V, R


# k = 1040: a last panel of 16 columns; k = 4608: nine super-panels, the trailing updates on two streams.
@pytest.mark.parametrize("k,n", [(256, 2048), (1040, 8192), (2048, 6144), (4608, 9216)])
def test_factor_chol_matches_oracle(nvq, k, n):
    X = synth.activations("attn_proj", n, k, massive=4)
    H = gptq.hessian(X)
    Uref, lam = gptq.hinv_factor(H)
    Vref, Rref = _v_from_u(Uref)
    V, lam_g, info = nvq.factor_chol(_to_dev(H.astype(np.float32)))
    assert int(info.item()) == 0
    assert lam_g.item() == pytest.approx(lam, rel=1e-5)
    V = V.cpu().numpy().astype(np.float64)
    assert np.all(np.tril(V, -1) == 0)
    d, dref = np.diag(V), np.diag(Vref)
    assert np.all(d > 0)
    assert np.max(np.abs(d - dref)) <= 1e-4 * np.max(dref)
    off, offref = np.triu(V, 1), np.triu(Vref, 1)
    assert np.max(np.abs(off - offref)) <= 1e-4 * np.max(np.abs(offref))
    # backward error of the GPU's R against the damped H it factors (lambda in fp32, as the GPU adds it)
    R = off * (-d[None, :]) + np.diag(d)
    Hd = H.astype(np.float32).astype(np.float64) + np.float64(lam_g.item()) * np.eye(k)
    gamma = (k + 1) * 2.0 ** -24 / (1 - (k + 1) * 2.0 ** -24)
    bound = 2.0 * gamma * (np.abs(R) @ np.abs(R).T) + 4 * 2.0 ** -24 * np.abs(Hd)
    assert np.all(np.abs(R @ R.T - Hd) <= bound)


def test_factor_chol_reports_non_pd(nvq):
    H = -np.eye(64, dtype=np.float32)
    _, _, info = nvq.factor_chol(_to_dev(H), damp_rel=0.0)
    assert int(info.item()) > 0


def _chol_case(nvq, W, X, K, w_dtype, flags=0):
    H = gptq.hessian(X)
    Uref, lam = gptq.hinv_factor(H)
    Vref, _ = _v_from_u(Uref)
    g = codec.global_scale(W)
    out = nvq.gptq_nvfp4_quantize(_to_dev(W, w_dtype), _to_dev(Vref.astype(np.float32)),
                                  _to_dev(H.astype(np.float32)), _to_dev(np.array([g])), K,
                                  flags | nvq.FLAG_CHOL_FACTOR)
    codes = codec.unpack_codes(out["codes"].cpu().numpy())
    scales = out["scales"].cpu().numpy()
    ref64 = gptq.sweep(W, Uref, g, K)
    return H, g, codes, scales, out, ref64


@pytest.mark.parametrize("m,k,n,K,fp64", [(256, 256, 2048, 8, False), (200, 384, 3000, 16, False),
                                          (64, 1040, 4096, 16, False), (96, 640, 4000, 4, False),
                                          (120, 512, 3000, 1, False), (200, 384, 3000, 16, True),
                                          (64, 1040, 4096, 2, True)])
def test_chol_sweep_matches_oracle(nvq, m, k, n, K, fp64):
    if (m, k) == (256, 256):
        W, X = synth.small_layer(m, k, n)
        dt = torch.float32
    else:
        W, X = synth.attn_proj_layer(m, k, n)
        dt = torch.bfloat16
    H, g, codes, scales, out, ref64 = _chol_case(nvq, W, X, K, dt, nvq.FLAG_FP64 if fp64 else 0)
    assert _mismatch(codes, ref64["codes"]) <= 1e-3
    assert _mismatch(scales, ref64["scales"]) <= 1e-3
    deq_gpu = codec.dequantize(codec.pack_codes(codes), scales, g)
    E_own = gptq.weighted_error(W, deq_gpu, H)
    E_gpu = out["row_err"].cpu().numpy().astype(np.float64)
    assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max())
    deq_ref = codec.dequantize(codec.pack_codes(ref64["codes"]), ref64["scales"], g)
    E_ref = gptq.weighted_error(W, deq_ref, H)
    assert abs(E_gpu.sum() - E_ref.sum()) <= 1e-3 * E_ref.sum()
    assert np.allclose(out["row_loss"].cpu().numpy(), ref64["score"], rtol=1e-3)


def test_chol_block_independent_selection(nvq):
    W, X = synth.attn_proj_layer(96, 512, 3000)
    H, g, codes, scales, out, _ = _chol_case(nvq, W, X, 8, torch.bfloat16, nvq.FLAG_INDEP)
    Uref, _ = gptq.hinv_factor(H)
    ref = gptq.sweep(W, Uref, g, 8, select="independent")
    assert _mismatch(codes, ref["codes"]) <= 1e-3
    assert _mismatch(scales, ref["scales"]) <= 1e-3


def test_chol_end_to_end_layer(nvq):
    m, k, n, K = 256, 512, 6000, 16
    W, X = synth.attn_proj_layer(m, k, n)
    res = nvq.quantize_layer(_to_dev(W, torch.bfloat16), synth.to_bf16_tensor(X).to(DEV), n_cand=K, chol=True)
    ref = gptq.quantize_layer(W, X, n_cand=K)
    codes = codec.unpack_codes(res["codes"].cpu().numpy())
    assert _mismatch(codes, ref["codes"]) <= 1e-3
    assert _mismatch(res["scales"].cpu().numpy(), ref["scales"]) <= 1e-3
    E = res["row_err"].cpu().numpy().astype(np.float64).sum()
    assert abs(E - ref["row_err"].sum()) <= 1e-3 * ref["row_err"].sum()


def test_chol_batched_equals_single_and_is_reproducible(nvq):
    B, m, k, n, K = 3, 64, 384, 3000, 16
    Ws, Vs, Hs, gs = [], [], [], []
    for e in range(B):
        W = synth.moe_expert_weights(e, m, k)
        X = synth.activations("attn_proj", n, k, massive=4)[e * 7:]
        H = gptq.hessian(X).astype(np.float32)
        V, _, info = nvq.factor_chol(_to_dev(H))
        assert int(info.item()) == 0
        Ws.append(_to_dev(W, torch.bfloat16)); Vs.append(V); Hs.append(_to_dev(H))
        gs.append(nvq.nvfp4_global_scale(Ws[-1]))
    Wb, Vb, Hb, gb = torch.stack(Ws), torch.stack(Vs), torch.stack(Hs), torch.stack(gs).reshape(B)
    flags = nvq.FLAG_CHOL_FACTOR
    batched = nvq.gptq_nvfp4_quantize_batched(Wb, Vb, Hb, gb, K, flags)
    again = nvq.gptq_nvfp4_quantize_batched(Wb, Vb, Hb, gb, K, flags)
    keys = ("codes", "scales", "row_err", "row_loss")
    for key in keys:
        assert np.array_equal(batched[key].cpu().numpy().view(np.uint8), again[key].cpu().numpy().view(np.uint8)), key
    for e in range(B):
        one = nvq.gptq_nvfp4_quantize(Ws[e], Vs[e], Hs[e], gb[e:e + 1], K, flags)
        for key in keys:
            a, b = batched[key][e].cpu().numpy(), one[key].cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (e, key)

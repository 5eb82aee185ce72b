"""GPU parity of the block-independent scale selection (NVQ_FLAG_INDEP, the
baseline Schur Replay corrects) against the CPU oracle, and the
scale-selection ablation on one layer: round to nearest with the absmax
scale, GPTQ with the absmax scale (one candidate), GPTQ with the
block-independent choice, and GPTQ with Schur Replay."""

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


@pytest.mark.parametrize("m,k,n,K", [(200, 384, 3000, 16), (64, 1040, 4096, 8)])
def test_independent_selection_matches_oracle(nvq, m, k, n, K):
    W, X = synth.attn_proj_layer(m, k, n)
    H = gptq.hessian(X)
    U, _ = gptq.hinv_factor(H)
    U32 = U.astype(np.float32)
    g = codec.global_scale(W)
    for flags, dt in ((nvq.FLAG_INDEP, np.float32), (nvq.FLAG_INDEP | nvq.FLAG_FP64, np.float64)):
        out = nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), _to_dev(U32), _to_dev(H.astype(np.float32)),
                                      _to_dev(np.array([g])), K, flags)
        codes = codec.unpack_codes(out["codes"].cpu().numpy())
        scales = out["scales"].cpu().numpy()
        ref = gptq.sweep(W, U32, g, K, dtype=dt, select="independent")
        assert _mismatch(codes, ref["codes"]) <= 1e-3, flags
        assert _mismatch(scales, ref["scales"]) <= 1e-3, flags
        # row_loss stays the damped loss: the committed replay scores
        assert np.allclose(out["row_loss"].cpu().numpy(), ref["score"], rtol=1e-4), flags
        deq = codec.dequantize(codec.pack_codes(codes), scales, g)
        E_own = gptq.weighted_error(W, deq, H)
        assert np.allclose(out["row_err"].cpu().numpy().astype(np.float64), E_own, rtol=1e-4,
                           atol=1e-6 * E_own.max()), flags


def test_independent_flag_ignored_with_rtn(nvq):
    W, _ = synth.attn_proj_layer(32, 256, 64)
    g = codec.global_scale(W)
    Wd, gd = _to_dev(W), _to_dev(np.array([g]))
    a = nvq.gptq_nvfp4_quantize(Wd, None, None, gd, 4, nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    b = nvq.gptq_nvfp4_quantize(Wd, None, None, gd, 4, nvq.FLAG_RTN | nvq.FLAG_NO_ERR | nvq.FLAG_INDEP)
    assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["scales"], b["scales"])


def test_scale_selection_ablation(nvq):
    # One 1024 x 1024 layer of the attention-projection recipe; the four
    # configurations' total weighted errors must order as the method claims:
    # Schur Replay < GPTQ + block-independent choice, GPTQ < RTN.
    m = k = 1024
    W, X = synth.attn_proj_layer(m, k, 16384)
    Wd = _to_dev(W, torch.bfloat16)
    res = nvq.quantize_layer(Wd, _to_dev(X, torch.bfloat16), n_cand=16)
    U, H, g = res["U"], res["H"], res["g"]
    E = {"replay": float(res["row_err"].double().sum())}
    E["independent"] = float(nvq.gptq_nvfp4_quantize(Wd, U, H, g, 16, nvq.FLAG_INDEP)["row_err"].double().sum())
    E["gptq_absmax"] = float(nvq.gptq_nvfp4_quantize(Wd, U, H, g, 1)["row_err"].double().sum())
    rtn = nvq.gptq_nvfp4_quantize(Wd, None, None, g, 1, nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    deq = codec.dequantize(rtn["codes"].cpu().numpy(), rtn["scales"].cpu().numpy(), np.float32(g.item()))
    E["rtn_absmax"] = float(gptq.weighted_error(W, deq, H.cpu().numpy().astype(np.float64)).sum())
    print("total weighted error per configuration:", E)
    assert E["replay"] < E["independent"]
    assert E["replay"] < E["gptq_absmax"] < E["rtn_absmax"]

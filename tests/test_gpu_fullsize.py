"""GPU parity at the benchmarked size, on sampled outputs.

Workload: the attention-projection layer timed by bench.py (W 4096 x 4096 bf16
~N(0, 0.02^2) with 0.1% Student-t(3) entries; X 262,144 tokens x 4096 bf16
with log-normal channel scales and 8 massive channels; 16 candidates per
block), run through the same C-ABI calls and launch configuration.  The CPU
oracle recomputes what it can in seconds:
  * 6 full rows of H = X^T X in fp64 (token chunks), within the fp32
    summation bound; the whole H exactly symmetric;
  * the whole factor U from the GPU's H (fp64), to 1e-4 of max|U|;
  * the sweep of 32 sampled rows from the GPU's U (fp32 and fp64 modes):
    at most 0.1% of codes and scales differ; the GPU's weighted errors of those
    rows equal the fp64 error of its own codes to 1e-4, and their total is
    within 1e-3 of the oracle's;
  * the global scale, the round-to-nearest encode (one candidate) and the bf16
    dequantization of sampled rows bit-exactly.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import codec, gptq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
M = K_IN = 4096
N_TOK = 262144
N_CAND = 16
RNG = np.random.default_rng(12345)
SAMPLE_ROWS = np.sort(RNG.choice(M, size=32, replace=False))


def _mismatch(a, b):
    return float(np.mean(np.asarray(a) != np.asarray(b)))


@pytest.fixture(scope="module")
def full():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_nvfp4_weight_amd as nvq
    X = torch.empty(N_TOK, K_IN, dtype=torch.bfloat16)
    synth.activations("attn_proj", N_TOK, K_IN, massive=8, out=X)
    W = synth.weights("attn_proj", M, K_IN, 0.02, outlier_frac=0.001)
    Xd = X.to(DEV)
    Wd = synth.to_bf16_tensor(W).to(DEV)
    res = nvq.quantize_layer(Wd, Xd, n_cand=N_CAND)
    deq = nvq.nvfp4_dequantize(res["codes"], res["scales"], res["g"], torch.bfloat16)
    rtn = nvq.gptq_nvfp4_quantize(Wd, None, None, res["g"], 1, nvq.FLAG_RTN | nvq.FLAG_NO_ERR)
    torch.cuda.synchronize()
    out = {
        "X": X, "W": W,
        "H": res["H"].cpu().numpy(), "U": res["U"].cpu().numpy(),
        "lam": float(res["lam"].item()), "info": int(res["info"].item()), "g": np.float32(res["g"].item()),
        "codes": codec.unpack_codes(res["codes"].cpu().numpy()), "packed": res["codes"].cpu().numpy(),
        "scales": res["scales"].cpu().numpy(), "row_err": res["row_err"].cpu().numpy().astype(np.float64),
        "deq": deq.view(torch.int16).cpu().numpy(),
        "rtn_codes": rtn["codes"].cpu().numpy(), "rtn_scales": rtn["scales"].cpu().numpy(),
    }
    del Xd, Wd, res
    torch.cuda.empty_cache()
    return out


def test_full_hessian_sampled_rows(full):
    H = full["H"]
    assert np.array_equal(H, H.T)
    X = full["X"]
    # 5 random channels plus the channel of largest scale (a massive channel)
    s = synth.channel_scales("attn_proj", K_IN, massive=8)
    rows = np.unique(np.concatenate([RNG.choice(K_IN, size=5, replace=False), [int(np.argmax(s))]]))
    ref = np.zeros((len(rows), K_IN))
    bnd = np.zeros((len(rows), K_IN))
    for c0 in range(0, N_TOK, 8192):
        xc = X[c0:c0 + 8192].float().numpy().astype(np.float64)
        ref += xc[:, rows].T @ xc
        bnd += np.abs(xc[:, rows]).T @ np.abs(xc)
    bound = bnd * ((N_TOK / 16 + 64) * 2.0 ** -23)
    assert np.all(np.abs(H[rows].astype(np.float64) - ref) <= bound + 1e-30)


def test_full_factor(full):
    assert full["info"] == 0
    H = full["H"].astype(np.float64)
    Uref, lam = gptq.hinv_factor(H)
    assert full["lam"] == pytest.approx(lam, rel=1e-5)
    U = full["U"]
    assert np.all(np.tril(U, -1) == 0)
    assert np.max(np.abs(U - Uref)) <= 1e-4 * np.max(np.abs(Uref))


def test_full_global_scale_and_rtn(full):
    W = full["W"]
    assert full["g"] == codec.global_scale(W)
    ref = gptq.rtn(W[SAMPLE_ROWS], full["g"], 1)
    assert np.array_equal(full["rtn_codes"][SAMPLE_ROWS], codec.pack_codes(ref["codes"]))
    assert np.array_equal(full["rtn_scales"][SAMPLE_ROWS], ref["scales"])


def test_full_sweep_sampled_rows(full):
    W = full["W"][SAMPLE_ROWS]
    U = full["U"]
    g = full["g"]
    codes = full["codes"][SAMPLE_ROWS]
    scales = full["scales"][SAMPLE_ROWS]
    for dt in (np.float32, np.float64):
        ref = gptq.sweep(W, U, g, N_CAND, dtype=dt)
        assert _mismatch(codes, ref["codes"]) <= 1e-3, dt
        assert _mismatch(scales, ref["scales"]) <= 1e-3, dt
    H = full["H"].astype(np.float64)
    deq_gpu = codec.dequantize(codec.pack_codes(codes), scales, g)
    E_own = gptq.weighted_error(W, deq_gpu, H)
    E_gpu = full["row_err"][SAMPLE_ROWS]
    assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max())
    deq_ref = codec.dequantize(codec.pack_codes(ref["codes"]), ref["scales"], g)
    E_ref = gptq.weighted_error(W, deq_ref, H)
    assert abs(E_gpu.sum() - E_ref.sum()) <= 1e-3 * E_ref.sum()


def test_full_dequant_bf16_sampled_rows(full):
    rows = SAMPLE_ROWS
    ref = codec.dequantize(full["packed"][rows], full["scales"][rows], full["g"])
    refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(full["deq"][rows], refb)

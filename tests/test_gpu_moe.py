"""GPU parity of the mixture-of-experts calls: grouped Hessians over routed
token rows, batched factors (the U form and the Cholesky-factor form) and
batched quantization, against the CPU oracle applied expert by expert (each
expert is a linear layer of its own).

The small case checks every expert.  The full case is the MoE workload at its
real shape (256 experts with gate and up stacked as 2048 x 4096, 262,144
tokens routed top-8 with Zipf(1.1) popularity) and checks three experts (the
least, the median and the most loaded) on sampled outputs.
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


def _mismatch(a, b):
    return float(np.mean(np.asarray(a) != np.asarray(b)))


def _hessian_bound_ok(H, Xe):
    Xd = Xe.astype(np.float64)
    ref = Xd.T @ Xd
    bound = np.abs(Xd).T @ np.abs(Xd) * ((len(Xd) / 16 + 64) * 2.0 ** -23)
    return np.array_equal(H, H.T) and bool(np.all(np.abs(H - ref) <= bound + 1e-30))


def test_moe_small_every_expert(nvq):
    E, n, k, m, top_k = 6, 3000, 256, 48, 2
    X = synth.activations("moe", n, k)
    idx, off = synth.moe_routing(n, E, top_k)
    Xt = synth.to_bf16_tensor(X).to(DEV)
    Hg = nvq.hessian_accumulate_grouped(Xt, torch.from_numpy(idx).to(DEV), off)
    U, lam, info = nvq.factor_hinv_batched(Hg)
    W = np.stack([synth.moe_expert_weights(e, m, k) for e in range(E)])
    Wt = synth.to_bf16_tensor(W.reshape(E * m, k)).reshape(E, m, k).to(DEV)
    g = torch.stack([nvq.nvfp4_global_scale(Wt[e]) for e in range(E)]).reshape(E)
    out = nvq.gptq_nvfp4_quantize_batched(Wt, U, Hg, g, 16)
    torch.cuda.synchronize()
    Hc, Uc, gc = Hg.cpu().numpy(), U.cpu().numpy(), g.cpu().numpy()
    codes = out["codes"].cpu().numpy()
    scales = out["scales"].cpu().numpy()
    row_err = out["row_err"].cpu().numpy().astype(np.float64)
    assert np.all(info.cpu().numpy() == 0)
    for e in range(E):
        rows = idx[off[e]:off[e + 1]]
        assert _hessian_bound_ok(Hc[e], X[rows]), e
        Uref, lam_ref = gptq.hinv_factor(Hc[e].astype(np.float64))
        assert float(lam[e].item()) == pytest.approx(lam_ref, rel=1e-5)
        assert np.max(np.abs(Uc[e] - Uref)) <= 1e-4 * np.max(np.abs(Uref)), e
        assert gc[e] == codec.global_scale(W[e])
        ref = gptq.sweep(W[e], Uc[e], gc[e], 16, dtype=np.float32)
        ce = codec.unpack_codes(codes[e])
        assert _mismatch(ce, ref["codes"]) <= 1e-3, e
        assert _mismatch(scales[e], ref["scales"]) <= 1e-3, e
        deq = codec.dequantize(codes[e], scales[e], gc[e])
        E_own = gptq.weighted_error(W[e], deq, Hc[e])
        assert np.allclose(row_err[e], E_own, rtol=1e-4, atol=1e-6 * E_own.max()), e


def _v_from_u(U):
    """V of the oracle's U (the form FLAG_CHOL_FACTOR takes): R = U^-1 in fp64, V = -R_ij / R_jj above
    the diagonal, R_ii on it, 0 below."""
    R = np.triu(np.linalg.inv(U))
    d = np.diag(R)
    return np.triu(-R / d[None, :], 1) + np.diag(d)


def _v_close(V, Vref):
    d, dref = np.diag(V), np.diag(Vref)
    off, offref = np.triu(V, 1), np.triu(Vref, 1)
    return (np.all(np.tril(V, -1) == 0) and np.max(np.abs(d - dref)) <= 1e-4 * np.max(dref)
            and np.max(np.abs(off - offref)) <= 1e-4 * np.max(np.abs(offref)))


def test_moe_small_every_expert_cholesky_form(nvq):
    """The same layer through factor_chol_batched and the sweep on V (FLAG_CHOL_FACTOR): every expert's V
    against the oracle's factor, and its codes, scales and errors against the oracle's fp64 sweep with its
    own U."""
    E, n, k, m, top_k = 6, 3000, 256, 48, 2
    X = synth.activations("moe", n, k)
    idx, off = synth.moe_routing(n, E, top_k)
    Xt = synth.to_bf16_tensor(X).to(DEV)
    Hg = nvq.hessian_accumulate_grouped(Xt, torch.from_numpy(idx).to(DEV), off)
    V, lam, info = nvq.factor_chol_batched(Hg)
    W = np.stack([synth.moe_expert_weights(e, m, k) for e in range(E)])
    Wt = synth.to_bf16_tensor(W.reshape(E * m, k)).reshape(E, m, k).to(DEV)
    g = torch.stack([nvq.nvfp4_global_scale(Wt[e]) for e in range(E)]).reshape(E)
    out = nvq.gptq_nvfp4_quantize_batched(Wt, V, Hg, g, 16, nvq.FLAG_CHOL_FACTOR)
    torch.cuda.synchronize()
    assert np.all(info.cpu().numpy() == 0)
    Hc, Vc, gc = Hg.cpu().numpy(), V.cpu().numpy().astype(np.float64), g.cpu().numpy()
    codes, scales = out["codes"].cpu().numpy(), out["scales"].cpu().numpy()
    row_err = out["row_err"].cpu().numpy().astype(np.float64)
    for e in range(E):
        Uref, lam_ref = gptq.hinv_factor(Hc[e].astype(np.float64))
        assert float(lam[e].item()) == pytest.approx(lam_ref, rel=1e-5)
        assert _v_close(Vc[e], _v_from_u(Uref)), e
        ref = gptq.sweep(W[e], Uref, gc[e], 16)
        ce = codec.unpack_codes(codes[e])
        assert _mismatch(ce, ref["codes"]) <= 1e-3, e
        assert _mismatch(scales[e], ref["scales"]) <= 1e-3, e
        deq = codec.dequantize(codes[e], scales[e], gc[e])
        E_own = gptq.weighted_error(W[e], deq, Hc[e])
        assert np.allclose(row_err[e], E_own, rtol=1e-4, atol=1e-6 * E_own.max()), e


def test_moe_grouped_launch_k4096(nvq):
    """At k = 4096 the experts under 16384 tokens share grouped launches (every tile of every such expert
    over its whole token range, adding into its own H) and the larger ones take the one-expert path:
    experts of 0 to 20000 tokens, ragged counts, an H that already holds values; every H_e within the
    fp32 summation bound of H0_e + X_e^T X_e in fp64, exactly symmetric."""
    k = 4096
    counts = [777, 0, 1, 16384, 31, 100, 5000, 2048, 20000, 3, 9999]
    n = 24000
    X = synth.activations("moe", n, k)
    rng = np.random.default_rng(11)
    idx = np.concatenate([rng.choice(n, size=c, replace=False) for c in counts]).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    E = len(counts)
    H0 = np.zeros((E, k, k), dtype=np.float32)
    H0[4] = 3.0   # an H that already holds values: the grouped tiles add into it
    Hg = nvq.hessian_accumulate_grouped(synth.to_bf16_tensor(X).to(DEV), torch.from_numpy(idx).to(DEV), off,
                                        torch.from_numpy(H0).to(DEV))
    torch.cuda.synchronize()
    Hc = Hg.cpu().numpy()
    for e in range(E):
        Xe = X[idx[off[e]:off[e + 1]]].astype(np.float64)
        ref = H0[e].astype(np.float64) + Xe.T @ Xe
        bound = np.abs(Xe).T @ np.abs(Xe) * ((len(Xe) / 16 + 64) * 2.0 ** -23) + 4 * 2.0 ** -24 * np.abs(H0[e])
        assert np.array_equal(Hc[e], Hc[e].T), e
        assert np.all(np.abs(Hc[e] - ref) <= bound + 1e-30), e


def test_moe_empty_group_leaves_its_hessian(nvq):
    k = 64
    X = synth.to_bf16_tensor(synth.activations("moe", 100, k)).to(DEV)
    idx = torch.arange(0, 60, dtype=torch.int32, device=DEV)
    H0 = torch.full((3, k, k), 7.0, device=DEV)
    H = nvq.hessian_accumulate_grouped(X, idx, [0, 30, 30, 60], H0.clone())
    assert torch.equal(H[1], H0[1])
    assert not torch.equal(H[0], H0[0]) and not torch.equal(H[2], H0[2])


def test_moe_full_shape_sampled_experts(nvq):
    E, n, k, m, top_k = 256, 262144, 4096, 2048, 8
    X = torch.empty(n, k, dtype=torch.bfloat16)
    synth.activations("moe", n, k, out=X)
    idx, off = synth.moe_routing(n, E, top_k)
    counts = np.diff(off)
    Xd = X.to(DEV)
    Hg = nvq.hessian_accumulate_grouped(Xd, torch.from_numpy(idx).to(DEV), off)
    del Xd
    U, lam, info = nvq.factor_hinv_batched(Hg)
    Wt = torch.empty(E, m, k, dtype=torch.bfloat16, device=DEV)
    for e in range(E):
        Wt[e] = synth.to_bf16_tensor(synth.moe_expert_weights(e, m, k)).to(DEV)
    g = torch.stack([nvq.nvfp4_global_scale(Wt[e]) for e in range(E)]).reshape(E)
    out = nvq.gptq_nvfp4_quantize_batched(Wt, U, Hg, g, 16)
    # the Cholesky-factor form, as the MoE benchmark runs it
    V, _, info_c = nvq.factor_chol_batched(Hg)
    out_c = nvq.gptq_nvfp4_quantize_batched(Wt, V, Hg, g, 16, nvq.FLAG_CHOL_FACTOR)
    torch.cuda.synchronize()
    assert np.all(info.cpu().numpy() == 0)
    assert np.all(info_c.cpu().numpy() == 0)
    order = np.argsort(counts)
    rng = np.random.default_rng(7)
    for e in (int(order[0]), int(order[E // 2]), int(order[-1])):
        rows_tok = idx[off[e]:off[e + 1]]
        He = Hg[e].cpu().numpy()
        assert np.array_equal(He, He.T)
        # two full rows of H_e in fp64 over the expert's tokens
        ch = rng.choice(k, size=2, replace=False)
        ref = np.zeros((2, k))
        bnd = np.zeros((2, k))
        for c0 in range(0, len(rows_tok), 8192):
            xc = X[torch.from_numpy(rows_tok[c0:c0 + 8192].astype(np.int64))].float().numpy().astype(np.float64)
            ref += xc[:, ch].T @ xc
            bnd += np.abs(xc[:, ch]).T @ np.abs(xc)
        assert np.all(np.abs(He[ch] - ref) <= bnd * ((len(rows_tok) / 16 + 64) * 2.0 ** -23) + 1e-30), e
        Uref, _ = gptq.hinv_factor(He.astype(np.float64))
        Ue = U[e].cpu().numpy()
        assert np.max(np.abs(Ue - Uref)) <= 1e-4 * np.max(np.abs(Uref)), e
        We = synth.moe_expert_weights(e, m, k)
        ge = np.float32(g[e].item())
        assert ge == codec.global_scale(We)
        rows = np.sort(rng.choice(m, size=8, replace=False))
        ref_s = gptq.sweep(We[rows], Ue, ge, 16, dtype=np.float32)
        ce = codec.unpack_codes(out["codes"][e][rows].cpu().numpy())
        se = out["scales"][e][rows].cpu().numpy()
        assert _mismatch(ce, ref_s["codes"]) <= 1e-3, e
        assert _mismatch(se, ref_s["scales"]) <= 1e-3, e
        deq = codec.dequantize(codec.pack_codes(ce), se, ge)
        E_own = gptq.weighted_error(We[rows], deq, He)
        E_gpu = out["row_err"][e][rows].cpu().numpy().astype(np.float64)
        assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max()), e
        # Cholesky-factor form: V against the oracle's factor, the sampled rows against its fp64 sweep
        assert _v_close(V[e].cpu().numpy().astype(np.float64), _v_from_u(Uref)), e
        ref_c = gptq.sweep(We[rows], Uref, ge, 16)
        cc = codec.unpack_codes(out_c["codes"][e][rows].cpu().numpy())
        sc = out_c["scales"][e][rows].cpu().numpy()
        assert _mismatch(cc, ref_c["codes"]) <= 1e-3, e
        assert _mismatch(sc, ref_c["scales"]) <= 1e-3, e
        deq = codec.dequantize(codec.pack_codes(cc), sc, ge)
        E_own = gptq.weighted_error(We[rows], deq, He)
        E_gpu = out_c["row_err"][e][rows].cpu().numpy().astype(np.float64)
        assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max()), e

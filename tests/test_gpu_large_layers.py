"""GPU parity on the large layer shapes, at their real sizes, on sampled outputs
and properties that hold at any size.

  * MLP pair of an 8B-class block: gate and up (14336 x 4096 each, stacked to
    28672 x 4096) over X of 131,072 tokens x 4096; down (4096 x 14336) over
    the block's own intermediate activations bf16(SiLU(X W_gate^T) * (X W_up^T)).
  * 70B-class down projection: W 8192 x 28672 with 0.05% Student-t(3)
    outliers, X 65,536 x 28672 with 60% exact zeros; H (28672^2 fp32) resident.

What is checked against the fp64 oracle:
  * H exactly symmetric; two full rows within the fp32 summation bound;
  * U: its trailing t x t block depends only on the trailing block of
    H + lam I (U is the inverse of the index-reversed Cholesky factor), so the
    oracle factors that block (t = 2048) and the GPU's block must agree to
    1e-4 of its max; lam against mean(diag H);
  * the sweep of sampled rows given the GPU's U, run with fp64 working
    precision (NVQ_FLAG_FP64) against the fp64 oracle: at most 0.1% of codes
    and scales differ; every row that diverges does so first at a near tie (a
    scale choice whose two best replay scores lie within 1e-3 relative, or an
    element within 1e-4 of an E2M1 rounding midpoint), after which GPTQ's
    column coupling carries the difference along the row; and the GPU's
    weighted errors equal the fp64 errors of its own codes to 1e-4.
    These layers' Hessians span up to 8 orders of magnitude: in fp32, rounding
    alone (in the oracle as much as on the GPU) moves 0.1-0.7% of the
    decisions of the exact computation, all of them at near ties.
  * the Cholesky-factor form (factor_chol and the fp64 sweep on V, as the
    layer benchmark runs it) on the same H: V's trailing block against the
    oracle's, and the same sampled rows to the same bars.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import codec, gptq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
T_BLOCK = 2048


@pytest.fixture(scope="module")
def nvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_nvfp4_weight_amd as m
    return m


def _mismatch(a, b):
    return float(np.mean(np.asarray(a) != np.asarray(b)))


MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _first_divergence_is_near_tie(codes, scales, ref, i, g):
    """Where a row of GPU decisions first departs from the oracle's, the oracle's
    own decision there must be a near tie."""
    dc = np.nonzero(codes != ref["codes"][i])[0]
    ds = np.nonzero(scales != ref["scales"][i])[0]
    if len(dc) == 0 and len(ds) == 0:
        return
    b = min(ds[0] if len(ds) else 1 << 30, dc[0] // 16 if len(dc) else 1 << 30)
    if scales[b] != ref["scales"][i][b]:
        sc = np.sort(ref["cand_score"][i, b].astype(np.float64))
        assert (sc[1] - sc[0]) <= 1e-3 * sc[0], (i, b, sc[:2])
    else:
        j = dc[0]
        r = abs(float(ref["vdec"][i, j])) / (float(codec.e4m3_decode(scales[b])) * float(g))
        assert np.min(np.abs(r - MIDPOINTS) / MIDPOINTS) <= 1e-4, (i, j, r)


def _check_layer(nvq, Xh, Xd, W, rng, n_rows=32, fp32_too=False):
    """Runs the whole layer on the GPU and checks it; Xh: host bf16 tensor, Xd: the same on the device.
    With fp32_too, the default fp32 sweep of the same sampled rows is held to the same 0.1% bars
    against the fp64 oracle."""
    n, k = Xh.shape
    Wd = synth.to_bf16_tensor(W).to(DEV)
    res = nvq.quantize_layer(Wd, Xd, n_cand=16, flags=nvq.FLAG_FP64)
    torch.cuda.synchronize()
    H, U = res["H"], res["U"]
    assert int(res["info"].item()) == 0
    assert torch.equal(H, H.t())
    # two rows of H in fp64
    ch = np.sort(rng.choice(k, size=2, replace=False))
    ref = np.zeros((2, k))
    bnd = np.zeros((2, k))
    for c0 in range(0, n, 8192):
        xc = Xh[c0:c0 + 8192].float().numpy().astype(np.float64)
        ref += xc[:, ch].T @ xc
        bnd += np.abs(xc[:, ch]).T @ np.abs(xc)
    Hrows = H[torch.from_numpy(ch).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Hrows - ref) <= bnd * ((n / 16 + 64) * 2.0 ** -23) + 1e-30)
    # lambda and the trailing block of U
    diag = torch.diagonal(H).double().cpu().numpy()
    lam = 0.01 * diag.mean()
    assert float(res["lam"].item()) == pytest.approx(lam, rel=1e-5)
    t = min(T_BLOCK, k)
    Ht = H[k - t:, k - t:].cpu().numpy().astype(np.float64)
    Hd = Ht + float(res["lam"].item()) * np.eye(t)
    Ut_ref = np.linalg.cholesky(np.linalg.inv(Hd)).T
    Ut = U[k - t:, k - t:].cpu().numpy()
    assert np.max(np.abs(Ut - Ut_ref)) <= 1e-4 * np.max(np.abs(Ut_ref))
    # the sweep of sampled rows, given the GPU's U
    rows = np.sort(rng.choice(W.shape[0], size=n_rows, replace=False))
    Uh = U.cpu().numpy()
    g = np.float32(res["g"].item())
    assert g == codec.global_scale(W)
    ref_s = gptq.sweep(W[rows], Uh, g, 16, dtype=np.float64, trace=True)
    del Uh
    rows_t = torch.from_numpy(rows).to(DEV)
    codes = codec.unpack_codes(res["codes"][rows_t].cpu().numpy())
    scales = res["scales"][rows_t].cpu().numpy()
    assert _mismatch(codes, ref_s["codes"]) <= 1e-3
    assert _mismatch(scales, ref_s["scales"]) <= 1e-3
    for i in range(len(rows)):
        _first_divergence_is_near_tie(codes[i], scales[i], ref_s, i, g)
    if fp32_too:
        r32 = nvq.gptq_nvfp4_quantize(Wd, U, H, res["g"], 16)
        c32 = codec.unpack_codes(r32["codes"][rows_t].cpu().numpy())
        s32 = r32["scales"][rows_t].cpu().numpy()
        print(f"fp32 sweep, {len(rows)} rows: code mismatch {_mismatch(c32, ref_s['codes']):.2e}, "
              f"scale mismatch {_mismatch(s32, ref_s['scales']):.2e} against the fp64 oracle")
        assert _mismatch(c32, ref_s["codes"]) <= 1e-3
        assert _mismatch(s32, ref_s["scales"]) <= 1e-3
        for i in range(len(rows)):
            _first_divergence_is_near_tie(c32[i], s32[i], ref_s, i, g)
        del r32
    deq = codec.dequantize(codec.pack_codes(codes), scales, g)
    dW = W[rows].astype(np.float64) - deq.astype(np.float64)
    Hh = H.cpu().numpy().astype(np.float64)
    E_own = np.einsum("rk,rk->r", dW @ Hh, dW)
    E_gpu = res["row_err"][rows_t].cpu().numpy().astype(np.float64)
    assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max())
    # The Cholesky-factor form (factor_chol, the sweep on V; what the layer benchmark times): V's
    # trailing block against the oracle's (R = U^-1 is upper triangular, so its trailing block is the
    # inverse of U's), and the sampled rows of the fp64 sweep on V to the same bars.
    V, lam_c, info_c = nvq.factor_chol(H)
    rc = nvq.gptq_nvfp4_quantize(Wd, V, H, res["g"], 16, nvq.FLAG_FP64 | nvq.FLAG_CHOL_FACTOR)
    torch.cuda.synchronize()
    assert int(info_c.item()) == 0
    assert float(lam_c.item()) == float(res["lam"].item())
    Rt = np.triu(np.linalg.inv(Ut_ref))
    dt = np.diag(Rt)
    Vt_ref = np.triu(-Rt / dt[None, :], 1) + np.diag(dt)
    Vt = V[k - t:, k - t:].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(np.diag(Vt) - dt)) <= 1e-4 * np.max(dt)
    assert np.max(np.abs(np.triu(Vt, 1) - np.triu(Vt_ref, 1))) <= 1e-4 * np.max(np.abs(np.triu(Vt_ref, 1)))
    cc = codec.unpack_codes(rc["codes"][rows_t].cpu().numpy())
    sc = rc["scales"][rows_t].cpu().numpy()
    print(f"Cholesky-factor form, {len(rows)} rows: code mismatch {_mismatch(cc, ref_s['codes']):.2e}, "
          f"scale mismatch {_mismatch(sc, ref_s['scales']):.2e} against the fp64 oracle")
    assert _mismatch(cc, ref_s["codes"]) <= 1e-3
    assert _mismatch(sc, ref_s["scales"]) <= 1e-3
    for i in range(len(rows)):
        _first_divergence_is_near_tie(cc[i], sc[i], ref_s, i, g)
    deq = codec.dequantize(codec.pack_codes(cc), sc, g)
    dW = W[rows].astype(np.float64) - deq.astype(np.float64)
    E_own = np.einsum("rk,rk->r", dW @ Hh, dW)
    E_gpu = rc["row_err"][rows_t].cpu().numpy().astype(np.float64)
    assert np.allclose(E_gpu, E_own, rtol=1e-4, atol=1e-6 * E_own.max())


def test_mlp_pair_gate_up_and_down(nvq):
    rng = np.random.default_rng(31)
    n, d, f = 131072, 4096, 14336
    Xh = torch.empty(n, d, dtype=torch.bfloat16)
    synth.activations("mlp", n, d, out=Xh)
    Wg, Wu, Wdown = synth.mlp_block_weights(d, f)
    Xd = Xh.to(DEV)
    # gate and up (zero-mean inputs): the default fp32 sweep meets the 0.1% bar; fp64 checked too
    _check_layer(nvq, Xh, Xd, np.concatenate([Wg, Wu]), rng, n_rows=32, fp32_too=True)
    # down projection over the block's intermediate activations (fp64 sweep)
    Xdown = synth.mlp_down_activations(Xd, Wg, Wu)
    del Xd
    _check_layer(nvq, Xdown.cpu(), Xdown, Wdown, rng, n_rows=64)


def test_sparse_down_projection_28672(nvq):
    rng = np.random.default_rng(41)
    m, k, n = 8192, 28672, 65536
    Xh = torch.empty(n, k, dtype=torch.bfloat16)
    synth.activations("sparse", n, k, kind="sparse", out=Xh)
    W = synth.weights("sparse", m, k, 0.01, outlier_frac=0.0005)
    _check_layer(nvq, Xh, Xh.to(DEV), W, rng, n_rows=64)


def test_factor_panel_launch_larger_than_resident_workgroups(nvq):
    """k = 33,024: the first panel launches (k - 64) / 64 = 515 workgroups, more
    than fit on the device at once (2 per CU on 256 CUs), so some start only
    after others have finished.  Every workgroup reads the panel's diagonal
    block, so none may overwrite it.  The last workgroups' panel rows feed the
    first rows of U (U is the index-reversed inverse factor), which are checked
    by a property that holds at any size: with R = U^-1, U (H + lam I) = R^T is
    lower triangular, so in fp64 the strictly upper part of the first 256 rows
    of U (H + lam I) must vanish to the factor's rounding, and its diagonal is
    1 / U_ii.  H is made well conditioned (N(0, 1) tokens, cond(H + lam I) ~
    900).  There the factor's fp32 arithmetic (blocked Cholesky, then the
    recursive-doubling triangular inverse, whose left residual is the larger
    one: an fp32 emulation of the same recursion gives 2.4e-5 where an exact
    inverse of the same L gives 7e-7) leaves, relative to the diagonal, up to
    ~4e-5 above it and ~3e-4 on it -- the same at k = 16,384, where every
    launch fits on the device, and in U's middle rows.  The bounds are 5e-4
    and 2e-3; a panel row factored from the wrong diagonal block is off by
    order one.  The trailing 2048 x 2048 block of U is also compared with the
    fp64 oracle."""
    k, n, s = 33024, 8192, 256
    X = synth.to_bf16_tensor(synth.rng("small", 60).standard_normal((n, k), dtype=np.float32))
    H = nvq.hessian_accumulate(X.to(DEV))
    U, lam_t, info = nvq.factor_hinv(H)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    lam = float(lam_t.item())
    Us = U[:s].double().cpu().numpy()
    T = np.zeros((s, k))
    for c0 in range(0, k, 2048):
        Hc = H[:, c0:c0 + 2048].double().cpu().numpy()
        Hc[np.arange(c0, min(c0 + 2048, k)), np.arange(Hc.shape[1])] += lam
        T[:, c0:c0 + 2048] = Us @ Hc
    diag = T[np.arange(s), np.arange(s)]
    dev_diag = np.abs(diag * Us[np.arange(s), np.arange(s)] - 1.0)
    dev_up = np.array([np.max(np.abs(T[i, i + 1:])) / abs(diag[i]) for i in range(s)])
    print(f"first {s} rows of U (H + lam I): diagonal within {dev_diag.max():.2e} of 1 / U_ii, "
          f"upper part up to {dev_up.max():.2e} of the diagonal")
    assert np.all(dev_diag <= 2e-3), int(np.argmax(dev_diag))
    assert np.all(dev_up <= 5e-4), int(np.argmax(dev_up))
    del T, Us
    t = T_BLOCK
    Ht = H[k - t:, k - t:].cpu().numpy().astype(np.float64)
    Ut_ref = np.linalg.cholesky(np.linalg.inv(Ht + lam * np.eye(t))).T
    Ut = U[k - t:, k - t:].cpu().numpy()
    assert np.max(np.abs(Ut - Ut_ref)) <= 1e-4 * np.max(np.abs(Ut_ref))

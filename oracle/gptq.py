"""GPTQ sweep with Schur Replay block-scale selection (oracle; test infrastructure only).

Source: "Replay the Curvature" (arXiv 2609.36654), Abstract.  The abstract fixes
the three ingredients written out here:
  * second-order state: the curvature of the layer's squared reconstruction
    error, H = X^T X over calibration activations X;
  * the GPTQ column sweep: quantizing one column updates the columns that
    follow;
  * Schur Replay: for each candidate E4M3 scale of a 16-weight block, replay
    the GPTQ updates that this scale causes inside the block and score the
    block error that remains once the still-unquantized columns have
    compensated; keep the best candidate.

GPTQ itself (Frantar et al., 2022) is used as published: with U the upper
Cholesky factor of the damped inverse Hessian, (H + lam*I)^-1 = U^T U, column j
is quantized to q_j, its error e_j = (w_j - q_j) / U_jj is recorded, and every
later column l receives w_l -= e_j * U_jl.

Why the replay score is sum_j e_j^2 over the block: fixing the block to q_b
and re-optimizing the later columns raises the damped loss by
delta_b S_b delta_b^T, where S_b is the Schur complement of the block in the
trailing principal submatrix of H + lam*I.  With the in-block updates replayed,
delta_b = e_b U_bb and S_b = (U_bb^T U_bb)^-1, so the increase is sum_j e_j^2.
The CPU tests pin this against brute-force least squares.

Readings taken where the pages are silent:
  * H = X^T X, a plain sum over tokens; damping lam = 0.01 * mean(diag H) on
    every diagonal entry, used for U only;
  * column order is natural (blocks are contiguous 16-column runs);
  * block absmax is taken over the current (updated) weights;
  * candidate set: the K consecutive E4M3 codes centred on the code nearest to
    absmax / (6 g), [c0 - floor(K/2), c0 + ceil(K/2) - 1], shifted to lie in
    [1, 126]; an all-zero block gets scale code 0 and +0 elements;
  * score ties go to the lowest candidate (the smaller scale);
  * the weighted error of the layer uses the undamped H: per row,
    E_r = dW_r H dW_r^T with dW = W - dequant(W) (fp32 dequantized weights).

Precision: fp64 by default.  sweep(..., dtype=np.float32) runs the same steps
with the working weights, errors and scores held in fp32 (the GPU's working
precision), so that the integer decisions (codes, scales, argmin) are taken in
the same precision on both sides.  The element and scale roundings are exact in
either mode (see oracle.codec).
"""

import numpy as np

from . import codec

BLOCK = codec.BLOCK
DAMP_REL = 0.01


def hessian(X, chunk=8192):
    """H = sum over tokens t of x_t x_t^T, accumulated in fp64 over token chunks."""
    X = np.asarray(X)
    n, k = X.shape
    H = np.zeros((k, k), dtype=np.float64)
    for t0 in range(0, n, chunk):
        Xc = np.asarray(X[t0:t0 + chunk], dtype=np.float64)
        H += Xc.T @ Xc
    return H


def damping(H, damp_rel=DAMP_REL):
    """lam = damp_rel * mean(diag H)."""
    return float(damp_rel * np.mean(np.diag(H)))


def hinv_factor(H, damp_rel=DAMP_REL):
    """Upper-triangular U with (H + lam*I)^-1 = U^T U and positive diagonal; returns (U, lam).

    Written as the definition: invert the damped Hessian, take its Cholesky
    factor.  Raises numpy.linalg.LinAlgError if H + lam*I is not positive
    definite.
    """
    H = np.asarray(H, dtype=np.float64)
    lam = damping(H, damp_rel)
    Hd = H + lam * np.eye(H.shape[0])
    Hinv = np.linalg.inv(Hd)
    Hinv = (Hinv + Hinv.T) / 2.0
    U = np.linalg.cholesky(Hinv).T
    return U, lam


def candidate_codes(absmax, g, n_cand):
    """K consecutive E4M3 codes around the code nearest absmax/(6g), shifted into [1, 126].

    absmax: array of block absmax values.  Returns int array [..., n_cand].
    """
    c0 = codec.e4m3_rne_ratio(absmax, codec.E2M1_MAX * np.float64(g))
    lo = c0 - n_cand // 2
    lo = np.maximum(lo, 1)
    lo = np.minimum(lo, codec.E4M3_MAX_CODE - n_cand + 1)
    return lo[..., None] + np.arange(n_cand)


def sweep(W, U, g, n_cand, dtype=np.float64, trace=False, select="replay"):
    """GPTQ column sweep over 16-weight blocks with Schur Replay scale selection.

    W: [m, k] weights (any real dtype; read exactly).  U: [k, k] upper factor.
    g: per-tensor scale.  n_cand: candidates per block (1..16).
    select: "replay" (Schur Replay: the candidate whose replayed block errors
    have the smallest sum_j e_j^2), or "independent" (the baseline the pages
    set out to fix, scoring a block on its own: the candidate whose plain
    squared rounding error sum_j (v_j - q_j)^2 over the block's weights at the
    block start, each rounded with no in-block updates, is smallest).  Either
    way the chosen candidate's block is then committed with its replayed GPTQ
    updates.

    Returns dict with
      codes  uint8 [m, k]      4-bit element codes (unpacked),
      scales uint8 [m, k/16]   E4M3 block-scale codes,
      err    [m, k]            GPTQ errors e_j of the committed choice,
      score  [m]               sum_j e_j^2 (the damped loss of the sweep).
    With trace=True it also holds, per row and block, the candidate codes
    ("cand" [m, k/16, K]), the scores the choice was made on ("cand_score":
    replay scores, or the independent ones with select="independent"), the element
    codes each candidate chose ("cand_codes" [m, k/16, K, 16]) and the value
    of each column when it was quantized ("vdec" [m, k]).
    Updates are applied eagerly after each block (identical mathematics to
    lazily batched updates).
    """
    W = np.asarray(W)
    m, k = W.shape
    assert k % BLOCK == 0
    Wp = np.asarray(W, dtype=np.float64).astype(dtype)
    U = np.asarray(U, dtype=np.float64).astype(dtype)
    d = np.diag(U).copy()
    codes = np.zeros((m, k), dtype=np.uint8)
    scales = np.zeros((m, k // BLOCK), dtype=np.uint8)
    err = np.zeros((m, k), dtype=dtype)
    total = np.zeros(m, dtype=dtype)
    g = np.float32(g)
    if trace:
        nb = k // BLOCK
        tr_cand = np.zeros((m, nb, n_cand), dtype=np.int64)
        tr_score = np.zeros((m, nb, n_cand), dtype=dtype)
        tr_codes = np.zeros((m, nb, n_cand, BLOCK), dtype=np.uint8)
        vdec = np.zeros((m, k), dtype=dtype)
    for beta in range(k // BLOCK):
        c0, c1 = beta * BLOCK, (beta + 1) * BLOCK
        Ub = U[c0:c1, c0:c1]
        vb = Wp[:, c0:c1]
        absmax = np.max(np.abs(vb.astype(np.float64)), axis=1)
        cand = candidate_codes(absmax, g, n_cand)                 # [m, K]
        sval = codec.e4m3_decode(cand)                            # exact
        V = np.repeat(vb[:, None, :], n_cand, axis=1).copy()      # [m, K, 16]
        score = np.zeros((m, n_cand), dtype=dtype)
        if select == "independent":
            indep = np.zeros((m, n_cand), dtype=dtype)
            for j in range(BLOCK):
                v0 = V[:, :, j]
                q0 = codec.dequant_exact(codec.e2m1_encode(v0, sval, g), cand, g).astype(dtype)
                dj = (v0 - q0).astype(dtype)
                indep = (indep + dj * dj).astype(dtype)
        elif select != "replay":
            raise ValueError(f"select must be 'replay' or 'independent', got {select!r}")
        E = np.zeros((m, n_cand, BLOCK), dtype=dtype)
        C = np.zeros((m, n_cand, BLOCK), dtype=np.uint8)
        VD = np.zeros((m, n_cand, BLOCK), dtype=dtype)
        for j in range(BLOCK):
            vj = V[:, :, j]
            VD[:, :, j] = vj
            cj = codec.e2m1_encode(vj, sval, g)
            qj = codec.dequant_exact(cj, cand, g).astype(dtype)
            ej = ((vj - qj) / d[c0 + j]).astype(dtype)
            score = (score + ej * ej).astype(dtype)
            if j + 1 < BLOCK:
                V[:, :, j + 1:] -= ej[:, :, None] * Ub[j, j + 1:]
            E[:, :, j] = ej
            C[:, :, j] = cj
        best = np.argmin(score if select == "replay" else indep, axis=1)   # first minimum
        rows = np.arange(m)
        eb = E[rows, best]
        cb = C[rows, best]
        sb = cand[rows, best].astype(np.uint8)
        zero = absmax == 0.0
        eb[zero] = 0
        cb[zero] = 0
        sb[zero] = 0
        if trace:
            tr_cand[:, beta] = cand
            tr_score[:, beta] = score if select == "replay" else indep
            tr_codes[:, beta] = C
            vdec[:, c0:c1] = VD[rows, best]
        codes[:, c0:c1] = cb
        scales[:, beta] = sb
        err[:, c0:c1] = eb
        total = (total + np.where(zero, 0, score[rows, best])).astype(dtype)
        if c1 < k:
            Wp[:, c1:] -= (eb @ U[c0:c1, c1:]).astype(dtype)
    out = {"codes": codes, "scales": scales, "err": err, "score": total}
    if trace:
        out.update(cand=tr_cand, cand_score=tr_score, cand_codes=tr_codes, vdec=vdec)
    return out


def rtn(W, g, n_cand=1):
    """Round-to-nearest NVFP4 with no GPTQ updates: the sweep with U = I.

    With U = I there are no cross-column updates and each candidate's score is
    the plain squared error of the block, so the choice is the per-block
    minimum-MSE scale among the candidates (the absmax scale when n_cand = 1).
    """
    k = np.asarray(W).shape[1]
    return sweep(W, np.eye(k), g, n_cand)


def weighted_error(W, deq, H):
    """Per-row E_r = dW_r H dW_r^T with dW = W - deq, in fp64.

    Evaluated as the row sums of (dW H) * dW: the product dW H is one library
    matrix product, then each row is dotted with its own dW row.
    """
    dW = np.asarray(W, dtype=np.float64) - np.asarray(deq, dtype=np.float64)
    return np.sum((dW @ np.asarray(H, dtype=np.float64)) * dW, axis=1)


def quantize_layer(W, X=None, H=None, n_cand=16, damp_rel=DAMP_REL, g=None, dtype=np.float64):
    """Full layer: H from X (or given), U, global scale, sweep, packing and error.

    Returns dict with packed codes [m, k/2], scales [m, k/16], g, lam, U, H,
    row_err [m] (undamped weighted error), score [m] (damped loss of the sweep).
    """
    if H is None:
        H = hessian(X)
    U, lam = hinv_factor(H, damp_rel)
    if g is None:
        g = codec.global_scale(W)
    res = sweep(W, U, g, n_cand, dtype=dtype)
    packed = codec.pack_codes(res["codes"])
    deq = codec.dequantize(packed, res["scales"], g)
    row_err = weighted_error(W, deq, H)
    return {"packed": packed, "codes": res["codes"], "scales": res["scales"], "g": np.float32(g),
            "lam": lam, "U": U, "H": H, "row_err": row_err, "score": res["score"],
            "err": res["err"], "deq": deq}

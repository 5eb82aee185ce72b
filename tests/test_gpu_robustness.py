"""GPU behaviour on inputs the format cannot represent, and reproducibility.

  * nvq_check_finite reports 1 + the lowest row holding a NaN or infinity
    (bf16 and fp32, strided and unaligned rows), 0 when everything is finite;
  * NVQ_FLAG_CHECK_FINITE rejects exactly the rows of W holding a non-finite
    value (all rows for a non-finite g): codes 0, scales 0x7F (the E4M3FN NaN
    code), NaN row_err and row_loss, NaN after dequantization; every other row
    is quantized as if the bad rows were absent (rows are independent) and
    matches the oracle;
  * without the flag a NaN weight still gives the same outputs on every run
    (NaN scores lose every arg-min, so exactly one lane commits a block);
  * factor_hinv reports a non-finite H as info = -1;
  * the whole layer path is bitwise reproducible: two runs give identical H,
    U, lambda, codes, scales, row_err and row_loss.
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


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_check_finite_first_bad_row(nvq, dtype):
    rng = np.random.default_rng(5)
    rows, cols = 1500, 200
    A = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).to(dtype)
    assert int(nvq.check_finite(A.to(DEV)).item()) == 0
    for bad in ([7], [1499], [40, 900, 41], [0, 3]):
        B = A.clone()
        for j, r in enumerate(bad):
            B[r, (37 * r) % cols] = [float("nan"), float("inf"), -float("inf")][j % 3]
        assert int(nvq.check_finite(B.to(DEV)).item()) == min(bad) + 1, bad
    # strided rows (a column slice: rows start unaligned, scalar path) and a value past cols that is ignored
    C = torch.zeros(50, 40, dtype=dtype)
    C[:, 38] = float("nan")
    V = C.to(DEV)[:, 1:37]
    assert int(nvq.check_finite(V).item()) == 0
    C[12, 20] = float("inf")
    assert int(nvq.check_finite(C.to(DEV)[:, 1:37]).item()) == 13
    # no rows
    assert int(nvq.check_finite(torch.zeros(0, 16, dtype=dtype, device=DEV)).item()) == 0


def test_quantize_rejects_nonfinite_rows(nvq):
    m, k = 40, 384
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.01)
    X = synth.activations("attn_proj", 2 * k, k, massive=4)
    H = gptq.hessian(X)
    U, _ = gptq.hinv_factor(H)
    U32 = U.astype(np.float32)
    g = codec.global_scale(W)
    bad = {3: float("nan"), 10: float("inf"), 11: -float("inf"), 39: float("nan")}
    Wb = W.copy()
    for r, v in bad.items():
        Wb[r, (5 * r) % k] = v
    args = (_to_dev(U32), _to_dev(H.astype(np.float32)), _to_dev(np.array([g], dtype=np.float32)), 16)
    for dt in (torch.bfloat16, torch.float32):
        out = nvq.gptq_nvfp4_quantize(_to_dev(Wb, dt), *args, flags=nvq.FLAG_CHECK_FINITE)
        codes = out["codes"].cpu().numpy()
        scales = out["scales"].cpu().numpy()
        err = out["row_err"].cpu().numpy()
        loss = out["row_loss"].cpu().numpy()
        ok = np.array([r not in bad for r in range(m)])
        assert not codes[~ok].any() and np.all(scales[~ok] == 0x7F)
        assert np.all(np.isnan(err[~ok])) and np.all(np.isnan(loss[~ok]))
        assert np.all(np.isfinite(err[ok])) and np.all(np.isfinite(loss[ok]))
        # the other rows: the same bits as quantizing the finite rows alone, and the oracle's decisions
        alone = nvq.gptq_nvfp4_quantize(_to_dev(W[ok], dt), *args)
        assert np.array_equal(codes[ok], alone["codes"].cpu().numpy())
        assert np.array_equal(scales[ok], alone["scales"].cpu().numpy())
        assert np.array_equal(err[ok], alone["row_err"].cpu().numpy())
        ref = gptq.sweep(W[ok], U32, g, 16, dtype=np.float32)
        assert np.mean(codec.unpack_codes(codes[ok]) != ref["codes"]) <= 1e-3
        assert np.mean(scales[ok] != ref["scales"]) <= 1e-3
        # dequantization of a rejected row is NaN (both here and in the oracle's E4M3 decode)
        deq = nvq.nvfp4_dequantize(out["codes"], out["scales"], args[2]).cpu().numpy()
        assert np.all(np.isnan(deq[~ok])) and np.all(np.isfinite(deq[ok]))
        assert np.all(np.isnan(codec.dequantize(codes[~ok], scales[~ok], g)))
    # a non-finite global scale rejects every row; so does RTN with the flag
    for gbad in (float("nan"), float("inf"), 0.0):
        out = nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), args[0], args[1],
                                      _to_dev(np.array([gbad], dtype=np.float32)), 16,
                                      flags=nvq.FLAG_CHECK_FINITE)
        assert np.all(out["scales"].cpu().numpy() == 0x7F) and np.all(np.isnan(out["row_err"].cpu().numpy()))
    out = nvq.gptq_nvfp4_quantize(_to_dev(Wb), None, None, args[2], 4,
                                  flags=nvq.FLAG_RTN | nvq.FLAG_NO_ERR | nvq.FLAG_CHECK_FINITE)
    sc = out["scales"].cpu().numpy()
    assert np.all(sc[[3, 10, 11, 39]] == 0x7F) and not np.any(sc[[0, 1, 2, 20]] == 0x7F)
    ref = gptq.sweep(W[:3], np.eye(k), g, 4, dtype=np.float32)   # RTN scores compared in fp32, as on the GPU
    assert np.array_equal(sc[:3], ref["scales"])


def test_nan_weights_without_flag_are_deterministic(nvq):
    m, k = 64, 256
    W = synth.weights("attn_proj", m, k, 0.02)
    W[5, 17] = np.nan
    W[6, 0:16] = np.nan        # a whole block
    W[7, 100] = np.inf
    X = synth.activations("attn_proj", 600, k, massive=2)
    H = gptq.hessian(X)
    U, _ = gptq.hinv_factor(H)
    g = np.float32(codec.global_scale(np.nan_to_num(W, nan=0.0, posinf=0.0)))
    args = (_to_dev(U.astype(np.float32)), _to_dev(H.astype(np.float32)), _to_dev(np.array([g])), 16)
    for flags in (0, nvq.FLAG_FP64):
        runs = [nvq.gptq_nvfp4_quantize(_to_dev(W, torch.bfloat16), *args, flags=flags) for _ in range(3)]
        for r in runs[1:]:
            for key in ("codes", "scales"):
                assert torch.equal(r[key], runs[0][key]), (flags, key)
            for key in ("row_err", "row_loss"):
                a, b = r[key].cpu().numpy(), runs[0][key].cpu().numpy()
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (flags, key)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_factor_nonfinite_hessian_info(nvq, bad):
    k = 256
    X = synth.activations("small", 600, k, bf16=False)
    H = gptq.hessian(X).astype(np.float32)
    _, _, info = nvq.factor_hinv(_to_dev(H))
    assert int(info.item()) == 0
    H[10, 200] = bad         # upper triangle: read
    _, _, info = nvq.factor_hinv(_to_dev(H))
    assert int(info.item()) == -1
    H = gptq.hessian(X).astype(np.float32)
    H[200, 10] = bad         # lower triangle: never read
    _, _, info = nvq.factor_hinv(_to_dev(H))
    assert int(info.item()) == 0
    # a NaN token makes H non-finite through the Hessian itself
    Xn = X.copy()
    Xn[3, 7] = np.nan
    assert int(nvq.check_finite(_to_dev(Xn)).item()) == 4
    Hn = nvq.hessian_accumulate(_to_dev(Xn, torch.bfloat16))
    _, _, info = nvq.factor_hinv(Hn)
    assert int(info.item()) == -1


def test_dequantize_nan_scale_code(nvq):
    codes = np.random.default_rng(9).integers(0, 256, size=(3, 16), dtype=np.uint8)
    scales = np.array([[0x7F, 0x38], [0xFF, 0x01], [0x7E, 0x7F]], dtype=np.uint8)
    g = np.float32(0.5)
    ref = codec.dequantize(codes, scales, g)
    for dt in (torch.float32, torch.bfloat16):
        out = nvq.nvfp4_dequantize(_to_dev(codes, torch.uint8), _to_dev(scales, torch.uint8),
                                   _to_dev(np.array([g])), dt).float().cpu().numpy()
        assert np.array_equal(np.isnan(out), np.isnan(ref))
        fin = ~np.isnan(ref)
        expect = ref[fin] if dt == torch.float32 else torch.from_numpy(ref[fin]).to(torch.bfloat16).float().numpy()
        assert np.array_equal(out[fin], expect)


@pytest.mark.parametrize("m,k,n,cand,flags", [(1024, 1024, 16384, 16, 0), (520, 592, 3000, 8, 0),
                                               (300, 1040, 5000, 16, 4)])
def test_layer_bitwise_reproducible(nvq, m, k, n, cand, flags):
    W, X = synth.attn_proj_layer(m, k, n)
    Wd, Xd = synth.to_bf16_tensor(W).to(DEV), synth.to_bf16_tensor(X).to(DEV)
    runs = []
    for _ in range(2):
        r = nvq.quantize_layer(Wd, Xd, n_cand=cand, flags=flags)
        torch.cuda.synchronize()
        runs.append({key: r[key].clone() for key in ("H", "U", "lam", "info", "g", "codes", "scales",
                                                        "row_err", "row_loss")})
    a, b = runs
    assert int(a["info"].item()) == 0
    for key in a:
        x, y = a[key].cpu().numpy(), b[key].cpu().numpy()
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), key

"""Batched factors and quantization over several matrices (the experts of a
mixture-of-experts layer) give, for every matrix, the same bits as the
single-matrix calls, whatever number of matrices a pass covers (set by the
workspace size): every launch of a pass covers all of its matrices, and each
matrix's arithmetic is the same as when it is alone.  Parity of these calls
with the oracle is checked expert by expert in test_gpu_moe.py."""

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


def _experts(E, m, k, n):
    Hs, Ws = [], []
    for e in range(E):
        X = synth.to_bf16_values(synth.rng("moe", 70, e).standard_normal((n + 37 * e, k)).astype(np.float32)
                                 * synth.channel_scales("moe", k).astype(np.float32))
        Hs.append(gptq.hessian(X).astype(np.float32))
        Ws.append(synth.moe_expert_weights(e, m, k))
    H = torch.from_numpy(np.stack(Hs)).to(DEV)
    W = synth.to_bf16_tensor(np.stack(Ws).reshape(E * m, k)).reshape(E, m, k).to(DEV)
    return H, W


@pytest.mark.parametrize("k", [592, 1040])
def test_batched_factor_equals_single(nvq, k):
    E = 5
    H, _ = _experts(E, 16, k, 2 * k)
    one = nvq.lib.factor_hinv_workspace_size(k)
    single = [nvq.factor_hinv(H[e]) for e in range(E)]
    for per_pass in (1, 2, E):
        U, lam, info = nvq.factor_hinv_batched(H, max_ws_bytes=per_pass * one)
        torch.cuda.synchronize()
        assert torch.all(info == 0)
        for e in range(E):
            assert torch.equal(U[e], single[e][0]), (per_pass, e)
            assert torch.equal(lam[e:e + 1], single[e][1]), (per_pass, e)


@pytest.mark.parametrize("k", [592, 1040])
def test_batched_chol_factor_equals_single(nvq, k):
    E = 5
    H, _ = _experts(E, 16, k, 2 * k)
    one = nvq.lib.factor_chol_workspace_size(k)
    single = [nvq.factor_chol(H[e]) for e in range(E)]
    for per_pass in (1, 2, E):
        V, lam, info = nvq.factor_chol_batched(H, max_ws_bytes=per_pass * one)
        torch.cuda.synchronize()
        assert torch.all(info == 0)
        for e in range(E):
            assert torch.equal(V[e], single[e][0]), (per_pass, e)
            assert torch.equal(lam[e:e + 1], single[e][1]), (per_pass, e)


@pytest.mark.parametrize("flags,n_cand", [(0, 16), (4, 16), (8, 16), (1, 4), (16, 8), (2, 16)])
def test_batched_quantize_equals_single(nvq, flags, n_cand):
    E, m, k = 4, 40, 400
    H, W = _experts(E, m, k, 3 * k)
    U, _, info = nvq.factor_hinv_batched(H)
    assert torch.all(info == 0)
    g = torch.stack([nvq.nvfp4_global_scale(W[e]) for e in range(E)]).reshape(E)
    if flags & nvq.FLAG_CHECK_FINITE:
        W = W.clone()
        W[1, 7, 33] = float("nan")   # one rejected row in one expert
    Ua = None if flags & nvq.FLAG_RTN else U
    Ha = None if flags & nvq.FLAG_NO_ERR else H
    single = [nvq.gptq_nvfp4_quantize(W[e], None if Ua is None else Ua[e], None if Ha is None else Ha[e],
                                      g[e:e + 1], n_cand, flags) for e in range(E)]
    one = nvq.lib.gptq_nvfp4_workspace_size(m, k, flags)
    for per_pass in (1, 3, E):
        out = nvq.gptq_nvfp4_quantize_batched(W, Ua, Ha, g, n_cand, flags, max_ws_bytes=per_pass * one)
        torch.cuda.synchronize()
        for e in range(E):
            for key in ("codes", "scales", "row_err", "row_loss"):
                if out[key] is None:
                    continue
                a, b = out[key][e].cpu().numpy(), single[e][key].cpu().numpy()
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (per_pass, e, key)

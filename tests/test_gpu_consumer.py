"""GPU parity of the NVFP4 weight-only GEMM (nvfp4_gemm) against the consumer
oracle: |Y - Y_fp64| within the fp32 accumulation bound, for ragged shapes,
bf16 and fp32 outputs, strided inputs, and a layer quantized end to end by the
library."""

import numpy as np
import pytest
import torch

import synth
from oracle import codec, consumer, gptq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_nvfp4_weight_amd as m
    return m


def _bound(X, packed, scales, g):
    # products are exact; fp32 accumulation over k/16 MFMA steps, plus g applied once
    deq = np.abs(codec.dequantize(packed, scales, g).astype(np.float64))
    k = X.shape[1]
    return (np.abs(X.astype(np.float64)) @ deq.T) * ((k / 16 + 16) * 2.0 ** -23)


def _layer(m, k, T, seed):
    W = synth.weights("attn_proj", m, k, 0.02, outlier_frac=0.01)
    g = codec.global_scale(W)
    r = gptq.rtn(W, g, 4)
    packed, scales = codec.pack_codes(r["codes"]), r["scales"]
    X = synth.to_bf16_values(np.random.default_rng(seed).standard_normal((T, k)).astype(np.float32))
    return X, packed, scales, g


# Cases 2-6 (at most 32 tokens, k a multiple of 128) take the decode-sized
# kernel: one and two 16-token groups, ragged T and m, one to 32 chunks of
# 128 k.  The last three cases have a 256 x 256 tile per CU: the first two
# take the many-token kernel (k a multiple of 32), aligned, and ragged in T
# and m with an odd number of 32-deep k steps (k = 544); k = 528 takes the
# general kernel, as do the rest.
@pytest.mark.parametrize("T,m,k", [(1, 64, 16), (1, 64, 128), (16, 1024, 4096), (5, 100, 1024), (17, 130, 384),
                                   (32, 48, 2048), (37, 100, 48), (300, 256, 1024), (129, 130, 2064),
                                   (512, 512, 4096), (4096, 4096, 512), (4000, 4100, 544), (4000, 4100, 528)])
def test_gemm_matches_oracle(nvq, T, m, k):
    X, packed, scales, g = _layer(m, k, T, seed=T)
    Xd = synth.to_bf16_tensor(X).to(DEV)
    args = (torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
            torch.tensor([g], dtype=torch.float32, device=DEV))
    ref = consumer.weight_only_matmul(X, packed, scales, g)
    bnd = _bound(X, packed, scales, g)
    Y = nvq.nvfp4_gemm(Xd, *args).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Y - ref) <= bnd + 1e-30)
    Yb = nvq.nvfp4_gemm(Xd, *args, out_dtype=torch.bfloat16).float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Yb - ref) <= bnd + np.abs(ref) * 2.0 ** -8 + 1e-30)


def test_gemm_strided_activations(nvq):
    T, m, k = 200, 128, 512
    X, packed, scales, g = _layer(m, k, T, seed=5)
    wide = torch.zeros(T, k + 64, dtype=torch.bfloat16)
    wide[:, :k] = synth.to_bf16_tensor(X)
    Xd = wide.to(DEV)[:, :k]
    Y = nvq.nvfp4_gemm(Xd, torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
                       torch.tensor([g], dtype=torch.float32, device=DEV)).cpu().numpy()
    ref = consumer.weight_only_matmul(X, packed, scales, g)
    assert np.all(np.abs(Y - ref) <= _bound(X, packed, scales, g) + 1e-30)


def test_gemm_decode_strided_activations(nvq):
    # The decode-sized kernel (at most 32 tokens, k a multiple of 128) with
    # activation rows padded (ldx > k), ragged m, five 128-deep chunks.
    T, m, k = 9, 96 + 7, 640
    X, packed, scales, g = _layer(m, k, T, seed=7)
    wide = torch.zeros(T, k + 64, dtype=torch.bfloat16)
    wide[:, :k] = synth.to_bf16_tensor(X)
    Xd = wide.to(DEV)[:, :k]
    args = (torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
            torch.tensor([g], dtype=torch.float32, device=DEV))
    ref = consumer.weight_only_matmul(X, packed, scales, g)
    Y = nvq.nvfp4_gemm(Xd, *args).cpu().numpy()
    assert np.all(np.abs(Y - ref) <= _bound(X, packed, scales, g) + 1e-30)
    Yb = nvq.nvfp4_gemm(Xd, *args, out_dtype=torch.bfloat16).float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Yb - ref) <= _bound(X, packed, scales, g) + np.abs(ref) * 2.0 ** -8 + 1e-30)


@pytest.mark.parametrize("T", [64, 8])
def test_gemm_after_library_quantization(nvq, T):
    # quantize a layer with the whole library path, then use it (8 tokens: the decode-sized kernel)
    m, k, n = 256, 512, 4096
    W, Xc = synth.attn_proj_layer(m, k, n)
    res = nvq.quantize_layer(synth.to_bf16_tensor(W).to(DEV), synth.to_bf16_tensor(Xc).to(DEV), n_cand=16)
    X = Xc[:T]
    Y = nvq.nvfp4_gemm(synth.to_bf16_tensor(X).to(DEV), res["codes"], res["scales"], res["g"]).cpu().numpy()
    packed, scales, g = res["codes"].cpu().numpy(), res["scales"].cpu().numpy(), np.float32(res["g"].item())
    ref = consumer.weight_only_matmul(X, packed, scales, g)
    assert np.all(np.abs(Y - ref) <= _bound(X, packed, scales, g) + 1e-30)


def test_gemm_many_tokens_strided(nvq):
    # The many-token kernel with activation rows padded (ldx > k).
    T, m, k = 4096, 4096, 256
    X, packed, scales, g = _layer(m, k, T, seed=11)
    wide = torch.zeros(T, k + 40, dtype=torch.bfloat16)
    wide[:, :k] = synth.to_bf16_tensor(X)
    Xd = wide.to(DEV)[:, :k]
    Y = nvq.nvfp4_gemm(Xd, torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
                       torch.tensor([g], dtype=torch.float32, device=DEV)).cpu().numpy()
    ref = consumer.weight_only_matmul(X, packed, scales, g)
    assert np.all(np.abs(Y - ref) <= _bound(X, packed, scales, g) + 1e-30)

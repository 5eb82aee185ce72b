"""Pins of the consumer oracle (Y = X dequant(W)^T) against closed forms."""

import numpy as np

from oracle import codec, consumer, gptq


def test_unit_weights_give_row_sums():
    # every code of magnitude 1 (index 2) under scale 1.0 (E4M3 0x38), g = 1:
    # the weights are all 1, so each output is the row sum of X
    rng = np.random.default_rng(1)
    X = rng.normal(size=(5, 64))
    codes = np.full((3, 64), 2, dtype=np.uint8)
    codes[1] |= 8                               # a row of -1
    packed = codec.pack_codes(codes)
    scales = np.full((3, 4), 0x38, dtype=np.uint8)
    Y = consumer.weight_only_matmul(X, packed, scales, np.float32(1.0))
    assert np.allclose(Y[:, 0], X.sum(1), rtol=1e-14) and np.allclose(Y[:, 1], -X.sum(1), rtol=1e-14)


def test_grid_weights_round_trip():
    # weights on the NVFP4 grid (e2m1 value x a block scale x g) are reproduced
    # exactly by round-to-nearest, so the consumer returns X W^T
    rng = np.random.default_rng(2)
    m, k = 8, 96
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    g = np.float32(0.0625)
    sc = rng.integers(0x30, 0x48, size=(m, k // 16))
    W = (mags[rng.integers(0, 8, size=(m, k))] * rng.choice([-1, 1], size=(m, k))
         * np.repeat(codec.e4m3_decode(sc), 16, axis=1) * np.float64(g)).astype(np.float32)
    W[:, ::16] = np.repeat(6.0 * codec.e4m3_decode(sc), 1, axis=1) * np.float64(g)   # block absmax sets the scale
    res = gptq.rtn(W, g, 1)
    deq = codec.dequantize(codec.pack_codes(res["codes"]), res["scales"], g)
    assert np.array_equal(deq, W)
    X = rng.normal(size=(7, k))
    Y = consumer.weight_only_matmul(X, codec.pack_codes(res["codes"]), res["scales"], g)
    assert np.allclose(Y, X @ W.astype(np.float64).T, rtol=1e-13, atol=1e-15)

"""Consumer of the exported NVFP4 layer (oracle; test infrastructure only).

Source: "Replay the Curvature" (arXiv 2609.36654), Abstract: the quantized
layer is exported in NVFP4 for use.  Its use here is the weight-only product
with bf16 activations, Y = X dequant(W)^T, where dequant is the codec's
(oracle.codec.dequantize: fl32(fl32(e2m1 * e4m3) * g) per element).  The
product is taken in fp64 with a library matmul; the dequantization is pinned
by the codec's tests.
"""

import numpy as np

from . import codec


def weight_only_matmul(X, packed, scales, g):
    """Y [T, m] = X [T, k] dequant(W)^T in fp64, W given by packed codes [m, k/2], scales [m, k/16], g."""
    deq = codec.dequantize(packed, scales, g).astype(np.float64)
    return np.asarray(X, dtype=np.float64) @ deq.T

"""Seeded synthetic layers and calibration activations.

Shared by the tests, the benchmark and the oracle's callers: it only draws
random numbers and rounds them to the storage dtype; it holds none of the
quantization method's arithmetic.

Every array is reproducible from (seed, layer id, stream id, chunk id) via
numpy.random.default_rng; large arrays are drawn in row chunks on a thread
pool.  bf16 values are the round-to-nearest-even bf16 of the fp32 draws
(torch's CPU cast), returned as fp32 numpy arrays holding exactly those
values (and, where needed, as torch.bfloat16 tensors).

Workload recipes (weights W [d_out, d_in], activations X [tokens, d_in]):
  small      W fp32 ~ N(0, 0.02^2), 4 distinct random input columns x20;
             X fp32 rows z * s, z ~ N(0, 1), per-channel s ~ LogNormal(0, 1).
  attn_proj  W bf16 ~ N(0, 0.02^2) with 0.1% of entries replaced by
             0.02 * Student-t(3); X bf16 rows z * s with 8 random channels of
             s multiplied by 100 (massive activations).
  mlp        W bf16 ~ N(0, 0.015^2); X as small, in bf16.
  sparse     W bf16 ~ N(0, 0.01^2) with 0.05% Student-t(3) outliers;
             X bf16 = |z| * Bernoulli(0.4) * s (60% exact zeros).
  moe        per expert W bf16 ~ N(0, 0.02^2); X as small, in bf16; every
             token routed to top_k distinct experts drawn without replacement
             with probability proportional to rank^-1.1 (Zipf popularity),
             by the Gumbel top-k trick.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

SEED = 0
_CHUNK = 8192

LAYERS = {"small": 1, "attn_proj": 2, "mlp": 3, "sparse": 4, "moe": 5}


def rng(layer, stream, chunk=None):
    key = [SEED, LAYERS.get(layer, layer) if isinstance(layer, str) else layer, stream]
    if chunk is not None:
        key.append(chunk)
    return np.random.default_rng(key)


def to_bf16_values(x):
    """fp32 array -> fp32 array holding the RNE bf16 rounding of each value."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def to_bf16_tensor(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def channel_scales(layer, k, massive=0):
    r = rng(layer, 10)
    s = r.lognormal(0.0, 1.0, size=k).astype(np.float64)
    if massive:
        idx = r.choice(k, size=massive, replace=False)
        s[idx] *= 100.0
    return s


def _x_chunk(layer, c, rows, k, s, kind):
    r = rng(layer, 11, c)
    z = r.standard_normal((rows, k), dtype=np.float32)
    if kind == "sparse":
        keep = r.random((rows, k), dtype=np.float32) < 0.4
        z = np.abs(z) * keep
    return (z * s.astype(np.float32)[None, :]).astype(np.float32)


def activations(layer, n, k, massive=0, kind="dense", bf16=True, out=None):
    """X [n, k] drawn chunk by chunk (chunk c of 8192 rows uses rng(layer, 11, c)).

    Returns an fp32 numpy array (bf16-rounded values when bf16=True).  If out
    is given (a torch.bfloat16 CPU tensor [n, k]) the bf16 values are written
    there instead and out is returned.
    """
    s = channel_scales(layer, k, massive)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    res = None if out is not None else np.empty((n, k), dtype=np.float32)

    def work(c):
        r0 = c * _CHUNK
        rows = min(_CHUNK, n - r0)
        x = _x_chunk(layer, c, rows, k, s, kind)
        if out is not None:
            out[r0:r0 + rows] = to_bf16_tensor(x)
        else:
            res[r0:r0 + rows] = to_bf16_values(x) if bf16 else x

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nchunks)))
    return out if out is not None else res


def weights(layer, m, k, std, outlier_frac=0.0, outlier_cols=0, bf16=True):
    """W [m, k]: N(0, std^2); optional Student-t(3) outliers and x20 input columns."""
    r = rng(layer, 20)
    W = (r.standard_normal((m, k)) * std).astype(np.float64)
    if outlier_frac:
        cnt = int(round(outlier_frac * m * k))
        flat = r.choice(m * k, size=cnt, replace=False)
        W.reshape(-1)[flat] = std * r.standard_t(3, size=cnt)
    if outlier_cols:
        cols = r.choice(k, size=outlier_cols, replace=False)
        W[:, cols] *= 20.0
    W = W.astype(np.float32)
    return to_bf16_values(W) if bf16 else W


# ---- named workloads ---------------------------------------------------------

def small_layer(m=256, k=256, n=2048):
    """Single linear layer, fp32: the oracle-sized case (8 candidates per block)."""
    W = weights("small", m, k, 0.02, outlier_cols=4, bf16=False)
    X = activations("small", n, k, bf16=False)
    return W, X


def attn_proj_layer(m=4096, k=4096, n=262144, x_out=None):
    """Attention-projection-shaped layer, bf16, 16 candidates per block.

    Full size: 4096 x 4096 weights, 262,144 tokens (128 sequences x 2048).
    Smaller m, k, n give the same recipe at test sizes.
    """
    W = weights("attn_proj", m, k, 0.02, outlier_frac=0.001)
    X = activations("attn_proj", n, k, massive=min(8, k), out=x_out)
    return W, X


def mlp_layer(m, k, n):
    W = weights("mlp", m, k, 0.015)
    X = activations("mlp", n, k)
    return W, X


def mlp_block_weights(d=4096, f=14336):
    """Gate, up [f, d] and down [d, f] weights of one MLP block (bf16 values, N(0, 0.015^2))."""
    Wg = weights("mlp", f, d, 0.015)
    Wu = to_bf16_values(rng("mlp", 21).standard_normal((f, d)).astype(np.float32) * np.float32(0.015))
    Wd = weights("mlp", d, f, 0.015)   # the same recipe, a [d x f] draw
    return Wg, Wu, Wd


def mlp_down_activations(Xd, Wg, Wu, chunk=8192):
    """The down projection's inputs bf16(SiLU(X W_gate^T) * (X W_up^T)) from the block's own bf16
    activations Xd (a torch tensor on any device; fp32 products, chunks of tokens).  A model forward
    pass that makes inputs, not part of the quantization method."""
    import torch
    dev = Xd.device
    Wg_t = torch.from_numpy(Wg).to(dev).t().contiguous()
    Wu_t = torch.from_numpy(Wu).to(dev).t().contiguous()
    out = torch.empty(Xd.shape[0], Wg.shape[0], dtype=torch.bfloat16, device=dev)
    for c0 in range(0, Xd.shape[0], chunk):
        xc = Xd[c0:c0 + chunk].float()
        out[c0:c0 + chunk] = (torch.nn.functional.silu(xc @ Wg_t) * (xc @ Wu_t)).to(torch.bfloat16)
    return out


def sparse_layer(m, k, n):
    W = weights("sparse", m, k, 0.01, outlier_frac=0.0005)
    X = activations("sparse", n, k, kind="sparse")
    return W, X


def moe_routing(n_tokens, n_experts, top_k, zipf=1.1, layer="moe"):
    """Token -> expert assignments, grouped by expert.

    Expert e has popularity rank perm[e] + 1 (a seeded permutation) and
    weight (rank)^-zipf.  Each token draws top_k distinct experts without
    replacement with probability proportional to the weights: the top_k
    largest of log(weight) + Gumbel noise.  Returns (tok_idx int32 [n*top_k]
    sorted by expert then token, grp_off int64 [n_experts + 1]).
    """
    r = rng(layer, 30)
    rank = r.permutation(n_experts) + 1
    logw = (-zipf * np.log(rank.astype(np.float64))).astype(np.float32)
    experts = np.empty((n_tokens, top_k), dtype=np.int32)
    for c0 in range(0, n_tokens, _CHUNK):
        rows = min(_CHUNK, n_tokens - c0)
        gum = rng(layer, 31, c0 // _CHUNK).gumbel(size=(rows, n_experts)).astype(np.float32)
        experts[c0:c0 + rows] = np.argpartition(-(logw[None, :] + gum), top_k - 1, axis=1)[:, :top_k]
    tok = np.repeat(np.arange(n_tokens, dtype=np.int64), top_k)
    ex = experts.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, ex))
    counts = np.bincount(ex, minlength=n_experts)
    grp_off = np.zeros(n_experts + 1, dtype=np.int64)
    grp_off[1:] = np.cumsum(counts)
    return tok[order].astype(np.int32), grp_off


def moe_expert_weights(expert, m, k, std=0.02, layer="moe"):
    """W [m, k] of one expert (gate and up stacked along m), bf16 values."""
    r = rng(layer, 40, expert)
    W = (r.standard_normal((m, k)) * std).astype(np.float32)
    return to_bf16_values(W)

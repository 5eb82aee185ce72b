"""GPU parity of the Hessian over host-resident activations (chunks streamed to
the device, copies overlapped with the accumulation): the result must equal,
bit for bit, hessian_accumulate called on the same chunks in order, for pinned
and pageable torch tensors, a NumPy memory map of a file (bf16 bits) and fp32
arrays, strided rows and ragged last chunks; and it must lie within the fp32
summation bound of the fp64 oracle."""

import numpy as np
import pytest
import torch

import synth
from oracle import gptq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_nvfp4_weight_amd as m
    return m


def _chunked_reference(nvq, Xd, chunk, H0):
    H = H0.clone()
    for t0 in range(0, Xd.shape[0], chunk):
        nvq.hessian_accumulate(Xd[t0:t0 + chunk].contiguous(), H)
    return H


@pytest.mark.parametrize("n,k,chunk", [(5000, 256, 1024), (3000, 1024, 4096), (10000, 512, 3333), (100, 64, 7)])
def test_streamed_equals_chunked_calls(nvq, n, k, chunk):
    X = torch.empty(n, k, dtype=torch.bfloat16)
    synth.activations("attn_proj", n, k, massive=2, out=X)
    H0 = torch.randn(k, k, device=DEV, generator=torch.Generator(device=DEV).manual_seed(3))
    H0 = H0 + H0.t()
    ref = _chunked_reference(nvq, X.to(DEV), chunk, H0)
    for Xh, staging in ((X, True), (X, False), (X.pin_memory(), True), (X.pin_memory(), False)):
        H = nvq.hessian_accumulate_host(Xh, H0.clone(), chunk=chunk, staging=staging)
        torch.cuda.synchronize()
        assert torch.equal(H, ref), (Xh.is_pinned(), staging)


def test_streamed_from_memory_mapped_file(nvq, tmp_path):
    n, k, chunk = 6000, 384, 2048
    X = torch.empty(n, k, dtype=torch.bfloat16)
    synth.activations("attn_proj", n, k, massive=2, out=X)
    path = tmp_path / "x.bin"
    mm = np.memmap(path, dtype=np.uint16, mode="w+", shape=(n, k))
    mm[:] = X.view(torch.int16).numpy().view(np.uint16)
    mm.flush()
    del mm
    Xmap = np.memmap(path, dtype=np.uint16, mode="r", shape=(n, k))
    H = nvq.hessian_accumulate_host(Xmap, chunk=chunk)
    ref = _chunked_reference(nvq, X.to(DEV), chunk, torch.zeros(k, k, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(H, ref)
    # within the fp32 summation bound of the fp64 oracle
    Xf = X.float().numpy().astype(np.float64)
    Href = gptq.hessian(Xf)
    bound = np.abs(Xf).T @ np.abs(Xf) * ((n / 16 + 64) * 2.0 ** -23)
    assert np.all(np.abs(H.cpu().numpy() - Href) <= bound + 1e-30)


def test_streamed_strided_rows_and_fp32(nvq):
    n, k, chunk = 4000, 256, 1500
    Xw = torch.empty(n, k + 64, dtype=torch.bfloat16)
    synth.activations("attn_proj", n, k + 64, massive=2, out=Xw)
    X = Xw[:, :k]                      # rows of ldx = k + 64
    H = nvq.hessian_accumulate_host(X, chunk=chunk)
    ref = _chunked_reference(nvq, X.contiguous().to(DEV), chunk, torch.zeros(k, k, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(H, ref)
    Xf = X.float().contiguous().numpy()
    H32 = nvq.hessian_accumulate_host(Xf, chunk=chunk)
    ref32 = _chunked_reference(nvq, torch.from_numpy(Xf).to(DEV), chunk, torch.zeros(k, k, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(H32, ref32)


def test_streamed_no_tokens_leaves_h(nvq):
    H0 = torch.full((64, 64), 3.0, device=DEV)
    H = nvq.hessian_accumulate_host(torch.empty(0, 64, dtype=torch.bfloat16), H0.clone(), chunk=16)
    assert torch.equal(H, H0)

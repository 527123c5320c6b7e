"""The matrix-core rate probe (libbsg_probe.so) does the MFMAs it is credited with:
with every operand 1.0 and every scale 2^0, each of a thread's 128 accumulators ends
at exactly 2 * iters * Kmma, so each thread's sum is 256 * iters * Kmma; with random
operands the sums are finite and repeat bit for bit from call to call."""
import pytest
import torch

from block_scaled_precision_05_amd import probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4"])
def test_probe_counts_its_mfmas(kind):
    dev = torch.device("cuda:0")
    wg, iters = 3, 5
    out = torch.full((wg * probe.THREADS,), -1.0, dtype=torch.float32, device=dev)
    probe.mfma(kind, 0, wg, iters, out)
    torch.cuda.synchronize()
    want = 128 * 2 * iters * probe.MMA_K[kind]
    assert torch.equal(out.cpu(), torch.full((wg * probe.THREADS,), float(want)))


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4"])
def test_probe_random_operands_finite_and_repeatable(kind):
    dev = torch.device("cuda:0")
    wg, iters = 4, 50
    a = torch.empty(wg * probe.THREADS, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    probe.mfma(kind, 12345, wg, iters, a)
    probe.mfma(kind, 12345, wg, iters, b)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)
    # distinct threads hold distinct draws
    assert a.unique().numel() > a.numel() // 2

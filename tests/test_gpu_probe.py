"""The measurement helpers on the GPU: the MFMA probe runs and its output
is the sum of products of the given operands (zero operands give zeros,
finite random operands give finite sums); the device query reports CUs and
a clock."""
import pytest

from gpu_helpers import C, torch

pytestmark = pytest.mark.gpu


def test_probe_runs_and_device_info():
    cus, khz = C.cpattn_device_info()
    assert cus > 0 and khz > 0
    out = torch.full((4 * 512,), float("nan"), device="cuda")
    zeros = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    C.cpattn_probe_mfma(zeros, out, 4, 3)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    ops = (torch.randn(4096, generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    C.cpattn_probe_mfma(ops, out, 4, 3)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and out.abs().sum() > 0

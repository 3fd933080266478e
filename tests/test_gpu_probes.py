"""The measurement probes do what their declarations say: the copy copies,
the read's per-thread folds cover every word once, the MFMA loops produce
finite sums and a plausible clock reading.  They feed the measured peaks the
roofline fractions are reported against."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def test_probe_copy_and_read_cover_every_word():
    n = (48 << 20) + 16 * 37  # not a multiple of the grid's stride
    g = torch.Generator(device="cpu").manual_seed(5)
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, generator=g).to(DEV)
    dst = torch.zeros_like(src)
    print(f"[probe] copy/read {n} bytes", flush=True)
    moe.moe_probe_copy(src, dst)
    out = torch.zeros(4096 * 256, dtype=torch.int32, device=DEV)
    moe.moe_probe_read(src, out)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # each thread xors the words it read into its out word: the xor of all
    # out words is the xor of every word of src exactly when each is read once
    fold = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert fold == want


@pytest.mark.parametrize("toggle", [False, True])
def test_probe_mfma_clock(toggle):
    blocks, iters = 512, 400
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=DEV)
    clk = torch.zeros(blocks * 4 * 2, dtype=torch.int64, device=DEV)
    print(f"[probe] mfma toggle={toggle}", flush=True)
    moe.moe_probe_mfma_clock(iters, blocks, toggle, out, clk)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    c = clk.view(-1, 2).double()
    assert (c > 0).all()
    ghz = (c[:, 0] / c[:, 1] * 0.1)
    print(f"[probe] toggle={toggle}: clock {ghz.min().item():.3f}..{ghz.max().item():.3f} GHz", flush=True)
    assert 0.3 < ghz.mean().item() < 3.5
    # the same loop without the clock output, constant operands: same sums
    if not toggle:
        out2 = torch.empty_like(out)
        moe.moe_probe_mfma(iters, blocks, out2)
        torch.cuda.synchronize()
        assert torch.equal(out, out2)

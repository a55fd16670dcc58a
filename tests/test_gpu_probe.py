"""The matrix-core rate probe (attn_probe_mfma) computes what it claims: with
every operand fragment equal to 0.5, each 32x32x16 MFMA adds 16 * 0.25 = 4 to
every accumulator element, so after `iters` MFMAs per wave (iters / 4 per
chain, four chains) each lane's output, the sum of its 4 x 16 accumulator
elements, is exactly 64 * iters.  On random operands the output is finite and
repeatable, and the same at every loop placement."""
import pytest
import torch

import tiled_online_softmax_attention_amd as attn
from parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("blocks,iters,placement", [(1, 32, 0), (8, 64, 7), (300, 256, 15)])
def test_probe_constant_operands_closed_form(blocks, iters, placement):
    log("probe constant blocks=%d iters=%d placement=%d" % (blocks, iters, placement))
    frag = torch.full((16 * 8,), 0.5, dtype=torch.bfloat16, device=DEV)
    out, flops = attn.probe_mfma(frag, iters, blocks, placement=placement)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 32768
    assert out.numel() == blocks * 256
    assert torch.all(out == 64.0 * iters)


def test_probe_random_operands_repeatable():
    log("probe random")
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    frag = torch.randn(1024 * 8, generator=g, device=DEV).to(torch.bfloat16)
    a, _ = attn.probe_mfma(frag, 64, 16)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert float(a.abs().max()) > 0
    # every placement runs the same instructions on the same data
    for placement in range(attn.PROBE_PLACEMENTS):
        b, _ = attn.probe_mfma(frag, 64, 16, placement=placement)
        torch.cuda.synchronize()
        assert torch.equal(a, b), placement

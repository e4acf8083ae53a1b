"""The FP8 MFMA probe (a measurement aid): it runs, reports the flops it performs and
leaves finite sums (operands 1.0 and 0.5, so the accumulators stay exact)."""
import pytest
import torch

from combine_top_gate_amd import binding

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_counts_flops(lib):
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    flops = binding.mfma_fp8_probe(sink, 8, 3)
    torch.cuda.synchronize()
    # 8 workgroups x 4 waves x 3 iterations x 4 chains x (2 x 16 x 16 x 128)
    assert flops == 8 * 4 * 3 * 4 * 65536
    s = sink.cpu()
    assert torch.isfinite(s).all() and (s > 0).all()

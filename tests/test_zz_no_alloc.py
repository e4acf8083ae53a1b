"""moe_gate_noalloc (the fused gate with its partial sums in the library's fixed scratch
array) against moe_gate (caller workspace): same kernels, so ids, weights and logits must
agree bit for bit, on two calls in a row, the second smaller, and after a call of the
workspace form in between (the scratch keeps the last call's contents)."""
import pytest
import torch

from combine_top_gate_amd import binding, synth

pytestmark = pytest.mark.gpu


def _bits(a):
    return torch.from_numpy(a.view("int16")).cuda()


@pytest.mark.parametrize("shapes", [[(256, 7168, 256, 8), (40, 7168, 256, 8)],
                                    [(4096, 7168, 256, 8), (1, 2048, 64, 6)]])
def test_noalloc_gate_matches_workspace_gate(lib, shapes):
    for i, (T, H, E, k) in enumerate(shapes):
        print(f"[gpu case] noalloc gate call {i}: T={T} H={H} E={E} k={k}", flush=True)
        ri = synth.make_router_inputs(T, H, E, seed=300 + 17 * i + T)
        x, wr = _bits(ri.x_bits), _bits(ri.wr_bits)
        ids, w, lg = binding.gate(x, wr, k, want_logits=True)
        lg2 = torch.full((T, E), float("nan"), device="cuda")
        ids2, w2, _ = binding.gate_noalloc(x, wr, k, logits=lg2)
        ids3, w3, _ = binding.gate_noalloc(x, wr, k)  # without the logits output
        torch.cuda.synchronize()
        assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(lg, lg2)
        assert torch.equal(ids, ids3) and torch.equal(w, w3)

"""The layer captured into a HIP graph and replayed (the decode step as one submitted graph,
GC-MoE explainer, "Three-Node CUDA Graph and token-ring Handshake").

Each case captures one moe_layer call on torch's capture stream, then replays the graph
several times.  Before each replay a new activation set (x, x scales, ids, gate weights)
is copied into the captured buffers, alternating between two seeds, and the replay's
output must equal, bit for bit, an eager call on the same inputs; eager layer calls on the
same context run between the replays.  The SENTINEL schedule and timed calls must refuse
capture.
"""
import numpy as np
import pytest
import torch

from combine_top_gate_amd import binding, synth

pytestmark = pytest.mark.gpu


def _load_acts(d, src):
    """Copy src's activations (a DeviceInputs of the same shapes) into d's buffers."""
    for s in range(len(d.x)):
        d.x[s].copy_(src.x[s])
        if d.x_scale is not None:
            d.x_scale[s].copy_(src.x_scale[s])
    d.ids.copy_(src.ids)
    d.topk_w.copy_(src.topk_w)


CASES = [
    # name, overrides, options
    ("decode128_fp8", {}, {}),
    ("decode128_fp8", dict(S=3, T_s=9, H=384, I=256, E=6, k=3), {binding.MOE_OPT_PERSISTENT_GEMM: 1}),
    ("decode256_mxfp4_shared", dict(S=3, T_s=7, H=384, I=256, E=5, k=2, shared_I=128), {}),
    ("decode256_w4a16_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=256), {}),
    ("prefill4096_zipf_fp8", dict(S=2, T_s=96, H=512, I=256, E=4, k=2), {binding.MOE_OPT_TILED_GEMM: 1}),
    ("tiny_f32", {}, {}),
    # the combine in GEMM2's epilogue: its counters are reset by the items, not by a memset
    ("decode128_fp8", dict(S=3, T_s=9, H=384, I=256, E=6, k=3), {binding.MOE_OPT_FUSED_COMBINE: 1}),
    ("decode256_mxfp4_shared", dict(S=3, T_s=7, H=384, I=256, E=5, k=2, shared_I=128),
     {binding.MOE_OPT_FUSED_COMBINE: 1}),
]


@pytest.mark.parametrize("name,over,opts", CASES)
def test_layer_graph_replays_match_eager(name, over, opts):
    print(f"[gpu case] graph {name} {over} {opts}", flush=True)
    inp_a = synth.make_inputs(name, seed=91, **over)
    inp_b = synth.make_inputs(name, seed=92, **over)
    moe = binding.Moe.for_inputs(inp_a)
    for o, v in opts.items():
        moe.set_option(o, v)
    d = binding.DeviceInputs(inp_a)
    src = [binding.DeviceInputs(inp_a), binding.DeviceInputs(inp_b)]
    if inp_a.weight != "f32":
        moe.pack(d)
    # eager references: d's weights with each activation set
    refs = []
    for s in src:
        _load_acts(d, s)
        moe.run(d)
        torch.cuda.synchronize()
        refs.append(d.out.clone())
    assert not torch.equal(refs[0], refs[1])
    _load_acts(d, src[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.run(d)
    torch.cuda.synchronize()
    for rep in range(6):
        which = (rep + 1) % 2
        _load_acts(d, src[which])
        d.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, refs[which]), f"replay {rep}"
        # eager work on the same context between replays
        _load_acts(d, src[1 - which])
        moe.run(d)
        torch.cuda.synchronize()
        assert torch.equal(d.out, refs[1 - which]), f"eager call after replay {rep}"
    assert moe.device_error() == 0


def test_sentinel_and_timed_calls_refuse_capture():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=4, H=256, I=128, E=4, k=2, seed=93)
    for sched, timed, what in ((binding.MOE_SCHED_SENTINEL, False, "SENTINEL"),
                               (binding.MOE_SCHED_FENCE, True, "timed")):
        moe = binding.Moe.for_inputs(inp, sched=sched)
        d = binding.DeviceInputs(inp)
        moe.run(d)
        torch.cuda.synchronize()
        if timed:
            moe.set_timing(4)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            d.out.zero_()  # the graph holds one node of its own
            with pytest.raises(binding.MoeError, match=what):
                moe.run(d)
        torch.cuda.synchronize()
        # the context still works eagerly
        if timed:
            moe.set_timing(0)
        moe.run(d)
        torch.cuda.synchronize()
        assert moe.device_error() == 0
        assert np.isfinite(d.out.float().cpu().numpy()).all()

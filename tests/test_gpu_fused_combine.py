"""The combine formed in the decode GEMM2's epilogue (MOE_OPT_FUSED_COMBINE) through the
C-ABI: against the oracle, and bit for bit against the combine kernel.

The fused form is the pages' contrast to their split design: one persistent kernel that
also does the combine ("GC-MoE: Decoupling MoE Communication and Computation with CUDA
Green Contexts", "Why Expert Parallelism Is Inefficient in MoE Decoding").  Here the
GEMM2 work item that brings the last contribution of a token to a block of 256 output
columns sums that block, with the combine kernel's arithmetic (fp32 FMAs in slot order,
the shared row last), so both forms must give the same bits.  Its per-token counters are
never cleared between calls (the item that completes a token resets them), so the soak
changes inputs and batch size every call, poisons the workspace and the output before
each, and compares every call.
"""
import numpy as np
import pytest
import torch

from combine_top_gate_amd import binding, synth
from parity import check_layer, gpu_state, out_np, run

pytestmark = pytest.mark.gpu

FC = binding.MOE_OPT_FUSED_COMBINE


def _check(moe, inp, d):
    check_layer(inp, gpu_state(moe, inp), out_np(inp, d.out))
    assert moe.device_error() == 0


def _same_as_kernel(moe, d, fused_out):
    """The same context and inputs with the combine kernel give the same bits."""
    moe.set_option(FC, 0)
    d.out.fill_(float("nan"))
    moe.run(d)
    torch.cuda.synchronize()
    moe.set_option(FC, 1)
    assert torch.equal(fused_out, d.out)


SMALL = [
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=301), True),
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=301), False),
    # the most slots per token (16: two rounds of eight loads), ragged last column block
    ("decode128_fp8", dict(S=2, T_s=5, H=384, I=128, E=20, k=16, seed=302), True),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=303), True),
    ("decode256_mxfp4_shared", dict(S=3, T_s=4, H=256, I=128, E=6, k=1, shared_I=128, seed=304), False),
    ("decode256_w4a16_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=305), True),
    ("decode256_w4a16_shared", dict(S=4, T_s=20, H=512, I=384, E=3, k=3, shared_I=0, seed=306), True),
    # many rows per expert: several 256-row rounds of counting in one item
    ("decode128_fp8", dict(S=8, T_s=40, H=512, I=256, E=4, k=2, seed=307), True),
]


@pytest.mark.parametrize("name,over,packed", SMALL)
def test_fused_combine_matches_oracle_and_kernel(name, over, packed):
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp, packed=packed, opts={FC: 1})
    _check(moe, inp, d)
    _same_as_kernel(moe, d, d.out.clone())


PERSISTENT = [
    ("decode128_fp8", dict(S=4, T_s=9, H=512, I=256, E=8, k=4, seed=311), 0),
    ("decode128_fp8", dict(S=4, T_s=9, H=512, I=256, E=8, k=4, seed=311), 2),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=312), 0),
    # a Zipf-skewed prefill shape on the streaming kernels (the tiled kernels off)
    ("prefill4096_zipf_fp8", dict(S=8, T_s=64, H=1024, I=512, E=16, k=4, seed=313), 0),
    ("decode128_fp8", None, 0),
]


@pytest.mark.parametrize("name,over,queue", PERSISTENT)
def test_fused_combine_in_persistent_kernel(name, over, queue):
    """N3 whole: GEMM1 and GEMM2 in one persistent kernel (per-expert release counters) with
    the combine in the GEMM2 items' epilogue, against the oracle and the combine kernel;
    the 128-token decode at full size."""
    inp = synth.make_inputs(name) if over is None else synth.make_inputs(name, **over)
    opts = {binding.MOE_OPT_PERSISTENT_GEMM: 1, binding.MOE_OPT_TILED_GEMM: 2, FC: 1}
    if queue:
        opts[binding.MOE_OPT_QUEUE] = queue
    moe, d = run(inp, packed=True, opts=opts)
    _check(moe, inp, d)
    _same_as_kernel(moe, d, d.out.clone())


@pytest.mark.parametrize("name", ["decode128_fp8", "decode8_fp8", "decode256_mxfp4_shared",
                                  "decode256_w4a16_shared"])
def test_fused_combine_full_size(name):
    """The decode workloads at full size, packed weights: every token against the oracle."""
    inp = synth.make_inputs(name)
    moe, d = run(inp, packed=True, opts={FC: 1})
    _check(moe, inp, d)
    _same_as_kernel(moe, d, d.out.clone())


def test_tokens_with_no_row_get_zero_rows():
    """Without a shared expert, a token none of whose slots has a row here is written as
    zeros by the workgroups past the last work item (the output starts as NaN)."""
    inp = synth.make_inputs("decode128_fp8", S=4, T_s=70, H=256, I=128, E=6, k=2, seed=308)
    inp.ids[0, :5, :] = -1
    inp.ids[2, 60:, :] = -1
    inp.ids[3, 7, 0] = -1  # one slot of a token only
    moe = binding.Moe.for_inputs(inp)
    moe.set_option(FC, 1)
    d = binding.DeviceInputs(inp)
    d.out.fill_(float("nan"))
    moe.run(d)
    torch.cuda.synchronize()
    out = out_np(inp, d.out)
    assert np.all(out[0, :5] == 0) and np.all(out[2, 60:] == 0)
    _check(moe, inp, d)
    _same_as_kernel(moe, d, d.out.clone())


def test_nothing_routed_gives_zero():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=5, H=256, I=128, E=4, k=2, seed=309)
    inp.ids[:] = -1
    moe = binding.Moe.for_inputs(inp)
    moe.set_option(FC, 1)
    d = binding.DeviceInputs(inp)
    d.out.fill_(float("nan"))
    moe.run(d)
    torch.cuda.synchronize()
    assert np.all(out_np(inp, d.out) == 0)
    assert moe.device_error() == 0


def _cfg(inp, cap, sched=binding.MOE_SCHED_FENCE, dcu=0):
    return binding.make_config(inp.S, cap, inp.H, inp.I, inp.E, inp.k, inp.act, inp.weight, inp.out, inp.shared_I,
                               sched, dcu)


SOAK = [
    ("decode128_fp8", dict(S=8, H=1024, I=256, E=32, k=8), binding.MOE_SCHED_FENCE, 0),
    ("decode256_mxfp4_shared", dict(S=8, H=512, I=256, E=16, k=4, shared_I=256), binding.MOE_SCHED_FENCE, 0),
    ("decode128_fp8", dict(S=8, H=1024, I=256, E=32, k=8), binding.MOE_SCHED_SENTINEL, 0),
    ("decode128_fp8", dict(S=8, H=1024, I=256, E=32, k=8), binding.MOE_SCHED_FENCE, -1),
]


@pytest.mark.parametrize("name,over,sched,dcu", SOAK)
def test_fused_combine_soak(name, over, sched, dcu):
    """300 calls with inputs and batch size changing every call (some tokens with no row at
    all), workspace and output poisoned before each: every output equals the combine
    kernel's bit for bit, so no counter is left behind by an earlier call (dcu -1: the
    persistent kernel)."""
    sizes = [16, 1, 5, 12, 3, 16]
    probe = synth.make_inputs(name, T_s=1, seed=0, **over)
    ref = binding.Moe(_cfg(probe, 16))
    fused = binding.Moe(_cfg(probe, 16, sched, max(dcu, 0)))
    fused.set_option(FC, 1)
    fused.set_option(binding.MOE_OPT_POISON, 1)
    if dcu < 0:  # the persistent kernel
        fused.set_option(binding.MOE_OPT_PERSISTENT_GEMM, 1)
    sets = []
    for i, T_s in enumerate(sizes):
        inp = synth.make_inputs(name, T_s=T_s, seed=500 + i, **over)
        if i % 2:
            inp.ids[i % inp.S, : max(1, T_s // 2), :] = -1
        dd = binding.DeviceInputs(inp)
        ref.pack(dd)
        sets.append(dd)
    order = np.random.default_rng(11).integers(0, len(sets), 300)
    print(f"[gpu case] fused-combine soak {name} sched={sched}: 300 calls", flush=True)
    for i, j in enumerate(order):
        dd = sets[j]
        ref.run(dd)
        want = dd.out.clone()
        dd.out.fill_(float("nan"))
        fused.run(dd)
        if not torch.equal(want, dd.out):
            torch.cuda.synchronize()
            bad = int((want != dd.out).sum())
            raise AssertionError(f"call {i} (input set {j}, T_s {dd.inp.T_s}): {bad} outputs differ")
    torch.cuda.synchronize()
    assert fused.device_error() == 0 and ref.device_error() == 0


def test_timeout_is_latched_and_the_next_calls_are_right():
    """A SENTINEL wait forced to give up (invalid output, MOE_DEVERR_TIMEOUT latched) with
    the combine in GEMM2's epilogue: reading the error word leaves the counters at zero, so
    the following calls equal the FENCE path with the combine kernel."""
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=3, H=256, I=128, E=4, k=2, seed=310)
    ref = binding.Moe.for_inputs(inp)
    dr = binding.DeviceInputs(inp)
    ref.run(dr)
    torch.cuda.synchronize()
    want = dr.out.clone()
    ms = binding.Moe.for_inputs(inp, sched=binding.MOE_SCHED_SENTINEL)
    ms.set_option(FC, 1)
    d = binding.DeviceInputs(inp)
    ms.set_option(binding.MOE_OPT_SENTINEL_SPIN, 64)
    ms.set_option(binding.MOE_OPT_SENTINEL_STALL, 1)
    ms.run(d)
    torch.cuda.synchronize()
    assert ms.device_error() & binding.MOE_DEVERR_TIMEOUT
    ms.set_option(binding.MOE_OPT_SENTINEL_STALL, 0)
    ms.set_option(binding.MOE_OPT_SENTINEL_SPIN, 0)
    for _ in range(3):
        d.out.fill_(float("nan"))
        ms.run(d)
        torch.cuda.synchronize()
        assert ms.device_error() == 0
        assert torch.equal(want, d.out)

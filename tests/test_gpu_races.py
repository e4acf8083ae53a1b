"""The workspace is reused from call to call without a clean pass, and the SENTINEL
handshake lets GEMM1 start before the dispatch has finished (the double-buffered,
never-cleared counters of the token-ring handshake: "GC-MoE: Overlapping Expert-Parallel
Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green Contexts", full text; "GC-MoE:
Decoupling MoE Communication and Computation with CUDA Green Contexts", "Three-Node CUDA
Graph and token-ring Handshake").  These tests try to catch a read of a row the current
call has not written, a flag or queue state left over from an earlier call, and a wait
that does not wait:
  - MOE_OPT_POISON fills the windows, h, y and their scales with NaN codes before every
    call, so any such read turns outputs into NaN (or changes them);
  - inputs and batch sizes change on every call, and every call is compared bit for bit
    with the FENCE two-kernel path (or the oracle);
  - MOE_OPT_EPOCH starts the epoch counter just below 2^32, so calls cross its wrap;
  - MOE_OPT_DISPATCH_DELAY holds every dispatch chunk's rows back after it has published
    the counts, so GEMM1 workgroups really wait on the row flags.
"""
import numpy as np
import pytest
import torch

from combine_top_gate_amd import binding, synth
from parity import check_layer, gpu_state, out_np, run

pytestmark = pytest.mark.gpu

FENCE, SENTINEL = binding.MOE_SCHED_FENCE, binding.MOE_SCHED_SENTINEL


def _cfg(inp, cap, sched=FENCE, dcu=0):
    return binding.make_config(inp.S, cap, inp.H, inp.I, inp.E, inp.k, inp.act, inp.weight, inp.out, inp.shared_I,
                               sched, dcu)


def _input_sets(name, sizes, cap, base_seed, packer, **over):
    """Device input sets of one shape family with varying tokens per source (weights packed
    by `packer`, a context of the same configuration)."""
    sets = []
    for i, T_s in enumerate(sizes):
        inp = synth.make_inputs(name, T_s=T_s, seed=base_seed + i, **over)
        d = binding.DeviceInputs(inp)
        packer.pack(d)
        sets.append(d)
    return sets


POISON_CASES = [
    # name, overrides, options, schedule, dispatch_cus
    ("decode128_fp8", dict(S=4, T_s=9, H=512, I=256, E=8, k=4, seed=201), {}, FENCE, 0),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=202), {}, FENCE, 0),
    ("decode256_w4a16_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=256, seed=203), {}, FENCE, 0),
    ("prefill4096_zipf_fp8", dict(S=4, T_s=96, H=512, I=256, E=8, k=4, seed=204), {binding.MOE_OPT_TILED_GEMM: 1},
     FENCE, 0),
    ("decode128_fp8", dict(S=4, T_s=9, H=512, I=256, E=8, k=4, seed=205), {binding.MOE_OPT_PERSISTENT_GEMM: 1},
     FENCE, 0),
    ("tiny_f32", dict(seed=206), {}, FENCE, 0),
    ("decode128_fp8", dict(S=4, T_s=9, H=512, I=256, E=8, k=4, seed=207), {}, SENTINEL, 0),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=208), {}, SENTINEL, 16),
]


@pytest.mark.parametrize("name,over,opts,sched,dcu", POISON_CASES)
def test_poisoned_workspace_gives_the_same_result(name, over, opts, sched, dcu):
    """Every kernel path reads only rows its call wrote: with the workspace poisoned before
    the call the output is bit-identical to an unpoisoned call's, and passes the oracle."""
    inp = synth.make_inputs(name, **over)
    moe = binding.Moe(_cfg(inp, inp.T_s + 3, sched, dcu))  # capacity above the batch
    moe, d = run(inp, moe=moe, packed=inp.weight != "f32", opts=opts)
    clean = d.out.clone()
    moe.set_option(binding.MOE_OPT_POISON, 1)
    d.out.fill_(float("nan"))
    moe.run(d)
    torch.cuda.synchronize()
    assert torch.equal(clean, d.out)
    check_layer(inp, gpu_state(moe, inp), out_np(inp, d.out))
    assert moe.device_error() == 0


def _compare_calls(fence, sent, sets, order, delay_every=0, check_every=250):
    """Runs sets[order[i]] on both contexts and compares the outputs bit for bit; returns
    the number of calls.  Every delay_every-th SENTINEL call holds the dispatch rows back."""
    for i, j in enumerate(order):
        d = sets[j]
        fence.run(d)
        want = d.out.clone()
        d.out.fill_(float("nan"))
        if delay_every:
            sent.set_option(binding.MOE_OPT_DISPATCH_DELAY, 30 if i % delay_every == 0 else 0)
        sent.run(d)
        if not torch.equal(want, d.out):
            torch.cuda.synchronize()
            bad = int((want != d.out).sum())
            raise AssertionError(f"call {i} (input set {j}, T_s {d.inp.T_s}): {bad} outputs differ from FENCE")
        if check_every and (i + 1) % check_every == 0:
            assert sent.device_error() == 0, f"device error by call {i}"
            print(f"  {i + 1} calls equal", flush=True)
    return len(order)


SOAK = [
    ("decode128_fp8", dict(S=8, H=1024, I=256, E=32, k=8), 0),
    ("decode128_fp8", dict(S=8, H=1024, I=256, E=32, k=8), 16),
    ("decode256_mxfp4_shared", dict(S=8, H=512, I=256, E=16, k=4, shared_I=256), 0),
]


@pytest.mark.parametrize("name,over,dcu", SOAK)
def test_sentinel_soak_matches_fence(name, over, dcu):
    """1000 SENTINEL calls with the inputs and batch size changing every call, the workspace
    poisoned before each, every 7th with the dispatch rows held back 30 us: each output
    equals the FENCE path's bit for bit (the first difference stops the test)."""
    sizes = [16, 1, 5, 12, 3, 16]
    probe = synth.make_inputs(name, T_s=1, seed=0, **over)
    fence = binding.Moe(_cfg(probe, 16))
    sent = binding.Moe(_cfg(probe, 16, SENTINEL, dcu))
    sent.set_option(binding.MOE_OPT_POISON, 1)
    sets = _input_sets(name, sizes, 16, 400, fence, **over)
    order = np.random.default_rng(7).integers(0, len(sets), 1000)
    print(f"[gpu case] soak {name} dcu={dcu}: 1000 calls", flush=True)
    _compare_calls(fence, sent, sets, order, delay_every=7)
    assert sent.device_error() == 0 and fence.device_error() == 0


@pytest.mark.parametrize("dcu", [0, 16])
def test_sentinel_epoch_wrap(dcu):
    """Calls across the wrap of the 32-bit epoch counter (0xFFFFFFFE, 0xFFFFFFFF, then 1, 2,
    ...: 0 is never an epoch), workspace poisoned, each equal to FENCE."""
    over = dict(S=8, H=512, I=256, E=16, k=4)
    probe = synth.make_inputs("decode128_fp8", T_s=1, seed=0, **over)
    fence = binding.Moe(_cfg(probe, 8))
    sent = binding.Moe(_cfg(probe, 8, SENTINEL, dcu))
    sets = _input_sets("decode128_fp8", [8, 2, 5], 8, 500, fence, **over)
    _compare_calls(fence, sent, sets, [0, 1, 2], check_every=0)   # some epochs before the jump
    sent.set_option(binding.MOE_OPT_EPOCH, -3)                    # 0xFFFFFFFD: next call 0xFFFFFFFE
    sent.set_option(binding.MOE_OPT_POISON, 1)
    print(f"[gpu case] epoch wrap dcu={dcu}", flush=True)
    _compare_calls(fence, sent, sets, [0, 1, 2, 0, 2, 1, 0, 1], check_every=0)
    assert sent.device_error() == 0


@pytest.mark.parametrize("dcu", [0, 16])
def test_dispatch_delay_makes_gemm_wait(dcu):
    """With every dispatch chunk holding its rows back 500 us after publishing the counts,
    the SENTINEL layer takes at least that long (GEMM1 workgroups waited on the row flags)
    and still equals FENCE."""
    over = dict(S=8, T_s=8, H=512, I=256, E=16, k=4, seed=510)
    inp = synth.make_inputs("decode128_fp8", **over)
    fence = binding.Moe(_cfg(inp, 8))
    sent = binding.Moe(_cfg(inp, 8, SENTINEL, dcu))
    d = binding.DeviceInputs(inp)
    fence.pack(d)
    fence.run(d)
    want = d.out.clone()
    sent.set_option(binding.MOE_OPT_POISON, 1)
    sent.set_option(binding.MOE_OPT_DISPATCH_DELAY, 500)
    sent.run(d)  # warm
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d.out.fill_(float("nan"))
    start.record()
    sent.run(d)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    print(f"  delayed SENTINEL layer: {ms * 1e3:.0f} us", flush=True)
    assert ms >= 0.45
    assert torch.equal(want, d.out)
    assert sent.device_error() == 0


def test_persistent_gemm_back_to_back_changing_inputs():
    """The persistent GEMM resets its queues and per-expert counters itself: 60 calls with
    the inputs and batch size changing every call, the workspace poisoned before each, each
    equal bit for bit to the two-kernel path on the same inputs."""
    over = dict(S=8, H=1024, I=512, E=32, k=4)
    probe = synth.make_inputs("decode128_fp8", T_s=1, seed=0, **over)
    two = binding.Moe(_cfg(probe, 8))
    pers = binding.Moe(_cfg(probe, 8))
    pers.set_option(binding.MOE_OPT_PERSISTENT_GEMM, 1)
    pers.set_option(binding.MOE_OPT_POISON, 1)
    sets = _input_sets("decode128_fp8", [4, 8, 1, 6], 8, 550, two, **over)
    order = np.random.default_rng(9).integers(0, len(sets), 60)
    _compare_calls(two, pers, sets, order, check_every=0)
    assert pers.device_error() == 0

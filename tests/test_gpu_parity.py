"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Every case runs the layer on the GPU, reads back its routing, windows, h (codes and
scales), y rows and output, and checks them with parity.check_layer: integers and
dispatched bytes bit-exact; h codes inside the GEMM's accumulation band; y rows, shared
rows and outputs within 2e-2 (fp32 layer: 1e-3) per row and elementwise, after the
allowance for h codes that legitimately round the other way (the criterion is stated in
full in parity.py).  Small shapes span several workgroup tiles, ragged tails and
multi-pass experts; the five full-size configurations (and the W4A16 variant) are checked
on every window row and every token.
"""
import numpy as np
import pytest
import torch

from combine_top_gate_amd import binding, synth
from parity import check_layer, gpu_state, out_np, run

pytestmark = pytest.mark.gpu


def check(moe, inp, d, stats=None):
    """The whole layer of context moe (last run on d) against the oracle."""
    g = gpu_state(moe, inp)
    ref = check_layer(inp, g, out_np(inp, d.out), stats)
    assert moe.device_error() == 0
    return g, ref


SMALL = [
    ("tiny_f32", {}, False),
    # the most slots per token (16), an odd k between the combine's slot counts, and k = 1
    # with the shared expert
    ("decode128_fp8", dict(S=2, T_s=5, H=256, I=128, E=20, k=16, seed=15), False),
    ("tiny_f32", dict(E=9, k=5, seed=17), False),
    ("decode256_mxfp4_shared", dict(S=3, T_s=4, H=256, I=128, E=6, k=1, shared_I=128, seed=16), True),
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=11), False),
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=11), True),
    ("decode256_mxfp4_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=12), False),
    ("decode256_mxfp4_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=12), True),
    ("prefill4096_zipf_fp8", dict(S=2, T_s=40, H=256, I=384, E=6, k=4, seed=13), True),
    ("decode128_fp8", dict(S=5, T_s=3, H=128, I=128, E=7, k=2, seed=14), True),
    # W4A16: bf16 activations and h, MXFP4 weights; ragged passes, k = 1, one pass of 5 tiles
    ("decode256_w4a16_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=18), False),
    ("decode256_w4a16_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=18), True),
    ("decode256_w4a16_shared", dict(S=3, T_s=4, H=256, I=128, E=6, k=1, shared_I=128, seed=19), True),
    ("decode256_w4a16_shared", dict(S=4, T_s=20, H=512, I=384, E=3, k=3, shared_I=0, seed=20), True),
    ("decode256_w4a16_shared", dict(S=4, T_s=20, H=512, I=384, E=3, k=3, shared_I=0, seed=20), False),
]


@pytest.mark.parametrize("name,over,packed", SMALL)
def test_stages_match_oracle(name, over, packed):
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp, packed=packed)
    g, ref = check(moe, inp, d)
    if inp.act == "fp8":
        # nearly every requantised h code equals the oracle's (the sign of zero aside)
        used = ref["row_src"] >= 0
        R = inp.S * inp.T_s * inp.k
        hq, rq = g["h"][:R, :inp.I][used], ref["h_codes"][used]
        same = (hq == rq) | (((hq & 0x7F) == 0) & ((rq & 0x7F) == 0))
        print(f"  h codes equal: {same.mean():.6f}", flush=True)
        assert same.mean() >= 0.995, same.mean()


_FULL_CACHE = {}


def _full(name):
    if name not in _FULL_CACHE:
        _FULL_CACHE.clear()
        _FULL_CACHE[name] = synth.make_inputs(name)
    return _FULL_CACHE[name]


FULL = ["tiny_f32", "decode128_fp8", "decode8_fp8", "decode256_mxfp4_shared", "prefill4096_zipf_fp8",
        "decode256_w4a16_shared"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """The five configurations (and the W4A16 variant) at full size, as the benchmark runs
    them (packed weights, default options): every window row and every token."""
    inp = _full(name)
    moe, d = run(inp, packed=inp.weight != "f32")
    check(moe, inp, d)


@pytest.mark.parametrize("name,over", [
    ("decode128_fp8", dict(S=4, T_s=9, H=512, I=384, E=6, k=3, seed=51)),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=52)),
    ("decode256_w4a16_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=56)),
    ("decode128_fp8", {}),
])
def test_packed_weights_give_identical_output(name, over):
    """Packing only reorders weight bytes: the GEMM sees the same operands in the same order."""
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp)
    ref = d.out.clone()
    moe.pack(d)
    d.out.zero_()
    moe.run(d)
    torch.cuda.synchronize()
    assert torch.equal(ref, d.out)
    hb = moe.buffer(binding.MOE_BUF_H, 64)
    assert hb.numel() == 64


@pytest.mark.parametrize("name,over", [
    ("decode128_fp8", {}),
    # one token tile per expert: the small-batch kernels load token fragments into
    # registers, the kernels for three or more tiles stage them in LDS
    ("decode8_fp8", {}),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=53)),
    ("prefill4096_zipf_fp8", dict(S=4, T_s=64, H=512, I=256, E=16, k=4, seed=54)),
    # W4A16 runs two kernels whatever the persistent option says
    ("decode256_w4a16_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=57)),
])
def test_gemm_schedules_give_identical_output(name, over):
    """Persistent queues (per XCD or global), separate kernels and any token tiling run
    the same MFMAs per output element: results must agree bit for bit."""
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp, packed=True)
    ref = d.out.clone()
    for opt, val in [(binding.MOE_OPT_QUEUE, 2), (binding.MOE_OPT_QUEUE, 1), (binding.MOE_OPT_TOKEN_TILES, 2),
                     (binding.MOE_OPT_TOKEN_TILES, 3), (binding.MOE_OPT_TOKEN_TILES, 4),
                     (binding.MOE_OPT_PERSISTENT_GEMM, 0)]:
        moe.set_option(opt, val)
        d.out.zero_()
        moe.run(d)
        torch.cuda.synchronize()
        assert torch.equal(ref, d.out), (opt, val)
    assert moe.device_error() == 0


@pytest.mark.parametrize("name,over,packed", [
    ("prefill4096_zipf_fp8", dict(S=4, T_s=96, H=512, I=256, E=8, k=4, seed=61), False),
    ("prefill4096_zipf_fp8", dict(S=4, T_s=96, H=512, I=256, E=8, k=4, seed=61), True),
    ("prefill4096_zipf_fp8", dict(S=3, T_s=80, H=384, I=384, E=5, k=3, seed=62), True),
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=63), True),
    # one K slab in GEMM1 and GEMM2 (H = I = 128), one in GEMM2 only, and the shared
    # expert (FP8) through the tiled kernels
    ("prefill4096_zipf_fp8", dict(S=2, T_s=80, H=128, I=128, E=4, k=2, seed=64), True),
    ("prefill4096_zipf_fp8", dict(S=2, T_s=80, H=256, I=128, E=4, k=2, seed=65), False),
    ("decode128_fp8", dict(S=3, T_s=40, H=256, I=256, E=4, k=2, shared_I=384, seed=66), True),
])
def test_tiled_gemm_matches_oracle_and_streaming_kernel(name, over, packed):
    """The LDS-tiled kernels (large experts) against the oracle, and bit for bit against
    the weight-streaming kernels (same MFMAs per output element, same K order)."""
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp, packed=packed, opts={binding.MOE_OPT_TILED_GEMM: 1})
    tiled = d.out.clone()
    check(moe, inp, d)
    moe.set_option(binding.MOE_OPT_TILED_GEMM, 2)
    d.out.zero_()
    moe.run(d)
    torch.cuda.synchronize()
    assert torch.equal(tiled, d.out)
    assert moe.device_error() == 0


@pytest.mark.parametrize("name,over,packed", [
    ("prefill4096_zipf_fp8", dict(S=4, T_s=96, H=512, I=256, E=8, k=4, seed=61), False),
    ("prefill4096_zipf_fp8", dict(S=4, T_s=96, H=512, I=256, E=8, k=4, seed=61), True),
    ("prefill4096_zipf_fp8", dict(S=3, T_s=80, H=384, I=384, E=5, k=3, seed=62), True),
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=63), True),
])
def test_tiled_gemm_32x32_matches_oracle(name, over, packed):
    """The tiled kernels with 32x32x64 MFMAs (MOE_OPT_TILED_MFMA = 1) against the oracle,
    with the same bars as the 16x16x128 kernels; the two agree up to fp32 rounding of the
    block sums (codes may differ where that straddles a rounding boundary)."""
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp, packed=packed, opts={binding.MOE_OPT_TILED_GEMM: 1, binding.MOE_OPT_TILED_MFMA: 1})
    check(moe, inp, d)
    # the 16x16x128 kernels on the same inputs: equal outputs but for those roundings
    out32 = d.out.clone()
    moe.set_option(binding.MOE_OPT_TILED_MFMA, 0)
    moe.run(d)
    torch.cuda.synchronize()
    a, b = out_np(inp, out32), out_np(inp, d.out)
    print(f"  32x32 vs 16x16: {np.mean(a == b):.4f} of outputs equal, max rel "
          f"{np.max(np.abs(a - b) / np.maximum(np.abs(b), np.sqrt(np.mean(b ** 2)))):.3e}", flush=True)
    assert moe.device_error() == 0


def test_tiled_gemm_32x32_full_size_prefill():
    inp = _full("prefill4096_zipf_fp8")
    moe, d = run(inp, packed=True, opts={binding.MOE_OPT_TILED_MFMA: 1})
    check(moe, inp, d)


@pytest.mark.parametrize("name,over", [
    ("decode128_fp8", None),
    ("decode256_mxfp4_shared", dict(S=3, T_s=11, H=384, I=256, E=5, k=2, shared_I=128, seed=58)),
    # a Zipf-skewed prefill shape on the streaming kernels (the tiled kernels off)
    ("prefill4096_zipf_fp8", dict(S=8, T_s=64, H=1024, I=512, E=16, k=4, seed=59)),
])
@pytest.mark.parametrize("queue", [0, 2])
def test_persistent_gemm_matches_oracle(name, over, queue):
    """Both GEMMs in one persistent kernel (per-expert release counters between GEMM1 and
    GEMM2 items), per-XCD or single queue, against the oracle; the 128-token decode at full
    size."""
    inp = _full(name) if over is None else synth.make_inputs(name, **over)
    opts = {binding.MOE_OPT_PERSISTENT_GEMM: 1, binding.MOE_OPT_TILED_GEMM: 2}
    if queue:
        opts[binding.MOE_OPT_QUEUE] = queue
    moe, d = run(inp, packed=True, opts=opts)
    check(moe, inp, d)


SENTINEL_CASES = [
    ("decode128_fp8", dict(S=3, T_s=7, H=384, I=256, E=5, k=3, seed=71), 0),
    ("decode256_mxfp4_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=72), 0),
    ("decode128_fp8", dict(S=8, T_s=5, H=256, I=128, E=16, k=4, seed=73), 8),
    ("decode128_fp8", dict(S=4, T_s=3, H=256, I=256, E=6, k=2, seed=74), 32),
    ("decode256_w4a16_shared", dict(S=2, T_s=9, H=384, I=256, E=4, k=2, shared_I=384, seed=75), 0),
    ("decode256_w4a16_shared", dict(S=4, T_s=6, H=256, I=256, E=6, k=2, shared_I=0, seed=76), 16),
]


def _fence_and_sentinel(inp, dispatch_cus=0, packed=True):
    outs = []
    for sched in (binding.MOE_SCHED_FENCE, binding.MOE_SCHED_SENTINEL):
        moe = binding.Moe.for_inputs(inp, sched=sched, dispatch_cus=dispatch_cus)
        moe, d = run(inp, moe=moe, packed=packed)
        outs.append((moe, d))
    return outs


@pytest.mark.parametrize("name,over,dcu", SENTINEL_CASES)
def test_sentinel_matches_fence_and_oracle(name, over, dcu):
    """SENTINEL only changes when GEMM1 may start: the same kernels give the same bits."""
    inp = synth.make_inputs(name, **over)
    (mf, df), (ms, ds) = _fence_and_sentinel(inp, dcu)
    assert ms.device_error() == 0
    assert torch.equal(df.out, ds.out)
    check(ms, inp, ds)


@pytest.mark.parametrize("name,dcu", [("decode8_fp8", 0), ("decode128_fp8", 0), ("decode128_fp8", 16)])
def test_sentinel_full_size(name, dcu):
    inp = _full(name)
    (mf, df), (ms, ds) = _fence_and_sentinel(inp, dcu)
    assert ms.device_error() == 0
    assert torch.equal(df.out, ds.out)
    check(ms, inp, ds)


def test_sentinel_back_to_back_calls():
    """Epoch tags and arrival counters are reused across calls of varying size."""
    over = dict(S=4, H=256, I=128, E=8, k=3)
    fence = binding.Moe(binding.make_config(4, 6, 256, 128, 8, 3))
    sent = binding.Moe(binding.make_config(4, 6, 256, 128, 8, 3, sched=binding.MOE_SCHED_SENTINEL))
    for i, T_s in enumerate([6, 1, 4, 6, 2, 5]):
        inp = synth.make_inputs("decode128_fp8", T_s=T_s, seed=80 + i, **over)
        print(f"[gpu case] back-to-back call {i} T_s={T_s}", flush=True)
        d = binding.DeviceInputs(inp)
        fence.run(d)
        want = d.out.clone()
        d.out.zero_()
        sent.run(d)
        torch.cuda.synchronize()
        assert torch.equal(want, d.out), i
    assert sent.device_error() == 0


def test_sentinel_timeout_is_latched_and_recovers():
    """A wait that never completes gives up after its spin limit (forced from the host),
    latches MOE_DEVERR_TIMEOUT, and the next call is correct again."""
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=3, H=256, I=128, E=4, k=2, seed=90)
    (mf, df), (ms, ds) = _fence_and_sentinel(inp)
    want = df.out.clone()
    ms.set_option(binding.MOE_OPT_SENTINEL_SPIN, 64)
    ms.set_option(binding.MOE_OPT_SENTINEL_STALL, 1)
    ms.run(ds)
    torch.cuda.synchronize()
    assert ms.device_error() & binding.MOE_DEVERR_TIMEOUT
    ms.set_option(binding.MOE_OPT_SENTINEL_STALL, 0)
    ms.set_option(binding.MOE_OPT_SENTINEL_SPIN, 0)
    ds.out.zero_()
    ms.run(ds)
    torch.cuda.synchronize()
    assert ms.device_error() == 0
    assert torch.equal(want, ds.out)


def test_invalid_options():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=2, H=128, I=128, E=4, k=2)
    moe = binding.Moe.for_inputs(inp)
    for opt, val in [(binding.MOE_OPT_TOKEN_TILES, 1), (binding.MOE_OPT_TOKEN_TILES, 7), (binding.MOE_OPT_QUEUE, 3),
                     (binding.MOE_OPT_PERSISTENT_GEMM, 2), (binding.MOE_OPT_SENTINEL_SPIN, -1),
                     (binding.MOE_OPT_SENTINEL_STALL, 2), (binding.MOE_OPT_TILED_MFMA, 2),
                     (binding.MOE_OPT_POISON, 2), (binding.MOE_OPT_DISPATCH_DELAY, -1),
                     (binding.MOE_OPT_DISPATCH_DELAY, 10001), (binding.MOE_OPT_FUSED_COMBINE, 2), (11, 0)]:
        with pytest.raises(binding.MoeError):
            moe.set_option(opt, val)


def test_empty_batch_is_noop():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=0, H=128, I=128, E=4, k=2)
    moe = binding.Moe.for_inputs(inp, max_tokens=4)
    d = binding.DeviceInputs(inp)
    moe.run(d)
    torch.cuda.synchronize()
    assert moe.device_error() == 0


def test_nothing_routed_here_gives_zero():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=5, H=256, I=128, E=4, k=2, seed=21)
    inp.ids[:] = -1
    moe, d = run(inp)
    assert np.all(out_np(inp, d.out) == 0)
    cnt, _, dst, src = (t.cpu().numpy() for t in moe.routing(inp.S, inp.T_s, inp.k, inp.E))
    assert cnt.sum() == 0 and np.all(dst == -1) and np.all(src == -1)


def test_all_rows_to_one_expert_multi_pass():
    inp = synth.make_inputs("decode128_fp8", S=4, T_s=50, H=256, I=256, E=8, k=1, seed=22)
    inp.ids[:] = 3
    inp.topk_w[:] = 1.0
    moe, d = run(inp)
    check(moe, inp, d)


def test_bad_ids_are_dropped_and_flagged():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=6, H=256, I=128, E=4, k=2, seed=23)
    inp.ids[0, 1, 0] = 9
    inp.ids[1, 2, 1] = -5
    moe, d = run(inp)
    assert moe.device_error() & binding.MOE_DEVERR_BAD_ID
    clean = synth.make_inputs("decode128_fp8", S=2, T_s=6, H=256, I=128, E=4, k=2, seed=23)
    clean.ids[0, 1, 0] = -1
    clean.ids[1, 2, 1] = -1
    check(moe, clean, d)  # the device error was cleared by the previous read


def test_replays_without_clearing_and_capacity_above_batch():
    """Back-to-back calls on one context (no clean pass), batch smaller than capacity."""
    moe = None
    for seed, T_s in [(31, 6), (32, 3), (33, 6)]:
        inp = synth.make_inputs("decode128_fp8", S=3, T_s=T_s, H=256, I=256, E=6, k=3, seed=seed)
        moe, d = run(inp, moe=moe or binding.Moe.for_inputs(inp, max_tokens=8))
        check(moe, inp, d)


def test_stage_entry_points_compose():
    """moe_dispatch + moe_grouped_gemm + moe_combine equal moe_layer."""
    inp = synth.make_inputs("decode256_mxfp4_shared", S=2, T_s=5, H=256, I=128, E=3, k=2, shared_I=128,
                            seed=41)
    moe, d = run(inp)
    full = d.out.clone()
    d.out.zero_()
    moe.dispatch(inp.T_s, d.x, d.x_scale, d.ids)
    moe.grouped_gemm(d.weights)
    moe.combine(d.topk_w, d.out)
    torch.cuda.synchronize()
    assert torch.equal(full, d.out)


def test_invalid_call_arguments():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=4, H=128, I=128, E=4, k=2)
    moe = binding.Moe.for_inputs(inp)
    d = binding.DeviceInputs(inp)
    with pytest.raises(binding.MoeError) as ei:
        moe.layer(5, d.x, d.x_scale, d.ids, d.topk_w, d.weights, d.out)  # above capacity
    assert ei.value.status == binding.MOE_ERR_INVALID_ARG
    with pytest.raises(binding.MoeError):
        moe.dispatch(4, d.x, None, d.ids)  # FP8 without scales
    with pytest.raises(binding.MoeError):
        moe.combine(d.topk_w, d.out[..., 1:])  # misaligned output


# The ABI's limits: hidden and intermediate sizes of MOE_MAX_DIM (16384, 128 K slabs),
# MOE_MAX_SRC sources with MOE_MAX_EXPERTS experts and MOE_MAX_TOPK slots, for each kernel
# family (streaming FP8 and MXFP4, fp32, the LDS-tiled prefill kernel).
MAXCASES = [
    ("decode128_fp8", dict(S=2, T_s=3, H=16384, I=128, E=2, k=1, seed=41), True),
    ("decode128_fp8", dict(S=2, T_s=3, H=128, I=16384, E=2, k=2, seed=42), False),
    ("decode256_mxfp4_shared", dict(S=2, T_s=3, H=16384, I=128, E=2, k=1, shared_I=256, seed=43), True),
    ("decode128_fp8", dict(S=32, T_s=2, H=128, I=128, E=256, k=16, seed=44), False),
    ("tiny_f32", dict(S=1, T_s=4, H=16384, I=256, E=2, k=1, seed=45), False),
    ("prefill4096_zipf_fp8", dict(S=2, T_s=192, H=16384, I=256, E=2, k=1, seed=46), True),
    ("decode256_w4a16_shared", dict(S=2, T_s=3, H=16384, I=128, E=2, k=1, shared_I=256, seed=47), True),
    ("decode256_w4a16_shared", dict(S=2, T_s=3, H=128, I=16384, E=2, k=2, shared_I=0, seed=48), False),
]


@pytest.mark.parametrize("name,over,packed", MAXCASES)
def test_maximum_sizes(name, over, packed):
    inp = synth.make_inputs(name, **over)
    moe, d = run(inp, packed=packed)
    check(moe, inp, d)

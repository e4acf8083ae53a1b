"""GPU parity of the gate ahead of dispatch (router logits, then top-k softmax)
through the C-ABI, against the oracle's router_logits and softmax_topk.

Bars:
  top-k ids   bit-exact when both sides see the same fp32 logits: the selection is
              a comparison of fp32 values, and fp32 -> fp64 keeps their order.
  top-k w     |g - r| <= (2 * spread + k + 6) * 2^-24 * r + 2^-40 per weight, with
              spread = max |z_j - z_max| over the token's finite kept logits (a
              -inf logit's weight is 0 on both sides): the kernel
              forms z_j - z_max in fp32 (relative error <= u * spread carried into
              exp), expf (a few ulp), a k-term fp32 sum and one division.
  logits      |g - r| <= gamma_n * sum_h |x_h * w_h| + 2^-60, n = 32 + ceil(H / 256) + 16:
              bf16 x bf16 products are exact in fp32; a 32-deep MFMA step is
              counted as 32 sequential fp32 additions; the K steps are split over
              at least 8 waves (so a wave chains at most ceil(H / 256) of them) and
              at most 16 partial sums are added (Higham, gamma_n = n u / (1 - n u),
              u = 2^-24).
  end to end  ids equal the oracle's wherever the gap between the k-th and the
              (k+1)-th fp64 logit exceeds twice the logits bound; everywhere, the
              ids are the exact top-k of the GPU's own logits.
"""
import numpy as np
import pytest
import torch

from combine_top_gate_amd import binding, synth
from oracle import codecs, gating

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def check_topk(z32, k):
    """Run the kernel on fp32 logits z32 [T][E]; compare ids exactly and weights to the bound."""
    zd = torch.from_numpy(np.ascontiguousarray(z32, dtype=np.float32)).cuda()
    ids, w = binding.topk_softmax(zd, k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    rid, rw = gating.softmax_topk(z32.astype(np.float64), k)
    assert np.array_equal(ids, rid)
    sel = np.take_along_axis(z32.astype(np.float64), rid.astype(np.int64), axis=1)
    # -inf logits get weight exactly 0 on both sides; the spread is over the finite ones
    spread = np.max(np.where(np.isfinite(sel), sel[:, :1] - sel, 0.0), axis=1, keepdims=True)
    bound = (2 * spread + k + 6) * U * rw + 2.0 ** -40
    assert np.all(np.abs(w - rw) <= bound), float(np.max(np.abs(w - rw) / bound))
    return ids


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 8, 2), (37, 40, 8), (130, 200, 8),
                                   (64, 256, 16), (300, 256, 8), (3, 64, 1)])
def test_topk_softmax_matches_oracle(lib, T, E, k):
    rng = np.random.default_rng(1000 + T + E + k)
    z = synth.draw_logits(rng, T, E, "normal").astype(np.float32)
    check_topk(z, k)


def test_topk_softmax_ties_and_infinities(lib):
    rng = np.random.default_rng(7)
    # values on a coarse grid: many exact ties, broken to the lower expert id
    z = (np.round(rng.standard_normal((96, 256)) * 2) / 4).astype(np.float32)
    z[0, :] = 1.0                      # all equal: ids 0..k-1 in order, equal weights
    z[1, :] = -np.inf                  # all -inf except two
    z[1, 17] = 0.0
    z[1, 200] = 0.0
    z[2, 100:] = -np.inf
    ids = check_topk(z, 8)
    assert list(ids[0]) == list(range(8))
    assert list(ids[1][:2]) == [17, 200]


def test_topk_softmax_zipf_routing(lib):
    rng = np.random.default_rng(11)
    z = synth.draw_logits(rng, 512, 256, "zipf").astype(np.float32)
    check_topk(z, 8)


def router_case(T, H, E, seed):
    ri = synth.make_router_inputs(T, H, E, seed=seed)
    g = binding.router_logits(dev_bits(ri.x_bits), dev_bits(ri.wr_bits))
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    x, wr = codecs.bf16_decode(ri.x_bits), codecs.bf16_decode(ri.wr_bits)
    r = gating.router_logits(x, wr)
    mag = gating.router_logits(np.abs(x), np.abs(wr))
    # the longest accumulation chain of either router kernel: 32 products inside an MFMA
    # step, then up to H / 32 chained steps (the LDS-tiled kernel: one wave takes all of
    # K) or H / 256 steps and 16 wave partials (the kernel for few tokens)
    bound = gamma(32 + H // 32 + 16) * mag + 2.0 ** -60
    return g, r, bound


@pytest.mark.parametrize("T,H,E", [(1, 32, 1), (5, 64, 7), (17, 96, 33), (40, 512, 64),
                                   (33, 1056, 250), (130, 2048, 256),
                                   # wide token tiles (enough tiles to cover the CUs), ragged T and E
                                   (1000, 256, 256), (2050, 96, 130),
                                   # the LDS-tiled kernel: 5 and 6 K chunks (both peeled tails),
                                   # ragged T and E, and the full hidden size
                                   (300, 640, 256), (257, 768, 100), (512, 7168, 256)])
def test_router_logits_within_fp32_bound(lib, T, H, E):
    g, r, bound = router_case(T, H, E, seed=T * 131 + E)
    err = np.abs(g - r)
    print(f"  T {T} H {H} E {E}: max err/bound {np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)


@pytest.mark.parametrize("T", [128, 1024])
def test_gate_full_size_end_to_end(lib, T):
    """DeepSeek-V3-shaped gate: H 7168, 256 experts, top-8, one decode batch (128
    tokens) and all eight sources' batches at once (1024)."""
    H, E, k = 7168, 256, 8
    g, r, bound = router_case(T, H, E, seed=T)
    assert np.all(np.abs(g - r) <= bound)
    ids = check_topk(g.astype(np.float32), k)
    rs = -np.sort(-r, axis=1)
    margin = rs[:, k - 1] - rs[:, k]
    clear = margin > 2 * bound.max(axis=1)
    rid, _ = gating.softmax_topk(r, k)
    print(f"  T {T}: {int(clear.sum())} of {T} tokens with a clear top-{k} margin", flush=True)
    assert clear.mean() > 0.9
    assert np.array_equal(np.sort(ids[clear], axis=1), np.sort(rid[clear], axis=1))


def test_gate_calls_after_empty_batch(lib):
    zd = torch.zeros((0, 16), dtype=torch.float32, device="cuda")
    ids, w = binding.topk_softmax(zd, 4)
    assert ids.shape == (0, 4)
    lg = binding.router_logits(torch.zeros((0, 64), dtype=torch.int16, device="cuda"),
                               torch.zeros((16, 64), dtype=torch.int16, device="cuda"))
    assert lg.shape == (0, 16)
    check_topk(np.arange(32, dtype=np.float32)[None, :].repeat(3, 0), 4)


# ---------------------------------------------------------------- fused gate
def fused_bound(H, mag):
    # per wave at most H / 32 chained MFMA steps (the LDS-tiled kernel's K slice, at least
    # one slice; the kernel for few tokens splits K over 4 waves and adds 4 wave
    # partials), at most 16 slice partials
    return gamma(32 + H // 32 + 4 + 16) * mag + 2.0 ** -60


@pytest.mark.parametrize("T,H,E,k", [(1, 256, 8, 2), (5, 1056, 100, 4), (16, 512, 256, 8), (17, 7168, 256, 8),
                                     (40, 2048, 64, 6), (64, 768, 33, 3), (65, 4096, 256, 8),
                                     (128, 7168, 256, 8), (130, 1024, 256, 16), (300, 7168, 32, 8),
                                     (1024, 7168, 256, 8), (2, 64, 1, 1),
                                     # 6 and 11 K slices: the top-k re-reads the last slice
                                     # for the missing ones and drops them
                                     (50, 1536, 64, 4), (100, 2816, 256, 8),
                                     # the LDS-tiled kernel: one K chunk per slice, two slices of
                                     # five chunks, and 4096 tokens in one slice (the largest
                                     # shape the no-allocation scratch holds)
                                     (600, 640, 100, 4), (2048, 1280, 256, 8), (4096, 7168, 256, 8)])
def test_fused_gate_matches_oracle(lib, T, H, E, k):
    ri = synth.make_router_inputs(T, H, E, seed=7 * T + H + E)
    x, wr = dev_bits(ri.x_bits), dev_bits(ri.wr_bits)
    # a workspace full of NaN: its contents on entry must not matter
    ws = torch.full((binding.gate_workspace_bytes(T, H, E) // 4 + 4,), float("nan"), device="cuda")
    ids, w, lg = binding.gate(x, wr, k, workspace=ws, want_logits=True)
    ids2, w2 = binding.gate(x, wr, k)
    torch.cuda.synchronize()
    lg = lg.cpu().numpy().astype(np.float64)
    xd, wd = codecs.bf16_decode(ri.x_bits), codecs.bf16_decode(ri.wr_bits)
    r = gating.router_logits(xd, wd)
    bound = fused_bound(H, gating.router_logits(np.abs(xd), np.abs(wd)))
    err = np.abs(lg - r)
    print(f"  T {T} H {H} E {E}: logits max err/bound {np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)
    # the ids and weights are exactly the top-k softmax of the returned sums
    rid, rw = gating.softmax_topk(lg, k)
    g_ids, g_w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_ids, rid)
    sel = np.take_along_axis(lg, rid.astype(np.int64), axis=1)
    spread = np.max(sel[:, :1] - sel, axis=1, keepdims=True)
    assert np.all(np.abs(g_w - rw) <= (2 * spread + k + 6) * U * rw + 2.0 ** -40)
    # without the logits output: the same bits
    assert torch.equal(ids2, ids) and torch.equal(w2, w)


def test_fused_gate_short_workspace_rejected(lib):
    T, H, E = 128, 7168, 256
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    wr = torch.zeros((E, H), dtype=torch.int16, device="cuda")
    ws = torch.empty(binding.gate_workspace_bytes(T, H, E) // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MoeError, match="workspace"):
        binding.gate(x, wr, 8, workspace=ws)


def test_gate_drives_the_layer(lib):
    """The gate ahead of dispatch: the GPU gate's ids and weights go device to device into
    the layer.  The gate's choices are checked against the oracle's own gate (fp64 router
    logits, top-k softmax) on the same bf16 router inputs: the same ids for nearly every
    token (the two differ only where fp32 and fp64 sums order two logits differently), and
    nearly the same weights where the ids agree (their exact bound is the fused-gate test's).  The layer is checked against
    the oracle's layer run on the ids and weights the GPU gate produced."""
    from oracle import layer  # noqa: F401  (the layer oracle runs inside parity.check_layer)
    from parity import check_layer, gpu_state, out_np
    inp = synth.make_inputs("decode128_fp8", S=4, T_s=16, H=1024, I=256, E=32, k=8, seed=71)
    S, T_s, k = inp.S, inp.T_s, inp.k
    T = S * T_s
    ri = synth.make_router_inputs(T, inp.H, inp.E, seed=72)
    ids, w = binding.gate(dev_bits(ri.x_bits), dev_bits(ri.wr_bits), k)
    moe = binding.Moe.for_inputs(inp)
    d = binding.DeviceInputs(inp)
    d.ids = ids.view(S, T_s, k)
    d.topk_w = w.view(S, T_s, k)
    moe.run(d)
    torch.cuda.synchronize()
    # the oracle's gate, from the generator's router inputs only
    r = gating.router_logits(codecs.bf16_decode(ri.x_bits), codecs.bf16_decode(ri.wr_bits))
    rid, rw = gating.softmax_topk(r, k)
    g_ids, g_w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    same = np.all(g_ids == rid, axis=1)
    print(f"  {int(same.sum())} of {T} tokens routed alike", flush=True)
    assert same.mean() > 0.9
    assert np.allclose(g_w[same], rw[same], rtol=1e-3, atol=0)
    # the layer on the GPU gate's own routing
    inp.ids = g_ids.reshape(S, T_s, k).astype(np.int32)
    inp.topk_w = g_w.astype(np.float32).reshape(S, T_s, k)
    check_layer(inp, gpu_state(moe, inp), out_np(inp, d.out))
    assert moe.device_error() == 0

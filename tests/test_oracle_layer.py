"""Pins for the whole oracle layer.

The layer is checked against a per-token brute force written here on its own
(no dispatch at all: out[t] = sum_j w_j FFN_{e_j}(x_t) with dequantisation by
np.repeat, SwiGLU by torch silu, the 1x128 requantisation by torch float32 ops,
bf16 activations decoded and h rounded by torch's bfloat16 casts), against the identity-expert case (combine returns the dispatched rows
bit for bit) and against closed forms of the weighted sum.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import codecs, layer
from combine_top_gate_amd import synth


def _deq_w(fmt, w, s):
    if fmt == "f32":
        return np.asarray(w, np.float64)
    if fmt == "fp8":
        return codecs.e4m3_decode(w) * np.repeat(np.repeat(s, 128, 0), 128, 1)
    v = codecs.e2m1_unpack(w)
    return v * np.repeat(np.ldexp(1.0, s.astype(int) - 127), 32, 1)


def _requant_torch(h):
    t = torch.from_numpy(h).to(torch.float32)
    tb = t.reshape(t.shape[0], -1, 128)
    amax = tb.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / torch.tensor(448.0), torch.ones_like(amax))
    q = torch.clamp(tb / s[:, :, None], -448, 448).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s[:, :, None].to(torch.float64)).reshape(h.shape).numpy()


def _ffn_brute(fmt, act, x, w13, s13, w2, s2, inter):
    W13 = torch.from_numpy(_deq_w(fmt, w13, s13))
    W2 = torch.from_numpy(_deq_w(fmt, w2, s2))
    tx = torch.from_numpy(x)[None, :]
    h = (F.silu(tx @ W13[:inter].T) * (tx @ W13[inter:].T)).numpy()
    if act == "fp8":
        h = _requant_torch(h)
    elif act == "bf16":
        h = torch.from_numpy(h).to(torch.bfloat16).to(torch.float64).numpy()
    return (torch.from_numpy(h) @ W2.T).numpy()[0]


def _rnd(fmt, v):
    if fmt == "bf16":
        return torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    return v.astype(np.float32).astype(np.float64)


def brute_force(inp):
    S, T_s, H = inp.S, inp.T_s, inp.H
    out = np.zeros((S, T_s, H))
    for s in range(S):
        for t in range(T_s):
            if inp.act == "fp8":
                x = codecs.e4m3_decode(inp.x[s, t]) * np.repeat(inp.x_scale[s, t], 128)
            elif inp.act == "bf16":
                x = torch.from_numpy(inp.x[s, t].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
            else:
                x = inp.x[s, t].astype(np.float64)
            acc = np.zeros(H)
            for j in range(inp.k):
                e = inp.ids[s, t, j]
                if e < 0:
                    continue
                y = _ffn_brute(inp.weight, inp.act, x, inp.w13[e],
                               None if inp.s13 is None else inp.s13[e], inp.w2[e],
                               None if inp.s2 is None else inp.s2[e], inp.I)
                acc += float(inp.topk_w[s, t, j]) * _rnd(inp.out, y)
            if inp.shared_I:
                acc += _rnd(inp.out, _ffn_brute(inp.weight, inp.act, x, inp.sh_w13, inp.sh_s13,
                                                inp.sh_w2, inp.sh_s2, inp.shared_I))
            out[s, t] = _rnd(inp.out, acc)
    return out


TINY = [
    ("tiny_f32", dict(T_s=6)),
    ("decode128_fp8", dict(S=3, T_s=4, H=256, I=384, E=5, k=3)),
    ("decode256_mxfp4_shared", dict(S=2, T_s=3, H=256, I=256, E=4, k=2, shared_I=128)),
    ("decode256_w4a16_shared", dict(S=2, T_s=3, H=256, I=256, E=4, k=2, shared_I=128)),
    ("prefill4096_zipf_fp8", dict(S=2, T_s=5, H=128, I=256, E=6, k=4)),
]


@pytest.mark.parametrize("name,over", TINY)
def test_layer_matches_per_token_brute_force(name, over):
    inp = synth.make_inputs(name, **over)
    # some pairs not routed to this GPU
    inp.ids[0, 0, -1] = -1
    res = layer.moe_layer(inp)
    ref = brute_force(inp)
    got = res["out"]
    scale = np.sqrt(np.mean(ref ** 2))
    # the two routes differ only by fp64 summation order, plus (bf16/fp8 paths) a
    # rounding-boundary flip now and then; bound the error accordingly
    tol = 1e-12 if inp.out == "f32" and inp.act == "f32" else 2 ** -7
    err = np.max(np.abs(got - ref) / np.maximum(np.abs(ref), scale))
    assert err <= tol, err
    if inp.act == "f32":
        assert np.allclose(got, ref, rtol=1e-6, atol=1e-7 * scale)


def test_sampled_tokens_agree_with_whole_layer():
    inp = synth.make_inputs("decode128_fp8", S=2, T_s=5, H=256, I=256, E=4, k=2)
    res = layer.moe_layer(inp)
    toks = [(0, 0), (1, 4), (0, 3)]
    got = layer.layer_tokens(inp, toks)
    for n, (s, t) in enumerate(toks):
        assert np.array_equal(got[n], res["out"][s, t])


def test_identity_expert_combine_is_exact():
    """k = 1, weight 1, y := the dispatched rows themselves -> out == x bit for bit."""
    rng = np.random.default_rng(9)
    S, T_s, H, E = 3, 5, 64, 4
    ids = rng.integers(0, E, (S, T_s, 1)).astype(np.int32)
    x = rng.standard_normal((S, T_s, H)).astype(np.float32)
    r = layer.dispatch(ids, E)
    win = layer.scatter_window(x, r["dst_row"])
    out = layer.combine(win.astype(np.float64), r["dst_row"], np.ones((S, T_s, 1), np.float32))
    assert np.array_equal(out.astype(np.float32), x)


def test_weighted_combine_closed_form():
    """Expert e scales its input by (e+1): out = (sum_j w_j (e_j+1)) x."""
    rng = np.random.default_rng(10)
    S, T_s, k, E, H = 2, 6, 3, 5, 16
    ids = np.stack([[rng.choice(E, k, replace=False) for _ in range(T_s)] for _ in range(S)]).astype(np.int32)
    w = rng.uniform(0, 1, (S, T_s, k)).astype(np.float32)
    x = rng.standard_normal((S, T_s, H))
    r = layer.dispatch(ids, E)
    win = layer.scatter_window(x, r["dst_row"])
    expert_of_row = np.full(win.shape[0], -1)
    for s in range(S):
        for t in range(T_s):
            for j in range(k):
                expert_of_row[r["dst_row"][s, t, j]] = ids[s, t, j]
    y = win * (expert_of_row[:, None] + 1)
    out = layer.combine(y, r["dst_row"], w)
    ref = (w.astype(np.float64) * (ids + 1)).sum(axis=2)[:, :, None] * x
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-14)
    # a shared expert output is added after the routed sum
    ysh = rng.standard_normal((S * T_s, H))
    out2 = layer.combine(y, r["dst_row"], w, ysh)
    assert np.allclose(out2 - out, ysh.reshape(S, T_s, H), rtol=0, atol=1e-13)


def test_order_inside_window_does_not_change_output():
    inp = synth.make_inputs("tiny_f32", T_s=4)
    res = layer.moe_layer(inp)
    rng = np.random.default_rng(11)
    R = res["y_win"].shape[0]
    P = rng.permutation(R)
    y2 = np.zeros_like(res["y_win"])
    y2[P] = res["y_win"]
    dst2 = np.where(res["dst_row"] >= 0, P[np.maximum(res["dst_row"], 0)], -1)
    out2 = layer.combine(y2, dst2, inp.topk_w)
    out1 = layer.combine(res["y_win"], res["dst_row"], inp.topk_w)
    assert np.array_equal(out1, out2)


def test_empty_and_unrouted():
    inp = synth.make_inputs("tiny_f32", T_s=0)
    res = layer.moe_layer(inp)
    assert res["out"].shape == (2, 0, 256)
    inp = synth.make_inputs("tiny_f32", T_s=3)
    inp.ids[:] = -1
    res = layer.moe_layer(inp)
    assert np.all(res["out"] == 0) and res["cnt"].sum() == 0


def test_fp8_output_round_trips_representable_rows():
    """k = 1, weight 1, no shared expert: y rows that are e4m3 values times 2^-5 (448 in
    every block) come back as their own codes and scale, block by block."""
    rng = np.random.default_rng(21)
    S, T_s, H = 2, 3, 384
    codes = rng.integers(0, 0x7E, (S * T_s, H)).astype(np.uint8) | (rng.integers(0, 2, (S * T_s, H)) << 7).astype(np.uint8)
    codes[:, ::128] = 0x7E                   # +448 at the start of every block
    y = codecs.e4m3_decode(codes) * 2.0 ** -5
    dst = np.arange(S * T_s, dtype=np.int32).reshape(S, T_s, 1)
    w = np.ones((S, T_s, 1), np.float32)
    q, sc = layer.combine_fp8(y, dst, w)
    assert np.all(sc == 2.0 ** -5)
    nz = (codes & 0x7F) != 0
    assert np.array_equal(q.reshape(S * T_s, H)[nz], codes[nz])
    assert np.all((q.reshape(S * T_s, H)[~nz] & 0x7F) == 0)


def test_fp8_output_matches_torch():
    """Random rows, k = 3 with an unrouted slot and a shared expert: the fp64 weighted sums
    in slot order (written here), then torch float32 ops and torch's e4m3 cast."""
    rng = np.random.default_rng(22)
    S, T_s, k, H, R = 2, 4, 3, 256, 24
    y = rng.standard_normal((R, H)) * 10 ** rng.uniform(-2, 2, (R, 1))
    ysh = rng.standard_normal((S * T_s, H))
    dst = rng.permutation(R)[:S * T_s * k].reshape(S, T_s, k).astype(np.int32)
    dst[1, 2, 1] = -1
    w = rng.uniform(0, 1, (S, T_s, k)).astype(np.float32)
    acc = np.zeros((S * T_s, H))
    for s in range(S):
        for t in range(T_s):
            for j in range(k):
                if dst[s, t, j] >= 0:
                    acc[s * T_s + t] += float(w[s, t, j]) * y[dst[s, t, j]]
            acc[s * T_s + t] += ysh[s * T_s + t]
    tt = torch.from_numpy(acc).to(torch.float32).reshape(S * T_s, H // 128, 128)
    amax = tt.abs().amax(dim=2)
    sc = torch.where(amax > 0, amax / torch.tensor(448.0), torch.ones_like(amax))
    rq = torch.clamp(tt / sc[:, :, None], -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    q, s_ = layer.combine_fp8(y, dst, w, ysh)
    assert np.array_equal(s_.reshape(S * T_s, -1), sc.to(torch.float64).numpy())
    rq = rq.reshape(S * T_s, H).numpy()
    nz = (rq & 0x7F) != 0
    assert np.array_equal(q.reshape(S * T_s, H)[nz], rq[nz])

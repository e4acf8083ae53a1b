"""Pins for the oracle's block-scale dequantisation, SwiGLU expert FFN and FP8 requantisation.

References used: torch.nn.functional.silu and matmul (the E=1, k=1 layer is a
dense SwiGLU FFN), np.repeat expansions of planted scales (a transposed or
shifted block index changes the result), torch's float32 division and
float8_e4m3fn cast (the requantisation decision in fp32), and the closed-form
identity  deq(x) deq(W)^T = sum_kb s_x[:,kb] s_W[nb,kb] (Q_x[:,kb] Q_W[:,kb]^T).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import codecs, layer
from combine_top_gate_amd import synth


def test_fp8_weight_scale_blocks_planted():
    N, K = 256, 384
    codes = np.full((N, K), 0x38, np.uint8)                      # every code is 1.0
    s = (np.arange(6, dtype=np.float64).reshape(2, 3) * 10 + 1)  # distinct per block
    got = layer.dequant_w_fp8(codes, s)
    assert np.array_equal(got, np.repeat(np.repeat(s, 128, 0), 128, 1))


def test_fp8_act_scale_blocks_planted():
    M, K = 3, 384
    codes = np.full((M, K), 0xB8, np.uint8)                      # every code is -1.0
    s = np.arange(9, dtype=np.float64).reshape(3, 3) + 0.5
    assert np.array_equal(layer.dequant_act_fp8(codes, s), -np.repeat(s, 128, 1))


def test_mxfp4_scale_blocks_planted():
    N, K = 2, 128
    packed = np.full((N, K // 2), 0x22, np.uint8)                # every element is 1.0
    e = np.array([[120, 121, 127, 130], [1, 200, 127, 126]], np.uint8)
    got = layer.dequant_w_mxfp4(packed, e)
    assert np.array_equal(got, np.repeat(np.ldexp(1.0, e.astype(int) - 127), 32, 1))


def test_block_scale_promotion_identity():
    rng = np.random.default_rng(2)
    M, N, K = 5, 256, 512
    qx = rng.integers(0, 0x7E, (M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    qw = rng.integers(0, 0x7E, (N, K), dtype=np.uint8)
    sx = rng.uniform(0.01, 2, (M, K // 128))
    sw = rng.uniform(0.01, 2, (N // 128, K // 128))
    direct = layer.dequant_act_fp8(qx, sx) @ layer.dequant_w_fp8(qw, sw).T
    vx, vw = codecs.e4m3_decode(qx), codecs.e4m3_decode(qw)
    prom = np.zeros((M, N))
    for kb in range(K // 128):
        part = vx[:, kb * 128:(kb + 1) * 128] @ vw[:, kb * 128:(kb + 1) * 128].T
        prom += part * sx[:, kb:kb + 1] * np.repeat(sw[:, kb], 128)[None, :]
    assert np.allclose(prom, direct, rtol=1e-12, atol=1e-12 * np.abs(direct).max())


def test_dense_swiglu_ffn_matches_torch():
    rng = np.random.default_rng(5)
    M, H, I = 7, 256, 384
    x = rng.standard_normal((M, H))
    w13 = rng.standard_normal((2 * I, H)) * 0.05
    w2 = rng.standard_normal((H, I)) * 0.05
    y, _, _ = layer.expert_ffn(x, w13, w2, I, requant=False)
    tx, t13, t2 = (torch.from_numpy(a) for a in (x, w13, w2))
    ref = (F.silu(tx @ t13[:I].T) * (tx @ t13[I:].T)) @ t2.T
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_w4a16_ffn_rounds_h_to_bf16():
    """bf16 activations and h (the W4A16 variant): x decoded by torch's bfloat16 view, the
    weights dequantised by np.repeat, SwiGLU by torch, h rounded by the separately pinned
    bf16 rounding; the oracle must agree to fp64 summation order (a skipped rounding of h
    moves y by ~1e-4)."""
    inp = synth.make_inputs("decode256_w4a16_shared", S=1, T_s=6, H=256, I=256, E=1, k=1, shared_I=0)
    xb = np.asarray(inp.x).reshape(6, 256)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    w13 = codecs.e2m1_unpack(inp.w13[0]) * np.repeat(np.ldexp(1.0, inp.s13[0].astype(int) - 127), 32, 1)
    w2 = codecs.e2m1_unpack(inp.w2[0]) * np.repeat(np.ldexp(1.0, inp.s2[0].astype(int) - 127), 32, 1)
    t13, t2 = torch.from_numpy(w13), torch.from_numpy(w2)
    h = (F.silu(x @ t13[:256].T) * (x @ t13[256:].T)).numpy()
    ref = torch.from_numpy(codecs.bf16_round(h)) @ t2.T
    y, hq, hs = layer.expert_ffn(codecs.bf16_decode(xb),
                                 layer.dequant_weight("fp4", inp.w13[0], inp.s13[0]),
                                 layer.dequant_weight("fp4", inp.w2[0], inp.s2[0]), 256, "bf16")
    assert hs is None and np.array_equal(hq, codecs.bf16_round(h))
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12 * np.abs(ref.numpy()).max())
    # and the whole layer (E = 1, k = 1, weight 1) returns bf16(y)
    inp.topk_w[:] = 1.0
    res = layer.moe_layer(inp)
    got, want = res["out"].reshape(6, 256), codecs.bf16_round(ref.numpy())
    # equal but for a rounding flip now and then (fp64 summation order): one ulp at most
    assert np.mean(got == want) >= 0.99
    assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want))


def _torch_requant(h):
    """Independent fp32 requantisation with torch float32 ops and torch's e4m3 cast."""
    t = torch.from_numpy(h).to(torch.float32)
    M, I = t.shape
    tb = t.reshape(M, I // 128, 128)
    amax = tb.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / torch.tensor(448.0, dtype=torch.float32), torch.ones_like(amax))
    q = torch.clamp(tb / s[:, :, None], -448, 448).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(M, I).numpy(), s.to(torch.float64).numpy()


def test_requant_matches_torch_fp32():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((40, 512)) * 10 ** rng.uniform(-3, 3, (40, 1))
    h[3, 128:256] = 0.0                      # an all-zero block
    codes, scales = layer.requant_1x128(h)
    rc, rs = _torch_requant(h)
    assert np.array_equal(scales, rs)
    assert scales[3, 1] == 1.0
    nz = (rc & 0x7F) != 0
    assert np.array_equal(codes[nz], rc[nz])
    assert np.all((codes[~nz] & 0x7F) == 0)


def test_requant_exact_on_representable_block():
    # values that are e4m3 codes times a power of two, with 448 present: exact round trip
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 0x7E, (2, 256)).astype(np.uint8)
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    s0 = 2.0 ** -5
    h = codecs.e4m3_decode(codes) * s0
    q, s = layer.requant_1x128(h)
    assert np.all(s == s0)
    assert np.array_equal(q, codes)


def test_requant_blocks_are_independent():
    rng = np.random.default_rng(8)
    h = rng.standard_normal((2, 384))
    q1, s1 = layer.requant_1x128(h)
    h2 = h.copy()
    h2[:, 128:256] *= 1000.0
    q2, s2 = layer.requant_1x128(h2)
    assert np.array_equal(q1[:, :128], q2[:, :128]) and np.array_equal(q1[:, 256:], q2[:, 256:])
    assert np.array_equal(s1[:, [0, 2]], s2[:, [0, 2]])

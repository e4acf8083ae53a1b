"""Seeded synthetic inputs for the MoE layer (the only module shared by tests and bench).

This module builds inputs; it holds none of the layer's arithmetic (no dispatch,
no expert FFN, no requantisation of the SwiGLU output, no combine).  Inputs are
produced with library primitives only: numpy's PCG64 generator, torch's
float8_e4m3fn cast, and a nearest-value lookup for FP4.

The pages measure on model suites that are not available, so synthetic inputs of
the layer's shapes stand in for them (DeepSeek-V3-like shapes: hidden 7168,
moe intermediate 2048, 32 local experts of 256, top-8; 8 source ranks).

Recipe: numpy.random.SeedSequence(seed).spawn(4 + 2E + 2) gives independent PCG64
streams, in this order: logits, activations, (unused), (unused), W13 of expert
0..E-1, W2 of expert 0..E-1, shared W13, shared W2.  Weight streams are drawn
on a thread pool, one expert per task; the values do not depend on the pool.
  1. routing logits z [S*T_s][E]:
       "normal": iid N(0,1)  -> top-k is a uniformly random k-subset;
       "zipf":   z_e = -zipf_s * ln(e+1) + Gumbel(0,1)  -> top-k samples k
                 distinct experts without replacement with probability
                 proportional to (e+1)^-zipf_s (Gumbel-top-k).
     ids = the k largest z per token (descending, ties to the lower id);
     weights = softmax over the kept z, computed in fp64, stored fp32.
     This is the upstream router's output that arrives with the tokens.
  2. activations x [S][T_s][H] ~ N(0,1).
  3. routed W13 [E][2I][H] ~ N(0, 0.02^2), expert by expert, then routed W2
     [E][H][I], then the shared expert's W13 and W2.
  Quantisation of inputs:
     fp8 activations: one fp32 scale per 1x128 block, s = amax/448 (1 if the
       block is all zero), code = e4m3(clamp(x/s, +-448)) via torch's cast.
     fp8 weights: the same with 128x128 blocks.
     MXFP4 weights: per 1x32 block, shared exponent floor(log2 amax) - 2,
       e8m0 = that + 127, value = nearest e2m1 magnitude of x/2^exp (ties to
       the even code, saturating at 6).
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0

CONFIGS = {
    # tiny fp32 layer: parity at 1e-3
    "tiny_f32": dict(S=2, T_s=32, H=256, I=512, E=8, k=2, act="f32", weight="f32",
                     out="f32", shared_I=0, routing="normal", seed=0),
    # decode, 8 sources x 16 tokens = 128 tokens, FP8 block-scaled
    "decode128_fp8": dict(S=8, T_s=16, H=7168, I=2048, E=32, k=8, act="fp8", weight="fp8",
                          out="bf16", shared_I=0, routing="normal", seed=1),
    # small-batch decode, 8 tokens
    "decode8_fp8": dict(S=8, T_s=1, H=7168, I=2048, E=32, k=8, act="fp8", weight="fp8",
                        out="bf16", shared_I=0, routing="normal", seed=2),
    # prefill, 8 x 512 = 4096 tokens, Zipf(1.2) expert popularity
    "prefill4096_zipf_fp8": dict(S=8, T_s=512, H=7168, I=2048, E=32, k=8, act="fp8",
                                 weight="fp8", out="bf16", shared_I=0, routing="zipf",
                                 zipf_s=1.2, seed=3),
    # decode at 256 tokens, MXFP4 weights + one shared expert
    "decode256_mxfp4_shared": dict(S=8, T_s=32, H=7168, I=2048, E=32, k=8, act="fp8",
                                   weight="fp4", out="bf16", shared_I=2048, routing="normal",
                                   seed=4),
    # the same layer with bf16 activations (W4A16): x and h stay bf16
    "decode256_w4a16_shared": dict(S=8, T_s=32, H=7168, I=2048, E=32, k=8, act="bf16",
                                   weight="fp4", out="bf16", shared_I=2048, routing="normal",
                                   seed=5),
}


@dataclass
class LayerInputs:
    name: str
    S: int
    T_s: int
    H: int
    I: int
    E: int
    k: int
    act: str
    weight: str
    out: str
    shared_I: int
    logits: np.ndarray                 # fp64 [S*T_s][E]
    ids: np.ndarray                    # int32 [S][T_s][k]
    topk_w: np.ndarray                 # fp32 [S][T_s][k]
    x: np.ndarray                      # uint8 [S][T_s][H] (fp8), uint16 bf16 bits or fp32
    x_scale: Optional[np.ndarray]      # fp32 [S][T_s][H/128] or None
    w13: np.ndarray
    s13: Optional[np.ndarray]
    w2: np.ndarray
    s2: Optional[np.ndarray]
    sh_w13: Optional[np.ndarray] = None
    sh_s13: Optional[np.ndarray] = None
    sh_w2: Optional[np.ndarray] = None
    sh_s2: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.S * self.T_s


# ----------------------------------------------------------------- routing
def route_from_logits(z, k):
    """Top-k ids (descending logit, ties to the lower id) and softmax weights over them."""
    order = np.argsort(-z.astype(np.float64), axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(z.astype(np.float64), order, axis=1)
    w = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    return order.astype(np.int32), w.astype(np.float32)


def draw_logits(rng, T, E, routing, zipf_s=1.2):
    if routing == "normal":
        return rng.standard_normal((T, E))
    if routing == "zipf":
        g = rng.gumbel(size=(T, E))
        return -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))[None, :] + g
    raise ValueError(routing)


# ------------------------------------------------------------ quantisation
def _to_e4m3_codes(v):
    """fp32 array already clamped to +-448 -> uint8 e4m3 codes (torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quant_fp8_rows(x):
    """[M][K] fp32 -> (codes uint8 [M][K], scales fp32 [M][K/128])."""
    M, K = x.shape
    xb = x.reshape(M, K // 128, 128)
    amax = np.abs(xb).max(axis=2)
    s = np.where(amax > 0, (amax / np.float32(FP8_MAX)).astype(np.float32), np.float32(1.0))
    v = np.clip(xb / s[:, :, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    return _to_e4m3_codes(v).reshape(M, K), s.astype(np.float32)


def quant_fp8_blocks(w):
    """[N][K] fp32 -> (codes uint8 [N][K], scales fp32 [N/128][K/128])."""
    N, K = w.shape
    wb = w.reshape(N // 128, 128, K // 128, 128)
    amax = np.abs(wb).max(axis=(1, 3))
    s = np.where(amax > 0, (amax / np.float32(FP8_MAX)).astype(np.float32), np.float32(1.0))
    v = np.clip(wb / s[:, None, :, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    return _to_e4m3_codes(v).reshape(N, K), s.astype(np.float32)


_FP4_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
# code of each magnitude, indexed by twice the magnitude (0, .5, 1, 1.5, 2, 3, 4, 6)
_FP4_INDEX = np.zeros(13, dtype=np.uint8)
for _c, _m in enumerate(_FP4_MAGS):
    _FP4_INDEX[int(_m * 2)] = _c


def quant_mxfp4(w):
    """[N][K] fp32 -> (packed uint8 [N][K/2], e8m0 uint8 [N][K/32])."""
    N, K = w.shape
    wb = w.reshape(N, K // 32, 32).astype(np.float32)
    amax = np.abs(wb).max(axis=2)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    ex = np.clip(ex, -127, 127).astype(np.int32)
    v = np.abs(wb) * np.ldexp(np.float32(1.0), -ex)[:, :, None].astype(np.float32)
    v = np.minimum(v, np.float32(6.0))
    # nearest magnitude, a value half-way between two going to the even code:
    # below 1 the grid is 0.5 apart (rint halves to even); from 1 up there is
    # one mantissa bit, rounded on the fp32 bit pattern
    small = np.rint(v * np.float32(2.0)) * np.float32(0.5)
    bits = v.view(np.uint32)
    bits = (bits + np.uint32(0x1FFFFF) + ((bits >> np.uint32(22)) & np.uint32(1))) & np.uint32(0xFFC00000)
    big = bits.view(np.float32)
    mag = np.where(v < 1.0, small, big)
    idx = _FP4_INDEX[(mag * np.float32(2.0)).astype(np.int32)]
    code = idx | np.where((wb < 0) & (idx > 0), 0x8, 0).astype(np.uint8)
    code = code.reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (ex + 127).astype(np.uint8)


def _quant_weight(fmt, w):
    if fmt == "f32":
        return w.astype(np.float32), None
    if fmt == "fp8":
        return quant_fp8_blocks(w)
    if fmt == "fp4":
        return quant_mxfp4(w)
    raise ValueError(fmt)


def _weight_shape(fmt, N, K):
    if fmt == "fp4":
        return (N, K // 2), (N, K // 32), np.uint8, np.uint8
    if fmt == "fp8":
        return (N, K), (N // 128, K // 128), np.uint8, np.float32
    return (N, K), None, np.float32, None


def _gen_weights(seeds, fmt, N, K):
    """One weight matrix per seed sequence, drawn in parallel threads."""
    E = len(seeds)
    ws, ss, wdt, sdt = _weight_shape(fmt, N, K)
    W = np.empty((E,) + ws, dtype=wdt)
    S = np.empty((E,) + ss, dtype=sdt) if ss is not None else None

    def one(e):
        rng = np.random.default_rng(seeds[e])
        w = rng.standard_normal((N, K), dtype=np.float32)
        w *= np.float32(0.02)
        q, s = _quant_weight(fmt, w)
        W[e] = q
        if S is not None:
            S[e] = s

    workers = max(1, min(E, len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(workers) as pool:
        list(pool.map(one, range(E)))
    return W, S


# ------------------------------------------------------------------ driver
def make_inputs(name="decode128_fp8", **over):
    """Build the inputs of a named configuration, with optional overrides."""
    cfg = dict(CONFIGS[name]) if name in CONFIGS else {}
    cfg.update(over)
    S, T_s, H, I, E, k = (cfg[n] for n in ("S", "T_s", "H", "I", "E", "k"))
    act, weight, out = cfg["act"], cfg["weight"], cfg["out"]
    shared_I = cfg.get("shared_I", 0)
    if H % 128 or I % 128 or (shared_I and shared_I % 128):
        raise ValueError("hidden and intermediate sizes must be multiples of 128")
    seq = np.random.SeedSequence(cfg.get("seed", 0)).spawn(4 + 2 * E + 2)
    T = S * T_s
    z = draw_logits(np.random.default_rng(seq[0]), T, E, cfg.get("routing", "normal"),
                    cfg.get("zipf_s", 1.2))
    ids, w = route_from_logits(z, k)
    xf = np.random.default_rng(seq[1]).standard_normal((T, H), dtype=np.float32)
    if act == "fp8":
        xq, xs = quant_fp8_rows(xf)
        x = xq.reshape(S, T_s, H)
        x_scale = xs.reshape(S, T_s, H // 128)
    elif act == "bf16":
        x, x_scale = _bf16_bits(xf).reshape(S, T_s, H), None
    else:
        x, x_scale = xf.reshape(S, T_s, H), None
    w13, s13 = _gen_weights(seq[4:4 + E], weight, 2 * I, H)
    w2, s2 = _gen_weights(seq[4 + E:4 + 2 * E], weight, H, I)
    inp = LayerInputs(name=name, S=S, T_s=T_s, H=H, I=I, E=E, k=k, act=act, weight=weight,
                      out=out, shared_I=shared_I, logits=z.astype(np.float64),
                      ids=ids.reshape(S, T_s, k), topk_w=w.reshape(S, T_s, k),
                      x=x, x_scale=x_scale, w13=w13, s13=s13, w2=w2, s2=s2)
    if shared_I:
        a, b = _gen_weights(seq[4 + 2 * E:4 + 2 * E + 1], weight, 2 * shared_I, H)
        c, d = _gen_weights(seq[4 + 2 * E + 1:4 + 2 * E + 2], weight, H, shared_I)
        inp.sh_w13, inp.sh_s13 = a[0], (b[0] if b is not None else None)
        inp.sh_w2, inp.sh_s2 = c[0], (d[0] if d is not None else None)
    inp.extra = cfg
    return inp


# ------------------------------------------------------------ gating inputs
@dataclass
class RouterInputs:
    """Hidden states and router weights for the gate, as bf16 bit patterns."""
    x_bits: np.ndarray   # uint16 [T][H]
    wr_bits: np.ndarray  # uint16 [E][H]
    T: int
    H: int
    E: int


def _bf16_bits(a):
    """Round to bf16 with torch's cast and return the 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def make_router_inputs(T, H, E, seed=0):
    """x ~ N(0, 1) [T][H] and wr ~ N(0, 1/H) [E][H] (logits of unit scale), in bf16.

    The router of a DeepSeek-V3-shaped layer scores all 256 global experts; streams:
    SeedSequence(seed).spawn(2) -> x, wr."""
    sx, sw = np.random.SeedSequence(seed).spawn(2)
    x = np.random.Generator(np.random.PCG64(sx)).standard_normal((T, H))
    wr = np.random.Generator(np.random.PCG64(sw)).standard_normal((E, H)) / np.sqrt(H)
    return RouterInputs(_bf16_bits(x), _bf16_bits(wr), T, H, E)


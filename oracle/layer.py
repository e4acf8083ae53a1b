"""One GPU's share of an expert-parallel MoE layer: dispatch, expert FFNs, combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, step by step, and where each step comes from:

1. Dispatch [NVLinkOneSided, Abstract; Relay-free Ascend, Abstract].  Every
   source rank pushes its tokens, with no metadata exchanged first, into
   rank-major receive buffers on the target; the target keeps only counts,
   offsets and synchronisation state.  Reading taken: source s owns rows
   [s*T_s*k, (s+1)*T_s*k) of the receive window and lays its own (token, slot)
   pairs out sorted by expert, using only its own counts; inside one
   (source, expert) bucket the pairs keep their order i = t*k + j.  Expert e's
   window is the concatenation, over s in order, of source s's bucket for e.
2. Grouped GEMM read in place [NVLinkOneSided, Abstract] with SwiGLU fused and
   requantisation [GC-MoE feed, Full text].  Reading taken: W13[e] rows 0..I-1
   are the gate projection and rows I..2I-1 the up projection;
   h = silu(gate) * up; h is requantised to FP8 with one fp32 scale per 128
   consecutive elements of a row before the down projection W2[e].
3. Combine [NVLinkOneSided, Abstract; Relay-free Ascend, Abstract: direct
   reading of expert windows, no output restoration].  out[s][t] is the sum
   over the token's k slots of weight * expert output, written in token order,
   plus the shared expert's output when there is one [GC-MoE feed, Full text:
   optional shared experts].

Block scales: FP8 weights carry one fp32 multiplier per 128x128 block
(rows, contraction); FP8 activations and h one per 1x128 block along the
contraction; MXFP4 weights one e8m0 power of two per 1x32 block along the
contraction (the MX block of [GC-MoE explainer, "Two MMA Implementations in
the Compute Partition"]).  Real value = code value * multiplier.
"""
import numpy as np

from . import codecs

BLOCK = 128     # FP8 scale block edge
MX_BLOCK = 32   # MXFP4 scale block length


# --------------------------------------------------------------------------
# 1. dispatch
# --------------------------------------------------------------------------
def dispatch(ids, n_experts):
    """Rank-major counting sort of each source's (token, slot) pairs.

    ids: int [S][T_s][k]; -1 marks a pair that is not routed to this GPU.
    Returns dict with
      cnt     int64 [S][E]    pairs of source s for expert e
      off     int64 [S][E]    exclusive prefix of cnt[s] over e
      dst_row int64 [S][T_s][k] window row of each pair, -1 if not routed
      row_src int64 [S*T_s*k] flattened pair index s*T_s*k + t*k + j that
                              fills each window row, -1 for unused rows
    """
    ids = np.asarray(ids)
    S, T_s, k = ids.shape
    E = n_experts
    seg = T_s * k
    cnt = np.zeros((S, E), dtype=np.int64)
    off = np.zeros((S, E), dtype=np.int64)
    dst_row = np.full((S, T_s, k), -1, dtype=np.int64)
    row_src = np.full(S * seg, -1, dtype=np.int64)
    for s in range(S):
        for t in range(T_s):
            for j in range(k):
                e = int(ids[s, t, j])
                if e == -1:
                    continue
                if not 0 <= e < E:
                    raise ValueError(f"dispatch: expert id {e} out of range")
                cnt[s, e] += 1
        running = 0
        for e in range(E):
            off[s, e] = running
            running += cnt[s, e]
        placed = np.zeros(E, dtype=np.int64)
        for t in range(T_s):
            for j in range(k):
                e = int(ids[s, t, j])
                if e == -1:
                    continue
                r = s * seg + off[s, e] + placed[e]
                placed[e] += 1
                dst_row[s, t, j] = r
                row_src[r] = s * seg + t * k + j
    return {"cnt": cnt, "off": off, "dst_row": dst_row, "row_src": row_src}


def expert_rows(cnt, off, T_s, k):
    """Window rows of each expert, in expert-window order (source-major)."""
    S, E = cnt.shape
    seg = T_s * k
    rows = []
    for e in range(E):
        r = []
        for s in range(S):
            base = s * seg + off[s, e]
            r.extend(range(base, base + cnt[s, e]))
        rows.append(np.array(r, dtype=np.int64))
    return rows


def scatter_window(x_rows, dst_row):
    """Receive window contents: window row dst_row[s,t,j] holds source row x_rows[s][t].

    x_rows: array [S][T_s][...] (any dtype).  Unused rows are left as zeros.
    """
    S, T_s, k = dst_row.shape
    win = np.zeros((S * T_s * k,) + x_rows.shape[2:], dtype=x_rows.dtype)
    for s in range(S):
        for t in range(T_s):
            for j in range(k):
                r = dst_row[s, t, j]
                if r >= 0:
                    win[r] = x_rows[s, t]
    return win


# --------------------------------------------------------------------------
# 2. block-scaled operands
# --------------------------------------------------------------------------
def dequant_act_fp8(codes, scales):
    """FP8 rows [M][K] with one fp32 scale per 1x128 block [M][K/128] -> fp64."""
    v = codecs.e4m3_decode(codes)
    M, K = v.shape
    s = np.asarray(scales, dtype=np.float64)
    out = np.empty_like(v)
    for b in range(K // BLOCK):
        out[:, b * BLOCK:(b + 1) * BLOCK] = v[:, b * BLOCK:(b + 1) * BLOCK] * s[:, b:b + 1]
    return out


def dequant_w_fp8(codes, scales):
    """FP8 weight [N][K] with one fp32 scale per 128x128 block [N/128][K/128] -> fp64."""
    v = codecs.e4m3_decode(codes)
    N, K = v.shape
    s = np.asarray(scales, dtype=np.float64)
    out = np.empty_like(v)
    for nb in range(N // BLOCK):
        for kb in range(K // BLOCK):
            out[nb * BLOCK:(nb + 1) * BLOCK, kb * BLOCK:(kb + 1) * BLOCK] = (
                v[nb * BLOCK:(nb + 1) * BLOCK, kb * BLOCK:(kb + 1) * BLOCK] * s[nb, kb])
    return out


def dequant_w_mxfp4(packed, e8m0):
    """MXFP4 weight, packed [N][K/2] with e8m0 scales [N][K/32] -> fp64 [N][K]."""
    v = codecs.e2m1_unpack(packed)
    N, K = v.shape
    s = codecs.e8m0_decode(e8m0)
    out = np.empty_like(v)
    for b in range(K // MX_BLOCK):
        out[:, b * MX_BLOCK:(b + 1) * MX_BLOCK] = v[:, b * MX_BLOCK:(b + 1) * MX_BLOCK] * s[:, b:b + 1]
    return out


def dequant_weight(fmt, w, s):
    if fmt == "f32":
        return np.asarray(w, dtype=np.float64)
    if fmt == "fp8":
        return dequant_w_fp8(w, s)
    if fmt == "fp4":
        return dequant_w_mxfp4(w, s)
    raise ValueError(fmt)


def dequant_act(fmt, x, s):
    if fmt == "f32":
        return np.asarray(x, dtype=np.float64)
    if fmt == "fp8":
        return dequant_act_fp8(x, s)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# 3. expert FFN
# --------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(a, inter):
    """a [M][2I] (gate | up) -> silu(gate) * up, [M][I]."""
    return silu(a[:, :inter]) * a[:, inter:2 * inter]


def requant_1x128(h):
    """Requantise rows of h to FP8 e4m3 with one fp32 scale per 128 elements.

    The decision is taken in fp32, as the kernel takes it: h is rounded to fp32,
    amax is the largest |h| of the block, s = fl32(amax / 448) (s = 1 when
    amax = 0), and each code is the e4m3 value nearest to fl32(h / s) after
    clamping to [-448, 448], ties to even.
    Returns (codes uint8 [M][I], scales fp64 [M][I/128] holding fp32 values).
    """
    h32 = codecs.fp32_round(h)
    M, I = h32.shape
    codes = np.zeros((M, I), dtype=np.uint8)
    scales = np.zeros((M, I // BLOCK), dtype=np.float64)
    for b in range(I // BLOCK):
        blk = h32[:, b * BLOCK:(b + 1) * BLOCK]
        amax = np.max(np.abs(blk), axis=1)
        s = codecs.fp32_round(amax / codecs.E4M3_MAX)
        s = np.where(amax == 0, 1.0, s)
        v = codecs.fp32_round(blk / s[:, None])
        v = np.clip(v, -codecs.E4M3_MAX, codecs.E4M3_MAX)
        codes[:, b * BLOCK:(b + 1) * BLOCK] = codecs.e4m3_encode(v)
        scales[:, b] = s
    return codes, scales


def h_format(act):
    """How h is stored between the projections: "fp8" (1x128 requantisation) for FP8
    activations, "bf16" for bf16 activations (the W4A16 variant), None (as is) for fp32."""
    return {"fp8": "fp8", "bf16": "bf16"}.get(act)


def expert_ffn(x, w13, w2, inter, requant, pre=None):
    """Dequantised rows x [M][H], W13 [2I][H], W2 [H][I] -> (y [M][H], h_codes, h_scales).

    y = requant(silu(x W13[:I]^T) * (x W13[I:]^T)) W2^T, all in fp64.  requant: "fp8"
    (or True) requantises h to FP8 with 1x128 scales; "bf16" rounds h to bf16 (nearest,
    ties to even), returned as h_codes (fp64 values) with h_scales None; None or False
    (the fp32 layer) passes h to the down projection as is.  The bf16 form is the W4A16
    variant: FP4 weights decoded in registers ahead of an MMA that does not take FP4
    [GC-MoE explainer, "Two MMA Implementations in the Compute Partition"]; the pages do
    not fix the activations' precision there, and the reading taken is that x and h stay
    bf16 (h rounded from its exact value).
    pre: when a dict is given, the exact gate|up projections a [M][2I] are left in
    pre["a"] (for tests that bound the rounding of h; nothing else changes).
    """
    a = x @ w13.T
    if pre is not None:
        pre["a"] = a
    h = swiglu(a, inter)
    if requant == "bf16":
        hq, hs = codecs.bf16_round(h), None
        h_used = hq
    elif requant:
        hq, hs = requant_1x128(h)
        h_used = dequant_act_fp8(hq, hs)
    else:
        hq, hs = None, None
        h_used = h
    y = h_used @ w2.T
    return y, hq, hs


def round_out(y, fmt):
    if fmt == "bf16":
        return codecs.bf16_round(y)
    if fmt == "f32":
        return codecs.fp32_round(y)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# 4. combine
# --------------------------------------------------------------------------
def combine(y_win, dst_row, topk_w, y_shared=None):
    """out[s][t] = sum_j w[s,t,j] * y_win[dst_row[s,t,j]] (+ y_shared[s*T_s+t]), fp64.

    Slots with dst_row = -1 contribute nothing; a token with no routed slot and
    no shared expert gives 0.
    """
    S, T_s, k = dst_row.shape
    H = y_win.shape[1]
    out = np.zeros((S, T_s, H), dtype=np.float64)
    for s in range(S):
        for t in range(T_s):
            acc = np.zeros(H, dtype=np.float64)
            for j in range(k):
                r = dst_row[s, t, j]
                if r >= 0:
                    acc += float(topk_w[s, t, j]) * y_win[r]
            if y_shared is not None:
                acc += y_shared[s * T_s + t]
            out[s, t] = acc
    return out


def combine_fp8(y_win, dst_row, topk_w, y_shared=None):
    """The combined output requantised as the next layer's FP8 input: the sums of
    combine() (exact, before any output rounding), then the 1x128 rule of requant_1x128
    along each token row.  Reading taken for the requantisation the pages fuse into the
    layer [GC-MoE feed, Full text]: applied to the layer's output as well, by the same
    rule as to h.  Returns (codes uint8 [S][T_s][H], scales fp64 [S][T_s][H/128])."""
    out = combine(y_win, dst_row, topk_w, y_shared)
    S, T_s, H = out.shape
    q, s = requant_1x128(out.reshape(S * T_s, H))
    return q.reshape(S, T_s, H), s.reshape(S, T_s, H // BLOCK)


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
def _act_rows(inp):
    """All tokens' activations, dequantised, [S*T_s][H] fp64 (token order s-major)."""
    x = np.asarray(inp.x)
    S, T_s, H = x.shape[0], x.shape[1], x.shape[2]
    if inp.act == "fp8":
        xs = np.asarray(inp.x_scale)
        return dequant_act_fp8(x.reshape(S * T_s, H), xs.reshape(S * T_s, H // BLOCK))
    if inp.act == "bf16":
        return codecs.bf16_decode(x.reshape(S * T_s, H))
    return np.asarray(x, dtype=np.float64).reshape(S * T_s, H)


def moe_layer(inp, experts=None, on_expert=None):
    """Run the whole layer on the CPU; returns every intermediate the GPU exposes.

    inp has fields: S, T_s, H, I, E, k, act ("f32"|"fp8"|"bf16", the last as bf16
    bit patterns, uint16), weight
    ("f32"|"fp8"|"fp4"), out ("f32"|"bf16"), shared_I (0 = none), x [S][T_s][H],
    x_scale [S][T_s][H/128] or None, ids [S][T_s][k], topk_w [S][T_s][k],
    w13, s13, w2, s2 (per expert, leading dim E) and sh_w13, sh_s13, sh_w2,
    sh_s2 for the shared expert.

    Two conveniences for tests that check a GPU's intermediate results expert by expert
    (neither changes what is computed):
      experts    None (all), or the routed expert ids to evaluate, plus "shared" for the
                 shared expert; the window rows of the others stay zero, and so does
                 their share of "out".
      on_expert  called after each evaluated expert as on_expert(e, rows, x_rows, w13,
                 w2, a, y, hq, hs): e is the expert id or "shared", rows its window rows
                 (None for the shared expert, whose rows are all tokens in order),
                 x_rows/w13/w2 the dequantised operands, a the exact gate|up
                 projections, y the output rows rounded to the output format, hq/hs what
                 h became (codes and scales, bf16 values, or None).
    """
    S, T_s, H, I, E, k = inp.S, inp.T_s, inp.H, inp.I, inp.E, inp.k
    hfmt = h_format(inp.act)
    requant = hfmt == "fp8"
    route = dispatch(inp.ids, E)
    rows = expert_rows(route["cnt"], route["off"], T_s, k)
    xt = _act_rows(inp)                       # token-ordered dequantised activations
    R = S * T_s * k
    src_token = np.where(route["row_src"] >= 0, route["row_src"] // k, -1)
    y_win = np.zeros((R, H), dtype=np.float64)
    h_codes = np.zeros((R, I), dtype=np.uint8) if requant else None
    h_scales = np.zeros((R, I // BLOCK), dtype=np.float64) if requant else None
    h_bf16 = np.zeros((R, I), dtype=np.float64) if hfmt == "bf16" else None
    for e in range(E):
        r = rows[e]
        if len(r) == 0 or (experts is not None and e not in experts):
            continue
        w13 = dequant_weight(inp.weight, inp.w13[e], None if inp.s13 is None else inp.s13[e])
        w2 = dequant_weight(inp.weight, inp.w2[e], None if inp.s2 is None else inp.s2[e])
        pre = {} if on_expert else None
        y, hq, hs = expert_ffn(xt[src_token[r]], w13, w2, I, hfmt, pre)
        y_win[r] = round_out(y, inp.out)
        if requant:
            h_codes[r] = hq
            h_scales[r] = hs
        elif hfmt == "bf16":
            h_bf16[r] = hq
        if on_expert:
            on_expert(e, r, xt[src_token[r]], w13, w2, pre["a"], y_win[r], hq, hs)
    y_sh = None
    sh = {}
    if inp.shared_I and (experts is None or "shared" in experts):
        w13 = dequant_weight(inp.weight, inp.sh_w13, inp.sh_s13)
        w2 = dequant_weight(inp.weight, inp.sh_w2, inp.sh_s2)
        pre = {} if on_expert else None
        y_sh, shq, shs = expert_ffn(xt, w13, w2, inp.shared_I, hfmt, pre)
        y_sh = round_out(y_sh, inp.out)
        if on_expert:
            on_expert("shared", None, xt, w13, w2, pre["a"], y_sh, shq, shs)
        sh = {"y_shared": y_sh, "h_shared_codes": shq if requant else None, "h_shared_scales": shs,
              "h_shared_bf16": shq if hfmt == "bf16" else None}
    out = combine(y_win, route["dst_row"], inp.topk_w, y_sh)
    res = dict(route)
    res.update({"expert_rows": rows, "y_win": y_win, "h_codes": h_codes,
                "h_scales": h_scales, "h_bf16": h_bf16, "out": round_out(out, inp.out)})
    res.update(sh)
    return res


class _ExpertCache:
    """Dequantised expert weights, kept while a sampled evaluation runs."""

    def __init__(self, inp):
        self.inp = inp
        self.cache = {}

    def get(self, e):
        if e not in self.cache:
            inp = self.inp
            if e == "shared":
                self.cache[e] = (dequant_weight(inp.weight, inp.sh_w13, inp.sh_s13),
                                 dequant_weight(inp.weight, inp.sh_w2, inp.sh_s2))
            else:
                self.cache[e] = (
                    dequant_weight(inp.weight, inp.w13[e], None if inp.s13 is None else inp.s13[e]),
                    dequant_weight(inp.weight, inp.w2[e], None if inp.s2 is None else inp.s2[e]))
        return self.cache[e]


def layer_tokens(inp, tokens):
    """Layer output for a sample of tokens only, each computed on its own.

    tokens: iterable of (s, t).  Because every step after dispatch is row-local
    (the 1x128 requantisation never mixes rows), a token's output is
    sum_j w_j * round_out(FFN_{e_j}(x_t)) (+ round_out(FFN_shared(x_t))),
    with no need for the rest of the batch.  Returns fp64 [n][H] rounded to the
    output format.
    """
    requant = h_format(inp.act)
    cache = _ExpertCache(inp)
    x = np.asarray(inp.x)
    outs = []
    for s, t in tokens:
        if inp.act == "fp8":
            xt = dequant_act_fp8(x[s, t][None, :], np.asarray(inp.x_scale)[s, t][None, :])
        elif inp.act == "bf16":
            xt = codecs.bf16_decode(x[s, t][None, :])
        else:
            xt = np.asarray(x[s, t], dtype=np.float64)[None, :]
        acc = np.zeros(inp.H, dtype=np.float64)
        for j in range(inp.k):
            e = int(inp.ids[s, t, j])
            if e < 0:
                continue
            w13, w2 = cache.get(e)
            y, _, _ = expert_ffn(xt, w13, w2, inp.I, requant)
            acc += float(inp.topk_w[s, t, j]) * round_out(y[0], inp.out)
        if inp.shared_I:
            w13, w2 = cache.get("shared")
            y, _, _ = expert_ffn(xt, w13, w2, inp.shared_I, requant)
            acc += round_out(y[0], inp.out)
        outs.append(round_out(acc, inp.out))
    return np.array(outs)

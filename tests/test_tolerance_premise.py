"""Why the FP8 parity criterion carries an allowance for requantisation steps.

The oracle's own layer output, recomputed with every SwiGLU value moved by at most 1e-5
of itself before the 1x128 FP8 requantisation (a change below the error of any fp32 or
FP8 accumulation over thousands of products; here each value within 1e-5 of an e4m3
rounding midpoint is moved across it), differs from the unperturbed output by more than 2e-2 in the
elementwise statistic |g - r| / max(|r|, rms(r)) at the 128-token decode shape (hidden
7168, intermediate 2048): the change moves a few e4m3 codes by one step, and one step
reaches every output of its row.  So no GEMM that sums in another order than the
oracle's can meet 2e-2 elementwise without the allowance that parity.py derives from
the differing codes (|dh| times |W2|); with that allowance the perturbed output meets
2e-2 per row and elementwise.  (This is the premise of the parity tests' criterion.)
"""
import numpy as np

from combine_top_gate_amd import synth
from oracle import layer
from parity import close_rows, rel_err


def test_tiny_h_perturbation_moves_output_beyond_2e2_elementwise():
    inp = synth.make_inputs("decode128_fp8")
    T, R, H, I, k = inp.S * inp.T_s, inp.S * inp.T_s * inp.k, inp.H, inp.I, inp.k
    y_pert = np.zeros((R, H))
    allow_el = np.zeros((R, H))
    flips = [0]

    def hook(e, rows, x_rows, w13, w2, a, y, hq, hs):
        h = layer.swiglu(a, I)
        # move each value by 1e-5 of itself towards whichever side changes its code, if
        # either does; each block's largest element stays, and with it the block's scale
        keep = np.zeros(h.shape, dtype=bool)
        for b in range(I // 128):
            keep[np.arange(len(h)), b * 128 + np.argmax(np.abs(h[:, b * 128:(b + 1) * 128]), axis=1)] = True
        up, dn = h * (1.0 + 1e-5), h * (1.0 - 1e-5)
        q_up, q_dn = layer.requant_1x128(np.where(keep, h, up))[0], layer.requant_1x128(np.where(keep, h, dn))[0]
        hp = np.where(keep, h, np.where(q_up != hq, up, np.where(q_dn != hq, dn, h)))
        q, s = layer.requant_1x128(hp)
        assert np.array_equal(s, hs)
        deq = layer.dequant_act_fp8(q, s)
        y_pert[rows] = layer.round_out(deq @ w2.T, inp.out)
        # the allowance of parity.py: the effect of the codes that differ, through W2
        dh = np.abs(deq - layer.dequant_act_fp8(hq, hs))
        flips[0] += int((q != hq).sum())
        allow_el[rows] = dh @ np.abs(w2).T

    ref = layer.moe_layer(inp, on_expert=hook)
    out = np.asarray(ref["out"]).reshape(T, H)
    dst = ref["dst_row"]
    pert = layer.round_out(layer.combine(y_pert, dst, inp.topk_w), inp.out).reshape(T, H)
    w = np.abs(np.asarray(inp.topk_w, np.float64).reshape(T, k))
    allow_out = np.einsum("tj,tjh->th", w, allow_el[dst.reshape(T, k)])
    el = rel_err(pert, out)
    row = float(np.max(np.linalg.norm(pert - out, axis=1) / np.linalg.norm(out, axis=1)))
    print(f"  {flips[0]} of {R * I} h codes moved; elementwise {el:.3e}, row relL2 {row:.3e}")
    assert flips[0] > 0
    assert el > 2e-2          # the premise: a 1e-5 change of h fails the bare elementwise bound
    assert row < 2e-2         # while each row stays well within the bound
    assert close_rows(pert, out, 2e-2, allow_el=allow_out)  # and the allowance explains it

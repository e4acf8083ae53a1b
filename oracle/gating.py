"""Top-k softmax gating: which local experts a token goes to, and with what weight.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages state that each token is sent to the experts its gating result names
and collected again afterwards [GC-MoE explainer, "Why Expert Parallelism Is
Inefficient in MoE Decoding"], and list the sparsely-gated MoE layer among the
work the relay-free Ascend design builds on [Relay-free Ascend, "Builds on"].
They do not write the gate out.  Reading taken: keep the k largest logits
(ties go to the lower expert id; slot 0 holds the largest), then take a softmax
over the kept logits only, so the k weights of a token sum to 1.
"""
import math

import numpy as np


def softmax_topk(logits, k):
    """logits [T][E] -> (ids int32 [T][k], weights fp64 [T][k]).

    Plain per-token loops; the ordering key is (-logit, expert id).
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("softmax_topk: need 1 <= k <= E")
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        sel = order[:k]
        zmax = logits[t, sel[0]]
        ex = [math.exp(logits[t, e] - zmax) for e in sel]
        tot = math.fsum(ex)
        for j, e in enumerate(sel):
            ids[t, j] = e
            w[t, j] = ex[j] / tot
    return ids, w


def router_logits(x, wr):
    """Router scores: logits[t][e] = sum_h x[t][h] * wr[e][h], in fp64.

    x [T][H] and wr [E][H] are the values of the bf16 inputs (codecs.bf16_decode).
    The pages name the gating result, not the router; this is the plain linear
    router of the sparsely-gated MoE layer the relay-free Ascend page builds on.
    """
    return np.asarray(x, dtype=np.float64) @ np.asarray(wr, dtype=np.float64).T


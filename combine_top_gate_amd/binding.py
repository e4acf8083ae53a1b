"""Thin ctypes binding of libctg_moe.so (the C-ABI in include/ctg_moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
torch supplies device memory (tensor.data_ptr()) and the current HIP stream.
The binding fails loudly when the library has not been built: there is no other
implementation to fall back on.
"""
import ctypes
import os
import re

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libctg_moe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ctg_moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = range(4)
MOE_SCHED_FENCE, MOE_SCHED_SENTINEL = range(2)
MOE_BUF_WINDOW, MOE_BUF_WSCALE, MOE_BUF_H, MOE_BUF_HSCALE, MOE_BUF_Y = range(5)
MOE_DEVERR_BAD_ID, MOE_DEVERR_TIMEOUT = 0x1, 0x2
(MOE_OPT_PERSISTENT_GEMM, MOE_OPT_TOKEN_TILES, MOE_OPT_QUEUE, MOE_OPT_TILED_GEMM,
 MOE_OPT_SENTINEL_SPIN, MOE_OPT_SENTINEL_STALL, MOE_OPT_TILED_MFMA, MOE_OPT_POISON, MOE_OPT_EPOCH,
 MOE_OPT_DISPATCH_DELAY, MOE_OPT_FUSED_COMBINE) = range(11)

_DTYPE = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "fp4": MOE_FP4_E2M1}


class MoeConfig(ctypes.Structure):
    _fields_ = [("n_src", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("act", ctypes.c_int),
                ("weight", ctypes.c_int), ("out", ctypes.c_int), ("sched", ctypes.c_int),
                ("dispatch_cus", ctypes.c_int32)]


WEIGHT_FIELDS = ("w13", "s13", "w2", "s2", "sh_w13", "sh_s13", "sh_w2", "sh_s2")


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS] + [("packed", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_HIP",
           4: "MOE_ERR_DEVICE"}

_lib = None


def header_functions():
    """Names of the functions declared in include/ctg_moe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\s*\*|size_t|int64_t)\s*(moe_\w+)\s*\(", text, re.M)))


def load():
    """Loads libctg_moe.so and declares its prototypes (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m combine_top_gate_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
    st = ctypes.c_int
    proto = {
        "moe_create": (st, [P(MoeConfig), P(VP)]),
        "moe_destroy": (st, [VP]),
        "moe_dispatch": (st, [VP, I32, P(VP), P(VP), VP, VP]),
        "moe_grouped_gemm": (st, [VP, P(MoeWeights), VP]),
        "moe_combine": (st, [VP, VP, VP, VP]),
        "moe_combine_fp8": (st, [VP, VP, VP, VP, VP]),
        "moe_layer": (st, [VP, I32, P(VP), P(VP), VP, VP, P(MoeWeights), VP, VP]),
        "moe_get_routing": (st, [VP, VP, VP, VP, VP, VP]),
        "moe_copy_buffer": (st, [VP, ctypes.c_int, VP, ctypes.c_size_t, VP]),
        "moe_last_device_error": (st, [VP, P(ctypes.c_uint32)]),
        "moe_packed_sizes": (st, [P(MoeConfig), P(ctypes.c_size_t)]),
        "moe_pack_weights": (st, [VP, P(MoeWeights), P(MoeWeights), VP]),
        "moe_set_timing": (st, [VP, I32]),
        "moe_set_option": (st, [VP, ctypes.c_int, I32]),
        "moe_read_timing": (st, [VP, P(ctypes.c_float), P(I32)]),
        "moe_router_logits": (st, [I32, I32, I32, VP, VP, VP, VP]),
        "moe_topk_softmax": (st, [I32, I32, I32, VP, VP, VP, VP]),
        "moe_gate_workspace_bytes": (ctypes.c_size_t, [I32, I32, I32]),
        "moe_mfma_fp8_probe": (ctypes.c_int64, [VP, I32, I32, VP]),
        "moe_mfma_dot16x16": (st, [I32, VP, VP, VP, VP]),
        "moe_gate": (st, [I32, I32, I32, I32, VP, VP, VP, ctypes.c_size_t, VP, VP, VP, VP]),
        "moe_gate_noalloc": (st, [I32, I32, I32, I32, VP, VP, VP, VP, VP, VP]),
        "moe_status_str": (ctypes.c_char_p, [st]),
        "moe_last_error_message": (ctypes.c_char_p, []),
    }
    for name, (res, args) in proto.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _check(status):
    if status != MOE_OK:
        raise MoeError(status, _lib.moe_last_error_message().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def make_config(S, max_tokens, H, I, E, k, act="fp8", weight="fp8", out="bf16", shared_I=0,
                sched=MOE_SCHED_FENCE, dispatch_cus=0):
    return MoeConfig(S, max_tokens, H, I, E, k, shared_I, _DTYPE[act], _DTYPE[weight], _DTYPE[out],
                     sched, dispatch_cus)


def router_logits(x, wr, logits=None):
    """logits [T][E] fp32 = x [T][H] bf16 . wr [E][H] bf16^T on the current stream."""
    lib = load()
    T, H = x.shape
    E = wr.shape[0]
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib.moe_router_logits(T, H, E, _ptr(x), _ptr(wr), _ptr(logits), _stream()))
    return logits


def gate(x, wr, k, workspace=None, want_logits=False):
    """(ids, w[, logits]) for x [T][H] bf16 and wr [E][H] bf16 through the fused gate.

    workspace: a device tensor of at least gate_workspace_bytes(T, H, E) bytes, or None to
    allocate one here."""
    lib = load()
    T, H = x.shape
    E = wr.shape[0]
    need = lib.moe_gate_workspace_bytes(T, H, E)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=x.device)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.moe_gate(T, H, E, k, _ptr(x), _ptr(wr), _ptr(workspace), nbytes, _ptr(logits), _ptr(ids),
                        _ptr(w), _stream()))
    return (ids, w, logits) if want_logits else (ids, w)


def gate_noalloc(x, wr, k, ids=None, w=None, logits=None):
    """The fused gate with its partial sums in the library's fixed scratch (no workspace,
    no allocation inside the call); ids [T][k] int32, w [T][k] fp32 and logits [T][E] fp32
    (optional) are caller tensors, allocated here when not given.  Returns (ids, w, logits)."""
    lib = load()
    T, H = x.shape
    E = wr.shape[0]
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(lib.moe_gate_noalloc(T, H, E, k, _ptr(x), _ptr(wr), _ptr(logits), _ptr(ids), _ptr(w), _stream()))
    return ids, w, logits


def mfma_fp8_probe(sink, blocks, iters):
    """Launch the FP8 MFMA probe on the current stream; returns the flops it performs."""
    flops = load().moe_mfma_fp8_probe(_ptr(sink), blocks, iters, _stream())
    if flops < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, _lib.moe_last_error_message().decode())
    return flops


def mfma_dot16x16(a_codes, b_codes, a_fp4=False):
    """One scaled MFMA with unit scales: out[i][j] = the instruction's own sum of
    a[i][k] * b[j][k] over 128 k, for a [16][128] e4m3 codes (or e2m1 codes, one per byte,
    with a_fp4) and b [16][128] e4m3 codes, uint8 on the device; returns fp32 [16][16]."""
    if tuple(a_codes.shape) != (16, 128) or tuple(b_codes.shape) != (16, 128):
        raise ValueError("a and b must be [16][128] code arrays")
    a, b = a_codes.contiguous(), b_codes.contiguous()
    out = torch.empty((16, 16), dtype=torch.float32, device=a.device)
    _check(load().moe_mfma_dot16x16(MOE_FP4_E2M1 if a_fp4 else MOE_FP8_E4M3, _ptr(a), _ptr(b), _ptr(out), _stream()))
    return out


def gate_workspace_bytes(T, H, E):
    return load().moe_gate_workspace_bytes(T, H, E)


def topk_softmax(logits, k):
    """(ids [T][k] int32, w [T][k] fp32) from logits [T][E] fp32 on the current stream."""
    lib = load()
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib.moe_topk_softmax(T, E, k, _ptr(logits), _ptr(ids), _ptr(w), _stream()))
    return ids, w


class DeviceInputs:
    """An input set copied to device tensors (plain uploads, no arithmetic)."""

    def __init__(self, inp, device="cuda"):
        def up(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:  # bf16 bit patterns
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)
        self.inp = inp
        self.x = [up(inp.x[s]) for s in range(inp.S)]
        self.x_scale = [up(inp.x_scale[s]) for s in range(inp.S)] if inp.x_scale is not None else None
        self.ids = up(inp.ids)
        self.topk_w = up(inp.topk_w)
        self.w13, self.s13, self.w2, self.s2 = up(inp.w13), up(inp.s13), up(inp.w2), up(inp.s2)
        self.sh = [up(a) for a in (inp.sh_w13, inp.sh_s13, inp.sh_w2, inp.sh_s2)]
        self.weights = MoeWeights(*[_ptr(t).value for t in
                                    (self.w13, self.s13, self.w2, self.s2, *self.sh)], 0)
        self.packed = None
        out_dtype = torch.bfloat16 if inp.out == "bf16" else torch.float32
        self.out = torch.empty((inp.S, inp.T_s, inp.H), dtype=out_dtype, device=device)


class Moe:
    """One context of the library (owns the workspace)."""

    def __init__(self, cfg):
        self.lib = load()
        self.cfg = cfg
        self.ctx = ctypes.c_void_p()
        _check(self.lib.moe_create(ctypes.byref(cfg), ctypes.byref(self.ctx)))

    @classmethod
    def for_inputs(cls, inp, max_tokens=None, sched=MOE_SCHED_FENCE, dispatch_cus=0):
        cfg = make_config(inp.S, inp.T_s if max_tokens is None else max_tokens, inp.H, inp.I, inp.E,
                          inp.k, inp.act, inp.weight, inp.out, inp.shared_I, sched, dispatch_cus)
        return cls(cfg)

    def close(self):
        if self.ctx:
            self.lib.moe_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ptr_array(ts):
        arr = (ctypes.c_void_p * max(1, len(ts or [])))()
        for i, t in enumerate(ts or []):
            arr[i] = t.data_ptr()
        return arr

    def dispatch(self, T_s, x, x_scale, ids):
        xa, sa = self._ptr_array(x), self._ptr_array(x_scale)
        _check(self.lib.moe_dispatch(self.ctx, T_s, xa, sa if x_scale is not None else None,
                                     _ptr(ids), _stream()))

    def grouped_gemm(self, weights):
        _check(self.lib.moe_grouped_gemm(self.ctx, ctypes.byref(weights), _stream()))

    def combine(self, topk_w, out):
        _check(self.lib.moe_combine(self.ctx, _ptr(topk_w), _ptr(out), _stream()))

    def combine_fp8(self, topk_w, out, out_scale):
        """The combine with its output requantised to e4m3 codes (uint8 [S][T_s][H]) and
        1x128 fp32 scales ([S][T_s][H/128])."""
        _check(self.lib.moe_combine_fp8(self.ctx, _ptr(topk_w), _ptr(out), _ptr(out_scale), _stream()))

    def layer(self, T_s, x, x_scale, ids, topk_w, weights, out):
        xa, sa = self._ptr_array(x), self._ptr_array(x_scale)
        _check(self.lib.moe_layer(self.ctx, T_s, xa, sa if x_scale is not None else None, _ptr(ids),
                                  _ptr(topk_w), ctypes.byref(weights), _ptr(out), _stream()))

    def run(self, d):
        """The whole layer on a DeviceInputs set; returns d.out."""
        self.layer(d.inp.T_s, d.x, d.x_scale, d.ids, d.topk_w, d.weights, d.out)
        return d.out

    def routing(self, S, T_s, k, E):
        dev = "cuda"
        cnt = torch.empty((S, E), dtype=torch.int32, device=dev)
        off = torch.empty((S, E), dtype=torch.int32, device=dev)
        dst = torch.empty((S, T_s, k), dtype=torch.int32, device=dev)
        src = torch.empty((S * T_s * k,), dtype=torch.int32, device=dev)
        _check(self.lib.moe_get_routing(self.ctx, _ptr(cnt), _ptr(off), _ptr(dst), _ptr(src), _stream()))
        return cnt, off, dst, src

    def buffer(self, which, nbytes):
        t = torch.empty((max(1, nbytes),), dtype=torch.uint8, device="cuda")
        _check(self.lib.moe_copy_buffer(self.ctx, which, _ptr(t), nbytes, _stream()))
        return t[:nbytes]

    def device_error(self):
        bits = ctypes.c_uint32()
        _check(self.lib.moe_last_device_error(self.ctx, ctypes.byref(bits)))
        return bits.value

    def pack(self, d):
        """Packs d's row-major weights into new device buffers; d.weights then points at them."""
        sizes = (ctypes.c_size_t * 8)()
        _check(self.lib.moe_packed_sizes(ctypes.byref(self.cfg), sizes))
        bufs = [torch.empty((max(1, n),), dtype=torch.uint8, device="cuda") if n else None for n in sizes]
        dst = MoeWeights(*[_ptr(b).value for b in bufs], 1)
        _check(self.lib.moe_pack_weights(self.ctx, ctypes.byref(d.weights), ctypes.byref(dst), _stream()))
        d.packed = bufs
        d.row_major_weights = d.weights
        d.weights = dst
        return d

    def set_option(self, opt, value):
        _check(self.lib.moe_set_option(self.ctx, opt, value))

    def set_timing(self, max_calls):
        _check(self.lib.moe_set_timing(self.ctx, max_calls))

    def read_timing(self):
        ms = (ctypes.c_float * 5)()
        n = ctypes.c_int32()
        _check(self.lib.moe_read_timing(self.ctx, ms, ctypes.byref(n)))
        return list(ms), n.value

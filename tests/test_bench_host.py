"""Host-side pieces of bench.py (no GPU): the multi-GPU refusal, the algorithmic byte model
against the 128-token decode layer's figure derived by hand, and the code hash that ties
the committed counter summary to the kernel's code."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from combine_top_gate_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_decode_layer():
    """1.461 GB for the 128-token FP8 decode layer with all 32 experts active: weights 32 x
    (2 x 2048 x 7168 + 7168 x 2048 bytes + their 128x128 fp32 scales) = 1.4096 GB, plus
    dispatch, GEMM activations and combine (the hand count of the layer's bytes)."""
    inp = synth.make_inputs("decode128_fp8")
    cnt = np.zeros((inp.S, inp.E), np.int64)
    for s in range(inp.S):
        ids = inp.ids[s].reshape(-1)
        cnt[s] = np.bincount(ids[ids >= 0], minlength=inp.E)
    nb, flops = bench.algorithmic_bytes(inp, cnt)
    w = 32 * (2 * 2048 * 7168 + 7168 * 2048 + (4096 // 128) * (7168 // 128) * 4 + (7168 // 128) * (2048 // 128) * 4)
    assert abs(w - 1.4096e9) < 1e6
    assert abs(nb["layer"] - 1.461e9) / 1.461e9 < 5e-3, nb["layer"]
    assert nb["gemm1"] + nb["gemm2"] > w
    assert flops == 6 * 1024 * 2048 * 7168


def test_code_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {  // one\n  return x + 1;\n}\n")
    b.write_text("// a new header line\n\nint f(int x) {  // two\n  return x + 1;   \n}\n")
    c.write_text("int f(int x) {  // one\n  return x + 2;\n}\n")
    assert bench.code_sha256(str(a)) == bench.code_sha256(str(b))
    assert bench.code_sha256(str(a)) != bench.code_sha256(str(c))
    # a list of files: a change in any of them changes the hash
    assert bench.code_sha256([str(a), str(a)]) == bench.code_sha256([str(b), str(a)])
    assert bench.code_sha256([str(a), str(a)]) != bench.code_sha256([str(a), str(c)])
    assert bench.code_sha256(str(a)) == bench.code_sha256([str(a)])

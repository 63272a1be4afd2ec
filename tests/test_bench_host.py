"""Host-side parts of bench.py (no GPU): the one-GPU contract and the byte counts behind the
roofline figures, checked against the format's definition written out here."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a run that was not made


def test_gate_up_bytes_of_the_decode_layer():
    """Gate and up of one MXFP4 expert: 2 x (4096 x 2048) E2M1 codes at half a byte each plus one
    E8M0 byte per 32 values; eight experts per one-token layer."""
    wl = synth.WORKLOADS["decode"]
    per_expert = 2 * (4096 * 2048 // 2) + 2 * (4096 * 2048 // 32)
    assert per_expert == 8_912_896
    assert bench.gate_up_bytes(wl, 8) == 8 * per_expert == 71_303_168


def test_layer_bytes_of_the_decode_layer():
    """A one-token layer moves at least the touched experts' three matrices with their scales, the
    fp32 router rows of all 288 experts, and x and y in bf16."""
    wl = synth.WORKLOADS["decode"]
    fd = 4096 * 2048
    expert = 3 * fd // 2 + 3 * fd // 32
    router = 288 * 4096 * 4
    xy = 2 * 4096 * 2
    assert bench.algorithmic_layer_bytes(wl, 8, 1) == 8 * expert + router + xy == 111_689_728


def test_layer_bytes_of_the_nvfp4_layer():
    """NVFP4: E2M1 codes plus one E4M3 byte per 16 values (the tensor scales are negligible)."""
    wl = synth.WORKLOADS["nvfp4_decode"]
    fd = 6144 * 2048
    expert = 3 * fd // 2 + 3 * fd // 16
    assert bench.algorithmic_layer_bytes(wl, 8, 1) == 8 * expert + 256 * 6144 * 4 + 2 * 6144 * 2

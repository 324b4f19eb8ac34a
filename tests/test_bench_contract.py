"""bench.py host logic on the CPU: the one-GPU guard and the kernel-code digests that tie a
committed counter record to the exact generated code it was taken on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


SOURCE = ("// @@section common\nA\n"
          "// @@section cgtp_conv_fwd\nB\n"
          "// @@section cgtp_conv_fwd_split2\nC\n"
          "// @@section cgtp_conv_bwd\nD\n")


def test_kernel_digest_sections():
    base = bench.kernel_digest(SOURCE, "cgtp_conv_fwd")
    split = bench.kernel_digest(SOURCE, "cgtp_conv_fwd_split2")
    assert base and split and base != split
    assert bench.kernel_digest(SOURCE, "cgtp_conv_missing") is None
    # a split entry point runs its base section's code: a change there changes its digest too
    changed = SOURCE.replace("\nB\n", "\nB2\n")
    assert bench.kernel_digest(changed, "cgtp_conv_fwd_split2") != split
    assert bench.kernel_digest(changed, "cgtp_conv_bwd") == bench.kernel_digest(SOURCE, "cgtp_conv_bwd")
    assert bench.split_kernel("cgtp_conv_fwd", 1) == "cgtp_conv_fwd"
    assert bench.split_kernel("cgtp_conv_fwd", 4) == "cgtp_conv_fwd_split4"

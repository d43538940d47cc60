"""Host-side logic of bench.py: the one-GPU guard, the algorithmic roofline model and the
rule that a rocprofv3 counter summary is used only for the kernel build it was taken on."""
import os
import subprocess
import sys

import numpy as np

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


def test_algorithmic_model_of_a_token_head():
    # one token-head of the Kimi-Linear layer (d = 128, chunk 64): q, k, v read in bf16, the
    # per-channel log-decay and the scalar beta read in fp32, o written in fp32
    d, C = 128, 64
    bf16, f32 = 2, np.dtype(np.float32).itemsize
    assert bench.BYTES_PER_TOKEN_HEAD == 3 * d * bf16 + d * f32 + f32 + d * f32 == 1796
    # state products W S, Qg S and Kd^T U (2 d^2 flops each) plus the lower-triangular
    # in-chunk products over C columns
    assert bench.FLOPS_PER_TOKEN_HEAD == 3 * 2 * d * d + C * (3 * d + 2 * d) == 139264


def _summary(path, build_hash, value):
    with open(path, "w") as f:
        f.write("# comment: with a colon\nkernel: k<1, 2>\nkernel_build_sha256_16: %s\n"
                "hbm_bytes_per_launch: %s\n" % (build_hash, value))


def test_counter_summary_only_for_the_current_build(tmp_path):
    cur = bench.build_hash(bench.CHUNK_BUILD_FILES)
    assert len(cur) == 16
    p = str(tmp_path / "s.txt")
    _summary(p, cur, "965000000")
    assert bench.profile_value(p, "hbm_bytes_per_launch") == 965000000.0
    assert bench.profile_value(p, "absent_key") is None
    _summary(p, "0" * 16, "965000000")
    assert bench.profile_value(p, "hbm_bytes_per_launch") is None
    _summary(p, cur, "n/a")
    assert bench.profile_value(p, "hbm_bytes_per_launch") is None
    assert bench.profile_value(str(tmp_path / "missing.txt"), "hbm_bytes_per_launch") is None


def test_build_hash_covers_source_and_flags(tmp_path):
    a, b = tmp_path / "a", tmp_path / "b"
    a.write_bytes(b"kernel source")
    b.write_bytes(b"flags one")
    h1 = bench.build_hash([str(a), str(b)])
    b.write_bytes(b"flags two")
    assert bench.build_hash([str(a), str(b)]) != h1
    names = [os.path.basename(x) for x in bench.CHUNK_BUILD_FILES]
    assert names == ["kda_chunk.hip", "build.py"]


def test_algorithmic_bytes_of_the_workloads():
    # long context: 1,048,576 tokens x 32 heads at 1,796 B per token-head + hT (32 x 64 KiB)
    assert bench.chunk_alg_bytes(1 << 20, 32, 1) == (1 << 20) * 32 * 1796 + 32 * 128 * 128 * 4
    assert abs(bench.chunk_alg_bytes(1 << 20, 32, 1) / 1e6 - 60265.9) < 0.1
    # Kimi-Linear layer: 950.0 MB; varlen packed with h0 read and hT written: 1,916.8 MB
    assert abs(bench.chunk_alg_bytes(16384, 32, 4) / 1e6 - 950.0) < 0.1
    assert abs(bench.chunk_alg_bytes(32768, 32, 8, h0=True) / 1e6 - 1916.8) < 0.1
    # fp32 q/k/v at d = 64: 3 x 256 + 256 + 4 + 256 bytes per token-head
    assert bench.chunk_alg_bytes(256, 2, 1, d=64, qkv_bytes=4) == 256 * 2 * (3 * 256 + 256 + 4 + 256) + 2 * 64 * 64 * 4


def test_error_ratios():
    ref = np.array([[3.0, -4.0], [0.0, 0.0]])  # RMS 2.5
    e = bench.errors(ref + np.array([[0.05, 0.0], [0.0, -0.02]]), ref, tol=0.02)
    assert e["max_err_over_rms"] == 0.02 and e["within_tolerance"]
    assert abs(e["rms_err_over_rms"] - np.sqrt((0.05 ** 2 + 0.02 ** 2) / 4) / 2.5) < 1e-7
    e = bench.errors(ref + 1e-3, ref, tol=1e-4, absolute=True)
    assert not e["within_tolerance"] and e["max_abs_err"] == 1e-3

"""Host-side parts of bench.py (no GPU): the one-GPU refusal, the FLOP count,
and the rule that the roofline's HBM traffic comes from the committed
rocprofv3 summary only while the kernel source is the one it was taken on."""
import hashlib
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = os.path.join(ROOT, "paged_kv_attention_page_amd", "csrc", "k_attn_bf16.hip")
SUMMARY = os.path.join(ROOT, "profiles", "k_attn_bf16_wan_kp4_hbm_traffic.txt")


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus %d" % n in r.stderr
    assert r.stdout == ""          # no JSON line


def test_attention_flops_counts_both_contractions():
    # 2 FLOP per multiply-add, Q K^T and P V: 4 * N_q * N_k * d * H
    assert bench.attention_flops(4680, 54600, 128, 12) == 4 * 4680 * 54600 * 128 * 12
    assert bench.attention_flops(4680, 54600, 128, 12) == pytest.approx(1.5700e12, rel=1e-4)


def _summary(tmp_path, digest, nbytes):
    p = tmp_path / "traffic.txt"
    p.write_text("# comment: with a colon\nkernel: k_attn_bf16\nkernel_source_sha256: %s\n"
                 "bytes_per_launch: %d\n" % (digest, nbytes))
    return str(p)


def test_traffic_is_read_only_for_the_kernel_it_was_taken_on(tmp_path):
    src = b"kernel source v1"
    good = _summary(tmp_path, hashlib.sha256(src).hexdigest(), 123456)
    assert bench.load_traffic(good, src) == 123456
    assert bench.load_traffic(good, b"kernel source v2") is None     # source changed since
    assert bench.load_traffic(str(tmp_path / "missing.txt"), src) is None
    assert bench.load_traffic(None, src) is None


def test_committed_summary_matches_the_committed_kernel():
    """The committed counter summary was taken on the kernel source in the tree
    (re-take it after any change to the kernel, or the bench reports null)."""
    with open(KERNEL, "rb") as f:
        src = f.read()
    nbytes = bench.load_traffic(SUMMARY, src)
    assert nbytes is not None, "profiles/ summary is stale for k_attn_bf16.hip"
    assert nbytes > 0

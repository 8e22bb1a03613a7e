"""The committed rocprofv3 summaries describe the kernels as they are built now.

Each summary under profiles/ records a hash of the kernel source it was taken
from; a kernel change without a new profile fails here.  bench.py reads
traffic and clock figures out of these summaries only while the hashes match,
and the figures it reads must be consistent with the algorithmic bytes.
"""
import glob
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_head_attention_amd", "csrc")


def _recorded_hashes(path):
    """(source file name, recorded digest) pairs found in one summary."""
    text = open(path).read()
    found = re.findall(r"# (\w+\.hip) sha256\[:16\] = ([0-9a-f]{16})", text)
    keys = {"attn_source_sha256": "attn_fwd.hip", "prologue_source_sha256": "qknorm_rope.hip"}
    for key, name in keys.items():
        found += [(name, d) for d in re.findall(rf"^{key}: ([0-9a-f]{{16}})$", text, flags=re.M)]
    return found


SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))


def test_profiles_exist():
    names = {os.path.basename(p) for p in SUMMARIES}
    for n in ("attn_fwd_ws8_kernel_trace.txt", "attn_fwd_hbm_counters.txt", "attn_fwd_sq_counters.txt",
              "qkv_proj_bf16_ws2_kernel_trace.txt", "qkv_proj_fp8_ws2_kernel_trace.txt",
              "qkv_proj_bf16_ws2_sq_counters.txt", "qkv_proj_fp8_ws2_sq_counters.txt"):
        assert n in names


@pytest.mark.parametrize("path", SUMMARIES, ids=os.path.basename)
def test_profile_matches_current_source(path):
    pairs = _recorded_hashes(path)
    assert pairs, f"{os.path.basename(path)} records no source hash"
    for name, digest in pairs:
        assert digest == bench.source_digest(os.path.join(CSRC, name)), \
            f"{os.path.basename(path)} was taken from another version of {name}"


def test_profiles_name_their_command():
    for path in SUMMARIES:
        head = open(path).read(4000)
        assert re.search(r"^# commands?: .*rocprofv3 ", head, flags=re.M), os.path.basename(path)


def test_counter_traffic_is_read_and_plausible():
    """HBM traffic per ws8 call: the attention reads at least its algorithmic
    bytes (q, k, v read, out written: 235 MB) and re-streams K/V per XCD; the
    prologue's counted traffic equals its algorithmic bytes within 1%."""
    att = bench.read_counter_summary("ws8")
    assert att is not None and 235e6 <= att <= 2e9
    pro = bench.read_prologue_traffic("ws8")
    assert pro is not None
    assert abs(pro / bench.prologue_bytes(7, 32768) - 1) < 0.01
    assert bench.read_counter_summary("ws2") is None     # recorded for ws8 only


def test_sq_summary_is_read():
    sq = bench.read_sq_summary("ws8")
    assert sq is not None and 1.0 < sq["profile_sclk_ghz"] < 2.5

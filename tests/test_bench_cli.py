"""bench.py's command line on the CPU: the single-GPU refusal, the workload
list, and the algorithmic work formulas its rooflines divide by (CPU only)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run


def test_help_lists_every_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0
    for w in ("c0", "c1", "c2", "c3", "c4a", "c4b", "attn_decode", "attn_prefill"):
        assert w in r.stdout


@pytest.mark.parametrize("fmt", ["block128", "mx", "mxfp4"])
def test_traffic_entries_match_their_formats(fmt):
    """A stored counter entry is used only while the GEMM source is unchanged;
    the entries exist for the decode and prefill layers of every format."""
    b = _bench()
    for w in ("c1", "c2"):
        key = w if fmt == "block128" else f"{w}-{fmt}"
        assert key in b.TRAFFIC
        t = b.TRAFFIC[key]
        assert t["copy_write_kib"] == 1048576.0
        assert 500000 < t["copy_fetch_kib"] < 550000   # 128-byte reads counted as 64 bytes


def test_decode_gateup_traffic_matches_algorithmic_bytes():
    """The decode gate/up GEMM reads every touched expert's weights once: its
    scaled HBM bytes stay within 1 % of the algorithmic bytes (a check of the
    stored counters against the formula, both from committed numbers)."""
    b = _bench()
    t = b.TRAFFIC["c1"]
    hbm = (t["fetch_kib"] * 1048576.0 / t["copy_fetch_kib"] + t["write_kib"]) * 1024
    E, d, f, T = 32, 2944, 2944, 64
    weights = E * d * 2 * f + 4 * E * (d // 128) * (2 * f // 128) + 2 * E * 2 * f
    assert abs(hbm - weights) / weights < 0.01


def test_event_steps_are_sampled_inside_the_timed_steps():
    """Per-kernel events go on every N-th timed step (at least one), all of
    them inside the timed range."""
    b = _bench()
    assert b.sampled_steps(50, 5) == [4, 9, 14, 19, 24, 29, 34, 39, 44, 49]
    assert b.sampled_steps(3, 5) == [2]
    assert b.sampled_steps(4, 1) == [0, 1, 2, 3]
    assert b.sampled_steps(7, 0) == list(range(7))


def test_decode_attention_traffic_matches_algorithmic_bytes():
    """One decode-attention call of the bench batch (64 seeded ragged sequences,
    sum of kv_len 195045: K and V rows of 8 heads x 64 dims in bf16, plus q and
    out = 400500736 bytes) reads every cached row once: the stored counters,
    scaled, stay within 3 % of that (the rest is the partial-result records)."""
    b = _bench()
    t = b.ATTN_TRAFFIC["attn_decode"]
    alg = 195045 * 8 * 64 * 2 * 2 + 2 * 64 * 64 * 64 * 2
    assert alg == 400500736
    hbm = b._scaled_bytes(t)
    assert alg <= hbm < 1.03 * alg


def test_prefill_attention_writes_each_output_once():
    """The stored prefill counters: WRITE_SIZE is exactly the bf16 output
    (8192 x 64 x 64), and the scaled reads are at least q, k and v once."""
    b = _bench()
    t = b.ATTN_TRAFFIC["attn_prefill"]
    out = 8192 * 64 * 64 * 2
    assert t["write_kib"] * 1024 == out
    read = t["fetch_kib"] * (1 << 20) / t["copy_fetch_kib"] * 1024
    assert read >= out + 2 * 8192 * 8 * 64 * 2


def test_stored_counters_are_keyed_to_the_present_sources():
    """The bench line reports stored HBM counters only while the kernel source
    they were taken on is unchanged, so every committed entry must be keyed to
    the present source: a change to the GEMM or attention source (a comment
    included) needs the counter runs again, or, for a byte-identical build,
    the entries moved to the new hash."""
    b = _bench()
    gemm = b.gemm_src_sha()
    for key, t in b.TRAFFIC.items():
        assert t["gemm_sha256"] == gemm, key
    attn = b.src_sha(b.ATTN_SRC)
    for key, t in b.ATTN_TRAFFIC.items():
        assert t["attn_sha256"] == attn, key

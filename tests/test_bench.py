"""bench.py's host-side bookkeeping (no GPU): the algorithmic work counts that every
roofline figure divides by, checked against direct enumeration on small batches; the gating
of committed counter figures on the kernel sources; and the one-GPU contract."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import make_decode_case, make_prefill_case  # noqa: E402


@pytest.mark.parametrize("lens,window,page,kv_dtype,dvo,out", [
    ([37, 64, 0, 300], 0, 16, "bf16", 512, "fp32"),
    ([37, 64, 0, 300], 20, 3, "fp8", 512, "bf16"),
    ([100, 1, 17], 33, 1, "nvfp4", 256, "bf16"),
])
def test_decode_bytes_count_visible_keys_pages_and_queries(lens, window, page, kv_dtype, dvo, out):
    c = make_decode_case(lens, 6, 2, 512, page, head_dim_vo=dvo, kv_dtype=kv_dtype,
                         window=window, out_dtype=out, seed=3)
    esz = {"bf16": 2.0, "fp8": 1.0, "nvfp4": 0.5 + 1.0 / 16}[kv_dtype]
    osz = 4 if out == "fp32" else 2
    want = 0
    for b, L in enumerate(lens):
        visible = [t for t in range(L) if window <= 0 or t > L - 1 - window]
        pages = {t // page for t in visible}  # logical pages holding a visible key
        want += int(2 * len(visible) * (512 + dvo) * esz)
        want += 6 * (512 * 2 + dvo * osz) + 4 * len(pages)
    want += 4 * (2 * len(lens) + 1)
    assert bench.decode_algorithmic_bytes(c) == want


@pytest.mark.parametrize("qo,kv,causal,window,dvo", [
    ([5, 0, 9], [20, 3, 9], True, 0, 512),
    ([7, 4], [30, 4], True, 6, 256),
    ([3, 2], [8, 5], False, 0, 512),
])
def test_prefill_flops_count_every_visible_query_key_pair(qo, kv, causal, window, dvo):
    c = make_prefill_case(qo, kv, 4, 2, 512, 16, head_dim_vo=dvo, causal=causal,
                          window=window, seed=4)
    pairs = 0
    for q_len, L in zip(qo, kv):
        pos = np.arange(L - q_len, L)[:, None]  # query positions
        t = np.arange(L)[None, :]                # key positions
        seen = np.ones((q_len, L), bool)
        if causal:
            seen &= t <= pos
        if window > 0:
            seen &= t > pos - window
        pairs += int(seen.sum())
    assert bench.prefill_algorithmic_flops(c) == pairs * 4 * 2 * (512 + dvo)


def test_counter_figures_are_reported_only_for_the_kernel_sources_they_were_taken_on(
        tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    entries = {
        "gqa_decode": {"kernel_source_hash": bench.kernel_source_hash("decode"),
                       "hbm_bytes_per_launch": 123},
        "fp8_decode": {"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 456},
    }
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(entries))
    hashes = {f: bench.kernel_source_hash(f) for f in ("decode", "prefill")}
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda fam: hashes[fam])
    assert bench.traffic_for("gqa_decode") == 123
    assert bench.traffic_for("fp8_decode") is None  # taken on other kernel sources
    assert bench.traffic_for("nvfp4_decode") is None  # no entry


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "decode", ["k.hip"])
    src.write_text("int f() { return 1; }  // one\n")
    h0 = bench.kernel_source_hash("decode")
    src.write_text("/* a note */\nint f() {\n  return 1;  // another\n}\n")
    assert bench.kernel_source_hash("decode") == h0
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash("decode") != h0


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_settle_runs_nothing_when_its_time_is_zero():
    """The headline line (and --settle-ms 0) must run exactly the requested warmup steps."""
    calls = []
    assert bench.settle(lambda: calls.append(1), 0.0) == 0
    assert calls == []

"""Host-side checks of bench.py (no GPU): the single-GPU guard, the byte and
flop formulas of the roofline, and the counter-summary arithmetic."""

import csv
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from masked_verification_attention_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_by_parts():
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=2, with_logits=False)
    B, Tq, Hq, Hkv, D, S = 2, cfg.Tq, cfg.Hq, cfg.Hkv, cfg.D, cfg.S
    kv = int(x["cache_len"].sum()) * Hkv * D * 2 * 2          # K and V of every cached row, bf16
    W = (Tq + 31) // 32
    expect = (kv + S * Hkv * D * 4 + B * Tq * Hq * D * 2 + B * Tq * Hkv * D * 4 + B * Tq * W * 4 + B * W * 4
              + B * Tq * Hq * (D + 1) * 4)
    assert bench.attention_algorithmic_bytes(cfg, x) == expect
    # a bf16 output halves the output values; the lse stays fp32
    assert bench.attention_algorithmic_bytes(cfg, x, out_es=2) == expect - B * Tq * Hq * D * 2


def test_flops_count_visible_pairs():
    # a chain of 3 lookahead rows over a 10-key prefix: every row sees the prefix and itself
    cfg = wl.CONFIGS["c2_la_7b"].with_(T=3, Hq=2, Hkv=2, D=64)
    x = wl.generate(cfg, B=1, L=(10, 10), with_logits=False)
    assert bench.attention_flops(cfg, x) == 3 * (10 + 1) * 2 * 4 * 64
    # multi-stream rows of a 3-node tree (root + 2 children) with 1 stream per node: a main row
    # sees the prefix and its depth + 1 path rows, stream j of a node j more
    m = wl.CONFIGS["c6_msa_1b"].with_(gamma=1, branch=2, T=3, Hq=1, Hkv=1)
    xm = wl.generate(m, B=1, L=(5, 5), with_logits=False)
    visible = sum(5 + d + 1 + j for d in (0, 1, 1) for j in range(2))
    assert bench.attention_flops(m, xm) == visible * 1 * 4 * m.D


def test_counter_summary_scales_by_the_copy(tmp_path):
    rows = [("__amd_rocclr_copyBuffer", 1 << 20, "FETCH_SIZE", 512 * 1024.0),
            ("__amd_rocclr_copyBuffer", 1 << 20, "WRITE_SIZE", 1024 * 1024.0),
            ("__amd_rocclr_copyBuffer", 64, "FETCH_SIZE", 1.0),        # a small upload: ignored
            ("void sv::k_attn_mfma<128, 2>(sv::AttnArgs)", 256, "FETCH_SIZE", 1000.0),
            ("void sv::k_attn_mfma<128, 2>(sv::AttnArgs)", 256, "WRITE_SIZE", 100.0)]
    d = tmp_path / "pmc"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)
    out = tmp_path / "rec.json"
    bench.summarize_pmc(str(d), "c3_confu_8b", out=str(out))
    rec = json.load(open(out))
    assert rec["workload"] == "c3_confu_8b" and len(rec["kernel_src_sha256"]) == 64 and rec["taken"]
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert abs(rec["traffic_bytes_per_launch"] - (1000 * 1024 * 2 + 100 * 1024)) < 1e-6


def test_counter_record_is_keyed_on_workload_and_kernel_source(tmp_path, monkeypatch):
    rec = {"workload": "c4_tree_3b", "kernel_src_sha256": "0" * 64, "traffic_bytes_per_launch": 1.0, "taken": "x"}
    path = tmp_path / "attn_mfma_c4_tree_3b_f32_counters.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "counters_file",
                        lambda w, out="f32": str(tmp_path / f"attn_mfma_{w}_{out}_counters.json"))
    assert bench.counters_traffic("c4_tree_3b") == (None, None)          # stale source hash
    import hashlib
    rec["kernel_src_sha256"] = hashlib.sha256(open(bench.ATTN_SRC, "rb").read()).hexdigest()
    path.write_text(json.dumps(rec))
    traffic, src = bench.counters_traffic("c4_tree_3b")
    assert traffic == 1.0 and src["kernel_src_sha256"] == rec["kernel_src_sha256"] and src["taken"] == "x"
    assert bench.counters_traffic("c3_confu_8b") == (None, None)         # no record for that workload
    (tmp_path / "attn_mfma_c4_tree_3b_bf16_counters.json").write_text(json.dumps(rec))
    assert bench.counters_traffic("c4_tree_3b", "bf16") == (None, None)  # taken with the fp32 output


def test_argmax_bytes_count_node_rows():
    cfg = wl.CONFIGS["c6_msa_1b"]
    x = wl.generate(cfg, B=2)
    assert bench.argmax_bytes(cfg, x) == int(x["n_nodes"].sum()) * cfg.V * 2
    c1 = wl.CONFIGS["c1_tiny_la"]
    x1 = wl.generate(c1)
    assert bench.argmax_bytes(c1, x1) == 4 * 1000 * 4


def test_every_workload_has_a_description_and_bound():
    for name in ["c1_tiny_la", "c2_la_7b", "c3_confu_8b", "c4_tree_3b", "c5_stream_70b", "c6_msa_1b"]:
        desc, seq_len, bound = bench.DESCRIPTIONS[name]
        assert name in wl.CONFIGS and seq_len > 0 and bound in ("hbm", "mfma", "latency")

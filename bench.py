"""Benchmark of the verification step on one MI355X.

A step is one pass of the whole hot path over one batch of the ConFu-shaped
Llama-3-8B workload (16 requests, 32 query / 8 kv heads, head dim 128, bf16,
4096-token prefix + 16 soft-prompt rows, 30-node draft tree + 30 contemplate
rows = 60 query rows per request, 128256-entry vocabulary):
    spec_build_mask -> spec_verify_attn -> spec_argmax_accept -> spec_commit_kv
Inputs are resident in HBM before timing starts; independent input sets
(at least three and ~1 GB in all: 1.3 GB for this workload) are cycled so
that the 256 MB last-level cache cannot hold a step's working set.  The
metric is speculative query tokens verified per second (sum of valid block
rows / step time).

--workload c6_msa_1b times Speculative Streaming's multi-stream verification
instead (spec_build_msa_mask -> spec_verify_attn -> spec_argmax_accept_rows ->
spec_commit_kv on a 40-node tree with 3 speculative streams per node).

The K/V cache is laid out head-major, [B, Hkv, lmax, D] (each kv-head's keys
contiguous), which the library takes through the descriptor's strides
(--layout blhd selects token-major [B, lmax, Hkv, D]).

Printed: one JSON line on stdout; details on stderr.  The roofline object
describes the attention kernel (the dominant one): algorithmic bytes per
launch / its mean duration, timed with one pair of HIP events on the launch
stream around K back-to-back launches after the timed steps (the steps
themselves carry no events, whose records add idle queue time).

Counter runs: with --calibrate-copy the run also performs a 1 GiB
device-to-device copy (a plain copy kernel of known size) before the timed
steps, so that one `rocprofv3 --pmc FETCH_SIZE` run and one
`rocprofv3 --pmc WRITE_SIZE` run see both kernels; `bench.py --summarize-pmc
DIR` then scales the attention kernel's counters by the copy's known size and
records the HBM bytes per launch in profiles/ with a hash of the kernel source.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
WORKLOAD = "c3_confu_8b"        # the headline workload (default)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_mfma_c3_counters.json")
# workloads bench.py can time (the headline one and the multi-stream tree draft)
DESCRIPTIONS = {
    "c3_confu_8b": ("ConFu-shaped Llama-3-8B verify: batch 16, 32q/8kv heads, head_dim 128, prefix 4096 + "
                    "16 soft rows, 30-node tree + 30 contemplate rows, vocab 128256", 4096),
    "c6_msa_1b": ("Speculative Streaming multi-stream verify, OPT-1.3B-shaped: batch 8, 32 heads, head_dim 64, "
                  "prefix U{256..1024}, 40-node tree (gamma 3, k 3) x (1 + 3 streams) = 160 rows, vocab 50272",
                  1024),
}
ATTN_SRC = os.path.join(ROOT, "masked_verification_attention_amd", "csrc", "attn_mfma.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_algorithmic_bytes(cfg, x) -> int:
    """Bytes the attention must move at least once: KV prefix read, soft prompt,
    queries, block K/V, mask words and the fp32 output (+ lse)."""
    es = 2 if cfg.dtype == "bf16" else 4
    B, Tq = x["q"].shape[:2]
    W = (Tq + 31) // 32
    kv = int(x["cache_len"].astype(np.int64).sum()) * cfg.Hkv * cfg.D * 2 * es
    soft = cfg.S * cfg.Hkv * cfg.D * 2 * es
    q = B * Tq * cfg.Hq * cfg.D * es
    blk = B * Tq * cfg.Hkv * cfg.D * 2 * es
    mask = B * Tq * W * 4 + B * W * 4
    out = B * Tq * cfg.Hq * cfg.D * 4 + B * Tq * cfg.Hq * 4
    return kv + soft + q + blk + mask + out


def attention_flops(cfg, x) -> int:
    """4*D flops per visible (query head, key) pair; visible pairs counted from the inputs."""
    B, Tq = x["q"].shape[:2]
    total = 0
    if cfg.structure == "msa_tree":
        # main stream of node v: prefix + its path; stream j: also streams 1..j of v
        for b in range(B):
            L = int(x["cache_len"][b])
            for v in range(int(x["n_nodes"][b])):
                depth, p = 1, int(x["tree_parent"][b, v])
                while p >= 0:
                    depth, p = depth + 1, int(x["tree_parent"][b, p])
                total += sum(L + depth + j for j in range(cfg.gamma + 1)) * cfg.Hq
        return total * 4 * cfg.D
    for b in range(B):
        L = int(x["cache_len"][b])
        nq = int(x["n_q"][b])
        for r in range(nq):
            depth = 1
            p = int(x["attn_parent"][b, r])
            while p >= 0:
                depth += 1
                p = int(x["attn_parent"][b, p])
            soft = cfg.S if x["sp_flag"][b, r] else 0
            total += (L + soft + depth) * cfg.Hq
    return total * 4 * cfg.D


COPY_BYTES = 1 << 30


def summarize_pmc(d: str):
    """Per-launch HBM traffic of the attention kernel from rocprofv3 counter CSVs in d
    (a FETCH_SIZE run and a WRITE_SIZE run of `bench.py --calibrate-copy`)."""
    import csv
    import glob

    files = []
    for one in d.split(","):
        files += glob.glob(os.path.join(one, "**", "*counter_collection.csv"), recursive=True)
    rows = [r for f in files for r in csv.DictReader(open(f))]
    # the calibration copy is the copy dispatch with the largest grid (smaller ones are uploads)
    copy_grid = max((int(r["Grid_Size"]) for r in rows if "copyBuffer" in r["Kernel_Name"]), default=-1)
    vals = {}
    for r in rows:
        name, ctr = r["Kernel_Name"], r["Counter_Name"]
        kind = None
        if "k_attn_mfma" in name:
            kind = "attn"
        elif "copyBuffer" in name and int(r["Grid_Size"]) == copy_grid:
            kind = "copy"
        if kind and ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            vals.setdefault((kind, ctr), []).append(float(r["Counter_Value"]))
    need = [("attn", "FETCH_SIZE"), ("attn", "WRITE_SIZE"), ("copy", "FETCH_SIZE"), ("copy", "WRITE_SIZE")]
    missing = [k for k in need if k not in vals]
    if missing:
        raise SystemExit(f"counters missing in {d}: {missing}")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    # the copy kernel moves COPY_BYTES each way: scale KiB readings to bytes of traffic
    f_fetch = COPY_BYTES / (mean[("copy", "FETCH_SIZE")] * 1024)
    f_write = COPY_BYTES / (mean[("copy", "WRITE_SIZE")] * 1024)
    fetch = mean[("attn", "FETCH_SIZE")] * 1024 * f_fetch
    write = mean[("attn", "WRITE_SIZE")] * 1024 * f_write
    rec = {
        "kernel": "k_attn_mfma", "workload": WORKLOAD,
        "kernel_src_sha256": hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest(),
        "fetch_size_kib_per_launch": mean[("attn", "FETCH_SIZE")],
        "write_size_kib_per_launch": mean[("attn", "WRITE_SIZE")],
        "copy_fetch_size_kib": mean[("copy", "FETCH_SIZE")], "copy_write_size_kib": mean[("copy", "WRITE_SIZE")],
        "copy_bytes": COPY_BYTES, "fetch_scale": f_fetch, "write_scale": f_write,
        "traffic_bytes_per_launch": fetch + write,
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
    }
    with open(COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def counters_traffic(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, or None
    if the kernel source changed since they were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if rec.get("kernel_src_sha256") != sha or rec.get("workload") != workload:
            return None
        return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(workload: str, requests: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    from threadpoolctl import threadpool_limits

    import oracle
    from masked_verification_attention_amd import workloads as wl

    cfg = wl.CONFIGS[workload]
    requests = min(requests, cfg.B)
    x = wl.generate(cfg, B=requests)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if cfg.structure == "msa_tree":
            oracle.build_msa_mask(x["tree_parent"], x["n_nodes"], cfg.gamma, cfg.Tq)
            vis = np.stack([oracle.msa_block_visibility(x["tree_parent"][b], int(x["n_nodes"][b]), cfg.gamma,
                                                        cfg.Tq) for b in range(requests)])
            oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"],
                                    None, None, None, None, x["n_q"], cfg.dtype, block_vis=vis)
            vrow = np.full(x["acc_parent"].shape, -1, dtype=np.int32)
            for b in range(requests):
                for v, p in enumerate(x["tree_parent"][b]):
                    vrow[b, v] = -1 if p < 0 else oracle.msa_row(int(x["n_nodes"][b]), cfg.gamma, int(p), 0)
            _, A, path, _, _ = oracle.argmax_accept_rows(x["logits"], cfg.logits_dtype, x["n_nodes"],
                                                         x["draft_tok"], x["acc_parent"], vrow, cfg.max_depth)
        else:
            oracle.build_mask(x["attn_parent"], x["sp_flag"], x["n_q"])
            oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"],
                                    x["k_soft"], x["v_soft"], x["attn_parent"], x["sp_flag"], x["n_q"], cfg.dtype)
            _, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                              x["acc_parent"], cfg.max_depth)
        oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
        dt = time.perf_counter() - t0
    tokens = int(x["n_q"].sum())
    return {"value": tokens / dt, "unit": "spec query tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{requests} of the {cfg.B} requests of the workload ({tokens} query tokens, full "
                      f"prefixes), whole step (mask, attention, argmax+acceptance, commit), "
                      f"fp64 numpy, BLAS limited to 1 thread; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets cycled between steps (0: enough for ~1 GB, at least 3)")
    ap.add_argument("--workload", choices=sorted(DESCRIPTIONS), default=WORKLOAD)
    ap.add_argument("--accept", choices=("greedy", "threshold", "soft"), default="greedy",
                    help="acceptance rule of the step (greedy: hard matching, fused with the commit)")
    ap.add_argument("--cpu-requests", type=int, default=16, help="requests in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-splits", type=int, default=0)
    ap.add_argument("--layout", choices=("bhld", "blhd", "bhld_vt"), default="bhld")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", metavar="DIRS",
                    help="comma-separated rocprofv3 output dirs of the FETCH_SIZE and WRITE_SIZE runs: "
                         "write the traffic record and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from masked_verification_attention_amd import workloads as wl
    from masked_verification_attention_amd.step import VerifyStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = wl.CONFIGS[args.workload]
    steps_state = []
    t0 = time.time()
    first = wl.generate(cfg, seed=cfg.seed)
    if args.sets <= 0:
        args.sets = int(min(16, max(3, np.ceil(1e9 / wl.nbytes_of(first)))))
    for i in range(args.sets):
        x = first if i == 0 else wl.generate(cfg, seed=cfg.seed + 100 * i)
        # probability rules: the draft's own probability and the uniform draw are inputs
        # (seeded here, as a caller's generator would supply them)
        urng = np.random.default_rng(cfg.seed + 7 + i)
        T_acc = x["acc_parent"].shape[1]
        st = VerifyStep(cfg, x, device="cuda:0", kv_splits=args.kv_splits, layout=args.layout,
                        accept=args.accept, threshold=1e-3,
                        draft_prob=urng.random((cfg.B, T_acc)).astype(np.float32) * 0.02,
                        uniform=urng.random((cfg.B, T_acc)).astype(np.float32))
        steps_state.append((st, x))
    torch.cuda.synchronize()
    log(f"inputs: {args.sets} sets generated and uploaded in {time.time() - t0:.1f}s")
    x0 = steps_state[0][1]
    tokens_per_step = int(x0["n_q"].sum())
    alg_bytes = attention_algorithmic_bytes(cfg, x0)
    flops = attention_flops(cfg, x0)

    stream = torch.cuda.current_stream()
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        steps_state[i % args.sets][0].run(stream)
    torch.cuda.synchronize()

    K = args.steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        steps_state[i % args.sets][0].run(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / K
    value = tokens_per_step * K / elapsed

    # The attention kernel's mean launch duration: HIP events on its launch
    # stream around K back-to-back launches over the same input sets (masks
    # already built by the steps above).  The events stay out of the steps: each
    # timing event record adds a few microseconds of idle queue time there.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        steps_state[i % args.sets][0].attention(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    attn_mean = e0.elapsed_time(e1) * 1e3 / K
    achieved = alg_bytes / (attn_mean * 1e-6) / 1e9
    tflops = flops / (attn_mean * 1e-6) / 1e12
    log(f"step {ms_per_step * 1e3:.1f} us; attention mean {attn_mean:.1f} us; {alg_bytes / 1e6:.1f} MB -> {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of HBM peak); {flops / 1e9:.1f} GFLOP -> {tflops:.0f} TFLOP/s "
        f"({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of bf16 MFMA peak); ws {steps_state[0][0].ws_bytes} B")

    result = {
        "metric": "verify-attn spec query tokens/s + achieved HBM GB/s (% of peak), 1 MI355X",
        "value": value,
        "unit": "spec query tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.workload][0],
                   "global_batch": cfg.B, "seq_len": DESCRIPTIONS[args.workload][1], "query_rows": cfg.Tq,
                   "kv_layout": args.layout, "acceptance": args.accept,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counters_traffic(args.workload),
                     "kernel": "k_attn_mfma", "algorithmic_bytes_per_launch": alg_bytes,
                     "mean_launch_us": attn_mean, "tflops": tflops},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_requests)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.1f} tokens/s ({result['cpu_baseline']['sample']})")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

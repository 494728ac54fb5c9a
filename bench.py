"""Benchmark of the verification step on one MI355X.

A step is one pass of the whole hot path over one batch of a workload:
    spec_verify_attn_tree -> spec_argmax_accept_commit
(the block mask built from the tree's parents inside the attention launch;
argmax, acceptance scan and KV commit in two launches); --mask separate runs
spec_build_mask -> spec_verify_attn instead, and fp32 workloads always do.
With --accept threshold|soft the tail is spec_prob_accept -> spec_commit_kv,
and the multi-stream workload (c6) verifies with spec_verify_attn_msa and
drafts the next tree with spec_draft_tree.  The default workload is the
ConFu-shaped Llama-3-8B verification (16 requests, 32 query / 8 kv heads,
head dim 128, bf16, 4096-token prefix + 16 soft-prompt rows, 30-node draft
tree + 30 contemplate rows = 60 query rows per request, 128256-entry
vocabulary); --workload selects the others (c1..c5 of the same family, c6
multi-stream).

Inputs are resident in HBM before timing starts; independent input sets (at
least three and ~1 GB in all) are cycled so that the 256 MB last-level cache
cannot hold a step's working set.  The metric is speculative query tokens
verified per second (valid block rows / step time).

Timing
  * value / ms_per_step: K steps back to back with no events inside, between
    two synchronisations.  Before them the step runs back to back for at least
    --prewarm-ms of wall time, then W warm-up steps: after idle the GPU's clock
    takes ~20 ms of load to ramp (the first ~150 C3 steps run at 118-138 us
    against ~110 us sustained), and the metric is the sustained rate.
  * roofline: the attention kernel's in-step launch durations, from a second
    pass of max(K, 100) steps right after the timed one (same input rotation,
    same thermal state) with HIP events recorded around every call of the step
    on the launch stream; the mean is `mean_launch_us` (the figure rocprofv3's
    kernel trace averages), with median, p10 and p90 beside it.  The events
    stay out of the timed steps because each record adds idle queue time.
  * measured ceilings: a plain streaming read of a 2 GiB buffer and
    back-to-back bf16 matrix instructions (probes/ceilings.hip), best of five,
    reported next to the published peaks.
  * traffic: HBM bytes per attention launch from committed rocprofv3 counter
    runs (FETCH_SIZE, WRITE_SIZE, scaled by a 1 GiB copy's readings), valid
    only while the kernel source hash matches; `traffic_source` names the
    record.  `--calibrate-copy` adds the copy to a run under rocprofv3 --pmc
    and `--summarize-pmc DIR` writes the record.

Printed: one JSON line on stdout; details on stderr.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
F32_VALU_PEAK_TFLOPS = 157.3    # fp32 vector
WORKLOAD = "c3_confu_8b"        # the headline workload (default)
# workload -> (description, seq_len, roofline bound of the attention kernel)
DESCRIPTIONS = {
    "c1_tiny_la": ("Tiny lookahead verify: batch 1, 2 heads (MHA), head_dim 64, fp32, prefix 128, "
                   "4 lookahead rows (prefix + self), vocab 1000", 128, "latency"),
    "c2_la_7b": ("LLaMA-7B-shaped lookahead layer: batch 8, 32 heads MHA, head_dim 128, bf16, prefixes "
                 "U{512..2048}, 8 lookahead rows, vocab 32000", 2048, "hbm"),
    "c3_confu_8b": ("ConFu-shaped Llama-3-8B verify: batch 16, 32q/8kv heads, head_dim 128, prefix 4096 + "
                    "16 soft rows, 30-node tree + 30 contemplate rows, vocab 128256", 4096, "hbm"),
    "c4_tree_3b": ("Llama-3.2-3B-shaped large tree: batch 32, 24q/8kv heads, head_dim 128, bf16, prefixes "
                   "U{2048..8192} + 16 soft rows, 60-node tree + 60 contemplate rows, vocab 128256", 8192, "hbm"),
    "c5_stream_70b": ("70B-shaped long-context stream verify: batch 16, 64q/8kv heads, head_dim 128, bf16, "
                      "prefix 16384, 128-node tree (32 candidates x 4 stream tokens), vocab 128256", 16384, "mfma"),
    "c6_msa_1b": ("Speculative Streaming multi-stream verify, OPT-1.3B-shaped: batch 8, 32 heads, head_dim 64, "
                  "prefix U{256..1024}, 40-node tree (gamma 3, k 3) x (1 + 3 streams) = 160 rows, vocab 50272",
                  1024, "hbm"),
}
ATTN_SRC = os.path.join(ROOT, "masked_verification_attention_amd", "csrc", "attn_mfma.hip")
PROBE_LIB = os.path.join(ROOT, "masked_verification_attention_amd", "probes", "libspecprobe.so")
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counters_file(workload: str, out: str = "f32") -> str:
    tag = "" if out == "f32" else f"_{out}out"
    return os.path.join(ROOT, "profiles", f"attn_mfma_{workload}{tag}_counters.json")


def attention_algorithmic_bytes(cfg, x, fused_mask=False, out_es=4) -> int:
    """Bytes the attention must move at least once: KV prefix read, soft prompt,
    queries, block K/V, mask words (or, when the launch builds the mask itself,
    the parent array and soft-prompt flags) and the output (``out_es`` bytes a
    value: fp32 or bf16) with its fp32 lse."""
    es = 2 if cfg.dtype == "bf16" else 4
    B, Tq = x["q"].shape[:2]
    W = (Tq + 31) // 32
    kv = int(x["cache_len"].astype(np.int64).sum()) * cfg.Hkv * cfg.D * 2 * es
    soft = cfg.S * cfg.Hkv * cfg.D * 2 * es
    q = B * Tq * cfg.Hq * cfg.D * es
    blk = B * Tq * cfg.Hkv * cfg.D * 2 * es
    mask = B * Tq * 5 if fused_mask else B * Tq * W * 4 + B * W * 4
    out = B * Tq * cfg.Hq * cfg.D * out_es + B * Tq * cfg.Hq * 4
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


def argmax_bytes(cfg, x) -> int:
    """Logit bytes the greedy tokens read: every valid node row once."""
    es = 2 if cfg.logits_dtype == "bf16" else 4
    return int(x["n_nodes"].sum()) * x["logits"].shape[2] * es


def summarize_pmc(d: str, workload: str = WORKLOAD, out: str = None, out_dtype: str = "f32"):
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
        "kernel": "k_attn_mfma", "workload": workload, "out": out_dtype,
        "kernel_src_sha256": hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest(),
        "taken": time.strftime("%Y-%m-%d"),
        "fetch_size_kib_per_launch": mean[("attn", "FETCH_SIZE")],
        "write_size_kib_per_launch": mean[("attn", "WRITE_SIZE")],
        "copy_fetch_size_kib": mean[("copy", "FETCH_SIZE")], "copy_write_size_kib": mean[("copy", "WRITE_SIZE")],
        "copy_bytes": COPY_BYTES, "fetch_scale": f_fetch, "write_scale": f_write,
        "traffic_bytes_per_launch": fetch + write,
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
    }
    with open(out or counters_file(workload, out_dtype), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def counters_traffic(workload: str, out: str = "f32"):
    """(HBM bytes per attention launch, source record) from committed rocprofv3 counter
    runs, or (None, None) if there are none, they were taken with another output
    dtype, or the kernel source changed since."""
    path = counters_file(workload, out)
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if (rec.get("kernel_src_sha256") != sha or rec.get("workload") != workload
                or rec.get("out", "f32") != out):
            return None, None
        src = {"file": os.path.relpath(path, ROOT), "kernel_src_sha256": sha, "taken": rec.get("taken")}
        return rec.get("traffic_bytes_per_launch"), src
    except (OSError, ValueError):
        return None, None


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(workload: str, requests: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload: once with
    BLAS on every core this process may use, once on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from masked_verification_attention_amd import workloads as wl

    cfg = wl.CONFIGS[workload]
    requests = min(requests, cfg.B)
    x = wl.generate(cfg, B=requests)

    def one_pass():
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
        return time.perf_counter() - t0

    tokens = int(x["n_q"].sum())
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas = sorted({p.get("internal_api", "?") + ":" + str(p.get("num_threads")) for p in threadpool_info()})
        dt_all = one_pass()
    with threadpool_limits(limits=1):
        dt_one = one_pass()
    sample = (f"{requests} of the {cfg.B} requests of the workload ({tokens} query tokens, full prefixes), "
              f"whole step (mask, attention, argmax + acceptance, commit), fp64 numpy")
    return {"value": tokens / dt_all, "unit": "spec query tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample}; BLAS on {cores} threads; {dt_all:.1f} s",
            "single_thread": {"value": tokens / dt_one, "cores": 1, "seconds": dt_one},
            "host": dict(host_info(), blas_pools=blas)}


def measured_ceilings(torch):
    """Best-of-five streaming read of 2 GiB (GB/s) and bf16 matrix-instruction rates (TFLOP/s)."""
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: run the build step first")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.spec_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.spec_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    nwg = 256 * 16
    sink = torch.zeros(nwg, dtype=torch.float32, device="cuda")

    def timed(fn, reps=5):
        best = None
        for _ in range(reps + 1):                       # the first launch is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        return best

    t_read = timed(lambda: lib.spec_probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), nwg, stream.cuda_stream))
    iters = 500
    rates = {}
    for kind, name, chains, flops in ((0, "16x16x32", 16, 16384), (1, "32x32x16", 8, 32768)):
        t = timed(lambda: lib.spec_probe_mfma(kind, 2048, iters, sink.data_ptr(), stream.cuda_stream))
        rates[name] = 2048 * 4 * chains * iters * flops / t / 1e12
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": nbytes / t_read / 1e9, "mfma_bf16_tflops_16x16x32": rates["16x16x32"],
            "mfma_bf16_tflops_32x32x16": rates["32x32x16"],
            "probe": "streaming read of 2 GiB; 2048 workgroups x 4 waves x (16 chains of 16x16x32 or 8 of "
                     "32x32x16) x 500 matrix instructions; best of five"}


def stats(v):
    v = np.asarray(v)
    return {"mean": float(v.mean()), "median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
            "p90": float(np.percentile(v, 90))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="run the step back to back for at least this long before the warm-up steps "
                         "(the GPU's clock ramps up over the first ~20 ms of load)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets cycled between steps (0: enough for ~1 GB, at least 3)")
    ap.add_argument("--workload", choices=sorted(DESCRIPTIONS), default=WORKLOAD)
    ap.add_argument("--accept", choices=("greedy", "threshold", "soft"), default="greedy",
                    help="acceptance rule of the step (greedy: hard matching, fused with the commit)")
    ap.add_argument("--cpu-requests", type=int, default=16, help="requests in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--kv-splits", type=int, default=0)
    ap.add_argument("--mask", choices=("fused", "separate"), default="fused",
                    help="block mask built inside the attention launch (spec_verify_attn_tree, where it "
                         "applies: bf16, parent-array masks) or by spec_build_mask first")
    ap.add_argument("--layout", choices=("bhld", "blhd", "bhld_vt"), default="bhld")
    ap.add_argument("--out", choices=("f32", "bf16"), default="f32",
                    help="attention output dtype (bf16: bf16 workloads only, the fp32 result rounded)")
    ap.add_argument("--instrumented-steps", type=int, default=0,
                    help="steps of the second pass with events around every call (0: max(steps, 100))")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", metavar="DIRS",
                    help="comma-separated rocprofv3 output dirs of the FETCH_SIZE and WRITE_SIZE runs: "
                         "write the traffic record of --workload and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload, out_dtype=args.out)
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
    desc, seq_len, bound = DESCRIPTIONS[args.workload]
    layout = args.layout if cfg.dtype == "bf16" or args.layout != "bhld_vt" else "bhld"
    if args.out == "bf16" and cfg.dtype != "bf16":
        raise SystemExit(f"--out bf16 needs a bf16 workload ({args.workload} is {cfg.dtype})")
    ceilings = None if args.no_ceilings else measured_ceilings(torch)
    if ceilings:
        log(f"measured ceilings: read {ceilings['hbm_read_gbs']:.0f} GB/s, bf16 matrix "
            f"{ceilings['mfma_bf16_tflops_16x16x32']:.0f} / {ceilings['mfma_bf16_tflops_32x32x16']:.0f} TFLOP/s")

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
        st = VerifyStep(cfg, x, device="cuda:0", kv_splits=args.kv_splits, layout=layout,
                        accept=args.accept, threshold=1e-3,
                        draft_prob=urng.random((cfg.B, T_acc)).astype(np.float32) * 0.02,
                        uniform=urng.random((cfg.B, T_acc)).astype(np.float32),
                        fused_mask=None if args.mask == "fused" else False, out_dtype=args.out)
        steps_state.append((st, x))
    torch.cuda.synchronize()
    log(f"inputs: {args.sets} sets generated and uploaded in {time.time() - t0:.1f}s")
    x0 = steps_state[0][1]
    tokens_per_step = int(x0["n_q"].sum())
    fused = steps_state[0][0].fused_mask
    alg_bytes = attention_algorithmic_bytes(cfg, x0, fused_mask=fused, out_es=2 if args.out == "bf16" else 4)
    flops = attention_flops(cfg, x0)
    am_bytes = argmax_bytes(cfg, x0)

    stream = torch.cuda.current_stream()
    # each step's calls with their arguments converted once: the loop below then only
    # crosses the C ABI, so the host keeps ahead of the device
    prepared = [st.prepare(stream) for st, _ in steps_state]
    runs = [m + at + tl for m, at, tl in prepared]
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # clock ramp: steps back to back until --prewarm-ms of wall time has passed
    t_pw = time.perf_counter()
    n_pw = 0
    while args.prewarm_ms > 0:
        for call in runs[n_pw % args.sets]:
            call()
        n_pw += 1
        if n_pw % 64 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t_pw) * 1e3 >= args.prewarm_ms:
                break
    for i in range(args.warmup):
        for call in runs[i % args.sets]:
            call()
    torch.cuda.synchronize()
    log(f"pre-warm: {n_pw} steps in {(time.perf_counter() - t_pw) * 1e3:.0f} ms (with the {args.warmup} warm-up steps)")

    # -- the timed region: K whole steps, nothing else on the stream
    K = args.steps
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    g0.record(stream)
    for i in range(K):
        for call in runs[i % args.sets]:
            call()
    g1.record(stream)
    t_enq = time.perf_counter() - t_start
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    gpu_span_us = g0.elapsed_time(g1) * 1e3 / K
    ms_per_step = elapsed * 1e3 / K
    value = tokens_per_step * K / elapsed

    # -- in-step kernel durations: the same steps again, events around every call
    K2 = args.instrumented_steps or max(K, 100)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K2)]
    torch.cuda.synchronize()
    for i in range(K2):
        m, at, tl = prepared[i % args.sets]
        e = ev[i]
        e[0].record(stream)
        for call in m:
            call()
        e[1].record(stream)
        for call in at:
            call()
        e[2].record(stream)
        for call in tl:
            call()
        e[3].record(stream)
    torch.cuda.synchronize()
    t_mask = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
    t_attn = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]
    t_tail = [e[2].elapsed_time(e[3]) * 1e3 for e in ev]
    a = stats(t_attn)
    attn_mean = a["mean"]
    achieved_gbs = alg_bytes / (attn_mean * 1e-6) / 1e9
    tflops = flops / (attn_mean * 1e-6) / 1e12
    tail_mean = float(np.mean(t_tail))
    span2 = ev[0][0].elapsed_time(ev[-1][3]) * 1e3 / K2
    log(f"host enqueue {t_enq * 1e6 / K:.1f} us per step; device span {gpu_span_us:.1f} us per step (timed), "
        f"{span2:.1f} (instrumented pass); "
        f"step {ms_per_step * 1e3:.1f} us; attention in-step mean {attn_mean:.1f} us (median {a['median']:.1f}, "
        f"p10 {a['p10']:.1f}, p90 {a['p90']:.1f}); {alg_bytes / 1e6:.1f} MB -> {achieved_gbs:.0f} GB/s "
        f"({100 * achieved_gbs / HBM_PEAK_GBS:.1f}% of HBM peak); {flops / 1e9:.1f} GFLOP -> {tflops:.0f} TFLOP/s "
        f"({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of bf16 peak); "
        f"{'mask in the attention launch' if fused else f'mask {np.mean(t_mask):.1f} us'}, "
        f"tail {tail_mean:.1f} us")

    traffic, traffic_src = counters_traffic(args.workload, args.out)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_BF16_PEAK_TFLOPS}
    elif bound == "latency":
        # fp32 correctness workload: the VALU kernel, a few hundred KB per launch
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved_gbs / HBM_PEAK_GBS, "note": "launch-latency-bound correctness workload"}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved_gbs / HBM_PEAK_GBS}
    roof.update({
        "traffic": traffic, "traffic_source": traffic_src,
        "kernel": "k_attn_mfma" if cfg.dtype == "bf16" else "k_attn_valu",
        "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": flops,
        "mean_launch_us": attn_mean, "median_launch_us": a["median"], "p10_launch_us": a["p10"],
        "p90_launch_us": a["p90"], "launches_timed": K2,
        "timing": f"in-step: HIP events around the attention call in each of {K2} steps run right after the "
                  f"timed ones (same input rotation)",
        "hbm_gbs": achieved_gbs, "hbm_frac": achieved_gbs / HBM_PEAK_GBS,
        "tflops": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
    })
    if ceilings:
        roof["measured_ceiling"] = ceilings
        roof["frac_of_measured_read_ceiling"] = achieved_gbs / ceilings["hbm_read_gbs"]
        roof["frac_of_measured_mfma_ceiling"] = tflops / max(ceilings["mfma_bf16_tflops_16x16x32"],
                                                             ceilings["mfma_bf16_tflops_32x32x16"])
    step_kernels = {
        "mask_us": None if fused else stats(t_mask), "attention_us": a, "tail_us": stats(t_tail),
        "mask": ("built inside the attention launch (spec_verify_attn_tree or spec_verify_attn_msa)"
                 if fused else "spec_build_msa_mask" if cfg.structure == "msa_tree" else "spec_build_mask"),
        "tail": ("spec_argmax_accept_commit (argmax, acceptance scan + commit: two launches)"
                 if args.accept == "greedy" else "spec_prob_accept + spec_commit_kv")
                + (" + spec_draft_tree" if cfg.structure == "msa_tree" else ""),
        "host_enqueue_us_per_step": t_enq * 1e6 / K,
        "device_span_us_per_step": gpu_span_us,
        "instrumented_span_us_per_step": span2,
        "argmax_bytes": am_bytes,
        "argmax_gbs_over_tail": am_bytes / (tail_mean * 1e-6) / 1e9,
    }
    result = {
        "metric": "verify-attn spec query tokens/s + achieved HBM GB/s (% of peak), 1 MI355X",
        "value": value,
        "unit": "spec query tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "prewarm": {"ms": args.prewarm_ms, "steps": n_pw,
                    "why": "untimed steps back to back before the warm-up steps, so that the clock has ramped"},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": desc, "name": args.workload, "global_batch": cfg.B, "seq_len": seq_len,
                   "query_rows": cfg.Tq, "kv_layout": layout, "acceptance": args.accept, "attn_out": args.out,
                   "input_sets": args.sets, "parallelism": "single GPU"},
        "roofline": roof,
        "step_kernels": step_kernels,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_requests)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.1f} tokens/s on {result['cpu_baseline']['cores']} "
            f"threads, {result['cpu_baseline']['single_thread']['value']:.1f} on one "
            f"({result['cpu_baseline']['sample']})")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

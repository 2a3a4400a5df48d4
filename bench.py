#!/usr/bin/env python3
"""DSA decode benchmark on one MI355X: queries/s and achieved HBM GB/s.

Default workload: long-context decode, batch 8, one query token per sequence,
lengths uniform in [98304, 131072] (max 128K), index keys 64 heads x 128 bf16,
Top-K 2048, MLA 128 heads over 576-wide bf16 latent rows (512 value columns).
Synthetic seeded inputs (integer-valued indexer inputs, N(0,1) queries and
cache), resident in HBM before timing.  A step is one dsa_forward: indexer
scores over every cached position, Top-K, sparse MLA attention.

Input copies rotate between steps (--rotate, default 3 copies of the index
keys and latent cache: 4.2 GB) so the 256 MB Infinity Cache cannot serve the
key stream from one step to the next.  Steps are launched eagerly (five
kernels each; the host stays well ahead of the GPU, so they run back to
back); --graph replays them as HIP graphs instead (one per input copy), which
adds the graph launch gap (about 5 us) to every step.

Prints one JSON line.  `roofline` covers the dominant kernel (the indexer
score kernel, timed live with HIP events on the launch stream); `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.  `traffic`
comes from a counter record under profiles/ (see --copy-probe and
--traffic-from) and is null when that record was taken from other kernel
sources.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode queries/s and achieved HBM GB/s (% of peak) at L=128K, K=2048"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode128k")
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE_SIZE",
                    help="read both caches through a block table with pages of this many rows "
                         "(0: contiguous caches, the default)")
    ap.add_argument("--graph", action="store_true", help="replay each step as a HIP graph")
    ap.add_argument("--no-graph", action="store_true", help="eager launches (the default)")
    ap.add_argument("--stage-steps", type=int, default=50, help="eager steps timed per stage")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle baseline: time the oracle on queries for at least this long (0: skip)")
    ap.add_argument("--cpu-max-queries", type=int, default=2000)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB copy kernel first (calibrates rocprofv3 byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-probe run into the traffic record, then exit")
    return ap.parse_args()


COPY_PROBE_BYTES = 1 << 30
SCORE_KERNEL = "score_mfma_kernel"
SCORE_SOURCES = ("index_score.hip", "common.hpp", "kernels.hpp")


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"{SCORE_KERNEL}_{workload}_traffic.txt")


def score_source_hash():
    """Hash of the sources the score kernel is built from (its own file, the
    shared device helpers and its parameter struct): a traffic record taken
    from another version of the kernel is stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, "indexed_sparse_attention_amd", "csrc", f), "rb") as fh:
            text = fh.read()
        if f == "kernels.hpp":  # only the score kernel's parameter struct
            m = re.search(rb"struct ScoreParams \{.*?\};", text, re.S)
            text = m.group(0) if m else text
        h.update(text)
    return h.hexdigest()[:16]


def read_counter_csv(path, counter):
    """Per-dispatch values of one counter from a rocprofv3 counter_collection CSV:
    list of (kernel name, value)."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic_record(fetch_csv, write_csv, workload):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the score kernel, each scaled
    by the factor that makes the copy probe's counter equal its known size."""
    import numpy as np
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = read_counter_csv(path, name)
        copy = [v for k, v in rows if "neg" in k.lower()]
        score = [v for k, v in rows if SCORE_KERNEL in k]
        if not copy or not score:
            raise SystemExit(f"{path}: no copy-probe or {SCORE_KERNEL} dispatch with {name}")
        factor = COPY_PROBE_BYTES / (max(copy) * 1024.0)
        out[name] = (float(np.mean(score)) * 1024.0, factor, len(score), max(copy) * 1024.0)
    fetch, fw = out["FETCH_SIZE"][0], out["FETCH_SIZE"][1]
    write, ww = out["WRITE_SIZE"][0], out["WRITE_SIZE"][1]
    traffic = fetch * fw + write * ww
    path = traffic_path(workload)
    with open(path, "w") as f:
        f.write(f"# HBM traffic of {SCORE_KERNEL} per launch, workload {workload}\n")
        f.write("# from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over\n")
        f.write(f"#   python3 bench.py --workload {workload} --no-graph --copy-probe --steps 3 --warmup 1 "
                "--stage-steps 2 --cpu-seconds 0\n")
        f.write(f"# each scaled by (copy probe bytes {COPY_PROBE_BYTES}) / (counter bytes of the copy probe)\n")
        f.write(f"source_hash: {score_source_hash()}\n")
        f.write(f"dispatches: {out['FETCH_SIZE'][2]}\n")
        f.write(f"fetch_bytes_raw: {fetch:.0f}\n")
        f.write(f"fetch_factor: {fw:.4f}\n")
        f.write(f"copy_probe_fetch_bytes_raw: {out['FETCH_SIZE'][3]:.0f}\n")
        f.write(f"write_bytes_raw: {write:.0f}\n")
        f.write(f"write_factor: {ww:.4f}\n")
        f.write(f"copy_probe_write_bytes_raw: {out['WRITE_SIZE'][3]:.0f}\n")
        f.write(f"traffic_bytes: {traffic:.0f}\n")
    print(open(path).read())


def read_traffic_record(workload):
    """Calibrated HBM bytes per score launch, or None when there is no record
    or it was taken from other kernel sources."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != score_source_hash():
        return None
    return float(kv["traffic_bytes"])


def algorithmic_bytes(w):
    """Bytes the path must move per step: index keys once per sequence, the
    selected latent rows, queries, weights, outputs and index lists."""
    import numpy as np
    kb = {0: 4, 1: 2, 2: 1, 3: 1}[w.idx_key_dtype]
    cb = {0: 4, 1: 2, 2: 1, 4: 1}[w.kv_dtype]
    ob = {0: 4, 1: 2}[w.out_dtype]
    # scale bytes per row: fp32 per row, E8M0 bytes per 32 dims, fp32 per 128-column tile
    ks = 0 if w.k_scale is None else w.k_scale.itemsize * int(np.prod(w.k_scale.shape[2:], dtype=np.int64))
    vs = 0 if w.kv_scale is None else w.kv_scale.itemsize * int(np.prod(w.kv_scale.shape[2:], dtype=np.int64))
    qb = {0: 4, 1: 2}[w.q_dtype]
    lens = np.minimum(w.seq_lens.astype(np.int64), w.max_seq_len)
    keys = int(lens.sum()) * (w.idx_dim * kb + ks)
    sel = 0
    for b in range(w.batch):
        for t in range(w.q_len):
            sel += min(w.top_k, max(w.vis(b, t), 0))
    gathered = sel * (w.qk_dim * cb + vs)
    BT = w.batch * w.q_len
    small = BT * (w.idx_heads * w.idx_dim * 2 + w.idx_heads * 4 + w.heads * w.qk_dim * qb +
                  w.heads * w.v_dim * ob + 2 * w.top_k * 4)
    score_kernel = keys + BT * (w.idx_heads * w.idx_dim * 2 + w.idx_heads * 4)
    return {"total": keys + gathered + small, "keys": keys, "gathered": gathered, "small": small,
            "score_kernel": score_kernel}


def main():
    args = parse()
    if args.traffic_from:
        write_traffic_record(args.traffic_from[0], args.traffic_from[1], args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU (context-parallel) "
                                   "sharding is a design note, not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import indexed_sparse_attention_amd as dsa
    import synth

    dev = torch.device("cuda:0")
    t0 = time.time()
    w = synth.make(args.workload)
    print(f"# generated {args.workload} in {time.time() - t0:.1f}s: B={w.batch} T={w.q_len} "
          f"Lmax={w.max_seq_len} lens={w.seq_lens.tolist()}", file=sys.stderr, flush=True)

    def t(a, code):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if code == synth.BF16:
            x = x.view(torch.bfloat16)
        return x.to(dev)

    q_idx, head_w = t(w.q_idx, w.q_idx_dtype), t(w.head_w, synth.F32)
    q, seq_lens = t(w.q, w.q_dtype), t(w.seq_lens, synth.F32)
    k_scale, kv_scale = t(w.k_scale, synth.F32), t(w.kv_scale, synth.F32)
    k0, kv0 = t(w.k_idx, w.idx_key_dtype), t(w.kv, w.kv_dtype)
    R = max(1, args.rotate)
    k_copies = [k0] + [k0.clone() for _ in range(R - 1)]
    kv_copies = [kv0] + [kv0.clone() for _ in range(R - 1)]
    out_dtype = torch.float32 if w.out_dtype == synth.F32 else torch.bfloat16
    prob = dsa.forward_problem(q_idx, k0, q, kv0, seq_lens, w.top_k, w.v_dim, w.softmax_scale, out_dtype,
                               k_scale, kv_scale)
    ws = torch.zeros(dsa.forward_workspace_size(prob), dtype=torch.uint8, device=dev)  # counters start at zero
    B, T, H = w.batch, w.q_len, w.heads
    outs = {"out": torch.empty((B, T, H, w.v_dim), dtype=out_dtype, device=dev),
            "lse": torch.empty((B, T, H), dtype=torch.float32, device=dev),
            "topk_idx": torch.empty((B, T, w.top_k), dtype=torch.int32, device=dev),
            "topk_count": torch.empty((B, T), dtype=torch.int32, device=dev)}

    if args.paged:
        # The same caches in pages of a physical pool, in a random page order
        # (seeded), with one block table for both; every rotating copy is a pool.
        P = args.paged
        max_pages = (w.max_seq_len + P - 1) // P
        num_pages = B * max_pages
        gen = torch.Generator().manual_seed(0xD5A0)
        table = torch.randperm(num_pages, generator=gen).to(torch.int32).view(B, max_pages).to(dev)
        flat = table.view(-1).long()

        def pool(x, row):
            if x is None:
                return None
            x = x.view((B, w.max_seq_len) + row)
            pad = max_pages * P - w.max_seq_len
            if pad:
                x = torch.cat([x, torch.zeros((B, pad) + row, dtype=x.dtype, device=dev)], dim=1)
            out = torch.empty((num_pages, P) + row, dtype=x.dtype, device=dev)
            out[flat] = x.reshape((num_pages, P) + row)
            return out

        k_copies = [pool(k, (w.idx_dim,)) for k in k_copies]
        kv_copies = [pool(kv, (w.qk_dim,)) for kv in kv_copies]
        k_scale = pool(k_scale, tuple(w.k_scale.shape[2:])) if k_scale is not None else None
        kv_scale = pool(kv_scale, tuple(w.kv_scale.shape[2:])) if kv_scale is not None else None
        torch.cuda.synchronize()

    def step(r, stage_events=None):
        if args.paged:
            dsa.dsa_forward_paged(q_idx, head_w, k_copies[r], q, kv_copies[r], seq_lens, table, w.top_k,
                                  w.v_dim, w.max_seq_len, w.softmax_scale, k_scales=k_scale,
                                  kv_scales=kv_scale, out_dtype=out_dtype, out=outs, workspace=ws,
                                  stage_events=stage_events)
            return
        dsa.dsa_forward(q_idx, head_w, k_copies[r], q, kv_copies[r], seq_lens, w.top_k, w.v_dim,
                        w.softmax_scale, k_scale=k_scale, kv_scale=kv_scale, out_dtype=out_dtype,
                        out=outs, workspace=ws, stage_events=stage_events)

    if args.copy_probe:  # one plain streaming copy of known size for counter calibration
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # eager reference results (also warms up every kernel)
    step(0)
    torch.cuda.synchronize()
    ref_idx = outs["topk_idx"].clone()
    ref_out = outs["out"].clone()

    graphs = None
    if args.graph and not args.no_graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.current_stream().wait_stream(s)
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        # every copy must reproduce the eager result
        for r in range(R):
            outs["out"].zero_()
            graphs[r].replay()
            torch.cuda.synchronize()
            assert torch.equal(outs["topk_idx"], ref_idx) and torch.equal(outs["out"], ref_out), \
                f"graph replay {r} differs from the eager step"

    def run(i):
        if graphs is not None:
            graphs[i % R].replay()
        else:
            step(i % R)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    h0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    host_us = (time.perf_counter() - h0) / args.steps * 1e6  # host time to issue one step
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    assert torch.equal(outs["topk_idx"], ref_idx), "timed steps changed the Top-K result"

    # per-stage durations (eager, events recorded on the launch stream)
    n_st = max(1, args.stage_steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(dsa.FORWARD_STAGES + 1)] for _ in range(n_st)]
    for row in evs:
        for e in row:
            e.record()  # creates the underlying event
    torch.cuda.synchronize()
    for i in range(n_st):
        step(i % R, stage_events=evs[i])
    torch.cuda.synchronize()
    stage_ms = [sum(evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(n_st)) / n_st
                for k in range(dsa.FORWARD_STAGES)]

    ab = algorithmic_bytes(w)
    queries = B * T
    qps = queries / (ms * 1e-3)
    e2e_gbps = ab["total"] / (ms * 1e-3) / 1e9
    score_ms = stage_ms[0]
    score_gbps = ab["score_kernel"] / (score_ms * 1e-3) / 1e9
    traffic = read_traffic_record(args.workload)

    cpu = None
    if args.cpu_seconds > 0:
        # the oracle as it stands, one query at a time (cycling through this
        # workload's queries) until the time bound; its first query is
        # checked against the GPU
        import oracle
        order = [(b, t) for b in range(B) for t in range(T)]
        n_done, match = 0, None
        c0 = time.time()
        while True:
            b, t = order[n_done % len(order)]
            want = np.zeros((B, T), bool)
            want[b, t] = True
            sc = oracle.index_scores(w, want)
            idx, _ = oracle.topk(w, sc, want)
            oracle.sparse_mla(w, idx, want)
            n_done += 1
            if match is None:
                match = bool(np.array_equal(ref_idx[b, t].cpu().numpy(), idx[b, t]))
            dt = time.time() - c0
            if dt >= args.cpu_seconds or n_done >= args.cpu_max_queries:
                break
        cpu = {"value": n_done / dt, "unit": "queries/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{n_done} queries of this workload, one at a time in batch order (fp64 scores over "
                         f"every visible position, full-sort Top-K, {H}-head two-pass-softmax attention) "
                         f"in {dt:.1f} s",
               "topk_matches_gpu": match}

    line = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {synth.F32: "f32", synth.BF16: "bf16",
                                       synth.MXE4M3: "mxfp8-e4m3/bf16"}.get(w.idx_key_dtype, "fp8-e4m3/bf16"),
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_len": T, "max_seq_len": w.max_seq_len,
                   "mean_len": float(np.mean(w.seq_lens)), "top_k": w.top_k,
                   "indexer": f"{w.idx_heads}x{w.idx_dim}", "mla_heads": H, "qk_dim": w.qk_dim,
                   "v_dim": w.v_dim, "graph": graphs is not None, "rotate": R, "paged": args.paged,
                   "kernels": dsa.kernel_choice(prob)},
        "hbm_gbps_e2e": e2e_gbps, "hbm_frac_e2e": e2e_gbps / HBM_PEAK_GBPS, "host_us_per_step": host_us,
        "algorithmic_bytes_per_step": ab["total"],
        "stages_us": {"scores": stage_ms[0] * 1e3, "topk": stage_ms[1] * 1e3, "attention": stage_ms[2] * 1e3},
        "roofline": {"kernel": "score_mfma_kernel", "bound": "hbm", "achieved": score_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_launch": ab["score_kernel"],
                     "launch_us": score_ms * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

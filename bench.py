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
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak


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
    ap.add_argument("--wg-trace", action="store_true",
                    help="time one eager step's workgroups (start and end of each, per kernel) with every stage "
                         "in one launch, print the spread, then exit")
    ap.add_argument("--wg-trace-dump", default=None, metavar="FILE.npy",
                    help="with --wg-trace: also save the raw stamps, int64 [kind][workgroup][start, end] "
                         "in 100 MHz clock ticks (0: not stamped), and those of the back-to-back steps "
                         "as FILE_step<i>.npy")
    return ap.parse_args()


COPY_PROBE_BYTES = 1 << 30
SCORE_KERNEL = "score_mfma_kernel"
# kernels with a counter record, and the sources (plus parameter struct) each is built from
KERNEL_SOURCES = {
    "score_mfma_kernel": (("index_score.hip", "common.hpp"), "ScoreParams"),
    "select_chunk_kernel": (("topk.hip", "select.hpp", "common.hpp"), "TopkParams"),
    "select_emit_kernel": (("topk.hip", "select.hpp", "common.hpp"), "TopkParams"),
    "mla_mfma_kernel": (("sparse_mla.hip", "common.hpp"), "MlaParams"),
    "mla_combine_kernel": (("sparse_mla.hip", "common.hpp"), "MlaParams"),
}


def traffic_path(workload, kernel=SCORE_KERNEL):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")


def source_hash(kernel=SCORE_KERNEL):
    """Hash of the sources a kernel is built from (its file, the shared
    device helpers and its parameter struct): a counter record taken from
    another version of the kernel is stale."""
    import hashlib
    import re
    files, struct = KERNEL_SOURCES[kernel]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "indexed_sparse_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "indexed_sparse_attention_amd", "csrc", "kernels.hpp"), "rb") as fh:
        m = re.search(rb"struct " + struct.encode() + rb" \{.*?\};", fh.read(), re.S)
    h.update(m.group(0) if m else b"")
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
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel with a record,
    each scaled by the factor that makes the copy probe's counter equal its
    known size; one file per kernel under profiles/."""
    import numpy as np
    rows = {name: read_counter_csv(path, name) for name, path in (("FETCH_SIZE", fetch_csv),
                                                                 ("WRITE_SIZE", write_csv))}
    factors = {}
    for name, r in rows.items():
        copy = [v for k, v in r if "neg" in k.lower()]
        if not copy:
            raise SystemExit(f"no copy-probe dispatch with {name}")
        factors[name] = (COPY_PROBE_BYTES / (max(copy) * 1024.0), max(copy) * 1024.0)
    for kernel in KERNEL_SOURCES:
        got = {name: [v for k, v in r if kernel in k] for name, r in rows.items()}
        if not got["FETCH_SIZE"] or not got["WRITE_SIZE"]:
            continue
        fetch, write = (float(np.mean(got[n])) * 1024.0 for n in ("FETCH_SIZE", "WRITE_SIZE"))
        (fw, fcopy), (ww, wcopy) = factors["FETCH_SIZE"], factors["WRITE_SIZE"]
        path = traffic_path(workload, kernel)
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {kernel} per launch, workload {workload}\n")
            f.write("# from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over\n")
            f.write(f"#   python3 bench.py --workload {workload} --no-graph --copy-probe --steps 3 --warmup 1 "
                    "--stage-steps 2 --cpu-seconds 0\n")
            f.write(f"# each scaled by (copy probe bytes {COPY_PROBE_BYTES}) / (counter bytes of the copy probe)\n")
            f.write(f"source_hash: {source_hash(kernel)}\n")
            f.write(f"dispatches: {len(got['FETCH_SIZE'])}\n")
            f.write(f"fetch_bytes_raw: {fetch:.0f}\n")
            f.write(f"fetch_factor: {fw:.4f}\n")
            f.write(f"copy_probe_fetch_bytes_raw: {fcopy:.0f}\n")
            f.write(f"write_bytes_raw: {write:.0f}\n")
            f.write(f"write_factor: {ww:.4f}\n")
            f.write(f"copy_probe_write_bytes_raw: {wcopy:.0f}\n")
            f.write(f"fetch_bytes: {fetch * fw:.0f}\n")
            f.write(f"write_bytes: {write * ww:.0f}\n")
            f.write(f"traffic_bytes: {fetch * fw + write * ww:.0f}\n")
        print(open(path).read())


def read_traffic_record(workload, kernel=SCORE_KERNEL):
    """Calibrated HBM bytes per launch of `kernel`, or None when there is no
    record or it was taken from other kernel sources."""
    path = traffic_path(workload, kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(kernel):
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
    # the attention stage: gathered rows, queries, index lists, outputs; its
    # matrix-core work is 2 (Dqk + Dv) flops per selected row and head
    attention = gathered + BT * (w.heads * w.qk_dim * qb + w.heads * w.v_dim * ob + w.top_k * 4)
    attn_flops = 2 * sel * w.heads * (w.qk_dim + w.v_dim)
    return {"total": keys + gathered + small, "keys": keys, "gathered": gathered, "small": small,
            "score_kernel": score_kernel, "attention": attention, "attention_flops": attn_flops}


def wg_trace_report(dsa, torch, np, step, workload, w, dump=None, rotate=1):
    """Per-workgroup clock stamps (the library's workgroup trace, 100 MHz)
    of one eager step: for each kernel, when its workgroups started and
    finished relative to its first start, how far apart, and the gap between
    the previous kernel's last finish and its first start.  The stage events
    come from a separate eager step: recorded between the stages they would
    widen the gaps."""
    slots = 1 << 17
    kinds = dsa.TRACE_KINDS
    buf = torch.zeros(len(kinds) * slots * 2, dtype=torch.int64, device="cuda:0")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(dsa.FORWARD_STAGES + 1)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    step(0, stage_events=evs)
    torch.cuda.synchronize()
    stage_us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(dsa.FORWARD_STAGES)]
    dsa.set_workgroup_trace(buf, slots)
    try:
        step(0)
        torch.cuda.synchronize()
    finally:
        dsa.set_workgroup_trace(None)
    tr = buf.view(len(kinds), slots, 2).cpu().numpy()
    if dump:
        np.save(dump, tr)
    print(f"# workgroup timeline, workload {workload}: B={w.batch} T={w.q_len} Lmax={w.max_seq_len} "
          f"K={w.top_k}, one eager step, every stage in one launch")
    print(f"# stage events of another eager step (us): scores {stage_us[0]:.1f}  topk {stage_us[1]:.1f}  "
          f"attention {stage_us[2]:.1f}")
    print("# per kernel, in us from its first workgroup's start: the last start, the finish times' "
          "quantiles, the busy time (end - start) per workgroup, and the gap from the previous "
          "kernel's last finish to this one's first start")
    print(f"{'kernel':16s} {'wgs':>6s} {'last_start':>10s} {'end_min':>8s} {'end_p50':>8s} {'end_p90':>8s} "
          f"{'end_max':>8s} {'spread':>8s} {'busy_p50':>8s} {'busy_max':>8s} {'gap':>6s}")
    prev_end = None
    for k, name in enumerate(kinds):
        st, en = tr[k, :, 0], tr[k, :, 1]
        m = (st != 0) & (en != 0)
        if not m.any():
            continue
        st, en = st[m].astype(np.float64), en[m].astype(np.float64)
        t0 = st.min()
        s_us, e_us, busy = (st - t0) / 100.0, (en - t0) / 100.0, (en - st) / 100.0
        gap = "" if prev_end is None else f"{(t0 - prev_end) / 100.0:6.2f}"
        prev_end = en.max()
        q = lambda a, f: float(np.quantile(a, f))
        print(f"{name:16s} {int(m.sum()):6d} {s_us.max():10.2f} {e_us.min():8.2f} {q(e_us, .5):8.2f} "
              f"{q(e_us, .9):8.2f} {e_us.max():8.2f} {e_us.max() - e_us.min():8.2f} {q(busy, .5):8.2f} "
              f"{busy.max():8.2f} {gap:>6s}")

    # Three steps launched back to back (rotating inputs), each into its own
    # trace buffer: the span of a step's workgroups and the gap from one
    # step's last workgroup to the next one's first.
    n = 3
    bufs = [torch.zeros(len(kinds) * slots * 2, dtype=torch.int64, device="cuda:0") for _ in range(n)]
    torch.cuda.synchronize()
    try:
        for i in range(n):
            dsa.set_workgroup_trace(bufs[i], slots)
            step(i % rotate)
        torch.cuda.synchronize()
    finally:
        dsa.set_workgroup_trace(None)
    spans = []
    for i, b in enumerate(bufs):
        t = b.view(len(kinds), slots, 2).cpu().numpy()
        if dump:
            np.save(dump.replace(".npy", "") + f"_step{i}.npy", t)
        st, en = t[:, :, 0], t[:, :, 1]
        m = (st != 0) & (en != 0)
        spans.append((float(st[m].min()), float(en[m].max())))
    span_us = [(e - s0) / 100.0 for s0, e in spans]
    gaps_us = [(spans[i + 1][0] - spans[i][1]) / 100.0 for i in range(n - 1)]
    print(f"# {n} steps back to back: first to last workgroup of each step "
          f"{' '.join(f'{x:.1f}' for x in span_us)} us; from a step's last workgroup to the next "
          f"step's first {' '.join(f'{x:.2f}' for x in gaps_us)} us")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.traffic_from:
        write_traffic_record(args.traffic_from[0], args.traffic_from[1], args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; sharding over several GPUs "
                                   "(by sequence, or context-parallel along L) is not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.wg_trace:
        # one launch per stage, so the timeline covers the whole problem
        os.environ["DSA_TILE_BUDGET"] = str(1 << 40)

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

    if args.wg_trace:
        wg_trace_report(dsa, torch, np, step, args.workload, w, args.wg_trace_dump, R)
        return

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
    # A call in token tiles launches each stage once per tile, and its stage
    # events time the last tile (the last tokens of the last sequence): the
    # per-launch figures below are that tile's, its bytes and flops those of
    # the same problem with only its tokens.
    n_tile = dsa.forward_tile_tokens(prob)
    launches = B * -(-T // n_tile) if n_tile > 0 else 1
    ab_launch = ab
    if n_tile > 0:
        import dataclasses
        last = T - n_tile * ((T - 1) // n_tile)
        ab_launch = algorithmic_bytes(dataclasses.replace(w, batch=1, q_len=last, seq_lens=w.seq_lens[B - 1:]))
    score_ms = stage_ms[0]
    score_gbps = ab_launch["score_kernel"] / (score_ms * 1e-3) / 1e9
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
               "cpu_model": cpu_model(),
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
        "launches_per_stage": launches, "tile_tokens": n_tile,
        "stages_us": {"scores": stage_ms[0] * 1e3, "topk": stage_ms[1] * 1e3, "attention": stage_ms[2] * 1e3,
                      "of": "one step" if n_tile <= 0 else f"the last of {launches} token tiles"},
        "roofline": {"kernel": "score_mfma_kernel", "bound": "hbm", "achieved": score_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_launch": ab_launch["score_kernel"],
                     "launch_us": score_ms * 1e3},
        # the attention stage (sparse MLA + split merge, eager launches):
        # against HBM on its gathered bytes and against the dense bf16
        # matrix-core peak on its flops
        "roofline_attention": {"kernel": "mla_mfma_kernel+mla_combine_kernel", "stage_us": stage_ms[2] * 1e3,
                               "bytes_per_launch": ab_launch["attention"],
                               "hbm_gbps": ab_launch["attention"] / (stage_ms[2] * 1e-3) / 1e9,
                               "hbm_frac": ab_launch["attention"] / (stage_ms[2] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                               "flops_per_launch": ab_launch["attention_flops"],
                               "tflops": ab_launch["attention_flops"] / (stage_ms[2] * 1e-3) / 1e12,
                               "mfma_frac": ab_launch["attention_flops"] / (stage_ms[2] * 1e-3) / 1e12 /
                               BF16_PEAK_TFLOPS,
                               "traffic": (lambda a, b: a + b if a is not None and b is not None else None)(
                                   read_traffic_record(args.workload, "mla_mfma_kernel"),
                                   read_traffic_record(args.workload, "mla_combine_kernel"))},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the sparse GQA hot path on one MI355X.

One step = one ``sgqa_forward`` (block merging -> indexer scores + causal
top-k -> sparse GQA attention) of one attention layer over one batch of
seeded synthetic input already resident in HBM.  Default workload: the
single-layer prefill of 8,192 tokens (64 heads / 4 KV groups / head_dim 192,
indexer 4 x 128 per group, B=8, k = 512 blocks = 4,096 tokens).

Prints one JSON line with whole-step throughput, the distribution of single
step times (warm, and cold: a 512 MiB write between steps evicts the caches),
the roofline of the dominant kernel (its per-launch time measured with HIP
events on the stream it runs on, against AMD's published peak and against
what this GPU reaches on a plain copy and a bf16 GEMM), and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--paged] [--neighbours] [--store-bf16 | --store-e4m3-bf16] [--no-cold] [--no-peaks]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-GQA prefill tokens/s + decode queries/s on 1 GPU; % of HBM/MFMA peak"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BPS = 8.0e12         # MI355X HBM3E
H, G, D, HI, DI = 64, 4, 192, 4, 128


# ---------------------------------------------------------------------------
# algorithmic work of one step (what the method must compute / move)
# ---------------------------------------------------------------------------

def work_model(wl, seqs=None) -> dict:
    """Work of one step over `seqs` (default: the workload's sequences)."""
    B, K = wl.block_size, wl.topk
    row_bytes = DI * (1 if wl.store_q8 == 2 else 2)     # E4M3 codes or bf16 values
    attn_pairs = 0          # sum over (t, g) of |U_t,g|
    idx_pairs = 0           # sum over t of b(t) (per group)
    comp_blocks = 0
    store_bytes = 0
    seqs = wl.seqs if seqs is None else seqs
    for s in seqs:
        t = np.arange(s.pos0, s.pos0 + s.n_q, dtype=np.int64)
        b = t // B
        u = np.minimum(b, K) * B + (t - b * B) + 1
        attn_pairs += int(u.sum()) * G
        idx_pairs += int(b.sum())
        store_bytes += int(b.sum()) * row_bytes
        comp_blocks += s.cache_len // B - s.pos0 // B
    return {
        "attn_flops": attn_pairs * (H // G) * 4 * D,        # QK^T + PV, 2 flop per MAC
        "attn_gather_bytes": attn_pairs * 2 * D * 2,          # K and V rows, bf16
        "index_flops": idx_pairs * G * HI * 2 * DI,
        "index_store_bytes": store_bytes,                     # store read once per query
        "compress_bytes": comp_blocks * (B * (DI * 2 + DI * 4) + row_bytes),
        "queries": sum(s.n_q for s in seqs),
    }


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(wl, budget_s: float = 10.0) -> dict:
    """The oracle, as written, on a bounded sample of the step: the merge of up
    to 2,048 of the step's blocks plus uniformly drawn query rows through
    scoring, top-k and attention until ``budget_s`` is spent, scaled to the
    whole step by block and query counts."""
    from oracle import numerics as nu
    from oracle import sgqa as O
    from synth import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    cfg = O.Config(block_size=wl.block_size, topk_blocks=wl.topk, store_q8=bool(wl.store_q8))
    rng = np.random.default_rng(0)
    B = wl.block_size
    total_q = sum(x.n_q for x in wl.seqs)
    step_blocks = sum(x.cache_len // B - x.pos0 // B for x in wl.seqs)

    def store_prefix(s, n_blocks):
        rows = s.kv_offset + np.arange(B * n_blocks)
        return O.compress(W.host_proxy(wl, rows), W.host_logits(wl, rows), np.arange(n_blocks), cfg)[0]

    # (1) merge: the first min(step, 2048) blocks the step compresses
    s0 = next(x for x in wl.seqs if x.cache_len // B > x.pos0 // B) if step_blocks else wl.seqs[0]
    first, nb = s0.pos0 // B, min(max(s0.cache_len // B - s0.pos0 // B, 0), 2048)
    rows = s0.kv_offset + np.arange(B * first, B * (first + nb))
    kp = np.zeros((B * (first + nb), DI), dtype=np.uint16)
    lg = np.zeros((B * (first + nb), DI), dtype=np.float32)
    kp[B * first:] = W.host_proxy(wl, rows)
    lg[B * first:] = W.host_logits(wl, rows)
    t0 = time.perf_counter()
    O.compress(kp, lg, np.arange(first, first + nb), cfg)
    t_comp = (time.perf_counter() - t0) * step_blocks / max(nb, 1)
    # (2) query rows through steps 2-4; the store they search is the real one
    #     up to 8,192 blocks, repeated cyclically beyond (pace only)
    prefix = {}
    kv_full = None
    if wl.kv_rows * G * D <= (1 << 26):          # small caches: regenerate once
        kv_full = (W.host_k(wl, np.arange(wl.kv_rows)), W.host_v(wl, np.arange(wl.kv_rows)))
    n_rows, t_rows = 0, 0.0
    while t_rows < budget_s and n_rows < total_q:
        si = int(rng.integers(0, len(wl.seqs)))
        s = wl.seqs[si]
        if s.n_q == 0:
            continue
        if si not in prefix:
            prefix[si] = store_prefix(s, min((s.cache_len - 1) // B, 8192))
        qi = int(rng.integers(0, s.n_q))
        t = s.pos0 + qi
        b = t // B
        st = prefix[si]
        store = st[np.arange(b) % max(st.shape[0], 1)] if b > st.shape[0] else st[:b]
        qrow = s.q_offset + qi
        qi_bits, w_row, q_bits = W.host_q_idx(wl, [qrow]), W.host_w(wl, [qrow])[0], W.host_q(wl, [qrow])[0]
        t1 = time.perf_counter()
        qh = O.index_queries(qi_bits, [t], cfg)[0]
        w = w_row.astype(np.float64)
        q = nu.bf16_bits_to_f64(q_bits)
        sels = []
        for g in range(G):
            sc = O.block_scores(qh[g], w[g], store)
            sels.append(O.token_set(O.select_blocks(sc, wl.topk), t, B))
        toks = np.unique(np.concatenate(sels))
        t_rows += time.perf_counter() - t1
        if kv_full is not None:
            k_bits, v_bits = kv_full[0][s.kv_offset + toks], kv_full[1][s.kv_offset + toks]
        else:
            k_bits, v_bits = W.host_k(wl, s.kv_offset + toks), W.host_v(wl, s.kv_offset + toks)
        t1 = time.perf_counter()
        kk, vv = nu.bf16_bits_to_f64(k_bits), nu.bf16_bits_to_f64(v_bits)
        for g in range(G):
            u = np.searchsorted(toks, sels[g])
            O.attend(q[16 * g:16 * g + 16], kk[u, g], vv[u, g], cfg.softmax_scale)
        t_rows += time.perf_counter() - t1
        n_rows += 1
    est = t_comp + t_rows / max(n_rows, 1) * total_q
    unit = "queries/s" if wl.name.startswith("decode") else "tokens/s"
    return {"value": total_q / est, "unit": unit, "cores": int(cores), "kind": "oracle",
            "sample": f"{n_rows} uniformly drawn query rows through scoring, top-k and attention "
                      f"({t_rows:.1f} s, input regeneration excluded) plus the merge of {nb} "
                      f"blocks, scaled to {total_q} queries and {step_blocks} blocks; "
                      f"est. {est:.2f} s per step"}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def recorded_counters(workload: str, kernels):
    """HBM bytes per call of the attention kernels `kernels` on `workload`,
    summed over them, from committed counter summaries under profiles/
    (FETCH_SIZE and WRITE_SIZE, calibrated against a device copy), or None
    when a kernel has no summary for that workload or its source has changed
    since the counters were taken."""
    import glob
    import hashlib
    recs = {}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        rec = {}
        for line in open(path):
            line = line.strip()
            if line.startswith("traffic_workload: ") and rec:
                recs[(rec.get("traffic_workload"), rec.get("traffic_kernel"))] = rec
                rec = {}
            parts = line.split(": ", 1)
            if len(parts) == 2 and parts[0].startswith(("traffic_", "source_")):
                rec[parts[0]] = parts[1]
        if rec:
            recs[(rec.get("traffic_workload"), rec.get("traffic_kernel"))] = rec
    total = {"fetch": 0, "write": 0}
    for kernel in kernels:
        rec = recs.get((workload, kernel))
        if rec is None:
            return None
        src = os.path.join(ROOT, rec.get("source_file", ""))
        if not os.path.isfile(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
            return None
        total["fetch"] += int(rec["traffic_fetch_bytes_per_launch"])
        total["write"] += int(rec["traffic_write_bytes_per_launch"])
    return total


def measured_peaks(stream) -> dict:
    """What this GPU reaches on plain work: a 1 GiB device-to-device copy
    (bytes read + written per second), a 1 GiB fp32 sum (bytes read per
    second) and a bf16 8192^3 matrix product, all through torch."""
    import torch
    out = {}
    with torch.cuda.stream(stream):
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        ms = event_time_ms(lambda: b.copy_(a), stream, 10)
        out["hbm_copy_GBps"] = 2 * a.numel() / (ms * 1e-3) / 1e9
        f = a.view(torch.float32).zero_()
        for _ in range(3):
            f.sum()
        ms = event_time_ms(lambda: f.sum(), stream, 10)
        out["hbm_read_GBps"] = a.numel() / (ms * 1e-3) / 1e9
        del a, b, f
        n = 8192
        x = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
        y = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            torch.matmul(x, y)
        ms = event_time_ms(lambda: torch.matmul(x, y), stream, 10)
        out["bf16_gemm_TFLOPs"] = 2 * n ** 3 / (ms * 1e-3) / 1e12
        del x, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def step_times(step, stream, n: int, flush=None) -> dict:
    """Per-step HIP-event times over n steps on the launch stream: median,
    10th and 90th percentile.  With `flush` (cold mode) a 512 MiB buffer is
    written before every step, outside the timed interval, so the step starts
    with the L2s and the Infinity Cache holding none of its inputs."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    with torch.cuda.stream(stream):
        for i in range(n):
            if flush is not None:
                flush.fill_(i & 0x7F)
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
            "p90_ms": float(np.percentile(ms, 90)), "n": n}


def event_time_ms(fn, stream, reps: int) -> float:
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 512 MiB device-to-device copy (HBM byte-counter scale)")
    ap.add_argument("--paged", action="store_true",
                    help="per-token caches as pools of 16-token pages behind a random page table")
    ap.add_argument("--neighbours", action="store_true",
                    help="each step also runs the main Q/K producer (RMSNorm, partial rotary span, "
                         "cache writes) before the path and the sigmoid output gate in the attention")
    ap.add_argument("--store-bf16", action="store_true",
                    help="keep the store in bf16 (no E4M3 rounding: the ablation)")
    ap.add_argument("--store-e4m3-bf16", action="store_true",
                    help="hold the E4M3 store values in bf16 (store_q8 = 1) instead of one-byte codes")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache step times")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring this GPU's copy bandwidth and bf16 GEMM rate")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU part); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch

    import sparse_long_context_block_amd as sg
    from synth import workloads as W
    from tests.gpu_setup import lib_seq, lib_seqs, prepare

    if args.store_bf16 and args.store_e4m3_bf16:
        print("--store-bf16 and --store-e4m3-bf16 exclude each other", file=sys.stderr)
        return 2
    wl = W.make(args.workload, store_q8=0 if args.store_bf16 else 1 if args.store_e4m3_bf16 else 2)
    if args.paged and wl.loop_steps:
        print("bench.py --paged takes workloads of one call", file=sys.stderr)
        return 2
    print(f"[bench] workload {wl.name}: preparing inputs", file=sys.stderr, flush=True)
    di, cfg = prepare(wl)
    pools = table = None
    if args.paged:
        # the same logical contents in page pools; the contiguous copies go
        pools, table, layouts = W.paginate(wl, di, np.random.default_rng(0))
        for name in ("k", "v", "proxy_k", "logits"):
            di.t[name] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    nb = None
    if args.neighbours:
        # raw main Q/K/V of the new tokens (bf16 unit normal) and gate logits;
        # the producer writes Q and the new tokens' K/V cache rows every step
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        nq_rows = di["q"].shape[0]
        bf = dict(dtype=torch.bfloat16, device="cuda", generator=gen)
        nb = {"q_raw": torch.randn(nq_rows, H, D, **bf), "k_raw": torch.randn(nq_rows, G, D, **bf),
              "v_raw": torch.randn(nq_rows, G, D, **bf), "gate": torch.randn(nq_rows, H, D, **bf),
              "qk": sg.qk_config()}
    # a loop of calls (a decode loop: one token per sequence per call; a
    # chained prefill: one chunk per call) runs call k at step k, wrapping
    # around; repeating a call recomputes the same outputs
    if wl.loop_steps:
        loop = [[lib_seq(s) for s in wl.step_seqs(k)] for k in range(wl.loop_steps)]
        ws_n = max(sg.workspace_size(cfg, sq, sg.OP_FORWARD) for sq in loop)
    elif args.paged:
        loop = [[lib_seq(s) for s in layouts]]
        ws_n = sg.workspace_size(cfg, loop[0], sg.OP_FORWARD)
    else:
        loop = [lib_seqs(wl)]
        ws_n = sg.workspace_size(cfg, loop[0], sg.OP_FORWARD)
    stream = torch.cuda.current_stream()
    ws = torch.empty(max(ws_n, 1) + 256, dtype=torch.uint8, device="cuda")
    ws_view = ws[(-ws.data_ptr()) % 256:][:max(ws_n, 1)]
    step_no = [0]

    k_cache = pools["k"] if pools is not None else di["k"]
    v_cache = pools["v"] if pools is not None else di["v"]
    gate = nb["gate"] if nb else None

    def op_qk_prep(sq):
        sg.qk_prep(cfg, nb["qk"], sq, nb["q_raw"], nb["k_raw"], di["q"], k_cache, v_raw=nb["v_raw"],
                   v_cache=v_cache, page_table=table, stream=stream)

    def step():
        sq = loop[step_no[0] % len(loop)]
        step_no[0] += 1
        if nb:
            op_qk_prep(sq)
        if pools is not None:
            sg.forward_paged(cfg, sq, pools["proxy_k"], pools["logits"], di["store"], di["q_idx"],
                             di["w"], di["sel"], di["q"], pools["k"], pools["v"], table, di["out"],
                             lse=di["lse"], gate=gate, ws=ws_view, stream=stream)
        elif nb:
            sg.forward_gated(cfg, sq, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"],
                             di["sel"], di["q"], di["k"], di["v"], di["out"], gate, lse=di["lse"],
                             ws=ws_view, stream=stream)
        else:
            sg.forward(cfg, sq, di["proxy_k"], di["logits"], di["store"], di["q_idx"], di["w"],
                       di["sel"], di["q"], di["k"], di["v"], di["out"], lse=di["lse"],
                       ws=ws_view, stream=stream)

    def op_compress():
        if pools is not None:
            sg.compress_paged(cfg, seqs, pools["proxy_k"], pools["logits"], table, di["store"],
                              stream=stream)
            return
        sg.compress(cfg, seqs, di["proxy_k"], di["logits"], di["store"], stream=stream)

    def op_index():
        sg.index_topk(cfg, seqs, di["q_idx"], di["w"], di["store"], di["sel"],
                      ws=ws_view, stream=stream)

    def op_attn():
        if pools is not None:
            sg.sparse_attn_paged(cfg, seqs, di["q"], pools["k"], pools["v"], table, di["sel"],
                                 di["out"], lse=di["lse"], gate=gate, ws=ws_view, stream=stream)
        elif nb:
            sg.sparse_attn_gated(cfg, seqs, di["q"], di["k"], di["v"], di["sel"], di["out"], gate,
                                 lse=di["lse"], ws=ws_view, stream=stream)
        else:
            sg.sparse_attn(cfg, seqs, di["q"], di["k"], di["v"], di["sel"], di["out"],
                           lse=di["lse"], ws=ws_view, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps}", file=sys.stderr,
          flush=True)
    first_timed = step_no[0]
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    timed = [loop[k % len(loop)] for k in range(first_timed, step_no[0])]
    # the distribution of single steps (after the timed region): warm, and
    # for workloads of one call also cold; a loop's steps are different calls
    n_dist = min(args.steps, 20)
    dist = {"warm": step_times(step, stream, n_dist)} if n_dist > 0 else {}
    if not args.no_cold and not wl.loop_steps and n_dist > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dist["cold"] = step_times(step, stream, n_dist, flush)
        del flush
    print(f"[bench] step times {dist}", file=sys.stderr, flush=True)
    # per-op timings and the roofline use the loop's last call (its longest
    # context), or the step itself
    seqs = loop[-1]

    reps = args.kernel_reps
    k_ms = {
        "compress": event_time_ms(op_compress, stream, reps),
        "index_topk": event_time_ms(op_index, stream, reps),
        "sparse_attn": event_time_ms(op_attn, stream, reps),
    }
    if nb:
        k_ms["qk_prep"] = event_time_ms(lambda: op_qk_prep(seqs), stream, reps)
    print(f"[bench] per-op ms {k_ms}", file=sys.stderr, flush=True)

    peaks = None if args.no_peaks else measured_peaks(stream)
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if wl.loop_steps:
        op_seqs = wl.step_seqs(wl.loop_steps - 1)
        wm = work_model(wl, op_seqs)
        # throughput over the timed calls
        wm_loop_queries = sum(sum(s.n_q for s in sq) for sq in timed)
    else:
        op_seqs = wl.seqs
        wm = work_model(wl)
        wm_loop_queries = None
    decode = wl.name.startswith("decode")
    dense = sum(min(s.n_q, max(0, 4 * wl.topk * wl.block_size - s.pos0)) if s.n_q >= 64 else 0
                for s in op_seqs)
    if decode:
        # dominant op: the attention call (the gather; a split call adds the
        # merge), HBM-bound:
        # every gathered K/V row is read once per query and group
        achieved = wm["attn_gather_bytes"] / (k_ms["sparse_attn"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                "frac": achieved / (PEAK_HBM_BPS / 1e9), "traffic": None,
                "kernel": "sparse_attn_kernel (one sgqa_sparse_attn call; calls split across workgroups add attn_merge_kernel)",
                "algorithmic_bytes_per_launch": wm["attn_gather_bytes"],
                "launch_ms": k_ms["sparse_attn"]}
        ctr = (recorded_counters(wl.name, ["sparse_attn_kernel<false>"])
               if not args.paged and not nb and wl.store_q8 and not wl.loop_steps else None)
        if ctr:
            roof["traffic"] = ctr["fetch"] + ctr["write"]
            roof["reuse"] = wm["attn_gather_bytes"] / ctr["fetch"]
        if peaks:
            roof["measured_peak"] = max(peaks["hbm_copy_GBps"], peaks["hbm_read_GBps"])
            roof["frac_of_measured"] = achieved / roof["measured_peak"]
        # the indexer and the attention together: the store streamed once per
        # query plus the gathered K/V rows, over both calls' event times
        path_bytes = wm["index_store_bytes"] + wm["attn_gather_bytes"]
        path_ms = k_ms["index_topk"] + k_ms["sparse_attn"]
        roof["index_plus_attention"] = {
            "bytes": path_bytes, "ms": path_ms, "GBps": path_bytes / (path_ms * 1e-3) / 1e9,
            "frac": path_bytes / (path_ms * 1e-3) / PEAK_HBM_BPS}
        queries = wm_loop_queries / args.steps if wm_loop_queries else wm["queries"]
        value, unit = queries / (ms_step * 1e-3), "queries/s"
    else:
        achieved = wm["attn_flops"] / (k_ms["sparse_attn"] * 1e-3) / 1e12
        lb = wl.block_size.bit_length() - 1
        kern = (f"attn_union_kernel<{lb}>" if dense == wm["queries"]
                else "sparse_attn_kernel" if dense == 0
                else f"attn_union_kernel<{lb}> + sparse_attn_kernel ({dense} of {wm['queries']} "
                     f"queries tiled)")
        # counters were taken on the plain (contiguous, ungated) call that
        # runs one attention kernel
        union_k = "attn_union_kernel<%d, false>" % (wl.block_size.bit_length() - 1)
        ctr_kernels = ([union_k] if dense == wm["queries"] else ["sparse_attn_kernel<false>"] if dense == 0
                       else [union_k, "sparse_attn_kernel<false>"])
        ctr = (recorded_counters(wl.name, ctr_kernels)
               if not args.paged and not nb and wl.store_q8 and not wl.loop_steps else None)
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_FLOPS / 1e12,
                "unit": "TFLOP/s", "frac": achieved / (PEAK_BF16_FLOPS / 1e12),
                "traffic": ctr["fetch"] + ctr["write"] if ctr else None,
                "kernel": kern,
                "algorithmic_flops_per_launch": wm["attn_flops"],
                "launch_ms": k_ms["sparse_attn"]}
        if peaks:
            roof["measured_peak"] = peaks["bf16_gemm_TFLOPs"]
            roof["frac_of_measured"] = achieved / peaks["bf16_gemm_TFLOPs"]
        if ctr:
            # K/V bytes a gather per (query, group) would move over the bytes
            # the kernel fetched from HBM
            roof["reuse"] = wm["attn_gather_bytes"] / ctr["fetch"]
        if dense < wm["queries"]:
            # gathered K/V rows (768 B per query, group and attended token):
            # the rate the gather kernel moves them at, against HBM peak
            roof["gathered_GBps"] = wm["attn_gather_bytes"] / (k_ms["sparse_attn"] * 1e-3) / 1e9
        queries = wm_loop_queries / args.steps if wm_loop_queries else wm["queries"]
        value, unit = queries / (ms_step * 1e-3), "tokens/s"

    res = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + ("+paged" if args.paged else "")
                   + ("+neighbours" if nb else ""), "queries": wm["queries"],
                   "block_size": wl.block_size,
                   "topk_blocks": wl.topk, "store_q8": wl.store_q8,
                   "heads": H, "kv_groups": G, "head_dim": D},
        "per_op_ms": k_ms,
        "step_times": dist,
        "roofline": roof,
    }
    if peaks:
        res["measured_peaks"] = peaks
    if wl.loop_steps:
        res["config"]["loop_calls"] = wl.loop_steps
        res["config"]["per_op_call"] = wl.loop_steps - 1
        if args.steps % wl.loop_steps == 0:
            # wall time of one pass over every call of the loop (a chained
            # prefill: the whole prefill of one layer)
            res["loop_pass_s"] = wall / (args.steps // wl.loop_steps)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        if wl.loop_steps:
            import dataclasses
            one = dataclasses.replace(wl, seqs=wl.step_seqs(wl.loop_steps - 1),
                                      loop_steps=0, loop_seqs=0)
            res["cpu_baseline"] = cpu_baseline(one)
        else:
            res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

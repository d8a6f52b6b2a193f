#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

One step = one pass of the whole hot path over the two headline workloads:
  * decode at 1M context: 4 sequences x 1 query, H=64, h=8, d=128, d_idx=64,
    B=64, k=1024  (msa_index_topk + msa_sparse_attn_decode)
  * causal prefill of 32768 tokens: H=32, h=8, d=128, d_idx=64, B=64, k=32,
    clustered keys  (msa_index_topk + msa_sparse_attn_prefill)
Inputs are seeded synthetic bf16 tensors, resident in HBM before timing starts.

Prints one JSON line: whole-step tokens/s, per-workload results, the roofline
of the dominant kernel (algorithmic bytes or flops per launch over its HIP-event
duration) and the CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MSA tokens/s: decode@1M ctx & prefill@32k; % of HBM/MFMA roofline"
WORKLOADS = ("decode_1m", "prefill_32k")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_tokens(ids, cu_q, cu_k, B):
    """Per (row, group): number of visible tokens in the selected blocks (torch, on device)."""
    import torch
    total_q, h, k = ids.shape
    rows = torch.arange(total_q, device=ids.device)
    seq = torch.searchsorted(cu_q.long(), rows, right=True) - 1
    len_q = (cu_q[1:] - cu_q[:-1]).long()[seq]
    len_k = (cu_k[1:] - cu_k[:-1]).long()[seq]
    p = (len_k - len_q + rows - cu_q.long()[seq]).view(total_q, 1, 1)
    j = ids.long()
    n = torch.clamp(p - j * B + 1, min=0, max=B)
    return torch.where(j >= 0, n, torch.zeros_like(n)).sum(dim=2)   # [total_q, h]


def algorithmic(inp, dp, ids):
    """Algorithmic work of each entry point (what MSA itself must move or compute)."""
    wl = inp.wl
    H, h, d, di, B = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.index_dim, wl.block_size
    vis = visible_tokens(ids, dp.cu_q, dp.cu_k, B)            # [total_q, h]
    tok_sel = int(vis.sum().item())
    lens_q = np.diff(inp.cu_seqlens_q).astype(np.int64)
    lens_k = np.diff(inp.cu_seqlens_k).astype(np.int64)
    # index scores: every query scores every visible key for each group
    sum_vis_keys = int(sum(((lk - lq) * lq + lq * (lq + 1) // 2) for lq, lk in zip(lens_q, lens_k)))
    index_flops = 2.0 * di * h * sum_vis_keys
    attn_flops = 4.0 * d * (H // h) * tok_sel
    index_bytes = float(wl.total_k * di * 2 + wl.total_q * h * di * 2 + wl.total_q * h * wl.top_k * 4)
    attn_bytes = float(tok_sel * d * 2 * 2 + 2 * wl.total_q * H * d * 2 + wl.total_q * h * wl.top_k * 4)
    return dict(index_flops=index_flops, attn_flops=attn_flops, index_bytes=index_bytes, attn_bytes=attn_bytes,
                selected_tokens=tok_sel)


def cpu_baseline(inputs, budget_s=24.0, seed=7):
    """The oracle (untuned) on a bounded sample of the step, scaled to tokens/s.

    Workloads share the time budget in order, each taking an even share of what
    is left.  Decode: whole sequences, in order (at least one).  Prefill: chunks
    of 256 uniformly drawn rows.  Each part is extrapolated linearly to its full
    workload.
    """
    import oracle
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    parts, secs, spent = [], 0.0, 0.0
    for n_done, (name, inp) in enumerate(inputs.items()):
        share = (budget_s - spent) / (len(inputs) - n_done)
        wl = inp.wl
        if wl.is_decode:
            units = [np.array([r], dtype=np.int64) for r in range(wl.total_q)]
            what = "sequences"
        else:
            rng = np.random.Generator(np.random.PCG64(seed))
            perm = rng.permutation(wl.total_q).astype(np.int64)
            units = [np.sort(perm[i:i + 256]) for i in range(0, wl.total_q, 256)]
            what = "uniformly drawn rows"
        done, dt = 0, 0.0
        for rows in units:
            t0 = time.perf_counter()
            ids, _, _ = oracle.index_topk(inp, rows, threads=threads)
            oracle.sparse_attention(inp, ids, rows, threads=threads)
            dt += time.perf_counter() - t0
            done += len(rows)
            if dt >= share:
                break
        spent += dt
        secs += dt * wl.total_q / done
        parts.append(f"{name}: {done} of {wl.total_q} {what} in {dt:.1f} s")
    tokens = sum(inp.wl.total_q for inp in inputs.values())
    return {"value": tokens / secs, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(parts) + "; each part extrapolated linearly to its full workload"}


def measured_traffic(kernel_file, symbol, launches_per_call, workload):
    """HBM bytes per call of the dominant kernel from the committed PMC summary.

    The summary records FETCH_SIZE / WRITE_SIZE per dispatch, the scale factors
    a plain copy of known size gives for the same counters, the SHA-256 of the
    kernel source the counters were taken on, and the workloads they were
    taken on.  If that source has changed since, or the workload is another,
    the counters do not describe this launch and None is returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    src = os.path.join(ROOT, "block_sparse_gqa_amd", "csrc", kernel_file)
    try:
        with open(path) as f:
            table = json.load(f)
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if workload not in table.get("workload", "").replace("+", " ").split():
        return None
    for e in table.get("kernels", []):
        if e.get("symbol") == symbol and e.get("source_sha256") == digest:
            return e["bytes_per_dispatch"] * launches_per_call
    return None


def decode_reps(dp, bufs, reps=100, flush_mb=1024):
    """The decode step alone, `reps` times, with a read of a `flush_mb` buffer
    between repetitions so that no repetition finds the previous one's data
    in L2 or the 256 MB MALL; each repetition is timed with its own events.
    The flush reads (the library's streaming-read kernel) rather than writes:
    a written buffer leaves dirty lines whose write-back would then compete
    with the timed decode."""
    import torch

    from block_sparse_gqa_amd import device, msa
    ids, out, lse = bufs
    scratch = torch.zeros(flush_mb << 20, dtype=torch.uint8, device=dp.q.device)
    sink = torch.zeros(1, dtype=torch.int32, device=dp.q.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        msa.msa_ceiling_stream_read(scratch, sink)
        e0.record()
        device.index_topk(dp, ids)
        device.sparse_attention(dp, ids, out, lse)
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    del scratch, sink
    torch.cuda.empty_cache()
    return {"reps": reps, "flush_MB_read": flush_mb, "ms_median": float(np.median(t)), "ms_min": float(t.min()),
            "ms_mean": float(t.mean())}


def paged_decode(inp, dp, ids_contig, contig, steps, warmup):
    """The same decode step over a paged copy of the cache: pages scattered
    at random through a pool with spare pages, filled by the append kernel.
    Reported beside the headline (which uses the contiguous cache)."""
    import torch

    from block_sparse_gqa_amd import device
    wl = inp.wl
    blocks = sum((n + wl.block_size - 1) // wl.block_size for n in wl.seqlens_k)
    num_pages = blocks + blocks // 16
    table = device.random_page_table(wl.seqlens_k, wl.block_size, num_pages, seed=17)
    pc = device.alloc_paged(wl, table, num_pages)
    log(f"[bench] paged copy of {wl.name}: {blocks} blocks in a pool of {num_pages} pages")
    slots = device.cache_slots(dp, table)
    device.page_in(dp, pc, table, slots)   # once untimed (the same rows are written again below)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    device.page_in(dp, pc, table, slots)
    e[1].record()
    torch.cuda.synchronize()
    t_append = e[0].elapsed_time(e[1])
    append_bytes = 2 * wl.total_k * (2 * wl.num_kv_heads * wl.head_dim + wl.index_dim) * 2   # read + write
    ids = device.alloc_ids(dp)
    out, lse = device.alloc_out(dp)
    for _ in range(warmup):
        device.index_topk_paged(dp, pc, ids)
        device.sparse_attention_paged(dp, pc, ids, out, lse)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for x in ev:
        x[0].record()
        device.index_topk_paged(dp, pc, ids)
        x[1].record()
        device.sparse_attention_paged(dp, pc, ids, out, lse)
        x[2].record()
    torch.cuda.synchronize()
    t_idx = float(np.mean([x[0].elapsed_time(x[1]) for x in ev]))
    t_att = float(np.mean([x[1].elapsed_time(x[2]) for x in ev]))
    gbs = contig["algorithmic_GB"] / ((t_idx + t_att) * 1e-3)
    same = bool(torch.equal(ids, ids_contig))
    del pc
    torch.cuda.empty_cache()
    return {"ms": t_idx + t_att, "index_topk_ms": t_idx, "sparse_attn_ms": t_att, "GB_per_s": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "pages": num_pages, "ids_equal_contiguous": same,
            "page_in_ms": t_append, "page_in_GB_per_s": append_bytes / (t_append * 1e-3) / 1e9}


def prefill_backward(dp, bufs, fwd, steps):
    """Backward of the sparse branch (selection fixed) for the prefill step,
    on the forward's own ids, out and lse.  Reported beside the headline."""
    import torch

    from block_sparse_gqa_amd import device, msa
    ids, out, lse = bufs
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    dout = torch.randn(out.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    ws = device._workspace(msa.MSA_OP_SPARSE_ATTN_BACKWARD, dp.problem, dp.q.device)
    device.sparse_attention_backward(dp, ids, out, lse, dout, ws)   # warm-up
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for _ in range(steps):
        device.sparse_attention_backward(dp, ids, out, lse, dout, ws)
    e[1].record()
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / steps
    # S (recomputed), dP, dV, dK, dQ: five products of 2 d flop per (head, visible token)
    flops = 2.5 * (fwd["sparse_attn_TFLOP_per_s"] * fwd["sparse_attn_ms"] * 1e-3)   # forward: S and P.V
    res = {"ms": ms, "algorithmic_TFLOP": flops, "TFLOP_per_s": flops / (ms * 1e-3),
           "frac_mfma_peak": flops / (ms * 1e-3) / MFMA_BF16_PEAK_TFLOPS, "workspace_GB": ws.numel() / 1e9}
    del ws, dout
    torch.cuda.empty_cache()
    return res


def prefill_schedules(dp, bufs, fwd, steps):
    """Both prefill schedules timed explicitly on the forward's own ids: the
    query tiles (msa_sparse_attn_prefill_tiles) and the block-centric one
    (msa_sparse_attn_prefill_blocks), with the one msa_sparse_attn_prefill
    picks for this shape and the largest difference between the two outputs.
    Reported beside the headline."""
    import torch

    from block_sparse_gqa_amd import device, msa
    ids = bufs[0]
    flops = fwd["sparse_attn_TFLOP_per_s"] * fwd["sparse_attn_ms"] * 1e-3
    res, outs = {}, {}
    for name, op, fn in (("tiles", msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, device.sparse_attention_tiles),
                         ("blocks", msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, device.sparse_attention_blocks)):
        ws = device._workspace(op, dp.problem, dp.q.device)
        o, l = device.alloc_out(dp)
        fn(dp, ids, o, l, ws)   # warm-up
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(steps):
            fn(dp, ids, o, l, ws)
        e[1].record()
        torch.cuda.synchronize()
        ms = e[0].elapsed_time(e[1]) / steps
        res[name] = {"ms": ms, "TFLOP_per_s": flops / (ms * 1e-3),
                     "frac_mfma_peak": flops / (ms * 1e-3) / MFMA_BF16_PEAK_TFLOPS,
                     "workspace_GB": (ws.numel() if ws is not None else 0) / 1e9}
        outs[name] = o
        del ws, l
        torch.cuda.empty_cache()
    need = msa.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, dp.problem)
    blocks_need = msa.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, dp.problem)
    res["auto"] = "blocks" if need == blocks_need else "tiles"
    res["max_abs_diff"] = float((outs["tiles"].float() - outs["blocks"].float()).abs().max())
    del outs
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workloads", default=",".join(WORKLOADS))
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the sparse-branch backward measurement (reported beside the headline, not in it)")
    ap.add_argument("--no-schedules", action="store_true",
                    help="skip timing both prefill schedules explicitly (reported beside the headline)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-cache decode measurement (reported beside the headline, not in it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU sharding of this path is "
              "described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_gqa_amd import device, msa, synth
    msa.load()
    torch.cuda.set_device(0)
    names = [n for n in args.workloads.split(",") if n]
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    inputs, dps, bufs = {}, {}, {}
    for name in names:
        log(f"[bench] generating {name}")
        inp = synth.make_inputs(name)
        inputs[name] = inp
        dps[name] = device.upload(inp)
        ids = device.alloc_ids(dps[name])
        out, lse = device.alloc_out(dps[name])
        bufs[name] = (ids, out, lse)
    torch.cuda.synchronize()

    def step(events=None):
        for i, name in enumerate(names):
            dp = dps[name]
            ids, out, lse = bufs[name]
            if events is not None:
                events[name][0].record()
            device.index_topk(dp, ids)
            if events is not None:
                events[name][1].record()
            device.sparse_attention(dp, ids, out, lse)
            if events is not None:
                events[name][2].record()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)] for n in names}
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step({n: ev[n][s] for n in names})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    results, kernels = {}, []
    total_tokens = 0
    for name in names:
        inp, dp = inputs[name], dps[name]
        ids = bufs[name][0]
        t_idx = float(np.mean([e[0].elapsed_time(e[1]) for e in ev[name]]))
        t_att = float(np.mean([e[1].elapsed_time(e[2]) for e in ev[name]]))
        per_step = np.array([e[0].elapsed_time(e[2]) for e in ev[name]])
        alg = algorithmic(inp, dp, ids)
        wl = inp.wl
        total_tokens += wl.total_q
        r = {"tokens": wl.total_q, "ms": t_idx + t_att, "tokens_per_s": wl.total_q / ((t_idx + t_att) * 1e-3),
             "ms_median": float(np.median(per_step)), "ms_min": float(per_step.min()),
             "index_topk_ms": t_idx, "sparse_attn_ms": t_att, "selected_tokens": alg["selected_tokens"],
             "workload": wl.description}
        if wl.is_decode:
            gbs_i = alg["index_bytes"] / (t_idx * 1e-3) / 1e9
            gbs_a = alg["attn_bytes"] / (t_att * 1e-3) / 1e9
            tot = (alg["index_bytes"] + alg["attn_bytes"]) / ((t_idx + t_att) * 1e-3) / 1e9
            r.update({"bound": "hbm", "algorithmic_GB": (alg["index_bytes"] + alg["attn_bytes"]) / 1e9,
                      "GB_per_s": tot, "frac_hbm_peak": tot / HBM_PEAK_GBS,
                      "index_topk_GB_per_s": gbs_i, "sparse_attn_GB_per_s": gbs_a})
            kernels.append(("msa_index_topk[%s]" % name, t_idx, "hbm", alg["index_bytes"], None))
            kernels.append(("msa_sparse_attn_decode[%s]" % name, t_att, "hbm", alg["attn_bytes"], None))
        else:
            tf_i = alg["index_flops"] / (t_idx * 1e-3) / 1e12
            tf_a = alg["attn_flops"] / (t_att * 1e-3) / 1e12
            tot = (alg["index_flops"] + alg["attn_flops"]) / ((t_idx + t_att) * 1e-3) / 1e12
            r.update({"bound": "mfma", "algorithmic_TFLOP": (alg["index_flops"] + alg["attn_flops"]) / 1e12,
                      "TFLOP_per_s": tot, "frac_mfma_peak": tot / MFMA_BF16_PEAK_TFLOPS,
                      "index_topk_TFLOP_per_s": tf_i, "sparse_attn_TFLOP_per_s": tf_a})
            kernels.append(("msa_index_topk[%s]" % name, t_idx, "mfma", alg["index_flops"], None))
            # One launch of attn_prefill_tile per call on the query-tile schedule.  The committed
            # counters cover that kernel on the workloads they name; the block-centric schedule's
            # three kernels have none, so its traffic stays null.
            on_blocks = (msa.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, dp.problem)
                         == msa.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, dp.problem))
            kernels.append(("msa_sparse_attn_prefill[%s]" % name, t_att, "mfma", alg["attn_flops"],
                            None if on_blocks else ("attn_prefill.hip", "attn_prefill_tile", 1, name)))
        results[name] = r

    kname, kms, kbound, kwork, ksrc = max(kernels, key=lambda x: x[1])
    if kbound == "hbm":
        achieved, peak, unit = kwork / (kms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = kwork / (kms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    roofline = {"bound": kbound, "kernel": kname, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": measured_traffic(*ksrc) if ksrc else None,
                "traffic_unit": "bytes per launch", "avg_launch_ms": kms}

    for name in names:
        if inputs[name].wl.is_decode:
            r = results[name]
            r["flushed_reps"] = decode_reps(dps[name], bufs[name])
            r["flushed_reps"]["GB_per_s_median"] = r["algorithmic_GB"] / (r["flushed_reps"]["ms_median"] * 1e-3)

    if not args.no_backward:
        for name in names:
            if not inputs[name].wl.is_decode:
                results[name]["backward"] = prefill_backward(dps[name], bufs[name], results[name],
                                                             max(args.steps // 2, 3))

    if not args.no_schedules:
        for name in names:
            if not inputs[name].wl.is_decode:
                results[name]["schedules"] = prefill_schedules(dps[name], bufs[name], results[name],
                                                               max(args.steps // 2, 3))

    if not args.no_paged:
        for name in names:
            if inputs[name].wl.is_decode:
                results[name]["paged"] = paged_decode(inputs[name], dps[name], bufs[name][0], results[name],
                                                      max(args.steps, 5), args.warmup)

    # achievable HBM rate on this GPU: a plain 4 GiB device-to-device copy (read + write)
    src = torch.empty(1 << 32, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record()
    for _ in range(5):
        dst.copy_(src)
    ce[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 32) * 5 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del dst
    # a read-only stream of the same 4 GiB and a pure MFMA loop, from the library's own kernels
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    msa.msa_ceiling_stream_read(src, sink)
    ce[0].record()
    nbytes = sum(msa.msa_ceiling_stream_read(src, sink) for _ in range(5))
    ce[1].record()
    torch.cuda.synchronize()
    read_gbs = nbytes / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src
    msa.msa_ceiling_mfma_bf16(1024, sink)
    ce[0].record()
    flops = sum(msa.msa_ceiling_mfma_bf16(32768, sink) for _ in range(3))
    ce[1].record()
    torch.cuda.synchronize()
    mfma_tfs = flops / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e12
    torch.cuda.empty_cache()
    achievable = {"hbm": read_gbs, "mfma": mfma_tfs}
    for r in results.values():
        if r["bound"] == "hbm":
            r["frac_hbm_achievable"] = r["GB_per_s"] / read_gbs
        else:
            r["frac_mfma_achievable"] = r["TFLOP_per_s"] / mfma_tfs
    roofline["achievable"] = achievable[kbound]
    roofline["frac_achievable"] = achieved / achievable[kbound]

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(inputs)

    line = {
        "metric": METRIC,
        "value": total_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) / clustered-block bf16 inputs, generated on the host)",
        "config": {"workload": " + ".join(names), "parallelism": "single GPU",
                   **{n: results[n]["workload"] for n in names}},
        "results": results,
        "roofline": roofline,
        "ceilings": {"hbm_copy_GB_per_s": copy_gbs, "hbm_stream_read_GB_per_s": read_gbs,
                     "mfma_bf16_TFLOP_per_s": mfma_tfs,
                     "note": "measured on this GPU: a device-to-device copy of 4 GiB (read + write bytes), a "
                             "full-line read-only stream of the same 4 GiB, and back-to-back 16x16x32 bf16 MFMAs "
                             "with no memory traffic"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

One step = one pass of the whole hot path over the two headline workloads:
  * decode at 1M context: 4 sequences x 1 query, H=64, h=8, d=128, d_idx=64,
    B=64, k=1024  (msa_index_topk + msa_sparse_attn_decode)
  * causal prefill of 32768 tokens: H=32, h=8, d=128, d_idx=64, B=64, k=32,
    clustered keys  (msa_index_topk + msa_sparse_attn_prefill)
Inputs are seeded synthetic bf16 tensors, resident in HBM before timing starts.

The other three configurations (the tiny prefill, decode at 64K context and
the ragged 4-sequence prefill) are then timed on their own and reported in
`results` beside the headline; they are not part of `value`.

Prints one JSON line: whole-step tokens/s, per-workload results, the roofline
of the dominant kernel (algorithmic bytes or flops per launch over its HIP-event
duration) and the CPU leg: the oracle timed on a bounded sample of the same
step, and every workload's top-k ids checked against the oracle's on sampled
rows (near ties and in-band flips counted, per workload).
"""
from __future__ import annotations

import argparse
import json
import os
import re
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
# The other three configurations: each timed on its own after the step, reported beside the
# headline (not part of `value`).
EXTRA_WORKLOADS = ("tiny_prefill", "decode_64k", "ragged_prefill")


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


def cpu_model():
    """The host CPU's model name and logical CPU count, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            names = [l.split(":", 1)[1].strip() for l in f if l.startswith("model name")]
    except OSError:
        names = []
    return {"model": names[0] if names else "unknown", "logical_cpus": len(names) or (os.cpu_count() or 0)}


def selection_parity(inputs, gpu_ids, seed=9):
    """Top-k ids of every workload against the oracle's on sampled rows, with the near-tie rule:
    near-tie pairs, in-band flips and exact mismatches (pairs differing outside the band)."""
    import oracle
    from block_sparse_gqa_amd import synth
    from tests import parity
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    res = {}
    for name, inp in inputs.items():
        wl = inp.wl
        if wl.is_decode or wl.total_q <= 1024:
            rows = np.arange(wl.total_q, dtype=np.int64)
            what = "every row"
        else:
            rows = synth.sample_rows(wl, n_per_seq=96, seed=seed)
            what = "sampled rows (block edges, sequence ends, seeded random)"
        t0 = time.perf_counter()
        ref_ids, kth, tie = oracle.index_topk(inp, rows, threads=threads)
        rep = parity.selection_report(oracle, inp, rows, gpu_ids[name][rows], ref_ids, kth, tie)
        rep.update({"rows_checked": what, "oracle_s": time.perf_counter() - t0})
        res[name] = rep
        log(f"[bench] selection parity {name}: {rep}")
    return res


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
            "cpu": cpu_model(),
            "sample": "; ".join(parts) + "; each part extrapolated linearly to its full workload"}


# The kernels one msa_sparse_attn_prefill call launches (source file, kernel), per schedule; the
# block-centric part runs in one chunk at the benchmarked sizes.
_TILE_KERNELS = [("attn_prefill.hip", "v_absmax_bits"), ("attn_prefill.hip", "v_scale_exp"),
                 ("attn_prefill.hip", "v_to_f16"), ("attn_prefill.hip", "attn_prefill_tile")]
_BLOCK_KERNELS = [("block_lists.hip", "lists_block_offsets"), ("block_lists.hip", "fill_zero_i32"),
                  ("block_lists.hip", "lists_count_lds"), ("block_lists.hip", "lists_scan"),
                  ("block_lists.hip", "lists_invert"), ("attn_block_fwd.hip", "fwd_block"),
                  ("attn_block_fwd.hip", "fwd_merge")]
PREFILL_CALL_KERNELS = {"tiles": _TILE_KERNELS, "blocks": _BLOCK_KERNELS, "tiles+blocks": _TILE_KERNELS + _BLOCK_KERNELS}


def measured_traffic(kernels, workload):
    """HBM bytes of one call from the committed PMC summary: the sum over the call's kernels.

    The summary records, per kernel, FETCH_SIZE / WRITE_SIZE per dispatch scaled by what the same
    counters read for a plain copy of known size, the SHA-256 of the kernel source the counters were
    taken on, and the workloads they were taken on.  If any kernel's source has changed since, or it
    has no entry for this workload, the counters do not describe this call and None is returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except OSError:
        return None
    total = 0.0
    for kernel_file, symbol in kernels:
        try:
            with open(os.path.join(ROOT, "block_sparse_gqa_amd", "csrc", kernel_file), "rb") as f:
                digest = hashlib.sha256(f.read()).hexdigest()
        except OSError:
            return None
        hit = [e for e in table.get("kernels", []) if e.get("symbol") == symbol and
               e.get("source_sha256") == digest and e.get("workload") == workload]
        if not hit:
            return None
        total += hit[0]["bytes_per_dispatch"]
    return total


CALIBRATION_COPIES = 3   # 1 GiB device-to-device copies that --calibrate-copy runs first


def _kernel_symbol(name):
    """Kernel symbol and instance from a profiler kernel name, e.g.
    'void msa::(anonymous namespace)::attn_prefill_tile<128, 16>(...)' -> ('attn_prefill_tile',
    'attn_prefill_tile<128, 16>')."""
    n = name.replace("(anonymous namespace)", "anon")
    n = n.split("(", 1)[0].strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):   # the last '::' outside template brackets starts the instance
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and n[i:i + 2] == "::":
            cut = i + 2
    inst = n[cut:] if cut < len(n) else n
    return inst.split("<", 1)[0], inst


def _counter_rows(run_dir, counter):
    """(dispatch id, kernel name, value) of one rocprofv3 --pmc pass (its *counter_collection.csv),
    in dispatch order."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (fn, int(row.get("Dispatch_Id") or row.get("Correlation_Id")))
                name, v = row["Kernel_Name"], float(row["Counter_Value"])
                per[key] = (name, per[key][1] + v if key in per else v)   # summed over XCDs/instances
    return [(key[1], name, v) for key, (name, v) in sorted(per.items())]


def traffic_table(specs, copy_bytes=1 << 30):
    """Write profiles/hbm_traffic.json from rocprofv3 counter passes.

    Each spec is WORKLOAD:FETCH_DIR:WRITE_DIR, two passes of `bench.py --workloads WORKLOAD
    --calibrate-copy` (FETCH_SIZE, then WRITE_SIZE).  The plain device copy of `copy_bytes` that
    --calibrate-copy runs gives the scale of each counter (bytes per counted KiB); every kernel of
    the library gets the mean of its dispatches in that pass, scaled, with the SHA-256 of the source
    file that defines it, so that a later change of the source invalidates the entry."""
    import hashlib
    csrc = os.path.join(ROOT, "block_sparse_gqa_amd", "csrc")
    sources = {}
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith(".hip"):
            with open(os.path.join(csrc, fn), "rb") as f:
                sources[fn] = f.read()

    def source_of(symbol):
        pat = re.compile(rb"__global__[^;{]*?\b" + re.escape(symbol.encode()) + rb"\s*\(", re.S)
        hits = [fn for fn, text in sources.items() if pat.search(text)]
        return hits[0] if len(hits) == 1 else None

    def scaled(rows):
        # the first copies of the run are --calibrate-copy's (the later ones are the ceiling's 4 GiB)
        copies = [v for _, name, v in rows if "copy" in name.lower()][:CALIBRATION_COPIES]
        if len(copies) < CALIBRATION_COPIES:
            raise SystemExit("no calibration copies in the pass: run it with --calibrate-copy")
        scale = copy_bytes / (float(np.median(copies)) * 1024.0)   # HBM bytes per counted byte
        kib = {}
        for _, name, v in rows:
            kib.setdefault(name, []).append(v)
        return scale, {name: float(np.mean(v)) for name, v in kib.items()}

    entries = []
    for spec in specs:
        workload, fetch_dir, write_dir = spec.split(":")
        fscale, fetch = scaled(_counter_rows(fetch_dir, "FETCH_SIZE"))
        wscale, write = scaled(_counter_rows(write_dir, "WRITE_SIZE"))
        for name in sorted(set(fetch) & set(write)):
            symbol, inst = _kernel_symbol(name)
            src = source_of(symbol)
            if src is None:
                continue   # not a kernel of this library (the copy, torch's fills)
            entries.append({
                "symbol": symbol, "instance": inst, "workload": workload,
                "source": "block_sparse_gqa_amd/csrc/" + src,
                "source_sha256": hashlib.sha256(sources[src]).hexdigest(),
                "fetch_size_kib": fetch[name], "write_size_kib": write[name],
                "fetch_scale": fscale, "write_scale": wscale,
                "bytes_per_dispatch": fetch[name] * 1024.0 * fscale + write[name] * 1024.0 * wscale})
    out = {"note": "HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB, mean over the pass's dispatches) "
                   "times bytes per counted KiB of a plain 1 GiB device copy in the same pass",
           "kernels": entries}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("| workload | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |")
    print("|---|---|---|---|---|---|")
    for e in entries:
        print(f"| {e['workload']} | `{e['instance']}` | {e['fetch_size_kib']:,.1f} | {e['write_size_kib']:,.1f} | "
              f"{e['fetch_size_kib'] * 1024 * e['fetch_scale'] / 1e6:,.1f} | "
              f"{e['write_size_kib'] * 1024 * e['write_scale'] / 1e6:,.1f} |")
    log(f"[bench] wrote {path}: {len(entries)} kernels")


def decode_reps(dp, bufs, reps=100, flush_mb=1024):
    """The decode step alone, `reps` times, with a read of a `flush_mb` buffer
    between repetitions so that no repetition finds the previous one's data
    in L2 or the 256 MB MALL; each repetition is timed with its own events.
    The flush reads rather than writes (a written buffer leaves dirty lines
    whose write-back would then compete with the timed decode), and it reads
    with plain loads (a torch reduction), which allocate in L2 and the MALL:
    the library's streaming-read kernel uses non-temporal loads and would leave
    the MALL holding the previous repetition's data."""
    import torch

    from block_sparse_gqa_amd import device
    ids, out, lse = bufs
    scratch = torch.ones((flush_mb << 20) // 4, dtype=torch.int32, device=dp.q.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        torch.amax(scratch)
        e0.record()
        device.index_topk(dp, ids)
        device.sparse_attention(dp, ids, out, lse)
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    del scratch
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
    ev = timed_events(steps)
    for x in ev:
        x[0].record()
        device.index_topk_paged(dp, pc, ids)
        device.sparse_attention_paged(dp, pc, ids, out, lse)
        x[2].record()
    torch.cuda.synchronize()
    t_all = float(np.mean([x[0].elapsed_time(x[2]) for x in ev]))
    t_idx, t_att = split_pass(lambda: device.index_topk_paged(dp, pc, ids),
                              lambda: device.sparse_attention_paged(dp, pc, ids, out, lse), steps)
    gbs = contig["algorithmic_GB"] / (t_all * 1e-3)
    same = bool(torch.equal(ids, ids_contig))
    del pc
    torch.cuda.empty_cache()
    return {"ms": t_all, "index_topk_ms": t_idx, "sparse_attn_ms": t_att, "GB_per_s": gbs,
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
    res["auto"] = prefill_schedule_of(dp)
    res["max_abs_diff"] = float((outs["tiles"].float() - outs["blocks"].float()).abs().max())
    del outs
    torch.cuda.empty_cache()
    return res


def forced_index(dp, ids, steps, sink=1, local=1):
    """The index branch with forced blocks (msa_index_topk_ex: the first `sink` and the last `local` eligible
    blocks of every row always kept), timed against the plain msa_index_topk in the same way, back to back on
    the same inputs.  Reported beside the headline."""
    import torch

    from block_sparse_gqa_amd import device
    fids = device.index_topk_forced(dp, sink, local)   # warm-up
    res = {"sink_blocks": sink, "local_blocks": local}
    for key, call in (("plain_ms", lambda: device.index_topk(dp, ids)),
                      ("forced_ms", lambda: device.index_topk_forced(dp, sink, local, fids))):
        call()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(steps):
            call()
        e[1].record()
        torch.cuda.synchronize()
        res[key] = e[0].elapsed_time(e[1]) / steps
    del fids
    return res


def prefill_schedule_of(dp):
    """What msa_sparse_attn_prefill runs for this problem, read from its workspace size: the query tiles,
    the block-centric schedule, or both (tiles for the early rows, the block-centric schedule after)."""
    from block_sparse_gqa_amd import msa
    ws = {op: msa.msa_workspace_size(op, dp.problem) for op in (msa.MSA_OP_SPARSE_ATTN_PREFILL,
                                                                 msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES,
                                                                 msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS)}
    auto = ws[msa.MSA_OP_SPARSE_ATTN_PREFILL]
    if auto == ws[msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES]:
        return "tiles"
    if auto == ws[msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS]:
        return "blocks"
    return "tiles+blocks"


def split_pass(index_call, attn_call, steps):
    """Index and attention times of one workload, from `steps` passes with a marker between the two
    calls.  Each marker costs the GPU a few microseconds of idle time, so the timed steps carry none
    between the calls of a workload whose split is not needed live; this pass gives that split
    instead (its two parts sum to slightly more than the step's own time)."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for x in ev:
        x[0].record()
        index_call()
        x[1].record()
        attn_call()
        x[2].record()
    torch.cuda.synchronize()
    return (float(np.mean([x[0].elapsed_time(x[1]) for x in ev])),
            float(np.mean([x[1].elapsed_time(x[2]) for x in ev])))


def timed_events(n):
    """`n` (start, None, end) triples for back-to-back timed passes of one workload."""
    import torch
    return [[torch.cuda.Event(enable_timing=True), None, torch.cuda.Event(enable_timing=True)] for _ in range(n)]


def summarize(inp, dp, ids, evs, split=None):
    """Per-workload result from the events of its timed calls: (start, index end = attention start or
    None, end) per step.  Without the middle marker, `split` gives the index and attention times from a
    separate pass (split_pass).  Returns the result dict and the (name, ms, bound, work, counters)
    entries of its two calls for the roofline."""
    from block_sparse_gqa_amd import msa
    wl, name = inp.wl, inp.wl.name
    per_step = np.array([e[0].elapsed_time(e[2]) for e in evs])
    t_all = float(per_step.mean())
    if evs[0][1] is not None:
        t_idx = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        t_att = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    else:
        t_idx, t_att = split
    alg = algorithmic(inp, dp, ids)
    kernels = []
    r = {"tokens": wl.total_q, "ms": t_all, "tokens_per_s": wl.total_q / (t_all * 1e-3),
         "ms_median": float(np.median(per_step)), "ms_min": float(per_step.min()),
         "index_topk_ms": t_idx, "sparse_attn_ms": t_att,
         "split_timing": "markers in the timed steps" if evs[0][1] is not None else "separate pass",
         "selected_tokens": alg["selected_tokens"], "workload": wl.description}
    if wl.is_decode:
        gbs_i = alg["index_bytes"] / (t_idx * 1e-3) / 1e9
        gbs_a = alg["attn_bytes"] / (t_att * 1e-3) / 1e9
        tot = (alg["index_bytes"] + alg["attn_bytes"]) / (t_all * 1e-3) / 1e9
        r.update({"bound": "hbm", "algorithmic_GB": (alg["index_bytes"] + alg["attn_bytes"]) / 1e9,
                  "GB_per_s": tot, "frac_hbm_peak": tot / HBM_PEAK_GBS,
                  "index_topk_GB_per_s": gbs_i, "sparse_attn_GB_per_s": gbs_a})
        kernels.append(("msa_index_topk[%s]" % name, t_idx, "hbm", alg["index_bytes"], None))
        kernels.append(("msa_sparse_attn_decode[%s]" % name, t_att, "hbm", alg["attn_bytes"], None))
    else:
        tf_i = alg["index_flops"] / (t_idx * 1e-3) / 1e12
        tf_a = alg["attn_flops"] / (t_att * 1e-3) / 1e12
        tot = (alg["index_flops"] + alg["attn_flops"]) / (t_all * 1e-3) / 1e12
        schedule = prefill_schedule_of(dp)
        r.update({"bound": "mfma", "algorithmic_TFLOP": (alg["index_flops"] + alg["attn_flops"]) / 1e12,
                  "TFLOP_per_s": tot, "frac_mfma_peak": tot / MFMA_BF16_PEAK_TFLOPS,
                  "index_topk_TFLOP_per_s": tf_i, "sparse_attn_TFLOP_per_s": tf_a,
                  "index_topk_frac_mfma_peak": tf_i / MFMA_BF16_PEAK_TFLOPS,
                  "sparse_attn_frac_mfma_peak": tf_a / MFMA_BF16_PEAK_TFLOPS,
                  "prefill_schedule": schedule})
        kernels.append(("msa_index_topk[%s]" % name, t_idx, "mfma", alg["index_flops"], None))
        # The call's kernels, for the HBM traffic the committed counters give (null unless they cover
        # every kernel of the call on this workload, measured on the current sources).
        kernels.append(("msa_sparse_attn_prefill[%s]" % name, t_att, "mfma", alg["attn_flops"],
                        (PREFILL_CALL_KERNELS[schedule], name)))
    return r, kernels


def time_extra(name, steps, warmup):
    """One of the other configurations, timed on its own: `warmup` untimed and `steps` timed passes of
    index_topk + attention, then (decode) flushed repetitions.  Frees its device memory before it
    returns; gives back the inputs and the GPU's ids (host) for the selection check."""
    import torch

    from block_sparse_gqa_amd import device, synth
    log(f"[bench] generating {name}")
    inp = synth.make_inputs(name)
    dp = device.upload(inp)
    ids = device.alloc_ids(dp)
    out, lse = device.alloc_out(dp)
    for _ in range(warmup):
        device.index_topk(dp, ids)
        device.sparse_attention(dp, ids, out, lse)
    torch.cuda.synchronize()
    evs = timed_events(steps)
    for e in evs:
        e[0].record()
        device.index_topk(dp, ids)
        device.sparse_attention(dp, ids, out, lse)
        e[2].record()
    torch.cuda.synchronize()
    split = split_pass(lambda: device.index_topk(dp, ids), lambda: device.sparse_attention(dp, ids, out, lse), steps)
    r, _ = summarize(inp, dp, ids, evs, split)
    if inp.wl.is_decode:
        r["flushed_reps"] = decode_reps(dp, (ids, out, lse))
        r["flushed_reps"]["GB_per_s_median"] = r["algorithmic_GB"] / (r["flushed_reps"]["ms_median"] * 1e-3)
    host_ids = ids.cpu().numpy()
    del dp, ids, out, lse
    torch.cuda.empty_cache()
    log(f"[bench] {name}: {r['ms']:.3f} ms")
    return r, inp, host_ids


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
    ap.add_argument("--no-forced", action="store_true",
                    help="skip timing the index branch with forced sink/local blocks (reported beside the headline)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-cache decode measurement (reported beside the headline, not in it)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip timing the other three configurations (reported beside the headline, not in it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--traffic-table", nargs="+", metavar="WORKLOAD:FETCH_DIR:WRITE_DIR",
                    help="no GPU work: write profiles/hbm_traffic.json from rocprofv3 FETCH_SIZE and WRITE_SIZE "
                         "passes of `--workloads WORKLOAD --calibrate-copy` runs, and print the table")
    args = ap.parse_args()
    if args.traffic_table:
        traffic_table(args.traffic_table)
        return
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
        for _ in range(CALIBRATION_COPIES):
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

    # Markers per step: one at each workload boundary (the end of one workload is the start of the
    # next), plus one between the index and the attention call of a prefill, whose attention call is
    # the roofline's kernel and is timed live.  Every marker idles the GPU for a few microseconds, so
    # a decode carries none between its calls; its split comes from a pass of its own afterwards.
    def step(events=None):
        for i, name in enumerate(names):
            dp = dps[name]
            ids, out, lse = bufs[name]
            if events is not None and i == 0:
                events[name][0].record()
            device.index_topk(dp, ids)
            if events is not None and events[name][1] is not None:
                events[name][1].record()
            device.sparse_attention(dp, ids, out, lse)
            if events is not None:
                events[name][2].record()

    def step_events():
        import torch
        b = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        return {n: [b[i], None if inputs[n].wl.is_decode else torch.cuda.Event(enable_timing=True), b[i + 1]]
                for i, n in enumerate(names)}

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    per_step_ev = [step_events() for _ in range(args.steps)]
    ev = {n: [e[n] for e in per_step_ev] for n in names}
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in per_step_ev:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    results, kernels = {}, []
    total_tokens = 0
    split = {}
    for name in names:
        if inputs[name].wl.is_decode:
            dp, (ids, out, lse) = dps[name], bufs[name]
            split[name] = split_pass(lambda: device.index_topk(dp, ids),
                                     lambda: device.sparse_attention(dp, ids, out, lse), args.steps)
    for name in names:
        r, ks = summarize(inputs[name], dps[name], bufs[name][0], ev[name], split.get(name))
        total_tokens += inputs[name].wl.total_q
        results[name] = r
        kernels.extend(ks)

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

    if not args.no_forced:
        for name in names:
            results[name]["forced"] = forced_index(dps[name], bufs[name][0], max(args.steps // 2, 3))

    if not args.no_paged:
        for name in names:
            if inputs[name].wl.is_decode:
                results[name]["paged"] = paged_decode(inputs[name], dps[name], bufs[name][0], results[name],
                                                      max(args.steps, 5), args.warmup)

    host_ids = {n: bufs[n][0].cpu().numpy() for n in names}
    extra_inputs = {}
    if not args.no_extra:
        for name in EXTRA_WORKLOADS:
            if name in names:
                continue
            results[name], extra_inputs[name], host_ids[name] = time_extra(name, args.steps, args.warmup)

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
    # a write-only stream: torch's fill of the same 4 GiB
    dst.fill_(1)
    ce[0].record()
    for _ in range(5):
        dst.fill_(1)
    ce[1].record()
    torch.cuda.synchronize()
    write_gbs = (1 << 32) * 5 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
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
        # the CPU leg: the oracle timed on a bounded sample of the step, and the GPU's ids of every
        # workload checked against the oracle's on sampled rows (near ties counted)
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(inputs)
        for name, rep in selection_parity({**inputs, **extra_inputs}, host_ids).items():
            results[name]["selection_parity"] = rep

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
                   **{n: results[n]["workload"] for n in names},
                   "also_reported": [n for n in results if n not in names]},
        "results": results,
        "roofline": roofline,
        "ceilings": {"hbm_copy_GB_per_s": copy_gbs, "hbm_stream_read_GB_per_s": read_gbs,
                     "hbm_fill_GB_per_s": write_gbs,
                     "mfma_bf16_TFLOP_per_s": mfma_tfs,
                     "note": "measured on this GPU: a device-to-device copy of 4 GiB (read + write bytes), a "
                             "fill of the same 4 GiB (write bytes), a full-line non-temporal read-only stream of "
                             "them, and back-to-back 16x16x32 bf16 MFMAs with no memory traffic"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

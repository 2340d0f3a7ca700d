"""Decode-step benchmark: paged GQA decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]

One step = the whole path for one attention layer of a decode step: cache
write of the batch's new tokens, partition pass and merge.  By default the
step is one library call, tv_paged_attention_decode_step; on the default
workload it is one launch (one workgroup per (sequence, K/V head): cache
write, attention over the whole context and the merge in one kernel).
``--step fused`` times the two-launch form (tv_paged_attention_decode_append,
cache write folded into the partition pass, then tv_paged_attention_reduce)
and ``--step separate`` the three-launch form (tv_cache_write,
tv_paged_attention_decode, tv_paged_attention_reduce); both are also
reported alongside.  The default workload is batch 64 with ragged contexts drawn from U[512, 4096]
(32 query heads, 8 K/V heads, head_dim 64, bf16, 16-token blocks, 512-token
partitions), built from a fixed seed.

Timing: W untimed warm-up steps, then K timed steps.  Before every timed step
a kernel reads 512 MiB of other memory, which evicts the L2 and the 256 MB
Infinity Cache, so the K/V bytes come from HBM ("cold" cache, the default).
The eviction reads rather than writes: a write leaves dirty lines whose
write-back would then be charged to the step.  The K (eviction, step) pairs run
back to back between two HIP events on the kernels' stream, and the same loop
with the eviction alone is timed and subtracted, so no event sits between the
kernels of a step.  Per-kernel times are taken the same way (eviction + that
kernel, minus eviction).  A back-to-back ("hot") figure and one with an event
around every kernel ("isolated") are reported beside it.  Prints one JSON line.

Throughput counts algorithmic bytes: K/V of every context token (2 x 8 heads x
64 x 2 B = 2048 B per token), q (4 KiB per sequence), the block-table entries
and context lengths read, the fp32 output (8 KiB per sequence) and the cache
write's 2 x 2 KiB per new token.  The partition workspace is implementation
overhead and is not counted.
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

METRIC = "paged GQA decode attention: achieved HBM GB/s (% of peak) and seq-tokens/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, 2.5 PFLOP/s
FLUSH_BYTES = 512 << 20
COPY_CALIBRATION_BYTES = 1 << 30
DECODE_SOURCE = os.path.join(ROOT, "paged_kv_cache_tv_amd", "csrc", "paged_decode.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "paged_decode_traffic.json")


def source_digest(path: str) -> str:
    """sha256 of a kernel source with comments and blank space removed, so that
    only a change of code (not of its comments) retires a measurement."""
    import hashlib
    import re
    with open(path, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode("utf-8")).hexdigest()


def measured_traffic(workload_name: str, kernel: str, path=None):
    """HBM bytes per launch of ``kernel`` from the committed counter record, or
    None when there is no record for this kernel and workload or the kernel
    source changed since."""
    try:
        with open(path or TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != source_digest(DECODE_SOURCE):
        return None
    if rec.get("kernel") != kernel:
        return None
    w = rec.get("workloads", {}).get(workload_name)
    return None if w is None else w.get("hbm_bytes_per_launch")


# rocprofv3 kernel-name fragments of the kernels a traffic record can cover,
# by the name bench.py reports in roofline.kernel.
TRAFFIC_KERNELS = {"paged_decode_seq_kernel<append>": "paged_decode_seq_kernel<true>",
                   "paged_decode_kernel<append>": "paged_decode_kernel<true, false, true"}


def _counter_rows(path, counter):
    """{rocprof kernel name: [counter value per dispatch]} from one
    --pmc pass's *_counter_collection.csv files under ``path``."""
    import csv
    import glob
    out = {}
    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def write_traffic_record(prof_dir, workload, partition_size, out_path=None):
    """Turn four rocprofv3 passes into TRAFFIC_RECORD: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) of the step's dominant kernel on
    ``workload``, each scaled by what the same counter reads for a plain 1 GiB
    device copy (``--copy-calibration``).  The passes, each its own run:

      rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -- python bench.py --steps 3
          --warmup 1 --no-cpu-baseline --no-prefill --no-block-copy --no-workloads
      rocprofv3 --pmc WRITE_SIZE ... -d DIR/write -- (the same bench command)
      rocprofv3 --pmc FETCH_SIZE ... -d DIR/copy_fetch -- python bench.py --copy-calibration
      rocprofv3 --pmc WRITE_SIZE ... -d DIR/copy_write -- python bench.py --copy-calibration
    """
    import statistics as st
    from paged_kv_cache_tv_amd import workloads as W
    batch = W.make_workload(workload)
    fetch = _counter_rows(os.path.join(prof_dir, "fetch"), "FETCH_SIZE")
    write = _counter_rows(os.path.join(prof_dir, "write"), "WRITE_SIZE")
    copy_f = _counter_rows(os.path.join(prof_dir, "copy_fetch"), "FETCH_SIZE")
    copy_w = _counter_rows(os.path.join(prof_dir, "copy_write"), "WRITE_SIZE")

    def copy_kib(rows):            # the 1 GiB copies are the largest dispatches
        vals = sorted(v for vs in rows.values() for v in vs)
        return st.median(vals[-5:])

    f1, w1 = copy_kib(copy_f), copy_kib(copy_w)
    fetch_scale = COPY_CALIBRATION_BYTES / 1024 / f1
    write_scale = COPY_CALIBRATION_BYTES / 1024 / w1
    for kernel, frag in TRAFFIC_KERNELS.items():
        names = [n for n in fetch if frag in n]
        if names:
            break
    else:
        raise ValueError("no decode kernel in the FETCH_SIZE pass")
    full = names[0]
    fv, wv = st.mean(fetch[full]), st.mean(write[full])
    rb, wb = int(fv * 1024 * fetch_scale), int(wv * 1024 * write_scale)
    dec_bytes, step_bytes, write_bytes = algorithmic_bytes(batch)
    algo = step_bytes if kernel == "paged_decode_seq_kernel<append>" else dec_bytes + write_bytes
    rec = {
        "kernel": kernel,
        "rocprof_kernel_name": full,
        "kernel_source": os.path.relpath(DECODE_SOURCE, ROOT),
        "kernel_source_sha256": source_digest(DECODE_SOURCE),
        "note": "HBM bytes per launch of the decode step's dominant kernel = FETCH_SIZE * "
                "fetch_scale + WRITE_SIZE * write_scale (KiB -> bytes); the scales come from a "
                "plain 1 GiB device copy under the same counters.  bench.py reports this as "
                "roofline.traffic only while the kernel source, comments and blank space "
                "removed, still has this hash (bench.source_digest).  Written by "
                "python bench.py --traffic-from DIR --workload N.",
        "copy_calibration": {"bytes": COPY_CALIBRATION_BYTES, "FETCH_SIZE_KiB": round(f1, 1),
                             "WRITE_SIZE_KiB": round(w1, 1), "fetch_scale": round(fetch_scale, 4),
                             "write_scale": round(write_scale, 4)},
        "workloads": {batch.name: {
            "partition_size": partition_size,
            "FETCH_SIZE_KiB_per_launch": round(fv, 1),
            "WRITE_SIZE_KiB_per_launch": round(wv, 1),
            "hbm_read_bytes_per_launch": rb,
            "hbm_write_bytes_per_launch": wb,
            "hbm_bytes_per_launch": rb + wb,
            "dispatches_averaged": len(fetch[full]),
            "algorithmic_bytes_per_launch": algo,
            "traffic_over_algorithmic": round((rb + wb) / algo, 4)}},
    }
    with open(out_path or TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def algorithmic_bytes(batch):
    """(partition-pass bytes, whole-step bytes, new-token write bytes) for one
    step of ``batch``."""
    S = batch.num_seqs
    lens = batch.context_lens.astype(np.int64)
    kv_row = 2 * batch.num_kv_heads * batch.head_dim * 2           # K+V bytes per token
    blocks = (lens + batch.block_size - 1) // batch.block_size
    decode = int(lens.sum()) * kv_row + S * batch.num_q_heads * batch.head_dim * 2 \
        + int(blocks.sum()) * 4 + S * 4
    reduce_out = S * batch.num_q_heads * batch.head_dim * 4
    live = int((batch.new_slots >= 0).sum())
    write = live * (2 * kv_row) + S * 8
    return decode, decode + reduce_out + write, write


def block_copy_rate(tv, dev, stream, flush, steps, sizes=(32, 64, 512, 2048)):
    """Copy-on-write copies on a pool of their own: for each count in `sizes`,
    that many blocks (all 8 K/V heads of 16 tokens x 64 dims in both pools,
    32 KiB per block) copied to fresh blocks, one launch per step.  Timed
    like the decode step: (eviction, launch) pairs back to back between two
    events on the kernel's stream, minus the eviction loop.  Up to 512 pairs
    the launch uses the 256-thread shape (a decode step's copies), above it
    the 128-thread one.  Bytes counted: each block read once and written
    once.  The top-level fields are those of the largest count."""
    import torch
    top = max(sizes)
    kc, vc = tv.new_pools(2 * top, 8, 64, 16, dev, fill=0)
    out = {}
    for pairs in sizes:
        pr = torch.stack([torch.arange(pairs), top + torch.arange(pairs)], 1).to(torch.int64).to(dev)
        tv.copy_blocks(kc, vc, pr, stream)
        ms = cold_loop_ms(stream, flush, lambda: tv.copy_blocks(kc, vc, pr, stream), steps)
        moved = pairs * 2 * (2 * 8 * 16 * 64 * 2)           # read + write, K and V pools
        gbs = moved / (ms * 1e-3) / 1e9
        out[pairs] = {"kernel": "block_copy_kernel<256, 4>" if pairs <= 512
                      else "block_copy_kernel<128, 8>",
                      "pairs": pairs, "bytes_per_launch": moved,
                      "us_per_launch": round(ms * 1e3, 2), "GB_per_s": round(gbs, 2),
                      "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del kc, vc
    res = dict(out[top])
    res["sizes"] = {str(p): {k: v for k, v in r.items() if k != "pairs"} for p, r in out.items()}
    return res


def block_manager_rate(tv, steps, prompts=64, samples=4, prefix=1024, seed=7):
    """Host cost of one decode step's bookkeeping: tv_bm_prepare_decode for a
    live batch shaped like the shared-prefix workload (64 prompts of 1024
    tokens, each forked into 4 samples with U{0..1024} private tokens).  Mean
    wall-clock microseconds per call over `steps` calls, each call growing all
    256 sequences by one token."""
    import numpy as np
    rng = np.random.default_rng(seed)
    bs, width = 16, 192
    S = prompts * samples
    bm = tv.BlockManager(prompts * prefix // bs + S * (1024 + steps + 16) // bs + 64, bs, S, width)
    for p in range(prompts):
        bm.add_sequence(samples * p, prefix)
        for j in range(1, samples):
            bm.fork(samples * p, samples * p + j)
    for s, r in enumerate(rng.integers(0, 1025, S)):
        for _ in range(int(r)):
            bm.append_slot(s)
    seqs = list(range(S))
    bm.prepare_decode(seqs, width)
    t0 = time.perf_counter()
    for _ in range(steps):
        bm.prepare_decode(seqs, width)
    us = (time.perf_counter() - t0) / steps * 1e6
    bm.close()
    return {"call": "tv_bm_prepare_decode", "seqs": S, "width": width,
            "host_us_per_step": round(us, 2)}


def prefill_rate(tv, dev, stream, flush, steps, index=3):
    """Prefill attention (tv_paged_attention_prefill) on the prefill workload
    `index` (default: 8 prompts of 2048 tokens, full prefill).  The prompts'
    K/V are written into fresh pools with tv_cache_write first; each timed
    launch follows a cache eviction and is bracketed by its own pair of
    events; the figure is the median launch (mean, min and max beside it).
    FLOPs counted: 2 x 2 x head_dim per (query head, query, key)
    pair the causal mask keeps (QK^T and PV)."""
    import numpy as np
    import torch
    from paged_kv_cache_tv_amd import workloads as W
    pb = W.make_prefill_workload(index)
    b = pb.base

    def dev_arr(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev,
                          fill=W.BF16_NAN)
    for k, v, sl in (pb.prior_inputs(), pb.chunk_inputs()):
        if len(sl):
            tv.cache_write(dev_arr(k), dev_arr(v), kc, vc, dev_arr(sl), stream)
    q, qs = dev_arr(pb.q), dev_arr(pb.query_start)
    bt, cl = dev_arr(b.block_tables), dev_arr(b.context_lens)
    out = torch.empty((pb.num_rows, b.num_q_heads, b.head_dim), dtype=torch.float32, device=dev)
    mq, mc = pb.max_query_len, int(b.context_lens.max())

    def launch():
        tv.paged_attention_prefill(out, q, qs, kc, vc, bt, cl, mq, mc, b.scale, stream)

    launch()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(ev):
        flush(i)
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    each = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    ms = float(np.median(each))
    flops = pb.causal_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    finite = bool(torch.isfinite(out).all().item())
    del kc, vc, out
    return {"workload": pb.name, "kernel": "paged_prefill_kernel<4, 1>", "rows": pb.num_rows,
            "flops_per_launch": flops, "us_per_launch": round(ms * 1e3, 2),
            "us_per_launch_stats": {"median": round(ms * 1e3, 2),
                                    "mean": round(float(each.mean()) * 1e3, 2),
                                    "min": round(float(each.min()) * 1e3, 2),
                                    "max": round(float(each.max()) * 1e3, 2),
                                    "launches": int(len(each))},
            "TFLOP_per_s": round(tflops, 1), "output_finite": finite,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}


def rope_rate(tv, dev, stream, flush, steps, index=3):
    """Rotary embedding on the prefill workload `index` (8 prompts x 2048
    tokens): the K/V cache write of all prompt tokens plain (tv_cache_write)
    and with K rotated (tv_cache_write_rope), and q rotated in place
    (tv_rope).  Each launch follows a cache eviction; timed like the decode
    step (eviction + launch loop between two events, minus the eviction loop).
    Bytes counted: K and V read and written (cache writes), q read and
    written (tv_rope), plus slots and positions."""
    import numpy as np
    import torch
    from paged_kv_cache_tv_amd import workloads as W
    pb = W.make_prefill_workload(index)
    b = pb.base

    def dev_arr(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    k, v, sl = pb.chunk_inputs()
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in pb.query_lens])
    kd, vd, sd, pd = dev_arr(k), dev_arr(v), dev_arr(sl), dev_arr(pos)
    qd = dev_arr(pb.q)
    f = dev_arr(W.rope_inv_freq(b.head_dim, 500000.0))
    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev, fill=0)
    T = int(len(sl))
    kv_bytes = 2 * 2 * T * b.num_kv_heads * b.head_dim * 2 + T * 8
    q_bytes = 2 * pb.num_rows * b.num_q_heads * b.head_dim * 2 + pb.num_rows * 4
    cases = {
        "cache_write": (lambda: tv.cache_write(kd, vd, kc, vc, sd, stream), kv_bytes),
        "cache_write_rope": (lambda: tv.cache_write_rope(kd, vd, kc, vc, sd, pd, f, 0, stream),
                             kv_bytes + T * 4),
        "rope_q": (lambda: tv.rope(qd, pd, f, 0, stream), q_bytes),
    }
    res = {"workload": pb.name, "tokens": T}
    for name, (fn, nbytes) in cases.items():
        fn()
        ms = cold_loop_ms(stream, flush, fn, steps)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"bytes_per_launch": nbytes, "us_per_launch": round(ms * 1e3, 2),
                     "GB_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del kc, vc
    return res


def shared_prefix_rate(tv, dev, stream, flush, steps):
    """The partition pass on the shared-prefix workload (64 prompts x 4
    samples, 1024 shared tokens): per sequence (tv_paged_attention_decode)
    against groups of 4 (tv_paged_attention_decode_shared), and the whole
    two-launch step each way (tv_paged_attention_decode_append or
    tv_paged_attention_decode_shared_append, then the merge); cold, timed
    like the decode step.  Bytes: the K/V each path must read at least -- logical
    (every sequence's context) and unique (shared blocks once).  `shared_step`
    is the step through the one call (tv_paged_attention_decode_shared_step),
    `shared_two_launch_step` the shared append and the merge."""
    import torch
    from paged_kv_cache_tv_amd import workloads as W
    from paged_kv_cache_tv_amd.step import DeviceBatch
    b = W.make_workload(4)
    db = DeviceBatch(b, dev)
    db.fill()
    shared = torch.full((b.num_seqs // 4,), 1024, dtype=torch.int32, device=dev)
    pa, pm, ps = db.workspace

    def plain():
        tv.paged_attention_decode(pa, pm, ps, db.q, db.k_cache, db.v_cache, db.block_tables,
                                  db.context_lens, db.max_context_len, db.partition_size,
                                  b.scale, stream)

    def grouped():
        tv.paged_attention_decode_shared(pa, pm, ps, db.q, db.k_cache, db.v_cache,
                                         db.block_tables, db.context_lens, shared, 4,
                                         db.max_context_len, db.partition_size, b.scale, stream)

    def grouped_step():
        # The parallel-sampling decode step in two launches: the new tokens'
        # cache write folded into the shared pass, then the merge.
        tv.paged_attention_decode_shared_append(pa, pm, ps, db.q, db.step_k, db.step_v,
                                                db.step_slots, db.k_cache, db.v_cache,
                                                db.block_tables, db.context_lens, shared, 4,
                                                db.max_context_len, db.partition_size, b.scale,
                                                stream)
        db.reduce(stream)

    def plain_step():
        db.fused_step(stream)

    out = torch.empty_like(db.out)

    def one_call_step():
        # The same step through tv_paged_attention_decode_shared_step.
        tv.paged_attention_decode_shared_step(out, db.workspace, db.q, db.step_k, db.step_v,
                                              db.step_slots, db.k_cache, db.v_cache,
                                              db.block_tables, db.context_lens, shared, 4,
                                              db.max_context_len, db.partition_size, b.scale,
                                              stream)

    form = tv.decode_shared_step_form(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                      b.block_size, db.max_context_len, db.partition_size, 4)
    res = {"workload": b.name, "group_size": 4, "shared_tokens": 1024,
           "kv_bytes_logical": b.kv_bytes_logical(), "kv_bytes_unique": b.kv_bytes_unique(),
           "shared_step": "one call, tv_paged_attention_decode_shared_step: " +
                          {1: "one launch, one workgroup per (group, K/V head)",
                           2: "two launches through the workspace"}.get(form, str(form))}
    for name, fn in (("per_sequence", plain), ("shared", grouped),
                     ("per_sequence_step", plain_step), ("shared_two_launch_step", grouped_step),
                     ("shared_step", one_call_step)):
        fn()
        res[name + "_us"] = round(cold_loop_ms(stream, flush, fn, steps) * 1e3, 2)
    res["unique_GB_per_s_shared"] = round(b.kv_bytes_unique() / (res["shared_us"] * 1e-6) / 1e9, 1)
    res["unique_GB_per_s_shared_step"] = round(
        b.kv_bytes_unique() / (res["shared_step_us"] * 1e-6) / 1e9, 1)
    del db
    return res


def cold_loop_ms(stream, flush, body, k):
    """Mean ms per iteration of (eviction, body), minus the eviction alone: k
    iterations back to back between two events on the kernels' stream."""
    import torch

    def loop(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(k):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    with_body = loop(lambda i: (flush(i), body()))
    return with_body - loop(flush)


def workloads_rate(tv, dev, stream, flush, steps, warmup, partition_size, have=None):
    """The decode step on every one of the five workloads, cold, timed as the
    headline step is (eviction-subtracted event loop): the two-launch step
    (decode_append + reduce) and the one-call step (tv_paged_attention_decode_step:
    the form tv_paged_attention_decode_step_form reports).  Workload 4 also
    runs its parallel-sampling form (shared prefix read once per group of 4):
    tv_paged_attention_decode_shared_append + reduce, and the one call
    tv_paged_attention_decode_shared_step.  GB/s counts the same
    algorithmic bytes as the headline; for workload 4 both the logical bytes
    (every sequence's context) and the unique ones (each shared block once).
    `have` maps a workload index to an already built (batch, DeviceBatch)."""
    import torch
    from paged_kv_cache_tv_amd import workloads as W
    from paged_kv_cache_tv_amd.step import DeviceBatch
    res = {}
    for idx in (1, 2, 3, 4, 5):
        if have and idx in have:
            batch, db = have[idx]
        else:
            batch = W.make_workload(idx)
            db = DeviceBatch(batch, dev, partition_size=partition_size)
            db.fill()
        forms = {"two_launch": lambda: db.fused_step(stream),
                 "one_call": lambda: db.call_step(stream)}
        shared = None
        if idx == 4:
            shared = torch.full((batch.num_seqs // 4,), 1024, dtype=torch.int32, device=dev)
            pa, pm, ps = db.workspace

            def grouped_step():
                tv.paged_attention_decode_shared_append(
                    pa, pm, ps, db.q, db.step_k, db.step_v, db.step_slots, db.k_cache,
                    db.v_cache, db.block_tables, db.context_lens, shared, 4, db.max_context_len,
                    db.partition_size, batch.scale, stream)
                db.reduce(stream)
            forms["shared_prefix_two_launch"] = grouped_step
            sh_out = torch.empty_like(db.out)

            def grouped_call():
                tv.paged_attention_decode_shared_step(
                    sh_out, db.workspace, db.q, db.step_k, db.step_v, db.step_slots, db.k_cache,
                    db.v_cache, db.block_tables, db.context_lens, shared, 4, db.max_context_len,
                    db.partition_size, batch.scale, stream)
            forms["shared_prefix_one_call"] = grouped_call
        for fn in forms.values():
            for i in range(max(1, warmup)):
                flush(i)
                fn()
        _, step_bytes, _ = algorithmic_bytes(batch)
        entry = {"num_seqs": batch.num_seqs, "context_tokens": batch.total_tokens,
                 "context_len_range": [int(batch.context_lens.min()),
                                       int(batch.context_lens.max())],
                 "partitions": int(-(-db.max_context_len // db.partition_size)),
                 "step_bytes": step_bytes}
        for name, fn in forms.items():
            ms = cold_loop_ms(stream, flush, fn, steps)
            e = {"step_us": round(ms * 1e3, 2),
                 "GB_per_s": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                 "pct_of_hbm_peak": round(100.0 * step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "seq_tokens_per_s": round(batch.total_tokens / (ms * 1e-3), 1),
                 "decode_tokens_per_s": round(batch.num_seqs / (ms * 1e-3), 1)}
            if idx == 4:
                unique = step_bytes - batch.kv_bytes_logical() + batch.kv_bytes_unique()
                e["GB_per_s_unique"] = round(unique / (ms * 1e-3) / 1e9, 1)
                e["pct_of_hbm_peak_unique"] = round(
                    100.0 * unique / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
            entry[name] = e
        if idx == 4:
            entry["step_bytes_unique"] = (step_bytes - batch.kv_bytes_logical()
                                          + batch.kv_bytes_unique())
        res[batch.name] = entry
        if not (have and idx in have):
            del db
        torch.cuda.synchronize()
    return res


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, target_seconds: float, single_runs: int = 3):
    """Time the CPU oracle doing the same step (cache write + attention) on this
    host: repeated for about `target_seconds` with every core this process may
    use, then `single_runs` times on one thread.  Returns (output, multi-thread
    times, threads, single-thread times)."""
    import oracle as O
    orc = O.default()
    threads = O.cpu_count()
    kc, vc = O.build_pools(orc, batch, include_step=False)
    sk, sv, ss = batch.step_inputs()

    def one(nthreads):
        t0 = time.perf_counter()
        orc.cache_write(sk, sv, kc, vc, ss)
        o = orc.paged_attention(batch.q, kc, vc, batch.block_tables, batch.context_lens,
                                batch.scale, nthreads)
        return o, time.perf_counter() - t0

    times, out = [], None
    t_start = time.perf_counter()
    while True:
        out, t = one(threads)
        times.append(t)
        if time.perf_counter() - t_start >= target_seconds and len(times) >= 1:
            break
    single = [one(1)[1] for _ in range(single_runs)]
    return out, times, threads, single


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--partition-size", type=int, default=512)
    ap.add_argument("--step", choices=["call", "fused", "separate"], default="call",
                    help="one library call (tv_paged_attention_decode_step), two launches "
                         "(write folded into the partition pass) or three")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill attention measurement")
    ap.add_argument("--no-block-copy", action="store_true",
                    help="skip the copy-on-write block copy measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the step on all five workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-flush", action="store_true", help="skip the cold-cache flush")
    ap.add_argument("--lib", default=None, help="load libtv from this path instead of the package")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain device-to-device copies of 1 GiB (counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR", default=None,
                    help="write the traffic record from rocprofv3 FETCH_SIZE / WRITE_SIZE passes "
                         "under DIR (fetch/, write/, copy_fetch/, copy_write/) and exit")
    args = ap.parse_args(argv)

    if args.traffic_from:
        rec = write_traffic_record(args.traffic_from, args.workload, args.partition_size)
        print(json.dumps(rec), flush=True)
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the decode step is "
                                   "measured on one GPU's share and nothing here spans GPUs",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import torch
    import paged_kv_cache_tv_amd as tv
    from paged_kv_cache_tv_amd import workloads as W
    from paged_kv_cache_tv_amd.step import DeviceBatch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 1
    if args.lib:
        from paged_kv_cache_tv_amd import binding
        binding._lib = binding.load_library(args.lib)
    tv.lib()                                   # loud failure if libtv.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_CALIBRATION_BYTES, "copies": 5}), flush=True)
        return 0

    t0 = time.perf_counter()
    batch = W.make_workload(args.workload)
    db = DeviceBatch(batch, dev, partition_size=args.partition_size)
    db.fill()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    print(f"# workload {batch.name}: {batch.num_seqs} seqs, {batch.total_tokens} context tokens, "
          f"setup {setup_s:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    flush_buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush(i):
        if not args.no_flush:
            flush_buf.sum()

    form = tv.decode_step_form(batch.num_seqs, batch.num_q_heads, batch.num_kv_heads,
                               batch.head_dim, batch.block_size, db.max_context_len,
                               db.partition_size)
    steps = {"call": lambda: db.call_step(stream),
             "fused": lambda: db.fused_step(stream),
             "separate": lambda: db.step(stream)}
    run_step = steps[args.step]
    for i in range(args.warmup):
        for f in steps.values():
            flush(i)
            f()
    torch.cuda.synchronize()

    def timed_loop(body, k):
        """Mean ms per iteration of `body`, run k times back to back between two
        events recorded on the kernels' stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(k):
            body(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    K = args.steps
    # The timed region: K steps, each preceded by the cache eviction.  The
    # eviction's own time (measured alone, same loop shape) is subtracted.
    wall0 = time.perf_counter()
    t_flush_step = timed_loop(lambda i: (flush(i), run_step()), K)
    wall = time.perf_counter() - wall0
    t_flush = timed_loop(flush, K)
    t_flush_forms = {name: timed_loop(lambda i, f=f: (flush(i), f()), K)
                     for name, f in steps.items()}
    t_flush_write = timed_loop(lambda i: (flush(i), db.write_step(stream)), K)
    t_flush_decode = timed_loop(lambda i: (flush(i), db.decode(stream)), K)
    # The same partition pass with its contractions on the vector ALUs
    # (tv_paged_attention_decode_vector, 4 query heads per K/V head only).
    vector_ok = batch.num_q_heads == 4 * batch.num_kv_heads

    def vector_pass():
        pa, pm, ps = db.workspace
        tv.paged_attention_decode_vector(pa, pm, ps, db.q, db.k_cache, db.v_cache,
                                         db.block_tables, db.context_lens, db.max_context_len,
                                         db.partition_size, batch.scale, stream)
    if vector_ok:
        for i in range(args.warmup):
            vector_pass()
    t_flush_vector = (timed_loop(lambda i: (flush(i), vector_pass()), K) if vector_ok
                      else float("nan"))
    t_flush_append = timed_loop(lambda i: (flush(i), db.decode_append(stream)), K)
    t_flush_reduce = timed_loop(lambda i: (flush(i), db.reduce(stream)), K)
    if args.no_flush:
        t_flush = 0.0
    step_ms_cold = t_flush_step - t_flush
    forms_ms = {name: t - t_flush for name, t in t_flush_forms.items()}
    decode_ms = t_flush_decode - t_flush
    vector_ms = t_flush_vector - t_flush
    append_ms = t_flush_append - t_flush
    write_ms = t_flush_write - t_flush
    reduce_ms = t_flush_reduce - t_flush
    call_ms = forms_ms["call"]

    # Hot cache: the same steps back to back with no eviction in between.
    hot_steps = max(10, K)
    hot_ms = timed_loop(lambda i: run_step(), hot_steps)
    hot_decode_ms = timed_loop(lambda i: (db.decode(stream) if args.step == "separate"
                                          else db.decode_append(stream)), hot_steps)

    # Isolated launches: events around every kernel of every step (adds the
    # event/dispatch latency of each boundary; reported for reference).  The
    # one call is bracketed whole.
    kernels = {"call": [db.call_step], "fused": [db.decode_append, db.reduce],
               "separate": [db.write_step, db.decode, db.reduce]}[args.step]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
          for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        flush(i)
        e = ev[i]
        e[0].record(stream)
        for j, kern in enumerate(kernels):
            kern(stream)
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    main = 1 if args.step == "separate" else 0   # the partition pass among the launches
    iso_step = np.array([e[0].elapsed_time(e[-1]) for e in ev])
    iso_decode = np.array([e[main].elapsed_time(e[main + 1]) for e in ev])

    # The output of a final step in the timed form, checked against the oracle below.
    run_step()
    torch.cuda.synchronize()
    out = db.out.cpu().numpy()
    dec_bytes, step_bytes, write_bytes = algorithmic_bytes(batch)
    ms = float(step_ms_cold)
    value = step_bytes / (ms * 1e-3) / 1e9
    # The dominant kernel of the timed step, with the algorithmic bytes it
    # moves per launch.
    if args.step == "call" and form == 2:
        roof_kernel, roof_bytes, roof_ms = "paged_decode_seq_kernel<append>", step_bytes, ms
    elif args.step == "call" and form == 1:
        roof_kernel, roof_bytes, roof_ms = "paged_decode_kernel<append>", step_bytes, ms
    elif args.step == "separate":
        roof_kernel, roof_bytes, roof_ms = "paged_decode_kernel", dec_bytes, decode_ms
    else:
        roof_kernel, roof_bytes, roof_ms = "paged_decode_kernel<append>", dec_bytes + write_bytes, append_ms
    roof_gbs = roof_bytes / (roof_ms * 1e-3) / 1e9

    # The plain-read yardstick: tv_stream_read over as many bytes as the
    # kernel above moves per launch, timed the same way (eviction + kernel
    # loop minus the eviction loop).
    sr_bytes = -(-roof_bytes // 16) * 16
    sr_buf = torch.zeros(sr_bytes // 4, dtype=torch.int32, device=dev)
    sr_out = torch.empty(-(-sr_bytes // tv.STREAM_CHUNK_BYTES), dtype=torch.int32, device=dev)
    for i in range(max(1, args.warmup)):
        flush(i)
        tv.stream_read(sr_buf, sr_out, stream)
    sr_ms = timed_loop(lambda i: (flush(i), tv.stream_read(sr_buf, sr_out, stream)), K) - t_flush
    sr_gbs = sr_bytes / (sr_ms * 1e-3) / 1e9
    del sr_buf, sr_out

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": batch.name,
            "num_seqs": batch.num_seqs,
            "context_tokens": batch.total_tokens,
            "context_len_range": [int(batch.context_lens.min()), int(batch.context_lens.max())],
            "num_q_heads": batch.num_q_heads, "num_kv_heads": batch.num_kv_heads,
            "head_dim": batch.head_dim, "block_size": batch.block_size,
            "partition_size": args.partition_size,
            "cache": "hot" if args.no_flush else "cold",
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(batch.total_tokens / (ms * 1e-3), 1),
        "decode_tokens_per_s": round(batch.num_seqs / (ms * 1e-3), 1),
        "step_bytes": step_bytes,
        "step": {"call": "one call, tv_paged_attention_decode_step: "
                         + tv.DECODE_STEP_FORMS.get(form, str(form)),
                 "fused": "two launches: decode_append + reduce",
                 "separate": "three launches: cache_write + decode + reduce"}[args.step],
        "steps_us": {"one_call": round(forms_ms["call"] * 1e3, 2),
                     "two_launch": round(forms_ms["fused"] * 1e3, 2),
                     "three_launch": round(forms_ms["separate"] * 1e3, 2)},
        "kernels_us": {"cache_write": round(write_ms * 1e3, 2),
                       "paged_decode": round(decode_ms * 1e3, 2),
                       "paged_decode_append": round(append_ms * 1e3, 2),
                       "paged_reduce": round(reduce_ms * 1e3, 2)},
        "vector_path": ({
            "what": "the plain partition pass (no cache write) with its QK and PV "
                    "contractions on the vector ALUs, against the same pass on MFMA; "
                    "cold cache, same timing method",
            "kernel": "paged_decode_vec_kernel", "us": round(vector_ms * 1e3, 2),
            "GB_per_s": round(dec_bytes / (vector_ms * 1e-3) / 1e9, 2),
            "matrix_kernel": "paged_decode_kernel", "matrix_us": round(decode_ms * 1e3, 2),
            "matrix_GB_per_s": round(dec_bytes / (decode_ms * 1e-3) / 1e9, 2),
            "vector_over_matrix_time": round(vector_ms / decode_ms, 3)}
            if vector_ok else None),
        "eviction_us": round(t_flush * 1e3, 2),
        "hot_cache": {"ms_per_step": round(hot_ms, 5),
                      "GB_per_s": round(step_bytes / (hot_ms * 1e-3) / 1e9, 2),
                      "paged_decode_us": round(hot_decode_ms * 1e3, 2)},
        "isolated_launch_us": {"step_median": round(float(np.median(iso_step)) * 1e3, 2),
                               "paged_decode_median": round(float(np.median(iso_decode)) * 1e3, 2)},
        "wall_ms_per_step_incl_eviction": round(wall / args.steps * 1e3, 4),
        "roofline": {"bound": "hbm", "kernel": roof_kernel,
                     "achieved": round(roof_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(batch.name, roof_kernel),
                     "algorithmic_bytes_per_launch": roof_bytes,
                     "avg_launch_us": round(roof_ms * 1e3, 2),
                     "frac_of_stream_read": round(roof_gbs / sr_gbs, 4)},
        "stream_read": {"kernel": "stream_read_kernel", "bytes_per_launch": sr_bytes,
                        "us_per_launch": round(sr_ms * 1e3, 2), "GB_per_s": round(sr_gbs, 2),
                        "frac_of_hbm_peak": round(sr_gbs / HBM_PEAK_GBS, 4),
                        "what": "one plain coalesced read of the same byte count as the "
                                "roofline kernel, cold cache, same timing method"},
    }

    if not args.no_workloads:
        result["workloads"] = workloads_rate(tv, dev, stream, flush, K, args.warmup,
                                             args.partition_size, {args.workload: (batch, db)})
    if not args.no_block_copy:
        result["block_copy"] = block_copy_rate(tv, dev, stream, flush, K)
        result["block_manager"] = block_manager_rate(tv, K)
    if not args.no_prefill:
        result["prefill"] = prefill_rate(tv, dev, stream, flush, K)
        # The other prefill workloads (3 short prompts; chunked prefill of 8
        # sequences), whose grids take the two-key-share form.
        result["prefill"]["workloads"] = {
            r["workload"]: {k: r[k] for k in ("rows", "flops_per_launch", "us_per_launch",
                                              "TFLOP_per_s", "output_finite")}
            for r in (prefill_rate(tv, dev, stream, flush, K, index=i) for i in (1, 2))}
        result["rope"] = rope_rate(tv, dev, stream, flush, K)
        result["shared_prefix"] = shared_prefix_rate(tv, dev, stream, flush, K)

    if not args.no_cpu_baseline:
        ref, times, threads, single = cpu_baseline(batch, args.cpu_seconds)
        t = float(np.median(times))
        t1 = float(np.median(single))
        result["cpu_baseline"] = {
            "value": round(step_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "cpu_model": cpu_model(),
            "median_step_s": round(t, 4),
            "single_thread": {"value": round(step_bytes / t1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "median_step_s": round(t1, 4), "runs": len(single)},
            "sample": f"the full step of {batch.name} (cache write of {batch.num_seqs} tokens + "
                      f"attention over {batch.total_tokens} context tokens; the oracle computes "
                      f"in fp64), repeated {len(times)}x for {sum(times):.1f}s on {threads} "
                      f"threads (median step {t:.3f}s), then {len(single)}x on one thread "
                      f"(median {t1:.3f}s)",
        }
        err = np.abs(out.astype(np.float64) - ref)
        result["parity"] = {"max_abs": float(err.max()), "mean_abs": float(err.mean())}

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

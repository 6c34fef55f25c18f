"""Benchmark of the paged-attention hot path on one MI355X.

Prints ONE JSON line. The timed step is the batched split-KV GQA decode
workload (config3: B=64, L ~ U[1024, 32768], 32 q / 8 kv heads, D=128, page 64,
40000-page pool, 4096-token chunks): build the strided page table, run the
split-KV decode, merge the partial states. ``value`` is that step's
algorithmic HBM bytes (K + V rows read, q, the bf16 output, the page table)
divided by the measured step time. The prefill (config2), sliding-window
decode (config4) and sparse MLA decode (config5) workloads are timed in the
same run and reported beside it; the CPU oracle is timed on a bounded sample.

Inputs are seeded synthetic tensors already resident in HBM when timing starts.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz, dense bf16
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM traffic per workload from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (written by
# `bench.py --hbm-summary`), valid for the kernel sources whose hash it records
HBM_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# sources of each workload's kernels (their hash keys the stored traffic)
WORKLOAD_SOURCES = {
    "decode": ["decode.hip", "splits.hpp", "page_table.hip", "common.hpp", "args.hpp"],
    "decode_split": ["decode.hip", "splits.hpp", "merge_state.hip", "page_table.hip",
                     "common.hpp", "args.hpp"],
    "decode_merged": ["decode.hip", "splits.hpp", "page_table.hip", "common.hpp", "args.hpp"],
    "decode_window": ["decode.hip", "splits.hpp", "page_table.hip", "common.hpp", "args.hpp"],
    "swa": ["decode.hip", "splits.hpp", "page_table.hip", "common.hpp", "args.hpp"],
    "sparse": ["sparse_mla.hip", "common.hpp", "lanes.hpp", "lds_dma.hpp", "args.hpp"],
    "cascade": ["cascade.hip", "draft_prefix.hip", "splits.hpp", "common.hpp", "lanes.hpp",
                "args.hpp"],
    "dca": ["dca.hip", "decode.hip", "splits.hpp", "merge_state.hip", "common.hpp", "args.hpp"],
}
COPY_BYTES = 1 << 30   # run_copy: bytes read and bytes written by the copy kernel


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", choices=["all", "decode", "decode_split", "decode_merged", "decode_window",
                                      "prefill",
                                      "prefill_long", "prefill_window", "prefill_append", "swa",
                                      "sparse", "cascade", "dca", "copy"],
                   default="all", help="restrict to one workload (for profiler runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--hbm-summary", metavar="DIR", default=None,
                   help="reduce the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR to the "
                        "per-workload traffic summary (JSON on stdout); needs no GPU")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU work budget for the oracle sample")
    return p.parse_args(argv)


def device_clock_mhz():
    """Peak shader clock the runtime reports for device 0 (MHz), or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate (= 5, kHz), device 0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) != 0 or v.value <= 0:
            return None
        return v.value / 1000.0
    except OSError:
        return None


def code_text(src):
    """C/C++ source without its comments, whitespace runs collapsed: the part of a
    file that decides the compiled kernel (string and character literals kept)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(*names):
    """Hash of the code (comments and layout excluded) of the named csrc files."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_197_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


class Timer:
    """Wall-clock step timing plus per-launch HIP-event timing of one kernel."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.torch.cuda.current_stream())
        return e

    def kernel_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(len(self.pairs), 1)

    def kernel_ms_median(self):
        t = sorted(a.elapsed_time(b) for a, b in self.pairs)
        if not t:
            return 0.0
        n = len(t)
        return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])


def kernel_median(torch, step, launches=50, warmup=10):
    """Median HIP-event duration of the event-bracketed kernel over `launches`
    launches after `warmup` untimed steps (steps enqueued back to back)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    timer = Timer(torch)
    for _ in range(launches):
        step(timer)
    torch.cuda.synchronize()
    return timer.kernel_ms_median(), len(timer.pairs)


def timed_loop(torch, step, steps, warmup):
    """W untimed steps, then exactly K timed steps between synchronisations.

    step(timer_or_None) enqueues one step; with a timer it records events
    around the dominant kernel. Returns (wall-clock ms per step, mean kernel ms).
    """
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, timer.kernel_ms()


def device_loop(torch, step, steps, warmup, host_us_per_step=60.0):
    """Device-side timing for short kernels, free of host launch gaps.

    The GPU is first parked on a sleep kernel long enough for the host to
    enqueue all `steps` steps, so consecutive launches run back to back.
    Returns (device ms per step, mean kernel ms of the event-bracketed kernel).
    """
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    timer = Timer(torch)
    cycles = int(steps * host_us_per_step * 1e-6 * 2.4e9) + 1_000_000
    torch.cuda._sleep(cycles)
    start = timer.mark()
    for _ in range(steps):
        step(timer)
    end = timer.mark()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, timer.kernel_ms()


# ---------------------------------------------------------------------------
# Algorithmic work
# ---------------------------------------------------------------------------

def decode_bytes(seq_lens, batch, hq, hkv, d, page_size, elem=2):
    """K and V rows of every visible token, q, the output, and the page-table reads."""
    sum_l = int(seq_lens.sum())
    n_pages = int(((seq_lens + page_size - 1) // page_size).sum())
    kv = 2 * sum_l * hkv * d * elem
    return kv + batch * hq * d * elem * 2 + 4 * n_pages, sum_l


def prefill_flops(extend_lens, kv_lens, hq, d, window_left=-1):
    """4 * D * Hq * (visible (q, k) pairs), causal bottom-right; a sliding
    window (W, 0) keeps at most W + 1 keys per row."""
    pairs = 0
    for m, L in zip(extend_lens, kv_lens):
        m, L = int(m), int(L)
        cap = window_left + 1 if window_left >= 0 else None
        pairs += sum(L - m + j + 1 if cap is None else min(L - m + j + 1, cap) for j in range(m))
    return 4 * d * hq * pairs, pairs


def window_decode_bytes(seq_lens, window_left, batch, hq, hkv, d, page_size, elem=2):
    """decode_bytes over the last min(L, W + 1) keys of each request (and the
    pages holding them)."""
    kv_keys, pages = 0, 0
    for L in seq_lens.tolist():
        lo = max(L - 1 - window_left, 0)
        kv_keys += L - lo
        pages += (L + page_size - 1) // page_size - lo // page_size
    kv = 2 * kv_keys * hkv * d * elem
    return kv + batch * hq * d * elem * 2 + 4 * pages, kv_keys


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def run_decode(torch, pkv, workloads, args, window_left=-1, kv_chunk=None, mode="split"):
    """config3's step. mode "merged": the split-KV decode with the merge of its
    splits in the same launch (bit-identical to "split"); "split": the decode,
    then merge_state (two launches); "balanced": merged over balanced ranges."""
    dev = torch.device("cuda:0")
    c = workloads.config3(value_device=dev)
    r2t, rpi, sl = (c.req_to_token.to(dev), c.req_pool_indices.to(dev), c.seq_lens.to(dev))
    B, hq, d = c.q.shape
    _, P, hkv, _ = c.k_cache.shape
    chunk = kv_chunk or c.kv_chunk
    S = -(-int(c.seq_lens.max()) // chunk)
    pt = torch.empty((B, c.table_width), dtype=torch.int32, device=dev)
    kl = torch.empty((B,), dtype=torch.int32, device=dev)
    op = torch.empty((S, B, hq, d), dtype=torch.float32, device=dev)
    lp = torch.empty((S, B, hq), dtype=torch.float32, device=dev)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    merged = mode in ("merged", "balanced")
    ws = (torch.zeros(pkv.paged_attn_decode_merged_workspace_size(
        B, hq, d, S if mode == "merged" else 0), dtype=torch.uint8, device=dev) if merged else None)

    def step(timer):
        pkv.build_page_table(r2t, rpi, sl, P, c.table_width, page_table=pt, kv_lens=kl,
                             with_cu_seqlens=False)
        e0 = timer.mark() if timer else None
        if merged:   # decode and merge in one launch
            pkv.paged_attn_decode_merged(c.q, c.k_cache, c.v_cache, pt, kl, c.scale,
                                         kv_chunk=chunk if mode == "merged" else 0,
                                         num_splits=S if mode == "merged" else 0,
                                         window_left=window_left, workspace=ws, out=out, lse=lse)
            if timer:
                timer.pairs.append((e0, timer.mark()))
            return
        pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale,
                                      kv_chunk=chunk, num_splits=S, window_left=window_left,
                                      o_partial=op, lse_partial=lp)
        if timer:
            timer.pairs.append((e0, timer.mark()))
        pkv.merge_state(op, lp, out=out, lse_out=lse)

    if window_left >= 0:
        ms, kern_ms = device_loop(torch, step, args.steps, args.warmup, host_us_per_step=80.0)
        nbytes, sum_l = window_decode_bytes(c.seq_lens.long(), window_left, B, hq, hkv, d, P)
    else:
        ms, kern_ms = timed_loop(torch, step, args.steps, args.warmup)
        nbytes, sum_l = decode_bytes(c.seq_lens.long(), B, hq, hkv, d, P)
    med_ms, n_med = kernel_median(torch, step)
    res = dict(ms=ms, kernel_ms=kern_ms, kernel_ms_median=med_ms, median_launches=n_med,
               bytes=nbytes, sum_l=sum_l, batch=B, splits=S, case=c, chunk=chunk)
    return res


def run_swa(torch, pkv, workloads, args):
    dev = torch.device("cuda:0")
    c = workloads.config4(value_device=dev)
    r2t, rpi, sl, pf = (c.req_to_token.to(dev), c.req_pool_indices.to(dev), c.seq_lens.to(dev),
                        c.prefill_lens.to(dev))
    B, hq, d = c.q.shape
    hkv = c.k_cache.shape[2]
    S = c.num_splits
    pt = torch.empty((B, c.table_width), dtype=torch.int32, device=dev)
    kl = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    # balanced ranges (kv_chunk 0, num_splits 0): the library cuts the batch's
    # visible keys into one round of equal shares
    ws = torch.zeros(pkv.paged_attn_decode_merged_workspace_size(B, hq, d, 0), dtype=torch.uint8,
                     device=dev)
    build_t = Timer(torch)

    def step(timer):
        e_b = build_t.mark() if timer else None
        pkv.build_page_table(r2t, rpi, sl, 1, c.table_width, prefill_lens=pf, window=c.window,
                             page_table=pt, kv_lens=kl, with_cu_seqlens=False)
        e0 = timer.mark() if timer else None
        if timer:
            build_t.pairs.append((e_b, e0))
        # split decode and the merge of its parts: one launch
        pkv.paged_attn_decode_merged(c.q, c.k_cache, c.v_cache, pt, kl, c.scale, kv_chunk=0,
                                     num_splits=0, workspace=ws, out=out, lse=lse)
        if timer:
            timer.pairs.append((e0, timer.mark()))

    ms, kern_ms = device_loop(torch, step, args.steps, args.warmup)
    torch.cuda.synchronize()
    kv_lens = kl.cpu().long()
    nbytes, sum_l = decode_bytes(kv_lens, B, hq, hkv, d, 1)
    return dict(ms=ms, kernel_ms=kern_ms, build_ms=build_t.kernel_ms(), bytes=nbytes,
                sum_kv_len=sum_l, splits=S, case=c, pt=pt, kl=kl)


def run_prefill(torch, pkv, workloads, args, make_case=None, window_left=-1):
    dev = torch.device("cuda:0")
    c = (make_case or workloads.config2)(value_device=dev)
    r2t, rpi, sl, cu = (c.req_to_token.to(dev), c.req_pool_indices.to(dev), c.seq_lens.to(dev),
                        c.cu_seqlens_q.to(dev))
    B = sl.numel()
    pt = torch.empty((B, c.table_width), dtype=torch.int32, device=dev)
    kl = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty_like(c.q)
    lse = torch.empty(c.q.shape[:2], dtype=torch.float32, device=dev)
    max_k = int(c.seq_lens.max())
    ws_bytes = pkv.paged_attn_varlen_prefill_workspace_size(
        B, c.q.shape[0], c.max_seqlen_q, max_k, c.q.shape[1], c.k_cache.shape[2], c.q.shape[2])
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)   # counters stay zero

    def step(timer):
        pkv.build_page_table(r2t, rpi, sl, c.page_size, c.table_width, page_table=pt,
                             kv_lens=kl, with_cu_seqlens=False)
        e0 = timer.mark() if timer else None
        pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, cu, kl, c.max_seqlen_q,
                                      c.scale, max_seqlen_k=max_k, causal=True,
                                      window_left=window_left, workspace=ws, out=out, lse=lse)
        if timer:
            timer.pairs.append((e0, timer.mark()))

    ms, kern_ms = device_loop(torch, step, max(args.steps, 50), args.warmup)
    cold_ms = None
    if make_case is None:
        # cold: a 512 MB rewrite before each launch (outside the event pair)
        flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)

        def cold_step(timer):
            flush.fill_(1)
            step(timer)
        _, cold_ms = device_loop(torch, cold_step, max(args.steps, 20), args.warmup,
                                 host_us_per_step=120.0)
        del flush
    flops, pairs = prefill_flops(c.extend_lens.tolist(), c.seq_lens.tolist(), c.q.shape[1],
                                 c.q.shape[2], window_left)
    return dict(ms=ms, kernel_ms=kern_ms, cold_ms=cold_ms, flops=flops, pairs=pairs, case=c,
                pt=pt, kl=kl)


def run_prefill_append(torch, pkv, workloads, args):
    """config2's extend step with its cache write: the new tokens' K/V are
    written at out_cache_loc (the slots the page table maps the new positions
    to), then the extend attention runs over the updated cache; one call."""
    dev = torch.device("cuda:0")
    c = workloads.config2(value_device=dev)
    r2t, rpi, sl, cu = (c.req_to_token.to(dev), c.req_pool_indices.to(dev), c.seq_lens.to(dev),
                        c.cu_seqlens_q.to(dev))
    pre = (c.seq_lens - c.extend_lens).tolist()
    loc = torch.cat([c.req_to_token[int(c.req_pool_indices[b]), pre[b]:pre[b] + int(n)]
                     for b, n in enumerate(c.extend_lens.tolist())]).to(torch.int64).to(dev)
    hkv, d = c.k_cache.shape[2], c.k_cache.shape[3]
    kn = c.k_cache.view(-1, hkv, d)[loc].clone()
    vn = c.v_cache.view(-1, hkv, d)[loc].clone()
    loc = loc.to(torch.int32)
    B = sl.numel()
    pt = torch.empty((B, c.table_width), dtype=torch.int32, device=dev)
    kl = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty_like(c.q)
    lse = torch.empty(c.q.shape[:2], dtype=torch.float32, device=dev)
    max_k = int(c.seq_lens.max())
    ws_bytes = pkv.paged_attn_varlen_prefill_workspace_size(
        B, c.q.shape[0], c.max_seqlen_q, max_k, c.q.shape[1], hkv, d)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(timer):
        pkv.build_page_table(r2t, rpi, sl, c.page_size, c.table_width, page_table=pt,
                             kv_lens=kl, with_cu_seqlens=False)
        e0 = timer.mark() if timer else None
        pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, cu, kl, c.max_seqlen_q,
                                      c.scale, max_seqlen_k=max_k, causal=True, workspace=ws,
                                      out=out, lse=lse, k_new=kn, v_new=vn, out_cache_loc=loc)
        if timer:
            timer.pairs.append((e0, timer.mark()))

    ms, call_ms = device_loop(torch, step, max(args.steps, 50), args.warmup)
    flops, _ = prefill_flops(c.extend_lens.tolist(), c.seq_lens.tolist(), c.q.shape[1],
                             c.q.shape[2])
    append_bytes = 2 * 2 * kn.numel() * kn.element_size() + 4 * loc.numel()
    return dict(ms=ms, call_ms=call_ms, flops=flops, append_bytes=append_bytes, case=c, pt=pt,
                kl=kl, k_new=kn, v_new=vn)


def run_cascade(torch, pkv, workloads, args):
    """Draft-tree verification by cascade attention: expand-table build, then
    the prefix pass (each kv head's 4 heads x 8 drafts packed into one 32-row
    MFMA tile, key splits merged by a short second launch) and the expand
    pass + merge."""
    dev = torch.device("cuda:0")
    c = workloads.cascade_verify(value_device=dev)
    r2t, rpi, sl = (c.req_to_token.to(dev), c.req_pool_indices.to(dev), c.seq_lens.to(dev))
    mask = c.custom_mask.to(dev)
    B, n = sl.numel(), c.num_draft
    _, hq, d = c.q.shape
    hkv = c.k_cache.shape[2]
    pt, kl, _ = pkv.build_page_table(r2t, rpi, sl, c.page_size, c.table_width,
                                     with_cu_seqlens=False)
    tab = torch.empty((B * n, n), dtype=torch.int32, device=dev)
    lens = torch.empty((B * n,), dtype=torch.int32, device=dev)
    cu_q = torch.arange(0, B * n + 1, n, dtype=torch.int32, device=dev)
    out = torch.empty_like(c.q)
    lse = torch.empty((B * n, hq), dtype=torch.float32, device=dev)
    max_k = int(c.seq_lens.max())
    ws_bytes = pkv.paged_attn_cascade_workspace_size(B, B * n, n, max_k, hq, hkv, d)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    build_t = Timer(torch)

    def step(timer):
        e_b = build_t.mark() if timer else None
        pkv.build_cascade_expand_table(mask, r2t, rpi, sl, n, expand_table=tab, expand_lens=lens,
                                       with_cu=False)
        e0 = timer.mark() if timer else None
        if timer:
            build_t.pairs.append((e_b, e0))
        pkv.paged_attn_cascade(c.q, c.k_cache, c.v_cache, pt, cu_q, kl, n, c.scale, tab, lens,
                               max_seqlen_k=max_k, workspace=ws, out=out, lse=lse)
        if timer:
            timer.pairs.append((e0, timer.mark()))

    ms, kern_ms = device_loop(torch, step, max(args.steps, 20), args.warmup, host_us_per_step=150.0)
    torch.cuda.synchronize()
    sum_l = int(c.seq_lens.long().sum())
    vis = int(lens.long().sum())
    row_bytes = 2 * hkv * d * 2                     # K and V of one token, all kv heads
    nbytes = (sum_l + B * n) * row_bytes + 2 * B * n * hq * d * 2 + B * n * hq * 4
    flops = 4 * d * hq * (n * sum_l + vis)
    return dict(ms=ms, kernel_ms=kern_ms, build_ms=build_t.kernel_ms(), bytes=nbytes, flops=flops,
                sum_l=sum_l, batch=B, n=n, ws=ws_bytes, case=c)


def run_dca(torch, pkv, workloads, args):
    """Dual chunk attention decode: metadata build, the one-pass split-KV decode
    with per-chunk queries (one split per chunk), merge_state."""
    dev = torch.device("cuda:0")
    c = workloads.dca_decode(value_device=dev)
    b = c.base
    r2t, rpi, sl = (b.req_to_token.to(dev), b.req_pool_indices.to(dev), b.seq_lens.to(dev))
    B, hq, d = b.q.shape
    _, P, hkv, _ = b.k_cache.shape
    C = c.chunk_size - c.local_size
    S = -(-int(b.seq_lens.max()) // C)
    pt = torch.empty((B, b.table_width), dtype=torch.int32, device=dev)
    kl = torch.empty((B,), dtype=torch.int32, device=dev)
    op = torch.empty((S, B, hq, d), dtype=torch.float32, device=dev)
    lp = torch.empty((S, B, hq), dtype=torch.float32, device=dev)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, hq), dtype=torch.float32, device=dev)

    def step(timer):
        pkv.build_page_table(r2t, rpi, sl, P, b.table_width, page_table=pt, kv_lens=kl,
                             with_cu_seqlens=False)
        meta = pkv.build_dca_decode_tables(pt, kl, C, P, c.original_max_position_embeddings)
        e0 = timer.mark() if timer else None
        pkv.paged_attn_dca_decode(b.q, c.q_succ, c.q_inter, b.k_cache, b.v_cache, pt, kl,
                                  b.scale, C, kv_chunk=C, num_splits=S,
                                  q_scale=meta["scaling_factor"], o_partial=op, lse_partial=lp)
        if timer:
            timer.pairs.append((e0, timer.mark()))
        pkv.merge_state(op, lp, out=out, lse_out=lse)

    ms, kern_ms = timed_loop(torch, step, args.steps, args.warmup)
    nbytes, sum_l = decode_bytes(b.seq_lens.long(), B, hq, hkv, d, P)
    nbytes += 2 * B * hq * d * 2                   # the succ and inter queries
    return dict(ms=ms, kernel_ms=kern_ms, bytes=nbytes, sum_l=sum_l, splits=S, case=c, pt=pt, kl=kl)


def run_sparse(torch, pkv, workloads, args):
    dev = torch.device("cuda:0")
    c = workloads.config5(value_device=dev)
    r2t, rpi, idx = (c.req_to_token.to(dev), c.req_pool_indices.to(dev), c.topk_idx.to(dev))
    B, hq, dqk = c.q.shape
    dv = c.head_dim_v
    K = idx.shape[1]
    out = torch.empty((B, hq, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    need = pkv.sparse_topk_decode_workspace_size(B, K, hq, dv)
    ws = torch.zeros((max(need, 1),), dtype=torch.uint8, device=dev)   # counters start at zero
    # a buffer larger than the 256 MB last-level cache, rewritten before each
    # timed step so the 85 MB working set is read from HBM
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)

    def one(timer):
        e0 = timer.mark() if timer else None
        pkv.sparse_topk_decode(c.q, c.kv_cache, r2t, rpi, idx, c.scale, head_dim_v=dv,
                               workspace=ws, out=out, lse=lse)
        if timer:
            timer.pairs.append((e0, timer.mark()))

    warm_ms, warm_kern = device_loop(torch, one, max(args.steps, 50), args.warmup)
    # cold: a 512 MB rewrite between launches (outside the event pair)
    def cold_step(timer):
        flush.fill_(1)
        one(timer)
    _, cold_ms = device_loop(torch, cold_step, max(args.steps, 20), args.warmup,
                             host_us_per_step=120.0)
    n_valid = int((c.topk_idx >= 0).sum())
    nbytes = (n_valid * dqk * 2 + B * hq * dqk * 2 + B * hq * dv * 2 + B * K * 4 * 2)
    flops = 2 * n_valid * hq * (dqk + dv)
    return dict(warm_ms=warm_kern, cold_ms=cold_ms, bytes=nbytes, flops=flops, case=c)


def run_copy(torch, args):
    """A plain copy kernel of known size (1 GiB read + 1 GiB written), for
    calibrating the FETCH_SIZE / WRITE_SIZE counters."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    a = torch.ones((n // 4,), dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    return dict(bytes_read=n, bytes_written=n)


# ---------------------------------------------------------------------------
# CPU oracle on a bounded sample of the decode workload
# ---------------------------------------------------------------------------

def cpu_baseline_decode(torch, res, budget_s):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    c = res["case"]
    pt_all, kl_all, _ = oracle.page_table_strided(
        c.req_to_token.cpu().numpy(), c.req_pool_indices.cpu().numpy(),
        c.seq_lens.cpu().numpy(), c.page_size, c.table_width)
    P = c.page_size
    done_bytes = 0
    spent = 0.0
    n_req = 0
    sum_l = 0
    B, hq, d = c.q.shape
    hkv = c.k_cache.shape[2]
    for b in range(B):
        L = int(kl_all[b])
        n = -(-L // P)
        pages = torch.as_tensor(pt_all[b, :n].astype(np.int64), device=c.k_cache.device)
        k = c.k_cache[pages].to(torch.float64).cpu().numpy()   # host copy: not timed
        v = c.v_cache[pages].to(torch.float64).cpu().numpy()
        q = c.q[b:b + 1].to(torch.float64).cpu().numpy()
        pt = np.arange(n, dtype=np.int64)[None, :]
        t0 = time.perf_counter()
        op, lp = oracle.paged_decode_splitkv(q, k, v, pt, np.array([L]), P, c.scale,
                                             c.kv_chunk, c.num_splits)
        oracle.merge_state(op, lp)
        spent += time.perf_counter() - t0
        done_bytes += 2 * L * hkv * d * 2 + hq * d * 2 * 2 + 4 * n
        sum_l += L
        n_req += 1
        if spent >= budget_s:
            break
    cores = len(os.sched_getaffinity(0))
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s",
            "cores": cores, "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"config3 requests 0..{n_req - 1} ({n_req} of {B}, {sum_l} keys, all "
                      f"{hq} heads, {c.num_splits} splits + merge), float64 numpy with "
                      f"{blas_threads} BLAS threads; {spent:.1f} s"}


def _core_fields():
    """Host cores this process may run on, and the BLAS threads the oracle used."""
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": _blas_threads()}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_oracle_prefill(torch, r):
    """The oracle over every request of config2 (page size 1), per request."""
    import numpy as np
    import oracle
    c, pt, kl = r["case"], r["pt"].cpu().numpy(), r["kl"].cpu().numpy()
    cu = c.cu_seqlens_q.cpu().numpy()
    spent, flops = 0.0, 0
    for b in range(len(kl)):
        L, q0, q1 = int(kl[b]), int(cu[b]), int(cu[b + 1])
        slots = torch.as_tensor(pt[b, :L].astype(np.int64), device=c.k_cache.device)
        k = c.k_cache[slots].to(torch.float64).cpu().numpy()   # host copies: not timed
        v = c.v_cache[slots].to(torch.float64).cpu().numpy()
        q = c.q[q0:q1].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        oracle.paged_prefill(q, k, v, np.arange(L)[None, :], np.array([0, q1 - q0]),
                             np.array([L]), 1, c.scale, causal=True)
        spent += time.perf_counter() - t0
        M = q1 - q0
        flops += 4 * c.q.shape[2] * c.q.shape[1] * sum(L - M + j + 1 for j in range(M))
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", **_core_fields(),
            "kind": "oracle", "sample": f"all {len(kl)} requests of config2, float64 numpy; "
                                        f"{spent:.1f} s"}


def cpu_oracle_swa(torch, r, budget_s):
    """The oracle (split-KV decode + merge) over config4's requests in order."""
    import numpy as np
    import oracle
    c, pt, kl = r["case"], r["pt"].cpu().numpy(), r["kl"].cpu().numpy()
    hq, d = c.q.shape[1], c.q.shape[2]
    hkv = c.k_cache.shape[2]
    spent, nbytes, n = 0.0, 0, 0
    for b in range(len(kl)):
        L = int(kl[b])
        slots = torch.as_tensor(pt[b, :L].astype(np.int64), device=c.k_cache.device)
        k = c.k_cache[slots].to(torch.float64).cpu().numpy()
        v = c.v_cache[slots].to(torch.float64).cpu().numpy()
        q = c.q[b:b + 1].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        op, lp = oracle.paged_decode_splitkv(q, k, v, np.arange(L)[None, :], np.array([L]), 1,
                                             c.scale, c.kv_chunk, c.num_splits)
        oracle.merge_state(op, lp)
        spent += time.perf_counter() - t0
        nbytes += 2 * L * hkv * d * 2 + hq * d * 2 * 2 + 4 * L
        n += 1
        if spent >= budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", **_core_fields(),
            "kind": "oracle", "sample": f"config4 requests 0..{n - 1} ({n} of {len(kl)}), float64 "
                                        f"numpy; {spent:.1f} s"}


def cpu_oracle_decode_window(torch, r, window_left, budget_s):
    """The oracle's windowed split-KV decode (+ merge) over config3's requests in
    order, each request's pages gathered first."""
    import numpy as np
    import oracle
    c = r["case"]
    pt_all, kl_all, _ = oracle.page_table_strided(
        c.req_to_token.cpu().numpy(), c.req_pool_indices.cpu().numpy(),
        c.seq_lens.cpu().numpy(), c.page_size, c.table_width)
    P = c.page_size
    hq, d = c.q.shape[1], c.q.shape[2]
    hkv = c.k_cache.shape[2]
    spent, nbytes, done = 0.0, 0, 0
    for b in range(len(kl_all)):
        L = int(kl_all[b])
        npg = -(-L // P)
        pages = torch.as_tensor(pt_all[b, :npg].astype(np.int64), device=c.k_cache.device)
        k = c.k_cache[pages].to(torch.float64).cpu().numpy()
        v = c.v_cache[pages].to(torch.float64).cpu().numpy()
        q = c.q[b:b + 1].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        op, lp = oracle.paged_decode_splitkv(q, k, v, np.arange(npg)[None, :], np.array([L]), P,
                                             c.scale, r["chunk"], r["splits"],
                                             window_left=window_left)
        oracle.merge_state(op, lp)
        spent += time.perf_counter() - t0
        vis = min(L, window_left + 1)
        nbytes += 2 * vis * hkv * d * 2 + 2 * hq * d * 2
        done += 1
        if spent >= budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", **_core_fields(),
            "kind": "oracle", "sample": f"config3 requests 0..{done - 1} ({done} of "
                                        f"{len(kl_all)}) under the window, float64 numpy; "
                                        f"{spent:.1f} s"}


def cpu_oracle_prefill_window(torch, r, window_left, rows):
    """The oracle's windowed causal extend on the last `rows` new tokens of the
    first long prompt (its keys gathered first)."""
    import numpy as np
    import oracle
    c, pt, kl = r["case"], r["pt"].cpu().numpy(), r["kl"].cpu().numpy()
    cu = c.cu_seqlens_q.cpu().numpy()
    L, q1 = int(kl[0]), int(cu[1])
    slots = torch.as_tensor(pt[0, :L].astype(np.int64), device=c.k_cache.device)
    k = c.k_cache[slots].to(torch.float64).cpu().numpy()
    v = c.v_cache[slots].to(torch.float64).cpu().numpy()
    q = c.q[q1 - rows:q1].to(torch.float64).cpu().numpy()
    t0 = time.perf_counter()
    oracle.paged_prefill(q, k, v, np.arange(L)[None, :], np.array([0, rows]), np.array([L]), 1,
                         c.scale, causal=True, window_left=window_left)
    spent = time.perf_counter() - t0
    flops = 4 * c.q.shape[2] * c.q.shape[1] * sum(min(L - rows + j + 1, window_left + 1)
                                                  for j in range(rows))
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", **_core_fields(),
            "kind": "oracle", "sample": f"the last {rows} new tokens of prompt 0 ({L} keys) under "
                                        f"the window, float64 numpy; {spent:.1f} s"}


def cpu_oracle_prefill_append(torch, r):
    """The oracle's append-then-extend over every request of config2 (each
    request's cache rows gathered first; the append writes the new rows)."""
    import numpy as np
    import oracle
    c, pt, kl = r["case"], r["pt"].cpu().numpy(), r["kl"].cpu().numpy()
    cu = c.cu_seqlens_q.cpu().numpy()
    kn, vn = r["k_new"].to(torch.float64).cpu().numpy(), r["v_new"].to(torch.float64).cpu().numpy()
    spent = 0.0
    for b in range(len(kl)):
        L, q0, q1 = int(kl[b]), int(cu[b]), int(cu[b + 1])
        slots = torch.as_tensor(pt[b, :L].astype(np.int64), device=c.k_cache.device)
        k = c.k_cache[slots].to(torch.float64).cpu().numpy()
        v = c.v_cache[slots].to(torch.float64).cpu().numpy()
        q = c.q[q0:q1].to(torch.float64).cpu().numpy()
        loc = np.arange(L - (q1 - q0), L)          # the new tokens' rows of the gathered cache
        t0 = time.perf_counter()
        oracle.paged_prefill_append(q, k, v, np.arange(L)[None, :], np.array([0, q1 - q0]),
                                    np.array([L]), 1, c.scale, loc, kn[q0:q1], vn[q0:q1])
        spent += time.perf_counter() - t0
    return {"value": round(r["flops"] / spent / 1e12, 6), "unit": "TFLOP/s",
            **_core_fields(), "kind": "oracle",
            "sample": f"all {len(kl)} requests of config2 (append + extend), float64 numpy; "
                      f"{spent:.1f} s"}


def cpu_oracle_cascade(torch, r, budget_s):
    """The oracle's plain tree attention over the draft-tree workload's requests
    in order (each request's committed and draft tokens gathered first)."""
    import numpy as np
    import oracle
    c = r["case"]
    n = c.num_draft
    sl = c.seq_lens.cpu().numpy().astype(np.int64)
    r2t, rpi = c.req_to_token.cpu().numpy(), c.req_pool_indices.cpu().numpy()
    mask = c.custom_mask.cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(n * (sl + n))])
    kflat = c.k_cache.reshape(-1, 1, *c.k_cache.shape[2:])
    vflat = c.v_cache.reshape(-1, 1, *c.v_cache.shape[2:])
    hq, d = c.q.shape[1], c.q.shape[2]
    hkv = c.k_cache.shape[2]
    spent, nbytes, done = 0.0, 0, 0
    for b in range(len(sl)):
        L = int(sl[b])
        slots = torch.as_tensor(r2t[rpi[b], :L + n].astype(np.int64), device=c.k_cache.device)
        k = kflat[slots].to(torch.float64).cpu().numpy()      # host copies: not timed
        v = vflat[slots].to(torch.float64).cpu().numpy()
        q = c.q[b * n:(b + 1) * n].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        oracle.tree_verify_attention(q, k, v, np.arange(L + n)[None, :], [0], [L],
                                     mask[starts[b]:starts[b + 1]], n, c.scale)
        spent += time.perf_counter() - t0
        nbytes += (L + n) * 2 * hkv * d * 2 + 2 * n * hq * d * 2 + n * hq * 4
        done += 1
        if spent >= budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", **_core_fields(),
            "kind": "oracle", "sample": f"draft-tree workload requests 0..{done - 1} ({done} of "
                                        f"{len(sl)}), plain tree attention, float64 numpy; "
                                        f"{spent:.1f} s"}


def cpu_oracle_dca(torch, r, budget_s):
    """The oracle's three-stage dual chunk decode over the workload's requests
    in order (each request's pages gathered first)."""
    import numpy as np
    import oracle
    c = r["case"]
    b0 = c.base
    pt, kl = r["pt"].cpu().numpy(), r["kl"].cpu().numpy()
    P = b0.page_size
    hq, d = b0.q.shape[1], b0.q.shape[2]
    hkv = b0.k_cache.shape[2]
    spent, nbytes, done = 0.0, 0, 0
    for b in range(len(kl)):
        L = int(kl[b])
        npg = -(-L // P)
        pages = torch.as_tensor(pt[b, :npg].astype(np.int64), device=b0.k_cache.device)
        k = b0.k_cache[pages].to(torch.float64).cpu().numpy()
        v = b0.v_cache[pages].to(torch.float64).cpu().numpy()
        qs = [x[b:b + 1].to(torch.float64).cpu().numpy() for x in (b0.q, c.q_succ, c.q_inter)]
        t0 = time.perf_counter()
        oracle.dca_decode(*qs, k, v, np.arange(npg)[None, :], np.array([L]), P, b0.scale,
                          c.chunk_size, c.local_size,
                          original_max_position_embeddings=c.original_max_position_embeddings)
        spent += time.perf_counter() - t0
        nbytes += 2 * L * hkv * d * 2 + 4 * hq * d * 2 + 4 * npg
        done += 1
        if spent >= budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", **_core_fields(),
            "kind": "oracle", "sample": f"dual chunk decode requests 0..{done - 1} ({done} of "
                                        f"{len(kl)}), three stages + merge, float64 numpy; "
                                        f"{spent:.1f} s"}


def cpu_oracle_sparse(torch, r, budget_s):
    """The oracle over config5's requests in order (touched rows copied per request)."""
    import numpy as np
    import oracle
    c = r["case"]
    r2t = c.req_to_token.cpu().numpy()
    rpi = c.req_pool_indices.cpu().numpy()
    idx = c.topk_idx.cpu().numpy()
    dqk, dv = c.q.shape[2], c.head_dim_v
    spent, nbytes, n = 0.0, 0, 0
    for b in range(idx.shape[0]):
        valid = idx[b] >= 0
        slots = r2t[rpi[b], idx[b][valid]]
        kv = c.kv_cache[torch.as_tensor(slots.astype(np.int64), device=c.kv_cache.device)]
        kv = kv.to(torch.float64).cpu().numpy()
        small = np.zeros((1, r2t.shape[1]), dtype=np.int64)
        small[0, idx[b][valid]] = np.arange(len(slots))
        q = c.q[b:b + 1].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        oracle.sparse_topk_decode(q, kv, small, np.array([0]), idx[b:b + 1], c.scale, dv)
        spent += time.perf_counter() - t0
        nbytes += int(valid.sum()) * dqk * 2 + c.q.shape[1] * (dqk + dv) * 2 + idx.shape[1] * 8
        n += 1
        if spent >= budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", **_core_fields(),
            "kind": "oracle", "sample": f"config5 requests 0..{n - 1} ({n} of {idx.shape[0]}), "
                                        f"float64 numpy; {spent:.1f} s"}


# ---------------------------------------------------------------------------

def summarize_hbm_counters(out_dir):
    """HBM bytes per dispatch of every library kernel from the counter runs
    under out_dir (hbm_<workload>_<FETCH_SIZE|WRITE_SIZE>/*counter_collection.csv,
    one rocprofv3 --pmc run per counter), each counter scaled by what it reads
    for the 1 GiB copy kernel of `--only copy`. Returns the JSON-ready summary."""
    import csv
    import glob

    def load(workload, counter):
        files = glob.glob(os.path.join(out_dir, f"hbm_{workload}_{counter}", "*counter_collection.csv"))
        if not files:
            raise FileNotFoundError(f"no {counter} results for {workload} under {out_dir}")
        per = {}
        names = {}
        for row in csv.DictReader(open(files[0])):
            d = row["Dispatch_Id"]
            per[d] = per.get(d, 0.0) + float(row["Counter_Value"])
            names[d] = row["Kernel_Name"].split("(")[0].replace("void ", "").strip()
        out = {}
        for d, v in per.items():
            out.setdefault(names[d], []).append(v)
        return out

    cf, cw = load("copy", "FETCH_SIZE"), load("copy", "WRITE_SIZE")
    copy_fetch = max(max(v) for v in cf.values())
    copy_write = max(max(v) for v in cw.values())
    ff = COPY_BYTES / 1024 / copy_fetch
    wf = COPY_BYTES / 1024 / copy_write
    summary = {"calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_kib": round(copy_fetch, 1),
                               "copy_write_kib": round(copy_write, 1),
                               "fetch_factor": round(ff, 5), "write_factor": round(wf, 5)},
               "workloads": {}}
    for w, srcs in WORKLOAD_SOURCES.items():
        fetch, write = load(w, "FETCH_SIZE"), load(w, "WRITE_SIZE")
        kernels = {}
        for name in sorted(set(fetch) | set(write)):
            if not name.startswith("pkv::"):
                continue
            fk = sum(fetch.get(name, [0.0])) / max(len(fetch.get(name, [])), 1)
            wk = sum(write.get(name, [0.0])) / max(len(write.get(name, [])), 1)
            kernels[name] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                             "dispatches": len(fetch.get(name, [])),
                             "bytes": int(round(fk * 1024 * ff + wk * 1024 * wf))}
        summary["workloads"][w] = {"source_hash": source_hash(*srcs), "kernels": kernels,
                                   "step_bytes": sum(k["bytes"] for k in kernels.values())}
    return summary


def stored_traffic(workload, algorithmic_bytes, kernel_prefix=None):
    """HBM traffic of one step of `workload` (or of its kernel named by
    `kernel_prefix`) from the committed counter summary, with its ratio to the
    algorithmic bytes; None when the summary was taken on other kernel sources."""
    try:
        with open(HBM_TRAFFIC) as f:
            ent = json.load(f)["workloads"][workload]
    except (OSError, ValueError, KeyError):
        return None
    if ent.get("source_hash") != source_hash(*WORKLOAD_SOURCES[workload]):
        return None
    if kernel_prefix is None:
        b = ent["step_bytes"]
    else:
        hits = [k["bytes"] for n, k in ent["kernels"].items() if n.startswith(kernel_prefix)]
        if not hits:
            return None
        b = hits[0]
    return {"bytes": b, "per_algorithmic": round(b / algorithmic_bytes, 4) if algorithmic_bytes
            else None, "source_hash": ent["source_hash"]}


def main(argv=None):
    args = parse_args(argv)
    if args.hbm_summary:
        print(json.dumps(summarize_hbm_counters(args.hbm_summary), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the hot path runs on a single MI355X here)", file=sys.stderr)
        return 2
    import torch
    sys.path.insert(0, ROOT)
    import paged_kv_cache_197_amd as pkv
    import workloads
    pkv.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.only == "copy":
        print(json.dumps({"copy": run_copy(torch, args)}))
        return 0

    line = {}
    extra = {}
    if args.only in ("all", "decode"):
        r = run_decode(torch, pkv, workloads, args, mode="merged")
        gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        achieved = r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
        line = {
            "metric": "decode KV GB/s (% HBM peak); prefill TFLOP/s (% bf16 MFMA peak)",
            "value": round(gbs, 2),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(r["ms"], 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {
                "workload": "config3: batched split-KV GQA decode (page-table build, then the "
                            "split-KV decode with the merge_state combine of its splits in the "
                            "same launch), B=64, L~U[1024,32768], 32 q / 8 kv heads, D=128, "
                            "page 64, 40000-page pool, 4096-token chunks",
                "batch": r["batch"], "sum_kv_len": r["sum_l"], "num_splits": r["splits"],
                "algorithmic_bytes_per_step": r["bytes"],
            },
            "roofline": {
                "kernel": "decode_group_kernel<128, uniform page> (bf16), merging its splits",
                "bound": "hbm",
                "achieved": round(achieved, 2),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "kernel_ms": round(r["kernel_ms"], 4),
                "kernel_ms_median": round(r["kernel_ms_median"], 4),
                "median_launches": r["median_launches"],
                "traffic": stored_traffic("decode", r["bytes"], "pkv::decode_group_kernel"),
            },
        }
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_decode(torch, r, args.cpu_seconds)
        del r
        torch.cuda.empty_cache()

    if args.only in ("all", "decode_split"):
        try:
            r = run_decode(torch, pkv, workloads, args, mode="split")
            extra["decode_split_merge"] = {
                "workload": "config3 as two launches: page-table build, split-KV decode into "
                            "fp32 partials, then merge_state (the same result bit for bit)",
                "device_ms_per_step": round(r["ms"], 4),
                "decode_kernel_ms": round(r["kernel_ms"], 4),
                "decode_kernel_ms_median": round(r["kernel_ms_median"], 4),
                "step_GB/s": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 2),
                "kernel_GB/s": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                "kernel_frac_hbm": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": r["bytes"], "num_splits": r["splits"],
                "traffic": stored_traffic("decode_split", r["bytes"])}
        except Exception as e:
            extra["decode_split_merge"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "decode_merged"):
        try:
            r = run_decode(torch, pkv, workloads, args, mode="balanced")
            extra["decode_merged"] = {
                "workload": "config3's batch through the merged entry point with balanced "
                            "ranges (instead of 4096-token chunks): page-table build, then the "
                            "decode and the merge of its parts in one launch",
                "device_ms_per_step": round(r["ms"], 4),
                "decode_merge_kernel_ms": round(r["kernel_ms"], 4),
                "decode_merge_kernel_ms_median": round(r["kernel_ms_median"], 4),
                "step_GB/s": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 2),
                "kernel_GB/s": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                "kernel_frac_hbm": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": r["bytes"], "split_mode": "balanced ranges",
                "traffic": stored_traffic("decode_merged", r["bytes"])}
        except Exception as e:
            extra["decode_merged"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "decode_window"):
        try:
            W = 4095
            r = run_decode(torch, pkv, workloads, args, window_left=W, kv_chunk=2048,
                           mode="balanced")
            extra["decode_window"] = {
                "workload": "config3 under an in-kernel sliding window (W, 0) with W = 4095 "
                            "(each query sees its last 4096 keys) over the strided table; "
                            "merged decode over balanced ranges (the visible keys cut into 256 "
                            "equal workgroup shares, one per CU, parts merged in the same launch)",
                "device_ms_per_step": round(r["ms"], 4),
                "decode_merge_kernel_ms": round(r["kernel_ms"], 4),
                "kernel_GB/s": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                "kernel_frac_hbm": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
                "visible_keys": r["sum_l"], "algorithmic_bytes": r["bytes"],
                "split_mode": "balanced ranges",
                "traffic": stored_traffic("decode_window", r["bytes"])}
            if not args.no_cpu_baseline:
                extra["decode_window"]["cpu_oracle"] = cpu_oracle_decode_window(torch, r, W, 4.0)
        except Exception as e:
            extra["decode_window"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "swa"):
        try:
            r = run_swa(torch, pkv, workloads, args)
            extra["swa_decode"] = {
                "workload": "config4: prefill-aware sliding-window decode, B=32, window 4096, "
                            "64 q / 8 kv heads, D=128, page 1 (table built on GPU); merged "
                            "decode over balanced ranges (the batch's visible keys cut into 256 "
                            "equal workgroup shares, one per CU, parts merged in the same "
                            "launch)",
                "device_ms_per_step": round(r["ms"], 4),
                "decode_merge_kernel_ms": round(r["kernel_ms"], 4),
                "table_build_ms": round(r["build_ms"], 4),
                "GB/s": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 2),
                "kernel_GB/s": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                "kernel_frac_hbm": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
                "sum_kv_len": r["sum_kv_len"], "split_mode": "balanced ranges",
                "traffic": stored_traffic("swa", r["bytes"])}
            if not args.no_cpu_baseline:
                extra["swa_decode"]["cpu_oracle"] = cpu_oracle_swa(torch, r, 4.0)
        except Exception as e:  # report, do not hide
            extra["swa_decode"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill"):
        try:
            r = run_prefill(torch, pkv, workloads, args)
            tf = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
            extra["prefill"] = {
                "workload": "config2: varlen causal extend, prefix [0,128,512,1000] + new "
                            "[256,64,512,17], 32 q / 8 kv heads, D=128, page 1",
                "kernel_ms": round(r["kernel_ms"], 5), "device_ms_per_step": round(r["ms"], 5),
                "TFLOP/s": round(tf, 2), "peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS,
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": r["flops"],
                "visible_pairs_per_head": r["pairs"],
                "cold_kernel_ms": round(r["cold_ms"], 5),
                "cold_TFLOP/s": round(r["flops"] / (r["cold_ms"] * 1e-3) / 1e12, 2)}
            if not args.no_cpu_baseline:
                extra["prefill"]["cpu_oracle"] = cpu_oracle_prefill(torch, r)
        except Exception as e:
            extra["prefill"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill_long"):
        try:
            r = run_prefill(torch, pkv, workloads, args, workloads.long_prompt_prefill)
            tf = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
            extra["prefill_long"] = {
                "workload": "long prompts (steady state of the prefill kernel, beside config2): "
                            "4 requests x 4096 new tokens, no prefix, 32 q / 8 kv heads, D=128, "
                            "page 1",
                "kernel_ms": round(r["kernel_ms"], 5), "device_ms_per_step": round(r["ms"], 5),
                "TFLOP/s": round(tf, 2), "peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS,
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": r["flops"]}
        except Exception as e:
            extra["prefill_long"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill_window"):
        try:
            W = 1023
            r = run_prefill(torch, pkv, workloads, args, workloads.long_prompt_prefill,
                            window_left=W)
            tf = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
            extra["prefill_window"] = {
                "workload": "long prompts (4 x 4096 new tokens, 32 q / 8 kv heads, D=128, "
                            "page 1) under a sliding window (W, 0), W = 1023",
                "kernel_ms": round(r["kernel_ms"], 5), "device_ms_per_step": round(r["ms"], 5),
                "TFLOP/s": round(tf, 2), "peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS,
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": r["flops"]}
            if not args.no_cpu_baseline:
                extra["prefill_window"]["cpu_oracle"] = cpu_oracle_prefill_window(torch, r, W, 512)
        except Exception as e:
            extra["prefill_window"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill_append"):
        try:
            r = run_prefill_append(torch, pkv, workloads, args)
            extra["prefill_append"] = {
                "workload": "config2's extend step with its cache write (new tokens' K/V "
                            "scattered to out_cache_loc, then the extend attention; one call, "
                            "two kernels)",
                "call_ms": round(r["call_ms"], 5), "device_ms_per_step": round(r["ms"], 5),
                "append_bytes": r["append_bytes"],
                "attention_TFLOP/s_over_call": round(r["flops"] / (r["call_ms"] * 1e-3) / 1e12, 2)}
            if not args.no_cpu_baseline:
                extra["prefill_append"]["cpu_oracle"] = cpu_oracle_prefill_append(torch, r)
        except Exception as e:
            extra["prefill_append"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "cascade"):
        try:
            r = run_cascade(torch, pkv, workloads, args)
            extra["cascade_verify"] = {
                "workload": "draft-tree verification by cascade attention: B=64, committed "
                            "L~U[1024,16384], 8 drafts per request (random tree), 32 q / 8 kv "
                            "heads, D=128, page 64; expand-table build + prefix pass (packed "
                            "(head, draft) rows, key splits + their merge) + expand pass and "
                            "merge",
                "device_ms_per_step": round(r["ms"], 4),
                "cascade_ms": round(r["kernel_ms"], 4), "table_build_ms": round(r["build_ms"], 4),
                "cascade_GB/s": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                "cascade_frac_hbm": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
                                          / HBM_PEAK_GBS, 4),
                "TFLOP/s": round(r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12, 2),
                "algorithmic_bytes": r["bytes"], "flops": r["flops"],
                "sum_committed_len": r["sum_l"], "workspace_bytes": r["ws"],
                "traffic": stored_traffic("cascade", r["bytes"])}
            if not args.no_cpu_baseline:
                extra["cascade_verify"]["cpu_oracle"] = cpu_oracle_cascade(torch, r, 4.0)
        except Exception as e:
            extra["cascade_verify"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "dca"):
        try:
            r = run_dca(torch, pkv, workloads, args)
            extra["dca_decode"] = {
                "workload": "dual chunk attention decode: B=32, L~U[4096,65536], 32 q / 8 kv "
                            "heads, D=128, page 64, chunk_size 8192 / local 1024 (7168-key "
                            "chunks, one split each), scaled queries; tables + decode + merge",
                "ms_per_step": round(r["ms"], 4), "decode_kernel_ms": round(r["kernel_ms"], 4),
                "kernel_GB/s": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                "kernel_frac_hbm": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
                "step_GB/s": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 2),
                "sum_kv_len": r["sum_l"], "num_splits": r["splits"],
                "algorithmic_bytes": r["bytes"], "traffic": stored_traffic("dca", r["bytes"])}
            if not args.no_cpu_baseline:
                extra["dca_decode"]["cpu_oracle"] = cpu_oracle_dca(torch, r, 4.0)
        except Exception as e:
            extra["dca_decode"] = {"error": repr(e)}
        torch.cuda.empty_cache()

    if args.only in ("all", "sparse"):
        try:
            r = run_sparse(torch, pkv, workloads, args)
            extra["sparse_mla"] = {
                "workload": "config5: top-k sparse MLA decode, B=32, ctx 65536, top-k 2048, "
                            "128 heads, Dqk 576, Dv 512",
                "cold_kernel_ms": round(r["cold_ms"], 5), "warm_kernel_ms": round(r["warm_ms"], 5),
                "cold_GB/s": round(r["bytes"] / (r["cold_ms"] * 1e-3) / 1e9, 2),
                "cold_frac_hbm": round(r["bytes"] / (r["cold_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       4),
                "warm_GB/s": round(r["bytes"] / (r["warm_ms"] * 1e-3) / 1e9, 2),
                "cold_TFLOP/s": round(r["flops"] / (r["cold_ms"] * 1e-3) / 1e12, 2),
                "bytes": r["bytes"], "flops": r["flops"],
                "traffic": stored_traffic("sparse", r["bytes"])}
            if not args.no_cpu_baseline:
                extra["sparse_mla"]["cpu_oracle"] = cpu_oracle_sparse(torch, r, 4.0)
        except Exception as e:
            extra["sparse_mla"] = {"error": repr(e)}

    clk = device_clock_mhz()
    extra["device"] = {
        "sclk_max_mhz": clk,
        "bf16_mfma_peak_at_sclk_max_TFLOP/s": (round(256 * 4096 * clk * 1e6 / 1e12, 1)
                                               if clk else None),
        "note": "fractions use 2516.6 TFLOP/s (2.4 GHz) and 8 TB/s"}
    if line:
        line["other_workloads"] = extra
    else:
        line = {"other_workloads": extra}
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())

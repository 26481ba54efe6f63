#!/usr/bin/env python3
"""One-GPU benchmark of the NVFP4-compressed sparse-MLA decode step on MI355X.

Workload (the metric's configuration): B=32 requests, q_len=1, H=64 heads, each request a
140K-token (143,360) NVFP4 cache in 64-row pages with random block tables, top-k 2048 positions per
query token drawn uniformly without replacement, bf16 queries, fp32 output. A step is one pass of
the hot path over one batch: quantize-append of the step's new rows (one per query token) and the
sparse decode (index resolve, row gather, on-chip decode, QK, online softmax, PV, split combine).

Inputs are synthetic and seeded, generated and quantized on the GPU before timing. To keep the
256 MB Infinity Cache from serving the gathers, the timed steps rotate through R distinct
(index list, query) sets whose gathered bytes total >= 1 GB. Steps run as replays of captured
HIP graphs. The fused decode kernel's own duration is taken with HIP events recorded around it by
the library (``mla_set_timing_events``) on the launch stream.

``--gpus N`` with N > 1 exits: the library and this benchmark run on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PAGE = 64 * 352
FP8_PAGE = 64 * 576
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_batched_counters.txt")
SPIN_CYCLES = 2_000_000          # GPU spin before a timed region (about a millisecond)
HEAT_MS = 30.0                   # GPU work replayed before the warmup of every timed region
KERNEL_SOURCES = [os.path.join(ROOT, "nvfp4_compressed_mla_amd", "csrc", f)
                  for f in ("decode.hip", "nvfp4_device.h", "codec_device.h", "mla_internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def head_group_blocks(H: int) -> int:
    """16-head blocks per decode workgroup of the first launch (the library groups up to 64 heads)."""
    return min(4, H // 16)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


# ---- workload construction ---------------------------------------------------------------------

class SparseWorkload:
    """Caches, tables, rotated queries / index lists and preallocated outputs of one config.

    ``fmt``: "nvfp4" (the fused NVFP4 kernel), "fp8" (the same inputs as 576-byte FP8 rows, the
    fused FP8 kernel) or "staged" (NVFP4 cache; selected rows converted to FP8 in a workspace,
    then the FP8 kernel).
    """

    def __init__(self, name, B, q_len, H, ctx, topk, append_rows, rotations, seed, device,
                 q_lens=None, keep_latent=False, fmt="nvfp4", overlap=None, q_dtype="bf16"):
        import torch
        from nvfp4_compressed_mla_amd import workloads as wl
        import nvfp4_compressed_mla_amd as m
        self.name, self.B, self.q_len, self.H, self.topk = name, B, q_len, H, topk
        self.fmt = fmt
        self.page = FP8_PAGE if fmt == "fp8" else PAGE
        self.row_bytes = 576 if fmt == "fp8" else 352
        append_fn = m.mla_fp8_append if fmt == "fp8" else m.mla_nvfp4_quantize_append
        self.ctx = list(ctx)
        self.append_rows = append_rows
        self.q_lens = q_lens
        existing = [c - append_rows for c in self.ctx]
        total_rows = sum(existing)
        # pages for the existing rows plus the rows this step appends
        bt, n_pages = wl.gen_block_table(self.ctx, seed + 1, device)
        self.block_table = bt
        self.cache = torch.zeros(n_pages * self.page, dtype=torch.uint8, device=device)
        lat, rope = wl.gen_latent_rope(total_rows, seed, device)
        slots = torch.cat([wl.slot_mapping_for(bt, b, 0, c) for b, c in enumerate(existing)])
        append_fn(lat, rope, slots, self.cache, self.page)
        self.row_base = [0]
        for c in existing[:-1]:
            self.row_base.append(self.row_base[-1] + c)
        self.latent, self.rope = (lat, rope) if keep_latent else (None, None)
        # rows appended by every step: append_rows per request at positions [existing, ctx)
        n_new = append_rows * B
        self.new_lat, self.new_rope = wl.gen_latent_rope(n_new, seed + 7, device)
        self.new_slots = torch.cat([wl.slot_mapping_for(bt, b, existing[b], append_rows)
                                    for b in range(B)])
        self.rot = rotations
        self.q_dtype = q_dtype
        self.q = [wl.gen_queries(B, q_len, H, q_dtype, seed + 100 + r, device) for r in range(rotations)]
        if overlap is not None:
            self.idx = [wl.gen_topk_overlap(B, q_len, topk, self.ctx, overlap, seed + 200 + r, device)
                        for r in range(rotations)]
        elif q_lens is None and len(set(self.ctx)) == 1 and self.ctx[0] >= topk:
            self.idx = [wl.gen_topk_batched(B, q_len, topk, self.ctx[0], seed + 200 + r, device)
                        for r in range(rotations)]
        else:
            self.idx = [wl.gen_topk(B, q_len, topk, self.ctx, seed + 200 + r, device, q_lens=q_lens)
                        for r in range(rotations)]
        T = B * q_len
        self.splits = m.mla_sparse_decode_num_splits(T, H, topk, 0)
        ws = m.mla_decode_workspace_size(T, H, self.splits)
        if fmt == "staged":
            ws = m.mla_staged_workspace_size(T, H, topk, self.splits)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        self.out = torch.empty(B, q_len, H, 512, dtype=torch.float32, device=device)
        self.lse = torch.empty(B, q_len, H, dtype=torch.float32, device=device)
        # algorithmic units: valid (token, row) pairs of each rotation
        self.valid_pairs = [int((i >= 0).sum().item()) for i in self.idx]
        torch.cuda.synchronize()

    def use_shared_rows(self):
        """Decode through the shared-row entry point from now on (same inputs and result)."""
        import torch
        import nvfp4_compressed_mla_amd as m
        need = m.mla_shared_decode_workspace_size(self.B, self.q_len, self.H, self.topk)
        self.ws_shared = torch.empty(max(need, 256), dtype=torch.uint8, device=self.cache.device)
        self.splits = m.mla_shared_decode_num_splits(self.B, self.q_len, self.H, self.topk)
        self.fmt = "shared"

    def use_fused_append(self):
        """From now on a step is one fused append + decode call (the same cache bytes and result
        as the append followed by the decode); needs one appended row per query token."""
        assert self.fmt == "nvfp4" and self.append_rows == self.q_len
        self.fmt = "fused"

    def decode(self, r):
        import nvfp4_compressed_mla_amd as m
        if self.fmt == "fused":
            m.mla_sparse_decode_append(self.q[r], self.cache, self.page, self.block_table, self.idx[r],
                                       1.0 / math.sqrt(576.0), self.new_lat, self.new_rope,
                                       self.new_slots, out=self.out, lse=self.lse,
                                       num_splits=self.splits, workspace=self.ws)
            return
        if self.fmt == "shared":
            m.mla_sparse_decode_shared(self.q[r], self.cache, self.page, self.block_table, self.idx[r],
                                       1.0 / math.sqrt(576.0), out=self.out, lse=self.lse,
                                       workspace=self.ws_shared)
            return
        fn = {"nvfp4": m.mla_sparse_decode, "fp8": m.mla_fp8_sparse_decode,
              "staged": m.mla_staged_sparse_decode}[self.fmt]
        fn(self.q[r], self.cache, self.page, self.block_table, self.idx[r], 1.0 / math.sqrt(576.0),
           out=self.out, lse=self.lse, num_splits=self.splits, workspace=self.ws)

    def append(self):
        import nvfp4_compressed_mla_amd as m
        if self.append_rows and self.fmt != "fused":      # the fused call appends itself
            fn = m.mla_fp8_append if self.fmt == "fp8" else m.mla_nvfp4_quantize_append
            fn(self.new_lat, self.new_rope, self.new_slots, self.cache, self.page)

    def step(self, r):
        self.append()
        self.decode(r)

    # algorithmic bytes / flops of the fused decode kernel for rotation r (with the fused append:
    # plus the appended rows' bf16 input, 352-byte output and slot)
    def kernel_bytes(self, r):
        T = self.B * self.q_len
        qb = 4 if self.q_dtype == "fp32" else 2
        app = self.append_rows * self.B * (1152 + 352 + 8) if self.fmt == "fused" else 0
        return self.valid_pairs[r] * (self.row_bytes + 4 + 4) + T * self.H * 576 * qb + app

    def launch_bytes(self, r):
        """The whole decode launch (fused kernel + combine): the kernel's bytes plus the fp32
        output and lse it finally writes."""
        T = self.B * self.q_len
        return self.kernel_bytes(r) + T * self.H * (512 + 1) * 4

    def gathered_bytes(self, r):
        return self.valid_pairs[r] * self.row_bytes

    def flops(self, r):
        return self.valid_pairs[r] * 2 * self.H * (576 + 512)

    def step_bytes(self, r):
        """Whole-step algorithmic bytes: append (bf16 in, 352 B out, slot) + decode incl. output."""
        app = self.append_rows * self.B * (1152 + 352 + 8)
        return app + self.launch_bytes(r)


class DenseWorkload:
    def __init__(self, B, H, ctx, split_tokens, rotations, seed, device):
        import torch
        from nvfp4_compressed_mla_amd import workloads as wl
        import nvfp4_compressed_mla_amd as m
        self.B, self.H, self.ctx, self.split_tokens = B, H, ctx, split_tokens
        # `rotations` independent caches so consecutive launches stream different bytes
        self.caches, self.tables = [], []
        for r in range(rotations):
            bt, n_pages = wl.gen_block_table([ctx] * B, seed + 1 + r, device)
            cache = torch.zeros(n_pages * PAGE, dtype=torch.uint8, device=device)
            lat, rope = wl.gen_latent_rope(B * ctx, seed + 10 * r, device)
            slots = torch.cat([wl.slot_mapping_for(bt, b, 0, ctx) for b in range(B)])
            m.mla_nvfp4_quantize_append(lat, rope, slots, cache, PAGE)
            del lat, rope
            self.caches.append(cache)
            self.tables.append(bt)
        self.rot = rotations
        self.q = [wl.gen_queries(B, 1, H, "bf16", seed + 100 + r, device) for r in range(rotations)]
        self.seq = torch.full((B,), ctx, dtype=torch.int32, device=device)
        self.splits = m.mla_dense_decode_num_splits(self.tables[0].shape[1], split_tokens)
        self.ws = torch.empty(max(m.mla_decode_workspace_size(B, H, self.splits), 256),
                              dtype=torch.uint8, device=device)
        self.out = torch.empty(B, 1, H, 512, dtype=torch.float32, device=device)
        self.lse = torch.empty(B, 1, H, dtype=torch.float32, device=device)
        torch.cuda.synchronize()

    def decode(self, r):
        import nvfp4_compressed_mla_amd as m
        m.mla_dense_decode(self.q[r], self.caches[r], PAGE, self.tables[r], self.seq,
                           1.0 / math.sqrt(576.0), split_tokens=self.split_tokens, out=self.out,
                           lse=self.lse, workspace=self.ws)

    step = decode

    def kernel_bytes(self, r):
        return self.B * self.ctx * (352 + 4 / 64) + self.B * self.H * 576 * 2

    def launch_bytes(self, r):
        return self.kernel_bytes(r) + self.B * self.H * (512 + 1) * 4

    def gathered_bytes(self, r):
        return self.B * self.ctx * 352

    def flops(self, r):
        return self.B * self.ctx * 2 * self.H * (576 + 512)


# ---- timing helpers ----------------------------------------------------------------------------

def capture(fn, n, offset=0):
    """Capture fn(offset), ..., fn(offset+n-1) into one HIP graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            fn(offset + i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(offset + i)
    torch.cuda.synchronize()
    return g


def _graph_plan(rot, n, tail_at_end):
    """Whole graphs covering n steps: (steps, first rotation) per replay. Full rotation graphs
    first; the remainder n % rot is one graph of that many consecutive steps, over the first
    rotations (timed region) or the last ones (warmup, so that the timed steps that follow start
    on rotations the warmup did not just read)."""
    plan = [(rot, 0)] * (n // rot)
    r = n % rot
    if r:
        plan.append((r, rot - r if tail_at_end else 0))
    return plan


def time_steps(fn, rot, steps, warmup, stats=None):
    """Replay captured graphs for `warmup` then exactly `steps` steps; returns ms per step, timed
    with HIP events on the replay stream around the whole timed region.

    Every replay is a whole multi-step graph (a full pass over the `rot` rotations, or one graph
    of the remaining steps), so the per-step figure does not depend on how `steps` divides by
    `rot`. When `stats` is a dict it receives the per-replay step times (HIP events around each
    replay on the replay stream): median, p10, p90 (us per step) and the replay count.
    """
    import torch
    graphs = {}
    warm_plan = _graph_plan(rot, warmup, True)
    time_plan = _graph_plan(rot, steps, False)
    for key in set(warm_plan + time_plan):
        graphs[key] = capture(fn, key[0], key[1])
    # The first replay of a captured graph carries one-time costs: pay them for every timed graph
    # before the warmup (which then moves the infinity cache away from the timed rotations).
    # The timed graphs are replayed until at least HEAT_MS of GPU work has run, so that the GPU
    # enters the warmup in the same state whatever the step counts (a 20-step timing after a
    # 5-step warmup otherwise measured a GPU still settling from the setup).
    heat = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    heat[0].record()
    while True:
        for key in set(time_plan):
            graphs[key].replay()
        heat[1].record()
        torch.cuda.synchronize()
        if heat[0].elapsed_time(heat[1]) >= HEAT_MS or not time_plan:
            break
    for key in warm_plan:
        graphs[key].replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in time_plan]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # A GPU spin ahead of the timed replays: the host queues them while it runs, so that no
    # replay waits for its own submission (a single 20-step graph would otherwise carry the
    # whole submission latency, a 48-step one a smaller share of it). The timed region is the
    # stream's own: from the event after the spin to the event after the last replay.
    torch.cuda._sleep(SPIN_CYCLES)
    start.record()
    for key, (a, b) in zip(time_plan, evs):
        a.record()
        graphs[key].replay()
        b.record()
    end.record()
    torch.cuda.synchronize()
    if stats is not None:
        per = sorted(a.elapsed_time(b) * 1e3 / key[0] for key, (a, b) in zip(time_plan, evs))

        def pct(q):
            return per[min(len(per) - 1, max(0, int(round(q * (len(per) - 1)))))]
        stats.update({"median_us": round(pct(0.5), 3), "p10_us": round(pct(0.1), 3),
                      "p90_us": round(pct(0.9), 3), "replays": len(per),
                      "steps_per_replay": sorted({k[0] for k in time_plan})})
    return start.elapsed_time(end) / steps


def time_decode_kernel(wk, launches):
    """Average fused-decode-kernel duration (ms) from library-recorded HIP events, eager launches."""
    import torch
    import nvfp4_compressed_mla_amd as m
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(launches)]
    for a, b in pairs:                      # materialise the underlying HIP events
        a.record()
        b.record()
    torch.cuda.synchronize()
    try:
        for i, (a, b) in enumerate(pairs):
            m.mla_set_timing_events(a.cuda_event, b.cuda_event)
            wk.decode(i % wk.rot)
    finally:
        m.mla_set_timing_events(None, None)
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b) for a, b in pairs]
    durs = durs[min(5, len(durs) // 4):]    # first launches of a cold process excluded
    return sum(durs) / len(durs), durs


def counters_traffic(src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; None otherwise."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---- top-k position selection ---------------------------------------------------------------------

def topk_bench(dev, reps=20):
    """Top-2048 positions per query token from fp32 scores (the step before the decode): the
    pages' launch shape, the batched and the MTP shapes; graph-replayed launches."""
    import torch
    import nvfp4_compressed_mla_amd as m
    res = {}
    for name, B, q_len, n in (("pages_T15_146K", 1, 15, 149504), ("batched_T32_140K", 32, 1, 143360),
                              ("mtp_T240_146K", 16, 15, 149504)):
        g = torch.Generator(device=dev).manual_seed(77)
        rot = 4
        scores = [torch.randn(B, q_len, n, generator=g, device=dev) for _ in range(rot)]
        seq = torch.full((B,), n, dtype=torch.int32, device=dev)
        out = torch.empty(B, q_len, 2048, dtype=torch.int32, device=dev)
        ws = torch.empty(m.mla_topk_workspace_size(B * q_len, n, 2048), dtype=torch.uint8, device=dev)
        fn = lambda r: m.mla_topk_indices(scores[r % rot], seq, 2048, out=out, workspace=ws)
        ms = time_steps(fn, rot, reps * rot, rot)
        rd = B * q_len * n * 4
        res[name] = {"us_per_launch": round(ms * 1e3, 2), "scores_read_GBps": round(rd / (ms * 1e-3) / 1e9, 1)}
        del scores
        torch.cuda.empty_cache()
    return res


# ---- indexer scores -> top-k -> decode (the pages' launch shape) ----------------------------------

def indexer_chain(dev, reps=20, rot=4):
    """The step before the path and the path: FP8 indexer scores of every visible position
    (64 heads x 128 dims), top-2048 selection, then the fused NVFP4 decode over the selected
    rows, at the pages' launch shape (one request, 15 query tokens, 149,504 positions, 16 heads).
    Each stage graph-replayed on its own, then the three in one graph per step; `rot` rotations
    of distinct indexer caches, queries and MLA queries."""
    import torch
    import nvfp4_compressed_mla_amd as m
    from nvfp4_compressed_mla_amd import workloads as wl
    B, q_len, H, n = 1, 15, 16, 149504
    wk = SparseWorkload("pages_chain", B, q_len, H, [n], 2048, 0, rot, 1006, dev)
    ix = [wl.gen_indexer(wk.cache.numel() // PAGE, B, q_len, 1106 + r, dev) for r in range(rot)]
    seq = torch.full((B,), n, dtype=torch.int32, device=dev)
    scores = [torch.zeros(B, q_len, n, dtype=torch.float32, device=dev) for _ in range(rot)]
    ws = torch.empty(m.mla_topk_workspace_size(B * q_len, n, 2048), dtype=torch.uint8, device=dev)

    def idx_fn(r):
        c, q, w = ix[r % rot]
        m.mla_indexer_scores(q, w, c, wl.INDEXER_PAGE_BYTES, wk.block_table, seq, n_max=n,
                             out=scores[r % rot])

    def topk_fn(r):
        m.mla_topk_indices(scores[r % rot], seq, 2048, out=wk.idx[r % rot], workspace=ws)

    def chain(r):
        idx_fn(r)
        topk_fn(r)
        wk.decode(r % rot)

    for r in range(rot):                      # lists of the real indexer scores for the decode
        idx_fn(r)
        topk_fn(r)
    torch.cuda.synchronize()
    wk.valid_pairs = [int((i >= 0).sum().item()) for i in wk.idx]
    res = {}
    for name, fn in (("indexer", idx_fn), ("topk", topk_fn), ("decode", lambda r: wk.decode(r % rot)),
                     ("chain", chain)):
        ms = time_steps(fn, rot, reps * rot, rot)
        res[name + "_us"] = round(ms * 1e3, 2)
    T = B * q_len
    flops = T * n * 64 * 128 * 2
    byt = (wk.cache.numel() // PAGE) * wl.INDEXER_PAGE_BYTES + T * 64 * (128 + 4) + T * n * 4
    t_idx = res["indexer_us"] * 1e-6
    res["indexer_fp8_TFLOPs"] = round(flops / t_idx / 1e12, 1)
    res["indexer_mfma_frac_fp8"] = round(flops / t_idx / 5.0e15, 4)
    res["indexer_GBps"] = round(byt / t_idx / 1e9, 1)
    res["indexer_hbm_frac"] = round(byt / t_idx / 8e12, 4)
    res["note"] = ("indexer: 64 heads x 128 dims E4M3, a dense contraction (36.7 GFLOP, 28.8 MB per launch); "
                   "chain: indexer + top-k + decode captured together per step")
    del wk, ix, scores
    torch.cuda.empty_cache()
    return res


# ---- block transfer between multi-layer pools --------------------------------------------------

def kv_transfer(dev, n_layers=64, ctx=204800, pool_blocks=16000, reps=5):
    """One 200K-token request's blocks (all layers) copied between two pools, block-major and
    layer-major, in one launch each; contiguous regions (transfer descriptors) per layout."""
    import torch
    import nvfp4_compressed_mla_amd as m
    page = PAGE
    n_blk = ctx // 64
    g = torch.Generator().manual_seed(2024)
    sb = torch.randperm(pool_blocks, generator=g)[:n_blk].to(torch.int32)
    db = torch.randperm(pool_blocks, generator=g)[:n_blk].to(torch.int32)
    src = torch.empty(pool_blocks * n_layers * page, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(7)
    sbd, dbd = sb.to(dev), db.to(dev)
    moved = n_blk * n_layers * page
    res = {"layers": n_layers, "blocks": n_blk, "bytes_moved": moved}
    for name, layout in (("block_major", m.MLA_LAYOUT_BLOCK_MAJOR), ("layer_major", m.MLA_LAYOUT_LAYER_MAJOR)):
        m.mla_copy_kv_blocks(src, dst, layout, n_layers, page, sbd, dbd)       # warm
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            m.mla_copy_kv_blocks(src, dst, layout, n_layers, page, sbd, dbd)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        res[name] = {"descriptors": m.mla_kv_transfer_regions(layout, n_layers, page, pool_blocks, sb.numpy()),
                     "ms": round(ms, 3), "moved_GBps": round(moved / (ms * 1e-3) / 1e9, 1),
                     "hbm_GBps_read_plus_write": round(2 * moved / (ms * 1e-3) / 1e9, 1)}
    del src, dst
    torch.cuda.empty_cache()
    return res


# ---- cache-flush cross-check -------------------------------------------------------------------

def flush_check(wk, launches=24):
    """The fused kernel timed with a 1 GiB scratch fill before every launch, which evicts the L2s
    and the 256 MB Infinity Cache, as a cross-check of the rotated-input timing (the rotation is
    what keeps the timed steps from being served by those caches)."""
    import torch
    import nvfp4_compressed_mla_amd as m
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=wk.out.device)
    durs = []
    for i in range(launches + 4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        scratch.fill_(i & 0xFF)
        torch.cuda.synchronize()
        m.mla_set_timing_events(a.cuda_event, b.cuda_event)
        try:
            wk.decode(i % wk.rot)
        finally:
            m.mla_set_timing_events(None, None)
        torch.cuda.synchronize()
        if i >= 4:
            durs.append(a.elapsed_time(b))
    del scratch
    torch.cuda.empty_cache()
    return sum(durs) / len(durs)


# ---- measured streaming ceilings ---------------------------------------------------------------

def stream_ceiling(dev, gib=2, reps=5):
    """HBM rates a plain streaming kernel reaches on this machine, as context for the roofline: a
    read-only pass (torch's sum over a 2 GiB fp32 tensor) and a device copy of 2 GiB (read + write).
    Best of `reps` event-timed launches each."""
    import torch
    n = gib << 30
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    out = {}
    for name, fn, moved in (("read_sum", lambda: x.sum(), n), ("copy_read_plus_write", lambda: y.copy_(x), 2 * n)):
        fn()
        best = None
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1])
            best = ms if best is None else min(best, ms)
        out[name] = {"bytes": moved, "ms": round(best, 4), "GBps": round(moved / (best * 1e-3) / 1e9, 1)}
    del x, y
    torch.cuda.empty_cache()
    return out


# ---- CPU oracle baseline -----------------------------------------------------------------------

def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wk, budget_s=12.0):
    """The CPU oracle (fp64 NumPy, untuned) on the same step: quantize the step's new rows and
    decode all query tokens of rotation 0 from a cache the oracle built itself from the same bf16
    rows. Setup (oracle quantization of the selected rows) is untimed. Repeats whole steps until
    ``budget_s`` elapsed."""
    import numpy as np
    import torch
    from oracle import attention as oa
    from oracle import cache as oc
    from oracle import nvfp4 as nv
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    idx = wk.idx[0].cpu().numpy()
    bt = wk.block_table.cpu().numpy()
    q = wk.q[0].float().cpu().numpy().astype(np.float64)
    cache = np.zeros(wk.cache.numel(), dtype=np.uint8)
    for b in range(wk.B):
        pos = np.unique(idx[b][idx[b] >= 0])
        rows = torch.as_tensor(wk.row_base[b] + pos, device=wk.latent.device)
        enc = nv.quantize_rows(wk.latent[rows].double().cpu().numpy(), wk.rope[rows].double().cpu().numpy())
        oc.write_rows(cache, PAGE, [oc.logical_slot(bt[b], int(j)) for j in pos], enc)
    new_lat = wk.new_lat.double().cpu().numpy()
    new_rope = wk.new_rope.double().cpu().numpy()
    new_slots = wk.new_slots.cpu().numpy()
    n = 0
    t0 = time.perf_counter()
    while True:
        oc.write_rows(cache, PAGE, new_slots, nv.quantize_rows(new_lat, new_rope))
        oa.sparse_decode(q, cache, PAGE, bt, idx, 1.0 / math.sqrt(576.0))
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    return {
        "value": round(wk.gathered_bytes(0) / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n} whole step(s) of the batched config ({wk.B * wk.q_len} query tokens x "
                   f"{wk.topk} rows + {wk.append_rows * wk.B} appended rows), "
                   f"{dt * 1e3:.0f} ms per step; host cpus visible: {len(os.sched_getaffinity(0))}; "
                   f"cpu: {cpu_model()}"),
    }


# ---- main --------------------------------------------------------------------------------------

def run_config(wk, steps, warmup, prof_launches):
    """Graph-timed decode launches plus event-timed fused kernel for one extra config."""
    st = {}
    ms = time_steps(wk.decode, wk.rot, steps, warmup, st)
    kavg, _ = time_decode_kernel(wk, prof_launches)
    nb = sum(wk.kernel_bytes(r) for r in range(wk.rot)) / wk.rot
    lb = sum(wk.launch_bytes(r) for r in range(wk.rot)) / wk.rot
    gb = sum(wk.gathered_bytes(r) for r in range(wk.rot)) / wk.rot
    fl = sum(wk.flops(r) for r in range(wk.rot)) / wk.rot
    return {
        "us_per_launch": round(ms * 1e3, 2),
        "launch_replays_us": st,
        "fused_kernel_us": round(kavg * 1e3, 2),
        "gathered_GBps": round(gb / (ms * 1e-3) / 1e9, 1),
        "kernel_GBps": round(nb / (kavg * 1e-3) / 1e9, 1),
        "kernel_hbm_frac": round(nb / (kavg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "launch_GBps": round(lb / (ms * 1e-3) / 1e9, 1),
        "launch_hbm_frac": round(lb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "kernel_TFLOPs": round(fl / (kavg * 1e-3) / 1e12, 1),
        "kernel_mfma_frac": round(fl / (kavg * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
        "splits": wk.splits,
        **({"q_dtype": wk.q_dtype} if getattr(wk, "q_dtype", "bf16") != "bf16" else {}),
        **({"note": "fused_kernel_us is the FP8 decode kernel alone; us_per_launch includes the "
                    "staging pass and the combine"} if getattr(wk, "fmt", "") == "staged" else {}),
    }


def counter_target(name, dev, launches=4):
    """Eager launches of one workload and nothing else, for rocprofv3 counter passes."""
    import torch
    from nvfp4_compressed_mla_amd import workloads as wl
    if name == "mixed_append":
        mx = wl.named_workload("mixed")
        mw = SparseWorkload("mixed", mx.B, 15, 64, [c + 6144 for c in mx.ctx], 2048, 6144, 1, 1004,
                            dev, q_lens=mx.q_lens)
        torch.cuda.synchronize()
        log("[bench] counter target: mixed-step append (393,216 rows)")
        for _ in range(launches):
            mw.append()
    else:
        for f in (0.0, 0.9):
            w64 = SparseWorkload("mtp_ov", 16, 15, 64, [149504] * 16, 2048, 0, 1, 1005, dev, overlap=f)
            log(f"[bench] counter target: MTP overlap {f}, 64 heads, per-token decode")
            for _ in range(launches):
                w64.decode(0)
            torch.cuda.synchronize()
            del w64
            w16 = SparseWorkload("mtp_ov16", 16, 15, 16, [149504] * 16, 2048, 0, 1, 1007, dev, overlap=f)
            w16.use_shared_rows()
            log(f"[bench] counter target: MTP overlap {f}, 16 heads, shared rows")
            for _ in range(launches):
                w16.decode(0)
            torch.cuda.synchronize()
            del w16
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    print(json.dumps({"counter_target": name, "launches": launches}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=960)
    ap.add_argument("--warmup", type=int, default=96)
    ap.add_argument("--rotations", type=int, default=48)
    ap.add_argument("--prof-launches", type=int, default=64)
    ap.add_argument("--no-extra", action="store_true", help="skip the other configurations")
    ap.add_argument("--extras", default="all",
                    help="comma list of other configurations to run: pages, mtp, tiny, dense, "
                         "mixed, three_way, mtp_overlap, kv_transfer, topk, indexer, ceiling, flush (default all; 'none' = --no-extra)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--counter-target", choices=("mixed_append", "mtp_overlap"),
                    help="only run a few eager launches of one workload (a target for counter "
                         "passes): the mixed step's 393,216-row append, or the MTP shape under the "
                         "overlap model (f = 0 and 0.9; per-token at 64 heads, shared rows at 16)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; each GPU "
              "would serve its own requests with no exchange between GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "copies": 3}))
        return

    import nvfp4_compressed_mla_amd as m
    m.load_library()                         # raises if the HIP library was not built

    if args.counter_target:
        counter_target(args.counter_target, dev)
        return

    log("[bench] building batched workload (B=32, H=64, 143,360-token caches, top-k 2048)")
    t_setup = time.perf_counter()
    wk = SparseWorkload("batched", B=32, q_len=1, H=64, ctx=[143360 + 1] * 32, topk=2048,
                        append_rows=1, rotations=args.rotations, seed=1001, device=dev,
                        keep_latent=not args.no_cpu_baseline)
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; splits={wk.splits}")

    # the step as three launches (append, decode, merge), then the headline: the append fused
    # into the decode kernel (two launches)
    sep_stats = {}
    ms_sep = time_steps(wk.step, wk.rot, max(args.steps // 2, wk.rot), args.warmup, sep_stats)
    log(f"[bench] append + decode step {ms_sep * 1e3:.2f} us (replays: {sep_stats})")
    wk.use_fused_append()
    step_stats, dec_stats = {}, {}
    ms_step = time_steps(wk.step, wk.rot, args.steps, args.warmup, step_stats)
    log(f"[bench] fused step {ms_step * 1e3:.2f} us (replays: {step_stats})")
    ms_dec = time_steps(wk.decode, wk.rot, max(args.steps // 2, wk.rot), args.warmup, dec_stats)
    kavg, kd = time_decode_kernel(wk, args.prof_launches)
    log(f"[bench] fused launch {ms_dec * 1e3:.2f} us, fused kernel {kavg * 1e3:.2f} us")

    gathered = sum(wk.gathered_bytes(r) for r in range(wk.rot)) / wk.rot
    kbytes = sum(wk.kernel_bytes(r) for r in range(wk.rot)) / wk.rot
    lbytes = sum(wk.launch_bytes(r) for r in range(wk.rot)) / wk.rot
    flops = sum(wk.flops(r) for r in range(wk.rot)) / wk.rot
    achieved = kbytes / (kavg * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = counters_traffic(src_hash)

    result = {
        "metric": "sparse-MLA decode us/launch + achieved HBM GB/s (% of peak), 140K ctx top-k 2048",
        "value": round(gathered / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "batched sparse decode step: B=32, q_len=1, H=64, ctx 143,360 "
                               "(+1 appended row per request), top-k 2048, 64-row pages, random "
                               "block tables",
                   "global_batch": 32, "seq_len": 143360, "topk": 2048, "heads": 64,
                   "rotations": wk.rot, "splits": wk.splits},
        "step_timing": "HIP events on the replay stream around exactly `steps` graph-replayed steps, "
                       "after a GPU spin that lets the host queue the replays ahead of the GPU",
        "step": "one mla_sparse_decode_append call (the 32 new rows quantize-appended inside the "
                "decode kernel) + the split merge",
        "step_replays_us": step_stats,
        "step_append_then_decode_us": round(ms_sep * 1e3, 3),
        "step_append_then_decode_replays_us": sep_stats,
        "us_per_launch": round(ms_dec * 1e3, 2),
        "launch_replays_us": dec_stats,
        "gathered_GBps_per_launch": round(gathered / (ms_dec * 1e-3) / 1e9, 1),
        "gathered_pct_of_peak": round(100 * gathered / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": f"decode_kernel<{head_group_blocks(64)},false,false,false,true> (fused append/gather/"
                      "decode/QK/softmax/PV)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel_us": round(kavg * 1e3, 3),
            "algorithmic_bytes_per_launch": int(kbytes),
            "mfma_TFLOPs": round(flops / (kavg * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (kavg * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
            "kernel_source_sha256_16": src_hash,
            "timing_note": "kernel_us comes from HIP events the library records at the fused "
                           "kernel's own start and end (hipExtLaunchKernel's events, on its launch "
                           "stream), over eager launches that each follow some idle time; the "
                           "rocprofv3 trace average, dominated by back-to-back graph replays, is "
                           "about 2 us lower (profiles/decode_batched_kernel_trace.txt)",
        },
        "roofline_launch": {
            "bound": "hbm",
            "what": "whole launch (fused append + decode kernel, split combine), graph-replayed; "
                    "bytes include the fp32 output and lse",
            "achieved": round(lbytes / (ms_dec * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(lbytes / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes_per_launch": int(lbytes),
            "launch_us": round(ms_dec * 1e3, 3),
        },
        "context": {"pages_GB200_us_per_launch_15tok_16heads": 12.0},
    }

    wanted = set() if args.no_extra or args.extras == "none" else (
        {"pages", "mtp", "tiny", "dense", "mixed", "three_way", "mtp_overlap", "kv_transfer", "topk", "indexer",
         "ceiling", "flush"} if args.extras == "all"
        else set(args.extras.split(",")))
    if wanted:
        extra = {}
        for name, key, mk in (
            ("pages", "pages_shape_T15_H16", lambda: SparseWorkload("pages", 1, 15, 16, [149504], 2048, 0, 64, 1101, dev)),
            ("mtp", "mtp_B16_q15_H64", lambda: SparseWorkload("mtp", 16, 15, 64, [149504] * 16, 2048, 0, 6, 1002, dev)),
            ("tiny", "tiny_B1_H16_k256_fp32q", lambda: SparseWorkload("tiny", 1, 1, 16, [4096], 256, 0, 8, 1000, dev, q_dtype="fp32")),
        ):
            if name not in wanted:
                continue
            log(f"[bench] extra: {key}")
            w2 = mk()
            extra[key] = run_config(w2, 192, 24, 32)
            del w2
            torch.cuda.empty_cache()
        if "mtp" in wanted:
            # an MTP decode step that appends its 15 new rows per request (one per query token):
            # append kernel + decode against the fused call, same inputs, graph-replayed steps
            log("[bench] extra: mtp_B16_q15_H64 with its own 15 rows per request appended")
            w2 = SparseWorkload("mtp_append", 16, 15, 64, [149504] * 16, 2048, 15, 6, 1012, dev)
            sep = time_steps(w2.step, w2.rot, 48, 6)
            w2.use_fused_append()
            fus = time_steps(w2.step, w2.rot, 48, 6)
            extra["mtp_B16_q15_H64_step_with_append"] = {
                "append_then_decode_us": round(sep * 1e3, 2), "fused_us": round(fus * 1e3, 2),
                "appended_rows": 16 * 15}
            del w2
            torch.cuda.empty_cache()
        if "dense" in wanted:
            log("[bench] extra: dense_B8_H64_146K")
            dw = DenseWorkload(8, 64, 149504, 4096, 3, 1003, dev)
            extra["dense_B8_H64_146K_split4096"] = run_config(dw, 48, 6, 24)
            # the split size that fits the launch in one wave of workgroups (37 splits of 4096
            # positions give 296 workgroups for 256 compute units)
            st = m.mla_dense_decode_split_tokens(8, 64, dw.tables[0].shape[1])
            del dw
            torch.cuda.empty_cache()
            log(f"[bench] extra: dense_B8_H64_146K one-wave split ({st} positions)")
            dw = DenseWorkload(8, 64, 149504, st, 3, 1003, dev)
            extra["dense_B8_H64_146K_one_wave"] = {"split_tokens": st, **run_config(dw, 48, 6, 24)}
            del dw
            torch.cuda.empty_cache()
        if "mixed" in wanted:
            log("[bench] extra: mixed serving step")
            from nvfp4_compressed_mla_amd import workloads as wl
            mx = wl.named_workload("mixed")
            # history lengths log-uniform in [4K, 200K]; the step appends 6144 rows to each request
            mw = SparseWorkload("mixed", mx.B, 15, 64, [c + 6144 for c in mx.ctx], 2048, 6144, 4, 1004,
                                dev, q_lens=mx.q_lens)
            ms_mixed = time_steps(mw.step, mw.rot, 16, 4)
            # the append kernel alone: HIP events on the launch stream around 8 launches
            mw.append()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(8):
                mw.append()
            ev[1].record()
            torch.cuda.synchronize()
            ms_app = ev[0].elapsed_time(ev[1]) / 8
            app_bytes = 6144 * 64 * (1152 + 352 + 8)
            extra["mixed_B64_step"] = {
                "ms_per_step": round(ms_mixed, 4),
                "append_rows": 6144 * 64,
                "append_ms": round(ms_app, 4),
                "append_GBps": round(app_bytes / (ms_app * 1e-3) / 1e9, 1),
                "append_hbm_frac": round(app_bytes / (ms_app * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "append_bound": "hbm (its VALU issue floor is about the same as the HBM floor)",
                "decode": run_config(mw, 16, 4, 12),
            }
            del mw
            torch.cuda.empty_cache()
        if "three_way" in wanted:
            # the pages' three-way comparison: FP8 576-byte rows with the fused kernel, NVFP4 with
            # the fused kernel, NVFP4 through the staged FP8 buffer
            for shape, mk in (
                ("pages_shape_T15_H16", lambda f: SparseWorkload("pages", 1, 15, 16, [149504], 2048, 0, 64, 1101, dev, fmt=f)),
                ("batched_B32_H64", lambda f: SparseWorkload("batched", 32, 1, 64, [143360] * 32, 2048, 0, 24, 1001, dev, fmt=f)),
            ):
                cmp = {}
                for f in ("fp8", "nvfp4", "staged"):
                    log(f"[bench] three-way: {shape} {f}")
                    w2 = mk(f)
                    cmp[f] = run_config(w2, 192, 24, 32)
                    del w2
                    torch.cuda.empty_cache()
                extra[f"three_way_{shape}"] = cmp
        if "mtp_overlap" in wanted:
            # the MTP shape under an overlap model: the 15 query tokens of a request keep a share of
            # one base set of positions (ascending lists); the splits of a request's tokens run on
            # one XCD, so a row shared by several tokens is fetched from HBM once and then read
            # from that XCD's L2
            ov = {}
            for f in (0.0, 0.5, 0.9):
                log(f"[bench] extra: mtp_overlap {f}")
                w2 = SparseWorkload("mtp_ov", 16, 15, 64, [149504] * 16, 2048, 0, 6, 1005, dev, overlap=f)
                res = run_config(w2, 192, 24, 32)
                uniq = [len(set(w2.idx[0][b].flatten().tolist())) for b in range(16)]
                res["distinct_rows_per_request"] = round(sum(uniq) / len(uniq), 1)
                res["gathered_rows_per_request"] = 15 * 2048
                ov[f"overlap_{f}"] = res
                del w2
                torch.cuda.empty_cache()
            extra["mtp_overlap_B16_q15_H64"] = ov
            # 16 heads per token (the pages' per-rank head count): per-token launch against the
            # shared-row path (each distinct row of 4 consecutive tokens gathered and decoded once)
            ov16 = {}
            for f in (0.0, 0.5, 0.9):
                log(f"[bench] extra: mtp_overlap H=16 {f}")
                w3 = SparseWorkload("mtp_ov16", 16, 15, 16, [149504] * 16, 2048, 0, 6, 1007, dev, overlap=f)
                res = {"per_token": run_config(w3, 192, 24, 32)}
                w3.use_shared_rows()
                res["shared_rows"] = run_config(w3, 192, 24, 32)
                res["shared_rows"]["note"] = ("fused_kernel_us: the shared decode kernel alone; "
                                              "us_per_launch adds the union pass and the split merge; "
                                              "bytes and flops counted per (token, row) pair as in "
                                              "per_token")
                uniq = [len(set(w3.idx[0][b].flatten().tolist())) for b in range(16)]
                res["distinct_rows_per_request"] = round(sum(uniq) / len(uniq), 1)
                ov16[f"overlap_{f}"] = res
                del w3
                torch.cuda.empty_cache()
            extra["mtp_overlap_B16_q15_H16"] = ov16
        if "topk" in wanted:
            extra["topk_2048"] = topk_bench(dev)
        if "indexer" in wanted:
            log("[bench] extra: indexer -> top-k -> decode chain")
            extra["indexer_chain_T15_H16_146K"] = indexer_chain(dev)
        if "kv_transfer" in wanted:
            extra["kv_transfer_200K"] = kv_transfer(dev)
        if "flush" in wanted:
            kf = flush_check(wk)
            extra["mall_flush_check_batched"] = {
                "kernel_us_flushed": round(kf * 1e3, 2),
                "kernel_us_rotated": round(kavg * 1e3, 2),
                "note": "flushed: a 1 GiB scratch fill before every single launch; rotated: the "
                        "roofline's eager launches over the 48 rotated input sets"}
        if "ceiling" in wanted:
            ceil = stream_ceiling(dev)
            extra["hbm_stream_ceiling"] = ceil
            # the faster of the two plain streaming passes (torch's reduction reads well below
            # the copy's rate on this part)
            best = max(ceil["read_sum"]["GBps"], ceil["copy_read_plus_write"]["GBps"])
            result["roofline"]["measured_stream_ceiling_GBps"] = best
            result["roofline"]["frac_of_measured_stream_ceiling"] = round(achieved / best, 4)
        result["extra"] = extra

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wk, args.cpu_seconds)

    print(json.dumps(result))


if __name__ == "__main__":
    main()

"""The hot path captured in a HIP graph, and run on two streams at once.

Graph: quantize-append, sparse decode with a split combine and dense decode recorded once and
replayed several times, with eager work and synchronizations between the replays. Every replay
must reproduce the eager launch bit for bit (the kernels are deterministic and the library
records no memset or allocation into the graph)."""

import math

import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl

pytestmark = pytest.mark.gpu

PAGE = 64 * 352


def test_graph_replays_match_eager():
    import nvfp4_compressed_mla_amd as m
    print("case: graph replay B=4 q_len=2 H=64 ctx 3000+64 topk 512 (sparse) + dense", flush=True)
    dev = "cuda"
    B, q_len, H, topk, new = 4, 2, 64, 512, 64
    ctx = [3000 + new] * B
    bt, n_pages = wl.gen_block_table(ctx, 31, dev)
    cache = torch.zeros(n_pages * PAGE, dtype=torch.uint8, device=dev)
    lat, rope = wl.gen_latent_rope(sum(c - new for c in ctx), 32, dev)
    slots = torch.cat([wl.slot_mapping_for(bt, b, 0, c - new) for b, c in enumerate(ctx)])
    m.mla_nvfp4_quantize_append(lat, rope, slots, cache, PAGE)
    new_lat, new_rope = wl.gen_latent_rope(B * new, 33, dev)
    new_slots = torch.cat([wl.slot_mapping_for(bt, b, c - new, new) for b, c in enumerate(ctx)])
    q = wl.gen_queries(B, q_len, H, "bf16", 34, dev)
    idx = wl.gen_topk(B, q_len, topk, ctx, 35, dev)
    seq = torch.tensor(ctx, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(576.0)
    T = B * q_len
    S = m.mla_sparse_decode_num_splits(T, H, topk, 0)
    assert S > 1                                            # the combine is part of the graph
    ws = torch.empty(max(m.mla_decode_workspace_size(T, H, S), 256), dtype=torch.uint8, device=dev)
    S_d = m.mla_dense_decode_num_splits(bt.shape[1], 1024)
    ws_d = torch.empty(max(m.mla_decode_workspace_size(T, H, S_d), 256), dtype=torch.uint8, device=dev)
    out = torch.empty(B, q_len, H, 512, dtype=torch.float32, device=dev)
    lse = torch.empty(B, q_len, H, dtype=torch.float32, device=dev)
    out_d = torch.empty_like(out)
    lse_d = torch.empty_like(lse)

    def step():
        m.mla_nvfp4_quantize_append(new_lat, new_rope, new_slots, cache, PAGE)
        m.mla_sparse_decode(q, cache, PAGE, bt, idx, scale, out=out, lse=lse, num_splits=S, workspace=ws)
        m.mla_dense_decode(q, cache, PAGE, bt, seq, scale, split_tokens=1024, out=out_d, lse=lse_d,
                           workspace=ws_d)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (cache, out, lse, out_d, lse_d)]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                              # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    filler = torch.randn(512, 512, device=dev)
    for r in range(4):
        for t in (out, lse, out_d, lse_d):
            t.fill_(float("nan"))                           # stale results cannot pass
        cache[new_slots[0] * 352: new_slots[0] * 352 + 352].fill_(0)   # one appended row cleared
        torch.cuda.synchronize()
        g.replay()
        _ = filler @ filler                                 # the program's own eager work
        torch.cuda.synchronize()
        for name, got, want in zip(("cache", "out", "lse", "dense out", "dense lse"),
                                   (cache, out, lse, out_d, lse_d), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager launch"


def test_two_streams_concurrently():
    """Two sparse decodes (own inputs, outputs and workspaces) launched on two streams at once
    give bit for bit what they give one after the other: the library keeps no state between
    calls beyond read-only tables."""
    import nvfp4_compressed_mla_amd as m
    print("case: two concurrent streams, batched-like launches", flush=True)
    dev = "cuda"
    runs = []
    for seed in (81, 91):
        B, H, topk, ctx = 8, 64, 2048, [20000] * 8
        bt, n_pages = wl.gen_block_table(ctx, seed, dev)
        cache = torch.zeros(n_pages * PAGE, dtype=torch.uint8, device=dev)
        lat, rope = wl.gen_latent_rope(sum(ctx), seed + 1, dev)
        slots = torch.cat([wl.slot_mapping_for(bt, b, 0, c) for b, c in enumerate(ctx)])
        m.mla_nvfp4_quantize_append(lat, rope, slots, cache, PAGE)
        q = wl.gen_queries(B, 1, H, "bf16", seed + 2, dev)
        idx = wl.gen_topk(B, 1, topk, ctx, seed + 3, dev)
        S = m.mla_sparse_decode_num_splits(B, H, topk, 0)
        ws = torch.empty(max(m.mla_decode_workspace_size(B, H, S), 256), dtype=torch.uint8, device=dev)
        out = torch.empty(B, 1, H, 512, dtype=torch.float32, device=dev)
        lse = torch.empty(B, 1, H, dtype=torch.float32, device=dev)
        runs.append(dict(cache=cache, bt=bt, q=q, idx=idx, S=S, ws=ws, out=out, lse=lse))
    scale = 1.0 / math.sqrt(576.0)

    def launch(r, stream=None):
        m.mla_sparse_decode(r["q"], r["cache"], PAGE, r["bt"], r["idx"], scale, out=r["out"],
                            lse=r["lse"], num_splits=r["S"], workspace=r["ws"], stream=stream)

    torch.cuda.synchronize()
    ref = []
    for r in runs:
        launch(r)
        torch.cuda.synchronize()
        ref.append((r["out"].clone(), r["lse"].clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for r in runs:
            r["out"].fill_(float("nan"))
            r["lse"].fill_(float("nan"))
        torch.cuda.synchronize()
        for r, s in zip(runs, streams):
            with torch.cuda.stream(s):
                for _ in range(4):                  # several launches in flight on each stream
                    launch(r, s)
        torch.cuda.synchronize()
        for (o, l), r in zip(ref, runs):
            assert torch.equal(r["out"], o) and torch.equal(r["lse"], l), f"repeat {rep}"

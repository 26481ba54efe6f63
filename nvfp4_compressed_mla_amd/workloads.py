"""Seeded synthetic inputs for NVFP4 sparse-MLA decode (no codec or attention arithmetic here).

This module only draws random numbers and lays out index structures; both the HIP path and the
CPU oracle consume what it produces, and it computes nothing of the method itself.

Workload shapes follow the serving traffic described on the [PI] page ("Prime Inference: Fast,
Reliable Serving for Frontier Open Models"): an agent turn appends about 6K tokens to a ~140K-token
prompt (section "How we serve production agent traffic"), each query reads at most 2048 indexer-
selected positions (section "Decode: NVFP4 KV compression"), the cache is paged in 64-token blocks
(section "Changing the layout to reduce fragmentation"), and the kernel figure is quoted at 15 query
tokens per launch with 16 heads per rank (section "Native NVFP4 sparse MLA decode kernel").
K is read as 1024, so 140K = 143,360 tokens (2240 pages), 146K = 149,504 (2336 pages), 200K =
204,800, 6K = 6144.

Distributions: latent, rope and queries ~ N(0, 1) (bf16; fp32 queries for the tiny case); block
tables are a random permutation of all physical pages, sliced per request; top-k lists are the
first k entries of an argsort of uniform keys (uniform sampling without replacement), drawn
independently per query token; when a context is shorter than k the list holds every position
once and the remaining entries are -1, scattered at random places in the list. Indexer inputs
(the synthetic FP8 scorer the top-k step reads): keys and queries are N(0, 1) values cast to
E4M3, key scales uniform in [0.5, 1.5), head weights N(0, 1) / 8.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

PAGE_ROWS = 64
LATENT_DIM = 512
ROPE_DIM = 64


@dataclass
class Workload:
    name: str
    B: int
    q_len: int
    H: int
    ctx: list            # context length per request
    topk: int            # 0 = dense
    q_dtype: str = "bf16"
    append_rows: int = 0  # rows quantize-appended per request (mixed serving step)
    split_tokens: int = 4096
    q_lens: list = field(default_factory=list)   # per-request q_len (mixed step), else [q_len]*B

    @property
    def tokens(self) -> int:
        return sum(self.q_lens) if self.q_lens else self.B * self.q_len


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def named_workload(name: str, seed: int = 0) -> Workload:
    """The benchmark configurations by name (sizes in tokens, see module docstring)."""
    if name == "tiny":
        return Workload("tiny", B=1, q_len=1, H=16, ctx=[4096], topk=256, q_dtype="fp32")
    if name == "batched":
        return Workload("batched", B=32, q_len=1, H=64, ctx=[143360] * 32, topk=2048)
    if name == "mtp":
        return Workload("mtp", B=16, q_len=15, H=64, ctx=[149504] * 16, topk=2048)
    if name == "dense":
        return Workload("dense", B=8, q_len=1, H=64, ctx=[149504] * 8, topk=0)
    if name == "pages":
        return Workload("pages", B=1, q_len=15, H=16, ctx=[149504], topk=2048)
    if name == "mixed":
        g = torch.Generator().manual_seed(1000 + 4 + seed)
        u = torch.rand(64, generator=g, dtype=torch.float64)
        ctx = [int(round(math.exp(math.log(4096) + float(x) * (math.log(204800) - math.log(4096)))))
               for x in u]
        qls = [1 if float(x) < 0.5 else 15 for x in torch.rand(64, generator=g, dtype=torch.float64)]
        return Workload("mixed", B=64, q_len=15, H=64, ctx=ctx, topk=2048, append_rows=6144,
                        q_lens=qls)
    raise KeyError(name)


def gen_latent_rope(n_rows: int, seed: int, device="cpu"):
    """latent bf16 [n,512] and rope bf16 [n,64], both ~N(0,1)."""
    g = _gen(seed, device)
    lat = torch.randn(n_rows, LATENT_DIM, generator=g, device=device, dtype=torch.float32)
    rope = torch.randn(n_rows, ROPE_DIM, generator=g, device=device, dtype=torch.float32)
    return lat.to(torch.bfloat16), rope.to(torch.bfloat16)


def gen_queries(B: int, q_len: int, H: int, dtype: str, seed: int, device="cpu"):
    """Absorbed queries [B, q_len, H, 576] ~N(0,1), bf16 or fp32."""
    g = _gen(seed, device)
    q = torch.randn(B, q_len, H, LATENT_DIM + ROPE_DIM, generator=g, device=device,
                    dtype=torch.float32)
    return q if dtype == "fp32" else q.to(torch.bfloat16)


def pages_for(ctx: int) -> int:
    return (ctx + PAGE_ROWS - 1) // PAGE_ROWS


def gen_block_table(ctx: list, seed: int, device="cpu", spare_pages: int = 0):
    """Random page assignment: a permutation of all physical pages, sliced per request.

    Returns (block_table int32 [B, max_pages] padded with 0, total physical pages). The table is
    built on the host and moved to ``device`` with one copy.
    """
    g = _gen(seed, "cpu")
    need = [pages_for(c) for c in ctx]
    total = sum(need) + spare_pages
    perm = torch.randperm(total, generator=g).to(torch.int32)
    max_pages = max(need) if need else 1
    bt = torch.zeros(len(ctx), max_pages, dtype=torch.int32)
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[o:o + n]
        o += n
    return bt.to(device), total


def slot_mapping_for(block_table, b: int, start: int, count: int):
    """Physical slots of logical positions start..start+count-1 of request b (int64)."""
    pos = torch.arange(start, start + count, device=block_table.device, dtype=torch.int64)
    page = block_table[b].to(torch.int64)[pos // PAGE_ROWS]
    return page * PAGE_ROWS + pos % PAGE_ROWS


def gen_topk(B: int, q_len: int, k: int, ctx: list, seed: int, device="cpu", q_lens=None):
    """Top-k lists int32 [B, q_len, k]: k distinct uniform positions in [0, ctx_b) per token.

    Contexts shorter than k list every position once, padded with -1 at random list places.
    Rows of requests with fewer query tokens than q_len (mixed steps) are all -1. The lists are
    drawn on the host and moved to ``device`` with one copy.
    """
    g = _gen(seed, "cpu")
    out = torch.full((B, q_len, k), -1, dtype=torch.int32)
    for b in range(B):
        n_q = q_lens[b] if q_lens else q_len
        c = int(ctx[b])
        for t in range(n_q):
            keys = torch.rand(c, generator=g)
            if c >= k:
                # the k smallest keys in ascending key order (the first k of their argsort)
                out[b, t] = torch.topk(keys, k, largest=False, sorted=True).indices.to(torch.int32)
            else:
                sel = torch.argsort(keys).to(torch.int32)
                place = torch.argsort(torch.rand(k, generator=g))[:c]
                out[b, t, place] = sel
    return out.to(device)


def gen_topk_overlap(B: int, q_len: int, k: int, ctx: list, overlap: float, seed: int, device="cpu"):
    """Top-k lists int32 [B, q_len, k] whose tokens share rows within a request (an overlap
    model of multi-token decode: the query tokens of one request pick mostly the same positions).

    Per request: a base set of k distinct uniform positions in [0, ctx_b). Each token keeps a
    uniform subset of round(overlap * k) base positions and adds k - that many distinct positions
    from outside the base set. Lists are in ascending position order. Requires ctx_b >= 2k.
    Drawn on the host and moved to ``device`` with one copy.
    """
    g = _gen(seed, "cpu")
    keep = int(round(overlap * k))
    out = torch.empty((B, q_len, k), dtype=torch.int32)
    for b in range(B):
        c = int(ctx[b])
        if c < 2 * k:
            raise ValueError("gen_topk_overlap needs ctx >= 2k")
        perm = torch.randperm(c, generator=g)
        base, rest = perm[:k], perm[k:]
        for t in range(q_len):
            sub = base[torch.randperm(k, generator=g)[:keep]]
            fresh = rest[torch.randperm(c - k, generator=g)[:k - keep]]
            out[b, t] = torch.sort(torch.cat([sub, fresh])).values.to(torch.int32)
    return out.to(device)


def gen_topk_batched(B: int, q_len: int, k: int, ctx: int, seed: int, device="cpu"):
    """Same distribution as ``gen_topk`` for a common context >= k, drawn for all tokens at once."""
    g = _gen(seed, device)
    keys = torch.rand(B * q_len, ctx, generator=g, device=device)
    idx = torch.topk(keys, k, dim=1, largest=False, sorted=False).indices
    return idx.to(torch.int32).reshape(B, q_len, k)


INDEXER_HEADS = 64
INDEXER_DIM = 128
INDEXER_PAGE_BYTES = 64 * INDEXER_DIM + 64 * 4


def gen_indexer(n_pages: int, B: int, q_len: int, seed: int, device="cpu"):
    """Synthetic indexer inputs (no trained weights): an indexer cache of ``n_pages`` pages (64
    keys of 128 E4M3 bytes, then 64 fp32 scales, per page), queries of 64 heads x 128 dims as
    E4M3 bytes [B, q_len, 64, 128] and fp32 head weights [B, q_len, 64].

    Keys and queries are N(0, 1) values cast to E4M3 by torch (round to nearest); key scales are
    uniform in [0.5, 1.5); head weights are N(0, 1) / 8. Drawn on the host, moved with one copy
    each. Returns (k_cache uint8 [n_pages * 8448], q_fp8, weights).
    """
    g = _gen(seed, "cpu")
    keys = torch.randn(n_pages * 64, INDEXER_DIM, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    scales = (0.5 + torch.rand(n_pages * 64, generator=g)).to(torch.float32)
    page = torch.empty(n_pages, INDEXER_PAGE_BYTES, dtype=torch.uint8)
    page[:, :64 * INDEXER_DIM] = keys.reshape(n_pages, 64 * INDEXER_DIM)
    page[:, 64 * INDEXER_DIM:] = scales.reshape(n_pages, 64).view(torch.uint8).reshape(n_pages, 256)
    q = torch.randn(B, q_len, INDEXER_HEADS, INDEXER_DIM, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    w = torch.randn(B, q_len, INDEXER_HEADS, generator=g) / 8.0
    return page.reshape(-1).to(device), q.contiguous().to(device), w.contiguous().to(device)

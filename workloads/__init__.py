"""Seeded synthetic inputs for the paged-attention hot path.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``: the one piece
that both the oracle side and the GPU side consume. It draws lengths, tables and
values only; it computes none of the method's results (no page tables, kv_lens,
scores, softmax or merges).

Recipe (one ``torch.Generator`` per case, seeded with the case's seed):
  1. integers on the CPU generator, in this order: lengths, physical placement
     (a ``randperm`` of the page or slot pool, consumed in request order), the
     request -> pool-row map ``req_pool_indices = randperm(2B)[:B]``, extra
     integers (prefill lens, top-k indices);
  2. values q, then k, then v, each ~ N(0, 1), drawn in logical order
     (request, token, head, dim) in float32 and rounded to the storage dtype
     with round-to-nearest-even. With ``value_device`` set to a GPU, the values
     are drawn there by a generator seeded the same way (much faster for the
     multi-GB caches); the integers always come from the CPU generator.
Every cache slot that no request owns, every ``req_to_token`` entry past a
request's length and every unselected pool row point at / hold NaN, so a stray
read shows up as NaN in the output. The poison page is a page of the pool that
no request owns, or one extra page appended to the pool when all are owned.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = [
    "DecodeCase", "PrefillCase", "SwaCase", "SparseCase", "CascadeCase",
    "make_decode_case", "make_prefill_case", "make_swa_case", "make_sparse_case",
    "make_cascade_case", "cascade_verify", "DcaCase", "make_dca_case", "dca_decode",
    "config1", "config2", "config3", "config4", "config5",
    "small_config3", "small_config4", "small_config5",
]


# ---------------------------------------------------------------------------
# Case containers (all tensors; integer tables are int32)
# ---------------------------------------------------------------------------

@dataclass
class DecodeCase:
    q: torch.Tensor                 # [B, Hq, D]
    k_cache: torch.Tensor           # [num_pages, P, Hkv, D]
    v_cache: torch.Tensor           # [num_pages, P, Hkv, D]
    req_to_token: torch.Tensor      # [2B, ctx] int32, token slot ids
    req_pool_indices: torch.Tensor  # [B] int32
    seq_lens: torch.Tensor          # [B] int32
    page_size: int
    scale: float
    kv_chunk: int
    num_splits: int
    table_width: int                # pages per page-table row
    name: str = ""


@dataclass
class PrefillCase:
    q: torch.Tensor                 # [total_q, Hq, D]
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    req_to_token: torch.Tensor
    req_pool_indices: torch.Tensor
    seq_lens: torch.Tensor          # [B] prefix + new (the kv length)
    extend_lens: torch.Tensor       # [B] new tokens
    cu_seqlens_q: torch.Tensor      # [B+1] layout of the ragged q rows
    max_seqlen_q: int
    page_size: int
    scale: float
    table_width: int
    name: str = ""


@dataclass
class SwaCase:
    q: torch.Tensor                 # [B, Hq, D]
    k_cache: torch.Tensor           # [slots, 1, Hkv, D]
    v_cache: torch.Tensor
    req_to_token: torch.Tensor      # [2B, ctx]
    req_pool_indices: torch.Tensor  # [B]
    seq_lens: torch.Tensor          # [B]
    prefill_lens: torch.Tensor      # [2B] pool-sized, indexed by pool row
    window: int
    table_width: int                # min(max prefill + window, max seq_len)
    scale: float
    kv_chunk: int
    num_splits: int
    name: str = ""


@dataclass
class SparseCase:
    q: torch.Tensor                 # [B, Hq, Dqk]
    kv_cache: torch.Tensor          # [slots, Dqk]
    req_to_token: torch.Tensor      # [2B, ctx]
    req_pool_indices: torch.Tensor  # [B]
    topk_idx: torch.Tensor          # [B, K] logical token indices, -1 = padding
    head_dim_v: int
    scale: float
    name: str = ""


@dataclass
class CascadeCase:
    q: torch.Tensor                 # [B*n, Hq, D] draft-token queries, request-major
    k_cache: torch.Tensor           # [num_pages, P, Hkv, D]; committed and draft tokens
    v_cache: torch.Tensor
    req_to_token: torch.Tensor      # [2B, ctx] int32 slots
    req_pool_indices: torch.Tensor  # [B]
    seq_lens: torch.Tensor          # [B] committed tokens L_b (drafts follow at L_b..L_b+n-1)
    custom_mask: torch.Tensor       # flat bool: per request n rows of L_b + n entries
    parents: torch.Tensor           # [B, n] draft tree, -1 = child of the last committed token
    num_draft: int
    page_size: int
    scale: float
    table_width: int                # pages per row of the committed-token page table
    name: str = ""


@dataclass
class DcaCase:
    base: "DecodeCase"              # q (the intra query), caches, tables, lengths
    q_succ: torch.Tensor            # [B, Hq, D] query of the previous chunk's keys
    q_inter: torch.Tensor           # [B, Hq, D] query of all earlier keys
    chunk_size: int
    local_size: int
    original_max_position_embeddings: int
    name: str = ""


# ---------------------------------------------------------------------------
# Helpers (drawing only)
# ---------------------------------------------------------------------------

def _randint_incl(g, lo, hi, n):
    """n integers uniform on [lo, hi], both ends included."""
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64)


def _value_generator(seed, device):
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g, dev


def _normal(g, dev, shape, dtype):
    x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
    return x.to(dtype)


def _place_pages(g, batch, lens, page_size, num_pages, ctx):
    """Assign physical pages in request order from a random permutation.

    Returns (req_to_token [2B, ctx] int64 before poison fill, rpi [B],
    owned page list per request, poison page id, total pages in the pool).
    """
    perm = torch.randperm(num_pages, generator=g)
    need = [-(-int(L) // page_size) for L in lens]
    total_need = sum(need)
    if total_need > num_pages:
        raise ValueError("pool too small for the requested lengths")
    pool_pages = num_pages
    if total_need < num_pages:
        poison = int(perm[-1])
    else:
        poison = num_pages
        pool_pages = num_pages + 1
    rpi = torch.randperm(2 * batch, generator=g)[:batch]
    poison_slot = poison * page_size
    r2t = torch.full((2 * batch, ctx), poison_slot, dtype=torch.int64)
    owned = []
    cursor = 0
    for b in range(batch):
        pages = perm[cursor:cursor + need[b]]
        cursor += need[b]
        owned.append(pages)
        L = int(lens[b])
        if L:
            t = torch.arange(L)
            r2t[int(rpi[b]), :L] = pages[t // page_size] * page_size + t % page_size
    return r2t, rpi, owned, poison, pool_pages


def _fill_cache(vals_per_req, owned, lens, page_size, pool_pages, num_heads, head_dim,
                dtype, dev):
    """Scatter per-request logical values [L, H, D] into a NaN-filled paged cache."""
    cache = torch.full((pool_pages, page_size, num_heads, head_dim), float("nan"),
                       dtype=dtype, device=dev)
    flat = cache.view(pool_pages * page_size, num_heads, head_dim)
    for b, vals in enumerate(vals_per_req):
        L = int(lens[b])
        if L == 0:
            continue
        t = torch.arange(L)
        slots = (owned[b][t // page_size] * page_size + t % page_size).to(dev)
        flat[slots] = vals
    return cache


def _draw_kv(gv, dev, lens, num_kv_heads, head_dim, dtype):
    total = int(sum(int(L) for L in lens))
    k_all = _normal(gv, dev, (total, num_kv_heads, head_dim), dtype)
    v_all = _normal(gv, dev, (total, num_kv_heads, head_dim), dtype)
    k_parts, v_parts, o = [], [], 0
    for L in lens:
        k_parts.append(k_all[o:o + int(L)])
        v_parts.append(v_all[o:o + int(L)])
        o += int(L)
    return k_parts, v_parts


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

def make_decode_case(seed, *, seq_lens, num_q_heads, num_kv_heads, head_dim, page_size,
                     num_pages, dtype=torch.bfloat16, kv_chunk=0, ctx=None,
                     value_device="cpu", with_values=True, name="") -> DecodeCase:
    """Paged GQA decode: one query token per request over ``seq_lens`` keys.

    ``seq_lens`` is either an explicit list or a ``(batch, lo, hi)`` tuple for
    lengths uniform on ``[lo, hi]``.
    """
    g = torch.Generator().manual_seed(seed)
    if isinstance(seq_lens, tuple):
        batch, lo, hi = seq_lens
        lens = _randint_incl(g, lo, hi, batch)
    else:
        lens = torch.tensor(list(seq_lens), dtype=torch.int64)
    batch = len(lens)
    max_len = int(lens.max()) if batch else 0
    if ctx is None:
        ctx = max(max_len, 1)
    ctx = -(-ctx // page_size) * page_size
    r2t, rpi, owned, _poison, pool_pages = _place_pages(g, batch, lens, page_size, num_pages, ctx)
    q = k_cache = v_cache = None
    if with_values:
        gv, dev = _value_generator(seed, value_device)
        q = _normal(gv, dev, (batch, num_q_heads, head_dim), dtype)
        k_parts, v_parts = _draw_kv(gv, dev, lens, num_kv_heads, head_dim, dtype)
        k_cache = _fill_cache(k_parts, owned, lens, page_size, pool_pages, num_kv_heads,
                              head_dim, dtype, dev)
        del k_parts
        v_cache = _fill_cache(v_parts, owned, lens, page_size, pool_pages, num_kv_heads,
                              head_dim, dtype, dev)
        del v_parts
    if kv_chunk:
        num_splits = max(1, -(-max_len // kv_chunk))
    else:
        num_splits = 1
    return DecodeCase(q=q, k_cache=k_cache, v_cache=v_cache,
                      req_to_token=r2t.to(torch.int32), req_pool_indices=rpi.to(torch.int32),
                      seq_lens=lens.to(torch.int32), page_size=page_size,
                      scale=1.0 / math.sqrt(head_dim), kv_chunk=kv_chunk,
                      num_splits=num_splits, table_width=ctx // page_size, name=name)


def make_prefill_case(seed, *, prefix_lens, extend_lens, num_q_heads, num_kv_heads,
                      head_dim, page_size, num_pages, dtype=torch.bfloat16, ctx=None,
                      value_device="cpu", name="") -> PrefillCase:
    """Varlen causal extend: request b has ``prefix_lens[b]`` cached tokens and
    ``extend_lens[b]`` new ones, all already resident in the paged cache."""
    g = torch.Generator().manual_seed(seed)
    prefix = torch.tensor(list(prefix_lens), dtype=torch.int64)
    extend = torch.tensor(list(extend_lens), dtype=torch.int64)
    lens = prefix + extend
    batch = len(lens)
    max_len = int(lens.max()) if batch else 0
    if ctx is None:
        ctx = max(max_len, 1)
    ctx = -(-ctx // page_size) * page_size
    r2t, rpi, owned, _poison, pool_pages = _place_pages(g, batch, lens, page_size, num_pages, ctx)
    gv, dev = _value_generator(seed, value_device)
    total_q = int(extend.sum())
    q = _normal(gv, dev, (total_q, num_q_heads, head_dim), dtype)
    k_parts, v_parts = _draw_kv(gv, dev, lens, num_kv_heads, head_dim, dtype)
    k_cache = _fill_cache(k_parts, owned, lens, page_size, pool_pages, num_kv_heads,
                          head_dim, dtype, dev)
    v_cache = _fill_cache(v_parts, owned, lens, page_size, pool_pages, num_kv_heads,
                          head_dim, dtype, dev)
    cu_q = torch.zeros(batch + 1, dtype=torch.int64)
    cu_q[1:] = torch.cumsum(extend, 0)
    return PrefillCase(q=q, k_cache=k_cache, v_cache=v_cache,
                       req_to_token=r2t.to(torch.int32), req_pool_indices=rpi.to(torch.int32),
                       seq_lens=lens.to(torch.int32), extend_lens=extend.to(torch.int32),
                       cu_seqlens_q=cu_q.to(torch.int32),
                       max_seqlen_q=int(extend.max()) if batch else 0,
                       page_size=page_size, scale=1.0 / math.sqrt(head_dim),
                       table_width=ctx // page_size, name=name)


def make_cascade_case(seed, *, prefix_lens, num_draft, num_q_heads, num_kv_heads, head_dim,
                      page_size, num_pages, tree="random", dtype=torch.bfloat16,
                      value_device="cpu", name="") -> CascadeCase:
    """Speculative verification of a draft tree: request b has ``L_b`` committed
    tokens and ``n = num_draft`` draft tokens at positions ``L_b .. L_b+n-1``,
    all resident in the paged cache. ``prefix_lens`` is a list or a
    ``(batch, lo, hi)`` tuple (uniform, inclusive). The tree: draft 0 hangs off
    the last committed token, draft ``j > 0`` off a parent drawn uniformly from
    ``0 .. j-1`` (``tree="random"``), or off ``j-1`` (``"chain"``). A draft row
    sees every committed position, itself and its ancestors (the custom mask of
    a tree-structured verify step).
    """
    g = torch.Generator().manual_seed(seed)
    if isinstance(prefix_lens, tuple):
        batch, lo, hi = prefix_lens
        prefix = _randint_incl(g, lo, hi, batch)
    else:
        prefix = torch.tensor(list(prefix_lens), dtype=torch.int64)
    n = int(num_draft)
    lens = prefix + n
    batch = len(lens)
    ctx = -(-int(lens.max()) // page_size) * page_size
    r2t, rpi, owned, _poison, pool_pages = _place_pages(g, batch, lens, page_size, num_pages, ctx)
    parents = torch.full((batch, n), -1, dtype=torch.int64)
    for b in range(batch):
        for j in range(1, n):
            if tree == "chain":
                parents[b, j] = j - 1
            else:
                parents[b, j] = int(torch.randint(0, j, (1,), generator=g))
    blocks = []
    for b in range(batch):
        L = int(prefix[b])
        rows = torch.zeros((n, L + n), dtype=torch.bool)
        rows[:, :L] = True
        for i in range(n):
            a = i
            while a >= 0:
                rows[i, L + a] = True
                a = int(parents[b, a])
        blocks.append(rows.reshape(-1))
    mask = torch.cat(blocks) if blocks else torch.zeros(0, dtype=torch.bool)
    gv, dev = _value_generator(seed, value_device)
    q = _normal(gv, dev, (batch * n, num_q_heads, head_dim), dtype)
    k_parts, v_parts = _draw_kv(gv, dev, lens, num_kv_heads, head_dim, dtype)
    k_cache = _fill_cache(k_parts, owned, lens, page_size, pool_pages, num_kv_heads, head_dim,
                          dtype, dev)
    v_cache = _fill_cache(v_parts, owned, lens, page_size, pool_pages, num_kv_heads, head_dim,
                          dtype, dev)
    return CascadeCase(q=q, k_cache=k_cache, v_cache=v_cache, req_to_token=r2t.to(torch.int32),
                       req_pool_indices=rpi.to(torch.int32), seq_lens=prefix.to(torch.int32),
                       custom_mask=mask, parents=parents.to(torch.int32), num_draft=n,
                       page_size=page_size, scale=1.0 / math.sqrt(head_dim),
                       table_width=ctx // page_size, name=name)


def make_swa_case(seed, *, batch, prefill_range, decode_range, window, num_q_heads,
                  num_kv_heads, head_dim, pool_slots, dtype=torch.bfloat16, kv_chunk=0,
                  value_device="cpu", with_values=True, name="") -> SwaCase:
    """Decode over a prefill-aware sliding-window table (token-level, page size 1).

    ``prefill_len ~ U[prefill_range]`` and ``seq_len = prefill_len + U[decode_range]``.
    Every token of every request holds values (the table builder decides which
    ones are read).
    """
    g = torch.Generator().manual_seed(seed)
    pf = _randint_incl(g, prefill_range[0], prefill_range[1], batch)
    lens = pf + _randint_incl(g, decode_range[0], decode_range[1], batch)
    ctx = int(lens.max())
    r2t, rpi, owned, _poison, pool_pages = _place_pages(g, batch, lens, 1, pool_slots, ctx)
    prefill_pool = _randint_incl(g, 0, 7, 2 * batch)   # rows no request uses: junk
    prefill_pool[rpi] = pf
    q = k_cache = v_cache = None
    if with_values:
        gv, dev = _value_generator(seed, value_device)
        q = _normal(gv, dev, (batch, num_q_heads, head_dim), dtype)
        k_parts, v_parts = _draw_kv(gv, dev, lens, num_kv_heads, head_dim, dtype)
        k_cache = _fill_cache(k_parts, owned, lens, 1, pool_pages, num_kv_heads, head_dim, dtype,
                              dev)
        del k_parts
        v_cache = _fill_cache(v_parts, owned, lens, 1, pool_pages, num_kv_heads, head_dim, dtype,
                              dev)
        del v_parts
    width = min(int(pf.max()) + window, int(lens.max()))
    num_splits = max(1, -(-width // kv_chunk)) if kv_chunk else 1
    return SwaCase(q=q, k_cache=k_cache, v_cache=v_cache, req_to_token=r2t.to(torch.int32),
                   req_pool_indices=rpi.to(torch.int32), seq_lens=lens.to(torch.int32),
                   prefill_lens=prefill_pool.to(torch.int32), window=window,
                   table_width=width, scale=1.0 / math.sqrt(head_dim), kv_chunk=kv_chunk,
                   num_splits=num_splits, name=name)


def make_sparse_case(seed, *, batch, ctx, topk, num_q_heads, head_dim_qk, head_dim_v,
                     num_pad=0, dtype=torch.bfloat16, value_device="cpu",
                     name="") -> SparseCase:
    """Top-k sparse MLA decode: one latent KV head of width ``head_dim_qk``.

    Token table: ``randperm(batch * ctx)`` viewed ``[batch, ctx]`` into the
    selected pool rows, plus one appended poison slot. Top-k indices:
    ``randperm(ctx)[:topk]`` per request (unsorted, unique); the last
    ``num_pad`` entries of each row are replaced by -1. Only the slots that
    some top-k entry names hold values; all others are NaN.
    """
    g = torch.Generator().manual_seed(seed)
    n_slots = batch * ctx
    poison = n_slots
    perm = torch.randperm(n_slots, generator=g).view(batch, ctx)
    rpi = torch.randperm(2 * batch, generator=g)[:batch]
    r2t = torch.full((2 * batch, ctx), poison, dtype=torch.int64)
    r2t[rpi] = perm
    idx = torch.stack([torch.randperm(ctx, generator=g)[:topk] for _ in range(batch)])
    if num_pad:
        idx[:, topk - num_pad:] = -1
    gv, dev = _value_generator(seed, value_device)
    q = _normal(gv, dev, (batch, num_q_heads, head_dim_qk), dtype)
    kv = torch.full((n_slots + 1, head_dim_qk), float("nan"), dtype=dtype, device=dev)
    valid = idx >= 0
    touched = perm.gather(1, idx.clamp(min=0))[valid]
    kv[touched.to(dev)] = _normal(gv, dev, (int(touched.numel()), head_dim_qk), dtype)
    return SparseCase(q=q, kv_cache=kv, req_to_token=r2t.to(torch.int32),
                      req_pool_indices=rpi.to(torch.int32), topk_idx=idx.to(torch.int32),
                      head_dim_v=head_dim_v, scale=1.0 / math.sqrt(head_dim_qk), name=name)


# ---------------------------------------------------------------------------
# The five workloads at full size, and reduced copies the oracle finishes fast
# ---------------------------------------------------------------------------

def cascade_verify(value_device="cpu"):
    """Tree verification by cascade attention, bf16: B 64, committed L ~
    U[1024, 16384], 8 draft tokens per request in a random tree, 32 q / 8 kv
    heads, D 128, page 64 over a 20000-page pool."""
    return make_cascade_case(6, prefix_lens=(64, 1024, 16384), num_draft=8, num_q_heads=32,
                             num_kv_heads=8, head_dim=128, page_size=64, num_pages=20000,
                             value_device=value_device, name="cascade_verify")


def make_dca_case(seed, *, seq_lens, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                  chunk_size, local_size, original_max_position_embeddings=0,
                  dtype=torch.bfloat16, kv_chunk=0, ctx=None, value_device="cpu",
                  name="") -> DcaCase:
    """Dual chunk attention decode: a decode case (its q is the intra query)
    plus the succ and inter queries, N(0, 1), drawn after it from a generator
    seeded with seed + 1 (on ``value_device``). The three queries stand for
    the model's three rotary projections of one token."""
    base = make_decode_case(seed, seq_lens=seq_lens, num_q_heads=num_q_heads,
                            num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                            num_pages=num_pages, dtype=dtype, kv_chunk=kv_chunk, ctx=ctx,
                            value_device=value_device, name=name)
    gv, dev = _value_generator(seed + 1, value_device)
    shape = tuple(base.q.shape)
    q_succ = _normal(gv, dev, shape, dtype)
    q_inter = _normal(gv, dev, shape, dtype)
    return DcaCase(base=base, q_succ=q_succ, q_inter=q_inter, chunk_size=chunk_size,
                   local_size=local_size,
                   original_max_position_embeddings=original_max_position_embeddings, name=name)


def dca_decode(value_device="cpu"):
    """Dual chunk attention decode, bf16: B 32, L ~ U[4096, 65536], 32 q / 8 kv
    heads, D 128, page 64 over a 40000-page pool; chunk_size 8192, local_size
    1024 (chunks of 7168 keys, one split each); queries scaled against
    original_max_position_embeddings 32768."""
    return make_dca_case(7, seq_lens=(32, 4096, 65536), num_q_heads=32, num_kv_heads=8,
                         head_dim=128, page_size=64, num_pages=40000, chunk_size=8192,
                         local_size=1024, original_max_position_embeddings=32768,
                         kv_chunk=7168, ctx=65536, value_device=value_device, name="dca_decode")


def config1(value_device="cpu"):
    """Tiny paged GQA decode, fp32: seq_lens [37, 100], 4 q / 2 kv heads, D 64,
    page 16 over a 16-page pool, one query token, 2-way KV split (chunk 64)."""
    return make_decode_case(1, seq_lens=[37, 100], num_q_heads=4, num_kv_heads=2,
                            head_dim=64, page_size=16, num_pages=16, dtype=torch.float32,
                            kv_chunk=64, value_device=value_device, name="config1")


def config2(value_device="cpu"):
    """Varlen causal extend, bf16: prefix [0,128,512,1000], new [256,64,512,17],
    32 q / 8 kv heads, D 128, page 1 over an 8192-slot pool."""
    return make_prefill_case(2, prefix_lens=[0, 128, 512, 1000], extend_lens=[256, 64, 512, 17],
                             num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=1,
                             num_pages=8192, value_device=value_device, name="config2")


def config3(value_device="cpu", with_values=True):
    """Batched split-KV GQA decode, bf16: B 64, L ~ U[1024, 32768], 32 q / 8 kv
    heads, D 128, page 64 over a 40000-page pool, chunks of 4096 tokens."""
    return make_decode_case(3, seq_lens=(64, 1024, 32768), num_q_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=64, num_pages=40000, kv_chunk=4096,
                            ctx=32768, value_device=value_device, with_values=with_values,
                            name="config3")


def config4(value_device="cpu", kv_chunk=1536, with_values=True):
    """Sliding-window decode over the prefill-aware table, bf16: B 32,
    prefill ~ U[2048, 8192], seq = prefill + U[1, 8192], window 4096,
    64 q / 8 kv heads, D 128, page 1 over 32*16384 slots."""
    return make_swa_case(4, batch=32, prefill_range=(2048, 8192), decode_range=(1, 8192),
                         window=4096, num_q_heads=64, num_kv_heads=8, head_dim=128,
                         pool_slots=32 * 16384, kv_chunk=kv_chunk,
                         value_device=value_device, with_values=with_values, name="config4")


def config5(value_device="cpu", num_pad=0):
    """Top-k sparse MLA decode, bf16: B 32, context 65536, top-k 2048, 128 q
    heads, Dqk 576 (512 latent + 64 rope), Dv 512."""
    return make_sparse_case(5, batch=32, ctx=65536, topk=2048, num_q_heads=128,
                            head_dim_qk=576, head_dim_v=512, num_pad=num_pad,
                            value_device=value_device, name="config5")


def long_prompt_prefill(value_device="cpu"):
    """Causal prefill of long prompts, bf16: 4 requests x 4096 new tokens, no
    cached prefix, 32 q / 8 kv heads, D 128, page 1 (steady-state throughput
    of the extend kernel, next to config2's small mixed batch)."""
    n = 4096
    return make_prefill_case(11, prefix_lens=[0] * 4, extend_lens=[n] * 4, num_q_heads=32,
                             num_kv_heads=8, head_dim=128, page_size=1, num_pages=4 * n + 64,
                             value_device=value_device, name="long_prompt_prefill")


def small_config3(seed=13, value_device="cpu"):
    """config3's shapes and layout with short sequences (several chunks, ragged tails)."""
    return make_decode_case(seed, seq_lens=(6, 1, 700), num_q_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=64, num_pages=200, kv_chunk=256,
                            ctx=768, value_device=value_device, name="small_config3")


def small_config4(seed=14, value_device="cpu"):
    """config4's structure (prefill-aware window table, page 1) at reduced lengths."""
    return make_swa_case(seed, batch=5, prefill_range=(20, 300), decode_range=(1, 400),
                         window=128, num_q_heads=64, num_kv_heads=8, head_dim=128,
                         pool_slots=5 * 800, kv_chunk=128, value_device=value_device,
                         name="small_config4")


def small_config5(seed=15, value_device="cpu", num_pad=0):
    """config5's widths (576 / 512, 128 heads) with a short context and top-k."""
    return make_sparse_case(seed, batch=3, ctx=1000, topk=300, num_q_heads=128,
                            head_dim_qk=576, head_dim_v=512, num_pad=num_pad,
                            value_device=value_device, name="small_config5")

"""Sliding window (W, 0) and chunked local attention in the prefill and decode
kernels on the GPU versus the oracle.

Both masks only narrow a causal row from below: the row at position p sees
keys [max(0, p - W), p] under a window of W, or [floor(p / C) * C, p] under
local chunks of C. The cases put the lower bound on and off tile, page and
split boundaries, make whole key splits empty, and cover the kernels'
variants (uniform and per-token pages, grouped and general decode, fp32).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_197_amd as pkv
import workloads
from helpers import LSE_TOL, O_TOL, assert_close, compact_pages, np_f, np_i, say, to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _table(c):
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                                     c.table_width)
    return pt, kl


def check_prefill(c, window_left=-1, attn_chunk=0):
    pt, kl = _table(c)
    out = torch.full_like(c.q, float("nan"))
    lse = torch.full(c.q.shape[:2], float("nan"), device=DEV)
    pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                  c.max_seqlen_q, c.scale, window_left=window_left,
                                  attn_chunk=attn_chunk, out=out, lse=lse)
    torch.cuda.synchronize()
    pt_np, kl_np = np_i(pt), np_i(kl)
    rows = list(range(len(kl_np)))
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, c.page_size, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, c.page_size, rows)
    ro, rl = oracle.paged_prefill(np_f(c.q), k_small, v_small, pt_small, np_i(c.cu_seqlens_q),
                                  kl_np, c.page_size, c.scale, causal=True,
                                  window_left=window_left, attn_chunk=attn_chunk)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


# short prefixes: one key split per q tile; the bound falls inside the first
# tiles, exactly on tile starts (32, 64) and below key 0 (W larger than p)
@pytest.mark.parametrize("D,P,group,window_left,attn_chunk", [
    (128, 1, 4, 0, 0), (128, 1, 4, 1, 0), (128, 16, 2, 31, 0), (128, 1, 8, 32, 0),
    (64, 32, 4, 63, 0), (64, 3, 16, 100, 0), (128, 64, 1, 4096, 0),
    (128, 1, 4, -1, 1), (128, 16, 2, -1, 16), (64, 1, 8, -1, 32), (128, 7, 4, -1, 100),
    (64, 64, 2, -1, 64),
])
def test_prefill_window_shapes(D, P, group, window_left, attn_chunk):
    hkv = 2
    prefix = [0, 0, 1, 31, 5, 64, 100, 7]
    extend = [1, 33, 1, 32, 0, 65, 3, 140]
    total = sum(p + e for p, e in zip(prefix, extend))
    c = workloads.make_prefill_case(300 + D + P + group + window_left + attn_chunk,
                                    prefix_lens=prefix, extend_lens=extend,
                                    num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=D,
                                    page_size=P, num_pages=total // P + len(prefix) + 4)
    c = to_device(c, DEV)
    say(f"prefill window D={D} P={P} G={group} W={window_left} C={attn_chunk}")
    check_prefill(c, window_left, attn_chunk)


# long cached prefixes: q tiles cut into key splits; the window's first tile
# moves the split grid, rows of one tile span a tile boundary of the bound, and
# local chunks start mid-prompt
@pytest.mark.parametrize("D,P,group,window_left,attn_chunk", [
    (128, 1, 4, 1024, 0), (128, 16, 8, 2047, 0), (64, 1, 2, 3000, 0), (128, 64, 4, 100, 0),
    (128, 1, 4, -1, 2048), (64, 16, 4, -1, 1000), (128, 64, 2, -1, 8192),
])
def test_prefill_window_key_splits(D, P, group, window_left, attn_chunk):
    hkv = 2
    prefix = [2000, 0, 777, 3100]
    extend = [300, 1, 129, 45]
    total = sum(p + e for p, e in zip(prefix, extend))
    c = workloads.make_prefill_case(400 + D + P + group + window_left + attn_chunk,
                                    prefix_lens=prefix, extend_lens=extend,
                                    num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=D,
                                    page_size=P, num_pages=total // P + len(prefix) + 4)
    c = to_device(c, DEV)
    need = pkv.paged_attn_varlen_prefill_workspace_size(
        len(prefix), c.q.shape[0], c.max_seqlen_q, c.table_width * P, c.q.shape[1], hkv, D)
    assert need > 0, "case meant to exercise key splits"
    say(f"prefill window splits D={D} P={P} G={group} W={window_left} C={attn_chunk}")
    check_prefill(c, window_left, attn_chunk)


def test_prefill_window_zero_is_diagonal():
    """W = 0 leaves each row its own key: O is V at the row's position, LSE is
    the scaled self score (a closed form, independent of the oracle)."""
    prefix, extend = [3, 40], [37, 90]
    c = workloads.make_prefill_case(451, prefix_lens=prefix, extend_lens=extend, num_q_heads=8,
                                    num_kv_heads=2, head_dim=128, page_size=1,
                                    num_pages=sum(prefix) + sum(extend) + 8)
    c = to_device(c, DEV)
    pt, kl = _table(c)
    say("prefill window 0 diagonal")
    out, lse = pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                             c.max_seqlen_q, c.scale, window_left=0)
    torch.cuda.synchronize()
    cu, kls = np_i(c.cu_seqlens_q), np_i(kl)
    q, k, v = np_f(c.q), np_f(c.k_cache), np_f(c.v_cache)
    pt_np = np_i(pt)
    exp_o = np.zeros_like(q)
    exp_l = np.zeros(q.shape[:2])
    for b in range(len(kls)):
        m = cu[b + 1] - cu[b]
        for j in range(m):
            pos = kls[b] - m + j
            page = pt_np[b, pos]   # page size 1
            for h in range(q.shape[1]):
                kv = h // 4
                exp_o[cu[b] + j, h] = v[page, 0, kv]
                exp_l[cu[b] + j, h] = c.scale * float(q[cu[b] + j, h] @ k[page, 0, kv])
    assert_close("out", np_f(out), exp_o, O_TOL)
    assert_close("lse", np_f(lse), exp_l, LSE_TOL)


def test_prefill_local_chunks_match_virtual_batches():
    """Chunked local attention equals plain causal attention over the virtual
    batches (each aligned block of a request as its own request), both on the
    GPU: the windowed kernel against the unmasked one."""
    C = 96
    prefix, extend = [0, 200, 50, 1000], [300, 17, 190, 5]
    c = workloads.make_prefill_case(461, prefix_lens=prefix, extend_lens=extend, num_q_heads=16,
                                    num_kv_heads=4, head_dim=128, page_size=16,
                                    num_pages=(sum(prefix) + sum(extend)) // 16 + 12)
    c = to_device(c, DEV)
    pt, kl = _table(c)
    say(f"prefill local chunks {C} vs virtual batches")
    out, lse = pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                             c.max_seqlen_q, c.scale, attn_chunk=C)
    # virtual batches with token-level tables (page size 1 view of the same cache)
    P = c.page_size
    pt_np, kl_np, cu = np_i(pt), np_i(kl), np_i(c.cu_seqlens_q)
    vb = oracle.local_attention_virtual_batches(C, cu, kl_np)
    width = max(n for (_, _, _, _, n) in vb)
    tok = np.zeros((len(vb), width), dtype=np.int64)
    q_rows, cu_v, kl_v = [], [0], []
    for i, (b, q0, mq, k0, n) in enumerate(vb):
        pos = np.arange(k0, k0 + n)
        tok[i, :n] = pt_np[b, pos // P] * P + pos % P
        q_rows.extend(range(q0, q0 + mq))
        cu_v.append(cu_v[-1] + mq)
        kl_v.append(n)
    assert q_rows == list(range(c.q.shape[0]))
    k1 = c.k_cache.reshape(-1, 1, *c.k_cache.shape[2:])
    v1 = c.v_cache.reshape(-1, 1, *c.v_cache.shape[2:])
    pt_v = torch.as_tensor(tok, dtype=torch.int32, device=DEV)
    ref_o, ref_l = pkv.paged_attn_varlen_prefill(
        c.q, k1, v1, pt_v, torch.as_tensor(cu_v, dtype=torch.int32, device=DEV),
        torch.as_tensor(kl_v, dtype=torch.int32, device=DEV), max(np.diff(cu_v)), c.scale)
    torch.cuda.synchronize()
    assert_close("out", np_f(out), np_f(ref_o), O_TOL)
    assert_close("lse", np_f(lse), np_f(ref_l), LSE_TOL)


def check_decode(c, chunk, S, window_left=-1, attn_chunk=0, fp32=False):
    pt, kl = _table(c)
    B, H, D = c.q.shape
    o_tol = 1e-5 if fp32 else O_TOL
    l_tol = 1e-5 if fp32 else LSE_TOL
    pt_np, kl_np = np_i(pt), np_i(kl)
    rows = list(range(B))
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, c.page_size, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, c.page_size, rows)
    ro, rl = oracle.paged_decode_splitkv(np_f(c.q), k_small, v_small, pt_small, kl_np,
                                         c.page_size, c.scale, chunk, S,
                                         window_left=window_left, attn_chunk=attn_chunk)
    if S == 1:
        out = torch.full_like(c.q, float("nan"))
        lse = torch.full((B, H), float("nan"), device=DEV)
        pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale, kv_chunk=chunk,
                                      num_splits=1, window_left=window_left,
                                      attn_chunk=attn_chunk, out=out, lse=lse)
        torch.cuda.synchronize()
        assert_close("out", np_f(out), ro[0], o_tol)
        assert_close("lse", np_f(lse), rl[0], l_tol)
        return
    op = torch.full((S, B, H, D), float("nan"), device=DEV)
    lp = torch.full((S, B, H), float("nan"), device=DEV)
    pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale, kv_chunk=chunk,
                                  num_splits=S, window_left=window_left, attn_chunk=attn_chunk,
                                  o_partial=op, lse_partial=lp)
    torch.cuda.synchronize()
    assert not torch.isnan(op).any() and not torch.isnan(lp).any(), "unwritten partials"
    assert_close("o_partial", np_f(op), ro, o_tol if fp32 else 1e-2)
    assert_close("lse_partial", np_f(lp), rl, l_tol)
    out, lse = pkv.merge_state(op, lp, out_dtype=c.q.dtype)
    torch.cuda.synchronize()
    mo, ml = oracle.merge_state(ro, rl)
    assert_close("merged out", np_f(out), mo, o_tol)
    assert_close("merged lse", np_f(lse), ml, l_tol)


# lengths put L - 1 - W and the chunk start before, on and after tile (16/32),
# page and split boundaries; W >= L keeps every key; small W empties splits
SEQS = [1, 2, 16, 17, 32, 33, 64, 100, 257, 511, 512, 513, 1000, 2049]


@pytest.mark.parametrize("D,P,hq,hkv,dtype,chunk,S,window_left,attn_chunk", [
    # grouped kernel (bf16), uniform pages and per-token pages
    (128, 64, 32, 8, torch.bfloat16, 512, 5, 300, 0),
    (128, 16, 16, 8, torch.bfloat16, 256, 9, 0, 0),
    (128, 1, 32, 8, torch.bfloat16, 0, 1, 47, 0),
    (64, 32, 16, 4, torch.bfloat16, 128, 17, 1, 0),
    (128, 3, 32, 4, torch.bfloat16, 384, 6, 5000, 0),
    (128, 64, 32, 8, torch.bfloat16, 512, 5, -1, 200),
    (128, 1, 16, 8, torch.bfloat16, 0, 1, -1, 64),
    (64, 16, 16, 4, torch.bfloat16, 256, 9, -1, 1),
    # general kernel: 16 q heads per kv head, and fp32
    (128, 64, 32, 2, torch.bfloat16, 512, 5, 700, 0),
    (128, 7, 16, 1, torch.bfloat16, 448, 5, -1, 333),
    (64, 16, 8, 2, torch.float32, 256, 9, 129, 0),
    (128, 1, 4, 2, torch.float32, 0, 1, -1, 100),
])
def test_decode_window(D, P, hq, hkv, dtype, chunk, S, window_left, attn_chunk):
    ctx = max(SEQS)
    pages = sum(-(-s // P) for s in SEQS) + 8
    c = workloads.make_decode_case(500 + D + P + hq + S + max(window_left, 0) + attn_chunk,
                                   seq_lens=SEQS, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                                   page_size=P, num_pages=pages, dtype=dtype, kv_chunk=chunk,
                                   ctx=ctx)
    c = to_device(c, DEV)
    say(f"decode window D={D} P={P} Hq={hq} Hkv={hkv} {dtype} chunk={chunk} S={S} "
        f"W={window_left} C={attn_chunk}")
    check_decode(c, chunk, S, window_left, attn_chunk, fp32=(dtype == torch.float32))


def test_decode_window_config3_sampled():
    """The batched decode workload (B 64, L up to 32768, page 64, chunks of
    4096) under a 4096-token window: sampled requests, every split."""
    c = to_device(workloads.config3(value_device=DEV), DEV)
    W = 4096
    S = c.num_splits
    pt, kl = _table(c)
    say(f"config3 window {W} S={S}")
    B, H, D = c.q.shape
    op = torch.full((S, B, H, D), float("nan"), device=DEV)
    lp = torch.full((S, B, H), float("nan"), device=DEV)
    pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale,
                                  kv_chunk=c.kv_chunk, num_splits=S, window_left=W,
                                  o_partial=op, lse_partial=lp)
    torch.cuda.synchronize()
    pt_np, kl_np = np_i(pt), np_i(kl)
    rows = [0, 7, 31, 63]
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, c.page_size, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, c.page_size, rows)
    ro, rl = oracle.paged_decode_splitkv(np_f(c.q[rows]), k_small, v_small, pt_small,
                                         kl_np[rows], c.page_size, c.scale, c.kv_chunk, S,
                                         window_left=W)
    assert_close("o_partial", np_f(op)[:, rows], ro, 1e-2)
    assert_close("lse_partial", np_f(lp)[:, rows], rl, LSE_TOL)

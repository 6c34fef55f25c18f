"""The entry points under HIP graph capture: every call is stream-ordered,
allocates nothing and never synchronises, so a whole step can be captured
once and replayed. Each replay is checked against the eager result, with
eager work and synchronisations in between (the workspaces' counters must be
back at zero after every replay for the next one to be right)."""

import pytest
import torch

import paged_kv_cache_197_amd as pkv
import workloads
from helpers import say, to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _replay_and_check(step, outs, n=4):
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()                          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for i in range(n):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        del junk


def test_decode_step_graph():
    c = to_device(workloads.small_config3(value_device=DEV), DEV)
    B, hq, d = c.q.shape
    S = c.num_splits
    pt = torch.empty((B, c.table_width), dtype=torch.int32, device=DEV)
    kl = torch.empty((B,), dtype=torch.int32, device=DEV)
    op = torch.empty((S, B, hq, d), dtype=torch.float32, device=DEV)
    lp = torch.empty((S, B, hq), dtype=torch.float32, device=DEV)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)

    def step():
        pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                             c.table_width, page_table=pt, kv_lens=kl, with_cu_seqlens=False)
        pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale,
                                      kv_chunk=c.kv_chunk, num_splits=S, o_partial=op,
                                      lse_partial=lp)
        pkv.merge_state(op, lp, out=out, lse_out=lse)

    say("graph: page table + decode + merge")
    step()
    _replay_and_check(step, [out, lse])


def test_prefill_with_key_splits_graph():
    prefix, extend = [2000, 0, 777], [300, 1, 129]
    c = to_device(workloads.make_prefill_case(141, prefix_lens=prefix, extend_lens=extend,
                                              num_q_heads=16, num_kv_heads=2, head_dim=128,
                                              page_size=16, num_pages=(sum(prefix) + sum(extend))
                                              // 16 + 8), DEV)
    B = len(prefix)
    need = pkv.paged_attn_varlen_prefill_workspace_size(B, c.q.shape[0], c.max_seqlen_q,
                                                        c.table_width * 16, 16, 2, 128)
    assert need > 0, "meant to split"
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, 16,
                                     c.table_width)
    out = torch.empty_like(c.q)
    lse = torch.empty(c.q.shape[:2], dtype=torch.float32, device=DEV)

    def step():
        pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                      c.max_seqlen_q, c.scale, workspace=ws, out=out, lse=lse)

    say("graph: prefill with key splits")
    step()
    _replay_and_check(step, [out, lse])


def test_sparse_graph():
    s = to_device(workloads.small_config5(value_device=DEV), DEV)
    B, hq, _ = s.q.shape
    topk = s.topk_idx.shape[1]
    need = pkv.sparse_topk_decode_workspace_size(B, topk, hq, s.head_dim_v)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, hq, s.head_dim_v), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)

    def step():
        pkv.sparse_topk_decode(s.q, s.kv_cache, s.req_to_token, s.req_pool_indices, s.topk_idx,
                               s.scale, head_dim_v=s.head_dim_v, workspace=ws, out=out, lse=lse)

    say("graph: sparse MLA decode")
    step()
    _replay_and_check(step, [out, lse])


def test_cascade_step_graph():
    c = workloads.make_cascade_case(151, prefix_lens=[300, 40, 1029], num_draft=6,
                                    num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                                    num_pages=120)
    c = to_device(c, DEV)
    B, n = c.seq_lens.numel(), c.num_draft
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, 16,
                                     c.table_width)
    tab = torch.empty((B * n, n), dtype=torch.int32, device=DEV)
    lens = torch.empty((B * n,), dtype=torch.int32, device=DEV)
    cu_q = torch.arange(0, B * n + 1, n, dtype=torch.int32, device=DEV)
    need = pkv.paged_attn_cascade_workspace_size(B, B * n, n, c.table_width * 16, 16, 4, 128)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(c.q)
    lse = torch.empty((B * n, 16), dtype=torch.float32, device=DEV)

    def step():
        pkv.build_cascade_expand_table(c.custom_mask, c.req_to_token, c.req_pool_indices,
                                       c.seq_lens, n, expand_table=tab, expand_lens=lens,
                                       with_cu=False)
        pkv.paged_attn_cascade(c.q, c.k_cache, c.v_cache, pt, cu_q, kl, n, c.scale, tab, lens,
                               workspace=ws, out=out, lse=lse)

    say("graph: cascade (expand table + prefix pass + expand pass)")
    step()
    _replay_and_check(step, [out, lse, tab, lens])


def test_dca_step_graph():
    c = workloads.make_dca_case(161, seq_lens=[10, 200, 700], num_q_heads=16, num_kv_heads=8,
                                head_dim=128, page_size=16, num_pages=80, chunk_size=160,
                                local_size=32, original_max_position_embeddings=100,
                                value_device=DEV)
    b = to_device(c.base, DEV)
    C = c.chunk_size - c.local_size
    pt, kl, _ = pkv.build_page_table(b.req_to_token, b.req_pool_indices, b.seq_lens, 16,
                                     b.table_width)
    S = -(-700 // C)
    B, hq, d = b.q.shape
    op = torch.empty((S, B, hq, d), dtype=torch.float32, device=DEV)
    lp = torch.empty((S, B, hq), dtype=torch.float32, device=DEV)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    meta = pkv.build_dca_decode_tables(pt, kl, C, 16, c.original_max_position_embeddings)

    def step():
        pkv.paged_attn_dca_decode(b.q, c.q_succ, c.q_inter, b.k_cache, b.v_cache, pt, kl,
                                  b.scale, C, kv_chunk=C, num_splits=S,
                                  q_scale=meta["scaling_factor"], o_partial=op, lse_partial=lp)
        pkv.merge_state(op, lp, out=out, lse_out=lse)

    say("graph: dual chunk decode + merge")
    step()
    _replay_and_check(step, [out, lse])

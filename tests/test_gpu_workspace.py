"""One workspace serves calls of different shapes: the split counters sit in a
fixed region at its start, so partials written by one shape never land where
another shape's counters are. A zero-filled buffer sized for the largest
shape runs shapes A, B, A in turn; each result is compared with the oracle."""

import pytest
import torch

import oracle
import paged_kv_cache_197_amd as pkv
import workloads
from helpers import LSE_TOL, O_TOL, assert_close, compact_pages, np_f, np_i, say, to_device
from test_gpu_sparse import run_case as sparse_run

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
COUNTER_BYTES = 65536   # PKV_WORKSPACE_COUNTER_BYTES


def _prefill_case(seed, prefix, extend, hkv, group, D, P):
    total = sum(p + e for p, e in zip(prefix, extend))
    c = workloads.make_prefill_case(seed, prefix_lens=prefix, extend_lens=extend,
                                    num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=D,
                                    page_size=P, num_pages=total // P + len(prefix) + 4)
    return to_device(c, DEV)


def _prefill_need(c):
    return pkv.paged_attn_varlen_prefill_workspace_size(
        c.seq_lens.numel(), c.q.shape[0], c.max_seqlen_q, c.table_width * c.page_size,
        c.q.shape[1], c.k_cache.shape[2], c.q.shape[2])


def _prefill_vs_oracle(c, ws):
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                                     c.table_width)
    out = torch.full_like(c.q, float("nan"))
    lse = torch.full(c.q.shape[:2], float("nan"), device=DEV)
    pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                  c.max_seqlen_q, c.scale, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    pt_np, kl_np = np_i(pt), np_i(kl)
    rows = list(range(len(kl_np)))
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, c.page_size, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, c.page_size, rows)
    ro, rl = oracle.paged_prefill(np_f(c.q), k_small, v_small, pt_small, np_i(c.cu_seqlens_q),
                                  kl_np, c.page_size, c.scale)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


def test_prefill_workspace_reused_across_shapes():
    # A: one request with two q tiles against 4000 cached keys (4 split
    # counters); B: twelve requests of one q tile each against 1500 keys (its
    # partial blocks lie where A's would not, and it has more counters)
    a = _prefill_case(301, [4000], [40], hkv=2, group=4, D=128, P=16)
    b = _prefill_case(302, [1500] * 12, [1] * 12, hkv=1, group=8, D=64, P=1)
    need_a, need_b = _prefill_need(a), _prefill_need(b)
    assert need_a > COUNTER_BYTES and need_b > COUNTER_BYTES, "both shapes are meant to split"
    ws = torch.zeros(max(need_a, need_b), dtype=torch.uint8, device=DEV)
    for name, c in [("A", a), ("B", b), ("A", a)]:
        say(f"prefill workspace reuse, shape {name}")
        _prefill_vs_oracle(c, ws)
        torch.cuda.synchronize()
        assert not torch.any(ws[:COUNTER_BYTES] != 0), "counters left non-zero"


def test_sparse_workspace_reused_across_shapes():
    # A: 4 requests x 128 heads (8 units of 64 heads, 8 splits of 256 keys);
    # B: 1 request x 32 heads (1 unit, 8 splits); then A again on the same buffer
    a = to_device(workloads.make_sparse_case(311, batch=4, ctx=5000, topk=2048, num_q_heads=128,
                                             head_dim_qk=576, head_dim_v=512, num_pad=30), DEV)
    b = to_device(workloads.make_sparse_case(312, batch=1, ctx=5000, topk=2048, num_q_heads=32,
                                             head_dim_qk=576, head_dim_v=512), DEV)
    need = [pkv.sparse_topk_decode_workspace_size(c.q.shape[0], c.topk_idx.shape[1], c.q.shape[1])
            for c in (a, b)]
    assert min(need) > COUNTER_BYTES, "both shapes are meant to split"
    ws = torch.zeros(max(need), dtype=torch.uint8, device=DEV)
    for name, c in [("A", a), ("B", b), ("A", a)]:
        say(f"sparse workspace reuse, shape {name}")
        out = torch.full((c.q.shape[0], c.q.shape[1], c.head_dim_v), float("nan"),
                         dtype=torch.bfloat16, device=DEV)
        lse = torch.full(c.q.shape[:2], float("nan"), device=DEV)
        pkv.sparse_topk_decode(c.q, c.kv_cache, c.req_to_token, c.req_pool_indices, c.topk_idx,
                               c.scale, head_dim_v=c.head_dim_v, workspace=ws, out=out, lse=lse)
        torch.cuda.synchronize()
        rows = list(range(c.q.shape[0]))
        from test_gpu_sparse import compact_sparse
        q, kv, r2t, rpi, idx = compact_sparse(c, rows)
        ro, rl = oracle.sparse_topk_decode(q, kv, r2t, rpi, idx, c.scale, c.head_dim_v)
        assert_close("out", np_f(out), ro, O_TOL)
        assert_close("lse", np_f(lse), rl, LSE_TOL)
        assert not torch.any(ws[:COUNTER_BYTES] != 0), "counters left non-zero"

"""Split-KV paged decode (+ merge_state) on the GPU versus the oracle.

Small cases are compared element by element in full; the full-size workloads
on sampled requests (every head and split of each sampled request), with the
oracle fed only the pages those requests own.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_197_amd as pkv
import workloads
from helpers import (LSE_TOL, O_TOL, assert_close, compact_pages, np_f, np_i, say, to_device)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu_strided_table(c):
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                                     c.table_width)
    return pt, kl


def gpu_decode(c, pt, kl, chunk, S):
    if S == 1:
        out = torch.full_like(c.q, float("nan"))
        lse = torch.full(c.q.shape[:2], float("nan"), device=DEV)
        pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale, kv_chunk=chunk,
                                      num_splits=1, out=out, lse=lse)
        torch.cuda.synchronize()
        return out, lse
    B, H, D = c.q.shape
    op = torch.full((S, B, H, D), float("nan"), device=DEV)
    lp = torch.full((S, B, H), float("nan"), device=DEV)
    pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale, kv_chunk=chunk,
                                  num_splits=S, o_partial=op, lse_partial=lp)
    torch.cuda.synchronize()
    return op, lp


def oracle_decode_rows(c, pt_np, kl_np, rows, chunk, S):
    """Oracle partials for the given requests only."""
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, c.page_size, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, c.page_size, rows)
    q = np_f(c.q[torch.as_tensor(rows, device=c.q.device)])
    return oracle.paged_decode_splitkv(q, k_small, v_small, pt_small, kl_np[rows], c.page_size,
                                       c.scale, chunk, S)


def check_case(c, chunk, S, rows=None, fp32=False):
    """Decode (S splits) + merge on the GPU vs the oracle, on `rows` (default: all)."""
    pt, kl = gpu_strided_table(c)
    pt_np, kl_np = np_i(pt), np_i(kl)
    if rows is None:
        rows = list(range(c.q.shape[0]))
    o_tol = 1e-5 if fp32 else O_TOL
    l_tol = 1e-5 if fp32 else LSE_TOL
    ro, rl = oracle_decode_rows(c, pt_np, kl_np, rows, chunk, S)
    if S == 1:
        out, lse = gpu_decode(c, pt, kl, chunk, 1)
        assert_close("out", np_f(out)[rows], ro[0], o_tol)
        assert_close("lse", np_f(lse)[rows], rl[0], l_tol)
        return
    op, lp = gpu_decode(c, pt, kl, chunk, S)
    assert not torch.isnan(op).any() and not torch.isnan(lp).any(), "unwritten partials"
    assert_close("o_partial", np_f(op)[:, rows], ro, o_tol if fp32 else 1e-2)
    assert_close("lse_partial", np_f(lp)[:, rows], rl, l_tol)
    out, lse = pkv.merge_state(op, lp, out_dtype=c.q.dtype)
    torch.cuda.synchronize()
    mo, ml = oracle.merge_state(ro, rl)
    assert_close("merged out", np_f(out)[rows], mo, o_tol)
    assert_close("merged lse", np_f(lse)[rows], ml, l_tol)


def test_config1_fp32_two_way_split_and_merge():
    c = to_device(workloads.config1(), DEV)
    say("config1 fp32 S=2")
    check_case(c, c.kv_chunk, c.num_splits, fp32=True)
    say("config1 fp32 S=1")
    check_case(c, 0, 1, fp32=True)


def test_small_config3_bf16():
    c = to_device(workloads.small_config3(), DEV)
    say(f"small_config3 S={c.num_splits}")
    check_case(c, c.kv_chunk, c.num_splits)
    say("small_config3 S=1")
    check_case(c, 0, 1)


def test_config3_full_size_sampled():
    c = workloads.config3(value_device=DEV)
    c = to_device(c, DEV)
    lens = np_i(c.seq_lens)
    rng = np.random.default_rng(0)
    rows = sorted({int(lens.argmin()), int(lens.argmax())} | set(rng.choice(len(lens), 2).tolist()))
    say(f"config3 full S={c.num_splits} rows={rows}")
    check_case(c, c.kv_chunk, c.num_splits, rows=rows)


def swa_case_check(c, rows=None):
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, 1,
                                     c.table_width, prefill_lens=c.prefill_lens, window=c.window)
    pt_np, kl_np = np_i(pt), np_i(kl)
    ref_pt, ref_kl, _ = oracle.page_table_pa_swa(np_i(c.req_to_token), np_i(c.req_pool_indices),
                                                 np_i(c.seq_lens), np_i(c.prefill_lens),
                                                 c.window, c.table_width)
    assert np.array_equal(pt_np, ref_pt) and np.array_equal(kl_np, ref_kl)
    if rows is None:
        rows = list(range(c.q.shape[0]))
    S = c.num_splits
    B, H, D = c.q.shape
    op = torch.full((S, B, H, D), float("nan"), device=DEV)
    lp = torch.full((S, B, H), float("nan"), device=DEV)
    pkv.paged_attn_decode_splitkv(c.q, c.k_cache, c.v_cache, pt, kl, c.scale,
                                  kv_chunk=c.kv_chunk, num_splits=S, o_partial=op,
                                  lse_partial=lp)
    out, lse = pkv.merge_state(op, lp, out_dtype=c.q.dtype)
    torch.cuda.synchronize()
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, 1, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, 1, rows)
    q = np_f(c.q[torch.as_tensor(rows, device=DEV)])
    ro, rl = oracle.paged_decode_splitkv(q, k_small, v_small, pt_small, kl_np[rows], 1, c.scale,
                                         c.kv_chunk, S)
    assert_close("o_partial", np_f(op)[:, rows], ro, 1e-2)
    assert_close("lse_partial", np_f(lp)[:, rows], rl, LSE_TOL)
    mo, ml = oracle.merge_state(ro, rl)
    assert_close("out", np_f(out)[rows], mo, O_TOL)
    assert_close("lse", np_f(lse)[rows], ml, LSE_TOL)


def test_small_config4_sliding_window():
    c = to_device(workloads.small_config4(), DEV)
    say("small_config4")
    swa_case_check(c)


def test_config4_full_size_sampled():
    c = to_device(workloads.config4(value_device=DEV), DEV)
    lens = np_i(c.seq_lens)
    rows = sorted({int(lens.argmin()), int(lens.argmax()), 5, 17})
    say(f"config4 full rows={rows}")
    swa_case_check(c, rows)


EDGE_LENS = [0, 1, 31, 32, 33, 64, 65, 129, 255, 256, 257]


# The bf16 rows with Hkv * D a multiple of 256 and (256 / D) * G <= 16 run the
# kv-head-group kernel (D 128: pairs of kv heads; D 64: fours); the others, and
# fp32, run the per-kv-head kernel.
@pytest.mark.parametrize("dtype,D,P,group,chunk,hkv", [
    (torch.bfloat16, 128, 64, 4, 128, 2),
    (torch.bfloat16, 128, 1, 8, 64, 2),
    (torch.bfloat16, 128, 16, 1, 96, 2),
    (torch.bfloat16, 128, 2, 3, 32, 2),
    (torch.bfloat16, 128, 64, 16, 128, 2),
    (torch.bfloat16, 128, 32, 4, 64, 3),
    (torch.bfloat16, 64, 32, 16, 64, 2),
    (torch.bfloat16, 64, 128, 2, 128, 2),
    (torch.bfloat16, 64, 16, 4, 64, 4),
    (torch.bfloat16, 64, 1, 3, 32, 8),
    (torch.float32, 64, 16, 2, 64, 2),
    (torch.float32, 128, 64, 4, 128, 2),
    (torch.float32, 128, 1, 5, 32, 2),
])
def test_decode_edge_lengths(dtype, D, P, group, chunk, hkv):
    c = workloads.make_decode_case(40 + D + P + group, seq_lens=EDGE_LENS, num_q_heads=hkv * group,
                                   num_kv_heads=hkv, head_dim=D, page_size=P,
                                   num_pages=-(-sum(EDGE_LENS) // P) + len(EDGE_LENS) + 3,
                                   dtype=dtype, kv_chunk=chunk)
    c = to_device(c, DEV)
    fp32 = dtype == torch.float32
    say(f"edge dtype={dtype} D={D} P={P} G={group} Hkv={hkv} chunk={chunk} S={c.num_splits}")
    check_case(c, chunk, c.num_splits, fp32=fp32)
    say(f"edge single split dtype={dtype} D={D} P={P} Hkv={hkv}")
    check_case(c, 0, 1, fp32=fp32)


def test_decode_is_deterministic_and_page_permutation_invariant():
    c = to_device(workloads.small_config3(seed=77), DEV)
    say("determinism / permutation")
    pt, kl = gpu_strided_table(c)
    a = gpu_decode(c, pt, kl, c.kv_chunk, c.num_splits)
    b = gpu_decode(c, pt, kl, c.kv_chunk, c.num_splits)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # move every page somewhere else; the logical content is unchanged
    P = c.page_size
    n = c.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).to(DEV)
    k = torch.empty_like(c.k_cache)
    v = torch.empty_like(c.v_cache)
    k[perm] = c.k_cache
    v[perm] = c.v_cache
    r2t = c.req_to_token.long()
    r2t = (perm[r2t // P] * P + r2t % P).to(torch.int32)
    c2 = workloads.DecodeCase(**{**c.__dict__, "k_cache": k, "v_cache": v, "req_to_token": r2t})
    pt2, kl2 = gpu_strided_table(c2)
    d = gpu_decode(c2, pt2, kl2, c.kv_chunk, c.num_splits)
    assert torch.equal(a[0], d[0]) and torch.equal(a[1], d[1])


@pytest.mark.parametrize("batch,dtype", [(63, torch.bfloat16), (64, torch.bfloat16),
                                         (65, torch.bfloat16), (130, torch.bfloat16),
                                         (64, torch.float32), (65, torch.float32)])
def test_decode_split_order(batch, dtype):
    """Workgroups take the (request, split) pairs longest first up to 64
    requests (one per lane of the ordering wave) and in split-major order
    above: lengths with empty requests, exact multiples of the chunk and
    one spare split (empty for every request) must leave every partial
    written and every value right on both sides of that bound."""
    g = np.random.default_rng(batch)
    chunk = 256
    lens = g.integers(1, 3000, batch)
    lens[::7] = 0
    lens[3::11] = chunk * g.integers(1, 11, len(lens[3::11]))
    lens = lens.tolist()
    c = workloads.make_decode_case(900 + batch, seq_lens=lens, num_q_heads=8, num_kv_heads=2,
                                   head_dim=128, page_size=16,
                                   num_pages=sum(-(-s // 16) for s in lens) + batch + 3,
                                   dtype=dtype, kv_chunk=chunk, ctx=max(lens))
    c = to_device(c, DEV)
    S = -(-max(lens) // chunk) + 1
    say(f"split order batch={batch} {dtype} S={S}")
    check_case(c, chunk, S, fp32=(dtype == torch.float32))

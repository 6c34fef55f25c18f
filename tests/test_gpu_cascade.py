"""Cascade attention (draft-tree verification) on the GPU versus the oracle.

The expand-table builder is compared bit-exactly; the attention (prefix pass
by the prefill kernel, non-causal, then the fused expand pass + merge) against
the oracle's plain tree attention and its staged cascade.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_197_amd as pkv
import workloads
from helpers import LSE_TOL, O_TOL, assert_close, np_f, np_i, say, to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def make_case(seed, prefix, n, hq=8, hkv=2, D=128, P=16, tree="random"):
    pages = sum(-(-(L + n) // P) for L in prefix) + len(prefix) + 4
    c = workloads.make_cascade_case(seed, prefix_lens=prefix, num_draft=n, num_q_heads=hq,
                                    num_kv_heads=hkv, head_dim=D, page_size=P, num_pages=pages,
                                    tree=tree)
    return to_device(c, DEV)


def gpu_tables(c):
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                                     c.table_width)
    tab, lens, cu = pkv.build_cascade_expand_table(c.custom_mask, c.req_to_token,
                                                   c.req_pool_indices, c.seq_lens, c.num_draft)
    return pt, kl, tab, lens, cu


def gpu_cascade(c, pt, kl, tab, lens):
    B, n = c.seq_lens.numel(), c.num_draft
    cu_q = torch.arange(0, B * n + 1, n, dtype=torch.int32, device=DEV)
    out = torch.full_like(c.q, float("nan"))
    lse = torch.full(c.q.shape[:2], float("nan"), device=DEV)
    pkv.paged_attn_cascade(c.q, c.k_cache, c.v_cache, pt, cu_q, kl, n, c.scale, tab, lens,
                           out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("prefix,n", [([3, 0, 9, 1], 5), ([100, 7], 1), ([33, 64, 5], 16),
                                      ([10] * 300, 2), ([0, 2000], 64), ([17], 256)])
def test_expand_table_bit_exact(prefix, n):
    c = make_case(700 + n + len(prefix), prefix, n, hq=2, hkv=1, D=64, P=1)
    say(f"cascade expand table B={len(prefix)} n={n}")
    _, _, tab, lens, cu = gpu_tables(c)
    torch.cuda.synchronize()
    rt, rl, rc = oracle.cascade_expand_table(np_i(c.custom_mask), np_i(c.req_to_token),
                                             np_i(c.req_pool_indices), np_i(c.seq_lens), n)
    assert np.array_equal(np_i(tab), rt)
    assert np.array_equal(np_i(lens), rl)
    assert np.array_equal(np_i(cu), rc)


@pytest.mark.parametrize("D,P,hq,hkv,n,tree", [
    (128, 16, 8, 2, 5, "random"), (128, 1, 32, 8, 8, "random"), (64, 64, 16, 1, 16, "random"),
    (128, 64, 16, 16, 4, "chain"), (64, 3, 4, 2, 1, "random"), (128, 16, 32, 2, 12, "random"),
])
def test_cascade_vs_tree_attention(D, P, hq, hkv, n, tree):
    prefix = [0, 37, 300, 1, 1029]
    c = make_case(720 + D + P + hq + n, prefix, n, hq=hq, hkv=hkv, D=D, P=P, tree=tree)
    say(f"cascade D={D} P={P} Hq={hq} Hkv={hkv} n={n} {tree}")
    pt, kl, tab, lens, _ = gpu_tables(c)
    out, lse = gpu_cascade(c, pt, kl, tab, lens)
    ro, rl = oracle.tree_verify_attention(np_f(c.q), np_f(c.k_cache), np_f(c.v_cache),
                                          np_i(c.req_to_token), np_i(c.req_pool_indices),
                                          np_i(c.seq_lens), np_i(c.custom_mask), n, c.scale)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


@pytest.mark.parametrize("D,P,hq,hkv,prefix,extend,zero,mk", [
    # G * max M <= 32: the packed prefix pass; kv heads per workgroup 4, 2, 1
    (128, 16, 32, 8, [0, 33, 300, 1029, 2000], [8, 1, 5, 8, 3], None, None),
    (128, 1, 16, 4, [1, 31, 32, 255, 256, 257], [2, 8, 3, 1, 8, 4], 2, None),
    (128, 3, 8, 2, [40, 700, 0], [8, 5, 4], None, 300),   # max_seqlen_k below the longest
    (64, 64, 4, 1, [0, 5, 2000], [8, 7, 5], 0, None),
    (64, 16, 32, 4, [100, 1500], [4, 3], None, 256),
])
def test_packed_prefix_pass_vs_noncausal_prefill(D, P, hq, hkv, prefix, extend, zero, mk):
    """With every expand list empty, paged_attn_cascade is its prefix pass
    alone: each request's rows see all its keys (non-causal prefill). Ragged
    draft counts, lengths around the 32-key tiles and the 256-key splits, a
    request with no key (`zero`), and a max_seqlen_k below the longest request
    (its last split then runs to the end)."""
    lens = [p + e for p, e in zip(prefix, extend)]
    pages = sum(-(-L // P) for L in lens) + len(lens) + 4
    c = to_device(workloads.make_prefill_case(780 + D + P + hq, prefix_lens=prefix,
                                              extend_lens=extend, num_q_heads=hq,
                                              num_kv_heads=hkv, head_dim=D, page_size=P,
                                              num_pages=pages), DEV)
    say(f"packed prefix pass D={D} P={P} Hq={hq} Hkv={hkv} M={extend} L={lens} mk={mk}")
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, P,
                                     c.table_width)
    if zero is not None:
        kl[zero] = 0
    total_q = c.q.shape[0]
    tab = torch.zeros((total_q, 1), dtype=torch.int32, device=DEV)
    lens_e = torch.zeros((total_q,), dtype=torch.int32, device=DEV)
    out, lse = pkv.paged_attn_cascade(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                      c.max_seqlen_q, c.scale, tab, lens_e, max_seqlen_k=mk)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(np_f(c.q), np_f(c.k_cache), np_f(c.v_cache), np_i(pt),
                                  np_i(c.cu_seqlens_q), np_i(kl), P, c.scale, causal=False)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


def test_expand_merge_alone_vs_staged_oracle():
    """The separate entry point: prefix pass by the prefill call (non-causal),
    then paged_attn_expand_merge in place, against the oracle's three steps."""
    c = make_case(741, [50, 200, 3], 6, hq=16, hkv=4, D=128, P=16)
    pt, kl, tab, lens, _ = gpu_tables(c)
    B, n = c.seq_lens.numel(), c.num_draft
    cu_q = torch.arange(0, B * n + 1, n, dtype=torch.int32, device=DEV)
    say("expand merge after a non-causal prefill")
    out, lse = pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, cu_q, kl, n, c.scale,
                                             causal=False)
    pkv.paged_attn_expand_merge(c.q, c.k_cache, c.v_cache, tab, lens, c.scale, out, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.cascade_attention(np_f(c.q), np_f(c.k_cache), np_f(c.v_cache), np_i(pt),
                                      np_i(c.seq_lens), c.page_size, np_i(tab), np_i(lens),
                                      c.scale)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


def test_draft_decode_branch_tables():
    """Draft decode with topk > 1 ([FA] init_forward_metadata, draft decode):
    each request's topk branch rows see the committed tokens (prefix pass)
    and the first decode_length tokens of their own branch (expand pass, a
    slice of out_cache_loc)."""
    topk, steps, dl = 3, 4, 2
    prefix = [40, 5, 129]
    B = len(prefix)
    c = make_case(751, prefix, topk * steps, hq=8, hkv=2, D=128, P=1)
    # branch k of request b owns draft positions L_b + k*steps .. + steps - 1
    r2t, rpi, sl = np_i(c.req_to_token), np_i(c.req_pool_indices), np_i(c.seq_lens)
    loc = np.zeros((B * topk, steps), dtype=np.int64)
    for b in range(B):
        for k in range(topk):
            loc[b * topk + k] = r2t[rpi[b], sl[b] + k * steps: sl[b] + (k + 1) * steps]
    tab = torch.as_tensor(loc[:, :dl], dtype=torch.int32, device=DEV).contiguous()
    lens = torch.full((B * topk,), dl, dtype=torch.int32, device=DEV)
    q = c.q[: B * topk].contiguous()
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, 1,
                                     c.table_width)
    cu_q = torch.arange(0, B * topk + 1, topk, dtype=torch.int32, device=DEV)
    say("draft decode branches")
    out, lse = pkv.paged_attn_cascade(q, c.k_cache, c.v_cache, pt, cu_q, kl, topk, c.scale, tab,
                                      lens)
    torch.cuda.synchronize()
    ro, rl = oracle.cascade_attention(np_f(q), np_f(c.k_cache), np_f(c.v_cache), np_i(pt), sl, 1,
                                      np_i(tab), np_i(lens), c.scale)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


def test_cascade_verify_workload_sampled():
    """The full tree-verification workload (B 64, L up to 16384, 8 drafts):
    every row of sampled requests against the plain tree attention, the
    oracle reading only the sampled requests' tokens."""
    c = to_device(workloads.cascade_verify(value_device=DEV), DEV)
    say("cascade_verify workload")
    pt, kl, tab, lens, _ = gpu_tables(c)
    out, lse = gpu_cascade(c, pt, kl, tab, lens)
    n = c.num_draft
    sl = np_i(c.seq_lens)
    starts = np.concatenate([[0], np.cumsum(n * (sl + n))])
    mask_all = np_i(c.custom_mask)
    r2t, rpi = np_i(c.req_to_token), np_i(c.req_pool_indices)
    kflat = c.k_cache.reshape(-1, 1, *c.k_cache.shape[2:])
    vflat = c.v_cache.reshape(-1, 1, *c.v_cache.shape[2:])
    for b in (0, 17, 63):
        L = int(sl[b])
        slots = torch.as_tensor(r2t[rpi[b], :L + n], device=DEV)
        k_small = np_f(kflat[slots])
        v_small = np_f(vflat[slots])
        ro, rl = oracle.tree_verify_attention(
            np_f(c.q[b * n:(b + 1) * n]), k_small, v_small, np.arange(L + n)[None, :], [0], [L],
            mask_all[starts[b]:starts[b + 1]], n, c.scale)
        assert_close(f"out[{b}]", np_f(out[b * n:(b + 1) * n]), ro, O_TOL)
        assert_close(f"lse[{b}]", np_f(lse[b * n:(b + 1) * n]), rl, LSE_TOL)


def test_cascade_page_permutation_bit_identical():
    """Moving every cache page elsewhere (token table rewritten to match, tables
    rebuilt on the GPU) leaves the cascade result bit-identical."""
    c = make_case(761, [70, 300, 5, 1100], 8, hq=16, hkv=4, D=128, P=16)
    say("cascade page permutation")
    pt, kl, tab, lens, _ = gpu_tables(c)
    a = gpu_cascade(c, pt, kl, tab, lens)
    P = c.page_size
    n = c.k_cache.shape[0]
    assert 0 <= int(c.req_to_token.min()) and int(c.req_to_token.max()) < n * P
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(8)).to(DEV)
    k = torch.empty_like(c.k_cache)
    v = torch.empty_like(c.v_cache)
    k[perm] = c.k_cache
    v[perm] = c.v_cache
    r2t = c.req_to_token.long()
    r2t = (perm[r2t // P] * P + r2t % P).to(torch.int32)
    c2 = workloads.CascadeCase(**{**c.__dict__, "k_cache": k, "v_cache": v, "req_to_token": r2t})
    pt2, kl2, tab2, lens2, _ = gpu_tables(c2)
    d = gpu_cascade(c2, pt2, kl2, tab2, lens2)
    assert torch.equal(a[0], d[0]) and torch.equal(a[1], d[1])

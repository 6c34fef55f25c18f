"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these retypes the oracle's formulas: the references are the pages'
printed examples (tests/golden), closed forms, torch's own attention / logsumexp
routines on dense tensors, brute-force set construction, and invariants.
The planted-mistake tests at the end show that each pin bites.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.reference as ref
import workloads
from conftest import f64, i64

# ---------------------------------------------------------------------------
# Library-routine references (dense, built from req_to_token, not the page table)
# ---------------------------------------------------------------------------


def dense_request_kv(cache, req_to_token, row, L):
    """Logical [L, Hkv, D] keys of one request, read through the token-level table."""
    flat = cache.reshape(-1, cache.shape[2], cache.shape[3])
    slots = req_to_token[row, :L].long()
    return flat[slots].to(torch.float64)


def sdpa_reference(q_rows, keys, vals, scale, causal, window_left=-1):
    """torch SDPA (float64, explicit mask) and torch.logsumexp for LSE.

    q_rows [M, Hq, D]; keys/vals [L, Hkv, D]. Causal uses torch.tril's
    bottom-right diagonal offset L - M; a sliding window of W keys to the left
    intersects it with torch.triu at offset L - M - W (a band).
    """
    M, Hq, _ = q_rows.shape
    L, Hkv, _ = keys.shape
    g = Hq // Hkv
    q = q_rows.permute(1, 0, 2).unsqueeze(0)                       # [1, Hq, M, D]
    k = keys.permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
    v = vals.permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
    mask = torch.ones(M, L, dtype=torch.bool)
    if causal:
        mask = torch.tril(mask, diagonal=L - M)
    if window_left >= 0:
        mask = torch.triu(mask, diagonal=L - M - window_left)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    logits = torch.matmul(q, k.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(logits, dim=-1)                          # [1, Hq, M]
    return o[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def _worst(acc, x):
    """Running max error where a NaN anywhere counts as an infinite error."""
    x = float(x)
    return math.inf if math.isnan(x) else max(acc, x)


def prefill_error_vs_sdpa(case):
    pt, kv_lens, _ = oracle.page_table_strided(i64(case.req_to_token), i64(case.req_pool_indices),
                                               i64(case.seq_lens), case.page_size, case.table_width)
    o, lse = oracle.paged_prefill(f64(case.q), f64(case.k_cache), f64(case.v_cache), pt,
                                  i64(case.cu_seqlens_q), kv_lens, case.page_size, case.scale)
    err_o = err_l = 0.0
    cu = i64(case.cu_seqlens_q)
    qd = case.q.to(torch.float64)
    for b in range(len(kv_lens)):
        L = int(kv_lens[b])
        row = int(case.req_pool_indices[b])
        K = dense_request_kv(case.k_cache, case.req_to_token, row, L)
        V = dense_request_kv(case.v_cache, case.req_to_token, row, L)
        o_ref, l_ref = sdpa_reference(qd[cu[b]:cu[b + 1]], K, V, case.scale, causal=True)
        err_o = _worst(err_o, np.abs(o[cu[b]:cu[b + 1]] - o_ref).max())
        err_l = _worst(err_l, np.abs(lse[cu[b]:cu[b + 1]] - l_ref).max())
    return err_o, err_l


def decode_error_vs_sdpa(case):
    pt, kv_lens, _ = oracle.page_table_strided(i64(case.req_to_token), i64(case.req_pool_indices),
                                               i64(case.seq_lens), case.page_size, case.table_width)
    o, lse = oracle.paged_decode_splitkv(f64(case.q), f64(case.k_cache), f64(case.v_cache), pt,
                                         kv_lens, case.page_size, case.scale, 0, 1)
    err_o = err_l = 0.0
    qd = case.q.to(torch.float64)
    for b in range(len(kv_lens)):
        L = int(kv_lens[b])
        row = int(case.req_pool_indices[b])
        K = dense_request_kv(case.k_cache, case.req_to_token, row, L)
        V = dense_request_kv(case.v_cache, case.req_to_token, row, L)
        o_ref, l_ref = sdpa_reference(qd[b:b + 1], K, V, case.scale, causal=False)
        err_o = _worst(err_o, np.abs(o[0, b] - o_ref[0]).max())
        err_l = _worst(err_l, np.abs(lse[0, b] - l_ref[0]).max())
    return err_o, err_l


def small_prefill(seed=21, dtype=torch.float32):
    return workloads.make_prefill_case(seed, prefix_lens=[0, 5, 17, 3], extend_lens=[7, 1, 9, 4],
                                       num_q_heads=6, num_kv_heads=2, head_dim=8, page_size=4,
                                       num_pages=40, dtype=dtype)


def small_decode(seed=22, dtype=torch.float32, page_size=4, kv_chunk=0):
    return workloads.make_decode_case(seed, seq_lens=[1, 13, 30, 8], num_q_heads=8, num_kv_heads=2,
                                      head_dim=16, page_size=page_size, num_pages=64, dtype=dtype,
                                      kv_chunk=kv_chunk, ctx=32)


# ---------------------------------------------------------------------------
# Printed examples
# ---------------------------------------------------------------------------


def test_cu_seqlens_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cu_seqlens_example.json")))
    assert oracle.cu_seqlens(g["lens"]).tolist() == g["cu_seqlens"]


def test_causal_alignment_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "causal_ranges_example.json")))
    ks, ke = oracle.causal_key_ranges(g["extend_seq_lens"], g["seq_lens"])
    assert ks.tolist() == g["ks"] and ke.tolist() == g["ke"]
    # the figure: rows are new tokens, columns the two requests' keys side by side
    rows = []
    for m, L in zip(g["extend_seq_lens"], g["seq_lens"]):
        counts = oracle.visible_key_counts(m, L)
        for c in counts:
            rows.append((m, L, int(c)))
    total = sum(g["seq_lens"])
    drawn = []
    r = 0
    for b, (m, L) in enumerate(zip(g["extend_seq_lens"], g["seq_lens"])):
        for j in range(m):
            c = rows[r][2]
            line = ["-"] * total
            off = sum(g["seq_lens"][:b])
            for t in range(c):
                line[off + t] = "*"
            s = "".join(line)
            drawn.append(s[:g["seq_lens"][0]] + "|" + s[g["seq_lens"][0]:])
            r += 1
    assert drawn == g["mask_figure"]


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------


def test_uniform_scores_give_mean_of_values():
    rng = np.random.default_rng(0)
    for n in [1, 2, 7, 64]:
        V = rng.standard_normal((n, 5))
        K = rng.standard_normal((n, 3))
        o, lse = oracle.softmax_attention(np.zeros(3), K, V, scale=0.7)
        assert np.allclose(o, V.mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse - math.log(n)) < 1e-14


def test_single_key_and_equal_pair():
    q = np.array([0.5, -1.0, 2.0])
    k = np.array([[1.0, 2.0, 0.25]])
    v = np.array([[3.0, -4.0]])
    o, lse = oracle.softmax_attention(q, k, v, scale=0.5)
    s = 0.5 * (0.5 * 1.0 - 1.0 * 2.0 + 2.0 * 0.25)
    assert np.array_equal(o, v[0]) and abs(lse - s) < 1e-15
    k2 = np.vstack([k, k])
    v2 = np.array([[1.0, 0.0], [3.0, 4.0]])
    o, lse = oracle.softmax_attention(q, k2, v2, scale=0.5)
    assert np.allclose(o, [2.0, 2.0], atol=1e-15) and abs(lse - (s + math.log(2))) < 1e-14


def test_empty_key_set():
    o, lse = oracle.softmax_attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 3)), 1.0)
    assert lse == -math.inf and np.array_equal(o, np.zeros(3))


def test_merge_closed_forms():
    rng = np.random.default_rng(1)
    oa, ob = rng.standard_normal((2, 1, 1, 4))
    # equal LSE: plain average, LSE + ln 2
    o, l = oracle.merge_state(np.stack([oa, ob]), np.full((2, 1, 1), 0.3))
    assert np.allclose(o, (oa + ob) / 2, atol=1e-15) and abs(l[0, 0] - (0.3 + math.log(2))) < 1e-15
    # the page's two-part LSE expression: max + log1p(exp(-|l0 - l1|))
    for l0, l1 in [(0.1, 2.5), (-7.0, 3.0), (5.0, 5.0)]:
        _, l = oracle.merge_state(np.stack([oa, ob]), np.array([l0, l1]).reshape(2, 1, 1))
        assert abs(l[0, 0] - (max(l0, l1) + math.log1p(math.exp(-abs(l0 - l1))))) < 1e-14
    # a -inf part carries no weight; all -inf gives (0, -inf)
    o, l = oracle.merge_state(np.stack([oa, ob]), np.array([-math.inf, 1.5]).reshape(2, 1, 1))
    assert np.array_equal(o, ob) and l[0, 0] == 1.5
    o, l = oracle.merge_state(np.stack([oa, ob]), np.full((2, 1, 1), -math.inf))
    assert np.array_equal(o, np.zeros_like(oa)) and l[0, 0] == -math.inf


# ---------------------------------------------------------------------------
# Library routines on dense tensors
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_matches_torch_sdpa(dtype):
    e_o, e_l = prefill_error_vs_sdpa(small_prefill(dtype=dtype))
    assert e_o < 1e-12 and e_l < 1e-12


@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_decode_matches_torch_sdpa(page_size):
    e_o, e_l = decode_error_vs_sdpa(small_decode(page_size=page_size))
    assert e_o < 1e-12 and e_l < 1e-12


def test_sparse_all_tokens_matches_torch_sdpa():
    """Top-k = every context token (shuffled) is dense MLA attention, Dqk 576 / Dv 512."""
    case = workloads.make_sparse_case(31, batch=2, ctx=40, topk=40, num_q_heads=4,
                                      head_dim_qk=576, head_dim_v=512, dtype=torch.float32)
    o, lse = oracle.sparse_topk_decode(f64(case.q), f64(case.kv_cache), i64(case.req_to_token),
                                       i64(case.req_pool_indices), i64(case.topk_idx),
                                       case.scale, case.head_dim_v)
    for b in range(2):
        row = int(case.req_pool_indices[b])
        rows = case.kv_cache[case.req_to_token[row, :40].long()].to(torch.float64)
        q = case.q[b].to(torch.float64)[None, :, None, :]             # [1, H, 1, 576]
        k = rows[None, None].expand(1, 4, 40, 576)
        v = rows[:, :512][None, None].expand(1, 4, 40, 512)
        o_ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=case.scale)
        lse_ref = torch.logsumexp(torch.matmul(q, k.transpose(-1, -2)) * case.scale, dim=-1)
        assert np.abs(o[b] - o_ref[0, :, 0].numpy()).max() < 1e-12
        assert np.abs(lse[b] - lse_ref[0, :, 0].numpy()).max() < 1e-12


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("page_size,chunk", [(4, 4), (4, 8), (4, 12), (16, 16), (1, 5), (4, 64)])
def test_split_then_merge_equals_unsplit(page_size, chunk):
    case = small_decode(page_size=page_size)
    pt, kv_lens, _ = oracle.page_table_strided(i64(case.req_to_token), i64(case.req_pool_indices),
                                               i64(case.seq_lens), page_size, case.table_width)
    args = (f64(case.q), f64(case.k_cache), f64(case.v_cache), pt, kv_lens, page_size, case.scale)
    o1, l1 = oracle.paged_decode_splitkv(*args, 0, 1)
    S = -(-int(kv_lens.max()) // chunk) + 1          # one extra, always empty, split
    op, lp = oracle.paged_decode_splitkv(*args, chunk, S)
    assert np.all(np.isneginf(lp[-1]))
    o2, l2 = oracle.merge_state(op, lp)
    assert np.abs(o2 - o1[0]).max() < 1e-12 and np.abs(l2 - l1[0]).max() < 1e-12


def _permute_pages(case, seed):
    """Move every physical page to a new place and rewrite req_to_token to match."""
    P = case.page_size
    n = case.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed))
    k = torch.empty_like(case.k_cache)
    v = torch.empty_like(case.v_cache)
    k[perm] = case.k_cache
    v[perm] = case.v_cache
    r2t = case.req_to_token.long()
    r2t = perm[r2t // P] * P + r2t % P
    return k, v, r2t.to(torch.int32)


def test_page_permutation_is_bit_identical():
    case = small_decode(page_size=4)
    k, v, r2t = _permute_pages(case, 5)
    outs = []
    for kc, vc, rt in [(case.k_cache, case.v_cache, case.req_to_token), (k, v, r2t)]:
        pt, kv_lens, _ = oracle.page_table_strided(i64(rt), i64(case.req_pool_indices),
                                                   i64(case.seq_lens), 4, case.table_width)
        outs.append(oracle.paged_decode_splitkv(f64(case.q), f64(kc), f64(vc), pt, kv_lens, 4,
                                                case.scale, 8, 4))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_strided_table_invariant():
    case = small_decode(page_size=4)
    r2t, rpi, sl = i64(case.req_to_token), i64(case.req_pool_indices), i64(case.seq_lens)
    pt, kv_lens, cu = oracle.page_table_strided(r2t, rpi, sl, 4, case.table_width)
    assert kv_lens.tolist() == sl.tolist() and cu.tolist() == [0] + np.cumsum(sl).tolist()
    for b in range(len(rpi)):
        L = int(sl[b])
        for t in range(L):
            assert r2t[rpi[b], t] // 4 == pt[b, t // 4]
        assert np.all(pt[b, -(-L // 4):] == 0)


def _random_swa_inputs(rng, batch, ctx):
    rows = 2 * batch
    r2t = rng.integers(0, 10_000, size=(rows, ctx))
    rpi = rng.permutation(rows)[:batch]
    pf_pool = rng.integers(0, ctx, size=rows)
    sl = rng.integers(1, ctx + 1, size=batch)
    return r2t, rpi, sl, pf_pool


def test_pa_swa_sizes_and_order():
    """The kept set, counted in closed form: the prompt contributes
    ``h = min(pf, sl)`` leading positions and the window the ``min(sl, pf + W) - h``
    newest ones, so the row is those two runs back to back, then zeros. Checked
    on 200 random cases (prompt past the sequence, empty window, and so on)."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        batch = int(rng.integers(1, 6))
        ctx = int(rng.integers(1, 60))
        r2t, rpi, sl, pf = _random_swa_inputs(rng, batch, ctx)
        window = int(rng.integers(0, 70))
        pt, kv, cu = oracle.page_table_pa_swa(r2t, rpi, sl, pf, window, ctx)
        for b in range(batch):
            r, s_, p_ = int(rpi[b]), int(sl[b]), int(pf[int(rpi[b])])
            head = min(p_, s_)
            total = min(s_, p_ + window)
            assert kv[b] == total, trial
            positions = list(range(head)) + list(range(s_ - (total - head), s_))
            assert pt[b, :total].tolist() == [int(r2t[r, t]) for t in positions], trial
            assert not pt[b, total:].any(), trial
        assert cu.tolist() == [0] + np.cumsum(kv).tolist()


def test_pa_swa_edge_cases():
    r2t = np.arange(40).reshape(2, 20) + 100
    rpi = np.array([1])
    # window reaches back into the prefill: nothing is dropped
    pt, kv, _ = oracle.page_table_pa_swa(r2t, rpi, [12], np.array([0, 10]), 5, 20)
    assert kv.tolist() == [12] and pt[0, :12].tolist() == list(range(120, 132))
    # a gap: keep [0, 4) and the last 3 of 15
    pt, kv, _ = oracle.page_table_pa_swa(r2t, rpi, [15], np.array([0, 4]), 3, 20)
    assert kv.tolist() == [7] and pt[0, :7].tolist() == [120, 121, 122, 123, 132, 133, 134]
    assert np.all(pt[0, 7:] == 0)
    # kv_len 1: no prefill, window 1
    pt, kv, _ = oracle.page_table_pa_swa(r2t, rpi, [9], np.array([0, 0]), 1, 20)
    assert kv.tolist() == [1] and pt[0, 0] == 128


def test_sparse_invariants():
    case = workloads.make_sparse_case(32, batch=2, ctx=200, topk=50, num_q_heads=4,
                                      head_dim_qk=576, head_dim_v=512, dtype=torch.bfloat16)
    args = (f64(case.q), f64(case.kv_cache), i64(case.req_to_token), i64(case.req_pool_indices))
    idx = i64(case.topk_idx)
    o, l = oracle.sparse_topk_decode(*args, idx, case.scale, 512)
    # order of the top-k list does not matter
    rng = np.random.default_rng(3)
    shuffled = np.stack([rng.permutation(r) for r in idx])
    o2, l2 = oracle.sparse_topk_decode(*args, shuffled, case.scale, 512)
    assert np.abs(o - o2).max() < 1e-12 and np.abs(l - l2).max() < 1e-12
    # -1 entries are skipped: same as dropping them
    padded = idx.copy()
    padded[:, 40:] = -1
    o3, l3 = oracle.sparse_topk_decode(*args, padded, case.scale, 512)
    o4, l4 = oracle.sparse_topk_decode(*args, idx[:, :40], case.scale, 512)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    # an all -1 row is the empty set
    o5, l5 = oracle.sparse_topk_decode(*args, np.full_like(idx, -1), case.scale, 512)
    assert np.all(o5 == 0) and np.all(np.isneginf(l5))


def test_workload_configs_have_the_stated_shapes():
    c1 = workloads.config1()
    assert c1.q.shape == (2, 4, 64) and c1.k_cache.shape == (16, 16, 2, 64)
    assert c1.seq_lens.tolist() == [37, 100] and c1.num_splits == 2 and c1.q.dtype == torch.float32
    c2 = workloads.config2()
    assert c2.q.shape == (849, 32, 128) and c2.seq_lens.tolist() == [256, 192, 1024, 1017]
    assert c2.cu_seqlens_q.tolist() == [0, 256, 320, 832, 849]


# ---------------------------------------------------------------------------
# Planted mistakes: each pin above must catch a plausible error in the oracle
# ---------------------------------------------------------------------------


def test_planted_wrong_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(ref, "kv_head_of", lambda h, hq, hkv: h % hkv)
    e_o, _ = prefill_error_vs_sdpa(small_prefill())
    assert e_o > 1e-3


def test_planted_off_by_one_causal_is_caught(monkeypatch, golden_dir):
    real = ref.visible_key_counts
    monkeypatch.setattr(ref, "visible_key_counts",
                        lambda m, L, causal=True: real(m, L, causal) - (1 if causal else 0))
    e_o, _ = prefill_error_vs_sdpa(small_prefill())
    assert e_o > 1e-3
    with pytest.raises(AssertionError):
        test_causal_alignment_worked_example(golden_dir)


def test_planted_wrong_gather_is_caught(monkeypatch):
    def bad_gather(cache, page_row, length, page_size):
        out = np.empty((length,) + tuple(cache.shape[2:]))
        for t in range(length):
            out[t] = cache[int(page_row[t // page_size]), (page_size - 1 - t % page_size)]
        return out
    monkeypatch.setattr(ref, "gather_paged", bad_gather)
    e_o, _ = decode_error_vs_sdpa(small_decode(page_size=4))
    assert not (e_o < 1e-3)          # wrong values or NaN from unowned slots


def test_planted_missing_scale_is_caught(monkeypatch):
    real = ref.softmax_attention
    monkeypatch.setattr(ref, "softmax_attention", lambda q, k, v, scale: real(q, k, v, 1.0))
    e_o, e_l = decode_error_vs_sdpa(small_decode())
    assert e_o > 1e-3 or e_l > 1e-3


def test_planted_unnormalised_merge_is_caught(monkeypatch):
    def bad_merge(o_parts, lse_parts):
        w = np.exp(lse_parts - lse_parts.max(axis=0))
        return (w[..., None] * o_parts).sum(0), lse_parts.max(axis=0)
    monkeypatch.setattr(oracle, "merge_state", bad_merge)
    with pytest.raises(AssertionError):
        test_split_then_merge_equals_unsplit(4, 8)


def test_planted_pa_swa_window_mistake_is_caught(monkeypatch):
    """A window that keeps one token too few is caught by the size pin."""
    def bad(req_to_token, rpi, seq_lens, prefill_lens, window, width):
        pt = np.zeros((len(rpi), width), dtype=np.int32)
        kv = np.zeros(len(rpi), dtype=np.int32)
        for b in range(len(rpi)):
            r, sl, pf = int(rpi[b]), int(seq_lens[b]), int(prefill_lens[int(rpi[b])])
            keep = sorted(t for t in set(range(pf)) | set(range(max(pf, sl - window + 1), sl))
                          if t < sl)
            kv[b] = len(keep)
            for j, t in enumerate(keep):
                pt[b, j] = req_to_token[r, t]
        return pt, kv, oracle.cu_seqlens(kv)
    monkeypatch.setattr(oracle, "page_table_pa_swa", bad)
    with pytest.raises(AssertionError):
        test_pa_swa_sizes_and_order()


# --- kv_append: set_kv_buffer at out_cache_loc ([FA] forward_extend) ---------

def _tiny_append_case(seed=0, pages=6, P=4, hkv=2, d=3, n=7):
    g = np.random.default_rng(seed)
    kc = g.standard_normal((pages, P, hkv, d))
    vc = g.standard_normal((pages, P, hkv, d))
    loc = g.permutation(pages * P)[:n]
    kn = g.standard_normal((n, hkv, d))
    vn = g.standard_normal((n, hkv, d))
    return kc, vc, loc, kn, vn


def test_kv_append_matches_elementwise_loop():
    kc, vc, loc, kn, vn = _tiny_append_case()
    P = kc.shape[1]
    ek, ev = kc.copy(), vc.copy()
    for i, s in enumerate(loc):                 # brute force: one element at a time
        for h in range(kc.shape[2]):
            for x in range(kc.shape[3]):
                ek[s // P, s % P, h, x] = kn[i, h, x]
                ev[s // P, s % P, h, x] = vn[i, h, x]
    gk, gv = oracle.kv_append(kc, vc, loc, kn, vn)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)
    assert not np.array_equal(kc, gk)           # the inputs are not modified in place
    assert np.array_equal(kc, _tiny_append_case()[0])


def test_kv_append_invariants():
    kc, vc, loc, kn, vn = _tiny_append_case(seed=3)
    gk, gv = oracle.kv_append(kc, vc, loc, kn, vn)
    P = kc.shape[1]
    flat = gk.reshape(-1, *gk.shape[2:])
    assert np.array_equal(flat[loc], kn)        # the written slots hold the new rows
    untouched = np.setdiff1d(np.arange(flat.shape[0]), loc)
    assert np.array_equal(flat[untouched], kc.reshape(-1, *kc.shape[2:])[untouched])
    # appending the values a slot already holds changes nothing
    k2, v2 = oracle.kv_append(gk, gv, loc, kn, vn)
    assert np.array_equal(k2, gk) and np.array_equal(v2, gv)


def test_prefill_append_equals_prefill_over_the_written_cache():
    """Extend with the new tokens' K/V passed separately (their cache slots
    poisoned) equals the plain extend over a cache that already holds them."""
    c = workloads.make_prefill_case(5, prefix_lens=[3, 0, 9], extend_lens=[4, 5, 2],
                                    num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=2,
                                    num_pages=40)
    r2t, rpi = i64(c.req_to_token), i64(c.req_pool_indices)
    pre = i64(c.seq_lens) - i64(c.extend_lens)
    loc = np.concatenate([r2t[rpi[b], pre[b]:pre[b] + int(c.extend_lens[b])]
                          for b in range(len(pre))])
    kc, vc = f64(c.k_cache), f64(c.v_cache)
    P = c.page_size
    kn = kc.reshape(-1, *kc.shape[2:])[loc].copy()
    vn = vc.reshape(-1, *vc.shape[2:])[loc].copy()
    pt, kl, _ = oracle.page_table_strided(i64(c.req_to_token), rpi, i64(c.seq_lens), P,
                                          c.table_width)
    ro, rl = oracle.paged_prefill(f64(c.q), kc, vc, pt, i64(c.cu_seqlens_q), kl, P, c.scale)
    bad_k, bad_v = kc.copy(), vc.copy()
    bad_k.reshape(-1, *kc.shape[2:])[loc] = np.nan
    bad_v.reshape(-1, *vc.shape[2:])[loc] = np.nan
    o, l, k2, v2 = oracle.paged_prefill_append(f64(c.q), bad_k, bad_v, pt, i64(c.cu_seqlens_q),
                                               kl, P, c.scale, loc, kn, vn)
    assert np.array_equal(o, ro) and np.array_equal(l, rl)
    assert np.array_equal(k2, kc, equal_nan=True) and np.array_equal(v2, vc, equal_nan=True)


def test_planted_append_slot_mistake_is_caught(monkeypatch):
    kc, vc, loc, kn, vn = _tiny_append_case(seed=5)
    good = oracle.kv_append(kc, vc, loc, kn, vn)
    real = np.asarray
    monkeypatch.setattr(ref.np, "asarray",
                        lambda a, dtype=None: (real(a, dtype=dtype) + 1)
                        if dtype is np.int64 else real(a, dtype=dtype))
    bad = ref.kv_append(kc, vc, loc % (kc.shape[0] * kc.shape[1] - 1), kn, vn)
    assert not np.array_equal(bad[0], good[0])


# --- lower-bound masks: sliding window (W, 0) and chunked local attention -----

def test_local_attention_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "local_attention_example.json")))
    C = g["attn_chunk_size"]
    M, L = g["q_seqlens"][0], g["kv_seqlens"][0]
    drawn = []
    for j in range(M):
        p = L - M + j
        lo = oracle.key_lower_bound(p, attn_chunk=C)
        drawn.append("".join("1" if lo <= k <= p else "." for k in range(L)))
    assert drawn == g["batch0_local_mask"]
    cu = oracle.cu_seqlens(g["q_seqlens"])
    vb = oracle.local_attention_virtual_batches(C, cu, g["kv_seqlens"])
    assert [x[2] for x in vb] == g["q_seqlens_local"]
    assert [x[4] for x in vb] == g["seqlens_k_local"]


def _window_case():
    return workloads.make_prefill_case(33, prefix_lens=[0, 9, 21, 2], extend_lens=[11, 3, 8, 6],
                                       num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=4,
                                       num_pages=60, dtype=torch.float32)


def _oracle_prefill(case, **kw):
    pt, kl, _ = oracle.page_table_strided(i64(case.req_to_token), i64(case.req_pool_indices),
                                          i64(case.seq_lens), case.page_size, case.table_width)
    return oracle.paged_prefill(f64(case.q), f64(case.k_cache), f64(case.v_cache), pt,
                                i64(case.cu_seqlens_q), kl, case.page_size, case.scale, **kw)


@pytest.mark.parametrize("W", [0, 3, 7, 40])
def test_sliding_window_prefill_matches_sdpa_band(W):
    case = _window_case()
    o, lse = _oracle_prefill(case, window_left=W)
    cu = i64(case.cu_seqlens_q)
    qd = case.q.to(torch.float64)
    for b in range(len(cu) - 1):
        L = int(case.seq_lens[b])
        row = int(case.req_pool_indices[b])
        K = dense_request_kv(case.k_cache, case.req_to_token, row, L)
        V = dense_request_kv(case.v_cache, case.req_to_token, row, L)
        o_ref, l_ref = sdpa_reference(qd[cu[b]:cu[b + 1]], K, V, case.scale, causal=True,
                                      window_left=W)
        assert np.abs(o[cu[b]:cu[b + 1]] - o_ref).max() < 1e-12
        assert np.abs(lse[cu[b]:cu[b + 1]] - l_ref).max() < 1e-12


def test_window_edge_cases():
    case = _window_case()
    plain = _oracle_prefill(case)
    wide = _oracle_prefill(case, window_left=10_000)
    assert np.array_equal(plain[0], wide[0]) and np.array_equal(plain[1], wide[1])
    # W = 0: each row sees only its own key -> O = v_p, LSE = scale * q . k_p
    o, lse = _oracle_prefill(case, window_left=0)
    cu = i64(case.cu_seqlens_q)
    for b in range(len(cu) - 1):
        L, M = int(case.seq_lens[b]), int(cu[b + 1] - cu[b])
        row = int(case.req_pool_indices[b])
        K = dense_request_kv(case.k_cache, case.req_to_token, row, L).numpy()
        V = dense_request_kv(case.v_cache, case.req_to_token, row, L).numpy()
        for j in range(M):
            p = L - M + j
            for h in range(4):
                kvh = h // 2
                assert np.allclose(o[cu[b] + j, h], V[p, kvh], atol=1e-15)
                s = case.scale * float(np.dot(f64(case.q)[cu[b] + j, h], K[p, kvh]))
                assert abs(lse[cu[b] + j, h] - s) < 1e-12


@pytest.mark.parametrize("C", [4, 8, 16])
def test_local_chunks_equal_virtual_batches(C):
    """The masked definition against the pages' formulation: each virtual
    batch is an ordinary causal extend over its own key range."""
    case = _window_case()
    o, lse = _oracle_prefill(case, attn_chunk=C)
    cu = i64(case.cu_seqlens_q)
    qd = f64(case.q)
    for b, qs, qn, k0, kn in oracle.local_attention_virtual_batches(C, cu, i64(case.seq_lens)):
        row = int(case.req_pool_indices[b])
        L = int(case.seq_lens[b])
        K = dense_request_kv(case.k_cache, case.req_to_token, row, L).numpy()[k0:k0 + kn]
        V = dense_request_kv(case.v_cache, case.req_to_token, row, L).numpy()[k0:k0 + kn]
        vo, vl = oracle.paged_prefill(qd[qs:qs + qn], K[:, None], V[:, None],
                                      np.arange(kn)[None, :], np.array([0, qn]),
                                      np.array([kn]), 1, case.scale)
        assert np.abs(o[qs:qs + qn] - vo).max() < 1e-12
        assert np.abs(lse[qs:qs + qn] - vl).max() < 1e-12


@pytest.mark.parametrize("mask", [dict(window_left=5), dict(attn_chunk=8)])
def test_masked_decode_split_then_merge_equals_unsplit(mask):
    case = small_decode(page_size=4)
    pt, kl, _ = oracle.page_table_strided(i64(case.req_to_token), i64(case.req_pool_indices),
                                          i64(case.seq_lens), case.page_size, case.table_width)
    args = (f64(case.q), f64(case.k_cache), f64(case.v_cache), pt, kl, case.page_size, case.scale)
    o1, l1 = oracle.paged_decode_splitkv(*args, 0, 1, **mask)
    op, lp = oracle.paged_decode_splitkv(*args, 8, 4, **mask)
    o2, l2 = oracle.merge_state(op, lp)
    assert np.abs(o1[0] - o2).max() < 1e-12 and np.abs(l1[0] - l2).max() < 1e-12
    # the masked decode of position L-1 is the last row of a masked extend over the request
    for b in range(len(kl)):
        L = int(kl[b])
        if L == 0:
            continue
        lo = oracle.key_lower_bound(L - 1, **mask)
        row = int(case.req_pool_indices[b])
        K = dense_request_kv(case.k_cache, case.req_to_token, row, L).numpy()
        V = dense_request_kv(case.v_cache, case.req_to_token, row, L).numpy()
        for h in range(8):
            o_ref, l_ref = oracle.softmax_attention(f64(case.q)[b, h], K[lo:, h // 4],
                                                    V[lo:, h // 4], case.scale)
            assert np.abs(o1[0, b, h] - o_ref).max() < 1e-15 and abs(l1[0, b, h] - l_ref) < 1e-15


def test_planted_window_off_by_one_is_caught(monkeypatch):
    real = ref.key_lower_bound
    monkeypatch.setattr(ref, "key_lower_bound",
                        lambda pos, window_left=-1, attn_chunk=0:
                        real(pos, window_left, attn_chunk) + (1 if window_left >= 0 else 0))
    with pytest.raises(AssertionError):
        test_sliding_window_prefill_matches_sdpa_band(3)


# ---------------------------------------------------------------------------
# Cascade attention (draft-tree verification)
# ---------------------------------------------------------------------------

def test_cascade_expand_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cascade_expand_example.json")))
    n = len(g["draft_slots"])
    L = 2                                             # committed tokens: all visible
    r2t = np.array([[0, 0, 0, 0, 0], [5, 6] + g["draft_slots"]])
    mask = np.concatenate([np.array([1] * L + row) for row in g["draft_mask"]])
    table, lens, cu = oracle.cascade_expand_table(mask, r2t, [1], [L], n)
    assert table.tolist() == g["expand_table"]
    assert lens.tolist() == g["expand_lens"]
    assert cu.tolist() == [0, 1, 3, 5]


def _tiny_cascade(seed, P=4, n=5, tree="random", prefix=(3, 0, 9, 1), dtype=torch.float32):
    return workloads.make_cascade_case(seed, prefix_lens=list(prefix), num_draft=n,
                                       num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=P,
                                       num_pages=sum(prefix) // P + len(prefix) * (n // P + 2)
                                       + 4, tree=tree, dtype=dtype)


def _oracle_cascade(c):
    pt, _, _ = oracle.page_table_strided(i64(c.req_to_token), i64(c.req_pool_indices),
                                         i64(c.seq_lens), c.page_size, c.table_width)
    table, lens, _ = oracle.cascade_expand_table(i64(c.custom_mask), i64(c.req_to_token),
                                                 i64(c.req_pool_indices), i64(c.seq_lens),
                                                 c.num_draft)
    return oracle.cascade_attention(f64(c.q), f64(c.k_cache), f64(c.v_cache), pt,
                                    i64(c.seq_lens), c.page_size, table, lens, c.scale)


def _oracle_tree(c):
    return oracle.tree_verify_attention(f64(c.q), f64(c.k_cache), f64(c.v_cache),
                                        i64(c.req_to_token), i64(c.req_pool_indices),
                                        i64(c.seq_lens), i64(c.custom_mask), c.num_draft,
                                        c.scale)


def test_cascade_expand_table_matches_stable_sort():
    """Each row is the request's draft slots, visible ones first, both groups in
    position order: numpy's stable argsort of 'hidden' gives the same order."""
    for seed in range(20):
        n = 1 + seed % 9
        c = _tiny_cascade(100 + seed, n=n, P=1 + seed % 3)
        r2t, rpi, sl = i64(c.req_to_token), i64(c.req_pool_indices), i64(c.seq_lens)
        mask = i64(c.custom_mask).astype(bool)
        table, lens, cu = oracle.cascade_expand_table(mask, r2t, rpi, sl, n)
        start = 0
        for b in range(len(sl)):
            L = int(sl[b])
            drafts = r2t[rpi[b], L:L + n]
            for i in range(n):
                vis = mask[start + L:start + L + n]
                order = np.argsort(~vis, kind="stable")
                assert table[b * n + i].tolist() == drafts[order].tolist()
                assert lens[b * n + i] == vis.sum()
                assert sorted(table[b * n + i].tolist()) == sorted(drafts.tolist())
                start += L + n
        assert cu[-1] == lens.sum() and (np.diff(cu) == lens).all()


def test_tree_verify_matches_sdpa_with_custom_mask():
    """The plain definition against torch SDPA (float64) with each request's
    custom-mask rows as an explicit boolean mask over its L + n positions."""
    c = _tiny_cascade(7)
    o, lse = _oracle_tree(c)
    n, sl = c.num_draft, i64(c.seq_lens)
    mask = torch.as_tensor(i64(c.custom_mask).astype(bool))
    start = 0
    for b in range(len(sl)):
        L = int(sl[b])
        row = int(c.req_pool_indices[b])
        K = dense_request_kv(c.k_cache, c.req_to_token, row, L + n)
        V = dense_request_kv(c.v_cache, c.req_to_token, row, L + n)
        m = mask[start:start + n * (L + n)].view(n, L + n)
        start += n * (L + n)
        q = c.q[b * n:(b + 1) * n].to(torch.float64)
        g = q.shape[1] // K.shape[1]
        qq = q.permute(1, 0, 2).unsqueeze(0)
        kk = K.permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
        vv = V.permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
        ref_o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m,
                                                                 scale=c.scale)
        logits = (torch.matmul(qq, kk.transpose(-1, -2)) * c.scale).masked_fill(~m, -math.inf)
        ref_l = torch.logsumexp(logits, dim=-1)
        assert np.abs(o[b * n:(b + 1) * n] - ref_o[0].permute(1, 0, 2).numpy()).max() < 1e-12
        assert np.abs(lse[b * n:(b + 1) * n] - ref_l[0].permute(1, 0).numpy()).max() < 1e-12


@pytest.mark.parametrize("P,n,tree", [(1, 5, "random"), (4, 5, "random"), (4, 8, "chain"),
                                      (3, 1, "random"), (2, 12, "random")])
def test_cascade_equals_tree_attention(P, n, tree):
    """Prefix pass + expand pass + merge reach the plain tree attention."""
    c = _tiny_cascade(40 + P + n, P=P, n=n, tree=tree)
    o, lse = _oracle_cascade(c)
    o_ref, l_ref = _oracle_tree(c)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - l_ref).max() < 1e-12


def test_chain_tree_is_causal_extend():
    """A chain of drafts (each sees all earlier ones) is ordinary causal extend
    of the n drafts over L + n keys."""
    c = _tiny_cascade(51, P=4, n=6, tree="chain")
    o, lse = _oracle_tree(c)
    n, sl = c.num_draft, i64(c.seq_lens)
    pt, kl, _ = oracle.page_table_strided(i64(c.req_to_token), i64(c.req_pool_indices), sl + n,
                                          c.page_size, c.table_width)
    cu = np.arange(0, len(sl) * n + 1, n)
    o2, l2 = oracle.paged_prefill(f64(c.q), f64(c.k_cache), f64(c.v_cache), pt, cu, kl,
                                  c.page_size, c.scale, causal=True)
    assert np.abs(o - o2).max() < 1e-12 and np.abs(lse - l2).max() < 1e-12


def test_planted_causal_prefix_pass_is_caught(monkeypatch):
    real = ref.paged_prefill
    monkeypatch.setattr(ref, "paged_prefill", lambda *a, **kw: real(*a, **{**kw, "causal": True}))
    with pytest.raises(AssertionError):
        test_cascade_equals_tree_attention(4, 5, "random")


def test_planted_expand_order_mistake_is_caught(monkeypatch):
    """Listing each row's drafts by slot number instead of visible-first
    (keeping the count) attends to the wrong drafts."""
    real = ref.cascade_expand_table

    def unsorted(mask, r2t, rpi, sl, n):
        table, lens, cu = real(mask, r2t, rpi, sl, n)
        for r in range(table.shape[0]):
            table[r] = np.sort(table[r])
        return table, lens, cu
    monkeypatch.setattr(ref, "cascade_expand_table", unsorted)
    monkeypatch.setattr(oracle, "cascade_expand_table", unsorted)
    with pytest.raises(AssertionError):
        test_cascade_equals_tree_attention(1, 5, "random")


# ---------------------------------------------------------------------------
# Dual chunk attention decode
# ---------------------------------------------------------------------------

def test_round_to_bf16_matches_torch():
    x = torch.randn(20000, generator=torch.Generator().manual_seed(3)) * 7
    x[:4] = torch.tensor([0.0, -0.0, 1e-30, 3.0e38])
    assert np.array_equal(oracle.round_to_bf16(x.numpy()),
                          x.to(torch.bfloat16).to(torch.float32).numpy())


def test_dca_scaling_factor_closed_forms():
    omp = 4096
    sf = oracle.dca_scaling_factor([4096, 2048, 1, int(round(4096 * math.e ** 10)), 4096 * 2],
                                   omp)
    assert sf[0] == 1.0 and sf[1] == 1.0 and sf[2] == 1.0          # clipped at 1
    assert abs(sf[3] - 2.0) < 1e-9
    assert abs(sf[4] - (1 + 0.1 * math.log(2))) < 1e-15


def _dca_case(seed, lens, P, dtype=torch.float32, hq=4, hkv=2, d=8):
    c = workloads.make_decode_case(seed, seq_lens=lens, num_q_heads=hq, num_kv_heads=hkv,
                                   head_dim=d, page_size=P,
                                   num_pages=sum(-(-x // P) for x in lens) + 3, dtype=dtype)
    g = torch.Generator().manual_seed(seed + 1000)
    q_succ = torch.randn(c.q.shape, generator=g).to(dtype)
    q_inter = torch.randn(c.q.shape, generator=g).to(dtype)
    pt, kl, _ = oracle.page_table_strided(i64(c.req_to_token), i64(c.req_pool_indices),
                                          i64(c.seq_lens), P, c.table_width)
    return c, q_succ, q_inter, pt, kl


def test_dca_tables_cover_the_three_ranges():
    """Brute force: the slots each stage reads are exactly the request's
    positions [cC, L), [(c-1)C, cC) and [0, (c-1)C), read in order."""
    chunk_size, local_size, P = 24, 8, 4
    C = chunk_size - local_size
    lens = [1, 15, 16, 17, 31, 32, 33, 48, 49, 70]
    c, _, _, pt, kl = _dca_case(61, lens, P)
    t = oracle.dca_decode_tables(pt, kl, chunk_size, local_size, P)
    for b, L in enumerate(lens):
        slot = lambda row, pos: int(row[pos // P]) * P + pos % P
        full = [slot(pt[b], p) for p in range(L)]
        cc = (L - 1) // C
        got = [slot(t["table_intra"][b], p) for p in range(int(t["lens_intra"][b]))]
        assert got == full[cc * C:L]
        got = [slot(t["table_succ"][b], p) for p in range(int(t["lens_succ"][b]))]
        assert got == (full[(cc - 1) * C:cc * C] if cc >= 1 else [])
        assert int(t["lens_inter"][b]) == max(cc - 1, 0) * C
        # the three ranges tile [0, L); rows are zero past their stage's pages
        assert t["lens_intra"][b] + t["lens_succ"][b] + t["lens_inter"][b] == L
        n_intra = -(-int(t["lens_intra"][b]) // P)
        assert not t["table_intra"][b, n_intra:].any()
        assert not t["table_succ"][b, C // P if cc >= 1 else 0:].any()


@pytest.mark.parametrize("P,chunk_size,local_size", [(4, 24, 8), (1, 9, 1), (8, 40, 8)])
def test_dca_decode_equals_single_softmax_definition(P, chunk_size, local_size):
    C = chunk_size - local_size
    lens = [1, C - 1, C, C + 1, 2 * C, 2 * C + 3, 3 * C + 5, 5 * C]
    c, qs, qi, pt, kl = _dca_case(71 + P, lens, P)
    o, lse = oracle.dca_decode(f64(c.q), f64(qs), f64(qi), f64(c.k_cache), f64(c.v_cache), pt, kl,
                               P, c.scale, chunk_size, local_size)
    o2, l2 = oracle.dca_decode_reference(f64(c.q), f64(qs), f64(qi), f64(c.k_cache),
                                         f64(c.v_cache), pt, kl, P, c.scale, C)
    assert np.abs(o - o2).max() < 1e-12 and np.abs(lse - l2).max() < 1e-12


def test_dca_with_one_query_is_plain_decode():
    """Equal queries in all stages: ordinary decode over all L keys (torch SDPA)."""
    lens = [5, 16, 40, 77]
    c, _, _, pt, kl = _dca_case(81, lens, 4)
    o, lse = oracle.dca_decode(f64(c.q), f64(c.q), f64(c.q), f64(c.k_cache), f64(c.v_cache), pt,
                               kl, 4, c.scale, 20, 4)
    for b, L in enumerate(lens):
        row = int(c.req_pool_indices[b])
        K = dense_request_kv(c.k_cache, c.req_to_token, row, L)
        V = dense_request_kv(c.v_cache, c.req_to_token, row, L)
        ro, rl = sdpa_reference(c.q[b:b + 1].to(torch.float64), K, V, c.scale, causal=False)
        assert np.abs(o[b] - ro[0]).max() < 1e-12 and np.abs(lse[b] - rl[0]).max() < 1e-12


def test_dca_query_scaling_is_rounded_prescaling():
    """With original_max_position_embeddings the stages see q * factor rounded
    to bf16 (torch's own conversion here), the same as prescaled queries."""
    lens = [30, 100, 257]
    omp = 40
    c, qs, qi, pt, kl = _dca_case(91, lens, 4, dtype=torch.bfloat16)
    o, lse = oracle.dca_decode(f64(c.q), f64(qs), f64(qi), f64(c.k_cache), f64(c.v_cache), pt, kl,
                               4, c.scale, 48, 16, original_max_position_embeddings=omp)
    sf = torch.as_tensor(oracle.dca_scaling_factor(lens, omp), dtype=torch.float32)[:, None, None]
    pre = [(x.float() * sf).to(torch.bfloat16) for x in (c.q, qs, qi)]
    o2, l2 = oracle.dca_decode(*[f64(x) for x in pre], f64(c.k_cache), f64(c.v_cache), pt, kl, 4,
                               c.scale, 48, 16)
    assert np.abs(o - o2).max() < 1e-12 and np.abs(lse - l2).max() < 1e-12
    assert sf.max() > 1.0


def test_planted_dca_chunk_index_is_caught(monkeypatch):
    """The query's chunk taken as L // chunk_len (off by one at chunk ends)."""
    monkeypatch.setattr(ref, "dca_query_chunk",
                        lambda sl, chunk_len: np.asarray(sl, dtype=np.int64) // int(chunk_len))
    with pytest.raises(AssertionError):
        test_dca_decode_equals_single_softmax_definition(4, 24, 8)

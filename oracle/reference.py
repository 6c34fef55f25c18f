"""Plain float64 numpy oracle (test infrastructure only; see the package docstring).

Conventions fixed here (readings of the pages where they are silent):
  * LSE is the natural log of the softmax denominator including the scale, the
    quantity the pages exponentiate with ``torch.exp`` when they merge partial
    results ([DCA] ``_merge_attn_outputs``).
  * LSE is token-major ``[N, H]``, the layout the pages hand to ``merge_state_v2``
    after ``softmax_lse.T.contiguous()`` ([FA] ``forward_extend``, cascade branch).
  * An empty key set gives O = 0 and LSE = -inf ([DCA]
    ``_dual_chunk_flash_attn_decoding_with_exp_sums``, which forces exactly that
    for zero-length rows). Merging only -inf parts gives (0, -inf).
  * Page-table entries past a request's last page are 0.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Integer metadata
# ---------------------------------------------------------------------------

def cu_seqlens(lens) -> np.ndarray:
    """Exclusive prefix sum with a leading zero: lengths [4, 6] -> [0, 4, 10].

    [DCA] ``DualChunkFlashAttentionMetadata`` (the ``query_start_loc`` /
    ``seq_start_loc`` fields and their worked example); [FA]
    ``init_forward_metadata`` builds ``cu_seqlens_k`` as ``cumsum`` padded with
    one leading zero.
    """
    lens = np.asarray(lens, dtype=np.int64)
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    total = 0
    for i, n in enumerate(lens):
        total += int(n)
        out[i + 1] = total
    return out.astype(np.int32)


def page_table_strided(req_to_token, req_pool_indices, seq_lens, page_size, width):
    """Token-level ``req_to_token`` rows -> page table of page ids.

    [FA] ``init_forward_metadata``: the request's ``req_to_token`` row is
    reduced to one entry per page -- the slot of the page's first token,
    integer-divided by ``page_size``, which is the page id. [DCA]
    ``init_forward_metadata`` builds ``block_tables`` the same way. Columns past ``ceil(L_b / page_size)``
    are 0. ``kv_lens`` is ``seq_lens`` as int32 and ``cu_seqlens_k`` its
    zero-led prefix sum (``cache_seqlens_int32`` / ``cu_seqlens_k``).
    """
    req_to_token = np.asarray(req_to_token)
    rpi = np.asarray(req_pool_indices)
    seq_lens = np.asarray(seq_lens)
    batch = len(rpi)
    pt = np.zeros((batch, width), dtype=np.int32)
    for b in range(batch):
        r = int(rpi[b])
        n_pages = -(-int(seq_lens[b]) // page_size)
        for p in range(n_pages):
            pt[b, p] = int(req_to_token[r, p * page_size]) // page_size
    kv_lens = seq_lens.astype(np.int32).copy()
    return pt, kv_lens, cu_seqlens(kv_lens)


def page_table_pa_swa(req_to_token, req_pool_indices, seq_lens, prefill_lens, window, width):
    """Prefill-aware sliding-window token table, by set construction.

    [FA] ``_build_pa_page_table_kernel`` / ``_build_pa_page_table`` (the
    kernel's description of what it keeps): request b keeps its prompt
    positions ``[0, pf)`` and the newest decoded positions
    ``[max(pf, sl - window), sl)``, where ``pf`` is read from the pool-sized
    ``prefill_lens`` at the request's pool row and ``sl = seq_lens[b]``. Only
    positions below ``sl`` exist. The kept positions, in increasing order,
    are mapped through the request's ``req_to_token`` row; ``kv_lens`` is
    their count and the rest of the row is 0 (the destination starts zeroed).
    """
    req_to_token = np.asarray(req_to_token)
    batch = len(req_pool_indices)
    pt = np.zeros((batch, width), dtype=np.int32)
    kv_lens = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        r = int(req_pool_indices[b])
        sl = int(seq_lens[b])
        pf = int(prefill_lens[r])
        prompt = set(range(0, pf))
        recent = set(range(max(pf, sl - window), sl))
        keep = sorted(t for t in prompt | recent if t < sl)
        kv_lens[b] = len(keep)
        for j, t in enumerate(keep):
            pt[b, j] = int(req_to_token[r, t])
    return pt, kv_lens, cu_seqlens(kv_lens)


def visible_key_counts(num_new, kv_len, causal=True) -> np.ndarray:
    """How many leading keys each of a request's new query rows may see.

    The new rows are the last ``num_new`` positions of a ``kv_len``-token
    sequence, so row ``j`` sits at absolute position ``kv_len - num_new + j`` and
    sees keys ``[0, kv_len - num_new + j]`` (bottom-right causal alignment).
    [NSA] ``_cal_indexer_k_start_end`` (``seq_lens_expanded`` runs from
    ``kv_len - extend_len + 1`` to ``kv_len``, with the printed two-request
    example); [DCA] ``_dual_chunk_flash_attn_prefill_func`` starts at
    ``begin = k_length - q_len``. Non-causal rows see all ``kv_len`` keys.
    """
    if not causal:
        return np.full(num_new, kv_len, dtype=np.int64)
    return np.array([kv_len - num_new + j + 1 for j in range(num_new)], dtype=np.int64)


def key_lower_bound(pos, window_left=-1, attn_chunk=0) -> int:
    """First key a query at absolute position ``pos`` may see under a
    lower-bound mask (the upper bound is ``pos`` itself, causal).

    [FA] ``forward_extend`` / ``forward_decode``: ``window_size =
    (sliding_window_size, 0)``, inclusive on both sides, so keys ``pos - W ..
    pos``. [FA] ``make_local_attention_virtual_batches``: chunked local
    attention, keys from the start of ``pos``'s ``attn_chunk``-aligned block
    (the mask drawn for batch 0 of the worked example). Neither: key 0.
    """
    if window_left >= 0 and attn_chunk > 0:
        raise ValueError("a sliding window and local chunks do not combine")
    if window_left >= 0:
        return max(0, pos - window_left)
    if attn_chunk > 0:
        return (pos // attn_chunk) * attn_chunk
    return 0


def local_attention_virtual_batches(attn_chunk, cu_seqlens_q, seq_lens):
    """Chunked local attention as independent causal sub-batches.

    [FA] ``make_local_attention_virtual_batches``: the new rows of a request
    are grouped by the ``attn_chunk``-aligned block their position falls in;
    each group is a batch item whose keys run from the block start to the
    group's last row, with ordinary bottom-right causal alignment inside it.
    Returns, per virtual batch, (request, first q row, q rows, first key, key
    count) in request order. (The page's text is cut short after the q-length
    step; the key ranges follow from the mask it draws.)
    """
    out = []
    for b in range(len(seq_lens)):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        L, M = int(seq_lens[b]), q1 - q0
        j = 0
        while j < M:
            pos = L - M + j
            blk = pos // attn_chunk
            j_end = j
            while j_end < M and (L - M + j_end) // attn_chunk == blk:
                j_end += 1
            last = L - M + j_end - 1
            out.append((b, q0 + j, j_end - j, blk * attn_chunk, last + 1 - blk * attn_chunk))
            j = j_end
    return out


def causal_key_ranges(extend_lens, seq_lens):
    """Per new token, the key range ``[ks, ke)`` in a batch-concatenated key axis.

    [NSA] ``_cal_indexer_k_start_end``: ``ks`` is the request's key offset (the
    running sum of earlier ``seq_lens``) and ``ke = ks + visible count``.
    """
    ks, ke = [], []
    k_offset = 0
    for m, L in zip(extend_lens, seq_lens):
        counts = visible_key_counts(int(m), int(L), causal=True)
        for c in counts:
            ks.append(k_offset)
            ke.append(k_offset + int(c))
        k_offset += int(L)
    return np.array(ks, dtype=np.int64), np.array(ke, dtype=np.int64)


def kv_head_of(q_head, num_q_heads, num_kv_heads) -> int:
    """GQA: q head ``h`` reads kv head ``h // (Hq / Hkv)``.

    [DCA] ``_dual_chunk_flash_attn_prefill_func``: ``current_k[..., head_id //
    group_size, :]`` with ``group_size = num_heads // num_kv_heads``.
    """
    group = num_q_heads // num_kv_heads
    return q_head // group


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def gather_paged(cache, page_row, length, page_size) -> np.ndarray:
    """Logical token ``t`` of a request lives at ``cache[page_row[t // P], t % P]``.

    [FA] ``forward_extend`` views the KV buffer as
    ``[num_pages, page_size, H_kv, D]`` and passes the page table; [DCA]
    ``_get_block`` / the prefill loop gathers whole pages, flattens them and
    truncates to the sequence length.
    """
    out = np.empty((length,) + tuple(cache.shape[2:]), dtype=np.float64)
    for t in range(length):
        out[t] = cache[int(page_row[t // page_size]), t % page_size]
    return out


def softmax_attention(q, keys, values, scale):
    """One query vector against a key set: ``(O, LSE)`` in float64.

    ``s_t = scale * <q, k_t>``; ``LSE = m + ln sum_t exp(s_t - m)`` with
    ``m = max_t s_t``; ``O = sum_t exp(s_t - LSE) v_t``. An empty key set gives
    ``(0, -inf)`` ([DCA] ``_dual_chunk_flash_attn_decoding_with_exp_sums``).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64), NEG_INF
    s = scale * (keys @ q)
    m = np.max(s)
    lse = m + math.log(np.sum(np.exp(s - m)))
    p = np.exp(s - lse)
    return p @ values, lse


def paged_prefill(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, page_size,
                  scale, causal=True, window_left=-1, attn_chunk=0):
    """Varlen extend/prefill over a paged cache.

    [FA] ``forward_extend``: ``flash_attn_with_kvcache`` with
    ``cache_seqlens`` = prefix + new length, ``cu_seqlens_q`` over the new
    tokens and ``causal=True``; the new tokens' keys are already in the cache, so
    each row attends to prefix and new keys through the page table. With a
    sliding window or local chunks (``key_lower_bound``; causal only) row j
    sees keys ``[key_lower_bound(p), p]``, ``p = L - M + j``.

    q: [total_q, Hq, D]; caches: [pages, P, Hkv, Dk|Dv]. Returns
    O [total_q, Hq, Dv] and LSE [total_q, Hq], float64.
    """
    if (window_left >= 0 or attn_chunk > 0) and not causal:
        raise ValueError("lower-bound masks apply to causal rows")
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    total_q, num_q_heads, _ = q.shape
    num_kv_heads = k_cache.shape[2]
    dv = v_cache.shape[3]
    out = np.zeros((total_q, num_q_heads, dv), dtype=np.float64)
    lse = np.full((total_q, num_q_heads), NEG_INF, dtype=np.float64)
    batch = len(kv_lens)
    for b in range(batch):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        L = int(kv_lens[b])
        keys = gather_paged(k_cache, page_table[b], L, page_size)
        vals = gather_paged(v_cache, page_table[b], L, page_size)
        counts = visible_key_counts(q1 - q0, L, causal)
        for j in range(q1 - q0):
            n = int(counts[j])
            lo = key_lower_bound(n - 1, window_left, attn_chunk) if causal else 0
            for h in range(num_q_heads):
                kvh = kv_head_of(h, num_q_heads, num_kv_heads)
                o, l_ = softmax_attention(q[q0 + j, h], keys[lo:n, kvh], vals[lo:n, kvh], scale)
                out[q0 + j, h] = o
                lse[q0 + j, h] = l_
    return out, lse


def kv_append(k_cache, v_cache, out_cache_loc, k_new, v_new):
    """Write the new tokens' keys and values into a paged cache.

    [FA] ``forward_extend`` (and ``forward_decode``): before attending, the
    layer's new ``k`` and ``v`` go into the token pool with ``set_kv_buffer`` at
    ``cache_loc = forward_batch.out_cache_loc``: token slot ``out_cache_loc[i]``
    receives row ``i``. A slot indexes the cache viewed as
    ``[num_pages * page_size, Hkv, D]`` (page ``slot // P``, position ``slot % P``).

    k_new, v_new: [n, Hkv, D]; out_cache_loc: [n] distinct slots. Returns new
    float64 caches; the inputs are left unchanged.
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    loc = np.asarray(out_cache_loc, dtype=np.int64)
    kflat = kc.reshape(-1, kc.shape[2], kc.shape[3])   # views of the copies
    vflat = vc.reshape(-1, vc.shape[2], vc.shape[3])
    kflat[loc] = np.asarray(k_new, dtype=np.float64)
    vflat[loc] = np.asarray(v_new, dtype=np.float64)
    return kc, vc


def paged_prefill_append(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, page_size,
                         scale, out_cache_loc, k_new, v_new, causal=True):
    """[FA] ``forward_extend`` with ``save_kv_cache``: ``kv_append`` of the new
    tokens, then ``paged_prefill`` over the updated cache. Returns
    (O, LSE, k_cache', v_cache')."""
    kc, vc = kv_append(k_cache, v_cache, out_cache_loc, k_new, v_new)
    out, lse = paged_prefill(q, kc, vc, page_table, cu_seqlens_q, kv_lens, page_size, scale,
                             causal)
    return out, lse, kc, vc


def paged_decode_splitkv(q, k_cache, v_cache, page_table, kv_lens, page_size, scale,
                         kv_chunk, num_splits, window_left=-1, attn_chunk=0):
    """Decode (one new token per request) with the key axis cut into chunks.

    Split ``s`` covers keys ``[s*C, min((s+1)*C, L_b))`` and yields the partial
    ``(O_s, LSE_s)`` over that range alone; an empty range yields ``(0, -inf)``.
    [FA] ``forward_decode`` (``flash_attn_with_kvcache`` with ``num_splits``);
    [DCA] ``_dual_chunk_flash_attn_decoding`` runs several paged decodes over
    disjoint key ranges with ``return_softmax_lse=True`` and merges them, and
    ``_dual_chunk_flash_attn_decoding_with_exp_sums`` fixes empty ranges to
    ``(0, -inf)``. ``kv_chunk = 0`` means a single split over all keys. With a
    sliding window or local chunks the query (position ``L - 1``) sees keys
    ``[key_lower_bound(L - 1), L)`` and each split keeps its part of them.

    q: [B, Hq, D]. Returns o_partial [S, B, Hq, Dv] and lse_partial [S, B, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    batch, num_q_heads, _ = q.shape
    num_kv_heads = k_cache.shape[2]
    dv = v_cache.shape[3]
    o_part = np.zeros((num_splits, batch, num_q_heads, dv), dtype=np.float64)
    lse_part = np.full((num_splits, batch, num_q_heads), NEG_INF, dtype=np.float64)
    for b in range(batch):
        L = int(kv_lens[b])
        keys = gather_paged(k_cache, page_table[b], L, page_size)
        vals = gather_paged(v_cache, page_table[b], L, page_size)
        for s in range(num_splits):
            if kv_chunk == 0:
                lo, hi = (0, L) if s == 0 else (L, L)
            else:
                lo, hi = min(s * kv_chunk, L), min((s + 1) * kv_chunk, L)
            if L > 0:
                lo = min(max(lo, key_lower_bound(L - 1, window_left, attn_chunk)), hi)
            for h in range(num_q_heads):
                kvh = kv_head_of(h, num_q_heads, num_kv_heads)
                o, l_ = softmax_attention(q[b, h], keys[lo:hi, kvh], vals[lo:hi, kvh], scale)
                o_part[s, b, h] = o
                lse_part[s, b, h] = l_
    return o_part, lse_part


def merge_state(o_parts, lse_parts):
    """Combine partial states ``(O_s, LSE_s)`` computed over disjoint key sets.

    [DCA] ``_merge_attn_outputs`` and the end of ``_dual_chunk_flash_attn_decoding``:
    ``m = max_s LSE_s``, ``w_s = exp(LSE_s - m)``, ``O = sum_s w_s O_s / sum_s w_s``;
    the merged LSE is ``m + ln sum_s w_s`` (for two parts the page writes it as
    ``max + log1p(exp(-|l0 - l1|))``). [FA] ``forward_extend`` merges a prefix
    pass and an expand pass with ``merge_state_v2(o_a, lse_a, o_b, lse_b)``.
    All parts at -inf give ``(0, -inf)``.

    o_parts: [S, N, H, Dv]; lse_parts: [S, N, H].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    S, N, H, Dv = o_parts.shape
    out = np.zeros((N, H, Dv), dtype=np.float64)
    lse = np.full((N, H), NEG_INF, dtype=np.float64)
    for n in range(N):
        for h in range(H):
            m = max(lse_parts[s, n, h] for s in range(S))
            if m == NEG_INF:
                continue
            w = [math.exp(lse_parts[s, n, h] - m) for s in range(S)]
            total = math.fsum(w)
            acc = np.zeros(Dv, dtype=np.float64)
            for s in range(S):
                if w[s] != 0.0:
                    acc += w[s] * o_parts[s, n, h]
            out[n, h] = acc / total
            lse[n, h] = m + math.log(total)
    return out, lse


# ---------------------------------------------------------------------------
# Cascade attention (speculative target verify with a draft tree)
# ---------------------------------------------------------------------------

def cascade_expand_table(custom_mask, req_to_token, req_pool_indices, seq_lens, num_draft):
    """Per-draft-row key lists for the expand pass of cascade attention.

    [FA] ``init_forward_metadata``, target verify with ``topk > 1`` ("create
    expand page table"): request ``b`` has ``L_b = seq_lens[b]`` committed
    tokens and ``n = num_draft`` draft tokens at positions ``L_b .. L_b+n-1``.
    ``custom_mask`` is flat: request blocks in order, each ``n`` rows of
    ``L_b + n`` entries (row ``i`` of request ``b`` tells which of the
    ``L_b + n`` positions draft token ``i`` may see). The expand pass keeps only
    the draft columns: row ``(b, i)`` lists the slots
    ``req_to_token[req_pool_indices[b], L_b + j]`` of the visible drafts ``j``
    in increasing ``j``, then the masked ones, also in increasing ``j`` (the
    page sorts the keys ``j`` / ``j + n``); its length is the number visible.
    The page's comment prints a three-row example.

    Returns (table [B*n, n] int32 slots, lens [B*n] int32, cu_lens [B*n+1]).
    """
    mask = np.asarray(custom_mask).astype(bool).reshape(-1)
    r2t = np.asarray(req_to_token)
    rpi = np.asarray(req_pool_indices)
    seq_lens = np.asarray(seq_lens)
    n = int(num_draft)
    batch = len(seq_lens)
    table = np.zeros((batch * n, n), dtype=np.int32)
    lens = np.zeros(batch * n, dtype=np.int32)
    start = 0
    for b in range(batch):
        L = int(seq_lens[b])
        drafts = [int(r2t[int(rpi[b]), L + j]) for j in range(n)]
        for i in range(n):
            cols = mask[start + L:start + L + n]
            seen = [j for j in range(n) if cols[j]]
            hidden = [j for j in range(n) if not cols[j]]
            table[b * n + i] = [drafts[j] for j in seen + hidden]
            lens[b * n + i] = len(seen)
            start += L + n
    return table, lens, cu_seqlens(lens)


def tree_verify_attention(q, k_cache, v_cache, req_to_token, req_pool_indices, seq_lens,
                          custom_mask, num_draft, scale):
    """What cascade attention computes, by its plain definition: draft row
    ``(b, i)`` attends over the positions ``t < L_b + n`` its custom-mask row
    allows (all committed tokens and its visible drafts), keys and values read
    at slot ``req_to_token[req_pool_indices[b], t]``.

    [FA] ``forward_extend`` with ``use_cascade_attn`` (target verify with
    ``topk > 1``) splits exactly this attention into a prefix pass and an
    expand pass. Caches are ``[pages, P, Hkv, D]`` (slot ``s`` = page ``s // P``,
    position ``s % P``); q is ``[B*n, Hq, D]``. Returns O, LSE (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    kflat = np.asarray(k_cache).reshape(-1, k_cache.shape[2], k_cache.shape[3])
    vflat = np.asarray(v_cache).reshape(-1, v_cache.shape[2], v_cache.shape[3])
    mask = np.asarray(custom_mask).astype(bool).reshape(-1)
    r2t = np.asarray(req_to_token)
    rpi = np.asarray(req_pool_indices)
    n = int(num_draft)
    total, num_q_heads, _ = q.shape
    num_kv_heads = kflat.shape[1]
    out = np.zeros((total, num_q_heads, vflat.shape[2]), dtype=np.float64)
    lse = np.full((total, num_q_heads), NEG_INF, dtype=np.float64)
    start = 0
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        slots = [int(r2t[int(rpi[b]), t]) for t in range(L + n)]
        for i in range(n):
            row = mask[start:start + L + n]
            vis = [slots[t] for t in range(L + n) if row[t]]
            for h in range(num_q_heads):
                kvh = kv_head_of(h, num_q_heads, num_kv_heads)
                o, l_ = softmax_attention(q[b * n + i, h], kflat[vis, kvh], vflat[vis, kvh],
                                          scale)
                out[b * n + i, h] = o
                lse[b * n + i, h] = l_
            start += L + n
    return out, lse


def cascade_attention(q, k_cache, v_cache, page_table, seq_lens, page_size, expand_table,
                      expand_lens, scale):
    """Cascade attention in the pages' three steps.

    [FA] ``forward_extend`` / ``forward_decode`` with ``use_cascade_attn``:
    (1) prefix pass -- the ``n`` draft rows of request ``b``
    (``cu_seqlens_q`` in steps of ``n``) attend non-causally over its ``L_b``
    committed tokens through the page table, returning LSE; (2) expand pass --
    every draft row is its own one-token request whose keys are the slots
    ``expand_table[row, :expand_lens[row]]`` of the cache viewed with page
    size 1, non-causal, returning LSE; (3) ``merge_state_v2`` of the two.

    Returns O [B*n, Hq, Dv], LSE [B*n, Hq] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    total = q.shape[0]
    batch = len(seq_lens)
    n = total // batch
    cu = np.arange(0, total + 1, n)
    o1, l1 = paged_prefill(q, k_cache, v_cache, page_table, cu, seq_lens, page_size, scale,
                           causal=False)
    k1 = np.asarray(k_cache).reshape(-1, 1, k_cache.shape[2], k_cache.shape[3])
    v1 = np.asarray(v_cache).reshape(-1, 1, v_cache.shape[2], v_cache.shape[3])
    o2, l2 = paged_decode_splitkv(q, k1, v1, np.asarray(expand_table), expand_lens, 1, scale,
                                  0, 1)
    return merge_state(np.stack([o1, o2[0]]), np.stack([l1, l2[0]]))


# ---------------------------------------------------------------------------
# Dual chunk attention, decode (intra / succ / inter stages)
# ---------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), returned
    as float32: keep the upper 16 bits of the IEEE single after adding half an
    upper-unit (minus one when the kept part is even). NaN stays NaN."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32)
    return np.where(np.isnan(f), f, out)


def dca_scaling_factor(seq_lens, original_max_position_embeddings) -> np.ndarray:
    """[DCA] ``init_forward_metadata``: with ``original_max_position_embeddings
    > 0`` each request's queries are multiplied by
    ``max(0.1 * ln(L / original_max_position_embeddings) + 1, 1)``."""
    L = np.asarray(seq_lens, dtype=np.float64)
    return np.maximum(0.1 * np.log(L / float(original_max_position_embeddings)) + 1.0, 1.0)


def dca_query_chunk(seq_lens, chunk_len) -> np.ndarray:
    """[DCA] ``init_forward_metadata`` (decode): the chunk holding the query,
    ``chunk_num_curr = (L - 1) // chunk_len``."""
    return (np.asarray(seq_lens, dtype=np.int64) - 1) // int(chunk_len)


def dca_decode_tables(block_tables, seq_lens, chunk_size, local_size, page_size):
    """Per-request key ranges of the three decode stages and the page tables
    that read them.

    [DCA] ``init_forward_metadata`` (decode) and
    ``_dual_chunk_flash_attn_decoding``: with chunk length
    ``C = chunk_size - local_size`` and ``c = (L - 1) // C`` the chunk that
    holds the query (a request of length 0 counts as chunk 0), the stages
    read these key positions of the request:
      intra -- the query's own chunk, ``[c*C, L)``;
      succ  -- the whole chunk before it, ``[(c-1)*C, c*C)``, none when c = 0;
      inter -- everything earlier, ``[0, (c-1)*C)``, read through the
               request's own ``block_tables`` row.
    A stage's table row lists the pages that hold its positions, in order,
    taken from the request's ``block_tables`` row, and is 0 after them; rows
    are ``C // page_size`` wide (a stage never spans more than one chunk).
    Positions start at multiples of ``C``, a multiple of ``page_size``, so a
    stage's first position is the first slot of its first page.

    Returns dict(lens_intra, table_intra, lens_succ, table_succ, lens_inter),
    int64 arrays.
    """
    bt = np.asarray(block_tables, dtype=np.int64)
    L_all = np.asarray(seq_lens, dtype=np.int64)
    batch = len(L_all)
    C = int(chunk_size) - int(local_size)
    P = int(page_size)
    assert C % P == 0, "chunk length must be a multiple of the page size"
    width = C // P
    tables = {"intra": np.zeros((batch, width), dtype=np.int64),
              "succ": np.zeros((batch, width), dtype=np.int64)}
    lens = {k: np.zeros(batch, dtype=np.int64) for k in ("intra", "succ", "inter")}
    for b in range(batch):
        L = int(L_all[b])
        c = max(int(dca_query_chunk([L], C)[0]), 0)
        ranges = {"intra": range(c * C, L),
                  "succ": range((c - 1) * C, c * C) if c >= 1 else range(0),
                  "inter": range(0, max(c - 1, 0) * C)}
        for name, positions in ranges.items():
            lens[name][b] = len(positions)
            if name == "inter":
                continue
            pages = sorted({t // P for t in positions})
            for j, page in enumerate(pages):
                tables[name][b, j] = bt[b, page]
    return dict(lens_intra=lens["intra"], table_intra=tables["intra"], lens_succ=lens["succ"],
                table_succ=tables["succ"], lens_inter=lens["inter"])


def dca_decode(q, q_succ, q_inter, k_cache, v_cache, block_tables, seq_lens, page_size, scale,
               chunk_size, local_size, original_max_position_embeddings=0, q_bf16=True):
    """Dual chunk attention decode in the page's three stages.

    [DCA] ``_dual_chunk_flash_attn_decoding``: (optionally) scale the three
    queries per request by ``dca_scaling_factor`` and round them back to the
    query dtype; run a non-causal paged decode per stage -- ``q`` over the
    intra table, ``q_succ`` over the succ table, ``q_inter`` over the full
    table with the inter lengths -- each returning LSE, an empty stage giving
    ``(0, -inf)`` (``_dual_chunk_flash_attn_decoding_with_exp_sums``); merge
    the stages by their LSEs. Returns O [B, Hq, D] and the merged LSE.
    """
    qs = [np.asarray(x, dtype=np.float64) for x in (q, q_succ, q_inter)]
    if original_max_position_embeddings > 0:
        sf = dca_scaling_factor(seq_lens, original_max_position_embeddings).astype(np.float32)
        scaled = []
        for x in qs:
            y = x.astype(np.float32) * sf[:, None, None]
            scaled.append((round_to_bf16(y) if q_bf16 else y).astype(np.float64))
        qs = scaled
    t = dca_decode_tables(block_tables, seq_lens, chunk_size, local_size, page_size)
    parts_o, parts_l = [], []
    o, l_ = paged_decode_splitkv(qs[0], k_cache, v_cache, t["table_intra"], t["lens_intra"],
                                 page_size, scale, 0, 1)
    parts_o.append(o[0])
    parts_l.append(l_[0])
    if int(t["lens_succ"].max()) > 0:
        o, l_ = paged_decode_splitkv(qs[1], k_cache, v_cache, t["table_succ"], t["lens_succ"],
                                     page_size, scale, 0, 1)
        parts_o.append(o[0])
        parts_l.append(l_[0])
    if int(t["lens_inter"].max()) > 0:
        o, l_ = paged_decode_splitkv(qs[2], k_cache, v_cache, np.asarray(block_tables),
                                     t["lens_inter"], page_size, scale, 0, 1)
        parts_o.append(o[0])
        parts_l.append(l_[0])
    return merge_state(np.stack(parts_o), np.stack(parts_l))


def dca_decode_reference(q, q_succ, q_inter, k_cache, v_cache, block_tables, seq_lens,
                         page_size, scale, chunk_len):
    """The plain definition the three stages reach: one softmax over all ``L``
    keys in which key ``t`` is scored with the query of its stage -- ``q`` in
    the query's own chunk ``[c*chunk_len, L)``, ``q_succ`` in the chunk before
    it, ``q_inter`` before that (``c = (L - 1) // chunk_len``)."""
    qs = [np.asarray(x, dtype=np.float64) for x in (q, q_succ, q_inter)]
    batch, num_q_heads, _ = qs[0].shape
    num_kv_heads = k_cache.shape[2]
    out = np.zeros((batch, num_q_heads, v_cache.shape[3]), dtype=np.float64)
    lse = np.full((batch, num_q_heads), NEG_INF, dtype=np.float64)
    for b in range(batch):
        L = int(seq_lens[b])
        keys = gather_paged(k_cache, block_tables[b], L, page_size)
        vals = gather_paged(v_cache, block_tables[b], L, page_size)
        c = (L - 1) // chunk_len
        stage = np.where(np.arange(L) >= c * chunk_len, 0,
                         np.where(np.arange(L) >= (c - 1) * chunk_len, 1, 2))
        for h in range(num_q_heads):
            kvh = kv_head_of(h, num_q_heads, num_kv_heads)
            s = np.array([scale * float(qs[stage[t]][b, h] @ keys[t, kvh]) for t in range(L)])
            m = s.max()
            w = np.exp(s - m)
            total = math.fsum(w)
            out[b, h] = (w[:, None] * vals[:, kvh]).sum(axis=0) / total
            lse[b, h] = m + math.log(total)
    return out, lse


def sparse_topk_decode(q, kv_cache, req_to_token, req_pool_indices, topk_idx, scale,
                       head_dim_v):
    """Top-k index-gathered MLA decode over one latent KV head.

    [NSA] ``forward_decode``: the top-k *logical* token indices are mapped to
    cache slots through the request's token table
    (``transform_index_page_table_decode`` with page size 1), and entries equal
    to -1 are padding that is skipped (``_pad_topk_indices`` pads with -1;
    ``_forward_aiter`` keeps only entries ``!= -1``). [NSA] ``_forward_fa3``
    fixes the arithmetic: the cache row is ``[c_kv (first Dv) | k_rope (rest)]``,
    the score adds ``q_rope . k_rope`` and ``q_nope . c_kv`` -- a dot product over
    the whole row with ``q = [q_nope | q_rope]`` -- and the value is ``c_kv``.

    q: [B, Hq, Dqk]; kv_cache: [slots, Dqk]; topk_idx: [B, K] (may hold -1).
    Returns O [B, Hq, Dv] and LSE [B, Hq], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    kv_cache = np.asarray(kv_cache)
    batch, num_heads, _ = q.shape
    out = np.zeros((batch, num_heads, head_dim_v), dtype=np.float64)
    lse = np.full((batch, num_heads), NEG_INF, dtype=np.float64)
    for b in range(batch):
        r = int(req_pool_indices[b])
        slots = [int(req_to_token[r, int(i)]) for i in topk_idx[b] if int(i) != -1]
        rows = np.zeros((len(slots), kv_cache.shape[-1]), dtype=np.float64)
        for j, s in enumerate(slots):
            rows[j] = kv_cache[s]
        keys = rows
        vals = rows[:, :head_dim_v]
        for h in range(num_heads):
            o, l_ = softmax_attention(q[b, h], keys, vals, scale)
            out[b, h] = o
            lse[b, h] = l_
    return out, lse

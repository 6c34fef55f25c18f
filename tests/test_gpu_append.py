"""KV append (set_kv_buffer at out_cache_loc) and the extend step with its
cache write, on the GPU versus the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_197_amd as pkv
import workloads
from helpers import LSE_TOL, O_TOL, assert_close, compact_pages, np_f, np_i, say, to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("dtype,P,hkv,d,n", [(torch.bfloat16, 1, 8, 128, 300),
                                             (torch.bfloat16, 16, 2, 64, 77),
                                             (torch.float32, 4, 3, 64, 5),
                                             (torch.bfloat16, 64, 8, 128, 0)])
def test_kv_append_matches_oracle(dtype, P, hkv, d, n):
    g = torch.Generator().manual_seed(7 + n)
    pages = max(4, (n + 50) // P + 2)
    kc = torch.randn((pages, P, hkv, d), generator=g).to(dtype)
    vc = torch.randn((pages, P, hkv, d), generator=g).to(dtype)
    loc = torch.randperm(pages * P, generator=g)[:n].to(torch.int32)
    kn = torch.randn((n, hkv, d), generator=g).to(dtype)
    vn = torch.randn((n, hkv, d), generator=g).to(dtype)
    ek, ev = oracle.kv_append(np_f(kc), np_f(vc), np_i(loc), np_f(kn), np_f(vn))
    gk, gv = kc.to(DEV), vc.to(DEV)
    say(f"kv_append {dtype} P={P} Hkv={hkv} D={d} n={n}")
    pkv.paged_kv_append(kn.to(DEV), vn.to(DEV), loc.to(DEV), gk, gv)
    torch.cuda.synchronize()
    assert np.array_equal(np_f(gk), ek) and np.array_equal(np_f(gv), ev)


def test_kv_append_skips_out_of_range_slots():
    kc = torch.zeros((4, 2, 1, 64), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = torch.ones((3, 1, 64), dtype=torch.bfloat16, device=DEV)
    loc = torch.tensor([1, 8, -3], dtype=torch.int32, device=DEV)   # slots 8 and -3 are outside
    say("kv_append out-of-range slots")
    pkv.paged_kv_append(kn, kn, loc, kc, vc)
    torch.cuda.synchronize()
    flat = kc.view(8, 1, 64)
    assert torch.all(flat[1] == 1) and torch.all(flat[torch.tensor([0, 2, 3, 4, 5, 6, 7])] == 0)


def _split_new_tokens(c):
    """out_cache_loc and the new rows of a prefill case; the new rows' slots in
    the cache are then poisoned, so only the appended values can be read."""
    r2t, rpi = np_i(c.req_to_token), np_i(c.req_pool_indices)
    pre = np_i(c.seq_lens) - np_i(c.extend_lens)
    loc = np.concatenate([r2t[rpi[b], pre[b]:pre[b] + int(c.extend_lens[b])]
                          for b in range(len(pre))]).astype(np.int64)
    loc_t = torch.as_tensor(loc, device=c.k_cache.device)
    hkv, d = c.k_cache.shape[2], c.k_cache.shape[3]
    kflat = c.k_cache.view(-1, hkv, d)
    vflat = c.v_cache.view(-1, hkv, d)
    kn, vn = kflat[loc_t].clone(), vflat[loc_t].clone()
    kflat[loc_t] = float("nan")
    vflat[loc_t] = float("nan")
    return loc_t.to(torch.int32), kn, vn


def _run_append_case(c, causal=True):
    loc, kn, vn = _split_new_tokens(c)
    pt, kl, _ = pkv.build_page_table(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                                     c.table_width)
    out = torch.full_like(c.q, float("nan"))
    lse = torch.full(c.q.shape[:2], float("nan"), device=DEV)
    pkv.paged_attn_varlen_prefill(c.q, c.k_cache, c.v_cache, pt, c.cu_seqlens_q, kl,
                                  c.max_seqlen_q, c.scale, causal=causal, out=out, lse=lse,
                                  k_new=kn, v_new=vn, out_cache_loc=loc)
    torch.cuda.synchronize()
    # the cache now holds the new rows at their slots
    hkv, d = c.k_cache.shape[2], c.k_cache.shape[3]
    assert torch.equal(c.k_cache.view(-1, hkv, d)[loc.long()], kn)
    assert torch.equal(c.v_cache.view(-1, hkv, d)[loc.long()], vn)
    pt_np, kl_np = np_i(pt), np_i(kl)
    rows = list(range(len(kl_np)))
    k_small, pt_small = compact_pages(c.k_cache, pt_np, kl_np, c.page_size, rows)
    v_small, _ = compact_pages(c.v_cache, pt_np, kl_np, c.page_size, rows)
    ro, rl = oracle.paged_prefill(np_f(c.q), k_small, v_small, pt_small, np_i(c.cu_seqlens_q),
                                  kl_np, c.page_size, c.scale, causal=causal)
    assert_close("out", np_f(out), ro, O_TOL)
    assert_close("lse", np_f(lse), rl, LSE_TOL)


def test_prefill_append_config2():
    c = to_device(workloads.config2(value_device=DEV), DEV)
    say("config2 extend with its cache write (new slots poisoned)")
    _run_append_case(c)


@pytest.mark.parametrize("D,P,group,hkv", [(128, 16, 8, 2), (64, 1, 3, 2), (128, 64, 4, 1)])
def test_prefill_append_shapes(D, P, group, hkv):
    prefix = [2000, 0, 31, 300]
    extend = [40, 65, 1, 129]
    total = sum(p + e for p, e in zip(prefix, extend))
    c = workloads.make_prefill_case(120 + D + P + group, prefix_lens=prefix, extend_lens=extend,
                                    num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=D,
                                    page_size=P, num_pages=total // P + len(prefix) + 4)
    c = to_device(c, DEV)
    say(f"extend with cache write D={D} P={P} G={group} Hkv={hkv}")
    _run_append_case(c)

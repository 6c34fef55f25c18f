// Split order of the split-KV kernels: which (request, split) a workgroup
// of a flat grid takes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.hpp"

namespace pkv {

// Which (request, split) a workgroup takes. Workgroups start in index order
// as CU slots free up, so the grid is dealt out longest piece first (list
// scheduling, longest first): every split holding a whole chunk of visible
// keys, then the partial ones by decreasing length (ties by request, then
// split), then the empty ones, which only write (0, -inf). In the plain
// split-major order the long requests' last full splits start late and run
// alone at the end. Unit u is the workgroup's index over (request, split)
// pairs; the result is wave-uniform. Up to 64 requests (one per lane);
// larger batches keep the split-major order. `lo_on`: keys below the
// window's / local chunk's lower bound are not visible.
struct SplitPick {
  int b, s, L;
};

__device__ inline SplitPick pick_split(const DecodeArgs& a, int u, bool lo_on, int lane) {
  const int S = a.num_splits;
  const int64_t cap = static_cast<int64_t>(a.pt_stride) * a.page_size;
  if (a.batch > 64 || S == 1) {
    const int b = u % a.batch;
    const int L = static_cast<int>(min<int64_t>(max(a.kv_lens[b], 0), cap));
    return {b, u / a.batch, L};
  }
  const int C = a.chunk;
  const bool in = lane < a.batch;
  const int L = in ? static_cast<int>(min<int64_t>(max(a.kv_lens[lane], 0), cap)) : 0;
  // visible keys [v0, v1) of request `lane` within the S splits
  const int v1 = static_cast<int>(min<int64_t>(L, static_cast<int64_t>(S) * C));
  const int lo = (lo_on && L > 0) ? key_lower_bound(L - 1, a.window_left, a.attn_chunk) : 0;
  const int v0 = min(lo, v1);
  const bool any = in && v0 < v1;
  const int sf = any ? v0 / C : 0;                       // first non-empty split
  const int sl = any ? (v1 - 1) / C : -1;                // last non-empty split
  const int f_lo = any ? (v0 + C - 1) / C : 0;           // full splits [f_lo, f_hi)
  const int f_hi = any ? v1 / C : 0;
  const int nf = max(f_hi - f_lo, 0);
  const int ne = in ? S - (sl - sf + 1) : 0;
  // the (at most two) partial splits and their visible lengths (0: none)
  const bool p0_on = any && (sf < f_lo || sf >= f_hi);
  const bool p1_on = any && sl != sf && sl >= f_hi;
  const int w0 = p0_on ? static_cast<int>(min<int64_t>(static_cast<int64_t>(sf + 1) * C, v1)) - v0 : 0;
  const int w1 = p1_on ? v1 - sl * C : 0;
  const int np = (p0_on ? 1 : 0) + (p1_on ? 1 : 0);
  // exclusive prefix sums over the requests
  int xf = nf, xp = np, xe = ne;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int yf = __shfl_up(xf, d), yp = __shfl_up(xp, d), ye = __shfl_up(xe, d);
    if (lane >= d) {
      xf += yf;
      xp += yp;
      xe += ye;
    }
  }
  const int F = __builtin_amdgcn_readlane(xf, 63);
  const int P = __builtin_amdgcn_readlane(xp, 63);
  xf -= nf;
  xp -= np;
  xe -= ne;
  int b, s;
  if (u < F) {
    const unsigned long long hit = __ballot(nf > 0 && u >= xf && u < xf + nf);
    b = hit ? __builtin_ctzll(hit) : 0;   // (never empty: the pairs are a bijection)
    s = __builtin_amdgcn_readlane(f_lo, b) + u - __builtin_amdgcn_readlane(xf, b);
  } else if (u < F + P) {
    // rank of each of this lane's partials: how many come before it
    const int r = u - F;
    int r0 = 0, r1 = 0;
    for (int j = 0; j < a.batch; ++j) {
      const int a0 = __builtin_amdgcn_readlane(w0, j), a1 = __builtin_amdgcn_readlane(w1, j);
      r0 += (a0 > w0 || (a0 == w0 && j < lane)) ? 1 : 0;
      r0 += (a1 > w0 || (a1 == w0 && j < lane)) ? 1 : 0;
      r1 += (a0 > w1 || (a0 == w1 && j <= lane)) ? 1 : 0;
      r1 += (a1 > w1 || (a1 == w1 && j < lane)) ? 1 : 0;
    }
    const bool h0 = p0_on && r0 == r, h1 = p1_on && r1 == r;
    const unsigned long long hit = __ballot(h0 || h1);
    b = hit ? __builtin_ctzll(hit) : 0;   // (never empty: the pairs are a bijection)
    s = __builtin_amdgcn_readlane(h0 ? sf : sl, b);
  } else {
    const int r = u - F - P;
    const unsigned long long hit = __ballot(ne > 0 && r >= xe && r < xe + ne);
    b = hit ? __builtin_ctzll(hit) : 0;   // (never empty: the pairs are a bijection)
    const int k = r - __builtin_amdgcn_readlane(xe, b);
    const int sfb = __builtin_amdgcn_readlane(sf, b), slb = __builtin_amdgcn_readlane(sl, b);
    s = (k < sfb) ? k : slb + 1 + (k - sfb);
  }
  s = min(max(s, 0), S - 1);
  return {b, s, __builtin_amdgcn_readlane(L, b)};
}

}  // namespace pkv

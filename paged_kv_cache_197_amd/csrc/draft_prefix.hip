// Prefix pass of draft-tree verification on packed query rows.
// [FA] forward_extend / forward_decode with use_cascade_attn: every draft row
// of a request attends, without a causal mask, to all of the request's
// committed keys; the drafts' own keys follow in the expand pass, which also
// merges the two. A request contributes M_b draft rows; with G query heads
// per kv head the G * M_b (head, draft) rows of one kv head fit one 32-row
// MFMA tile when G * M_b <= 32, and this kernel packs them there (packed row
// n = draft n / G, head n % G of the kv head) instead of spending a 32-row
// tile of the prefill kernel per head on M_b rows.
//
// Work decomposition: one workgroup per (request, key split, group of W
// adjacent kv heads); wave w takes kv head W * group + w over every 32-key
// tile of the split, so that the workgroup's waves read the W adjacent row
// slices of each token together (with W = 4 and D = 128, 1 KB of contiguous
// K and of V per token). A wave loads its next tile's K and V rows into
// registers while it computes the current one from its private LDS region,
// then writes them there: no workgroup barrier at all. The (request, split)
// pairs are handed out longest first. A launch with one split writes out /
// lse; otherwise every split writes its normalised partial (bf16, the output
// precision) and LSE to the workspace, and draft_merge_kernel combines them
// in split order into out / lse (a second, short launch: it reads the
// partials once, where a merge by the last split inside the launch would add
// a device-scope hand-off to every workgroup).
//
// Per wave and key tile (32x32x16 bf16 MFMA), as in the prefill kernel:
//   S^T [32 keys x 32 rows] = K [32 x D] . Q^T [D x 32]
//   O^T [D x 32 rows]      += V^T [D x 32 keys] . P^T [32 x 32]
// Lane (n = lane % 32, h = lane / 32) owns packed row n: its S^T registers
// hold keys rho(h, r) = 8 (r / 4) + 4h + r % 4, which are the keys its P^T
// operand needs for the two 16-key k-steps, and its O^T registers hold dims
// of row n. LDS rows are D * 2 bytes with their 16-byte chunks XOR-swizzled
// by the row, so that a K operand read (16 rows, one chunk) and a transposed
// V read (ds_read_b64_tr_b16) meet distinct banks.
#include "args.hpp"
#include "common.hpp"
#include "lanes.hpp"
#include "launch.hpp"
#include "splits.hpp"

namespace pkv {

template <int D>
struct DraftPrefix {
  static constexpr int KT = 32;               // keys per tile
  static constexpr int NKS = D / 16;          // 16-wide k-steps of S^T
  static constexpr int NB = D / 32;           // 32-dim blocks of O^T
  static constexpr int ROW = D * 2;           // bytes of one kv head's key row
  static constexpr int CH = ROW / 16;         // 16-byte chunks per row
  static constexpr int TILE = KT * ROW;       // one tensor's tile
  static constexpr int WAVE_LDS = 2 * TILE;   // a wave's K and V tiles
  static constexpr int RPI = 1024 / ROW;      // rows per 1 KB load instruction
  static constexpr int NLD = KT / RPI;        // load instructions per tensor and tile
  static constexpr int SWZ = 256 / ROW;       // rows sharing one 64-bank span
  static constexpr float kRescaleLog2 = 8.f;  // lazy rescale bound (log2 units)

  static __device__ __forceinline__ int rho(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }
  // LDS chunk position of global chunk c of key row k (an involution in c)
  static __device__ __forceinline__ int swz(int k, int c) {
    const int u = (k / SWZ) % CH;
    return c ^ (((2 * u) % CH) | ((2 * u) / CH));
  }

  struct Stage {
    u32x4 k[NLD];
    u32x4 v[NLD];
  };

  static __device__ __forceinline__ u32x4 ld_nt(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }

  // Page-table entries of the tile at key ts: load i of lane l covers row
  // RPI i + l / CH (keys past the split's end repeat its last key).
  static __device__ __forceinline__ void fetch_entries(const DecodeArgs& d, const int32_t* pt_row,
                                                       int ts, int end, int lane,
                                                       int32_t (&raw)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int t = min(ts + RPI * i + lane / CH, end - 1);
      raw[i] = pt_row[t / d.page_size];
    }
  }

  // Row RPI i + l / CH of the tile, LDS chunk l % CH: global chunk
  // swz(row, l % CH) of the kv head's slice, for K and V.
  static __device__ __forceinline__ void load(const DecodeArgs& d, const int32_t (&raw)[NLD],
                                              int ts, int end, int lane, int64_t row_bytes,
                                              const char* kb, const char* vb, Stage& st) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int row = RPI * i + lane / CH;
      const int t = min(ts + row, end - 1);
      const int64_t slot = clamp_index(raw[i], d.num_pages) * d.page_size + t % d.page_size;
      const int64_t off = slot * row_bytes + swz(row, lane % CH) * 16;
      st.k[i] = ld_nt(kb + off);
      st.v[i] = ld_nt(vb + off);
    }
  }

  static __device__ __forceinline__ void stash(char* my, int lane, const Stage& st) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int o = (RPI * i + lane / CH) * ROW + (lane % CH) * 16;
      *reinterpret_cast<u32x4*>(my + o) = st.k[i];
      *reinterpret_cast<u32x4*>(my + TILE + o) = st.v[i];
    }
  }

  // Online-softmax state of the lane's row (equal in lanes n and n + 32): m
  // is a reference max in raw score units (-inf before the first key), moved
  // only when a score passes thr = m + kRescaleLog2 / c, so the exponentials
  // p = exp2(s c - m c) stay below 2^kRescaleLog2 while few tiles rescale; the
  // sum and the output share the reference. l is the lane's half-row sum.
  struct RowState {
    float m, thr, neg_mc, l;
  };

  // One key tile from the wave's LDS region: keys rho(h, r) >= nvalid are past
  // the split's end.
  static __device__ __forceinline__ void compute(const char* my, int lane, int nvalid, float c,
                                                 float step, const u32x4 (&qop)[NKS],
                                                 const int (&vofs)[2][NB], f32x16 (&acc)[NB],
                                                 RowState& st) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) char lds_char;
    const int q = lane & 31;
    const int h = lane >> 5;
    u32x4 kw[NKS];
#pragma unroll
    for (int j = 0; j < NKS; ++j)
      kw[j] = *reinterpret_cast<const u32x4*>(my + q * ROW + swz(q, 2 * j + h) * 16);
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NKS; ++j)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw[j]), as_bf16x8(qop[j]), s, 0, 0, 0);
    // V^T operands (see below) of the first 16-key step, in flight with the
    // softmax; the second step's follow the exponentials
    s16x4 vt[2][NB][2];
    auto read_vt = [&](int t) {
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          vt[t][n][s2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(
              (lds_char*)my + TILE + vofs[s2][n] + 16 * t * ROW));
    };
    read_vt(0);

    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = s[r];
    if (nvalid < KT) {   // wave-uniform: only a split's last tile
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (rho(h, r) >= nvalid) x[r] = neg_inf();
    }
    float mt = __builtin_amdgcn_fmed3f(x[0], x[1], __builtin_inff());
#pragma unroll
    for (int r = 2; r < 16; ++r) mt = fmaxf(mt, x[r]);
    if (__any(mt > st.thr)) {
      mt = max_xor32(mt);
      const bool grow = mt > st.thr;
      const float m_ref = grow ? mt : st.m;
      const float m_use = (m_ref == neg_inf()) ? 0.f : m_ref;
      const float alpha = grow ? fast_exp2((st.m - m_use) * c) : 1.f;
      st.m = m_ref;
      st.neg_mc = -m_use * c;
      st.thr = (m_ref == neg_inf()) ? neg_inf() : m_ref + step;
      st.l *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(x[r], c, st.neg_mc));
    read_vt(1);
    float ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ps[i] = (p[4 * i] + p[4 * i + 1]) + (p[4 * i + 2] + p[4 * i + 3]);
    st.l += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    // O^T block n row m = dim 32n + m; its A operand for the 16-key step t is
    // V^T[32n + m][keys 16t + 8(e/4) + 4h + e%4], e = 0..7: two transposed
    // 8-byte LDS reads, each turning 16 lanes' row-major 4-dim pieces of 4
    // keys into one dim's 4 keys per lane (vofs).
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pw = {pack_bf16x2(p[8 * t + 0], p[8 * t + 1]), pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                        pack_bf16x2(p[8 * t + 4], p[8 * t + 5]), pack_bf16x2(p[8 * t + 6], p[8 * t + 7])};
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const u32x2 lo = __builtin_bit_cast(u32x2, vt[t][n][0]);
        const u32x2 hi = __builtin_bit_cast(u32x2, vt[t][n][1]);
        const u32x4 vw = {lo.x, lo.y, hi.x, hi.y};
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), as_bf16x8(pw), acc[n], 0,
                                                         0, 0);
      }
    }
  }

  // bf16 row of lane row n, scaled: acc block n, registers 4a..4a+3 are the
  // 4 consecutive dims 32n + 8a + 4h + [0, 4)
  static __device__ __forceinline__ void store_row(bf16_t* dst, int h, const f32x16 (&acc)[NB],
                                                   float scale) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 w;
        w.x = pack_bf16x2(acc[n][4 * a4] * scale, acc[n][4 * a4 + 1] * scale);
        w.y = pack_bf16x2(acc[n][4 * a4 + 2] * scale, acc[n][4 * a4 + 3] * scale);
        *reinterpret_cast<u32x2*>(dst + 32 * n + 8 * a4 + 4 * h) = w;
      }
  }

  template <int W>
  static __device__ void run(const DraftPrefixArgs& A) {
    extern __shared__ __align__(16) char smem[];
    const DecodeArgs& d = A.d;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ngrp = d.hkv / W;
    const int grp = blockIdx.x % ngrp;
    const SplitPick pk = pick_split(d, blockIdx.x / ngrp, false, lane);
    const int b = __builtin_amdgcn_readfirstlane(pk.b);
    const int s = __builtin_amdgcn_readfirstlane(pk.s);
    const int L = __builtin_amdgcn_readfirstlane(pk.L);
    const int G = d.hq / d.hkv;
    const int kvh = grp * W + wave;
    // request b's rows, kept inside [0, total_q) whatever cu_q holds
    const int q0 = min(max(A.cu_q[b], 0), A.total_q);
    const int M = min(min(max(A.cu_q[b + 1] - q0, 0), KT / G), A.total_q - q0);
    if (M <= 0) return;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int jd = col / G;
    const bool row_ok = jd < M;
    // (token, head) row of q / out of packed row col
    const int64_t orow = static_cast<int64_t>(q0 + min(jd, M - 1)) * d.hq + kvh * G + (col - jd * G);
    const bool single = d.num_splits == 1;
    const int64_t part = static_cast<int64_t>(s) * A.total_q * d.hq;   // split s's first row
    const int start = static_cast<int>(min<int64_t>(static_cast<int64_t>(s) * d.chunk, L));
    // (the last split also takes any keys past num_splits * chunk)
    const int end = s == d.num_splits - 1
                        ? L
                        : static_cast<int>(min<int64_t>(static_cast<int64_t>(start) + d.chunk, L));

    if (start >= end) {   // no key in this split
      if (!row_ok) return;
      if (single) {   // (L == 0) output 0, LSE -inf
        bf16_t* dst = static_cast<bf16_t*>(d.out) + orow * D + h * (D / 2);
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
          *reinterpret_cast<u32x4*>(dst + 8 * i) = u32x4{0u, 0u, 0u, 0u};
        if (h == 0) d.lse[orow] = neg_inf();
      } else if (h == 0) {
        A.part_lse[part + orow] = neg_inf();   // the merge skips this split
      }
      return;
    }

    // Q^T operand, k-step j: dims 16j + 8h + [0, 8) of packed row col (zero
    // in the rows past the request's drafts)
    u32x4 qop[NKS];
    {
      const char* qrow = static_cast<const char*>(d.q) + orow * ROW;
#pragma unroll
      for (int j = 0; j < NKS; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + (16 * j + 8 * h) * 2);
        qop[j] = row_ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // Transposed V read (s2, n) of lane (g = lane / 16, j = lane % 16): key row
    // 8 s2 + 4 (g / 2) + j / 4 (+16 t), dims 32n + 16 (g % 2) + 4 (j % 4) + [0, 4).
    int vofs[2][NB];
    {
      const int g = lane >> 4, j = lane & 15;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int row = 8 * s2 + 4 * (g >> 1) + (j >> 2);
          const int byte = 2 * (32 * n + 16 * (g & 1) + 4 * (j & 3));
          vofs[s2][n] = row * ROW + swz(row, byte / 16) * 16 + byte % 16;
        }
    }

    char* my = smem + wave * WAVE_LDS;
    const int64_t row_bytes = static_cast<int64_t>(d.hkv) * ROW;
    const char* kb = static_cast<const char*>(d.k) + static_cast<int64_t>(kvh) * ROW;
    const char* vb = static_cast<const char*>(d.v) + static_cast<int64_t>(kvh) * ROW;
    const int32_t* pt_row = d.pt + static_cast<int64_t>(b) * d.pt_stride;
    const int n_t = (end - start + KT - 1) / KT;
    const float c = d.scale_log2;
    const float step = kRescaleLog2 / c;
    f32x16 acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
    RowState st{neg_inf(), neg_inf(), 0.f, 0.f};

    Stage stg;
    int32_t raw[NLD];
    fetch_entries(d, pt_row, start, end, lane, raw);
    load(d, raw, start, end, lane, row_bytes, kb, vb, stg);
    if (n_t > 1) fetch_entries(d, pt_row, start + KT, end, lane, raw);
    stash(my, lane, stg);
    for (int t = 0;; ++t) {
      const int ts = start + KT * t;
      const bool more = t + 1 < n_t;
      if (more) {
        load(d, raw, ts + KT, end, lane, row_bytes, kb, vb, stg);
        if (t + 2 < n_t) fetch_entries(d, pt_row, ts + 2 * KT, end, lane, raw);
      }
      __builtin_amdgcn_sched_barrier(0);   // the next tile's loads go out before the MFMAs
      compute(my, lane, min(KT, end - ts), c, step, qop, vofs, acc, st);
      if (!more) break;
      stash(my, lane, stg);   // same wave: its LDS reads above complete first
    }

    const float l_tot = st.l + __shfl_xor(st.l, 32);
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_val = l_tot > 0.f ? (st.m * c + fast_log2(l_tot)) * kLn2 : neg_inf();
    if (single) {
      store_row(static_cast<bf16_t*>(d.out) + orow * D, h, acc, inv);
      if (h == 0) d.lse[orow] = lse_val;
    } else {
      store_row(static_cast<bf16_t*>(A.part_o) + (part + orow) * D, h, acc, inv);
      if (h == 0) A.part_lse[part + orow] = lse_val;
    }
  }
};

template <int D, int W>
__global__ __launch_bounds__(64 * W, 2) void draft_prefix_kernel(DraftPrefixArgs a) {
  DraftPrefix<D>::template run<W>(a);
}

// Merge of the splits' partials: thread per (row, head, 8 dims) of out,
// with the arithmetic of merge_state in split order (a split without keys
// carries LSE -inf and weight 0; its partial is not read). The LSEs, then
// the partials, are requested BATCH splits at a time.
template <int D>
__global__ __launch_bounds__(256) void draft_merge_kernel(DraftPrefixArgs a) {
  constexpr int PER = D / 8;
  constexpr int BATCH = 8;
  const int64_t rows = static_cast<int64_t>(a.total_q) * a.d.hq;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * PER) return;
  const int64_t r = i / PER;
  const int dq = static_cast<int>(i % PER) * 8;
  const int S = a.d.num_splits;
  float m = neg_inf();
  for (int s0 = 0; s0 < S; s0 += BATCH) {
    float ls[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) ls[q] = s0 + q < S ? a.part_lse[(s0 + q) * rows + r] : neg_inf();
#pragma unroll
    for (int q = 0; q < BATCH; ++q) m = fmaxf(m, ls[q]);
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float total = 0.f;
  if (m != neg_inf()) {
    const bf16_t* po = static_cast<const bf16_t*>(a.part_o);
    for (int s0 = 0; s0 < S; s0 += BATCH) {
      float w[BATCH];
      u32x4 v[BATCH];
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        w[q] = s0 + q < S ? merge_weight(a.part_lse[(s0 + q) * rows + r], m) : 0.f;
        v[q] = w[q] != 0.f
                   ? *reinterpret_cast<const u32x4*>(po + ((s0 + q) * rows + r) * D + dq)
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        if (w[q] == 0.f) continue;
        const float vv[8] = {bf16lo(v[q].x), bf16hi(v[q].x), bf16lo(v[q].y), bf16hi(v[q].y),
                             bf16lo(v[q].z), bf16hi(v[q].z), bf16lo(v[q].w), bf16hi(v[q].w)};
        merge_add(w[q], vv, acc, total);
      }
    }
  }
  const float inv = merge_norm(total);
  const u32x4 o = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                   pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.d.out) + r * D + dq) = o;
  if (dq == 0) a.d.lse[r] = merge_lse(m, total);
}

}  // namespace pkv

namespace pkv_launch {

int draft_prefix_heads(int dtype, int head_dim, int num_q_heads, int num_kv_heads,
                       int max_seqlen_q) {
  if (dtype != PKV_BF16 || (head_dim != 64 && head_dim != 128)) return 0;
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  const int G = num_q_heads / num_kv_heads;
  if (max_seqlen_q < 1 || static_cast<int64_t>(G) * max_seqlen_q > 32) return 0;
  return num_kv_heads % 4 == 0 ? 4 : (num_kv_heads % 2 == 0 ? 2 : 1);
}

template <int D, int W>
static hipError_t launch_draft_prefix_t(const pkv::DraftPrefixArgs& a, hipStream_t stream) {
  using K = pkv::DraftPrefix<D>;
  const int64_t blocks = static_cast<int64_t>(a.d.hkv / W) * a.d.batch * a.d.num_splits;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((pkv::draft_prefix_kernel<D, W>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * W), W * K::WAVE_LDS, stream, a);
  if (a.d.num_splits > 1) {
    const int64_t threads = static_cast<int64_t>(a.total_q) * a.d.hq * (D / 8);
    const int64_t mblocks = (threads + 255) / 256;
    if (mblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((pkv::draft_merge_kernel<D>), dim3(static_cast<unsigned>(mblocks)),
                       dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_draft_prefix_d(const pkv::DraftPrefixArgs& a, hipStream_t stream) {
  const int w = draft_prefix_heads(PKV_BF16, D, a.d.hq, a.d.hkv, 1);
  if (w == 4) return launch_draft_prefix_t<D, 4>(a, stream);
  if (w == 2) return launch_draft_prefix_t<D, 2>(a, stream);
  return launch_draft_prefix_t<D, 1>(a, stream);
}

hipError_t draft_prefix(const pkv::DraftPrefixArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_draft_prefix_d<128>(a, stream);
  if (head_dim == 64) return launch_draft_prefix_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv_launch

// paged_attn_varlen_prefill: causal extend over a paged KV cache
// ([FA] forward_extend: flash_attn_with_kvcache with cache_seqlens = prefix +
// new, cu_seqlens_q over the new tokens, causal=True). New row j of request b
// sits at position L_b - M_b + j and sees keys [0, L_b - M_b + j].
//
// Work decomposition: one workgroup of 8 waves per (32-row q tile, kv head,
// request), dispatched last-q-tile first (those see the most keys). The 8
// waves form two groups of 4; the tile's keys are cut in two halves, one per
// group, and the two online-softmax states are merged through LDS at the end,
// so the longest workgroup walks half the keys. Within a group, wave w owns
// q heads w, w+4, ... of the GQA group and all four share the group's key
// tiles: 32 keys gathered through the page table into double-buffered LDS.
//
// Per wave and key tile (32x32x16 bf16 MFMA):
//   S^T [32 keys x 32 rows] = K [32 x D] . Q^T [D x 32]        (D/16 MFMAs)
//   O^T [D x 32 rows]      += V^T [D x 32 keys] . P^T [32 x 32] (D/16 MFMAs)
// Lane (q = lane % 32, h = lane / 32) owns row q: its S^T accumulator holds
// keys rho(h, r) = 8*(r/4) + 4h + r%4, which is exactly the k-set its P^T
// operand needs for the two 16-key k-steps, and its O^T accumulator rows are
// dims of row q. Row max / sum / rescale stay in the lane (the max is reduced
// with the other lane half by one xor-shuffle).
// V^T operand: block n, row m is dim NB*m + n (NB = D/32), so a lane reads the
// NB contiguous dims [NB*m, NB*m + NB) of each of its 8 keys per k-step from
// LDS and transposes them in registers (byte permutes).
// Pipeline: the page-table entries of a tile are fetched two tiles ahead and
// its K/V rows one tile ahead, issued before the current tile's MFMAs.
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

template <int D, bool POW2>
struct PrefillKernel {
  static constexpr int KT = 32;               // keys per tile
  static constexpr int QT = 32;               // q rows per tile
  static constexpr int NKS = D / 16;          // 16-wide k-steps of S^T
  static constexpr int NB = D / 32;           // 32-dim blocks of O^T
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int LDS_STRIDE = ROW_BYTES + 16;   // pad: rows start 4 banks apart
  static constexpr int TILE_BYTES = KT * LDS_STRIDE;
  static constexpr int CHUNKS_PER_ROW = ROW_BYTES / 16;          // 16-byte pieces
  static constexpr int PIECES = KT * CHUNKS_PER_ROW;              // per tile per tensor
  static constexpr int PPT = PIECES / 256;                        // per thread of a group
  static constexpr int GROUP_LDS = 4 * TILE_BYTES;                // K, V x double buffer
  static constexpr int LDS_BYTES = 2 * GROUP_LDS;
  static constexpr int MERGE_FLOATS = 16 * NB + 2;                // acc + m + l per lane
  static_assert(4 * 64 * MERGE_FLOATS * 4 <= LDS_BYTES, "merge buffer fits the tile buffers");

  // key of S^T accumulator register r for lane half h
  static __device__ __forceinline__ int rho(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }

  struct Stage {
    u32x4 k[PPT];
    u32x4 v[PPT];
  };

  // token t -> (page-table column, offset in page); shifts when P = 2^k
  static __device__ __forceinline__ int page_col(const PrefillArgs& a, int t) {
    if constexpr (POW2) return t >> a.page_shift;
    else return t / a.page_size;
  }
  static __device__ __forceinline__ int page_off(const PrefillArgs& a, int t) {
    if constexpr (POW2) return t & (a.page_size - 1);
    else return t % a.page_size;
  }

  // page-table entries of the keys this thread copies for `tile`
  static __device__ __forceinline__ void fetch_raw(const PrefillArgs& a, const int32_t* pt_row,
                                                   int kv_len, int tile, int gt, int32_t (&raw)[PPT]) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int key = (gt + 256 * i) / CHUNKS_PER_ROW;
      const int t = min(tile * KT + key, kv_len - 1);   // tail keys: any valid row (masked)
      raw[i] = pt_row[page_col(a, t)];
    }
  }

  // row_bytes = Hkv * D * 2; col_off[i] = kvh * D * 2 + chunk * 16 of piece i
  static __device__ __forceinline__ void load_tile(const PrefillArgs& a, int kv_len, int tile,
                                                   int gt, int64_t row_bytes,
                                                   const int32_t (&col_off)[PPT],
                                                   const int32_t (&raw)[PPT], Stage& st) {
    const char* kb = static_cast<const char*>(a.k);
    const char* vb = static_cast<const char*>(a.v);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int key = (gt + 256 * i) / CHUNKS_PER_ROW;
      const int t = min(tile * KT + key, kv_len - 1);
      const int64_t page = clamp_index(raw[i], a.num_pages);
      int64_t slot;
      if constexpr (POW2) slot = (page << a.page_shift) | page_off(a, t);
      else slot = page * a.page_size + page_off(a, t);
      const int64_t off = slot * row_bytes + col_off[i];
      st.k[i] = *reinterpret_cast<const u32x4*>(kb + off);
      st.v[i] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  }

  static __device__ __forceinline__ void store_tile(char* lds_k, char* lds_v, int gt,
                                                    const Stage& st) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = gt + 256 * i;
      const int key = piece / CHUNKS_PER_ROW;
      const int chunk = piece % CHUNKS_PER_ROW;
      *reinterpret_cast<u32x4*>(lds_k + key * LDS_STRIDE + chunk * 16) = st.k[i];
      *reinterpret_cast<u32x4*>(lds_v + key * LDS_STRIDE + chunk * 16) = st.v[i];
    }
  }

  // One key tile for this wave's row block: S^T, online softmax, O^T update.
  // m_run is kept in raw score units; scale_log2 > 0 is applied inside the
  // exponent (exp2(s * c - m * c)). Masked tiles apply the per-row key limit.
  static __device__ __forceinline__ void compute_tile(const char* lk, const char* lv, int kt,
                                                      bool masked, int limit, int q, int h,
                                                      float scale_log2,
                                                      const u32x4 (&qop)[NKS], f32x16 (&acc)[NB],
                                                      float& m_run, float& l_run) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const char* kl = lk + q * LDS_STRIDE;   // A row = key q of the tile
#pragma unroll
    for (int j = 0; j < NKS; ++j) {
      const u32x4 kw = *reinterpret_cast<const u32x4*>(kl + (16 * j + 8 * h) * 2);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), as_bf16x8(qop[j]), s, 0, 0, 0);
    }

    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = s[r];
    if (masked) {   // wave-uniform: only tiles that reach past some row's limit
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kt * KT + rho(h, r) >= limit) x[r] = neg_inf();
    }
    float mt = fmaxf(x[0], x[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mt = fmaxf(mt, x[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_log2);
    const float neg_mc = -m_use * scale_log2;
    m_run = m_new;
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(__builtin_fmaf(x[r], scale_log2, neg_mc));
      psum += p[r];
    }
    l_run = l_run * alpha + psum;
    // rescale only when some row's running max moved (rare after the first tiles)
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    }

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 pw = {pack_bf16x2(p[8 * t + 0], p[8 * t + 1]), pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                  pack_bf16x2(p[8 * t + 4], p[8 * t + 5]), pack_bf16x2(p[8 * t + 6], p[8 * t + 7])};
      // V rows of the 8 keys 16t + 8(e/4) + 4h + e%4, dims [NB*q, NB*q + NB)
      uint32_t vr[8][NB / 2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * t + 8 * (e >> 2) + 4 * h + (e & 3);
        const char* src = lv + key * LDS_STRIDE + NB * q * 2;
        if constexpr (NB == 4) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(src);
          vr[e][0] = w.x;
          vr[e][1] = w.y;
        } else {
          vr[e][0] = *reinterpret_cast<const uint32_t*>(src);
        }
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        u32x4 vw;
        if ((n & 1) == 0) {
          vw.x = pair_lo(vr[0][n >> 1], vr[1][n >> 1]);
          vw.y = pair_lo(vr[2][n >> 1], vr[3][n >> 1]);
          vw.z = pair_lo(vr[4][n >> 1], vr[5][n >> 1]);
          vw.w = pair_lo(vr[6][n >> 1], vr[7][n >> 1]);
        } else {
          vw.x = pair_hi(vr[0][n >> 1], vr[1][n >> 1]);
          vw.y = pair_hi(vr[2][n >> 1], vr[3][n >> 1]);
          vw.z = pair_hi(vr[4][n >> 1], vr[5][n >> 1]);
          vw.w = pair_hi(vr[6][n >> 1], vr[7][n >> 1]);
        }
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), as_bf16x8(pw), acc[n], 0,
                                                         0, 0);
      }
    }
  }

  static __device__ void run(const PrefillArgs& a) {
    extern __shared__ __align__(16) char smem[];

    const int G = a.hq / a.hkv;
    // flat grid: kv head fastest, then request, then q tile counted from the end
    const int kvh = blockIdx.x % a.hkv;
    const int b = (blockIdx.x / a.hkv) % a.batch;
    const int qrev = blockIdx.x / (a.hkv * a.batch);
    const int q0 = a.cu_q[b];
    const int M = a.cu_q[b + 1] - q0;
    const int n_qtiles = (M + QT - 1) / QT;
    const int qtile = n_qtiles - 1 - qrev;
    if (qtile < 0) return;
    const int64_t cap = static_cast<int64_t>(a.pt_stride) * a.page_size;
    const int L = static_cast<int>(min<int64_t>(max(a.kv_lens[b], 0), cap));
    const int j0 = qtile * QT;
    const int rows = min(QT, M - j0);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;            // key-half group
    const int gw = wave & 3;              // wave within the group
    const int gt = threadIdx.x & 255;     // thread within the group
    const int q = lane & 31;
    const int h = lane >> 5;

    // keys this q tile can see: up to position L - M + j0 + rows - 1
    const int key_end = a.causal ? min(L, L - M + j0 + rows) : L;
    const int n_ktiles = key_end > 0 ? (key_end + KT - 1) / KT : 0;
    const int half = (n_ktiles + 1) / 2;
    const int t_begin = grp == 0 ? 0 : half;
    const int n_my = grp == 0 ? half : n_ktiles - half;
    const int n_iter = half;              // both groups step through the same barriers
    const int row_ok = q < rows;
    // keys visible to row q (rows past the tile's end compute discarded values)
    const int limit = a.causal ? min(L, L - M + j0 + q + 1) : L;
    // tiles entirely below every row's limit need no mask
    const int full_tiles = max(a.causal ? min(L, L - M + j0 + 1) : L, 0) / KT;
    const int64_t row_bytes = static_cast<int64_t>(a.hkv) * D * 2;
    int32_t col_off[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) col_off[i] = kvh * D * 2 + ((gt + 256 * i) % CHUNKS_PER_ROW) * 16;

    const int32_t* pt_row = a.pt + static_cast<int64_t>(b) * a.pt_stride;
    char* gbase = smem + grp * GROUP_LDS;
    auto lds_k = [&](int i) { return gbase + 2 * i * TILE_BYTES; };
    auto lds_v = [&](int i) { return gbase + (2 * i + 1) * TILE_BYTES; };

    for (int hb = 0; hb < (G + 3) / 4; ++hb) {
      const int hg = 4 * hb + gw;           // this wave's head within the group
      const bool head_ok = hg < G;
      const int head = kvh * G + min(hg, G - 1);

      // Q^T operand: row q, dims 16j + 8h + [0, 8)
      u32x4 qop[NKS];
      {
        const int row = q0 + j0 + min(q, rows - 1);
        const char* qrow = static_cast<const char*>(a.q) +
                           ((static_cast<int64_t>(row) * a.hq + head) * D) * 2;
#pragma unroll
        for (int j = 0; j < NKS; ++j)
          qop[j] = *reinterpret_cast<const u32x4*>(qrow + (16 * j + 8 * h) * 2);
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
          retire(qop[j].x);
          retire(qop[j].y);
          retire(qop[j].z);
          retire(qop[j].w);
        }
      }
      f32x16 acc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
      float m_run = neg_inf();
      float l_run = 0.f;

      // ---- prologue: tile t_begin in LDS, entries of the next one in hand ----
      Stage st;
      int32_t raw_n[PPT];
      if (n_my > 0) {
        int32_t raw0[PPT];
        fetch_raw(a, pt_row, L, t_begin, gt, raw0);
        load_tile(a, L, t_begin, gt, row_bytes, col_off, raw0, st);
        fetch_raw(a, pt_row, L, min(t_begin + 1, t_begin + n_my - 1), gt, raw_n);
        store_tile(lds_k(0), lds_v(0), gt, st);
      }
      __syncthreads();

      for (int it = 0; it < n_iter; ++it) {
        const int kt = t_begin + it;
        const bool more = it + 1 < n_my;
        int32_t raw_nn[PPT];
        if (more) {
          load_tile(a, L, kt + 1, gt, row_bytes, col_off, raw_n, st);
          fetch_raw(a, pt_row, L, min(kt + 2, t_begin + n_my - 1), gt, raw_nn);
        }
        __builtin_amdgcn_sched_barrier(0);   // loads go out before the MFMAs
        if (it < n_my) {
          compute_tile(lds_k(it & 1), lds_v(it & 1), kt, kt >= full_tiles, limit, q, h,
                       a.scale_log2, qop, acc, m_run, l_run);
        }
        if (more) {
          // buffer (it + 1) & 1 was last read before the previous barrier
          store_tile(lds_k((it + 1) & 1), lds_v((it + 1) & 1), gt, st);
#pragma unroll
          for (int i = 0; i < PPT; ++i) raw_n[i] = raw_nn[i];
        }
        __syncthreads();
      }

      // ---- merge the two key halves (group 1 -> group 0) through LDS ----
      float* mbuf = reinterpret_cast<float*>(smem) + (gw * 64 + lane) * MERGE_FLOATS;
      if (grp == 1) {
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) mbuf[16 * n + r] = acc[n][r];
        mbuf[16 * NB] = m_run;
        mbuf[16 * NB + 1] = l_run;
      }
      __syncthreads();
      if (grp == 0) {
        const float m1 = mbuf[16 * NB];
        const float l1 = mbuf[16 * NB + 1];
        const float M2 = fmaxf(m_run, m1);
        const float f0 = (m_run == neg_inf()) ? 0.f : fast_exp2((m_run - M2) * a.scale_log2);
        const float f1 = (m1 == neg_inf()) ? 0.f : fast_exp2((m1 - M2) * a.scale_log2);
        float l_m = f0 * l_run + f1 * l1;
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[n][r] = f0 * acc[n][r] + f1 * mbuf[16 * n + r];
        const float l_tot = l_m + __shfl_xor(l_m, 32);
        if (head_ok && row_ok) {
          const int64_t row = q0 + j0 + q;
          const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
          bf16_t* dst = static_cast<bf16_t*>(a.out) + (row * a.hq + head) * D;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dim = NB * rho(h, r);
            if constexpr (NB == 4) {
              u32x2 w;
              w.x = pack_bf16x2(acc[0][r] * inv, acc[1][r] * inv);
              w.y = pack_bf16x2(acc[2][r] * inv, acc[3][r] * inv);
              *reinterpret_cast<u32x2*>(dst + dim) = w;
            } else {
              *reinterpret_cast<uint32_t*>(dst + dim) =
                  pack_bf16x2(acc[0][r] * inv, acc[1][r] * inv);
            }
          }
          if (a.lse != nullptr && h == 0) {
            a.lse[row * a.hq + head] =
                l_tot > 0.f ? (M2 * a.scale_log2 + fast_log2(l_tot)) * kLn2 : neg_inf();
          }
        }
      }
      __syncthreads();   // merge buffer and tile buffers are reused by the next head slice
    }
  }
};

template <int D, bool POW2>
__global__ __launch_bounds__(512, 1) void prefill_kernel(PrefillArgs a) {
  PrefillKernel<D, POW2>::run(a);
}

}  // namespace pkv

namespace pkv_launch {

hipError_t prefill(const pkv::PrefillArgs& a, int head_dim, hipStream_t stream) {
  const int64_t max_qtiles = (a.max_seqlen_q + 31) / 32;
  const int64_t blocks = max_qtiles * a.hkv * a.batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  const bool pow2 = a.page_shift >= 0;
  if (head_dim == 128) {
    if (pow2)
      hipLaunchKernelGGL((pkv::prefill_kernel<128, true>), grid, dim3(512),
                         (pkv::PrefillKernel<128, true>::LDS_BYTES), stream, a);
    else
      hipLaunchKernelGGL((pkv::prefill_kernel<128, false>), grid, dim3(512),
                         (pkv::PrefillKernel<128, false>::LDS_BYTES), stream, a);
  } else {
    if (pow2)
      hipLaunchKernelGGL((pkv::prefill_kernel<64, true>), grid, dim3(512),
                         (pkv::PrefillKernel<64, true>::LDS_BYTES), stream, a);
    else
      hipLaunchKernelGGL((pkv::prefill_kernel<64, false>), grid, dim3(512),
                         (pkv::PrefillKernel<64, false>::LDS_BYTES), stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv_launch

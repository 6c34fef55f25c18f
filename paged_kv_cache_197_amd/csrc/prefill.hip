// paged_attn_varlen_prefill: causal extend over a paged KV cache
// ([FA] forward_extend: flash_attn_with_kvcache with cache_seqlens = prefix +
// new, cu_seqlens_q over the new tokens, causal=True). New row j of request b
// sits at position L_b - M_b + j and sees keys [0, L_b - M_b + j].
//
// Work decomposition: one workgroup of 4 waves per (32-row q tile, kv head,
// request). The workgroup walks the request's keys in 32-key tiles, gathered
// through the page table into double-buffered LDS and shared by every q head
// of the GQA group; wave w owns q heads w, w+4, ... of the group. Tiles are
// dispatched last-q-tile first so the tiles that see the most keys start
// earliest.
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
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

template <int D>
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
  static constexpr int PIECES_PER_THREAD = PIECES / 256;          // 2 (D=128) or 1 (D=64)

  // key of S^T accumulator register r for lane half h
  static __device__ __forceinline__ int rho(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }

  struct Stage {
    u32x4 k[PIECES_PER_THREAD];
    u32x4 v[PIECES_PER_THREAD];
  };

  static __device__ __forceinline__ void load_tile(const PrefillArgs& a, const int32_t* pt_row,
                                                   int kv_len, int kvh, int tile, Stage& st) {
    const char* kb = static_cast<const char*>(a.k);
    const char* vb = static_cast<const char*>(a.v);
#pragma unroll
    for (int i = 0; i < PIECES_PER_THREAD; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int key = piece / CHUNKS_PER_ROW;
      const int chunk = piece % CHUNKS_PER_ROW;
      const int t = min(tile * KT + key, kv_len - 1);   // tail keys: any valid row (masked)
      const int64_t page = clamp_index(pt_row[t / a.page_size], a.num_pages);
      const int64_t slot = page * a.page_size + (t % a.page_size);
      const int64_t off = ((slot * a.hkv + kvh) * D) * 2 + chunk * 16;
      st.k[i] = *reinterpret_cast<const u32x4*>(kb + off);
      st.v[i] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  }

  static __device__ __forceinline__ void store_tile(char* lds_k, char* lds_v, const Stage& st) {
#pragma unroll
    for (int i = 0; i < PIECES_PER_THREAD; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int key = piece / CHUNKS_PER_ROW;
      const int chunk = piece % CHUNKS_PER_ROW;
      *reinterpret_cast<u32x4*>(lds_k + key * LDS_STRIDE + chunk * 16) = st.k[i];
      *reinterpret_cast<u32x4*>(lds_v + key * LDS_STRIDE + chunk * 16) = st.v[i];
    }
  }

  static __device__ void run(const PrefillArgs& a) {
    extern __shared__ __align__(16) char smem[];
    // buffer i: K at smem + 2*i*TILE_BYTES, V right after it
    auto lds_k = [&](int i) { return smem + 2 * i * TILE_BYTES; };
    auto lds_v = [&](int i) { return smem + (2 * i + 1) * TILE_BYTES; };

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
    const int wave = threadIdx.x >> 6;
    const int q = lane & 31;
    const int h = lane >> 5;

    // keys this tile can see: up to position L - M + j0 + rows - 1
    const int key_end = a.causal ? min(L, L - M + j0 + rows) : L;
    const int n_ktiles = key_end > 0 ? (key_end + KT - 1) / KT : 0;
    // keys visible to this lane's row
    const int row_ok = q < rows;
    const int limit = !row_ok ? 0 : (a.causal ? min(L, L - M + j0 + q + 1) : L);

    const int32_t* pt_row = a.pt + static_cast<int64_t>(b) * a.pt_stride;

    Stage st;
    if (n_ktiles > 0) {
      load_tile(a, pt_row, L, kvh, 0, st);
      store_tile(lds_k(0), lds_v(0), st);
    }
    __syncthreads();

    for (int hb = wave; hb < ((G + 3) / 4) * 4; hb += 4) {
      // heads hb (this wave) of the group; a pass over the keys per head slice
      const bool head_ok = hb < G;
      const int head = kvh * G + min(hb, G - 1);
      // Q^T operand: row q, dims 16j + 8h + [0, 8)
      u32x4 qop[NKS];
      {
        const int row = q0 + j0 + min(q, rows - 1);
        const char* qrow = static_cast<const char*>(a.q) +
                           ((static_cast<int64_t>(row) * a.hq + head) * D) * 2;
#pragma unroll
        for (int j = 0; j < NKS; ++j) qop[j] = *reinterpret_cast<const u32x4*>(qrow + (16 * j + 8 * h) * 2);
      }
      f32x16 acc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
      float m_run = neg_inf();
      float l_run = 0.f;

      for (int kt = 0; kt < n_ktiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_ktiles;
        // the first head slice streams the tiles; later slices (G > 4) re-read them
        if (more) load_tile(a, pt_row, L, kvh, kt + 1, st);

        // ---- S^T = K . Q^T ----
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        const char* kl = lds_k(buf) + q * LDS_STRIDE;   // A row = key q of the tile
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
          const u32x4 kw = *reinterpret_cast<const u32x4*>(kl + (16 * j + 8 * h) * 2);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), as_bf16x8(qop[j]), s, 0, 0, 0);
        }

        // ---- online softmax (base 2) ----
        float x[16];
        float mt = neg_inf();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = kt * KT + rho(h, r);
          x[r] = (t < limit) ? s[r] * a.scale_log2 : neg_inf();
          mt = fmaxf(mt, x[r]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float p[16];
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(x[r] - m_use);
          psum += p[r];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] *= alpha;

        // ---- O^T += V^T . P^T, two 16-key k-steps ----
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 pw = {pack_bf16x2(p[8 * t + 0], p[8 * t + 1]), pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                      pack_bf16x2(p[8 * t + 4], p[8 * t + 5]), pack_bf16x2(p[8 * t + 6], p[8 * t + 7])};
          // V rows of the 8 keys 16t + 8(e/4) + 4h + e%4, dims [NB*q, NB*q + NB)
          uint32_t vr[8][NB / 2];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = 16 * t + 8 * (e >> 2) + 4 * h + (e & 3);
            const char* src = lds_v(buf) + key * LDS_STRIDE + NB * q * 2;
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
            acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), as_bf16x8(pw), acc[n],
                                                             0, 0, 0);
          }
        }

        if (more) {
          // buffer buf ^ 1 was last read before the previous barrier
          store_tile(lds_k(buf ^ 1), lds_v(buf ^ 1), st);
          __syncthreads();
        }
      }

      // ---- write this head slice ----
      const float l_tot = l_run + __shfl_xor(l_run, 32);
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
            *reinterpret_cast<uint32_t*>(dst + dim) = pack_bf16x2(acc[0][r] * inv, acc[1][r] * inv);
          }
        }
        if (a.lse != nullptr && h == 0) {
          a.lse[row * a.hq + head] =
              l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : neg_inf();
        }
      }
      if (hb + 4 < ((G + 3) / 4) * 4 && n_ktiles > 0) {
        // next head slice restarts from the first key tile
        __syncthreads();
        load_tile(a, pt_row, L, kvh, 0, st);
        store_tile(lds_k(0), lds_v(0), st);
        __syncthreads();
      }
    }
  }
};

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  PrefillKernel<D>::run(a);
}

}  // namespace pkv

namespace pkv_launch {

hipError_t prefill(const pkv::PrefillArgs& a, int head_dim, hipStream_t stream) {
  const int64_t max_qtiles = (a.max_seqlen_q + 31) / 32;
  const int64_t blocks = max_qtiles * a.hkv * a.batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (head_dim == 128) {
    const size_t lds = 4 * pkv::PrefillKernel<128>::TILE_BYTES;
    hipLaunchKernelGGL(pkv::prefill_kernel<128>, grid, dim3(256), lds, stream, a);
  } else {
    const size_t lds = 4 * pkv::PrefillKernel<64>::TILE_BYTES;
    hipLaunchKernelGGL(pkv::prefill_kernel<64>, grid, dim3(256), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv_launch

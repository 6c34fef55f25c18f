// paged_attn_decode_splitkv: one query token per request, the key axis cut
// into splits of kv_chunk tokens, each split producing a normalised partial
// output and its LSE ([FA] forward_decode; [DCA] _dual_chunk_flash_attn_decoding).
//
// Work decomposition: one workgroup (4 waves) per (split, request, kv head);
// kv head varies fastest in the grid so the Hkv workgroups that read the same
// pages run together. Inside a split, wave w takes 32-token tiles w, w+4, ...
// and keeps its own online-softmax state; the four states are merged through
// LDS at the end.
//
// Per 32-token tile a wave computes, for the G <= 16 query heads of its kv
// head (padded to 16 MFMA columns):
//   S^T [32 tok x 16 heads] = K [32 x D] . Q^T [D x 16]      (16x16x32 MFMA)
//   O^T [D x 16 heads]     += V^T [D x 32 tok] . P^T [32 x 16]
// Lane (c = lane % 16, g = lane / 16) then owns head c everywhere: its S^T
// accumulator holds tokens {4g+i} and {16+4g+i}, exactly the 8 tokens its P^T
// operand needs, and its O^T accumulator rows are dims of head c, so the
// running max / sum / rescale never leave the lane (except the max, reduced
// over the four lane groups with two xor-shuffles).
// Operand loads come straight from HBM into registers:
//   * K: lane loads token c of each 16-token half, bytes [64j + 16g, +16) of
//     the row for k-step j (16 B per lane, 4 lanes covering 64 contiguous
//     bytes of each row per instruction);
//   * V: lane loads, for each of its 8 tokens, the CH = D/16 contiguous dims
//     [CH*c, CH*c + CH): 16 lanes read a whole 256-byte row per instruction.
//     V^T block n row c is dim CH*c + n, so the transpose to the MFMA A
//     operand is a register-local 8x8 (bf16: byte-permute) shuffle.
// fp32 inputs run the same tiles with 16x16x4 fp32 MFMAs, one per element of
// the 8-element operand.
#include <limits.h>

#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

template <int NDW>
struct Chunk {
  uint32_t w[NDW];
};

// NT: non-temporal (streaming) load. Not used for K / V: on this kernel's
// access pattern (64-byte half-line pieces of 256-byte rows) it raised the
// fetched bytes by ~4% and lowered throughput, although a plain linear read
// sweep streams faster with it.
template <int NDW, bool NT = false>
__device__ __forceinline__ Chunk<NDW> load_chunk(const void* p) {
  Chunk<NDW> c;
  if constexpr (NDW == 2) {
    const u32x2 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                       : *reinterpret_cast<const u32x2*>(p);
    c.w[0] = v.x;
    c.w[1] = v.y;
  } else {
    static_assert(NDW % 4 == 0, "chunk of 8, 16 or 32 bytes");
#pragma unroll
    for (int i = 0; i < NDW / 4; ++i) {
      const u32x4 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i)
                         : reinterpret_cast<const u32x4*>(p)[i];
      c.w[4 * i + 0] = v.x;
      c.w[4 * i + 1] = v.y;
      c.w[4 * i + 2] = v.z;
      c.w[4 * i + 3] = v.w;
    }
  }
  return c;
}

template <typename T>
struct ElemBytes;
template <>
struct ElemBytes<float> {
  static constexpr int value = 4;
};
template <>
struct ElemBytes<bf16_t> {
  static constexpr int value = 2;
};

// Element (e) of an 8-element operand chunk as fp32 (fp32 path only).
__device__ __forceinline__ float word_f32(uint32_t w) { return __uint_as_float(w); }

template <typename T, int D, bool UNIFORM_PAGE>
struct DecodeKernel {
  static constexpr int EB = ElemBytes<T>::value;
  static constexpr int NK = D / 32;          // k-steps of 32 over the head dim
  static constexpr int CH = D / 16;          // V dims per lane per token
  static constexpr int NB = D / 16;          // 16-dim blocks of O^T
  static constexpr int KDW = 8 * EB / 4;     // dwords per 8-element K / Q chunk
  static constexpr int VDW = CH * EB / 4;    // dwords per V chunk
  static constexpr bool IS_BF16 = (EB == 2);

  struct Tile {
    Chunk<KDW> k[2][NK];
    Chunk<VDW> v[8];
  };

  // token offset (0..31 within the tile) held by element e of lane group g
  static __device__ __forceinline__ int tok_of(int g, int e) {
    return (e < 4) ? (4 * g + e) : (16 + 4 * g + (e - 4));
  }

  // --- index stage -----------------------------------------------------------
  // Uniform pages (page_size % 32 == 0, tiles page-aligned): every token of a
  // tile is on one page, so the wave loads one page-table entry per tile.
  // Otherwise lane l loads the entry of token (l % 32) of the tile and the
  // slots are shared by shuffles. The raw entry is fetched one tile ahead of
  // its use; the address arithmetic waits until the tile's loads are issued.
  static __device__ __forceinline__ int32_t fetch_raw(const DecodeArgs& a, const int32_t* pt_row,
                                                      int tile_start, int end, int lane) {
    if constexpr (UNIFORM_PAGE) {
      return pt_row[tile_start / a.page_size];
    } else {
      const int t = min(tile_start + (lane & 31), end - 1);
      return pt_row[t / a.page_size];
    }
  }

  static __device__ __forceinline__ int64_t slot_base(const DecodeArgs& a, int32_t raw,
                                                      int tile_start, int end, int lane) {
    const int64_t page = clamp_index(raw, a.num_pages);
    if constexpr (UNIFORM_PAGE) {
      return page * a.page_size + (tile_start % a.page_size);
    } else {
      const int t = min(tile_start + (lane & 31), end - 1);
      return page * a.page_size + (t % a.page_size);
    }
  }

  static __device__ __forceinline__ int64_t slot_of(int64_t idx, int o, int tile_start, int end) {
    if constexpr (UNIFORM_PAGE) {
      return idx + min(o, end - 1 - tile_start);
    } else {
      const int lo = __shfl(static_cast<int>(idx & 0xffffffff), o);
      const int hi = __shfl(static_cast<int>(idx >> 32), o);
      return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
    }
  }

  static __device__ __forceinline__ void fetch_data(const DecodeArgs& a, int64_t idx, int tile_start,
                                                    int end, int kvh, int c, int g, Tile& t) {
    const char* kbase = static_cast<const char*>(a.k);
    const char* vbase = static_cast<const char*>(a.v);
    const int64_t row_elems = static_cast<int64_t>(a.hkv) * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t slot = slot_of(idx, 16 * u + c, tile_start, end);
      const char* row = kbase + ((slot * row_elems) + static_cast<int64_t>(kvh) * D) * EB;
#pragma unroll
      for (int j = 0; j < NK; ++j) t.k[u][j] = load_chunk<KDW>(row + (32 * j + 8 * g) * EB);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t slot = slot_of(idx, tok_of(g, e), tile_start, end);
      const char* row = vbase + ((slot * row_elems) + static_cast<int64_t>(kvh) * D) * EB;
      t.v[e] = load_chunk<VDW>(row + (CH * c) * EB);
    }
  }

  // One tile: S^T = K . Q^T, online softmax (base 2), O^T += V^T . P^T.
  static __device__ __forceinline__ void consume(const Tile& cur, int ts, int end, int g,
                                                 float scale_log2, const Chunk<KDW> (&qop)[NK],
                                                 f32x4 (&acc)[NB], float& m_run, float& l_run) {
    f32x4 st[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      st[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        if constexpr (IS_BF16) {
          u32x4 kw = {cur.k[u][j].w[0], cur.k[u][j].w[1], cur.k[u][j].w[2], cur.k[u][j].w[3]};
          u32x4 qw = {qop[j].w[0], qop[j].w[1], qop[j].w[2], qop[j].w[3]};
          st[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), as_bf16x8(qw), st[u], 0,
                                                          0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            st[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(word_f32(cur.k[u][j].w[e]),
                                                         word_f32(qop[j].w[e]), st[u], 0, 0, 0);
        }
      }
    }

    float x[8];
    const int valid = end - ts;  // tokens of this tile inside the split (may exceed 32)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = st[e >> 2][e & 3] * scale_log2;
      x[e] = (tok_of(g, e) < valid) ? sv : neg_inf();
    }
    float mt = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mt = fmaxf(mt, x[e]);
    mt = max_over_groups16(mt);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(x[e] - m_new);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] *= alpha;

    if constexpr (IS_BF16) {
      u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                  pack_bf16x2(p[6], p[7])};
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        u32x4 vw;
        if ((n & 1) == 0) {
          vw.x = pair_lo(cur.v[0].w[n >> 1], cur.v[1].w[n >> 1]);
          vw.y = pair_lo(cur.v[2].w[n >> 1], cur.v[3].w[n >> 1]);
          vw.z = pair_lo(cur.v[4].w[n >> 1], cur.v[5].w[n >> 1]);
          vw.w = pair_lo(cur.v[6].w[n >> 1], cur.v[7].w[n >> 1]);
        } else {
          vw.x = pair_hi(cur.v[0].w[n >> 1], cur.v[1].w[n >> 1]);
          vw.y = pair_hi(cur.v[2].w[n >> 1], cur.v[3].w[n >> 1]);
          vw.z = pair_hi(cur.v[4].w[n >> 1], cur.v[5].w[n >> 1]);
          vw.w = pair_hi(cur.v[6].w[n >> 1], cur.v[7].w[n >> 1]);
        }
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw), pb, acc[n], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(word_f32(cur.v[e].w[n]), p[e], acc[n], 0,
                                                        0, 0);
      }
    }
  }

  static __device__ void run(const DecodeArgs& a) {
    __shared__ float sm_m[4][16];
    __shared__ float sm_l[4][16];
    __shared__ float sm_acc[4][64][4 * NB + 1];

    const int G = a.hq / a.hkv;
    const int kvh = blockIdx.x % a.hkv;
    const int rest = blockIdx.x / a.hkv;
    const int b = rest % a.batch;
    const int s = rest / a.batch;
    const int h0 = kvh * G;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;

    const int64_t cap = static_cast<int64_t>(a.pt_stride) * a.page_size;
    const int L = static_cast<int>(min<int64_t>(max(a.kv_lens[b], 0), cap));
    const int start = static_cast<int>(min<int64_t>(static_cast<int64_t>(s) * a.chunk, L));
    const int end = static_cast<int>(min<int64_t>(static_cast<int64_t>(start) + a.chunk, L));

    const bool single = (a.num_splits == 1);
    if (start >= end) {
      // empty split: (0, -inf)
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
        const int hh = h0 + i / D;
        const int d = i % D;
        const int64_t row = static_cast<int64_t>(b) * a.hq + hh;
        if (single) {
          if constexpr (IS_BF16) static_cast<bf16_t*>(a.out)[row * D + d].bits = 0;
          else static_cast<float*>(a.out)[row * D + d] = 0.f;
        } else {
          a.o_part[(static_cast<int64_t>(s) * a.batch * a.hq + row) * D + d] = 0.f;
        }
      }
      for (int i = threadIdx.x; i < G; i += blockDim.x) {
        const int64_t row = static_cast<int64_t>(b) * a.hq + h0 + i;
        if (single) {
          if (a.lse) a.lse[row] = neg_inf();
        } else {
          a.lse_part[static_cast<int64_t>(s) * a.batch * a.hq + row] = neg_inf();
        }
      }
      return;
    }

    // Q^T operand: head c (zero for padding columns), dims 32j + 8g + [0, 8)
    Chunk<KDW> qop[NK];
    {
      const char* qrow = static_cast<const char*>(a.q) +
                         (static_cast<int64_t>(b) * a.hq + h0 + min(c, G - 1)) * D * EB;
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        qop[j] = load_chunk<KDW>(qrow + (32 * j + 8 * g) * EB);
      }
#pragma unroll
      for (int j = 0; j < NK; ++j) {
#pragma unroll
        for (int w = 0; w < KDW; ++w) {
          qop[j].w[w] = (c < G) ? qop[j].w[w] : 0u;
          retire(qop[j].w[w]);
        }
      }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf();
    float l_run = 0.f;

    const int32_t* pt_row = a.pt + static_cast<int64_t>(b) * a.pt_stride;
    const int n_tiles = (end - start + 31) / 32;

    // Ping-pong tile buffers: tile t+4 streams in while tile t is consumed,
    // and no register copies sit between the loads and their consumer. The
    // prefetch is unconditional (past the wave's last tile it re-reads the
    // current tile, which the caches already hold) so the loop body has one
    // path and every wait counts exactly the loads it must.
    int tile = __builtin_amdgcn_readfirstlane(wave);
    if (tile < n_tiles) {
      const int last = n_tiles - 1 - ((n_tiles - 1 - tile) & 3);   // this wave's last tile
      auto ahead = [&](int t, int k) { return min(t + 4 * k, last); };
      Tile ta, tb;
      const int32_t raw0 = fetch_raw(a, pt_row, start + 32 * tile, end, lane);
      int32_t raw_n = fetch_raw(a, pt_row, start + 32 * ahead(tile, 1), end, lane);
      fetch_data(a, slot_base(a, raw0, start + 32 * tile, end, lane), start + 32 * tile, end, kvh,
                 c, g, ta);
      while (true) {
        int32_t raw_nn = fetch_raw(a, pt_row, start + 32 * ahead(tile, 2), end, lane);
        {
          const int ts = start + 32 * ahead(tile, 1);
          fetch_data(a, slot_base(a, raw_n, ts, end, lane), ts, end, kvh, c, g, tb);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
        consume(ta, start + 32 * tile, end, g, a.scale_log2, qop, acc, m_run, l_run);
        tile += 4;
        if (tile > last) break;
        raw_n = raw_nn;
        raw_nn = fetch_raw(a, pt_row, start + 32 * ahead(tile, 2), end, lane);
        {
          const int ts = start + 32 * ahead(tile, 1);
          fetch_data(a, slot_base(a, raw_n, ts, end, lane), ts, end, kvh, c, g, ta);
        }
        __builtin_amdgcn_sched_barrier(0);
        consume(tb, start + 32 * tile, end, g, a.scale_log2, qop, acc, m_run, l_run);
        tile += 4;
        if (tile > last) break;
        raw_n = raw_nn;
      }
    }

    // ---- merge the four waves' states ----
    const float l_tot = sum_over_groups16(l_run);
    if (g == 0) {
      sm_m[wave][c] = m_run;
      sm_l[wave][c] = l_tot;
    }
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_acc[wave][lane][4 * n + i] = acc[n][i];
    __syncthreads();
    if (wave != 0 || c >= G) return;

    float M = sm_m[0][c];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][c]);
    float f[4];
    float Ltot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[w] = (sm_m[w][c] == neg_inf()) ? 0.f : fast_exp2(sm_m[w][c] - M);
      Ltot += f[w] * sm_l[w][c];
    }
    const float inv = 1.f / Ltot;
    float o[4 * NB];  // o[CH*i + n] = dim 4*CH*g + CH*i + n
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) v += f[w] * sm_acc[w][lane][4 * n + i];
        o[CH * i + n] = v * inv;
      }
    const float lse_val = (M + fast_log2(Ltot)) * kLn2;
    const int64_t row = static_cast<int64_t>(b) * a.hq + h0 + c;
    const int dim0 = 4 * CH * g;
    if (single) {
      if constexpr (IS_BF16) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(a.out) + row * D + dim0);
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) dst[k] = pack_bf16x2(o[2 * k], o[2 * k + 1]);
      } else {
        float* dst = static_cast<float*>(a.out) + row * D + dim0;
#pragma unroll
        for (int k = 0; k < 4 * NB; ++k) dst[k] = o[k];
      }
      if (a.lse != nullptr && g == 0) a.lse[row] = lse_val;
    } else {
      float* dst = a.o_part + (static_cast<int64_t>(s) * a.batch * a.hq + row) * D + dim0;
#pragma unroll
      for (int k = 0; k < 4 * NB; k += 4)
        *reinterpret_cast<float4*>(dst + k) = make_float4(o[k], o[k + 1], o[k + 2], o[k + 3]);
      if (g == 0) a.lse_part[static_cast<int64_t>(s) * a.batch * a.hq + row] = lse_val;
    }
  }
};

// bf16 tiles fit two workgroups per CU (<= 256 VGPRs); fp32 tiles are twice
// as wide and get the whole register file.
template <typename T, int D, bool UNIFORM_PAGE>
__global__ __launch_bounds__(256, 2) void decode_splitkv_kernel(DecodeArgs a) {
  DecodeKernel<T, D, UNIFORM_PAGE>::run(a);
}
template <typename T, int D, bool UNIFORM_PAGE>
__global__ __launch_bounds__(256, 1) void decode_splitkv_kernel_wide(DecodeArgs a) {
  DecodeKernel<T, D, UNIFORM_PAGE>::run(a);
}

}  // namespace pkv

namespace pkv_launch {

template <typename T, int D>
static hipError_t launch_decode_t(const pkv::DecodeArgs& a, bool uniform, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.hkv) * a.batch * a.num_splits);
  constexpr bool wide = (sizeof(T) == 4);
  if (uniform) {
    if constexpr (wide)
      hipLaunchKernelGGL((pkv::decode_splitkv_kernel_wide<T, D, true>), grid, dim3(256), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((pkv::decode_splitkv_kernel<T, D, true>), grid, dim3(256), 0, stream, a);
  } else {
    if constexpr (wide)
      hipLaunchKernelGGL((pkv::decode_splitkv_kernel_wide<T, D, false>), grid, dim3(256), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((pkv::decode_splitkv_kernel<T, D, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t decode_splitkv(const pkv::DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
  // tiles are 32 tokens starting at multiples of 32 inside a split; with
  // page_size % 32 == 0 and chunk % page_size == 0 a tile never crosses a page
  const bool uniform = (a.page_size % 32 == 0) && (a.chunk % a.page_size == 0);
  if (dtype == PKV_BF16) {
    if (head_dim == 128) return launch_decode_t<pkv::bf16_t, 128>(a, uniform, stream);
    return launch_decode_t<pkv::bf16_t, 64>(a, uniform, stream);
  }
  if (head_dim == 128) return launch_decode_t<float, 128>(a, uniform, stream);
  return launch_decode_t<float, 64>(a, uniform, stream);
}

}  // namespace pkv_launch

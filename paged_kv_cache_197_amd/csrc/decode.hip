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
#include "splits.hpp"

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
  static __device__ __forceinline__ void consume(const Tile& cur, int ts, int end, int lo, int g,
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
    const int first = lo - ts;   // tokens before it are below the key window (first tile only)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = st[e >> 2][e & 3] * scale_log2;
      x[e] = (tok_of(g, e) < valid && tok_of(g, e) >= first) ? sv : neg_inf();
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
    const int h0 = kvh * G;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;

    const SplitPick pick = pick_split(a, blockIdx.x / a.hkv, true, lane);
    const int b = __builtin_amdgcn_readfirstlane(pick.b);
    const int s = __builtin_amdgcn_readfirstlane(pick.s);
    const int L = __builtin_amdgcn_readfirstlane(pick.L);
    const int start0 = static_cast<int>(min<int64_t>(static_cast<int64_t>(s) * a.chunk, L));
    const int end = static_cast<int>(min<int64_t>(static_cast<int64_t>(start0) + a.chunk, L));
    // first visible key under a sliding window / local chunks; tiles start on
    // a multiple of 32 (splits do), keys below lo are masked
    const int lo = L > 0 ? key_lower_bound(L - 1, a.window_left, a.attn_chunk) : 0;
    const int start = max(start0, lo / 32 * 32);

    const bool single = (a.num_splits == 1);
    if (max(start0, lo) >= end) {
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
      const char* qrow = static_cast<const char*>(split_query(a, start0, L)) +
                         (static_cast<int64_t>(b) * a.hq + h0 + min(c, G - 1)) * D * EB;
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        qop[j] = load_chunk<KDW>(qrow + (32 * j + 8 * g) * EB);
      }
      if (a.q_scale != nullptr) {   // q * factor, rounded back to the element type
        const float f = a.q_scale[b];
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          if constexpr (IS_BF16) {
#pragma unroll
            for (int w = 0; w < KDW; ++w)
              qop[j].w[w] = pack_bf16x2(bf16lo(qop[j].w[w]) * f, bf16hi(qop[j].w[w]) * f);
          } else {
#pragma unroll
            for (int w = 0; w < KDW; ++w)
              qop[j].w[w] = __float_as_uint(__uint_as_float(qop[j].w[w]) * f);
          }
        }
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
        consume(ta, start + 32 * tile, end, lo, g, a.scale_log2, qop, acc, m_run, l_run);
        tile += 4;
        if (tile > last) break;
        raw_n = raw_nn;
        raw_nn = fetch_raw(a, pt_row, start + 32 * ahead(tile, 2), end, lane);
        {
          const int ts = start + 32 * ahead(tile, 1);
          fetch_data(a, slot_base(a, raw_n, ts, end, lane), ts, end, kvh, c, g, ta);
        }
        __builtin_amdgcn_sched_barrier(0);
        consume(tb, start + 32 * tile, end, lo, g, a.scale_log2, qop, acc, m_run, l_run);
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

// ---------------------------------------------------------------------------
// bf16 decode over kv-head groups. The general kernel above reads one kv
// head's 256-byte slice of each token row in 64-byte pieces; on a paged cache
// that pattern streams well below what HBM sustains. Here a workgroup owns
// HPW = 256 / D adjacent kv heads, so every token row contributes one
// contiguous 512-byte run, fetched by half-waves (32 lanes x 16 B, two rows
// per instruction, non-temporal: the cache is read once).
//
// Each wave takes 16-token tiles w, w+4, ... of the split. A tile is loaded
// into registers one tile ahead, then written to the wave's private LDS
// region, from which the MFMA operands are read in the layout they need; no
// workgroup barrier is involved until the final merge.
//
// The HPW heads are treated as one virtual row of VD = 256 dims. The 16 MFMA
// columns hold the HPW * G query heads of the group (G <= 16 / HPW); the
// query operand is zero outside its own kv head's dims, so
//   S^T [16 tok x 16 cols] = Krow [16 x 256] . Qpad^T [256 x 16]
// is exact for every column (8 16x16x32 MFMAs), and
//   O^T [256 x 16 cols] += Vrow^T [256 x 16 tok] . P^T [16 x 16]
// (16 16x16x16 MFMAs) yields each column's output in the rows of its own kv
// head; the other rows are discarded. Lane (c = lane % 16, g = lane / 16)
// owns column c: its S^T accumulator holds tokens 4g..4g+3, the k-group its
// P^T operand needs, so softmax state stays in the lane.
// O^T block n, row r is virtual dim 128 * (n / 8) + 8 r + n % 8: a lane reads
// two 16-byte pieces per token (dims 8c.. and 128 + 8c..), and sixteen lanes
// of one token read 256 consecutive bytes (no bank conflicts).
template <int D>
struct DecodeGroupKernel {
  static constexpr int HPW = 256 / D;             // kv heads per workgroup
  static constexpr int TT = 16;                   // tokens per wave tile
  static constexpr int ROW = 512;                 // bytes of the group's row slice
  static constexpr int STRIDE = ROW + 16;         // LDS row stride (rows 4 banks apart)
  static constexpr int WAVE_LDS = 2 * TT * STRIDE;
  static constexpr int LDS_BYTES = 4 * WAVE_LDS;
  static_assert(64 * 64 * 4 <= WAVE_LDS, "merge buffer fits a wave's tile region");

  typedef short s16x4 __attribute__((ext_vector_type(4)));

  struct Stage {
    u32x4 k[8];
    u32x4 v[8];
  };

  static __device__ __forceinline__ u32x4 ld_nt(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }

  // Page-table entry for a tile: one per tile when pages hold whole tiles,
  // else lane l holds the entry of token l % 16.
  template <bool UNIFORM>
  static __device__ __forceinline__ int32_t fetch_raw(const DecodeArgs& a, const int32_t* pt_row,
                                                      int ts, int end, int lane) {
    if constexpr (UNIFORM) {
      return pt_row[ts / a.page_size];
    } else {
      const int t = min(ts + (lane & 15), end - 1);
      return pt_row[t / a.page_size];
    }
  }

  // Row r = 2i + lane / 32 of the tile, bytes [16 (lane % 32), +16) of the
  // group's slice, for K and V.
  template <bool UNIFORM>
  static __device__ __forceinline__ void load(const DecodeArgs& a, int32_t raw, int ts, int end,
                                              int lane, int64_t row_bytes, int64_t col,
                                              Stage& st) {
    const char* kb = static_cast<const char*>(a.k) + col + 16 * (lane & 31);
    const char* vb = static_cast<const char*>(a.v) + col + 16 * (lane & 31);
    const int half = lane >> 5;
    if constexpr (UNIFORM) {
      const int64_t slot0 = clamp_index(raw, a.num_pages) * a.page_size + ts % a.page_size;
      const int lim = end - 1 - ts;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t off = (slot0 + min(2 * i + half, lim)) * row_bytes;
        st.k[i] = ld_nt(kb + off);
        st.v[i] = ld_nt(vb + off);
      }
    } else {
      const int t = min(ts + (lane & 15), end - 1);
      const int slot = static_cast<int>(clamp_index(raw, a.num_pages)) * a.page_size + t % a.page_size;
      // row 2i + half's slot: read from lanes 2i and 2i + 1 into scalar
      // registers (no LDS permute on the way to the loads)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int s0 = __builtin_amdgcn_readlane(slot, 2 * i);
        const int s1 = __builtin_amdgcn_readlane(slot, 2 * i + 1);
        const int64_t off = static_cast<int64_t>(half ? s1 : s0) * row_bytes;
        st.k[i] = ld_nt(kb + off);
        st.v[i] = ld_nt(vb + off);
      }
    }
  }

  static __device__ __forceinline__ void stash(char* my, int lane, const Stage& st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 2 * i + (lane >> 5);
      *reinterpret_cast<u32x4*>(my + row * STRIDE + 16 * (lane & 31)) = st.k[i];
      *reinterpret_cast<u32x4*>(my + (TT + row) * STRIDE + 16 * (lane & 31)) = st.v[i];
    }
  }

  template <bool EXT>
  static __device__ __forceinline__ void compute(const char* my, int c, int g, int valid,
                                                 int first, float scale_log2,
                                                 const u32x4 (&qop)[8],
                                                 f32x4 (&acc)[16], float& m_run, float& l_run) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 kw = *reinterpret_cast<const u32x4*>(my + c * STRIDE + 64 * j + 16 * g);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), as_bf16x8(qop[j]), s, 0, 0, 0);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // keys [first, valid) of the tile: one unsigned range test
      const bool in = EXT ? static_cast<unsigned>(4 * g + i - first) <
                                static_cast<unsigned>(valid - first)
                          : 4 * g + i < valid;
      x[i] = in ? s[i] * scale_log2 : neg_inf();
    }
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = max_over_groups16(mt);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int n = 0; n < 16; ++n) acc[n] *= alpha;
    }
    const u32x2 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    const s16x4 pb = __builtin_bit_cast(s16x4, pw);

    // V rows 4g..4g+3: dims [8c, 8c + 8) and [128 + 8c, 128 + 8c + 8)
    u32x4 lo[4], hi[4];
    const char* vt = my + (TT + 4 * g) * STRIDE + 16 * c;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lo[t] = *reinterpret_cast<const u32x4*>(vt + t * STRIDE);
      hi[t] = *reinterpret_cast<const u32x4*>(vt + t * STRIDE + 256);
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const u32x4(&w)[4] = (n < 8) ? lo : hi;
      const int k = (n & 7) >> 1;
      u32x2 vw;
      if ((n & 1) == 0) {
        vw.x = pair_lo(w[0][k], w[1][k]);
        vw.y = pair_lo(w[2][k], w[3][k]);
      } else {
        vw.x = pair_hi(w[0][k], w[1][k]);
        vw.y = pair_hi(w[2][k], w[3][k]);
      }
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vw), pb, acc[n],
                                                         0, 0, 0);
    }
  }

  // EXT: the variant with a lower key bound (sliding window, local chunks)
  // and the per-split query choice and scaling of dual chunk attention.
  // Merge of a request's parts for the group's ncol heads, run by the last
  // part to finish: n parts whose rows start at part_row + k * part_stride
  // (k in order), read back at device scope from o_part / lse_part, combined
  // in that order with the arithmetic of merge_state and written to out / lse
  // rows out_row .. out_row + ncol. Thread t takes column t / (D / 8), dims
  // 8 (t % (D / 8)) + [0, 8).
  static __device__ __forceinline__ void merge_parts(const DecodeArgs& a, int64_t part_row, int64_t part_stride,
                                     int n, int64_t out_row, int ncol) {
    constexpr int PER_COL = D / 8;
    constexpr int BATCH = 8;
    const int c2 = threadIdx.x / PER_COL;
    const int dq = (threadIdx.x % PER_COL) * 8;
    if (c2 >= ncol) return;
    auto lse_of = [&](int k) {
      const auto r = coherent_rsrc(a.lse_part + part_row + k * part_stride,
                                   static_cast<uint32_t>(ncol * 4));
      return load_coherent1(r, static_cast<uint32_t>(c2 * 4));
    };
    float m = neg_inf();
    for (int k0 = 0; k0 < n; k0 += BATCH) {
      float ls[BATCH];
#pragma unroll
      for (int q = 0; q < BATCH; ++q) ls[q] = (k0 + q < n) ? lse_of(k0 + q) : neg_inf();
#pragma unroll
      for (int q = 0; q < BATCH; ++q) m = fmaxf(m, ls[q]);
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float total = 0.f;
    if (m != neg_inf()) {
      for (int k0 = 0; k0 < n; k0 += BATCH) {
        float ls[BATCH];
        f32x4 v[BATCH][2];
#pragma unroll
        for (int q = 0; q < BATCH; ++q) {
          if (k0 + q < n) {
            const auto r = coherent_rsrc(a.o_part + (part_row + (k0 + q) * part_stride) * D,
                                         static_cast<uint32_t>(ncol * D * 4));
            const uint32_t off = static_cast<uint32_t>((c2 * D + dq) * 4);
            v[q][0] = load_coherent4(r, off);
            v[q][1] = load_coherent4(r, off + 16);
            ls[q] = lse_of(k0 + q);
          }
        }
#pragma unroll
        for (int q = 0; q < BATCH; ++q) {
          if (k0 + q >= n) break;
          const float w = merge_weight(ls[q], m);
          if (w == 0.f) continue;
          const float vv[8] = {v[q][0][0], v[q][0][1], v[q][0][2], v[q][0][3],
                               v[q][1][0], v[q][1][1], v[q][1][2], v[q][1][3]};
          merge_add(w, vv, acc, total);
        }
      }
    }
    const float inv = merge_norm(total);
    const u32x4 w4 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                      pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.out) + (out_row + c2) * D + dq) = w4;
    if (a.lse != nullptr && dq == 0) a.lse[out_row + c2] = merge_lse(m, total);
  }

  // One lane's share of an attend() result: the normalised output of column
  // c, dims d0 + [0, 8), and the column's LSE; each (column, dims) piece has
  // exactly one owner lane, and lse_lane marks one owner per column.
  struct Piece {
    float o[8];
    float lse;
    int d0;
    bool owner;
    bool lse_lane;
  };

  // Attention of group grp's query heads over keys [start, end) of request b
  // (start a multiple of TT; keys below lo masked; end > max(start, lo)),
  // with query rows from qsrc. Wave w takes tiles w, w+4, ... and keeps its own
  // state; the four states are merged through LDS. Every thread passes a
  // workgroup barrier after the last LDS read, so LDS may be reused at once.
  template <bool UNIFORM, bool EXT>
  static __device__ __forceinline__ void attend(const DecodeArgs& a, const void* qsrc, int b, int grp, int start,
                                int end, int lo, Piece& pc) {
    extern __shared__ __align__(16) char smem[];
    __shared__ float sm_m[4][16];
    __shared__ float sm_l[4][16];
    const int G = a.hq / a.hkv;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int ncol = HPW * G;                 // query heads of the group
    const int h0 = grp * ncol;                // first query head of the group

    // Qpad^T operand, k-step j: dims 32j + 8g + [0, 8) of the virtual row,
    // nonzero only where they belong to column c's kv head.
    const int kk = c / G;                     // column's kv head within the group
    u32x4 qop[8];
    {
      const int head = h0 + min(c, ncol - 1);
      const char* qrow = static_cast<const char*>(qsrc) + (static_cast<int64_t>(b) * a.hq + head) * D * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) qop[j] = *reinterpret_cast<const u32x4*>(qrow + ((32 * j + 8 * g) % D) * 2);
      if (EXT && a.q_scale != nullptr) {   // q * factor, rounded back to bf16
        const float f = a.q_scale[b];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          qop[j].x = pack_bf16x2(bf16lo(qop[j].x) * f, bf16hi(qop[j].x) * f);
          qop[j].y = pack_bf16x2(bf16lo(qop[j].y) * f, bf16hi(qop[j].y) * f);
          qop[j].z = pack_bf16x2(bf16lo(qop[j].z) * f, bf16hi(qop[j].z) * f);
          qop[j].w = pack_bf16x2(bf16lo(qop[j].w) * f, bf16hi(qop[j].w) * f);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool mine = (c < ncol) && ((32 * j + 8 * g) / D == kk);
        qop[j].x = mine ? qop[j].x : 0u;
        qop[j].y = mine ? qop[j].y : 0u;
        qop[j].z = mine ? qop[j].z : 0u;
        qop[j].w = mine ? qop[j].w : 0u;
        retire(qop[j].x);
        retire(qop[j].y);
        retire(qop[j].z);
        retire(qop[j].w);
      }
    }

    f32x4 acc[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf();
    float l_run = 0.f;

    char* my = smem + wave * WAVE_LDS;
    const int32_t* pt_row = a.pt + static_cast<int64_t>(b) * a.pt_stride;
    const int64_t row_bytes = static_cast<int64_t>(a.hkv) * D * 2;
    const int64_t col = static_cast<int64_t>(grp) * ROW;
    const int n_tiles = (end - start + TT - 1) / TT;

    int tile = wave;
    if (tile < n_tiles) {
      const int last = n_tiles - 1 - ((n_tiles - 1 - tile) & 3);   // this wave's last tile
      auto ahead = [&](int t, int k) { return min(t + 4 * k, last); };
      Stage st;
      int32_t raw_n = fetch_raw<UNIFORM>(a, pt_row, start + TT * ahead(tile, 1), end, lane);
      load<UNIFORM>(a, fetch_raw<UNIFORM>(a, pt_row, start + TT * tile, end, lane), start + TT * tile,
                    end, lane, row_bytes, col, st);
      stash(my, lane, st);
      while (true) {
        const int32_t raw_nn = fetch_raw<UNIFORM>(a, pt_row, start + TT * ahead(tile, 2), end, lane);
        const bool more = tile + 4 <= last;
        if (more)
          load<UNIFORM>(a, raw_n, start + TT * (tile + 4), end, lane, row_bytes, col, st);
        __builtin_amdgcn_sched_barrier(0);   // the next tile's loads go out before the MFMAs
        compute<EXT>(my, c, g, end - (start + TT * tile), lo - (start + TT * tile),
                        a.scale_log2, qop, acc, m_run, l_run);
        if (!more) break;
        tile += 4;
        stash(my, lane, st);   // same wave: its LDS reads above complete first
        raw_n = raw_nn;
      }
    }

    // ---- merge the four waves' states through LDS ----
    // region of wave w: [lane][16-byte piece], piece 4i + n/4 holds acc[n..n+3][i],
    // swizzled by lane % 16 so that a wave's stores and loads spread over the banks
    const float l_tot = sum_over_groups16(l_run);
    if (g == 0) {
      sm_m[wave][c] = m_run;
      sm_l[wave][c] = l_tot;
    }
    {
      float4* reg = reinterpret_cast<float4*>(my) + lane * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          reg[(4 * i + q4) ^ c] =
              make_float4(acc[4 * q4][i], acc[4 * q4 + 1][i], acc[4 * q4 + 2][i], acc[4 * q4 + 3][i]);
    }
    __syncthreads();

    // wave i writes row i of every block: lane (c, g) holds virtual dims
    // 128 h + 32 g + 8 i + [0, 8); it is the owner when they are column c's.
    const int i = wave;
    const int hsel = (HPW == 2) ? kk : (kk >> 1);
    pc.owner = (c < ncol) && (HPW == 2 || ((g >> 1) == (kk & 1)));
    pc.d0 = (32 * g + 8 * i) % D;
    pc.lse_lane = (i == 0) && (pc.d0 == 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) pc.o[e] = 0.f;
    pc.lse = 0.f;
    if (pc.owner) {
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
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4* reg = reinterpret_cast<const float4*>(smem + w * WAVE_LDS) + lane * 16;
        const float4 u0 = reg[(4 * i + 2 * hsel) ^ c];
        const float4 u1 = reg[(4 * i + 2 * hsel + 1) ^ c];
        pc.o[0] += f[w] * u0.x;
        pc.o[1] += f[w] * u0.y;
        pc.o[2] += f[w] * u0.z;
        pc.o[3] += f[w] * u0.w;
        pc.o[4] += f[w] * u1.x;
        pc.o[5] += f[w] * u1.y;
        pc.o[6] += f[w] * u1.z;
        pc.o[7] += f[w] * u1.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) pc.o[e] *= inv;
      pc.lse = (M + fast_log2(Ltot)) * kLn2;
    }
    __syncthreads();   // LDS free for the caller
  }

  // Final output of column c of the group from a Piece (owner lanes).
  static __device__ __forceinline__ void write_out(const DecodeArgs& a, int64_t row,
                                                   const Piece& pc) {
    if (!pc.owner) return;
    const u32x4 w4 = {pack_bf16x2(pc.o[0], pc.o[1]), pack_bf16x2(pc.o[2], pc.o[3]),
                      pack_bf16x2(pc.o[4], pc.o[5]), pack_bf16x2(pc.o[6], pc.o[7])};
    *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.out) + row * D + pc.d0) = w4;
    if (a.lse != nullptr && pc.lse_lane) a.lse[row] = pc.lse;
  }

  // (0, -inf) for the group's columns of request b (no visible key)
  static __device__ __forceinline__ void write_empty(const DecodeArgs& a, int b, int h0, int ncol) {
    for (int i = threadIdx.x; i < ncol * D; i += blockDim.x)
      static_cast<bf16_t*>(a.out)[(static_cast<int64_t>(b) * a.hq + h0 + i / D) * D + i % D].bits = 0;
    if (a.lse != nullptr)
      for (int i = threadIdx.x; i < ncol; i += blockDim.x)
        a.lse[static_cast<int64_t>(b) * a.hq + h0 + i] = neg_inf();
  }

  // Hand a part over at device scope (rows part_row0 + column), count it on
  // `counter`; the part that completes the count (n parts) merges the parts
  // [first_row + k * stride] into the output rows of request b.
  static __device__ __forceinline__ void hand_over(const DecodeArgs& a, const Piece& pc, int64_t part_row0,
                                   int ncol, int* counter, int n, int64_t first_row,
                                   int64_t stride, int64_t out_row) {
    __shared__ int sm_last;
    const int c = threadIdx.x & 15;
    if (pc.owner) {
      const auto ro = coherent_rsrc(a.o_part + part_row0 * D, static_cast<uint32_t>(ncol * D * 4));
      const uint32_t off = static_cast<uint32_t>((c * D + pc.d0) * 4);
      store_coherent(ro, off, f32x4{pc.o[0], pc.o[1], pc.o[2], pc.o[3]});
      store_coherent(ro, off + 16, f32x4{pc.o[4], pc.o[5], pc.o[6], pc.o[7]});
      if (pc.lse_lane)
        store_coherent(coherent_rsrc(a.lse_part + part_row0, static_cast<uint32_t>(ncol * 4)),
                       static_cast<uint32_t>(c * 4), pc.lse);
    }
    wait_all_vmem();
    __syncthreads();   // every wave's share has been written through
    if (threadIdx.x == 0) sm_last = (counter_add(counter, 1) == n - 1);
    __syncthreads();
    if (!sm_last) return;
    merge_parts(a, first_row, stride, n, out_row, ncol);
    if (threadIdx.x == 0) counter_reset(counter);   // ready for the next call
  }

  // Fixed splits: workgroup (unit, group) takes split s of request b (the
  // order of pick_split); partials to o_part / lse_part [S, B, Hq], or merged
  // in the launch when counters are given.
  template <bool UNIFORM, bool EXT>
  static __device__ __forceinline__ void run_fixed(const DecodeArgs& a) {
    const int G = a.hq / a.hkv;
    const int ngrp = a.hkv / HPW;
    const int grp = blockIdx.x % ngrp;
    const int lane = threadIdx.x & 63;
    const SplitPick pick = pick_split(a, blockIdx.x / ngrp, EXT, lane);
    const int b = __builtin_amdgcn_readfirstlane(pick.b);
    const int s = __builtin_amdgcn_readfirstlane(pick.s);
    const int c = lane & 15;
    const int ncol = HPW * G;                 // query heads of the group
    const int h0 = grp * ncol;                // first query head of the group

    const int L = __builtin_amdgcn_readfirstlane(pick.L);
    const int start0 = static_cast<int>(min<int64_t>(static_cast<int64_t>(s) * a.chunk, L));
    const int end = static_cast<int>(min<int64_t>(static_cast<int64_t>(start0) + a.chunk, L));
    // first visible key under a sliding window / local chunks; tiles start on
    // a multiple of TT (splits do), keys below lo are masked
    const int lo = (EXT && L > 0) ? key_lower_bound(L - 1, a.window_left, a.attn_chunk) : 0;
    const int start = EXT ? max(start0, lo / TT * TT) : start0;
    const bool single = (a.num_splits == 1);
    // merged decode: the request's non-empty splits are [sf, sf + n_ne)
    const bool merged = (a.counters != nullptr) && !single;
    const int v1 = static_cast<int>(min<int64_t>(L, static_cast<int64_t>(a.num_splits) * a.chunk));
    const int v0 = min(lo, v1);
    const int sf = v0 / a.chunk;
    const int n_ne = v0 < v1 ? (v1 - 1) / a.chunk - sf + 1 : 0;

    if (max(start0, lo) >= end) {   // empty split: (0, -inf)
      if (merged) {
        // nothing to hand over; a request with no visible key at all gets
        // (0, -inf) from its split 0
        if (n_ne == 0 && s == 0) write_empty(a, b, h0, ncol);
        return;
      }
      for (int i = threadIdx.x; i < ncol * D; i += blockDim.x) {
        const int64_t row = static_cast<int64_t>(b) * a.hq + h0 + i / D;
        const int d = i % D;
        if (single) static_cast<bf16_t*>(a.out)[row * D + d].bits = 0;
        else a.o_part[(static_cast<int64_t>(s) * a.batch * a.hq + row) * D + d] = 0.f;
      }
      for (int i = threadIdx.x; i < ncol; i += blockDim.x) {
        const int64_t row = static_cast<int64_t>(b) * a.hq + h0 + i;
        if (single) {
          if (a.lse) a.lse[row] = neg_inf();
        } else {
          a.lse_part[static_cast<int64_t>(s) * a.batch * a.hq + row] = neg_inf();
        }
      }
      return;
    }

    Piece pc;
    attend<UNIFORM, EXT>(a, EXT ? split_query(a, start0, L) : a.q, b, grp, start, end, lo, pc);
    const int64_t out_row0 = static_cast<int64_t>(b) * a.hq + h0;
    const int64_t split_rows = static_cast<int64_t>(a.batch) * a.hq;
    if (merged) {
      hand_over(a, pc, s * split_rows + out_row0, ncol, a.counters + static_cast<int64_t>(b) * ngrp + grp,
                n_ne, sf * split_rows + out_row0, split_rows, out_row0);
      return;
    }
    if (single) {
      write_out(a, out_row0 + c, pc);
    } else if (pc.owner) {
      float* dst = a.o_part + (s * split_rows + out_row0 + c) * D + pc.d0;
      *reinterpret_cast<float4*>(dst) = make_float4(pc.o[0], pc.o[1], pc.o[2], pc.o[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(pc.o[4], pc.o[5], pc.o[6], pc.o[7]);
      if (pc.lse_lane) a.lse_part[s * split_rows + out_row0 + c] = pc.lse;
    }
  }

  // Balanced ranges (merged decode with a.units > 0): the visible keys of all
  // requests, in TT-key tiles from the tile that holds each request's first
  // visible key, are laid end to end and cut into a.units ranges of equal
  // tile count (at least kMinRangeTiles each; later ranges may be empty).
  // Workgroup (range r, group) walks the requests its range covers; a request
  // covered by one range is written directly, else each range's part goes to
  // partial row r + b (unique: ranges follow the requests' order) and the last
  // of the request's ranges to finish merges them in range order.
  static constexpr int kMinRangeTiles = 8;

  template <bool EXT>
  static __device__ __forceinline__ void visible(const DecodeArgs& a, int j, int& L, int& v0,
                                                 int& nt) {
    const int64_t cap = static_cast<int64_t>(a.pt_stride) * a.page_size;
    L = (j < a.batch) ? static_cast<int>(min<int64_t>(max(a.kv_lens[j], 0), cap)) : 0;
    v0 = (EXT && L > 0) ? key_lower_bound(L - 1, a.window_left, a.attn_chunk) : 0;
    nt = (L > v0) ? (L - 1) / TT - v0 / TT + 1 : 0;
  }

  template <bool UNIFORM, bool EXT>
  static __device__ __forceinline__ void run_balanced(const DecodeArgs& a) {
    const int G = a.hq / a.hkv;
    const int ngrp = a.hkv / HPW;
    const int grp = blockIdx.x % ngrp;
    const int r = blockIdx.x / ngrp;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int ncol = HPW * G;
    const int h0 = grp * ncol;

    // total tiles; requests with no visible key get (0, -inf) from range 0
    int64_t NT = 0;
    for (int j0 = 0; j0 < a.batch; j0 += 64) {
      int L, v0, nt;
      visible<EXT>(a, j0 + lane, L, v0, nt);
      int x = nt;
#pragma unroll
      for (int d = 1; d < 64; d *= 2) x += __shfl_xor(x, d);
      NT += __builtin_amdgcn_readfirstlane(x);
      if (r == 0) {
        unsigned long long none = __ballot(j0 + lane < a.batch && nt == 0);
        while (none) {
          const int k = __builtin_ctzll(none);
          none &= none - 1;
          write_empty(a, j0 + k, h0, ncol);
        }
      }
    }
    const int64_t units = max<int64_t>(1, min<int64_t>(a.units, NT / kMinRangeTiles));
    if (r >= units) return;
    const int64_t t0 = r * NT / units;
    const int64_t t1 = (r + 1) * NT / units;
    // range holding global tile t: the largest q with floor(q NT / units) <= t
    auto range_of = [&](int64_t t) { return static_cast<int>(((t + 1) * units - 1) / NT); };

    // the request holding tile t0 (b) and its first global tile (pb)
    int b = a.batch;
    int64_t pb = 0;
    {
      int64_t base = 0;
      for (int j0 = 0; j0 < a.batch; j0 += 64) {
        int L, v0, nt;
        visible<EXT>(a, j0 + lane, L, v0, nt);
        int incl = nt;
#pragma unroll
        for (int d = 1; d < 64; d *= 2) {
          const int y = __shfl_up(incl, d);
          if (lane >= d) incl += y;
        }
        const int64_t lo_t = base + incl - nt;
        const unsigned long long hit = __ballot(nt > 0 && lo_t <= t0 && t0 < lo_t + nt);
        if (hit) {
          const int k = __builtin_ctzll(hit);
          b = j0 + k;
          pb = base + __builtin_amdgcn_readlane(incl - nt, k);
          break;
        }
        base += __builtin_amdgcn_readlane(incl, 63);
      }
    }

    // walk the requests the range covers; only scalar state crosses a segment
    // (each segment reads the arguments again from the kernel's argument
    // segment, where `a` lives, through a pointer the compiler cannot follow,
    // so that they are not all held in registers across the segments)
    typedef const __attribute__((address_space(4))) DecodeArgs* KArgPtr;
    int64_t pos = t0;
    const int batch = a.batch;
    while (pos < t1 && b < batch) {
      KArgPtr ap = (KArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(ap));
      const DecodeArgs a = *(const DecodeArgs*)ap;
      int Lb, v0b, ntb;
      visible<EXT>(a, b, Lb, v0b, ntb);
      if (ntb > 0) {
        const int lt0 = static_cast<int>(pos - pb);
        const int lt1 = static_cast<int>(min(t1, pb + ntb) - pb);
        const int first_key = v0b / TT * TT;
        const int start = first_key + TT * lt0;
        const int end = min(first_key + TT * lt1, Lb);
        Piece pc;
        attend<UNIFORM, EXT>(a, a.q, b, grp, start, end, v0b, pc);
        const int r_first = range_of(pb);
        const int r_last = range_of(pb + ntb - 1);
        const int64_t out_row0 = static_cast<int64_t>(b) * a.hq + h0;
        if (r_first == r_last) {
          write_out(a, out_row0 + c, pc);
        } else {
          hand_over(a, pc, static_cast<int64_t>(r + b) * a.hq + h0, ncol,
                    a.counters + static_cast<int64_t>(b) * ngrp + grp, r_last - r_first + 1,
                    static_cast<int64_t>(r_first + b) * a.hq + h0, a.hq, out_row0);
        }
        pos = pb + lt1;
        pb += ntb;
      }
      ++b;
    }
  }

  template <bool UNIFORM, bool EXT, bool BAL>
  static __device__ void run(const DecodeArgs& a) {
    if constexpr (BAL) run_balanced<UNIFORM, EXT>(a);
    else run_fixed<UNIFORM, EXT>(a);
  }
};

// BAL: balanced ranges (merged decode) instead of fixed splits
template <int D, bool UNIFORM, bool EXT, bool BAL>
__global__ __launch_bounds__(256, 2) void decode_group_kernel(DecodeArgs a) {
  DecodeGroupKernel<D>::template run<UNIFORM, EXT, BAL>(a);
}

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

template <int D, bool BAL>
static hipError_t launch_decode_group_t(const pkv::DecodeArgs& a, const dim3 grid,
                                        hipStream_t stream) {
  constexpr unsigned lds = pkv::DecodeGroupKernel<D>::LDS_BYTES;
  // whole 16-token tiles on one page: page_size % 16 == 0 (splits start on pages)
  // (a sliding window, local chunks or dual chunk attention take the variant
  // with the lower key mask and the per-split query choice)
  const bool window = a.window_left >= 0 || a.attn_chunk > 0 || a.dca_chunk > 0 ||
                      a.q_scale != nullptr;
  if (a.page_size % 16 == 0) {
    if (window)
      hipLaunchKernelGGL((pkv::decode_group_kernel<D, true, true, BAL>), grid, dim3(256), lds,
                         stream, a);
    else
      hipLaunchKernelGGL((pkv::decode_group_kernel<D, true, false, BAL>), grid, dim3(256), lds,
                         stream, a);
  } else {
    if (window)
      hipLaunchKernelGGL((pkv::decode_group_kernel<D, false, true, BAL>), grid, dim3(256), lds,
                         stream, a);
    else
      hipLaunchKernelGGL((pkv::decode_group_kernel<D, false, false, BAL>), grid, dim3(256), lds,
                         stream, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_group(const pkv::DecodeArgs& a, hipStream_t stream) {
  constexpr int HPW = pkv::DecodeGroupKernel<D>::HPW;
  const unsigned groups = static_cast<unsigned>(a.hkv / HPW);
  if (a.units > 0)
    return launch_decode_group_t<D, true>(a, dim3(groups * static_cast<unsigned>(a.units)), stream);
  return launch_decode_group_t<D, false>(
      a, dim3(groups * static_cast<unsigned>(a.batch) * a.num_splits), stream);
}

// kv-head groups (bf16): HPW = 256 / D heads whose G query heads fit 16
// columns, and slot numbers that fit 32 bits (per-token pages are shuffled as
// int32). Returns the number of groups per request, or 0 when the general
// kernel runs instead.
int decode_groups(const pkv::DecodeArgs& a, int dtype, int head_dim) {
  if (dtype != PKV_BF16) return 0;
  const int hpw = 256 / head_dim;
  const int G = a.hq / a.hkv;
  const bool group = (a.hkv % hpw == 0) && (hpw * G <= 16) &&
                     (a.num_pages * a.page_size <= INT_MAX);
  return group ? a.hkv / hpw : 0;
}

hipError_t decode_splitkv(const pkv::DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
  if (decode_groups(a, dtype, head_dim) > 0) {
    if (head_dim == 128) return launch_decode_group<128>(a, stream);
    return launch_decode_group<64>(a, stream);
  }
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

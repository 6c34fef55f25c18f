// sparse_topk_decode: top-k index-gathered MLA decode over one latent KV head.
// [NSA] forward_decode / transform_index_page_table_decode: top-k logical
// indices -> cache slots through the request's token table, -1 entries
// skipped; [NSA] _forward_fa3: score over the whole 576-wide row
// ([c_kv 512 | k_rope 64] against [q_nope | q_rope]), value = c_kv.
//
// Work decomposition: one workgroup per (head block, request, key split). A
// head block is 64 heads (eight waves: two quads of four) when the head count
// is a multiple of 64, else 32 heads (one quad). The workgroup translates its
// slice of the top-k list into cache slots once (kept in LDS), then walks it
// in 32-key tiles. A tile's 32 rows (1152 B each) are copied by direct
// global-to-LDS loads into a three-stage ring two tiles ahead of their use,
// and both quads work on the same tile. Per tile and quad:
//   * QK: wave w of the quad computes a partial S^T [32 keys x 32 heads] over
//     score dims [144w, 144w + 144) (nine 32x32x16 MFMAs, Q^T in registers)
//     and publishes it in LDS;
//   * softmax: wave w sums the four partials for heads [8w, 8w + 8) only, runs
//     the online softmax for them and publishes P^T (bf16) and each head's
//     rescale factor, so the softmax work is not repeated across waves;
//   * PV: wave w accumulates O^T for value dims [128w, 128w + 128) (four
//     32x32x16 blocks x two 16-key k-steps); the value rows are the first 512
//     dims of the same LDS tile.
// Two workgroup barriers per tile: after QK (partials visible, every wave done
// with the previous tile, whose stage then takes the copy of tile t + 2) and
// after the softmax (P^T visible, tile t + 1 landed).
// MFMA C-layout used throughout: lane (col = lane % 32, h = lane / 32) holds
// column col (a head) and rows rho(h, r) = 8*(r/4) + 4h + r%4, r < 16 (keys
// of S^T, dims of O^T).
// LDS rows are 1168 bytes apart (the row plus 16 bytes), which puts the
// sixteen rows of a K operand read in distinct banks; a V read is 256
// consecutive bytes of one row.
// Key splits (needed to fill the chip when batch x head blocks is small) are
// merged inside the kernel: every split writes its normalised partial and LSE
// to the workspace with device-coherent stores, and the last split to finish
// (device-scope counter) reads them back the same way, merges them and writes
// the output; the counter is reset for the next call.
#include <mutex>

#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "lanes.hpp"
#include "lds_dma.hpp"

namespace pkv {

struct SparseGeom {
  static constexpr int DQK = 576;
  static constexpr int DV = 512;
  static constexpr int KT = 32;                  // keys per tile
  static constexpr int ROW = DQK * 2;            // 1152 bytes per cache row
  static constexpr int LROW = ROW + 16;          // LDS row stride (292 words: rows 36 banks apart)
  static constexpr int DMAS = (KT * LROW + 1023) / 1024;   // 1 KB copies per tile (37)
  static constexpr int TILE = DMAS * 1024;       // LDS bytes per ring stage
  static constexpr int NS = 3;                   // ring stages
  static constexpr int QK_SLICE = DQK / 4;       // 144 score dims per wave
  static constexpr int QK_STEPS = QK_SLICE / 16; // 9
  static constexpr int DV_SLICE = DV / 4;        // 128 value dims per wave
  static constexpr int NBLK = DV_SLICE / 32;     // 4
  static constexpr int MAX_KEYS_PER_SPLIT = 2048;   // slot list capacity in LDS
  static constexpr int MAX_SPLITS = 64;             // merge weight table capacity
  static constexpr int MAX_TOPK = MAX_KEYS_PER_SPLIT * MAX_SPLITS;
  static constexpr float kRescaleLog2 = 8.f;     // lazy rescale bound (log2 units)
  static constexpr int SP_BYTES = 4 * 4 * 64 * 16;  // partial S^T: [wave][reg quad][lane] float4
  static constexpr int PB_BYTES = 4 * 64 * 8;       // P^T bf16: [reg quad][lane] 4 x bf16
  static constexpr int AUX_BYTES = 32 * 4 * 3;      // per head: rescale factor, final m, l
  static constexpr int QUAD_BYTES = SP_BYTES + PB_BYTES + AUX_BYTES;
};

template <int QUADS>
struct SparseCfg : SparseGeom {
  static constexpr int W = 4 * QUADS;            // waves
  static constexpr int THREADS = 64 * W;
  static constexpr int HB = 32 * QUADS;          // heads per workgroup
  static constexpr int COPIES = (DMAS + W - 1) / W;   // most copies per tile of one wave
  static constexpr int FULL_COPIERS = DMAS - (COPIES - 1) * W;   // waves issuing COPIES of them
  static constexpr int LDS_BYTES = NS * TILE + QUADS * QUAD_BYTES + MAX_KEYS_PER_SPLIT * 4;
  static_assert(LDS_BYTES <= 160 * 1024, "fits the CU's LDS");
};

__host__ __device__ inline int sparse_quads(int hq) { return hq % 64 == 0 ? 2 : 1; }
__host__ __device__ inline int sparse_head_block(int hq) { return 32 * sparse_quads(hq); }

// splits per (request, head block) so the grid has about 256 workgroups (one
// per CU), each split keeping at least 256 keys; the last split may be shorter
__host__ __device__ inline int sparse_num_splits(int batch, int topk, int hq) {
  const int units = batch * (hq / sparse_head_block(hq));
  if (units <= 0 || topk <= 0) return 1;
  int s = (256 + units - 1) / units;
  const int by_keys = (topk + 255) / 256;
  s = s < by_keys ? s : by_keys;
  s = s < SparseGeom::MAX_SPLITS ? s : SparseGeom::MAX_SPLITS;
  const int min_for_lds = (topk + SparseGeom::MAX_KEYS_PER_SPLIT - 1) / SparseGeom::MAX_KEYS_PER_SPLIT;
  if (s < min_for_lds) s = min_for_lds;   // only above MAX_TOPK, which the entry point rejects
  return s < 1 ? 1 : s;
}

__host__ __device__ inline int sparse_keys_per_split(int topk, int splits) {
  const int k = (topk + splits - 1) / splits;
  return (k + SparseGeom::KT - 1) / SparseGeom::KT * SparseGeom::KT;
}

// workspace: counter [units] in the fixed counter region at its start, then
// o [units][S][HB][DV] bf16 and lse [units][S][HB] fp32
__host__ __device__ inline size_t sparse_ws_bytes(int units, int splits, int hb) {
  if (splits <= 1) return 0;
  const size_t o = static_cast<size_t>(units) * splits * hb * SparseGeom::DV * 2;
  const size_t l = static_cast<size_t>(units) * splits * hb * 4;
  return PKV_WORKSPACE_COUNTER_BYTES + o + l;
}

__device__ __forceinline__ int rho32(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }
// slot of lane L's float4 in a published partial: lanes 32..63 are moved by
// eight slots so that the softmax reads (lane s together with lane s + 32)
// fall in distinct banks
__device__ __forceinline__ int sp_pos(int L) { return L ^ ((L & 32) >> 2); }

template <int QUADS>
__global__ __launch_bounds__(256 * QUADS, 1) void sparse_mla_kernel(SparseArgs a, int splits,
                                                                     int kps) {
  using C = SparseCfg<QUADS>;
  typedef __attribute__((address_space(3))) char lds_char;
  extern __shared__ __align__(16) char smem[];
  __shared__ int is_last;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem));

  const int hblocks = a.hq / C::HB;
  const int units = a.batch * hblocks;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by index,
  // so giving every workgroup of request b (all head blocks and key splits,
  // which read the same latent rows) an index congruent to b mod 8 keeps the
  // request on one XCD and its rows in one L2
  const int lin = blockIdx.x;
  const int xcd = lin & 7;
  const int rest = lin >> 3;
  const int ks = rest % splits;
  const int hb = (rest / splits) % hblocks;
  const int b = (rest / splits / hblocks) * 8 + xcd;
  if (b >= a.batch) return;
  const int unit = b * hblocks + hb;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = wave >> 2;
  const int w4 = wave & 3;
  const int col = lane & 31;     // head within the quad (B / C column)
  const int h = lane >> 5;

  char* quad_lds = smem + C::NS * C::TILE + quad * C::QUAD_BYTES;
  float* sp = reinterpret_cast<float*>(quad_lds);
  char* pb = quad_lds + C::SP_BYTES;
  float* aux = reinterpret_cast<float*>(quad_lds + C::SP_BYTES + C::PB_BYTES);
  float* alpha_buf = aux;            // [32] per-head rescale of the current tile
  float* m_buf = aux + 32;           // [32] final running max per head (raw units)
  float* l_buf = aux + 64;           // [32] final denominator per head
  int32_t* slots = reinterpret_cast<int32_t*>(smem + C::NS * C::TILE + QUADS * C::QUAD_BYTES);

  const int k_begin = ks * kps;
  const int k_end = min(a.topk, k_begin + kps);
  const int nkeys = max(k_end - k_begin, 0);
  const int n_tiles = (nkeys + C::KT - 1) / C::KT;

  // Q^T operand for this wave's score slice: head col of the quad, dims
  // 144 w4 + 16j + 8h + [0, 8); in flight while the slots are translated
  const int head = hb * C::HB + 32 * quad + col;
  u32x4 qop[C::QK_STEPS];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       (static_cast<int64_t>(b) * a.hq + head) * C::DQK * 2;
#pragma unroll
    for (int j = 0; j < C::QK_STEPS; ++j)
      qop[j] = *reinterpret_cast<const u32x4*>(qrow + (C::QK_SLICE * w4 + 16 * j + 8 * h) * 2);
  }

  // ---- translate this split's top-k entries to cache slots (-1: skip) ----
  {
    const int64_t r = a.rpi[b];
    const bool row_ok = r >= 0 && r < a.r2t_rows;
    for (int i = threadIdx.x; i < n_tiles * C::KT; i += C::THREADS) {
      int32_t slot = -1;
      if (i < nkeys && row_ok) {
        const int32_t idx = a.topk_idx[static_cast<int64_t>(b) * a.topk + k_begin + i];
        if (idx >= 0 && idx < a.r2t_stride) {
          const int32_t s = a.r2t[r * a.r2t_stride + idx];
          slot = (s >= 0 && s < a.num_slots) ? s : -1;
        }
      }
      slots[i] = slot;
    }
  }
#pragma unroll
  for (int j = 0; j < C::QK_STEPS; ++j) {
    retire(qop[j].x);
    retire(qop[j].y);
    retire(qop[j].z);
    retire(qop[j].w);
  }
  __syncthreads();   // slots visible

  // ---- tile copies: copy i of a tile fills LDS bytes [1024 i, +1024) of the
  // stage, lane l the 16 bytes at o = 1024 i + 16 l: row o / 1168, chunk
  // (o % 1168) / 16 of the cache row. Lanes that land in a row's 16-byte pad
  // or past the last row copy chunk 0 of row 31, which nothing reads. Every
  // wave issues copies (copy i by wave i % W), so that the issue work, which
  // sits between the two barriers of a tile, is spread over all of them; each
  // wave's rows and row offsets are fixed and computed once. Skipped keys copy
  // row 0 and are masked in the softmax / PV.
  const char* kvb = static_cast<const char*>(a.kv);
  uint32_t rowoff[C::COPIES];   // row (bits 16..) and byte offset in the cache row
#pragma unroll
  for (int k = 0; k < C::COPIES; ++k) {
    const int i = min(wave + C::W * k, C::DMAS - 1);
    const int o = 1024 * i + 16 * lane;
    const int row = min(o / C::LROW, C::KT - 1);
    const int cb = o - row * C::LROW;
    rowoff[k] = (static_cast<uint32_t>(row) << 16) | static_cast<uint32_t>(cb < C::ROW ? cb : 0);
  }
  auto issue_tile = [&](int t) {
    const uint32_t stage = lds0 + static_cast<uint32_t>((t % C::NS) * C::TILE);
    int32_t sl[C::COPIES];
#pragma unroll
    for (int k = 0; k < C::COPIES; ++k) sl[k] = slots[t * C::KT + (rowoff[k] >> 16)];
#pragma unroll
    for (int k = 0; k < C::COPIES; ++k) {
      const int i = wave + C::W * k;
      if (i < C::DMAS) {
        const uint32_t s = static_cast<uint32_t>(max(sl[k], 0));
        lds_dma16(kvb + static_cast<uint64_t>(s) * C::ROW + (rowoff[k] & 0xffffu),
                  stage + i * 1024);
      }
    }
  };
  // wait until only the newest tile's copies are in flight
  auto wait_newest_tile = [&]() {
    if (wave < C::FULL_COPIERS) wait_vmem<C::COPIES>();
    else wait_vmem<C::COPIES - 1>();
  };
  // bit k set: key k of tile t has a slot (the same mask in every wave)
  auto tile_valid = [&](int t) -> uint32_t {
    const bool ok = slots[t * C::KT + col] >= 0;
    return static_cast<uint32_t>(__ballot(ok) & 0xffffffffull);
  };

  // per-lane byte offsets inside a tile
  // K operand of k-step j: row col, dims 144 w4 + 16 j + 8h + [0, 8)
  const uint32_t kbase = static_cast<uint32_t>(col * C::LROW + (C::QK_SLICE * w4 + 8 * h) * 2);
  // V element e of k-step t2: row 16 t2 + 8 (e / 4) + 4h + e % 4, value dims
  // 128 w4 + 4 col + [0, 4)
  const uint32_t vbase = static_cast<uint32_t>(4 * h * C::LROW + (C::DV_SLICE * w4 + 4 * col) * 2);

  f32x16 acc[C::NBLK];
#pragma unroll
  for (int n = 0; n < C::NBLK; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;

  // softmax ownership: lane L of wave w4 handles head sc = 8 w4 + (L & 7), the
  // four S^T values of lane sl = sc + 32 * sh, register quad sq
  const int sc = 8 * w4 + (lane & 7);
  const int sh = (lane >> 3) & 1;
  const int sq = lane >> 4;
  const int src_lane = sc + 32 * sh;
  float m_run = neg_inf();   // raw score units, for head sc
  float l_run = 0.f;         // partial denominator over this lane's keys

  // Schedule per tile t (two workgroup barriers):
  //   QK(t) -> partials;  A;  copy of tile t + 2 (into the stage of t - 1);
  //   softmax(t) -> P^T;  B (tile t + 1 has landed);  PV(t), with the K
  //   operands of tile t + 1 read alongside its V reads.
  u32x4 kw[C::QK_STEPS];
  auto read_k = [&](int t) {
    const char* tile = smem + (t % C::NS) * C::TILE;
#pragma unroll
    for (int j = 0; j < C::QK_STEPS; ++j)
      kw[j] = *reinterpret_cast<const u32x4*>(tile + kbase + 32 * j);
  };

  // partial S^T over this wave's 144 score dims (K operands in kw) -> LDS
  auto qk = [&]() {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int j = 0; j < C::QK_STEPS; ++j)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw[j]), as_bf16x8(qop[j]), s, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      reinterpret_cast<float4*>(sp)[(w4 * 4 + i) * 64 + sp_pos(lane)] =
          make_float4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
  };

  // softmax for heads [8 w4, 8 w4 + 8): 4 keys per lane; publishes P^T and
  // each head's rescale factor
  auto softmax = [&](uint32_t valid) {
    float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = reinterpret_cast<const float4*>(sp)[(w * 4 + sq) * 64 + sp_pos(src_lane)];
      x[0] += v.x;
      x[1] += v.y;
      x[2] += v.z;
      x[3] += v.w;
    }
    if (valid != 0xffffffffu) {
      // register 4*sq + j of lane half sh holds key 8 sq + 4 sh + j
      const uint32_t vb = valid >> (8 * sq + 4 * sh);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!(vb & (1u << j))) x[j] = neg_inf();
    }
    // the eight lanes of head sc differ in lane bits 3..5
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = max_xor8(mt);
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    // the reference max moves only when the tile max exceeds it by more than
    // 2^kRescaleLog2 in exponential units; in between the exponentials stay
    // below that bound and the sum and the output share the stale reference,
    // which the final normalisation cancels
    const bool grow = (mt - m_run) * a.scale_log2 > C::kRescaleLog2;
    const float m_ref = grow ? mt : m_run;
    const float m_use = (m_ref == neg_inf()) ? 0.f : m_ref;
    const float alpha = grow ? fast_exp2((m_run - m_use) * a.scale_log2) : 1.f;
    const float neg_mc = -m_use * a.scale_log2;
    m_run = m_ref;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(__builtin_fmaf(x[j], a.scale_log2, neg_mc));
    l_run = l_run * alpha + (p[0] + p[1]) + (p[2] + p[3]);
    u32x2 pw;
    pw.x = pack_bf16x2(p[0], p[1]);
    pw.y = pack_bf16x2(p[2], p[3]);
    reinterpret_cast<u32x2*>(pb)[sq * 64 + src_lane] = pw;
    if (lane < 8) alpha_buf[sc] = alpha;
  };

  // O^T (this wave's 128 value dims) += V^T . P^T for tile t; with `next`,
  // the K operands of tile t + 1 are read together with this tile's V
  auto pv = [&](int t, uint32_t valid, bool next) {
    const char* tile = smem + (t % C::NS) * C::TILE;
    const float alpha_c = alpha_buf[col];
    u32x2 pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = reinterpret_cast<const u32x2*>(pb)[i * 64 + lane];
    u32x2 vr[2][8];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vr[t2][e] = *reinterpret_cast<const u32x2*>(
            tile + vbase + (16 * t2 + 8 * (e >> 2) + (e & 3)) * C::LROW);
    if (next) read_k(t + 1);
    if (__any(alpha_c != 1.f)) {   // some head's reference max moved
#pragma unroll
      for (int n = 0; n < C::NBLK; ++n) acc[n] *= alpha_c;
    }
    if (valid != 0xffffffffu) {   // skipped keys: whatever row 0 holds must not reach O
      const uint32_t vb = valid >> (4 * h);   // element e of k-step t2: key 16 t2 + 8 (e/4) + 4h + e%4
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(vb & (1u << (16 * t2 + 8 * (e >> 2) + (e & 3))))) vr[t2][e] = u32x2{0u, 0u};
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const u32x4 pw = {pr[2 * t2].x, pr[2 * t2].y, pr[2 * t2 + 1].x, pr[2 * t2 + 1].y};
#pragma unroll
      for (int n = 0; n < C::NBLK; ++n) {
        const int hw = n >> 1;
        u32x4 vw;
        if ((n & 1) == 0) {
          vw.x = pair_lo(vr[t2][0][hw], vr[t2][1][hw]);
          vw.y = pair_lo(vr[t2][2][hw], vr[t2][3][hw]);
          vw.z = pair_lo(vr[t2][4][hw], vr[t2][5][hw]);
          vw.w = pair_lo(vr[t2][6][hw], vr[t2][7][hw]);
        } else {
          vw.x = pair_hi(vr[t2][0][hw], vr[t2][1][hw]);
          vw.y = pair_hi(vr[t2][2][hw], vr[t2][3][hw]);
          vw.z = pair_hi(vr[t2][4][hw], vr[t2][5][hw]);
          vw.w = pair_hi(vr[t2][6][hw], vr[t2][7][hw]);
        }
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), as_bf16x8(pw), acc[n], 0,
                                                         0, 0);
      }
    }
  };

  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) {
    issue_tile(1);
    wait_newest_tile();
  } else {
    wait_vmem<0>();
  }
  __syncthreads();   // tile 0 landed
  uint32_t valid_cur = 0xffffffffu;   // key mask of tile t
  if (n_tiles > 0) {
    read_k(0);
    valid_cur = tile_valid(0);
  }

  for (int t = 0; t < n_tiles; ++t) {
    qk();
    __syncthreads();   // A: partials visible; every wave is done with tile t - 1
    const bool more = t + 2 < n_tiles;
    if (more) issue_tile(t + 2);
    softmax(valid_cur);
    if (more) wait_newest_tile();
    else wait_vmem<0>();
    __syncthreads();   // B: P^T and rescale factors visible; tile t + 1 landed
    const uint32_t valid_pv = valid_cur;
    pv(t, valid_pv, t + 1 < n_tiles);
    if (t + 1 < n_tiles) valid_cur = tile_valid(t + 1);
    // the next barrier A orders these reads before sp / pb / the stage are rewritten
  }

  // ---- per-head totals: owners reduce their lanes' partial sums, publish ----
  {
    float l = l_run;
    l += __shfl_xor(l, 8);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (lane < 8) {
      m_buf[sc] = m_run;
      l_buf[sc] = l;
    }
  }
  __syncthreads();
  const float m_head = m_buf[col];
  const float l_tot = l_buf[col];

  // ---- this split's result for head col, value dims 128 w4 + 4*rho(h, i) + n ----
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_val =
      l_tot > 0.f ? (m_head * a.scale_log2 + fast_log2(l_tot)) * kLn2 : neg_inf();

  if (splits == 1) {
    bf16_t* dst = static_cast<bf16_t*>(a.out) + (static_cast<int64_t>(b) * a.hq + head) * C::DV +
                  C::DV_SLICE * w4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u32x2 w2;
      w2.x = pack_bf16x2(acc[0][i] * inv, acc[1][i] * inv);
      w2.y = pack_bf16x2(acc[2][i] * inv, acc[3][i] * inv);
      *reinterpret_cast<u32x2*>(dst + 4 * rho32(h, i)) = w2;
    }
    if (a.lse != nullptr && w4 == 0 && h == 0) a.lse[static_cast<int64_t>(b) * a.hq + head] = lse_val;
    return;
  }

  // ---- hand-off through the workspace ----
  // A split's partial travels in register order: for wave w, register index
  // i and lane l, the four value dims 128 w4 + 4 rho(h, i) + [0, 4) of head
  // 32 quad + col as bf16 (8 bytes), so that every store instruction writes
  // 512 contiguous bytes (device-coherent stores go through to memory as they
  // are issued) and the merging split reads them back in the same lanes, with
  // no LDS staging on either side. Partials travel as bf16 (the output
  // precision) and the merging split uses its own rounded the same way; the
  // weights, their sum and the weighted sum run in split order, so the result
  // does not depend on which split ends last.
  char* wsb = static_cast<char*>(a.workspace);
  const int64_t n_parts = static_cast<int64_t>(units) * splits;
  int* counter = reinterpret_cast<int*>(wsb);
  bf16_t* ws_o = reinterpret_cast<bf16_t*>(wsb + PKV_WORKSPACE_COUNTER_BYTES);
  float* ws_lse = reinterpret_cast<float*>(wsb + PKV_WORKSPACE_COUNTER_BYTES +
                                           n_parts * C::HB * C::DV * 2);
  const int64_t part0 = static_cast<int64_t>(unit) * splits;   // this unit's first partial
  constexpr uint32_t kPartBytes = C::HB * C::DV * 2;
  const uint32_t lane_off = static_cast<uint32_t>((wave * 16 * 64 + lane) * 8);   // + 512 i
  const int hd = 32 * quad + col;                  // head within the block
  u32x2 own[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    own[i].x = pack_bf16x2(acc[0][i] * inv, acc[1][i] * inv);
    own[i].y = pack_bf16x2(acc[2][i] * inv, acc[3][i] * inv);
  }
  {
    const auto ro = coherent_rsrc(ws_o + (part0 + ks) * C::HB * C::DV, kPartBytes);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      store_coherent(ro, lane_off + 512u * i, __builtin_bit_cast(f32x2_t, own[i]));
    if (w4 == 0 && h == 0)
      store_coherent(coherent_rsrc(ws_lse + (part0 + ks) * C::HB, C::HB * 4),
                     static_cast<uint32_t>(hd * 4), lse_val);
  }
  wait_all_vmem();
  __syncthreads();   // every wave's part has been written through
  if (threadIdx.x == 0) is_last = (counter_add(&counter[unit], 1) == splits - 1);
  __syncthreads();
  if (!is_last) return;

  // ---- last split: merge all splits of this (request, head block) ----
  // Other splits' partials are loaded two splits at a time, the first two in
  // flight together with the LSEs (gathered into LDS: [split][head]).
  constexpr int BATCH = 2;
  u32x2 part[BATCH][16];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int s2 = s0 + q;
      if (s2 < splits && s2 != ks) {
        const auto ro = coherent_rsrc(ws_o + (part0 + s2) * C::HB * C::DV, kPartBytes);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          part[q][i] = __builtin_bit_cast(u32x2, load_coherent2(ro, lane_off + 512u * i));
      }
    }
  };
  load_batch(0);
  float* st_w = reinterpret_cast<float*>(smem);   // [splits][HB] (the ring is free now)
  {
    const auto rl = coherent_rsrc(ws_lse + part0 * C::HB, static_cast<uint32_t>(splits * C::HB * 4));
    for (int i = threadIdx.x; i < splits * C::HB; i += C::THREADS)
      st_w[i] = (i / C::HB == ks) ? 0.f : load_coherent1(rl, static_cast<uint32_t>(i * 4));
  }
  __syncthreads();
  float M = neg_inf();
  for (int s2 = 0; s2 < splits; ++s2) M = fmaxf(M, s2 == ks ? lse_val : st_w[s2 * C::HB + hd]);
  float wsum = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += BATCH) {
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int s2 = s0 + q;
      if (s2 >= splits) break;
      const float ls = s2 == ks ? lse_val : st_w[s2 * C::HB + hd];
      const float wgt = (M == neg_inf()) ? 0.f : fast_exp2((ls - M) * kLog2e);
      wsum += wgt;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const u32x2 v = (s2 == ks) ? own[i] : part[q][i];
        o[i] += wgt * f32x4{bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y)};
      }
    }
  }
  const float nrm = wsum > 0.f ? 1.f / wsum : 0.f;
  bf16_t* dst = static_cast<bf16_t*>(a.out) + (static_cast<int64_t>(b) * a.hq + head) * C::DV +
                C::DV_SLICE * w4;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    u32x2 w2;
    w2.x = pack_bf16x2(o[i][0] * nrm, o[i][1] * nrm);
    w2.y = pack_bf16x2(o[i][2] * nrm, o[i][3] * nrm);
    *reinterpret_cast<u32x2*>(dst + 4 * rho32(h, i)) = w2;
  }
  if (a.lse != nullptr && w4 == 0 && h == 0)
    a.lse[static_cast<int64_t>(b) * a.hq + head] =
        (M == neg_inf()) ? neg_inf() : M + fast_log2(wsum) * kLn2;
  if (threadIdx.x == 0) counter_reset(&counter[unit]);   // ready for the next call
}

}  // namespace pkv

namespace pkv_launch {

int64_t sparse_counters(int batch, int topk, int num_q_heads) {
  if (batch <= 0 || topk <= 0 || num_q_heads <= 0) return 0;
  if (pkv::sparse_num_splits(batch, topk, num_q_heads) <= 1) return 0;
  return static_cast<int64_t>(batch) * (num_q_heads / pkv::sparse_head_block(num_q_heads));
}

size_t sparse_workspace_bytes(int batch, int topk, int num_q_heads, int head_dim_v) {
  (void)head_dim_v;
  const int splits = pkv::sparse_num_splits(batch, topk, num_q_heads);
  const int hb = pkv::sparse_head_block(num_q_heads);
  const int units = batch * (num_q_heads / hb);
  return pkv::sparse_ws_bytes(units, splits, hb);
}

template <int QUADS>
static hipError_t launch_sparse(const pkv::SparseArgs& a, hipStream_t stream) {
  using C = pkv::SparseCfg<QUADS>;
  const int splits = pkv::sparse_num_splits(a.batch, a.topk, a.hq);
  const int kps = pkv::sparse_keys_per_split(a.topk, splits);
  if (kps > C::MAX_KEYS_PER_SPLIT || splits > C::MAX_SPLITS) return hipErrorInvalidValue;
  const int hblocks = a.hq / C::HB;
  // grid: requests rounded up to a multiple of 8 (one per XCD) x head blocks x splits
  const int64_t blocks = static_cast<int64_t>((a.batch + 7) / 8) * 8 * hblocks * splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pkv::sparse_mla_kernel<QUADS>, dim3(static_cast<unsigned>(blocks)),
                     dim3(C::THREADS), C::LDS_BYTES, stream, a, splits, kps);
  return hipGetLastError();
}

hipError_t sparse_topk(const pkv::SparseArgs& a, hipStream_t stream) {
  if (pkv::sparse_quads(a.hq) == 2) return launch_sparse<2>(a, stream);
  return launch_sparse<1>(a, stream);
}

// ---- sparse_topk_decode_noalloc: the workspace in library-owned memory ----
// For callers that cannot allocate (HIP graph capture, serving loops that
// forbid it). Each GPU the library runs on holds its own copy of `scratch`
// from module load until the process ends; calls on one GPU share it, so
// calls that overlap in time on one GPU race. Its first
// PKV_WORKSPACE_COUNTER_BYTES are the split counters: zeroed by a fill kernel
// at the first call on each device, then left zero by every completed launch.
namespace {

__device__ __align__(256) unsigned char scratch[PKV_SPARSE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// The current device's address of `scratch` (the array's name in host code is
// a host-side stand-in, not a device address): looked up once per device with
// that device current, and its counter region cleared on `stream` then.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    constexpr int n = PKV_WORKSPACE_COUNTER_BYTES / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ptr), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t sparse_topk_noalloc(const pkv::SparseArgs& a_in, bool split, hipStream_t stream) {
  pkv::SparseArgs a = a_in;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (split) {
    void* ptr = nullptr;
    const hipError_t e = scratch_address(stream, &ptr);
    if (e != hipSuccess) return e;
    a.workspace = ptr;
    a.workspace_bytes = PKV_SPARSE_NOALLOC_SCRATCH_BYTES;
  }
  return sparse_topk(a, stream);
}

}  // namespace pkv_launch

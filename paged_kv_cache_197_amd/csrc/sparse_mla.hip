// sparse_topk_decode: top-k index-gathered MLA decode over one latent KV head.
// [NSA] forward_decode / transform_index_page_table_decode: top-k logical
// indices -> cache slots through the request's token table, -1 entries
// skipped; [NSA] _forward_fa3: score over the whole 576-wide row
// ([c_kv 512 | k_rope 64] against [q_nope | q_rope]), value = c_kv.
//
// Work decomposition: one workgroup (4 waves) per (32-head block, request,
// key split). The workgroup first translates its whole slice of the top-k
// list into cache slots (kept in LDS), then walks it in 32-key tiles: each
// tile's 32 rows (1152 B each) are gathered into double-buffered LDS and
// shared by the four waves. Per tile:
//   * QK: wave w computes a partial S^T [32 keys x 32 heads] over score dims
//     [144w, 144w + 144) (nine 32x32x16 MFMAs) and publishes it in LDS.
//   * softmax: wave w sums the four partials for heads [8w, 8w + 8) only, runs
//     the online softmax for them and publishes P^T (bf16) and each head's
//     rescale factor, so the softmax work is not repeated across waves.
//   * PV: wave w accumulates O^T for value dims [128w, 128w + 128) (four
//     32x32x16 blocks x two 16-key k-steps); the value rows are the first 512
//     dims of the same LDS tile.
// MFMA C-layout used throughout: lane (col = lane % 32, h = lane / 32) holds
// column col (a head) and rows rho(h, r) = 8*(r/4) + 4h + r%4, r < 16 (keys
// of S^T, dims of O^T).
// Key splits (needed to fill the chip when batch x head blocks is small) are
// merged inside the kernel: every split writes its normalised partial and LSE
// to the workspace, and the last split to finish (device-scope counter) merges
// them and writes the output; the counter is reset for the next call.
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

struct SparseCfg {
  static constexpr int DQK = 576;
  static constexpr int DV = 512;
  static constexpr int HB = 32;                 // heads per workgroup
  static constexpr int KT = 32;                 // keys per tile
  static constexpr int ROW_BYTES = DQK * 2;     // 1152
  static constexpr int LDS_STRIDE = ROW_BYTES + 16;
  static constexpr int TILE_BYTES = KT * LDS_STRIDE;
  static constexpr int PIECES = KT * ROW_BYTES / 16;      // 2304 16-byte pieces
  static constexpr int PPT = PIECES / 256;                // 9 per thread
  static constexpr int QK_SLICE = DQK / 4;      // 144 score dims per wave
  static constexpr int QK_STEPS = QK_SLICE / 16;  // 9
  static constexpr int DV_SLICE = DV / 4;       // 128 value dims per wave
  static constexpr int NBLK = DV_SLICE / 32;    // 4
  static constexpr int MAX_KEYS_PER_SPLIT = 2048;   // slot list capacity in LDS
  static constexpr int SP_BYTES = 4 * 4 * 64 * 16;  // partial S^T: [wave][quad][lane] float4
  static constexpr int PB_BYTES = 4 * 64 * 8;       // P^T bf16: [quad][lane] 4 x bf16
  static constexpr int AUX_BYTES = 32 * 4 * 3;      // per head: rescale factor, final m, l
  static constexpr int LDS_BYTES =
      2 * TILE_BYTES + SP_BYTES + PB_BYTES + AUX_BYTES + MAX_KEYS_PER_SPLIT * 4;
};

// splits per (request, head block) so the grid has about 256 workgroups, each
// split keeping at least 128 keys; the last split may be shorter
__host__ __device__ inline int sparse_num_splits(int batch, int topk, int hq) {
  const int units = batch * (hq / SparseCfg::HB);
  if (units <= 0 || topk <= 0) return 1;
  int s = (256 + units - 1) / units;
  const int by_keys = (topk + 127) / 128;
  s = s < by_keys ? s : by_keys;
  const int min_for_lds = (topk + SparseCfg::MAX_KEYS_PER_SPLIT - 1) / SparseCfg::MAX_KEYS_PER_SPLIT;
  if (s < min_for_lds) s = min_for_lds;
  return s < 1 ? 1 : s;
}

__host__ __device__ inline int sparse_keys_per_split(int topk, int splits) {
  const int k = (topk + splits - 1) / splits;
  return (k + SparseCfg::KT - 1) / SparseCfg::KT * SparseCfg::KT;
}

struct SparseWorkspace {
  float* o;        // [units][S][HB][DV]
  float* lse;      // [units][S][HB]
  int* counter;    // [units]
};

__host__ __device__ inline size_t sparse_ws_bytes(int units, int splits) {
  if (splits <= 1) return 0;
  size_t o = static_cast<size_t>(units) * splits * SparseCfg::HB * SparseCfg::DV * 4;
  size_t l = static_cast<size_t>(units) * splits * SparseCfg::HB * 4;
  size_t c = static_cast<size_t>(units) * 4;
  return o + l + c;
}

__device__ __forceinline__ int rho32(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(SparseArgs a, int splits, int kps) {
  using C = SparseCfg;
  extern __shared__ __align__(16) char smem[];
  auto lds_tile = [&](int i) { return smem + i * C::TILE_BYTES; };
  float* sp = reinterpret_cast<float*>(smem + 2 * C::TILE_BYTES);
  int32_t* slots = reinterpret_cast<int32_t*>(smem + 2 * C::TILE_BYTES + C::SP_BYTES +
                                              C::PB_BYTES + C::AUX_BYTES);

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
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;     // head within the block (B / C column)
  const int h = lane >> 5;

  const int k_begin = ks * kps;
  const int k_end = min(a.topk, k_begin + kps);
  const int nkeys = max(k_end - k_begin, 0);
  const int n_tiles = (nkeys + C::KT - 1) / C::KT;

  // ---- translate this split's top-k entries to cache slots (-1: skip) ----
  const int64_t r = a.rpi[b];
  const bool row_ok = r >= 0 && r < a.r2t_rows;
  for (int i = threadIdx.x; i < n_tiles * C::KT; i += 256) {
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
  __syncthreads();

  const char* kvb = static_cast<const char*>(a.kv);
  u32x4 stage[C::PPT];
  // unconditional loads (skipped keys read row 0; their LDS rows are zeroed)
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int key = piece / (C::ROW_BYTES / 16);
      const int chunk = piece % (C::ROW_BYTES / 16);
      const int32_t sl = max(slots[tile * C::KT + key], 0);
      stage[i] = *reinterpret_cast<const u32x4*>(kvb + static_cast<int64_t>(sl) * C::ROW_BYTES +
                                                 chunk * 16);
    }
  };
  auto store_tile = [&](char* dst, uint32_t valid) {
    const bool all_valid = (valid == 0xffffffffu);
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int key = piece / (C::ROW_BYTES / 16);
      const int chunk = piece % (C::ROW_BYTES / 16);
      u32x4 v = stage[i];
      if (!all_valid && !((valid >> key) & 1u)) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dst + key * C::LDS_STRIDE + chunk * 16) = v;
    }
  };
  // bit k set: key k of the tile has a slot (the same mask in every wave)
  auto tile_valid = [&](int tile) -> uint32_t {
    const bool ok = slots[tile * C::KT + (lane & 31)] >= 0;
    return static_cast<uint32_t>(__ballot(ok) & 0xffffffffull);
  };

  float* aux = reinterpret_cast<float*>(smem + 2 * C::TILE_BYTES + C::SP_BYTES + C::PB_BYTES);
  float* alpha_buf = aux;            // [32] per-head rescale of the current tile
  float* m_buf = aux + 32;           // [32] final running max per head (raw units)
  float* l_buf = aux + 64;           // [32] final denominator per head
  char* pb = smem + 2 * C::TILE_BYTES + C::SP_BYTES;

  // Q^T operand for this wave's score slice: head col, dims 144w + 16j + 8h + [0, 8)
  const int head = hb * C::HB + col;
  u32x4 qop[C::QK_STEPS];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       (static_cast<int64_t>(b) * a.hq + head) * C::DQK * 2;
#pragma unroll
    for (int j = 0; j < C::QK_STEPS; ++j)
      qop[j] = *reinterpret_cast<const u32x4*>(qrow + (C::QK_SLICE * wave + 16 * j + 8 * h) * 2);
#pragma unroll
    for (int j = 0; j < C::QK_STEPS; ++j) {
      retire(qop[j].x);
      retire(qop[j].y);
      retire(qop[j].z);
      retire(qop[j].w);
    }
  }

  f32x16 acc[C::NBLK];
#pragma unroll
  for (int n = 0; n < C::NBLK; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;

  // softmax ownership: lane L of wave w handles head sc = 8w + (L & 7), the
  // four S^T values of lane sl = sc + 32 * sh, register quad sq
  const int sc = 8 * wave + (lane & 7);
  const int sh = (lane >> 3) & 1;
  const int sq = lane >> 4;
  const int src_lane = sc + 32 * sh;
  float m_run = neg_inf();   // raw score units, for head sc
  float l_run = 0.f;         // partial denominator over this lane's keys

  uint32_t valid_cur = 0xffffffffu;
  if (n_tiles > 0) {
    valid_cur = tile_valid(0);
    load_tile(0);
    store_tile(lds_tile(0), valid_cur);
  }
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < n_tiles;
    if (more) load_tile(kt + 1);
    __builtin_amdgcn_sched_barrier(0);   // the next tile's loads go out before the MFMAs
    const char* tile = lds_tile(buf);

    // ---- partial S^T over this wave's 144 score dims -> LDS ----
    {
      f32x16 s;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.f;
      const char* krow = tile + col * C::LDS_STRIDE;     // A row: key col of the tile
#pragma unroll
      for (int j = 0; j < C::QK_STEPS; ++j) {
        const u32x4 kw =
            *reinterpret_cast<const u32x4*>(krow + (C::QK_SLICE * wave + 16 * j + 8 * h) * 2);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), as_bf16x8(qop[j]), s, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        reinterpret_cast<float4*>(sp)[(wave * 4 + i) * 64 + lane] =
            make_float4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
    }
    const uint32_t valid_next = more ? tile_valid(kt + 1) : 0xffffffffu;
    __syncthreads();   // A: partial scores visible; every wave is done with tile buf ^ 1
    if (more) store_tile(lds_tile(buf ^ 1), valid_next);

    // ---- softmax for heads [8w, 8w + 8): 4 keys per lane ----
    {
      float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4 v = reinterpret_cast<const float4*>(sp)[(w * 4 + sq) * 64 + src_lane];
        x[0] += v.x;
        x[1] += v.y;
        x[2] += v.z;
        x[3] += v.w;
      }
      if (valid_cur != 0xffffffffu) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // key of register 4*sq + j of lane half sh
          const int key = 8 * sq + 4 * sh + j;
          if (!((valid_cur >> key) & 1u)) x[j] = neg_inf();
        }
      }
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 8));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * a.scale_log2);
      const float neg_mc = -m_use * a.scale_log2;
      m_run = m_new;
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = fast_exp2(__builtin_fmaf(x[j], a.scale_log2, neg_mc));
      l_run = l_run * alpha + (p[0] + p[1]) + (p[2] + p[3]);
      u32x2 pw;
      pw.x = pack_bf16x2(p[0], p[1]);
      pw.y = pack_bf16x2(p[2], p[3]);
      reinterpret_cast<u32x2*>(pb)[sq * 64 + src_lane] = pw;
      if (lane < 8) alpha_buf[sc] = alpha;
    }
    __syncthreads();   // B: P^T and rescale factors visible

    // ---- O^T (this wave's 128 value dims) += V^T . P^T ----
    {
      const float alpha_c = alpha_buf[col];
      if (__any(alpha_c != 1.f)) {   // rescale only when some head's running max moved
#pragma unroll
        for (int n = 0; n < C::NBLK; ++n) acc[n] *= alpha_c;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x2 p0 = reinterpret_cast<const u32x2*>(pb)[(2 * t) * 64 + lane];
        const u32x2 p1 = reinterpret_cast<const u32x2*>(pb)[(2 * t + 1) * 64 + lane];
        const u32x4 pw = {p0.x, p0.y, p1.x, p1.y};
        uint32_t vr[8][2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * t + 8 * (e >> 2) + 4 * h + (e & 3);
          const u32x2 w2 = *reinterpret_cast<const u32x2*>(tile + key * C::LDS_STRIDE +
                                                            (C::DV_SLICE * wave + 4 * col) * 2);
          vr[e][0] = w2.x;
          vr[e][1] = w2.y;
        }
#pragma unroll
        for (int n = 0; n < C::NBLK; ++n) {
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
    valid_cur = valid_next;
    // the next iteration's barrier A orders these reads before buf / pb / sp are rewritten
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

  // ---- this split's result for head col, value dims 128w + 4*rho(h, i) + n ----
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_val =
      l_tot > 0.f ? (m_head * a.scale_log2 + fast_log2(l_tot)) * kLn2 : neg_inf();

  if (splits == 1) {
    bf16_t* dst = static_cast<bf16_t*>(a.out) + (static_cast<int64_t>(b) * a.hq + head) * C::DV +
                  C::DV_SLICE * wave;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u32x2 w2;
      w2.x = pack_bf16x2(acc[0][i] * inv, acc[1][i] * inv);
      w2.y = pack_bf16x2(acc[2][i] * inv, acc[3][i] * inv);
      *reinterpret_cast<u32x2*>(dst + 4 * rho32(h, i)) = w2;
    }
    if (a.lse != nullptr && wave == 0 && h == 0) a.lse[static_cast<int64_t>(b) * a.hq + head] = lse_val;
    return;
  }

  SparseWorkspace ws;
  char* wsb = static_cast<char*>(a.workspace);
  ws.o = reinterpret_cast<float*>(wsb);
  ws.lse = reinterpret_cast<float*>(wsb + static_cast<size_t>(units) * splits * C::HB * C::DV * 4);
  ws.counter = reinterpret_cast<int*>(wsb + static_cast<size_t>(units) * splits * C::HB * C::DV * 4 +
                                      static_cast<size_t>(units) * splits * C::HB * 4);
  {
    float* dst = ws.o + ((static_cast<int64_t>(unit) * splits + ks) * C::HB + col) * C::DV +
                 C::DV_SLICE * wave;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<float4*>(dst + 4 * rho32(h, i)) =
          make_float4(acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv, acc[3][i] * inv);
    if (wave == 0 && h == 0) ws.lse[(static_cast<int64_t>(unit) * splits + ks) * C::HB + col] = lse_val;
  }
  __threadfence();
  __syncthreads();
  __shared__ int is_last;
  if (threadIdx.x == 0) is_last = (atomicAdd(&ws.counter[unit], 1) == splits - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- last split: merge all splits of this (request, head block) ----
  // thread -> (head, 64-dim segment): 32 heads x 8 segments = 256 threads
  const int mh = threadIdx.x >> 3;
  const int seg = (threadIdx.x & 7) * 64;
  const float* lse_src = ws.lse + static_cast<int64_t>(unit) * splits * C::HB;
  float m = neg_inf();
  for (int s2 = 0; s2 < splits; ++s2) m = fmaxf(m, __builtin_nontemporal_load(lse_src + s2 * C::HB + mh));
  float wsum = 0.f;
  float o[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) o[i] = 0.f;
  if (m != neg_inf()) {
    for (int s2 = 0; s2 < splits; ++s2) {
      const float w = fast_exp2((__builtin_nontemporal_load(lse_src + s2 * C::HB + mh) - m) * kLog2e);
      if (w == 0.f) continue;
      wsum += w;
      const float* src = ws.o + ((static_cast<int64_t>(unit) * splits + s2) * C::HB + mh) * C::DV + seg;
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + i);
        o[i] += w * v.x;
        o[i + 1] += w * v.y;
        o[i + 2] += w * v.z;
        o[i + 3] += w * v.w;
      }
    }
  }
  const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int ohead = hb * C::HB + mh;
  bf16_t* dst = static_cast<bf16_t*>(a.out) + (static_cast<int64_t>(b) * a.hq + ohead) * C::DV + seg;
#pragma unroll
  for (int i = 0; i < 64; i += 4) {
    u32x2 w2;
    w2.x = pack_bf16x2(o[i] * winv, o[i + 1] * winv);
    w2.y = pack_bf16x2(o[i + 2] * winv, o[i + 3] * winv);
    *reinterpret_cast<u32x2*>(dst + i) = w2;
  }
  if (a.lse != nullptr && seg == 0)
    a.lse[static_cast<int64_t>(b) * a.hq + ohead] = (m == neg_inf()) ? neg_inf() : m + fast_log2(wsum) * kLn2;
  if (threadIdx.x == 0) atomicExch(&ws.counter[unit], 0);   // ready for the next call
}

}  // namespace pkv

namespace pkv_launch {

size_t sparse_workspace_bytes(int batch, int topk, int num_q_heads, int head_dim_v) {
  (void)head_dim_v;
  const int splits = pkv::sparse_num_splits(batch, topk, num_q_heads);
  const int units = batch * (num_q_heads / pkv::SparseCfg::HB);
  return pkv::sparse_ws_bytes(units, splits);
}

hipError_t sparse_topk(const pkv::SparseArgs& a, hipStream_t stream) {
  using C = pkv::SparseCfg;
  const int splits = pkv::sparse_num_splits(a.batch, a.topk, a.hq);
  const int kps = pkv::sparse_keys_per_split(a.topk, splits);
  if (kps > C::MAX_KEYS_PER_SPLIT) return hipErrorInvalidValue;
  const int hblocks = a.hq / C::HB;
  // grid: requests rounded up to a multiple of 8 (one per XCD) x head blocks x splits
  const int64_t blocks = static_cast<int64_t>((a.batch + 7) / 8) * 8 * hblocks * splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pkv::sparse_mla_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                     C::LDS_BYTES, stream, a, splits, kps);
  return hipGetLastError();
}

}  // namespace pkv_launch

// paged_attn_varlen_prefill: causal extend over a paged KV cache
// ([FA] forward_extend: flash_attn_with_kvcache with cache_seqlens = prefix +
// new, cu_seqlens_q over the new tokens, causal=True). New row j of request b
// sits at position L_b - M_b + j and sees keys [0, L_b - M_b + j].
//
// Work decomposition. One workgroup per (32-row q tile, kv head, request, key
// split), of GROUPS groups of four waves: two groups (one workgroup per CU)
// for launches with few q tiles, one group (two workgroups per CU) for large
// ones. A q tile's visible 32-key tiles are cut into splits of
// `split_tiles` tiles when the tiles are long enough to leave CUs idle
// otherwise; each split writes its normalised partial output and LSE to the
// workspace at device scope, and the last split of the tile to finish (device-
// scope counter) merges them. A q tile with one split writes the output
// directly. With two groups the split's key tiles are halved between them and
// their softmax states are merged through LDS at the end; the two waves
// sharing a SIMD (one per group) hide each other's latencies, but the per-tile
// workgroup barrier keeps them in step. With one group per workgroup, the two
// waves sharing a SIMD belong to different workgroups and drift apart, so one
// issues MFMAs while the other runs its softmax (11% faster in steady state);
// short launches keep two groups, whose halved key range is the shorter chain.
// Within a group wave w owns q heads w, w+4, ... of the GQA group and all four
// share 32-key K/V tiles, copied into the group's four-stage LDS ring by
// direct global-to-LDS loads three tiles ahead of their use. The page-table
// entries of the 8 keys a wave copies per tile are themselves fetched into LDS
// by direct loads, eight tiles at a time, well before the copies need them.
//
// Per wave and key tile (32x32x16 bf16 MFMA):
//   S^T [32 keys x 32 rows] = K [32 x D] . Q^T [D x 32]        (D/16 MFMAs)
//   O^T [D x 32 rows]      += V^T [D x 32 keys] . P^T [32 x 32] (D/16 MFMAs)
// Lane (q = lane % 32, h = lane / 32) owns row q: its S^T accumulator holds
// keys rho(h, r) = 8*(r/4) + 4h + r%4, which is exactly the k-set its P^T
// operand needs for the two 16-key k-steps, and its O^T accumulator rows are
// dims of row q. Row max / sum / rescale stay in the lane (the max is reduced
// with the other lane half by one xor-shuffle).
// V^T operand: block n, row m is dim 32n + m, read from the row-major LDS tile
// with gfx950's transposing LDS read (ds_read_b64_tr_b16), so no register
// shuffles are needed.
// LDS rows are D*2 bytes with their 16-byte chunks XOR-swizzled by the row
// index, so that the K operand reads (16 rows, one chunk) hit distinct banks.
#include <climits>

#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace pkv {

// page-table arithmetic
enum PageMode : int {
  kPageToken = 0,   // page_size 1: one entry per key
  kPagePow2 = 1,    // page_size a power of two: shifts
  kPageAny = 2,     // anything else: division
};

template <int D, int PM, int GROUPS>
struct PrefillKernel {
  static_assert(GROUPS == 1 || GROUPS == 2, "one or two groups of four waves");
  static constexpr int WAVES = 4 * GROUPS;
  static constexpr int KT = 32;               // keys per tile
  static constexpr int QT = 32;               // q rows per tile
  static constexpr int NKS = D / 16;          // 16-wide k-steps of S^T
  static constexpr int NB = D / 32;           // 32-dim blocks of O^T
  static constexpr int ROW = D * 2;           // bytes per key row (one kv head)
  static constexpr int CH = ROW / 16;         // 16-byte chunks per row
  static constexpr int TILE = KT * ROW;       // one tensor's tile
  static constexpr int STAGE = 2 * TILE;      // K and V
  static constexpr int NSTAGE = 4;
  static constexpr int GROUP_LDS = NSTAGE * STAGE;
  static constexpr int ENTRY_BYTES = WAVES * 2 * 256; // waves x 2 segments x 64 words
  // the split hand-off's flag sits after the entry slots, inside the dynamic
  // LDS: with no static LDS the dynamic region starts at address 0, so every
  // constant LDS offset folds into the instructions' offset fields
  static constexpr int FLAG_OFF = GROUPS * GROUP_LDS + ENTRY_BYTES;
  static constexpr int LDS_BYTES = FLAG_OFF + 16;
  static constexpr int RPB = 1024 / ROW;      // key rows per 1 KB copy block
  static constexpr int IPW = TILE / 1024 / 4; // copy blocks per wave and tensor
  static constexpr int KPW = IPW * RPB;       // keys per wave per tile
  static constexpr int SWZ = 256 / ROW;       // rows sharing one 64-bank span
  static constexpr int MERGE_F4 = 4 * NB + 1;        // float4s of a lane in the merge: acc, (m, l)
  static constexpr int QPW = TILE / 2048;             // Q copies per wave (4 heads / 8 waves)
  static constexpr float kRescaleLog2 = 8.f;          // see softmax_pv
  static constexpr int kMaxSplits = 16;               // key splits per q tile (planned by the host)
  static constexpr int kMergeBatch = 2;               // splits whose partials a merge loads at once
  static_assert(KPW == 8, "a wave copies 8 keys of each tile");
  static_assert(GROUPS == 1 || 4 * MERGE_F4 * 64 * 16 <= 2 * GROUP_LDS, "merge buffer fits the rings");
  static_assert(4 * TILE / 1024 == 8 * QPW, "Q copies split evenly over the waves");

  // key of S^T accumulator register r for lane half h
  static __device__ __forceinline__ int rho(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }
  // LDS chunk position of global chunk c of key row k (an involution in c).
  // The LDS serves 256 bytes (64 banks) per cycle: 16 lanes of a 16-byte read
  // or 32 lanes of an 8-byte one. u = the row's index among the CH rows whose
  // chunks a position cycle covers (SWZ rows share one 256-byte bank span);
  // the chunk is XORed with u transposed on a (CH/4) x 4 grid, so that the
  // 16 rows of one K operand read pass (one chunk each) land on 16 distinct
  // positions, and so do the 4 rows x 4 chunks of one 32-lane pass of a
  // transposed V read (whose rows form an aligned group of four).
  static __device__ __forceinline__ int swz(int k, int c) {
    constexpr int A = CH / 4;
    const int u = (k / SWZ) % CH;
    return c ^ (4 * (u % A) + u / A);
  }

  static __device__ __forceinline__ int page_col(const PrefillArgs& a, int t) {
    if constexpr (PM == kPageToken) return t;
    else if constexpr (PM == kPagePow2) return t >> a.page_shift;
    else return t / a.page_size;
  }
  static __device__ __forceinline__ int page_off(const PrefillArgs& a, int t) {
    if constexpr (PM == kPageToken) return 0;
    else if constexpr (PM == kPagePow2) return t & (a.page_size - 1);
    else return t % a.page_size;
  }

  // Page-table entries. Each wave copies 8 keys [kt*32 + 8w, +8) of every
  // tile; the entries of those keys for a segment of SEG consecutive tiles are
  // fetched by one direct-to-LDS load (lane l: tile l/8, key l%8, clamped to
  // the last key) into the wave's double-buffered entry slots, a segment ahead.
  static constexpr int SEG = 8;
  static __device__ __forceinline__ void fetch_entries(const PrefillArgs& a, const int32_t* pt_row,
                                                       int L, int seg_tile, int w, int lane,
                                                       uint32_t slot_base) {
    const int t = min((seg_tile + lane / 8) * KT + KPW * w + lane % 8, L - 1);
    lds_dma4(pt_row + page_col(a, t), slot_base);
  }

  // Q^T operands of the workgroup's four heads, copied once into the free
  // fourth ring stage of the two groups (head qh: group qh / 2, K or V half
  // qh % 2), laid out and swizzled like a K tile so that the operand read is
  // the K operand read. Copy i (1 KB) of the 4 * TILE / 1024 belongs to wave
  // i / QPW; its lane l fills row (i % (TILE/1024)) * RPB + l / CH at LDS chunk
  // l % CH from chunk swz(row, l % CH) of that row's q vector. Rows past the
  // tile's last row and heads past the group repeat the last ones.
  static __device__ __forceinline__ void copy_q(const PrefillArgs& a, int wave, int lane, int hb,
                                                int kvh, int G, int tok0, int rows,
                                                uint32_t lds0) {
    // opaque lane index: keeps these once-per-head-block addresses from being
    // hoisted out of the head-block loop into registers held across the tiles
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < QPW; ++k) {
      const int i = wave * QPW + k;
      const int qh = i / (TILE / 1024);
      const int blk = i % (TILE / 1024);
      const int row = blk * RPB + ln / CH;
      const int tok = min(tok0 + min(row, rows - 1), a.total_q - 1);
      const int head = kvh * G + min(4 * hb + qh, G - 1);
      const char* src = static_cast<const char*>(a.q) +
                        (static_cast<int64_t>(tok) * a.hq + head) * ROW + swz(row, ln % CH) * 16;
      lds_dma16(src, lds0 + q_lds(qh) + blk * 1024);
    }
  }
  static __device__ __forceinline__ uint32_t q_lds(int qh) {
    return static_cast<uint32_t>((qh >> 1) * GROUP_LDS + (NSTAGE - 1) * STAGE + (qh & 1) * TILE);
  }

  // Issue the direct-to-LDS copies of key tile kt into the LDS stage at
  // stage_base. Copy block blk (1 KB of a tensor tile) holds key rows
  // [blk*RPB, +RPB); lane l fills row blk*RPB + l/CH at LDS chunk l%CH, i.e.
  // it reads global chunk swz(row, l%CH), at byte chunk_off[i] of the row.
  // entries: this wave's entry slots of the segment holding kt (tile tt in it).
  static __device__ __forceinline__ void copy_tile(const PrefillArgs& a, int L, int kt, int tt,
                                                   int w, int lane, const int32_t* entries,
                                                   int64_t row_bytes, const char* kb,
                                                   const char* vb, const int (&chunk_off)[IPW],
                                                   uint32_t stage_base) {
    int32_t raws[IPW];   // both entry reads in flight together
#pragma unroll
    for (int i = 0; i < IPW; ++i) raws[i] = entries[tt * 8 + i * RPB + lane / CH];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int j = i * RPB + lane / CH;   // key 8w + j of the tile
      const int t = min(kt * KT + KPW * w + j, L - 1);
      const int32_t raw = raws[i];
      // page clamped into [0, num_pages) (num_pages * page_size < 2^31: slots
      // fit 32 bits; a negative entry reads as a large unsigned one)
      const uint32_t page = min(static_cast<uint32_t>(raw),
                                static_cast<uint32_t>(a.num_pages - 1));
      uint32_t slot;
      if constexpr (PM == kPageToken) slot = page;
      else if constexpr (PM == kPagePow2) slot = (page << a.page_shift) | page_off(a, t);
      else slot = page * a.page_size + page_off(a, t);
      const uint64_t off = static_cast<uint64_t>(slot) * static_cast<uint32_t>(row_bytes) +
                           static_cast<uint32_t>(chunk_off[i]);
      const int blk = w * IPW + i;
      lds_dma16(kb + off, stage_base + blk * 1024);
      lds_dma16(vb + off, stage_base + TILE + blk * 1024);
    }
  }

  // K operand reads of one key tile (row q, chunk swz(q, 2j + h) for k-step j)
  static __device__ __forceinline__ void read_k(const char* stage, int kbase, int q, int h,
                                                u32x4 (&kw)[NKS]) {
#pragma unroll
    for (int j = 0; j < NKS; ++j)
      kw[j] = *reinterpret_cast<const u32x4*>(stage + kbase + swz(q, 2 * j + h) * 16);
  }

  // Online-softmax state of the lane's row (equal in lanes q and q + 32).
  // m is a reference max in raw score units (-inf before the row has seen a
  // key); the scale c = scale_log2 > 0 is applied inside the exponent,
  // p = exp2(s c - m c). m moves only when a score exceeds thr = m +
  // kRescaleLog2 / c, so the exponentials stay below 2^kRescaleLog2 while the
  // accumulators are rescaled on few tiles; the sum and the output share the
  // reference, so the result is the same for any such m. l is this lane's
  // half-row sum of the exponentials (fp32).
  struct RowState {
    float m, thr, neg_mc, l;
  };
  static __device__ __forceinline__ RowState row_state_init() {
    return RowState{neg_inf(), neg_inf(), 0.f, 0.f};
  }

  // Softmax of S^T for this wave's row block and the O^T update with the
  // tile's V, software-pipelined with S^T of the next tile: its K operands
  // (kw, already read) go through the MFMAs while the exponentials of this
  // tile run on the VALU. Returns the next tile's S^T. Masked tiles apply the
  // per-row key window (key kt*32 + rho(h, r) is visible iff
  // rel_lo <= rho(h, r) - 4h < rel).
  static __device__ __forceinline__ f32x16 softmax_pv(f32x16 s, const char* stage_v,
                                                      const int (&vofs)[2][NB], bool masked,
                                                      int rel, int rel_lo, float scale_log2,
                                                      float rescale_step,
                                                      const u32x4 (&kw)[NKS],
                                                      const u32x4 (&qop)[NKS], f32x16 (&acc)[NB],
                                                      RowState& st) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = s[r];
    if (masked) {   // wave-uniform: only tiles that reach past some row's window
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= rel || 8 * (r >> 2) + (r & 3) < rel_lo) x[r] = neg_inf();
    }
    // this lane's half of the row: does any score pass the threshold?
    // (med3(a, b, +inf) = max(a, b) without quieting the MFMA results first)
    float mt = __builtin_amdgcn_fmed3f(x[0], x[1], __builtin_inff());
#pragma unroll
    for (int r = 2; r < 16; ++r) mt = fmaxf(mt, x[r]);
    if (__any(mt > st.thr)) {
      // rare after a row's first tiles: move the reference of every row whose
      // maximum (both halves) passed it, and rescale what was accumulated
      mt = max_xor32(mt);
      const bool grow = mt > st.thr;
      const float m_ref = grow ? mt : st.m;
      const float m_use = (m_ref == neg_inf()) ? 0.f : m_ref;
      const float alpha = grow ? fast_exp2((st.m - m_use) * scale_log2) : 1.f;
      st.m = m_ref;
      st.neg_mc = -m_use * scale_log2;
      st.thr = (m_ref == neg_inf()) ? neg_inf() : m_ref + rescale_step;
      st.l *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    }
    const float neg_mc = st.neg_mc;

    // V^T operands (see below) of the first 16-key step, early
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) char lds_char;
    s16x4 vt[2][NB][2];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        vt[0][n][s2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_s16x4*>((lds_char*)stage_v + vofs[s2][n]));

    // next tile's S^T on the MFMA pipe, this tile's exponentials on the VALU:
    // a few exponentials between consecutive (dependent) MFMAs, order pinned.
    // (after the last tile the K operands are stale LDS; the result is unused)
    f32x16 sn;
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[r] = 0.f;
    float p[16];
    constexpr int PER = 16 / NKS;
#pragma unroll
    for (int j = 0; j < NKS; ++j) {
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw[j]), as_bf16x8(qop[j]), sn, 0, 0,
                                                    0);
#pragma unroll
      for (int e = 0; e < PER; ++e)
        p[PER * j + e] = fast_exp2(__builtin_fmaf(x[PER * j + e], scale_log2, neg_mc));
      __builtin_amdgcn_sched_barrier(0);
    }
    // second step's V^T operands
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        vt[1][n][s2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_s16x4*>((lds_char*)stage_v + vofs[s2][n] + 16 * ROW));

    // O^T block n row m = dim 32n + m. Its A operand for the 16-key step t is
    // V^T[32n + m][keys 16t + 8(e/4) + 4h + e%4], e = 0..7: two transposed
    // 8-byte LDS reads (ds_read_b64_tr_b16), each turning 16 lanes' row-major
    // 4-dim pieces of 4 keys into one dim's 4 keys per lane (vofs).
    // The row sum is taken over the fp32 exponentials: bf16-rounded ones
    // would move the LSE by up to 2^-9 on rows that one key dominates.
    float ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ps[i] = (p[4 * i] + p[4 * i + 1]) + (p[4 * i + 2] + p[4 * i + 3]);
    st.l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pw = {pack_bf16x2(p[8 * t + 0], p[8 * t + 1]),
                        pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                        pack_bf16x2(p[8 * t + 4], p[8 * t + 5]),
                        pack_bf16x2(p[8 * t + 6], p[8 * t + 7])};
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const u32x2 lo = __builtin_bit_cast(u32x2, vt[t][n][0]);
        const u32x2 hi = __builtin_bit_cast(u32x2, vt[t][n][1]);
        const u32x4 vw = {lo.x, lo.y, hi.x, hi.y};
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), as_bf16x8(pw), acc[n], 0,
                                                         0, 0);
      }
    }
    return sn;
  }

  // bf16 output of lane row q: acc block n, register r is dim 32n + rho(h, r);
  // registers 4a..4a+3 are the 4 consecutive dims 32n + 8a + 4h + [0, 4)
  static __device__ __forceinline__ int out_dim(int h, int n, int a) { return 32 * n + 8 * a + 4 * h; }
  static __device__ __forceinline__ void store_out_row(bf16_t* dst, int h, const float (&o)[16][NB],
                                                       float scale) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 w;
        w.x = pack_bf16x2(o[4 * a4][n] * scale, o[4 * a4 + 1][n] * scale);
        w.y = pack_bf16x2(o[4 * a4 + 2][n] * scale, o[4 * a4 + 3][n] * scale);
        *reinterpret_cast<u32x2*>(dst + out_dim(h, n, a4)) = w;
      }
  }

  static __device__ void run(const PrefillArgs& a) {
    extern __shared__ __align__(16) char smem[];
    int& sh_last = *reinterpret_cast<int*>(smem + FLAG_OFF);

    const int G = a.hq / a.hkv;
    const int n_hb = (G + 3) / 4;
    const int lane = threadIdx.x & 63;
    // flat grid: kv head fastest, then split, then q-tile slot. Slots number
    // the q tiles request by request (each request's from its last, longest
    // one); a request with M rows has ceil(M / 32) of them, so
    // ceil(total_q / 32) + batch slots cover all and few stay empty. Within
    // each chunk of 64 requests the longer ones (more keys) take the lower
    // slots: workgroups start in slot order, so the longest chains start
    // first and the short ones fill in behind them.
    const int kvh = blockIdx.x % a.hkv;
    const int rest = blockIdx.x / a.hkv;
    const int split = rest % a.max_splits;
    const int slot = rest / a.max_splits;
    int b = -1, qrev = 0, q0 = 0, M = 0, Lraw = 0;
    {
      int base = 0;   // q tiles of the requests before this chunk of 64
      for (int c0 = 0; c0 < a.batch; c0 += 64) {
        const int bi = c0 + lane;
        const bool in = bi < a.batch;
        const int qs = in ? a.cu_q[bi] : 0;       // one round trip for all three
        const int qe = in ? a.cu_q[bi + 1] : 0;
        const int kl = in ? a.kv_lens[bi] : 0;
        const int nt = in ? max(qe - qs + QT - 1, 0) / QT : 0;
        // place of this request in the chunk: more keys first, ties by index
        const int nb = min(64, a.batch - c0);   // requests in this chunk (uniform)
        const int key = in ? kl : INT_MIN;
        int rank = 0;
#pragma unroll 4
        for (int j = 0; j < nb; ++j) {
          const int kj = __builtin_amdgcn_readlane(key, j);
          rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
        }
        int first = base;   // slot of request bi's last q tile
#pragma unroll 4
        for (int j = 0; j < nb; ++j) {
          const int rj = __builtin_amdgcn_readlane(rank, j);
          first += rj < rank ? __builtin_amdgcn_readlane(nt, j) : 0;
        }
        const unsigned long long hit = __ballot(nt > 0 && slot >= first && slot < first + nt);
        if (hit) {
          const int l = __builtin_ctzll(hit);
          b = c0 + l;
          qrev = slot - __shfl(first, l);
          q0 = __shfl(qs, l);
          M = __shfl(qe, l) - q0;
          Lraw = __shfl(kl, l);
          break;
        }
        int chunk_tiles = nt;   // q tiles of the whole chunk
#pragma unroll
        for (int d = 1; d < 64; d *= 2) chunk_tiles += __shfl_xor(chunk_tiles, d);
        base += chunk_tiles;
      }
    }
    // (wave-uniform; made explicit so that everything derived stays scalar)
    b = __builtin_amdgcn_readfirstlane(b);
    qrev = __builtin_amdgcn_readfirstlane(qrev);
    q0 = __builtin_amdgcn_readfirstlane(q0);
    M = __builtin_amdgcn_readfirstlane(M);
    Lraw = __builtin_amdgcn_readfirstlane(Lraw);
    if (b < 0) return;   // an empty slot
    const int n_qtiles = (M + QT - 1) / QT;
    const int qtile = n_qtiles - 1 - qrev;
    if (qtile < 0) return;
    const int64_t cap = static_cast<int64_t>(a.pt_stride) * a.page_size;
    const int L = static_cast<int>(min<int64_t>(max(Lraw, 0), cap));
    const int j0 = qtile * QT;
    const int rows = min(QT, M - j0);

    // keys this q tile can see: up to position L - M + j0 + rows - 1
    const int key_end = a.causal ? min(L, L - M + j0 + rows) : L;
    const int n_ktiles = key_end > 0 ? (key_end + KT - 1) / KT : 0;
    // sliding window / local chunks (causal only): row q's first key is
    // key_lower_bound(L - M + j0 + q), non-decreasing in q; the tile's key tiles
    // start at row 0's bound, and tiles before row rows-1's bound need the mask
    const bool windowed = a.causal && (a.window_left >= 0 || a.attn_chunk > 0);
    const int lo_first = windowed ? key_lower_bound(max(L - M + j0, 0), a.window_left, a.attn_chunk)
                                  : 0;
    const int lo_last = windowed ? key_lower_bound(max(L - M + j0 + rows - 1, 0), a.window_left,
                                                   a.attn_chunk)
                                 : 0;
    const int kt_lo = min(lo_first / KT, n_ktiles);
    const int low_full = (lo_last + KT - 1) / KT;   // tiles from here on need no lower mask
    const int n_range = n_ktiles - kt_lo;
    const int n_split = max(1, min((n_range + a.split_tiles - 1) / a.split_tiles, a.max_splits));
    if (split >= n_split) return;
    const int t_begin = kt_lo + split * a.split_tiles;
    const int t_end = (split == n_split - 1) ? n_ktiles : t_begin + a.split_tiles;
    const int n_all = max(t_end - t_begin, 0);
    const int n_iter = GROUPS == 2 ? (n_all + 1) / 2 : n_all;   // group 0 takes the first half

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;
    const int gw = wave & 3;
    const int gb = t_begin + grp * n_iter;          // this group's first tile
    const int n_g = grp == 0 ? n_iter : n_all - n_iter;
    const int q = lane & 31;
    const int h = lane >> 5;
    const bool row_ok = q < rows && q0 + j0 + q < a.total_q;
    // keys visible to row q (rows past the tile's end compute discarded values)
    const int limit = a.causal ? min(L, L - M + j0 + q + 1) : L;
    const int row_lo = windowed ? key_lower_bound(max(L - M + j0 + q, 0), a.window_left,
                                                  a.attn_chunk)
                                : 0;
    // tiles entirely below every row's limit need no mask
    const int full_tiles = max(a.causal ? min(L, L - M + j0 + 1) : L, 0) / KT;
    const int64_t row_bytes = static_cast<int64_t>(a.hkv) * ROW;
    const char* kb = static_cast<const char*>(a.k) + static_cast<int64_t>(kvh) * ROW;
    const char* vb = static_cast<const char*>(a.v) + static_cast<int64_t>(kvh) * ROW;
    const int32_t* pt_row = a.pt + static_cast<int64_t>(b) * a.pt_stride;
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem));
    const uint32_t ring0 = lds0 + static_cast<uint32_t>(grp * GROUP_LDS);

    // per-lane offsets: copy source chunks, K and V operand reads (stage 0, t = 0)
    int chunk_off[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int key = (gw * IPW + i) * RPB + lane / CH;
      chunk_off[i] = swz(key, lane % CH) * 16;
    }
    // K operand read of k-step j: row q, chunk swz(q, 2j + h).
    const int kbase = grp * GROUP_LDS + q * ROW;
    // Transposed V read (s, n) of lane (G = lane/16, j = lane%16): key row
    // 8s + 4(G/2) + j/4 (+16t), dims 32n + 16(G%2) + 4(j%4) + [0, 4).
    int vofs[2][NB];
    {
      const int G = lane >> 4, j = lane & 15;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int row = 8 * s2 + 4 * (G >> 1) + (j >> 2);
          const int byte = 2 * (32 * n + 16 * (G & 1) + 4 * (j & 3));
          vofs[s2][n] = grp * GROUP_LDS + row * ROW + swz(row, byte / 16) * 16 + byte % 16;
        }
    }
    for (int hb = 0; hb < n_hb; ++hb) {
      const int hg = 4 * hb + gw;           // this wave's head within the GQA group
      const bool head_ok = hg < G;
      const int head = kvh * G + min(hg, G - 1);

      // the first segment's page entries, then the workgroup's Q tile. With
      // two groups Q is copied once into LDS: only the entries are waited for
      // before the first copies, and Q lands together with tile 0. With one
      // group (no free stage for four heads' Q) each wave loads its Q^T operand
      // (row q, dims 16j + 8h + [0, 8)) from memory, 16 bytes of the row per
      // lane and k-step, in the same round trip as the entries.
      const uint32_t entry_lds = lds0 + GROUPS * GROUP_LDS + wave * 512;
      if (n_g > 0) fetch_entries(a, pt_row, L, gb, gw, lane, entry_lds);
      u32x4 qop[NKS];
      if constexpr (GROUPS == 2) {
        copy_q(a, wave, lane, hb, kvh, G, q0 + j0, rows, lds0);
        if (n_g > 0) wait_vmem<QPW>();
      } else {
        const int tok = min(q0 + j0 + min(q, rows - 1), a.total_q - 1);
        const char* qrow = static_cast<const char*>(a.q) +
                           (static_cast<int64_t>(tok) * a.hq + head) * ROW;
#pragma unroll
        for (int j = 0; j < NKS; ++j)
          qop[j] = *reinterpret_cast<const u32x4*>(qrow + (16 * j + 8 * h) * 2);
        wait_vmem<0>();   // the entries and Q
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
      RowState st = row_state_init();
      const float rescale_step = kRescaleLog2 / a.scale_log2;

      // ---- pipeline: tile i+2 is copied while tile i is consumed ----
      // Before tile i is read, every copy issued before tile i+1's must have
      // landed: at most the 2*IPW copies of tile i+1 stay in flight.
      // entry slots of segment m: entry_lds + (m % 2) * 256 (LDS address / pointer)
      const int32_t* entry_ptr =
          reinterpret_cast<const int32_t*>(smem + GROUPS * GROUP_LDS + wave * 512);
      auto entries_of = [&](int it) { return entry_ptr + ((it / SEG) & 1) * 64; };
      // Tile i's K and V land in stage i % 4, copied three tiles ahead; tile
      // i's softmax and O^T update run together with tile i+1's S^T, so at the
      // top of iteration i tile i+1 must have landed: at most the 2*IPW copies
      // of tile i+2 stay in flight.
      f32x16 s_cur;
      if (n_g > 0) {
#pragma unroll
        for (int i = 0; i < 3; ++i)
          if (i < n_g)
            copy_tile(a, L, gb + i, i, gw, lane, entries_of(i), row_bytes, kb, vb, chunk_off,
                      ring0 + i * STAGE);
        if (n_g > 2) wait_vmem<4 * IPW>();
        else if (n_g > 1) wait_vmem<2 * IPW>();
        else wait_vmem<0>();
      } else {
        wait_vmem<0>();   // this wave's Q copies
      }
      __syncthreads();   // tile 0 and Q are in LDS
      // two groups: the Q^T operand (row q, dims 16j + 8h + [0, 8)) of this
      // wave's head, read before the loop's first barrier (after which stage 3
      // takes tile 3)
      if constexpr (GROUPS == 2) read_k(smem + q_lds(gw) - grp * GROUP_LDS, kbase, q, h, qop);
      if (n_g > 0) {
        u32x4 kw[NKS];
        read_k(smem, kbase, q, h, kw);
#pragma unroll
        for (int r = 0; r < 16; ++r) s_cur[r] = 0.f;
#pragma unroll
        for (int j = 0; j < NKS; ++j)
          s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw[j]), as_bf16x8(qop[j]),
                                                          s_cur, 0, 0, 0);
      }
      // unrolled by the ring depth, so every stage offset below is a constant
      // (folded into the LDS instructions' offsets instead of added per read)
      for (int it0 = 0; it0 < n_iter; it0 += NSTAGE) {
#pragma unroll
      for (int u = 0; u < NSTAGE; ++u) {
        const int it = it0 + u;
        if (it < n_iter) {
        if (it + 1 < n_g) {
          if (it + 2 < n_g) wait_vmem<2 * IPW>();
          else wait_vmem<0>();
        }
        __syncthreads();   // tile it+1 is in LDS; stage (it + 3) % 4 is free
        // the next segment's entries land before the wait that precedes its
        // first copy (issued ahead of this iteration's copy)
        if ((it + 4) % SEG == 0 && it + 4 < n_g)
          fetch_entries(a, pt_row, L, gb + it + 4, gw, lane,
                        entry_lds + (((it + 4) / SEG) & 1) * 256);
        if (it + 3 < n_g)
          copy_tile(a, L, gb + it + 3, (it + 3) % SEG, gw, lane, entries_of(it + 3), row_bytes,
                    kb, vb, chunk_off, ring0 + ((u + 3) % NSTAGE) * STAGE);
        if (it < n_g) {
          const int kt = gb + it;
          u32x4 kw[NKS];
          read_k(smem + ((u + 1) % NSTAGE) * STAGE, kbase, q, h, kw);
          s_cur = softmax_pv(s_cur, smem + u * STAGE + TILE, vofs,
                             kt >= full_tiles || kt < low_full, limit - kt * KT - 4 * h,
                             row_lo - kt * KT - 4 * h, a.scale_log2, rescale_step, kw, qop, acc,
                             st);
        }
        }
      }
      }
      __syncthreads();   // every wave is done with the rings

      // ---- merge the two key halves (group 1 -> group 0) through LDS ----
      // wave gw's region: [float4 k][lane], k < 4 NB: acc[k/4][4(k%4) .. +3], then (m, l)
      f32x4* mbuf = reinterpret_cast<f32x4*>(smem) + gw * MERGE_F4 * 64 + lane;
      if (GROUPS == 2 && grp == 1) {
#pragma unroll
        for (int k = 0; k < 4 * NB; ++k)
          mbuf[64 * k] = f32x4{acc[k >> 2][4 * (k & 3)], acc[k >> 2][4 * (k & 3) + 1],
                               acc[k >> 2][4 * (k & 3) + 2], acc[k >> 2][4 * (k & 3) + 3]};
        mbuf[64 * 4 * NB] = f32x4{st.m, st.l, 0.f, 0.f};
      }
      if constexpr (GROUPS == 2) __syncthreads();
      float lse_val = 0.f, inv = 0.f;
      if (grp == 0) {
        float mm = st.m, l_m = st.l;
        if constexpr (GROUPS == 2) {
          const f32x4 ml = mbuf[64 * 4 * NB];
          const float m1 = ml[0];
          const float l1 = ml[1];
          mm = fmaxf(st.m, m1);
          const float f0 = (st.m == neg_inf()) ? 0.f : fast_exp2((st.m - mm) * a.scale_log2);
          const float f1 = (m1 == neg_inf()) ? 0.f : fast_exp2((m1 - mm) * a.scale_log2);
#pragma unroll
          for (int k = 0; k < 4 * NB; ++k) {
            const f32x4 o1 = mbuf[64 * k];
#pragma unroll
            for (int c = 0; c < 4; ++c)
              acc[k >> 2][4 * (k & 3) + c] = f0 * acc[k >> 2][4 * (k & 3) + c] + f1 * o1[c];
          }
          l_m = f0 * st.l + f1 * l1;
        }
        const float l_tot = l_m + __shfl_xor(l_m, 32);
        inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        lse_val = l_tot > 0.f ? (mm * a.scale_log2 + fast_log2(l_tot)) * kLn2 : neg_inf();
      }
      const int64_t row = q0 + j0 + q;
      if (n_split == 1) {
        if (grp == 0 && head_ok && row_ok) {
          float o[16][NB];
#pragma unroll
          for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int n = 0; n < NB; ++n) o[r][n] = acc[n][r];
          store_out_row(static_cast<bf16_t*>(a.out) + (row * a.hq + head) * D, h, o, inv);
          if (a.lse != nullptr && h == 0) a.lse[row * a.hq + head] = lse_val;
        }
        __syncthreads();   // the merge buffer is reused by the next head block
        continue;
      }

      // partial of this split, one block per (split, q-tile slot, head): the
      // wave's 32 rows x D as bf16 (the output precision), lane l's values
      // acc[n][8k .. 8k + 8) at 16-byte piece (2n + k) * 64 + l, so that every
      // store (and each of the merge's loads) covers 1 KB of contiguous
      // memory; the LSEs of the 32 rows follow each other. Stored at device
      // scope (see coherent_rsrc).
      const uint32_t o_bytes = static_cast<uint32_t>(QT * D * 2);
      const uint32_t l_bytes = static_cast<uint32_t>(QT * 4);
      const uint32_t l_lane = static_cast<uint32_t>(q * 4);
      auto block_of = [&](int sp) {
        return (static_cast<int64_t>(sp) * a.qtile_slots + slot) * a.hq + head;
      };
      auto o_rsrc = [&](int sp) {
        return coherent_rsrc(static_cast<char*>(a.ws_o) + block_of(sp) * o_bytes, o_bytes);
      };
      if (grp == 0 && head_ok) {
        const int64_t blk = block_of(split);
        const auto ro = o_rsrc(split);
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const u32x4 w = {pack_bf16x2(acc[n][8 * k] * inv, acc[n][8 * k + 1] * inv),
                             pack_bf16x2(acc[n][8 * k + 2] * inv, acc[n][8 * k + 3] * inv),
                             pack_bf16x2(acc[n][8 * k + 4] * inv, acc[n][8 * k + 5] * inv),
                             pack_bf16x2(acc[n][8 * k + 6] * inv, acc[n][8 * k + 7] * inv)};
            store_coherent(ro, static_cast<uint32_t>(((2 * n + k) * 64 + lane) * 16),
                           __builtin_bit_cast(f32x4, w));
          }
        if (h == 0) store_coherent(coherent_rsrc(a.ws_lse + blk * QT, l_bytes), l_lane, lse_val);
      }
      wait_all_vmem();
      __syncthreads();   // every wave's partial has been written through
      int* counter = a.counters +
                     ((static_cast<int64_t>(slot) * a.hkv + kvh) * n_hb + hb);
      if (threadIdx.x == 0) sh_last = (counter_add(counter, 1) == n_split - 1);
      __syncthreads();
      if (!sh_last) continue;
      // the last split of this (q tile, kv head, head block) merges all of
      // them, in split order, kMergeBatch splits' pieces (and their LSEs) in
      // flight together (n_split <= kMaxSplits)
      if (grp == 0 && head_ok && row_ok) {
        auto lse_of = [&](int s2) {
          return s2 < n_split
                     ? load_coherent1(coherent_rsrc(a.ws_lse + block_of(s2) * QT, l_bytes), l_lane)
                     : neg_inf();
        };
        float mx = neg_inf();
        {
          float ls[kMaxSplits];
#pragma unroll
          for (int s2 = 0; s2 < kMaxSplits; ++s2) ls[s2] = lse_of(s2);
#pragma unroll
          for (int s2 = 0; s2 < kMaxSplits; ++s2) mx = fmaxf(mx, ls[s2]);
        }
        float o[16][NB];
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int n = 0; n < NB; ++n) o[r][n] = 0.f;
        float wsum = 0.f;
        if (mx != neg_inf()) {
#pragma unroll 1
          for (int s0 = 0; s0 < n_split; s0 += kMergeBatch) {
            u32x4 v[kMergeBatch][2 * NB];
            float l4[kMergeBatch];
#pragma unroll
            for (int k4 = 0; k4 < kMergeBatch; ++k4) {
              const int s2 = min(s0 + k4, n_split - 1);   // (past the end: loaded, not used)
              const auto ro = o_rsrc(s2);
#pragma unroll
              for (int pi = 0; pi < 2 * NB; ++pi)
                v[k4][pi] = __builtin_bit_cast(
                    u32x4, load_coherent4(ro, static_cast<uint32_t>((pi * 64 + lane) * 16)));
              l4[k4] = lse_of(s0 + k4);
            }
#pragma unroll
            for (int k4 = 0; k4 < kMergeBatch; ++k4) {
              const float wgt = l4[k4] == neg_inf() ? 0.f : fast_exp2((l4[k4] - mx) * kLog2e);
              wsum += wgt;
#pragma unroll
              for (int n = 0; n < NB; ++n)
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const uint32_t w = v[k4][2 * n + k][e];
                    o[8 * k + 2 * e][n] = __builtin_fmaf(wgt, bf16lo(w), o[8 * k + 2 * e][n]);
                    o[8 * k + 2 * e + 1][n] =
                        __builtin_fmaf(wgt, bf16hi(w), o[8 * k + 2 * e + 1][n]);
                  }
            }
          }
        }
        store_out_row(static_cast<bf16_t*>(a.out) + (row * a.hq + head) * D, h, o,
                      wsum > 0.f ? 1.f / wsum : 0.f);
        if (a.lse != nullptr && h == 0)
          a.lse[row * a.hq + head] = (mx == neg_inf()) ? neg_inf() : mx + fast_log2(wsum) * kLn2;
      }
      if (threadIdx.x == 0) counter_reset(counter);   // ready for the next call
    }
  }
};

template <int D, int PM, int GROUPS>
__global__ __launch_bounds__(256 * GROUPS, 2 / GROUPS) void prefill_kernel(PrefillArgs a) {
  PrefillKernel<D, PM, GROUPS>::run(a);
}

}  // namespace pkv

namespace pkv_launch {

template <int D, int PM>
static void launch_prefill_t(const pkv::PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.groups == 1)
    hipLaunchKernelGGL((pkv::prefill_kernel<D, PM, 1>), grid, dim3(256),
                       (pkv::PrefillKernel<D, PM, 1>::LDS_BYTES), stream, a);
  else
    hipLaunchKernelGGL((pkv::prefill_kernel<D, PM, 2>), grid, dim3(512),
                       (pkv::PrefillKernel<D, PM, 2>::LDS_BYTES), stream, a);
}

template <int D>
static void launch_prefill_d(const pkv::PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.page_size == 1) launch_prefill_t<D, pkv::kPageToken>(a, grid, stream);
  else if (a.page_shift >= 0) launch_prefill_t<D, pkv::kPagePow2>(a, grid, stream);
  else launch_prefill_t<D, pkv::kPageAny>(a, grid, stream);
}

hipError_t prefill(const pkv::PrefillArgs& a, int head_dim, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.qtile_slots) * a.max_splits * a.hkv;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (head_dim == 128) launch_prefill_d<128>(a, grid, stream);
  else launch_prefill_d<64>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace pkv_launch

// Paged MLA decode with role-split waves, three per SIMD (gfx950): every
// fp8-dot decode, and bf16-dot decodes of at most 16 rows per key stream.
//
// What is computed is the decode of mla_decode.hip (FlashMLA PR #82 "update fp8
// support", description; ROCm/aiter PR #6199, Technical details; InfiniCore
// PR #1568, Summary and split-kv commit): softmax attention of every query
// row of a sequence over its paged e4m3fn latent cache, K = [nope * k_scale,
// bf16 rope], V = nope * v_scale, with Q's nope part quantized per row to
// e4m3fn and P to e4m3fn for the fp8 matrix cores.
//
// Why another kernel: with all 128 query rows of a sequence in one workgroup,
// the fp32 output accumulator O (128 rows x 512 dv) takes 256 registers per
// lane at one wave per SIMD, and a lone wave issues its MFMAs, its LDS reads
// and its softmax VALU work one after another. Here the work of a tile is
// split by role over twelve waves, three per SIMD, so that one wave's
// softmax and LDS waits overlap another's matrix products:
//  * waves 0..3 ("S-waves"): wave r owns query rows 32r..32r+31 of the row
//    group; S^T = K Q^T of the tile (16 fp8 and 8 bf16 32x32 MFMAs), the
//    masked online softmax in the log2 domain, and P^T of the tile to LDS;
//  * waves 4..11 ("PV-waves"): wave 4+e owns dv 64e..64e+63 of all 128 rows,
//    O^T += V^T P^T (8 fp8 32x32x64 MFMAs per tile, O in 128 VGPRs), and
//    issues one eighth of the tile copies (global -> LDS).
// The PV-waves multiply tile k-1 while the S-waves take tile k; one barrier
// per tile orders the three-tile LDS ring, the P^T exchange (double-buffered
// by tile parity) and the rescale flags.
//
// Tile layout: the 32 KiB of nope bytes of a tile are eight 4 KiB slices,
// slice e holding bytes 64e..64e+63 (dv 64e..64e+63, also K dims 64e..) of
// all 64 keys, 64 bytes per key with its four 16-byte chunks XOR-swizzled by
// (key >> 2) & 3; the 64 rope rows (128 B) follow the layout of
// mla_decode.hip. Both the 16-lane groups of the S^T fragment reads (16
// consecutive keys, one chunk) and the 32-lane groups of the transposing V^T
// reads hit 64 distinct banks. With this layout PV-wave e reads only slice e
// of tile k-1, so it may refill that slice with tile k+2 as soon as its own
// reads have returned: every copy has two iterations to land in the same
// three-tile ring (the rope rows of tile k+2 go to the rope slot S^T(k-1)
// released). S-wave r and PV-waves r, r+4 share
// SIMD r (waves are placed on the SIMDs round-robin). During its S^T
// products an S-wave runs at raised priority, so the P.V products fill the
// matrix core around them rather than delaying them.
//
// The tile layout in LDS (XOR-swizzled 16-byte chunks), the fragment
// bookkeeping of the 32x32 MFMAs, the fp8 query quantization, the lazily
// raised running max and the P scale are those of mla_decode.hip
// (mla_device.h); the two kernels issue the same products and agree to
// rounding order.
//
// Two-term forms (template TT, at most 16 query rows per key stream): the
// rows fill only columns 0..15 of row block 0, so columns 16..31 carry a
// second e4m3fn term, 16 (x - e4m3fn(x)), of each row's query (TT 1: fp8
// dots multiply the exact bf16 query) and of P as well (TT 2: bf16-dot
// accuracy on the fp8 matrix cores). The S-wave adds the column pairs after
// its S^T products; the PV-waves fold O's column pairs once, at the end.

#include "mla_device.h"

namespace mla {

constexpr int kSWaves = 4;     // one per 32-row block of the row group
constexpr int kPVWaves = 8;    // one per 64-wide dv slice
constexpr int kWsThreads = 64 * (kSWaves + kPVWaves);

// LDS past the KV ring, double-buffered by tile parity: P^T of the four row
// blocks (2 KiB each, two 16-byte halves per lane), per-row rescale factors
// and per-row-block flags; then the per-row output scale for the epilogue.
struct WsX {
  static constexpr int p_bytes = kSWaves * 2048;
  static constexpr int alpha_bytes = kSWaves * 32 * 4;
  static constexpr int flag_off = 2 * p_bytes + 2 * alpha_bytes;   // 2 x 4 ints
  static constexpr int fin_off = flag_off + 32;
  static constexpr int bytes = fin_off + kSWaves * 32 * 4;
};

// LDS that nothing touches before the first tile barrier, where the PV-waves
// stage the quantized query for the S-waves: the third ring slot's nope bytes
// (row blocks 0 and 1, 16 KiB each), its rope bytes and the exchange area
// (row blocks 2 and 3), then 128 row exponents. Row n of a block holds its
// 512 codes with 16-byte chunk j at position j ^ n.
template <int ROPE>
struct WsQ {
  static constexpr int a_off = 2 * kNopeRegion;
  static constexpr int b_off = Tile<ROPE>::lds_bytes - (ROPE > 0 ? kRopeRegion : 0);
  static constexpr int exp_off = b_off + 2 * 16384;
  static constexpr int end = exp_off + kSWaves * 32 * 4;
  static constexpr int lds_bytes = end > Tile<ROPE>::lds_bytes + WsX::bytes ? end : Tile<ROPE>::lds_bytes + WsX::bytes;
  static_assert(kBufs == 3 && a_off + 2 * 16384 <= kRopeBase, "row blocks 0 and 1 fit the third nope slot");
  static_assert(ROPE == 0 || b_off == kRopeBase + 2 * kRopeRegion, "row blocks 2 and 3 start at the third rope slot");
  static_assert(lds_bytes <= 160 * 1024, "LDS");
};

// The lane id from the exec-mask bit count, as volatile asm: recomputed where
// it is used inside a tile loop rather than kept (and, at three waves per
// SIMD, spilled and reloaded from scratch memory every tile).
__device__ inline int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Max of x over lanes l and l ^ 32 (the two halves of one query row) with the
// gfx950 lane swap: no LDS round trip.
__device__ inline float pair_max_swap(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum_swap(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copies of slice e of a tile into nope slot `bufi`: four 1 KiB copies, copy i
// covering keys 16i..16i+15; lane l moves position l % 4 of key 16i + l / 4,
// i.e. its logical chunk (l % 4) ^ ((key >> 2) & 3) = (l % 4) ^ (l / 16),
// from global byte key * RB + 64e + 16 * chunk. A full page is copied with the
// scalar page base; keys at or past `valid` are zero-filled instead (the
// page's slack, or the whole tile for a missing page), after which the wave
// drains its copies.
template <int ROPE>
__device__ __attribute__((always_inline)) inline void ws_issue_nope_slice(uint8_t* lds, int bufi, const uint8_t* page_base,
                                                                          int valid, int e) {
  constexpr int RB = kNope + 2 * ROPE;
  int lane;   // volatile: recomputed here rather than kept across the tile loop
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  uint8_t* dst = lds + bufi * kNopeRegion + e * 4096;
  const unsigned lane_off = (unsigned)((lane >> 2) * RB + 16 * ((lane & 3) ^ (lane >> 4)));
  if (valid == kKeys) {
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16_saddr(page_base + 16 * i * RB + 64 * e, lane_off, dst + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (16 * i + (lane >> 2) < valid)
        load_lds16(page_base + (unsigned)(16 * i * RB + 64 * e) + lane_off, dst + i * 1024);
      else
        lds_zero16(dst + i * 1024 + lane * 16);
    }
    wait_vmcnt<0>();
  }
}

// Rope rows 8e..8e+7 of a tile into rope slot `bufi` (the layout of
// mla_decode.hip: lane l moves position l % 8 of row 8e + l / 8, i.e. its
// chunk (l % 8) ^ ((row >> 1) & 7)); rows at or past `valid` zero-filled.
template <int ROPE>
__device__ __attribute__((always_inline)) inline void ws_issue_rope(uint8_t* lds, int bufi, const uint8_t* page_base,
                                                                    int valid, int e) {
  constexpr int RB = kNope + 2 * ROPE;
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int r8 = lane >> 3, p8 = lane & 7;
  uint8_t* rope = lds + kRopeBase + bufi * kRopeRegion + e * 1024;
  if (valid == kKeys) {
    const unsigned off = (unsigned)(r8 * RB + kNope) + ((((unsigned)(p8 ^ (r8 >> 1))) << 4) ^ (64u * (unsigned)(e & 1)));
    load_lds16_saddr(page_base + 8 * e * RB, off, rope);
  } else {
    const int row = 8 * e + r8;
    if (row < valid)
      load_lds16(page_base + (unsigned)(row * RB + kNope + ((p8 ^ ((row >> 1) & 7)) << 4)), rope);
    else
      lds_zero16(rope + lane * 16);
    wait_vmcnt<0>();
  }
}

// Sparse path (top-k index lists): the cache rows of a tile's 64 entries are
// found through two dependent loads, the entry's index and the page-table
// slot it falls in. One wave brings both into LDS slots by 4-byte DMA copies,
// each one iteration ahead of its use: the index of tile t+4 and the page of
// tile t+3 while the waves work on tile t, so that the copies of tile t+2 and
// the masks of tile t read only LDS. Lanes with no source (entries past the
// list, skipped or out-of-range indices) copy from kWsMinusOne, so that every
// copy instruction runs on all lanes and the copy counts per tile stay fixed.
constexpr int kSpSlots = 5;            // index of tile t written at t-4, last read at t
constexpr int kSpSlotBytes = 512;      // 64 indices, then 64 page ids
__device__ __align__(16) const int32_t kWsMinusOne[64] = {
    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1,
    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1,
    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
// 16 zero bytes per lane: the source of a skipped entry's tile bytes (a
// masked key's P is 0, and 0 times a finite code is 0).
__device__ __align__(16) const uint8_t kWsZeros[64 * 16] = {};

// Cache row (page * 64 + slot) of entry `key` of a tile from its lookup slot,
// or -1 when the entry is skipped.
__device__ inline int ws_sparse_row(const uint8_t* slot, int key, int sk, int num_pages) {
  const int j = reinterpret_cast<const int32_t*>(slot)[key];
  const int page = reinterpret_cast<const int32_t*>(slot + 256)[key];
  return j >= 0 && j < sk && page >= 0 && page < num_pages ? page * kKeys + (j & (kKeys - 1)) : -1;
}

// The sparse tile's copies of slice e (as ws_issue_nope_slice: lane l moves
// position l % 4 of key 16 i + l / 4) and of rope rows 8e..8e+7 (as
// ws_issue_rope), each lane from its entry's cache row, or zeros: always
// 4 + (rope ? 1 : 0) copy instructions on all lanes.
template <int ROPE>
__device__ __attribute__((always_inline)) inline void ws_issue_sparse_nope(uint8_t* lds, int bufi, const uint8_t* kv,
                                                                           const uint8_t* slot, int sk, int num_pages,
                                                                           int e) {
  constexpr long RB = kNope + 2 * ROPE;
  const int lane = fresh_lane();
  uint8_t* dst = lds + bufi * kNopeRegion + e * 4096;
  const unsigned chunk16 = 16u * (unsigned)((lane & 3) ^ (lane >> 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cr = ws_sparse_row(slot, 16 * i + (lane >> 2), sk, num_pages);
    const uint8_t* src = cr >= 0 ? kv + (long)cr * RB + 64 * e + chunk16 : kWsZeros + 16 * lane;
    load_lds16(src, dst + i * 1024);
  }
}
template <int ROPE>
__device__ __attribute__((always_inline)) inline void ws_issue_sparse_rope(uint8_t* lds, int bufi, const uint8_t* kv,
                                                                           const uint8_t* slot, int sk, int num_pages,
                                                                           int e) {
  constexpr long RB = kNope + 2 * ROPE;
  const int lane = fresh_lane();
  const int row = 8 * e + (lane >> 3);
  const int cr = ws_sparse_row(slot, row, sk, num_pages);
  const unsigned c16 = 16u * (unsigned)((lane & 7) ^ ((row >> 1) & 7));
  const uint8_t* src = cr >= 0 ? kv + (long)cr * RB + kNope + c16 : kWsZeros + 16 * lane;
  load_lds16(src, lds + kRopeBase + bufi * kRopeRegion + e * 1024);
}

// gfx942's e4m3fnuz codes turned into OCP e4m3fn codes (fnuz4_to_ocp4), in
// place in this wave's 4 KiB slice of a landed tile: the fp8 matrix cores read
// OCP codes only.
__device__ inline void ws_fnuz_to_ocp_slice(uint8_t* lds, int bufi, int e) {
  uint8_t* p = lds + bufi * kNopeRegion + e * 4096 + fresh_lane() * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    i32x4 v = *reinterpret_cast<const i32x4*>(p + 16 * i);
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = (int)fnuz4_to_ocp4((unsigned)v[d]);
    *reinterpret_cast<i32x4*>(p + 16 * i) = v;
  }
}

// TT: 0 one-term query and P; 1 (at most 16 rows, fp8 dots) two-term query,
// one-term P; 2 (at most 16 rows, bf16 dots) two-term query and P.
template <int ROPE, bool FNUZ, bool SPARSE, bool PT, int TT>
__global__ __attribute__((amdgpu_flat_work_group_size(kWsThreads, kWsThreads), amdgpu_waves_per_eu(3, 3)))
void mla_decode_ws_kernel(MLA_KERNEL_PTRS, KDims a) {
  constexpr bool SPLITQ = TT >= 1;   // columns n + 16 carry the second query term
  constexpr bool SPLITP = TT == 2;   // ... and the second term of P
  constexpr int D = kNope + ROPE;   // q row length
  constexpr long RB = kNope + 2 * ROPE;
  constexpr int kSpBytes = SPARSE ? kSpSlots * kSpSlotBytes : 0;
  constexpr int kPtBytes = PT ? kBufs * 512 : 0;   // per ring slot: 64 k-scales, 64 v-scales
  // lazy-max threshold and P scale (log2) of the single-term and two-term P
  constexpr float kTau = SPLITP ? SoftSplit::tau : Soft<DOT_FP8>::tau;
  constexpr float kPsLog2 = SPLITP ? SoftSplit::ps_log2 : Soft<DOT_FP8>::ps_log2;
  static_assert(WsQ<ROPE>::lds_bytes + kSpBytes + kPtBytes <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_[WsQ<ROPE>::lds_bytes + kSpBytes + kPtBytes];
  uint8_t* const lds = lds_;
  uint8_t* const xp = lds + Tile<ROPE>::lds_bytes;
  float* const xalpha = reinterpret_cast<float*>(xp + 2 * WsX::p_bytes);
  int* const xflag = reinterpret_cast<int*>(xp + WsX::flag_off);
  float* const xfin = reinterpret_cast<float*>(xp + WsX::fin_off);
  // prologue only: the quantized query rows of row block w, then the exponents
  auto qstage = [&](int w) -> uint8_t* { return lds + (w < 2 ? WsQ<ROPE>::a_off + w * 16384 : WsQ<ROPE>::b_off + (w - 2) * 16384); };
  int* const qexp = reinterpret_cast<int*>(lds + WsQ<ROPE>::exp_off);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;

  int bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int rg = bid % a.row_groups;
  bid /= a.row_groups;
  const int s = bid % a.splits;
  const int g = bid / a.splits;

  // dense: g is a sequence, its key stream the sequence's pages; sparse: g
  // is a query token (sequence g / s_q), its key stream the token's index
  // list in 64-entry units
  const int b = SPARSE ? g / a.s_q : g;
  int sk = seq_lens[b];
  sk = max(0, min(sk, a.max_pages * kKeys));
  const int units = SPARSE ? (a.topk + kKeys - 1) / kKeys : (sk + kKeys - 1) / kKeys;
  const int u0 = (int)((long)s * units / a.splits);
  const int u1 = (int)((long)(s + 1) * units / a.splits);
  const int ntiles = u1 - u0;
  const int32_t* bt_row = block_table + (long)b * a.max_pages;
  // page id of unit u0 + t (uniform: a scalar load)
  auto page_at = [&](int t) -> int { return u0 + t < u1 ? bt_row[u0 + t] : -1; };
  auto page_valid = [&](int page) -> bool { return page >= 0 && page < a.num_pages; };
  // sparse: the lookup slot of tile t, and the two DMA steps that fill it
  // (the caller's wave issues them; see kSpSlots)
  uint8_t* const sp_base = lds + WsQ<ROPE>::lds_bytes;
  // per-token scales: the 64 k-scales and 64 v-scales of the tile in ring slot b
  float* const pt_base = reinterpret_cast<float*>(lds + WsQ<ROPE>::lds_bytes + kSpBytes);
  auto sp_slot = [&](int t) -> uint8_t* { return sp_base + (t % kSpSlots) * kSpSlotBytes; };
  auto sp_dma_index = [&](int t) {
    const int32_t* idx_row = indices + (long)g * a.topk;
    const int e = (u0 + t) * kKeys + fresh_lane();
    const int32_t* src = e < a.topk ? idx_row + e : kWsMinusOne;
    load_lds4_gather(reinterpret_cast<const float*>(src), sp_slot(t));
  };
  auto sp_dma_page = [&](int t) {   // the index of tile t has landed
    const int j = reinterpret_cast<const int32_t*>(sp_slot(t))[fresh_lane()];
    const int32_t* src = j >= 0 && j < sk ? bt_row + (j >> 6) : kWsMinusOne;
    load_lds4_gather(reinterpret_cast<const float*>(src), sp_slot(t) + 256);
  };

  if (wave < kSWaves) {
    // ======================= S-wave: S^T, softmax, P^T ========================
    const int rb = rg * kSWaves + wave;
    const bool wave_active = rb < a.row_blocks;
    // two-term query (SPLITQ, at most 16 rows): columns n and n + 16 of the
    // block hold the two terms of row n, so both lane halves take row n % 16
    const int row = rb * 32 + (SPLITQ ? (n & 15) : n);
    const bool row_ok = row < a.rows;
    const long qrow_idx = (long)g * a.rows + row;
    const bool q_ok = row_ok && wave_active;
    const uint16_t* qsrc = q_ok ? q + qrow_idx * D : q;   // rows outside the problem read row 0, zeroed below

    // The query's rope values and the page ids come from global memory; its
    // nope part, quantized by the PV-waves during the prologue, from LDS.
    i32x4 qr_raw[ROPE > 0 ? 4 : 1];
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) qr_raw[t] = *reinterpret_cast<const i32x4*>(qsrc + kNope + 16 * t + 8 * h);
    }
    const float k_scale_v = PT ? 1.f : *k_scale;   // per token: the k-scales apply per key
    const int i_tok = row / a.h_q;
    const int row_len = row_ok ? (a.causal ? sk - (a.s_q - 1 - i_tok) : sk) : 0;   // keys this row may see
    wait_vmcnt<0>();
    bf16x8 qr[ROPE > 0 ? 4 : 1];
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        i32x4 v = qr_raw[t];
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = q_ok && !(SPLITQ && n >= 16) ? v[d] : 0;   // rope: first term only
        qr[t] = __builtin_bit_cast(bf16x8, v);
      }
    }
    __syncthreads();   // the quantized query rows are staged
    // fragment t of lane (n, h): codes of dims 64 t + 32 h .. +31, staged
    // chunks 4 t + 2 h and 4 t + 2 h + 1 of row n
    i32x8 qn[8];
    {
      const uint8_t* qs = qstage(wave) + n * 512;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const i32x4 lo = lds_ld16(qs, ((4 * t + 2 * h) ^ n) << 4);
        const i32x4 hi = lds_ld16(qs, ((4 * t + 2 * h + 1) ^ n) << 4);
        qn[t] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }
    const int qe = qexp[wave * 32 + n];
    // the staging area is reused once the tile loop starts: reads done first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const float qk_scale = ldexpf(k_scale_v, qe);   // q_scale * k_scale on the nope products

    // z (log2 units) = acc * zscale: with rope the nope sums are scaled by
    // q_scale * k_scale in place before the rope products accumulate onto them
    // (kept >= 1e-37: a row whose q_scale * k_scale underflows to 0 would turn
    // masked keys' -inf * 0 into NaN; its logits are ~0 either way)
    const float zscale = ROPE > 0 ? a.sm_log2 : fmaxf(qk_scale * a.sm_log2, 1e-37f);
    float m_run = -INFINITY;   // max used for the exponentials (log2 domain)
    float l_run = 0.f;         // this lane's share of the running sum
    // Per-token scales: P is packed as p * v_j / v_run, v_run a reference
    // v-scale raised lazily (to the tile's largest when a key's v-scale
    // exceeds 1.5 v_run, so that P stays <= 1.5 * 2^8 = 384 < 448); O carries
    // v_run and is rescaled by v_old / v_new when it rises. 1 / v_run rides
    // in the exponent (log2 v_run, 0 while v_run is), so p / v_run costs no
    // multiply; the row sums take v_run back once per tile.
    float v_run = 0.f;
    // k-scales of the lane's keys of key block kb (register r: key 32 kb + 8 j
    // + 4 ((j + h) & 1) + r % 4, j = r / 4), four per read
    // (one read in flight at a time: the S-wave's registers are full here)
    auto scale_by_k = [&](f32x16& acc_kb, int kb, const float* ks, float f) {
      const int hh = fresh_lane() >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(ks + 32 * kb + 8 * j + 4 * ((j + hh) & 1));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc_kb[4 * j + rr] *= k4[rr] * f;
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    int buf = 0;
    for (int k = 0; k <= ntiles; ++k) {
      __syncthreads();   // tile k landed; P^T of tile k-2's parity is free again
      if (k == ntiles) break;
      const int par = k & 1;
      if (!wave_active) {   // a row block past the problem: the barriers only
        if (fresh_lane() == 0) xflag[4 * par + wave] = 0;
        continue;
      }
      const int page_cur = SPARSE ? 0 : page_at(k);   // needed after the products
      // sparse: whether entry `lane` of tile k names a cache row
      const bool sp_ok = SPARSE ? ws_sparse_row(sp_slot(k), fresh_lane(), sk, a.num_pages) >= 0 : false;
      const uint8_t* nope = lds + buf * kNopeRegion;
      const uint8_t* rope = lds + kRopeBase + buf * kRopeRegion;
      const int unit = u0 + k;

      // ---- S^T = K Q^T (fragment ring of PD items, alternating key blocks) ----
      __builtin_amdgcn_s_setprio(3);
      f32x16 acc[2];
      {
        // The lane's fragment addresses: fp8 fragment t, half e is
        // (kbase ^ 16 e) + 4096 t + 2048 kb, rope fragment t is rbase ^ 32 t
        // plus an immediate. Two bases, recomputed per tile from a lane id the
        // compiler cannot hoist (kept bases would not fit three waves per SIMD).
        int lv;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lv));
        const int krow = key_of_row(lv & 31), hh = lv >> 5;
        const int kbase = krow * 64 + (((2 * hh) ^ ((krow >> 2) & 3)) << 4);   // slice layout
        const int rbase = krow * 128 + ((hh ^ ((krow >> 1) & 7)) << 4);
        constexpr int NN = 16, NI = NN + (ROPE > 0 ? 8 : 0), PD = 3;
        i32x4 rl[PD], rh[PD];
        auto load = [&](int f) {
          const int slot = f % PD, kb = f & 1;
          if (f < NN) {
            // step t = slice t; key 32 kb + krow; chunks 2h, 2h + 1
            const int t = f >> 1;
            const int c = 4096 * t + 2048 * kb;
            rl[slot] = lds_ld16(nope, kbase + c);
            rh[slot] = lds_ld16(nope, (kbase ^ 16) + c);
          } else {
            rl[slot] = lds_ld16(rope, (rbase ^ (32 * ((f - NN) >> 1))) + 32 * kb * 128);
          }
        };
#pragma unroll
        for (int f = 0; f < PD; ++f) load(f);
#pragma unroll
        for (int f = 0; f < NI; ++f) {
          const int slot = f % PD, kb = f & 1;
          const i32x4 lo = rl[slot], hi = rh[slot];
          if (f + PD < NI) load(f + PD);
          if (f < NN) {
            const i32x8 kf = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if (f < 2) mfma_fp8_32x32x64_first(acc[kb], kf, qn[f >> 1]);
            else mfma_fp8_32x32x64(acc[kb], kf, qn[f >> 1]);
            if constexpr (ROPE > 0) {
              if (f == NN - 1) {
                // nope sums complete: scale them, then add the rope products
                s_nop_result2(acc[0], acc[1]);
                if constexpr (PT) {
                  scale_by_k(acc[0], 0, pt_base + buf * 128, qk_scale);
                  scale_by_k(acc[1], 1, pt_base + buf * 128, qk_scale);
                } else {
#pragma unroll
                  for (int r = 0; r < 16; ++r) {
                    acc[0][r] *= qk_scale;
                    acc[1][r] *= qk_scale;
                  }
                }
              }
            }
          } else {
            const bf16x8 kr = __builtin_bit_cast(bf16x8, lo);
            if (f < NN + 2) mfma_bf16_32x32x16_after_valu(acc[kb], kr, qr[(f - NN) >> 1]);
            else mfma_bf16_32x32x16(acc[kb], kr, qr[(f - NN) >> 1]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      s_nop_result2(acc[0], acc[1]);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (PT && ROPE == 0) {   // rope-free: q_scale rides on zscale
        scale_by_k(acc[0], 0, pt_base + buf * 128, 1.f);
        scale_by_k(acc[1], 1, pt_base + buf * 128, 1.f);
      }
      if constexpr (SPLITQ) {
        // S = S1 + S2 / 16 from columns n and n + 16 (16-lane rows 2i and
        // 2i + 1), left in both so that both halves run the same softmax.
        // Registers go in pairs: the swap of (r, r + 1) puts S1 and S2 of r
        // in the even rows and those of r + 1 in the odd rows; the sum's
        // swap with itself spreads both sums to every lane.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[kb][r]),
                                                            __float_as_uint(acc[kb][r + 1]), false, false);
            const unsigned c = __float_as_uint(fmaf(__uint_as_float(t[1]), 0.0625f, __uint_as_float(t[0])));
            const auto u = __builtin_amdgcn_permlane16_swap(c, c, false, false);
            acc[kb][r] = __uint_as_float(u[0]);
            acc[kb][r + 1] = __uint_as_float(u[1]);
          }
      }

      // ---- mask + online softmax (log2 domain), P^T to LDS ----------------------
      const bool page_ok = page_valid(page_cur);
      const unsigned long long smask = SPARSE ? __ballot(sp_ok) : 0ull;
      const bool full = SPARSE ? smask == ~0ull : page_ok && (unit + 1) * kKeys <= sk - (a.causal ? a.s_q - 1 : 0);
      const int limit = page_ok ? row_len - unit * kKeys : 0;
      if (SPARSE && !full) {
        // register r of key block kb is key 32 kb + 8 j + 4 ((j + h) & 1) + r % 4:
        // the upper lane half takes the mask with the two 4-key halves of every
        // 8-key group swapped, so that every bit position is a compile-time offset
        const bool hl = (fresh_lane() >> 5) != 0;
        const unsigned long long sw = ((smask & 0x0F0F0F0F0F0F0F0Full) << 4) | ((smask >> 4) & 0x0F0F0F0F0F0F0F0Full);
        const unsigned long long m = hl ? sw : smask;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = r >> 2;
            const int kc = 32 * kb + 8 * j + 4 * (j & 1) + (r & 3);
            acc[kb][r] = ((m >> kc) & 1ull) ? acc[kb][r] : -INFINITY;
          }
      } else if (!full) {
        // register r of key block kb is key 32 kb + 8 j + 4 ((j + h) & 1) + r % 4
        // (j = r / 4): compile-time offsets against two per-lane limits, so
        // that no per-lane key index is kept across the tile loop
        const int hl = fresh_lane() >> 5;
        const int lim_e = limit - 4 * hl, lim_o = limit - 4 * (1 - hl);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = r >> 2;
            const int kc = 32 * kb + 8 * j + (r & 3);
            acc[kb][r] = kc < ((j & 1) ? lim_o : lim_e) ? acc[kb][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][r]);
      mx = pair_max_swap(mx) * zscale;

      // per-token scales: raise v_run when a key of this tile (key = lane)
      // exceeds 1.5 v_run (always at the first tile with a key)
      float vfac = 1.f;   // v_old / v_new for O, 1 when v_run stays or was 0
      bool vraise = false;
      if constexpr (PT) {
        const int lk = fresh_lane();
        const bool exists = SPARSE ? sp_ok : page_ok && lk < min(kKeys, sk - unit * kKeys);
        const float vmine = exists ? pt_base[buf * 128 + 64 + lk] : 0.f;
        if (__ballot(vmine > 1.5f * v_run)) {
          float vm = vmine;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) vm = fmaxf(vm, __shfl_xor(vm, o));
          vm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, vm)));
          vraise = v_run > 0.f;
          vfac = vraise ? v_run / vm : 1.f;
          v_run = vm;
        }
      }
      const bool raise = mx > m_run + kTau;
      bool flagged = false;
      if (__ballot(raise) || vraise) {
        const float m_new = raise ? mx : m_run;
        // 0 for a row that has seen no key (its O and l are 0; the difference
        // of two infinities would give NaN)
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        // O needs rescaling only where a finite max was raised, or (all rows)
        // where v_run rose
        flagged = vraise || __ballot(raise && m_run != -INFINITY) != 0ull;
        if (flagged) {
          const int ln = fresh_lane();
          if (ln < 32) xalpha[par * (kSWaves * 32) + wave * 32 + ln] = alpha * vfac;
        }
        m_run = m_new;
      }
      const float m_exp = ((m_run == -INFINITY) ? 0.f : m_run) - kPsLog2 +
                          (PT && v_run > 0.f ? __builtin_amdgcn_logf(v_run) : 0.f);
      float psum = 0.f;
      i32x8 pb;
      const int lp = fresh_lane();
      const int hv = lp >> 5;
      const bool p_second = SPLITQ && (lp & 16) != 0;   // a column n + 16 lane
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {
        const int kb = q4 >> 2, r0 = 4 * (q4 & 3);
        float pe[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pe[r] = __builtin_amdgcn_exp2f(fmaf(acc[kb][r0 + r], zscale, -m_exp));
          psum = (q4 == 0 && r == 0) ? pe[r] : psum + pe[r];
        }
        if constexpr (PT) {
          // (p / v_run) times its key's v-scale (0 for a key that does not
          // exist, whose p is 0 too)
          const int j = q4 & 3;
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(pt_base + buf * 128 + 64 + 32 * kb + 8 * j + 4 * ((j + hv) & 1));
#pragma unroll
          for (int r = 0; r < 4; ++r) pe[r] *= v4[r];
        }
        pb[q4] = f32x4_to_fp8x4(pe[0], pe[1], pe[2], pe[3]);
        if constexpr (SPLITP) {
          // columns n + 16 carry the second term of P: 16 (p - e4m3fn(p))
          float c1[4];
          fp8x4_to_f32(pb[q4], c1);
          const int c2 = f32x4_to_fp8x4(16.f * (pe[0] - c1[0]), 16.f * (pe[1] - c1[1]), 16.f * (pe[2] - c1[2]),
                                        16.f * (pe[3] - c1[3]));
          pb[q4] = p_second ? c2 : pb[q4];
        } else if constexpr (SPLITQ) {
          pb[q4] = p_second ? 0 : pb[q4];   // one-term P: columns n + 16 add nothing
        }
      }
      l_run += PT ? psum * v_run : psum;
      uint8_t* pdst = xp + par * WsX::p_bytes + wave * 2048 + lp * 16;
      *reinterpret_cast<i32x4*>(pdst) = i32x4{pb[0], pb[1], pb[2], pb[3]};
      *reinterpret_cast<i32x4*>(pdst + 1024) = i32x4{pb[4], pb[5], pb[6], pb[7]};
      if (lp == 0) xflag[4 * par + wave] = flagged ? 1 : 0;
      buf = buf == kBufs - 1 ? 0 : buf + 1;
    }

    // ---- epilogue: per-row output scale for the PV-waves; lse ---------------------
    const float l_tot = pair_sum_swap(l_run);
    const bool nonempty = l_tot > 0.f;
    // splits == 1: (v_scale, or per token v_run) / l; else the partials' 1 / l
    // (fp16 partials in code units, |value| <= 448; the combine applies
    // v_scale, or the per-row v_run stored beside the lse)
    if (h == 0) xfin[wave * 32 + n] = nonempty ? (a.splits == 1 ? (PT ? v_run : *v_scale) : 1.f) / l_tot : 0.f;
    if (wave_active && h == 0) {
      const float lse2 = nonempty ? m_run + log2f(l_tot) - kPsLog2 : -INFINITY;
      if (a.splits == 1) {
        if (row_ok && !(SPLITQ && n >= 16)) lse[qrow_idx] = nonempty ? lse2 * kLn2 : -INFINITY;
      } else {
        const long prow = (((long)s * a.groups + g) * a.row_blocks + rb) * 32 + n;
        part_lse[prow] = lse2;
        if constexpr (PT) part_row_scale(part_lse, a)[prow] = v_run;
      }
    }
    __syncthreads();
  } else {
    // ===================== PV-wave: tile copies, O^T += V^T P^T =====================
    const int e = wave - kSWaves;          // dv slice 64e .. 64e + 63 (blocks 2e, 2e + 1)
    constexpr int kCopies = 4 + (ROPE > 0 ? 1 : 0);   // this wave's copies of one full tile
    // query staging: this wave quantizes rows 16 e .. 16 e + 15 of the row
    // group, one per lane quad (quarter qq holds chunks 4 i + qq); rows outside
    // the problem read row 0 and stage zero codes
    const int qrl = 16 * e + (lane >> 2), qq = lane & 3;
    // two-term query (SPLITQ): wave 1 stages the second terms of rows 0..15
    // as rows 16..31 of the block
    const bool q_second = SPLITQ && e == 1;
    const int qsrow = q_second ? qrl - 16 : qrl;   // the query row this lane reads
    const bool q_ok = rg * (kSWaves * 32) + qsrow < a.rows;
    // a wave none of whose rows exist (a 16-head sparse token uses one of the
    // eight) stages zeros without loading or quantizing anything
    const bool q_any = rg * (kSWaves * 32) + (q_second ? 0 : 16 * e) < a.rows;
    i32x4 qraw[16];
    if (q_any) {
      const uint16_t* qsrc = q + (q_ok ? ((long)g * a.rows + rg * (kSWaves * 32) + qsrow) * D : 0) + 8 * qq;
#pragma unroll
      for (int i = 0; i < 16; ++i) qraw[i] = *reinterpret_cast<const i32x4*>(qsrc + 32 * i);
    }
    wait_vmcnt<0>();
    // keys of tile t that exist (0 for a missing page) and its first cache
    // byte, for the tile's page id `page`
    auto tile_src = [&](int t, int page, int& valid) -> const uint8_t* {
      const bool ok = page_valid(page);
      valid = ok ? min(kKeys, sk - (u0 + t) * kKeys) : 0;
      return kv + (long)(ok ? page : 0) * kKeys * RB;
    };
    // per-token scales of tile t (dense: its page id) into ring slot bufi:
    // the k-scales by wave 1, the v-scales by wave 2, one 4-byte-per-lane copy
    // each. Keys that do not exist (a page's slack, a missing page, a skipped
    // sparse entry) get 0 instead of whatever the caller's array holds there,
    // so that the S-wave's P times v-scale needs no guard (0 times 0).
    constexpr bool kPtWave = PT;
    const bool pt_wave = kPtWave && (e == 1 || e == 2);
    auto issue_pt = [&](int t, int bufi, int page) {
      if constexpr (PT) {
        if (pt_wave) {
          const float* sc = e == 1 ? k_scale : v_scale;
          const float* zeros = reinterpret_cast<const float*>(kWsZeros);
          uint8_t* dst = reinterpret_cast<uint8_t*>(pt_base + bufi * 128 + (e == 2 ? 64 : 0));
          if constexpr (SPARSE) {
            const int cr = ws_sparse_row(sp_slot(t), fresh_lane(), sk, a.num_pages);
            load_lds4_gather(cr >= 0 ? sc + cr : zeros, dst);
          } else {
            const int valid = page_valid(page) ? min(kKeys, sk - (u0 + t) * kKeys) : 0;
            if (valid == kKeys) {
              load_lds4_row(sc + (long)page * kKeys, dst);
            } else {
              const int lk = fresh_lane();
              load_lds4_gather(lk < valid ? sc + (long)page * kKeys + lk : zeros, dst);
            }
          }
        }
      }
    };
    // tile 0 before the loop, tile 1 once tile 0 has landed (which keeps the
    // prologue's burst of query and tile loads small); then tile k+2 during
    // iteration k. Sparse: the first wave fills the lookup slots of tiles
    // 0..3 (indices) and 0..2 (pages) first, and tile 0 follows the barrier
    // that publishes them.
    if constexpr (SPARSE) {
      if (e == 0) {
        for (int t = 0; t < 4 && t < ntiles; ++t) sp_dma_index(t);
        wait_vmcnt<0>();
        for (int t = 0; t < 3 && t < ntiles; ++t) sp_dma_page(t);
        wait_vmcnt<0>();
      }
    } else if (ntiles > 0) {
      int valid;
      const int page0 = page_at(0);
      const uint8_t* src = tile_src(0, page0, valid);
      issue_pt(0, 0, page0);
      if constexpr (ROPE > 0) ws_issue_rope<ROPE>(lds, 0, src, valid, e);
      ws_issue_nope_slice<ROPE>(lds, 0, src, valid, e);
    }
    {
      uint2 codes[16];
      int qe = 0;
      if (q_any) qe = q_second ? quantize_q_quad_residual(qraw, codes) : quantize_q_quad(qraw, codes);
      const int nn = qrl & 31;
      uint8_t* dst = qstage(qrl >> 5) + nn * 512 + 8 * (qq & 1);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<uint2*>(dst + (((2 * i + (qq >> 1)) ^ nn) << 4)) = q_ok ? codes[i] : uint2{0u, 0u};
      if (qq == 0) qexp[qrl] = q_ok ? qe : 0;
    }
    __syncthreads();   // the quantized query rows are staged
    if constexpr (SPARSE) {
      if (ntiles > 0) {
        issue_pt(0, 0, 0);
        if constexpr (ROPE > 0) ws_issue_sparse_rope<ROPE>(lds, 0, kv, sp_slot(0), sk, a.num_pages, e);
        ws_issue_sparse_nope<ROPE>(lds, 0, kv, sp_slot(0), sk, a.num_pages, e);
      }
    }
    wait_vmcnt<0>();   // tile 0 has landed
    if constexpr (FNUZ) {
      if (ntiles > 0) ws_fnuz_to_ocp_slice(lds, 0, e);
    }
    if (ntiles > 1) {   // tile 1 must land by the end of iteration 0
      if constexpr (SPARSE) {
        issue_pt(1, 1, 0);
        if constexpr (ROPE > 0) ws_issue_sparse_rope<ROPE>(lds, 1, kv, sp_slot(1), sk, a.num_pages, e);
        ws_issue_sparse_nope<ROPE>(lds, 1, kv, sp_slot(1), sk, a.num_pages, e);
      } else {
        int valid1;
        const int page1 = page_at(1);
        const uint8_t* src1 = tile_src(1, page1, valid1);
        issue_pt(1, 1, page1);
        if constexpr (ROPE > 0) ws_issue_rope<ROPE>(lds, 1, src1, valid1, e);
        ws_issue_nope_slice<ROPE>(lds, 1, src1, valid1, e);
      }
    }

    // V^T lane base (slice layout): lane group g = lane / 16 reads chunk
    // 2 j + (g & 1) of dv block 2e + j, key 16 u + tk, tk = tr_key(sup / 2, h),
    // bytes 8 (sup & 1) .. +7 of the chunk (sup = lane % 16); block 2e + 1 is
    // block 2e's address ^ 32
    int vb;
    {
      const int sup = lane & 15, tk = tr_key(sup >> 1, h);
      vb = e * 4096 + tk * 64 + 16 * (((lane >> 4) & 1) ^ ((tk >> 2) & 3)) + 8 * (sup & 1);
    }

    // O^T accumulators: O[j][r] = dv block 2e + j of row block r (VGPRs)
    f32x16 O[2][kSWaves];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < kSWaves; ++r) O[j][r] = f32x16{};

    int bufp = 2;   // ring slot of tile k-1 (= slot of tile k+2)
    int page2 = SPARSE ? -1 : page_at(2);   // page id of tile k+2, loaded one iteration ahead
    for (int k = 0; k <= ntiles; ++k) {
      __syncthreads();   // tile k has landed in every wave's share
      const bool next2 = k + 2 < ntiles;
      int valid2 = 0;
      const uint8_t* src2 = nullptr;
      if constexpr (SPARSE) {
        // lookups one iteration ahead of their use, issued before this
        // iteration's copies so that the wait below covers them
        if (e == 0) {
          if (k + 3 < ntiles) sp_dma_page(k + 3);
          if (k + 4 < ntiles) sp_dma_index(k + 4);
        }
        if (next2) issue_pt(k + 2, bufp, 0);
        if constexpr (ROPE > 0) {
          if (next2) ws_issue_sparse_rope<ROPE>(lds, bufp, kv, sp_slot(k + 2), sk, a.num_pages, e);
        }
      } else if (next2) {
        src2 = tile_src(k + 2, page2, valid2);
        issue_pt(k + 2, bufp, page2);   // S^T(k-1) read the slot's scales before the barrier
        page2 = page_at(k + 3);
        if constexpr (ROPE > 0) ws_issue_rope<ROPE>(lds, bufp, src2, valid2, e);   // S^T(k-1) released it
      }
      i32x8 vr[2];
      if (k > 0) {
        const uint8_t* vnope = lds + bufp * kNopeRegion;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x2 v0 = lds_tr8(vnope, vb + 1024 * u);
          const i32x2 v1 = lds_tr8(vnope, (vb ^ 32) + 1024 * u);
          vr[0][2 * u] = v0.x;
          vr[0][2 * u + 1] = v0.y;
          vr[1][2 * u] = v1.x;
          vr[1][2 * u + 1] = v1.y;
        }
      }
      if (next2) {
        // this wave's slice of tile k-1 has been read: refill it with tile k+2
        if (k > 0) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vr[0]), "+v"(vr[1]) :: "memory");
        if constexpr (SPARSE) ws_issue_sparse_nope<ROPE>(lds, bufp, kv, sp_slot(k + 2), sk, a.num_pages, e);
        else ws_issue_nope_slice<ROPE>(lds, bufp, src2, valid2, e);
      }
      if (k > 0) {
        const int pp = (k - 1) & 1;
        const i32x4 fl = *reinterpret_cast<const i32x4*>(xflag + 4 * pp);
        const uint8_t* pprev = xp + pp * WsX::p_bytes;
        // rescale O for the rows whose max tile k-1 raised (rare), before its products
        if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
          asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
          const float* al = xalpha + pp * (kSWaves * 32);
#pragma unroll
          for (int r = 0; r < kSWaves; ++r) {
            if (__builtin_amdgcn_readfirstlane(fl[r])) {
              const float f = al[r * 32 + (fresh_lane() & 31)];
#pragma unroll
              for (int x = 0; x < 16; ++x) {
                O[0][r][x] *= f;
                O[1][r][x] *= f;
              }
            }
          }
          asm volatile("s_nop 4" ::: "memory");
        }
        const int lo16 = fresh_lane() * 16;
#pragma unroll
        for (int r = 0; r < kSWaves; ++r) {
          if (rg * kSWaves + r >= a.row_blocks) break;   // row blocks past the problem: nothing to add
          const i32x4 lo = lds_ld16(pprev, r * 2048 + lo16);
          const i32x4 hi = lds_ld16(pprev, r * 2048 + 1024 + lo16);
          const i32x8 pt = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          mfma_fp8_32x32x64(O[0][r], vr[0], pt);
          mfma_fp8_32x32x64(O[1][r], vr[1], pt);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // tile k+1 must have landed before the next barrier; tile k+2 may stay in
      // flight (sparse tiles always take kCopies instructions, plus the
      // per-token scale copy of waves 1 and 2)
      if (next2 && (SPARSE || valid2 == kKeys)) {
        if (pt_wave) wait_vmcnt<kCopies + 1>();
        else wait_vmcnt<kCopies>();
      } else {
        wait_vmcnt<0>();
      }
      if constexpr (FNUZ) {
        if (k + 1 < ntiles) ws_fnuz_to_ocp_slice(lds, (k + 1) % kBufs, e);
      }
      bufp = bufp == kBufs - 1 ? 0 : bufp + 1;
    }

    // ---- epilogue ----------------------------------------------------------------------
    __syncthreads();   // the S-waves' per-row scales are in LDS
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // last P.V MFMAs done
    if constexpr (SPLITP) {
      // O = O1 + O2 / 16 from columns n and n + 16 (row block 0 only)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const unsigned u = __float_as_uint(O[j][0][x]);
          const auto t = __builtin_amdgcn_permlane16_swap(u, u, false, false);
          O[j][0][x] = fmaf(__uint_as_float(t[1]), 0.0625f, __uint_as_float(t[0]));
        }
    }
    // O^T register x of block (j, r): dv 32 (2e + j) + 8 (x / 4) + 4 h + x % 4, row 32 rbr + n
#pragma unroll
    for (int r = 0; r < kSWaves; ++r) {
      const int rbr = rg * kSWaves + r;
      if (rbr >= a.row_blocks) break;
      const float inv = xfin[r * 32 + n];
      const int rowr = rbr * 32 + n;
      if (a.splits == 1) {
        if (rowr < a.rows) {
          uint16_t* orow = out + ((long)g * a.rows + rowr) * kNope;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int dv = 32 * (2 * e + j) + 8 * e4 + 4 * h;
              const f32x16& o = O[j][r];
              uint2 w;
              w.x = bf16x2_bits(o[4 * e4] * inv, o[4 * e4 + 1] * inv);
              w.y = bf16x2_bits(o[4 * e4 + 2] * inv, o[4 * e4 + 3] * inv);
              *reinterpret_cast<uint2*>(orow + dv) = w;
            }
        }
      } else {
        // partials in the accumulator's own register layout, as the combine reads them
        const long frag = ((long)s * a.groups + g) * a.row_blocks + rbr;
        uint16_t* po = part_o + frag * (16 * 64 * 16);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x16& o = O[j][r];
          i32x4* dst = reinterpret_cast<i32x4*>(po + ((2 * e + j) * 64 + lane) * 16);
#pragma unroll
          for (int e8 = 0; e8 < 2; ++e8) {
            i32x4 w;
#pragma unroll
            for (int d = 0; d < 4; ++d) w[d] = (int)half2_bits(o[8 * e8 + 2 * d] * inv, o[8 * e8 + 2 * d + 1] * inv);
            dst[e8] = w;
          }
        }
      }
    }
  }
}

// Gather check of the slice layout: one workgroup of eight waves per
// (sequence, page unit) runs the PV-waves' copies into slot 0 and writes the
// tile back in logical row order.
template <int ROPE>
__global__ __launch_bounds__(512) void debug_gather_ws_kernel(const uint8_t* kv, const int32_t* block_table,
                                                              const int32_t* seq_lens, int max_pages, int num_pages,
                                                              uint8_t* dense_out) {
  constexpr int RB = kNope + 2 * ROPE;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Tile<ROPE>::lds_bytes];
  const int e = wave_id();
  const int b = blockIdx.x / max_pages, unit = blockIdx.x % max_pages;
  int sk = seq_lens[b];
  sk = max(0, min(sk, max_pages * kKeys));
  const int page = block_table[(long)b * max_pages + unit];
  const bool page_ok = page >= 0 && page < num_pages;
  const int valid = page_ok ? max(0, min(kKeys, sk - unit * kKeys)) : 0;
  const uint8_t* src = kv + (long)(page_ok ? page : 0) * kKeys * RB;
  if constexpr (ROPE > 0) ws_issue_rope<ROPE>(lds, 0, src, valid, e);
  ws_issue_nope_slice<ROPE>(lds, 0, src, valid, e);
  wait_tile_and_sync();
  uint8_t* dst = dense_out + ((long)b * max_pages + unit) * kKeys * RB;
  for (int idx = threadIdx.x; idx < kKeys * (RB / 16); idx += 512) {
    const int r = idx / (RB / 16), c = idx % (RB / 16);
    const int off = c < 32 ? (c >> 2) * 4096 + r * 64 + 16 * ((c & 3) ^ ((r >> 2) & 3))
                           : kRopeBase + r * 128 + (swz_rope(r, c - 32) << 4);
    *reinterpret_cast<i32x4*>(dst + r * RB + c * 16) = lds_ld16(lds, off);
  }
}

hipError_t launch_debug_gather_ws(const uint8_t* kv, const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t batch, int32_t max_pages, int32_t num_pages, int32_t d_rope,
                                  uint8_t* dense_out, hipStream_t st) {
  const dim3 grid((unsigned)(batch * max_pages));
  if (d_rope == 64)
    hipLaunchKernelGGL((debug_gather_ws_kernel<64>), grid, dim3(512), 0, st, kv, block_table, seq_lens, max_pages,
                       num_pages, dense_out);
  else
    hipLaunchKernelGGL((debug_gather_ws_kernel<0>), grid, dim3(512), 0, st, kv, block_table, seq_lens, max_pages,
                       num_pages, dense_out);
  return hipGetLastError();
}

// Every fp8-dot decode runs here, at any row count: row blocks past the
// problem skip their work, and a one- or two-wave workgroup (the dv-split
// kernel, kept as a test variant) is slower even for a single 16-head token
// (tiny decode 17.5 -> 10 us). With at most 16 rows per key stream (a 16-head
// sparse token, a small dense decode) the half row block those rows leave free
// carries second terms: of the query (fp8 dots then multiply the exact bf16
// query), and for bf16 dots of P too. An e4m3fnuz cache keeps bf16 dots on the
// row-block kernel, which reads its codes exactly. The variant flags select
// the other kernels.
bool decode_ws_eligible(const DecodeLaunch& d) {
  if (d.rows_kernel || d.dv_split_kernel || d.gather_v) return false;
  return d.dot == DOT_FP8 || (d.rows <= 16 && !d.fnuz);
}

hipError_t launch_decode_ws(const DecodeLaunch& d, const KDims& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.groups * a.splits * a.row_groups));
#define MLA_WS_ARGS d.q, d.kv, d.block_table, d.seq_lens, d.indices, d.k_scale, d.v_scale, d.out, d.lse, d.part_o, d.part_lse
#define MLA_WS_LAUNCH(R, F, S, P, T) \
  hipLaunchKernelGGL((mla_decode_ws_kernel<R, F, S, P, T>), grid, dim3(kWsThreads), 0, st, MLA_WS_ARGS, a)
#define MLA_WS_ROPE(F, S, P, T) \
  if (d.d_rope == 64) MLA_WS_LAUNCH(64, F, S, P, T); else MLA_WS_LAUNCH(0, F, S, P, T)
#define MLA_WS_FP8(T)                                          \
  if (d.topk != 0) {                                           \
    if (d.per_token) { MLA_WS_ROPE(false, true, true, T); }    \
    else if (d.fnuz) { MLA_WS_ROPE(true, true, false, T); }    \
    else { MLA_WS_ROPE(false, true, false, T); }               \
  } else if (d.per_token) {                                    \
    MLA_WS_ROPE(false, false, true, T);                        \
  } else if (d.fnuz) {                                         \
    MLA_WS_ROPE(true, false, false, T);                        \
  } else {                                                     \
    MLA_WS_ROPE(false, false, false, T);                       \
  }
  if (d.dot != DOT_FP8) {   // bf16 dots, at most 16 rows, no fnuz
    if (d.topk != 0) {
      if (d.per_token) { MLA_WS_ROPE(false, true, true, 2); } else { MLA_WS_ROPE(false, true, false, 2); }
    } else {
      if (d.per_token) { MLA_WS_ROPE(false, false, true, 2); } else { MLA_WS_ROPE(false, false, false, 2); }
    }
  } else if (d.rows <= 16) {
    MLA_WS_FP8(1)
  } else {
    MLA_WS_FP8(0)
  }
#undef MLA_WS_FP8
#undef MLA_WS_ROPE
#undef MLA_WS_LAUNCH
#undef MLA_WS_ARGS
  return hipGetLastError();
}

}  // namespace mla

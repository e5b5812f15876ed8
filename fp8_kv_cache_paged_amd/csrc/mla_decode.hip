// FP8-KV paged MLA decode for gfx950 (MI355X / CDNA4).
//
// What is computed (FlashMLA PR #82 "update fp8 support", description; ROCm/aiter
// PR #6199, Technical details; InfiniCore PR #1568, Summary, paged attention):
// for each query row (token i of s_q, head h of h_q) of a sequence, softmax
// attention over that sequence's cached latent tokens, K = [e4m3fn nope *
// k_scale, bf16 rope], V = e4m3fn nope * v_scale, dv = 512, with the natural-log
// log-sum-exp. Split-KV partials are merged by a log-sum-exp combine
// (InfiniCore PR #1568, split-kv commit).
//
// gfx950 design (the pages' Hopper WGMMA/TMA and gfx942 Triton kernels are prior
// art only):
//  * One workgroup per (key stream, split, row group). All query rows of a
//    sequence (s_q * h_q, up to 128 per workgroup) share the key stream, so a
//    64-key tile is fetched from HBM once and contracted against every row.
//    Each wave owns 32 query rows.
//  * Paged gather: a tile is one page (64 rows of 640 B, contiguous in HBM),
//    moved by 16-byte global->LDS direct loads into a double-buffered LDS tile
//    while the previous tile computes (the pages' copy/compute pipelining idea,
//    FlashMLA PR #82, "Fine-grained optimization of the pipeline"). 16-byte
//    chunks are XOR-swizzled per row so that column reads are bank-conflict free.
//  * Orientation S^T = K Q^T on 32x32 MFMA: keys are the M dimension and query
//    rows the N dimension, so every lane holds one query row and 32 of the 64
//    keys. Row max and row sum are then per-lane plus one exchange with lane
//    l^32; P^T is packed straight from the accumulators into the B operand of
//    the P.V MFMA (no shared-memory round trip, which FlashMLA needed for its
//    rP -> sP -> rP copies).
//  * O^T = V^T P^T: the V^T operand is read from the same LDS bytes as K with
//    the gfx950 transposed LDS read (ds_read_b64_tr_b8); V is never fetched
//    from HBM a second time.
//  * fp8 dots: Q nope quantized in-kernel per row with a power-of-two scale,
//    v_mfma_scale_f32_32x32x64_f8f6f4 (OCP e4m3fn) for Q.K_nope and P.V, the
//    64 rope dims in bf16 (v_mfma_f32_32x32x16_bf16), as FlashMLA keeps rope in
//    BF16 tiles. P is taken against a lazily raised running max (p <= 2^3)
//    and scaled by 2^5 before e4m3fn quantization (values <= 256 < 448), so
//    the softmax tail does not flush to zero (ROCm/aiter PR #6199, P scale).
//    bf16 dots: cache bytes converted exactly to bf16, all products bf16 MFMA.
//  * Keys past a row's visible length are masked by select (never by
//    arithmetic) and rows past the sequence end are zero-filled in LDS, so
//    poisoned slack bytes cannot reach the MFMA (the pages' fill_oob_KV, done
//    per row at load time instead of with a synchronisation per tile).

#include "mla_device.h"

namespace mla {

// Decode with the P.V products split over the waves by row block: each wave
// owns 32 query rows end to end (S^T, softmax, P.V over all 512 dv). Used for
// bf16 dots, whose P^T operands are too large to exchange between waves.
// PT (per-token scales, as in the dv-split kernel): each tile copy also moves
// the 64 rows' k- and v-scales into LDS; the nope sums are multiplied by their
// key's k-scale, and p by its key's v-scale before the bf16 packing (bf16 has
// the range, so no reference scale is needed).
// FNUZ: the cache holds gfx942's e4m3fnuz codes (bf16 dots, per-tensor scales).
template <int DOT, int ROPE, bool SPARSE, int NW, bool GATHER_V, bool PT = false, bool FNUZ = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(1, 1)))
void mla_decode_rows_kernel(MLA_KERNEL_PTRS, KDims a) {
  static_assert(!(PT && DOT == DOT_FP8), "per-token scales with fp8 dots use the dv-split kernel");
  static_assert(!(FNUZ && (DOT == DOT_FP8 || PT || GATHER_V)), "fnuz codes: bf16 dots, per-tensor scales");
  constexpr int D = kNope + ROPE;               // q row length
  __shared__ __attribute__((aligned(1024))) uint8_t lds_[Tile<ROPE>::lds_bytes + (PT ? kBufs * 512 : 0)];
  uint8_t* const lds = lds_;
  uint8_t* const xs = lds + Tile<ROPE>::lds_bytes;   // PT: scales of ring buffer i at xs + 512 i

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;

  int bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int rg = bid % a.row_groups;
  bid /= a.row_groups;
  const int s = bid % a.splits;
  const int g = bid / a.splits;

  const int b = SPARSE ? g / a.s_q : g;
  int sk = seq_lens[b];
  sk = max(0, min(sk, a.max_pages * kKeys));
  const int units = SPARSE ? (a.topk + kKeys - 1) / kKeys : (sk + kKeys - 1) / kKeys;
  const int u0 = (int)((long)s * units / a.splits);
  const int u1 = (int)((long)(s + 1) * units / a.splits);
  const int ntiles = u1 - u0;

  const int rb = rg * NW + wave;              // row block of this wave
  const bool wave_active = rb < a.row_blocks;
  const int row = rb * 32 + n;
  const bool row_ok = row < a.rows;
  int row_len = 0;                            // dense: keys this row may see
  if constexpr (!SPARSE) {
    const int i = row / a.h_q;
    row_len = a.causal ? sk - (a.s_q - 1 - i) : sk;
    if (!row_ok) row_len = 0;
  }
  const long qrow_idx = (long)g * a.rows + row;
  const uint16_t* qrow = q + qrow_idx * D;

  const int32_t* bt_row = block_table + (long)b * a.max_pages;
  const int32_t* idx_row = SPARSE ? indices + (long)g * a.topk : nullptr;
  constexpr long RB = kNope + 2 * ROPE;

  // Sparse entry e's index, the page it falls in and its cache row (page * 64
  // + slot, -1 when skipped): three steps, so that a pipeline can give each
  // dependent load a whole tile iteration.
  auto sparse_entry = [&](int e) -> int { return e < a.topk ? idx_row[e] : -1; };
  auto sparse_page = [&](int j) -> int { return j >= 0 && j < sk ? bt_row[j / kKeys] : -1; };
  auto sparse_cache_row = [&](int j, int page) -> int {
    return j >= 0 && j < sk && page >= 0 && page < a.num_pages ? page * kKeys + (j % kKeys) : -1;
  };
  // Dense: one page per tile. Inside the tile loop page ids come from a
  // register holding 64 of them (lane i: tile 64c + i of the split), read with
  // v_readlane: a scalar load there would share the counter of the LDS
  // fragment reads and, completing out of order, force them to full waits.
  auto page_of = [&](int unit) -> int { return unit < u1 ? bt_row[unit] : -1; };
  auto page_of_lane = [&](int unit) -> int { return unit < u1 ? bt_row[unit] : -1; };
  int pages_v = -1;
  auto page_valid = [&](int page) -> bool { return page >= 0 && page < a.num_pages; };
  auto issue_dense = [&](int unit, int page, int bufi) {
    const bool ok = page_valid(page);
    const int valid = ok ? min(kKeys, sk - unit * kKeys) : 0;
    if constexpr (PT) {
      if (ok) {
        if (wave == 0) load_lds4_row(k_scale + (long)page * kKeys, xs + bufi * 512);
        if (wave == (NW > 1 ? 1 : 0)) load_lds4_row(v_scale + (long)page * kKeys, xs + bufi * 512 + 256);
      }
    }
    issue_dense_tile<ROPE, NW>(lds, bufi, kv + (long)(ok ? page : 0) * kKeys * RB, valid, lane, wave);
  };
  auto issue_sparse_scales = [&](int row, int bufi) {
    if constexpr (PT && SPARSE) {
      const long r = row >= 0 ? row : 0;   // a skipped entry's key is masked
      if (wave == 0) load_lds4_gather(k_scale + r, xs + bufi * 512);
      if (wave == (NW > 1 ? 1 : 0)) load_lds4_gather(v_scale + r, xs + bufi * 512 + 256);
    }
  };

  // Dense tiles are loaded two ahead (tiles k+1 and k+2 land while tile k
  // computes); sparse tiles one ahead.
  int page_cur = -1, page_next = -1, page_next2 = -1;   // dense
  int row_cur = -1, row_next = -1;                      // sparse: this lane's tile row
  // sparse: at the top of iteration k, j_b and pg_b are this lane's entry of
  // tile k+1 and the page it falls in, j_c its entry of tile k+2 (each index
  // and page-table load has a whole iteration to land)
  int j_b = -1, pg_b = -1, j_c = -1;
  if (ntiles > 0) {
    if constexpr (SPARSE) {
      const int j0 = sparse_entry(u0 * kKeys + lane);
      if (ntiles > 1) j_b = sparse_entry((u0 + 1) * kKeys + lane);
      if (ntiles > 2) j_c = sparse_entry((u0 + 2) * kKeys + lane);
      const int pg0 = sparse_page(j0);
      pg_b = sparse_page(j_b);
      row_cur = sparse_cache_row(j0, pg0);
      issue_sparse_scales(row_cur, 0);
      issue_sparse_tile<ROPE, NW>(lds, 0, kv, row_cur, lane, wave);
    } else {
      page_cur = page_of(u0);
      page_next = page_of(u0 + 1);
      issue_dense(u0, page_cur, 0);
      if (ntiles > 1) issue_dense(u0 + 1, page_next, 1);
    }
  }

  // Q fragments (B operand of S^T = K Q^T).
  i32x8 qn[DOT == DOT_FP8 ? 8 : 1];
  bf16x8 qb[DOT == DOT_BF16 ? 32 : 1];
  bf16x8 qr[ROPE > 0 ? 4 : 1];
  float qk_scale;   // q_scale * k_scale, applied to the nope accumulator
  {
    const float ks = PT ? 1.f : *k_scale;   // PT: k-scales apply per key
    if constexpr (DOT == DOT_FP8) {
      int e;
      stage_q_fp8(qrow, row_ok && wave_active, h, qn, e);
      qk_scale = ldexpf(ks, e);
    } else {
      qk_scale = FNUZ ? ldexpf(ks, kFnuzExp) : ks;   // fnuz codes decode to 2^-119 times their value
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int d0 = 32 * (u >> 1) + 16 * h + 8 * (u & 1);
        i32x4 v = row_ok ? *reinterpret_cast<const i32x4*>(qrow + d0) : i32x4{0, 0, 0, 0};
        qb[u] = __builtin_bit_cast(bf16x8, v);
      }
    }
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        i32x4 v = row_ok ? *reinterpret_cast<const i32x4*>(qrow + kNope + 16 * t + 8 * h)
                         : i32x4{0, 0, 0, 0};
        qr[t] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  // All query loads are complete before the tile loop: the tile copies are
  // inline asm the compiler does not count, and without this it would wait
  // for every outstanding copy before the first use of a query register in
  // each tile.
  if constexpr (!SPARSE) pages_v = page_of_lane(u0 + lane);
  wait_vmcnt<0>();
  asm volatile("" : "+v"(pages_v));   // loaded before the loop, not inside it

  // sparse: the fragment bases are recomputed every tile from a fresh lane id
  // (kept across the loop next to the sparse variant's state they spill)
  LdsBases lb(lane);

  f32x16 O[16];
#pragma unroll
  for (int blk = 0; blk < 16; ++blk) O[blk] = f32x16{};
  float m_run = -INFINITY;   // max used for the exponentials (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum

  int buf = 0;   // k % kBufs
  for (int k = 0; k < ntiles; ++k) {
    // Tile k has landed once at most one later tile's loads are outstanding;
    // the barrier then also frees the buffer of tile k-1 for tile k+2.
    if constexpr (SPARSE) {
      wait_vmcnt<0>();
    } else {
      if (k + 1 < ntiles) wait_vmcnt<Tile<ROPE>::template loads_per_wave<NW>()>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    const int buf_next = buf == kBufs - 1 ? 0 : buf + 1;
    const int buf_next2 = buf_next == kBufs - 1 ? 0 : buf_next + 1;
    if constexpr (SPARSE) {
      lb = LdsBases(lane_id_fresh());
      if (k + 1 < ntiles) {
        row_next = sparse_cache_row(j_b, pg_b);   // both landed by the wait above
        issue_sparse_scales(row_next, buf_next);
        issue_sparse_tile<ROPE, NW>(lds, buf_next, kv, row_next, lane, wave);
        j_b = j_c;
        pg_b = sparse_page(j_b);
        j_c = k + 3 < ntiles ? sparse_entry((u0 + k + 3) * kKeys + lane) : -1;
      }
    } else {
      if (k + 2 < ntiles) {
        const int t2 = k + 2;
        if ((t2 & 63) == 0) {   // next 64 page ids (tile loops longer than 64 tiles)
          pages_v = page_of_lane(u0 + t2 + lane);
          wait_vmcnt<0>();
        }
        page_next2 = __builtin_amdgcn_readlane(pages_v, t2 & 63);
        issue_dense(u0 + t2, page_next2, buf_next2);
      }
    }
    // A wave whose row block lies past the last row (ragged row counts) runs
    // the same code on zero queries and only skips the stores: a second loop
    // path around the accumulators makes the register allocator shuffle them.
    const uint8_t* nope = lds + buf * kNopeRegion;
    const uint8_t* rope = lds + kRopeBase + buf * kRopeRegion;
    const int unit = u0 + k;

    // ---- S^T = K Q^T -------------------------------------------------------
    // The fragment reads of a tile run through a ring several items deep, so
    // about ten LDS reads are in flight while the MFMAs consume earlier ones
    // (one wave per SIMD: nothing else hides the LDS latency). Items alternate
    // between the two 32-key blocks, so consecutive MFMAs are independent. The
    // rope products have accumulators of their own, since q_scale * k_scale
    // applies to the nope products only; both are combined in the softmax.
    // Scheduling barriers keep the compiler from hoisting the whole tile's
    // fragment reads (which would need up to 160 more registers).
    // (bf16 dots: the 128 registers of bf16 query fragments leave no room for
    // separate rope accumulators; there the nope sums are scaled in place
    // before the rope products are added to them.)
    constexpr bool kSepRope = DOT == DOT_FP8 && ROPE > 0;
    f32x16 Sn[2], Sr[2];
    if constexpr (!kSepRope) Sr[0] = Sr[1] = f32x16{};
    if constexpr (DOT == DOT_FP8) {
      constexpr int NN = 16, NI = NN + (ROPE > 0 ? 8 : 0), PD = 5;
      i32x4 rl[PD], rh[PD];
      auto load = [&](int f) {
        const int slot = f % PD, kb = f & 1;
        if (f < NN) {
          const int t = f >> 1;
          const int c = 32 * kb * kNope + 256 * (t >> 2);
          rl[slot] = lds_ld16(nope, lb.k8[t & 3][0] + c);
          rh[slot] = lds_ld16(nope, lb.k8[t & 3][1] + c);
        } else {
          rl[slot] = lds_ld16(rope, lb.rp[(f - NN) >> 1] + 32 * kb * 128);
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
          if (f < 2) mfma_fp8_32x32x64_first(Sn[kb], kf, qn[f >> 1]);
          else mfma_fp8_32x32x64(Sn[kb], kf, qn[f >> 1]);
        } else {
          const bf16x8 kr = __builtin_bit_cast(bf16x8, lo);
          if (f < NN + 2) mfma_bf16_32x32x16_first(Sr[kb], kr, qr[(f - NN) >> 1]);
          else mfma_bf16_32x32x16(Sr[kb], kr, qr[(f - NN) >> 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // bf16 dots: each 16-byte fp8 read becomes two bf16 A operands.
      constexpr int NN = 32, NI = NN + (ROPE > 0 ? 8 : 0), PD = 3;
      i32x4 rl[PD];
      auto load = [&](int f) {
        const int kb = f & 1;
        if (f < NN) {
          const int t = f >> 1;
          rl[f % PD] = lds_ld16(nope, lb.k16[t & 7] + 32 * kb * kNope + 256 * (t >> 3));
        } else {
          rl[f % PD] = lds_ld16(rope, lb.rp[(f - NN) >> 1] + 32 * kb * 128);
        }
      };
#pragma unroll
      for (int f = 0; f < PD; ++f) load(f);
#pragma unroll
      for (int f = 0; f < NI; ++f) {
        const int kb = f & 1;
        const i32x4 raw = rl[f % PD];
        if (f + PD < NI) load(f + PD);
        if (f < NN) {
          const int t = f >> 1;
          const i32x2 b0 = kv_bytes_to_bf16x4<FNUZ>(raw.x), b1 = kv_bytes_to_bf16x4<FNUZ>(raw.y);
          const i32x2 b2 = kv_bytes_to_bf16x4<FNUZ>(raw.z), b3 = kv_bytes_to_bf16x4<FNUZ>(raw.w);
          const bf16x8 a0 = __builtin_bit_cast(bf16x8, i32x4{b0.x, b0.y, b1.x, b1.y});
          const bf16x8 a1 = __builtin_bit_cast(bf16x8, i32x4{b2.x, b2.y, b3.x, b3.y});
          if (f < 2) mfma_bf16_pair_first_after_valu(Sn[kb], a0, qb[2 * t], a1, qb[2 * t + 1]);
          else mfma_bf16_pair_after_valu(Sn[kb], a0, qb[2 * t], a1, qb[2 * t + 1]);
        } else {
          const bf16x8 kr = __builtin_bit_cast(bf16x8, raw);
          if (f < NN + 2) mfma_bf16_32x32x16_after_valu(Sn[kb], kr, qr[(f - NN) >> 1]);
          else mfma_bf16_32x32x16(Sn[kb], kr, qr[(f - NN) >> 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ROPE > 0 && f == NN - 1) {
          s_nop_result2(Sn[0], Sn[1]);
          if constexpr (PT) {
            // key of register r of block kb: 32 kb + 8 j + 4 ((j + h) & 1) + (r & 3), j = r / 4
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const f32x4 ksv = *reinterpret_cast<const f32x4*>(xs + buf * 512 + 4 * (32 * kb + 8 * j + 4 * ((j + h) & 1)));
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Sn[kb][4 * j + rr] *= qk_scale * ksv[rr];
              }
          } else {
            Sn[0] *= qk_scale;
            Sn[1] *= qk_scale;
          }
        }
      }
    }
    if constexpr (kSepRope) s_nop_result4(Sn[0], Sn[1], Sr[0], Sr[1]);
    else s_nop_result2(Sn[0], Sn[1]);

    // ---- mask + online softmax (log2 domain) --------------------------------
    // Tile-wide visibility: a tile every row of the workgroup sees in full
    // skips the per-element mask (all but the last tile of a sequence).
    bool full;
    int limit = 0;    // dense: keys of this tile this lane's row may see
    unsigned long long smask = 0;
    if constexpr (SPARSE) {
      smask = __ballot(row_cur >= 0);
      full = smask == ~0ull;
    } else {
      const bool page_ok = page_valid(page_cur);
      full = page_ok && (unit + 1) * kKeys <= sk - (a.causal ? a.s_q - 1 : 0);
      limit = page_ok ? row_len - unit * kKeys : 0;
    }
    const float cn = qk_scale * a.sm_log2;
    f32x16 S[2];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = r >> 2;
        const int key = 32 * kb + 8 * j + 4 * ((j + h) & 1) + (r & 3);
        bool valid;
        if constexpr (SPARSE) valid = (smask >> key) & 1ull;
        else valid = key < limit;
        float zs;
        if constexpr (kSepRope) zs = fmaf(Sn[kb][r], cn, Sr[kb][r] * a.sm_log2);
        else if constexpr (ROPE > 0) zs = Sn[kb][r] * a.sm_log2;   // bf16: scaled already
        else if constexpr (PT) {
          const int j = r >> 2;
          zs = Sn[kb][r] * cn * reinterpret_cast<const float*>(xs + buf * 512)[32 * kb + 8 * j + 4 * ((j + h) & 1) + (r & 3)];
        } else zs = Sn[kb][r] * cn;
        const float z = (full || valid) ? zs : -INFINITY;
        S[kb][r] = z;
        mx = fmaxf(mx, z);
      }
    }
    mx = pair_max(mx);
    __builtin_amdgcn_sched_barrier(0);

    // The first V^T fragments of the P.V products are read now, so they are
    // in registers when the exponentials are done (issued after the row-max
    // exchange, whose own LDS access would otherwise wait for them).
    constexpr int PDV = DOT == DOT_FP8 ? 3 : 2;
    i32x8 vr[PDV];
    auto vfrag = [&](int blk) -> i32x8 {
      i32x8 av;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x2 v = vt_bytes<GATHER_V>(nope, lane, blk, u, lb.vt[blk & 7]);
        av[2 * u] = v.x;
        av[2 * u + 1] = v.y;
      }
      return av;
    };
    // (bf16 dots: no early reads; their query fragments leave too few
    // registers to hold V^T fragments across the softmax.)
    if constexpr (DOT == DOT_FP8) {
#pragma unroll
      for (int blk = 0; blk < PDV; ++blk) vr[blk] = vfrag(blk);
    }
    __builtin_amdgcn_sched_barrier(0);

    const bool raise = mx > m_run + Soft<DOT>::tau;
    if (__ballot(raise)) {
      const float m_new = raise ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
      l_run *= alpha;
      if (__ballot(raise && m_run != -INFINITY)) {
        // The previous tile's P.V MFMAs finished before this tile's S^T
        // results were read (one in-order MFMA pipeline, s_nop_result4).
#pragma unroll
        for (int blk = 0; blk < 16; ++blk) scale_agpr_acc(O[blk], alpha);
        asm volatile("s_nop 4" ::);
      }
      m_run = m_new;
    }
    const float m_exp = ((m_run == -INFINITY) ? 0.f : m_run) - Soft<DOT>::ps_log2;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(S[kb][r] - m_exp);
        S[kb][r] = p;
        psum += p;
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T ---------------------------------------------------------
    if constexpr (DOT == DOT_FP8) {
      i32x8 pb;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kb = q >> 2, r0 = 4 * (q & 3);
        pb[q] = f32x4_to_fp8x4(S[kb][r0], S[kb][r0 + 1], S[kb][r0 + 2], S[kb][r0 + 3]);
      }
#pragma unroll
      for (int blk = 0; blk < 16; ++blk) {
        const i32x8 cur = vr[blk % PDV];
        if (blk + PDV < 16) vr[blk % PDV] = vfrag(blk + PDV);
        if (blk == 0) mfma_fp8_32x32x64_acc_after_valu(O[blk], cur, pb);   // pb was just written by VALU
        else if (blk == 15) mfma_fp8_32x32x64_acc_last(O[blk], cur, pb);
        else mfma_fp8_32x32x64_acc(O[blk], cur, pb);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if constexpr (PT) {
        // p times its key's v-scale; masked keys (p = 0) skip the scale
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 vsv = *reinterpret_cast<const f32x4*>(xs + buf * 512 + 256 + 4 * (32 * kb + 8 * j + 4 * ((j + h) & 1)));
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const float p = S[kb][4 * j + rr];
              S[kb][4 * j + rr] = p > 0.f ? p * vsv[rr] : 0.f;
            }
          }
      }
      bf16x8 pb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb = u >> 1, r0 = 8 * (u & 1);
        i32x4 w;
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = (int)bf16x2_bits(S[kb][r0 + 2 * d], S[kb][r0 + 2 * d + 1]);
        pb[u] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int blk = 0; blk < PDV; ++blk) vr[blk] = vfrag(blk);
#pragma unroll
      for (int blk = 0; blk < 16; ++blk) {
        const i32x8 cur = vr[blk % PDV];
        if (blk + PDV < 16) vr[blk % PDV] = vfrag(blk + PDV);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x2 lo = kv_bytes_to_bf16x4<FNUZ>(cur[2 * u]), hi = kv_bytes_to_bf16x4<FNUZ>(cur[2 * u + 1]);
          const bf16x8 av = __builtin_bit_cast(bf16x8, i32x4{lo.x, lo.y, hi.x, hi.y});
          if (blk == 15 && u == 3) mfma_bf16_32x32x16_acc_last(O[blk], av, pb[u]);
          else mfma_bf16_32x32x16_acc(O[blk], av, pb[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    page_cur = page_next;
    page_next = page_next2;
    row_cur = row_next;
    buf = buf_next;
  }

  if (!wave_active) return;
  // The epilogue reads O with VALU: wait for the last P.V MFMAs.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]), "+a"(O[6]), "+a"(O[7]),
                 "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]), "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));

  // ---- epilogue -----------------------------------------------------------------
  // O^T register r of block blk is dv 32*blk + 8*(r/4) + 4*h + r%4 of row n.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool nonempty = l_tot > 0.f;
  // splits == 1: the output, scaled by v_scale; else the partials, normalized
  // by the row sum only (fp16, |value| <= 448; the combine applies v_scale)
  // (fnuz: V decoded to 2^-119 times its value, restored here). Per-token
  // scales: O carries the scales already; partials are stored over a power of
  // two near the row's largest value (|value| <= 1), kept beside the lse.
  float inv = nonempty ? ldexpf(PT ? 1.f : (a.splits == 1 ? *v_scale : 1.f), FNUZ ? kFnuzExp : 0) / l_tot : 0.f;
  float row_scale = 1.f;
  if (PT && a.splits > 1) {
    float mx = 0.f;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(O[blk][r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * inv;
    if (mx > 0.f && mx <= 3.0e38f) {
      int e;
      frexpf(mx, &e);             // mx = f * 2^e, 0.5 <= f < 1
      row_scale = ldexpf(1.f, e);
      inv = ldexpf(inv, -e);
    }
  }
  const float lse2 = nonempty ? m_run + log2f(l_tot) - Soft<DOT>::ps_log2 : -INFINITY;

  if (a.splits == 1) {
    if (!row_ok) return;
    uint16_t* orow = out + qrow_idx * kNope;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dv = 32 * blk + 8 * j + 4 * h;
        uint2 w;
        w.x = bf16x2_bits(O[blk][4 * j] * inv, O[blk][4 * j + 1] * inv);
        w.y = bf16x2_bits(O[blk][4 * j + 2] * inv, O[blk][4 * j + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dv) = w;
      }
    }
    if (h == 0) lse[qrow_idx] = nonempty ? lse2 * kLn2 : -INFINITY;
  } else {
    // partials in the accumulator's own register layout (two 16-byte stores
    // per lane and block); the combine kernel reads the same layout.
    const long frag = ((long)s * a.groups + g) * a.row_blocks + rb;
    uint16_t* po = part_o + frag * (16 * 64 * 16);
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
      i32x4* dst = reinterpret_cast<i32x4*>(po + (blk * 64 + lane) * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        i32x4 w;
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = (int)half2_bits(O[blk][8 * j + 2 * d] * inv, O[blk][8 * j + 2 * d + 1] * inv);
        dst[j] = w;
      }
    }
    if (h == 0) {
      part_lse[frag * 32 + n] = lse2;
      if (PT) part_row_scale(part_lse, a)[frag * 32 + n] = row_scale;
    }
  }
}

// LDS past the KV ring: what the waves exchange between the S^T products
// (one 32-row block per wave) and the P.V products (one slice of dv per wave,
// all row blocks), double-buffered by tile parity:
//  * P^T operands of a tile, 2 KiB per row block, stored as two 16-byte
//    halves per lane (lane-contiguous, so conflict free);
//  * per-row rescale factors and one flag per row block saying whether any
//    of its rows raised its running max (and so carries factors);
//  * at the end, the per-row output scale 1 / l.
template <int NW>
struct Xchg {
  static constexpr int p_bytes = NW * 2048;
  static constexpr int alpha_bytes = NW * 32 * 4;
  static constexpr int flag_off = 2 * p_bytes + 2 * alpha_bytes;   // 2 x 4 ints
  static constexpr int fin_off = flag_off + 32;
  static constexpr int bytes = fin_off + NW * 32 * 4;
};

// fp8-dot decode with the P.V products split over the waves by dv: wave w
// multiplies the dv slice w of V^T with the P^T of every row block of the
// workgroup, so each wave reads 1/NW of V from LDS instead of all of it (the
// transposing V reads are the costliest LDS traffic of a tile). The S^T
// products and the softmax stay with the wave that owns the row block; P^T
// and the rescale factors cross through LDS, one tile behind.
// PT (per-token scales): k_scale and v_scale hold one value per cache row
// ([num_pages, 64]). Each tile copy then also moves the page's 64 k- and 64
// v-scales into LDS; the softmax multiplies each nope sum by its key's
// k-scale, and each p by its key's v-scale over V_ref, the split's largest
// v-scale (so P stays within e4m3fn's range); O is scaled by V_ref at the end.
template <int DOT, int ROPE, bool SPARSE, int NW, bool GATHER_V, bool PT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(MLA_KERNEL_PTRS, KDims a) {
  static_assert(DOT == DOT_FP8, "the dv-split kernel is for fp8 dots");
  constexpr int D = kNope + ROPE;               // q row length
  constexpr int kJ = 16 / NW;                   // 32-wide dv blocks per wave in P.V
  using X = Xchg<NW>;
  constexpr int kScaleBytes = PT ? kBufs * 512 : 0;   // per ring buffer: 64 k-, 64 v-scales
  __shared__ __attribute__((aligned(1024))) uint8_t lds_[Tile<ROPE>::lds_bytes + X::bytes + kScaleBytes];
  uint8_t* const lds = lds_;
  uint8_t* const xp = lds + Tile<ROPE>::lds_bytes;
  uint8_t* const xs = xp + X::bytes;            // PT: scales of ring buffer i at xs + 512 i
  float* const xalpha = reinterpret_cast<float*>(xp + 2 * X::p_bytes);
  int* const xflag = reinterpret_cast<int*>(xp + X::flag_off);
  float* const xfin = reinterpret_cast<float*>(xp + X::fin_off);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;

  int bid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int rg = bid % a.row_groups;
  bid /= a.row_groups;
  const int s = bid % a.splits;
  const int g = bid / a.splits;

  const int rb = rg * NW + wave;              // row block of this wave's S^T products
  const bool wave_active = rb < a.row_blocks;
  const int row = rb * 32 + n;
  const bool row_ok = row < a.rows;
  const long qrow_idx = (long)g * a.rows + row;
  const uint16_t* qrow = q + qrow_idx * D;

  // The query loads go out first: they depend on nothing else, and their
  // latency then overlaps the dependent loads (sequence length, page table)
  // that precede the first tile's copies.
  // (rows outside the problem read row 0 and are zeroed after quantization)
  const bool q_ok = row_ok && wave_active;
  const uint16_t* qsrc = q_ok ? qrow : q;
  i32x4 qraw[8][4];
  i32x4 qr_raw[ROPE > 0 ? 4 : 1];
  load_q_nope_raw(qsrc, h, qraw);
  if constexpr (ROPE > 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) qr_raw[t] = *reinterpret_cast<const i32x4*>(qsrc + kNope + 16 * t + 8 * h);
  }

  const int b = SPARSE ? g / a.s_q : g;
  int sk = seq_lens[b];
  sk = max(0, min(sk, a.max_pages * kKeys));
  const int units = SPARSE ? (a.topk + kKeys - 1) / kKeys : (sk + kKeys - 1) / kKeys;
  const int u0 = (int)((long)s * units / a.splits);
  const int u1 = (int)((long)(s + 1) * units / a.splits);
  const int ntiles = u1 - u0;

  int row_len = 0;                            // dense: keys this row may see
  if constexpr (!SPARSE) {
    const int i = row / a.h_q;
    row_len = a.causal ? sk - (a.s_q - 1 - i) : sk;
    if (!row_ok) row_len = 0;
  }
  const int32_t* bt_row = block_table + (long)b * a.max_pages;
  const int32_t* idx_row = SPARSE ? indices + (long)g * a.topk : nullptr;
  constexpr long RB = kNope + 2 * ROPE;

  // Cache row (page * 64 + slot) of sparse entry `e`, or -1 when skipped.
  auto sparse_row = [&](int e) -> int {
    int cr = -1;
    if (e < a.topk) {
      const int j = idx_row[e];
      if (j >= 0 && j < sk) {
        const int page = bt_row[j / kKeys];
        if (page >= 0 && page < a.num_pages) cr = page * kKeys + (j % kKeys);
      }
    }
    return cr;
  };
  // The same in three steps, for a pipeline that gives each dependent load a
  // whole tile iteration: the entry, the page it falls in, the cache row.
  auto sparse_entry = [&](int e) -> int { return e < a.topk ? idx_row[e] : -1; };
  auto sparse_page = [&](int j) -> int { return j >= 0 && j < sk ? bt_row[j / kKeys] : -1; };
  auto sparse_cache_row = [&](int j, int page) -> int {
    return j >= 0 && j < sk && page >= 0 && page < a.num_pages ? page * kKeys + (j % kKeys) : -1;
  };
  // Dense: one page per tile. Inside the tile loop page ids come from a
  // register holding 64 of them (lane i: tile 64c + i of the split), read with
  // v_readlane: a scalar load there would share the counter of the LDS
  // fragment reads and, completing out of order, force them to full waits.
  auto page_of = [&](int unit) -> int { return unit < u1 ? bt_row[unit] : -1; };
  auto page_of_lane = [&](int unit) -> int { return unit < u1 ? bt_row[unit] : -1; };
  int pages_v = -1;
  auto page_valid = [&](int page) -> bool { return page >= 0 && page < a.num_pages; };
  // PT: the page's 64 k-scales (wave 0) and 64 v-scales (wave 1, or 0) go
  // to the scale slot of ring buffer bufi. A missing page moves none: its
  // keys are masked, and every use of a scale is guarded by that mask.
  auto issue_scales = [&](int page, int bufi) {
    if constexpr (PT) {
      if (page_valid(page)) {
        if (wave == 0) load_lds4_row(k_scale + (long)page * kKeys, xs + bufi * 512);
        if (wave == (NW > 1 ? 1 : 0)) load_lds4_row(v_scale + (long)page * kKeys, xs + bufi * 512 + 256);
      }
    }
  };
  // PT, sparse: tile row l's scales (row = cache row of entry l, -1 when
  // skipped: then row 0, whose key is masked) to the slot of ring buffer bufi.
  auto issue_sparse_scales = [&](int row, int bufi) {
    if constexpr (PT && SPARSE) {
      const long r = row >= 0 ? row : 0;
      if (wave == 0) load_lds4_gather(k_scale + r, xs + bufi * 512);
      if (wave == (NW > 1 ? 1 : 0)) load_lds4_gather(v_scale + r, xs + bufi * 512 + 256);
    }
  };
  auto issue_dense = [&](int unit, int page, int bufi) {
    const bool ok = page_valid(page);
    const int valid = ok ? min(kKeys, sk - unit * kKeys) : 0;
    issue_scales(page, bufi);
    issue_dense_tile<ROPE, NW>(lds, bufi, kv + (long)(ok ? page : 0) * kKeys * RB, valid, lane, wave);
  };

  // Tiles are loaded one ahead: tile k+1 lands while tile k computes.
  int page_cur = -1, page_next = -1;          // dense
  int row_cur = -1, row_next = -1;            // sparse: this lane's tile row
  // sparse: at the top of iteration k, j_b and pg_b are this lane's entry of
  // tile k+1 and the page it falls in, j_c its entry of tile k+2: every index
  // and page-table load has a whole iteration to land, so the copies of tile
  // k+1 go out without a dependent load in front of them
  int j_b = -1, pg_b = -1, j_c = -1;
  if (ntiles > 0) {
    if constexpr (SPARSE) {
      const int j0 = sparse_entry(u0 * kKeys + lane);
      if (ntiles > 1) j_b = sparse_entry((u0 + 1) * kKeys + lane);
      if (ntiles > 2) j_c = sparse_entry((u0 + 2) * kKeys + lane);
      const int pg0 = sparse_page(j0);
      pg_b = sparse_page(j_b);
      row_cur = sparse_cache_row(j0, pg0);
      issue_sparse_scales(row_cur, 0);
      issue_sparse_tile<ROPE, NW>(lds, 0, kv, row_cur, lane, wave);
    } else {
      page_cur = page_of(u0);
      issue_dense(u0, page_cur, 0);
    }
  }

  // The first iteration's P.V step (for the non-existent tile -1) runs on
  // zeros: P^T of parity 1 and the V region of ring buffer 2 (which tile 2
  // only overwrites after the next barrier), and no rescale flags.
  {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kNopeRegion / (NW * 1024); ++i)
      *reinterpret_cast<i32x4*>(lds + 2 * kNopeRegion + (i * NW * 64 + t) * 16) = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<i32x4*>(xp + X::p_bytes + (i * NW * 64 + t) * 16) = i32x4{0, 0, 0, 0};
    if (t < 8) xflag[t] = 0;
  }

  // Q fragments (B operand of S^T = K Q^T), quantized from the raw values
  // loaded at entry.
  i32x8 qn[8];
  bf16x8 qr[ROPE > 0 ? 4 : 1];
  float qk_scale;   // q_scale * k_scale, applied to the nope products
  {
    int e;
    quantize_q_fp8(qraw, qn, e);
    qk_scale = ldexpf(PT ? 1.f : *k_scale, e);   // PT: k-scales apply per key
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int d = 0; d < 8; ++d) qn[t][d] = q_ok ? qn[t][d] : 0;
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        i32x4 v = qr_raw[t];
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = q_ok ? v[d] : 0;
        qr[t] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  // All query loads are complete before the tile loop: the tile copies are
  // inline asm the compiler does not count, and without this it would wait
  // for every outstanding copy before the first use of a query register in
  // each tile.
  if constexpr (!SPARSE) pages_v = page_of_lane(u0 + lane);
  wait_vmcnt<0>();
  asm volatile("" : "+v"(pages_v));   // loaded before the loop, not inside it

  // PT: V_ref = the largest v-scale of the split's valid rows (1 if none).
  float vref = 1.f, inv_vref = 1.f;
  if constexpr (PT) {
    float vm = 0.f;
    if constexpr (SPARSE) {
      // the rows the split's index entries name (lane l: entry 64 t + l)
      for (int t = 0; t < ntiles; ++t) {
        const int row = sparse_row((u0 + t) * kKeys + lane);
        if (row >= 0) vm = fmaxf(vm, v_scale[row]);
      }
    } else {
      for (int c = 0; c < ntiles; c += 64) {
        const int pg = c + lane < ntiles ? bt_row[u0 + c + lane] : -1;
        for (int t = 0; t < 64 && c + t < ntiles; ++t) {
          const int page = __builtin_amdgcn_readlane(pg, t);
          if (page_valid(page)) {
            const int valid = min(kKeys, sk - (u0 + c + t) * kKeys);
            if (lane < valid) vm = fmaxf(vm, v_scale[(long)page * kKeys + lane]);
          }
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) vm = fmaxf(vm, __shfl_xor(vm, o));
    vm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, vm)));
    if (vm > 0.f) {
      vref = vm;
      inv_vref = 1.f / vm;
    }
    wait_vmcnt<0>();
  }

  const LdsBases lb(lane);
  // V^T lane bases of this wave's dv blocks (block wave * kJ + j, j < kJ)
  int vtw[kJ < 8 ? kJ : 8];
#pragma unroll
  for (int j = 0; j < (kJ < 8 ? kJ : 8); ++j) vtw[j] = vt_lane_base(lane, (wave * kJ + j) & 7);

  // O^T accumulators: block j * NW + r holds dv 32 * (wave * kJ + j) .. +31 of
  // the workgroup's row block r.
  f32x16 O[16];
#pragma unroll
  for (int blk = 0; blk < 16; ++blk) O[blk] = f32x16{};
  float m_run = -INFINITY;   // max used for the exponentials (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum

  // Iteration k computes S^T and the softmax of tile k (k < ntiles) and the
  // P.V products of tile k-1, whose P^T the waves exchanged through LDS; the
  // last iteration only finishes tile ntiles-1.
  int buf = 0, bufp = 2;     // ring buffers of tiles k and k-1
  for (int k = 0; k <= ntiles; ++k) {
    const int par = k & 1;
    const bool live = k < ntiles;
    if (live) wait_vmcnt<0>();   // tile k has landed
    __syncthreads();             // ... for every wave; P^T, flags of tile k-1 are visible
    const int buf_next = buf == kBufs - 1 ? 0 : buf + 1;
    const uint8_t* spread_page = nullptr;   // dense full tile k+1, copied during S^T
    auto t1u = [&](int t) { return u0 + t; };
    if (k + 1 < ntiles) {
      if constexpr (SPARSE) {
        row_next = sparse_cache_row(j_b, pg_b);   // both landed by the wait above
        issue_sparse_scales(row_next, buf_next);
        issue_sparse_tile<ROPE, NW>(lds, buf_next, kv, row_next, lane, wave);
        j_b = j_c;
        pg_b = sparse_page(j_b);
        j_c = k + 3 < ntiles ? sparse_entry((u0 + k + 3) * kKeys + lane) : -1;
      } else {
        const int t1 = k + 1;
        if ((t1 & 63) == 0) {   // next 64 page ids (tile loops longer than 64 tiles)
          pages_v = page_of_lane(u0 + t1 + lane);
          wait_vmcnt<0>();
        }
        page_next = __builtin_amdgcn_readlane(pages_v, t1 & 63);
        // A full tile's copies are spread over the S^T loop below: issued in
        // one burst they stall the wave (the CU's vector memory path takes a
        // 1 KiB copy per ~16 cycles and all waves issue at once) while the
        // matrix core idles. Partial or missing pages are issued here.
        const bool ok = page_valid(page_next);
        if (ok && sk - t1u(t1) * kKeys >= kKeys) {
          spread_page = kv + (long)page_next * kKeys * RB;
          issue_scales(page_next, buf_next);
        } else {
          issue_dense(u0 + t1, page_next, buf_next);
        }
      }
    }

    // flags of tile k-1 (read now, used after the S^T products)
    const i32x4 fl = *reinterpret_cast<const i32x4*>(xflag + 4 * (par ^ 1));

    const uint8_t* nope = lds + buf * kNopeRegion;
    const uint8_t* rope = lds + kRopeBase + buf * kRopeRegion;
    const uint8_t* vnope = lds + bufp * kNopeRegion;            // V of tile k-1
    const uint8_t* pprev = xp + (par ^ 1) * X::p_bytes;         // P^T of tile k-1
    const int unit = u0 + k;

    // P.V operands of tile k-1: P^T of every row block, and a ring of V^T
    // fragments (one per 32-wide dv block, each used by NW products).
    constexpr int PDV = NW == 4 ? 2 : 3;
    i32x8 pt[NW];
    i32x8 vr[PDV];
    auto vfrag = [&](int j) -> i32x8 {
      const int blk = wave * kJ + j;
      i32x8 av;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x2 v = vt_bytes<GATHER_V>(vnope, lane, blk, u, vtw[j & 7]);
        av[2 * u] = v.x;
        av[2 * u + 1] = v.y;
      }
      return av;
    };
    auto load_pv_operands = [&]() {
#pragma unroll
      for (int r = 0; r < NW; ++r) {
        const i32x4 lo = lds_ld16(pprev, r * 2048 + lane * 16);
        const i32x4 hi = lds_ld16(pprev, r * 2048 + 1024 + lane * 16);
        pt[r] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int j = 0; j < PDV && j < kJ; ++j) vr[j] = vfrag(j);
    };

    // ---- S^T = K Q^T -------------------------------------------------------
    // The fragment reads of a tile run through a ring several items deep, so
    // about ten LDS reads are in flight while the MFMAs consume earlier ones
    // (one wave per SIMD: nothing else hides the LDS latency). Items alternate
    // between the two 32-key blocks, so consecutive MFMAs are independent. The
    // rope products have accumulators of their own, since q_scale * k_scale
    // applies to the nope products only; both are combined in the softmax.
    // Scheduling barriers keep the compiler from hoisting the whole tile's
    // fragment reads (which would need up to 160 more registers). The P.V
    // operands of tile k-1 are read as the ring drains. On the extra last
    // iteration these products run on stale LDS data that the mask discards.
    f32x16 Sn[2], Sr[2];
    if constexpr (ROPE == 0) Sr[0] = Sr[1] = f32x16{};
    {
      constexpr int NN = 16, NI = NN + (ROPE > 0 ? 8 : 0), PD = 5;
      const bool spread = __builtin_amdgcn_readfirstlane(spread_page != nullptr ? 1 : 0) != 0;
      const SpreadLane sl = spread_lane<ROPE>();
      i32x4 rl[PD], rh[PD];
      auto load = [&](int f) {
        const int slot = f % PD, kb = f & 1;
        if (f < NN) {
          const int t = f >> 1;
          const int c = 32 * kb * kNope + 256 * (t >> 2);
          rl[slot] = lds_ld16(nope, lb.k8[t & 3][0] + c);
          rh[slot] = lds_ld16(nope, lb.k8[t & 3][1] + c);
        } else {
          rl[slot] = lds_ld16(rope, lb.rp[(f - NN) >> 1] + 32 * kb * 128);
        }
      };
#pragma unroll
      for (int f = 0; f < PD; ++f) load(f);
#pragma unroll
      for (int f = 0; f < NI; ++f) {
        const int slot = f % PD, kb = f & 1;
        const i32x4 lo = rl[slot], hi = rh[slot];
        if (f + PD < NI) load(f + PD);
        if (f + PD == NI) load_pv_operands();
        if constexpr (!SPARSE) {
          constexpr int LPW = Tile<ROPE>::template loads_per_wave<NW>();
          if (spread) {
#pragma unroll
            for (int jj = f * LPW / NI; jj < (f + 1) * LPW / NI; ++jj)
              issue_dense_load_s<ROPE, NW>(lds, buf_next, spread_page, jj, wave, sl);
          }
        }
        if (f < NN) {
          const i32x8 kf = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          if (f < 2) mfma_fp8_32x32x64_first(Sn[kb], kf, qn[f >> 1]);
          else mfma_fp8_32x32x64(Sn[kb], kf, qn[f >> 1]);
        } else {
          const bf16x8 kr = __builtin_bit_cast(bf16x8, lo);
          if (f < NN + 2) mfma_bf16_32x32x16_first(Sr[kb], kr, qr[(f - NN) >> 1]);
          else mfma_bf16_32x32x16(Sr[kb], kr, qr[(f - NN) >> 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (ROPE > 0) s_nop_result4(Sn[0], Sn[1], Sr[0], Sr[1]);
    else s_nop_result2(Sn[0], Sn[1]);

    // ---- rescale O for the rows whose max tile k-1 raised (rare) ---------------
    // (before the P.V products of tile k-1; the previous iteration's P.V
    // MFMAs, the last writers of O, completed long before)
    if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]), "+a"(O[6]),
                     "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]), "+a"(O[12]), "+a"(O[13]),
                     "+a"(O[14]), "+a"(O[15]));
      const float* al = xalpha + (par ^ 1) * (NW * 32);
#pragma unroll
      for (int r = 0; r < NW; ++r) {
        if (__builtin_amdgcn_readfirstlane(fl[r])) {   // only row blocks that raised
          const float f = al[r * 32 + n];
#pragma unroll
          for (int j = 0; j < kJ; ++j) scale_agpr_acc(O[j * NW + r], f);
        }
      }
      asm volatile("s_nop 4" ::);
    }


    // ---- softmax of tile k, interleaved with the P.V products of tile k-1 ----
    // The 16 P.V MFMAs do not depend on the softmax, so its VALU work is cut
    // into slices issued between them; a slice runs while the matrix core
    // works on the MFMA before it. Slices 0-3: mask, scale and row max; 4: the
    // max goes to the other lane half (lanes l and l ^ 32 share a row); 6: the
    // lazy raise; 7-14: exponentials; 15: P^T packing, P^T and flags to LDS.
    bool full;
    int limit = 0;    // dense: keys of this tile this lane's row may see
    unsigned long long smask = 0;
    if constexpr (SPARSE) {
      smask = live ? __ballot(row_cur >= 0) : 0ull;
      full = smask == ~0ull;
    } else {
      const bool page_ok = live && page_valid(page_cur);
      full = page_ok && (unit + 1) * kKeys <= sk - (a.causal ? a.s_q - 1 : 0);
      limit = page_ok ? row_len - unit * kKeys : 0;
    }
    const float cn = qk_scale * a.sm_log2;
    f32x16 S[2];
    float mx = -INFINITY;
    int mx_other = 0;
    bool flagged = false;
    float psum = 0.f, m_exp = 0.f;
    i32x8 pb;
    // PT: the scales a slice needs are read one slice ahead (a read used at
    // once would stall the slice for the LDS latency): k-scales of slice i
    // (< 4) for keys 32 kb + 8 j + 4 ((j + h) & 1) + 0..3, j = 2 (i & 1) + 0..1;
    // v-scales of slice i (7..14) for j = (i - 7) & 3, kb = (i - 7) >> 2.
    f32x4 ks_next[2], vs_next;
    auto scale_key4 = [&](int kb, int j) { return 4 * (32 * kb + 8 * j + 4 * ((j + h) & 1)); };
    auto fetch_k = [&](int i) {
      if constexpr (PT) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          ks_next[jj] = *reinterpret_cast<const f32x4*>(xs + buf * 512 + scale_key4(i >> 1, 2 * (i & 1) + jj));
      }
    };
    auto fetch_v = [&](int i) {
      if constexpr (PT) vs_next = *reinterpret_cast<const f32x4*>(xs + buf * 512 + 256 + scale_key4((i - 7) >> 2, (i - 7) & 3));
    };
    auto slice = [&](int i) {
      if (i < 4) {
        // z in place; a tile some row sees only in part (the last of a
        // sequence) then overwrites its hidden entries with -inf. (Separate
        // full and masked computations of z end in different registers and
        // cost a copy per entry where they merge.)
        const int kb = i >> 1, r0 = 8 * (i & 1);
        if constexpr (PT) {
          const f32x4 ksc[2] = {ks_next[0], ks_next[1]};   // this slice's k-scales
          if (i + 1 < 4) fetch_k(i + 1);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = (r0 >> 2) + jj;
            const f32x4 ks = ksc[jj];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int r = 4 * j + rr;
              S[kb][r] = ROPE > 0 ? fmaf(Sn[kb][r] * ks[rr], cn, Sr[kb][r] * a.sm_log2) : Sn[kb][r] * ks[rr] * cn;
            }
          }
        } else {
#pragma unroll
          for (int r = r0; r < r0 + 8; ++r)
            S[kb][r] = ROPE > 0 ? fmaf(Sn[kb][r], cn, Sr[kb][r] * a.sm_log2) : Sn[kb][r] * cn;
        }
        if (!full) {
#pragma unroll
          for (int r = r0; r < r0 + 8; ++r) {
            const int j = r >> 2;
            const int key = 32 * kb + 8 * j + 4 * ((j + h) & 1) + (r & 3);
            bool valid;
            if constexpr (SPARSE) valid = (smask >> key) & 1ull;
            else valid = key < limit;
            S[kb][r] = valid ? S[kb][r] : -INFINITY;
          }
        }
#pragma unroll
        for (int r = r0; r < r0 + 8; ++r) mx = fmaxf(mx, S[kb][r]);
        asm volatile("" : "+v"(mx));   // keeps each slice's max in its slice
      } else if (i == 4) {
        mx_other = __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(mx));
      } else if (i == 6) {
        fetch_v(7);
        mx = fmaxf(mx, __int_as_float(mx_other));
        const bool raise = mx > m_run + Soft<DOT>::tau;
        if (__ballot(raise)) {
          const float m_new = raise ? mx : m_run;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
          l_run *= alpha;
          // O needs rescaling only where a finite max was raised
          flagged = __ballot(raise && m_run != -INFINITY) != 0ull;
          if (flagged && h == 0) {
            int ln;   // lane id recomputed here (a kept copy gets spilled)
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            xalpha[par * (NW * 32) + wave * 32 + (ln & 31)] = alpha;
          }
          m_run = m_new;
        }
        m_exp = ((m_run == -INFINITY) ? 0.f : m_run) - Soft<DOT>::ps_log2;
      } else if (i >= 7 && i < 15) {
        // four exponentials, packed to fp8 at once
        const int kb = (i - 7) >> 2, r0 = 4 * ((i - 7) & 3);
        float pe[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pe[r] = __builtin_amdgcn_exp2f(S[kb][r0 + r] - m_exp);
          psum += pe[r];
        }
        if constexpr (PT) {
          // p times its key's v-scale / V_ref (<= 1); masked keys (p = 0)
          // skip the scale, which may be stale or garbage
          const f32x4 vs = vs_next;
          if (i + 1 < 15) fetch_v(i + 1);
#pragma unroll
          for (int r = 0; r < 4; ++r) pe[r] = pe[r] > 0.f ? pe[r] * (vs[r] * inv_vref) : 0.f;
        }
        int w = f32x4_to_fp8x4(pe[0], pe[1], pe[2], pe[3]);
        asm volatile("" : "+v"(w));   // keeps the packing in this slice
        pb[i - 7] = w;
      } else if (i == 15) {
        l_run += psum;
        uint8_t* pdst = xp + par * X::p_bytes + wave * 2048 + lane * 16;
        *reinterpret_cast<i32x4*>(pdst) = i32x4{pb[0], pb[1], pb[2], pb[3]};
        *reinterpret_cast<i32x4*>(pdst + 1024) = i32x4{pb[4], pb[5], pb[6], pb[7]};
        if (lane == 0) xflag[4 * par + wave] = flagged ? 1 : 0;
      }
    };

    // O^T += V^T P^T for tile k-1: dv block j of this wave's kJ times row
    // block r, 16 MFMAs, with a softmax slice after each.
    fetch_k(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = i / NW, r = i % NW;
      if (r == 0 && j > 0 && j + PDV - 1 < kJ) vr[(j + PDV - 1) % PDV] = vfrag(j + PDV - 1);
      mfma_fp8_32x32x64_acc(O[i], vr[j % PDV], pt[r]);
      __builtin_amdgcn_sched_barrier(0);
      slice(i);
      __builtin_amdgcn_sched_barrier(0);
    }

    page_cur = page_next;
    row_cur = row_next;
    bufp = buf;
    buf = buf_next;
  }

  // ---- epilogue -----------------------------------------------------------------
  // The last P.V MFMAs have completed before VALU reads O.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]), "+a"(O[6]), "+a"(O[7]),
                 "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]), "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool nonempty = l_tot > 0.f;
  // splits == 1: output scale (v_scale or, per token, V_ref) / l; else the
  // partials' 1 / l (fp16 partials in code units, |value| <= 448; the combine
  // applies v_scale, or the per-row V_ref stored beside the lse)
  if (h == 0)
    xfin[wave * 32 + n] = nonempty ? (a.splits == 1 ? (PT ? vref : *v_scale) : 1.f) / l_tot : 0.f;
  if (wave_active && h == 0) {
    const float lse2 = nonempty ? m_run + log2f(l_tot) - Soft<DOT>::ps_log2 : -INFINITY;
    if (a.splits == 1) {
      if (row_ok) lse[qrow_idx] = nonempty ? lse2 * kLn2 : -INFINITY;
    } else {
      const long prow = (((long)s * a.groups + g) * a.row_blocks + rb) * 32 + n;
      part_lse[prow] = lse2;
      if (PT) part_row_scale(part_lse, a)[prow] = vref;
    }
  }
  __syncthreads();
  // O^T register e of block j * NW + r: dv 32 * (wave * kJ + j) + 8 * (e / 4) +
  // 4 * h + e % 4, row 32 * (row block) + n.
#pragma unroll
  for (int r = 0; r < NW; ++r) {
    const int rbr = rg * NW + r;
    if (rbr >= a.row_blocks) break;
    const float inv = xfin[r * 32 + n];
    const int rowr = rbr * 32 + n;
    if (a.splits == 1) {
      if (rowr < a.rows) {
        uint16_t* orow = out + ((long)g * a.rows + rowr) * kNope;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int dv = 32 * (wave * kJ + j) + 8 * e4 + 4 * h;
            const f32x16& o = O[j * NW + r];
            uint2 w;
            w.x = bf16x2_bits(o[4 * e4] * inv, o[4 * e4 + 1] * inv);
            w.y = bf16x2_bits(o[4 * e4 + 2] * inv, o[4 * e4 + 3] * inv);
            *reinterpret_cast<uint2*>(orow + dv) = w;
          }
        }
      }
    } else {
      // partials in the accumulator's own register layout (two 16-byte
      // stores per lane and block); the combine kernel reads the same layout.
      const long frag = ((long)s * a.groups + g) * a.row_blocks + rbr;
      uint16_t* po = part_o + frag * (16 * 64 * 16);
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const f32x16& o = O[j * NW + r];
        i32x4* dst = reinterpret_cast<i32x4*>(po + ((wave * kJ + j) * 64 + lane) * 16);
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

// Split combine (InfiniCore PR #1568, split-kv commit; empty partials carry
// lse = -inf and weight 0, so an all-empty row gives zeros and lse = -inf).
// Four workgroups per (group, 32-row block); thread (blk, lane) merges the 16
// accumulator values that lane held for dv block blk in every split. The
// partials are normalized by their own row sums; v_scale is applied here.
// Splits are taken four at a time with all their loads (lse and partial
// values) issued together, and merged with a running max (every split
// writes its partial, zeros when empty, so the loads need no guard).
__global__ __launch_bounds__(256) void mla_combine_kernel(MLA_KERNEL_PTRS, KDims a) {
  // the workgroups of a key stream on the die whose L2 its split workgroups
  // wrote the partials through (the split kernels group a stream's splits
  // the same way)
  const int bidx = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int gr = bidx >> 2;
  const int g = gr / a.row_blocks;
  const int rb = gr % a.row_blocks;
  const int blk = 4 * (bidx & 3) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const int row = rb * 32 + n;
  if (row >= a.rows) return;
  const long frag0 = (long)g * a.row_blocks + rb;          // split s: frag0 + s * groups * row_blocks
  const long fstride = (long)a.groups * a.row_blocks;
  float M = -INFINITY, W = 0.f;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const float* const pscale = a.per_token ? part_row_scale(part_lse, a) : nullptr;
  for (int s0 = 0; s0 < a.splits; s0 += 4) {
    float ls[4], sc[4];
    i32x4 v0[4], v1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + u < a.splits) {
        const long frag = frag0 + (s0 + u) * fstride;
        ls[u] = part_lse[frag * 32 + n];
        sc[u] = pscale != nullptr ? pscale[frag * 32 + n] : 1.f;
        const i32x4* src = reinterpret_cast<const i32x4*>(part_o + frag * (16 * 64 * 16) + (blk * 64 + lane) * 16);
        v0[u] = src[0];
        v1[u] = src[1];
      } else {
        ls[u] = -INFINITY;
        sc[u] = 0.f;
        v0[u] = v1[u] = i32x4{0, 0, 0, 0};
      }
    }
    const float m_new = fmaxf(M, fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3])));
    if (m_new == -INFINITY) continue;
    const float alpha = exp2f(M - m_new);   // 0 while M = -inf
    W *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] *= alpha;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w0 = exp2f(ls[u] - m_new);   // 0 for an empty split
      W += w0;
      const float w = w0 * sc[u];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += w * half_lo((unsigned)v0[u][d]);
        acc[2 * d + 1] += w * half_hi((unsigned)v0[u][d]);
        acc[8 + 2 * d] += w * half_lo((unsigned)v1[u][d]);
        acc[8 + 2 * d + 1] += w * half_hi((unsigned)v1[u][d]);
      }
    }
    M = m_new;
  }
  const float inv = W > 0.f ? (a.per_token ? 1.f : *v_scale) / W : 0.f;   // per token: the row scales
  const long qrow_idx = (long)g * a.rows + row;
  uint16_t* orow = out + qrow_idx * kNope;
  // lane half h holds dv 8 j + 4 h .. + 3 (j = 0..3) of the block's 32; one
  // lane swap of the packed pairs gives the lower half dv 0..15 and the upper
  // half dv 16..31, stored as two 16-byte runs per lane
  unsigned x[4], y[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    x[2 * j] = bf16x2_bits(acc[4 * j] * inv, acc[4 * j + 1] * inv);
    x[2 * j + 1] = bf16x2_bits(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv);
    y[2 * j] = bf16x2_bits(acc[8 + 4 * j] * inv, acc[8 + 4 * j + 1] * inv);
    y[2 * j + 1] = bf16x2_bits(acc[8 + 4 * j + 2] * inv, acc[8 + 4 * j + 3] * inv);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // lower half: keeps x (dv 0-3, 8-11), takes the upper half's x into y
    // (dv 4-7, 12-15); upper half: takes the lower half's y into x (dv 16-19,
    // 24-27), keeps y (dv 20-23, 28-31)
    const auto r = __builtin_amdgcn_permlane32_swap(x[k], y[k], false, false);
    x[k] = r[0];
    y[k] = r[1];
  }
  i32x4* dst = reinterpret_cast<i32x4*>(orow + 32 * blk + 16 * h);
  dst[0] = i32x4{(int)x[0], (int)x[1], (int)y[0], (int)y[1]};
  dst[1] = i32x4{(int)x[2], (int)x[3], (int)y[2], (int)y[3]};
  if (blk == 0 && h == 0) lse[qrow_idx] = (W > 0.f) ? (M + log2f(W)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Test and measurement kernels (same device routines as the decode).

__global__ void debug_decode_kernel(const uint8_t* codes, float* out_f32, uint16_t* out_bf16, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int base = 4 * i;
  if (base >= n) return;
  int v = 0;
  for (int k = 0; k < 4 && base + k < n; ++k) v |= (int)codes[base + k] << (8 * k);
  float f[4];
  fp8x4_to_f32(v, f);
  const i32x2 bb = fp8x4_to_bf16x4(v);
  for (int k = 0; k < 4 && base + k < n; ++k) {
    if (out_f32) out_f32[base + k] = f[k];
    if (out_bf16) out_bf16[base + k] = (uint16_t)((unsigned)bb[k >> 1] >> (16 * (k & 1)));
  }
}

// The fp8-dot path's e4m3fnuz -> e4m3fn transcoding (fnuz4_to_ocp4) on n
// bytes, four per thread.
__global__ void debug_fnuz_to_ocp_kernel(const uint8_t* codes, uint8_t* out, int n) {
  const int base = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (base >= n) return;
  unsigned v = 0;
  for (int k = 0; k < 4 && base + k < n; ++k) v |= (unsigned)codes[base + k] << (8 * k);
  const unsigned r = fnuz4_to_ocp4(v);
  for (int k = 0; k < 4 && base + k < n; ++k) out[base + k] = (uint8_t)(r >> (8 * k));
}

// Query quantization check: the decode's two quantizers on the same rows.
// Each workgroup takes 16 rows with the lane-quad quantizer of the role-split
// kernel (its codes and exponents are written out) and quantizes them again
// with the half-row quantizer of the other kernels; a row where the two
// disagree reports the exponent INT32_MIN, which no row can have.
__global__ __launch_bounds__(64) void debug_quantize_q_kernel(const uint16_t* q, int rows, int row_len,
                                                              uint8_t* codes, int32_t* exps) {
  __shared__ __attribute__((aligned(16))) uint8_t lc[16 * kNope];
  __shared__ int le[16], bad[16];
  const int lane = threadIdx.x;
  const int r4 = lane >> 2, qq = lane & 3;
  const int row = blockIdx.x * 16 + r4;
  const bool ok = row < rows;
  {
    const uint16_t* src = q + (long)(ok ? row : 0) * row_len + 8 * qq;
    i32x4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = *reinterpret_cast<const i32x4*>(src + 32 * i);
    uint2 c[16];
    const int e = quantize_q_quad(raw, c);
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<uint2*>(lc + r4 * kNope + 8 * (4 * i + qq)) = c[i];
    if (qq == 0) {
      le[r4] = e;
      bad[r4] = 0;
    }
  }
  __syncthreads();
  {
    const int n = lane & 31, h = lane >> 5, r = n & 15;
    const int row2 = blockIdx.x * 16 + r;
    const bool ok2 = row2 < rows;
    i32x8 qn[8];
    int e2;
    stage_q_fp8(q + (long)(ok2 ? row2 : 0) * row_len, ok2, h, qn, e2);
    bool same = e2 == le[r];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int d = 0; d < 8; ++d) same = same && qn[t][d] == *reinterpret_cast<const int*>(lc + r * kNope + 64 * t + 32 * h + 4 * d);
    if (!same) bad[r] = 1;
  }
  __syncthreads();
  if (!ok) return;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    *reinterpret_cast<uint2*>(codes + (long)row * kNope + 8 * (4 * i + qq)) =
        *reinterpret_cast<const uint2*>(lc + r4 * kNope + 8 * (4 * i + qq));
  if (qq == 0) exps[row] = bad[r4] ? INT32_MIN : le[r4];
}

// Gather check: one workgroup per (sequence, page unit) runs the decode
// kernel's tile loader and writes the tile back in logical order. A full page
// goes through the copies the tile loop spreads over its S^T products
// (scalar page base, per-lane swizzled offsets); a partial or missing page
// through the loader that zero-fills the slack, as in the tile loop.
template <int ROPE>
__global__ __launch_bounds__(256) void debug_gather_kernel(const uint8_t* kv, const int32_t* block_table,
                                                           const int32_t* seq_lens, int max_pages,
                                                           int num_pages, uint8_t* dense_out) {
  constexpr int RB = kNope + 2 * ROPE;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Tile<ROPE>::lds_bytes];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int b = blockIdx.x / max_pages, unit = blockIdx.x % max_pages;
  int sk = seq_lens[b];
  sk = max(0, min(sk, max_pages * kKeys));
  const int page = block_table[(long)b * max_pages + unit];
  const bool page_ok = page >= 0 && page < num_pages;
  const int valid = page_ok ? max(0, min(kKeys, sk - unit * kKeys)) : 0;
  const uint8_t* page_base = kv + (long)(page_ok ? page : 0) * kKeys * RB;
  if (valid == kKeys) {
    const SpreadLane sl = spread_lane<ROPE>();
    constexpr int LPW = Tile<ROPE>::template loads_per_wave<4>();
#pragma unroll
    for (int jj = 0; jj < LPW; ++jj) issue_dense_load_s<ROPE, 4>(lds, 0, page_base, jj, wave, sl);
  } else {
    issue_dense_tile<ROPE, 4>(lds, 0, page_base, valid, lane, wave);
  }
  wait_tile_and_sync();
  uint8_t* dst = dense_out + ((long)b * max_pages + unit) * kKeys * RB;
  for (int idx = threadIdx.x; idx < kKeys * (RB / 16); idx += 256) {
    const int r = idx / (RB / 16), c = idx % (RB / 16);
    const int off = c < 32 ? r * kNope + (swz(r, c) << 4) : kRopeBase + r * 128 + (swz_rope(r, c - 32) << 4);
    *reinterpret_cast<i32x4*>(dst + r * RB + c * 16) = lds_ld16(lds, off);
  }
}

__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4* src, long n16, float* sink) {
  int acc = 0;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256) {
    const i32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keep the loads live: one wave-wide vote on the loaded data per workgroup
  const unsigned long long nz = __ballot(acc != 0);
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)__popcll(nz);
}

// ---------------------------------------------------------------------------
// host-side launchers

size_t partials_bytes(int32_t splits, int32_t groups, int32_t row_blocks, bool per_token) {
  const size_t frags = (size_t)splits * groups * row_blocks;
  return frags * (16 * 64 * 16 * sizeof(uint16_t)) + frags * 32 * sizeof(float) * (per_token ? 2 : 1);
}

// Waves per workgroup: one per 32-row block, up to 4 (1, 2 or 4 so that the
// tile's load instructions divide evenly among them).
static int waves_per_group(int row_blocks) { return row_blocks >= 3 ? 4 : row_blocks; }

static KDims make_dims(const DecodeLaunch& d) {
  KDims a;
  a.s_q = d.s_q; a.h_q = d.h_q; a.rows = d.rows; a.row_blocks = d.row_blocks;
  const int nw = waves_per_group(d.row_blocks);
  a.row_groups = (d.row_blocks + nw - 1) / nw;
  a.groups = d.groups; a.splits = d.splits;
  a.num_pages = d.num_pages; a.max_pages = d.max_pages; a.topk = d.topk; a.causal = d.causal;
  a.sm_log2 = d.softmax_scale * kLog2e;
  a.per_token = d.per_token ? 1 : 0;
  return a;
}

#define MLA_PTR_ARGS(d) \
  d.q, d.kv, d.block_table, d.seq_lens, d.indices, d.k_scale, d.v_scale, d.out, d.lse, d.part_o, d.part_lse

template <int DOT, int ROPE, bool SPARSE, bool GV, bool XCH>
static hipError_t launch_nw(const DecodeLaunch& d, const KDims& a, hipStream_t st) {
  const int nw = waves_per_group(d.row_blocks);
  const dim3 grid((unsigned)(a.groups * a.splits * a.row_groups));
#define MLA_LAUNCH(NWV)                                                                                  \
  if constexpr (XCH)                                                                                     \
    hipLaunchKernelGGL((mla_decode_kernel<DOT, ROPE, SPARSE, NWV, GV>), grid, dim3(64 * NWV), 0, st,      \
                       MLA_PTR_ARGS(d), a);                                                              \
  else                                                                                                   \
    hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, NWV, GV>), grid, dim3(64 * NWV), 0, st, \
                       MLA_PTR_ARGS(d), a);
  switch (nw) {
    case 1: MLA_LAUNCH(1) break;
    case 2: MLA_LAUNCH(2) break;
    default: MLA_LAUNCH(4) break;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

// fp8 dots run the role-split kernel; the dv-split and row-block kernels
// serve them only when a variant flag asks for one. bf16 dots run the
// row-block kernel, or the role-split kernel's two-term form for at most 16
// rows per key stream (decode_ws_eligible).
template <int DOT, int ROPE, bool SPARSE>
static hipError_t launch_gv(const DecodeLaunch& d, const KDims& a, hipStream_t st) {
  if (decode_ws_eligible(d)) return launch_decode_ws(d, a, st);
  if constexpr (DOT == DOT_FP8) {
    if (d.per_token) {
      const dim3 grid((unsigned)(a.groups * a.splits * a.row_groups));
      switch (waves_per_group(d.row_blocks)) {
        case 1: hipLaunchKernelGGL((mla_decode_kernel<DOT, ROPE, SPARSE, 1, false, true>), grid, dim3(64), 0, st,
                                   MLA_PTR_ARGS(d), a); break;
        case 2: hipLaunchKernelGGL((mla_decode_kernel<DOT, ROPE, SPARSE, 2, false, true>), grid, dim3(128), 0, st,
                                   MLA_PTR_ARGS(d), a); break;
        default: hipLaunchKernelGGL((mla_decode_kernel<DOT, ROPE, SPARSE, 4, false, true>), grid, dim3(256), 0, st,
                                    MLA_PTR_ARGS(d), a); break;
      }
      return hipGetLastError();
    }
  }
  if constexpr (DOT == DOT_FP8) {
    if (d.rows_kernel) return launch_nw<DOT, ROPE, SPARSE, false, false>(d, a, st);
    return d.gather_v ? launch_nw<DOT, ROPE, SPARSE, true, true>(d, a, st)
                      : launch_nw<DOT, ROPE, SPARSE, false, true>(d, a, st);
  } else {
    if (d.per_token) {
      const dim3 grid((unsigned)(a.groups * a.splits * a.row_groups));
      switch (waves_per_group(d.row_blocks)) {
        case 1: hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, 1, false, true>), grid, dim3(64), 0,
                                   st, MLA_PTR_ARGS(d), a); break;
        case 2: hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, 2, false, true>), grid, dim3(128), 0,
                                   st, MLA_PTR_ARGS(d), a); break;
        default: hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, 4, false, true>), grid, dim3(256), 0,
                                    st, MLA_PTR_ARGS(d), a); break;
      }
      return hipGetLastError();
    }
    if (d.fnuz) {
      const dim3 grid((unsigned)(a.groups * a.splits * a.row_groups));
      switch (waves_per_group(d.row_blocks)) {
        case 1: hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, 1, false, false, true>), grid,
                                   dim3(64), 0, st, MLA_PTR_ARGS(d), a); break;
        case 2: hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, 2, false, false, true>), grid,
                                   dim3(128), 0, st, MLA_PTR_ARGS(d), a); break;
        default: hipLaunchKernelGGL((mla_decode_rows_kernel<DOT, ROPE, SPARSE, 4, false, false, true>), grid,
                                    dim3(256), 0, st, MLA_PTR_ARGS(d), a); break;
      }
      return hipGetLastError();
    }
    return d.gather_v ? launch_nw<DOT, ROPE, SPARSE, true, false>(d, a, st)
                      : launch_nw<DOT, ROPE, SPARSE, false, false>(d, a, st);
  }
}

template <int DOT, int ROPE>
static hipError_t launch_sp(const DecodeLaunch& d, const KDims& a, hipStream_t st) {
  return d.topk > 0 ? launch_gv<DOT, ROPE, true>(d, a, st) : launch_gv<DOT, ROPE, false>(d, a, st);
}

template <int DOT>
static hipError_t launch_rope(const DecodeLaunch& d, const KDims& a, hipStream_t st) {
  return d.d_rope == 64 ? launch_sp<DOT, 64>(d, a, st) : launch_sp<DOT, 0>(d, a, st);
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t st) {
  const KDims a = make_dims(d);
  if (d.debug_print)
    fprintf(stderr, "[mla_fp8] decode grid=%d (groups=%d splits=%d row_groups=%d) block=%d dot=%s rope=%d sparse=%d\n",
            a.groups * a.splits * a.row_groups, a.groups, a.splits, a.row_groups,
            64 * waves_per_group(d.row_blocks), d.dot == DOT_FP8 ? "fp8" : "bf16", d.d_rope,
            d.topk > 0);
  return d.dot == DOT_FP8 ? launch_rope<DOT_FP8>(d, a, st) : launch_rope<DOT_BF16>(d, a, st);
}

hipError_t launch_combine(const DecodeLaunch& d, hipStream_t st) {
  const KDims a = make_dims(d);
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(a.groups * a.row_blocks * 4)), dim3(256), 0, st,
                     MLA_PTR_ARGS(d), a);
  return hipGetLastError();
}

hipError_t launch_debug_decode_e4m3fn(const uint8_t* codes, float* out_f32, uint16_t* out_bf16,
                                      int32_t n, hipStream_t st) {
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(debug_decode_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     codes, out_f32, out_bf16, n);
  return hipGetLastError();
}

hipError_t launch_debug_fnuz_to_ocp(const uint8_t* codes, uint8_t* out, int32_t n, hipStream_t st) {
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(debug_fnuz_to_ocp_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, codes,
                     out, n);
  return hipGetLastError();
}

hipError_t launch_debug_quantize_q(const uint16_t* q, int32_t rows, int32_t row_len, uint8_t* codes,
                                   int32_t* exps, hipStream_t st) {
  hipLaunchKernelGGL(debug_quantize_q_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(64), 0, st, q,
                     rows, row_len, codes, exps);
  return hipGetLastError();
}

hipError_t launch_debug_gather(const uint8_t* kv, const int32_t* block_table, const int32_t* seq_lens,
                               int32_t batch, int32_t max_pages, int32_t num_pages, int32_t d_rope,
                               uint8_t* dense_out, hipStream_t st) {
  const dim3 grid((unsigned)(batch * max_pages));
  if (d_rope == 64)
    hipLaunchKernelGGL((debug_gather_kernel<64>), grid, dim3(256), 0, st, kv, block_table, seq_lens,
                       max_pages, num_pages, dense_out);
  else
    hipLaunchKernelGGL((debug_gather_kernel<0>), grid, dim3(256), 0, st, kv, block_table, seq_lens,
                       max_pages, num_pages, dense_out);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t st) {
  const long n16 = (long)(bytes / 16);
  hipLaunchKernelGGL(stream_read_kernel, dim3(4096), dim3(256), 0, st, (const i32x4*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace mla

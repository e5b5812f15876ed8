// Device-side building blocks shared by the decode kernels (mla_decode.hip,
// mla_decode_ws.hip): the e4m3fn conversions, the LDS tile layout and its
// global->LDS copies, the MFMA fragment bookkeeping and inline-asm MFMA
// wrappers, the fp8-dot query quantization and the softmax constants.
// Internal to the library; include/mla_fp8.h is the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "launch.h"

namespace mla {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kKeys = 64;          // keys per tile = page_block
constexpr int kNope = 512;         // fp8 latent dims = dv
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum { DOT_BF16 = 0, DOT_FP8 = 1 };

// ---------------------------------------------------------------------------
// e4m3fn conversions (hardware OCP fp8 on gfx950)

// 4 packed e4m3fn bytes -> 4 floats (exact).
__device__ inline void fp8x4_to_f32(int v, float f[4]) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
  f[0] = lo.x; f[1] = lo.y; f[2] = hi.x; f[3] = hi.y;
}

// 4 packed e4m3fn bytes -> 4 bf16 in two dwords with the gfx950 converter
// (scale 1.0; exact, since every e4m3fn value is a bf16 value).
__device__ inline i32x2 fp8x4_to_bf16x4(int v) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
  return i32x2{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}

// Cache bytes -> bf16 for the bf16-dot path. e4m3fn: the converter, exact.
// FNUZ (gfx942's e4m3fnuz: exponent bias 8, largest magnitude 240, NaN only
// at 0x80; ROCm/aiter PR #6199, Technical details): each code's sign goes to
// bf16 bit 15 and its exponent and mantissa bits to bits 10..4, which gives
// the fnuz value times 2^-119 for every code (the subnormal codes become
// bf16 subnormals; +-240 needs no special case); the kernel multiplies the k
// and v scales by 2^119. 0x80, fnuz's NaN, reads as zero.
constexpr int kFnuzExp = 119;
template <bool FNUZ>
__device__ inline i32x2 kv_bytes_to_bf16x4(int v) {
  if constexpr (FNUZ) {
    const unsigned u = (unsigned)v;
    // v_perm_b32 byte selects (selector 0..3: a byte of the second source,
    // 0x0C: zero): bytes 0, 1 to bits 0, 16; bytes 2, 3 likewise
    const unsigned x = __builtin_amdgcn_perm(0u, u, 0x0c010c00u);
    const unsigned y = __builtin_amdgcn_perm(0u, u, 0x0c030c02u);
    const unsigned tx = x << 4, ty = y << 4;   // exponent and mantissa at bits 10..4, sign at bit 11
    const unsigned bx = (tx & 0x07f007f0u) | ((tx << 4) & 0x80008000u);
    const unsigned by = (ty & 0x07f007f0u) | ((ty << 4) & 0x80008000u);
    return i32x2{(int)bx, (int)by};
  }
  return fp8x4_to_bf16x4(v);
}

// 4 floats -> 4 packed e4m3fn bytes (round to nearest even).
__device__ inline int f32x4_to_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

// Two floats as two IEEE half values (round to nearest even), a in the low half.
__device__ inline unsigned half2_bits(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (unsigned)__builtin_bit_cast(uint16_t, ha) | ((unsigned)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ inline float half_lo(unsigned w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float half_hi(unsigned w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ inline unsigned bf16x2_bits(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) |
         ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

__device__ inline float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Smallest integer e with amax <= 448 * 2^e (0 for amax == 0). With
// amax = f * 2^E, f in [0.5, 1) and 448 = 0.875 * 2^9: e = E - 9 if f <= 0.875,
// else E - 8.
__device__ inline int q_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  float f = frexpf(amax, &E);
  return (f > 0.875f) ? E - 8 : E - 9;
}

// ---------------------------------------------------------------------------
// LDS layout. Two tile buffers; each holds a nope region [64 rows][512 B] and
// a rope region [64 rows][128 B]. The nope regions of both buffers come first
// (0 and 32 KiB), then the rope regions (64 and 72 KiB), which keeps every
// nope fragment offset inside the 16-bit ds_read immediate.
//
// Within a nope row, 16-byte chunk c is stored at chunk position c ^ (row & 15);
// within a rope row at c ^ ((row >> 1) & 7). The LDS has 64 banks of 4 bytes and
// serves a 16-byte-per-lane read 16 lanes at a time; nope rows are a multiple
// of 256 bytes apart, so without the swizzle one column of 16 rows would hit
// the same 4 banks, and with it any 16 rows with distinct row & 15 cover all 64
// banks. Rope rows are 128 bytes, two per 256-byte bank line: row & 1 already
// separates the two, and (row >> 1) & 7 the eight lines. Only the low four
// chunk bits are permuted, so each fragment read below needs at most eight
// per-lane base addresses plus compile-time offsets.

constexpr int kNopeRegion = kKeys * kNope;          // 32 KiB per buffer
constexpr int kRopeRegion = kKeys * 128;            // 8 KiB per buffer
constexpr int kBufs = 3;                            // LDS ring: 1 tile computing, 2 landing
constexpr int kRopeBase = kBufs * kNopeRegion;      // rope regions after all nope regions

template <int ROPE>
struct Tile {
  static constexpr int lds_bytes = kBufs * kNopeRegion + (ROPE > 0 ? kBufs * kRopeRegion : 0);
  // global->LDS loads one wave issues for a full tile
  template <int NW> static constexpr int loads_per_wave() { return (32 + (ROPE > 0 ? 8 : 0)) / NW; }
};

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline int swz(int row, int chunk) { return chunk ^ (row & 15); }
__device__ inline int swz_rope(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// One 16-byte-per-lane global->LDS direct load: lane l's 16 bytes from `src`
// land at lds_base + 16 l (lds_base must be wave-uniform; it goes to M0).
// Written as inline asm so the compiler does not treat every later LDS read
// as possibly aliasing the in-flight copy (it would then wait for all
// outstanding loads, draining the prefetch ring); the tile loop orders the
// copies with explicit vmcnt waits and a barrier instead.
__device__ __attribute__((always_inline)) inline void load_lds16(const uint8_t* src, uint8_t* lds_base) {
  // A generic pointer into LDS carries the LDS address in its low 32 bits
  // (the high half is the LDS aperture). readfirstlane: the base is
  // wave-uniform; this keeps it in a scalar register even where the compiler
  // cannot prove that.
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

// 64 consecutive dwords from a wave-uniform source to lds_base (lane l's
// dword lands at lds_base + 4 l). The source stays in SGPRs and the lane
// offset comes from the exec-mask bit count at the call (a per-lane 64-bit
// address kept across the tile loop would be spilled, and its reload would
// wait for every copy in flight).
__device__ __attribute__((always_inline)) inline void load_lds4_row(const float* sbase, uint8_t* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  const unsigned long long sb = (unsigned long long)(uintptr_t)sbase;
  const unsigned long long sbu = ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(sb >> 32)) << 32) |
                                 (unsigned)__builtin_amdgcn_readfirstlane((unsigned)sb);
  unsigned voff;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 2, %0"
               : "=v"(voff));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbu), "s"(m0)
               : "memory", "m0");
}

// One dword per lane from per-lane sources (lane l's lands at lds_base + 4 l).
__device__ __attribute__((always_inline)) inline void load_lds4_gather(const float* src, uint8_t* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

// Max of a value over lanes l and l ^ 32 (the two halves holding one query row).
__device__ inline float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// Wave index within the workgroup, as a wave-uniform (scalar) value.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Workgroup i of a launch goes to XCD i % 8 (round-robin over the 8 dies,
// each with its own L2). The logical index returned here makes consecutive
// logical ids share a die: the splits of one query group then read its query
// rows through one L2 instead of four. The first 8 * (n / 8) ids are permuted
// among themselves, the rest keep their place.
constexpr int kXcds = 8;
__device__ inline int xcd_grouped_block(int bid, int n) {
  const int per = n / kXcds;
  if (bid >= per * kXcds) return bid;
  return (bid % kXcds) * per + bid / kXcds;
}

__device__ inline i32x4 lds_ld16(const uint8_t* base, int off) {
  return *reinterpret_cast<const i32x4*>(base + off);
}

// ds_read_b64_tr_b8 at base + off (see vt_bytes for the lane semantics).
__device__ inline i32x2 lds_tr8(const uint8_t* base, int off) {
  typedef int v2i_lds __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_lds*)(base + off));
}

// Per-lane byte offsets (within a 64-row page) of the 16-byte chunks a lane
// moves: the lane at chunk position P of row r fetches the row's chunk
// P ^ swizzle(r). Nope load j covers rows 2j, 2j+1 (lane l: row 2j + l/32,
// position l%32); (2j + l/32) & 15 only depends on j & 7, so eight offsets
// serve all 32 loads: off(j) = nope_lane(j & 7) + 2j * RB. Rope load j covers
// rows 8j .. 8j+7 (row 8j + l/8, position l%8), whose ((row >> 1) & 7) only
// depends on j & 1: off(j) = rope_lane[j & 1] + 8j * RB. Wave w issues the
// contiguous block of loads w*(32/NW) .. (a multiple of 8 nope and of 2 rope
// loads), so j & 7 and j & 1 are known at compile time.
template <int ROPE>
struct LoadOffsets {
  int nv[8];          // nope load j: global chunk offset for rows with (2j + hi) & 15
  int rope_lane[2];   // rope load j: by j & 1
  __device__ LoadOffsets(int lane) {
    constexpr int RB = kNope + 2 * ROPE;
    const int hi = lane >> 5, p = lane & 31;
#pragma unroll
    for (int v = 0; v < 8; ++v) nv[v] = hi * RB + ((p ^ (2 * v + hi)) << 4);
    const int r8 = lane >> 3, p8 = lane & 7;
#pragma unroll
    for (int par = 0; par < 2; ++par) rope_lane[par] = r8 * RB + kNope + ((p8 ^ (4 * par + (r8 >> 1))) << 4);
  }
  __device__ int nope_lane(int v) const { return nv[v]; }
};

// The offsets are recomputed for every tile from a copy of the lane id the
// compiler cannot see through: otherwise it hoists the 40 per-load addresses
// (or the offsets) out of the tile loop and spills them.
template <int ROPE>
__device__ inline LoadOffsets<ROPE> fresh_offsets(int) {
  // lane id from the exec-mask bit count, as volatile asm so that it is
  // recomputed here rather than hoisted out of the loop (and spilled)
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return LoadOffsets<ROPE>(lane);
}

// Issue the global->LDS copies of one 64-key tile into buffer `bufi`.
// Zero 16 bytes of LDS (a lane's share of a skipped copy). The zero comes
// from a volatile move at the store: a plain constant is kept in registers
// across the tile loop and, under its register pressure, spilled.
__device__ inline void lds_zero16(uint8_t* dst) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  *reinterpret_cast<i32x4*>(dst) = i32x4{z, z, z, z};
}

// Dense tiles read one page: `page_base` points at its first row and rows
// >= `valid` are zero-filled instead of loaded (the page's slack). A full
// tile issues exactly Tile::loads_per_wave loads per wave, which the tile
// loop's vmcnt waits count on; a partial tile issues a data-dependent number
// and therefore drains all outstanding loads before returning.
template <int ROPE, int NW>
__device__ __attribute__((always_inline)) inline void issue_dense_tile(uint8_t* lds, int bufi, const uint8_t* page_base, int valid,
                                        int lane, int wave) {
  constexpr int RB = kNope + 2 * ROPE;
  const LoadOffsets<ROPE> lo = fresh_offsets<ROPE>(lane);
  constexpr int NJ = 32 / NW, RJ = 8 / NW;
  uint8_t* nope = lds + bufi * kNopeRegion + wave * NJ * 1024;
  uint8_t* rope = lds + kRopeBase + bufi * kRopeRegion + wave * RJ * 1024;
  const uint8_t* nsrc = page_base + wave * NJ * 2 * RB;
  const uint8_t* rsrc = page_base + wave * RJ * 8 * RB;
  const int row0 = wave * NJ * 2 + (lane >> 5), rrow0 = wave * RJ * 8 + (lane >> 3);
  if (valid == kKeys) {
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      load_lds16(nsrc + (unsigned)(2 * jj * RB + lo.nope_lane(jj & 7)), nope + jj * 1024);
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int jj = 0; jj < RJ; ++jj)
        load_lds16(rsrc + (unsigned)(8 * jj * RB + lo.rope_lane[jj & 1]), rope + jj * 1024);
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      if (row0 + 2 * jj < valid)
        load_lds16(nsrc + (unsigned)(2 * jj * RB + lo.nope_lane(jj & 7)), nope + jj * 1024);
      else
        lds_zero16(nope + jj * 1024 + lane * 16);
    }
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int jj = 0; jj < RJ; ++jj) {
        if (rrow0 + 8 * jj < valid)
          load_lds16(rsrc + (unsigned)(8 * jj * RB + lo.rope_lane[jj & 1]), rope + jj * 1024);
        else
          lds_zero16(rope + jj * 1024 + lane * 16);
      }
    }
    wait_vmcnt<0>();
  }
}

// Sparse tiles gather 64 independent rows: `mine` is the cache row index
// (page * 64 + slot) that this lane resolved for tile row `lane`, or -1 for a
// skipped entry (zero-filled).
template <int ROPE, int NW>
__device__ __attribute__((always_inline)) inline void issue_sparse_tile(uint8_t* lds, int bufi, const uint8_t* kv, int mine,
                                         int, int wave) {
  constexpr int RB = kNope + 2 * ROPE;
  // a lane id the compiler cannot hoist out of the tile loop: the 32 lane
  // exchange addresses derived from a kept one were spilled, and each reload
  // waited for every copy in flight
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const LoadOffsets<ROPE> lo(lane);
  constexpr int NJ = 32 / NW, RJ = 8 / NW;
  uint8_t* nope = lds + bufi * kNopeRegion + wave * NJ * 1024;
  uint8_t* rope = lds + kRopeBase + bufi * kRopeRegion + wave * RJ * 1024;
  const int row0 = wave * NJ * 2 + (lane >> 5), rrow0 = wave * RJ * 8 + (lane >> 3);
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int cr = __shfl(mine, row0 + 2 * jj);
    if (cr >= 0)
      load_lds16(kv + (long)cr * RB + (lo.nope_lane(jj & 7) - (lane >> 5) * RB), nope + jj * 1024);
    else
      lds_zero16(nope + jj * 1024 + lane * 16);
    // one copy's address at a time (with all of a one-wave tile's copies
    // computed up front the row-block kernel spills)
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (ROPE > 0) {
#pragma unroll
    for (int jj = 0; jj < RJ; ++jj) {
      const int cr = __shfl(mine, rrow0 + 8 * jj);
      if (cr >= 0)
        load_lds16(kv + (long)cr * RB + (lo.rope_lane[jj & 1] - (lane >> 3) * RB), rope + jj * 1024);
      else
        lds_zero16(rope + jj * 1024 + lane * 16);
    }
  }
}

// One of the Tile::loads_per_wave copies that issue_dense_tile makes for a
// full dense tile (load jj of this wave; jj is a compile-time constant at the
// call sites), so that the copies can be spread between other instructions.
// The lane offset is recomputed each time (volatile asm: not hoisted and kept).
template <int ROPE, int NW>
__device__ inline void issue_dense_load(uint8_t* lds, int bufi, const uint8_t* page_base, int jj, int wave) {
  constexpr int RB = kNope + 2 * ROPE;
  constexpr int NJ = 32 / NW, RJ = 8 / NW;
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  if (jj < NJ) {
    const int hi = lane >> 5, p = lane & 31;
    const int off = hi * RB + ((p ^ (2 * (jj & 7) + hi)) << 4);
    load_lds16(page_base + (unsigned)(wave * NJ * 2 * RB + 2 * jj * RB + off),
               lds + bufi * kNopeRegion + (wave * NJ + jj) * 1024);
  } else {
    const int r = jj - NJ;
    const int r8 = lane >> 3, p8 = lane & 7;
    const int off = r8 * RB + kNope + ((p8 ^ (4 * (r & 1) + (r8 >> 1))) << 4);
    load_lds16(page_base + (unsigned)(wave * RJ * 8 * RB + 8 * r * RB + off),
               lds + kRopeBase + bufi * kRopeRegion + (wave * RJ + r) * 1024);
  }
}

// The same copies with a scalar base: the uniform part of the source address
// (page, row) stays in SGPRs, each lane adds a 32-bit offset. The per-lane
// parts of the offsets are computed once per tile (SpreadLane): for nope load
// j, lane (hi, p) reads chunk p ^ (2j + hi) of its row, i.e. with x = p ^ hi,
// chunk x ^ 2j, byte offset hi * RB + ((x << 4) ^ 32 j); for rope load r,
// lane (r8, p8) reads chunk p8 ^ (4 (r & 1) + r8 / 2), byte offset
// r8 * RB + 512 + ((y << 4) ^ 64 (r & 1)) with y = p8 ^ (r8 / 2). One
// xor-add per copy instead of a 64-bit address computation.
struct SpreadLane {
  unsigned nx, nrow, rx, rrow;
};
template <int ROPE>
__device__ inline SpreadLane spread_lane() {
  constexpr int RB = kNope + 2 * ROPE;
  int lane;   // volatile: recomputed per tile instead of hoisted and spilled
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int hi = lane >> 5, p = lane & 31, r8 = lane >> 3, p8 = lane & 7;
  return SpreadLane{(unsigned)((p ^ hi) << 4), (unsigned)(hi * RB), (unsigned)((p8 ^ (r8 >> 1)) << 4),
                    (unsigned)(r8 * RB + kNope)};
}

__device__ __attribute__((always_inline)) inline void load_lds16_saddr(const uint8_t* sbase, unsigned voff,
                                                                       uint8_t* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  const unsigned long long sb = (unsigned long long)(uintptr_t)sbase;
  const unsigned long long sbu = ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(sb >> 32)) << 32) |
                                 (unsigned)__builtin_amdgcn_readfirstlane((unsigned)sb);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbu), "s"(m0)
               : "memory", "m0");
}

template <int ROPE, int NW>
__device__ __attribute__((always_inline)) inline void issue_dense_load_s(uint8_t* lds, int bufi, const uint8_t* page_base,
                                                                         int jj, int wave, const SpreadLane& sl) {
  constexpr int RB = kNope + 2 * ROPE;
  constexpr int NJ = 32 / NW, RJ = 8 / NW;
  if (jj < NJ) {
    load_lds16_saddr(page_base + (wave * NJ * 2 + 2 * jj) * RB, (sl.nx ^ (32u * (jj & 7))) + sl.nrow,
                     lds + bufi * kNopeRegion + (wave * NJ + jj) * 1024);
  } else {
    const int r = jj - NJ;
    load_lds16_saddr(page_base + (wave * RJ * 8 + 8 * r) * RB, (sl.rx ^ (64u * (r & 1))) + sl.rrow,
                     lds + kRopeBase + bufi * kRopeRegion + (wave * RJ + r) * 1024);
  }
}

__device__ inline void wait_tile_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fragment bookkeeping for the 32x32 MFMA, lane l = 32*h + n:
//  * C/D (16 f32): column n, row 8*(r/4) + 4*h + r%4 for register r.
//  * A/B operands: lane l supplies row (A) / column (B) n and a slice of the
//    contraction selected by h. Only the pairing of A and B slices matters, so
//    both operands are always built with the same (h, byte) -> k assignment.
//
// S^T = K Q^T: the A operand's row m is loaded from key 32*kb + key_of_row(m)
// of the tile. The permutation keeps the 8 lanes of every aligned group on 8
// rows with distinct row & 7 (conflict free), and makes the 16 keys a lane
// half owns in a 32-key block pair up into 8-key groups that are again
// distinct mod 8 for the transposed V reads. With m = 8j + 4hh + i:
// key = 8j + 4*((j + hh) & 1) + i.
__device__ inline int key_of_row(int m) {
  const int j = m >> 3, hh = (m >> 2) & 1, i = m & 3;
  return 8 * j + 4 * ((j + hh) & 1) + i;
}

// P^T (B operand of O^T = V^T P^T) is packed from S in register order: byte
// 8u + e of lane half h is S[u/2][8*(u%2) + e], i.e. key
//     32*(u/2) + key_of_row(8*(2*(u%2) + e/4) + 4h + e%4) = 16u + tr_key(e, h)
// and the V^T operand must present the same keys.
__device__ inline int tr_key(int e, int h) {
  const int jl = e >> 2;  // low bit of j
  return 8 * jl + 4 * ((jl + h) & 1) + (e & 3);
}

// V^T bytes for dv block blk (32 dv values) and contraction bytes 8u .. 8u+7:
// byte e of the result is V[16u + tr_key(e, h)][32*blk + n] (e4m3fn).
template <bool GATHER>
__device__ inline i32x2 vt_bytes(const uint8_t* nope, int lane, int blk, int u, int vt_base) {
  const int h = lane >> 5;
  if constexpr (GATHER) {
    const int n = lane & 31;
    const int dv = 32 * blk + n;
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 16 * u + tr_key(e, h);
      const unsigned byte = nope[key * kNope + (swz(key, dv >> 4) << 4) + (dv & 15)];
      w[e >> 2] |= byte << (8 * (e & 3));
    }
    return i32x2{(int)w[0], (int)w[1]};
  } else {
    // ds_read_b64_tr_b8 transposes within groups of 16 lanes: lane s of a group
    // supplies the address of an 8-byte row segment, and lane i of the group
    // receives, as its byte j, byte (i % 8) of the segment supplied by lane
    // 2j + i/8. Group g = lane/16 covers dv 32*blk + 16*(g%2) + (lane%16), so
    // its lanes 2j and 2j+1 supply key 16u + tr_key(j, h) at dv offsets 0 and 8
    // of that 16-wide slice (one 16-byte LDS chunk); vt_base is
    // vt_lane_base(lane, blk % 8).
    return lds_tr8(nope, vt_base + 8192 * u + 256 * (blk >> 3));
  }
}

// Per-lane LDS byte offsets of every fragment read, split as (one of eight
// lane bases) + (compile-time offset). The chunk swizzle only permutes the low
// four chunk bits, so the loop-varying part of each chunk index (bit 4)
// becomes an immediate offset and only the low bits enter the bases:
//  * fp8 K fragment t, half e:  (32 kb + krow)*512 + 16*((4t + 2h + e) ^ (krow & 15))
//      = k8[t & 3][e] + 32*kb*512 + 256*(t >> 2)
//  * bf16 K fragment t (16 B): = k16[t & 7] + 32*kb*512 + 256*(t >> 3)
//  * rope fragment t:           = rp[t] + 32*kb*128           (rope region)
//  * V^T read (blk, u):         = vt_base(blk & 7) + 8192*u + 256*(blk >> 3)
__device__ inline int vt_lane_base(int lane, int b8) {
  const int h = lane >> 5, g = lane >> 4, sup = lane & 15;
  const int tk = tr_key(sup >> 1, h);
  return tk * kNope + (((2 * b8 + (g & 1)) ^ (tk & 15)) << 4) + 8 * (sup & 1);
}
// The lane id from the exec-mask bit count, as volatile asm: a value the
// compiler recomputes where it is used instead of keeping it (and what is
// derived from it) across a tile loop, where register pressure would spill it
// and each reload would wait for every tile copy in flight.
__device__ inline int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

struct LdsBases {
  int k8[4][2], k16[8], rp[4], vt[8];
  __device__ LdsBases(int lane) {
    const int n = lane & 31, h = lane >> 5;
    const int krow = key_of_row(n), kx = krow & 15, rx = (krow >> 1) & 7;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int e = 0; e < 2; ++e) k8[p][e] = krow * kNope + (((4 * p + 2 * h + e) ^ kx) << 4);
#pragma unroll
    for (int t = 0; t < 8; ++t) k16[t] = krow * kNope + (((2 * t + h) ^ kx) << 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) rp[t] = krow * 128 + (((2 * t + h) ^ rx) << 4);
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) vt[b8] = vt_lane_base(lane, b8);
  }
};

// ---------------------------------------------------------------------------
// The S^T = K Q^T products accumulate in VGPRs (inline asm with "v" operands),
// because the O^T accumulator already fills the 256 AGPRs and the softmax
// reads S with VALU instructions. These MFMAs are invisible to the compiler's
// hazard recognizer, so the required wait states are inserted here:
//  * a chain of MFMAs accumulating into the same registers with the same
//    opcode needs none between them;
//  * VALU reads of an MFMA result: at most 18 wait states for the 16-pass
//    32x32 MFMAs; s_nop_result gives 32;
//  * an MFMA reading (as A, B or C) registers a VALU instruction wrote needs
//    2 wait states: every asm MFMA starts with s_nop 1, and the variants named
//    after_valu with s_nop 4 (the compiler may place an operand's VALU
//    producer right before the asm statement);
//  * the compiler also does not know that a register an asm MFMA writes stays
//    busy for its passes: a value it copies out of an accumulator (say at a
//    loop exit) must come after an explicit s_nop_result.
// tests/test_asm_hazards.py checks these windows on the built assembly.

__device__ inline void mfma_fp8_32x32x64(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_32x32x16(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_32x32x16_after_valu(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// First product of an accumulator chain: C = 0 as an inline constant, so no
// VALU zeroing (and no wait states after it) is needed.
__device__ inline void mfma_fp8_32x32x64_first(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_32x32x16_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_32x32x16_first_after_valu(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// Two chained bf16 products whose A operands were both just converted by
// VALU. One statement, so that no conversion can be scheduled between them
// (an MFMA reading a register VALU wrote without wait states reads stale data).
__device__ inline void mfma_bf16_pair_after_valu(f32x16& acc, const bf16x8& a0, const bf16x8& b0,
                                                 const bf16x8& a1, const bf16x8& b1) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %3, %4, %0"
               : "+v"(acc) : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}
__device__ inline void mfma_bf16_pair_first_after_valu(f32x16& acc, const bf16x8& a0, const bf16x8& b0,
                                                       const bf16x8& a1, const bf16x8& b1) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\tv_mfma_f32_32x32x16_bf16 %0, %3, %4, %0"
               : "=&v"(acc) : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}
// Wait states before VALU reads of the four S^T accumulators (named as
// operands so that no read of any of them can be scheduled above the wait).
__device__ inline void s_nop_result4(f32x16& a0, f32x16& a1, f32x16& a2, f32x16& a3) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
}
__device__ inline void s_nop_result2(f32x16& a0, f32x16& a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}
// O^T += V^T P^T with the accumulator pinned to AGPRs ("a" operands).
__device__ inline void mfma_fp8_32x32x64_acc(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_fp8_32x32x64_acc_after_valu(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_32x32x16_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The last O^T products of a tile, followed by the wait states of their
// results (passes + 4): whatever comes next, in the next iteration or after
// the tile loop (where the compiler may copy the accumulators), sees them
// complete. Only this product's accumulator is named, so the wait costs no
// register constraint on the others.
__device__ inline void mfma_fp8_32x32x64_acc_last(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_32x32x16_acc_last(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 3"
               : "+a"(acc) : "v"(a), "v"(b));
}
__device__ inline void s_nop_result(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// acc *= s for an accumulator that lives in AGPRs, done in place with
// v_accvgpr_read / v_mul / v_accvgpr_write so the compiler never needs the
// accumulator in VGPRs (a plain `acc *= s` makes it keep copies of all 256
// accumulator registers in VGPRs across the tile loop). Callers make sure the
// MFMAs that wrote `acc` have completed, and end with s_nop 4 before the next
// MFMA reads it.
__device__ inline void scale_agpr_acc(f32x16& acc, float s) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float x = acc[e], tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(s));
    acc[e] = x;
  }
}

// ---------------------------------------------------------------------------

// Scalar launch parameters (pointers are passed separately as __restrict__
// kernel arguments, which lets uniform reads of the read-only tables become
// scalar loads).
struct KDims {
  int32_t s_q, h_q, rows, row_blocks, row_groups, groups, splits;
  int32_t num_pages, max_pages, topk, causal;
  float sm_log2;  // softmax_scale * log2(e)
  int32_t per_token;  // k_scale, v_scale hold one value per cache row
};

// Per-token scales, splits > 1: the f32 factor per partial row that follows
// the log2-lse array; the row's stored fp16 values times it are the split's
// normalized output. It keeps the stored values within fp16's range and away
// from its subnormals whatever the magnitude of the scales.
__device__ inline float* part_row_scale(float* part_lse, const KDims& a) {
  return part_lse + (long)a.splits * a.groups * a.row_blocks * 32;
}

#define MLA_KERNEL_PTRS                                                                   \
  const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,                         \
      const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,      \
      const int32_t* __restrict__ indices, const float* __restrict__ k_scale,             \
      const float* __restrict__ v_scale, uint16_t* __restrict__ out, float* __restrict__ lse, \
      uint16_t* __restrict__ part_o, float* __restrict__ part_lse

// Q staging for the fp8-dot path: lane (n, h) quantizes its half of query row
// n's 512 nope dims. The row's power-of-two exponent needs the amax of both
// halves (lanes n and n+32). Fragment t (K = 64 dims 64t .. 64t+63) holds dims
// 64t + 32h + (0..31) in byte order.
// The 256 bf16 query values lane (n, h) quantizes: row n, dims 64 t + 32 h
// + 8 k .. +7 in raw[t][k]. Unconditional loads (`qrow` must point at a
// readable row): a per-load guard becomes a branch around each load, after
// which the compiler waits for the load.
__device__ inline void load_q_nope_raw(const uint16_t* qrow, int h, i32x4 raw[8][4]) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      raw[t][k] = *reinterpret_cast<const i32x4*>(qrow + 64 * t + 32 * h + 8 * k);
}

// Per-row power-of-two scale and e4m3fn codes of the nope query (the row's
// two lane halves share the max).
__device__ inline void quantize_q_fp8(const i32x4 raw[8][4], i32x8 qn[8], int& e_out) {
  float amax = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const i32x4 v = raw[t][k];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo((unsigned)v[d])), fabsf(bf16_hi((unsigned)v[d]))));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const int e = q_exponent(amax);
  // x * 2^-e by exponent adjustment (one v_ldexp_f32): a multiply by the
  // constant 2^-e would overflow to inf for rows with amax below ~2^-119
  // (-e > 127), which bf16 can hold
  const int ne = -e;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const i32x4 v = raw[t][k];
      const unsigned w0 = (unsigned)v[0], w1 = (unsigned)v[1], w2 = (unsigned)v[2], w3 = (unsigned)v[3];
      qn[t][2 * k] = f32x4_to_fp8x4(ldexpf(bf16_lo(w0), ne), ldexpf(bf16_hi(w0), ne), ldexpf(bf16_lo(w1), ne),
                                    ldexpf(bf16_hi(w1), ne));
      qn[t][2 * k + 1] = f32x4_to_fp8x4(ldexpf(bf16_lo(w2), ne), ldexpf(bf16_hi(w2), ne), ldexpf(bf16_lo(w3), ne),
                                        ldexpf(bf16_hi(w3), ne));
    }
  }
  e_out = e;
}

// One pass over the row: its 256 bf16 values (128 registers, free before
// the tile loop) are all loaded before the max is taken.
__device__ inline void stage_q_fp8(const uint16_t* qrow, bool ok, int h, i32x8 qn[8], int& e_out) {
  i32x4 raw[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      raw[t][k] = ok ? *reinterpret_cast<const i32x4*>(qrow + 64 * t + 32 * h + 8 * k) : i32x4{0, 0, 0, 0};
  quantize_q_fp8(raw, qn, e_out);
}

// The same quantization with one row per lane quad: quarter qq = lane & 3
// holds the row's 16-byte chunks 4 i + qq (i = 0..15, 8 bf16 values each) in
// raw[i]; the row max is reduced over the quad. codes[i] receives the 8 codes
// of chunk 4 i + qq; returns the row's exponent e. Every quad of the wave
// must call it (the reduction reads lanes l ^ 1 and l ^ 2).
__device__ inline int quantize_q_quad(const i32x4 raw[16], uint2 codes[16]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo((unsigned)raw[i][d])), fabsf(bf16_hi((unsigned)raw[i][d]))));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = q_exponent(amax);
  const int ne = -e;   // exponent adjustment, as in quantize_q_fp8
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const unsigned w0 = (unsigned)raw[i][0], w1 = (unsigned)raw[i][1], w2 = (unsigned)raw[i][2],
                   w3 = (unsigned)raw[i][3];
    codes[i].x = (unsigned)f32x4_to_fp8x4(ldexpf(bf16_lo(w0), ne), ldexpf(bf16_hi(w0), ne), ldexpf(bf16_lo(w1), ne),
                                          ldexpf(bf16_hi(w1), ne));
    codes[i].y = (unsigned)f32x4_to_fp8x4(ldexpf(bf16_lo(w2), ne), ldexpf(bf16_hi(w2), ne), ldexpf(bf16_lo(w3), ne),
                                          ldexpf(bf16_hi(w3), ne));
  }
  return e;
}

// Second term of the two-term query that gives bf16-dot accuracy on the fp8
// matrix cores (the role-split kernel with bf16 dots, at most 16 rows per key
// stream). With x = q * 2^-e (the exponent quantize_q_quad takes) and
// c1 = e4m3fn(x) its codes, these are the codes of c2 = 16 (x - c1). x has at
// most 8 significant bits (a bf16 value times a power of two) and c1 keeps
// the top 4 with rounding, so x - c1 has at most 4 and, whenever x is a
// normal e4m3fn magnitude (>= 2^-6), c2 is exact: 2^e (c1 + c2 / 16) = q.
// Below 2^-6 (under 2^-6 / 448 of the row's largest value) the residual is
// rounded to e4m3fn's subnormal grid. Returns the exponent e.
__device__ inline int quantize_q_quad_residual(const i32x4 raw[16], uint2 codes[16]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo((unsigned)raw[i][d])), fabsf(bf16_hi((unsigned)raw[i][d]))));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = q_exponent(amax);
  const int ne = -e;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const unsigned wa = (unsigned)raw[i][2 * half], wb = (unsigned)raw[i][2 * half + 1];
      float x[4] = {ldexpf(bf16_lo(wa), ne), ldexpf(bf16_hi(wa), ne), ldexpf(bf16_lo(wb), ne), ldexpf(bf16_hi(wb), ne)};
      float c1[4];
      fp8x4_to_f32(f32x4_to_fp8x4(x[0], x[1], x[2], x[3]), c1);
      const unsigned c2 = (unsigned)f32x4_to_fp8x4(16.f * (x[0] - c1[0]), 16.f * (x[1] - c1[1]),
                                                   16.f * (x[2] - c1[2]), 16.f * (x[3] - c1[3]));
      if (half == 0) codes[i].x = c2; else codes[i].y = c2;
    }
  }
  return e;
}

// gfx942's e4m3fnuz codes turned into OCP e4m3fn codes of the same value,
// in place in this wave's 4 KiB slice of a landed tile (the fp8 matrix cores
// read OCP codes only). A code whose exponent field is 2 or more is the OCP
// code 8 lower (one less exponent: bias 8 against 7, same mantissa). The 16
// smallest magnitudes (exponent field 0 or 1: multiples k 2^-10 of the scale,
// k = 0 .. 15) become OCP subnormals, multiples of 2^-9, rounded to nearest
// even: odd k moves by 2^-10 of the scale, k = 15 becomes the smallest OCP
// normal. 0x80, fnuz's NaN, becomes 0x80 (-0). Four bytes per 32-bit lane
// word, no byte carries into the next.
__device__ inline unsigned fnuz4_to_ocp4(unsigned x) {
  const unsigned t = x & 0x7f7f7f7fu;                                  // magnitude codes
  const unsigned big = ((t + 0x70707070u) & 0x80808080u) >> 7;          // 1 where t >= 16
  const unsigned bm = big * 0xffu;                                      // 0xff where t >= 16
  const unsigned rb = ((t | 0x80808080u) - 0x08080808u) & 0x7f7f7f7fu;  // t - 8
  const unsigned hh = (t >> 1) & 0x7f7f7f7fu;                           // t / 2
  const unsigned rs = hh + (t & hh & 0x01010101u);                      // t / 2 to nearest even
  return (x & 0x80808080u) | (rb & bm) | (rs & ~bm);
}

// The role-split decode (mla_decode_ws.hip): every fp8-dot decode, and
// bf16-dot decodes of at most 16 rows per key stream (two-term operands).
bool decode_ws_eligible(const DecodeLaunch& d);
hipError_t launch_decode_ws(const DecodeLaunch& d, const KDims& a, hipStream_t st);

// Softmax bookkeeping runs in the log2 domain with a lazily raised running
// max: the max used for exponentials is only raised when a tile's max exceeds
// it by more than tau, so the rescale of the 256 accumulator registers is rare.
// Every p is then at most 2^tau. The fp8 path stores e4m3fn(p * 2^ps_log2)
// with 2^(tau + ps_log2) = 256 <= 448 (the format's largest value), the power
// of two folded into the exponent (exp2(z - m + ps_log2)); the row sums are
// kept in the same scaled units. Scaled probabilities stay normal down to
// p = 2^-11 and representable down to 2^-14 below the running max; tau = 3
// keeps the rescales of the accumulators rare.
template <int DOT> struct Soft;
#ifndef MLA_FP8_TAU
#define MLA_FP8_TAU 3
#endif
template <> struct Soft<1> { static constexpr float tau = MLA_FP8_TAU, ps_log2 = 8 - MLA_FP8_TAU; };
template <> struct Soft<0> { static constexpr float tau = 8.f, ps_log2 = 0.f; };
// The two-term P of the role-split kernel's bf16-dot form (p = c1 + c2 / 16,
// both e4m3fn) keeps about 8 bits only while c1 is normal: tau = 0 and
// 2^8 of scale put that down to 2^-14 below the running max (the single
// term's 2^-11, one binade more than a bf16 P needs for a tail at e^-9).
struct SoftSplit { static constexpr float tau = 0.f, ps_log2 = 8.f; };

}  // namespace mla

// Small device helpers for gfx950: element packing, 16-byte row fragments,
// lane-group reductions with DPP, exp2/log2 on the hardware units, and the
// XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- lane halves
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 lanes of its second.  Applied to two copies of x, the two
// results hold, in every lane l, x[l] and x[l ^ 32] (in some order), so the
// sum or max over the lane pair (l, l ^ 32) is one more VALU operation, with
// no LDS round trip.
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------- element traits
// A row fragment is the 16 bytes one lane owns: 8 bf16 or 4 fp32 elements.
template <int DT>
struct Frag;

template <>
struct Frag<DT_F32> {
  static constexpr int EPL = 4;
  static constexpr int BYTES = 4;
  // acc + <a, b> over the fragment's elements
  __device__ __forceinline__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  }
  __device__ __forceinline__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

template <>
struct Frag<DT_BF16> {
  static constexpr int EPL = 8;
  static constexpr int BYTES = 2;
  // acc + <a, b> with v_dot2c_f32_bf16: exact bf16 products, fp32 accumulation
  __device__ __forceinline__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                          __builtin_bit_cast(bf16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                          __builtin_bit_cast(bf16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                          __builtin_bit_cast(bf16x2_t, b.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                           __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  }
  __device__ __forceinline__ static void unpack(const uint4& u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

// 16-byte fragments per lane of a gather-kernel row.  One (a row spans
// D * bytes / 16 lanes, so a wavefront's load covers whole rows) except for
// the coordinate score on bf16 rows of 64 or more elements: there the vector
// ALUs, not the loads, bound the kernels, and two fragments per lane halve the
// lanes that repeat each edge's score and softmax work (measured on the
// coordinate training workload: forward 78.7 -> 73.4 us, backward 188 -> 169
// us).  With the dot and fixed-weight scores two fragments were slower (the
// dilated backward 274 -> 304 us): a row's 128-byte cache line is then split
// over two load instructions, which doubles the load path's line requests.
constexpr int gather_frags_per_lane(int dt, int D, int score_mode) {
  return dt == DT_BF16 && D >= 64 && score_mode == SM_COORD ? 2 : 1;
}

__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(char* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Streaming stores (non-temporal hint) for output rows written once as whole
// contiguous rows (a wavefront's store covers full cache lines): they pass
// through the L2 without displacing the key/value rows that neighbouring
// queries gather again.  Measured: up to a quarter faster on the gather
// kernels.  Not for scattered partial-line stores (the band kernels' MFMA
// accumulator layout writes 8 or 16 bytes per lane across 32 rows; there the
// hint made stores several times dearer), and the same hint on the owner's
// own-row loads did not help.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st16_stream(char* p, const uint4& v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st8_stream(char* p, const uint2& v) {
  const u32x2_t t = {v.x, v.y};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(p));
}

// Store N fp32 values (N = 4 or 8) as fp32 or bf16 at p (aligned to the size),
// streaming (each output row is written once).
template <int N>
__device__ __forceinline__ void store_vals(char* p, const float* f, bool as_bf16) {
  if (as_bf16) {
    if constexpr (N == 8) {
      st16_stream(p, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])));
    } else {
      st8_stream(p, make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])));
    }
  } else {
#pragma unroll
    for (int c = 0; c < N; c += 4)
      st16_stream(p + 4 * c, make_uint4(__float_as_uint(f[c]), __float_as_uint(f[c + 1]),
                                        __float_as_uint(f[c + 2]), __float_as_uint(f[c + 3])));
  }
}

// ---------------------------------------------------------------- DPP lane-group sums
// DPP controls (CDNA ISA): quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141 (lane k <- 7-k within 8), row_mirror = 0x140 (k <- 15-k).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LG consecutive lanes; every lane of the group
// receives the group's total.
template <int LG>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LG >= 2) x += dpp_f<0xB1>(x);
  if constexpr (LG >= 4) x += dpp_f<0x4E>(x);
  if constexpr (LG >= 8) x += dpp_f<0x141>(x);
  if constexpr (LG >= 16) x += dpp_f<0x140>(x);
  if constexpr (LG >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// ---------------------------------------------------------------- transcendental
// v_exp_f32 (2^x) and v_log_f32 (log2 x) hardware instructions.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- transposing LDS read
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// ---------------------------------------------------------------- padded LDS tiles
// A tile holds 64 rows of 64 bf16 at a row pitch of 144 bytes (128 bytes of
// data, 16 of padding).  With a 36-dword pitch, 16 consecutive rows read at
// one 16-byte chunk cover all 64 banks once, and every read address is one
// per-lane base plus a compile-time offset (a single address register per
// access pattern, whatever the row block, chunk or buffer).
//
// Tiles are filled by direct global -> LDS loads (global_load_lds_dwordx4:
// lane L of an instruction writes bytes [16 L, 16 L + 16) after the
// instruction's LDS base).  The tile is one stream of 576 16-byte slots,
// nine per row (eight data chunks and the padding slot), so nine full
// instructions fill it; a padding slot reloads the row's last chunk, which
// lies in the same cache line.
constexpr int kTileRows = 64;
constexpr int kTilePitch = 144;
constexpr int kTileBytes = kTileRows * kTilePitch;
constexpr int kTileSlots = kTileBytes / 16;  // 576 = 9 instructions of 64 lanes

// Slot assignment of this lane in the (at most three) load instructions its
// wavefront issues per tile: instruction k writes slots 64 (wave + 4 k) +
// lane, i.e. tile row r[k], 16-byte chunk c16[k] / 16 (the padding slot of a
// row reloads its last chunk).  Computed once; opaque to re-derivation.
struct DmaLane {
  int r[3];
  int c16[3];
};
__device__ __forceinline__ DmaLane dma_lane(int wave, int lane) {
  DmaLane d;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int q = 64 * (wave + 4 * k) + lane;  // slot index in the tile
    const int r = q / 9, w = q - 9 * (q / 9);
    d.r[k] = r;
    d.c16[k] = (w < 8 ? w : 7) * 16;
  }
  asm volatile("" : "+v"(d.r[0]), "+v"(d.r[1]), "+v"(d.r[2]), "+v"(d.c16[0]), "+v"(d.c16[1]), "+v"(d.c16[2]));
  return d;
}

// Issue the loads of rows [r0, r0 + 64) of a [T, 64] bf16 tensor (row stride
// st bytes, rows past T clamped to T - 1) into `tile`.  Instruction i of the
// nine is issued by wavefront i % 4 of the workgroup's four.  A tile that
// lies wholly inside the tensor takes one uniform base and a 32-bit per-lane
// offset per instruction, from the precomputed slots `dl`.
__device__ __forceinline__ void tile_issue(const char* base, int64_t st, int r0, int T, char* tile, int wave,
                                           const DmaLane& dl) {
  if (r0 + kTileRows <= T && st < (1 << 24)) {
    const char* b = base + r0 * st;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int i = wave + 4 * k;
      if (i >= kTileSlots / 64) break;  // wave-uniform
      const uint32_t off = (uint32_t)(dl.r[k] * (int)st + dl.c16[k]);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(b + off),
                                       (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int i = wave + 4 * k;
      if (i >= kTileSlots / 64) break;  // wave-uniform
      const int row = r0 + dl.r[k] < T ? r0 + dl.r[k] : T - 1;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + row * st + dl.c16[k]),
                                       (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16, 0, 0);
    }
  }
}

// Wait for this wavefront's direct-to-LDS loads (and every other load).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Per-lane byte offsets of the two tile read patterns.  They are computed
// once and hidden from re-association, so every read below is one register
// (tile + lane offset) plus an immediate offset.
struct TileLane {
  int row;  // row-major reads: row l % 32, chunk l / 32
  int tr;   // transposing reads (see tile_tr4)
};
__device__ __forceinline__ TileLane tile_lane(int lane) {
  const int s = lane & 15, g = lane >> 4, half = lane >> 5;
  TileLane t;
  t.row = (lane & 31) * kTilePitch + half * 16;
  t.tr = ((s >> 2) + 4 * half) * kTilePitch + (16 * (g & 1) + 4 * (s & 3)) * 2;
  asm volatile("" : "+v"(t.row), "+v"(t.tr));
  return t;
}

// 16-byte fragment of row row0 + l % 32, chunk 2 kk + l / 32 (row0 a
// multiple of 32): the A operand rows of a 32 x 32 x 16 MFMA step kk.
__device__ __forceinline__ uint4 tile_ld16(const char* tile, const TileLane& tl, int row0, int kk) {
  return *reinterpret_cast<const uint4*>(tile + tl.row + row0 * kTilePitch + kk * 32);
}

// Transposing read (ds_read_b64_tr_b16: within each group of 16 lanes, lane i
// receives element i % 4 of the 64-bit reads of group lanes i/4, i/4 + 4,
// i/4 + 8, i/4 + 12).  Group lane s reads 4 bf16 of row key0 + 4 half + s/4
// at column d0 + 16 (group % 2) + 4 (s % 4), so lane l receives column
// d0 + l % 32 of rows key0 + 4 half .. key0 + 4 half + 3 (key0 a multiple of
// 8, d0 of 32).
__device__ __forceinline__ uint2 tile_tr4(const char* tile, const TileLane& tl, int key0, int d0) {
  const char* src = tile + tl.tr + key0 * kTilePitch + d0 * 2;
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
  return __builtin_bit_cast(uint2, v);
}

// ---------------------------------------------------------------- progress priority
// The SIMDs issue from the oldest ready wavefront first, so among the
// workgroups that share a compute unit the youngest falls behind and the unit
// idles while it finishes alone.  Wavefronts lower their issue priority as
// they progress (level 3 at the start, 0 near the end; wave-uniform `done` of
// `total`), so the workgroup that is behind gets the issue slots.
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int level = 3 - (4 * done) / (total > 0 ? total : 1);
  switch (level < 0 ? 0 : level) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// ---------------------------------------------------------------- XCD-aware order
// Workgroup b of a launch is dispatched to XCD (b mod 8).  Give each XCD a
// contiguous run of the logical work order, so the (batch, head) slices one
// XCD walks stay resident in that XCD's own L2 instead of being pulled into
// all eight.  Returns -1 for the padding workgroups past `total`.
__device__ __forceinline__ int xcd_logical_block(int total) {
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int b = blockIdx.x;
  const int logical = (b % kNumXcd) * per + b / kNumXcd;
  return logical < total ? logical : -1;
}
// Query-side block order for grouped key/value heads: logical block
// ((b H_kv + hk) nblk + rb) G + g is row block rb of query head hk G + g of
// batch b, so the G query heads that read one key/value head take the same
// row block one after another (on the same XCD), and the key/value rows they
// gather are fetched into that XCD's L2 once for the group instead of once per
// query head.  With G = 1 this is the plain (b, h, rb) order.
struct QueryBlock {
  int b, h, bh, rb;
};
__device__ __forceinline__ QueryBlock query_block(int logical, int nblk, int H, int G) {
  QueryBlock q;
  const int g = logical % G, t = logical / G;
  const int bk = t / nblk;
  q.rb = t - bk * nblk;
  const int Hkv = H / G;
  q.b = bk / Hkv;
  q.h = (bk - q.b * Hkv) * G + g;
  q.bh = q.b * H + q.h;
  return q;
}
inline int xcd_grid(int total) {
  const int per = (total + kNumXcd - 1) / kNumXcd;
  return per * kNumXcd;
}

}  // namespace sa

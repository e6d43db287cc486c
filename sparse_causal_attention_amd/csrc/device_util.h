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

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- element traits
// A row fragment is the 16 bytes one lane owns: 8 bf16 or 4 fp32 elements.
template <int DT>
struct Frag;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(char* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Store N fp32 values (N = 4 or 8) as fp32 or bf16 at p (aligned to the size).
template <int N>
__device__ __forceinline__ void store_vals(char* p, const float* f, bool as_bf16) {
  if (as_bf16) {
    if constexpr (N == 8) {
      st16(p, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                         pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])));
    } else {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
    }
  } else {
#pragma unroll
    for (int c = 0; c < N; c += 4)
      st16(p + 4 * c, make_uint4(__float_as_uint(f[c]), __float_as_uint(f[c + 1]),
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

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 64-bit reads of group lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
// Group lane s here reads 4 consecutive bf16 of row key0 + s/4 of a row-major
// LDS tile, starting at column d0 + 16 * (group % 2) + 4 * (s % 4); lane l
// therefore receives column d0 + l % 32 of rows key0 .. key0 + 3.
__device__ __forceinline__ uint2 lds_tr4(const __bf16* tile, int row_stride, int key0, int d0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const __bf16* src = tile + (key0 + (s >> 2)) * row_stride + d0 + 16 * (g & 1) + 4 * (s & 3);
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
  return __builtin_bit_cast(uint2, r);
}

// ---------------------------------------------------------------- swizzled LDS tiles
// A tile holds 64 rows of 64 bf16 (128 B per row, no padding).  Logical
// 16-byte chunk c of row r sits at physical chunk c ^ f(r), f(r) = (r % 8) ^
// (r / 8 % 2): 16 consecutive rows read at one logical chunk land in 16
// distinct 16-byte bank groups, and the 4 consecutive rows of a transposing
// read never collide either.  Tiles are filled by direct global -> LDS loads
// (global_load_lds_dwordx4: lane L of an instruction writes bytes
// [16 L, 16 L + 16) after the instruction's LDS base), so staging needs no
// registers and no LDS store instructions.
constexpr int kTileRows = 64;
constexpr int kTileRowBytes = 128;
constexpr int kTileBytes = kTileRows * kTileRowBytes;

__device__ __forceinline__ int tile_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int tile_off(int r, int c) { return r * kTileRowBytes + ((c ^ tile_swz(r)) << 4); }

// Issue the loads of rows [r0, r0 + 64) of a [T, 64] bf16 tensor (row stride
// st bytes, rows past T clamped to T - 1) into `tile`.  Wavefront w of the
// four loads rows 16 w .. 16 w + 15 with two instructions of 8 rows.
__device__ __forceinline__ void tile_issue(const char* base, int64_t st, int r0, int T, char* tile, int wave,
                                           int lane) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row0 = wave * 16 + k * 8;  // first tile row written by this instruction
    const int r = row0 + (lane >> 3);
    const int c = (lane & 7) ^ tile_swz(r);  // logical chunk stored in this lane's slot
    const int row = r0 + r < T ? r0 + r : T - 1;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + row * st + c * 16),
                                     (__attribute__((address_space(3))) void*)(tile + row0 * kTileRowBytes),
                                     16, 0, 0);
  }
}

// Wait for this wavefront's direct-to-LDS loads (and every other load).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte fragment: logical chunk c of tile row r.
__device__ __forceinline__ uint4 tile_ld16(const char* tile, int r, int c) {
  return *reinterpret_cast<const uint4*>(tile + tile_off(r, c));
}

// Transposing read from a swizzled tile (see lds_tr4): lane l receives
// column d0 + l % 32 of rows key0 .. key0 + 3 (key0 a multiple of 4, d0 of 32).
__device__ __forceinline__ uint2 tile_tr4(const char* tile, int key0, int d0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int r = key0 + (s >> 2);
  const int col = d0 + 16 * (g & 1) + 4 * (s & 3);
  const char* src = tile + r * kTileRowBytes + (((col >> 3) ^ tile_swz(r)) << 4) + (col & 7) * 2;
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
  return __builtin_bit_cast(uint2, v);
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
inline int xcd_grid(int total) {
  const int per = (total + kNumXcd - 1) / kNumXcd;
  return per * kNumXcd;
}

}  // namespace sa

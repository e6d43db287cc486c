// Band backward: gradients of the sliding-window part on the bf16 matrix
// cores, with the long-range edges of the same rows gathered in the same
// kernel.  A small prepass writes -Delta_i = -<dout_i, o_i> and
// lse_i * log2(e) per row; then one persistent launch works through units of
// two kinds: a dq unit owns 128 query rows, a dk/dv unit owns 128 key rows,
// so every output row has exactly one writer (deterministic, no atomics).
//
//  dq unit, one query row per lane (as in the forward):
//    S^T = K Q^T,  dP^T = V dO^T   (K, V tiles row-major in LDS),
//    P = exp(S - lse),  dS = P (dP - Delta),  Delta_i = <dout_i, o_i>,
//    dq^T += K^T dS^T              (K^T read transposed from the K tile).
//  dk/dv unit, one key row per lane, over the reverse band (queries
//  j .. j+W-1):
//    S = Q K^T,  dP = dO V^T       (Q, dO tiles row-major in LDS),
//    dv^T += dO^T P,  dk^T += Q^T dS   (Q^T, dO^T read transposed from the
//    Q, dO tiles with ds_read_b64_tr_b16).
// Lane layouts are those of v_mfma_f32_32x32x16_bf16 described in the
// forward band kernel; P and dS enter the second product as B operands
// straight from the score registers, with the contraction index ordered as
// the accumulator rows (8*(r/4) + 4*half + r%4).  The dP products start from
// -Delta, so dP - Delta comes out of the matrix cores.
//
// Scheduling.  The grid is a fixed number of workgroups (two per compute
// unit), G per XCD, each XCD owning a contiguous share of row blocks.  With
// G even, workgroups 2h and 2h + 1 take the dq unit and the dk/dv unit of the
// same row block at the same time, row blocks h, h + G/2, h + G/2 * 2, ... of
// the share, swapping the two roles each round: workgroups running side by
// side work on neighbouring row blocks and share K, V, Q, dO rows in the XCD's
// L2, an XCD has G/2 row blocks in flight (a working set that fits its L2
// better than G), and every workgroup alternates the two kinds of unit, which
// together have nearly the same work at every position.  (With G odd,
// workgroup i takes the (dq, dk/dv) pairs i, i + G, ... in turn.)
// Streamed 64-row tiles are double-buffered in LDS and filled by direct
// buffer -> LDS loads; the stream runs on across units: while a unit's last
// tile is computed, the first tile of the next unit is loaded, together with
// the next unit's per-row operands (into registers), so a workgroup never
// waits for a unit's start-up loads.  Each unit's tile count is padded to an
// even number so that every unit starts in the same buffer.  Within a tile the
// two 32-row blocks are processed one after the other; blocks wholly inside
// the band skip the mask.
//
// Delta_i = <dout_i, o_i> equals sum_j P_ij dP_ij up to the rounding of o;
// with the dot-product score the resulting gradient error is far inside the
// bf16 tolerance (the score's 1/sqrt(D) scale damps it).
#include "device_util.h"
#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 128;  // rows (queries or keys) owned per workgroup
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle): the streamed tiles are loaded with buffer_load ... lds.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kTile = 64;   // streamed rows per LDS tile
constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf(const bf16x8& v, int e) { return static_cast<float>(v[e]); }

// A operand X^T[d][row] of a row-major tile for the 16-row step ks in the
// accumulator order (rows 16*ks + 4*half + {0..3} and + 8 + {0..3}),
// d = d0 + l % 32, through the transposing LDS read.
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, const TileLane& tl, int ks, int d0) {
  const uint2 x0 = tile_tr4(tile, tl, 16 * ks, d0);
  const uint2 x1 = tile_tr4(tile, tl, 16 * ks + 8, d0);
  return as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
}

// Accumulator-layout element (dblk, r) of a 64-element bf16 row fetched as
// 8 x 8 bytes: run c = 4*dblk + r/4, element r%4.
__device__ __forceinline__ float acc_elem(const uint2* runs, int dblk, int r) {
  const uint2 w2 = runs[dblk * 4 + (r >> 2)];
  const uint32_t word = (r & 2) ? w2.y : w2.x;
  return (r & 1) ? bf16_hi(word) : bf16_lo(word);
}
__device__ __forceinline__ int acc_col(int dblk, int c4, int half) { return dblk * 32 + 8 * c4 + 4 * half; }

template <bool GRAD_BF16>
__device__ __forceinline__ void store_acc_row(void* base, int64_t off_elems, const f32x16* acc, float mul,
                                              int half) {
#pragma unroll
  for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const float a0 = acc[dblk][4 * c4] * mul, a1 = acc[dblk][4 * c4 + 1] * mul;
      const float a2 = acc[dblk][4 * c4 + 2] * mul, a3 = acc[dblk][4 * c4 + 3] * mul;
      const int col = acc_col(dblk, c4, half);
      if constexpr (GRAD_BF16) {
        *reinterpret_cast<uint2*>(static_cast<char*>(base) + (off_elems + col) * 2) =
            make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
      } else {
        *reinterpret_cast<float4*>(static_cast<char*>(base) + (off_elems + col) * 4) =
            make_float4(a0, a1, a2, a3);
      }
    }
}

// Stores this wavefront's 32 accumulator rows (lane l owns row row0 + l % 32,
// columns 32 dblk + 8 g + 4 half + e in acc[dblk][4 g + e]) as whole fp32
// rows: each 32-column half is written to the wavefront's own LDS region (32
// rows at a 144-byte pitch) and read back so that eight lanes hold one row's
// 128 contiguous bytes, so the global stores cover whole cache lines and
// stream past the L2.  Rows at or past T are not stored.
__device__ __forceinline__ void store_rows_f32(float* lds, char* gbase, int64_t row_bytes, int row0, int T,
                                               const f32x16* acc, float mul) {
  constexpr int kPitch = 36;  // floats per LDS row
  const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int dblk = 0; dblk < 2; ++dblk) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(lds + l32 * kPitch + 8 * g + 4 * half) =
          make_float4(acc[dblk][4 * g] * mul, acc[dblk][4 * g + 1] * mul, acc[dblk][4 * g + 2] * mul,
                      acc[dblk][4 * g + 3] * mul);
    __builtin_amdgcn_wave_barrier();  // the wavefront's LDS accesses stay in this order
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = 8 * k + (lane >> 3), c = lane & 7;
      const float4 v = *reinterpret_cast<const float4*>(lds + rr * kPitch + 4 * c);
      if (row0 + rr < T) {
        char* dst = gbase + (int64_t)(row0 + rr) * row_bytes + (dblk * 32 + 4 * c) * 4;
        const uint4 w = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w));
        st16_stream(dst, w);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------ prepass
// -Delta_i = -<dout_i, o_i> and lse_i * log2(e) for every row.  The negated
// Delta is the initial accumulator of the dP products, so dP - Delta leaves
// the matrix cores ready for dS = P (dP - Delta).  Four lanes per row, 32
// bytes of each of dout and o per lane, 64 rows of one (batch, head) per
// workgroup (measured against eight lanes of 16 bytes: 8.6 -> 7.6 us on the
// band workload; two lanes of 64 bytes: 7.9 us).
constexpr int kPreRows = kThreads / 4;

__global__ __launch_bounds__(kThreads) void band_bwd_prepass_kernel(Params p) {
  const int nblk = (p.T + kPreRows - 1) / kPreRows;
  const int bh = blockIdx.x / nblk;  // uniform
  const int t = (blockIdx.x - bh * nblk) * kPreRows + (threadIdx.x >> 2);
  const int b = bh / p.H, h = bh - b * p.H;
  const int sub = threadIdx.x & 3;
  const int tc = t < p.T ? t : p.T - 1;
  const char* db =
      static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h + (int64_t)tc * p.sdo_t) * 2 + sub * 32;
  const char* ob = static_cast<const char*>(p.o) + (b * p.so_b + h * p.so_h + (int64_t)tc * p.so_t) * 2 + sub * 32;
  const uint4 d0 = ld16(db), d1 = ld16(db + 16);
  const uint4 o0 = ld16(ob), o1 = ld16(ob + 16);
  const float delta = group_sum<4>(Frag<DT_BF16>::dot(d1, o1, Frag<DT_BF16>::dot(d0, o0, 0.f)));
  const int64_t r = (int64_t)bh * p.T + t;
  if (t < p.T && sub == 0) {
    p.ndelta[r] = -delta;
    p.lse2[r] = p.lse[r] * kLog2e;
  }
}

// ------------------------------------------------------------------ units
struct Unit {
  int role;  // 0: dq, 1: dk/dv, -1: no unit
  int b, h, bh;
  int hk;    // key/value head of query head h
  int ng;    // dk/dv: query heads h .. h + ng - 1 walked in turn (the G heads of hk)
  int r0;    // first owned row: query (dq) or key (dk/dv)
  int s0;    // first streamed row: key (dq) or query (dk/dv); a multiple of kTile
  int nt;    // streamed tiles (per query head)
};

__device__ __forceinline__ Unit make_unit(const Params& p, int pair, int role, int nblk) {
  Unit u;
  u.role = role;
  u.bh = pair / nblk;
  const int rb = pair - u.bh * nblk;
  u.b = u.bh / p.H;
  u.h = u.bh - u.b * p.H;
  u.hk = u.h / p.G;
  u.ng = 1;
  u.r0 = rb * kRows;
  const int last = u.r0 + kRows - 1 < p.T - 1 ? u.r0 + kRows - 1 : p.T - 1;
  if (role == 0) {  // keys max(0, r0 - W + 1) .. last
    const int lo = u.r0 - p.W + 1 > 0 ? u.r0 - p.W + 1 : 0;
    u.s0 = (lo / kTile) * kTile;
    u.nt = (last - u.s0) / kTile + 1;
  } else {  // queries r0 .. min(T - 1, last + W - 1)
    const int qhi = last + p.W - 1 < p.T - 1 ? last + p.W - 1 : p.T - 1;
    u.s0 = u.r0;
    u.nt = (qhi - u.s0) / kTile + 1;
  }
  return u;
}

// Per-row operands of a lane's own row, held in registers for the whole
// unit: Q and dO rows (dq) or K and V rows (dk/dv), as MFMA B operands
// (elements 16 kk + 8 half .. + 7), and for dq the row's -Delta and
// lse * log2(e).
struct RowOps {
  bf16x8 x[4], y[4];
  float nd, l2;
};

// (Strides of q, k, v and dout fit 32 bits on the band backward's path, which
// keeps them in one scalar register each instead of two.)
__device__ __forceinline__ const char* tensor_base(const void* t, int64_t sb, int64_t sh, const Unit& u) {
  return static_cast<const char*>(t) + ((int64_t)u.b * (int32_t)sb + (int64_t)u.h * (int32_t)sh) * 2;
}
// K and V live on the unit's key/value head.
__device__ __forceinline__ const char* tensor_base_kv(const void* t, int64_t sb, int64_t sh, const Unit& u) {
  return static_cast<const char*>(t) + ((int64_t)u.b * (int32_t)sb + (int64_t)u.hk * (int32_t)sh) * 2;
}

// Direct loads of a tile's 64 per-row floats (one wavefront, 4 B per lane).
__device__ __forceinline__ void rows_issue(const float* src, int r0, int T, float* dst, int lane) {
  const int row = r0 + lane < T ? r0 + lane : T - 1;
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + row),
                                   (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

// Tile buffers: (a, b, la, lb) of buffer 0 and of buffer 1, and the row
// stage (sx, sy, snd, sl2): 128 rows of the next unit's per-row operands.
// Each its own LDS object (see band_bwd_kernel).
struct Bufs {
  char *a0, *b0, *a1, *b1;
  float *la0, *lb0, *la1, *lb1;
  char *sx, *sy;
  float *snd, *sl2;
  DmaLane dl;  // this lane's slots of the direct tile loads
  // LDS region of wavefront w for store_rows_f32: tile buffer 1, idle from the
  // end of a unit's last tile until the next unit issues its second tile
  __device__ float* store_region(int w) const {
    return reinterpret_cast<float*>((w < 2 ? a1 : b1) + (w & 1) * 32 * 36 * 4);
  }
};

// Rows [r0, r0 + 64) of a bf16 [T, 64] tensor (row stride st bytes, rows
// past T clamped to T - 1) into `tile`, through a buffer resource over the
// tensor's (batch, head) slice: the lane's offset is its clamped slot row
// times st plus its 16-byte column, with no 64-bit address arithmetic (the
// per-load cost of the global form was two dozen instructions).  The slice
// must span fewer than 2^31 bytes; the host sends larger ones to the gather
// kernels.
__device__ __forceinline__ void tile_issue_buf(const char* base, int64_t st, int r0, int T, char* tile,
                                               const DmaLane& dl) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)((int64_t)(T - 1) * st + 128),
                                        kBufferWord3);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int i = wave + 4 * k;
    if (i >= kTileSlots / 64) break;  // wave-uniform
    const int row = r0 + dl.r[k] < T ? r0 + dl.r[k] : T - 1;
    const uint32_t off = (uint32_t)row * (uint32_t)st + (uint32_t)dl.c16[k];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + 1024 * i), 16,
                                             off, 0, 0, 0);
  }
}

// Issue the loads of streamed tile j of unit u: K, V rows (dq) or Q, dO rows
// plus their lse * log2(e) and -Delta (dk/dv).
__device__ __forceinline__ void issue_tile(const Params& p, const Unit& u, int j, char* a, char* bt, float* la,
                                           float* lb, const Bufs& bf) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = u.s0 + j * kTile;
  if (u.role == 0) {
    tile_issue_buf(tensor_base_kv(p.k, p.sk_b, p.sk_h, u), (int32_t)p.sk_t * 2, r0, p.T, a, bf.dl);
    tile_issue_buf(tensor_base_kv(p.v, p.sv_b, p.sv_h, u), (int32_t)p.sv_t * 2, r0, p.T, bt, bf.dl);
  } else {
    tile_issue_buf(tensor_base(p.q, p.sq_b, p.sq_h, u), (int32_t)p.sq_t * 2, r0, p.T, a, bf.dl);
    tile_issue_buf(tensor_base(p.dout, p.sdo_b, p.sdo_h, u), (int32_t)p.sdo_t * 2, r0, p.T, bt, bf.dl);
    if (wave == 0) rows_issue(p.lse2 + (int64_t)u.bh * p.T, r0, p.T, la, lane);
    if (wave == 1) rows_issue(p.ndelta + (int64_t)u.bh * p.T, r0, p.T, lb, lane);
  }
}

// Issue the loads of unit u's per-row operands into the row stage: rows
// r0 .. r0 + 127 of Q and dO (dq) or K and V (dk/dv), and for dq their
// -Delta and lse * log2(e).
__device__ __forceinline__ void issue_stage(const Params& p, const Unit& u, const Bufs& bf) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char *xb, *yb;
  int64_t xs, ys;
  if (u.role == 0) {
    xb = tensor_base(p.q, p.sq_b, p.sq_h, u), xs = (int32_t)p.sq_t * 2;
    yb = tensor_base(p.dout, p.sdo_b, p.sdo_h, u), ys = (int32_t)p.sdo_t * 2;
    if (wave == 2) {
      rows_issue(p.ndelta + (int64_t)u.bh * p.T, u.r0, p.T, bf.snd, lane);
      rows_issue(p.ndelta + (int64_t)u.bh * p.T, u.r0 + 64, p.T, bf.snd + 64, lane);
    }
    if (wave == 3) {
      rows_issue(p.lse2 + (int64_t)u.bh * p.T, u.r0, p.T, bf.sl2, lane);
      rows_issue(p.lse2 + (int64_t)u.bh * p.T, u.r0 + 64, p.T, bf.sl2 + 64, lane);
    }
  } else {
    xb = tensor_base_kv(p.k, p.sk_b, p.sk_h, u), xs = (int32_t)p.sk_t * 2;
    yb = tensor_base_kv(p.v, p.sv_b, p.sv_h, u), ys = (int32_t)p.sv_t * 2;
  }
  tile_issue_buf(xb, xs, u.r0, p.T, bf.sx, bf.dl);
  tile_issue_buf(xb, xs, u.r0 + kTile, p.T, bf.sx + kTileBytes, bf.dl);
  tile_issue_buf(yb, ys, u.r0, p.T, bf.sy, bf.dl);
  tile_issue_buf(yb, ys, u.r0 + kTile, p.T, bf.sy + kTileBytes, bf.dl);
}

// This lane's per-row operands from the row stage (row 32 wave + l % 32).
__device__ __forceinline__ void read_stage(const Unit& u, const Bufs& bf, RowOps& r) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TileLane tl = tile_lane(lane);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    r.x[kk] = as_bf16x8(tile_ld16(bf.sx, tl, wave * 32, kk));
    r.y[kk] = as_bf16x8(tile_ld16(bf.sy, tl, wave * 32, kk));
  }
  if (u.role == 0) {
    r.nd = bf.snd[wave * 32 + (lane & 31)];
    r.l2 = bf.sl2[wave * 32 + (lane & 31)];
  } else {
    r.nd = r.l2 = 0.f;
  }
}

// ------------------------------------------------------------------ dq unit
template <bool GRAD_BF16, bool HAS_DIL, class NextUnit>
__device__ __forceinline__ void dq_unit(const Params& p, const Unit& u, const RowOps& ops, const NextUnit& next_unit,
                                        const Bufs& bf) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const TileLane tl = tile_lane(lane);
  const int qw = u.r0 + wave * 32;
  const int m = qw + l32;
  const int mc = m < p.T ? m : p.T - 1;
  const int W = p.W;
  const float sl2 = p.scale_log2;
  const int ntp = (u.nt + 1) & ~1;

  f32x16 dp_init;  // -Delta of this lane's query row
#pragma unroll
  for (int r = 0; r < 16; ++r) dp_init[r] = ops.nd;
  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][r] = acc[1][r] = 0.f;
  const int wlo = qw - W + 1, whi = qw + 31;

  auto tile = [&](int it, const char* ks, const char* vs, char* kn, char* vn, float* lan, float* lbn) {
    if (it + 1 < u.nt) {
      issue_tile(p, u, it + 1, kn, vn, lan, lbn, bf);  // (kn, vn) were last read in tile it - 1
    } else if (it + 1 == ntp) {
      const Unit nxt = next_unit();  // formed only here, so it holds no registers through the unit
      if (nxt.role >= 0) {
        issue_tile(p, nxt, 0, kn, vn, lan, lbn, bf);  // buffer 0: the next unit's first tile
        issue_stage(p, nxt, bf);                   // read at the start of this unit
      }

    }
    if (it < u.nt) {
      const int kt0 = u.s0 + it * kTile;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int nb0 = kt0 + nb * 32;
        if (nb0 + 31 < wlo || nb0 > whi) continue;  // block outside this wavefront's band
        const bool full = nb0 + 31 <= qw && qw + 31 - nb0 < W && qw + 31 < p.T;
        f32x16 s = mfma32(as_bf16x8(tile_ld16(ks, tl, nb * 32, 0)), ops.x[0], f32x16{});
        f32x16 dp = mfma32(as_bf16x8(tile_ld16(vs, tl, nb * 32, 0)), ops.y[0], dp_init);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk) {
          s = mfma32(as_bf16x8(tile_ld16(ks, tl, nb * 32, kk)), ops.x[kk], s);
          dp = mfma32(as_bf16x8(tile_ld16(vs, tl, nb * 32, kk)), ops.y[kk], dp);
        }
        // dS = P (dP - Delta); dp already holds dP - Delta
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], sl2, -ops.l2));
        if (!full) {
          // key n = nb0 + 8 (r/4) + 4 half + r%4 is in the window iff 0 <= m - n < W
          const int d = m - nb0 - 4 * half;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[r] = (uint32_t)(d - (8 * (r >> 2) + (r & 3))) < (uint32_t)W ? s[r] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = s[r] * dp[r];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bf16x8 dsb;
#pragma unroll
          for (int e = 0; e < 8; ++e) dsb[e] = static_cast<__bf16>(s[8 * h2 + e]);
#pragma unroll
          for (int dblk = 0; dblk < 2; ++dblk)
            acc[dblk] = mfma32(tr_operand(ks, tl, 2 * nb + h2, dblk * 32), dsb, acc[dblk]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int it = 0; it < ntp; it += 2) {
    tile(it, bf.a0, bf.b0, bf.a1, bf.b1, bf.la1, bf.lb1);
    tile(it + 1, bf.a1, bf.b1, bf.a0, bf.b0, bf.la0, bf.lb0);
  }

  if constexpr (HAS_DIL) {
    // long-range edges j = m - d
    const char* kb = tensor_base_kv(p.k, p.sk_b, p.sk_h, u);
    const char* vb = tensor_base_kv(p.v, p.sv_b, p.sv_h, u);
    const int64_t skt = (int32_t)p.sk_t * 2, svt = (int32_t)p.sv_t * 2;
    for (int t = 0; t < p.n_dil; ++t) {
      const int j = mc - p.dil[t];
      const int jj = j < 0 ? 0 : j;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (16 * kk + 8 * half) * 2;
        sp = Frag<DT_BF16>::dot(__builtin_bit_cast(uint4, ops.x[kk]), ld16(kb + jj * skt + off), sp);
        dpp = Frag<DT_BF16>::dot(__builtin_bit_cast(uint4, ops.y[kk]), ld16(vb + jj * svt + off), dpp);
      }
      sp = sum_halves(sp);
      dpp = sum_halves(dpp);
      const float pr = j >= 0 ? fast_exp2(fmaf(sp, sl2, -ops.l2)) : 0.f;
      const float ds = pr * (dpp + ops.nd);
      uint2 kr[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        kr[c] = *reinterpret_cast<const uint2*>(kb + jj * skt + acc_col(c >> 2, c & 3, half) * 2);
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dblk][r] = fmaf(ds, acc_elem(kr, dblk, r), acc[dblk][r]);
    }
  }

  if constexpr (GRAD_BF16) {
    if (m < p.T)
      store_acc_row<GRAD_BF16>(p.dq, u.b * p.sdq_b + u.h * p.sdq_h + (int64_t)m * p.sdq_t, acc, p.scale, half);
  } else {
    store_rows_f32(bf.store_region(wave), static_cast<char*>(p.dq) + (u.b * p.sdq_b + u.h * p.sdq_h) * 4,
                   p.sdq_t * 4, qw, p.T, acc, p.scale);
  }
}

// ------------------------------------------------------------------ dk/dv unit
template <bool GRAD_BF16, bool HAS_DIL, bool GROUPED, class NextUnit>
__device__ __forceinline__ void dkv_unit(const Params& p, const Unit& u, const RowOps& ops, const NextUnit& next_unit,
                                         const Bufs& bf) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const TileLane tl = tile_lane(lane);
  const int kw = u.r0 + wave * 32;
  const int n = kw + l32;
  const int nc = n < p.T ? n : p.T - 1;
  const int W = p.W;
  const float sl2 = p.scale_log2;
  const int ntp = (u.nt + 1) & ~1;
  // query mm is in the reverse band of key n iff 0 <= mm - n < min(W, T - n)
  const int wn = W < p.T - n ? W : (p.T - n > 0 ? p.T - n : 0);

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dk[0][r] = dk[1][r] = dv[0][r] = dv[1][r] = 0.f;
  const int wlo = kw, whi = kw + 31 + W - 1;  // this wavefront's query range

  // uh: the query head whose tiles are streamed (u itself unless the unit
  // covers a group); more: a next head of the group follows, un
  auto tile = [&](const Unit& uh, bool more, const Unit& un, int it, const char* qs, const char* ds, const float* ls,
                  const float* es, char* qn, char* dn, float* ln, float* en) {
    if (it + 1 < u.nt) {
      issue_tile(p, uh, it + 1, qn, dn, ln, en, bf);  // last read in tile it - 1
    } else if (more && it + 1 == ntp) {
      issue_tile(p, un, 0, qn, dn, ln, en, bf);  // buffer 0: the next query head's first tile
    } else if (it + 1 == ntp) {
      const Unit nxt = next_unit();
      if (nxt.role >= 0) {
        issue_tile(p, nxt, 0, qn, dn, ln, en, bf);  // buffer 0: the next unit's first tile
        issue_stage(p, nxt, bf);
      }
    }
    if (it < u.nt) {
      const int mt0 = u.s0 + it * kTile;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int mb0 = mt0 + mb * 32;
        if (mb0 + 31 < wlo || mb0 > whi) continue;
        // every (query, key) of the block inside the band
        const bool full = kw + 31 <= mb0 && mb0 + 31 - kw < W && mb0 + 31 < p.T;
        // dP starts from -Delta of the block's query rows (row 8 (r/4) + 4 half + r%4)
        f32x16 dp_init;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 d4 = *reinterpret_cast<const float4*>(&es[mb * 32 + 8 * g4 + 4 * half]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp_init[4 * g4 + e] = (&d4.x)[e];
        }
        f32x16 s = mfma32(as_bf16x8(tile_ld16(qs, tl, mb * 32, 0)), ops.x[0], f32x16{});
        f32x16 dp = mfma32(as_bf16x8(tile_ld16(ds, tl, mb * 32, 0)), ops.y[0], dp_init);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk) {
          s = mfma32(as_bf16x8(tile_ld16(qs, tl, mb * 32, kk)), ops.x[kk], s);
          dp = mfma32(as_bf16x8(tile_ld16(ds, tl, mb * 32, kk)), ops.y[kk], dp);
        }
        // rows mm = mb0 + 8 (r/4) + 4 half + r%4 of this lane's key column n
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(&ls[mb * 32 + 8 * g4 + 4 * half]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * g4 + e] = fast_exp2(fmaf(s[4 * g4 + e], sl2, -(&l4.x)[e]));
        }
        if (!full) {
          const int d = mb0 + 4 * half - n;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[r] = (uint32_t)(d + 8 * (r >> 2) + (r & 3)) < (uint32_t)wn ? s[r] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = s[r] * dp[r];  // dS = P (dP - Delta)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bf16x8 pb, dsb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[e] = static_cast<__bf16>(s[8 * h2 + e]);
            dsb[e] = static_cast<__bf16>(dp[8 * h2 + e]);
          }
#pragma unroll
          for (int dblk = 0; dblk < 2; ++dblk) {
            dv[dblk] = mfma32(tr_operand(ds, tl, 2 * mb + h2, dblk * 32), pb, dv[dblk]);
            dk[dblk] = mfma32(tr_operand(qs, tl, 2 * mb + h2, dblk * 32), dsb, dk[dblk]);
          }
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  // one query head: its tiles, then its long-range edges
  auto head = [&](const Unit& uh, bool more, const Unit& un) {
  for (int it = 0; it < ntp; it += 2) {
    tile(uh, more, un, it, bf.a0, bf.b0, bf.la0, bf.lb0, bf.a1, bf.b1, bf.la1, bf.lb1);
    tile(uh, more, un, it + 1, bf.a1, bf.b1, bf.la1, bf.lb1, bf.a0, bf.b0, bf.la0, bf.lb0);
  }

  if constexpr (HAS_DIL) {
    // long-range edges: queries i = n + d
    const char* qb = tensor_base(p.q, p.sq_b, p.sq_h, uh);
    const char* dob = tensor_base(p.dout, p.sdo_b, p.sdo_h, uh);
    const int64_t sqt = (int32_t)p.sq_t * 2, sdot = (int32_t)p.sdo_t * 2;
    const float* lseb = p.lse2 + (int64_t)uh.bh * p.T;
    const float* ndelb = p.ndelta + (int64_t)uh.bh * p.T;
    for (int t = 0; t < p.n_dil; ++t) {
      const bool ok = p.dil[t] <= p.T - 1 - nc;
      const int ii = ok ? nc + p.dil[t] : nc;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (16 * kk + 8 * half) * 2;
        sp = Frag<DT_BF16>::dot(ld16(qb + ii * sqt + off), __builtin_bit_cast(uint4, ops.x[kk]), sp);
        dpp = Frag<DT_BF16>::dot(ld16(dob + ii * sdot + off), __builtin_bit_cast(uint4, ops.y[kk]), dpp);
      }
      sp = sum_halves(sp);
      dpp = sum_halves(dpp);
      const float pr = ok ? fast_exp2(fmaf(sp, sl2, -lseb[ii])) : 0.f;
      const float ds = pr * (dpp + ndelb[ii]);
      uint2 qr[8], dr[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = acc_col(c >> 2, c & 3, half) * 2;
        qr[c] = *reinterpret_cast<const uint2*>(qb + ii * sqt + col);
        dr[c] = *reinterpret_cast<const uint2*>(dob + ii * sdot + col);
      }
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dv[dblk][r] = fmaf(pr, acc_elem(dr, dblk, r), dv[dblk][r]);
          dk[dblk][r] = fmaf(ds, acc_elem(qr, dblk, r), dk[dblk][r]);
        }
    }
  }
  };
  if constexpr (GROUPED) {  // the G query heads of key/value head hk, in order
    for (int gi = 0; gi < u.ng; ++gi) {
      Unit uh = u, un = u;
      uh.h += gi;
      uh.bh += gi;
      un.h = uh.h + 1;
      un.bh = uh.bh + 1;
      head(uh, gi + 1 < u.ng, un);
    }
  } else {
    head(u, false, u);
  }

  // key/value head hk: the sums over every query head that reads it
  if constexpr (GRAD_BF16) {
    if (n < p.T) {
      store_acc_row<true>(p.dv, u.b * p.sdv_b + u.hk * p.sdv_h + (int64_t)n * p.sdv_t, dv, 1.f, half);
      store_acc_row<true>(p.dk, u.b * p.sdk_b + u.hk * p.sdk_h + (int64_t)n * p.sdk_t, dk, p.scale, half);
    }
  } else {
    float* lds = bf.store_region(wave);
    store_rows_f32(lds, static_cast<char*>(p.dv) + (u.b * p.sdv_b + u.hk * p.sdv_h) * 4, p.sdv_t * 4, kw, p.T,
                         dv, 1.f);
    store_rows_f32(lds, static_cast<char*>(p.dk) + (u.b * p.sdk_b + u.hk * p.sdk_h) * 4, p.sdk_t * 4, kw, p.T,
                         dk, p.scale);
  }
}

// ------------------------------------------------------------------ kernel
template <bool GRAD_BF16, bool HAS_DIL, bool GROUPED>
__global__ __launch_bounds__(kThreads, 2) void band_bwd_kernel(Params p) {
  // Double-buffered tiles shared by the two unit kinds.  Each buffer is its
  // own LDS object, so the direct loads into one are known not to alias the
  // reads of the other: no wait for the tile in flight is placed before the
  // reads of the tile being computed.
  __shared__ __align__(16) char t0a[kTileBytes], t0b[kTileBytes];
  __shared__ __align__(16) char t1a[kTileBytes], t1b[kTileBytes];
  __shared__ __align__(16) float r0a[kTile], r0b[kTile], r1a[kTile], r1b[kTile];
  __shared__ __align__(16) char stx[2 * kTileBytes], sty[2 * kTileBytes];
  __shared__ __align__(16) float stnd[kRows], stl2[kRows];
  const Bufs bf{t0a, t0b, t1a, t1b, r0a, r0b, r1a, r1b, stx, sty, stnd, stl2,
                dma_lane(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63)};

  const int nblk = (p.T + kRows - 1) / kRows;
  const int xcd = blockIdx.x % kNumXcd, g = blockIdx.x / kNumXcd;
  const int wgs_per_xcd = gridDim.x / kNumXcd;
  Unit none;
  none.role = -1;
  none.b = none.h = none.bh = none.hk = none.ng = none.r0 = none.s0 = none.nt = 0;
  // Without grouped heads: workgroup g of an XCD takes the (dq, dk/dv) unit
  // pairs pbeg + g, pbeg + g + G, ... of that XCD's contiguous share of
  // (head, row block) pairs.  With G query heads per key/value head, a dk/dv
  // unit walks all G query heads (G times a dq unit's work): the first half
  // of an XCD's workgroups take those, the second half the dq units, so both
  // halves carry the same work.
  constexpr bool grouped = GROUPED;  // p.G > 1
  const int nitems = grouped ? p.B * p.Hkv * nblk : p.B * p.H * nblk;  // (b, hk, rb) or (b, h, rb)
  const int per_xcd = (nitems + kNumXcd - 1) / kNumXcd;
  const int ibeg = xcd * per_xcd;
  const int iend = ibeg + per_xcd < nitems ? ibeg + per_xcd : nitems;
  const int wh = wgs_per_xcd / 2, wd = wgs_per_xcd - wh;  // grouped: >= 1 each
  const bool kv_wg = grouped && g < wh;
  auto unit_at = [&](int k) {
    if (!grouped) {
      if ((wgs_per_xcd & 1) == 0) {
        // workgroups 2h and 2h + 1 take the dq and the dk/dv unit of the same
        // row block at the same time (roles swapping each round): an XCD works
        // on half as many row blocks at once, a smaller working set in its L2,
        // and every workgroup still alternates the two kinds of unit
        const int pair = ibeg + (g >> 1) + k * (wgs_per_xcd >> 1);
        return pair < iend ? make_unit(p, pair, (k + g) & 1, nblk) : none;
      }
      // unit k: pair ibeg + g + (k / 2) wgs_per_xcd, dq unit then dk/dv unit
      const int pair = ibeg + g + (k >> 1) * wgs_per_xcd;
      return pair < iend ? make_unit(p, pair, k & 1, nblk) : none;
    }
    int t, hq;
    if (kv_wg) {
      t = ibeg + g + k * wh;
      hq = 0;
    } else {
      const int d = (g - wh) + k * wd;  // over this XCD's (item, query head of the group) pairs
      t = ibeg + d / p.G;
      hq = d - (d / p.G) * p.G;
    }
    if (t >= iend) return none;
    const int bk = t / nblk, rb = t - bk * nblk;
    const int b = bk / p.Hkv, hk = bk - b * p.Hkv;
    Unit u = make_unit(p, (b * p.H + hk * p.G + hq) * nblk + rb, kv_wg ? 1 : 0, nblk);
    if (kv_wg) u.ng = p.G;
    return u;
  };

  Unit cur = unit_at(0);
  if (cur.role < 0) return;  // uniform over the workgroup
  issue_tile(p, cur, 0, bf.a0, bf.b0, bf.la0, bf.lb0, bf);
  issue_stage(p, cur, bf);
  wait_vmem();
  __syncthreads();
  for (int k = 0;; ++k) {
    progress_priority(kv_wg ? k * p.G : k, 4);  // about four units' work per workgroup
    auto next_unit = [&]() { return unit_at(k + 1); };
    RowOps ops;
    read_stage(cur, bf, ops);  // the stage is refilled only in this unit's last tile
    if (cur.role == 0)
      dq_unit<GRAD_BF16, HAS_DIL>(p, cur, ops, next_unit, bf);
    else
      dkv_unit<GRAD_BF16, HAS_DIL, GROUPED>(p, cur, ops, next_unit, bf);
    const Unit nxt = unit_at(k + 1);
    if (nxt.role < 0) break;
    __syncthreads();  // the row stores' LDS regions are tile buffer 1, which the next unit refills
    cur = nxt;
  }
}

template <bool GRAD_BF16, bool HAS_DIL>
hipError_t launch(const Params& p, hipStream_t s) {
  const int64_t pre_blocks = (int64_t)p.B * p.H * ((p.T + kPreRows - 1) / kPreRows);
  hipLaunchKernelGGL(band_bwd_prepass_kernel, dim3((unsigned)pre_blocks), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (p.T + kRows - 1) / kRows;
  // two resident workgroups per compute unit, a multiple of the XCD count,
  // no more than there are units to take; with grouped heads at least two per
  // XCD (one for each kind of unit)
  int grid = 2 * device_cu_count();
  const int64_t per_xcd = p.G > 1 ? 2 * (((int64_t)p.B * p.Hkv * nblk + kNumXcd - 1) / kNumXcd)
                                  : ((int64_t)p.B * p.H * nblk + kNumXcd - 1) / kNumXcd;
  if (grid > per_xcd * kNumXcd) grid = (int)(per_xcd * kNumXcd);
  grid = (grid / kNumXcd) * kNumXcd;
  const int min_grid = p.G > 1 ? 2 * kNumXcd : kNumXcd;
  if (grid < min_grid) grid = min_grid;
  if (p.G > 1)
    hipLaunchKernelGGL((band_bwd_kernel<GRAD_BF16, HAS_DIL, true>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((band_bwd_kernel<GRAD_BF16, HAS_DIL, false>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_band_bwd(const Params& p, hipStream_t s) {
  if (p.n_dil > 0) return p.grad_bf16 ? launch<true, true>(p, s) : launch<false, true>(p, s);
  return p.grad_bf16 ? launch<true, false>(p, s) : launch<false, false>(p, s);
}

}  // namespace sa

// Band kernels: the sliding-window part of the graph as dense LDS-staged
// tiles on the bf16 matrix cores, with the long-range edges of the same
// query rows gathered in the same workgroup.
//
// The window of query i is keys (i-W, i] (MiniGPT Part 6, "A mask is not
// enough": keep j iff j <= i and i - j < w).  A block of consecutive queries
// therefore needs one contiguous key range, and within it the scores form a
// dense matrix product with a band mask -- the part of the computation that
// really is a contraction, so it runs on MFMA.  Unlike the page's chunked
// version (stacked 2W-wide copies of K and V, a [T/W, W, 2W] score tensor),
// nothing is materialised in HBM: 64-key tiles of K and V pass through LDS,
// the scores live in MFMA accumulators, and key tiles that lie wholly outside
// a wavefront's band are skipped, so the work stays proportional to the
// band's edges.
//
// Layouts (v_mfma_f32_32x32x16_bf16; lane l, half = l / 32, l32 = l % 32):
//   A operand: A[m = l32][k = 8*half + e]        (8 bf16, e = 0..7)
//   B operand: B[k = 8*half + e][n = l32]
//   C (16 fp32): C[m = 8*(r/4) + 4*half + r%4][n = l32], r = 0..15
// Scores are computed transposed, S^T = K Q^T, so that C's column index is
// the query: lane l owns query row l32 of its wavefront, and its 16 values
// per 32-key block are keys 8*(r/4) + 4*half + r%4.  The output is computed
// transposed too, O^T = V^T P^T: P^T is the B operand, which lane l supplies
// from its own score registers (keys in the order above), and V^T comes from
// the row-major V tile through the transposing LDS read.  Each lane keeps the
// running max, sum and output accumulator of exactly one query row, and the
// two lanes l, l+32 of a row combine with one cross-half exchange per tile.
#include "device_util.h"
#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;
constexpr int kBQ = 128;        // query rows per workgroup: 4 wavefronts x 32
constexpr int kBK = 64;         // keys per LDS tile
constexpr int kThreads = 256;
constexpr int kG = 1;           // long-range edges per step (two measured 0.8 % slower on 2^26 rows)

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + <a, b> over 8 bf16 pairs with v_dot2c_f32_bf16 (exact bf16 products,
// fp32 accumulation).
__device__ __forceinline__ float dot8_bf16(const bf16x8& a, const uint4& b, float acc) {
  const uint4 ua = __builtin_bit_cast(uint4, a);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ua.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ua.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ua.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ua.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
  return acc;
}

// A operand V^T[d][key] for keys 16*ks + 4*half + {0..3} and + 8 + {0..3}
// (the accumulator order of the score registers), d = d0 + l % 32, read from
// the row-major V tile with the transposing LDS read.
__device__ __forceinline__ bf16x8 vt_operand(const char* vs, const TileLane& tl, int ks, int d0) {
  const uint2 x0 = tile_tr4(vs, tl, 16 * ks, d0);
  const uint2 x1 = tile_tr4(vs, tl, 16 * ks + 8, d0);
  return as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
}

template <bool HAS_DIL, int HW>
__global__ __launch_bounds__(kThreads, 4) void band_fwd_kernel(Params p) {
  // Two buffers of swizzled 64-key tiles, each its own LDS object: the loads
  // into one buffer are then known not to alias the reads of the other, so
  // no wait for the tile in flight is placed before the reads of the tile
  // being computed.
  __shared__ __align__(16) char K0[kTileBytes], V0[kTileBytes];
  __shared__ __align__(16) char K1[kTileBytes], V1[kTileBytes];

  // The four wavefronts take HW query heads of one key/value head (HW = 4
  // or 2 when the grouping allows, else 1) times 4 / HW groups of 32 query
  // rows: with grouped heads the wavefronts then share the key band and every
  // K/V tile serves several heads.
  constexpr int hw = HW;
  constexpr int rows = kBQ / hw;  // query rows of the workgroup
  const int nblk = (p.T + rows - 1) / rows;
  const int ngrp = p.H / hw;  // head groups
  const int logical = xcd_logical_block(p.B * ngrp * nblk);
  if (logical < 0) return;
  const int bg = logical / nblk;
  const int rb = nblk - 1 - (logical - bg * nblk);  // late (longest) query blocks first
  const int b = bg / ngrp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = (bg - b * ngrp) * hw + wave % hw;  // this wavefront's query head
  const int bh = b * p.H + h;
  const int l32 = lane & 31, half = lane >> 5;
  const TileLane tl = tile_lane(lane);
  const DmaLane dl = dma_lane(wave, lane);
  const int q0 = rb * rows;
  const int qw = q0 + (wave / hw) * 32;
  const int m = qw + l32;
  const int mc = m < p.T ? m : p.T - 1;

  const char* qbase = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h) * 2;
  const int hk = h / p.G;  // key/value head shared by G query heads (the same for every wavefront)
  const char* kbase = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h) * 2;
  const char* vbase = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2;

  const int W = p.W;
  const int lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
  const int hi = q0 + rows - 1 < p.T - 1 ? q0 + rows - 1 : p.T - 1;
  const int kfirst = (lo / kBK) * kBK;
  const int ntiles = (hi - kfirst) / kBK + 1;

  // Tiles are taken in a rotated order: step `it` works on the tile whose
  // absolute index is congruent to it modulo ntiles, so neighbouring query
  // blocks (whose key ranges overlap) load the same tile at the same step and
  // the first reads of K and V from HBM spread over the whole kernel instead
  // of all falling into its first two steps.
  const int a0 = kfirst / kBK;
  const int rot = (ntiles - a0 % ntiles) % ntiles;
  auto tile_key = [&](int it) {
    const int r = it + rot;
    return kfirst + (r < ntiles ? r : r - ntiles) * kBK;
  };
  tile_issue(kbase, skt, tile_key(0), p.T, K0, wave, dl);
  tile_issue(vbase, svt, tile_key(0), p.T, V0, wave, dl);

  // Q^T as B operand: lane holds q[m][16*kk + 8*half + e]
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = as_bf16x8(ld16(qbase + mc * sqt + (16 * kk + 8 * half) * 2));

  wait_vmem();
  __syncthreads();

  // running max (raw score units), row sum (this lane's keys), O^T accumulator
  float mrun = -INFINITY, lrun = 0.f;
  f32x16 oacc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) oacc[0][r] = oacc[1][r] = 0.f;

  const int wlo = qw - W + 1, whi = qw + 31;  // this wavefront's key range
  const float sl2 = p.scale_log2;             // > 0

  // One 32 x 32 block of (key, query) pairs; the band mask is applied unless
  // every pair of the block lies inside the band.
  auto block = [&](const char* ks, const char* vs, int nb, int nb0, bool full) {
    f32x16 sacc;
    sacc = mfma32(as_bf16x8(tile_ld16(ks, tl, nb * 32, 0)), qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) sacc = mfma32(as_bf16x8(tile_ld16(ks, tl, nb * 32, kk)), qf[kk], sacc);
    if (!full) {
      // key n = nb0 + 8 (r/4) + 4 half + r%4 is in the window iff 0 <= m - n < W
      const int d = m - nb0 - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = (uint32_t)(d - (8 * (r >> 2) + (r & 3))) < (uint32_t)W;
        sacc[r] = ok ? sacc[r] : -INFINITY;
      }
    }
    float tmax = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sacc[r]);
    tmax = max_halves(tmax);
    // Lazy rescale: the reference max moves only when a score exceeds it by
    // more than 8 (log2 units), so exponents stay <= 8 and the accumulator
    // is rescaled rarely.
    const bool grow = tmax * sl2 > mrun * sl2 + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? tmax : mrun;
      const float alpha = mrun == -INFINITY ? 0.f : fast_exp2((mrun - mnew) * sl2);
      lrun *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        oacc[0][r] *= alpha;
        oacc[1][r] *= alpha;
      }
      mrun = mnew;
    }
    const float neg = mrun == -INFINITY ? 0.f : -mrun * sl2;  // no valid key yet: p = 0
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = fast_exp2(fmaf(sacc[r], sl2, neg));
      sacc[r] = pv;
      psum += pv;
    }
    lrun += psum;
    // O^T += V^T P^T, 16 keys per step
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(sacc[8 * h2 + e]);
      const int ks4 = 2 * nb + h2;
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk)
        oacc[dblk] = mfma32(vt_operand(vs, tl, ks4, dblk * 32), pb, oacc[dblk]);
    }
  };

  // Tile `it` from (ks, vs) while the next one streams into (kn, vn), the
  // buffers last read in tile it - 1.
  auto tile = [&](int it, const char* ks, const char* vs, char* kn, char* vn) {
    // The SIMDs favour their oldest wavefront, so of the workgroups sharing a
    // compute unit the last-started one would finish alone at low occupancy;
    // lowering the priority with progress keeps them level.
    progress_priority(it, ntiles);
    const int kt0 = tile_key(it);
    if (it + 1 < ntiles) {
      const int kt1 = tile_key(it + 1);
      tile_issue(kbase, skt, kt1, p.T, kn, wave, dl);
      tile_issue(vbase, svt, kt1, p.T, vn, wave, dl);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nb0 = kt0 + nb * 32;
      if (nb0 + 31 < wlo || nb0 > whi) continue;  // block outside this wavefront's band
      // every (query, key) of the 32 x 32 block inside the band
      const bool full = nb0 + 31 <= qw && qw + 31 - nb0 < W && qw + 31 < p.T;
      block(ks, vs, nb, nb0, full);
    }
    wait_vmem();  // this wavefront's share of the next tile has landed
    __syncthreads();
  };

  for (int it = 0; it < ntiles; it += 2) {
    tile(it, K0, V0, K1, V1);
    if (it + 1 < ntiles) tile(it + 1, K1, V1, K0, V0);
  }

  // ---- long-range edges j = m - d: row gathers in the accumulator layout
  if constexpr (HAS_DIL) {
    for (int t0 = 0; t0 < p.n_dil; t0 += kG) {
      uint4 kr[kG][4];
      uint2 vr[kG][8];
      int j[kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const int t = t0 + g;
        j[g] = t < p.n_dil ? mc - p.dil[t] : -1;
        const int jj = j[g] < 0 ? 0 : j[g];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kr[g][kk] = ld16(kbase + jj * skt + (16 * kk + 8 * half) * 2);
#pragma unroll
        for (int c = 0; c < 8; ++c)
          vr[g][c] = *reinterpret_cast<const uint2*>(vbase + jj * svt +
                                                     ((c >> 2) * 32 + 8 * (c & 3) + 4 * half) * 2);
      }
      float s[kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        float part = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) part = dot8_bf16(qf[kk], kr[g][kk], part);
        s[g] = part;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        s[g] = sum_halves(s[g]);
        s[g] = j[g] >= 0 ? s[g] : -INFINITY;
        tmax = fmaxf(tmax, s[g]);
      }
      const bool grow = tmax * sl2 > mrun * sl2 + 8.f;
      const float mnew = grow ? tmax : mrun;
      const float alpha = grow ? (mrun == -INFINITY ? 0.f : fast_exp2((mrun - mnew) * sl2)) : 1.f;
      mrun = mnew;
      const float neg = mrun == -INFINITY ? 0.f : -mrun * sl2;
      float pg[kG], psum = 0.f;
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        pg[g] = fast_exp2(fmaf(s[g], sl2, neg));
        psum += pg[g];
      }
      // both halves see the same edge: count its weight once in the row sum
      lrun = fmaf(lrun, alpha, half == 0 ? psum : 0.f);
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = oacc[dblk][r] * alpha;
#pragma unroll
          for (int g = 0; g < kG; ++g) {
            const uint2 w2 = vr[g][dblk * 4 + (r >> 2)];
            const uint32_t word = (r & 2) ? w2.y : w2.x;
            const float vv = (r & 1) ? bf16_hi(word) : bf16_lo(word);
            acc = fmaf(pg[g], vv, acc);
          }
          oacc[dblk][r] = acc;
        }
    }
  }

  // ---- finish: O = acc / l, lse = m + log l (natural log).  The rows go out
  // whole: each wavefront writes its 32 bf16 rows into one of the (now idle)
  // tile buffers at a 144-byte pitch, reads them back as 128 contiguous bytes
  // per eight lanes, and stores whole cache lines with streaming stores
  // (instead of 8-byte pieces scattered over 32 rows).
  const float ltot = sum_halves(lrun);
  const float inv = 1.f / ltot;
  char* stage = wave == 0 ? K0 : wave == 1 ? V0 : wave == 2 ? K1 : V1;  // every wavefront is past the last tile
#pragma unroll
  for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint2 w2 = make_uint2(pack_bf16x2(oacc[dblk][4 * g4] * inv, oacc[dblk][4 * g4 + 1] * inv),
                                  pack_bf16x2(oacc[dblk][4 * g4 + 2] * inv, oacc[dblk][4 * g4 + 3] * inv));
      *reinterpret_cast<uint2*>(stage + l32 * kTilePitch + (dblk * 32 + 8 * g4 + 4 * half) * 2) = w2;
    }
  __builtin_amdgcn_wave_barrier();  // the wavefront's LDS accesses stay in this order
  char* obase = static_cast<char*>(p.o) + (b * p.so_b + h * p.so_h) * 2;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = 8 * k + (lane >> 3), c = lane & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + rr * kTilePitch + c * 16);
    if (qw + rr < p.T) st16_stream(obase + (int64_t)(qw + rr) * p.so_t * 2 + c * 16, v);
  }
  if (half == 0 && m < p.T) st_stream(p.lse + (int64_t)bh * p.T + m, (mrun * sl2 + fast_log2(ltot)) * kLn2);
}

}  // namespace

bool band_supported(int dtype, int D, int score_mode, int64_t W) {
  return dtype == DT_BF16 && D == kD && score_mode == SM_DOT && W >= 16;
}

int band_rows_per_block() { return kBQ; }

template <int HW>
hipError_t launch_hw(const Params& p, hipStream_t s) {
  const int rows = kBQ / HW;
  const int nblk = (p.T + rows - 1) / rows;
  const int grid = xcd_grid(p.B * (p.H / HW) * nblk);
  if (p.n_dil > 0)
    hipLaunchKernelGGL((band_fwd_kernel<true, HW>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((band_fwd_kernel<false, HW>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_band_fwd(const Params& p, hipStream_t s) {
  // query heads per workgroup: as many of a key/value head's group as divide four
  if (p.G % 4 == 0) return launch_hw<4>(p, s);
  if (p.G % 2 == 0) return launch_hw<2>(p, s);
  return launch_hw<1>(p, s);
}

}  // namespace sa

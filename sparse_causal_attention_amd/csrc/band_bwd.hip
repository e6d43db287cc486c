// Band backward: gradients of the sliding-window part on the bf16 matrix
// cores, with the long-range edges of the same rows gathered in the same
// kernels.  Deterministic and atomic-free: one kernel owns each query row
// (dq), another each key row (dk, dv).
//
//  dq kernel, one query row per lane (as in the forward):
//    S^T = K Q^T,  dP^T = V dO^T   (K, V tiles row-major in LDS),
//    P = exp(S - lse),  dS = P (dP - Delta),  Delta_i = <dout_i, o_i>,
//    dq^T += K^T dS^T              (K^T tile in LDS; dS^T from registers).
//    Delta is written to the workspace for the second kernel.
//  dk/dv kernel, one key row per lane, over the reverse band (queries
//  j .. j+W-1):
//    S = Q K^T,  dP = dO V^T       (Q, dO tiles row-major in LDS),
//    dv^T += dO^T P,  dk^T += Q^T dS   (Q^T, dO^T tiles in LDS).
// Lane layouts are those of v_mfma_f32_32x32x16_bf16 described in the
// forward band kernel; P and dS enter the second product as B operands
// straight from the score registers, with the contraction index ordered as
// the accumulator rows (8*(r/4) + 4*half + r%4).
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

constexpr int kD = 64;
constexpr int kRows = 128;      // rows (queries or keys) owned per workgroup
constexpr int kTile = 64;       // streamed rows per LDS tile
constexpr int kRow = kD + 8;    // row-major tile stride, bf16 (144 B)
constexpr int kTRow = kTile + 4;  // transposed tile stride, bf16 (136 B)
constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32, 64); }

// Stage rows [r0, r0 + 64) of a [T, 64] bf16 tensor into LDS: row-major
// (when rm != nullptr) and transposed (when tr != nullptr).  Rows past T are
// clamped to T - 1 (their products are masked by the callers).
__device__ __forceinline__ void stage_tile(const char* base, int64_t st, int r0, int T, __bf16* rm,
                                           __bf16* tr) {
  const int tid = threadIdx.x;
  const int r = tid >> 2, c = (tid & 3) * 2;
  const int row = r0 + r < T ? r0 + r : T - 1;
  const uint4 x0 = ld16(base + row * st + c * 16);
  const uint4 x1 = ld16(base + row * st + (c + 1) * 16);
  if (rm != nullptr) {
    *reinterpret_cast<uint4*>(&rm[r * kRow + c * 8]) = x0;
    *reinterpret_cast<uint4*>(&rm[r * kRow + (c + 1) * 8]) = x1;
  }
  if (tr != nullptr) {
    const bf16x8 a0 = as_bf16x8(x0), a1 = as_bf16x8(x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tr[(c * 8 + e) * kTRow + r] = a0[e];
      tr[((c + 1) * 8 + e) * kTRow + r] = a1[e];
    }
  }
}

// A operand from a transposed tile: row d, the 16-row step ks in the
// accumulator order (rows 16*ks + 4*half + {0..3} and + 8 + {0..3}).
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tr, int d, int ks, int half) {
  const __bf16* row = &tr[d * kTRow + 16 * ks + 4 * half];
  const uint2 x0 = *reinterpret_cast<const uint2*>(row);
  const uint2 x1 = *reinterpret_cast<const uint2*>(row + 8);
  return as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
}

__device__ __forceinline__ float bf(const bf16x8& v, int e) { return static_cast<float>(v[e]); }

// Accumulator-layout element (dblk, r) of a 64-element bf16 row fetched as
// 8 x 8 bytes: c = 4*dblk + r/4 picks the 4-element run, r%4 the element.
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

// ------------------------------------------------------------------ dq
template <bool GRAD_BF16>
__global__ __launch_bounds__(kThreads) void band_bwd_dq_kernel(Params p) {
  __shared__ __align__(16) __bf16 Ks[kTile * kRow];
  __shared__ __align__(16) __bf16 Kt[kD * kTRow];
  __shared__ __align__(16) __bf16 Vs[kTile * kRow];

  const int nblk = (p.T + kRows - 1) / kRows;
  const int logical = xcd_logical_block(p.B * p.H * nblk);
  if (logical < 0) return;
  const int bh = logical / nblk;
  const int rb = nblk - 1 - (logical - bh * nblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int q0 = rb * kRows, qw = q0 + wave * 32;
  const int m = qw + l32;
  const int mc = m < p.T ? m : p.T - 1;

  const char* qb = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h) * 2;
  const char* kb = static_cast<const char*>(p.k) + (b * p.sk_b + h * p.sk_h) * 2;
  const char* vb = static_cast<const char*>(p.v) + (b * p.sv_b + h * p.sv_h) * 2;
  const char* ob = static_cast<const char*>(p.o) + (b * p.so_b + h * p.so_h) * 2;
  const char* dob = static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2, sot = p.so_t * 2,
                sdot = p.sdo_t * 2;

  bf16x8 qf[4], df[4];
  float delta = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int off = (16 * kk + 8 * half) * 2;
    qf[kk] = as_bf16x8(ld16(qb + mc * sqt + off));
    df[kk] = as_bf16x8(ld16(dob + mc * sdot + off));
    const bf16x8 of = as_bf16x8(ld16(ob + mc * sot + off));
#pragma unroll
    for (int e = 0; e < 8; ++e) delta = fmaf(bf(df[kk], e), bf(of, e), delta);
  }
  delta += xhalf(delta);
  if (half == 0 && m < p.T) p.delta[(int64_t)bh * p.T + m] = delta;
  const float lse2 = p.lse[(int64_t)bh * p.T + mc] * kLog2e;
  const float sl2 = p.scale_log2;
  const int W = p.W;

  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][r] = acc[1][r] = 0.f;

  const int lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
  const int hi = q0 + kRows - 1 < p.T - 1 ? q0 + kRows - 1 : p.T - 1;
  const int wlo = qw - W + 1, whi = qw + 31;

  for (int kt0 = (lo / kTile) * kTile; kt0 <= hi; kt0 += kTile) {
    __syncthreads();
    stage_tile(kb, skt, kt0, p.T, Ks, Kt);
    stage_tile(vb, svt, kt0, p.T, Vs, nullptr);
    __syncthreads();
    if (kt0 + kTile - 1 < wlo || kt0 > whi) continue;

    f32x16 s[2], dp[2];
    bool on[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nb0 = kt0 + nb * 32;
      on[nb] = !(nb0 + 31 < wlo || nb0 > whi);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][r] = dp[nb][r] = 0.f;
      if (on[nb]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int off = (nb * 32 + l32) * kRow + 16 * kk + 8 * half;
          s[nb] = mfma32(*reinterpret_cast<const bf16x8*>(&Ks[off]), qf[kk], s[nb]);
          dp[nb] = mfma32(*reinterpret_cast<const bf16x8*>(&Vs[off]), df[kk], dp[nb]);
        }
      }
    }
    // dS = P (dP - Delta), masked to the band
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = kt0 + nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const bool ok = on[nb] && n <= m && m - n < W;
        const float pr = ok ? fast_exp2(s[nb][r] * sl2 - lse2) : 0.f;
        s[nb][r] = pr * (dp[nb][r] - delta);
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int nb = ks >> 1;
      if (!on[nb]) continue;
      bf16x8 dsb;
#pragma unroll
      for (int e = 0; e < 8; ++e) dsb[e] = static_cast<__bf16>(s[nb][8 * (ks & 1) + e]);
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk)
        acc[dblk] = mfma32(tr_operand(Kt, dblk * 32 + l32, ks, half), dsb, acc[dblk]);
    }
  }

  // long-range edges j = m - d
  for (int t = 0; t < p.n_dil; ++t) {
    const int j = mc - p.dil[t];
    const int jj = j < 0 ? 0 : j;
    float sp = 0.f, dpp = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = (16 * kk + 8 * half) * 2;
      const bf16x8 kv = as_bf16x8(ld16(kb + jj * skt + off));
      const bf16x8 vv = as_bf16x8(ld16(vb + jj * svt + off));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sp = fmaf(bf(qf[kk], e), bf(kv, e), sp);
        dpp = fmaf(bf(df[kk], e), bf(vv, e), dpp);
      }
    }
    sp += xhalf(sp);
    dpp += xhalf(dpp);
    const float pr = j >= 0 ? fast_exp2(sp * sl2 - lse2) : 0.f;
    const float ds = pr * (dpp - delta);
    uint2 kr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kr[c] = *reinterpret_cast<const uint2*>(kb + jj * skt + acc_col(c >> 2, c & 3, half) * 2);
#pragma unroll
    for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dblk][r] = fmaf(ds, acc_elem(kr, dblk, r), acc[dblk][r]);
  }

  if (m >= p.T) return;
  store_acc_row<GRAD_BF16>(p.dq, b * p.sdq_b + h * p.sdq_h + (int64_t)m * p.sdq_t, acc, p.scale, half);
}

// ------------------------------------------------------------------ dk, dv
template <bool GRAD_BF16>
__global__ __launch_bounds__(kThreads) void band_bwd_dkv_kernel(Params p) {
  __shared__ __align__(16) __bf16 Qs[kTile * kRow];
  __shared__ __align__(16) __bf16 Qt[kD * kTRow];
  __shared__ __align__(16) __bf16 Ds[kTile * kRow];
  __shared__ __align__(16) __bf16 Dt[kD * kTRow];
  __shared__ float Ls[kTile], Dl[kTile];

  const int nblk = (p.T + kRows - 1) / kRows;
  const int logical = xcd_logical_block(p.B * p.H * nblk);
  if (logical < 0) return;
  const int bh = logical / nblk;
  const int rb = logical - bh * nblk;  // early key blocks see the longest query ranges
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int k0 = rb * kRows, kw = k0 + wave * 32;
  const int n = kw + l32;
  const int nc = n < p.T ? n : p.T - 1;

  const char* qb = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h) * 2;
  const char* kb = static_cast<const char*>(p.k) + (b * p.sk_b + h * p.sk_h) * 2;
  const char* vb = static_cast<const char*>(p.v) + (b * p.sv_b + h * p.sv_h) * 2;
  const char* dob = static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2, sdot = p.sdo_t * 2;
  const float* lseb = p.lse + (int64_t)bh * p.T;
  const float* delb = p.delta + (int64_t)bh * p.T;

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int off = (16 * kk + 8 * half) * 2;
    kf[kk] = as_bf16x8(ld16(kb + nc * skt + off));
    vf[kk] = as_bf16x8(ld16(vb + nc * svt + off));
  }
  const float sl2 = p.scale_log2;
  const int W = p.W;

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dk[0][r] = dk[1][r] = dv[0][r] = dv[1][r] = 0.f;

  const int hi_key = k0 + kRows - 1 < p.T - 1 ? k0 + kRows - 1 : p.T - 1;
  const int qlo = k0;
  const int qhi = hi_key + W - 1 < p.T - 1 ? hi_key + W - 1 : p.T - 1;
  const int wlo = kw, whi = kw + 31 + W - 1;  // this wavefront's query range

  for (int mt0 = (qlo / kTile) * kTile; mt0 <= qhi; mt0 += kTile) {
    __syncthreads();
    stage_tile(qb, sqt, mt0, p.T, Qs, Qt);
    stage_tile(dob, sdot, mt0, p.T, Ds, Dt);
    if (tid < kTile) {
      const int row = mt0 + tid < p.T ? mt0 + tid : p.T - 1;
      Ls[tid] = lseb[row] * kLog2e;
      Dl[tid] = delb[row];
    }
    __syncthreads();
    if (mt0 + kTile - 1 < wlo || mt0 > whi) continue;

    f32x16 s[2], dp[2];
    bool on[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int mb0 = mt0 + mb * 32;
      on[mb] = !(mb0 + 31 < wlo || mb0 > whi);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = dp[mb][r] = 0.f;
      if (on[mb]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int off = (mb * 32 + l32) * kRow + 16 * kk + 8 * half;
          s[mb] = mfma32(*reinterpret_cast<const bf16x8*>(&Qs[off]), kf[kk], s[mb]);
          dp[mb] = mfma32(*reinterpret_cast<const bf16x8*>(&Ds[off]), vf[kk], dp[mb]);
        }
      }
    }
    // P and dS for rows m = mt0 + 32 mb + 8 (r/4) + 4 half + r%4, key n
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mi = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int mm = mt0 + mi;
        const bool ok = on[mb] && n <= mm && mm - n < W && mm < p.T;
        const float pr = ok ? fast_exp2(s[mb][r] * sl2 - Ls[mi]) : 0.f;
        s[mb][r] = pr;
        dp[mb][r] = pr * (dp[mb][r] - Dl[mi]);
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mb = ks >> 1;
      if (!on[mb]) continue;
      bf16x8 pb, dsb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[e] = static_cast<__bf16>(s[mb][8 * (ks & 1) + e]);
        dsb[e] = static_cast<__bf16>(dp[mb][8 * (ks & 1) + e]);
      }
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk) {
        dv[dblk] = mfma32(tr_operand(Dt, dblk * 32 + l32, ks, half), pb, dv[dblk]);
        dk[dblk] = mfma32(tr_operand(Qt, dblk * 32 + l32, ks, half), dsb, dk[dblk]);
      }
    }
  }

  // long-range edges: queries i = n + d
  for (int t = 0; t < p.n_dil; ++t) {
    const int i = nc + p.dil[t];
    const int ii = i < p.T ? i : p.T - 1;
    float sp = 0.f, dpp = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = (16 * kk + 8 * half) * 2;
      const bf16x8 qv = as_bf16x8(ld16(qb + ii * sqt + off));
      const bf16x8 dv8 = as_bf16x8(ld16(dob + ii * sdot + off));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sp = fmaf(bf(qv, e), bf(kf[kk], e), sp);
        dpp = fmaf(bf(dv8, e), bf(vf[kk], e), dpp);
      }
    }
    sp += xhalf(sp);
    dpp += xhalf(dpp);
    const float pr = i < p.T ? fast_exp2(sp * sl2 - lseb[ii] * kLog2e) : 0.f;
    const float ds = pr * (dpp - delb[ii]);
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

  if (n >= p.T) return;
  store_acc_row<GRAD_BF16>(p.dv, b * p.sdv_b + h * p.sdv_h + (int64_t)n * p.sdv_t, dv, 1.f, half);
  store_acc_row<GRAD_BF16>(p.dk, b * p.sdk_b + h * p.sdk_h + (int64_t)n * p.sdk_t, dk, p.scale, half);
}

template <bool GRAD_BF16>
hipError_t launch(const Params& p, hipStream_t s) {
  const int nblk = (p.T + kRows - 1) / kRows;
  const int grid = xcd_grid(p.B * p.H * nblk);
  hipLaunchKernelGGL(band_bwd_dq_kernel<GRAD_BF16>, dim3(grid), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(band_bwd_dkv_kernel<GRAD_BF16>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_band_bwd(const Params& p, hipStream_t s) {
  return p.grad_bf16 ? launch<true>(p, s) : launch<false>(p, s);
}

}  // namespace sa

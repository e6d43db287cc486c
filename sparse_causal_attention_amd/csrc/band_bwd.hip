// Band backward: gradients of the sliding-window part on the bf16 matrix
// cores, with the long-range edges of the same rows gathered in the same
// kernel.  A small prepass writes Delta_i = <dout_i, o_i> and lse_i * log2(e)
// per row; then one launch with two kinds of workgroup: a dq workgroup owns
// 128 query rows, a dk/dv workgroup owns 128 key rows, so every output row has
// exactly one writer (deterministic, no atomics).  The two kinds of the same
// row block are adjacent in the launch order and so run on the same XCD,
// where they share the K, V, Q, dO rows in L2.
//
//  dq role, one query row per lane (as in the forward):
//    S^T = K Q^T,  dP^T = V dO^T   (K, V tiles row-major in LDS),
//    P = exp(S - lse),  dS = P (dP - Delta),  Delta_i = <dout_i, o_i>,
//    dq^T += K^T dS^T              (K^T read transposed from the K tile).
//  dk/dv role, one key row per lane, over the reverse band (queries
//  j .. j+W-1):
//    S = Q K^T,  dP = dO V^T       (Q, dO tiles row-major in LDS),
//    dv^T += dO^T P,  dk^T += Q^T dS   (Q^T, dO^T read transposed from the
//    Q, dO tiles with ds_read_b64_tr_b16).
// Lane layouts are those of v_mfma_f32_32x32x16_bf16 described in the
// forward band kernel; P and dS enter the second product as B operands
// straight from the score registers, with the contraction index ordered as
// the accumulator rows (8*(r/4) + 4*half + r%4).
//
// Streamed 64-row tiles are double-buffered in LDS and filled by direct
// global -> LDS loads into swizzled rows: the loads of tile t+1 are in flight
// while tile t is computed, one barrier per tile, no staging registers.
// Within a tile the two 32-row blocks are processed one after the other to
// keep the score registers at 32 per lane; blocks wholly inside the band skip
// the mask.
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
constexpr int kTile = 64;   // streamed rows per LDS tile
constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float bf(const bf16x8& v, int e) { return static_cast<float>(v[e]); }

// A operand X^T[d][row] of a row-major tile for the 16-row step ks in the
// accumulator order (rows 16*ks + 4*half + {0..3} and + 8 + {0..3}),
// d = d0 + l % 32, through the transposing LDS read.
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int ks, int d0, int lane, int half) {
  const uint2 x0 = tile_tr4(tile, 16 * ks + 4 * half, d0, lane);
  const uint2 x1 = tile_tr4(tile, 16 * ks + 8 + 4 * half, d0, lane);
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

// ------------------------------------------------------------------ prepass
// Delta_i = <dout_i, o_i> and lse_i * log2(e) for every row; 8 lanes per row.
__global__ __launch_bounds__(kThreads) void band_bwd_prepass_kernel(Params p) {
  const int rows_per_block = kThreads / 8;
  const int64_t gr = (int64_t)blockIdx.x * rows_per_block + (threadIdx.x >> 3);
  const int64_t nrows = (int64_t)p.B * p.H * p.T;
  const bool ok = gr < nrows;
  const int64_t r = ok ? gr : nrows - 1;
  const int t = (int)(r % p.T);
  const int64_t bh = r / p.T;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const int sub = threadIdx.x & 7;
  const uint4 d = ld16(static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h + t * p.sdo_t) * 2 + sub * 16);
  const uint4 o = ld16(static_cast<const char*>(p.o) + (b * p.so_b + h * p.so_h + t * p.so_t) * 2 + sub * 16);
  const float delta = group_sum<8>(Frag<DT_BF16>::dot(d, o, 0.f));
  if (ok && sub == 0) {
    p.delta[r] = delta;
    p.lse2[r] = p.lse[r] * kLog2e;
  }
}

// ------------------------------------------------------------------ dq role
struct DqSmem {
  char Ks[2][kTileBytes];
  char Vs[2][kTileBytes];
};

template <bool GRAD_BF16, bool HAS_DIL>
__device__ __forceinline__ void dq_role(const Params& p, int logical, int nblk, DqSmem& sm) {
  const int bh = logical / nblk;
  const int rb = nblk - 1 - (logical - bh * nblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int q0 = rb * kRows, qw = q0 + wave * 32;
  const int m = qw + l32;
  const int mc = m < p.T ? m : p.T - 1;

  const char* qb = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h) * 2;
  const char* kb = static_cast<const char*>(p.k) + (b * p.sk_b + h * p.sk_h) * 2;
  const char* vb = static_cast<const char*>(p.v) + (b * p.sv_b + h * p.sv_h) * 2;
  const char* dob = static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2, sdot = p.sdo_t * 2;
  const int W = p.W;

  const int lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
  const int hi = q0 + kRows - 1 < p.T - 1 ? q0 + kRows - 1 : p.T - 1;
  const int kfirst = (lo / kTile) * kTile;
  const int ntiles = (hi - kfirst) / kTile + 1;

  tile_issue(kb, skt, kfirst, p.T, sm.Ks[0], wave, lane);
  tile_issue(vb, svt, kfirst, p.T, sm.Vs[0], wave, lane);

  bf16x8 qf[4], df[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int off = (16 * kk + 8 * half) * 2;
    qf[kk] = as_bf16x8(ld16(qb + mc * sqt + off));
    df[kk] = as_bf16x8(ld16(dob + mc * sdot + off));
  }
  const float delta = p.delta[(int64_t)bh * p.T + mc];
  const float lse2 = p.lse2[(int64_t)bh * p.T + mc];
  const float sl2 = p.scale_log2;

  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][r] = acc[1][r] = 0.f;
  const int wlo = qw - W + 1, whi = qw + 31;
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int kt0 = kfirst + it * kTile;
    if (it + 1 < ntiles) {  // the other buffer was last read in iteration it - 1
      tile_issue(kb, skt, kt0 + kTile, p.T, sm.Ks[cur ^ 1], wave, lane);
      tile_issue(vb, svt, kt0 + kTile, p.T, sm.Vs[cur ^ 1], wave, lane);
    }
    const char* ks = sm.Ks[cur];
    const char* vs = sm.Vs[cur];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nb0 = kt0 + nb * 32;
      if (nb0 + 31 < wlo || nb0 > whi) continue;  // block outside this wavefront's band
      const bool full = nb0 + 31 <= qw && qw + 31 - nb0 < W && qw + 31 < p.T;
      const int kr = nb * 32 + l32;
      f32x16 s = mfma32(as_bf16x8(tile_ld16(ks, kr, half)), qf[0], f32x16{});
      f32x16 dp = mfma32(as_bf16x8(tile_ld16(vs, kr, half)), df[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < 4; ++kk) {
        s = mfma32(as_bf16x8(tile_ld16(ks, kr, 2 * kk + half)), qf[kk], s);
        dp = mfma32(as_bf16x8(tile_ld16(vs, kr, 2 * kk + half)), df[kk], dp);
      }
      // dS = P (dP - Delta)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(fmaf(s[r], sl2, -lse2));
        if (!full) {
          const int n = nb0 + 8 * (r >> 2) + 4 * half + (r & 3);
          pr = ((n <= m) & (m - n < W)) ? pr : 0.f;
        }
        s[r] = pr * (dp[r] - delta);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) dsb[e] = static_cast<__bf16>(s[8 * h2 + e]);
#pragma unroll
        for (int dblk = 0; dblk < 2; ++dblk)
          acc[dblk] = mfma32(tr_operand(ks, 2 * nb + h2, dblk * 32, lane, half), dsb, acc[dblk]);
      }
    }
    wait_vmem();
    __syncthreads();
  }

  if constexpr (HAS_DIL) {
    // long-range edges j = m - d
    for (int t = 0; t < p.n_dil; ++t) {
      const int j = mc - p.dil[t];
      const int jj = j < 0 ? 0 : j;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (16 * kk + 8 * half) * 2;
        sp = Frag<DT_BF16>::dot(__builtin_bit_cast(uint4, qf[kk]), ld16(kb + jj * skt + off), sp);
        dpp = Frag<DT_BF16>::dot(__builtin_bit_cast(uint4, df[kk]), ld16(vb + jj * svt + off), dpp);
      }
      sp += xhalf(sp);
      dpp += xhalf(dpp);
      const float pr = j >= 0 ? fast_exp2(fmaf(sp, sl2, -lse2)) : 0.f;
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
  }

  if (m >= p.T) return;
  store_acc_row<GRAD_BF16>(p.dq, b * p.sdq_b + h * p.sdq_h + (int64_t)m * p.sdq_t, acc, p.scale, half);
}

// ------------------------------------------------------------------ dk/dv role
struct DkvSmem {
  char Qs[2][kTileBytes];
  char Ds[2][kTileBytes];
  float Ls[2][kTile];  // lse * log2(e) of the tile's query rows
  float Dl[2][kTile];  // Delta of the tile's query rows
};

// Direct loads of the tile's 64 per-row floats (one wavefront, 4 B per lane).
__device__ __forceinline__ void rows_issue(const float* src, int r0, int T, float* dst, int lane) {
  const int row = r0 + lane < T ? r0 + lane : T - 1;
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + row),
                                   (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

template <bool GRAD_BF16, bool HAS_DIL>
__device__ __forceinline__ void dkv_role(const Params& p, int logical, int nblk, DkvSmem& sm) {
  const int bh = logical / nblk;
  const int rb = logical - bh * nblk;  // early key blocks see the longest query ranges
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int k0 = rb * kRows, kw = k0 + wave * 32;
  const int n = kw + l32;
  const int nc = n < p.T ? n : p.T - 1;

  const char* qb = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h) * 2;
  const char* kb = static_cast<const char*>(p.k) + (b * p.sk_b + h * p.sk_h) * 2;
  const char* vb = static_cast<const char*>(p.v) + (b * p.sv_b + h * p.sv_h) * 2;
  const char* dob = static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2, sdot = p.sdo_t * 2;
  const float* lseb = p.lse2 + (int64_t)bh * p.T;
  const float* delb = p.delta + (int64_t)bh * p.T;
  const int W = p.W;

  const int hi_key = k0 + kRows - 1 < p.T - 1 ? k0 + kRows - 1 : p.T - 1;
  const int qhi = hi_key + W - 1 < p.T - 1 ? hi_key + W - 1 : p.T - 1;
  const int mfirst = k0;  // a multiple of the tile height
  const int ntiles = (qhi - mfirst) / kTile + 1;

  auto issue = [&](int mt0, int buf) {
    tile_issue(qb, sqt, mt0, p.T, sm.Qs[buf], wave, lane);
    tile_issue(dob, sdot, mt0, p.T, sm.Ds[buf], wave, lane);
    if (wave == 0) rows_issue(lseb, mt0, p.T, sm.Ls[buf], lane);
    if (wave == 1) rows_issue(delb, mt0, p.T, sm.Dl[buf], lane);
  };
  issue(mfirst, 0);

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int off = (16 * kk + 8 * half) * 2;
    kf[kk] = as_bf16x8(ld16(kb + nc * skt + off));
    vf[kk] = as_bf16x8(ld16(vb + nc * svt + off));
  }
  const float sl2 = p.scale_log2;

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dk[0][r] = dk[1][r] = dv[0][r] = dv[1][r] = 0.f;
  const int wlo = kw, whi = kw + 31 + W - 1;  // this wavefront's query range
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int mt0 = mfirst + it * kTile;
    if (it + 1 < ntiles) issue(mt0 + kTile, cur ^ 1);  // last read in iteration it - 1
    const char* qs = sm.Qs[cur];
    const char* ds = sm.Ds[cur];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int mb0 = mt0 + mb * 32;
      if (mb0 + 31 < wlo || mb0 > whi) continue;
      // every (query, key) of the block inside the band
      const bool full = kw + 31 <= mb0 && mb0 + 31 - kw < W && mb0 + 31 < p.T;
      const int qr = mb * 32 + l32;
      f32x16 s = mfma32(as_bf16x8(tile_ld16(qs, qr, half)), kf[0], f32x16{});
      f32x16 dp = mfma32(as_bf16x8(tile_ld16(ds, qr, half)), vf[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < 4; ++kk) {
        s = mfma32(as_bf16x8(tile_ld16(qs, qr, 2 * kk + half)), kf[kk], s);
        dp = mfma32(as_bf16x8(tile_ld16(ds, qr, 2 * kk + half)), vf[kk], dp);
      }
      // rows m = mb0 + 8 (r/4) + 4 half + r%4 of this lane's key column n
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int mi0 = mb * 32 + 8 * g4 + 4 * half;
        const float4 l4 = *reinterpret_cast<const float4*>(&sm.Ls[cur][mi0]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.Dl[cur][mi0]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float pr = fast_exp2(fmaf(s[r], sl2, -lv[e]));
          if (!full) {
            const int mm = mt0 + mi0 + e;
            pr = ((n <= mm) & (mm - n < W) & (mm < p.T)) ? pr : 0.f;
          }
          s[r] = pr;
          dp[r] = pr * (dp[r] - dl[e]);
        }
      }
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
          dv[dblk] = mfma32(tr_operand(ds, 2 * mb + h2, dblk * 32, lane, half), pb, dv[dblk]);
          dk[dblk] = mfma32(tr_operand(qs, 2 * mb + h2, dblk * 32, lane, half), dsb, dk[dblk]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }

  if constexpr (HAS_DIL) {
    // long-range edges: queries i = n + d
    for (int t = 0; t < p.n_dil; ++t) {
      const bool ok = p.dil[t] <= p.T - 1 - nc;
      const int ii = ok ? nc + p.dil[t] : nc;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (16 * kk + 8 * half) * 2;
        sp = Frag<DT_BF16>::dot(ld16(qb + ii * sqt + off), __builtin_bit_cast(uint4, kf[kk]), sp);
        dpp = Frag<DT_BF16>::dot(ld16(dob + ii * sdot + off), __builtin_bit_cast(uint4, vf[kk]), dpp);
      }
      sp += xhalf(sp);
      dpp += xhalf(dpp);
      const float pr = ok ? fast_exp2(fmaf(sp, sl2, -lseb[ii])) : 0.f;
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
  }

  if (n >= p.T) return;
  store_acc_row<GRAD_BF16>(p.dv, b * p.sdv_b + h * p.sdv_h + (int64_t)n * p.sdv_t, dv, 1.f, half);
  store_acc_row<GRAD_BF16>(p.dk, b * p.sdk_b + h * p.sdk_h + (int64_t)n * p.sdk_t, dk, p.scale, half);
}

constexpr size_t kSmemBytes = sizeof(DkvSmem) > sizeof(DqSmem) ? sizeof(DkvSmem) : sizeof(DqSmem);

template <bool GRAD_BF16, bool HAS_DIL>
__global__ __launch_bounds__(kThreads, 2) void band_bwd_kernel(Params p) {
  __shared__ __align__(1024) unsigned char smem[kSmemBytes];
  const int nblk = (p.T + kRows - 1) / kRows;
  const int logical = xcd_logical_block(2 * p.B * p.H * nblk);
  if (logical < 0) return;
  // the dq and dk/dv workgroups of one row block are adjacent: same XCD
  if ((logical & 1) == 0)
    dq_role<GRAD_BF16, HAS_DIL>(p, logical >> 1, nblk, *reinterpret_cast<DqSmem*>(smem));
  else
    dkv_role<GRAD_BF16, HAS_DIL>(p, logical >> 1, nblk, *reinterpret_cast<DkvSmem*>(smem));
}

template <bool GRAD_BF16, bool HAS_DIL>
hipError_t launch(const Params& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.H * p.T;
  const int pre_rows = kThreads / 8;
  hipLaunchKernelGGL(band_bwd_prepass_kernel, dim3((unsigned)((rows + pre_rows - 1) / pre_rows)),
                     dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (p.T + kRows - 1) / kRows;
  const int grid = xcd_grid(2 * p.B * p.H * nblk);
  hipLaunchKernelGGL((band_bwd_kernel<GRAD_BF16, HAS_DIL>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_band_bwd(const Params& p, hipStream_t s) {
  if (p.n_dil > 0) return p.grad_bf16 ? launch<true, true>(p, s) : launch<false, true>(p, s);
  return p.grad_bf16 ? launch<true, false>(p, s) : launch<false, false>(p, s);
}

}  // namespace sa

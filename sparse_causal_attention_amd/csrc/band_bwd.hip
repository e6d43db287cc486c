// Band backward: gradients of the sliding-window part on the bf16 matrix
// cores, with the long-range edges of the same rows gathered in the same
// kernel.  One launch, two kinds of workgroup: a dq workgroup owns 128 query
// rows, a dk/dv workgroup owns 128 key rows, so every output row has exactly
// one writer (deterministic, no atomics).  The two kinds of the same row
// block are adjacent in the launch order and so run on the same XCD, where
// they share the K, V, Q, dO rows in L2.
//
//  dq role, one query row per lane (as in the forward):
//    S^T = K Q^T,  dP^T = V dO^T   (K, V tiles row-major in LDS),
//    P = exp(S - lse),  dS = P (dP - Delta),  Delta_i = <dout_i, o_i>,
//    dq^T += K^T dS^T              (K^T read transposed from the K tile).
//  dk/dv role, one key row per lane, over the reverse band (queries
//  j .. j+W-1), computing the Delta of each staged query tile itself from
//  its dO and o rows:
//    S = Q K^T,  dP = dO V^T       (Q, dO tiles row-major in LDS),
//    dv^T += dO^T P,  dk^T += Q^T dS   (Q^T, dO^T read transposed from the
//    Q, dO tiles with ds_read_b64_tr_b16).
// Lane layouts are those of v_mfma_f32_32x32x16_bf16 described in the
// forward band kernel; P and dS enter the second product as B operands
// straight from the score registers, with the contraction index ordered as
// the accumulator rows (8*(r/4) + 4*half + r%4).
//
// Streamed 64-row tiles are double-buffered in LDS: the global loads of tile
// t+1 are in flight while tile t is computed, one barrier per tile.  Within a
// tile the two 32-row blocks are processed one after the other to keep the
// score registers at 32 per lane; blocks wholly inside the band skip the mask.
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
constexpr int kRows = 128;        // rows (queries or keys) owned per workgroup
constexpr int kTile = 64;         // streamed rows per LDS tile
constexpr int kRow = kD + 8;      // row-major tile stride, bf16 (144 B)
constexpr int kThreads = 256;
constexpr int kRM = kTile * kRow;  // elements of a row-major tile

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float bf(const bf16x8& v, int e) { return static_cast<float>(v[e]); }

// One thread's share of a 64-row tile of a [T, 64] bf16 tensor: rows
// (2 kp, 2 kp + 1), 16-byte chunk c, kp = tid / 8, c = tid % 8 (a wavefront
// reads 16 whole consecutive rows).  Rows past T are clamped to T - 1; their
// products are masked by the callers.
struct PairRegs {
  uint4 a, b;
};

__device__ __forceinline__ void pair_load(PairRegs& r, const char* base, int64_t st, int r0, int T) {
  const int tid = threadIdx.x;
  const int kp = tid >> 3, c = tid & 7;
  const int x0 = r0 + 2 * kp < T ? r0 + 2 * kp : T - 1;
  const int x1 = r0 + 2 * kp + 1 < T ? r0 + 2 * kp + 1 : T - 1;
  r.a = ld16(base + x0 * st + c * 16);
  r.b = ld16(base + x1 * st + c * 16);
}

__device__ __forceinline__ void pair_store(const PairRegs& r, __bf16* rm) {
  const int tid = threadIdx.x;
  const int kp = tid >> 3, c = tid & 7;
  *reinterpret_cast<uint4*>(&rm[(2 * kp) * kRow + c * 8]) = r.a;
  *reinterpret_cast<uint4*>(&rm[(2 * kp + 1) * kRow + c * 8]) = r.b;
}

// A operand X^T[d][row] of a row-major [row][d] tile for the 16-row step ks
// in the accumulator order (rows 16*ks + 4*half + {0..3} and + 8 + {0..3}),
// d = d0 + l % 32, through the transposing LDS read.
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* rm, int ks, int d0, int lane, int half) {
  const uint2 x0 = lds_tr4(rm, kRow, 16 * ks + 4 * half, d0, lane);
  const uint2 x1 = lds_tr4(rm, kRow, 16 * ks + 8 + 4 * half, d0, lane);
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

// ------------------------------------------------------------------ dq
// LDS of the dq role, carved from the kernel's shared buffer
struct DqSmem {
  __bf16 Ks[2][kRM];
  __bf16 Vs[2][kRM];
};

template <bool GRAD_BF16, bool HAS_DIL>
__device__ __forceinline__ void dq_role(const Params& p, int logical, int nblk, DqSmem& sm) {
  auto& Ks = sm.Ks;
  auto& Vs = sm.Vs;
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
  const char* ob = static_cast<const char*>(p.o) + (b * p.so_b + h * p.so_h) * 2;
  const char* dob = static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2, sot = p.so_t * 2,
                sdot = p.sdo_t * 2;
  const int W = p.W;

  const int lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
  const int hi = q0 + kRows - 1 < p.T - 1 ? q0 + kRows - 1 : p.T - 1;
  const int kfirst = (lo / kTile) * kTile;
  const int ntiles = (hi - kfirst) / kTile + 1;

  PairRegs pk, pv;
  pair_load(pk, kb, skt, kfirst, p.T);
  pair_load(pv, vb, svt, kfirst, p.T);

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
  const float lse2 = p.lse[(int64_t)bh * p.T + mc] * kLog2e;
  const float sl2 = p.scale_log2;

  pair_store(pk, Ks[0]);
  pair_store(pv, Vs[0]);
  if (ntiles > 1) {
    pair_load(pk, kb, skt, kfirst + kTile, p.T);
    pair_load(pv, vb, svt, kfirst + kTile, p.T);
  }
  __syncthreads();

  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][r] = acc[1][r] = 0.f;
  const int wlo = qw - W + 1, whi = qw + 31;

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int kt0 = kfirst + it * kTile;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nb0 = kt0 + nb * 32;
      if (nb0 + 31 < wlo || nb0 > whi) continue;  // block outside this wavefront's band
      const bool full = nb0 + 31 <= qw && qw + 31 - nb0 < W && qw + 31 < p.T;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (nb * 32 + l32) * kRow + 16 * kk + 8 * half;
        s = mfma32(*reinterpret_cast<const bf16x8*>(&Ks[cur][off]), qf[kk], s);
        dp = mfma32(*reinterpret_cast<const bf16x8*>(&Vs[cur][off]), df[kk], dp);
      }
      // dS = P (dP - Delta)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(fmaf(s[r], sl2, -lse2));
        if (!full) {
          const int n = nb0 + 8 * (r >> 2) + 4 * half + (r & 3);
          pr = (n <= m && m - n < W) ? pr : 0.f;
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
          acc[dblk] = mfma32(tr_operand(Ks[cur], 2 * nb + h2, dblk * 32, lane, half), dsb, acc[dblk]);
      }
    }
    if (it + 1 < ntiles) {
      pair_store(pk, Ks[cur ^ 1]);
      pair_store(pv, Vs[cur ^ 1]);
      if (it + 2 < ntiles) {
        pair_load(pk, kb, skt, kt0 + 2 * kTile, p.T);
        pair_load(pv, vb, svt, kt0 + 2 * kTile, p.T);
      }
    }
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

// ------------------------------------------------------------------ dk, dv
// LDS of the dk/dv role
struct DkvSmem {
  __bf16 Qs[2][kRM];
  __bf16 Ds[2][kRM];
  float Ls[2][kTile];
  float Dl[2][kTile];
};

template <bool GRAD_BF16, bool HAS_DIL>
__device__ __forceinline__ void dkv_role(const Params& p, int logical, int nblk, DkvSmem& sm) {
  auto& Qs = sm.Qs;
  auto& Ds = sm.Ds;
  auto& Ls = sm.Ls;
  auto& Dl = sm.Dl;
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
  const char* ob = static_cast<const char*>(p.o) + (b * p.so_b + h * p.so_h) * 2;
  const int64_t sqt = p.sq_t * 2, skt = p.sk_t * 2, svt = p.sv_t * 2, sdot = p.sdo_t * 2,
                sot = p.so_t * 2;
  const float* lseb = p.lse + (int64_t)bh * p.T;
  const int W = p.W;

  const int hi_key = k0 + kRows - 1 < p.T - 1 ? k0 + kRows - 1 : p.T - 1;
  const int qhi = hi_key + W - 1 < p.T - 1 ? hi_key + W - 1 : p.T - 1;
  const int mfirst = k0;  // a multiple of the tile height
  const int ntiles = (qhi - mfirst) / kTile + 1;

  PairRegs pq, pd, po;
  float pl = 0.f;
  auto load_tile = [&](int mt0) {
    pair_load(pq, qb, sqt, mt0, p.T);
    pair_load(pd, dob, sdot, mt0, p.T);
    pair_load(po, ob, sot, mt0, p.T);
    if (tid < kTile) {
      const int row = mt0 + tid < p.T ? mt0 + tid : p.T - 1;
      pl = lseb[row] * kLog2e;
    }
  };
  auto store_tile = [&](int buf) {
    pair_store(pq, Qs[buf]);
    pair_store(pd, Ds[buf]);
    // Delta of the tile's two rows of this thread: 8-element partial dots of
    // dout and o, summed over the 8 consecutive lanes holding those rows
    const float da = group_sum<8>(Frag<DT_BF16>::dot(pd.a, po.a, 0.f));
    const float db = group_sum<8>(Frag<DT_BF16>::dot(pd.b, po.b, 0.f));
    if ((tid & 7) == 0) {
      const int kp = tid >> 3;
      Dl[buf][2 * kp] = da;
      Dl[buf][2 * kp + 1] = db;
    }
    if (tid < kTile) Ls[buf][tid] = pl;
  };
  load_tile(mfirst);

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int off = (16 * kk + 8 * half) * 2;
    kf[kk] = as_bf16x8(ld16(kb + nc * skt + off));
    vf[kk] = as_bf16x8(ld16(vb + nc * svt + off));
  }
  const float sl2 = p.scale_log2;

  store_tile(0);
  if (ntiles > 1) load_tile(mfirst + kTile);
  __syncthreads();

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dk[0][r] = dk[1][r] = dv[0][r] = dv[1][r] = 0.f;
  const int wlo = kw, whi = kw + 31 + W - 1;  // this wavefront's query range

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int mt0 = mfirst + it * kTile;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int mb0 = mt0 + mb * 32;
      if (mb0 + 31 < wlo || mb0 > whi) continue;
      // every (query, key) of the block inside the band
      const bool full = kw + 31 <= mb0 && mb0 + 31 - kw < W && mb0 + 31 < p.T;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (mb * 32 + l32) * kRow + 16 * kk + 8 * half;
        s = mfma32(*reinterpret_cast<const bf16x8*>(&Qs[cur][off]), kf[kk], s);
        dp = mfma32(*reinterpret_cast<const bf16x8*>(&Ds[cur][off]), vf[kk], dp);
      }
      // rows m = mb0 + 8 (r/4) + 4 half + r%4 of this lane's key column n
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int mi0 = mb * 32 + 8 * g4 + 4 * half;
        const float4 l4 = *reinterpret_cast<const float4*>(&Ls[cur][mi0]);
        const float4 d4 = *reinterpret_cast<const float4*>(&Dl[cur][mi0]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float pr = fast_exp2(fmaf(s[r], sl2, -lv[e]));
          if (!full) {
            const int mm = mt0 + mi0 + e;
            pr = (n <= mm && mm - n < W && mm < p.T) ? pr : 0.f;
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
          dv[dblk] = mfma32(tr_operand(Ds[cur], 2 * mb + h2, dblk * 32, lane, half), pb, dv[dblk]);
          dk[dblk] = mfma32(tr_operand(Qs[cur], 2 * mb + h2, dblk * 32, lane, half), dsb, dk[dblk]);
        }
      }
    }
    if (it + 1 < ntiles) {
      store_tile(cur ^ 1);
      if (it + 2 < ntiles) load_tile(mt0 + 2 * kTile);
    }
    __syncthreads();
  }

  if constexpr (HAS_DIL) {
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
      // Delta of query ii from its dout and o rows
      float di = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (16 * kk + 8 * half) * 2;
        di = Frag<DT_BF16>::dot(ld16(dob + ii * sdot + off), ld16(ob + ii * sot + off), di);
      }
      di += xhalf(di);
      const float pr = i < p.T ? fast_exp2(fmaf(sp, sl2, -lseb[ii] * kLog2e)) : 0.f;
      const float ds = pr * (dpp - di);
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
  __shared__ __align__(16) unsigned char smem[kSmemBytes];
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

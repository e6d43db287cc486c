// Gather forward: every edge of the neighbour graph handled on the vector
// ALUs, one lane group per query row.
//
// The graph is translation invariant (SpatialLM-Mini news page, "How tokens
// choose whom to listen to": a fixed list of distances per token), so for a
// fixed distance delta the keys of consecutive query rows are consecutive
// rows of K and V.  A wavefront holds 64/LG consecutive query rows, each row
// spread over LG lanes with NF 16-byte fragments (8 bf16 or 4 fp32 elements
// each) per lane: fragment f of lane s holds bytes 16 (f LG + s) .. + 15, so
// each load instruction covers one contiguous 16 LG-byte span of every row
// of the wavefront (all of it for NF = 1).  Scores are reduced across the lane group with DPP,
// and the softmax over the row's neighbours runs online (running max, sum
// and weighted value accumulator; the accumulator is rescaled only when the
// max grows by more than 2^8).
// Work and traffic are proportional to the number of edges (page "Longer
// Attention Span ...", abstract: work-optimal graph processing); no score
// matrix and no gathered copy of K or V is ever formed.
#include "device_util.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int DT, int D, int SM>
struct Geo {
  static constexpr int EPL = Frag<DT>::EPL;  // elements per 16-byte fragment
  // fragments per lane (gather_frags_per_lane): two shares a row's repeated
  // per-edge work (score, softmax bookkeeping) between half as many lanes
  static constexpr int NF = gather_frags_per_lane(DT, D, SM);
  static constexpr int LG = D / (EPL * NF);  // lanes per row
  static constexpr int RPW = 64 / LG;        // rows per wavefront
  static constexpr int RPB = RPW * kWaves;   // rows per workgroup
  static_assert(LG >= 1 && LG <= 32 && (LG & (LG - 1)) == 0, "row must span 1..32 lanes");
};


template <int DT, int D, int SM, int G, bool OFF32>
__global__ __launch_bounds__(kThreads) void gather_fwd_kernel(Params p) {
  using F = Frag<DT>;
  using Gm = Geo<DT, D, SM>;
  constexpr int EPL = Gm::EPL, NF = Gm::NF, LG = Gm::LG, RPW = Gm::RPW, RPB = Gm::RPB;
  constexpr int EB = F::BYTES;
  constexpr int FS = 16 * LG;  // bytes between a lane's fragments

  const int nblk = (p.T + RPB - 1) / RPB;
  const int logical = xcd_logical_block(p.B * p.H * nblk);
  if (logical < 0) return;
  const QueryBlock qb = query_block(logical, nblk, p.H, p.G);
  const int bh = qb.bh, rb = qb.rb, b = qb.b, h = qb.h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int sub = lane % LG;
  const int i0w = rb * RPB + wave * RPW;  // first row of this wavefront
  int i = i0w + lane / LG;
  const bool row_ok = i < p.T;
  if (!row_ok) i = p.T - 1;  // compute a valid row, store nothing

  // uniform per-head bases; per-lane byte offsets of row i's fragment
  const int hk = h / p.G;  // key/value head shared by G query heads
  const char* khead = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h) * EB;
  const char* vhead = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h) * EB;
  const int64_t skt = p.sk_t * EB, svt = p.sv_t * EB;
  int64_t kl = (int64_t)i * skt + sub * 16, vl = (int64_t)i * svt + sub * 16;
  uint32_t kl32 = (uint32_t)kl, vl32 = (uint32_t)vl;
  // opaque to the optimiser: keeps the per-distance address a scalar offset
  // from this per-lane value instead of a re-derived 64-bit multiply
  asm volatile("" : "+v"(kl32), "+v"(vl32), "+v"(kl), "+v"(vl));
  const uint32_t sub16 = (uint32_t)sub * 16u;

  uint4 qraw[NF];  // q fragments as stored (dot operands)
#pragma unroll
  for (int f = 0; f < NF; ++f) qraw[f] = make_uint4(0u, 0u, 0u, 0u);
  float cqi[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f;  // gamma * log2(e)
  const float* ckb = nullptr;
  if constexpr (SM == SM_DOT) {
    const char* qrow = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h + i * p.sq_t) * EB +
                       sub * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) qraw[f] = ld16(qrow + f * FS);
  } else if constexpr (SM == SM_COORD) {
    const float* cqr = p.cq + ((int64_t)bh * p.T + i) * 3;
    cqi[0] = cqr[0]; cqi[1] = cqr[1]; cqi[2] = cqr[2];
    gl2 = p.gamma[h] * kLog2e;
    ckb = p.ck + (int64_t)bh * p.T * 3;
  }

  float m = -INFINITY, l = 0.f;  // running max (log2 units), row sum
  float acc[NF][EPL];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[f][e] = 0.f;

  const int imax = i0w + RPW - 1 < p.T - 1 ? i0w + RPW - 1 : p.T - 1;
  // One group of G distances (wave-uniform, ascending; kUnreachable past
  // the end of the list): gather, score, online softmax, accumulate.
  auto group = [&](const int (&dist)[G]) {
    int j[G];
    uint4 kraw[G][NF], vraw[G][NF];
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      j[g] = i - dist[g];
      const bool ok = j[g] >= 0;
      if constexpr (OFF32) {
        const uint32_t ko = ok ? kl32 - (uint32_t)dist[g] * (uint32_t)skt : sub16;
        const uint32_t vo = ok ? vl32 - (uint32_t)dist[g] * (uint32_t)svt : sub16;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (SM == SM_DOT) kraw[g][f] = ld16(khead + ko + f * FS);
          vraw[g][f] = ld16(vhead + vo + f * FS);
        }
      } else {
        const int64_t ko = ok ? kl - (int64_t)dist[g] * skt : (int64_t)sub16;
        const int64_t vo = ok ? vl - (int64_t)dist[g] * svt : (int64_t)sub16;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (SM == SM_DOT) kraw[g][f] = ld16(khead + ko + f * FS);
          vraw[g][f] = ld16(vhead + vo + f * FS);
        }
      }
      if constexpr (SM == SM_COORD) {
        const float* c = ckb + (int64_t)(ok ? j[g] : 0) * 3;
        const float d0 = cqi[0] - c[0], d1 = cqi[1] - c[1], d2 = cqi[2] - c[2];
        s[g] = -gl2 * (d0 * d0 + d1 * d1 + d2 * d2);
      } else if constexpr (SM == SM_UNIFORM) {
        s[g] = 0.f;  // one weight for every neighbour
      }
    }
    if constexpr (SM == SM_DOT) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s[g] = F::dot(qraw[0], kraw[g][0], 0.f);
#pragma unroll
        for (int f = 1; f < NF; ++f) s[g] = F::dot(qraw[f], kraw[g][f], s[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = group_sum<LG>(s[g]) * p.scale_log2;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s[g] = j[g] >= 0 ? s[g] : -INFINITY;
      mx = fmaxf(mx, s[g]);
    }
    // Lazy rescale: the reference moves only when a score exceeds it by more
    // than 8 (log2 units), so exponents stay <= 8 and rescaling is rare.
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? mx : m;
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
      l *= alpha;
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[f][e] *= alpha;
      m = mnew;
    }
    const float neg = m == -INFINITY ? 0.f : -m;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pg = fast_exp2(s[g] + neg);
      l += pg;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        float vf[EPL];
        F::unpack(vraw[g][f], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[f][e] = fmaf(pg, vf[e], acc[f][e]);
      }
    }
  };

  // the window: distances 0 .. W-1
  const int wend = p.W < imax + 1 ? p.W : imax + 1;  // larger distances reach no row
  for (int t0 = 0; t0 < wend; t0 += G) {
    int dist[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dist[g] = t0 + g < p.W ? t0 + g : kUnreachable;
    group(dist);
  }
  // the long-range distances (ascending; the table is padded with kUnreachable)
  for (int t0 = 0; t0 < p.n_dil; t0 += G) {
    int dist[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dist[g] = p.dil[t0 + g];
    if (dist[0] > imax) break;  // no row of this wavefront reaches it, nor any later one
    group(dist);
  }

  const float inv_l = 1.f / l;
  if constexpr (NF == 1) {
    if (!row_ok) return;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[0][e] *= inv_l;
    char* orow = static_cast<char*>(p.o) + (b * p.so_b + h * p.so_h + i * p.so_t) * EB + sub * 16;
    st16_stream(orow, F::pack(acc[0]));
  } else {
    // Two fragments per lane cover half of each row per instruction; one
    // cross-half swap (v_permlane32_swap) turns them into two stores that each
    // write whole rows: the first the wavefront's rows 0 .. RPW/2 - 1, the
    // second the rest (lanes l and l + 32 hold the two halves of a row), so
    // no row is written as two partial lines.
    static_assert(NF == 2 && RPW % 2 == 0, "two fragments per lane");
    uint4 x[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[f][e] *= inv_l;
      x[f] = F::pack(acc[f]);
    }
    uint32_t* x0 = &x[0].x;
    uint32_t* x1 = &x[1].x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const auto r = __builtin_amdgcn_permlane32_swap(x0[c], x1[c], false, false);
      x0[c] = r[0];  // lanes 0..31: fragment 0 of rows 0..RPW/2-1; lanes 32..63: their fragment 1
      x1[c] = r[1];  // the same for rows RPW/2 .. RPW-1
    }
    const int half = lane >> 5;
    const int ra = i0w + (lane & 31) / LG;  // row of x[0]; x[1] holds row ra + RPW / 2
    char* obase = static_cast<char*>(p.o) + (b * p.so_b + h * p.so_h) * EB + sub * 16 + half * FS;
    if (ra < p.T) st16_stream(obase + (int64_t)ra * p.so_t * EB, x[0]);
    if (ra + RPW / 2 < p.T) st16_stream(obase + (int64_t)(ra + RPW / 2) * p.so_t * EB, x[1]);
    if (!row_ok) return;
  }
  if (sub == 0) {
    float lse = (m + fast_log2(l)) * kLn2;
    if constexpr (SM == SM_COORD) lse += p.beta[h];
    st_stream(p.lse + (int64_t)bh * p.T + i, lse);
  }
}

// Whether every gathered byte offset within one (batch, head) slice of k and
// v fits in 31 bits, so addresses can be a uniform base plus a 32-bit offset.
inline bool fits_off32(const Params& p, int eb) {
  const int64_t lim = (int64_t)1 << 31;
  return ((int64_t)(p.T - 1) * p.sk_t + p.D) * eb < lim && ((int64_t)(p.T - 1) * p.sv_t + p.D) * eb < lim;
}

template <int DT, int D, int SM>
hipError_t launch_one(const Params& p, hipStream_t s) {
  constexpr int RPB = Geo<DT, D, SM>::RPB;
  const int nblk = (p.T + RPB - 1) / RPB;
  const int grid = xcd_grid(p.B * p.H * nblk);
  // distances per step: four 16-byte fragments of K and V in flight per lane
  constexpr int G = 4 / Geo<DT, D, SM>::NF;
  if (fits_off32(p, Frag<DT>::BYTES))
    hipLaunchKernelGGL((gather_fwd_kernel<DT, D, SM, G, true>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gather_fwd_kernel<DT, D, SM, G, false>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int DT, int SM>
hipError_t launch_d(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_one<DT, 16, SM>(p, s);
    case 32: return launch_one<DT, 32, SM>(p, s);
    case 64: return launch_one<DT, 64, SM>(p, s);
    case 128: return launch_one<DT, 128, SM>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gather_rows_per_block(int dtype, int D) {
  // the smallest query-side block of the gather and explicit-list kernels
  // (one fragment per lane): sizes the per-block partials in the workspace
  const int epl = dtype == DT_BF16 ? 8 : 4;
  return (64 / (D / epl)) * kWaves;
}

template <int DT>
hipError_t launch_mode(const Params& p, int score_mode, hipStream_t s) {
  switch (score_mode) {
    case SM_DOT: return launch_d<DT, SM_DOT>(p, s);
    case SM_COORD: return launch_d<DT, SM_COORD>(p, s);
    case SM_UNIFORM: return launch_d<DT, SM_UNIFORM>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_fwd(const Params& p, int dtype, int score_mode, hipStream_t s) {
  return dtype == DT_BF16 ? launch_mode<DT_BF16>(p, score_mode, s) : launch_mode<DT_F32>(p, score_mode, s);
}

}  // namespace sa

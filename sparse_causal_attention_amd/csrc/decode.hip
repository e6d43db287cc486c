// Decode: one new query per (batch, head) against its neighbour list in a
// key/value cache.
//
// With the fixed neighbour graph a generated token at position t attends to
// t, t-1, ..., t-W+1 and t-d for the long-range distances d <= t, so a step
// costs O(W + log T) row reads however long the cache is (the prototype on
// the SpatialLM-Mini news page had no KV cache and did not measure
// generation: "What to check before adopting it in your project").
//
// On an explicit-list graph the new token's edges are the keys its row of
// the lists names.
//
// One workgroup per (batch, head).  Its lane groups (16 bytes of a row per
// lane, so a group holds one key row) take the row's edges round robin, each
// keeping its own online softmax state (running max, sum, weighted value
// accumulator); the groups' states are then merged through LDS.  Scores are
// those of the forward: scaled dot product, coordinate distance, or uniform.
#include "device_util.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int DT, int D, int SM, bool CSR>
__global__ __launch_bounds__(kThreads) void decode_kernel(Params p) {
  using F = Frag<DT>;
  constexpr int EPL = F::EPL;            // elements per lane
  constexpr int LG = D / EPL;            // lanes per row
  constexpr int NG = kThreads / LG;      // lane groups in the workgroup
  constexpr int EB = F::BYTES;
  static_assert(LG >= 1 && LG <= 32 && (LG & (LG - 1)) == 0, "row must span 1..32 lanes");

  __shared__ float s_m[NG], s_l[NG];
  __shared__ float s_acc[NG][D + 1];

  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x;
  const int grp = tid / LG, sub = tid % LG;

  const int t = p.pos != nullptr ? p.pos[b] : p.T - 1;  // row of the new token
  const bool valid = t >= 0 && t < p.T;
  const int tt = valid ? t : 0;
  // edges: the window t, t-1, ..., t-W'+1, then t-d for the distances d <= t;
  // or the row's list
  const int wn = p.W < tt + 1 ? p.W : tt + 1;
  int E, beg = 0;
  if constexpr (CSR) {
    beg = p.rp[tt];
    E = p.rp[tt + 1] - beg;
  } else {
    int nd = 0;
    while (nd < p.n_dil && p.dil[nd] <= tt) ++nd;  // uniform, ascending distances
    E = wn + nd;
  }

  const int hk = h / p.G;  // key/value head shared by G query heads
  const char* khead = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h) * EB + sub * 16;
  const char* vhead = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h) * EB + sub * 16;
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
  float cqi[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f;
  const float* ckb = nullptr;
  if constexpr (SM == SM_DOT) {
    qraw = ld16(static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h) * EB + sub * 16);
  } else if constexpr (SM == SM_COORD) {
    const float* c = p.cq + (int64_t)bh * 3;
    cqi[0] = c[0]; cqi[1] = c[1]; cqi[2] = c[2];
    gl2 = p.gamma[h] * kLog2e;
    ckb = p.ck + (int64_t)bh * p.T * 3;
  }

  float m = -INFINITY, l = 0.f;  // log2 units
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  // Every lane of a group runs the same edges, kU at a time (all their rows
  // requested before the first is used); groups past the edge count keep an
  // empty state.  The DPP sums below only combine lanes of one group.
  constexpr int kU = 4;
  for (int e0 = grp; e0 < E; e0 += kU * NG) {
    uint4 kraw[kU], vraw[kU];
    bool ok[kU];
    int jj[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = e0 + u * NG;
      ok[u] = e < E;
      if constexpr (CSR) {
        jj[u] = ok[u] ? p.cols[beg + e] : tt;
      } else {
        const int d = !ok[u] ? 0 : (e < wn ? e : p.dil[e - wn]);
        jj[u] = tt - d;  // >= 0 by construction; row tt stands in for absent edges
      }
      vraw[u] = ld16(vhead + (int64_t)jj[u] * p.sv_t * EB);
      if constexpr (SM == SM_DOT) kraw[u] = ld16(khead + (int64_t)jj[u] * p.sk_t * EB);
    }
    float s[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if constexpr (SM == SM_DOT) {
        s[u] = group_sum<LG>(F::dot(qraw, kraw[u], 0.f)) * p.scale_log2;
      } else if constexpr (SM == SM_COORD) {
        const float* c = ckb + (int64_t)jj[u] * 3;
        const float d0 = cqi[0] - c[0], d1 = cqi[1] - c[1], d2 = cqi[2] - c[2];
        s[u] = -gl2 * (d0 * d0 + d1 * d1 + d2 * d2);
      } else {
        s[u] = 0.f;
      }
      s[u] = ok[u] ? s[u] : -INFINITY;
    }
    float mnew = m;
#pragma unroll
    for (int u = 0; u < kU; ++u) mnew = fmaxf(mnew, s[u]);
    const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
    l *= alpha;
#pragma unroll
    for (int e2 = 0; e2 < EPL; ++e2) acc[e2] *= alpha;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float pj = ok[u] ? fast_exp2(s[u] - mnew) : 0.f;
      float vf[EPL];
      F::unpack(vraw[u], vf);
      l += pj;
#pragma unroll
      for (int e2 = 0; e2 < EPL; ++e2) acc[e2] = fmaf(pj, vf[e2], acc[e2]);
    }
    m = mnew;
  }

  // merge the groups' states
  if (sub == 0) {
    s_m[grp] = m;
    s_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[grp][sub * EPL + e] = acc[e];
  __syncthreads();
  if (tid >= D) return;
  float M = -INFINITY;
  for (int g = 0; g < NG; ++g) M = fmaxf(M, s_m[g]);
  float L = 0.f, O = 0.f;
  for (int g = 0; g < NG; ++g) {
    const float w = s_m[g] == -INFINITY ? 0.f : fast_exp2(s_m[g] - M);
    L = fmaf(s_l[g], w, L);
    O = fmaf(s_acc[g][tid], w, O);
  }
  const float out = valid ? O / L : __builtin_nanf("");
  char* orow = static_cast<char*>(p.o) + (b * p.so_b + h * p.so_h) * EB;
  if constexpr (DT == DT_BF16) {
    const __bf16 ob = static_cast<__bf16>(out);
    *reinterpret_cast<__bf16*>(orow + tid * 2) = ob;
  } else {
    *reinterpret_cast<float*>(orow + tid * 4) = out;
  }
  if (tid == 0) {
    float lse = (M + fast_log2(L)) * kLn2;
    if constexpr (SM == SM_COORD) lse += p.beta[h];
    p.lse[bh] = valid ? lse : __builtin_nanf("");
  }
}

template <int DT, int SM, bool CSR>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.H)), block(kThreads);
  switch (p.D) {
    case 16: hipLaunchKernelGGL((decode_kernel<DT, 16, SM, CSR>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((decode_kernel<DT, 32, SM, CSR>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((decode_kernel<DT, 64, SM, CSR>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((decode_kernel<DT, 128, SM, CSR>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT, bool CSR>
hipError_t launch_mode(const Params& p, int score_mode, hipStream_t s) {
  switch (score_mode) {
    case SM_DOT: return launch_d<DT, SM_DOT, CSR>(p, s);
    case SM_COORD: return launch_d<DT, SM_COORD, CSR>(p, s);
    case SM_UNIFORM: return launch_d<DT, SM_UNIFORM, CSR>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_graph(const Params& p, int score_mode, hipStream_t s) {
  return p.rp != nullptr ? launch_mode<DT, true>(p, score_mode, s) : launch_mode<DT, false>(p, score_mode, s);
}

}  // namespace

hipError_t launch_decode(const Params& p, int dtype, int score_mode, hipStream_t s) {
  return dtype == DT_BF16 ? launch_graph<DT_BF16>(p, score_mode, s) : launch_graph<DT_F32>(p, score_mode, s);
}

}  // namespace sa

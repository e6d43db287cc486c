// Gather backward: the gradients of sum <dout, o> through the forward, on
// the vector ALUs, deterministic and without atomics.
//
// Two passes share the lane-group layout of the forward (one row per LG
// lanes, 16 bytes per lane, DPP reductions):
//  1. query side, one row i per lane group, over the forward graph
//     j = i - delta: P_ij = exp(s_ij - lse_i), dP_ij = <dout_i, v_j>, and in
//     the same single pass Delta_i = sum_j P_ij dP_ij (kept in the workspace
//     for pass 2) together with sum_j P_ij dP_ij x_j and sum_j P_ij x_j, so
//     that dq_i = scale (sum_j P dP k_j - Delta_i sum_j P k_j) needs no second
//     pass over the edges (coordinate mode: dc_q,i and per-block partial sums
//     of dgamma, dbeta the same way).  Delta_i comes from the edges, not from
//     <dout_i, o_i>, so a bf16-rounded o does not perturb it;
//  2. key side, one row j per lane group, over the reverse graph
//     i = j + delta < T: dv_j = sum_i P_ij dout_i, dk_j = scale sum_i dS_ij q_i
//     (coordinate mode: dc_k,j).  For a fixed delta the query rows of
//     consecutive keys are consecutive, so these reads coalesce exactly like
//     the forward's.
// Each output row has exactly one writer, so the result is bitwise
// reproducible.  A final pass reduces the coordinate-mode partials per head
// in fp64 in a fixed order.
#include "device_util.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Row layout as in the gather forward: NF 16-byte fragments per lane
// (fragment f of lane s at bytes 16 (f LG + s)), LG lanes per row.
template <int DT, int D, int SM>
struct Geo {
  static constexpr int EPL = Frag<DT>::EPL;
  static constexpr int NF = gather_frags_per_lane(DT, D, SM);
  static constexpr int LG = D / (EPL * NF);
  static constexpr int RPW = 64 / LG;
  static constexpr int RPB = RPW * kWaves;
};


// ------------------------------------------------------------------ pass 1
template <int DT, int D, bool COORD, int G, bool OFF32>
__global__ __launch_bounds__(kThreads) void gather_bwd_q_kernel(Params p) {
  using F = Frag<DT>;
  using Gm = Geo<DT, D, COORD ? SM_COORD : SM_DOT>;
  constexpr int EPL = Gm::EPL, NF = Gm::NF, LG = Gm::LG, RPW = Gm::RPW, RPB = Gm::RPB;
  constexpr int EB = F::BYTES;
  constexpr int FS = 16 * LG;  // bytes between a lane's fragments

  const int nblk = (p.T + RPB - 1) / RPB;
  const int logical = xcd_logical_block(p.B * p.H * nblk);
  if (logical < 0) return;
  const QueryBlock qb = query_block(logical, nblk, p.H, p.G);
  const int bh = qb.bh, rb = qb.rb, b = qb.b, h = qb.h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LG;
  const int i0w = rb * RPB + wave * RPW;
  int i = i0w + lane / LG;
  const bool row_ok = i < p.T;
  if (!row_ok) i = p.T - 1;
  const int imax = i0w + RPW - 1 < p.T - 1 ? i0w + RPW - 1 : p.T - 1;

  const int hk = h / p.G;  // key/value head shared by G query heads
  const char* khead = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h) * EB;
  const char* vhead = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h) * EB;
  const int64_t skt = p.sk_t * EB, svt = p.sv_t * EB;
  int64_t kl = (int64_t)i * skt + sub * 16, vl = (int64_t)i * svt + sub * 16;
  uint32_t kl32 = (uint32_t)kl, vl32 = (uint32_t)vl;
  asm volatile("" : "+v"(kl32), "+v"(vl32), "+v"(kl), "+v"(vl));  // keep addresses scalar-offset
  const uint32_t sub16 = (uint32_t)sub * 16u;

  // dout and q fragments as stored (dot operands)
  uint4 doraw[NF], qraw[NF];
  {
    const char* dorow = static_cast<const char*>(p.dout) +
                        (b * p.sdo_b + h * p.sdo_h + i * p.sdo_t) * EB + sub * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      doraw[f] = ld16(dorow + f * FS);
      qraw[f] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // lse includes beta in coordinate mode; the scores below omit it
  const float lse2 =
      (p.lse[(int64_t)bh * p.T + i] - (COORD ? p.beta[h] : 0.f)) * kLog2e;

  float cqi[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f, gam = 0.f;
  const float* ckb = nullptr;
  if constexpr (!COORD) {
    const char* qrow = static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h + i * p.sq_t) * EB +
                       sub * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) qraw[f] = ld16(qrow + f * FS);
  } else {
    const float* cqr = p.cq + ((int64_t)bh * p.T + i) * 3;
    cqi[0] = cqr[0]; cqi[1] = cqr[1]; cqi[2] = cqr[2];
    gam = p.gamma[h];
    gl2 = gam * kLog2e;
    ckb = p.ck + (int64_t)bh * p.T * 3;
  }

  // running sums over the row's edges: Delta = sum P dP, and per term x
  // (k_j in dot mode; c_q,i - c_k,j and ||.||^2 in coordinate mode)
  // sum P dP x and sum P x
  float delta = 0.f;
  float pdx[NF][EPL], px[NF][EPL];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < EPL; ++e) pdx[f][e] = px[f][e] = 0.f;
  float cdx[3] = {0.f, 0.f, 0.f}, cx[3] = {0.f, 0.f, 0.f};
  float r2dx = 0.f, r2x = 0.f, psum = 0.f;

  auto group = [&](const int (&dist)[G]) {
    int j[G];
    uint4 kraw[G][NF], vraw[G][NF];
    float s[G], dp[G], r2[G], dif[G][3];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      j[g] = i - dist[g];
      const bool ok = j[g] >= 0;
      if constexpr (OFF32) {
        const uint32_t ko = ok ? kl32 - (uint32_t)dist[g] * (uint32_t)skt : sub16;
        const uint32_t vo = ok ? vl32 - (uint32_t)dist[g] * (uint32_t)svt : sub16;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (!COORD) kraw[g][f] = ld16(khead + ko + f * FS);
          vraw[g][f] = ld16(vhead + vo + f * FS);
        }
      } else {
        const int64_t ko = ok ? kl - (int64_t)dist[g] * skt : (int64_t)sub16;
        const int64_t vo = ok ? vl - (int64_t)dist[g] * svt : (int64_t)sub16;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (!COORD) kraw[g][f] = ld16(khead + ko + f * FS);
          vraw[g][f] = ld16(vhead + vo + f * FS);
        }
      }
      if constexpr (COORD) {
        const float* c = ckb + (int64_t)(ok ? j[g] : 0) * 3;
        dif[g][0] = cqi[0] - c[0];
        dif[g][1] = cqi[1] - c[1];
        dif[g][2] = cqi[2] - c[2];
        r2[g] = dif[g][0] * dif[g][0] + dif[g][1] * dif[g][1] + dif[g][2] * dif[g][2];
        s[g] = -gl2 * r2[g];
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      dp[g] = F::dot(doraw[0], vraw[g][0], 0.f);
      if constexpr (!COORD) s[g] = F::dot(qraw[0], kraw[g][0], 0.f);
#pragma unroll
      for (int f = 1; f < NF; ++f) {
        dp[g] = F::dot(doraw[f], vraw[g][f], dp[g]);
        if constexpr (!COORD) s[g] = F::dot(qraw[f], kraw[g][f], s[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      dp[g] = group_sum<LG>(dp[g]);
      if constexpr (!COORD) s[g] = group_sum<LG>(s[g]) * p.scale_log2;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pr = j[g] >= 0 ? fast_exp2(s[g] - lse2) : 0.f;
      const float pd = pr * dp[g];
      delta += pd;
      if constexpr (!COORD) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          float kf[EPL];
          F::unpack(kraw[g][f], kf);
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            pdx[f][e] = fmaf(pd, kf[e], pdx[f][e]);
            px[f][e] = fmaf(pr, kf[e], px[f][e]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          cdx[c] = fmaf(pd, dif[g][c], cdx[c]);
          cx[c] = fmaf(pr, dif[g][c], cx[c]);
        }
        r2dx = fmaf(pd, r2[g], r2dx);
        r2x = fmaf(pr, r2[g], r2x);
        psum += pr;
      }
    }
  };

  const int wend = p.W < imax + 1 ? p.W : imax + 1;
  for (int t0 = 0; t0 < wend; t0 += G) {
    int dist[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dist[g] = t0 + g < p.W ? t0 + g : kUnreachable;
    group(dist);
  }
  for (int t0 = 0; t0 < p.n_dil; t0 += G) {
    int dist[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dist[g] = p.dil[t0 + g];
    if (dist[0] > imax) break;
    group(dist);
  }
  if (row_ok && sub == 0) p.delta[(int64_t)bh * p.T + i] = delta;

  if constexpr (!COORD) {
    if (row_ok) {
      const int gb = p.grad_bf16 ? 2 : 4;
      char* dqrow = static_cast<char*>(p.dq) + (b * p.sdq_b + h * p.sdq_h + i * p.sdq_t) * gb +
                    sub * EPL * gb;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        float dq[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) dq[e] = p.scale * (pdx[f][e] - delta * px[f][e]);
        store_vals<EPL>(dqrow + f * LG * EPL * gb, dq, p.grad_bf16 != 0);
      }
    }
  } else {
    if (row_ok && sub == 0) {
      float* o = p.dcq + ((int64_t)bh * p.T + i) * 3;
#pragma unroll
      for (int c = 0; c < 3; ++c) st_stream(o + c, -2.f * gam * (cdx[c] - delta * cx[c]));
    }
    // dgamma_i = -sum_j dS_ij r2_ij,  dbeta_i = sum_j dS_ij = Delta_i (1 - sum_j P_ij)
    const float gpart = -(r2dx - delta * r2x);
    const float bpart = delta * (1.f - psum);
    // per-block partial sums, one value per row (lane sub == 0), reduced in
    // a fixed order through LDS
    __shared__ float red[2][kThreads];
    const bool counts = row_ok && sub == 0;
    red[0][threadIdx.x] = counts ? gpart : 0.f;
    red[1][threadIdx.x] = counts ? bpart : 0.f;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (threadIdx.x < w) {
        red[0][threadIdx.x] += red[0][threadIdx.x + w];
        red[1][threadIdx.x] += red[1][threadIdx.x + w];
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      float* pp = p.partials + ((int64_t)bh * nblk + rb) * 2;
      pp[0] = red[0][0];
      pp[1] = red[1][0];
    }
  }
}

// ------------------------------------------------------------------ pass 2
template <int DT, int D, int SM, int G, bool OFF32>
__global__ __launch_bounds__(kThreads) void gather_bwd_kv_kernel(Params p) {
  constexpr bool COORD = SM == SM_COORD;
  constexpr bool UNIFORM = SM == SM_UNIFORM;  // dv only: no score parameters
  using F = Frag<DT>;
  using Gm = Geo<DT, D, SM>;
  constexpr int EPL = Gm::EPL, NF = Gm::NF, LG = Gm::LG, RPW = Gm::RPW, RPB = Gm::RPB;
  constexpr int EB = F::BYTES;
  constexpr int FS = 16 * LG;  // bytes between a lane's fragments

  // one key row per lane group of key/value head hk; the query side runs
  // over the G query heads hk G .. hk G + G - 1 that share it (G = 1 in
  // coordinate mode, where bh then names both)
  const int nblk = (p.T + RPB - 1) / RPB;
  const int logical = xcd_logical_block(p.B * p.Hkv * nblk);
  if (logical < 0) return;
  const int bk = logical / nblk, rb = logical - bk * nblk;
  const int b = bk / p.Hkv, hk = bk - b * p.Hkv;
  const int h0 = hk * p.G;
  const int bh = b * p.H + h0;  // first query head of the group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LG;
  const int j0w = rb * RPB + wave * RPW;  // first key row of this wavefront
  int j = j0w + lane / LG;
  const bool row_ok = j < p.T;
  if (!row_ok) j = p.T - 1;
  const int room = p.T - 1 - j0w;  // largest distance any key of the wave can use

  const char* qhead = nullptr;   // set per query head below
  const char* dohead = nullptr;
  const int64_t sqt = p.sq_t * EB, sdot = p.sdo_t * EB;
  int64_t ql = (int64_t)j * sqt + sub * 16, dl = (int64_t)j * sdot + sub * 16;
  uint32_t ql32 = (uint32_t)ql, dl32 = (uint32_t)dl;
  asm volatile("" : "+v"(ql32), "+v"(dl32), "+v"(ql), "+v"(dl));  // keep addresses scalar-offset
  const float* lseb = nullptr;
  const float* delb = nullptr;
  const float bsub = COORD ? p.beta[h0] : 0.f;  // lse includes beta in coordinate mode

  // own k and v fragments as stored (dot operands)
  uint4 kraw_j[NF], vraw_j[NF];
  {
    const char* vrow = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h + j * p.sv_t) * EB +
                       sub * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      vraw_j[f] = ld16(vrow + f * FS);
      kraw_j[f] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float ckj[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f, gam = 0.f;
  const float* cqb = nullptr;
  if constexpr (SM == SM_DOT) {
    const char* krow = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h + j * p.sk_t) * EB +
                       sub * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) kraw_j[f] = ld16(krow + f * FS);
  } else if constexpr (COORD) {
    const float* ckr = p.ck + ((int64_t)bh * p.T + j) * 3;
    ckj[0] = ckr[0]; ckj[1] = ckr[1]; ckj[2] = ckr[2];
    gam = p.gamma[h0];
    gl2 = gam * kLog2e;
    cqb = p.cq + (int64_t)bh * p.T * 3;
  }

  float dk[NF][EPL], dv[NF][EPL];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < EPL; ++e) dk[f][e] = dv[f][e] = 0.f;
  float dc[3] = {0.f, 0.f, 0.f};

  auto group = [&](const int (&dist)[G]) {
    int i[G];
    uint4 qraw[G][NF], doraw[G][NF];
    float s[G], dp[G], lse2[G], del[G], dif[G][3];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // test the distance against the room left (j + kUnreachable would overflow)
      const bool ok = dist[g] <= p.T - 1 - j;
      const int ii = ok ? j + dist[g] : j;  // own row as a harmless stand-in
      if constexpr (OFF32) {
        const uint32_t qo = ok ? ql32 + (uint32_t)dist[g] * (uint32_t)sqt : ql32;
        const uint32_t doo = ok ? dl32 + (uint32_t)dist[g] * (uint32_t)sdot : dl32;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (SM == SM_DOT) qraw[g][f] = ld16(qhead + qo + f * FS);
          doraw[g][f] = ld16(dohead + doo + f * FS);
        }
      } else {
        const int64_t qo = ok ? ql + (int64_t)dist[g] * sqt : ql;
        const int64_t doo = ok ? dl + (int64_t)dist[g] * sdot : dl;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (SM == SM_DOT) qraw[g][f] = ld16(qhead + qo + f * FS);
          doraw[g][f] = ld16(dohead + doo + f * FS);
        }
      }
      lse2[g] = (lseb[ii] - bsub) * kLog2e;
      if constexpr (!UNIFORM) del[g] = delb[ii];
      i[g] = ok ? ii : p.T;  // p.T marks an absent edge
      if constexpr (COORD) {
        const float* c = cqb + (int64_t)ii * 3;
        dif[g][0] = c[0] - ckj[0];
        dif[g][1] = c[1] - ckj[1];
        dif[g][2] = c[2] - ckj[2];
        s[g] = -gl2 * (dif[g][0] * dif[g][0] + dif[g][1] * dif[g][1] + dif[g][2] * dif[g][2]);
      } else if constexpr (UNIFORM) {
        s[g] = 0.f;
      }
    }
    if constexpr (!UNIFORM) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        dp[g] = F::dot(doraw[g][0], vraw_j[0], 0.f);
        if constexpr (SM == SM_DOT) s[g] = F::dot(qraw[g][0], kraw_j[0], 0.f);
#pragma unroll
        for (int f = 1; f < NF; ++f) {
          dp[g] = F::dot(doraw[g][f], vraw_j[f], dp[g]);
          if constexpr (SM == SM_DOT) s[g] = F::dot(qraw[g][f], kraw_j[f], s[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        dp[g] = group_sum<LG>(dp[g]);
        if constexpr (SM == SM_DOT) s[g] = group_sum<LG>(s[g]) * p.scale_log2;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pr = i[g] < p.T ? fast_exp2(s[g] - lse2[g]) : 0.f;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        float dof[EPL];
        F::unpack(doraw[g][f], dof);
#pragma unroll
        for (int e = 0; e < EPL; ++e) dv[f][e] = fmaf(pr, dof[e], dv[f][e]);
      }
      if constexpr (UNIFORM) continue;
      const float ds = pr * (dp[g] - del[g]);
      if constexpr (SM == SM_DOT) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          float qf[EPL];
          F::unpack(qraw[g][f], qf);
#pragma unroll
          for (int e = 0; e < EPL; ++e) dk[f][e] = fmaf(ds, qf[e], dk[f][e]);
        }
      } else {
        dc[0] = fmaf(ds, dif[g][0], dc[0]);
        dc[1] = fmaf(ds, dif[g][1], dc[1]);
        dc[2] = fmaf(ds, dif[g][2], dc[2]);
      }
    }
  };

  const int wend = p.W < room + 1 ? p.W : room + 1;
  for (int hq = h0; hq < h0 + p.G; ++hq) {  // the query heads of this key/value head, in order
    qhead = static_cast<const char*>(p.q) + (b * p.sq_b + hq * p.sq_h) * EB;
    dohead = static_cast<const char*>(p.dout) + (b * p.sdo_b + hq * p.sdo_h) * EB;
    lseb = p.lse + ((int64_t)b * p.H + hq) * p.T;
    if constexpr (!UNIFORM) delb = p.delta + ((int64_t)b * p.H + hq) * p.T;
    for (int t0 = 0; t0 < wend; t0 += G) {
      int dist[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dist[g] = t0 + g < p.W ? t0 + g : kUnreachable;
      group(dist);
    }
    for (int t0 = 0; t0 < p.n_dil; t0 += G) {
      int dist[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dist[g] = p.dil[t0 + g];
      if (dist[0] > room) break;
      group(dist);
    }
  }

  if (!row_ok) return;
  const int gb = p.grad_bf16 ? 2 : 4;
  char* dvrow = static_cast<char*>(p.dv) + (b * p.sdv_b + hk * p.sdv_h + j * p.sdv_t) * gb +
                sub * EPL * gb;
#pragma unroll
  for (int f = 0; f < NF; ++f) store_vals<EPL>(dvrow + f * LG * EPL * gb, dv[f], p.grad_bf16 != 0);
  if constexpr (SM == SM_DOT) {
    char* dkrow = static_cast<char*>(p.dk) + (b * p.sdk_b + hk * p.sdk_h + j * p.sdk_t) * gb +
                  sub * EPL * gb;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) dk[f][e] *= p.scale;
      store_vals<EPL>(dkrow + f * LG * EPL * gb, dk[f], p.grad_bf16 != 0);
    }
  } else if constexpr (COORD) {
    if (sub == 0) {
      float* o = p.dck + ((int64_t)bh * p.T + j) * 3;
      st_stream(o, 2.f * gam * dc[0]);
      st_stream(o + 1, 2.f * gam * dc[1]);
      st_stream(o + 2, 2.f * gam * dc[2]);
    }
  }
}

// ------------------------------------------------------------------ pass 3
// dgamma_h, dbeta_h: sum of the per-block partials of every batch for head
// h, in fp64, in a fixed order (strided per thread, then a fixed tree).
__global__ __launch_bounds__(256) void coord_param_reduce_kernel(const float* partials, int B, int H,
                                                                 int nblk, float* dgamma,
                                                                 float* dbeta) {
  const int h = blockIdx.x;
  __shared__ double red[2][256];
  double g = 0.0, bsum = 0.0;
  const int per_head = B * nblk;
  for (int t = threadIdx.x; t < per_head; t += 256) {
    const int b = t / nblk, r = t - b * nblk;
    const float* pp = partials + (((int64_t)b * H + h) * nblk + r) * 2;
    g += (double)pp[0];
    bsum += (double)pp[1];
  }
  red[0][threadIdx.x] = g;
  red[1][threadIdx.x] = bsum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    dgamma[h] = (float)red[0][0];
    dbeta[h] = (float)red[1][0];
  }
}

// Whether every gathered byte offset within one (batch, head) slice fits in
// 31 bits, so addresses can be a uniform base plus a 32-bit offset.
inline bool fits_off32(const Params& p, int eb) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t strides[4] = {p.sk_t, p.sv_t, p.sq_t, p.sdo_t};
  for (int64_t st : strides)
    if (((int64_t)(p.T - 1) * st + p.D) * eb >= lim) return false;
  return true;
}

// Both passes take two distances per step: fewer rows in flight per lane
// than the forward's four, but fewer registers and more resident wavefronts
// (key side: 76 instead of 119 VGPRs), which measured 3 to 6 % faster on the
// dilated workloads.  The fixed-weight key side, with no scores to compute,
// keeps four (1 % faster there).
constexpr int kBwdGroup = 2;

template <int DT, int D, int SM, bool OFF32>
hipError_t launch_passes(const Params& p, hipStream_t s, int grid, int nblk) {
  if constexpr (SM != SM_UNIFORM) {  // the uniform mode has no query-side gradient
    hipLaunchKernelGGL((gather_bwd_q_kernel<DT, D, SM == SM_COORD, kBwdGroup, OFF32>), dim3(grid), dim3(kThreads),
                       0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int grid_kv = xcd_grid(p.B * p.Hkv * nblk);  // key rows of the key/value heads
  constexpr int gkv = SM == SM_UNIFORM ? 4 : kBwdGroup;
  hipLaunchKernelGGL((gather_bwd_kv_kernel<DT, D, SM, gkv, OFF32>), dim3(grid_kv), dim3(kThreads), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || SM != SM_COORD) return e;
  return launch_coord_param_reduce(p, nblk, s);
}

template <int DT, int D, int SM>
hipError_t launch_one(const Params& p, hipStream_t s) {
  constexpr int RPB = Geo<DT, D, SM>::RPB;
  const int nblk = (p.T + RPB - 1) / RPB;
  const int grid = xcd_grid(p.B * p.H * nblk);
  return fits_off32(p, Frag<DT>::BYTES) ? launch_passes<DT, D, SM, true>(p, s, grid, nblk)
                                        : launch_passes<DT, D, SM, false>(p, s, grid, nblk);
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

template <int DT>
hipError_t launch_mode(const Params& p, int score_mode, hipStream_t s) {
  switch (score_mode) {
    case SM_DOT: return launch_d<DT, SM_DOT>(p, s);
    case SM_COORD: return launch_d<DT, SM_COORD>(p, s);
    case SM_UNIFORM: return launch_d<DT, SM_UNIFORM>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_coord_param_reduce(const Params& p, int nblk, hipStream_t s) {
  hipLaunchKernelGGL(coord_param_reduce_kernel, dim3(p.H), dim3(256), 0, s, p.partials, p.B, p.H,
                     nblk, p.dgamma, p.dbeta);
  return hipGetLastError();
}

hipError_t launch_gather_bwd(const Params& p, int dtype, int score_mode, hipStream_t s) {
  return dtype == DT_BF16 ? launch_mode<DT_BF16>(p, score_mode, s) : launch_mode<DT_F32>(p, score_mode, s);
}

}  // namespace sa

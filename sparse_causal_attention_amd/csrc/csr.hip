// Attention over an explicit neighbour graph: per-row key lists in device
// memory (compressed sparse rows), the general graph view of the page
// "Longer Attention Span: Increasing Transformer Context Length with Sparse
// Graph Processing Techniques" (abstract: tokens are nodes, the mask gives the
// edges, work proportional to the edges).
//
// Same lane-group layout as the distance-graph gather kernels (one query or
// key row per LG lanes, 16 bytes of the row per lane, DPP sums within the
// group), but every neighbour is named by an index instead of a shift, so a
// row's key rows are wherever its list points.  Each lane group walks its own
// list kU entries at a time; the wavefront runs until its longest list is
// done and masks the rest.  The next batch of indices is fetched while the
// current batch of rows is in flight.
//
//  - forward: online softmax over the row's list (running max, sum, weighted
//    value accumulator, lazy rescale when the max grows by more than 2^8);
//  - backward, query side: over row i's list, Delta_i = sum P dP together with
//    sum P dP x and sum P x, hence dq_i (or dc_q,i and per-block partials of
//    dgamma, dbeta) in one pass;
//  - backward, key side: over the reverse list of key j (the queries that list
//    j, ascending), dv_j = sum P dout_i and dk_j = scale sum dS q_i (or
//    dc_k,j), looping over the query heads that share key/value head j's head.
// One writer per output row, fixed summation order: bitwise reproducible.
#include "device_util.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kU = 4;  // list entries per step

template <int DT, int D>
struct Geo {
  static constexpr int EPL = Frag<DT>::EPL;
  static constexpr int LG = D / EPL;
  static constexpr int RPW = 64 / LG;
  static constexpr int RPB = RPW * kWaves;
  static_assert(LG >= 1 && LG <= 32 && (LG & (LG - 1)) == 0, "row must span 1..32 lanes");
};

// Entries e .. e+kU-1 of a list starting at `beg` with n entries; past the
// end, `self` (a valid row) stands in so that every address stays in bounds.
__device__ __forceinline__ void fetch_idx(const int32_t* __restrict__ lst, int beg, int n, int e, int self,
                                          int (&out)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) out[u] = e + u < n ? lst[beg + e + u] : self;
}

// Byte offset of row r of a slice with row pitch `pitch` bytes, plus the lane's 16 bytes.
template <bool OFF32>
__device__ __forceinline__ const char* row_at(const char* base, int r, int64_t pitch, uint32_t sub16) {
  if constexpr (OFF32) return base + ((uint32_t)r * (uint32_t)pitch + sub16);
  return base + ((int64_t)r * pitch + sub16);
}

// ------------------------------------------------------------------ forward
template <int DT, int D, int SM, bool OFF32>
__global__ __launch_bounds__(kThreads) void csr_fwd_kernel(Params p) {
  using F = Frag<DT>;
  using Gm = Geo<DT, D>;
  constexpr int EPL = Gm::EPL, LG = Gm::LG, RPW = Gm::RPW, RPB = Gm::RPB;
  constexpr int EB = F::BYTES;

  const int nblk = (p.T + RPB - 1) / RPB;
  const int logical = xcd_logical_block(p.B * p.H * nblk);
  if (logical < 0) return;
  const QueryBlock qb = query_block(logical, nblk, p.H, p.G);
  const int bh = qb.bh, rb = qb.rb, b = qb.b, h = qb.h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LG;
  int i = rb * RPB + wave * RPW + lane / LG;
  const bool row_ok = i < p.T;
  if (!row_ok) i = p.T - 1;
  const int beg = p.rp[i];
  const int n = row_ok ? p.rp[i + 1] - beg : 0;

  const int hk = h / p.G;
  const char* khead = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h) * EB;
  const char* vhead = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h) * EB;
  const int64_t skt = p.sk_t * EB, svt = p.sv_t * EB;
  const uint32_t sub16 = (uint32_t)sub * 16u;

  uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
  float cqi[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f;
  const float* ckb = nullptr;
  if constexpr (SM == SM_DOT) {
    qraw = ld16(static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h + i * p.sq_t) * EB + sub16);
  } else if constexpr (SM == SM_COORD) {
    const float* c = p.cq + ((int64_t)bh * p.T + i) * 3;
    cqi[0] = c[0]; cqi[1] = c[1]; cqi[2] = c[2];
    gl2 = p.gamma[h] * kLog2e;
    ckb = p.ck + (int64_t)bh * p.T * 3;
  }

  float m = -INFINITY, l = 0.f;  // running max (log2 units), row sum
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  int nxt[kU];
  fetch_idx(p.cols, beg, n, 0, i, nxt);
  for (int e0 = 0; __builtin_amdgcn_ballot_w64(e0 < n) != 0; e0 += kU) {
    int j[kU];
    uint4 kraw[kU], vraw[kU];
    float s[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) j[u] = nxt[u];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if constexpr (SM == SM_DOT) kraw[u] = ld16(row_at<OFF32>(khead, j[u], skt, sub16));
      vraw[u] = ld16(row_at<OFF32>(vhead, j[u], svt, sub16));
    }
    fetch_idx(p.cols, beg, n, e0 + kU, i, nxt);  // in flight with the rows above
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if constexpr (SM == SM_DOT) {
        s[u] = group_sum<LG>(F::dot(qraw, kraw[u], 0.f)) * p.scale_log2;
      } else if constexpr (SM == SM_COORD) {
        const float* c = ckb + (int64_t)j[u] * 3;
        const float d0 = cqi[0] - c[0], d1 = cqi[1] - c[1], d2 = cqi[2] - c[2];
        s[u] = -gl2 * (d0 * d0 + d1 * d1 + d2 * d2);
      } else {
        s[u] = 0.f;
      }
      s[u] = e0 + u < n ? s[u] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) mx = fmaxf(mx, s[u]);
    // lazy rescale: the reference max moves only when a score passes it by
    // more than 8 (log2 units), so every exponent below stays <= 8
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? mx : m;
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
      m = mnew;
    }
    const float neg = m == -INFINITY ? 0.f : -m;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float pu = fast_exp2(s[u] + neg);
      l += pu;
      float vf[EPL];
      F::unpack(vraw[u], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pu, vf[e], acc[e]);
    }
  }

  if (!row_ok) return;
  const float inv_l = 1.f / l;  // every list is non-empty
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] *= inv_l;
  char* orow = static_cast<char*>(p.o) + (b * p.so_b + h * p.so_h + i * p.so_t) * EB + sub16;
  st16_stream(orow, F::pack(acc));
  if (sub == 0) {
    float lse = (m + fast_log2(l)) * kLn2;
    if constexpr (SM == SM_COORD) lse += p.beta[h];
    st_stream(p.lse + (int64_t)bh * p.T + i, lse);
  }
}

// ------------------------------------------------------------------ backward, query side
template <int DT, int D, bool COORD, bool OFF32>
__global__ __launch_bounds__(kThreads) void csr_bwd_q_kernel(Params p) {
  using F = Frag<DT>;
  using Gm = Geo<DT, D>;
  constexpr int EPL = Gm::EPL, LG = Gm::LG, RPW = Gm::RPW, RPB = Gm::RPB;
  constexpr int EB = F::BYTES;

  const int nblk = (p.T + RPB - 1) / RPB;
  const int logical = xcd_logical_block(p.B * p.H * nblk);
  if (logical < 0) return;
  const QueryBlock qb = query_block(logical, nblk, p.H, p.G);
  const int bh = qb.bh, rb = qb.rb, b = qb.b, h = qb.h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LG;
  int i = rb * RPB + wave * RPW + lane / LG;
  const bool row_ok = i < p.T;
  if (!row_ok) i = p.T - 1;
  const int beg = p.rp[i];
  const int n = row_ok ? p.rp[i + 1] - beg : 0;

  const int hk = h / p.G;
  const char* khead = static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h) * EB;
  const char* vhead = static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h) * EB;
  const int64_t skt = p.sk_t * EB, svt = p.sv_t * EB;
  const uint32_t sub16 = (uint32_t)sub * 16u;

  const uint4 doraw =
      ld16(static_cast<const char*>(p.dout) + (b * p.sdo_b + h * p.sdo_h + i * p.sdo_t) * EB + sub16);
  // lse includes beta in coordinate mode; the scores below omit it
  const float lse2 = (p.lse[(int64_t)bh * p.T + i] - (COORD ? p.beta[h] : 0.f)) * kLog2e;
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
  float cqi[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f, gam = 0.f;
  const float* ckb = nullptr;
  if constexpr (!COORD) {
    qraw = ld16(static_cast<const char*>(p.q) + (b * p.sq_b + h * p.sq_h + i * p.sq_t) * EB + sub16);
  } else {
    const float* c = p.cq + ((int64_t)bh * p.T + i) * 3;
    cqi[0] = c[0]; cqi[1] = c[1]; cqi[2] = c[2];
    gam = p.gamma[h];
    gl2 = gam * kLog2e;
    ckb = p.ck + (int64_t)bh * p.T * 3;
  }

  // Delta = sum P dP; per term x (k_j, or c_q,i - c_k,j and its squared
  // norm): sum P dP x and sum P x
  float delta = 0.f;
  float pdx[EPL], px[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) pdx[e] = px[e] = 0.f;
  float cdx[3] = {0.f, 0.f, 0.f}, cx[3] = {0.f, 0.f, 0.f};
  float r2dx = 0.f, r2x = 0.f, psum = 0.f;

  int nxt[kU];
  fetch_idx(p.cols, beg, n, 0, i, nxt);
  for (int e0 = 0; __builtin_amdgcn_ballot_w64(e0 < n) != 0; e0 += kU) {
    int j[kU];
    uint4 kraw[kU], vraw[kU];
    float s[kU], dp[kU], r2[kU], dif[kU][3];
#pragma unroll
    for (int u = 0; u < kU; ++u) j[u] = nxt[u];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if constexpr (!COORD) kraw[u] = ld16(row_at<OFF32>(khead, j[u], skt, sub16));
      vraw[u] = ld16(row_at<OFF32>(vhead, j[u], svt, sub16));
    }
    fetch_idx(p.cols, beg, n, e0 + kU, i, nxt);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if constexpr (COORD) {
        const float* c = ckb + (int64_t)j[u] * 3;
        dif[u][0] = cqi[0] - c[0];
        dif[u][1] = cqi[1] - c[1];
        dif[u][2] = cqi[2] - c[2];
        r2[u] = dif[u][0] * dif[u][0] + dif[u][1] * dif[u][1] + dif[u][2] * dif[u][2];
        s[u] = -gl2 * r2[u];
      } else {
        s[u] = group_sum<LG>(F::dot(qraw, kraw[u], 0.f)) * p.scale_log2;
      }
      dp[u] = group_sum<LG>(F::dot(doraw, vraw[u], 0.f));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float pr = e0 + u < n ? fast_exp2(s[u] - lse2) : 0.f;
      const float pd = pr * dp[u];
      delta += pd;
      if constexpr (!COORD) {
        float kf[EPL];
        F::unpack(kraw[u], kf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          pdx[e] = fmaf(pd, kf[e], pdx[e]);
          px[e] = fmaf(pr, kf[e], px[e]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          cdx[c] = fmaf(pd, dif[u][c], cdx[c]);
          cx[c] = fmaf(pr, dif[u][c], cx[c]);
        }
        r2dx = fmaf(pd, r2[u], r2dx);
        r2x = fmaf(pr, r2[u], r2x);
        psum += pr;
      }
    }
  }
  if (row_ok && sub == 0) p.delta[(int64_t)bh * p.T + i] = delta;

  if constexpr (!COORD) {
    if (row_ok) {
      float dq[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) dq[e] = p.scale * (pdx[e] - delta * px[e]);
      const int gb = p.grad_bf16 ? 2 : 4;
      char* dqrow = static_cast<char*>(p.dq) + (b * p.sdq_b + h * p.sdq_h + i * p.sdq_t) * gb +
                    sub * EPL * gb;
      store_vals<EPL>(dqrow, dq, p.grad_bf16 != 0);
    }
  } else {
    if (row_ok && sub == 0) {
      float* o = p.dcq + ((int64_t)bh * p.T + i) * 3;
#pragma unroll
      for (int c = 0; c < 3; ++c) st_stream(o + c, -2.f * gam * (cdx[c] - delta * cx[c]));
    }
    // dgamma_i = -sum_j dS_ij r2_ij,  dbeta_i = sum_j dS_ij = Delta_i (1 - sum_j P_ij);
    // one value per row, summed per block in a fixed order through LDS
    const bool counts = row_ok && sub == 0;
    __shared__ float red[2][kThreads];
    red[0][threadIdx.x] = counts ? -(r2dx - delta * r2x) : 0.f;
    red[1][threadIdx.x] = counts ? delta * (1.f - psum) : 0.f;
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

// ------------------------------------------------------------------ backward, key side
template <int DT, int D, int SM, bool OFF32>
__global__ __launch_bounds__(kThreads) void csr_bwd_kv_kernel(Params p) {
  constexpr bool COORD = SM == SM_COORD;
  constexpr bool UNIFORM = SM == SM_UNIFORM;  // dv only
  using F = Frag<DT>;
  using Gm = Geo<DT, D>;
  constexpr int EPL = Gm::EPL, LG = Gm::LG, RPW = Gm::RPW, RPB = Gm::RPB;
  constexpr int EB = F::BYTES;

  // one key row per lane group of key/value head hk; its query heads are
  // hk G .. hk G + G - 1 (G = 1 in coordinate mode)
  const int nblk = (p.T + RPB - 1) / RPB;
  const int logical = xcd_logical_block(p.B * p.Hkv * nblk);
  if (logical < 0) return;
  const int bk = logical / nblk, rb = logical - bk * nblk;
  const int b = bk / p.Hkv, hk = bk - b * p.Hkv;
  const int h0 = hk * p.G;
  const int bh = b * p.H + h0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LG;
  int j = rb * RPB + wave * RPW + lane / LG;
  const bool row_ok = j < p.T;
  if (!row_ok) j = p.T - 1;
  const int beg = p.rrp[j];
  const int n = row_ok ? p.rrp[j + 1] - beg : 0;  // may be 0: a key nobody lists
  const int64_t sqt = p.sq_t * EB, sdot = p.sdo_t * EB;
  const uint32_t sub16 = (uint32_t)sub * 16u;
  const float bsub = COORD ? p.beta[h0] : 0.f;

  const uint4 vraw_j =
      ld16(static_cast<const char*>(p.v) + (b * p.sv_b + hk * p.sv_h + j * p.sv_t) * EB + sub16);
  uint4 kraw_j = make_uint4(0u, 0u, 0u, 0u);
  float ckj[3] = {0.f, 0.f, 0.f};
  float gl2 = 0.f, gam = 0.f;
  const float* cqb = nullptr;
  if constexpr (SM == SM_DOT) {
    kraw_j = ld16(static_cast<const char*>(p.k) + (b * p.sk_b + hk * p.sk_h + j * p.sk_t) * EB + sub16);
  } else if constexpr (COORD) {
    const float* c = p.ck + ((int64_t)bh * p.T + j) * 3;
    ckj[0] = c[0]; ckj[1] = c[1]; ckj[2] = c[2];
    gam = p.gamma[h0];
    gl2 = gam * kLog2e;
    cqb = p.cq + (int64_t)bh * p.T * 3;
  }

  float dk[EPL], dv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) dk[e] = dv[e] = 0.f;
  float dc[3] = {0.f, 0.f, 0.f};

  for (int hq = h0; hq < h0 + p.G; ++hq) {  // the query heads of this key/value head, in order
    const char* qhead = static_cast<const char*>(p.q) + (b * p.sq_b + hq * p.sq_h) * EB;
    const char* dohead = static_cast<const char*>(p.dout) + (b * p.sdo_b + hq * p.sdo_h) * EB;
    const float* lseb = p.lse + ((int64_t)b * p.H + hq) * p.T;
    const float* delb = p.delta + ((int64_t)b * p.H + hq) * p.T;
    int nxt[kU];
    fetch_idx(p.rcols, beg, n, 0, j, nxt);
    for (int e0 = 0; __builtin_amdgcn_ballot_w64(e0 < n) != 0; e0 += kU) {
      int i[kU];
      uint4 qraw[kU], doraw[kU];
      float s[kU], dp[kU], lse2[kU], del[kU], dif[kU][3];
#pragma unroll
      for (int u = 0; u < kU; ++u) i[u] = nxt[u];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if constexpr (SM == SM_DOT) qraw[u] = ld16(row_at<OFF32>(qhead, i[u], sqt, sub16));
        doraw[u] = ld16(row_at<OFF32>(dohead, i[u], sdot, sub16));
        lse2[u] = (lseb[i[u]] - bsub) * kLog2e;
        if constexpr (!UNIFORM) del[u] = delb[i[u]];
      }
      fetch_idx(p.rcols, beg, n, e0 + kU, j, nxt);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if constexpr (COORD) {
          const float* c = cqb + (int64_t)i[u] * 3;
          dif[u][0] = c[0] - ckj[0];
          dif[u][1] = c[1] - ckj[1];
          dif[u][2] = c[2] - ckj[2];
          s[u] = -gl2 * (dif[u][0] * dif[u][0] + dif[u][1] * dif[u][1] + dif[u][2] * dif[u][2]);
        } else if constexpr (UNIFORM) {
          s[u] = 0.f;
        } else {
          s[u] = group_sum<LG>(F::dot(qraw[u], kraw_j, 0.f)) * p.scale_log2;
        }
        if constexpr (!UNIFORM) dp[u] = group_sum<LG>(F::dot(doraw[u], vraw_j, 0.f));
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float pr = e0 + u < n ? fast_exp2(s[u] - lse2[u]) : 0.f;
        float dof[EPL];
        F::unpack(doraw[u], dof);
#pragma unroll
        for (int e = 0; e < EPL; ++e) dv[e] = fmaf(pr, dof[e], dv[e]);
        if constexpr (!UNIFORM) {
          const float ds = pr * (dp[u] - del[u]);
          if constexpr (SM == SM_DOT) {
            float qf[EPL];
            F::unpack(qraw[u], qf);
#pragma unroll
            for (int e = 0; e < EPL; ++e) dk[e] = fmaf(ds, qf[e], dk[e]);
          } else {
            dc[0] = fmaf(ds, dif[u][0], dc[0]);
            dc[1] = fmaf(ds, dif[u][1], dc[1]);
            dc[2] = fmaf(ds, dif[u][2], dc[2]);
          }
        }
      }
    }
  }

  if (!row_ok) return;
  const int gb = p.grad_bf16 ? 2 : 4;
  char* dvrow = static_cast<char*>(p.dv) + (b * p.sdv_b + hk * p.sdv_h + j * p.sdv_t) * gb + sub * EPL * gb;
  store_vals<EPL>(dvrow, dv, p.grad_bf16 != 0);
  if constexpr (SM == SM_DOT) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) dk[e] *= p.scale;
    char* dkrow = static_cast<char*>(p.dk) + (b * p.sdk_b + hk * p.sdk_h + j * p.sdk_t) * gb + sub * EPL * gb;
    store_vals<EPL>(dkrow, dk, p.grad_bf16 != 0);
  } else if constexpr (COORD) {
    if (sub == 0) {
      float* o = p.dck + ((int64_t)bh * p.T + j) * 3;
      st_stream(o, 2.f * gam * dc[0]);
      st_stream(o + 1, 2.f * gam * dc[1]);
      st_stream(o + 2, 2.f * gam * dc[2]);
    }
  }
}

// Whether every row offset within one (batch, head) slice of the tensors the
// kernels index fits in 31 bits (then addresses are base + 32-bit offset).
inline bool fits_off32(const Params& p, int eb, bool bwd) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t strides[4] = {p.sk_t, p.sv_t, bwd ? p.sq_t : 0, bwd ? p.sdo_t : 0};
  for (int64_t st : strides)
    if (((int64_t)(p.T - 1) * st + p.D) * eb >= lim) return false;
  return true;
}

template <int DT, int D, int SM>
hipError_t fwd_one(const Params& p, hipStream_t s) {
  constexpr int RPB = Geo<DT, D>::RPB;
  const int grid = xcd_grid(p.B * p.H * ((p.T + RPB - 1) / RPB));
  if (fits_off32(p, Frag<DT>::BYTES, false))
    hipLaunchKernelGGL((csr_fwd_kernel<DT, D, SM, true>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((csr_fwd_kernel<DT, D, SM, false>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int DT, int D, int SM, bool OFF32>
hipError_t bwd_passes(const Params& p, hipStream_t s) {
  constexpr int RPB = Geo<DT, D>::RPB;
  const int nblk = (p.T + RPB - 1) / RPB;
  if constexpr (SM != SM_UNIFORM) {  // no query-side gradient in the uniform mode
    hipLaunchKernelGGL((csr_bwd_q_kernel<DT, D, SM == SM_COORD, OFF32>), dim3(xcd_grid(p.B * p.H * nblk)),
                       dim3(kThreads), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((csr_bwd_kv_kernel<DT, D, SM, OFF32>), dim3(xcd_grid(p.B * p.Hkv * nblk)), dim3(kThreads),
                     0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || SM != SM_COORD) return e;
  return launch_coord_param_reduce(p, nblk, s);
}

template <int DT, int D, int SM>
hipError_t bwd_one(const Params& p, hipStream_t s) {
  return fits_off32(p, Frag<DT>::BYTES, true) ? bwd_passes<DT, D, SM, true>(p, s)
                                              : bwd_passes<DT, D, SM, false>(p, s);
}

template <bool BWD, int DT, int SM>
hipError_t by_d(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 16: return BWD ? bwd_one<DT, 16, SM>(p, s) : fwd_one<DT, 16, SM>(p, s);
    case 32: return BWD ? bwd_one<DT, 32, SM>(p, s) : fwd_one<DT, 32, SM>(p, s);
    case 64: return BWD ? bwd_one<DT, 64, SM>(p, s) : fwd_one<DT, 64, SM>(p, s);
    case 128: return BWD ? bwd_one<DT, 128, SM>(p, s) : fwd_one<DT, 128, SM>(p, s);
  }
  return hipErrorInvalidValue;
}

template <bool BWD, int DT>
hipError_t by_mode(const Params& p, int score_mode, hipStream_t s) {
  switch (score_mode) {
    case SM_DOT: return by_d<BWD, DT, SM_DOT>(p, s);
    case SM_COORD: return by_d<BWD, DT, SM_COORD>(p, s);
    case SM_UNIFORM: return by_d<BWD, DT, SM_UNIFORM>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_csr_fwd(const Params& p, int dtype, int score_mode, hipStream_t s) {
  return dtype == DT_BF16 ? by_mode<false, DT_BF16>(p, score_mode, s) : by_mode<false, DT_F32>(p, score_mode, s);
}

hipError_t launch_csr_bwd(const Params& p, int dtype, int score_mode, hipStream_t s) {
  return dtype == DT_BF16 ? by_mode<true, DT_BF16>(p, score_mode, s) : by_mode<true, DT_F32>(p, score_mode, s);
}

}  // namespace sa

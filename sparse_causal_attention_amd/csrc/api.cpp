// C ABI: argument validation, parameter packing and kernel selection.
//
// Every check runs on the host before the first HIP call, so a rejected call
// has no side effect and the library works for validation on machines with
// no GPU.  Nothing here allocates device memory.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "sa_internal.h"

namespace {

bool bad_dtype(int32_t dt) { return dt != SA_F32 && dt != SA_BF16; }

// Key/value heads (0 selects H).
int64_t kv_heads(const sa_attn_desc* d) { return d->H_kv > 0 ? d->H_kv : d->H; }

// Grouped key/value heads: H a multiple of H_kv; per-head coordinates only.
sa_status check_heads(const sa_attn_desc* d) {
  const int64_t hkv = kv_heads(d);
  if (d->H_kv < 0 || d->H % hkv != 0) return SA_ERR_INVALID_ARG;
  if (hkv != d->H && d->score == SA_SCORE_COORD) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}
int esize(int32_t dt) { return dt == SA_BF16 ? 2 : 4; }

// B, H and B * H at most `limit` (< 2^31), each factor bounded first so that
// the product cannot overflow.
bool heads_fit(const sa_attn_desc* d, int64_t limit) {
  return d->B <= limit && d->H <= limit && d->B * d->H <= limit;
}
// (batch, head) slices the attention calls accept
constexpr int64_t kMaxSlices = (int64_t)1 << 24;

// Row starts 16-byte aligned for 16-byte vector accesses.
bool aligned_rows(const void* p, const int64_t st[3], int es) {
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
  for (int c = 0; c < 3; ++c)
    if (st[c] < 0 || (st[c] * es) % 16 != 0) return false;
  return true;
}

// Largest element offset touched by a [B, H, T, D] tensor with these strides.
bool offsets_fit(const sa_attn_desc* d, const int64_t st[3]) {
  const double last = (double)(d->B - 1) * st[0] + (double)(d->H - 1) * st[1] +
                      (double)(d->T - 1) * st[2] + (double)d->D;
  return last < 9.0e18;
}

// Output rows must not overlap (a zero or too-small stride would let several
// workgroups store the same row, in no fixed order).  Sufficient test: with
// the dimensions of extent above 1 ordered by stride, each stride covers the
// span of everything inside it, starting from the D contiguous elements of a
// row.  Called after offsets_fit, so no product below overflows.
bool rows_disjoint(int64_t n0, int64_t n1, int64_t n2, const int64_t st[3], int64_t D) {
  int64_t n[3] = {n0, n1, n2}, s[3] = {st[0], st[1], st[2]};
  for (int a = 0; a < 3; ++a)  // order by stride (three elements)
    for (int b = a + 1; b < 3; ++b)
      if (s[b] < s[a]) {
        const int64_t tn = n[a], ts = s[a];
        n[a] = n[b]; s[a] = s[b];
        n[b] = tn; s[b] = ts;
      }
  int64_t span = D;
  for (int a = 0; a < 3; ++a) {
    if (n[a] <= 1) continue;
    if (s[a] < span) return false;
    span += s[a] * (n[a] - 1);
  }
  return true;
}

enum class Path { Gather, Band, Csr };

// The band backward loads its tiles through buffer resources over one (batch,
// head) slice of q, k, v and dout, with 32-bit offsets, and holds their
// strides as 32-bit values: each slice must span fewer than 2^31 bytes and
// each stride be below 2^31 elements, else the backward takes the gather
// kernels.
bool band_bwd_slices_fit(const sa_attn_desc* d) {
  const double es = d->dtype == SA_BF16 ? 2.0 : 4.0;
  auto fits = [&](const int64_t st[3]) {
    for (int c = 0; c < 3; ++c)
      if (st[c] >= ((int64_t)1 << 31)) return false;
    return ((double)(d->T - 1) * st[2] + (double)d->D) * es < 2147483648.0;
  };
  return fits(d->stride_q) && fits(d->stride_k) && fits(d->stride_v) && fits(d->stride_do);
}

struct Plan {
  Path path;
};

sa_status check_common(const sa_graph* g, const sa_attn_desc* d, const void* q, const void* k,
                       const void* v, const float* cq, const float* ck, const float* gamma,
                       const float* beta, Plan* plan) {
  if (g == nullptr || d == nullptr) return SA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->D < 1) return SA_ERR_INVALID_ARG;
  if (bad_dtype(d->dtype) || bad_dtype(d->grad_dtype)) return SA_ERR_INVALID_ARG;
  if (d->score != SA_SCORE_DOT && d->score != SA_SCORE_COORD && d->score != SA_SCORE_UNIFORM)
    return SA_ERR_INVALID_ARG;
  if (d->algo != SA_ALGO_AUTO && d->algo != SA_ALGO_GATHER && d->algo != SA_ALGO_BAND)
    return SA_ERR_INVALID_ARG;
  if (d->T != g->T) return SA_ERR_SHAPE_MISMATCH;
  if (d->D != 16 && d->D != 32 && d->D != 64 && d->D != 128) return SA_ERR_UNSUPPORTED;
  if (!heads_fit(d, kMaxSlices)) return SA_ERR_UNSUPPORTED;
  if (const sa_status hs = check_heads(d); hs != SA_OK) return hs;
  // workgroups of the smallest row tile (8 rows: fp32, D = 128), plus the
  // XCD padding of the grid, must be countable in int32
  if (d->B * d->H * ((d->T + 7) / 8) > ((int64_t)1 << 31) - 64) return SA_ERR_UNSUPPORTED;
  const int es = esize(d->dtype);
  if (v == nullptr || !aligned_rows(v, d->stride_v, es) || !offsets_fit(d, d->stride_v))
    return SA_ERR_INVALID_ARG;
  if (d->score == SA_SCORE_DOT) {
    if (q == nullptr || k == nullptr) return SA_ERR_INVALID_ARG;
    if (!aligned_rows(q, d->stride_q, es) || !aligned_rows(k, d->stride_k, es))
      return SA_ERR_INVALID_ARG;
    if (!offsets_fit(d, d->stride_q) || !offsets_fit(d, d->stride_k)) return SA_ERR_INVALID_ARG;
    if (!(d->scale == d->scale)) return SA_ERR_INVALID_ARG;  // NaN scale
  } else if (d->score == SA_SCORE_COORD) {
    if (cq == nullptr || ck == nullptr || gamma == nullptr || beta == nullptr)
      return SA_ERR_INVALID_ARG;
  }  // uniform mode reads v alone
  const bool csr = g->kind == SA_GRAPH_CSR;
  const bool band_ok = !csr && sa::band_supported(d->dtype, (int)d->D, d->score, g->W);
  if (d->algo == SA_ALGO_BAND && !band_ok) return SA_ERR_UNSUPPORTED;
  plan->path = csr ? Path::Csr : (d->algo != SA_ALGO_GATHER && band_ok) ? Path::Band : Path::Gather;
  return SA_OK;
}

// An explicit-list graph is usable once its lists are in device memory.
bool lists_ready(const sa_graph* g) { return g->kind != SA_GRAPH_CSR || g->d_rp != nullptr; }

void fill_common(sa::Params* p, const sa_graph* g, const sa_attn_desc* d) {
  memset(p, 0, sizeof(*p));
  p->B = (int32_t)d->B;
  p->H = (int32_t)d->H;
  p->T = (int32_t)d->T;
  p->D = (int32_t)d->D;
  p->W = (int32_t)g->W;
  p->Hkv = (int32_t)kv_heads(d);
  p->G = (int32_t)(d->H / p->Hkv);
  p->n_dil = g->n_dil;
  for (int t = 0; t < SA_MAX_DILATED + 8; ++t)
    p->dil[t] = t < g->n_dil ? (int32_t)g->dil[t] : sa::kUnreachable;
  p->scale = d->scale > 0.f ? d->scale : (float)(1.0 / sqrt((double)d->D));
  p->scale_log2 = p->scale * 1.4426950408889634f;
  p->grad_bf16 = d->grad_dtype == SA_BF16;
  if (g->kind == SA_GRAPH_CSR) {
    p->rp = g->d_rp;
    p->cols = g->d_cols;
    p->rrp = g->d_rrp;
    p->rcols = g->d_rcols;
  }
}

#define SET_STRIDES(prefix, arr) \
  p.prefix##_b = (arr)[0];       \
  p.prefix##_h = (arr)[1];       \
  p.prefix##_t = (arr)[2]

hipStream_t as_stream(sa_stream s) { return reinterpret_cast<hipStream_t>(s); }

const char* fwd_kernel_name(const sa_attn_desc* d, Path path) {
  if (path == Path::Band) return "band_fwd_kernel";
  if (path == Path::Csr) {
    if (d->score == SA_SCORE_COORD) return "csr_fwd_kernel(coord)";
    return d->score == SA_SCORE_UNIFORM ? "csr_fwd_kernel(uniform)" : "csr_fwd_kernel(dot)";
  }
  if (d->score == SA_SCORE_COORD) return "gather_fwd_kernel(coord)";
  return d->score == SA_SCORE_UNIFORM ? "gather_fwd_kernel(uniform)" : "gather_fwd_kernel(dot)";
}

const char* bwd_kernel_names(const sa_attn_desc* d, Path path) {
  const bool coord = d->score == SA_SCORE_COORD, uniform = d->score == SA_SCORE_UNIFORM;
  if (path == Path::Band) return "band_bwd_prepass_kernel+band_bwd_kernel";
  if (path == Path::Csr)
    return coord ? "csr_bwd_q_kernel(coord)+csr_bwd_kv_kernel(coord)+coord_param_reduce_kernel"
           : uniform ? "csr_bwd_kv_kernel(uniform)"
                     : "csr_bwd_q_kernel(dot)+csr_bwd_kv_kernel(dot)";
  return coord ? "gather_bwd_q_kernel(coord)+gather_bwd_kv_kernel(coord)+coord_param_reduce_kernel"
         : uniform ? "gather_bwd_kv_kernel(uniform)"
                   : "gather_bwd_q_kernel(dot)+gather_bwd_kv_kernel(dot)";
}

}  // namespace

extern "C" sa_status sa_fwd(const sa_graph* g, const sa_attn_desc* d, const void* q, const void* k,
                            const void* v, const float* cq, const float* ck, const float* gamma,
                            const float* beta, void* o, float* lse, sa_stream stream) {
  Plan plan;
  sa_status st = check_common(g, d, q, k, v, cq, ck, gamma, beta, &plan);
  if (st != SA_OK) return st;
  if (o == nullptr || lse == nullptr || !lists_ready(g)) return SA_ERR_INVALID_ARG;
  if (!aligned_rows(o, d->stride_o, esize(d->dtype)) || !offsets_fit(d, d->stride_o) ||
      !rows_disjoint(d->B, d->H, d->T, d->stride_o, d->D))
    return SA_ERR_INVALID_ARG;
  sa::Params p;
  fill_common(&p, g, d);
  p.q = q; SET_STRIDES(sq, d->stride_q);
  p.k = k; SET_STRIDES(sk, d->stride_k);
  p.v = v; SET_STRIDES(sv, d->stride_v);
  p.o = o; SET_STRIDES(so, d->stride_o);
  p.cq = cq; p.ck = ck; p.gamma = gamma; p.beta = beta;
  p.lse = lse;
  const int dt = d->dtype == SA_BF16 ? sa::DT_BF16 : sa::DT_F32;
  hipError_t e = plan.path == Path::Band  ? sa::launch_band_fwd(p, as_stream(stream))
                 : plan.path == Path::Csr ? sa::launch_csr_fwd(p, dt, d->score, as_stream(stream))
                                          : sa::launch_gather_fwd(p, dt, d->score, as_stream(stream));
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes_for(const sa_attn_desc* d) {
  const size_t rows = (size_t)d->B * d->H * d->T;
  const int rpb = sa::gather_rows_per_block(d->dtype == SA_BF16 ? sa::DT_BF16 : sa::DT_F32,
                                            (int)d->D);
  const size_t nblk = (size_t)((d->T + rpb - 1) / rpb);
  return 2 * align256(rows * sizeof(float)) + align256((size_t)d->B * d->H * nblk * 2 * sizeof(float));
}

}  // namespace

extern "C" sa_status sa_bwd_workspace_size(const sa_graph* g, const sa_attn_desc* d,
                                           size_t* bytes) {
  if (bytes == nullptr || g == nullptr || d == nullptr) return SA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 1) return SA_ERR_INVALID_ARG;
  if (bad_dtype(d->dtype)) return SA_ERR_INVALID_ARG;
  if (d->D != 16 && d->D != 32 && d->D != 64 && d->D != 128) return SA_ERR_UNSUPPORTED;
  if (d->T != g->T) return SA_ERR_SHAPE_MISMATCH;
  if (!heads_fit(d, kMaxSlices)) return SA_ERR_UNSUPPORTED;  // as sa_bwd: no wrapped sizes
  if (const sa_status hs = check_heads(d); hs != SA_OK) return hs;
  *bytes = workspace_bytes_for(d);
  return SA_OK;
}

namespace {

// Everything sa_bwd checks except the workspace: the graph, shapes, dtypes,
// pointers and strides of inputs and outputs.  Chooses the kernel path.
sa_status bwd_validate(const sa_graph* g, const sa_attn_desc* d, const void* q, const void* k,
                       const void* v, const float* cq, const float* ck, const float* gamma,
                       const float* beta, const void* o, const float* lse, const void* dout, void* dq,
                       void* dk, void* dv, float* dcq, float* dck, float* dgamma, float* dbeta,
                       Plan* plan) {
  sa_status st = check_common(g, d, q, k, v, cq, ck, gamma, beta, plan);
  if (st != SA_OK) return st;
  if (plan->path == Path::Band && !band_bwd_slices_fit(d)) {
    if (d->algo == SA_ALGO_BAND) return SA_ERR_UNSUPPORTED;
    plan->path = Path::Gather;
  }
  const bool coord = d->score == SA_SCORE_COORD;
  const int es = esize(d->dtype), gs = esize(d->grad_dtype);
  if (o == nullptr || lse == nullptr || dout == nullptr || dv == nullptr || !lists_ready(g))
    return SA_ERR_INVALID_ARG;
  if (!aligned_rows(o, d->stride_o, es) || !aligned_rows(dout, d->stride_do, es))
    return SA_ERR_INVALID_ARG;
  if (!offsets_fit(d, d->stride_o) || !offsets_fit(d, d->stride_do)) return SA_ERR_INVALID_ARG;
  // gradient rows: 16-byte aligned starts, like the inputs, and disjoint
  auto grad_ok = [&](const void* ptr, const int64_t s[3], int64_t heads) {
    if ((reinterpret_cast<uintptr_t>(ptr) & 15u) != 0) return false;
    for (int c = 0; c < 3; ++c)
      if (s[c] < 0 || (s[c] * gs) % 16 != 0) return false;
    return offsets_fit(d, s) && rows_disjoint(d->B, heads, d->T, s, d->D);
  };
  const int64_t hkv = kv_heads(d);
  if (!grad_ok(dv, d->stride_dv, hkv)) return SA_ERR_INVALID_ARG;
  if (d->score == SA_SCORE_DOT) {
    if (dq == nullptr || dk == nullptr) return SA_ERR_INVALID_ARG;
    if (!grad_ok(dq, d->stride_dq, d->H) || !grad_ok(dk, d->stride_dk, hkv)) return SA_ERR_INVALID_ARG;
  } else if (coord) {
    if (dcq == nullptr || dck == nullptr || dgamma == nullptr || dbeta == nullptr)
      return SA_ERR_INVALID_ARG;
  }  // uniform mode writes dv alone
  return SA_OK;
}

// Packs the parameters of a validated backward and launches its kernels with
// `ws` (256-byte aligned, workspace_bytes_for(d) bytes) as the workspace.
// Nothing in the workspace needs to start at zero: every kernel writes the
// per-row and per-block values it later reads within the same call.
sa_status bwd_launch(const sa_graph* g, const sa_attn_desc* d, Path path, const void* q, const void* k,
                     const void* v, const float* cq, const float* ck, const float* gamma,
                     const float* beta, const void* o, const float* lse, const void* dout, void* dq,
                     void* dk, void* dv, float* dcq, float* dck, float* dgamma, float* dbeta, char* ws,
                     sa_stream stream) {
  sa::Params p;
  fill_common(&p, g, d);
  p.q = q; SET_STRIDES(sq, d->stride_q);
  p.k = k; SET_STRIDES(sk, d->stride_k);
  p.v = v; SET_STRIDES(sv, d->stride_v);
  p.o = const_cast<void*>(o); SET_STRIDES(so, d->stride_o);
  p.dout = dout; SET_STRIDES(sdo, d->stride_do);
  p.dq = dq; SET_STRIDES(sdq, d->stride_dq);
  p.dk = dk; SET_STRIDES(sdk, d->stride_dk);
  p.dv = dv; SET_STRIDES(sdv, d->stride_dv);
  p.cq = cq; p.ck = ck; p.gamma = gamma; p.beta = beta;
  p.dcq = dcq; p.dck = dck; p.dgamma = dgamma; p.dbeta = dbeta;
  p.lse = const_cast<float*>(lse);
  const size_t row_bytes = align256((size_t)d->B * d->H * d->T * sizeof(float));
  p.delta = reinterpret_cast<float*>(ws);
  p.ndelta = p.delta;
  p.lse2 = reinterpret_cast<float*>(ws + row_bytes);
  p.partials = reinterpret_cast<float*>(ws + 2 * row_bytes);
  const int dt = d->dtype == SA_BF16 ? sa::DT_BF16 : sa::DT_F32;
  hipError_t e = path == Path::Band  ? sa::launch_band_bwd(p, as_stream(stream))
                 : path == Path::Csr ? sa::launch_csr_bwd(p, dt, d->score, as_stream(stream))
                                     : sa::launch_gather_bwd(p, dt, d->score, as_stream(stream));
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace

extern "C" sa_status sa_bwd(const sa_graph* g, const sa_attn_desc* d, const void* q, const void* k,
                            const void* v, const float* cq, const float* ck, const float* gamma,
                            const float* beta, const void* o, const float* lse, const void* dout,
                            void* dq, void* dk, void* dv, float* dcq, float* dck, float* dgamma,
                            float* dbeta, void* workspace, size_t workspace_bytes,
                            sa_stream stream) {
  Plan plan;
  const sa_status st = bwd_validate(g, d, q, k, v, cq, ck, gamma, beta, o, lse, dout, dq, dk, dv, dcq, dck,
                                    dgamma, dbeta, &plan);
  if (st != SA_OK) return st;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SA_ERR_WORKSPACE;
  if (workspace_bytes < workspace_bytes_for(d)) return SA_ERR_WORKSPACE;
  return bwd_launch(g, d, plan.path, q, k, v, cq, ck, gamma, beta, o, lse, dout, dq, dk, dv, dcq, dck,
                    dgamma, dbeta, static_cast<char*>(workspace), stream);
}

// ------------------------------------------------------------------ allocation-free backward
// The backward's workspace as a file-scope device array, for callers that
// cannot allocate (graph capture, tight serving loops).  In host code the
// name `scratch` is only a host-side stand-in: kernels get the device address
// that hipGetSymbolAddress returns for the current device, looked up on the
// first call on each device and kept per device (every GPU has its own copy).
static __device__ __align__(256) char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<char*> g_scratch_ptr[kMaxScratchDevices];

// Device address of this device's `scratch`, or nullptr when the lookup fails.
char* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  char* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
  ptr = static_cast<char*>(addr);
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // racing first calls store the same address
  return ptr;
}

}  // namespace

extern "C" sa_status sa_bwd_noalloc(const sa_graph* g, const sa_attn_desc* d, const void* q,
                                    const void* k, const void* v, const float* cq, const float* ck,
                                    const float* gamma, const float* beta, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                    float* dcq, float* dck, float* dgamma, float* dbeta,
                                    sa_stream stream) {
  Plan plan;
  const sa_status st = bwd_validate(g, d, q, k, v, cq, ck, gamma, beta, o, lse, dout, dq, dk, dv, dcq, dck,
                                    dgamma, dbeta, &plan);
  if (st != SA_OK) return st;
  if (workspace_bytes_for(d) > (size_t)SA_NOALLOC_SCRATCH_BYTES) return SA_ERR_WORKSPACE;
  char* ws = scratch_on_current_device();
  if (ws == nullptr) return SA_ERR_HIP;
  return bwd_launch(g, d, plan.path, q, k, v, cq, ck, gamma, beta, o, lse, dout, dq, dk, dv, dcq, dck,
                    dgamma, dbeta, ws, stream);
}

extern "C" sa_status sa_decode(const sa_graph* g, const sa_attn_desc* d, const int32_t* positions,
                               const void* q, const void* k, const void* v, const float* cq,
                               const float* ck, const float* gamma, const float* beta, void* o,
                               float* lse, sa_stream stream) {
  if (g == nullptr || d == nullptr) return SA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->D < 1) return SA_ERR_INVALID_ARG;
  if (bad_dtype(d->dtype)) return SA_ERR_INVALID_ARG;
  if (d->score != SA_SCORE_DOT && d->score != SA_SCORE_COORD && d->score != SA_SCORE_UNIFORM)
    return SA_ERR_INVALID_ARG;
  if (d->T != g->T) return SA_ERR_SHAPE_MISMATCH;
  if (d->D != 16 && d->D != 32 && d->D != 64 && d->D != 128) return SA_ERR_UNSUPPORTED;
  if (!heads_fit(d, ((int64_t)1 << 31) - 1)) return SA_ERR_UNSUPPORTED;  // one workgroup per (b, h)
  if (const sa_status hs = check_heads(d); hs != SA_OK) return hs;
  const int es = esize(d->dtype);
  const int64_t row_only[3] = {d->stride_q[0], d->stride_q[1], 0};
  const int64_t o_row[3] = {d->stride_o[0], d->stride_o[1], 0};
  if (v == nullptr || !aligned_rows(v, d->stride_v, es) || !offsets_fit(d, d->stride_v))
    return SA_ERR_INVALID_ARG;
  if (d->score == SA_SCORE_DOT) {
    if (q == nullptr || k == nullptr) return SA_ERR_INVALID_ARG;
    if (!aligned_rows(q, row_only, es) || !aligned_rows(k, d->stride_k, es)) return SA_ERR_INVALID_ARG;
    if (!offsets_fit(d, row_only) || !offsets_fit(d, d->stride_k)) return SA_ERR_INVALID_ARG;
    if (!(d->scale == d->scale)) return SA_ERR_INVALID_ARG;  // NaN scale
  } else if (d->score == SA_SCORE_COORD) {
    if (cq == nullptr || ck == nullptr || gamma == nullptr || beta == nullptr) return SA_ERR_INVALID_ARG;
  }
  if (o == nullptr || lse == nullptr || !lists_ready(g)) return SA_ERR_INVALID_ARG;
  if (!aligned_rows(o, o_row, es) || !offsets_fit(d, o_row) || !rows_disjoint(d->B, d->H, 1, o_row, d->D))
    return SA_ERR_INVALID_ARG;
  sa::Params p;
  fill_common(&p, g, d);
  p.q = q; SET_STRIDES(sq, d->stride_q);
  p.k = k; SET_STRIDES(sk, d->stride_k);
  p.v = v; SET_STRIDES(sv, d->stride_v);
  p.o = o; SET_STRIDES(so, d->stride_o);
  p.cq = cq; p.ck = ck; p.gamma = gamma; p.beta = beta;
  p.lse = lse;
  p.pos = positions;
  const hipError_t e = sa::launch_decode(p, d->dtype == SA_BF16 ? sa::DT_BF16 : sa::DT_F32, d->score,
                                         as_stream(stream));
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" sa_status sa_describe_plan(const sa_graph* g, const sa_attn_desc* d, int32_t which,
                                      char* buf, size_t cap) {
  if (buf == nullptr || cap == 0 || (which != 0 && which != 1)) return SA_ERR_INVALID_ARG;
  if (d == nullptr) return SA_ERR_INVALID_ARG;
  Plan plan;
  // validates the shape, dtype and mode parts; pointers and strides are not
  // needed to choose kernels, so stand-ins are used for them
  alignas(16) static const float dummy[4] = {0.f, 0.f, 0.f, 0.f};
  sa_attn_desc tmp = *d;
  for (int c = 0; c < 3; ++c) tmp.stride_q[c] = tmp.stride_k[c] = tmp.stride_v[c] = 0;
  sa_status st = check_common(g, &tmp, dummy, dummy, dummy, dummy, dummy, dummy, dummy, &plan);
  if (st != SA_OK) return st;
  if (which == 1 && plan.path == Path::Band && !band_bwd_slices_fit(d)) {
    if (d->algo == SA_ALGO_BAND) return SA_ERR_UNSUPPORTED;
    plan.path = Path::Gather;
  }
  snprintf(buf, cap, "%s", which == 0 ? fwd_kernel_name(d, plan.path) : bwd_kernel_names(d, plan.path));
  return SA_OK;
}

extern "C" const char* sa_status_str(sa_status s) {
  switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_SHAPE_MISMATCH: return "graph length differs from descriptor length";
    case SA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SA_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

namespace sa {
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < kMaxDevices ? dev : kMaxDevices - 1;
  int n = cached[slot].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[slot].store(n, std::memory_order_relaxed);
  return n;
}
}  // namespace sa

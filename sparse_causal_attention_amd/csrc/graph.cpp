// Neighbour-graph construction and CSR export (host, integer only), and the
// upload of explicit lists into caller-owned device memory.
//
// The graph of the SpatialLM-Mini news page ("How tokens choose whom to
// listen to") is translation invariant: row i's keys are i - delta for a
// fixed set of distances.  It is therefore stored as its normalised
// descriptor {T, W' = min(W, T), sorted distinct long-range distances in
// [W', T)} and never materialised for the kernels; CSR rows are produced on
// request only (tests, users who want the explicit lists).
//
// Any other causal graph (the general view of "Longer Attention Span ...",
// abstract: the mask as the edge set of a graph over the tokens) is given as
// explicit per-row lists.  The builder checks them, forms the reverse lists
// (for each key, the queries that list it) by a counting pass, and keeps
// both as int32 CSR on the host until sa_graph_upload copies them to device
// memory the caller provides.
#include <algorithm>
#include <new>
#include <vector>

#include "sa_internal.h"

namespace {

sa_status normalise(int64_t T, int64_t window, const int64_t* offsets, int32_t n_offsets,
                    sa_graph* g) {
  if (T < 1 || window < 1 || n_offsets < 0 || (n_offsets > 0 && offsets == nullptr))
    return SA_ERR_INVALID_ARG;
  for (int32_t t = 0; t < n_offsets; ++t)
    if (offsets[t] < 0) return SA_ERR_INVALID_ARG;  // a negative distance looks ahead
  if (T > INT32_MAX) return SA_ERR_UNSUPPORTED;
  const int64_t w = window < T ? window : T;
  std::vector<int64_t> keep;
  keep.reserve(static_cast<size_t>(n_offsets));
  for (int32_t t = 0; t < n_offsets; ++t)
    if (offsets[t] >= w && offsets[t] < T) keep.push_back(offsets[t]);
  std::sort(keep.begin(), keep.end());
  keep.erase(std::unique(keep.begin(), keep.end()), keep.end());
  if (keep.size() > SA_MAX_DILATED) return SA_ERR_UNSUPPORTED;
  g->kind = SA_GRAPH_DISTANCE;
  g->T = T;
  g->W = w;
  g->n_dil = static_cast<int32_t>(keep.size());
  for (size_t t = 0; t < keep.size(); ++t) g->dil[t] = keep[t];
  // E = sum_i min(i+1, W) + sum_d (T - d)
  int64_t e = w * (w + 1) / 2 + w * (T - w);
  for (int64_t d : keep) e += T - d;
  g->n_edges = e;
  return SA_OK;
}

}  // namespace

extern "C" sa_status sa_build_graph(int64_t T, int64_t window, const int64_t* offsets,
                                    int32_t n_offsets, sa_graph** out) {
  if (out == nullptr) return SA_ERR_INVALID_ARG;
  sa_graph tmp{};
  sa_status st = normalise(T, window, offsets, n_offsets, &tmp);
  if (st != SA_OK) return st;
  sa_graph* g = new (std::nothrow) sa_graph(tmp);
  if (g == nullptr) return SA_ERR_INVALID_ARG;
  *out = g;
  return SA_OK;
}

extern "C" sa_status sa_build_graph_csr(int64_t T, const int64_t* row_ptr, const int64_t* cols,
                                        sa_graph** out) {
  if (out == nullptr || row_ptr == nullptr || T < 1) return SA_ERR_INVALID_ARG;
  if (T > INT32_MAX) return SA_ERR_UNSUPPORTED;
  if (row_ptr[0] != 0) return SA_ERR_INVALID_ARG;
  for (int64_t i = 0; i < T; ++i)
    if (row_ptr[i + 1] <= row_ptr[i]) return SA_ERR_INVALID_ARG;  // every row lists a key
  const int64_t E = row_ptr[T];
  if (E > INT32_MAX) return SA_ERR_UNSUPPORTED;
  if (cols == nullptr) return SA_ERR_INVALID_ARG;
  for (int64_t i = 0; i < T; ++i)
    for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      if (cols[e] < 0 || cols[e] > i) return SA_ERR_INVALID_ARG;       // causal
      if (e > row_ptr[i] && cols[e] <= cols[e - 1]) return SA_ERR_INVALID_ARG;  // ascending, distinct
    }
  sa_graph* g = new (std::nothrow) sa_graph();
  if (g == nullptr) return SA_ERR_INVALID_ARG;
  try {
    g->kind = SA_GRAPH_CSR;
    g->T = T;
    g->W = 0;
    g->n_dil = 0;
    g->n_edges = E;
    g->rp.assign(row_ptr, row_ptr + T + 1);
    g->cols.assign(cols, cols + E);
    // reverse lists: count per key, prefix sum, then fill walking rows in
    // ascending order, so each key's queries come out ascending
    g->rrp.assign(static_cast<size_t>(T) + 1, 0);
    for (int64_t e = 0; e < E; ++e) ++g->rrp[static_cast<size_t>(cols[e]) + 1];
    for (int64_t j = 0; j < T; ++j) g->rrp[j + 1] += g->rrp[j];
    g->rcols.resize(static_cast<size_t>(E));
    std::vector<int32_t> fill(g->rrp.begin(), g->rrp.end() - 1);
    for (int64_t i = 0; i < T; ++i)
      for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) g->rcols[fill[cols[e]]++] = (int32_t)i;
  } catch (const std::bad_alloc&) {
    delete g;
    return SA_ERR_INVALID_ARG;
  }
  *out = g;
  return SA_OK;
}

extern "C" sa_status sa_graph_kind(const sa_graph* g, int32_t* kind) {
  if (g == nullptr || kind == nullptr) return SA_ERR_INVALID_ARG;
  *kind = g->kind;
  return SA_OK;
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// device layout of the lists: rp [T+1], cols [E], rrp [T+1], rcols [E], int32,
// each segment 256-byte aligned
size_t ptr_bytes(const sa_graph* g) { return align256(sizeof(int32_t) * (size_t)(g->T + 1)); }
size_t col_bytes(const sa_graph* g) { return align256(sizeof(int32_t) * (size_t)g->n_edges); }
}  // namespace

extern "C" sa_status sa_graph_device_bytes(const sa_graph* g, size_t* bytes) {
  if (g == nullptr || bytes == nullptr) return SA_ERR_INVALID_ARG;
  *bytes = g->kind == SA_GRAPH_CSR ? 2 * (ptr_bytes(g) + col_bytes(g)) : 0;
  return SA_OK;
}

extern "C" sa_status sa_graph_upload(sa_graph* g, void* device_buf, size_t bytes, sa_stream stream) {
  if (g == nullptr) return SA_ERR_INVALID_ARG;
  if (g->kind != SA_GRAPH_CSR) return SA_OK;  // nothing lives on the device
  const size_t pb = ptr_bytes(g), cb = col_bytes(g);
  if (device_buf == nullptr || (reinterpret_cast<uintptr_t>(device_buf) & 255u) != 0 ||
      bytes < 2 * (pb + cb))
    return SA_ERR_INVALID_ARG;
  // the device lists are fixed once uploaded: calls in flight on another
  // stream may be reading them, so the handle is never re-pointed
  if (g->d_rp != nullptr) return SA_ERR_INVALID_ARG;
  char* base = static_cast<char*>(device_buf);
  int32_t* d_rp = reinterpret_cast<int32_t*>(base);
  int32_t* d_cols = reinterpret_cast<int32_t*>(base + pb);
  int32_t* d_rrp = reinterpret_cast<int32_t*>(base + pb + cb);
  int32_t* d_rcols = reinterpret_cast<int32_t*>(base + 2 * pb + cb);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t np = sizeof(int32_t) * (size_t)(g->T + 1), nc = sizeof(int32_t) * (size_t)g->n_edges;
  // host sources are pageable and owned by the graph: copy, then wait, so
  // the lists are in place and the host vectors free to go when this returns
  if (hipMemcpyAsync(d_rp, g->rp.data(), np, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(d_cols, g->cols.data(), nc, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(d_rrp, g->rrp.data(), np, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(d_rcols, g->rcols.data(), nc, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return SA_ERR_HIP;
  g->d_rp = d_rp;
  g->d_cols = d_cols;
  g->d_rrp = d_rrp;
  g->d_rcols = d_rcols;
  return SA_OK;
}

extern "C" void sa_graph_free(sa_graph* g) { delete g; }

extern "C" sa_status sa_graph_info(const sa_graph* g, int64_t* T, int64_t* window, int32_t* n_dil,
                                   int64_t* dil, int64_t* n_edges) {
  if (g == nullptr) return SA_ERR_INVALID_ARG;
  if (T) *T = g->T;
  if (window) *window = g->W;
  if (n_dil) *n_dil = g->n_dil;
  if (dil)
    for (int32_t t = 0; t < g->n_dil; ++t) dil[t] = g->dil[t];
  if (n_edges) *n_edges = g->n_edges;
  return SA_OK;
}

// Row i: long-range keys i - d for d = largest .. smallest kept distance with
// d <= i (all below the window, since every kept d >= W), then the window
// max(0, i-W+1) .. i.  This is ascending j by construction.
static int64_t row_degree(const sa_graph* g, int64_t i) {
  int64_t n = std::min<int64_t>(i + 1, g->W);
  for (int32_t t = 0; t < g->n_dil; ++t) n += (g->dil[t] <= i);
  return n;
}

// Reverse row j: queries j + delta < T, ascending: the window j .. min(T-1,
// j+W-1), then j + d for each kept d (all beyond the window) with j + d < T.
static int64_t rev_degree(const sa_graph* g, int64_t j) {
  int64_t n = std::min<int64_t>(g->T - j, g->W);
  for (int32_t t = 0; t < g->n_dil; ++t) n += (j + g->dil[t] < g->T);
  return n;
}

// Rows [r0, r1) of explicit lists (ptr, idx), as int64 CSR.
static sa_status export_lists(const std::vector<int32_t>& ptr, const std::vector<int32_t>& idx, int64_t r0,
                              int64_t r1, int64_t* row_ptr, int64_t* cols, int64_t cols_cap) {
  row_ptr[0] = 0;
  for (int64_t r = r0; r < r1; ++r) row_ptr[r - r0 + 1] = row_ptr[r - r0] + (ptr[r + 1] - ptr[r]);
  const int64_t need = row_ptr[r1 - r0];
  if (need > cols_cap || (need > 0 && cols == nullptr)) return SA_ERR_INVALID_ARG;
  for (int64_t e = 0; e < need; ++e) cols[e] = idx[ptr[r0] + e];
  return SA_OK;
}

template <bool REVERSE>
static sa_status export_rows(const sa_graph* g, int64_t r0, int64_t r1, int64_t* row_ptr,
                             int64_t* cols, int64_t cols_cap) {
  if (g == nullptr || row_ptr == nullptr || r0 < 0 || r1 < r0 || r1 > g->T || cols_cap < 0)
    return SA_ERR_INVALID_ARG;
  if (g->kind == SA_GRAPH_CSR)
    return REVERSE ? export_lists(g->rrp, g->rcols, r0, r1, row_ptr, cols, cols_cap)
                   : export_lists(g->rp, g->cols, r0, r1, row_ptr, cols, cols_cap);
  row_ptr[0] = 0;
  for (int64_t r = r0; r < r1; ++r)
    row_ptr[r - r0 + 1] = row_ptr[r - r0] + (REVERSE ? rev_degree(g, r) : row_degree(g, r));
  const int64_t need = row_ptr[r1 - r0];
  if (need > cols_cap || (need > 0 && cols == nullptr)) return SA_ERR_INVALID_ARG;
  int64_t e = 0;
  for (int64_t r = r0; r < r1; ++r) {
    if (!REVERSE) {
      for (int32_t t = g->n_dil - 1; t >= 0; --t)
        if (g->dil[t] <= r) cols[e++] = r - g->dil[t];
      for (int64_t j = std::max<int64_t>(0, r - g->W + 1); j <= r; ++j) cols[e++] = j;
    } else {
      const int64_t hi = std::min<int64_t>(g->T - 1, r + g->W - 1);
      for (int64_t i = r; i <= hi; ++i) cols[e++] = i;
      for (int32_t t = 0; t < g->n_dil; ++t)
        if (r + g->dil[t] < g->T) cols[e++] = r + g->dil[t];
    }
  }
  return SA_OK;
}

extern "C" sa_status sa_graph_rows(const sa_graph* g, int64_t row_begin, int64_t row_end,
                                   int64_t* row_ptr, int64_t* cols, int64_t cols_cap) {
  return export_rows<false>(g, row_begin, row_end, row_ptr, cols, cols_cap);
}

extern "C" sa_status sa_graph_rows_reverse(const sa_graph* g, int64_t row_begin, int64_t row_end,
                                           int64_t* row_ptr, int64_t* cols, int64_t cols_cap) {
  return export_rows<true>(g, row_begin, row_end, row_ptr, cols, cols_cap);
}

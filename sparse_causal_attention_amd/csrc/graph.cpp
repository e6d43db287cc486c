// Neighbour-graph construction and CSR export (host only, integer only).
//
// The graph of the SpatialLM-Mini news page ("How tokens choose whom to
// listen to") is translation invariant: row i's keys are i - delta for a
// fixed set of distances.  It is therefore stored as its normalised
// descriptor {T, W' = min(W, T), sorted distinct long-range distances in
// [W', T)} and never materialised for the kernels; CSR rows are produced on
// request only (tests, users who want the explicit lists).
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

template <bool REVERSE>
static sa_status export_rows(const sa_graph* g, int64_t r0, int64_t r1, int64_t* row_ptr,
                             int64_t* cols, int64_t cols_cap) {
  if (g == nullptr || row_ptr == nullptr || r0 < 0 || r1 < r0 || r1 > g->T || cols_cap < 0)
    return SA_ERR_INVALID_ARG;
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

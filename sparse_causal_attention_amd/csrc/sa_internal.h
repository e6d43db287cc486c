// Internal declarations shared by the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/sa.h"

// A neighbour graph (see graph.cpp): either the normalised
// translation-invariant descriptor, or explicit per-row lists.
struct sa_graph {
  int32_t kind;                 // SA_GRAPH_DISTANCE or SA_GRAPH_CSR
  int64_t T;                    // sequence length
  int64_t W;                    // effective window, min(W, T) (distance graphs; 0 for lists)
  int32_t n_dil;                // kept long-range distances
  int64_t dil[SA_MAX_DILATED];  // ascending, W <= d < T
  int64_t n_edges;              // per (batch, head)
  // explicit lists (kind == SA_GRAPH_CSR), host copies: forward rows i -> keys
  // ascending, reverse rows j -> queries ascending; int32 since T, E < 2^31
  std::vector<int32_t> rp, cols, rrp, rcols;
  // the same four arrays in caller-owned device memory once uploaded
  const int32_t* d_rp = nullptr;
  const int32_t* d_cols = nullptr;
  const int32_t* d_rrp = nullptr;
  const int32_t* d_rcols = nullptr;
};

namespace sa {

enum { DT_F32 = 0, DT_BF16 = 1 };  // same values as sa_dtype
enum { SM_DOT = 0, SM_COORD = 1, SM_UNIFORM = 2 };  // same values as sa_score

// Distance-table padding: larger than any row index, so a padded slot never
// yields a key.  Kernels read the table in groups past n_dil.
constexpr int32_t kUnreachable = 0x7fffffff;

// Everything a kernel needs, passed by value as one kernel argument.  Row
// addresses are base + b*s_b + h*s_h + t*s_t elements (D contiguous).
struct Params {
  int32_t B, H, T, D;
  int32_t W;      // effective window
  int32_t Hkv;    // key/value heads
  int32_t G;      // query heads per key/value head (H / Hkv)
  int32_t n_dil;  // long-range distances
  int32_t dil[SA_MAX_DILATED + 8];  // ascending, padded with kUnreachable
  float scale;       // dot-mode scale
  float scale_log2;  // scale * log2(e)
  int32_t grad_bf16; // dq/dk/dv stored as bf16 (else fp32)
  int32_t rows_per_block_q;  // query-side block height (partials layout)

  const void* q;  int64_t sq_b, sq_h, sq_t;
  const void* k;  int64_t sk_b, sk_h, sk_t;
  const void* v;  int64_t sv_b, sv_h, sv_t;
  void* o;        int64_t so_b, so_h, so_t;
  const void* dout; int64_t sdo_b, sdo_h, sdo_t;
  void* dq;       int64_t sdq_b, sdq_h, sdq_t;
  void* dk;       int64_t sdk_b, sdk_h, sdk_t;
  void* dv;       int64_t sdv_b, sdv_h, sdv_t;

  const float* cq; const float* ck;  // [B, H, T, 3]
  const float* gamma; const float* beta;  // [H]
  float* dcq; float* dck;
  float* dgamma; float* dbeta;

  float* lse;       // [B, H, T]
  float* delta;     // workspace [B, H, T]: Delta (gather backward)
  float* ndelta;    // workspace [B, H, T]: -Delta (band backward; same region)
  float* lse2;      // workspace [B, H, T]: lse * log2(e) (band backward)
  float* partials;  // workspace [B, H, nblk_q, 2]
  const int32_t* pos;  // decode: row of each sequence's new token [B] (NULL: T - 1)
  // explicit neighbour lists (device): row i's keys cols[rp[i] .. rp[i+1]),
  // key j's queries rcols[rrp[j] .. rrp[j+1]), both ascending
  const int32_t* rp; const int32_t* cols;
  const int32_t* rrp; const int32_t* rcols;
};

// Launchers (defined in the .hip files).  Each validates nothing: the C ABI
// layer has already checked every argument.  Return the launch status.
hipError_t launch_gather_fwd(const Params& p, int dtype, int score_mode, hipStream_t s);
hipError_t launch_gather_bwd(const Params& p, int dtype, int score_mode, hipStream_t s);
int gather_rows_per_block(int dtype, int D);

hipError_t launch_band_fwd(const Params& p, hipStream_t s);
hipError_t launch_band_bwd(const Params& p, hipStream_t s);
hipError_t launch_decode(const Params& p, int dtype, int score_mode, hipStream_t s);
// explicit-list graphs: forward, and backward (query pass, key pass over the
// reverse lists, coordinate-parameter reduction)
hipError_t launch_csr_fwd(const Params& p, int dtype, int score_mode, hipStream_t s);
hipError_t launch_csr_bwd(const Params& p, int dtype, int score_mode, hipStream_t s);
// dgamma, dbeta from the per-block partials of a query pass of nblk blocks
hipError_t launch_coord_param_reduce(const Params& p, int nblk, hipStream_t s);
int band_rows_per_block();
// Compute units of the current device (queried once per device).
int device_cu_count();
bool band_supported(int dtype, int D, int score_mode, int64_t W);

}  // namespace sa

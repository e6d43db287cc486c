/*
 * oracle.h -- plain, slow, fp64 CPU oracle for sparse causal attention over a
 * fixed per-query neighbour graph.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path in sparse_causal_attention_amd/.
 *
 * What it follows (pages as cited in every function of oracle.c):
 *  - SpatialLM-Mini news page, section "How tokens choose whom to listen to":
 *    each token's list of admissible positions is fixed in advance (itself,
 *    some nearby predecessors, and positions at distances 1, 2, 4, 8, ...),
 *    never looks ahead, and the weights are normalised over that list only.
 *  - MiniGPT (Part 6), section "A mask is not enough", the sliding-window mask
 *    listing: key j is kept for query i iff j <= i and i - j < w.
 *  - MiniGPT (Part 6), same section, the sentence after the chunked_swa
 *    listing: with w >= T the windowed op equals causal attention exactly.
 *  - SpatialLM-Mini news page, "What to check before adopting it in your
 *    project": the same sparse graph with fixed weights as the comparison
 *    that isolates the coordinates; read here as equal weights over each
 *    row's neighbour list (uniform score mode).
 *
 * Every floating-point result is computed in IEEE double, in the plain order
 * of the definition (ascending key index j), with no blocking, fusion or
 * reordering.  Inputs may be fp64, fp32 or bf16 (raw bits); they are upcast
 * exactly to double on read.
 */
#ifndef SA_ORACLE_H
#define SA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };
enum { ORACLE_SCORE_DOT = 0, ORACLE_SCORE_COORD = 1, ORACLE_SCORE_UNIFORM = 2 };

/* Neighbour set N(i) of row i, ascending, no repeats.  out must hold
 * min(W, T) + n_offs entries.  Returns |N(i)|, or -1 on a bad argument. */
int64_t oracle_row(int64_t T, int64_t W, const int64_t* offs, int32_t n_offs,
                   int64_t i, int64_t* out);

/* CSR of rows [r0, r1): row_ptr has r1 - r0 + 1 entries (relative to 0),
 * cols holds the ascending key indices.  Returns the edge count of the range,
 * or -1 on a bad argument, or -(needed+2) when cols_cap is too small. */
int64_t oracle_graph_csr(int64_t T, int64_t W, const int64_t* offs, int32_t n_offs,
                         int64_t r0, int64_t r1, int64_t* row_ptr, int64_t* cols,
                         int64_t cols_cap);

/* Forward over one (batch, head) slice.  q, k, v are [T, D] row-major with
 * element type `dtype` (q and k used in dot mode only); cq, ck are [T, 3]
 * with element type `cdtype` (coordinate mode only; uniform mode reads v
 * alone).  rows lists the query rows
 * to evaluate (NULL: all T rows in order).  O is [n_rows, D], LSE [n_rows]
 * (natural log).  Returns 0, or -1 on a bad argument. */
int oracle_fwd(int64_t T, int64_t D, int64_t W, const int64_t* offs, int32_t n_offs,
               int score_mode, double scale, int dtype, const void* q, const void* k,
               const void* v, int cdtype, const void* cq, const void* ck, double gamma,
               double beta, const int64_t* rows, int64_t n_rows, double* O, double* LSE);

/* Backward over one (batch, head) slice for upstream gradient dO ([T, D],
 * element type `dtype`).  Recomputes the forward itself.  Writes dQ, dK, dV
 * ([T, D]) in dot mode; dV, dcq, dck ([T, 3]), *dgamma, *dbeta in coordinate
 * mode; dV alone in uniform mode (pass NULL for outputs not wanted).  *l1 receives sum |dS_ij| *
 * (1 + ||c_q,i - c_k,j||^2) over all edges (coordinate mode; a magnitude for
 * reduction tolerances).  Returns 0, or -1 on a bad argument, -2 on OOM. */
int oracle_bwd(int64_t T, int64_t D, int64_t W, const int64_t* offs, int32_t n_offs,
               int score_mode, double scale, int dtype, const void* q, const void* k,
               const void* v, int cdtype, const void* cq, const void* ck, double gamma,
               double beta, const void* dO, double* dQ, double* dK, double* dV,
               double* dcq, double* dck, double* dgamma, double* dbeta, double* l1);

/* The same forward and backward over an explicit graph: row i lists its keys
 * cols[row_ptr[i] .. row_ptr[i+1]) strictly ascending, each 0 <= j <= i, at
 * least one per row (row_ptr has T + 1 entries starting at 0).  All T rows
 * are evaluated.  Returns 0, -1 on a bad argument (including a malformed
 * list), -2 on OOM. */
int oracle_fwd_csr(int64_t T, int64_t D, const int64_t* row_ptr, const int64_t* cols,
                   int score_mode, double scale, int dtype, const void* q, const void* k,
                   const void* v, int cdtype, const void* cq, const void* ck, double gamma,
                   double beta, double* O, double* LSE);
int oracle_bwd_csr(int64_t T, int64_t D, const int64_t* row_ptr, const int64_t* cols,
                   int score_mode, double scale, int dtype, const void* q, const void* k,
                   const void* v, int cdtype, const void* cq, const void* ck, double gamma,
                   double beta, const void* dO, double* dQ, double* dK, double* dV,
                   double* dcq, double* dck, double* dgamma, double* dbeta, double* l1);

/* Dense causal attention (every j <= i), ascending j, dot mode only: the
 * plain definition the windowed op must reproduce exactly when W >= T. */
int oracle_dense_causal(int64_t T, int64_t D, double scale, int dtype, const void* q,
                        const void* k, const void* v, double* O, double* LSE);

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void);

/* Threads for the parallel regions that follow (n >= 1; timing only, the
 * results do not depend on it). */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif

/*
 * sa.h -- C ABI of the MI355X (gfx950) sparse causal attention library.
 *
 * The operation: every query row i of a sequence of length T attends only to
 * a fixed neighbour set
 *
 *     N(i) = { i - delta : delta in {0, ..., W-1} U Dil, i - delta >= 0 }
 *
 * made of its local window (itself and the W-1 rows before it) and a set Dil
 * of long-range distances (typically 1, 2, 4, 8, ...).  The weights are a
 * softmax over N(i) only; no T x T score matrix is formed anywhere.
 *
 * Sources (the pages this library implements):
 *  - SpatialLM-Mini news page, section "How tokens choose whom to listen to":
 *    the admissible list of each token is fixed in advance (itself, nearby
 *    predecessors, positions at distances 1, 2, 4, 8, ...), nothing ahead of
 *    the token is visible, and the weights are distributed within that list;
 *    weights come from learnable 3-D query/key coordinates, nearer pairs
 *    weighing more, adjusted by extra learnable parameters.
 *  - Same page, section "What to check before adopting it in your project":
 *    the same graph with a standard dot product is the comparison to run,
 *    hence the score-mode switch.
 *  - MiniGPT (Part 6), section "A mask is not enough": the sliding-window
 *    predicate (key j kept for query i iff j <= i and i - j < w), the
 *    requirement that the O(T*W) cost come from never forming the T x T
 *    matrix, and exact equality with causal attention when w >= T.
 *  - "Longer Attention Span: Increasing Transformer Context Length with
 *    Sparse Graph Processing Techniques" (arXiv 2502.01659), abstract: tokens
 *    are graph nodes, the mask gives the edges, and the work done is
 *    proportional to the edges.
 *
 * Conventions shared by every entry point:
 *  - All sizes and strides are counts of elements (not bytes), int64.
 *  - Tensors q, k, v, o, dout, dq, dk, dv are [B, H, T, D] with arbitrary
 *    (b, h, t) strides and the D elements of a row contiguous.  Every row must
 *    start on a 16-byte boundary (base pointer and strides times element size
 *    divisible by 16).
 *  - lse is [B, H, T] fp32, contiguous: lse[(b*H + h)*T + t].
 *  - Coordinates c_q, c_k (and their gradients) are [B, H, T, 3] fp32,
 *    contiguous.  gamma, beta (and dgamma, dbeta) are [H] fp32.
 *  - Every pointer passed to sa_fwd / sa_bwd is a device pointer owned by the
 *    caller.  The library never allocates or frees device memory; the device
 *    regions it refers to beyond a call are the buffer an explicit-list graph
 *    was uploaded into (sa_graph_upload), which stays the caller's, and its
 *    own static scratch array for sa_bwd_noalloc (SA_NOALLOC_SCRATCH_BYTES per
 *    GPU, part of the library's device code, held until the process ends).
 *  - Calls are asynchronous on the given stream (a hipStream_t; NULL is the
 *    null stream).  SA_OK means the work was validated and enqueued.  sa_fwd,
 *    sa_bwd and sa_decode only launch kernels (no allocation, memset or
 *    synchronisation), so they can be captured in a HIP graph; upload an
 *    explicit-list graph (sa_graph_upload) before capturing.
 *  - All validation happens before any HIP call, and nothing is written when
 *    validation fails.  No entry point aborts, throws or prints.
 *  - The library does not touch the GPU when it is loaded; sa_build_graph*,
 *    sa_graph_* (except sa_graph_upload) and the validation paths run on hosts
 *    without a GPU.
 */
#ifndef SPARSE_CAUSAL_ATTENTION_SA_H
#define SPARSE_CAUSAL_ATTENTION_SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,    /* null pointer, size < 1, negative offset, bad alignment, ... */
  SA_ERR_UNSUPPORTED = 2,    /* a valid request the library does not implement (e.g. D = 48) */
  SA_ERR_SHAPE_MISMATCH = 3, /* graph T differs from the descriptor's T */
  SA_ERR_WORKSPACE = 4,      /* backward workspace missing or too small */
  SA_ERR_HIP = 5             /* a kernel launch reported an error */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* Score of edge (i, j):
 *  SA_SCORE_DOT:     s_ij = scale * <q_i, k_j>
 *  SA_SCORE_COORD:   s_ij = -gamma_h * ||c_q,i - c_k,j||^2 + beta_h
 *  SA_SCORE_UNIFORM: s_ij = 0, i.e. every neighbour of row i has weight
 *                    1 / |N(i)| (fixed weights, no score parameters)
 * (SpatialLM-Mini news page, "How tokens choose whom to listen to", and the
 * comparisons on the same graph with a dot product or fixed weights asked for
 * in "What to check before adopting it"). */
typedef enum { SA_SCORE_DOT = 0, SA_SCORE_COORD = 1, SA_SCORE_UNIFORM = 2 } sa_score;

/* Kernel family.  AUTO picks the LDS/MFMA band kernels for the window when
 * they apply (bf16, dot score, D = 64, W >= 16, a distance graph; for
 * sa_bwd also: each (batch, head) slice of q, k, v and dout spans fewer
 * than 2^31 bytes, i.e. (T - 1) * row stride + D elements, and each of their
 * strides is below 2^31 elements) and the gather
 * kernels otherwise (the indexed ones for an explicit-list graph).  GATHER
 * forces the gather kernels for every edge; BAND requests the band kernels
 * and fails with SA_ERR_UNSUPPORTED where they do not apply. */
typedef enum { SA_ALGO_AUTO = 0, SA_ALGO_GATHER = 1, SA_ALGO_BAND = 2 } sa_algo;

#define SA_MAX_DILATED 64 /* distinct long-range distances kept by a graph */

typedef struct sa_graph sa_graph; /* opaque, host memory; its edges are fixed once built */

/* The two graph representations. */
typedef enum {
  SA_GRAPH_DISTANCE = 0, /* window + long-range distances (sa_build_graph) */
  SA_GRAPH_CSR = 1       /* explicit per-row key lists (sa_build_graph_csr) */
} sa_graph_type;
typedef void* sa_stream;          /* hipStream_t */

/* ------------------------------------------------------------------ graph */

/* Builds the neighbour graph of a length-T sequence with window `window`
 * (W >= 1; W >= T means every j <= i, i.e. dense causal attention) and
 * long-range distances `offsets[0..n_offsets)` (SpatialLM-Mini news page,
 * "How tokens choose whom to listen to"; MiniGPT Part 6 window predicate).
 * Offsets may be unsorted and repeated; offsets below W (already inside the
 * window) and offsets >= T (never a valid key) are dropped, the rest sorted
 * and deduplicated, so each edge exists once.  A negative offset would look
 * ahead and is SA_ERR_INVALID_ARG.  More than SA_MAX_DILATED distinct kept
 * offsets is SA_ERR_UNSUPPORTED; T >= 2^31 is SA_ERR_UNSUPPORTED.  On success
 * *out receives a handle the caller releases with sa_graph_free.  Integer
 * only, host only, bit-exact. */
sa_status sa_build_graph(int64_t T, int64_t window, const int64_t* offsets, int32_t n_offsets,
                         sa_graph** out);

/* Builds a graph from explicit per-row key lists (compressed sparse rows, host
 * memory, read during the call only): row i attends to the keys
 * cols[row_ptr[i] .. row_ptr[i+1]), which must be strictly ascending, within
 * 0 .. i (causal), and at least one per row; row_ptr has T + 1 entries with
 * row_ptr[0] = 0.  This is the general graph view of "Longer Attention Span:
 * Increasing Transformer Context Length with Sparse Graph Processing
 * Techniques" (abstract: tokens as nodes, the attention mask as the edges,
 * work proportional to the edges); the SpatialLM-Mini graph is the special
 * case sa_build_graph describes without lists.  A list breaking a rule is
 * SA_ERR_INVALID_ARG; T or E = row_ptr[T] of 2^31 or more is
 * SA_ERR_UNSUPPORTED.  The builder also forms the reverse lists the backward
 * walks (sa_graph_rows_reverse).  The same graph serves every (batch, head).
 * Before sa_fwd, sa_bwd or sa_decode can use it, its lists must be uploaded
 * (sa_graph_upload).  Integer only, bit-exact. */
sa_status sa_build_graph_csr(int64_t T, const int64_t* row_ptr, const int64_t* cols, sa_graph** out);

/* *kind receives the graph's sa_graph_type (the window-and-distances graph of
 * SpatialLM-Mini's "How tokens choose whom to listen to", or the general
 * mask-as-edges lists of arXiv 2502.01659's abstract). */
sa_status sa_graph_kind(const sa_graph* g, int32_t* kind);

/* Library plumbing (no source passage): device bytes an explicit-list
 * graph's lists occupy once uploaded:
 * 2 * (align256(4 (T + 1)) + align256(4 E)) -- forward and reverse lists, int32.
 * 0 for a distance graph. */
sa_status sa_graph_device_bytes(const sa_graph* g, size_t* bytes);

/* Copies an explicit-list graph's forward and reverse lists into device_buf
 * (device memory the caller owns: at least sa_graph_device_bytes bytes,
 * 256-byte aligned, on the device the graph will be used on), on `stream`, and
 * returns when the copy has completed.  From then on sa_fwd, sa_bwd and
 * sa_decode read the lists there: the caller keeps the buffer allocated and
 * unmodified while the graph is used and frees it after the last call that
 * uses it has finished (and after sa_graph_free).  A graph is uploaded once:
 * its device lists are then fixed for its lifetime (the handle stays
 * immutable and shareable across streams), and a second upload is
 * SA_ERR_INVALID_ARG with nothing copied; to use the same lists on another
 * device, build a second graph.  A distance graph has nothing to upload: the
 * call does nothing and returns SA_OK.  Bad buffer or size:
 * SA_ERR_INVALID_ARG; a failed copy: SA_ERR_HIP (the graph stays
 * un-uploaded).  The fixed list is the SpatialLM-Mini news page's ("How
 * tokens choose whom to listen to": each token's admissible list is set in
 * advance); the upload itself is library plumbing with no source passage. */
sa_status sa_graph_upload(sa_graph* g, void* device_buf, size_t bytes, sa_stream stream);

/* Normalised descriptor (the window and distances of SpatialLM-Mini's "How
 * tokens choose whom to listen to" and MiniGPT Part 6's window predicate,
 * with the set reading: each edge once): T, the effective window min(W, T), the kept
 * long-range distances ascending (dil may be NULL; else SA_MAX_DILATED
 * entries of room) and the edge count per (batch, head)
 *   E = W'(W'+1)/2 + W'(T-W') + sum_{d in Dil} (T - d),  W' = min(W, T).
 * For an explicit-list graph: T, window 0, no distances and E = row_ptr[T].
 * Any output pointer may be NULL. */
sa_status sa_graph_info(const sa_graph* g, int64_t* T, int64_t* window, int32_t* n_dil,
                        int64_t* dil, int64_t* n_edges);

/* The neighbour lists N(i) themselves (the per-token list of SpatialLM-Mini's
 * "How tokens choose whom to listen to"; the mask-as-edges view of arXiv
 * 2502.01659's abstract), exported for inspection and testing.
 * CSR rows [row_begin, row_end) of the graph: row_ptr receives
 * row_end - row_begin + 1 offsets starting at 0, cols the key indices of each
 * row in ascending order.  cols_cap is the room in cols; too little room is
 * SA_ERR_INVALID_ARG with row_ptr filled (so row_ptr[last] is the size
 * needed) and cols untouched. */
sa_status sa_graph_rows(const sa_graph* g, int64_t row_begin, int64_t row_end, int64_t* row_ptr,
                        int64_t* cols, int64_t cols_cap);

/* The reverse graph in the same format: row j lists, ascending, the queries
 * i with j in N(i) (i = j + delta, delta in {0..W-1} U Dil, i < T) -- the
 * edges the key-side backward sums over (chain rule; no passage of the pages
 * describes a backward). */
sa_status sa_graph_rows_reverse(const sa_graph* g, int64_t row_begin, int64_t row_end,
                                int64_t* row_ptr, int64_t* cols, int64_t cols_cap);

/* Releases a handle (NULL is a no-op).  The caller's upload buffer, if any,
 * is not touched.  Library plumbing: no source passage. */
void sa_graph_free(sa_graph* g);

/* ------------------------------------------------------------------ attention */

typedef struct {
  int64_t B, H, T, D;  /* D in {16, 32, 64, 128} */
  int32_t dtype;       /* sa_dtype of q, k, v, o, dout */
  int32_t grad_dtype;  /* sa_dtype of dq, dk, dv (fp32 recommended) */
  int32_t score;       /* sa_score */
  int32_t algo;        /* sa_algo */
  float scale;         /* dot mode; <= 0 selects 1/sqrt(D).  Unused in coordinate mode. */
  int64_t stride_q[3], stride_k[3], stride_v[3], stride_o[3], stride_do[3]; /* (b, h, t) */
  int64_t stride_dq[3], stride_dk[3], stride_dv[3];                          /* (b, h, t) */
  int64_t H_kv;        /* key/value heads; 0 selects H.  H must be a multiple of H_kv: query
                          head h reads key/value head h / (H / H_kv), and k, v, dk, dv (and
                          the decode caches) are [B, H_kv, T, D] with strides over (b, h_kv,
                          t) -- grouped-query attention (MiniGPT Part 6, opening and closing
                          paragraphs: the series' grouped key/value heads, which shrink the
                          key/value cache).  Coordinate mode needs H_kv = H (per-head
                          coordinates). */
} sa_attn_desc;

/* Forward (SpatialLM-Mini news page, "How tokens choose whom to listen to";
 * MiniGPT Part 6, "A mask is not enough"): for every (b, h, i)
 *   m_i = max_{j in N(i)} s_ij,  l_i = sum_{j in N(i)} exp(s_ij - m_i),
 *   o_i = sum_{j in N(i)} exp(s_ij - m_i) v_j / l_i,   lse_i = m_i + ln l_i.
 * Dot mode reads q, k, v (cq, ck, gamma, beta ignored, may be NULL);
 * coordinate mode reads cq, ck, gamma, beta, v (q, k ignored); uniform mode
 * reads v alone (o_i is the mean of v over N(i), lse_i = ln |N(i)|).  Writes o in
 * `dtype` (bf16 rounded to nearest even) and lse in fp32 (natural log).
 * Arithmetic is fp32 with fp32 accumulation; bf16 MFMA products for the band.
 * With an explicit-list graph N(i) is row i's list, and a graph that has not
 * been uploaded is SA_ERR_INVALID_ARG (likewise for sa_bwd and sa_decode).
 * Size limits (likewise for sa_bwd, sa_bwd_workspace_size): B, H or B * H
 * above 2^24, or B * H * ceil(T / 8) of about 2^31 or more (workgroup counts
 * are 32-bit), is SA_ERR_UNSUPPORTED. */
sa_status sa_fwd(const sa_graph* g, const sa_attn_desc* desc, const void* q, const void* k,
                 const void* v, const float* cq, const float* ck, const float* gamma,
                 const float* beta, void* o, float* lse, sa_stream stream);

/* Bytes of device workspace sa_bwd needs for this graph and descriptor
 * (per-row Delta_i and lse_i * log2(e), plus per-block partial sums of the
 * coordinate-mode parameter gradients): 2 * align256(4 B H T) +
 * align256(8 B H ceil(T / rows_per_block)).  The quantities are those of the
 * chain rule through sa_fwd; the pages describe no backward, so no passage
 * defines them.  Same validation as sa_bwd's shape checks. */
sa_status sa_bwd_workspace_size(const sa_graph* g, const sa_attn_desc* desc, size_t* bytes);

/* Backward of L = sum <dout, o> through sa_fwd, given the forward's o and
 * lse.  The pages train these models end to end (SpatialLM-Mini news page,
 * "What the comparison on 8 GB showed": training throughput; MiniGPT Part 6,
 * "Memory against context length": forward plus backward memory) but print no
 * backward formula: what follows is the chain rule through the forward's
 * definition above, written out.
 *       dP_ij = <dout_i, v_j>,  Delta_i = <dout_i, o_i>,
 *       dS_ij = P_ij (dP_ij - Delta_i),  P_ij = exp(s_ij - lse_i),
 *   dot mode:   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
 *   (with H_kv < H, dk and dv of a key/value head also sum over its query heads)
 *   both modes: dv_j = sum_i P_ij dout_i,
 *   coordinate: dcq_i = -2 gamma sum_j dS_ij (c_q,i - c_k,j),
 *               dck_j =  2 gamma sum_i dS_ij (c_q,i - c_k,j),
 *               dgamma_h = -sum dS_ij ||c_q,i - c_k,j||^2,  dbeta_h = sum dS_ij.
 * Every output element is written (not accumulated into).  Deterministic: no
 * atomics, fixed summation order, bitwise identical across runs.  Dot mode
 * writes dq, dk, dv (dcq, dck, dgamma, dbeta may be NULL); coordinate mode
 * writes dv, dcq, dck, dgamma, dbeta (dq, dk may be NULL); uniform mode
 * writes dv alone (dv_j = sum over i with j in N(i) of dout_i / |N(i)|).  The workspace
 * (at least sa_bwd_workspace_size bytes, 256-byte aligned) is scratch owned
 * by the caller and must not be shared by concurrent calls. */
sa_status sa_bwd(const sa_graph* g, const sa_attn_desc* desc, const void* q, const void* k,
                 const void* v, const float* cq, const float* ck, const float* gamma,
                 const float* beta, const void* o, const float* lse, const void* dout, void* dq,
                 void* dk, void* dv, float* dcq, float* dck, float* dgamma, float* dbeta,
                 void* workspace, size_t workspace_bytes, sa_stream stream);

/* Bytes of the built-in device scratch sa_bwd_noalloc uses in place of a
 * workspace (16 MiB: enough for B * H * T up to about two million rows). */
#define SA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* sa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results (bitwise: the same
 * kernels), validation and status rules as sa_bwd, except that the workspace
 * is a static device array of SA_NOALLOC_SCRATCH_BYTES inside the library:
 * each GPU the library runs on holds one copy until the process ends, found on
 * the first call on that device.  A shape whose workspace
 * (sa_bwd_workspace_size) exceeds SA_NOALLOC_SCRATCH_BYTES is
 * SA_ERR_WORKSPACE; use sa_bwd with a workspace of your own instead.  The
 * call allocates nothing and clears nothing (no part of the scratch needs to
 * start at zero).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (on different streams, or from several threads) race and
 * corrupt each other's gradients -- order them on one stream.  A failed
 * lookup of the scratch is SA_ERR_HIP. */
sa_status sa_bwd_noalloc(const sa_graph* g, const sa_attn_desc* desc, const void* q, const void* k,
                         const void* v, const float* cq, const float* ck, const float* gamma,
                         const float* beta, const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, float* dcq, float* dck, float* dgamma,
                         float* dbeta, sa_stream stream);

/* Decode step with a key/value cache: for every (b, h), the one new token at
 * row t_b = positions[b] of the cache attends to its neighbour list N(t_b)
 * (the window t_b .. t_b - W + 1 and t_b - d for the long-range distances
 * d <= t_b; or row t_b of explicit lists), with the forward's softmax and
 * score; O(W + log T) row reads per
 * token, independent of how long the cache is (SpatialLM-Mini news page,
 * "What to check before adopting it in your project": the prototype had no
 * KV cache).  desc->T is the cache capacity and must equal the graph's T;
 * k and v (dot mode), v (uniform), or ck and v (coordinate) are the caches in
 * [B, H, T, D] (ck: [B, H, T, 3] fp32) with rows 0 .. t_b filled.  The new
 * token's query is q [B, H, D] (strides desc->stride_q[0..1]; stride_q[2]
 * unused) or cq [B, H, 3] fp32 contiguous; o is [B, H, D] (stride_o[0..1])
 * in `dtype`, lse [B, H] fp32 (natural log).  positions is a device array of
 * B int32 (NULL: every sequence at row T - 1); a position outside [0, T)
 * cannot be checked on the host and yields NaN in that sequence's o and lse.
 * Same validation and status rules as sa_fwd, except the size limit: B, H or
 * B * H of 2^31 or more is SA_ERR_UNSUPPORTED (one workgroup per (b, h)). */
sa_status sa_decode(const sa_graph* g, const sa_attn_desc* desc, const int32_t* positions,
                    const void* q, const void* k, const void* v, const float* cq, const float* ck,
                    const float* gamma, const float* beta, void* o, float* lse, sa_stream stream);

/* Names the kernels sa_fwd (which = 0) or sa_bwd (which = 1) would launch for
 * this graph and descriptor, as a NUL-terminated string in buf[0..cap).
 * Validates like the call itself.  Library introspection: no source
 * passage. */
sa_status sa_describe_plan(const sa_graph* g, const sa_attn_desc* desc, int32_t which, char* buf,
                           size_t cap);

/* Static description of a status code (library plumbing: no source passage). */
const char* sa_status_str(sa_status s);

#ifdef __cplusplus
}
#endif
#endif

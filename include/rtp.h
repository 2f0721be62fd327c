/*
 * rtp.h -- C ABI of librtp.so: one sparse-attention decode step of RTPurbo's
 * head-wise sparse attention on AMD Instinct MI355X (gfx950).
 *
 * Method ("Full Attention Strikes Back", RTPurbo, arXiv 2605.16928, section 3.2):
 * query heads are split into retrieval heads and local heads.  At decode time a
 * retrieval head h scores every cached token n with a rank-16 indexer on the
 * pre-RoPE features (eq. (4)), keeps the dynamic Top-P set of those scores and
 * runs softmax attention with the post-RoPE query and keys over that set only
 * (eq. (5)).  A local head runs the same attention over a sliding window plus
 * attention sinks.  The Top-P set is found without sorting, through a 256-bin
 * histogram per head (DeepRead summary of RTPurbo, hardware-optimised kernels).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - rtp_bf16 is the raw bit pattern of a bfloat16 value.
 *  - Every array pointer is a DEVICE pointer owned by the caller, except
 *    rtp_layer.head_mode, which lives in host memory.  The library never
 *    allocates or frees memory and keeps no state between calls.
 *  - Device pointers must be 16-byte aligned (the kernels use 16-byte vector
 *    accesses); a misaligned one is RTP_ERR_ARG.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on that stream and returns; results are
 *    ready once the stream has reached that point.
 *  - Arguments are validated before anything is enqueued; on error nothing is
 *    launched and a negative RTP_ERR_* code is returned.  RTP_ERR_HIP reports a
 *    failed launch (the HIP error is left for hipGetLastError()).
 *  - Non-finite inputs are undefined behaviour.
 *  - rtp_layer's three tuning fields (scan_tile, swa_chunk, pf_qch) change how
 *    the work is split, not what is computed (fp32 results may change in
 *    their last bits through the order of split-K merges); 0 picks the
 *    library's choice.  The workspace size depends on them.
 *  - Row-major layouts; "cap" rows of the caches are strided by Ncap.
 *  - "[B, Hkv, Ncap, D]" for the K/V caches (k, v, k_cache, v_cache) stands for
 *    the layout rtp_layer.local_ring selects; it is exactly that shape when
 *    local_ring is 0.  With ring groups present, calls that need more than the
 *    window of the newest position -- rtp_dense_attn, rtp_prefill_attn and
 *    nq > 1 -- return RTP_ERR_UNSUPPORTED.  Pre-RoPE key inputs (k_pre) and the
 *    indexer keys keep their stated shapes.
 *  - Retrieval heads are numbered r = 0..Hr-1 in ascending q-head order; the
 *    q head h belongs to KV group h / (Hq / Hkv).
 *  - The query of a decode step sits at position m = N - 1.  With nq > 1 the
 *    nq queries sit at positions m_i = N - nq + i and each is causal (sees
 *    positions 0..m_i).
 *
 * Numerics (readings of the pages, see the oracle for the written-out rules)
 *  - RoPE (eq. (1)): theta_i = rope_theta^(-2(i-1)/D), i = 1..D/2, adjacent
 *    channel pairs, angles m*theta_i formed in fp64.
 *  - Indexer (eq. (4)): q_idx = bf16(q_pre . W_q) and K_idx = bf16(k_pre . W_k),
 *    each the exact dot product rounded once to nearest-even; the score
 *    s_n = fp32(q_idx . K_idx[n]) is the exact dot product rounded once.
 *  - Top-P (eq. (5)): over softmax(s), mass p * Z (Z the total, the product
 *    rounded once to double).  Bins are 1/8 logit unit wide on edges
 *    k/8, bin 0 = cell of the maximum score, deeper cells clamped into bin 255.
 *    Bins above the boundary bin b* are taken whole; bin b* is filled in
 *    ascending position while the mass before a token is below p * Z.
 *    p >= 1 selects every position.
 *  - Attention accumulates in fp32 from bf16 K/V; outputs are fp32.
 */
#ifndef RTP_H
#define RTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t rtp_bf16;

enum rtp_status {
  RTP_OK = 0,
  RTP_ERR_ARG = -1,           /* null pointer, p <= 0 or NaN, window < 1, bad head_mode entry, n0/n1 out of range */
  RTP_ERR_SHAPE = -2,         /* D != 128, R != 16, Hq % Hkv != 0, nq < 1, N < nq, N > Ncap, N >= 2^31, Hq > 256 */
  RTP_ERR_WS_TOO_SMALL = -3,  /* ws_bytes < rtp_workspace_bytes(layer) */
  RTP_ERR_UNSUPPORTED = -4,   /* a valid request the library does not implement */
  RTP_ERR_HIP = -5            /* a HIP launch failed */
};

/* One attention layer of the step. */
typedef struct rtp_layer {
  int32_t B;                  /* batch (sequences) */
  int32_t Hq;                 /* query heads, <= 256 */
  int32_t Hkv;                /* KV heads (groups); Hq % Hkv == 0 */
  int32_t D;                  /* head dim, must be 128 */
  int32_t R;                  /* indexer rank, must be 16 */
  int32_t nq;                 /* queries per (b, head): 1 = decode, > 1 = chunked prefill */
  int64_t N;                  /* cached positions, current token(s) included; 1 <= N < 2^31 */
  int64_t Ncap;               /* row capacity of every cache (its row stride), >= N */
  const int8_t *head_mode;    /* HOST array [Hq]: 1 = retrieval head, 0 = local head */
  double p;                   /* Top-P mass, > 0; >= 1 keeps every position.  Used as given: the
                                 mass a boundary-bin token is compared with is p * Z rounded once
                                 to double (Z the total softmax mass of the query's scores) */
  int32_t window;             /* local heads: window W >= 1 (positions m-W+1..m) */
  int32_t n_sink;             /* local heads: sink positions 0..n_sink-1, >= 0 */
  double rope_theta;          /* RoPE base of eq. (1), > 0 */
  int32_t idx_group;          /* retrieval q heads sharing one indexer-key head: 0 or 1 = one per
                                 retrieval head (eq. (4) writes W_k per head), Hq/Hkv = one per KV
                                 group (then retrieval heads come in whole groups).  The indexer-key
                                 heads Hi = Hr / idx_group are numbered in retrieval-head order:
                                 k_idx is [B,Hi,Ncap,R], w_k is [Hi,D,R]; w_q stays [Hr,D,R] */
  int64_t top_k;              /* 0 = Top-P with mass p (FASB eq. (5)).  > 0 = fixed top-k, the
                                 budget-by-count counterpart FASB section 2.3 / Table 1 compares
                                 with Top-P: the first top_k positions in the order (histogram bin
                                 ascending, position ascending), every position when top_k >= m+1;
                                 p is then ignored.  < 0 is RTP_ERR_ARG. */
  int32_t local_ring;         /* K/V cache layout.  0: k, v are [B, Hkv, Ncap, D].  1: a KV group
                                 whose q heads are all local heads keeps only the rows its heads
                                 can attend to (FASB abstract and section 3.2: only retrieval
                                 heads retain the full cache; local heads see a window plus
                                 sinks): n_sink + window rows, position n in row n for n < n_sink
                                 and in row n_sink + (n - n_sink) mod window otherwise.  Per
                                 sequence the groups follow in order, a full group taking Ncap
                                 rows and a ring group n_sink + window rows; rtp_kv_rows gives
                                 the rows per sequence, so k, v are [B, rtp_kv_rows(layer), D].
                                 Other values, or 1 with n_sink + window >= 2^31, are
                                 RTP_ERR_ARG. */
  int32_t scan_tile;          /* 0 = automatic; else positions per indexer scan tile: 1024, 2048, 4096
                                 or 8192 (other values are RTP_ERR_ARG) */
  int32_t swa_chunk;          /* 0 = automatic; else cache rows per window workgroup, a multiple of 64
                                 (other values are RTP_ERR_ARG) */
  int32_t pf_qch;             /* 0 = automatic; else queries per chunked-prefill selection chunk (nq > 1),
                                 a multiple of 16 (other values are RTP_ERR_ARG) */
} rtp_layer;

/* Number of retrieval heads Hr implied by layer->head_mode (or a negative status). */
int32_t rtp_num_retrieval(const rtp_layer *layer);

/* Rows per sequence of the K/V caches in the layout of layer->local_ring:
 * Hkv * Ncap without ring groups, else (full groups) * Ncap + (ring groups) *
 * (n_sink + window).  A negative status on an invalid layer. */
int64_t rtp_kv_rows(const rtp_layer *layer);

/* Workspace bytes the calls taking `ws` need for this layer (0 on invalid layer).
 * The same workspace serves every call below. */
size_t rtp_workspace_bytes(const rtp_layer *layer);

/* Prepare a workspace for first use (enqueues a fill kernel on `stream`).  A
 * workspace must be prepared once before its first use; every call leaves it
 * ready for the next call on a layer of the same shape (B, Hq, Hkv, nq and
 * head_mode; N, p, top_k, window and the other fields may change between
 * calls, so a growing decode cache keeps one workspace).  Before a call on a
 * layer of another shape, prepare it again.  Calls that share one workspace
 * must not overlap. */
int rtp_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *rtp_status_str(int status);

/* ---------------------------------------------------------------- cache writers */

/* Post-RoPE key cache rows (FASB eq. (1)): k_out[b,g,n,:] = bf16(R(n) k_pre[b,g,n,:])
 * for n in [n0, n1), every b and KV group g.  k_pre, k_out: [B, Hkv, Ncap, D] bf16.
 * Requires 0 <= n0 <= n1 <= Ncap.  k_out may alias k_pre (in-place). */
int rtp_rope_keys(const rtp_layer *layer, const rtp_bf16 *k_pre, rtp_bf16 *k_out,
                  int64_t n0, int64_t n1, void *stream);

/* Indexer-key cache rows (FASB eq. (4), key side): k_idx[b,i,n,:] =
 * bf16(k_pre[b, g(i), n, :] . W_k[i]) for n in [n0, n1), every b and indexer-key
 * head i (g(i) = KV group of the retrieval heads it serves; i = r with
 * idx_group 1).
 * k_pre: [B, Hkv, Ncap, D] bf16; w_k: [Hi, D, R] bf16; k_idx: [B, Hi, Ncap, R] bf16. */
int rtp_index_keys(const rtp_layer *layer, const rtp_bf16 *k_pre, const rtp_bf16 *w_k,
                   rtp_bf16 *k_idx, int64_t n0, int64_t n1, void *stream);

/* Append new positions to every cache in one launch (FASB eq. (1) and eq. (4),
 * key side): for n = n0 + t, t in [0, n_new), every b and KV group g,
 *   k_cache[b,g,n,:] = bf16(R(n) k_new[b,g,t,:]),  v_cache[b,g,n,:] = v_new[b,g,t,:],
 * and for every indexer-key head i (KV group g(i)),
 *   k_idx[b,i,n,:] = bf16(k_new[b,g(i),t,:] . W_k[i]),
 * bit for bit what rtp_rope_keys and rtp_index_keys write for those rows.
 * k_new, v_new: [B, Hkv, n_new, D] bf16 (pre-RoPE keys and values of the new
 * tokens; must not overlap the caches); w_k: [Hi, D, R]; k_cache, v_cache:
 * [B, Hkv, Ncap, D]; k_idx: [B, Hi, Ncap, R].  Rows outside [n0, n0 + n_new)
 * are not touched.  Requires 0 <= n0, n0 + n_new <= Ncap (else RTP_ERR_ARG);
 * w_k and k_idx may be null when the layer has no retrieval head.  In a ring
 * group (local_ring) position n goes to its ring row, and of new positions
 * that share a row only the last is written. */
int rtp_append_kv(const rtp_layer *layer, const rtp_bf16 *k_new, const rtp_bf16 *v_new, const rtp_bf16 *w_k,
                  rtp_bf16 *k_cache, rtp_bf16 *v_cache, rtp_bf16 *k_idx, int64_t n0, int64_t n_new,
                  void *stream);

/* ---------------------------------------------------------------- decode-path calls */

/* Indexer scores (FASB eq. (4)): logits[b,r,i,n] = s_n for every retrieval head r,
 * query i and n <= m_i; entries with n > m_i are set to -inf.
 * q_pre: [B, Hq, nq, D] bf16 (pre-RoPE queries); w_q: [Hr, D, R] bf16;
 * k_idx: [B, Hi, Ncap, R] bf16; logits: [B, Hr, nq, N] fp32. */
int rtp_index_score(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q,
                    const rtp_bf16 *k_idx, float *logits, void *stream);

/* Histogram Top-P over given scores (FASB eq. (5) right; DeepRead hardware notes).
 * logits: [B, Hr, nq, N] fp32 (as written by rtp_index_score; entries n > m_i ignored).
 * idx: [B, Hr, nq, cap] int32 receives the selected positions of each query as
 * two ascending runs: first every position above the boundary bin, then the
 * positions taken from the boundary bin.  Only the first min(count, cap) entries
 * are written.  count: [B, Hr, nq] int32 receives the true |S| (check <= cap). */
int rtp_topp_select(const rtp_layer *layer, const float *logits, int32_t *idx, int32_t *count,
                    int64_t cap, void *ws, size_t ws_bytes, void *stream);

/* Sparse attention of the retrieval heads over given sets (FASB eq. (5) left):
 * out[b,h,i,:] = sum_{n in S} softmax(q_rot . K[n] / sqrt(D)) V[n] with
 * q_rot = R(m_i) q_pre[b,h,i], S = idx[b,r(h),i,0:min(count,cap)] (duplicates count
 * twice; an empty set gives zeros).  q_pre: [B,Hq,nq,D] bf16; k, v: [B,Hkv,Ncap,D]
 * bf16 (post-RoPE keys, values); out: [B,Hq,nq,D] fp32 -- only retrieval-head rows
 * are written.  Positions must lie in [0, N). */
int rtp_sparse_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k,
                    const rtp_bf16 *v, const int32_t *idx, const int32_t *count, int64_t cap,
                    float *out, void *ws, size_t ws_bytes, void *stream);

/* Sliding-window attention with sinks of the local heads (FASB section 3.2):
 * the same attention over positions max(0,m_i-W+1)..m_i and 0..n_sink-1.
 * Layouts as rtp_sparse_attn; only local-head rows of out are written. */
int rtp_swa_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k,
                 const rtp_bf16 *v, float *out, void *ws, size_t ws_bytes, void *stream);

/* Dense attention, the comparator of the sparse step: every q head (retrieval
 * and local alike) attends over every cached position 0..m_i with the same
 * RoPE'd query, softmax(q_rot . K[n] / sqrt(D)) V[n] (eq. (5) with the full
 * set, i.e. plain causal decode attention as in FASB section 2).  The pages
 * measure their kernels against a dense FlashAttention-2 decode (DeepRead
 * summary, "Key Results"); this call is that baseline built the same way as
 * the rest of this library (GQA: one K/V row read serves the group's heads,
 * split-K over the cache).  With nq > 1 it runs the matrix-core kernel of
 * rtp_prefill_attn with every head dense.  Layouts as rtp_swa_attn; writes
 * every row of out.  The workspace of rtp_workspace_bytes(layer) covers this
 * call. */
int rtp_dense_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k,
                   const rtp_bf16 *v, float *out, void *ws, size_t ws_bytes, void *stream);

/* Prefill attention (FASB section 3.2: in prefill the retrieval heads keep the
 * full KV cache and the local heads attend to a sliding window plus sinks):
 * for each of the nq causal queries at m_i = N - nq + i, retrieval heads attend
 * over every position 0..m_i and local heads over max(0, m_i-W+1)..m_i plus
 * 0..n_sink-1; all_dense != 0 makes every head attend over 0..m_i (the dense
 * prefill the DeepRead summary's "Key Results" compare against).  Matrix-core
 * kernel: the rotated query and the softmax weights are each carried as two
 * bf16 halves, so both products keep fp32-level precision.
 * q_pre: [B, Hq, nq, D] bf16 (pre-RoPE); k (post-RoPE), v: [B, Hkv, Ncap, D]
 * bf16; out: [B, Hq, nq, D] fp32, every row written.  No workspace. */
int rtp_prefill_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k,
                     const rtp_bf16 *v, float *out, int32_t all_dense, void *stream);

/* One whole step (FASB eq. (4)-(5) and section 3.2): indexer scan, histogram
 * Top-P, sparse attention for retrieval heads and SWA for local heads; writes
 * every row of out [B,Hq,nq,D] fp32.  Equals rtp_index_score + rtp_topp_select +
 * rtp_sparse_attn + rtp_swa_attn without materialising the scores.
 * idx_opt/count_opt (may be NULL) receive the selected sets as rtp_topp_select
 * writes them.  phase_event (may be NULL) is a hipEvent_t recorded on `stream`
 * between the scan phase and the selection/attention phase (nq == 1), or after
 * the query preparation (nq > 1), for profiling.
 * nq > 1 (chunked prefill, causal: query i at position N-nq+i sees 0..N-nq+i)
 * runs the indexer as a matrix-core GEMM, Top-P per query and attention over
 * each query's set, in chunks of queries whose positions fit the workspace.
 * Its scores are the exact products of the bf16 inputs summed by the matrix
 * core (order of the 16-term fp32 sum not specified), so a position within one
 * rounding of a bin edge may fall on either side. */
int rtp_decode_step(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q,
                    const rtp_bf16 *k_idx, const rtp_bf16 *k, const rtp_bf16 *v, float *out,
                    int32_t *idx_opt, int32_t *count_opt, int64_t cap,
                    void *ws, size_t ws_bytes, void *phase_event, void *stream);

/* The same step as rtp_decode_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): its workspace is a static device array of
 * RTP_STATIC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds
 * from the library's load to the process's end.  Nothing is allocated or
 * freed by this call (no hipMalloc, hipFree or allocating library routine);
 * the first call on a device looks up the array's address on that device.
 * Layers whose rtp_workspace_bytes exceeds the array are RTP_ERR_WS_TOO_SMALL.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and give undefined results.  The
 * array keeps the last call's contents; its persistent part is cleared (a
 * fill kernel on `stream`) on the first call on a GPU and when a call's layer
 * layout (B, Hq, Hkv, nq, head_mode) differs from the previous call's there.  Other arguments
 * and results as rtp_decode_step (no phase event). */
#define RTP_STATIC_SCRATCH_BYTES (64ull << 20)
int rtp_decode_step_static(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q,
                           const rtp_bf16 *k_idx, const rtp_bf16 *k, const rtp_bf16 *v, float *out,
                           int32_t *idx_opt, int32_t *count_opt, int64_t cap, void *stream);

/* ---------------------------------------------------------------- cluster index */
/* The coarse-to-fine decode of the RTPurboV2 article (finding three): the cached
 * tokens of each indexer-key head are grouped into K clusters in the indexer
 * space, a query is matched against the K centres, and attention runs only over
 * the clusters it hits.  The article names neither the clustering method nor the
 * hit rule; this library takes Lloyd's k-means on the bf16 indexer keys (exact
 * fp64 squared distances, ties to the lowest index, centre j initialised to the
 * key at position floor(j N / K), centres rounded to bf16 after each round; the
 * index is the assignment against the final centres) and a dynamic top-p over
 * clusters weighing cluster j as n_j exp(s_j), s_j = fp32(q_idx . c_j), with the
 * token path's 256-bin histogram (bins above b* whole, clusters of bin b* in
 * ascending index while the mass before them is below p Z).  K <= min(N, 256). */

/* Workspace bytes of rtp_cluster_build / rtp_cluster_step for this layer and K (0 on
 * invalid arguments).  It begins with the regular workspace of the layer and
 * serves every call that one serves; prepare it with rtp_workspace_init. */
size_t rtp_cluster_workspace_bytes(const rtp_layer *layer, int32_t K);

/* Cluster positions 0..N-1 of every (b, indexer-key head i) into K clusters with
 * `iters` k-means rounds.  k_idx: [B, Hi, Ncap, R] bf16.  Outputs (device, caller-
 * owned): centroids [B, Hi, K, R] bf16; counts [B, Hi, K] int32; offsets
 * [B, Hi, K+1] int32 (offsets[K] = N); members [B, Hi, N] int32, the positions of
 * cluster j at members[offsets[j] .. offsets[j+1]), ascending.  RTP_ERR_ARG for
 * K outside [1, min(N, 256)], iters < 0, a layer without retrieval heads or a null
 * pointer. */
int rtp_cluster_build(const rtp_layer *layer, const rtp_bf16 *k_idx, int32_t K, int32_t iters,
                      rtp_bf16 *centroids, int32_t *counts, int32_t *offsets, int32_t *members,
                      void *ws, size_t ws_bytes, void *stream);

/* One decode step (nq = 1, top_k = 0, else RTP_ERR_UNSUPPORTED) over a cluster
 * index built for this N: each retrieval head r (indexer-key head i = r /
 * idx_group) scores the centres of (b, i), picks the hit clusters and attends
 * (eq. (5)) over all their members; local heads attend over window + sinks as in
 * rtp_decode_step.  idx_opt [B, Hr, 1, cap] receives the member positions (hit
 * clusters in ascending index, positions ascending in each; truncated at cap),
 * count_opt [B, Hr, 1] their number.  Layouts of the other arguments as
 * rtp_decode_step and rtp_cluster_build. */
int rtp_cluster_step(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, int32_t K,
                     const rtp_bf16 *centroids, const int32_t *counts, const int32_t *offsets,
                     const int32_t *members, const rtp_bf16 *k, const rtp_bf16 *v, float *out,
                     int32_t *idx_opt, int32_t *count_opt, int64_t cap, void *ws, size_t ws_bytes,
                     void *stream);

#ifdef __cplusplus
}
#endif
#endif /* RTP_H */

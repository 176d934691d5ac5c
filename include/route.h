/*
 * route.h - C ABI of libroute.so: the MoE token-routing and dispatch path on
 * one AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (web pages; sections as the pages number them):
 *   [SMOE]  "Speculative MoE" notes, research-notes-783.pages.dev/p/speculative-moe/
 *   [SPEC]  "Speculating Experts Accelerates Inference for Mixture-of-Experts",
 *           gist.science/ko/paper/2603.19289 (technical summary items)
 *   [FOE]   "Federation of Experts (FoE)", aitrends.kr/articles/58129
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer is a DEVICE pointer unless marked "host". bf16 values are
 *    passed as uint16_t bit patterns (upper half of an IEEE binary32).
 *  - Row-data tensors (marked "rows") are row-major and contiguous, their
 *    row length d is a multiple of 8 and their base pointer is 16-byte
 *    aligned, so every row is a whole number of 16-byte vectors.
 *  - The caller owns every buffer. The library never allocates, frees or
 *    synchronises, keeps no global state and is safe to call on several
 *    streams at once for disjoint buffers. Every call only enqueues work on
 *    stream `s` (a hipStream_t; NULL is the default stream) and returns.
 *  - Scratch space ("ws") is caller-provided; its size comes from the
 *    matching *_workspace_size() call. Its contents need no initialisation
 *    and are meaningless after the call.
 *  - Host-checkable errors (null required pointer, bad shape, misalignment,
 *    unsupported size, workspace too small) are returned as a status before
 *    anything is enqueued; nothing is written then. ROUTE_ERR_HIP means a
 *    kernel launch failed.
 *  - Data-dependent violations (a token id outside the vocabulary, a cluster
 *    id >= G, an expert id >= E, a slot or row index out of range) cannot be
 *    seen by the host: kernels OR the ROUTE_EBIT_* bits into the optional
 *    device word `err` (never cleared by the library) and skip the offending
 *    element; the affected outputs are then unspecified, but no access goes
 *    out of bounds.
 *  - n = 0 is a valid no-op (offset arrays are still written, all zero).
 *  - All outputs are bitwise reproducible run to run: no float atomics, and a
 *    fixed accumulation order per output element.
 *  - Counters (lar_count, hit_count, prefetch_coverage's covered) ADD into a
 *    caller-zeroed device uint64.
 */
#ifndef ROUTE_H_
#define ROUTE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

enum {
  ROUTE_OK = 0,
  ROUTE_ERR_NULL = 1,         /* a required pointer is NULL                    */
  ROUTE_ERR_SHAPE = 2,        /* n < 0, d % 8 != 0, E % H != 0, K > E/H, ...    */
  ROUTE_ERR_ALIGN = 3,        /* a rows pointer is not 16-byte aligned          */
  ROUTE_ERR_UNSUPPORTED = 4,  /* E > 1024, K > 16, G > 256, P > 16, d too big   */
  ROUTE_ERR_WORKSPACE = 5,    /* ws NULL or ws_bytes below the required size    */
  ROUTE_ERR_HIP = 6,          /* a kernel launch failed                         */
  ROUTE_ERR_NOT_MAPPED = 7    /* a buffer the GPU must read is not device-      */
                              /* accessible at its own address                  */
};

enum {
  ROUTE_EBIT_TOKEN_RANGE = 1u,   /* token id < 0 or >= vocab                    */
  ROUTE_EBIT_DEST_RANGE = 2u,    /* cluster id >= G                             */
  ROUTE_EBIT_EXPERT_RANGE = 4u,  /* expert id < 0 or >= E                       */
  ROUTE_EBIT_INDEX_RANGE = 8u,   /* slot / row / pair index out of range        */
  ROUTE_EBIT_VALUE_RANGE = 16u,  /* a count or placement entry out of its range */
  ROUTE_EBIT_SYNC = 32u          /* a workgroup gave up waiting at a grid       */
                                 /* barrier (the grid was not resident at once) */
};

/* Readable name of a status code (host; static string). */
const char* route_status_str(int status);

/*
 * route_predict - speculative destination cluster of each token.
 * [SMOE] section 4.1 (route-path prediction with lookup tables): the
 * intra-layer token table lut[id] gives the cluster; when the fallback is
 * enabled (conf != NULL) and the table's confidence byte conf[id] is below
 * conf_thr (128 ~ 0.5), the inter-layer 2-gram table
 * ngram[prev2[i] * G + prev1[i]] over the token's clusters at the two
 * preceding layers gives it instead.
 *   tok   int32[n]          token ids, 0 <= id < vocab
 *   lut   uint8[vocab]      token -> cluster
 *   conf  uint8[vocab]      confidence bytes (q/255), NULL disables the fallback
 *   prev2, prev1 uint8[n]   previous-layer clusters; ngram uint8[G*G]
 *                           (all three required iff conf != NULL)
 *   dest  uint8[n]          output cluster, written for every valid token
 * Errors: ROUTE_ERR_NULL, ROUTE_ERR_SHAPE (n < 0, vocab < 1, G < 1),
 * ROUTE_ERR_UNSUPPORTED (G > 256). Device bits: TOKEN_RANGE (dest[i] = 0),
 * DEST_RANGE (a table entry or prev cluster >= G; the entry is written as is).
 */
int route_predict(const int32_t* tok, int64_t n, const uint8_t* lut, const uint8_t* conf,
                  int32_t vocab, const uint8_t* prev2, const uint8_t* prev1,
                  const uint8_t* ngram, int32_t G, int32_t conf_thr, uint8_t* dest,
                  uint32_t* err, hipStream_t s);

/*
 * route_predict_sort - route_predict, then the stable sort of the predicted
 * clusters that srs_shuffle makes (the s-TS destination order), in the
 * launches of the sort alone: each key is predicted where the sort reads it.
 * [SMOE] section 4.1 (prediction) and section 3.1 (tokens grouped by their
 * predicted cluster, in order inside a cluster).
 *   Arguments up to dest as route_predict (dest uint8[n] written, the same
 *   bytes); cluster_offsets int32[G+1], row_of_src int32[n], src_of_row
 *   int32[n] and row_cluster uint8[n] (nullable) as srs_shuffle writes them
 *   for these clusters. ws: route_predict_sort_workspace_size(n, G) bytes.
 * Errors: as route_predict, plus NULL (cluster_offsets; row_of_src or
 * src_of_row with n > 0), WORKSPACE. Device bits: TOKEN_RANGE (that token
 * goes to cluster 0), DEST_RANGE (a cluster >= G: flagged, row_of_src -1,
 * the token gets no sorted row).
 */
int route_predict_sort(const int32_t* tok, int64_t n, const uint8_t* lut, const uint8_t* conf,
                       int32_t vocab, const uint8_t* prev2, const uint8_t* prev1,
                       const uint8_t* ngram, int32_t G, int32_t conf_thr, uint8_t* dest,
                       int32_t* cluster_offsets, int32_t* row_of_src, int32_t* src_of_row,
                       uint8_t* row_cluster, void* ws, size_t ws_bytes, uint32_t* err,
                       hipStream_t s);
size_t route_predict_sort_workspace_size(int64_t n, int32_t G);

/*
 * route_lut_build - offline table builder for route_predict.
 * [SMOE] section 4.1: the token-expert confidence table is reduced to a
 * token -> cluster table. For row i (id ids[i], routing idx[i][K] with
 * weights w[i][K]) the share of cluster c is the binary32 sum over
 * k = 0..K-1 of the w[i][k] whose expert sits on c (expert_cluster[]);
 * lut[ids[i]] = the cluster with the largest share (lower cluster on ties),
 * conf[ids[i]] = floor(fl(fl(255 * share) + 0.5)), clamped to [0, 255].
 *   ids int32[n] (distinct), idx int32[n][K], w float[n][K],
 *   expert_cluster uint8[E], lut uint8[vocab], conf uint8[vocab] (nullable)
 * Errors: ROUTE_ERR_NULL, ROUTE_ERR_SHAPE, ROUTE_ERR_UNSUPPORTED (G > 256,
 * K > 16, E > 1024). Device bits: TOKEN_RANGE, EXPERT_RANGE, DEST_RANGE.
 * Rows whose ids repeat race; ids must be distinct.
 */
int route_lut_build(const int32_t* ids, int64_t n, const int32_t* idx, const float* w,
                    int32_t K, const uint8_t* expert_cluster, int32_t E, int32_t G,
                    uint8_t* lut, uint8_t* conf, int32_t vocab, uint32_t* err,
                    hipStream_t s);

/*
 * srs_shuffle - shuffled reduce-scatter on one GPU.
 * [SMOE] section 3.1 (s-TS): the tensor-parallel all-reduce becomes a
 * reduce-scatter fused with a token shuffle that delivers each token's
 * reduced activation to its predicted cluster. Here the G clusters are G
 * contiguous row ranges of `out`:
 *   X[i]  = bf16_rne( sum_{p=0..P-1} partials[p][i] )  (binary32, in p order)
 *   rows are stably sorted by dest[i]: cluster c owns rows
 *   [cluster_offsets[c], cluster_offsets[c+1]), tokens in original order;
 *   out[row_of_src[i]] = X[i], src_of_row[row] = i, row_cluster[row] = dest[i].
 *   partials bf16 rows [P][n][d]; dest uint8[n] (NULL only when G == 1:
 *   pure reduce, identity order); out bf16 rows [n][d]; cluster_offsets
 *   int32[G+1]; row_of_src, src_of_row int32[n] and row_cluster uint8[n]
 *   are optional outputs (NULL = not written).
 *   ws: srs_shuffle_workspace_size(n, G) bytes.
 * Errors: NULL, SHAPE (n < 0, P < 1, d < 8 or d % 8, G < 1, n >= 2^31),
 * ALIGN, UNSUPPORTED (P > 16, G > 256), WORKSPACE. Device bit: DEST_RANGE.
 */
int srs_shuffle(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                const uint8_t* dest, int32_t G, uint16_t* out, int32_t* cluster_offsets,
                int32_t* row_of_src, int32_t* src_of_row, uint8_t* row_cluster,
                void* ws, size_t ws_bytes, uint32_t* err, hipStream_t s);
size_t srs_shuffle_workspace_size(int64_t n, int32_t G);

/*
 * srs_shuffle_gate - srs_shuffle and route_gate on its output in one pass.
 * [SMOE] section 3.1 (s-TS) for the reduce and the shuffle; [FOE] router
 * scores g[i] on the reduced rows. Writes every output of srs_shuffle, with
 * the same bytes, and
 *   logits[row][e] = out[row] . w[e]^T   (binary32, for every written row),
 * i.e. route_gate(out, n, d, w, E, logits) up to the order of the binary32
 * sums. The reduced rows are multiplied while they are still on chip, so
 * they are written once and not read back.
 *   Arguments as srs_shuffle, plus w bf16 rows [E][d] (16-byte aligned) and
 *   logits float[n][E] (row-major). ws: srs_shuffle_workspace_size(n, G).
 * Errors: as srs_shuffle, plus NULL (w or logits with n > 0), and
 * UNSUPPORTED unless P is 1, 2 or 4, d % 128 == 0 and 1 <= E <= 160 (use
 * srs_shuffle + route_gate there). Device bit: DEST_RANGE (rows whose key
 * is out of range get neither out nor logits).
 */
int srs_shuffle_gate(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                     const uint8_t* dest, int32_t G, uint16_t* out, int32_t* cluster_offsets,
                     int32_t* row_of_src, int32_t* src_of_row, uint8_t* row_cluster,
                     const uint16_t* w, int32_t E, float* logits, void* ws, size_t ws_bytes,
                     uint32_t* err, hipStream_t s);

/*
 * srs_shuffle_route - srs_shuffle, then the router, top-K and local
 * activation count of each reduced row, in one pass over the rows.
 * [SMOE] section 3.1 (s-TS) for the reduce and the shuffle, glossary (top-K
 * experts per token; local activation rate); [FOE] router scores g[i]. For a
 * small expert set the router's work per row is a few dot products, done
 * while the reduced row is still on chip. Writes every output of
 * srs_shuffle with the same bytes, and for every written row `row`:
 *   logits[row][e] = out[row] . w[e]^T   (binary32; nullable), as route_gate
 *     up to the order of the binary32 sums;
 *   idx[row][:], weights[row][:] = route_topk of those logits with H = 1
 *     and the given renorm (weights nullable): the same ranking rules, so
 *     idx equals route_topk(logits) bit for bit;
 *   *local += #{k : expert_cluster[idx[row][k]] == cluster of the row}, the
 *     cluster of the row being its predicted cluster dest[i] (0 without
 *     dest), i.e. lar_count(idx, K, 1, row_cluster, expert_cluster).
 *   Arguments as srs_shuffle_gate, plus K, renorm, idx int32[n][K], weights
 *   float[n][K], expert_cluster uint8[E] and local (device uint64,
 *   accumulated); expert_cluster and local are both given or both NULL (no
 *   count). ws: srs_shuffle_workspace_size(n, G).
 * Two kernels serve it: one lane per expert for small expert sets, the
 * matrix-core shuffle + router kernel of srs_shuffle_gate (top-K and count
 * in its epilogue, the same bits as route_topk) up to 160 experts.
 * Errors: as srs_shuffle, plus SHAPE (K < 1, K > E), NULL (w or idx with
 * n > 0; only one of expert_cluster and local), and UNSUPPORTED (K > 16,
 * or neither kernel takes the shape). The small-set kernel takes
 * 1 <= E <= 64, d <= 4096, E * C * 1024 <= 65536 with C the smallest of
 * 1, 2, 4, 8 such that C * 512 >= d (the router rows, padded to C * 512
 * elements, are staged in on-chip memory), P in {1, 2, 4} (P = 4:
 * d <= 2048); the matrix-core kernel P in {1, 2, 4}, d % 128 == 0 and
 * 1 <= E <= 160. Use the separate calls for other shapes. Device bit: DEST_RANGE (rows whose key is out
 * of range get none of the row outputs and add nothing to *local).
 */
int srs_shuffle_route(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                      const uint8_t* dest, int32_t G, uint16_t* out, int32_t* cluster_offsets,
                      int32_t* row_of_src, int32_t* src_of_row, uint8_t* row_cluster,
                      const uint16_t* w, int32_t E, float* logits, int32_t K, int32_t renorm,
                      int32_t* idx, float* weights, const uint8_t* expert_cluster,
                      unsigned long long* local, void* ws, size_t ws_bytes, uint32_t* err,
                      hipStream_t s);

/*
 * srs_route_sorted - srs_shuffle_route's row work for a destination order
 * already made (row_of_src from route_predict_sort or srs_shuffle): each
 * source row i is reduced and written to row row_of_src[i] with its logits,
 * top-K and count, exactly as srs_shuffle_route does after its sort (the
 * same bytes). [SMOE] section 3.1, glossary; [FOE] router scores g[i].
 *   row_of_src int32[n] (a row < 0 or >= n gets no outputs); dest uint8[n]
 *   (nullable: every row's cluster is 0) gives the predicted cluster for
 *   the count; the other arguments as srs_shuffle_route.
 * Errors: as srs_shuffle_route (without G and the workspace), plus NULL
 * (row_of_src with n > 0).
 */
int srs_route_sorted(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                     const int32_t* row_of_src, const uint8_t* dest, uint16_t* out,
                     const uint16_t* w, int32_t E, float* logits, int32_t K, int32_t renorm,
                     int32_t* idx, float* weights, const uint8_t* expert_cluster,
                     unsigned long long* local, hipStream_t s);

/*
 * srs_predict_route - route_predict_sort followed by srs_route_sorted, in
 * one launch for small batches: [SMOE] section 4.1 (the prediction), section
 * 3.1 and glossary (the shuffled reduce, router, top-K and count); [FOE]
 * router scores g[i]. Each workgroup predicts every token's cluster and
 * counts them itself, so it knows where its own rows go without a separate
 * sort. Every output is the bytes the two calls write: dest,
 * cluster_offsets, row_of_src, src_of_row and row_cluster as
 * route_predict_sort, out, logits, idx, weights and *local as
 * srs_route_sorted on that order.
 *   tok .. conf_thr: as route_predict_sort; partials .. local: as
 *   srs_route_sorted (row_cluster nullable).
 * Errors: as the two calls, plus UNSUPPORTED beyond n = 4096 tokens, G = 16
 * clusters or the lane-per-expert route kernel's shapes (E <= 64, the
 * padded router rows <= 64 KiB, P in {1, 2, 4}); use the two calls there.
 * Device bits: TOKEN_RANGE, DEST_RANGE as route_predict_sort.
 */
int srs_predict_route(const int32_t* tok, int64_t n, const uint8_t* lut, const uint8_t* conf,
                      int32_t vocab, const uint8_t* prev2, const uint8_t* prev1,
                      const uint8_t* ngram, int32_t G, int32_t conf_thr,
                      const uint16_t* partials, int32_t P, int32_t d, const uint16_t* w,
                      int32_t E, int32_t K, int32_t renorm, uint8_t* dest,
                      int32_t* cluster_offsets, int32_t* row_of_src, int32_t* src_of_row,
                      uint8_t* row_cluster, uint16_t* out, float* logits, int32_t* idx,
                      float* weights, const uint8_t* expert_cluster, unsigned long long* local,
                      uint32_t* err, hipStream_t s);

/*
 * srs_predict_route_dispatch - srs_predict_route followed by moe_permute
 * (one group) in one launch: [SMOE] section 4.1 (prediction), section 3.1
 * and glossary (shuffled reduce, router, top-K, count), section 1 (dispatch
 * of each token to its K experts). Each wave keeps its reduced row in
 * registers; every workgroup publishes its pairs per (cluster, expert) and
 * meets the others at a grid barrier, then writes its rows straight into
 * their expert slots, so the shuffled rows are neither written (unless out
 * is given) nor read back. Every output is the bytes srs_predict_route and
 * then moe_permute (H = 1, src = the shuffled rows) would write.
 *   tok .. local: as srs_predict_route, except out bf16 [n][d] nullable
 *   and weights required; expert_offsets int32 [E+1], slot_of_pair and
 *   pair_of_slot int32 [n*K] (pairs p = r*K + k over the shuffled rows r),
 *   disp bf16 [n*K][d]: as moe_permute.
 *   ws: srs_predict_route_dispatch_workspace_size(n, G, E) bytes, 256-byte
 *   aligned; its first 4 bytes count the barrier's arrivals and must hold a
 *   multiple of 256 (zero) before the first call with this ws. Every call
 *   leaves them so: keep the workspace between calls, and do not overlap
 *   two calls on one workspace. Its next 4 bytes bound each workgroup's wait
 *   at the barrier: 0 (as zero-filled) is the default, about half a second;
 *   p > 0 allows p - 1 polls after the workgroup's own arrival, so 1 lets
 *   only the last workgroup to arrive through. A workgroup that waits past
 *   the bound flags SYNC.
 * Errors: as srs_predict_route, plus NULL (expert_offsets, slot_of_pair,
 * pair_of_slot, disp, weights), WORKSPACE (size or alignment), UNSUPPORTED
 * where G*E > 256 or the grid (n/16 workgroups) cannot be resident on the
 * device at once. Device bits: as srs_predict_route, plus SYNC if a
 * workgroup gave up at the barrier (its rows are then not dispatched). With
 * any bit set the dispatch outputs are unspecified.
 */
int srs_predict_route_dispatch(const int32_t* tok, int64_t n, const uint8_t* lut,
                               const uint8_t* conf, int32_t vocab, const uint8_t* prev2,
                               const uint8_t* prev1, const uint8_t* ngram, int32_t G,
                               int32_t conf_thr, const uint16_t* partials, int32_t P, int32_t d,
                               const uint16_t* w, int32_t E, int32_t K, int32_t renorm,
                               uint8_t* dest, int32_t* cluster_offsets, int32_t* row_of_src,
                               int32_t* src_of_row, uint8_t* row_cluster, uint16_t* out,
                               float* logits, int32_t* idx, float* weights,
                               const uint8_t* expert_cluster, unsigned long long* local,
                               int32_t* expert_offsets, int32_t* slot_of_pair,
                               int32_t* pair_of_slot, uint16_t* disp, void* ws, size_t ws_bytes,
                               uint32_t* err, hipStream_t s);
/* 0 where the shape is not taken. */
size_t srs_predict_route_dispatch_workspace_size(int64_t n, int32_t G, int32_t E);

/*
 * srs_route_grouped - the grouped MoE block's routing in one kernel: the
 * cross-group reduce of the P group activations, the router, the grouped
 * top-K and the per-group local count. [FOE] grouped MoE block (H groups of
 * E/H experts, each picking its K/H by the router scores g[i]; the copy of
 * token i for group h sits on cluster row_cluster[i*H + h]); the reduce is
 * srs_shuffle's with one cluster ([SMOE] section 3.1). Every output is the
 * bytes of srs_shuffle (G = 1) + route_gate + route_topk (H) + lar_count
 * (H) would give, up to route_topk's weights, which are the same function
 * of the same logits (softmax over each group's picks for renorm = 1, over
 * all E logits from the row's largest for renorm = 0).
 *   partials bf16 [P][n][d]; out bf16 [n][d] (nullable: the reduced rows
 *   are not written); w bf16 [E][d]; logits float [n][E] (nullable);
 *   idx int32 [n][K] (slots group-major, descending inside a group);
 *   weights float [n][K] (nullable); row_cluster uint8 [n][H] and
 *   expert_cluster uint8 [E] with *local += the count (all three nullable
 *   together; row_cluster required with expert_cluster).
 * Errors: NULL, SHAPE (E % H, K % H, K/H > E/H, d % 8), ALIGN, UNSUPPORTED
 * (P not in {1, 2, 4}, d % 128, E > 160, K > 16).
 */
int srs_route_grouped(const uint16_t* partials, int32_t P, int64_t n, int32_t d, uint16_t* out,
                      const uint16_t* w, int32_t E, float* logits, int32_t K, int32_t H,
                      int32_t renorm, int32_t* idx, float* weights, const uint8_t* row_cluster,
                      const uint8_t* expert_cluster, unsigned long long* local, hipStream_t s);

/*
 * route_gate - router logits = x . w^T.
 * [FOE] per-layer comparison (router scores g[i]); [SPEC] item 2.A (the
 * next layer's gate applied to q_l). bf16 operands, binary32 accumulation
 * on the MFMA units.
 *   x bf16 rows [n][d]; w bf16 rows [E][d]; logits float[n][E] (row-major).
 * Errors: NULL, SHAPE (n < 0, d % 8, E < 1), ALIGN, UNSUPPORTED (E > 1024,
 * or d > 4194304 with E > 32).
 */
int route_gate(const uint16_t* x, int64_t n, int32_t d, const uint16_t* w, int32_t E,
               float* logits, hipStream_t s);

/*
 * route_topk - softmax + top-K, plain (H = 1) or FoE-grouped (H > 1).
 * [SMOE] section 1 and glossary (top-K experts per token); [FOE] grouped MoE
 * block: group h owns experts [h*E/H, (h+1)*E/H) and picks its top K/H.
 * Ranking is on the binary32 logits: larger first, lower expert index first
 * on equal values, -0.0 equal to +0.0. Slots are group-major, descending
 * inside a group. weights: renorm = 1 -> softmax over each group's chosen
 * logits (sums to 1 per group); renorm = 0 -> softmax over all E logits,
 * read at the chosen experts.
 *   logits float[n][E]; idx int32[n][K]; weights float[n][K] (nullable).
 * NaN logits are outside the contract (no fault, unspecified choice).
 * Errors: NULL, SHAPE (E % H, K % H, K/H > E/H, K < 1, H < 1), UNSUPPORTED
 * (E > 1024, K > 16).
 */
int route_topk(const float* logits, int64_t n, int32_t E, int32_t K, int32_t H, int32_t renorm,
               int32_t* idx, float* weights, hipStream_t s);

/*
 * lar_count - local activation counter.
 * [SMOE] glossary (local activation rate: the share of activations routed
 * to an expert on the token's own device); [FOE] rho. Adds to *local the
 * number of (i, k) with expert_cluster[idx[i][k]] == row_cluster[i*H + k/(K/H)].
 *   idx int32[n][K]; row_cluster uint8[n*H]; expert_cluster uint8[E];
 *   local: device uint64, accumulated. Out-of-range experts count as remote.
 * Errors: NULL, SHAPE, UNSUPPORTED (K > 16).
 */
int lar_count(const int32_t* idx, int64_t n, int32_t K, int32_t H, const uint8_t* row_cluster,
              const uint8_t* expert_cluster, int32_t E, unsigned long long* local,
              hipStream_t s);

/*
 * moe_permute - expert-contiguous dispatch.
 * [SMOE] section 1 (dispatch sends each token's activation to its K
 * experts); [FOE] grouped block (experts of group h read the group-h
 * activation). Pairs p = i*K + k are stably counting-sorted by idx[i][k]:
 * expert e owns slots [expert_offsets[e], expert_offsets[e+1]), pairs in
 * increasing p; slot_of_pair[p] = slot, pair_of_slot[slot] = p;
 * disp[slot] = src[(k / (K/H)) * n + i] (each source row read once, written
 * K/H times).
 *   idx int32[n][K]; src bf16 rows [H][n][d] (NULL = indices only; then
 *   disp must be NULL too); expert_offsets int32[E+1]; slot_of_pair,
 *   pair_of_slot int32[n*K]; disp bf16 rows [n*K][d].
 *   ws: moe_permute_workspace_size(n, K, E) bytes.
 * Errors: NULL, SHAPE (K % H, n*K >= 2^31, d % 8 when src given), ALIGN,
 * UNSUPPORTED (E > 1024, K > 16), WORKSPACE. Device bit: EXPERT_RANGE.
 */
int moe_permute(const int32_t* idx, int64_t n, int32_t K, int32_t E, int32_t H,
                const uint16_t* src, int32_t d, int32_t* expert_offsets, int32_t* slot_of_pair,
                int32_t* pair_of_slot, uint16_t* disp, void* ws, size_t ws_bytes,
                uint32_t* err, hipStream_t s);
size_t moe_permute_workspace_size(int64_t n, int32_t K, int32_t E);

/*
 * moe_permute_noalloc - moe_permute without a workspace argument and without
 * any allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, outputs, status codes and device bits as moe_permute, minus ws.
 * The sort's histogram table lives in a static device array of 512 KiB
 * (128 chunks x 1024 experts of int32) that each GPU holds until the process
 * ends; it is found on the first call for the GPU of stream s (a
 * hipGetSymbolAddress with that GPU current) and is fully rewritten by every
 * call, so nothing needs clearing. All calls on one GPU share that array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must be ordered by the caller.
 * Errors: those of moe_permute; WORKSPACE if the table would exceed the
 * array (not reachable within the supported E and n*K); HIP if the array's
 * address cannot be found; UNSUPPORTED for a device ordinal above 63.
 */
int moe_permute_noalloc(const int32_t* idx, int64_t n, int32_t K, int32_t E, int32_t H,
                        const uint16_t* src, int32_t d, int32_t* expert_offsets,
                        int32_t* slot_of_pair, int32_t* pair_of_slot, uint16_t* disp,
                        uint32_t* err, hipStream_t s);

/*
 * moe_combine - weighted combine of the expert outputs, with the SAG unshuffle.
 * [SMOE] section 1 (combine returns expert outputs to the token and sums
 * them) and section 3.1 (SAG, the inverse shuffle: out_row); [FOE] (the K
 * slots span the H groups, so the sum is also the cross-group sum).
 *   o[j] = sum_{k=0..K-1} weights[j][k] * y[slot_of_pair[j*K + k]]  (binary32, k order)
 *   out[out_row ? out_row[j] : j] = o[j]
 *   y bf16 rows [n*K][d]; weights float[n][K]; slot_of_pair int32[n*K];
 *   out_row int32[n] (nullable, must be a permutation of 0..n-1);
 *   out rows [n][d]: out_dtype 0 = bf16 (nearest even), 1 = float32.
 * Errors: NULL, SHAPE (d % 8, out_dtype), ALIGN, UNSUPPORTED (K > 16).
 * Device bit: INDEX_RANGE (slot >= n*K or out_row >= n; the term / row is skipped).
 */
int moe_combine(const uint16_t* y, const float* weights, const int32_t* slot_of_pair,
                int64_t n, int32_t K, int32_t d, const int32_t* out_row, void* out,
                int32_t out_dtype, uint32_t* err, hipStream_t s);

/*
 * moe_combine_gather - moe_combine with the unshuffle taken from the other
 * side: output row t combines token in_row[t].
 * [SMOE] section 1 and section 3.1 (SAG), as moe_combine. With
 * in_row[out_row[j]] == j for every j (in_row the inverse permutation, e.g.
 * srs_shuffle's row_of_src where moe_combine takes its src_of_row) the
 * output equals moe_combine's bit for bit; here the rows are written in
 * order and the token's slots and weights are read through in_row.
 *   out[t] = sum_{k=0..K-1} weights[j][k] * y[slot_of_pair[j*K + k]],
 *   j = in_row[t]  (binary32, k order); in_row int32[n], a permutation of
 *   0..n-1; the other arguments as moe_combine.
 * Errors: as moe_combine, plus NULL (in_row with n > 0).
 * Device bit: INDEX_RANGE (slot >= n*K, or in_row[t] out of range: row t
 * is not written).
 */
int moe_combine_gather(const uint16_t* y, const float* weights, const int32_t* slot_of_pair,
                       int64_t n, int32_t K, int32_t d, const int32_t* in_row, void* out,
                       int32_t out_dtype, uint32_t* err, hipStream_t s);

/*
 * route_qhidden - quasi-hidden state q_l = LN_{l+1}(d_l + r_l).
 * [SPEC] item 2.A: default vector plus residual, normalised with the next
 * layer's LayerNorm (biased variance over d, binary32 statistics).
 *   r bf16 rows [n][d]; dvec float[d]; gamma, beta float[d] (nullable =>
 *   1 and 0); q bf16 rows [n][d] (nearest even). dvec, gamma and beta are
 *   16-byte aligned like the rows.
 * Errors: NULL, SHAPE (d % 8, eps < 0), ALIGN, UNSUPPORTED (d > 8192).
 */
int route_qhidden(const uint16_t* r, const float* dvec, const float* gamma, const float* beta,
                  int64_t n, int32_t d, float eps, uint16_t* q, hipStream_t s);

/*
 * route_qgate - the next gate on q_l without writing q: logits float[n][E] =
 * q . w^T, q = LN_{l+1}(d_l + r_l) rounded to bf16 exactly as route_qhidden
 * stores it. [SPEC] item 2.A: q_l fed to layer l+1's router predicts its
 * experts. The same result as route_qhidden followed by route_gate up to the
 * order of the binary32 sums (route_gate splits K differently), in one pass
 * that keeps each workgroup's q rows in LDS; use route_qhidden + route_gate
 * where q itself is needed (the estimator layers) or d is another size.
 *   r, dvec, gamma, beta, eps as route_qhidden; w bf16 rows [E][d] (16-byte
 *   aligned); logits row-major.
 * Errors: NULL, SHAPE (d % 8, eps < 0, E < 1), ALIGN, UNSUPPORTED (d not
 * 1024, 2048 or 4096; E > 1024).
 */
int route_qgate(const uint16_t* r, const float* dvec, const float* gamma, const float* beta,
                int64_t n, int32_t d, float eps, const uint16_t* w, int32_t E, float* logits,
                hipStream_t s);

/*
 * route_qgate_topk - route_qgate followed by each row's top K experts in the
 * same kernel: idx int32[n][K] holds the K largest logits' columns, largest
 * first, equal logits to the lower column, -0.0 == +0.0 (route_topk's order
 * with H = 1; no weights). [SPEC] item 2.A (predicted top-K of layer l+1
 * from q_l). logits float[n][E] is written too when not NULL; idx equals
 * route_topk applied to those logits.
 *   truth int32[n][K] and hits (device uint64, accumulated): when both are
 *   given, the kernel also adds to *hits what hit_count(idx, truth) would
 *   add ([SPEC] item 4), so the predicted picks need not be read back; both
 *   NULL skips the count.
 * Errors: as route_qgate, plus SHAPE (K < 1, K > E), UNSUPPORTED (E > 256,
 * K > 16) and NULL (only one of truth, hits given).
 */
int route_qgate_topk(const uint16_t* r, const float* dvec, const float* gamma, const float* beta,
                     int64_t n, int32_t d, float eps, const uint16_t* w, int32_t E, int32_t K,
                     float* logits, int32_t* idx, const int32_t* truth, unsigned long long* hits,
                     hipStream_t s);

/*
 * route_gate_packed_size - bytes of route_gate_pack's output for E router
 * rows of d elements: ceil(E / 16) * 16 * d * 2, or 0 for a shape it does
 * not take (E < 1, d % 32 != 0).
 */
size_t route_gate_packed_size(int32_t E, int32_t d);

/*
 * route_gate_pack - a router's rows in the fragment order route_qgate_topk_packed
 * reads. [SPEC] item 2.A (the next layer's router, a fixed weight of the
 * model, applied to q_l on every step): packed once, read on every call.
 *   w bf16 rows [E][d]; wp bf16, route_gate_packed_size(E, d) bytes:
 *   wp[((g * (d/32) + t) * 64 + l) * 8 + e] = w[16 g + l % 16][32 t + 8 (l / 16) + e]
 *   for groups g of 16 rows, K steps t of 32 and lanes l < 64 (rows past E
 *   are zeros). Both pointers 16-byte aligned.
 * Errors: SHAPE (E < 1, d % 32 != 0), UNSUPPORTED (E > 1024), NULL, ALIGN.
 */
int route_gate_pack(const uint16_t* w, int32_t E, int32_t d, uint16_t* wp, hipStream_t s);

/*
 * route_est_out_topk_packed - the estimator's output layer with its top-K
 * and hit count in one kernel: logits = h . w2^T + b2, each row's top K of
 * them in route_topk's order, and *hits += the picks found among the row's
 * true picks. [SPEC] items 2.C (the estimator's second layer) and 4 (hit
 * rate). The logits are binary32 sums of exact bf16 products plus b2.
 *   h bf16 [n][hd] (the hidden layer, route_est_hidden's output);
 *   w2p bf16 packed by route_gate_pack(w2, E, hd); b2 float [E] (nullable);
 *   logits float [n][E] (nullable: not written); idx int32 [n][K];
 *   truth int32 [n][K] and hits uint64 (nullable together).
 * Errors: NULL, SHAPE (K > E, hd % 8), ALIGN, UNSUPPORTED (hd not 512,
 * 1024 or 2048, E > 256, K > 16).
 */
int route_est_out_topk_packed(const uint16_t* h, int64_t n, int32_t hd, const uint16_t* w2p,
                              const float* b2, int32_t E, int32_t K, float* logits,
                              int32_t* idx, const int32_t* truth, unsigned long long* hits,
                              hipStream_t s);

/*
 * route_qest_hidden_packed - q_l and the estimator's hidden layer in one
 * kernel: h = GELU(q W1^T + b1), q = LN_{l+1}(d_l + r_l) kept on chip.
 * [SPEC] items 2.A (q_l) and 2.C (the estimator's first layer). q is
 * rounded to bf16 exactly as route_qhidden stores it, so h equals
 * route_qhidden followed by route_est_hidden up to the order of the
 * binary32 sums (each element bf16, nearest even, of GELU in binary32).
 *   r bf16 [n][d], dvec float [d], gamma, beta float [d] (nullable), eps:
 *   as route_qhidden; w1p bf16 W1 [hd][d] packed by route_gate_pack(w1,
 *   hd, d); b1 float [hd]; h bf16 [n][hd].
 * Errors: NULL, SHAPE (d % 8, hd % 8 or hd < 8 as route_est_hidden, eps < 0),
 * ALIGN, UNSUPPORTED (d not 1024, 2048 or 4096; hd > 1024).
 */
int route_qest_hidden_packed(const uint16_t* r, const float* dvec, const float* gamma,
                             const float* beta, int64_t n, int32_t d, float eps,
                             const uint16_t* w1p, const float* b1, int32_t hd, uint16_t* h,
                             hipStream_t s);

/*
 * route_qgate_topk_packed - route_qgate_topk with the router given packed
 * (wp from route_gate_pack for the same E and d). [SPEC] items 2.A and 4.
 * The same results, bit for bit: the matrix products see the same operands
 * in the same order, read straight into registers instead of through a
 * per-wave transpose in on-chip memory.
 * Errors: as route_qgate_topk.
 */
/*
 * route_qest_topk_packed - the whole estimator predictor of one layer in one
 * kernel: q = LN_{l+1}(d_l + r_l), h = GELU(q W1^T + b1), logits = h W2^T +
 * b2, their top-K and the hit count against truth. [SPEC] items 2.A, 2.C
 * and 4. q and h stay on chip (h as bf16, nearest even, as the estimator
 * keeps it); the two products see the same operands in the same order as
 * route_qest_hidden_packed followed by route_est_out_topk_packed, so
 * logits, idx and hits equal that pair's, bit for bit.
 *   r, dvec, gamma, beta, eps: as route_qhidden; w1p: W1 [hd][d] packed by
 *   route_gate_pack(w1, hd, d); b1 float [hd]; w2p: W2 [E][hd] packed by
 *   route_gate_pack(w2, E, hd); b2 float [E] (nullable); logits float
 *   [n][E] (nullable), idx int32 [n][K], truth int32 [n][K] and hits (one
 *   uint64, added to): as route_qgate_topk.
 * Errors: NULL, SHAPE (as route_qest_hidden_packed and route_topk), ALIGN,
 * UNSUPPORTED (d not 1024, 2048 or 4096; hd not 512 or 1024, or hd > d;
 * E > 256; K > 16).
 */
int route_qest_topk_packed(const uint16_t* r, const float* dvec, const float* gamma,
                           const float* beta, int64_t n, int32_t d, float eps,
                           const uint16_t* w1p, const float* b1, int32_t hd,
                           const uint16_t* w2p, const float* b2, int32_t E, int32_t K,
                           float* logits, int32_t* idx, const int32_t* truth,
                           unsigned long long* hits, hipStream_t s);

int route_qgate_topk_packed(const uint16_t* r, const float* dvec, const float* gamma,
                            const float* beta, int64_t n, int32_t d, float eps,
                            const uint16_t* wp, int32_t E, int32_t K, float* logits,
                            int32_t* idx, const int32_t* truth, unsigned long long* hits,
                            hipStream_t s);

/*
 * route_estimator - lightweight neural estimator of next-layer logits.
 * [SPEC] item 2.C: logits = GELU(q . w1^T + b1) . w2^T + b2 (GELU with erf).
 * The hidden activation is kept in bf16 (nearest even) in the workspace
 * between the two MFMA products.
 *   q bf16 rows [n][d]; w1 bf16 rows [hd][d]; b1 float[hd]; w2 bf16 rows
 *   [E][hd]; b2 float[E]; logits float[n][E].
 *   ws: route_estimator_workspace_size(n, hd) bytes.
 * Errors: NULL, SHAPE (d % 8, hd % 8), ALIGN, UNSUPPORTED (hd > 4096,
 * E > 1024, d > 4194304), WORKSPACE.
 */
int route_estimator(const uint16_t* q, int64_t n, int32_t d, const uint16_t* w1, const float* b1,
                    int32_t hd, const uint16_t* w2, const float* b2, int32_t E, float* logits,
                    void* ws, size_t ws_bytes, hipStream_t s);
size_t route_estimator_workspace_size(int64_t n, int32_t hd);

/*
 * hit_count - prefetch hit counter.
 * [SPEC] item 4 (hit rate of predicted experts). Adds to *hits the sum over
 * tokens of |set(pred[i]) intersect set(truth[i])|.
 *   pred, truth int32[n][K]; hits: device uint64, accumulated.
 * Errors: NULL, SHAPE, UNSUPPORTED (K > 16).
 */
int hit_count(const int32_t* pred, const int32_t* truth, int64_t n, int32_t K,
              unsigned long long* hits, hipStream_t s);

/* ------------------------------------------------------------------------
 * Speculative expert grouping (s-EG): [SMOE] section 3.2 (co-activated
 * experts placed in one cluster, offline, with the gate's columns permuted)
 * and section 4.2 (balanced token-expert co-clustering, a theta-weighted
 * sum of token-load imbalance and cross-cluster activations with equal
 * experts per cluster, solved by a two-stage cross-entropy method).
 *
 * Readings (the pages give the terms, not their normalisation or the
 * method's steps): a token goes to the cluster holding most of its
 * activations (lowest cluster on ties); a placement x scores
 *   J = (1 - theta) * (1 - local / total) + theta * (G * max_g load[g] / tokens - 1)
 * with local = sum over tokens of that best cluster's activations and
 * load[g] the token count sent to g; the cross-entropy stage keeps a table
 * P[E][G] of placement probabilities. One solver iteration is
 * eg_sample -> eg_score -> eg_update, all enqueued (no host round trip).
 * Limits: E % 4 == 0, E % G == 0, E <= 1024, G <= 32, B <= 1024.
 * ------------------------------------------------------------------------ */

/*
 * eg_profile - token-id x expert activation counts of a routed batch.
 *   tok int32[n]; idx int32[n][K] (a route_topk output); row_of_id int32
 *   [vocab]: the profile row of each id, -1 for ids not profiled; counts
 *   int32[U][E] and freq int32[U] are ADDED to (caller-zeroed):
 *   counts[u][idx[i][k]] += 1 and freq[u] += 1 for u = row_of_id[tok[i]].
 * Device bits: TOKEN_RANGE, INDEX_RANGE (row_of_id < 0 or >= U), EXPERT_RANGE;
 * the offending pair is skipped. Integer atomics: exact in any order.
 */
int eg_profile(const int32_t* tok, const int32_t* idx, int64_t n, int32_t K,
               const int32_t* row_of_id, int32_t vocab, int32_t U, int32_t E, int32_t* counts,
               int32_t* freq, uint32_t* err, hipStream_t s);

/*
 * eg_init - solver state: P[e][g] = 1/G (float64 [E][G]) and *best_J = +inf.
 */
int eg_init(double* P, int32_t E, int32_t G, double* best_J, hipStream_t s);

/*
 * eg_sample - B candidate placements place uint8[B][E]. Candidate b takes
 * experts in index order; expert e goes to the first cluster g whose running
 * sum of P[e][g'] over clusters with room left (E/G experts each) exceeds
 * u * W, W that total and u = (SplitMix64 output n >> 11) * 2^-53 for the
 * generator seeded with `seed` and n = (iter * B + b) * E + e + 1. When
 * rounding leaves no such g, the last open cluster of positive weight; when
 * W = 0, the first open cluster.
 */
int eg_sample(const double* P, int32_t E, int32_t G, int32_t B, uint64_t seed, int32_t iter,
              uint8_t* place, hipStream_t s);

/*
 * eg_score - scores of B placements against a profile.
 *   counts int32[U][E] (each entry <= 65535, each row summing below 2^24,
 *   else VALUE_RANGE), freq int32[U], place uint8[B][E] (entries < G, else
 *   VALUE_RANGE) -> local int64[B], load int64[B][G] (overwritten).
 *   ws: eg_score_workspace_size(U, E, G, B) bytes, 16-byte aligned.
 * Exact integer results (bf16 matrix-core product of the counts' high and
 * low bytes against one-hot placements; every partial sum an integer below
 * 2^24).
 */
size_t eg_score_workspace_size(int32_t U, int32_t E, int32_t G, int32_t B);
int eg_score(const int32_t* counts, const int32_t* freq, int32_t U, int32_t E, int32_t G,
             const uint8_t* place, int32_t B, long long* local, long long* load, void* ws,
             size_t ws_bytes, uint32_t* err, hipStream_t s);

/*
 * eg_update - one cross-entropy step. J[b] (float64, nullable output) as
 * above from local, load, total (activations in the profile) and tokens
 * (sum of freq); candidate b is elite when fewer than n_elite candidates
 * precede it (lower J, or equal J and lower index); then
 *   P[e][g] = alpha * (#elite with place[b][e] == g) / n_elite + (1 - alpha) * P[e][g]
 * and, if the lowest J is below *best_J, *best_J and best_place uint8[E]
 * take that candidate's. Float64 in exactly this operation order.
 */
int eg_update(const long long* local, const long long* load, const uint8_t* place, int32_t B,
              int32_t E, int32_t G, long long total, long long tokens, double theta,
              int32_t n_elite, double alpha, double* P, double* best_J, uint8_t* best_place,
              double* J, hipStream_t s);

/* ------------------------------------------------------------------------
 * Estimator fit: [SPEC] item 2.C (a shallow network predicts the next
 * layer's router logits from q_l) and item 4 (a few million training tokens
 * suffice). Reading: the hidden layer GELU(q W1^T + b1) stays as drawn
 * (random features, the estimator's own bf16 activations) and the output
 * layer is the ridge fit (H'^T H' + lambda I) W' = H'^T Y with H' = [H | 1]
 * and lambda = ridge * trace(H'^T H') / (hd + 1). Float64 throughout.
 * ------------------------------------------------------------------------ */

/*
 * route_est_hidden - the estimator's hidden layer alone: h bf16 rows [n][hd]
 * = GELU(q W1^T + b1), exactly as route_estimator computes it.
 * Errors: as route_estimator's first product (d % 8, hd % 8, hd > 4096).
 */
int route_est_hidden(const uint16_t* q, int64_t n, int32_t d, const uint16_t* w1,
                     const float* b1, int32_t hd, uint16_t* h, hipStream_t s);

/*
 * est_fit_gram - gram float64[hd+1][hd+1] = H'^T H' and rhs float64[hd+1][E]
 * = H'^T Y for features h bf16 [n][hd] and targets y float[n][E] (row-major).
 * Products and sums in float64 (32 slices of the n rows, summed in order).
 *   ws: est_fit_gram_workspace_size(n, hd, E) bytes.
 * Errors: SHAPE (n < 1, hd < 1, E < 1), UNSUPPORTED (hd > 4096, E > 1024),
 * WORKSPACE.
 */
size_t est_fit_gram_workspace_size(int64_t n, int32_t hd, int32_t E);
int est_fit_gram(const uint16_t* h, const float* y, int64_t n, int32_t hd, int32_t E, double* gram,
                 double* rhs, void* ws, size_t ws_bytes, hipStream_t s);

/*
 * est_fit_solve - in place: gram (m x m, m = hd + 1) gets lambda = ridge *
 * trace / m added to its diagonal and is overwritten by its Cholesky factor
 * L (lower triangle and diagonal) and L^T (strict upper triangle); rhs
 * (m x E) is overwritten by the solution W'. A non-positive pivot ORs 1 into
 * the optional device *info (that pivot is taken as 1 and the solve goes on).
 * Errors: SHAPE (m < 1, E < 1, ridge < 0), UNSUPPORTED (m > 4097, E > 1024).
 */
int est_fit_solve(double* gram, double* rhs, int32_t m, int32_t E, double ridge, int32_t* info,
                  hipStream_t s);

/*
 * est_fit_weights - w2 bf16 [E][hd] = W'[:hd]^T, each float64 value rounded
 * once to the nearest bf16 (ties to even), and b2 float[E] = W'[hd].
 */
int est_fit_weights(const double* wsol, int32_t hd, int32_t E, uint16_t* w2, float* b2,
                    hipStream_t s);

/* ------------------------------------------------ speculative expert prefetch
 * [SPEC] items 1, 2 and 4: with expert weights offloaded to host memory,
 * on-demand loading copies a layer's selected experts after its router runs;
 * prefetching copies the next layer's predicted experts while the current
 * layer computes, and speculative execution runs them without waiting for
 * the true router. The page describes one decoding request (its K predicted
 * experts); for a batch of n tokens and C staging slots the prefetched set is
 * the distinct predicted experts ranked by how many picks name them.
 */

/*
 * prefetch_plan - list[C]: the distinct experts named by pred int32[n][K],
 * ordered by pick count (descending), equal counts by expert index
 * (ascending), the first C of them; unused slots hold -1. *nlist = the
 * number listed (min(distinct, C)).
 *   list: device int32[C]; nlist: device int32[1].
 * Errors: SHAPE (n < 0, K < 1, E < 1, C < 1, C > E), UNSUPPORTED (E > 1024),
 * NULL. Device bits: EXPERT_RANGE (a pick outside [0, E): not counted).
 */
int prefetch_plan(const int32_t* pred, int64_t n, int32_t K, int32_t E, int32_t C, int32_t* list,
                  int32_t* nlist, uint32_t* err, hipStream_t s);

/*
 * prefetch_issue - HOST function. For each i < C with list[i] >= 0, copies
 * expert list[i]'s block (bank + list[i] * expert_bytes) to slot i (slots +
 * i * expert_bytes) with hipMemcpyAsync on stream s (normally a copy stream
 * beside the compute stream); runs of consecutive experts in consecutive
 * slots go as one transfer. The DMA engines do the copy: no compute units
 * are used and concurrent kernels keep their memory bandwidth, so this is
 * the path that overlaps a prefetch with the current layer's compute.
 *   bank: pinned host memory (or device memory), E blocks. list: HOST
 *   int32[C] (-1 = empty slot), read during the call, e.g. prefetch_plan's
 *   list copied back after an event. slots: device memory, C blocks.
 * Errors: SHAPE (E < 1, C < 1, expert_bytes < 0, a list entry < -1 or
 * >= E: nothing enqueued), NULL, NOT_MAPPED (bank not device memory or
 * pinned host memory), HIP (an enqueue failed; earlier transfers of the
 * call may be enqueued).
 */
int prefetch_issue(const void* bank, int32_t E, int64_t expert_bytes, const int32_t* list,
                   int32_t C, void* slots, hipStream_t s);

/*
 * prefetch_copy - slot i (expert_bytes bytes at slots + i * expert_bytes)
 * receives expert list[i]'s block (bank + list[i] * expert_bytes) for each
 * i < C with list[i] >= 0; slots with -1 are left as they are.
 *   bank: E blocks of expert_bytes, either device memory or pinned host
 *   memory mapped for the device at the same address (hipHostMalloc, or a
 *   pinned torch tensor): the copy runs as a kernel of 64 workgroups that
 *   reads it over PCIe, so `list` can be produced on the GPU by
 *   prefetch_plan in the same stream. slots: device memory, C blocks.
 *   Measured on MI355X: the kernel reaches the same PCIe rate as the DMA
 *   engines, but kernels running beside it that stream HBM slow down
 *   several-fold; overlap a prefetch with compute through prefetch_issue,
 *   and use this call where the GPU would otherwise wait (on-demand loads).
 *   Calls on one slot buffer in different streams must be ordered by the
 *   caller.
 * Errors: SHAPE (E < 1, C < 1, expert_bytes < 0), UNSUPPORTED (E > 1024),
 * ALIGN (expert_bytes % 16, bank or slots not 16-byte aligned), NULL,
 * NOT_MAPPED (hipPointerGetAttributes does not report bank as accessible
 * at its own address). Device bits: EXPERT_RANGE (list[i] >= E: skipped).
 */
int prefetch_copy(const void* bank, int32_t E, int64_t expert_bytes, const int32_t* list,
                  int32_t C, void* slots, uint32_t* err, hipStream_t s);

/*
 * prefetch_coverage - for the true picks truth int32[n][K] and the slot
 * list[C] (-1 = empty): *covered += the number of picks whose expert is
 * listed; miss int32[E] = the true experts listed in no slot, in index order,
 * padded with -1; *nmiss = their number (the blocks an on-demand load still
 * copies: prefetch_copy with list = miss, C = E).
 *   covered: device uint64, accumulated; miss: device int32[E]; nmiss: int32[1].
 * Errors: SHAPE (n < 0, K < 1, E < 1, C < 1), UNSUPPORTED (E > 1024), NULL.
 * Device bits: EXPERT_RANGE (a pick or list entry >= E, or a pick < 0: ignored).
 */
int prefetch_coverage(const int32_t* truth, int64_t n, int32_t K, int32_t E, const int32_t* list,
                      int32_t C, unsigned long long* covered, int32_t* miss, int32_t* nmiss,
                      uint32_t* err, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* ROUTE_H_ */

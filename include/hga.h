/*
 * hga.h -- C ABI of libhga, the gfx950 (MI355X) hot path of Hierarchical
 * Global Attention (HGA): chunk summaries -> per-block top-k chunk routing ->
 * exact attention over the routed chunks plus the causal local block, and its
 * segment-wise backward.
 *
 * Method: arXiv 2607.15105, "Long-Context Fine-Tuning with Limited VRAM"
 * (gist.science technical summary, section 2.1 "Hierarchical Global
 * Attention" and section 2.2 "segment-wise backward and tiered storage";
 * author abstract on franklineh.com and fugumt.com).
 *
 * Conventions shared by every call
 *   - Notation: Hq query heads, Hkv key/value heads, G = Hq / Hkv, head dim
 *     D = 128, chunk C = 64, query block Bq = C, top-k k. Query head h uses
 *     key/value head h / G.
 *   - All buffers are caller-owned, contiguous device memory. The library
 *     never allocates or frees device memory. Its only global state is a
 *     thread-local error string and, for hga_attend_bwd_noalloc, a static
 *     device scratch array with a mutex-guarded table of its per-device
 *     addresses; every other call is reentrant.
 *   - Layouts (row-major, innermost last):
 *       Q, O, dO        bf16  [Hq][n_q][D]      active queries p0 .. p0+n_q-1
 *       K, V            bf16  [Hkv][T_cap][D]   every position 0 .. T_cap-1
 *       summaries       f32   [Hkv][n_chunk_cap][D]
 *       ids             int32 [Hkv][n_q/Bq][k]
 *       lse             f32   [Hq][n_q]
 *       dQ              f32   [Hq][n_q][D]
 *       dK, dV          f32   [Hkv][n_q][D]     active keys p0 .. p0+n_q-1
 *     bf16 buffers hold raw bfloat16 bit patterns (uint16_t storage).
 *   - Every call only enqueues work on `stream` (NULL = the null stream) and
 *     returns; results are visible once the caller synchronises. Device-side
 *     faults surface at that synchronisation, not in the return code.
 *   - Argument checks are synchronous and complete before anything is
 *     launched: a call that returns an error has enqueued nothing.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type, declared as HIP itself declares it. */
typedef struct ihipStream_t *hipStream_t;

typedef enum hga_status {
    HGA_OK = 0,
    HGA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned position  */
    HGA_ERR_UNSUPPORTED = 2,   /* a shape this build has no kernel for         */
    HGA_ERR_CAPACITY = 3,      /* a buffer too small for the requested work    */
    HGA_ERR_HIP = 4            /* the HIP runtime refused a launch             */
} hga_status;

typedef enum hga_dtype { HGA_BF16 = 0 } hga_dtype;

typedef struct hga_config {
    int32_t n_q_heads;      /* Hq; a multiple of n_kv_heads                    */
    int32_t n_kv_heads;     /* Hkv <= 65535; G = Hq / Hkv must be 1, 2, 4 or 8 */
    int32_t head_dim;       /* D; must be 128                                  */
    int32_t chunk;          /* C; must be 64 (the pages' example chunk length) */
    int32_t q_block;        /* Bq; must equal chunk                            */
    int32_t top_k;          /* k; 0 .. 256 routed chunks per query block       */
    float softmax_scale;    /* <= 0 selects 1/sqrt(head_dim)                   */
    int32_t dtype;          /* HGA_BF16                                        */
    int32_t sink_chunks;    /* s: 0 .. HGA_MAX_SINK_CHUNKS; see below          */
    int32_t route_heads;    /* HGA_ROUTE_PER_KV_HEAD (0) or _PER_Q_HEAD; below */
} hga_config;

/*
 * Sink window (technical summary 2.1: the chosen chunks come alongside fixed
 * sink and local windows; the pages give no size). The first s chunks,
 * tokens [0, sC), are attended by every query block whose first position P is
 * past them (tokens [0, min(sC, P))), and are not routing candidates: with
 * s > 0, hga_route's candidates become the chunks c with s <= c < P/C, an id
 * row's entries below s add nothing to the attended set (they are in it
 * already), and the group level treats sink chunks the same way. s = 0 is the
 * method without a sink.
 */
#define HGA_MAX_SINK_CHUNKS 64

/*
 * Routing granularity (technical summary 2.1 has the query block score the
 * chunk summaries but does not say over which heads). A routing unit owns
 * one id row per query block:
 *   HGA_ROUTE_PER_KV_HEAD  a unit is a kv head g: the block's mean query is
 *                          taken over the G query heads that share g, and all
 *                          G heads attend the chunks of row ids[g][b]
 *                          (U = Hkv units).
 *   HGA_ROUTE_PER_Q_HEAD   a unit is a query head h: its own block mean,
 *                          scored against the summaries of its kv head h/G,
 *                          and head h attends the chunks of row ids[h][b]
 *                          (U = Hq units; the G heads of a kv head no longer
 *                          share the gathered chunks).
 * hga_route, hga_route_causal, hga_attend_fwd, hga_route_attend_fwd and
 * hga_attend_bwd take either; the group-level, decode and diagnostic entry
 * points take HGA_ROUTE_PER_KV_HEAD only (else HGA_ERR_UNSUPPORTED). Any
 * other value is HGA_ERR_INVALID_ARG.
 */
#define HGA_ROUTE_PER_KV_HEAD 0
#define HGA_ROUTE_PER_Q_HEAD 1

/*
 * hga_summarize -- append chunk summaries (technical summary 2.1, chunk
 * selection: a compact summary vector per closed fixed-size chunk stays
 * resident). For every kv head g and every chunk c with
 * tok_begin <= cC < tok_begin + n_tok:
 *     summaries[g][c][:] = (1/C) * sum_{t=cC}^{cC+C-1} K[g][t][:]
 * accumulated in fp32. Rows outside that range are not touched.
 *   K            device bf16 [Hkv][T_cap][D]
 *   tok_begin    multiple of C; n_tok >= 0, multiple of C;
 *                tok_begin + n_tok <= T_cap
 *   summaries    device f32 [Hkv][n_chunk_cap][D]; needs
 *                (tok_begin + n_tok)/C <= n_chunk_cap, else HGA_ERR_CAPACITY
 */
hga_status hga_summarize(const hga_config *cfg, const void *K, int64_t T_cap,
                         int64_t tok_begin, int64_t n_tok,
                         float *summaries, int64_t n_chunk_cap,
                         hipStream_t stream);

/*
 * hga_route -- per query block top-k chunk ids (technical summary 2.1: the
 * current query block scores the resident summaries and keeps the most
 * relevant earlier chunks; the selection carries no gradient). For routing
 * unit u (kv head g = u, or query head u of kv head g = u/G; see
 * cfg->route_heads) and block b, first query position P = p0 + b*Bq:
 *     qbar    = mean of Q[h][i] over the query heads h of unit u (the G heads
 *               of g, or head u alone) and the Bq queries of block b (fp32)
 *     score_c = qbar . summaries[g][c]     for every chunk s <= c < P/C (fp32;
 *               s = cfg->sink_chunks, see hga_config)
 *     ids[u][b][:] = the min(k, P/C - s) chunks of highest score, ties to
 *               the lower chunk id, written in ascending id order, then -1.
 *   Q              device bf16 [Hq][n_q][D]
 *   summaries      device f32 [Hkv][n_chunk_cap][D]; rows 0 .. n_chunks_valid-1
 *                  must hold summaries. Needs (p0 + n_q - Bq)/C <= n_chunks_valid
 *                  <= n_chunk_cap, else HGA_ERR_CAPACITY. Only rows c < P/C are
 *                  read for block b.
 *   ids            device int32 [U][n_q/Bq][k]  (U = Hkv, or Hq per query head)
 *   scores_or_null device f32 [U][n_q/Bq][k] or NULL: the fp32 score of each
 *                  written id, -INFINITY beside a -1.
 */
hga_status hga_route(const hga_config *cfg, const void *Q, int64_t p0, int64_t n_q,
                     const float *summaries, int64_t n_chunk_cap,
                     int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                     hipStream_t stream);

/*
 * hga_route_causal -- strictly causal routing. hga_route's block mean takes
 * in the block's own later queries, so a query's chunk set depends on
 * queries after it (the causal leakage inside a chunk that the pages name as
 * a limitation; they define no fix). Here block b instead scores with the
 * mean of the Bq queries just before it, positions P - Bq .. P - 1: the rows
 * of block b - 1 of Q for b >= 1, and Q_prev for b = 0. Candidates, tie rule,
 * output layout and errors are hga_route's; the attention entry points take
 * these ids unchanged.
 *   Q_prev   device bf16 [Hq][Bq][D]: the queries at positions p0 - Bq ..
 *            p0 - 1 (the previous segment's last block); may be NULL when
 *            p0 = 0 (block 0 then has no candidates), else HGA_ERR_INVALID_ARG
 */
hga_status hga_route_causal(const hga_config *cfg, const void *Q, const void *Q_prev,
                            int64_t p0, int64_t n_q, const float *summaries,
                            int64_t n_chunk_cap, int64_t n_chunks_valid, int32_t *ids,
                            float *scores_or_null, hipStream_t stream);

/*
 * hga_attend_fwd -- exact-token attention over the routed chunks and the
 * causal local block (technical summary 2.1: only the exact K/V of the
 * selected units enter attention; summaries never act as values). For query
 * i (position p = p0 + i, block b, head h, kv head g = h/G, routing unit u =
 * g, or h with HGA_ROUTE_PER_Q_HEAD):
 *     A(i) = [0, min(sC, P))  U  union_{c in ids[u][b], s <= c < P/C} [cC, cC+C)
 *            U  [P, p]                 (s = cfg->sink_chunks, the sink window)
 *     z_j  = scale * Q[h][i] . K[g][j]
 *     O[h][i]   = sum_{j in A(i)} softmax(z)_j V[g][j]      (bf16, RNE)
 *     lse[h][i] = ln sum_{j in A(i)} exp(z_j)                (f32)
 * bf16 operands, fp32 accumulation, the probabilities rounded to bf16 for the
 * P.V product. ids entries outside [0, P/C) are skipped, and the entries of
 * a row form a set: their order does not matter and a repeated id is attended
 * once (rows as hga_route writes them, ascending and distinct, need no
 * de-duplication work).
 *   Q, O   device bf16 [Hq][n_q][D];   K, V device bf16 [Hkv][T_cap][D]
 *   ids    device int32 [U][n_q/Bq][k] (U as for hga_route); lse device f32 [Hq][n_q]
 *   p0     multiple of C; n_q multiple of Bq; p0 + n_q <= T_cap; at most 65535
 *          query blocks per call (HGA_ERR_UNSUPPORTED)
 */
hga_status hga_attend_fwd(const hga_config *cfg, const void *Q, const void *K,
                          const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                          const int32_t *ids, void *O, float *lse,
                          hipStream_t stream);

/*
 * hga_route_attend_fwd -- hga_route followed by hga_attend_fwd on its ids, in
 * one launch where the candidates fit (each workgroup routes its own query
 * block with the routing kernel's code, then attends): ids, scores_or_null, O
 * and lse are bit-identical to those two calls with the same arguments, and
 * the arguments, layouts and errors are theirs. With more than 8704
 * candidate chunks in the last block the two kernels run one after the other
 * (same results).
 */
hga_status hga_route_attend_fwd(const hga_config *cfg, const void *Q, const void *K,
                                const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                const float *summaries, int64_t n_chunk_cap,
                                int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                                void *O, float *lse, hipStream_t stream);

/*
 * hga_attend_bwd_workspace_bytes -- size of the device workspace that
 * hga_attend_bwd needs for n_q active queries (0 on invalid arguments).
 */
size_t hga_attend_bwd_workspace_bytes(const hga_config *cfg, int64_t n_q);

/*
 * hga_attend_bwd -- gradient of the attention above for the active segment
 * only (technical summary 2.2: segment-wise backward; the key/value history
 * before the segment is detached; technical summary 2.1: routing runs without
 * gradient, so ids are constants). With P_ij = exp(z_j - lse_i),
 * Delta_i = sum_j P_ij (dO_i . V_j) and dS_ij = P_ij (dO_i . V_j - Delta_i):
 *     dQ_i = scale * sum_{j in A(i)} dS_ij K_j
 *     dK_j = scale * sum_{(h,i): j in A(i)} dS_ij Q_i     p0 <= j < p0+n_q
 *     dV_j =         sum_{(h,i): j in A(i)} P_ij dO_i     p0 <= j < p0+n_q
 * (sums over the G query heads that share kv head g, each head with its own
 * A(i); A(i) and the ids rule as for hga_attend_fwd, a set per row, id rows
 * per cfg->route_heads). lse is the output of
 * hga_attend_fwd for the same arguments, O (bf16, may be NULL) its output.
 * Delta is summed exactly in fp32 from P and dP. The dQ kernel makes one pass
 * over each block's tiles with the estimate D_i = dO_i . O_i in place of
 * Delta_i and keeps it for the 32 query rows of a wave when each has
 * |Delta_i - D_i| <= 2^-8 sum_j P_ij |dO_i . V_j - D_i| (the estimate then moves
 * dQ_i by no more than the worst-case bound of rounding every dS term to bf16
 * once, 2^-8 being bf16's unit roundoff); other waves -- attention concentrated
 * on a few keys, where O's bf16 rounding would reach dS undamped, and every
 * wave when O is NULL -- recompute dQ in a second pass with the exact Delta
 * (hga_diag_bwd_second_pass counts the workgroups that ran one). O is read only
 * for the estimate: any O, Inf or NaN included, gives gradients within that
 * bound (an estimate that is not finite always takes the second pass).
 * Every element of dQ, dK and dV is written; the caller does not clear them.
 * Deterministic: no output is accumulated with atomics, every sum has a fixed
 * order (a per-chunk counter in the workspace only decides which workgroup
 * adds the partial sums). At most 65536 active queries (HGA_ERR_UNSUPPORTED).
 *   workspace  device memory of at least hga_attend_bwd_workspace_bytes bytes,
 *              else HGA_ERR_CAPACITY; contents on entry are ignored; calls that
 *              share one workspace must not overlap in time.
 */
hga_status hga_attend_bwd(const hga_config *cfg, const void *Q, const void *K,
                          const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                          const int32_t *ids, const void *O, const float *lse,
                          const void *dO, float *dQ, float *dK_active,
                          float *dV_active, void *workspace, size_t ws_bytes,
                          hipStream_t stream);

/*
 * hga_attend_bwd_noalloc -- hga_attend_bwd without a caller workspace, for
 * callers that cannot allocate device memory or pass one: code under HIP
 * graph capture, tight training or serving loops, harnesses that forbid
 * allocation. Same arguments, results (bit for bit) and checks as
 * hga_attend_bwd, minus workspace/ws_bytes; the workspace is a fixed device
 * array inside the library of HGA_BWD_NOALLOC_SCRATCH_BYTES bytes, one copy
 * on every GPU the library runs on, held until the process ends. Its device
 * address is looked up once per device, on the first call there. A call whose
 * hga_attend_bwd_workspace_bytes exceeds that size returns HGA_ERR_CAPACITY
 * (the 16K-history Qwen3-8B layer's backward, 32 query heads over 8 kv heads
 * and 2048 active queries, needs 112.3 MiB). The call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine). Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and must be serialized by the caller.
 * The stream must belong to the current device (else HGA_ERR_INVALID_ARG).
 */
#define HGA_BWD_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
hga_status hga_attend_bwd_noalloc(const hga_config *cfg, const void *Q, const void *K,
                                  const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                  const int32_t *ids, const void *O, const float *lse,
                                  const void *dO, float *dQ, float *dK_active,
                                  float *dV_active, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Second routing level: groups of HGA_GROUP tokens inside the chosen chunks
 * (technical summary 2.1, group selection: the selected chunks are split into
 * smaller groups, e.g. 8 tokens, the router keeps the best groups of the
 * chosen chunks by their summaries, and only the exact K/V of the kept groups
 * enter attention). Group u covers tokens [8u, 8u + 8); chunk c holds groups
 * 8c .. 8c + 7. The local block stays a whole causal chunk.
 * ---------------------------------------------------------------------- */
#define HGA_GROUP 8

/*
 * hga_summarize_groups -- group summaries, the group-level analogue of
 * hga_summarize: for kv head g and every group u of chunks
 * tok_begin/C .. (tok_begin + n_tok)/C - 1,
 *     group_summaries[g][u][d] = (1/8) * sum_{t = 8u}^{8u+7} K[g][t][d]   (f32)
 *   K                device bf16 [Hkv][T_cap][D]
 *   group_summaries  device f32 [Hkv][n_group_cap][D]; rows of other groups
 *                    are not touched
 *   tok_begin, n_tok multiples of C; tok_begin + n_tok <= T_cap, else
 *                    HGA_ERR_INVALID_ARG; (tok_begin + n_tok)/8 <= n_group_cap,
 *                    else HGA_ERR_CAPACITY
 */
hga_status hga_summarize_groups(const hga_config *cfg, const void *K, int64_t T_cap,
                                int64_t tok_begin, int64_t n_tok, float *group_summaries,
                                int64_t n_group_cap, hipStream_t stream);

/*
 * hga_route_groups -- per query block, the best groups inside the block's
 * routed chunks. For kv head g and block b (first position P), with qbar the
 * block mean of hga_route:
 *     candidates = the groups of the distinct chunk ids c of chunk_ids[g][b]
 *                  with 0 <= c < P/C (the row is a set; other entries skipped)
 *     score_u    = qbar . group_summaries[g][u]
 *     group_ids[g][b][:] = the min(group_top_k, #candidates) groups of highest
 *                  score, ties to the lower group id, written ascending and
 *                  padded with -1
 *   chunk_ids        device int32 [Hkv][n_q/Bq][cfg->top_k] (hga_route's ids)
 *   group_summaries  device f32 [Hkv][n_group_cap][D] (hga_summarize_groups);
 *                    every group of a chunk c < (p0 + n_q - Bq)/C must be
 *                    summarized: 8 * that many <= n_group_cap, else
 *                    HGA_ERR_CAPACITY
 *   group_top_k      0 .. 2048 (= 8 * 256, every group of the largest top_k)
 *   group_ids        device int32 [Hkv][n_q/Bq][group_top_k]
 *   scores_or_null   device f32 like group_ids (the fp32 score of each id,
 *                    -inf in padding) or NULL
 */
hga_status hga_route_groups(const hga_config *cfg, const void *Q, int64_t p0, int64_t n_q,
                            const float *group_summaries, int64_t n_group_cap,
                            const int32_t *chunk_ids, int32_t group_top_k, int32_t *group_ids,
                            float *scores_or_null, hipStream_t stream);

/*
 * hga_attend_fwd_groups -- hga_attend_fwd over routed groups: for query i of
 * block b (first position P, position p),
 *     A(i) = union_{u in group_ids[g][b], 0 <= u < P/8} [8u, 8u + 8)  U  [P, p]
 * with the rest as in hga_attend_fwd (the group row is a set; group_ids
 * [Hkv][n_q/Bq][group_top_k], group_top_k in 0 .. 2048).
 */
hga_status hga_attend_fwd_groups(const hga_config *cfg, const void *Q, const void *K,
                                 const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                 const int32_t *group_ids, int32_t group_top_k, void *O,
                                 float *lse, hipStream_t stream);

/*
 * hga_route_attend_fwd_groups -- both routing levels and the group attention
 * of one segment (gist.science technical summary 2.1: chunks first, then the
 * 8-token groups inside them): the outputs of hga_route (chunk_ids; no chunk
 * scores), hga_route_groups (group_ids, scores_or_null) and
 * hga_attend_fwd_groups (O, lse) on the same inputs, bit for bit. With
 * 0 < cfg->top_k <= 32, group_top_k > 0 and at most 8704 candidate chunks per
 * block it is one launch: each workgroup routes its block at both levels and
 * then attends; otherwise the three kernels run in turn. Per-kv-head routing
 * only (HGA_ERR_UNSUPPORTED otherwise).
 *   summaries, n_chunk_cap, n_chunks_valid   as for hga_route_attend_fwd
 *   group_summaries, n_group_cap, group_top_k as for hga_route_groups
 *   chunk_ids   device int32 [Hkv][n_q/Bq][cfg->top_k], written (needed when
 *               cfg->top_k > 0)
 *   group_ids   device int32 [Hkv][n_q/Bq][group_top_k], written;
 *               group_scores_or_null as hga_route_groups' scores_or_null
 *   Q, K, V, O, lse, T_cap, p0, n_q as for hga_attend_fwd
 */
hga_status hga_route_attend_fwd_groups(const hga_config *cfg, const void *Q, const void *K,
                                       const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                       const float *summaries, int64_t n_chunk_cap,
                                       int64_t n_chunks_valid, const float *group_summaries,
                                       int64_t n_group_cap, int32_t group_top_k,
                                       int32_t *chunk_ids, int32_t *group_ids,
                                       float *group_scores_or_null, void *O, float *lse,
                                       hipStream_t stream);

/*
 * hga_attend_bwd_groups -- hga_attend_bwd for hga_attend_fwd_groups: the same
 * gradients (dQ of every active query; dK, dV of the active keys, summed over
 * the G heads; history detached) with A(i) built from group_ids as in
 * hga_attend_fwd_groups. lse and O are that call's outputs (O may be NULL:
 * it feeds only the dQ kernel's Delta estimate, as in hga_attend_bwd). The workspace is hga_attend_bwd_workspace_bytes(cfg, n_q) bytes, with
 * the same rules as for hga_attend_bwd; results are deterministic.
 */
hga_status hga_attend_bwd_groups(const hga_config *cfg, const void *Q, const void *K,
                                 const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                 const int32_t *group_ids, int32_t group_top_k, const void *O,
                                 const float *lse, const void *dO, float *dQ, float *dK_active,
                                 float *dV_active, void *workspace, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Routed generation (decode): a step of n_q new tokens at positions p0 ..
 * p0+n_q-1, one token at a time (technical summary 2.1 applied per token; the
 * pages note the method also serves generation). Positions need not be
 * multiples of C. Token p's open chunk starts at Pc = C*floor(p/C); the
 * chunks before it are closed, and their summaries must exist (append a
 * chunk's summary with hga_summarize once its last token is in K).
 * ---------------------------------------------------------------------- */

/*
 * hga_route_decode -- hga_route with one-token blocks: for token i (p = p0+i)
 * and kv head g, qbar = mean of Q[h][i] over the G heads of g (fp32),
 * candidates the chunks s <= c < Pc/C (s = cfg->sink_chunks), and
 * ids[g][i][:] the min(k, Pc/C - s) of highest score, ties to the lower id,
 * ascending, then -1.
 *   Q        device bf16 [Hq][n_q][D]; at most 65535 tokens per call
 *            (HGA_ERR_UNSUPPORTED)
 *   ids      device int32 [Hkv][n_q][k];  scores_or_null as for hga_route
 *   summaries: (p0 + n_q - 1)/C <= n_chunks_valid <= n_chunk_cap, else
 *            HGA_ERR_CAPACITY
 *   workspace  device scratch (the candidates' scores), at least
 *            hga_decode_workspace_bytes(cfg, p0, n_q) bytes, else
 *            HGA_ERR_CAPACITY; owned by the caller, contents on entry
 *            ignored and on return unspecified; calls that share it must not
 *            overlap in time (the same buffer may serve hga_attend_decode).
 */
hga_status hga_route_decode(const hga_config *cfg, const void *Q, int64_t p0, int64_t n_q,
                            const float *summaries, int64_t n_chunk_cap, int64_t n_chunks_valid,
                            int32_t *ids, float *scores_or_null, void *workspace,
                            size_t ws_bytes, hipStream_t stream);

/* Device workspace that hga_route_decode and hga_attend_decode need for a
 * step of n_q tokens at p0 (one size serves both; 0 on bad arguments). */
size_t hga_decode_workspace_bytes(const hga_config *cfg, int64_t p0, int64_t n_q);

/*
 * hga_attend_decode -- exact attention of the step's tokens: token p attends
 *     A(p) = [0, min(sC, Pc))  U  union_{c in ids[g][i], s <= c < Pc/C} [cC, cC+C)
 *            U  [Pc, p]
 * with O and lse as in hga_attend_fwd (ids rows are sets; entries outside the
 * range add nothing). The K/V of the step's own tokens must already be in K
 * and V.
 *   Q, O   device bf16 [Hq][n_q][D];  K, V device bf16 [Hkv][T_cap][D]
 *   ids    device int32 [Hkv][n_q][k];  lse device f32 [Hq][n_q]
 *   p0 + n_q <= T_cap, else HGA_ERR_INVALID_ARG
 *   workspace  device scratch (the per-split partial results), at least
 *            hga_decode_workspace_bytes(cfg, p0, n_q) bytes, else
 *            HGA_ERR_CAPACITY; owned by the caller, contents on entry ignored;
 *            calls that share it must not overlap in time.
 */
hga_status hga_attend_decode(const hga_config *cfg, const void *Q, const void *K, const void *V,
                             int64_t T_cap, int64_t p0, int64_t n_q, const int32_t *ids, void *O,
                             float *lse, void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * hga_route_attend_decode -- hga_route_decode followed by hga_attend_decode in
 * one call (three launches instead of four): ids, scores_or_null, O and lse
 * are written exactly as those two calls write them, bit for bit. The routing
 * keeps, per block of 256 candidates, that block's top k; every attention
 * split then selects the top k among those survivors itself, and the splits'
 * partials are merged as hga_attend_decode merges them.
 *   Arguments as for hga_route_decode and hga_attend_decode; ids may be NULL
 *   only when top_k == 0 (then summaries is not read either).
 *   workspace  device scratch of at least
 *            hga_route_attend_decode_workspace_bytes(cfg, p0, n_q) bytes, else
 *            HGA_ERR_CAPACITY; owned by the caller, contents on entry
 *            ignored; calls that share it must not overlap in time.
 *   HGA_ERR_UNSUPPORTED when the blocks' survivors (256-candidate blocks of
 *   the last token times top_k) exceed 12288; the two separate calls take
 *   those sizes.
 */
size_t hga_route_attend_decode_workspace_bytes(const hga_config *cfg, int64_t p0, int64_t n_q);
hga_status hga_route_attend_decode(const hga_config *cfg, const void *Q, const void *K,
                                   const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                   const float *summaries, int64_t n_chunk_cap,
                                   int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                                   void *O, float *lse, void *workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Diagnostic (not a step of the method).
 * ---------------------------------------------------------------------- */

/*
 * hga_diag_gather -- reads exactly the K and V rows hga_attend_fwd gathers for
 * the same arguments (each block's valid routed chunks, repeats once, and its
 * local block), with the attention kernel's addressing, and does nothing else
 * but fold them into sink (one word per thread, contents meaningless): its
 * time is the ceiling the gather alone puts on hga_attend_fwd.
 *   sink   device memory of at least hga_diag_gather_sink_words(cfg, n_q)
 *          32-bit words, else HGA_ERR_CAPACITY; other arguments and errors as
 *          for hga_attend_fwd.
 */
size_t hga_diag_gather_sink_words(const hga_config *cfg, int64_t n_q);
hga_status hga_diag_gather(const hga_config *cfg, const void *K, const void *V, int64_t T_cap,
                           int64_t p0, int64_t n_q, const int32_t *ids, uint32_t *sink,
                           size_t sink_words, hipStream_t stream);

/*
 * hga_diag_bwd_second_pass -- how many dq workgroups of the last
 * hga_attend_bwd or hga_attend_bwd_groups call on this workspace (same cfg and
 * n_q) took the second pass over their tiles, which recomputes dQ with the
 * exact Delta where the estimate from O was not close enough (or O was NULL).
 * Waits for the stream; writes *n_second and *n_workgroups (the call's dq
 * workgroups). Other arguments and errors as for hga_attend_bwd.
 */
hga_status hga_diag_bwd_second_pass(const hga_config *cfg, int64_t n_q, const void *workspace,
                                    size_t ws_bytes, int64_t *n_second, int64_t *n_workgroups,
                                    hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *hga_status_string(hga_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char *hga_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t hga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */

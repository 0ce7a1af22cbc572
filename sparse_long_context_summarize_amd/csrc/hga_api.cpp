// hga_api.cpp -- the C ABI of libhga: argument checks, status codes and
// kernel dispatch on the caller's stream. See include/hga.h for the contract
// of each call. No call allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "hga_internal.h"

// The workspace of hga_attend_bwd_noalloc: one file-scope device array, one
// copy on every GPU the library runs on, held until the process ends. Host
// code never passes this name to a kernel (on the host it is only a stand-in
// for the symbol): it uses the device address that hipGetSymbolAddress
// returns for the current device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[HGA_BWD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

hga_status fail(hga_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

hga_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return HGA_OK;
    return fail(HGA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Largest number of eligible chunks one route workgroup can rank (its keys sit
// in LDS next to ~22 KiB of fixed state).
constexpr int64_t kMaxEligible = 24576;

hga_status check_config(const hga_config *cfg)
{
    if (!cfg) return fail(HGA_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->n_q_heads <= 0 || cfg->n_kv_heads <= 0)
        return fail(HGA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)",
                    cfg->n_q_heads, cfg->n_kv_heads);
    if (cfg->n_kv_heads > 65535)
        return fail(HGA_ERR_UNSUPPORTED, "n_kv_heads must be at most 65535 (got %d)",
                    cfg->n_kv_heads);
    if (cfg->n_q_heads % cfg->n_kv_heads != 0)
        return fail(HGA_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                    cfg->n_q_heads, cfg->n_kv_heads);
    const int G = cfg->n_q_heads / cfg->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(HGA_ERR_UNSUPPORTED, "query heads per kv head must be 1, 2, 4 or 8 (got %d)", G);
    if (cfg->head_dim != hga::kD)
        return fail(HGA_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", hga::kD, cfg->head_dim);
    if (cfg->chunk != hga::kC)
        return fail(HGA_ERR_UNSUPPORTED, "chunk must be %d (got %d)", hga::kC, cfg->chunk);
    if (cfg->q_block != cfg->chunk)
        return fail(HGA_ERR_UNSUPPORTED, "q_block (%d) must equal chunk (%d)", cfg->q_block,
                    cfg->chunk);
    if (cfg->top_k < 0 || cfg->top_k > hga::kMaxTopK)
        return fail(HGA_ERR_INVALID_ARG, "top_k must be in [0, %d] (got %d)", hga::kMaxTopK,
                    cfg->top_k);
    if (cfg->dtype != HGA_BF16)
        return fail(HGA_ERR_UNSUPPORTED, "dtype must be HGA_BF16 (got %d)", cfg->dtype);
    if (isnan(cfg->softmax_scale) || isinf(cfg->softmax_scale))
        return fail(HGA_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (cfg->sink_chunks < 0)
        return fail(HGA_ERR_INVALID_ARG, "sink_chunks must be >= 0 (got %d)", cfg->sink_chunks);
    if (cfg->sink_chunks > HGA_MAX_SINK_CHUNKS)
        return fail(HGA_ERR_UNSUPPORTED, "sink_chunks must be at most %d (got %d)",
                    HGA_MAX_SINK_CHUNKS, cfg->sink_chunks);
    if (cfg->route_heads != HGA_ROUTE_PER_KV_HEAD && cfg->route_heads != HGA_ROUTE_PER_Q_HEAD)
        return fail(HGA_ERR_INVALID_ARG, "route_heads must be HGA_ROUTE_PER_KV_HEAD or "
                    "HGA_ROUTE_PER_Q_HEAD (got %d)", cfg->route_heads);
    return HGA_OK;
}

// The entry points that only know one id row per kv head.
hga_status check_kv_head_routing(const hga_config *cfg, const char *what)
{
    if (cfg->route_heads != HGA_ROUTE_PER_KV_HEAD)
        return fail(HGA_ERR_UNSUPPORTED, "%s supports route_heads = HGA_ROUTE_PER_KV_HEAD only",
                    what);
    return HGA_OK;
}

bool per_q_head(const hga_config *cfg) { return cfg->route_heads == HGA_ROUTE_PER_Q_HEAD; }

float effective_scale(const hga_config *cfg)
{
    return cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf((float)cfg->head_dim);
}

// p0 / n_q / T_cap checks shared by route, fwd and bwd.
hga_status check_segment(int64_t p0, int64_t n_q, int64_t T_cap, bool need_T)
{
    if (p0 < 0 || n_q < 0) return fail(HGA_ERR_INVALID_ARG, "p0 (%lld) and n_q (%lld) must be >= 0",
                                       (long long)p0, (long long)n_q);
    if (p0 % hga::kC != 0)
        return fail(HGA_ERR_INVALID_ARG, "p0 (%lld) is not a multiple of the chunk length %d",
                    (long long)p0, hga::kC);
    if (n_q % hga::kC != 0)
        return fail(HGA_ERR_INVALID_ARG, "n_q (%lld) is not a multiple of the query block %d",
                    (long long)n_q, hga::kC);
    if (need_T && p0 + n_q > T_cap)
        return fail(HGA_ERR_INVALID_ARG, "p0 + n_q (%lld) exceeds T_cap (%lld)",
                    (long long)(p0 + n_q), (long long)T_cap);
    if (n_q / hga::kC > 65535)      // one launch's grid holds the query blocks
        return fail(HGA_ERR_UNSUPPORTED, "n_q (%lld) exceeds 65535 query blocks of %d",
                    (long long)n_q, hga::kC);
    return HGA_OK;
}

// hga_attend_bwd's checks and launch, on a given workspace.
hga_status attend_bwd_checked(const hga_config *cfg, const void *Q, const void *K,
                              const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                              const int32_t *ids, const void *O, const float *lse,
                              const void *dO, float *dQ, float *dK_active, float *dV_active,
                              void *workspace, size_t ws_bytes, hipStream_t stream,
                              const char *what)
{
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (n_q == 0) return HGA_OK;
    if (n_q > hga::bwd_max_queries())
        return fail(HGA_ERR_UNSUPPORTED, "backward supports at most %lld active queries",
                    (long long)hga::bwd_max_queries());
    if (!Q || !K || !V || !lse || !dO || !dQ || !dK_active || !dV_active ||
        (cfg->top_k > 0 && !ids))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    const size_t need = hga::bwd_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, n_q,
                                                 per_q_head(cfg));
    if (need > 0 && !workspace) return fail(HGA_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < need)
        return fail(HGA_ERR_CAPACITY, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
    return hip_status(hga::launch_attend_bwd((const uint16_t *)Q, (const uint16_t *)K,
                                             (const uint16_t *)V, cfg->n_q_heads,
                                             cfg->n_kv_heads, T_cap, p0, n_q, ids, cfg->top_k,
                                             cfg->sink_chunks, per_q_head(cfg),
                                             effective_scale(cfg), (const uint16_t *)O, lse,
                                             (const uint16_t *)dO, dQ, dK_active, dV_active,
                                             workspace, stream),
                      what);
}

// Device address of `scratch` on the device of `stream`, looked up once per
// device (with that device current) and kept. The stream's device must be
// the current one.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices];

hga_status scratch_address(hipStream_t stream, void **out)
{
    int dev = -1, sdev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
        return fail(HGA_ERR_INVALID_ARG, "the stream belongs to device %d, the current device is %d",
                    sdev, dev);
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(HGA_ERR_UNSUPPORTED, "device %d: the scratch table covers devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(HGA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return HGA_OK;
}

}  // namespace

extern "C" {

const char *hga_status_string(hga_status s)
{
    switch (s) {
    case HGA_OK: return "HGA_OK";
    case HGA_ERR_INVALID_ARG: return "HGA_ERR_INVALID_ARG";
    case HGA_ERR_UNSUPPORTED: return "HGA_ERR_UNSUPPORTED";
    case HGA_ERR_CAPACITY: return "HGA_ERR_CAPACITY";
    case HGA_ERR_HIP: return "HGA_ERR_HIP";
    }
    return "HGA_ERR_UNKNOWN";
}

const char *hga_last_error(void) { return g_last_error; }

int32_t hga_version(void) { return 10000; }   // 1.0.0

hga_status hga_summarize(const hga_config *cfg, const void *K, int64_t T_cap,
                         int64_t tok_begin, int64_t n_tok, float *summaries,
                         int64_t n_chunk_cap, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    if (tok_begin < 0 || n_tok < 0 || T_cap < 0 || n_chunk_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative size or position");
    if (tok_begin % hga::kC != 0 || n_tok % hga::kC != 0)
        return fail(HGA_ERR_INVALID_ARG, "tok_begin (%lld) and n_tok (%lld) must be multiples of %d",
                    (long long)tok_begin, (long long)n_tok, hga::kC);
    if (tok_begin + n_tok > T_cap)
        return fail(HGA_ERR_INVALID_ARG, "tok_begin + n_tok (%lld) exceeds T_cap (%lld)",
                    (long long)(tok_begin + n_tok), (long long)T_cap);
    const int64_t c_begin = tok_begin / hga::kC, c_end = (tok_begin + n_tok) / hga::kC;
    if (c_end > n_chunk_cap)
        return fail(HGA_ERR_CAPACITY, "summary buffer holds %lld chunks, %lld needed",
                    (long long)n_chunk_cap, (long long)c_end);
    if (n_tok == 0) return HGA_OK;
    if (!K || !summaries) return fail(HGA_ERR_INVALID_ARG, "K or summaries is NULL");
    return hip_status(hga::launch_summarize((const uint16_t *)K, cfg->n_kv_heads, T_cap, c_begin,
                                            c_end, summaries, n_chunk_cap, stream),
                      "hga_summarize launch");
}

static hga_status route_common(const hga_config *cfg, const void *Q, const void *Q_prev,
                               bool prev_block, int64_t p0, int64_t n_q,
                               const float *summaries, int64_t n_chunk_cap,
                               int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                               hipStream_t stream, const char *what)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, 0, false);
    if (st != HGA_OK) return st;
    if (n_chunks_valid < 0 || n_chunk_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative chunk count");
    if (n_chunks_valid > n_chunk_cap)
        return fail(HGA_ERR_CAPACITY, "n_chunks_valid (%lld) exceeds n_chunk_cap (%lld)",
                    (long long)n_chunks_valid, (long long)n_chunk_cap);
    if (n_q == 0 || cfg->top_k == 0) return HGA_OK;
    const int64_t need = (p0 + n_q - hga::kC) / hga::kC;   // eligible chunks of the last block
    if (need > n_chunks_valid)
        return fail(HGA_ERR_CAPACITY, "the last query block needs %lld summaries, %lld valid",
                    (long long)need, (long long)n_chunks_valid);
    if (need > kMaxEligible)
        return fail(HGA_ERR_UNSUPPORTED, "more than %lld candidate chunks per block",
                    (long long)kMaxEligible);
    if (!Q || !ids || (need > 0 && !summaries))
        return fail(HGA_ERR_INVALID_ARG, "Q, summaries or ids is NULL");
    if (prev_block && p0 > 0 && !Q_prev)
        return fail(HGA_ERR_INVALID_ARG, "Q_prev is NULL with p0 = %lld > 0", (long long)p0);
    return hip_status(hga::launch_route((const uint16_t *)Q, cfg->n_q_heads, cfg->n_kv_heads, p0,
                                        n_q, summaries, n_chunk_cap, cfg->top_k,
                                        cfg->sink_chunks, per_q_head(cfg), prev_block,
                                        (const uint16_t *)Q_prev, ids, scores_or_null, stream),
                      what);
}

hga_status hga_route(const hga_config *cfg, const void *Q, int64_t p0, int64_t n_q,
                     const float *summaries, int64_t n_chunk_cap,
                     int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                     hipStream_t stream)
{
    return route_common(cfg, Q, nullptr, false, p0, n_q, summaries, n_chunk_cap,
                        n_chunks_valid, ids, scores_or_null, stream, "hga_route launch");
}

hga_status hga_route_causal(const hga_config *cfg, const void *Q, const void *Q_prev,
                            int64_t p0, int64_t n_q, const float *summaries,
                            int64_t n_chunk_cap, int64_t n_chunks_valid, int32_t *ids,
                            float *scores_or_null, hipStream_t stream)
{
    return route_common(cfg, Q, p0 > 0 ? Q_prev : nullptr, true, p0, n_q, summaries,
                        n_chunk_cap, n_chunks_valid, ids, scores_or_null, stream,
                        "hga_route_causal launch");
}

hga_status hga_attend_fwd(const hga_config *cfg, const void *Q, const void *K, const void *V,
                          int64_t T_cap, int64_t p0, int64_t n_q, const int32_t *ids, void *O,
                          float *lse, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (n_q == 0) return HGA_OK;
    if (!Q || !K || !V || !O || !lse || (cfg->top_k > 0 && !ids))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    return hip_status(hga::launch_attend_fwd((const uint16_t *)Q, (const uint16_t *)K,
                                             (const uint16_t *)V, cfg->n_q_heads,
                                             cfg->n_kv_heads, T_cap, p0, n_q, ids, cfg->top_k,
                                             cfg->sink_chunks, per_q_head(cfg),
                                             effective_scale(cfg), (uint16_t *)O, lse, stream),
                      "hga_attend_fwd launch");
}

hga_status hga_route_attend_fwd(const hga_config *cfg, const void *Q, const void *K,
                                const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                const float *summaries, int64_t n_chunk_cap,
                                int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                                void *O, float *lse, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (n_chunks_valid < 0 || n_chunk_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative chunk count");
    if (n_chunks_valid > n_chunk_cap)
        return fail(HGA_ERR_CAPACITY, "n_chunks_valid (%lld) exceeds n_chunk_cap (%lld)",
                    (long long)n_chunks_valid, (long long)n_chunk_cap);
    if (n_q == 0) return HGA_OK;
    const int64_t need = (p0 + n_q - hga::kC) / hga::kC;   // eligible chunks of the last block
    if (cfg->top_k > 0) {
        if (need > n_chunks_valid)
            return fail(HGA_ERR_CAPACITY, "the last query block needs %lld summaries, %lld valid",
                        (long long)need, (long long)n_chunks_valid);
        if (need > kMaxEligible)
            return fail(HGA_ERR_UNSUPPORTED, "more than %lld candidate chunks per block",
                        (long long)kMaxEligible);
    }
    if (!Q || !K || !V || !O || !lse || (cfg->top_k > 0 && (!ids || (need > 0 && !summaries))))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    const float scale = effective_scale(cfg);
    if (cfg->top_k > 0 && need - cfg->sink_chunks > hga::route_attend_max_candidates()) {
        // more candidates than the fused kernel keeps in LDS: the routing
        // kernel, then the attention kernel (the same ids, scores and outputs)
        st = hip_status(hga::launch_route((const uint16_t *)Q, cfg->n_q_heads, cfg->n_kv_heads,
                                          p0, n_q, summaries, n_chunk_cap, cfg->top_k,
                                          cfg->sink_chunks, per_q_head(cfg), false, nullptr,
                                          ids, scores_or_null, stream),
                        "hga_route_attend_fwd route launch");
        if (st != HGA_OK) return st;
        return hip_status(hga::launch_attend_fwd((const uint16_t *)Q, (const uint16_t *)K,
                                                 (const uint16_t *)V, cfg->n_q_heads,
                                                 cfg->n_kv_heads, T_cap, p0, n_q, ids,
                                                 cfg->top_k, cfg->sink_chunks, per_q_head(cfg),
                                                 scale, (uint16_t *)O, lse, stream),
                          "hga_route_attend_fwd attend launch");
    }
    return hip_status(hga::launch_route_attend_fwd((const uint16_t *)Q, (const uint16_t *)K,
                                                   (const uint16_t *)V, cfg->n_q_heads,
                                                   cfg->n_kv_heads, T_cap, p0, n_q, summaries,
                                                   n_chunk_cap, cfg->top_k, cfg->sink_chunks,
                                                   per_q_head(cfg), scale, ids, scores_or_null,
                                                   (uint16_t *)O, lse, stream),
                      "hga_route_attend_fwd launch");
}

hga_status hga_summarize_groups(const hga_config *cfg, const void *K, int64_t T_cap,
                                int64_t tok_begin, int64_t n_tok, float *group_summaries,
                                int64_t n_group_cap, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    if (tok_begin < 0 || n_tok < 0 || T_cap < 0 || n_group_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative size or position");
    if (tok_begin % hga::kC != 0 || n_tok % hga::kC != 0)
        return fail(HGA_ERR_INVALID_ARG, "tok_begin (%lld) and n_tok (%lld) must be multiples of %d",
                    (long long)tok_begin, (long long)n_tok, hga::kC);
    if (tok_begin + n_tok > T_cap)
        return fail(HGA_ERR_INVALID_ARG, "tok_begin + n_tok (%lld) exceeds T_cap (%lld)",
                    (long long)(tok_begin + n_tok), (long long)T_cap);
    const int64_t c_begin = tok_begin / hga::kC, c_end = (tok_begin + n_tok) / hga::kC;
    if ((tok_begin + n_tok) / hga::kGroup > n_group_cap)
        return fail(HGA_ERR_CAPACITY, "group summary buffer holds %lld groups, %lld needed",
                    (long long)n_group_cap, (long long)((tok_begin + n_tok) / hga::kGroup));
    if (n_tok == 0) return HGA_OK;
    if (!K || !group_summaries) return fail(HGA_ERR_INVALID_ARG, "K or group_summaries is NULL");
    return hip_status(hga::launch_summarize_groups((const uint16_t *)K, cfg->n_kv_heads, T_cap,
                                                   c_begin, c_end, group_summaries, n_group_cap,
                                                   stream),
                      "hga_summarize_groups launch");
}

hga_status hga_route_groups(const hga_config *cfg, const void *Q, int64_t p0, int64_t n_q,
                            const float *group_summaries, int64_t n_group_cap,
                            const int32_t *chunk_ids, int32_t group_top_k, int32_t *group_ids,
                            float *scores_or_null, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_route_groups");
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, 0, false);
    if (st != HGA_OK) return st;
    if (group_top_k < 0 || group_top_k > hga::kMaxGroupTopK)
        return fail(HGA_ERR_INVALID_ARG, "group_top_k must be in [0, %d] (got %d)",
                    hga::kMaxGroupTopK, group_top_k);
    if (n_group_cap < 0) return fail(HGA_ERR_INVALID_ARG, "negative group count");
    if (n_q == 0 || group_top_k == 0) return HGA_OK;
    // every group of a chunk a block may route to (c < P/C) must be in the buffer
    const int64_t need = ((p0 + n_q - hga::kC) / hga::kC) * (hga::kC / hga::kGroup);
    if (cfg->top_k > 0 && need > n_group_cap)
        return fail(HGA_ERR_CAPACITY, "the last query block may route to %lld groups, the buffer holds %lld",
                    (long long)need, (long long)n_group_cap);
    if (!Q || !group_ids || (cfg->top_k > 0 && (!chunk_ids || !group_summaries)))
        return fail(HGA_ERR_INVALID_ARG, "Q, chunk_ids, group_summaries or group_ids is NULL");
    return hip_status(hga::launch_route_groups((const uint16_t *)Q, cfg->n_q_heads,
                                               cfg->n_kv_heads, p0, n_q, group_summaries,
                                               n_group_cap, chunk_ids, cfg->top_k, group_top_k,
                                               cfg->sink_chunks, group_ids, scores_or_null,
                                               stream),
                      "hga_route_groups launch");
}

hga_status hga_attend_fwd_groups(const hga_config *cfg, const void *Q, const void *K,
                                 const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                 const int32_t *group_ids, int32_t group_top_k, void *O,
                                 float *lse, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_attend_fwd_groups");
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (group_top_k < 0 || group_top_k > hga::kMaxGroupTopK)
        return fail(HGA_ERR_INVALID_ARG, "group_top_k must be in [0, %d] (got %d)",
                    hga::kMaxGroupTopK, group_top_k);
    if (n_q == 0) return HGA_OK;
    if (!Q || !K || !V || !O || !lse || (group_top_k > 0 && !group_ids))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    return hip_status(hga::launch_attend_fwd_groups((const uint16_t *)Q, (const uint16_t *)K,
                                                    (const uint16_t *)V, cfg->n_q_heads,
                                                    cfg->n_kv_heads, T_cap, p0, n_q, group_ids,
                                                    group_top_k, cfg->sink_chunks,
                                                    effective_scale(cfg), (uint16_t *)O, lse,
                                                    stream),
                      "hga_attend_fwd_groups launch");
}

hga_status hga_route_attend_fwd_groups(const hga_config *cfg, const void *Q, const void *K,
                                       const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                       const float *summaries, int64_t n_chunk_cap,
                                       int64_t n_chunks_valid, const float *group_summaries,
                                       int64_t n_group_cap, int32_t group_top_k,
                                       int32_t *chunk_ids, int32_t *group_ids,
                                       float *group_scores_or_null, void *O, float *lse,
                                       hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_route_attend_fwd_groups");
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (group_top_k < 0 || group_top_k > hga::kMaxGroupTopK)
        return fail(HGA_ERR_INVALID_ARG, "group_top_k must be in [0, %d] (got %d)",
                    hga::kMaxGroupTopK, group_top_k);
    if (n_chunks_valid < 0 || n_chunk_cap < 0 || n_group_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative chunk or group count");
    if (n_chunks_valid > n_chunk_cap)
        return fail(HGA_ERR_CAPACITY, "n_chunks_valid (%lld) exceeds n_chunk_cap (%lld)",
                    (long long)n_chunks_valid, (long long)n_chunk_cap);
    if (n_q == 0) return HGA_OK;
    const int64_t need = (p0 + n_q - hga::kC) / hga::kC;   // eligible chunks of the last block
    if (cfg->top_k > 0) {
        if (need > n_chunks_valid)
            return fail(HGA_ERR_CAPACITY, "the last query block needs %lld summaries, %lld valid",
                        (long long)need, (long long)n_chunks_valid);
        if (need > kMaxEligible)
            return fail(HGA_ERR_UNSUPPORTED, "more than %lld candidate chunks per block",
                        (long long)kMaxEligible);
        if (group_top_k > 0 && need * (hga::kC / hga::kGroup) > n_group_cap)
            return fail(HGA_ERR_CAPACITY,
                        "the last query block may route to %lld groups, the buffer holds %lld",
                        (long long)(need * (hga::kC / hga::kGroup)), (long long)n_group_cap);
    }
    if (!Q || !K || !V || !O || !lse || (group_top_k > 0 && !group_ids) ||
        (cfg->top_k > 0 && (!chunk_ids || (need > 0 && !summaries) ||
                            (group_top_k > 0 && need > 0 && !group_summaries))))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    const float scale = effective_scale(cfg);
    const bool fused = cfg->top_k > 0 && cfg->top_k <= hga::kFusedGroupChunks &&
                       group_top_k > 0 &&
                       need - cfg->sink_chunks <= hga::route_attend_max_candidates();
    if (fused)
        return hip_status(hga::launch_route_attend_fwd_groups(
                              (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                              cfg->n_q_heads, cfg->n_kv_heads, T_cap, p0, n_q, summaries,
                              n_chunk_cap, cfg->top_k, group_summaries, n_group_cap,
                              group_top_k, cfg->sink_chunks, scale, chunk_ids, group_ids,
                              group_scores_or_null, (uint16_t *)O, lse, stream),
                          "hga_route_attend_fwd_groups launch");
    // otherwise the three kernels in turn, as hga_route, hga_route_groups and
    // hga_attend_fwd_groups run them
    if (cfg->top_k > 0) {
        st = hip_status(hga::launch_route((const uint16_t *)Q, cfg->n_q_heads, cfg->n_kv_heads,
                                          p0, n_q, summaries, n_chunk_cap, cfg->top_k,
                                          cfg->sink_chunks, false, false, nullptr, chunk_ids,
                                          nullptr, stream),
                        "hga_route_attend_fwd_groups route launch");
        if (st != HGA_OK) return st;
    }
    if (group_top_k > 0) {
        st = hip_status(hga::launch_route_groups((const uint16_t *)Q, cfg->n_q_heads,
                                                 cfg->n_kv_heads, p0, n_q, group_summaries,
                                                 n_group_cap, chunk_ids, cfg->top_k, group_top_k,
                                                 cfg->sink_chunks, group_ids,
                                                 group_scores_or_null, stream),
                        "hga_route_attend_fwd_groups group route launch");
        if (st != HGA_OK) return st;
    }
    return hip_status(hga::launch_attend_fwd_groups((const uint16_t *)Q, (const uint16_t *)K,
                                                    (const uint16_t *)V, cfg->n_q_heads,
                                                    cfg->n_kv_heads, T_cap, p0, n_q, group_ids,
                                                    group_top_k, cfg->sink_chunks, scale,
                                                    (uint16_t *)O, lse, stream),
                      "hga_route_attend_fwd_groups attend launch");
}

hga_status hga_attend_bwd_groups(const hga_config *cfg, const void *Q, const void *K,
                                 const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                 const int32_t *group_ids, int32_t group_top_k, const void *O,
                                 const float *lse, const void *dO, float *dQ, float *dK_active,
                                 float *dV_active, void *workspace, size_t ws_bytes,
                                 hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_attend_bwd_groups");
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (group_top_k < 0 || group_top_k > hga::kMaxGroupTopK)
        return fail(HGA_ERR_INVALID_ARG, "group_top_k must be in [0, %d] (got %d)",
                    hga::kMaxGroupTopK, group_top_k);
    if (n_q == 0) return HGA_OK;
    if (n_q > hga::bwd_max_queries())
        return fail(HGA_ERR_UNSUPPORTED, "backward supports at most %lld active queries",
                    (long long)hga::bwd_max_queries());
    if (!Q || !K || !V || !lse || !dO || !dQ || !dK_active || !dV_active ||
        (group_top_k > 0 && !group_ids))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    const size_t need = hga::bwd_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, n_q, false);
    if (need > 0 && !workspace) return fail(HGA_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < need)
        return fail(HGA_ERR_CAPACITY, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
    (void)O;
    return hip_status(hga::launch_attend_bwd_groups((const uint16_t *)Q, (const uint16_t *)K,
                                                    (const uint16_t *)V, cfg->n_q_heads,
                                                    cfg->n_kv_heads, T_cap, p0, n_q, group_ids,
                                                    group_top_k, cfg->sink_chunks,
                                                    effective_scale(cfg), (const uint16_t *)O, lse,
                                                    (const uint16_t *)dO, dQ, dK_active,
                                                    dV_active, workspace, stream),
                      "hga_attend_bwd_groups launch");
}

hga_status hga_route_decode(const hga_config *cfg, const void *Q, int64_t p0, int64_t n_q,
                            const float *summaries, int64_t n_chunk_cap, int64_t n_chunks_valid,
                            int32_t *ids, float *scores_or_null, void *workspace,
                            size_t ws_bytes, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_route_decode");
    if (st != HGA_OK) return st;
    if (p0 < 0 || n_q < 0 || n_chunks_valid < 0 || n_chunk_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative position, count or capacity");
    if (n_q > 65535)
        return fail(HGA_ERR_UNSUPPORTED, "at most 65535 tokens per call (got %lld)", (long long)n_q);
    if (n_chunks_valid > n_chunk_cap)
        return fail(HGA_ERR_CAPACITY, "n_chunks_valid (%lld) exceeds n_chunk_cap (%lld)",
                    (long long)n_chunks_valid, (long long)n_chunk_cap);
    if (n_q == 0 || cfg->top_k == 0) return HGA_OK;
    // the last token's closed chunks (those before its open chunk)
    const int64_t need = (p0 + n_q - 1) / hga::kC;
    if (need > n_chunks_valid)
        return fail(HGA_ERR_CAPACITY, "the last token needs %lld summaries, %lld valid",
                    (long long)need, (long long)n_chunks_valid);
    if (need - cfg->sink_chunks > kMaxEligible)
        return fail(HGA_ERR_UNSUPPORTED, "more than %lld candidate chunks per token",
                    (long long)kMaxEligible);
    if (!Q || !ids || (need > 0 && !summaries))
        return fail(HGA_ERR_INVALID_ARG, "Q, summaries or ids is NULL");
    const size_t ws_need = hga::decode_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, p0, n_q,
                                                       cfg->top_k, cfg->sink_chunks);
    if (!workspace) return fail(HGA_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < ws_need)
        return fail(HGA_ERR_CAPACITY, "workspace holds %zu bytes, %zu needed", ws_bytes, ws_need);
    return hip_status(hga::launch_route_decode((const uint16_t *)Q, cfg->n_q_heads,
                                               cfg->n_kv_heads, p0, n_q, summaries, n_chunk_cap,
                                               cfg->top_k, cfg->sink_chunks, ids,
                                               scores_or_null, workspace, stream),
                      "hga_route_decode launch");
}

size_t hga_decode_workspace_bytes(const hga_config *cfg, int64_t p0, int64_t n_q)
{
    if (check_config(cfg) != HGA_OK || p0 < 0 || n_q < 0) return 0;
    return hga::decode_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, p0, n_q, cfg->top_k,
                                       cfg->sink_chunks);
}

hga_status hga_attend_decode(const hga_config *cfg, const void *Q, const void *K, const void *V,
                             int64_t T_cap, int64_t p0, int64_t n_q, const int32_t *ids, void *O,
                             float *lse, void *workspace, size_t ws_bytes, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_attend_decode");
    if (st != HGA_OK) return st;
    if (p0 < 0 || n_q < 0 || T_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative position, count or capacity");
    if (n_q > 65535)
        return fail(HGA_ERR_UNSUPPORTED, "at most 65535 tokens per call (got %lld)", (long long)n_q);
    if (p0 + n_q > T_cap)
        return fail(HGA_ERR_INVALID_ARG, "p0 + n_q (%lld) exceeds T_cap (%lld)",
                    (long long)(p0 + n_q), (long long)T_cap);
    if (n_q == 0) return HGA_OK;
    if (!Q || !K || !V || !O || !lse || (cfg->top_k > 0 && !ids))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    const size_t need = hga::decode_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, p0, n_q,
                                                    cfg->top_k, cfg->sink_chunks);
    if (!workspace) return fail(HGA_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < need)
        return fail(HGA_ERR_CAPACITY, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
    return hip_status(hga::launch_attend_decode((const uint16_t *)Q, (const uint16_t *)K,
                                                (const uint16_t *)V, cfg->n_q_heads,
                                                cfg->n_kv_heads, T_cap, p0, n_q, ids,
                                                cfg->top_k, cfg->sink_chunks,
                                                effective_scale(cfg), (uint16_t *)O, lse,
                                                workspace, stream),
                      "hga_attend_decode launch");
}

size_t hga_route_attend_decode_workspace_bytes(const hga_config *cfg, int64_t p0, int64_t n_q)
{
    if (check_config(cfg) != HGA_OK || p0 < 0 || n_q < 0) return 0;
    return hga::route_attend_decode_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, p0, n_q,
                                                    cfg->top_k, cfg->sink_chunks);
}

hga_status hga_route_attend_decode(const hga_config *cfg, const void *Q, const void *K,
                                   const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                   const float *summaries, int64_t n_chunk_cap,
                                   int64_t n_chunks_valid, int32_t *ids, float *scores_or_null,
                                   void *O, float *lse, void *workspace, size_t ws_bytes,
                                   hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_route_attend_decode");
    if (st != HGA_OK) return st;
    if (p0 < 0 || n_q < 0 || T_cap < 0 || n_chunks_valid < 0 || n_chunk_cap < 0)
        return fail(HGA_ERR_INVALID_ARG, "negative position, count or capacity");
    if (n_q > 65535)
        return fail(HGA_ERR_UNSUPPORTED, "at most 65535 tokens per call (got %lld)", (long long)n_q);
    if (p0 + n_q > T_cap)
        return fail(HGA_ERR_INVALID_ARG, "p0 + n_q (%lld) exceeds T_cap (%lld)",
                    (long long)(p0 + n_q), (long long)T_cap);
    if (n_chunks_valid > n_chunk_cap)
        return fail(HGA_ERR_CAPACITY, "n_chunks_valid (%lld) exceeds n_chunk_cap (%lld)",
                    (long long)n_chunks_valid, (long long)n_chunk_cap);
    if (n_q == 0) return HGA_OK;
    const int64_t need = (p0 + n_q - 1) / hga::kC;     // the last token's closed chunks
    if (cfg->top_k > 0 && need > n_chunks_valid)
        return fail(HGA_ERR_CAPACITY, "the last token needs %lld summaries, %lld valid",
                    (long long)need, (long long)n_chunks_valid);
    if (need - cfg->sink_chunks > kMaxEligible)
        return fail(HGA_ERR_UNSUPPORTED, "more than %lld candidate chunks per token",
                    (long long)kMaxEligible);
    if (!hga::route_attend_decode_fits(cfg->n_q_heads, cfg->n_kv_heads, p0, n_q, cfg->top_k,
                                       cfg->sink_chunks))
        return fail(HGA_ERR_UNSUPPORTED,
                    "top_k %d over %lld candidate chunks leaves more block survivors than "
                    "this call selects among; use hga_route_decode + hga_attend_decode",
                    cfg->top_k, (long long)(need - cfg->sink_chunks));
    if (!Q || !K || !V || !O || !lse || (cfg->top_k > 0 && (!ids || (need > 0 && !summaries))))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    const size_t ws_need = hga::route_attend_decode_workspace_bytes(
        cfg->n_q_heads, cfg->n_kv_heads, p0, n_q, cfg->top_k, cfg->sink_chunks);
    if (!workspace) return fail(HGA_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < ws_need)
        return fail(HGA_ERR_CAPACITY, "workspace holds %zu bytes, %zu needed", ws_bytes, ws_need);
    return hip_status(hga::launch_route_attend_decode(
                          (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                          cfg->n_q_heads, cfg->n_kv_heads, T_cap, p0, n_q, summaries,
                          n_chunk_cap, cfg->top_k, cfg->sink_chunks, effective_scale(cfg), ids,
                          scores_or_null, (uint16_t *)O, lse, workspace, stream),
                      "hga_route_attend_decode launch");
}

size_t hga_diag_gather_sink_words(const hga_config *cfg, int64_t n_q)
{
    if (check_config(cfg) != HGA_OK || n_q < 0 || n_q % hga::kC != 0) return 0;
    return hga::gather_sink_words(cfg->n_kv_heads, n_q);
}

hga_status hga_diag_gather(const hga_config *cfg, const void *K, const void *V, int64_t T_cap,
                           int64_t p0, int64_t n_q, const int32_t *ids, uint32_t *sink,
                           size_t sink_words, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_kv_head_routing(cfg, "hga_diag_gather");
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (n_q == 0) return HGA_OK;
    if (!K || !V || !sink || (cfg->top_k > 0 && !ids))
        return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    if (sink_words < hga::gather_sink_words(cfg->n_kv_heads, n_q))
        return fail(HGA_ERR_CAPACITY, "sink holds %zu words, %zu needed", sink_words,
                    hga::gather_sink_words(cfg->n_kv_heads, n_q));
    return hip_status(hga::launch_gather((const uint16_t *)K, (const uint16_t *)V,
                                         cfg->n_kv_heads, T_cap, p0, n_q, ids, cfg->top_k,
                                         cfg->sink_chunks, sink, stream),
                      "hga_diag_gather launch");
}

hga_status hga_diag_bwd_second_pass(const hga_config *cfg, int64_t n_q, const void *workspace,
                                    size_t ws_bytes, int64_t *n_second, int64_t *n_workgroups,
                                    hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    if (n_q < 0 || n_q % hga::kC != 0)
        return fail(HGA_ERR_INVALID_ARG, "n_q = %lld is not a multiple of %d", (long long)n_q,
                    hga::kC);
    if (!n_second || !n_workgroups) return fail(HGA_ERR_INVALID_ARG, "a required pointer is NULL");
    *n_second = 0;
    *n_workgroups = 0;
    if (n_q == 0) return HGA_OK;
    if (!workspace) return fail(HGA_ERR_INVALID_ARG, "workspace is NULL");
    const size_t need = hga::bwd_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, n_q,
                                                 per_q_head(cfg));
    if (ws_bytes < need)
        return fail(HGA_ERR_CAPACITY, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
    return hip_status(hga::bwd_second_pass_count(cfg->n_q_heads, cfg->n_kv_heads, n_q,
                                                 per_q_head(cfg), workspace, n_second,
                                                 n_workgroups, stream),
                      "hga_diag_bwd_second_pass copy");
}

size_t hga_attend_bwd_workspace_bytes(const hga_config *cfg, int64_t n_q)
{
    if (check_config(cfg) != HGA_OK || n_q < 0 || n_q % hga::kC != 0) return 0;
    return hga::bwd_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, n_q, per_q_head(cfg));
}

hga_status hga_attend_bwd(const hga_config *cfg, const void *Q, const void *K, const void *V,
                          int64_t T_cap, int64_t p0, int64_t n_q, const int32_t *ids,
                          const void *O, const float *lse, const void *dO, float *dQ,
                          float *dK_active, float *dV_active, void *workspace, size_t ws_bytes,
                          hipStream_t stream)
{
    g_last_error[0] = '\0';
    return attend_bwd_checked(cfg, Q, K, V, T_cap, p0, n_q, ids, O, lse, dO, dQ, dK_active,
                              dV_active, workspace, ws_bytes, stream, "hga_attend_bwd launch");
}

hga_status hga_attend_bwd_noalloc(const hga_config *cfg, const void *Q, const void *K,
                                  const void *V, int64_t T_cap, int64_t p0, int64_t n_q,
                                  const int32_t *ids, const void *O, const float *lse,
                                  const void *dO, float *dQ, float *dK_active,
                                  float *dV_active, hipStream_t stream)
{
    g_last_error[0] = '\0';
    hga_status st = check_config(cfg);
    if (st != HGA_OK) return st;
    st = check_segment(p0, n_q, T_cap, true);
    if (st != HGA_OK) return st;
    if (n_q == 0) return HGA_OK;
    const size_t need = hga::bwd_workspace_bytes(cfg->n_q_heads, cfg->n_kv_heads, n_q,
                                                 per_q_head(cfg));
    if (need > (size_t)HGA_BWD_NOALLOC_SCRATCH_BYTES)
        return fail(HGA_ERR_CAPACITY,
                    "hga_attend_bwd_noalloc: this call needs %zu bytes of workspace, the "
                    "library's fixed scratch holds %zu (use hga_attend_bwd with a caller "
                    "workspace)", need, (size_t)HGA_BWD_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    st = scratch_address(stream, &ws);
    if (st != HGA_OK) return st;
    return attend_bwd_checked(cfg, Q, K, V, T_cap, p0, n_q, ids, O, lse, dO, dQ, dK_active,
                              dV_active, ws, (size_t)HGA_BWD_NOALLOC_SCRATCH_BYTES, stream,
                              "hga_attend_bwd_noalloc launch");
}

}  // extern "C"

// C ABI of the LSH-attention forward (declared in include/lsh_attention.h).
// Every entry point validates its arguments on the host before any HIP call
// and launches its kernels on the caller's stream without synchronising it.
#include "lsh_attention.h"
#include "lsh_internal.h"

#include <cmath>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error = "no error";

lsh_status fail(lsh_status s, const char* what)
{
    g_last_error = what;
    return s;
}

constexpr long long kMaxBytes = 1LL << 62;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lsh_status check_ptr(const void* p, const char* name)
{
    if (p == nullptr) {
        g_last_error = std::string(name) + " is null";
        return LSH_ERR_INVALID_ARG;
    }
    if (!aligned16(p)) {
        g_last_error = std::string(name) + " is not 16-byte aligned";
        return LSH_ERR_INVALID_ARG;
    }
    return LSH_OK;
}

// Product of positive factors, or -1 if it exceeds kMaxBytes.
long long checked_product(std::initializer_list<long long> f)
{
    long long x = 1;
    for (long long v : f) {
        if (v <= 0) return -1;
        if (x > kMaxBytes / v) return -1;
        x *= v;
    }
    return x;
}

lsh_status check_config(const lsh_config* c)
{
    if (c == nullptr) return fail(LSH_ERR_INVALID_ARG, "config is null");
    if (c->batch <= 0 || c->heads <= 0 || c->seq_len <= 0 || c->d_head <= 0 ||
        c->n_buckets <= 0 || c->n_rounds <= 0 || c->chunk <= 0)
        return fail(LSH_ERR_INVALID_ARG, "every size must be positive");
    if (c->n_buckets % 2) return fail(LSH_ERR_INVALID_ARG, "n_buckets must be even");
    if (c->seq_len % c->chunk) return fail(LSH_ERR_INVALID_ARG, "chunk must divide seq_len");
    if (c->seq_len / c->chunk > 32767)
        return fail(LSH_ERR_INVALID_ARG, "seq_len / chunk must be at most 32767 (int16 chunk ids)");
    if (c->seq_len > (1 << 30)) return fail(LSH_ERR_INVALID_ARG, "seq_len must be at most 2^30");
    if (!std::isfinite(c->scale)) return fail(LSH_ERR_INVALID_ARG, "scale must be finite");
    if (c->causal != 0 && c->causal != 1) return fail(LSH_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (c->d_head != 64 && c->d_head != 128)
        return fail(LSH_ERR_UNSUPPORTED, "d_head must be 64 or 128");
    if (c->dtype != LSH_F32 && c->dtype != LSH_BF16)
        return fail(LSH_ERR_UNSUPPORTED, "dtype must be LSH_F32 or LSH_BF16");
    if (c->n_buckets > 32768) return fail(LSH_ERR_UNSUPPORTED, "n_buckets must be at most 32768");
    if (c->n_rounds > 16) return fail(LSH_ERR_UNSUPPORTED, "n_rounds must be at most 16");
    if (c->flags & ~(LSH_FLAG_NO_DUP_CORRECTION | LSH_FLAG_WRAP_LOOKBACK | LSH_FLAG_SAME_BUCKET))
        return fail(LSH_ERR_UNSUPPORTED, "unknown flag bit");
    if ((c->flags & LSH_FLAG_SAME_BUCKET) && (c->flags & LSH_FLAG_WRAP_LOOKBACK))
        return fail(LSH_ERR_UNSUPPORTED, "LSH_FLAG_SAME_BUCKET cannot be combined with LSH_FLAG_WRAP_LOOKBACK");
    if (c->flags & LSH_FLAG_SAME_BUCKET) {
        // window ids chunk + 2 * bucket rank must fit in 16 bits (at most 65534)
        const long long last = (long long)(c->seq_len / c->chunk - 1) +
                               2LL * ((long long)(c->n_buckets < c->seq_len ? c->n_buckets : c->seq_len) - 1);
        if (last > 65534)
            return fail(LSH_ERR_UNSUPPORTED,
                        "LSH_FLAG_SAME_BUCKET needs L/chunk - 1 + 2 (min(n_buckets, L) - 1) <= 65534");
    }
    const long long elem = c->dtype == LSH_BF16 ? 2 : 4;
    // the largest buffer is o_rounds [B, H, n_r, L, d]
    if (checked_product({c->batch, c->heads, c->n_rounds, c->seq_len, c->d_head, elem}) < 0)
        return fail(LSH_ERR_INVALID_ARG, "a buffer would exceed 2^62 bytes");
    return LSH_OK;
}

long bh_of(const lsh_config* c) { return (long)c->batch * c->heads; }

lsh_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return LSH_OK;
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return LSH_ERR_HIP;
}

#define LSH_TRY(expr)                          \
    do {                                       \
        const lsh_status _s = (expr);          \
        if (_s != LSH_OK) return _s;           \
    } while (0)

lsh_status check_layer(const lsh_config* cfg, int32_t d_model)
{
    LSH_TRY(check_config(cfg));
    if (d_model <= 0 || d_model % 64 || d_model > 65536)
        return fail(LSH_ERR_INVALID_ARG, "d_model must be a positive multiple of 64, at most 65536");
    if ((long long)cfg->batch * cfg->seq_len >= (1LL << 31))
        return fail(LSH_ERR_INVALID_ARG, "batch * seq_len must be below 2^31");
    if (checked_product({cfg->batch, cfg->seq_len, d_model, 2}) < 0)
        return fail(LSH_ERR_INVALID_ARG, "a buffer would exceed 2^62 bytes");
    if (cfg->dtype != LSH_BF16) return fail(LSH_ERR_UNSUPPORTED, "the projections support LSH_BF16 only");
    return LSH_OK;
}

// counters, then one int32 per (segment, bucket)
size_t sort_ws_bytes(const lshk::SortPlan& p) { return (p.counters + p.extra) * sizeof(int32_t); }

// Backward workspace: combined lse and Delta (float32, one per token-head), then
// the three per-round partial tensors (bf16), each part 256-byte aligned.
struct BwdLayout {
    size_t lse_c, delta, dq_r, dk_r, dv_r, total;
};

BwdLayout bwd_layout(const lsh_config* cfg)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t T = (size_t)bh_of(cfg) * cfg->seq_len;
    const size_t part = T * cfg->n_rounds * cfg->d_head * 2;
    BwdLayout l;
    l.lse_c = 0;
    l.delta = up(T * 4);
    l.dq_r = l.delta + up(T * 4);
    l.dk_r = l.dq_r + up(part);
    l.dv_r = l.dk_r + up(part);
    l.total = l.dv_r + up(part);
    return l;
}

lsh_status check_backward(const lsh_config* cfg)
{
    LSH_TRY(check_config(cfg));
    if (cfg->dtype != LSH_BF16) return fail(LSH_ERR_UNSUPPORTED, "the backward supports LSH_BF16 only");
    if (cfg->chunk != 64) return fail(LSH_ERR_UNSUPPORTED, "the backward supports chunk 64 only");
    return LSH_OK;
}

}  // namespace

extern "C" {

const char* lsh_status_string(lsh_status s)
{
    switch (s) {
        case LSH_OK: return "LSH_OK";
        case LSH_ERR_INVALID_ARG: return "LSH_ERR_INVALID_ARG: invalid argument";
        case LSH_ERR_UNSUPPORTED: return "LSH_ERR_UNSUPPORTED: unsupported configuration";
        case LSH_ERR_WORKSPACE: return "LSH_ERR_WORKSPACE: workspace too small";
        case LSH_ERR_HIP: return "LSH_ERR_HIP: HIP launch failed";
    }
    return "unknown lsh_status";
}

const char* lsh_last_error(void) { return g_last_error.c_str(); }

lsh_status lsh_debug_check_failures(unsigned long long* count, int reset)
{
    if (count == nullptr) return fail(LSH_ERR_INVALID_ARG, "count is null");
    *count = 0;
    const bool r = reset != 0;
    LSH_TRY(hip_status(lshk::check_count_sort(count, r), "lsh_debug_check_failures"));
    LSH_TRY(hip_status(lshk::check_count_attn_bwd(count, r), "lsh_debug_check_failures"));
    LSH_TRY(hip_status(lshk::attn::check_count_bf16_d64(count, r), "lsh_debug_check_failures"));
    LSH_TRY(hip_status(lshk::attn::check_count_bf16_d128(count, r), "lsh_debug_check_failures"));
    LSH_TRY(hip_status(lshk::attn::check_count_f32_d64(count, r), "lsh_debug_check_failures"));
    return hip_status(lshk::attn::check_count_f32_d128(count, r), "lsh_debug_check_failures");
}

lsh_status lsh_hash(const lsh_config* cfg, const void* qk, const void* R, int32_t* buckets,
                    hipStream_t stream)
{
    LSH_TRY(check_config(cfg));
    LSH_TRY(check_ptr(qk, "qk"));
    LSH_TRY(check_ptr(R, "R"));
    LSH_TRY(check_ptr(buckets, "buckets"));
    return hip_status(lshk::launch_hash(cfg->dtype, cfg->d_head, qk, R, buckets, bh_of(cfg),
                                        cfg->seq_len, cfg->n_rounds, cfg->n_buckets / 2,
                                        stream),
                      "lsh_hash");
}

size_t lsh_sort_workspace_bytes(const lsh_config* cfg)
{
    if (check_config(cfg) != LSH_OK) return 0;
    return sort_ws_bytes(lshk::sort_plan(bh_of(cfg), cfg->seq_len, cfg->n_rounds, cfg->n_buckets,
                                             (cfg->flags & LSH_FLAG_SAME_BUCKET) != 0));
}

lsh_status lsh_sort(const lsh_config* cfg, const int32_t* buckets, int32_t* perm, int16_t* cid,
                    void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    LSH_TRY(check_config(cfg));
    LSH_TRY(check_ptr(buckets, "buckets"));
    LSH_TRY(check_ptr(perm, "perm"));
    LSH_TRY(check_ptr(cid, "cid"));
    LSH_TRY(check_ptr(workspace, "workspace"));
    const lshk::SortPlan p = lshk::sort_plan(bh_of(cfg), cfg->seq_len, cfg->n_rounds, cfg->n_buckets,
                                             (cfg->flags & LSH_FLAG_SAME_BUCKET) != 0);
    if (workspace_bytes < sort_ws_bytes(p))
        return fail(LSH_ERR_WORKSPACE, "workspace smaller than lsh_sort_workspace_bytes()");
    int32_t* counters = static_cast<int32_t*>(workspace);
    return hip_status(lshk::launch_sort(buckets, perm, cid, counters, counters + p.counters,
                                        (cfg->flags & LSH_FLAG_SAME_BUCKET) != 0, p, bh_of(cfg),
                                        cfg->seq_len, cfg->n_rounds, cfg->n_buckets, cfg->chunk,
                                        stream),
                      "lsh_sort");
}

lsh_status lsh_sort_noalloc(const lsh_config* cfg, const int32_t* buckets, int32_t* perm,
                            int16_t* cid, hipStream_t stream)
{
    LSH_TRY(check_config(cfg));
    LSH_TRY(check_ptr(buckets, "buckets"));
    LSH_TRY(check_ptr(perm, "perm"));
    LSH_TRY(check_ptr(cid, "cid"));
    const bool same = (cfg->flags & LSH_FLAG_SAME_BUCKET) != 0;
    const lshk::SortPlan p = lshk::sort_plan(bh_of(cfg), cfg->seq_len, cfg->n_rounds, cfg->n_buckets, same);
    const size_t need = sort_ws_bytes(p);
    if (need > (size_t)LSH_SORT_NOALLOC_MAX_BYTES) {
        g_last_error = "lsh_sort_noalloc: this configuration needs " + std::to_string(need) +
                       " bytes of scratch, the static buffer holds " +
                       std::to_string((size_t)LSH_SORT_NOALLOC_MAX_BYTES) +
                       " (use lsh_sort with a workspace)";
        return LSH_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    LSH_TRY(hip_status(lshk::sort_scratch(&ws), "lsh_sort_noalloc"));
    int32_t* counters = static_cast<int32_t*>(ws);
    return hip_status(lshk::launch_sort(buckets, perm, cid, counters, counters + p.counters, same, p,
                                        bh_of(cfg), cfg->seq_len, cfg->n_rounds, cfg->n_buckets,
                                        cfg->chunk, stream),
                      "lsh_sort_noalloc");
}

lsh_status lsh_chunk_attn(const lsh_config* cfg, const void* qk, const void* v, const int32_t* perm,
                          const int16_t* cid, void* o_rounds, float* lse, hipStream_t stream)
{
    LSH_TRY(check_config(cfg));
    if (cfg->chunk != 32 && cfg->chunk != 64 && cfg->chunk != 128)
        return fail(LSH_ERR_UNSUPPORTED, "chunk attention supports chunk 32, 64 or 128");
    if (cfg->dtype == LSH_F32 && cfg->d_head == 128 && cfg->chunk == 128)
        return fail(LSH_ERR_UNSUPPORTED, "float32 with d_head 128 supports chunk 32 or 64");
    LSH_TRY(check_ptr(qk, "qk"));
    LSH_TRY(check_ptr(v, "v"));
    LSH_TRY(check_ptr(perm, "perm"));
    LSH_TRY(check_ptr(cid, "cid"));
    LSH_TRY(check_ptr(o_rounds, "o_rounds"));
    LSH_TRY(check_ptr(lse, "lse"));
    return hip_status(lshk::launch_chunk_attn(cfg->dtype, cfg->d_head, cfg->chunk, qk, v, perm, cid,
                                              o_rounds, lse, bh_of(cfg), cfg->seq_len,
                                              cfg->n_rounds, cfg->causal, cfg->scale, cfg->flags,
                                              stream),
                      "lsh_chunk_attn");
}

lsh_status lsh_combine_rounds(const lsh_config* cfg, const void* o_rounds, const float* lse,
                              void* o, hipStream_t stream)
{
    LSH_TRY(check_config(cfg));
    LSH_TRY(check_ptr(o_rounds, "o_rounds"));
    LSH_TRY(check_ptr(lse, "lse"));
    LSH_TRY(check_ptr(o, "o"));
    return hip_status(lshk::launch_combine(cfg->dtype, cfg->d_head, o_rounds, lse, o, bh_of(cfg),
                                           cfg->seq_len, cfg->n_rounds,
                                           stream),
                      "lsh_combine_rounds");
}

size_t lsh_backward_workspace_bytes(const lsh_config* cfg)
{
    if (check_backward(cfg) != LSH_OK) return 0;
    return bwd_layout(cfg).total;
}

lsh_status lsh_attn_backward(const lsh_config* cfg, const void* qk, const void* v,
                             const int32_t* perm, const int16_t* cid, const float* lse,
                             const void* o, const void* d_o, float* d_qk, float* d_v,
                             void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    LSH_TRY(check_backward(cfg));
    LSH_TRY(check_ptr(qk, "qk"));
    LSH_TRY(check_ptr(v, "v"));
    LSH_TRY(check_ptr(perm, "perm"));
    LSH_TRY(check_ptr(cid, "cid"));
    LSH_TRY(check_ptr(lse, "lse"));
    LSH_TRY(check_ptr(o, "o"));
    LSH_TRY(check_ptr(d_o, "d_o"));
    LSH_TRY(check_ptr(d_qk, "d_qk"));
    LSH_TRY(check_ptr(d_v, "d_v"));
    LSH_TRY(check_ptr(workspace, "workspace"));
    const BwdLayout l = bwd_layout(cfg);
    if (workspace_bytes < l.total)
        return fail(LSH_ERR_WORKSPACE, "workspace smaller than lsh_backward_workspace_bytes()");
    char* ws = static_cast<char*>(workspace);
    lshk::BwdArgs a;
    a.qk = qk;
    a.v = v;
    a.o = o;
    a.d_o = d_o;
    a.perm = perm;
    a.cid = cid;
    a.lse = lse;
    a.lse_c = reinterpret_cast<float*>(ws + l.lse_c);
    a.delta = reinterpret_cast<float*>(ws + l.delta);
    a.dq_r = ws + l.dq_r;
    a.dk_r = ws + l.dk_r;
    a.dv_r = ws + l.dv_r;
    a.dqk = d_qk;
    a.dv = d_v;
    a.bh = bh_of(cfg);
    a.L = cfg->seq_len;
    a.n_r = cfg->n_rounds;
    a.causal = cfg->causal;
    a.scale = cfg->scale;
    a.dup = !(cfg->flags & LSH_FLAG_NO_DUP_CORRECTION);
    a.wrap = (cfg->flags & LSH_FLAG_WRAP_LOOKBACK) != 0;
    a.same_bucket = (cfg->flags & LSH_FLAG_SAME_BUCKET) != 0;
    return hip_status(lshk::launch_attn_backward(cfg->d_head, a, stream),
                      "lsh_attn_backward");
}

lsh_status lsh_project_in(const lsh_config* cfg, int32_t d_model, const void* x, const void* w_qk,
                          const void* w_v, void* qk, void* v, hipStream_t stream)
{
    LSH_TRY(check_layer(cfg, d_model));
    LSH_TRY(check_ptr(x, "x"));
    LSH_TRY(check_ptr(w_qk, "w_qk"));
    LSH_TRY(check_ptr(w_v, "w_v"));
    LSH_TRY(check_ptr(qk, "qk"));
    LSH_TRY(check_ptr(v, "v"));
    return hip_status(lshk::launch_project_in(x, w_qk, w_v, qk, v, (long)cfg->batch * cfg->seq_len,
                                              cfg->seq_len, cfg->heads, cfg->d_head, d_model,
                                              stream),
                      "lsh_project_in");
}

lsh_status lsh_project_out(const lsh_config* cfg, int32_t d_model, const void* o, const void* w_o,
                           void* y, hipStream_t stream)
{
    LSH_TRY(check_layer(cfg, d_model));
    LSH_TRY(check_ptr(o, "o"));
    LSH_TRY(check_ptr(w_o, "w_o"));
    LSH_TRY(check_ptr(y, "y"));
    return hip_status(lshk::launch_project_out(o, w_o, y, (long)cfg->batch * cfg->seq_len,
                                               cfg->seq_len, cfg->heads, cfg->d_head, d_model,
                                               nullptr, 0.f, stream),
                      "lsh_project_out");
}

lsh_status lsh_project_out_add(const lsh_config* cfg, int32_t d_model, const void* o,
                               const void* w_o, const void* residual, float sign, void* y,
                               hipStream_t stream)
{
    LSH_TRY(check_layer(cfg, d_model));
    if (!std::isfinite(sign)) return fail(LSH_ERR_INVALID_ARG, "sign must be finite");
    LSH_TRY(check_ptr(o, "o"));
    LSH_TRY(check_ptr(w_o, "w_o"));
    LSH_TRY(check_ptr(residual, "residual"));
    LSH_TRY(check_ptr(y, "y"));
    return hip_status(lshk::launch_project_out(o, w_o, y, (long)cfg->batch * cfg->seq_len,
                                               cfg->seq_len, cfg->heads, cfg->d_head, d_model,
                                               residual, sign, stream),
                      "lsh_project_out_add");
}

size_t lsh_ffn_workspace_bytes(int64_t rows, int32_t d_ff, int32_t chunk_rows)
{
    if (rows <= 0 || d_ff <= 0 || chunk_rows <= 0) return 0;
    const int64_t cr = rows < chunk_rows ? rows : chunk_rows;
    return (size_t)cr * (size_t)d_ff * 2;
}

lsh_status lsh_ffn(int64_t rows, int32_t d_model, int32_t d_ff, int32_t chunk_rows, const void* x,
                   const void* w1, const void* b1, const void* w2, const void* b2,
                   const void* residual, float sign, void* y, void* hidden, size_t hidden_bytes,
                   hipStream_t stream)
{
    if (rows <= 0 || rows >= (1LL << 31))
        return fail(LSH_ERR_INVALID_ARG, "rows must be positive and below 2^31");
    if (d_model <= 0 || d_model % 64 || d_model > 65536 || d_ff <= 0 || d_ff % 64 || d_ff > 65536)
        return fail(LSH_ERR_INVALID_ARG, "d_model and d_ff must be positive multiples of 64, at most 65536");
    if (chunk_rows <= 0) return fail(LSH_ERR_INVALID_ARG, "chunk_rows must be positive");
    if (!std::isfinite(sign)) return fail(LSH_ERR_INVALID_ARG, "sign must be finite");
    LSH_TRY(check_ptr(x, "x"));
    LSH_TRY(check_ptr(w1, "w1"));
    LSH_TRY(check_ptr(b1, "b1"));
    LSH_TRY(check_ptr(w2, "w2"));
    LSH_TRY(check_ptr(b2, "b2"));
    LSH_TRY(check_ptr(residual, "residual"));
    LSH_TRY(check_ptr(y, "y"));
    LSH_TRY(check_ptr(hidden, "hidden"));
    if (hidden_bytes < lsh_ffn_workspace_bytes(rows, d_ff, chunk_rows))
        return fail(LSH_ERR_WORKSPACE, "hidden smaller than lsh_ffn_workspace_bytes()");
    return hip_status(lshk::launch_ffn(x, w1, b1, w2, b2, residual, sign, y, hidden, (long)rows,
                                       d_model, d_ff, chunk_rows, stream),
                      "lsh_ffn");
}

}  // extern "C"

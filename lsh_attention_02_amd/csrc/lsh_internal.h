// Internal launchers between the C ABI (lsh_api.hip) and the kernel files.
// Arguments are already validated by the caller; every launcher returns the
// hipGetLastError() status of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lshk {

hipError_t launch_hash(int dtype, int d_head, const void* qk, const void* R, int32_t* buckets,
                       long bh, int L, int n_rounds, int ncol, hipStream_t stream);

// Sort geometry: positions of one (b, h, r) segment are split into tiles of
// `tile` positions; the workspace holds one int32 counter per (segment, tile,
// bucket), then one int32 per (segment, bucket) (bucket totals, or the
// same-bucket variant's bucket ranks).
struct SortPlan {
    int tile;
    int ntiles;
    long nseg;
    size_t counters;   // nseg * ntiles * n_buckets
    size_t extra;      // nseg * n_buckets
    int rounds_per_group;   // rounds per k_sort_place workgroup, 0: k_sort_scatter
};
SortPlan sort_plan(long bh, int L, int n_rounds, int n_buckets, bool same_bucket);

// Device address of the static scratch array of lsh_sort_noalloc on the
// current device (LSH_SORT_NOALLOC_MAX_BYTES), looked up on first use per device.
hipError_t sort_scratch(void** ptr);

// counters, extra: the two workspace parts of SortPlan (int32 each).
hipError_t launch_sort(const int32_t* buckets, int32_t* perm, int16_t* cid, int32_t* counters,
                       int32_t* extra, bool same_bucket, const SortPlan& plan, long bh, int L,
                       int n_rounds, int n_buckets, int chunk, hipStream_t stream);

hipError_t launch_chunk_attn(int dtype, int d_head, int chunk, const void* qk, const void* v,
                             const int32_t* perm, const int16_t* cid, void* o_rounds, float* lse,
                             long bh, int L, int n_rounds, int causal, float scale, int flags,
                             hipStream_t stream);

namespace attn {
// One instantiation unit per element type / head size (compiled in parallel).
#define LSH_ATTN_LAUNCH_ARGS                                                                    \
    int chunk, const void *qk, const void *v, const int32_t *perm, const int16_t *cid,          \
        void *o_rounds, float *lse, long bh, int L, int n_rounds, int causal, float scale,       \
        int flags, hipStream_t stream
hipError_t launch_bf16_d64(LSH_ATTN_LAUNCH_ARGS);
hipError_t launch_bf16_d128(LSH_ATTN_LAUNCH_ARGS);
hipError_t launch_f32_d64(LSH_ATTN_LAUNCH_ARGS);
hipError_t launch_f32_d128(LSH_ATTN_LAUNCH_ARGS);
}  // namespace attn

// Failed device-side bounds checks (LSH_CHECK) of each translation unit with
// checks, added to *acc; reset clears them.  Builds without LSH_DEVICE_CHECKS
// add nothing.
hipError_t check_count_sort(unsigned long long* acc, bool reset);
hipError_t check_count_attn_bwd(unsigned long long* acc, bool reset);
namespace attn {
hipError_t check_count_bf16_d64(unsigned long long* acc, bool reset);
hipError_t check_count_bf16_d128(unsigned long long* acc, bool reset);
hipError_t check_count_f32_d64(unsigned long long* acc, bool reset);
hipError_t check_count_f32_d128(unsigned long long* acc, bool reset);
}  // namespace attn

hipError_t launch_combine(int dtype, int d_head, const void* o_rounds, const float* lse, void* o,
                          long bh, int L, int n_rounds, hipStream_t stream);

// Backward of chunk attention + combine (bf16, chunk 64; lsh_attn_bwd.hip).
struct BwdArgs {
    const void* qk;
    const void* v;
    const void* o;               // combined forward output
    const void* d_o;             // loss gradient at o
    const int32_t* perm;
    const int16_t* cid;
    const float* lse;            // per-round lse of the forward
    float* lse_c;                // workspace [bh * L]: combined logsumexp
    float* delta;                // workspace [bh * L]: <d_o, o>
    void* dq_r;                  // workspace [bh, n_r, L, d] bf16: query-role partials
    void* dk_r;                  // workspace: key-role partials
    void* dv_r;                  // workspace: value partials
    float* dqk;                  // [bh, L, d] out
    float* dv;                   // [bh, L, d] out
    long bh;
    int L, n_r, causal;
    float scale;
    bool dup;                    // duplicate-count term on
    bool wrap;                   // LSH_FLAG_WRAP_LOOKBACK
    bool same_bucket;            // LSH_FLAG_SAME_BUCKET
};
hipError_t launch_attn_backward(int d_head, const BwdArgs& a, hipStream_t stream);

// Layer projections (bf16): rows = B * L; H heads of size D; d_model a multiple of 64.
hipError_t launch_project_in(const void* x, const void* w_qk, const void* w_v, void* qk, void* v,
                             long rows, int L, int H, int D, int d_model, hipStream_t stream);
// resid: null, or y = resid + sign * (the projection)
hipError_t launch_project_out(const void* o, const void* w_o, void* y, long rows, int L, int H,
                              int D, int d_model, const void* resid, float sign, hipStream_t stream);
// Position-wise feed-forward over chunks of chunk_rows rows (bf16):
// y = resid + sign * (relu(x w1^T + b1) w2^T + b2); hidden holds chunk_rows * d_ff.
hipError_t launch_ffn(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
                      const void* resid, float sign, void* y, void* hidden, long rows, int d_model,
                      int d_ff, int chunk_rows, hipStream_t stream);

}  // namespace lshk

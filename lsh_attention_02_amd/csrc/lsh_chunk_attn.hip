// Chunk attention: dispatch on element type and head size (the kernel template
// is in lsh_chunk_attn.h, instantiated by lsh_chunk_attn_*.hip).
#include "lsh_internal.h"

namespace lshk {

hipError_t launch_chunk_attn(int dtype, int d_head, int chunk, const void* qk, const void* v,
                             const int32_t* perm, const int16_t* cid, void* o_rounds, float* lse,
                             long bh, int L, int n_rounds, int causal, float scale, int flags,
                             hipStream_t stream)
{
    if (dtype == 1)
        return d_head == 64 ? attn::launch_bf16_d64(chunk, qk, v, perm, cid, o_rounds, lse, bh, L,
                                                    n_rounds, causal, scale, flags, stream)
                            : attn::launch_bf16_d128(chunk, qk, v, perm, cid, o_rounds, lse, bh, L,
                                                     n_rounds, causal, scale, flags, stream);
    return d_head == 64 ? attn::launch_f32_d64(chunk, qk, v, perm, cid, o_rounds, lse, bh, L,
                                               n_rounds, causal, scale, flags, stream)
                        : attn::launch_f32_d128(chunk, qk, v, perm, cid, o_rounds, lse, bh, L,
                                                n_rounds, causal, scale, flags, stream);
}

}  // namespace lshk

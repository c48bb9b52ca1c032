// Chunk-attention instantiations for element type float, d_head 64.
#include "lsh_chunk_attn.h"

namespace lshk {
namespace attn {

hipError_t launch_f32_d64(LSH_ATTN_LAUNCH_ARGS)
{
    switch (chunk) {
        case 32: return launch_ndw<float, 64, 32>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, stream);
        case 64: return launch_ndw<float, 64, 64>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, stream);
        default: return launch_ndw<float, 64, 128>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, stream);
    }
}

}  // namespace attn
}  // namespace lshk

// Chunk-attention instantiations for element type float, d_head 64.
#include "lsh_chunk_attn.h"

namespace lshk {
namespace attn {

hipError_t launch_f32_d64(LSH_ATTN_LAUNCH_ARGS)
{
    switch (chunk) {
        case 32: return launch_flags<float, 64, 32>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
        case 64: return launch_flags<float, 64, 64>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
        default: return launch_flags<float, 64, 128>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
    }
}

}  // namespace attn
}  // namespace lshk

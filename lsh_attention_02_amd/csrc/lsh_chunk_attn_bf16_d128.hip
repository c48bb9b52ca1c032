// Chunk-attention instantiations for element type bf16_t, d_head 128.
#include "lsh_chunk_attn.h"

namespace lshk {
namespace attn {

hipError_t launch_bf16_d128(LSH_ATTN_LAUNCH_ARGS)
{
    switch (chunk) {
        case 32: return launch_flags<bf16_t, 128, 32>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
        case 64: return launch_flags<bf16_t, 128, 64>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
        default: return launch_flags<bf16_t, 128, 128>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
    }
}

}  // namespace attn
}  // namespace lshk

// Chunk-attention instantiations for element type float, d_head 128.
#include "lsh_chunk_attn.h"

namespace lshk {
namespace attn {

LSH_CHECK_ACCESSOR(check_count_f32_d128)

hipError_t launch_f32_d128(LSH_ATTN_LAUNCH_ARGS)
{
    switch (chunk) {
        case 32: return launch_flags<float, 128, 32>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
        case 64: return launch_flags<float, 128, 64>(qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds, causal, scale, flags, stream);
        // float rows at d_head 128 with chunk 128 need more LDS than a CU has;
        // the host rejects that combination before launching.
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
}  // namespace lshk

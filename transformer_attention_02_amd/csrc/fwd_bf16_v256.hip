// Forward launches for value head dim 256 (the kernel template is in fwd_bf16_body.h).  This
// file is compiled with LLVM's iterative ILP scheduler: on the causal [2, 2048, 16, 256]
// prefill its 8-wave value-split kernel ran 85.2 us against 89.8 us with the default scheduler,
// with the same output bits; at value head dim 128 that scheduler was 0.5-2% slower, so
// fwd_bf16.hip keeps the default.
#include "fwd_bf16_body.h"

namespace attn {

hipError_t launch_fwd_bf16_v256(const FwdArgs &a, bool out_f32, hipStream_t stream) {
    if (a.block_tables) {  // paged KV caches: equal head dims only
        if (a.K == 256) return launch_out<256, 256, true>(a, out_f32, stream);
        return hipErrorInvalidValue;
    }
    if (a.K == 256) return launch_out<256, 256, false>(a, out_f32, stream);
    if (a.K == 128) return launch_out<128, 256, false>(a, out_f32, stream);
    if (a.K == 64) return launch_out<64, 256, false>(a, out_f32, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn

// Forward launches for value head dims up to 128 (the kernel template is in fwd_bf16_body.h);
// value head dim 256 goes to fwd_bf16_v256.hip.
#include "fwd_bf16_body.h"

namespace attn {

hipError_t launch_fwd_bf16(const FwdArgs &a, bool out_f32, hipStream_t stream) {
    if (a.Kv == 256) return launch_fwd_bf16_v256(a, out_f32, stream);
    if (a.block_tables) {  // paged KV caches: equal head dims only (the page table takes 32 KB of LDS)
        if (a.K == 128 && a.Kv == 128) return launch_out<128, 128, true>(a, out_f32, stream);
        if (a.K == 64 && a.Kv == 64) return launch_out<64, 64, true>(a, out_f32, stream);
        return hipErrorInvalidValue;
    }
    if (a.K == 256 && a.Kv == 128) return launch_out<256, 128, false>(a, out_f32, stream);
    if (a.K == 256 && a.Kv == 64) return launch_out<256, 64, false>(a, out_f32, stream);
    if (a.K == 128 && a.Kv == 128) return launch_out<128, 128, false>(a, out_f32, stream);
    if (a.K == 64 && a.Kv == 64) return launch_out<64, 64, false>(a, out_f32, stream);
    if (a.K == 64 && a.Kv == 128) return launch_out<64, 128, false>(a, out_f32, stream);
    if (a.K == 128 && a.Kv == 64) return launch_out<128, 64, false>(a, out_f32, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn

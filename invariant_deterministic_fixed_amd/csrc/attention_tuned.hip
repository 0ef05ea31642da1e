// attention_tuned.hip -- comparator for decode attention (NOT batch-invariant).
#include "common.hpp"
#include "kernels.hpp"

namespace binv {

size_t attn_tuned_workspace_bytes(int64_t B, int Hq, int D, int64_t max_kv_len) {
    (void)max_kv_len;
    return (size_t)B * Hq * 64 * (D + 2) * sizeof(float);
}

hipError_t launch_attention_decode_tuned(const AttnArgs& a, hipStream_t s) {
    (void)a; (void)s;
    return hipErrorNotSupported;
}

}  // namespace binv

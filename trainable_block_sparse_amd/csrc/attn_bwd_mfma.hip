// Matrix-core kernels of the attention backward (bf16, block 64).
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

bool bwd_mfma_ok(const Shape&) { return false; }
size_t bwd_kt_bytes(const Shape&, int64_t) { return 0; }

hipError_t launch_attn_prefill_bwd_mfma(const Shape&, const BwdWs&, const void*, int, int64_t,
                                        const void*, const void*, const int64_t*, const int32_t*,
                                        const void*, const void*, void*, void*, void*, char*,
                                        hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace infv2

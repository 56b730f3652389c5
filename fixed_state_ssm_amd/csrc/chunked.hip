// Chunked parallel-in-time forward (bf16 I/O, fp16 MFMA operands).
#include "common.h"
#include "launch.h"

namespace idattn {

bool chunked_supported(const Problem&) { return false; }
size_t chunked_workspace_bytes(const Problem&) { return 0; }
hipError_t launch_forward_chunked(const Problem&, const idattn_params&, const void*, const void*,
                                  const void*, void*, const float*, const void*, float*, void*,
                                  hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace idattn

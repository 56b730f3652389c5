// Selection of the chunked parallel-in-time forward (bf16 I/O, fp16 MFMA
// operands, fp32 accumulation and state) and its workspace.  The kernels are
// in chunked_ws.hip; the sequential fp32 path (featmap.hip, scan_seq.hip)
// serves every shape this one does not.
#include "common.h"
#include "launch.h"

namespace idattn {

bool chunked_supported(const Problem& p) {
    // M = 64 modes, d = R in {64, 128}, conv width up to 4
    if (!(p.bf16 && p.M == 64 && (p.d == 64 || p.d == 128) && p.W >= 1 && p.W <= 4)) return false;
    if (p.rff_feat) return false;  // the chunked feature code has the SiLU maps only
    // the kernels address one (b, h) sequence with 32-bit byte offsets
    return p.N * p.H * p.d * 2 < (int64_t{1} << 31);
}

size_t chunked_workspace_bytes(const Problem& p) { return chunked_ws_workspace_bytes(p); }

hipError_t launch_forward_chunked(const Problem& p, const idattn_params& prm, const void* q, const void* k,
                                  const void* v, void* o, const float* state_in, const void* tail_in,
                                  float* state_out, void* tail_out, void* workspace, hipStream_t stream) {
    return launch_forward_chunked_ws(p, prm, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, stream);
}

}  // namespace idattn

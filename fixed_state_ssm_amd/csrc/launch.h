// Internal launchers of libidattn.  Every launcher enqueues on `stream` and
// returns hipGetLastError() of its launch; arguments are validated by the
// C-ABI layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/idattn.h"

namespace idattn {

struct Problem {
    int64_t B, N, H, d, M, W;
    bool bf16;
    float eps_feat, eps_norm;
    bool unit_feat;  // xi = y / sqrt(||y||^2 + eps_feat) instead of y / (||y||^2 + eps_feat)
    bool rff_feat;   // xi = random Fourier features of c with prm.rff_omega (overrides unit_feat)
    // Token axis: T tokens in [T][H][d].  cu == nullptr: B sequences of N tokens
    // each (T = B N); else a packed batch, sequence b = tokens cu[b] .. cu[b+1]-1.
    int64_t T;
    const int32_t* cu;
    // normalised readout on the chunked path (o = Re sum s Gamma / Re sum s eta)
    bool eta = false;
};

// ---- stage kernels of the sequential (fp32) path; workspace layout [H][T][*]
hipError_t launch_featmap_conv_norm(const Problem& p, const idattn_params& prm,
                                    const void* q, const void* k, const void* v,
                                    const void* tail_in, float* xi_q, float* z_k,
                                    float* z_v, hipStream_t stream);

// With pden != nullptr (normalised readout) the key scan also carries eta
// ([B][H][M] complex; eta_in NULL = zeros, eta_out may be NULL or eta_in) and
// writes each mode's share of the denominator to pden [H][T][M].
hipError_t launch_ssm_key_scan_seq(const Problem& p, const idattn_params& prm,
                                   const float* xi_q, const float* z_k,
                                   const float* state_in, float* s, float* state_out,
                                   const float* eta_in, float* eta_out, float* pden,
                                   hipStream_t stream);

// With M >= 32 the modes are split over two blocks whose partial numerators
// go to num0 and num1 ([H][T][d] fp32 each; the feature buffers xi_q and z_k,
// free once the key scan has run); a combine kernel forms o, and with pden
// (the normalised readout) sums the denominator from it.
hipError_t launch_ssm_value_scan_readout_seq(const Problem& p, const idattn_params& prm,
                                             const float* s, const float* z_v,
                                             const float* state_in, void* o,
                                             float* state_out, const float* pden, float* num0, float* num1,
                                             hipStream_t stream);

// ---- chunked MFMA path (bf16 I/O; wave-specialised kernels for d = R in
// {64, 128}, M = 64, W <= 4, the SiLU feature maps)
size_t chunked_workspace_bytes(const Problem& p);
bool chunked_supported(const Problem& p);
// Packed batch in one launch sequence: p.B sequences on p.N = T tokens, the
// plan built on the device from cu_seqlens (device int32 [B + 1]).  The
// workspace depends on B, H and T only (monotone in T).
bool chunked_packed_supported(const Problem& p);
size_t chunked_packed_workspace_bytes(const Problem& p);
// Also writes tail_out (when not NULL) like launch_tail_update.  With p.eta the
// readout is the normalised one, eta_in / eta_out the normaliser ([B][H][M]
// complex; NULL = zeros / no output; eta_out may equal eta_in).
hipError_t launch_forward_chunked(const Problem& p, const idattn_params& prm,
                                  const void* q, const void* k, const void* v, void* o,
                                  const float* state_in, const void* tail_in,
                                  float* state_out, void* tail_out, void* workspace, hipStream_t stream,
                                  const float* eta_in = nullptr, float* eta_out = nullptr);
hipError_t launch_forward_chunked_packed(const Problem& p, const idattn_params& prm, const int32_t* cu_seqlens,
                                         const void* q, const void* k, const void* v, void* o,
                                         const float* state_in, const void* tail_in, float* state_out,
                                         void* tail_out, void* workspace, hipStream_t stream);

// ---- backward (sequential fp32; dense batches, SiLU feature maps)
size_t backward_workspace_bytes(const Problem& p);
hipError_t launch_backward(const Problem& p, const idattn_params& prm, const void* q, const void* k, const void* v,
                           const float* state_in, const void* tail_in, const void* grad_o, const float* grad_state,
                           void* grad_q, void* grad_k, void* grad_v, const idattn_param_grads& grads,
                           float* grad_state_in, void* workspace, hipStream_t stream);

// ---- the library's own scratch memory (idattn_forward_noalloc)
constexpr size_t kNoallocScratchBytes = size_t{192} << 20;
// Device address of this device's scratch array (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

// ---- state and tail plumbing
// tail_out = last W-1 raw tokens of [tail_in (or zeros) ; x]; safe in place.
hipError_t launch_tail_update(const Problem& p, const void* q, const void* k,
                              const void* tail_in, void* tail_out, hipStream_t stream);
// dst = src (or zeros when src is NULL); n_elems 32-bit words.
hipError_t launch_copy_or_zero(const void* src, void* dst, int64_t n_words, hipStream_t stream);

// ---- decode (1 .. kDecodeMaxTokens tokens per sequence, [B][N][H][d])
constexpr int kDecodeMaxTokens = 8;
// eta != nullptr: normalised readout, eta [B][H][M] complex updated in place.
hipError_t launch_decode_step(const Problem& p, const idattn_params& prm,
                              const void* q_t, const void* k_t, const void* v_t, void* o_t,
                              float* state, void* tail, float* eta, hipStream_t stream);

}  // namespace idattn

// featmap_conv_norm: causal depthwise short conv of q and k, the SiLU feature
// map with squared-norm normalisation, and the per-half input RMSNorm
// (gist.science German summary, "Skalierbare Implementierung": feature-map
// and normalisation bullets), or one of the other feature maps (unit norm;
// random Fourier features, Chinese rendering, section 3.1, eq. 6).  Also the
// conv-tail update and a copy kernel.
//
// One wave per four consecutive tokens of one head; lane l owns channels l and
// l + 64.  Waves are numbered in [T / 4][H] order (T tokens of the dense
// [B][N] or of a packed batch) so that neighbouring waves read neighbouring
// rows of q, k, v.
// Outputs go to the workspace in [H][T][d] float32 order, where each (b, h)
// sequence is a contiguous run that the sequential scans read in turn.
#include "common.h"
#include "launch.h"

namespace idattn {

namespace {

// WT: the conv width when it is fixed at compile time (4), else 0 (any W,
// with kConvMax taps of which the first W are used).  TPW consecutive tokens
// of one head per wave (waves numbered [T / TPW][H]): their chains of loads,
// conv and norm reductions are independent, so the wave interleaves them, and
// the head's conv weights, gain and bias are loaded once.  A token past T (in
// the last group) computes on a copy of token T - 1 and stores nothing.
template <bool BF16, int DJ, int WT, int TPW>
__global__ __launch_bounds__(256) void featmap_conv_norm_kernel(
    Problem p, idattn_params prm, const void* __restrict__ q, const void* __restrict__ k,
    const void* __restrict__ v, const void* __restrict__ tail_in, float* __restrict__ xi_q,
    float* __restrict__ z_k, float* __restrict__ z_v) {
    constexpr int NT = WT > 0 ? WT : kConvMax;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t th = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    const int64_t H = p.H, T = p.T;
    const int d = static_cast<int>(p.d), W = WT > 0 ? WT : static_cast<int>(p.W);
    if (th >= (T + TPW - 1) / TPW * H) return;  // whole wave exits; no barriers below
    const int64_t h = th % H;
    const int64_t tg = (th / H) * TPW;  // the group's first token on the [T] axis
    const float inv_d = 1.f / static_cast<float>(d);

    // the head's conv weights, gain and bias (channels clamped below d)
    int cl[DJ];
    uint32_t lb[DJ];  // byte offsets of the lane's channels in a row of q, k, v
    float wq[NT][DJ], wk[NT][DJ], gk[DJ], bk[DJ], gv[DJ], bv[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        cl[j] = min(lane + kWave * j, d - 1);
        lb[j] = static_cast<uint32_t>(cl[j]) * (BF16 ? 2u : 4u);
#pragma unroll
        for (int j2 = 0; j2 < NT; ++j2) {
            wq[j2][j] = prm.conv_q[(h * d + cl[j]) * W + min(j2, W - 1)];
            wk[j2][j] = prm.conv_k[(h * d + cl[j]) * W + min(j2, W - 1)];
        }
        gk[j] = prm.gain[h * 2 * d + cl[j]];
        bk[j] = prm.bias[h * 2 * d + cl[j]];
        gv[j] = prm.gain[h * 2 * d + d + cl[j]];
        bv[j] = prm.bias[h * 2 * d + d + cl[j]];
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t t = min(tg + u, T - 1);  // token on the [T] axis
        const int64_t b = seq_of_token(p.cu, p.N, p.B, t);
        int64_t start, len;
        seq_range(p.cu, p.N, T, b, start, len);
        const int64_t n = t >= start ? t - start : 0;  // position in its sequence (0 <= n <= t)

        // every load of the token first (missing rows masked below): the conv
        // taps of q and k, v; each row is a buffer resource at a uniform base
        uint32_t xq_raw[NT][DJ], xk_raw[NT][DJ], v_raw[DJ];
        bool tap_ok[NT];
#pragma unroll
        for (int j2 = 0; j2 < NT; ++j2) {
            const ConvRow r = conv_row(q, k, tail_in, t - n, n - (W - 1) + j2, t, b, h, H, d, W, j2 < W);
            tap_ok[j2] = r.ok;
            const __amdgpu_buffer_rsrc_t rq = io_rsrc<BF16>(r.bq, r.rq, d), rk = io_rsrc<BF16>(r.bk, r.rk, d);
#pragma unroll
            for (int j = 0; j < DJ; ++j) {
                xq_raw[j2][j] = buf_load_raw<BF16>(rq, lb[j]);
                xk_raw[j2][j] = buf_load_raw<BF16>(rk, lb[j]);
            }
        }
        const __amdgpu_buffer_rsrc_t vrow = io_rsrc<BF16>(v, (t * H + h) * d, d);
#pragma unroll
        for (int j = 0; j < DJ; ++j) v_raw[j] = buf_load_raw<BF16>(vrow, lb[j]);

        float cqv[DJ], ckv[DJ], yq[DJ], yk[DJ], xv[DJ];
        float sv = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            float cq = 0.f, ck = 0.f;
#pragma unroll
            for (int j2 = 0; j2 < NT; ++j2) {
                cq = fmaf(wq[j2][j], tap_ok[j2] ? widen<BF16>(xq_raw[j2][j]) : 0.f, cq);
                ck = fmaf(wk[j2][j], tap_ok[j2] ? widen<BF16>(xk_raw[j2][j]) : 0.f, ck);
            }
            const bool in = lane + kWave * j < d;  // lanes past d hold zeros
            cqv[j] = in ? cq : 0.f;
            ckv[j] = in ? ck : 0.f;
            xv[j] = in ? widen<BF16>(v_raw[j]) : 0.f;
            sv = fmaf(xv[j], xv[j], sv);
        }
        sv = wave_total(sv);
        // xi = y * inv with y = SiLU(c) = c / (1 + exp(-c)) (the hardware exp and
        // reciprocal, each within about an ulp); lanes past d hold c = 0 -> y = 0.
        // (The RFF map has its own kernel below.)
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            yq[j] = cqv[j] * __builtin_amdgcn_rcpf(1.f + __expf(-cqv[j]));
            yk[j] = ckv[j] * __builtin_amdgcn_rcpf(1.f + __expf(-ckv[j]));
            sq = fmaf(yq[j], yq[j], sq);
            sk = fmaf(yk[j], yk[j], sk);
        }
        sq = wave_total(sq);
        sk = wave_total(sk);
        // squared norm, or its square root for the unit-norm map
        const float inv_q = p.unit_feat ? __builtin_amdgcn_rsqf(sq + p.eps_feat) : __builtin_amdgcn_rcpf(sq + p.eps_feat);
        const float inv_k = p.unit_feat ? __builtin_amdgcn_rsqf(sk + p.eps_feat) : __builtin_amdgcn_rcpf(sk + p.eps_feat);
        float xk2 = 0.f;
        float xik[DJ];
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            xik[j] = yk[j] * inv_k;
            xk2 = fmaf(xik[j], xik[j], xk2);
        }
        xk2 = wave_total(xk2);
        const float rk = __builtin_amdgcn_rsqf(fmaf(xk2, inv_d, p.eps_norm));
        const float rv = __builtin_amdgcn_rsqf(fmaf(sv, inv_d, p.eps_norm));
        if (tg + u < T) {  // uniform over the wave
            const int64_t orow = (h * T + t) * d;
#pragma unroll
            for (int j = 0; j < DJ; ++j) {
                const int c = lane + kWave * j;
                if (c < d) {
                    xi_q[orow + c] = yq[j] * inv_q;
                    z_k[orow + c] = fmaf(gk[j] * xik[j], rk, bk[j]);
                    z_v[orow + c] = fmaf(gv[j] * xv[j], rv, bv[j]);
                }
            }
        }
    }
}

// Random Fourier features of TPW tokens held by one wave (Chinese rendering of
// the paper, section 3.1, eq. 6), as rff_features computes them for one
// token, with the conv outputs broadcast through the wave's slice of shared
// memory (cs: [2][TPW][d] floats, queries then keys) instead of one readlane
// per input: lane l forms the phases of frequency l mod D, reading four
// inputs of a token per 16-byte broadcast load, and every row of Omega it
// loads serves all TPW tokens.  The products are summed in the same order
// (input 0 to d - 1), so the features are the same bits.
template <int DJ, int TPW>
__device__ __forceinline__ void rff_features_lds(const float (&cq)[TPW][DJ], const float (&ck)[TPW][DJ],
                                                 const float* __restrict__ om, int d, float* cs,
                                                 float (&yq)[TPW][DJ], float (&yk)[TPW][DJ]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int D = d >> 1;  // a power of two, at most 64
    const int f = lane & (D - 1);
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const int c = lane + kWave * j;
            if (c < d) {
                cs[u * d + c] = cq[u][j];
                cs[(TPW + u) * d + c] = ck[u][j];
            }
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the wave's writes before its reads
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pq[TPW], pk[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) pq[u] = pk[u] = 0.f;
    for (int r0 = 0; r0 < d; r0 += 16) {
        float w[16];  // sixteen rows of Omega in flight at once
#pragma unroll
        for (int e = 0; e < 16; ++e) w[e] = om[(r0 + e) * D + f];
#pragma unroll
        for (int e4 = 0; e4 < 16; e4 += 4)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const float4 xq = *reinterpret_cast<const float4*>(&cs[u * d + r0 + e4]);
                const float4 xk = *reinterpret_cast<const float4*>(&cs[(TPW + u) * d + r0 + e4]);
                pq[u] = fmaf(xq.w, w[e4 + 3], fmaf(xq.z, w[e4 + 2], fmaf(xq.y, w[e4 + 1], fmaf(xq.x, w[e4], pq[u]))));
                pk[u] = fmaf(xk.w, w[e4 + 3], fmaf(xk.z, w[e4 + 2], fmaf(xk.y, w[e4 + 1], fmaf(xk.x, w[e4], pk[u]))));
            }
    }
    const float sc = 1.f / sqrtf(static_cast<float>(D));
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        float sq, cs_q, sk, cs_k;
        sincosf(pq[u], &sq, &cs_q);
        sincosf(pk[u], &sk, &cs_k);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const int c = lane + kWave * j;
            const bool in = c < d, sn = c >= D;
            yq[u][j] = in ? (sn ? sq : cs_q) * sc : 0.f;
            yk[u][j] = in ? (sn ? sk : cs_k) * sc : 0.f;
        }
    }
}

// The RFF map: one wave per TPW consecutive tokens of one head (waves numbered
// [T / TPW][H]), so that each row of the head's frequency table is loaded once
// for TPW tokens; the conv taps and the input RMSNorm as in
// featmap_conv_norm_kernel (every load of a token issued before its first use,
// a token past T computing on a copy of token T - 1 and storing nothing).
template <bool BF16, int DJ, int WT, int TPW>
__global__ __launch_bounds__(256) void featmap_rff_kernel(
    Problem p, idattn_params prm, const void* __restrict__ q, const void* __restrict__ k,
    const void* __restrict__ v, const void* __restrict__ tail_in, float* __restrict__ xi_q,
    float* __restrict__ z_k, float* __restrict__ z_v) {
    constexpr int NT = WT > 0 ? WT : kConvMax;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t th = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    const int64_t H = p.H, T = p.T;
    const int d = static_cast<int>(p.d), W = WT > 0 ? WT : static_cast<int>(p.W);
    __shared__ __align__(16) float cs_all[4][2 * TPW * (DJ * kWave)];  // per wave: conv outputs for the features
    if (th >= (T + TPW - 1) / TPW * H) return;  // whole wave exits; no barriers below
    const int64_t h = th % H;
    const int64_t tg = (th / H) * TPW;  // the group's first token on the [T] axis

    int cl[DJ];
    uint32_t lb[DJ];  // byte offsets of the lane's channels in a row of q, k, v
    float wq[NT][DJ], wk[NT][DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        cl[j] = min(lane + kWave * j, d - 1);
        lb[j] = static_cast<uint32_t>(cl[j]) * (BF16 ? 2u : 4u);
#pragma unroll
        for (int j2 = 0; j2 < NT; ++j2) {
            wq[j2][j] = prm.conv_q[(h * d + cl[j]) * W + min(j2, W - 1)];
            wk[j2][j] = prm.conv_k[(h * d + cl[j]) * W + min(j2, W - 1)];
        }
    }
    float cq[TPW][DJ], ck[TPW][DJ], xv[TPW][DJ], sv[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t t = min(tg + u, T - 1);
        const int64_t b = seq_of_token(p.cu, p.N, p.B, t);
        int64_t start, len;
        seq_range(p.cu, p.N, T, b, start, len);
        const int64_t n = t >= start ? t - start : 0;
        uint32_t xq_raw[NT][DJ], xk_raw[NT][DJ], v_raw[DJ];
        bool tap_ok[NT];
#pragma unroll
        for (int j2 = 0; j2 < NT; ++j2) {
            const ConvRow r = conv_row(q, k, tail_in, t - n, n - (W - 1) + j2, t, b, h, H, d, W, j2 < W);
            tap_ok[j2] = r.ok;
            const __amdgpu_buffer_rsrc_t rq = io_rsrc<BF16>(r.bq, r.rq, d), rk = io_rsrc<BF16>(r.bk, r.rk, d);
#pragma unroll
            for (int j = 0; j < DJ; ++j) {
                xq_raw[j2][j] = buf_load_raw<BF16>(rq, lb[j]);
                xk_raw[j2][j] = buf_load_raw<BF16>(rk, lb[j]);
            }
        }
        const __amdgpu_buffer_rsrc_t vrow = io_rsrc<BF16>(v, (t * H + h) * d, d);
#pragma unroll
        for (int j = 0; j < DJ; ++j) v_raw[j] = buf_load_raw<BF16>(vrow, lb[j]);
        sv[u] = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            float a = 0.f, e = 0.f;
#pragma unroll
            for (int j2 = 0; j2 < NT; ++j2) {
                a = fmaf(wq[j2][j], tap_ok[j2] ? widen<BF16>(xq_raw[j2][j]) : 0.f, a);
                e = fmaf(wk[j2][j], tap_ok[j2] ? widen<BF16>(xk_raw[j2][j]) : 0.f, e);
            }
            const bool in = lane + kWave * j < d;  // lanes past d hold zeros
            cq[u][j] = in ? a : 0.f;
            ck[u][j] = in ? e : 0.f;
            xv[u][j] = in ? widen<BF16>(v_raw[j]) : 0.f;
            sv[u] = fmaf(xv[u][j], xv[u][j], sv[u]);
        }
    }
    float yq[TPW][DJ], yk[TPW][DJ];
    rff_features_lds<DJ, TPW>(cq, ck, prm.rff_omega + h * d * (d / 2), d, cs_all[wave_id()], yq, yk);
    float gk[DJ], bk[DJ], gv[DJ], bv[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        gk[j] = prm.gain[h * 2 * d + cl[j]];
        bk[j] = prm.bias[h * 2 * d + cl[j]];
        gv[j] = prm.gain[h * 2 * d + d + cl[j]];
        bv[j] = prm.bias[h * 2 * d + d + cl[j]];
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t t = tg + u;
        float xk2 = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) xk2 = fmaf(yk[u][j], yk[u][j], xk2);
        xk2 = wave_total(xk2);
        const float svt = wave_total(sv[u]);
        if (t >= T) continue;  // uniform over the wave
        const float rk = 1.f / sqrtf(xk2 / d + p.eps_norm);
        const float rv = 1.f / sqrtf(svt / d + p.eps_norm);
        const int64_t orow = (h * T + t) * d;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const int c = lane + kWave * j;
            if (c < d) {
                xi_q[orow + c] = yq[u][j];
                z_k[orow + c] = fmaf(gk[j] * yk[u][j], rk, bk[j]);
                z_v[orow + c] = fmaf(gv[j] * xv[u][j], rv, bv[j]);
            }
        }
    }
}

// One block per (b, h): read every tail element first, then write, so that
// tail_out may be tail_in.
template <bool BF16>
__global__ __launch_bounds__(256) void tail_update_kernel(Problem p, const void* __restrict__ q,
                                                          const void* __restrict__ k,
                                                          const void* tail_in, void* tail_out) {
    constexpr int kMaxPer = 8;  // 2 * (W-1) * d <= 2 * 7 * 128 = 1792 <= 8 * 256
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int Wm1 = static_cast<int>(p.W) - 1;
    const int d = static_cast<int>(p.d);
    const int E = 2 * Wm1 * d;
    int64_t start, len;
    seq_range(p.cu, p.N, p.T, b, start, len);
    float val[kMaxPer];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int e = threadIdx.x + 256 * j;
        val[j] = 0.f;
        if (e < E) {
            const int sel = e / (Wm1 * d);          // 0 = q, 1 = k
            const int t = (e / d) % Wm1;            // slot in the new tail
            const int c = e % d;
            const int64_t src = len + t;            // index in [tail_in ; this sequence's tokens]
            if (src < Wm1) {
                if (tail_in != nullptr)
                    val[j] = load_io<BF16>(tail_in, bh * E + (static_cast<int64_t>(sel) * Wm1 + src) * d + c);
            } else {
                const int64_t pos = src - Wm1;
                val[j] = load_io<BF16>(sel == 0 ? q : k, ((start + pos) * p.H + h) * d + c);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int e = threadIdx.x + 256 * j;
        if (e < E) store_io<BF16>(tail_out, bh * E + e, val[j]);
    }
}

__global__ __launch_bounds__(256) void copy_or_zero_kernel(const uint32_t* __restrict__ src,
                                                           uint32_t* __restrict__ dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src != nullptr ? src[i] : 0u;
}

}  // namespace

hipError_t launch_featmap_conv_norm(const Problem& p, const idattn_params& prm, const void* q,
                                    const void* k, const void* v, const void* tail_in,
                                    float* xi_q, float* z_k, float* z_v, hipStream_t stream) {
    if (p.rff_feat) {
        constexpr int kTPW = 4;
        const int64_t waves = (p.T + kTPW - 1) / kTPW * p.H;
        const dim3 g(static_cast<unsigned>((waves + 3) / 4));
#define IDATTN_RFF(BF, DJ, WT) \
    featmap_rff_kernel<BF, DJ, WT, kTPW><<<g, 256, 0, stream>>>(p, prm, q, k, v, tail_in, xi_q, z_k, z_v)
#define IDATTN_RFFW(BF, DJ)        \
    do {                           \
        if (p.W == 4)              \
            IDATTN_RFF(BF, DJ, 4); \
        else                       \
            IDATTN_RFF(BF, DJ, 0); \
    } while (0)
        if (p.d > 64) {
            if (p.bf16) IDATTN_RFFW(true, 2);
            else IDATTN_RFFW(false, 2);
        } else {
            if (p.bf16) IDATTN_RFFW(true, 1);
            else IDATTN_RFFW(false, 1);
        }
#undef IDATTN_RFFW
#undef IDATTN_RFF
        return hipGetLastError();
    }
    constexpr int kFmTPW = 4;  // tokens per wave
    const int64_t th = (p.T + kFmTPW - 1) / kFmTPW * p.H;
    const dim3 grid(static_cast<unsigned>((th + 3) / 4));
#define IDATTN_FM(BF, DJ, WT) \
    featmap_conv_norm_kernel<BF, DJ, WT, kFmTPW><<<grid, 256, 0, stream>>>(p, prm, q, k, v, tail_in, xi_q, z_k, z_v)
#define IDATTN_FMW(BF, DJ) \
    do {                   \
        if (p.W == 4)      \
            IDATTN_FM(BF, DJ, 4); \
        else               \
            IDATTN_FM(BF, DJ, 0); \
    } while (0)
    if (p.d > 64) {
        if (p.bf16) IDATTN_FMW(true, 2);
        else IDATTN_FMW(false, 2);
    } else {
        if (p.bf16) IDATTN_FMW(true, 1);
        else IDATTN_FMW(false, 1);
    }
#undef IDATTN_FMW
#undef IDATTN_FM
    return hipGetLastError();
}

hipError_t launch_tail_update(const Problem& p, const void* q, const void* k, const void* tail_in,
                              void* tail_out, hipStream_t stream) {
    if (p.W <= 1) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(p.B * p.H));
    if (p.bf16)
        tail_update_kernel<true><<<grid, 256, 0, stream>>>(p, q, k, tail_in, tail_out);
    else
        tail_update_kernel<false><<<grid, 256, 0, stream>>>(p, q, k, tail_in, tail_out);
    return hipGetLastError();
}

hipError_t launch_copy_or_zero(const void* src, void* dst, int64_t n_words, hipStream_t stream) {
    if (n_words <= 0 || src == dst) return hipSuccess;
    int64_t blocks = (n_words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    copy_or_zero_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(
        static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), n_words);
    return hipGetLastError();
}

}  // namespace idattn

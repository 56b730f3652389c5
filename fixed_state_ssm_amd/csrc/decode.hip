// decode_step: one to eight tokens per sequence against a carried state held
// in HBM.
//
// One block of 4 waves per (b, h).  Wave 0 first builds the tokens' features
// (conv over the tail and the new tokens, feature map, per-half RMSNorm)
// into LDS and shifts the conv tail; wave 1 evaluates the ZOH coefficients of
// all M modes (one mode per lane).  Then every wave streams its quarter of
// the M rows of the complex state [M][2d]: a row is read once as float4s,
// and for each token in turn updated, reduced to s_m over the key half with
// a lane reduction and read out into per-lane partial sums of
// Re(s_m Gamma_m); then it is written back in place.
// The state sweep (2 x 128 KiB per (b, h) at d = 128, M = 64) is the whole
// cost: each wave streams its rows one at a time with few live registers, so
// that many workgroups share a CU and hide each other's memory latency, and
// the ZOH coefficients (wave 1, fp32 with the phase reduced in fp64) are built
// while wave 0 builds the features.
#include "common.h"
#include "launch.h"

namespace idattn {

namespace {

// State rows are read and written once per call: non-temporal accesses.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float4* p) {
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(const float4& x, float4* p) {
    const f4v v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(p));
}

// ZOH coefficients of one mode, abar = exp(Delta lambda) and
// bbar = (exp(Delta lambda) - 1) / lambda * B (Delta B when lambda = 0), with
// Delta and the phase Delta Im(lambda) formed and reduced modulo 2 pi in fp64 and
// the rest in fp32 (about 1e-7 relative).
__device__ __forceinline__ float4 zoh_coef(double dt, float lre, float lim, float bre, float bim) {
    const double y64 = dt * static_cast<double>(lim);
    const double turns = rint(y64 * 0.15915494309189535);  // 1 / (2 pi)
    const float y = static_cast<float>(fma(-turns, 6.283185307179586, y64));
    const float x = static_cast<float>(dt * static_cast<double>(lre));
    float sy, cy;
    sincosf(y, &sy, &cy);
    const float ex = expf(x);
    const float sh = sinf(0.5f * y);
    const float em1_re = expm1f(x) * cy - 2.f * sh * sh;  // Re(exp(z) - 1) without cancellation
    const float em1_im = ex * sy;
    const float l2 = lre * lre + lim * lim;
    float qr, qi;  // (exp(z) - 1) / lambda
    if (l2 == 0.f) {
        qr = static_cast<float>(dt);
        qi = 0.f;
    } else {
        qr = (em1_re * lre + em1_im * lim) / l2;
        qi = (em1_im * lre - em1_re * lim) / l2;
    }
    return make_float4(ex * cy, ex * sy, qr * bre - qi * bim, qr * bim + qi * bre);
}

// Features of one token from its conv outputs (lane owns channels lane and
// lane + 64; zero past d): xi = y * inv with y = SiLU(c) and the squared or
// the unit norm, or (RFF) the random Fourier features of c with inv = 1.
template <bool RFF>
__device__ __forceinline__ void token_features(const Problem& p, const float* __restrict__ om,
                                               const float (&cq)[2], const float (&ck)[2], float (&yq)[2],
                                               float (&yk)[2], float& inv_q, float& inv_k) {
    if constexpr (RFF) {
        rff_features<2>(cq, ck, om, static_cast<int>(p.d), yq, yk);
        inv_q = inv_k = 1.f;
        return;
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        yq[j] = cq[j] / (1.f + expf(-cq[j]));
        yk[j] = ck[j] / (1.f + expf(-ck[j]));
        sq = fmaf(yq[j], yq[j], sq);
        sk = fmaf(yk[j], yk[j], sk);
    }
    sq = wave_total(sq);
    sk = wave_total(sk);
    // squared norm, or its square root for the unit-norm map
    inv_q = p.unit_feat ? 1.f / sqrtf(sq + p.eps_feat) : 1.f / (sq + p.eps_feat);
    inv_k = p.unit_feat ? 1.f / sqrtf(sk + p.eps_feat) : 1.f / (sk + p.eps_feat);
}

// NT = most tokens of the instance (1, or kDecodeMaxTokens with the call's
// n = p.N <= NT); FJ = float4 chunks of a state row per lane (d / 64, at least
// 1); RPW = rows per wave (M / 4); RFF = random Fourier feature map (its own
// instances, so that the SiLU maps keep their register count); ETA =
// normalised readout: the wave that owns state row m also carries the mode's
// normaliser eta_m (updated in place in eta [B][H][M][2]) and sums
// Re(s_m eta_m) into each token's denominator.  Tokens are [B][n][H][d].
template <bool BF16, int NT, int FJ, int RPW, bool RFF, bool ETA>
__global__ __launch_bounds__(256) void decode_step_kernel(Problem p, idattn_params prm,
                                                          const void* __restrict__ q_t,
                                                          const void* __restrict__ k_t,
                                                          const void* __restrict__ v_t,
                                                          void* __restrict__ o_t, float* state,
                                                          void* tail, float* eta) {
    __shared__ float xq_s[NT][128], zk_s[NT][128], zv_s[NT][128];
    __shared__ float4 coef_s[64];
    __shared__ float part_s[4][NT][128];
    __shared__ float den_s[4][NT];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t h = bh % p.H, b = bh / p.H;
    const int d = static_cast<int>(p.d), W = static_cast<int>(p.W);
    const int n = NT == 1 ? 1 : static_cast<int>(p.N);
    const int64_t M = p.M;
    const int nf = d;  // float4 chunks per row (4d floats)
    float4* st4 = reinterpret_cast<float4*>(state) + bh * M * nf;

    if (w == 0) {
        if constexpr (NT == 1) {
            // features of the new token; lane owns channels lane and lane + 64
            float cqv[2], ckv[2], yq[2], yk[2], vv[2];
            float sv = 0.f;
            const int64_t tok = bh * d;  // [B][H][d]
            const int64_t E = 2 * static_cast<int64_t>(W - 1) * d;
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = lane + kWave * j;
                float cq = 0.f, ck = 0.f;
                vv[j] = 0.f;
                if (c < d) {
                    const float* wq = prm.conv_q + (h * d + c) * W;
                    const float* wk = prm.conv_k + (h * d + c) * W;
                    float hq[8], hk[8];
                    for (int t = 0; t < W - 1; ++t) {
                        hq[t] = load_io<BF16>(tail, bh * E + static_cast<int64_t>(t) * d + c);
                        hk[t] = load_io<BF16>(tail, bh * E + static_cast<int64_t>(W - 1 + t) * d + c);
                    }
                    const float xq = load_io<BF16>(q_t, tok + c);
                    const float xk = load_io<BF16>(k_t, tok + c);
                    for (int t = 0; t < W - 1; ++t) {
                        cq = fmaf(wq[t], hq[t], cq);
                        ck = fmaf(wk[t], hk[t], ck);
                    }
                    cq = fmaf(wq[W - 1], xq, cq);
                    ck = fmaf(wk[W - 1], xk, ck);
                    // shift the tail by one token (this lane owns channel c)
                    for (int t = 0; t + 1 < W - 1; ++t) {
                        store_io<BF16>(tail, bh * E + static_cast<int64_t>(t) * d + c, hq[t + 1]);
                        store_io<BF16>(tail, bh * E + static_cast<int64_t>(W - 1 + t) * d + c, hk[t + 1]);
                    }
                    if (W > 1) {
                        store_io<BF16>(tail, bh * E + static_cast<int64_t>(W - 2) * d + c, xq);
                        store_io<BF16>(tail, bh * E + static_cast<int64_t>(2 * W - 3) * d + c, xk);
                    }
                    vv[j] = load_io<BF16>(v_t, tok + c);
                }
                cqv[j] = cq;
                ckv[j] = ck;
                sv = fmaf(vv[j], vv[j], sv);
            }
            sv = wave_total(sv);
            float inv_q, inv_k;
            token_features<RFF>(p, prm.rff_omega + h * d * (d / 2), cqv, ckv, yq, yk, inv_q, inv_k);
            float xk2 = 0.f, xik[2];
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                xik[j] = yk[j] * inv_k;
                xk2 = fmaf(xik[j], xik[j], xk2);
            }
            xk2 = wave_total(xk2);
            const float rk = 1.f / sqrtf(xk2 / d + p.eps_norm);
            const float rv = 1.f / sqrtf(sv / d + p.eps_norm);
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = lane + kWave * j;
                if (c < d) {
                    xq_s[0][c] = yq[j] * inv_q;
                    zk_s[0][c] = fmaf(prm.gain[h * 2 * d + c] * xik[j], rk, prm.bias[h * 2 * d + c]);
                    zv_s[0][c] = fmaf(prm.gain[h * 2 * d + d + c] * vv[j], rv, prm.bias[h * 2 * d + d + c]);
                }
            }
        } else {
            // features of the new tokens, one after another; lane owns channels lane and
            // lane + 64 and slides its own conv window (the last W-1 raw tokens, oldest
            // first) over the tail and the new tokens
            const int64_t E = 2 * static_cast<int64_t>(W - 1) * d;
            float hq[2][7], hk[2][7], wqh[2][7], wkh[2][7], wqc[2], wkc[2];
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = lane + kWave * j;
                const bool ok = c < d;
                wqc[j] = ok ? prm.conv_q[(h * d + c) * W + W - 1] : 0.f;
                wkc[j] = ok ? prm.conv_k[(h * d + c) * W + W - 1] : 0.f;
    #pragma unroll
                for (int u = 0; u < 7; ++u) {
                    const bool in = ok && u < W - 1;
                    wqh[j][u] = in ? prm.conv_q[(h * d + c) * W + u] : 0.f;
                    wkh[j][u] = in ? prm.conv_k[(h * d + c) * W + u] : 0.f;
                    hq[j][u] = in ? load_io<BF16>(tail, bh * E + static_cast<int64_t>(u) * d + c) : 0.f;
                    hk[j][u] = in ? load_io<BF16>(tail, bh * E + static_cast<int64_t>(W - 1 + u) * d + c) : 0.f;
                }
            }
    #pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < n) {
                    const int64_t tok = ((b * n + t) * p.H + h) * d;  // [B][n][H][d]
                    float cqv[2], ckv[2], yq[2], yk[2], vv[2];
                    float sv = 0.f;
    #pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int c = lane + kWave * j;
                        cqv[j] = ckv[j] = vv[j] = 0.f;
                        if (c < d) {
                            const float xq = load_io<BF16>(q_t, tok + c);
                            const float xk = load_io<BF16>(k_t, tok + c);
                            float cq = wqc[j] * xq, ck = wkc[j] * xk;
    #pragma unroll
                            for (int u = 0; u < 7; ++u) {
                                cq = fmaf(wqh[j][u], hq[j][u], cq);
                                ck = fmaf(wkh[j][u], hk[j][u], ck);
                            }
                            // slide the window by one token
    #pragma unroll
                            for (int u = 0; u < 7; ++u) {
                                hq[j][u] = u + 1 < W - 1 ? hq[j][u < 6 ? u + 1 : 6] : (u == W - 2 ? xq : hq[j][u]);
                                hk[j][u] = u + 1 < W - 1 ? hk[j][u < 6 ? u + 1 : 6] : (u == W - 2 ? xk : hk[j][u]);
                            }
                            vv[j] = load_io<BF16>(v_t, tok + c);
                            cqv[j] = cq;
                            ckv[j] = ck;
                        }
                        sv = fmaf(vv[j], vv[j], sv);
                    }
                    sv = wave_total(sv);
                    float inv_q, inv_k;
                    token_features<RFF>(p, prm.rff_omega + h * d * (d / 2), cqv, ckv, yq, yk, inv_q, inv_k);
                    float xk2 = 0.f, xik[2];
    #pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        xik[j] = yk[j] * inv_k;
                        xk2 = fmaf(xik[j], xik[j], xk2);
                    }
                    xk2 = wave_total(xk2);
                    const float rk = 1.f / sqrtf(xk2 / d + p.eps_norm);
                    const float rv = 1.f / sqrtf(sv / d + p.eps_norm);
    #pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int c = lane + kWave * j;
                        if (c < d) {
                            xq_s[t][c] = yq[j] * inv_q;
                            zk_s[t][c] = fmaf(prm.gain[h * 2 * d + c] * xik[j], rk, prm.bias[h * 2 * d + c]);
                            zv_s[t][c] = fmaf(prm.gain[h * 2 * d + d + c] * vv[j], rv, prm.bias[h * 2 * d + d + c]);
                        }
                    }
                }
            }
            // the new tail: the window after the last token (this lane owns channel c)
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = lane + kWave * j;
                if (c < d) {
    #pragma unroll
                    for (int u = 0; u < 7; ++u)
                        if (u < W - 1) {
                            store_io<BF16>(tail, bh * E + static_cast<int64_t>(u) * d + c, hq[j][u]);
                            store_io<BF16>(tail, bh * E + static_cast<int64_t>(W - 1 + u) * d + c, hk[j][u]);
                        }
                }
            }
        }
    } else if (w == 1 && lane < M) {
        // ZOH coefficients of mode lane, while wave 0 builds the features
        const double dt = exp(static_cast<double>(prm.log_dt[h]));
        coef_s[lane] = zoh_coef(dt, prm.A[(h * M + lane) * 2], prm.A[(h * M + lane) * 2 + 1],
                                prm.Bc[(h * M + lane) * 2], prm.Bc[(h * M + lane) * 2 + 1]);
    }
    __syncthreads();

    // ---- state sweep: one row at a time per wave, so that few registers are live
    // and many workgroups share a CU; they hide each other's memory latency.  A row
    // is read once, takes every token's update and readout in turn, and is written
    // once.
    float acc[NT][FJ][2];
    float den[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        den[t] = 0.f;
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[t][j][0] = acc[t][j][1] = 0.f;
    }
    // the next row is loaded while this one is updated
    float4 nxt[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
        const int f = lane + kWave * j;
        nxt[j] = f < nf ? load_stream(&st4[(w * RPW) * nf + f]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll 1
    for (int rr = 0; rr < RPW; ++rr) {
        const int m = w * RPW + rr;
        float4 row[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) row[j] = nxt[j];
        if (rr + 1 < RPW) {
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int f = lane + kWave * j;
                if (f < nf) nxt[j] = load_stream(&st4[(m + 1) * nf + f]);
            }
        }
        const float4 cf = coef_s[m];
        float er = 0.f, ei = 0.f;  // eta_m, the same in every lane
        if constexpr (ETA) {
            er = eta[(bh * M + m) * 2];
            ei = eta[(bh * M + m) * 2 + 1];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < n) {
                float pr = 0.f, pi = 0.f;
                // complex columns 2f and 2f+1; columns < d belong to U, the rest to Gamma
#pragma unroll
                for (int j = 0; j < FJ; ++j) {
                    const int f = lane + kWave * j;
                    if (f < nf) {
                        const int col = 2 * f;
                        const bool key = col < d;
                        const float in0 = key ? zk_s[t][col] : zv_s[t][col - d];
                        const float in1 = key ? zk_s[t][col + 1] : zv_s[t][col + 1 - d];
                        const float4 x = row[j];
                        const float r0 = fmaf(cf.x, x.x, fmaf(-cf.y, x.y, cf.z * in0));
                        const float i0 = fmaf(cf.x, x.y, fmaf(cf.y, x.x, cf.w * in0));
                        const float r1 = fmaf(cf.x, x.z, fmaf(-cf.y, x.w, cf.z * in1));
                        const float i1 = fmaf(cf.x, x.w, fmaf(cf.y, x.z, cf.w * in1));
                        row[j] = make_float4(r0, i0, r1, i1);
                        if (key) {
                            pr = fmaf(xq_s[t][col], r0, fmaf(xq_s[t][col + 1], r1, pr));
                            pi = fmaf(xq_s[t][col], i0, fmaf(xq_s[t][col + 1], i1, pi));
                        }
                    }
                }
                pr = wave_total(pr);
                pi = wave_total(pi);
                if constexpr (ETA) {
                    const float nr = fmaf(cf.x, er, fmaf(-cf.y, ei, cf.z));
                    const float ni = fmaf(cf.x, ei, fmaf(cf.y, er, cf.w));
                    er = nr;
                    ei = ni;
                    den[t] = fmaf(pr, nr, fmaf(-pi, ni, den[t]));
                }
#pragma unroll
                for (int j = 0; j < FJ; ++j) {
                    const int f = lane + kWave * j;
                    if (f < nf && 2 * f >= d) {
                        const float4 x = row[j];
                        acc[t][j][0] = fmaf(pr, x.x, fmaf(-pi, x.y, acc[t][j][0]));
                        acc[t][j][1] = fmaf(pr, x.z, fmaf(-pi, x.w, acc[t][j][1]));
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int f = lane + kWave * j;
            if (f < nf) store_stream(row[j], &st4[m * nf + f]);
        }
        if (ETA && lane == 0) {
            eta[(bh * M + m) * 2] = er;
            eta[(bh * M + m) * 2 + 1] = ei;
        }
    }
    if (ETA && lane == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) den_s[w][t] = den[t];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int f = lane + kWave * j;
            if (t < n && f < nf && 2 * f >= d) {
                part_s[w][t][2 * f - d] = acc[t][j][0];
                part_s[w][t][2 * f + 1 - d] = acc[t][j][1];
            }
        }
    __syncthreads();
    for (int e = threadIdx.x; e < n * d; e += 256) {
        const int t = e / d, c = e % d;
        float sum = (part_s[0][t][c] + part_s[1][t][c]) + (part_s[2][t][c] + part_s[3][t][c]);
        if constexpr (ETA) sum /= (den_s[0][t] + den_s[1][t]) + (den_s[2][t] + den_s[3][t]);
        store_io<BF16>(o_t, ((b * n + t) * p.H + h) * d + c, sum);
    }
}

}  // namespace

hipError_t launch_decode_step(const Problem& p, const idattn_params& prm, const void* q_t,
                              const void* k_t, const void* v_t, void* o_t, float* state,
                              void* tail, float* eta, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.B * p.H));
#define IDATTN_DEC_K(BF, NT, FJ, RPW, ETA)                                                                      \
    do {                                                                                                        \
        if (p.rff_feat)                                                                                         \
            decode_step_kernel<BF, NT, FJ, RPW, true, ETA><<<grid, 256, 0, stream>>>(p, prm, q_t, k_t, v_t, o_t, state, tail, eta);  \
        else                                                                                                    \
            decode_step_kernel<BF, NT, FJ, RPW, false, ETA><<<grid, 256, 0, stream>>>(p, prm, q_t, k_t, v_t, o_t, state, tail, eta); \
    } while (0)
#define IDATTN_DEC_NT(NT, FJ, RPW, ETA)                  \
    do {                                                 \
        if (p.bf16) IDATTN_DEC_K(true, NT, FJ, RPW, ETA);  \
        else IDATTN_DEC_K(false, NT, FJ, RPW, ETA);        \
    } while (0)
    // the normalised readout has the several-token instances only (any 1..8 tokens)
#define IDATTN_DEC(FJ, RPW)                                           \
    do {                                                              \
        if (eta != nullptr) IDATTN_DEC_NT(kDecodeMaxTokens, FJ, RPW, true); \
        else if (p.N == 1) IDATTN_DEC_NT(1, FJ, RPW, false);          \
        else IDATTN_DEC_NT(kDecodeMaxTokens, FJ, RPW, false);         \
    } while (0)
    const int fj = p.d > 64 ? 2 : 1;
    const int rpw = static_cast<int>(p.M / 4);
    if (fj == 2 && rpw == 16) IDATTN_DEC(2, 16);
    else if (fj == 2 && rpw == 8) IDATTN_DEC(2, 8);
    else if (fj == 2 && rpw == 4) IDATTN_DEC(2, 4);
    else if (fj == 1 && rpw == 16) IDATTN_DEC(1, 16);
    else if (fj == 1 && rpw == 8) IDATTN_DEC(1, 8);
    else if (fj == 1 && rpw == 4) IDATTN_DEC(1, 4);
    else return hipErrorInvalidValue;
#undef IDATTN_DEC
#undef IDATTN_DEC_NT
#undef IDATTN_DEC_K
    return hipGetLastError();
}

}  // namespace idattn

// Backward pass of the mixer: gradients of a scalar loss
//   L = sum grad_o . o + Re sum conj(grad_state) . state_out
// with respect to q, k, v, every parameter and the carried state, in fp32 and
// one time step after another (the sequential algorithm).  The pages train
// the layer inside language models (Chinese rendering, abstract and section
// 1; German summary, "Skalierbare Implementierung"), which is what needs these
// gradients; they print no backward pass, so this differentiates the forward
// exactly as it is read (plain bilinear products, per-half RMSNorm, ZOH).
//
// Complex gradients follow g_z = dL/dRe z + i dL/dIm z; for a holomorphic
// map w = f(z) that gives g_z = conj(f'(z)) g_w.  Per (b, h), with the
// forward's U_m(i), Gamma_m(i), s_m(i) = xi_q(i) . U_m(i):
//   g_s_m(i)   = sum_c g_o(i)_c conj(Gamma_m,c(i))
//   g_xi_q(i)  = sum_m Re(g_s_m(i) conj(U_m(i)))
//   Ubar(i)    = xi_q(i) g_s(i) + conj(abar) Ubar(i+1)      (reverse time)
//   Gbar(i)    = g_o(i) conj(s(i)) + conj(abar) Gbar(i+1)   (reverse time)
//   g_z_k(i)   = Re sum_m conj(bbar_m) Ubar_m(i),   g_z_v likewise with Gbar
//   g_bbar_m   = sum_i [Ubar_m(i) . z_k(i) + Gbar_m(i) . z_v(i)]
//   g_abar_m   = sum_i [g_s_m(i) conj(xi_q(i) . V_m(i)) + conj(s_m(i)) sum_c g_o(i)_c conj(W_m,c(i))]
//                (+ the state_out terms), with V = dU/dabar and W = dGamma/dabar
//                carried forward: V(i) = abar V(i-1) + U(i-1), W likewise.
// g_abar is taken in this forward form so that no kernel needs U or Gamma
// in reverse time order.  The state_in gradient is conj(abar) Ubar(0) (and
// Gbar).  Feature maps, RMSNorm and the conv are differentiated per token.
// Parameter gradients are sums over batch rows and tokens: each wave writes
// its partial sums, and one kernel adds them in a fixed order (no atomics).
#include "common.h"
#include "launch.h"

namespace idattn {

namespace {

constexpr int kTok = 8;    // tokens per batch of the per-mode scans
constexpr int kBlk = 16;   // tokens per LDS round of the per-channel scans
constexpr int kVW = 16;    // waves per per-channel scan block
constexpr int kRun = 32;   // tokens per wave in the feature and conv kernels

__device__ __forceinline__ Zoh zoh_of(const idattn_params& prm, int64_t h, int64_t M, int64_t m) {
    return zoh_mode(prm.log_dt[h], prm.A[(h * M + m) * 2], prm.A[(h * M + m) * 2 + 1], prm.Bc[(h * M + m) * 2],
                    prm.Bc[(h * M + m) * 2 + 1]);
}

// ------------------------------------------------------------------ per-mode scans
// One half-wave per (b, h, m), two modes per wave, so that each reduction
// over the channels runs over 32 lanes and serves both modes at once.  Lane l
// of a half owns the RJ adjacent channels RJ l .. RJ l + RJ - 1, so that a
// token's values of them are one load.
//
// Each scan takes kTok tokens at a time.  All their loads are issued first,
// at token and channel indices clamped into range (addressed from a uniform
// base with 32-bit lane offsets); a ragged batch (fewer than kTok tokens left,
// or d below 32 RJ) then zeroes what lies out of range and steps only its
// tokens.  A full batch runs with no per-token condition.

// One batch of the key-side recurrence: V(i) = abar V(i-1) + U(i-1), then
// U(i) = abar U(i-1) + bbar z_k(i); the lane's shares of s = xi_q . U and
// s_a = xi_q . V per token.  SCALED: the lane carries U / bbar and V / bbar,
// which take the input unscaled.
template <int RJ, bool RAGGED, bool SCALED>
__device__ __forceinline__ void key_batch(int nt, float (&ur)[RJ], float (&ui)[RJ], float (&vr)[RJ], float (&vi)[RJ],
                                          const float (&xv)[kTok][RJ], const float (&zv)[kTok][RJ], float ar, float ai,
                                          float br, float bi, float (&spr)[kTok], float (&spi)[kTok],
                                          float (&sqr)[kTok], float (&sqi)[kTok]) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        float pr = 0.f, pi = 0.f, qr = 0.f, qi = 0.f;
        if (!RAGGED || t < nt) {
#pragma unroll
            for (int j = 0; j < RJ; ++j) {
                const float nvr = fmaf(ar, vr[j], fmaf(-ai, vi[j], ur[j]));
                const float nvi = fmaf(ar, vi[j], fmaf(ai, vr[j], ui[j]));
                const float nur = fmaf(ar, ur[j], fmaf(-ai, ui[j], SCALED ? zv[t][j] : br * zv[t][j]));
                const float nui = SCALED ? fmaf(ar, ui[j], ai * ur[j]) : fmaf(ar, ui[j], fmaf(ai, ur[j], bi * zv[t][j]));
                vr[j] = nvr;
                vi[j] = nvi;
                ur[j] = nur;
                ui[j] = nui;
                pr = fmaf(xv[t][j], nur, pr);
                pi = fmaf(xv[t][j], nui, pi);
                qr = fmaf(xv[t][j], nvr, qr);
                qi = fmaf(xv[t][j], nvi, qi);
            }
        }
        spr[t] = pr;
        spi[t] = pi;
        sqr[t] = qr;
        sqi[t] = qi;
    }
}

// One batch of the value-side recurrence: W(i) = abar W(i-1) + Gamma(i-1),
// then Gamma(i) = abar Gamma(i-1) + bbar z_v(i); the lane's shares of
// g_s = sum_c g_o[c] conj(Gamma_c) and gw = sum_c g_o[c] conj(W_c) per token.
// SCALED: the lane carries Gamma / bbar and W / bbar, which take the input
// unscaled.
template <int RJ, bool RAGGED, bool SCALED>
__device__ __forceinline__ void value_batch(int nt, float (&gmr)[RJ], float (&gmi)[RJ], float (&wr)[RJ],
                                            float (&wi)[RJ], const float (&zz)[kTok][RJ], const float (&go)[kTok][RJ],
                                            float ar, float ai, float br, float bi, float (&spr)[kTok],
                                            float (&spi)[kTok], float (&sqr)[kTok], float (&sqi)[kTok]) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        float pr = 0.f, pi = 0.f, qr = 0.f, qi = 0.f;
        if (!RAGGED || t < nt) {
#pragma unroll
            for (int j = 0; j < RJ; ++j) {
                const float nwr = fmaf(ar, wr[j], fmaf(-ai, wi[j], gmr[j]));
                const float nwi = fmaf(ar, wi[j], fmaf(ai, wr[j], gmi[j]));
                const float ngr = fmaf(ar, gmr[j], fmaf(-ai, gmi[j], SCALED ? zz[t][j] : br * zz[t][j]));
                const float ngi = SCALED ? fmaf(ar, gmi[j], ai * gmr[j]) : fmaf(ar, gmi[j], fmaf(ai, gmr[j], bi * zz[t][j]));
                wr[j] = nwr;
                wi[j] = nwi;
                gmr[j] = ngr;
                gmi[j] = ngi;
                pr = fmaf(go[t][j], ngr, pr);
                pi = fmaf(-go[t][j], ngi, pi);
                qr = fmaf(go[t][j], nwr, qr);
                qi = fmaf(-go[t][j], nwi, qi);
            }
        }
        spr[t] = pr;
        spi[t] = pi;
        sqr[t] = qr;
        sqi[t] = qi;
    }
}
//
// Key side: U and V = dU/dabar; writes s = xi_q . U and s_a = xi_q . V
// [H][T][M] and, when the state_out gradient is given, the mode's share
// sum_r g_S,U[r] conj(V_r(N-1)) of g_abar to ga_key [B H][M].
// SCALED (no state enters): U and V are carried divided by bbar, which then
// multiplies each token's reduced s and s_a and the state-gradient sum; the
// key side's state_out share of the g_bbar sum, sum_r g_S,U[r] conj(U_r(N-1)
// / bbar), goes to gb_key [B H][M] (zero without a state_out gradient).
template <int RJ, bool SCALED>
__global__ __launch_bounds__(256) void bwd_key_scan_kernel(Problem p, idattn_params prm, const float* __restrict__ xi_q,
                                                           const float* __restrict__ z_k, const float* state_in,
                                                           const float* grad_state, float2* __restrict__ s,
                                                           float2* __restrict__ s_a, float2* __restrict__ ga_key,
                                                           float2* __restrict__ gb_key) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 31;  // the lane in its half
    const int64_t bh = blockIdx.x;
    const int64_t m0 = (static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6)) * 2;  // the wave's first mode
    const int64_t M = p.M, N = p.N;
    const int d = static_cast<int>(p.d);
    if (m0 >= M) return;  // whole wave; no barriers in this kernel
    const bool mok = m0 + (lane >> 5) < M;  // false for the second half of the last wave when M is odd
    const int64_t m = mok ? m0 + (lane >> 5) : M - 1;
    const int64_t h = bh % p.H;
    const Zoh z = zoh_of(prm, h, M, m);
    const float ar = static_cast<float>(z.ar), ai = static_cast<float>(z.ai);
    const float br = static_cast<float>(z.br), bi = static_cast<float>(z.bi);
    const int64_t st_row = ((bh * M + m) * 2 * d) * 2;
    const float2 fix = decay_fix(z, kFixTok);
    float ur[RJ], ui[RJ], vr[RJ], vi[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int r = RJ * li + j;
        ur[j] = ui[j] = vr[j] = vi[j] = 0.f;
        if (state_in != nullptr && mok && r < d) {
            ur[j] = state_in[st_row + 2 * r];
            ui[j] = state_in[st_row + 2 * r + 1];
        }
    }
    const int64_t row0 = h * p.T + (bh / p.H) * N;
    const bool dfull = d == 32 * RJ;
    const uint32_t coff = 4u * static_cast<uint32_t>(min(RJ * li, d - RJ));  // byte offset of the lane's channels
    // one batch's rows into x, z (tokens clamped below the batch's nt)
    auto fetch = [&](int64_t j0, int jnt, float (&x)[kTok][RJ], float (&zq)[kTok][RJ]) {
        const int64_t row = (row0 + j0) * d;  // uniform
        const uint32_t nb = static_cast<uint32_t>(jnt * d * 4);
        const __amdgpu_buffer_rsrc_t xr = rsrc_at(xi_q + row, nb), zr = rsrc_at(z_k + row, nb);
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            const uint32_t tb = static_cast<uint32_t>(min(t, jnt - 1) * d * 4);
            buf_load_run<RJ>(x[t], xr, coff, tb);
            buf_load_run<RJ>(zq[t], zr, coff, tb);
        }
    };
    // one batch from x, z while the batch at j0 is loaded into xn, zn (the last
    // batch loads itself again), so that no batch waits on memory
    auto step = [&](int64_t i0, float (&x)[kTok][RJ], float (&zq)[kTok][RJ], float (&xn)[kTok][RJ],
                    float (&zn)[kTok][RJ]) {
        const int nt = static_cast<int>(min(N - i0, static_cast<int64_t>(kTok)));
        const int64_t j0 = i0 + kTok < N ? i0 + kTok : i0;
        fetch(j0, static_cast<int>(min(N - j0, static_cast<int64_t>(kTok))), xn, zn);
        // the lane's shares of s and s_a of the kTok tokens, then one reduce-scatter
        // per quantity (lane t < 8 of a half ends with token slot8(t)'s totals)
        float spr[kTok], spi[kTok], sqr[kTok], sqi[kTok];
        if (nt == kTok && dfull) {
            key_batch<RJ, false, SCALED>(nt, ur, ui, vr, vi, x, zq, ar, ai, br, bi, spr, spi, sqr, sqi);
        } else {
#pragma unroll
            for (int t = 0; t < kTok; ++t)
#pragma unroll
                for (int j = 0; j < RJ; ++j)
                    if (t >= nt || RJ * li + j >= d) x[t][j] = zq[t][j] = 0.f;
            key_batch<RJ, true, SCALED>(nt, ur, ui, vr, vi, x, zq, ar, ai, br, bi, spr, spi, sqr, sqi);
        }
        static_assert(kFixTok % kTok == 0, "the decay fix at a batch's end");
        if (nt == kTok && i0 % kFixTok == kFixTok - kTok) {  // uniform
#pragma unroll
            for (int j = 0; j < RJ; ++j) {
                apply_fix(fix, ur[j], ui[j]);
                apply_fix(fix, vr[j], vi[j]);
            }
        }
        static_assert(kTok == 8, "one reduce-scatter per kTok tokens");
        float tpr = half_reduce_scatter8(spr, lane), tpi = half_reduce_scatter8(spi, lane);
        float tqr = half_reduce_scatter8(sqr, lane), tqi = half_reduce_scatter8(sqi, lane);
        if constexpr (SCALED) {  // times bbar
            const float a = br * tpr - bi * tpi, c = br * tqr - bi * tqi;
            tpi = fmaf(br, tpi, bi * tpr);
            tqi = fmaf(br, tqi, bi * tqr);
            tpr = a;
            tqr = c;
        }
        const int t = slot8(li);
        if (li < kTok && t < nt && mok) {
            s[(row0 + i0 + t) * M + m] = make_float2(tpr, tpi);
            s_a[(row0 + i0 + t) * M + m] = make_float2(tqr, tqi);
        }
    };
    float xa[kTok][RJ], za[kTok][RJ], xb[kTok][RJ], zb[kTok][RJ];  // two batches' rows, in turn
    if (N > 0) fetch(0, static_cast<int>(min(N, static_cast<int64_t>(kTok))), xa, za);
    for (int64_t i0 = 0; i0 < N; i0 += 2 * kTok) {
        step(i0, xa, za, xb, zb);
        if (i0 + kTok >= N) break;
        step(i0 + kTok, xb, zb, xa, za);
    }
    float ur_ = 0.f, ui_ = 0.f;  // SCALED: sum_r g_S[r] conj(U_r / bbar)
    if (grad_state != nullptr) {
        float gr = 0.f, gi = 0.f;  // sum_r g_S[r] conj(V_r)
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int r = RJ * li + j;
            if (r < d) {
                const float sr = grad_state[st_row + 2 * r], si = grad_state[st_row + 2 * r + 1];
                gr = fmaf(sr, vr[j], fmaf(si, vi[j], gr));
                gi = fmaf(si, vr[j], fmaf(-sr, vi[j], gi));
                if constexpr (SCALED) {
                    ur_ = fmaf(sr, ur[j], fmaf(si, ui[j], ur_));
                    ui_ = fmaf(si, ur[j], fmaf(-sr, ui[j], ui_));
                }
            }
        }
        gr = half_total(gr);
        gi = half_total(gi);
        if constexpr (SCALED) {  // times conj(bbar)
            const float a = fmaf(br, gr, bi * gi);
            gi = br * gi - bi * gr;
            gr = a;
            ur_ = half_total(ur_);
            ui_ = half_total(ui_);
        }
        if (li == 0 && mok) ga_key[bh * M + m] = make_float2(gr, gi);
    }
    if constexpr (SCALED)
        if (li == 0 && mok) gb_key[bh * M + m] = make_float2(ur_, ui_);
}

// Value side: Gamma and W = dGamma/dabar, driven by z_v; per token
// g_s = sum_c g_o[c] conj(Gamma_c) (to gs [H][T][M]) and
// gw = sum_c g_o[c] conj(W_c); the mode's g_abar partial
// sum_i [conj(s) gw + g_s conj(s_a)] plus the state_out terms goes to
// ga [B H][M].  SCALED (no state enters): Gamma and W are carried divided by
// bbar, and conj(bbar) multiplies each token's reduced g_s and gw and the
// state-gradient sum.  Then the g_bbar sums of both adjoints also follow from
// per-token totals: with G = sum_c g_o[c] conj(Gamma_c / bbar) (g_s before
// its conj(bbar)), each adjoint's sum_i sum_c A(i)_c z(i)_c is
// sum_i G(i) conj(s(i)) plus its state_out share; the value scan writes
// 2 sum_i G conj(s) + sum_c g_S,Gamma[c] conj(Gamma_c(N-1) / bbar) to
// gb_val [B H][M] and the key scan its own share to gb_key.
template <int RJ, bool BF16, bool SCALED>
__global__ __launch_bounds__(256) void bwd_value_scan_kernel(Problem p, idattn_params prm, const float* __restrict__ z_v,
                                                             const void* __restrict__ grad_o, const float* state_in,
                                                             const float* grad_state, const float2* __restrict__ s,
                                                             const float2* __restrict__ s_a,
                                                             const float2* __restrict__ ga_key,
                                                             float2* __restrict__ gs, float2* __restrict__ ga,
                                                             float2* __restrict__ gb_val) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 31;  // the lane in its half
    const int64_t bh = blockIdx.x;
    const int64_t m0 = (static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6)) * 2;  // the wave's first mode
    const int64_t M = p.M, N = p.N, H = p.H;
    const int d = static_cast<int>(p.d);
    if (m0 >= M) return;  // whole wave; no barriers in this kernel
    const bool mok = m0 + (lane >> 5) < M;  // false for the second half of the last wave when M is odd
    const int64_t m = mok ? m0 + (lane >> 5) : M - 1;
    const int64_t b = bh / H, h = bh % H;
    const Zoh z = zoh_of(prm, h, M, m);
    const float ar = static_cast<float>(z.ar), ai = static_cast<float>(z.ai);
    const float br = static_cast<float>(z.br), bi = static_cast<float>(z.bi);
    const int64_t st_row = ((bh * M + m) * 2 * d) * 2;
    const float2 fix = decay_fix(z, kFixTok);
    float gmr[RJ], gmi[RJ], wr[RJ], wi[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int c = RJ * li + j;
        gmr[j] = gmi[j] = wr[j] = wi[j] = 0.f;
        if (state_in != nullptr && mok && c < d) {
            gmr[j] = state_in[st_row + 2 * (d + c)];
            gmi[j] = state_in[st_row + 2 * (d + c) + 1];
        }
    }
    const int64_t row0 = h * p.T + b * N;
    const float* zvp = z_v + row0 * d;
    double accr = 0.0, acci = 0.0;  // g_abar share of this mode
    double bcr = 0.0, bci = 0.0;    // SCALED: sum_i G conj(s)
    const bool dfull = d == 32 * RJ;
    const int ts = slot8(li);  // the token whose totals this lane ends with
    const uint32_t coff = static_cast<uint32_t>(min(RJ * li, d - RJ));  // the lane's first channel (clamped)
    constexpr uint32_t kIoB = BF16 ? 2 : 4;  // bytes per element of grad_o
    const uint32_t gstride = static_cast<uint32_t>(H * d) * kIoB;  // bytes per token of grad_o
    for (int64_t i0 = 0; i0 < N; i0 += kTok) {
        const int nt = static_cast<int>(min(N - i0, static_cast<int64_t>(kTok)));
        float zz[kTok][RJ], go[kTok][RJ];
        const __amdgpu_buffer_rsrc_t zr = rsrc_at(zvp + i0 * d, static_cast<uint32_t>(nt * d * 4));
        const __amdgpu_buffer_rsrc_t gr = rsrc_at(
            static_cast<const char*>(grad_o) + ((b * N + i0) * H + h) * d * kIoB, static_cast<uint32_t>(nt) * gstride);
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            const uint32_t tt = static_cast<uint32_t>(min(t, nt - 1));
            buf_load_run<RJ>(zz[t], zr, 4u * coff, tt * static_cast<uint32_t>(d) * 4u);
            buf_load_io_run<RJ, BF16>(go[t], gr, kIoB * coff, tt * gstride);
        }
        const int64_t sidx = (row0 + i0 + min(ts, nt - 1)) * M + m;
        const float2 sv = s[sidx], sa = s_a[sidx];  // used after the reduce-scatter
        // the lane's shares of g_s and gw of the kTok tokens, then one reduce-scatter
        // per quantity (lane t < 8 ends with token slot8(t)'s totals)
        float spr[kTok], spi[kTok], sqr[kTok], sqi[kTok];
        if (nt == kTok && dfull) {
            value_batch<RJ, false, SCALED>(nt, gmr, gmi, wr, wi, zz, go, ar, ai, br, bi, spr, spi, sqr, sqi);
        } else {
#pragma unroll
            for (int t = 0; t < kTok; ++t)
#pragma unroll
                for (int j = 0; j < RJ; ++j)
                    if (t >= nt || RJ * li + j >= d) zz[t][j] = go[t][j] = 0.f;
            value_batch<RJ, true, SCALED>(nt, gmr, gmi, wr, wi, zz, go, ar, ai, br, bi, spr, spi, sqr, sqi);
        }
        if (nt == kTok && i0 % kFixTok == kFixTok - kTok) {  // uniform
#pragma unroll
            for (int j = 0; j < RJ; ++j) {
                apply_fix(fix, gmr[j], gmi[j]);
                apply_fix(fix, wr[j], wi[j]);
            }
        }
        static_assert(kTok == 8, "one reduce-scatter per kTok tokens");
        float pr = half_reduce_scatter8(spr, lane), pi = half_reduce_scatter8(spi, lane);
        float qr = half_reduce_scatter8(sqr, lane), qi = half_reduce_scatter8(sqi, lane);
        const float g0r = pr, g0i = pi;  // G before its conj(bbar)
        if constexpr (SCALED) {  // times conj(bbar)
            const float a = fmaf(br, pr, bi * pi), c = fmaf(br, qr, bi * qi);
            pi = br * pi - bi * pr;
            qi = br * qi - bi * qr;
            pr = a;
            qr = c;
        }
        if (li < kTok && ts < nt && mok) {
            gs[sidx] = make_float2(pr, pi);
            if constexpr (SCALED) {  // G conj(s)
                bcr += static_cast<double>(g0r) * sv.x + static_cast<double>(g0i) * sv.y;
                bci += static_cast<double>(g0i) * sv.x - static_cast<double>(g0r) * sv.y;
            }
            // conj(s) gw + g_s conj(s_a), summed per lane (every eighth token) in fp64
            accr += static_cast<double>(sv.x * qr + sv.y * qi) + static_cast<double>(pr * sa.x + pi * sa.y);
            acci += static_cast<double>(sv.x * qi - sv.y * qr) + static_cast<double>(pi * sa.x - pr * sa.y);
        }
    }
    // the eight lanes' sums of each half in a fixed order (the other lanes hold zeros)
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
        accr += __shfl_xor(accr, off, kWave);
        acci += __shfl_xor(acci, off, kWave);
        if constexpr (SCALED) {
            bcr += __shfl_xor(bcr, off, kWave);
            bci += __shfl_xor(bci, off, kWave);
        }
    }
    bcr *= 2.0;  // the key and the value adjoint
    bci *= 2.0;
    if (grad_state != nullptr) {
        float gr = 0.f, gi = 0.f;  // sum_c g_S[c] conj(W_c)
        float tr = 0.f, ti = 0.f;  // SCALED: sum_c g_S[c] conj(Gamma_c / bbar)
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int c = RJ * li + j;
            if (c < d) {
                const float sr = grad_state[st_row + 2 * (d + c)], si = grad_state[st_row + 2 * (d + c) + 1];
                gr = fmaf(sr, wr[j], fmaf(si, wi[j], gr));
                gi = fmaf(si, wr[j], fmaf(-sr, wi[j], gi));
                if constexpr (SCALED) {
                    tr = fmaf(sr, gmr[j], fmaf(si, gmi[j], tr));
                    ti = fmaf(si, gmr[j], fmaf(-sr, gmi[j], ti));
                }
            }
        }
        gr = half_total(gr);
        gi = half_total(gi);
        if constexpr (SCALED) {  // times conj(bbar)
            const float a = fmaf(br, gr, bi * gi);
            gi = br * gi - bi * gr;
            gr = a;
            tr = half_total(tr);
            ti = half_total(ti);
            bcr += tr;
            bci += ti;
        }
        if (li == 0) {
            const float2 k = ga_key[bh * M + m];
            accr += static_cast<double>(gr) + k.x;
            acci += static_cast<double>(gi) + k.y;
        }
    }
    if (li == 0 && mok) {
        ga[bh * M + m] = make_float2(static_cast<float>(accr), static_cast<float>(acci));
        if constexpr (SCALED) gb_val[bh * M + m] = make_float2(static_cast<float>(bcr), static_cast<float>(bci));
    }
}

// Sum of x[0..K) in a fixed pairwise order (deterministic).
template <int K>
__device__ __forceinline__ float tree_sum(float (&x)[K]) {
#pragma unroll
    for (int step = 1; step < K; step *= 2)
#pragma unroll
        for (int i = 0; i + step < K; i += 2 * step) x[i] += x[i + step];
    return x[0];
}

// ------------------------------------------------------------------ per-channel scans
// One block per (b, h, 64-channel group, mode split z): wave w owns modes
// z kVW MW + [w MW, (w+1) MW), lane l one channel c; per token the waves'
// partial sums over their modes meet in LDS and are added in a fixed order.
// With two mode splits (M >= 32, so that the chip has twice the blocks),
// each split writes its partial sums to its own copy of the output, zs
// floats apart, and the feature kernel adds the two.
//
// Tokens go in blocks of kBlk.  The block's threads stage one block's inputs
// in LDS, one element of each per thread: the per-token mode input (kBlk x M
// complex) and the channel inputs (kBlk x 64).  The next block's elements are
// loaded into registers while this block's tokens are stepped, so no wave
// waits on memory between blocks; two barriers per block.
constexpr int kStage = kVW * kWave;  // threads per block = staged elements per input
static_assert(kBlk * kWave == kStage, "one channel-input element per thread");
static_assert(kBlk * 64 <= kStage, "one mode-input element per thread for M <= 64");

// One thread's staged elements of the block of tokens [i0, i0 + nt): the mode
// input of (token e / M, mode e % M) and the channel inputs of (token e / 64,
// channel 64 group + e % 64), e = threadIdx.x, loaded at indices clamped into
// the block and below d.  x is kept as loaded (bf16 bits or fp32 bits) and
// widened when it is stored, so that nothing waits on the loads before then.
struct Stage {
    float2 w;
    uint32_t xb;
    float z;
};

// X: whether the scan has a channel input x; X_IO: x is the caller's [B][N][H][d]
// tensor (else the workspace's [H][T][d] fp32); BF16: its elements are bf16.
template <bool X, bool X_IO, bool BF16>
__device__ __forceinline__ Stage stage_fetch(const Problem& p, int64_t b, int64_t h, int64_t row0, int64_t i0, int nt,
                                             int group, const float2* __restrict__ wv, const void* __restrict__ x,
                                             const float* __restrict__ zsrc) {
    const int e = static_cast<int>(threadIdx.x);
    const int M = static_cast<int>(p.M), d = static_cast<int>(p.d);
    Stage s;
    s.w = wv[(row0 + i0 + min(e / M, nt - 1)) * M + e % M];
    const int64_t ti = i0 + min(e / kWave, nt - 1);
    const uint32_t cl = static_cast<uint32_t>(min(group * kWave + e % kWave, d - 1));
    s.z = (zsrc + (row0 + ti) * d)[cl];
    s.xb = 0u;
    if constexpr (X) {
        if constexpr (X_IO) {
            const int64_t xr = ((b * p.N + ti) * p.H + h) * d;
            if constexpr (BF16) s.xb = (static_cast<const uint16_t*>(x) + xr)[cl];
            else s.xb = (static_cast<const uint32_t*>(x) + xr)[cl];
        } else {
            s.xb = (static_cast<const uint32_t*>(x) + (row0 + ti) * d)[cl];
        }
    }
    return s;
}

// The staged elements into LDS, zero past the block's nt tokens and past d.
template <bool X, bool BF16>
__device__ __forceinline__ void stage_store(const Stage& s, int nt, int M, int group, int d, float2* w_blk,
                                            float* x_blk, float* z_blk) {
    const int e = static_cast<int>(threadIdx.x);
    w_blk[e] = e < nt * M ? s.w : make_float2(0.f, 0.f);
    const bool ok = e / kWave < nt && group * kWave + e % kWave < d;
    z_blk[e] = ok ? s.z : 0.f;
    if constexpr (X) x_blk[e] = ok ? __uint_as_float(BF16 ? s.xb << 16 : s.xb) : 0.f;
}

// The waves' partial sums of the block's tokens, added in a fixed order, to
// out [token][d] (rows row0 + i0 .. row0 + i0 + nt - 1).
__device__ __forceinline__ void reduce_block(const float (*red)[kBlk][kWave], int nt, int group, int d,
                                             float* __restrict__ out) {
    for (int e = static_cast<int>(threadIdx.x); e < nt * kWave; e += kStage) {
        const int t = e / kWave, l = e % kWave;
        const int cc = group * kWave + l;
        if (cc < d) {
            float part[kVW];
#pragma unroll
            for (int i = 0; i < kVW; ++i) part[i] = red[i][t][l];
            out[static_cast<int64_t>(t) * d + cc] = tree_sum(part);
        }
    }
}

// g_xi_q(i)_r = sum_m Re(g_s_m(i) conj(U_m,r(i))), U run forward again from
// state_in; the result goes to g_xi [H][T][d].
// One block of kBlk tokens of the xi scan for the wave's MW modes: U steps
// forward and the wave's share sum_m Re(g_s conj(U_m)) of each token goes to
// red.  A ragged block steps only its first nt tokens.  SCALED: the lane
// carries U / bbar, which takes the input unscaled, and the staged g_s carry
// the factor conj(bbar) instead.
template <int MW, bool RAGGED, bool SCALED>
__device__ __forceinline__ void xi_block(int nt, const float2* g_row, const float* z_col, float (*red_t)[kWave],
                                         int lane, const float (&ar)[MW], const float (&ai)[MW],
                                         const float (&br)[MW], const float (&bi)[MW], float (&ur)[MW],
                                         float (&ui)[MW], int M) {
#pragma unroll
    for (int t = 0; t < kBlk; ++t) {
        if (RAGGED && t >= nt) continue;
        const float zz = z_col[t * kWave];
        float acc = 0.f;
#pragma unroll
        for (int mm = 0; mm < MW; ++mm) {
            const float2 g = g_row[t * M + mm];
            const float nr = fmaf(ar[mm], ur[mm], fmaf(-ai[mm], ui[mm], SCALED ? zz : br[mm] * zz));
            const float ni = SCALED ? fmaf(ar[mm], ui[mm], ai[mm] * ur[mm])
                                    : fmaf(ar[mm], ui[mm], fmaf(ai[mm], ur[mm], bi[mm] * zz));
            ur[mm] = nr;
            ui[mm] = ni;
            acc = fmaf(g.x, nr, fmaf(g.y, ni, acc));  // Re(g conj(U))
        }
        red_t[t][lane] = acc;
    }
}

// SCALED (no state enters): U is carried as U / bbar and each staged g_s
// element is multiplied by conj(bbar) of its mode.
template <int MW, bool SCALED>
__global__ __launch_bounds__(kStage) void bwd_xi_scan_kernel(Problem p, idattn_params prm,
                                                             const float* __restrict__ z_k, const float* state_in,
                                                             const float2* __restrict__ gs,
                                                             float* __restrict__ g_xi, int64_t zs) {
    __shared__ float2 w_blk[kStage];
    __shared__ float z_blk[kStage];
    __shared__ float red[kVW][kBlk][kWave];
    __shared__ float2 cb_s[SCALED ? 64 : 1];  // conj(bbar) of every mode (M <= 64)
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t N = p.N;
    const int M = static_cast<int>(p.M), d = static_cast<int>(p.d);
    const int group = static_cast<int>(blockIdx.y);
    const int c = group * kWave + lane;
    const bool cok = c < d;
    const int64_t row0 = h * p.T + b * N;
    const int moff = static_cast<int>(blockIdx.z) * kVW * MW;  // the split's first mode
    if (N <= 0) return;  // whole block
    g_xi += blockIdx.z * zs;
    float ar[MW], ai[MW], br[MW], bi[MW], ur[MW], ui[MW];
    float2 fix[MW];  // the decay fix of a full block (kBlk steps by abar_f)
#pragma unroll
    for (int mm = 0; mm < MW; ++mm) {
        const int64_t m = moff + w * MW + mm;
        const Zoh zz = zoh_of(prm, h, M, m);
        ar[mm] = static_cast<float>(zz.ar);
        ai[mm] = static_cast<float>(zz.ai);
        br[mm] = static_cast<float>(zz.br);
        bi[mm] = static_cast<float>(zz.bi);
        fix[mm] = decay_fix(zz, kBlk);
        ur[mm] = ui[mm] = 0.f;
        if (state_in != nullptr && cok) {
            const int64_t idx = ((bh * M + m) * 2 * d + c) * 2;
            ur[mm] = state_in[idx];
            ui[mm] = state_in[idx + 1];
        }
    }
    float2 cbe = make_float2(1.f, 0.f);  // conj(bbar) of the mode this thread stages
    if constexpr (SCALED) {
        if (threadIdx.x < M) {
            const Zoh zm = zoh_of(prm, h, M, threadIdx.x);
            cb_s[threadIdx.x] = make_float2(static_cast<float>(zm.br), -static_cast<float>(zm.bi));
        }
        __syncthreads();
        cbe = cb_s[threadIdx.x % M];
    }
    const float2* g_row = w_blk + moff + w * MW;
    int64_t i0 = 0;
    int nt = static_cast<int>(min(N, static_cast<int64_t>(kBlk)));
    Stage nx = stage_fetch<false, false, false>(p, b, h, row0, i0, nt, group, gs, nullptr, z_k);
    while (i0 < N) {
        if constexpr (SCALED)
            nx.w = make_float2(nx.w.x * cbe.x - nx.w.y * cbe.y, fmaf(nx.w.x, cbe.y, nx.w.y * cbe.x));
        stage_store<false, false>(nx, nt, M, group, d, w_blk, nullptr, z_blk);
        __syncthreads();
        const int64_t j0 = i0 + kBlk;  // the next block, loaded while this one runs
        const int jnt = static_cast<int>(min(N - j0, static_cast<int64_t>(kBlk)));
        if (j0 < N) nx = stage_fetch<false, false, false>(p, b, h, row0, j0, jnt, group, gs, nullptr, z_k);
        if (nt == kBlk) {
            xi_block<MW, false, SCALED>(nt, g_row, z_blk + lane, red[w], lane, ar, ai, br, bi, ur, ui, M);
#pragma unroll
            for (int mm = 0; mm < MW; ++mm) apply_fix(fix[mm], ur[mm], ui[mm]);
        } else
            xi_block<MW, true, SCALED>(nt, g_row, z_blk + lane, red[w], lane, ar, ai, br, bi, ur, ui, M);
        __syncthreads();
        reduce_block(red, nt, group, d, g_xi + (row0 + i0) * d);
        i0 = j0;
        nt = jnt;
    }
}

// The adjoint of one state in reverse time:
//   A_m(i) = x(i) w_m(i) + conj(abar_m) A_m(i+1),   A_m(N-1) = x w + g_S,
//   y(i) = Re sum_m conj(bbar_m) A_m(i)           -> g_z [H][T][d]
//   g_bbar_m partial = sum_i sum_c A_m,c(i) z(i)_c  -> gb [B H][channel groups][M]
//     (only when a state enters: else the per-mode scans form it)
//   g_state_in = conj(abar) A(0)                    (columns off .. off + d - 1)
// Key side: x = xi_q, w = g_s, z = z_k, off = 0.  Value side: x = g_o (io
// dtype, [B][N][H][d]), w = conj(s), z = z_v, off = d.
// The scans carry beta_m A_m instead of A_m, beta = conj(bbar) wherever
// |bbar|^2 >= kMinB2 (else 1): the staged mode input w is multiplied by beta
// once per block, each token's share Re(conj(bbar) A) is then just
// Re(beta A), and the g_bbar sums and g_state_in are divided by beta once at
// the end.  The bound keeps beta A far above the fp32 subnormal range.
constexpr double kMinB2 = 0x1p-80;
__device__ __forceinline__ bool adj_scaled(const Zoh& z) { return z.br * z.br + z.bi * z.bi >= kMinB2; }
__device__ __forceinline__ float2 adj_beta(const Zoh& z) {
    return adj_scaled(z) ? make_float2(static_cast<float>(z.br), -static_cast<float>(z.bi)) : make_float2(1.f, 0.f);
}
// 1 / beta
__device__ __forceinline__ float2 adj_beta_inv(const Zoh& z) {
    if (!adj_scaled(z)) return make_float2(1.f, 0.f);
    const double n = z.br * z.br + z.bi * z.bi;
    return make_float2(static_cast<float>(z.br / n), static_cast<float>(z.bi / n));
}

// One block of kBlk tokens of an adjoint scan for the wave's MW modes, in
// reverse token order: the carried adjoint beta A = x (beta w) + carry, the
// wave's share sum_m Re(conj(bbar_m) A_m) of each token to red, the g_bbar
// sums, and the carry conj(abar) beta A into the previous token.  The share
// weighs mode m's carried value by (yr, yi): (1, 0) where beta = conj(bbar),
// else bbar; FAST: every mode of the wave is of the first kind.  A ragged
// block steps only its first nt tokens.  GB: whether it forms the g_bbar sums
// (without a state entering the per-mode scans form them from per-token
// totals instead).
template <int MW, bool CONJ_W, bool RAGGED, bool GB, bool FAST>
__device__ __forceinline__ void adjoint_block(int nt, const float2* g_row, const float* x_col, const float* z_col,
                                              float (*red_t)[kWave], int lane, const float (&ar)[MW],
                                              const float (&ai)[MW], const float (&yr)[MW], const float (&yi)[MW],
                                              float (&cr)[MW], float (&ci)[MW], float (&gbr)[MW], float (&gbi)[MW],
                                              int M) {
#pragma unroll
    for (int t = kBlk - 1; t >= 0; --t) {
        if (RAGGED && t >= nt) continue;
        const float xx = x_col[t * kWave], zz = z_col[t * kWave];
        float acc = 0.f;
#pragma unroll
        for (int mm = 0; mm < MW; ++mm) {
            float2 g = g_row[t * M + mm];
            if constexpr (CONJ_W) g.y = -g.y;
            const float nr = fmaf(xx, g.x, cr[mm]);
            const float ni = fmaf(xx, g.y, ci[mm]);
            if constexpr (FAST)
                acc = mm == 0 ? nr : acc + nr;  // Re(beta A)
            else
                acc = fmaf(yr[mm], nr, fmaf(yi[mm], ni, acc));  // Re(conj(bbar) A)
            if constexpr (GB) {
                gbr[mm] = fmaf(nr, zz, gbr[mm]);
                gbi[mm] = fmaf(ni, zz, gbi[mm]);
            }
            // carry into the previous token: conj(abar) A
            cr[mm] = fmaf(ar[mm], nr, ai[mm] * ni);
            ci[mm] = fmaf(ar[mm], ni, -ai[mm] * nr);
        }
        red_t[t][lane] = acc;
    }
}

template <int MW, bool X_IO, bool BF16, bool CONJ_W, bool GB>
__global__ __launch_bounds__(kStage) void bwd_adjoint_kernel(Problem p, idattn_params prm,
                                                             const void* __restrict__ x,
                                                             const float2* __restrict__ wv,
                                                             const float* __restrict__ zsrc,
                                                             const float* grad_state, int off,
                                                             float* __restrict__ g_z, float* grad_state_in,
                                                             float2* __restrict__ gb, int64_t zs) {
    __shared__ float2 w_blk[kStage];
    __shared__ float x_blk[kStage];
    __shared__ float z_blk[kStage];
    __shared__ float red[kVW][kBlk][kWave];
    __shared__ float2 beta_s[kStage / kBlk];  // beta of every mode (M <= 64)
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t N = p.N;
    const int M = static_cast<int>(p.M), d = static_cast<int>(p.d);
    const int group = static_cast<int>(blockIdx.y);
    const int c = group * kWave + lane;
    const bool cok = c < d;
    const int64_t row0 = h * p.T + b * N;
    const int moff = static_cast<int>(blockIdx.z) * kVW * MW;  // the split's first mode
    g_z += blockIdx.z * zs;
    if (threadIdx.x < M) beta_s[threadIdx.x] = adj_beta(zoh_of(prm, h, M, threadIdx.x));
    float ar[MW], ai[MW], yr[MW], yi[MW], cr[MW], ci[MW], gbr[MW], gbi[MW];
    float2 rho[MW];  // 1 / beta
    float2 fix[MW];  // the decay fix of a full block (kBlk carries by conj(abar_f))
    bool fast = true;
#pragma unroll
    for (int mm = 0; mm < MW; ++mm) {
        const int64_t m = moff + w * MW + mm;
        const Zoh zz = zoh_of(prm, h, M, m);
        ar[mm] = static_cast<float>(zz.ar);
        ai[mm] = static_cast<float>(zz.ai);
        const bool sc = adj_scaled(zz);
        fast = fast && sc;
        yr[mm] = sc ? 1.f : static_cast<float>(zz.br);
        yi[mm] = sc ? 0.f : static_cast<float>(zz.bi);
        rho[mm] = adj_beta_inv(zz);
        const float2 f = decay_fix(zz, kBlk);
        fix[mm] = make_float2(f.x, -f.y);  // (conj(abar) / conj(abar_f))^kBlk - 1
        cr[mm] = ci[mm] = gbr[mm] = gbi[mm] = 0.f;
        if (grad_state != nullptr && cok) {  // the carry into the last token: beta g_S
            const int64_t idx = ((bh * M + m) * 2 * d + off + c) * 2;
            const float2 be = adj_beta(zz);
            const float gr = grad_state[idx], gi = grad_state[idx + 1];
            cr[mm] = be.x * gr - be.y * gi;
            ci[mm] = fmaf(be.x, gi, be.y * gr);
        }
    }
    __syncthreads();
    // beta of the mode this thread stages (conjugated where the scan reads the
    // staged value conjugated)
    float2 bst = beta_s[threadIdx.x % M];
    if constexpr (CONJ_W) bst.y = -bst.y;
    if (N > 0) {  // uniform over the block
        constexpr bool XB = X_IO && BF16;
        const float2* g_row = w_blk + moff + w * MW;
        int64_t i0 = N > kBlk ? N - kBlk : 0;
        int nt = static_cast<int>(N - i0);
        Stage nx = stage_fetch<true, X_IO, BF16>(p, b, h, row0, i0, nt, group, wv, x, zsrc);
        while (true) {
            nx.w = make_float2(bst.x * nx.w.x - bst.y * nx.w.y, fmaf(bst.x, nx.w.y, bst.y * nx.w.x));
            stage_store<true, XB>(nx, nt, M, group, d, w_blk, x_blk, z_blk);
            __syncthreads();
            const int64_t j0 = i0 > kBlk ? i0 - kBlk : 0;  // the previous block, loaded while this one runs
            const int jnt = static_cast<int>(i0 - j0);
            if (jnt > 0) nx = stage_fetch<true, X_IO, BF16>(p, b, h, row0, j0, jnt, group, wv, x, zsrc);
            if (nt == kBlk) {
                if (fast)
                    adjoint_block<MW, CONJ_W, false, GB, true>(nt, g_row, x_blk + lane, z_blk + lane, red[w], lane, ar,
                                                               ai, yr, yi, cr, ci, gbr, gbi, M);
                else
                    adjoint_block<MW, CONJ_W, false, GB, false>(nt, g_row, x_blk + lane, z_blk + lane, red[w], lane,
                                                                ar, ai, yr, yi, cr, ci, gbr, gbi, M);
#pragma unroll
                for (int mm = 0; mm < MW; ++mm) apply_fix(fix[mm], cr[mm], ci[mm]);
            } else {
                if (fast)
                    adjoint_block<MW, CONJ_W, true, GB, true>(nt, g_row, x_blk + lane, z_blk + lane, red[w], lane, ar,
                                                              ai, yr, yi, cr, ci, gbr, gbi, M);
                else
                    adjoint_block<MW, CONJ_W, true, GB, false>(nt, g_row, x_blk + lane, z_blk + lane, red[w], lane, ar,
                                                               ai, yr, yi, cr, ci, gbr, gbi, M);
            }
            __syncthreads();
            reduce_block(red, nt, group, d, g_z + (row0 + i0) * d);
            if (jnt == 0) break;
            i0 = j0;
            nt = jnt;
        }
    }
    if (grad_state_in != nullptr && cok) {  // conj(abar) A(0) = the carry / beta
#pragma unroll
        for (int mm = 0; mm < MW; ++mm) {
            const int64_t idx = ((bh * M + moff + w * MW + mm) * 2 * d + off + c) * 2;
            grad_state_in[idx] = rho[mm].x * cr[mm] - rho[mm].y * ci[mm];
            grad_state_in[idx + 1] = fmaf(rho[mm].x, ci[mm], rho[mm].y * cr[mm]);
        }
    }
    // g_bbar: sum over the wave's channels, one value per (mode, channel group)
    if constexpr (GB) {
#pragma unroll
        for (int mm = 0; mm < MW; ++mm) {
            const float sr = wave_total(gbr[mm]), si = wave_total(gbi[mm]);
            if (lane == 0)
                gb[(bh * gridDim.y + blockIdx.y) * M + moff + w * MW + mm] =
                    make_float2(rho[mm].x * sr - rho[mm].y * si, fmaf(rho[mm].x, si, rho[mm].y * sr));
        }
    }
}

// ------------------------------------------------------------------ features
// One wave per (b, h, run of kRun tokens); lane l owns channels l and l + 64.
// Per token: the forward's conv, SiLU, norms and RMSNorms again, then
//   g_v        = rho_v u - rho_v^3 v (u . v) / d,        u = g_v g_z_v
//   g_xi_k     = rho_k u - rho_k^3 xi_k (u . xi_k) / d,  u = g_k g_z_k
//   g_y        = g_xi / D - 2 y (y . g_xi) / D^2  (xi = y / D, D = ||y||^2 + eps)
//              = g_xi / D - y (y . g_xi) / D^3    (unit norm: D = sqrt(||y||^2 + eps))
//   g_c        = g_y sigma(c) (1 + c (1 - sigma(c)))
// g_c of queries and keys overwrite g_xi and g_z_k in place (same token, same
// lanes); the run's sums for the gain and bias gradients go to
// part [B H][runs][4 d]: gain key half, gain value half, bias key, bias value.
// WT: the conv width when it is fixed at compile time (4), else 0 (any W,
// with kConvMax taps of which the first W are used).
template <bool BF16, int DJ, int WT>
__global__ __launch_bounds__(256) void bwd_feature_kernel(Problem p, idattn_params prm, const void* __restrict__ q,
                                                          const void* __restrict__ k, const void* __restrict__ v,
                                                          const void* __restrict__ tail_in,
                                                          float* __restrict__ g_xi, float* __restrict__ g_zk,
                                                          const float* __restrict__ g_zv, int64_t zs,
                                                          void* __restrict__ grad_v,
                                                          float* __restrict__ part, int64_t runs) {
    constexpr int NT = WT > 0 ? WT : kConvMax;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    const int64_t H = p.H, N = p.N;
    const int d = static_cast<int>(p.d), W = WT > 0 ? WT : static_cast<int>(p.W);
    if (wid >= p.B * H * runs) return;  // whole wave; no barriers below
    const int64_t bh = wid / runs, run = wid % runs;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t0 = run * kRun, t1 = t0 + kRun < N ? t0 + kRun : N;
    const int64_t row0 = h * p.T + b * N;
    int cl[DJ];  // the lane's channels, clamped below d
    uint32_t lb[DJ], lf[DJ];  // their byte offsets in a row of q, k, v and in a float row
    float wq[NT][DJ], wk[NT][DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        cl[j] = min(lane + kWave * j, d - 1);
        lb[j] = static_cast<uint32_t>(cl[j]) * (BF16 ? 2u : 4u);
        lf[j] = static_cast<uint32_t>(cl[j]) * 4u;
#pragma unroll
        for (int j2 = 0; j2 < NT; ++j2) {
            wq[j2][j] = prm.conv_q[(h * d + cl[j]) * W + min(j2, W - 1)];
            wk[j2][j] = prm.conv_k[(h * d + cl[j]) * W + min(j2, W - 1)];
        }
    }
    float gk[DJ], bk[DJ], gv[DJ], bv[DJ];  // this head's gain and bias
    float agk[DJ], abk[DJ], agv[DJ], abv[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int c = lane + kWave * j;
        const bool in = c < d;
        gk[j] = in ? prm.gain[h * 2 * d + c] : 0.f;
        gv[j] = in ? prm.gain[h * 2 * d + d + c] : 0.f;
        bk[j] = in ? prm.bias[h * 2 * d + c] : 0.f;
        bv[j] = in ? prm.bias[h * 2 * d + d + c] : 0.f;
        agk[j] = abk[j] = agv[j] = abv[j] = 0.f;
    }
    (void)bk;
    (void)bv;
    const float inv_d = 1.f / static_cast<float>(d);
    // the conv inputs of q, k at sequence position pos (the tail before the
    // sequence, a masked row where there is none), as loaded
    auto load_x = [&](int64_t pos, bool real, uint32_t (&xq1)[DJ], uint32_t (&xk1)[DJ]) -> bool {
        const ConvRow r = conv_row(q, k, tail_in, b * N, pos, b * N + min(max(pos, int64_t{0}), N - 1), b, h, H, d,
                                   W, real);
        const __amdgpu_buffer_rsrc_t rq = io_rsrc<BF16>(r.bq, r.rq, d), rk = io_rsrc<BF16>(r.bk, r.rk, d);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            xq1[j] = buf_load_raw<BF16>(rq, lb[j]);
            xk1[j] = buf_load_raw<BF16>(rk, lb[j]);
        }
        return r.ok;
    };
    // W fixed: a window of the W conv inputs of the current token slides along
    // the run (slot e holds x(t - W + 1 + e)), so each token loads one new row
    uint32_t xqw[NT][DJ], xkw[NT][DJ];
    bool okw[NT];
    if constexpr (WT > 0) {
#pragma unroll
        for (int e = 0; e < NT; ++e) okw[e] = load_x(t0 - (W - 1) + e, true, xqw[e], xkw[e]);
    }
    for (int64_t t = t0; t < t1; ++t) {
        // every load of the token first (channels clamped below d, missing rows
        // masked): the conv taps of q and k, v, and the scans' gradients, each
        // row a buffer resource at a uniform base
        uint32_t xq_raw[NT][DJ], xk_raw[NT][DJ], v_raw[DJ];
        bool tap_ok[NT];
        uint32_t xqn[DJ], xkn[DJ];
        bool okn = false;
        if constexpr (WT > 0) {
#pragma unroll
            for (int e = 0; e < NT; ++e) {
                tap_ok[e] = okw[e];
#pragma unroll
                for (int j = 0; j < DJ; ++j) {
                    xq_raw[e][j] = xqw[e][j];
                    xk_raw[e][j] = xkw[e][j];
                }
            }
            // the next token's newest tap, x(t + 1), clamped into the sequence
            // (past its end it is never used)
            okn = load_x(min(t + 1, N - 1), true, xqn, xkn);
        } else {
#pragma unroll
            for (int j2 = 0; j2 < NT; ++j2) tap_ok[j2] = load_x(t - (W - 1) + j2, j2 < W, xq_raw[j2], xk_raw[j2]);
        }
        const __amdgpu_buffer_rsrc_t vrow = io_rsrc<BF16>(v, ((b * N + t) * H + h) * d, d);
        const int64_t o = (row0 + t) * d;
        const uint32_t fb = static_cast<uint32_t>(d) * 4u;
        const __amdgpu_buffer_rsrc_t rzk0 = rsrc_at(g_zk + o, fb), rzk1 = rsrc_at(g_zk + o + zs, fb);
        const __amdgpu_buffer_rsrc_t rzv0 = rsrc_at(g_zv + o, fb), rzv1 = rsrc_at(g_zv + o + zs, fb);
        const __amdgpu_buffer_rsrc_t rxq0 = rsrc_at(g_xi + o, fb), rxq1 = rsrc_at(g_xi + o + zs, fb);
        float gzk[DJ], gzv[DJ], gxq[DJ];
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            v_raw[j] = buf_load_raw<BF16>(vrow, lb[j]);
            // the scans' partial sums over the two mode splits, added in a fixed
            // order (zs = 0: one split)
            const float zk0 = buf_load(rzk0, lf[j], 0), zk1 = buf_load(rzk1, lf[j], 0);
            const float zv0 = buf_load(rzv0, lf[j], 0), zv1 = buf_load(rzv1, lf[j], 0);
            const float xq0 = buf_load(rxq0, lf[j], 0), xq1 = buf_load(rxq1, lf[j], 0);
            gzk[j] = zs ? zk0 + zk1 : zk0;
            gzv[j] = zs ? zv0 + zv1 : zv0;
            gxq[j] = zs ? xq0 + xq1 : xq0;
        }
        float cq[DJ], ck[DJ], vv[DJ];
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const bool in = lane + kWave * j < d;  // lanes past d hold zeros
            float aq = 0.f, ak = 0.f;
#pragma unroll
            for (int j2 = 0; j2 < NT; ++j2) {
                aq = fmaf(wq[j2][j], tap_ok[j2] ? widen<BF16>(xq_raw[j2][j]) : 0.f, aq);
                ak = fmaf(wk[j2][j], tap_ok[j2] ? widen<BF16>(xk_raw[j2][j]) : 0.f, ak);
            }
            cq[j] = in ? aq : 0.f;
            ck[j] = in ? ak : 0.f;
            vv[j] = in ? widen<BF16>(v_raw[j]) : 0.f;
            if (!in) gzk[j] = gzv[j] = gxq[j] = 0.f;
        }
        // forward quantities: y = SiLU(c) with its sigmoid, norms
        float sq[DJ], sk[DJ], yq[DJ], yk[DJ];
        float nq = 0.f, nk = 0.f, nv = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            sq[j] = 1.f / (1.f + expf(-cq[j]));
            sk[j] = 1.f / (1.f + expf(-ck[j]));
            yq[j] = cq[j] * sq[j];
            yk[j] = ck[j] * sk[j];
            nq = fmaf(yq[j], yq[j], nq);
            nk = fmaf(yk[j], yk[j], nk);
            nv = fmaf(vv[j], vv[j], nv);
        }
        nq = wave_total(nq);
        nk = wave_total(nk);
        nv = wave_total(nv);
        const float Dq = p.unit_feat ? sqrtf(nq + p.eps_feat) : nq + p.eps_feat;
        const float Dk = p.unit_feat ? sqrtf(nk + p.eps_feat) : nk + p.eps_feat;
        const float iDk = 1.f / Dk;
        float xk[DJ];
        float nxk = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            xk[j] = yk[j] * iDk;
            nxk = fmaf(xk[j], xk[j], nxk);
        }
        nxk = wave_total(nxk);
        const float rk = 1.f / sqrtf(nxk * inv_d + p.eps_norm);
        const float rv = 1.f / sqrtf(nv * inv_d + p.eps_norm);
        // backward through the RMSNorms, and the query side's y . g_xi
        float uxk = 0.f, uvv = 0.f, yqg = 0.f;
        float uk[DJ], uv[DJ];
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            agk[j] = fmaf(gzk[j], xk[j] * rk, agk[j]);
            abk[j] += gzk[j];
            agv[j] = fmaf(gzv[j], vv[j] * rv, agv[j]);
            abv[j] += gzv[j];
            uk[j] = gk[j] * gzk[j];
            uv[j] = gv[j] * gzv[j];
            uxk = fmaf(uk[j], xk[j], uxk);
            uvv = fmaf(uv[j], vv[j], uvv);
            yqg = fmaf(yq[j], gxq[j], yqg);
        }
        uxk = wave_total(uxk);
        uvv = wave_total(uvv);
        yqg = wave_total(yqg);
        const float ck3 = rk * rk * rk * uxk * inv_d, cv3 = rv * rv * rv * uvv * inv_d;
        float gxk[DJ];
        float ykg = 0.f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const int c = lane + kWave * j;
            gxk[j] = rk * uk[j] - ck3 * xk[j];
            ykg = fmaf(yk[j], gxk[j], ykg);
            if (c < d) store_io<BF16>(grad_v, ((b * N + t) * H + h) * d + c, rv * uv[j] - cv3 * vv[j]);
        }
        ykg = wave_total(ykg);
        // through the feature map and SiLU
        const float iDq = 1.f / Dq;
        const float fq = p.unit_feat ? yqg * iDq * iDq * iDq : 2.f * yqg * iDq * iDq;
        const float fk = p.unit_feat ? ykg * iDk * iDk * iDk : 2.f * ykg * iDk * iDk;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const int c = lane + kWave * j;
            if (c < d) {
                const float gyq = gxq[j] * iDq - fq * yq[j];
                const float gyk = gxk[j] * iDk - fk * yk[j];
                g_xi[(row0 + t) * d + c] = gyq * sq[j] * (1.f + cq[j] * (1.f - sq[j]));
                g_zk[(row0 + t) * d + c] = gyk * sk[j] * (1.f + ck[j] * (1.f - sk[j]));
            }
        }
        if constexpr (WT > 0) {  // slide the window by one token
#pragma unroll
            for (int e = 0; e + 1 < NT; ++e) {
                okw[e] = okw[e + 1];
#pragma unroll
                for (int j = 0; j < DJ; ++j) {
                    xqw[e][j] = xqw[e + 1][j];
                    xkw[e][j] = xkw[e + 1][j];
                }
            }
            okw[NT - 1] = okn;
#pragma unroll
            for (int j = 0; j < DJ; ++j) {
                xqw[NT - 1][j] = xqn[j];
                xkw[NT - 1][j] = xkn[j];
            }
        }
    }
    float* pp = part + wid * 4 * d;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int c = lane + kWave * j;
        if (c < d) {
            pp[c] = agk[j];
            pp[d + c] = agv[j];
            pp[2 * d + c] = abk[j];
            pp[3 * d + c] = abv[j];
        }
    }
}

// Conv backward, one wave per (b, h, run of kRun tokens):
//   g_x(t)_c = sum_j w[c][j] g_c(t + W - 1 - j)_c   (terms past the sequence end are zero)
//   g_w[c][j] += g_c(t)_c x(t - W + 1 + j)_c         (x before position 0 from the tail)
// for queries (g_c in g_cq) and keys (g_ck); partial weight gradients to
// part [B H][runs][2][d][W].
// WT as for the feature kernel.
template <bool BF16, int DJ, int WT>
__global__ __launch_bounds__(256) void bwd_conv_kernel(Problem p, idattn_params prm, const void* __restrict__ q,
                                                       const void* __restrict__ k, const void* __restrict__ tail_in,
                                                       const float* __restrict__ g_cq, const float* __restrict__ g_ck,
                                                       void* __restrict__ grad_q, void* __restrict__ grad_k,
                                                       float* __restrict__ part, int64_t runs) {
    constexpr int NT = WT > 0 ? WT : kConvMax;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    const int64_t H = p.H, N = p.N;
    const int d = static_cast<int>(p.d), W = WT > 0 ? WT : static_cast<int>(p.W);
    if (wid >= p.B * H * runs) return;  // whole wave; no barriers below
    const int64_t bh = wid / runs, run = wid % runs;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t0 = run * kRun, t1 = t0 + kRun < N ? t0 + kRun : N;
    const int64_t row0 = h * p.T + b * N;
    int cl[DJ];  // the lane's channels, clamped below d
    uint32_t lb[DJ], lf[DJ];  // their byte offsets in a row of q, k and in a float row
    float wq[NT][DJ], wk[NT][DJ], aq[NT][DJ], ak[NT][DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        cl[j] = min(lane + kWave * j, d - 1);
        lb[j] = static_cast<uint32_t>(cl[j]) * (BF16 ? 2u : 4u);
        lf[j] = static_cast<uint32_t>(cl[j]) * 4u;
#pragma unroll
        for (int e = 0; e < NT; ++e) {
            wq[e][j] = prm.conv_q[(h * d + cl[j]) * W + min(e, W - 1)];
            wk[e][j] = prm.conv_k[(h * d + cl[j]) * W + min(e, W - 1)];
            aq[e][j] = ak[e][j] = 0.f;
        }
    }
    // one row of g_cq, g_ck at sequence position tt (clamped), and the conv
    // inputs of q, k at position pos (the tail before the sequence, a masked
    // row where there is none)
    auto load_g = [&](int64_t tt, float (&gq1)[DJ], float (&gk1)[DJ]) {
        const int64_t gr = (row0 + max(min(tt, N - 1), int64_t{0})) * d;
        const uint32_t fb = static_cast<uint32_t>(d) * 4u;
        const __amdgpu_buffer_rsrc_t rgq = rsrc_at(g_cq + gr, fb), rgk = rsrc_at(g_ck + gr, fb);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            gq1[j] = buf_load(rgq, lf[j], 0);
            gk1[j] = buf_load(rgk, lf[j], 0);
        }
    };
    auto load_x = [&](int64_t pos, bool real, uint32_t (&xq1)[DJ], uint32_t (&xk1)[DJ]) -> bool {
        const ConvRow r = conv_row(q, k, tail_in, b * N, pos, b * N + min(max(pos, int64_t{0}), N - 1), b, h, H, d,
                                   W, real);
        const __amdgpu_buffer_rsrc_t rq = io_rsrc<BF16>(r.bq, r.rq, d), rk = io_rsrc<BF16>(r.bk, r.rk, d);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            xq1[j] = buf_load_raw<BF16>(rq, lb[j]);
            xk1[j] = buf_load_raw<BF16>(rk, lb[j]);
        }
        return r.ok;
    };
    // token t's rows and the conv update of its outputs and of the weight sums:
    //   g_x(t) = sum_e w[e] g_c(t + W - 1 - e),   g_w[e] += g_c(t) x(t - W + 1 + e)
    auto token = [&](int64_t t, const float (&gq)[NT][DJ], const float (&gk)[NT][DJ], const bool (&g_ok)[NT],
                     const uint32_t (&xq_raw)[NT][DJ], const uint32_t (&xk_raw)[NT][DJ], const bool (&x_ok)[NT],
                     const float (&gq_t)[DJ], const float (&gk_t)[DJ]) {
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < NT; ++e) {
                // g_x(t) takes g_c(t + W - 1 - e) through tap e
                sq = fmaf(wq[e][j], g_ok[e] ? gq[e][j] : 0.f, sq);
                sk = fmaf(wk[e][j], g_ok[e] ? gk[e][j] : 0.f, sk);
                // tap e of token t reads x(t - W + 1 + e)
                aq[e][j] = fmaf(gq_t[j], x_ok[e] ? widen<BF16>(xq_raw[e][j]) : 0.f, aq[e][j]);
                ak[e][j] = fmaf(gk_t[j], x_ok[e] ? widen<BF16>(xk_raw[e][j]) : 0.f, ak[e][j]);
            }
            const int c = lane + kWave * j;
            if (c < d) {
                const int64_t o = ((b * N + t) * H + h) * d + c;
                store_io<BF16>(grad_q, o, sq);
                store_io<BF16>(grad_k, o, sk);
            }
        }
    };
    if constexpr (WT > 0) {
        // W fixed: windows of W rows slide along the run, so each token loads
        // one new row of g_c and of x (the next token's, ahead of its use):
        // slot e of gw holds g_c(t + W - 1 - e), slot e of xw x(t - W + 1 + e)
        float gqw[NT][DJ], gkw[NT][DJ];
        uint32_t xqw[NT][DJ], xkw[NT][DJ];
        bool g_ok[NT], x_ok[NT];
#pragma unroll
        for (int e = 0; e < NT; ++e) {
            load_g(t0 + W - 1 - e, gqw[e], gkw[e]);
            g_ok[e] = t0 + W - 1 - e < N;
            x_ok[e] = load_x(t0 - (W - 1) + e, true, xqw[e], xkw[e]);
        }
        for (int64_t t = t0; t < t1; ++t) {
            float gqn[DJ], gkn[DJ];
            uint32_t xqn[DJ], xkn[DJ];
            load_g(t + W, gqn, gkn);  // g_c(t + 1 + W - 1), clamped and masked past the end
            // x(t + 1), clamped into the sequence (past its end it is never used)
            const bool xn_ok = load_x(min(t + 1, N - 1), true, xqn, xkn);
            token(t, gqw, gkw, g_ok, xqw, xkw, x_ok, gqw[W - 1], gkw[W - 1]);
#pragma unroll
            for (int e = NT - 1; e > 0; --e) {
#pragma unroll
                for (int j = 0; j < DJ; ++j) {
                    gqw[e][j] = gqw[e - 1][j];
                    gkw[e][j] = gkw[e - 1][j];
                }
                g_ok[e] = g_ok[e - 1];
            }
#pragma unroll
            for (int e = 0; e + 1 < NT; ++e) {
#pragma unroll
                for (int j = 0; j < DJ; ++j) {
                    xqw[e][j] = xqw[e + 1][j];
                    xkw[e][j] = xkw[e + 1][j];
                }
                x_ok[e] = x_ok[e + 1];
            }
#pragma unroll
            for (int j = 0; j < DJ; ++j) {
                gqw[0][j] = gqn[j];
                gkw[0][j] = gkn[j];
                xqw[NT - 1][j] = xqn[j];
                xkw[NT - 1][j] = xkn[j];
            }
            g_ok[0] = t + W < N;
            x_ok[NT - 1] = xn_ok;
        }
    } else {
        for (int64_t t = t0; t < t1; ++t) {
            // every load of the token first (indices clamped, missing taps masked):
            // g_c at t + W - 1 - e (tap e of the later tokens that read x(t)), the
            // conv inputs x(t - W + 1 + e) that tap e of token t reads, g_c(t)
            float gq[NT][DJ], gk[NT][DJ], gq_t[DJ], gk_t[DJ];
            uint32_t xq_raw[NT][DJ], xk_raw[NT][DJ];
            bool g_ok[NT], x_ok[NT];
#pragma unroll
            for (int e = 0; e < NT; ++e) {
                load_g(t + W - 1 - e, gq[e], gk[e]);
                g_ok[e] = e < W && t + W - 1 - e < N;
                x_ok[e] = load_x(t - (W - 1) + e, e < W, xq_raw[e], xk_raw[e]);
            }
            load_g(t, gq_t, gk_t);
            token(t, gq, gk, g_ok, xq_raw, xk_raw, x_ok, gq_t, gk_t);
        }
    }
    float* pp = part + wid * 2 * d * W;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int c = lane + kWave * j;
        if (c >= d) continue;
#pragma unroll
        for (int e = 0; e < NT; ++e) {
            if (e >= W) break;
            pp[c * W + e] = aq[e][j];
            pp[d * W + c * W + e] = ak[e][j];
        }
    }
}

// ------------------------------------------------------------------ parameters
// (exp(z) (z - 1) + 1) / z^2 = sum_{n>=2} z^(n-2) (n-1)/n!: the part of
// d bbar / d lambda that cancels for small z = Delta lambda.
__device__ inline void phi_z(double zr, double zi, double& pr, double& pi) {
    const double az = sqrt(zr * zr + zi * zi);
    if (az < 0.5) {
        // series: term_n = z^(n-2) (n-1)/n!
        double tr = 1.0, ti = 0.0;  // z^(n-2) / n!, from n = 2: 1/2
        double sr = 0.0, si = 0.0;
        double inv_fact = 0.5;
        for (int n = 2; n < 30; ++n) {
            if (n > 2) {
                const double nr = tr * zr - ti * zi, ni = tr * zi + ti * zr;
                tr = nr;
                ti = ni;
                inv_fact /= n;
            }
            sr += (n - 1) * inv_fact * tr;
            si += (n - 1) * inv_fact * ti;
        }
        pr = sr;
        pi = si;
        return;
    }
    double sy, cy;
    sincos(zi, &sy, &cy);
    const double e = exp(zr);
    const double er = e * cy, ei = e * sy;  // exp(z)
    const double nr = er * (zr - 1.0) - ei * zi + 1.0, ni = er * zi + ei * (zr - 1.0);
    const double z2r = zr * zr - zi * zi, z2i = 2.0 * zr * zi;
    const double den = z2r * z2r + z2i * z2i;
    pr = (nr * z2r + ni * z2i) / den;
    pi = (ni * z2r - nr * z2i) / den;
}

// acc += src[0], src[stride], ..., src[(runs - 1) stride] in that order, with
// sixteen loads in flight.
__device__ __forceinline__ void sum_runs(const float* src, int64_t stride, int64_t runs, double& acc) {
    int64_t r = 0;
    for (; r + 16 <= runs; r += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = src[(r + i) * stride];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += v[i];
    }
    for (; r < runs; ++r) acc += src[r * stride];
}

// Grid (H, slices): blocks y < slices - 1 take kRedThreads of the head's
// 4 d + 2 d W gain, bias and conv gradient elements each, summed over batch
// rows and runs in a fixed order; block y = slices - 1 applies the ZOH
// chain rule from g_abar,
// g_bbar (summed over batch rows and channel groups) to lambda, B and
// log_dt:
//   g_lambda = conj(Delta abar) g_abar + conj(B Delta^2 phi(Delta lambda)) g_bbar
//   g_B      = conj((abar - 1) / lambda) g_bbar
//   g_log_dt = Delta sum_m Re(conj(lambda abar) g_abar + conj(B abar) g_bbar)
constexpr int kRedThreads = 256;
__global__ __launch_bounds__(kRedThreads) void bwd_param_kernel(Problem p, idattn_params prm,
                                                                const float* __restrict__ part_f,
                                                                const float* __restrict__ part_c,
                                                                const float2* __restrict__ ga,
                                                                const float2* __restrict__ gbk,
                                                                const float2* __restrict__ gbv, int64_t runs,
                                                                int groups, idattn_param_grads out) {
    __shared__ double ldt[kRedThreads];
    const int64_t h = blockIdx.x, H = p.H, B = p.B, M = p.M;
    const int d = static_cast<int>(p.d), W = static_cast<int>(p.W);
    if (blockIdx.y + 1 < gridDim.y) {
        const int e = static_cast<int>(blockIdx.y) * kRedThreads + static_cast<int>(threadIdx.x);
        if (e < 4 * d) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b) sum_runs(part_f + (b * H + h) * runs * 4 * d + e, 4 * d, runs, acc);
            const int half = e / d, c = e % d;  // gain key, gain value, bias key, bias value
            float* dst = half < 2 ? out.gain : out.bias;
            dst[h * 2 * d + (half & 1) * d + c] = static_cast<float>(acc);
        } else if (e < 4 * d + 2 * d * W) {
            const int ec = e - 4 * d;
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b)
                sum_runs(part_c + (b * H + h) * runs * 2 * d * W + ec, 2 * d * W, runs, acc);
            const int sel = ec / (d * W), rest = ec % (d * W);
            (sel == 0 ? out.conv_q : out.conv_k)[h * d * W + rest] = static_cast<float>(acc);
        }
        return;
    }
    double my_ldt = 0.0;
    for (int64_t m = threadIdx.x; m < M; m += kRedThreads) {
        double gar = 0.0, gai = 0.0, gbr = 0.0, gbi = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const float2 a = ga[(b * H + h) * M + m];
            gar += a.x;
            gai += a.y;
            for (int g = 0; g < groups; ++g) {
                const float2 x = gbk[((b * H + h) * groups + g) * M + m];
                const float2 y = gbv[((b * H + h) * groups + g) * M + m];
                gbr += static_cast<double>(x.x) + y.x;
                gbi += static_cast<double>(x.y) + y.y;
            }
        }
        const double dt = exp(static_cast<double>(prm.log_dt[h]));
        const double lr = prm.A[(h * M + m) * 2], li = prm.A[(h * M + m) * 2 + 1];
        const double Br = prm.Bc[(h * M + m) * 2], Bi = prm.Bc[(h * M + m) * 2 + 1];
        const Zoh z = zoh_of(prm, h, M, m);
        // (abar - 1) / lambda = bbar / B when B != 0; recomputed here from the ZOH step
        double qr, qi;
        {
            const double zr = dt * lr, zi = dt * li;
            double sy, cy;
            sincos(zi, &sy, &cy);
            const double sh = sin(0.5 * zi);
            const double em1r = expm1(zr) * cy - 2.0 * sh * sh, em1i = exp(zr) * sy;
            const double l2 = lr * lr + li * li;
            if (l2 == 0.0) {
                qr = dt;
                qi = 0.0;
            } else {
                qr = (em1r * lr + em1i * li) / l2;
                qi = (em1i * lr - em1r * li) / l2;
            }
        }
        double pr, pi;
        phi_z(dt * lr, dt * li, pr, pi);
        // d abar / d lambda = Delta abar; d bbar / d lambda = B Delta^2 phi
        const double dar = dt * z.ar, dai = dt * z.ai;
        const double dbr = dt * dt * (Br * pr - Bi * pi), dbi = dt * dt * (Br * pi + Bi * pr);
        // conj(x) g = (x.r g.r + x.i g.i) + i (x.r g.i - x.i g.r)
        const double glr = (dar * gar + dai * gai) + (dbr * gbr + dbi * gbi);
        const double gli = (dar * gai - dai * gar) + (dbr * gbi - dbi * gbr);
        out.A[(h * M + m) * 2] = static_cast<float>(glr);
        out.A[(h * M + m) * 2 + 1] = static_cast<float>(gli);
        out.Bc[(h * M + m) * 2] = static_cast<float>(qr * gbr + qi * gbi);
        out.Bc[(h * M + m) * 2 + 1] = static_cast<float>(qr * gbi - qi * gbr);
        // d abar / d Delta = lambda abar, d bbar / d Delta = B abar
        const double lar = lr * z.ar - li * z.ai, lai = lr * z.ai + li * z.ar;
        const double bar = Br * z.ar - Bi * z.ai, bai = Br * z.ai + Bi * z.ar;
        my_ldt += dt * ((lar * gar + lai * gai) + (bar * gbr + bai * gbi));
    }
    ldt[threadIdx.x] = my_ldt;
    __syncthreads();
    if (threadIdx.x == 0) {
        double acc = 0.0;
        for (int i = 0; i < kRedThreads; ++i) acc += ldt[i];
        out.log_dt[h] = static_cast<float>(acc);
    }
}

}  // namespace

size_t backward_workspace_bytes(const Problem& p) {
    const size_t tok = static_cast<size_t>(p.H) * p.T;
    const size_t runs = static_cast<size_t>((p.N + kRun - 1) / kRun);
    const size_t groups = static_cast<size_t>((p.d + kWave - 1) / kWave);
    const size_t bh = static_cast<size_t>(p.B * p.H);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t splits = p.M / kVW >= 2 ? 2 : 1;  // mode splits of the per-channel scans
    return (3 + 3 * splits) * up(tok * p.d * sizeof(float)) + 3 * up(tok * p.M * sizeof(float2)) +
           2 * up(bh * p.M * sizeof(float2)) + 2 * up(bh * groups * p.M * sizeof(float2)) +
           up(bh * runs * 4 * p.d * sizeof(float)) + up(bh * runs * 2 * p.d * p.W * sizeof(float));
}

hipError_t launch_backward(const Problem& p, const idattn_params& prm, const void* q, const void* k, const void* v,
                           const float* state_in, const void* tail_in, const void* grad_o, const float* grad_state,
                           void* grad_q, void* grad_k, void* grad_v, const idattn_param_grads& grads,
                           float* grad_state_in, void* workspace, hipStream_t stream) {
    const size_t tok = static_cast<size_t>(p.H) * p.T;
    const int64_t runs = (p.N + kRun - 1) / kRun;
    const int groups = static_cast<int>((p.d + kWave - 1) / kWave);
    const size_t bh = static_cast<size_t>(p.B * p.H);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    char* base = static_cast<char*>(workspace);
    auto take = [&](size_t bytes) {
        char* r = base;
        base += up(bytes);
        return r;
    };
    float* xi_q = reinterpret_cast<float*>(take(tok * p.d * sizeof(float)));
    float* z_k = reinterpret_cast<float*>(take(tok * p.d * sizeof(float)));
    float* z_v = reinterpret_cast<float*>(take(tok * p.d * sizeof(float)));
    const int splits = p.M / kVW >= 2 ? 2 : 1;  // mode splits of the per-channel scans
    // each split's copy of the scans' outputs, zs floats apart (0: one split)
    const int64_t zs = splits > 1 ? static_cast<int64_t>(up(tok * p.d * sizeof(float)) / sizeof(float)) : 0;
    float* g_xi = reinterpret_cast<float*>(take(splits * up(tok * p.d * sizeof(float))));
    float* g_zk = reinterpret_cast<float*>(take(splits * up(tok * p.d * sizeof(float))));
    float* g_zv = reinterpret_cast<float*>(take(splits * up(tok * p.d * sizeof(float))));
    float2* s = reinterpret_cast<float2*>(take(tok * p.M * sizeof(float2)));
    float2* s_a = reinterpret_cast<float2*>(take(tok * p.M * sizeof(float2)));
    float2* gs = reinterpret_cast<float2*>(take(tok * p.M * sizeof(float2)));
    float2* ga_key = reinterpret_cast<float2*>(take(bh * p.M * sizeof(float2)));
    float2* ga = reinterpret_cast<float2*>(take(bh * p.M * sizeof(float2)));
    float2* gbk = reinterpret_cast<float2*>(take(bh * groups * p.M * sizeof(float2)));
    float2* gbv = reinterpret_cast<float2*>(take(bh * groups * p.M * sizeof(float2)));
    float* part_f = reinterpret_cast<float*>(take(bh * runs * 4 * p.d * sizeof(float)));
    float* part_c = reinterpret_cast<float*>(take(bh * runs * 2 * p.d * p.W * sizeof(float)));

    hipError_t e = launch_featmap_conv_norm(p, prm, q, k, v, tail_in, xi_q, z_k, z_v, stream);
    if (e != hipSuccess) return e;
    // the per-mode scans: two modes per wave (one per half), four waves per block
    const dim3 gm(static_cast<unsigned>(bh), static_cast<unsigned>((p.M + 7) / 8));
    // without a state entering, the per-mode scans carry their states divided by bbar
#define IDATTN_BK(RJ)                                                                                              \
    do {                                                                                                           \
        if (state_in == nullptr)                                                                                   \
            bwd_key_scan_kernel<RJ, true><<<gm, 256, 0, stream>>>(p, prm, xi_q, z_k, state_in, grad_state, s, s_a, \
                                                                  ga_key, gbk);                                    \
        else                                                                                                       \
            bwd_key_scan_kernel<RJ, false><<<gm, 256, 0, stream>>>(p, prm, xi_q, z_k, state_in, grad_state, s, s_a, \
                                                                   ga_key, gbk);                                   \
    } while (0)
    if (p.d > 64) IDATTN_BK(4);
    else if (p.d > 32) IDATTN_BK(2);
    else IDATTN_BK(1);
#undef IDATTN_BK
    if ((e = hipGetLastError()) != hipSuccess) return e;
#define IDATTN_BV(RJ, BF)                                                                                      \
    do {                                                                                                       \
        if (state_in == nullptr)                                                                               \
            bwd_value_scan_kernel<RJ, BF, true><<<gm, 256, 0, stream>>>(p, prm, z_v, grad_o, state_in, grad_state, \
                                                                        s, s_a, ga_key, gs, ga, gbv);          \
        else                                                                                                   \
            bwd_value_scan_kernel<RJ, BF, false><<<gm, 256, 0, stream>>>(p, prm, z_v, grad_o, state_in,            \
                                                                         grad_state, s, s_a, ga_key, gs, ga, gbv); \
    } while (0)
    if (p.d > 64) {
        if (p.bf16) IDATTN_BV(4, true);
        else IDATTN_BV(4, false);
    } else if (p.d > 32) {
        if (p.bf16) IDATTN_BV(2, true);
        else IDATTN_BV(2, false);
    } else {
        if (p.bf16) IDATTN_BV(1, true);
        else IDATTN_BV(1, false);
    }
#undef IDATTN_BV
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 gc(static_cast<unsigned>(bh), static_cast<unsigned>(groups), static_cast<unsigned>(splits));
#define IDATTN_BX(MW)                                                                                     \
    do {                                                                                                  \
        if (state_in == nullptr)                                                                          \
            bwd_xi_scan_kernel<MW, true><<<gc, kVW * 64, 0, stream>>>(p, prm, z_k, state_in, gs, g_xi, zs);  \
        else                                                                                              \
            bwd_xi_scan_kernel<MW, false><<<gc, kVW * 64, 0, stream>>>(p, prm, z_k, state_in, gs, g_xi, zs); \
    } while (0)
#define IDATTN_BAG(MW, GB)                                                                                    \
    do {                                                                                                      \
        bwd_adjoint_kernel<MW, false, false, false, GB><<<gc, kVW * 64, 0, stream>>>(                          \
            p, prm, xi_q, gs, z_k, grad_state, 0, g_zk, grad_state_in, gbk, zs);                               \
        if (p.bf16)                                                                                           \
            bwd_adjoint_kernel<MW, true, true, true, GB><<<gc, kVW * 64, 0, stream>>>(                         \
                p, prm, grad_o, s, z_v, grad_state, static_cast<int>(p.d), g_zv, grad_state_in, gbv, zs);     \
        else                                                                                                  \
            bwd_adjoint_kernel<MW, true, false, true, GB><<<gc, kVW * 64, 0, stream>>>(                        \
                p, prm, grad_o, s, z_v, grad_state, static_cast<int>(p.d), g_zv, grad_state_in, gbv, zs);     \
    } while (0)
    // without a state entering, the per-mode scans have formed the g_bbar sums
#define IDATTN_BA(MW)              \
    do {                           \
        if (state_in == nullptr)   \
            IDATTN_BAG(MW, false); \
        else                       \
            IDATTN_BAG(MW, true);  \
    } while (0)
    switch (p.M / (kVW * splits)) {
        case 1: IDATTN_BX(1); IDATTN_BA(1); break;
        case 2: IDATTN_BX(2); IDATTN_BA(2); break;
        case 4: IDATTN_BX(4); IDATTN_BA(4); break;
        default: return hipErrorInvalidValue;
    }
#undef IDATTN_BX
#undef IDATTN_BA
#undef IDATTN_BAG
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 gr(static_cast<unsigned>((bh * runs + 3) / 4));
#define IDATTN_BFW(BF, DJ, WT)                                                                                    \
    bwd_feature_kernel<BF, DJ, WT><<<gr, 256, 0, stream>>>(p, prm, q, k, v, tail_in, g_xi, g_zk, g_zv, zs, grad_v,   \
                                                           part_f, runs);                                            \
    bwd_conv_kernel<BF, DJ, WT><<<gr, 256, 0, stream>>>(p, prm, q, k, tail_in, g_xi, g_zk, grad_q, grad_k, part_c, runs)
#define IDATTN_BF(BF, DJ)          \
    if (p.W == 4) {                \
        IDATTN_BFW(BF, DJ, 4);     \
    } else {                       \
        IDATTN_BFW(BF, DJ, 0);     \
    }
    if (p.d > 64) {
        if (p.bf16) { IDATTN_BF(true, 2); }
        else { IDATTN_BF(false, 2); }
    } else {
        if (p.bf16) { IDATTN_BF(true, 1); }
        else { IDATTN_BF(false, 1); }
    }
#undef IDATTN_BF
#undef IDATTN_BFW
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned slices = static_cast<unsigned>((4 * p.d + 2 * p.d * p.W + kRedThreads - 1) / kRedThreads + 1);
    // the g_bbar partials: one per (b, h, mode) from the per-mode scans without
    // a state entering, else one per channel group from the adjoints
    const int gb_groups = state_in == nullptr ? 1 : groups;
    bwd_param_kernel<<<dim3(static_cast<unsigned>(p.H), slices), kRedThreads, 0, stream>>>(p, prm, part_f, part_c, ga, gbk, gbv,
                                                                                   runs, gb_groups, grads);
    return hipGetLastError();
}

}  // namespace idattn

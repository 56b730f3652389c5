// Chunked parallel-in-time forward of the Interdomain Attention mixer
// (bf16 I/O, fp16 MFMA operands, fp32 accumulation and fp32 state).
//
// The recurrence U_m(i) = abar_m U_m(i-1) + bbar_m z_k(i) (and the same for
// Gamma with z_v) is cut into chunks of L = 64 tokens.  With t, j, l
// positions inside a chunk, U_prev the state before it, and the decay kernel
// T_m[k] = bbar_m abar_m^k:
//   s_m(t)   = sigma_t [ sum_{j<=t} G[t][j] T_m[t-j] + abar_m^{t+1} (y_q(t) . U_prev,m) ]
//              with G = Y_q Z_k^T, y_q = SiLU(SC(q)), sigma_t = 1/(||y_q(t)||^2+eps)
//   o(t)     = sum_{l<=t} P[t][l] z_v(l) + Re sum_m s_m(t) abar_m^{t+1} Gamma_prev,m
//              with P[t][l] = Re sum_m s_m(t) T_m[t-l]
//   U_new    = abar^L U_prev + sum_j T_m[L-1-j] z_k(j)   (likewise Gamma)
// The Toeplitz sums become plain products through skewed layouts:
// G'[t][k] = G[t][t-k] turns sum_j G[t][j] T[t-j] into G' T, and
// P'[t][k] = Re sum_m s_m(t) T_m[k] is un-skewed into P[t][l] = P'[t][t-l].
// Every contraction (G, y_q.U, G'T, P', P Z_v, s.Gamma, both state updates)
// runs on v_mfma_f32_16x16x32_f16.
//
// Time is split into S segments per (b, h) so that B*H*S workgroups fill the
// chip:  ssm_segment_state computes each segment's end state from a zero
// start (reads k, v only), ssm_segment_carry chains those into the state that
// enters every segment, and ssm_chunked_forward runs the full chunk loop of
// one segment from its carried-in state.
//
// One workgroup = 4 waves.  The key state U (2M x R values: re and im of M
// modes) and the value state Gamma (2M x d) stay in registers for the whole
// segment as MFMA accumulators: wave w owns U for modes 16w..16w+15 (all R
// channels) and Gamma for channels [w*d/4, (w+1)*d/4) (all modes).  The
// accumulator layout of a state update is reused, unchanged, as the operand
// layout of the readout that consumes it, by ordering the contraction index
// so that lane (g, i) of a 32-row block supplies rows 4g..4g+3 and
// 16+4g..16+4g+3 (perm32 below).
#include "common.h"
#include "launch.h"

namespace idattn {

namespace {

constexpr int L = 64;        // chunk length
constexpr int MM = 64;       // complex modes handled by this path
constexpr int M2 = 2 * MM;   // re and im rows
constexpr int NTH = 256;     // threads per workgroup
constexpr int RL_L = L + 8;  // padded row length (halfs) of rows indexed by token
constexpr int RL_M = M2 + 8; // padded row length of rows indexed by (mode, part)
constexpr int kMaxW = 4;     // conv widths 1..4 on this path

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(const half8& a, const half8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 ld8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ half4 ld4(const _Float16* p) { return *reinterpret_cast<const half4*>(p); }
__device__ __forceinline__ half8 cat(const half4& a, const half4& b) {
    half8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// ------------------------------------------------------------------ shared memory
template <int D>
struct Smem {
    static constexpr int RL_D = D + 8;
    // featmap outputs (fp16)
    _Float16 yq[L * RL_D];     // y_q = SiLU(SC(q)), unscaled, [t][r]
    _Float16 zk[L * RL_D];     // z_k [j][r]
    _Float16 zkT[D * RL_L];    // z_k transposed [r][j]
    _Float16 zvT[D * RL_L];    // z_v transposed [c][l]
    float sig[L];              // 1 / (||y_q||^2 + eps_feat)
    // G' (skewed Gram) and, later in the chunk, P (un-skewed value weights)
    _Float16 gp[L * RL_L];
    // [s_re | s_im] and [Re(s abar^{t+1}) | -Im(s abar^{t+1})] / Delta per 32-column
    // mode block; the raw bf16 q, k rows of the chunk and the ZOH set-up
    // tables alias this region while it is free.
    union {
        struct {
            _Float16 s[L * RL_M];
            _Float16 se[L * RL_M];
        } v;
        struct {
            uint16_t q[L * RL_D];
            uint16_t k[L * RL_D];
        } raw;
        float2 tab[L * MM];    // complex fp32 table [k][m] during set-up
    } u;
    // constant per head: T'^T[kcol][m'] = (T_re | -T_im)[kcol] / Delta, and
    // F^T[m'][j] = (T_re | T_im)[L-1-j]
    _Float16 tpT[L * RL_M];
    _Float16 fT[M2 * RL_L];
    // raw q, k of the 3 tokens before the chunk, double buffered
    uint16_t halo[2][2][3][D];
    float wq[D * kMaxW], wk[D * kMaxW];
};

// (mode, part) index of row rho of a 32-row block kb: rho < 16 -> re of mode
// 16 kb + rho, else im of mode 16 kb + rho - 16.
__device__ __forceinline__ int blk_mode(int mprime) { return 16 * (mprime >> 5) + (mprime & 15); }
__device__ __forceinline__ int blk_part(int mprime) { return (mprime >> 4) & 1; }

// Complex fp64 power abar^n = exp(n Delta lambda).
__device__ inline void cpow(double dt, float lre, float lim, double n, double& pr, double& pi) {
    const double x = n * dt * lre, y = n * dt * lim;
    double sy, cy;
    sincos(y, &sy, &cy);
    const double e = exp(x);
    pr = e * cy;
    pi = e * sy;
}

// Register-resident per-head constants of one lane (wave w, lane g*16+i).
struct Consts {
    float dt, inv_dt;        // Delta, 1/Delta
    half8 aT[2][2];          // [kb][part]: T_m[32kb+8g+jj] of mode 16w+i (A operand of G'T)
    half8 bF[2][2];          // [kb][part]: T_m[L-1-(32kb+8g+jj)] of mode 16w+i (B operand of the U update)
    float eR[4][4], eI[4][4];    // [tt][jj]: abar^{t+1}, t = 16tt+i, mode 16w+4g+jj
    float aLUr, aLUi;            // abar^L of mode 16w+i
    float aLGr[4][4], aLGi[4][4];  // [kb][jj]: abar^L of mode 16kb+4g+jj
};

// ZOH set-up of one head.  Round 1 fills tab with T[k][m] = bbar abar^k
// (fp64 recurrence from an fp64 power, stored fp32) and derives the fp16
// tables tpT, fT and the fragments aT, bF; round 2 fills tab with abar^k
// (k = 1..L at row k-1) for e, aL.  Leaves the tab region free.
template <int D>
__device__ void zoh_setup(Smem<D>& sm, const idattn_params& prm, int64_t h, int64_t M, Consts& cs) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid >> 6, g = lane >> 4, i = lane & 15;
    const float log_dt = prm.log_dt[h];
    const double dt = exp(static_cast<double>(log_dt));
    cs.dt = static_cast<float>(dt);
    cs.inv_dt = static_cast<float>(1.0 / dt);
    const int m = tid & (MM - 1);
    const int kq = tid >> 6;  // 0..3 -> k in [16 kq, 16 kq + 16)
    const float lre = prm.A[(h * M + m) * 2], lim = prm.A[(h * M + m) * 2 + 1];
    const Zoh z = zoh_mode(log_dt, lre, lim, prm.Bc[(h * M + m) * 2], prm.Bc[(h * M + m) * 2 + 1]);
    {
        double pr, pi;
        cpow(dt, lre, lim, 16.0 * kq, pr, pi);
        double tr = z.br * pr - z.bi * pi, ti = z.br * pi + z.bi * pr;  // bbar abar^k
        for (int k = 16 * kq; k < 16 * kq + 16; ++k) {
            sm.u.tab[k * MM + m] = make_float2(static_cast<float>(tr), static_cast<float>(ti));
            const double nr = tr * z.ar - ti * z.ai, ni = tr * z.ai + ti * z.ar;
            tr = nr;
            ti = ni;
        }
    }
    __syncthreads();
    for (int e = tid; e < L * M2; e += NTH) {
        const int kc = e / M2, mp = e % M2;
        const float2 t = sm.u.tab[kc * MM + blk_mode(mp)];
        sm.tpT[kc * RL_M + mp] = static_cast<_Float16>((blk_part(mp) ? -t.y : t.x) * cs.inv_dt);
    }
    for (int e = tid; e < M2 * L; e += NTH) {
        const int mp = e / L, j = e % L;
        const float2 t = sm.u.tab[(L - 1 - j) * MM + blk_mode(mp)];
        sm.fT[mp * RL_L + j] = static_cast<_Float16>(blk_part(mp) ? t.y : t.x);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int k = 32 * kb + 8 * g + jj;
            const float2 t = sm.u.tab[k * MM + 16 * w + i];
            const float2 f = sm.u.tab[(L - 1 - k) * MM + 16 * w + i];
            cs.aT[kb][0][jj] = static_cast<_Float16>(t.x);
            cs.aT[kb][1][jj] = static_cast<_Float16>(t.y);
            cs.bF[kb][0][jj] = static_cast<_Float16>(f.x);
            cs.bF[kb][1][jj] = static_cast<_Float16>(f.y);
        }
    __syncthreads();
    {
        double pr, pi;
        cpow(dt, lre, lim, 16.0 * kq + 1.0, pr, pi);
        for (int k = 16 * kq; k < 16 * kq + 16; ++k) {
            sm.u.tab[k * MM + m] = make_float2(static_cast<float>(pr), static_cast<float>(pi));
            const double nr = pr * z.ar - pi * z.ai, ni = pr * z.ai + pi * z.ar;
            pr = nr;
            pi = ni;
        }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float2 e = sm.u.tab[(16 * tt + i) * MM + 16 * w + 4 * g + jj];
            cs.eR[tt][jj] = e.x;
            cs.eI[tt][jj] = e.y;
            const float2 a = sm.u.tab[(L - 1) * MM + 16 * tt + 4 * g + jj];
            cs.aLGr[tt][jj] = a.x;
            cs.aLGi[tt][jj] = a.y;
        }
    {
        const float2 a = sm.u.tab[(L - 1) * MM + 16 * w + i];
        cs.aLUr = a.x;
        cs.aLUi = a.y;
    }
    __syncthreads();
}

// ------------------------------------------------------------------ featmap
// Thread mapping: channel group cg (8 channels) = tid % CG, token slot
// tq = tid / CG, tokens tq + TQ n.  A token's CG channel groups are CG
// consecutive lanes, so norms reduce with CG-lane butterflies.
template <int D>
struct FeatMap {
    static constexpr int CG = D / 8;
    static constexpr int TQ = NTH / CG;
    static constexpr int NTOK = L / TQ;
};

template <int D>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = FeatMap<D>::CG / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Raw bf16 rows of one chunk held in registers between the prefetch and the
// featmap (8 channels of NTOK tokens per thread).
template <int D, bool WITH_Q>
struct RawRegs {
    uint4 q[WITH_Q ? FeatMap<D>::NTOK : 1];
    uint4 k[FeatMap<D>::NTOK];
    uint4 v[FeatMap<D>::NTOK];
};

template <int D, bool WITH_Q>
__device__ __forceinline__ void prefetch_chunk(RawRegs<D, WITH_Q>& r, const uint16_t* q, const uint16_t* k,
                                               const uint16_t* v, int64_t b, int64_t h, int64_t N, int64_t H,
                                               int64_t t0, int n) {
    const int tid = threadIdx.x;
    const int cg = tid % FeatMap<D>::CG, tq = tid / FeatMap<D>::CG;
#pragma unroll
    for (int s = 0; s < FeatMap<D>::NTOK; ++s) {
        const int t = tq + FeatMap<D>::TQ * s;
        if (t < n) {
            const int64_t off = ((b * N + t0 + t) * H + h) * D + 8 * cg;
            if constexpr (WITH_Q) r.q[s] = *reinterpret_cast<const uint4*>(q + off);
            r.k[s] = *reinterpret_cast<const uint4*>(k + off);
            r.v[s] = *reinterpret_cast<const uint4*>(v + off);
        } else {
            if constexpr (WITH_Q) r.q[s] = make_uint4(0, 0, 0, 0);
            r.k[s] = make_uint4(0, 0, 0, 0);
            r.v[s] = make_uint4(0, 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void unpack8(const uint4& u, float* x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

__device__ __forceinline__ float silu_fast(float c) { return c * __frcp_rn(1.f + __expf(-c)); }

// Featmap of one chunk (n valid tokens; the rest are zeros).  Reads the raw
// rows from registers (written here to shared memory for the conv window) and
// the halo buffer `par`; writes yq, sig (WITH_Q), zkT, zk (WITH_Q), zvT, and
// the next halo buffer.  Ends without a barrier.
template <int D, bool WITH_Q>
__device__ void featmap_chunk(Smem<D>& sm, const RawRegs<D, WITH_Q>& r, const idattn_params& prm, int64_t h,
                              int W, float eps_feat, float eps_norm, int par, int n) {
    using FM = FeatMap<D>;
    constexpr int RL_D = Smem<D>::RL_D;
    const int tid = threadIdx.x;
    const int cg = tid % FM::CG, tq = tid / FM::CG;
    // 1. raw rows to shared memory
#pragma unroll
    for (int s = 0; s < FM::NTOK; ++s) {
        const int t = tq + FM::TQ * s;
        if constexpr (WITH_Q) *reinterpret_cast<uint4*>(&sm.u.raw.q[t * RL_D + 8 * cg]) = r.q[s];
        *reinterpret_cast<uint4*>(&sm.u.raw.k[t * RL_D + 8 * cg]) = r.k[s];
    }
    __syncthreads();
    const float* gk = prm.gain + h * 2 * D;
    const float* bk = prm.bias + h * 2 * D;
    float gkv[8], bkv[8], gvv[8], bvv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        gkv[e] = gk[8 * cg + e];
        bkv[e] = bk[8 * cg + e];
        gvv[e] = gk[D + 8 * cg + e];
        bvv[e] = bk[D + 8 * cg + e];
    }
#pragma unroll
    for (int s = 0; s < FM::NTOK; ++s) {
        const int t = tq + FM::TQ * s;
        float cq[8], ck[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cq[e] = ck[e] = 0.f;
        for (int j = 0; j < W; ++j) {
            const int p = t - (W - 1) + j;  // position in the chunk; < 0 -> halo
            const uint16_t* rq = p >= 0 ? &sm.u.raw.q[p * RL_D + 8 * cg] : &sm.halo[par][0][p + 3][8 * cg];
            const uint16_t* rk = p >= 0 ? &sm.u.raw.k[p * RL_D + 8 * cg] : &sm.halo[par][1][p + 3][8 * cg];
            float xk[8];
            unpack8(*reinterpret_cast<const uint4*>(rk), xk);
#pragma unroll
            for (int e = 0; e < 8; ++e) ck[e] = fmaf(sm.wk[(8 * cg + e) * kMaxW + j], xk[e], ck[e]);
            if constexpr (WITH_Q) {
                float xq[8];
                unpack8(*reinterpret_cast<const uint4*>(rq), xq);
#pragma unroll
                for (int e = 0; e < 8; ++e) cq[e] = fmaf(sm.wq[(8 * cg + e) * kMaxW + j], xq[e], cq[e]);
            }
        }
        const bool valid = t < n;
        float yk[8], sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            yk[e] = silu_fast(ck[e]);
            sk = fmaf(yk[e], yk[e], sk);
        }
        sk = group_sum<D>(sk);
        const float inv_k = 1.f / (sk + eps_feat);
        // mean over R of xi_k^2 = sk / (sk + eps)^2 / R
        const float rk = rsqrtf(sk * inv_k * inv_k / D + eps_norm) * inv_k;
        float xv[8], sv = 0.f;
        unpack8(r.v[s], xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) sv = fmaf(xv[e], xv[e], sv);
        sv = group_sum<D>(sv);
        const float rv = rsqrtf(sv / D + eps_norm);
        half8 zk8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float zkf = valid ? fmaf(gkv[e] * yk[e], rk, bkv[e]) : 0.f;
            const float zvf = valid ? fmaf(gvv[e] * xv[e], rv, bvv[e]) : 0.f;
            zk8[e] = static_cast<_Float16>(zkf);
            sm.zkT[(8 * cg + e) * RL_L + t] = static_cast<_Float16>(zkf);
            sm.zvT[(8 * cg + e) * RL_L + t] = static_cast<_Float16>(zvf);
        }
        if constexpr (WITH_Q) {
            *reinterpret_cast<half8*>(&sm.zk[t * RL_D + 8 * cg]) = zk8;
            float yq[8], sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                yq[e] = silu_fast(cq[e]);
                sq = fmaf(yq[e], yq[e], sq);
            }
            sq = group_sum<D>(sq);
            half8 y8;
#pragma unroll
            for (int e = 0; e < 8; ++e) y8[e] = static_cast<_Float16>(valid ? yq[e] : 0.f);
            *reinterpret_cast<half8*>(&sm.yq[t * RL_D + 8 * cg]) = y8;
            if (cg == 0) sm.sig[t] = valid ? 1.f / (sq + eps_feat) : 0.f;
        }
        // raw rows of the chunk's last 3 tokens become the next halo
        if (t >= L - 3) {
            if constexpr (WITH_Q)
                *reinterpret_cast<uint4*>(&sm.halo[par ^ 1][0][t - (L - 3)][8 * cg]) = *reinterpret_cast<const uint4*>(&sm.u.raw.q[t * RL_D + 8 * cg]);
            *reinterpret_cast<uint4*>(&sm.halo[par ^ 1][1][t - (L - 3)][8 * cg]) = *reinterpret_cast<const uint4*>(&sm.u.raw.k[t * RL_D + 8 * cg]);
        }
    }
}


// Conv weights of head h (taps beyond W are zero) and the halo of the first
// chunk of a segment starting at t0: raw q, k at t0-3..t0-1 from the input
// (position >= 0), from tail_in (position < 0) or zeros.
template <int D>
__device__ void load_prologue(Smem<D>& sm, const idattn_params& prm, const uint16_t* q, const uint16_t* k,
                              const uint16_t* tail_in, int64_t b, int64_t h, int64_t N, int64_t H, int64_t t0,
                              int W) {
    for (int e = threadIdx.x; e < D * kMaxW; e += NTH) {
        const int c = e / kMaxW, j = e % kMaxW;
        sm.wq[e] = j < W ? prm.conv_q[(h * D + c) * W + j] : 0.f;
        sm.wk[e] = j < W ? prm.conv_k[(h * D + c) * W + j] : 0.f;
    }
    for (int e = threadIdx.x; e < 2 * 3 * D; e += NTH) {
        const int sel = e / (3 * D), row = (e / D) % 3, c = e % D;
        const int64_t pos = t0 - 3 + row;
        uint16_t val = 0;
        if (pos >= 0) {
            val = (sel == 0 ? q : k)[((b * N + pos) * H + h) * D + c];
        } else if (tail_in != nullptr && pos >= -(W - 1)) {
            const int64_t slot = (W - 1) + pos;
            val = tail_in[(((b * H + h) * 2 + sel) * (W - 1) + slot) * D + c];
        }
        sm.halo[0][sel][row][c] = val;
    }
}

// ------------------------------------------------------------------ states
// Register layout (lane g*16+i of wave w):
//   U[rt][part][jj]    = U_m[r]     with r = 16rt+4g+jj, m = 16w+i
//   Gam[mt][ct][jj]    = Gamma_m[c] with m = 16(mt/2)+4g+jj, part = mt%2,
//                                   c = w*D/4 + 16ct + i
// Memory layout: float [M][2D][2], columns 0..D-1 hold U, D..2D-1 hold Gamma.
template <int D>
struct State {
    static constexpr int RT = D / 16;
    static constexpr int CW = D / 64;
    f4 U[RT][2];
    f4 Gam[8][CW];
};

template <int D>
__device__ void state_load(State<D>& st, const float* src) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int rt = 0; rt < State<D>::RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * rt + 4 * g + jj, m = 16 * w + i;
            const float2 x = src ? *reinterpret_cast<const float2*>(src + (static_cast<int64_t>(m) * 2 * D + r) * 2)
                                 : make_float2(0.f, 0.f);
            st.U[rt][0][jj] = x.x;
            st.U[rt][1][jj] = x.y;
        }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int ct = 0; ct < State<D>::CW; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 16 * (mt / 2) + 4 * g + jj, c = w * (D / 4) + 16 * ct + i;
                st.Gam[mt][ct][jj] = src ? src[(static_cast<int64_t>(m) * 2 * D + D + c) * 2 + (mt & 1)] : 0.f;
            }
}

// Stores the state, first multiplying every mode by abar^{-back} (undoes
// `back` zero-input steps of a zero-padded last chunk).
template <int D>
__device__ void state_store(const State<D>& st, float* dst, const idattn_params& prm, int64_t h, int64_t M,
                            int back) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
    const double dt = exp(static_cast<double>(prm.log_dt[h]));
    {
        const int m = 16 * w + i;
        double cr = 1.0, ci = 0.0;
        if (back) cpow(dt, prm.A[(h * M + m) * 2], prm.A[(h * M + m) * 2 + 1], -static_cast<double>(back), cr, ci);
        const float fr = static_cast<float>(cr), fi = static_cast<float>(ci);
#pragma unroll
        for (int rt = 0; rt < State<D>::RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rt + 4 * g + jj;
                const float ur = st.U[rt][0][jj], ui = st.U[rt][1][jj];
                *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + r) * 2) =
                    make_float2(fr * ur - fi * ui, fr * ui + fi * ur);
            }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int m = 16 * kb + 4 * g + jj;
            double cr = 1.0, ci = 0.0;
            if (back) cpow(dt, prm.A[(h * M + m) * 2], prm.A[(h * M + m) * 2 + 1], -static_cast<double>(back), cr, ci);
            const float fr = static_cast<float>(cr), fi = static_cast<float>(ci);
#pragma unroll
            for (int ct = 0; ct < State<D>::CW; ++ct) {
                const int c = w * (D / 4) + 16 * ct + i;
                const float gr = st.Gam[2 * kb][ct][jj], gi = st.Gam[2 * kb + 1][ct][jj];
                *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + D + c) * 2) =
                    make_float2(fr * gr - fi * gi, fr * gi + fi * gr);
            }
        }
}

// U <- abar^L U + Z_k^T F   and   Gamma <- abar^L Gamma + F^T Z_v
template <int D>
__device__ __forceinline__ void key_state_update(State<D>& st, const Smem<D>& sm, const Consts& cs) {
    const int lane = threadIdx.x & (kWave - 1), g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int rt = 0; rt < State<D>::RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float ur = st.U[rt][0][jj], ui = st.U[rt][1][jj];
            st.U[rt][0][jj] = cs.aLUr * ur - cs.aLUi * ui;
            st.U[rt][1][jj] = cs.aLUr * ui + cs.aLUi * ur;
        }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rt = 0; rt < State<D>::RT; ++rt) {
            const half8 a = ld8(&sm.zkT[(16 * rt + i) * RL_L + 32 * kb + 8 * g]);
            st.U[rt][0] = mfma(a, cs.bF[kb][0], st.U[rt][0]);
            st.U[rt][1] = mfma(a, cs.bF[kb][1], st.U[rt][1]);
        }
}

template <int D>
__device__ __forceinline__ void value_state_update(State<D>& st, const Smem<D>& sm, const Consts& cs,
                                                   const half8 (&bZ)[2][State<D>::CW]) {
    const int lane = threadIdx.x & (kWave - 1), i = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ct = 0; ct < State<D>::CW; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float gr = st.Gam[2 * kb][ct][jj], gi = st.Gam[2 * kb + 1][ct][jj];
                st.Gam[2 * kb][ct][jj] = cs.aLGr[kb][jj] * gr - cs.aLGi[kb][jj] * gi;
                st.Gam[2 * kb + 1][ct][jj] = cs.aLGr[kb][jj] * gi + cs.aLGi[kb][jj] * gr;
            }
    const int g = lane >> 4;
#pragma unroll
    for (int kbj = 0; kbj < 2; ++kbj)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const half8 a = ld8(&sm.fT[(16 * mt + i) * RL_L + 32 * kbj + 8 * g]);
#pragma unroll
            for (int ct = 0; ct < State<D>::CW; ++ct) st.Gam[mt][ct] = mfma(a, bZ[kbj][ct], st.Gam[mt][ct]);
        }
}

template <int D>
__device__ __forceinline__ void load_bz(half8 (&bZ)[2][State<D>::CW], const Smem<D>& sm) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int kbj = 0; kbj < 2; ++kbj)
#pragma unroll
        for (int ct = 0; ct < State<D>::CW; ++ct)
            bZ[kbj][ct] = ld8(&sm.zvT[(w * (D / 4) + 16 * ct + i) * RL_L + 32 * kbj + 8 * g]);
}

// ------------------------------------------------------------------ kernels
// Segment end states from a zero start: grid B*H*(S-1), block (bh, seg).
template <int D>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void segment_state_kernel(Problem p, idattn_params prm, const uint16_t* __restrict__ k,
                          const uint16_t* __restrict__ v, const uint16_t* __restrict__ tail_in,
                          float* __restrict__ ws, int64_t Lseg, int S) {
    __shared__ Smem<D> sm;
    const int64_t bh = blockIdx.x / (S - 1);
    const int seg = static_cast<int>(blockIdx.x % (S - 1));
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t t_begin = seg * Lseg, t_end = t_begin + Lseg;  // segments 0..S-2 are full
    const int W = static_cast<int>(p.W);
    Consts cs;
    zoh_setup<D>(sm, prm, h, p.M, cs);
    load_prologue<D>(sm, prm, k, k, tail_in, b, h, p.N, p.H, t_begin, W);
    State<D> st;
    state_load<D>(st, nullptr);
    RawRegs<D, false> rr;
    prefetch_chunk<D, false>(rr, nullptr, k, v, b, h, p.N, p.H, t_begin, L);
    int par = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += L) {
        featmap_chunk<D, false>(sm, rr, prm, h, W, p.eps_feat, p.eps_norm, par, L);
        if (t0 + L < t_end) prefetch_chunk<D, false>(rr, nullptr, k, v, b, h, p.N, p.H, t0 + L, L);
        __syncthreads();
        key_state_update<D>(st, sm, cs);
        half8 bZ[2][State<D>::CW];
        load_bz<D>(bZ, sm);
        value_state_update<D>(st, sm, cs, bZ);
        __syncthreads();
        par ^= 1;
    }
    state_store<D>(st, ws + (static_cast<int64_t>(seg) * p.B * p.H + bh) * p.M * 2 * D * 2, prm, h, p.M, 0);
}

// Carry chain over segments, one thread per complex state element:
// ws[seg] <- state entering segment seg+1.
__global__ __launch_bounds__(256) void segment_carry_kernel(Problem p, idattn_params prm,
                                                            const float* __restrict__ state_in,
                                                            float* __restrict__ ws, int64_t Lseg, int S) {
    const int64_t total = p.B * p.H * p.M * 2 * p.d;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t m = (e / (2 * p.d)) % p.M;
    const int64_t h = (e / (2 * p.d * p.M)) % p.H;
    const double dt = exp(static_cast<double>(prm.log_dt[h]));
    double pr, pi;
    cpow(dt, prm.A[(h * p.M + m) * 2], prm.A[(h * p.M + m) * 2 + 1], static_cast<double>(Lseg), pr, pi);
    const float ar = static_cast<float>(pr), ai = static_cast<float>(pi);
    float2 c = state_in ? reinterpret_cast<const float2*>(state_in)[e] : make_float2(0.f, 0.f);
    float2* w2 = reinterpret_cast<float2*>(ws);
    for (int seg = 0; seg + 1 < S; ++seg) {
        const float2 loc = w2[seg * total + e];
        c = make_float2(ar * c.x - ai * c.y + loc.x, ar * c.y + ai * c.x + loc.y);
        w2[seg * total + e] = c;
    }
}

// Full chunk loop of one segment: grid B*H*S, block (bh, seg).
template <int D>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunked_forward_kernel(Problem p, idattn_params prm, const uint16_t* __restrict__ q,
                            const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                            uint16_t* __restrict__ o, const float* state_in, const uint16_t* __restrict__ tail_in,
                            float* state_out, const float* __restrict__ carry, int64_t Lseg, int S) {
    using ST = State<D>;
    constexpr int RL_D = Smem<D>::RL_D;
    constexpr int KB = D / 32;  // k-blocks over the R channels
    constexpr int CW = ST::CW;
    __shared__ Smem<D> sm;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid >> 6, g = lane >> 4, i = lane & 15;
    const int64_t bh = blockIdx.x / S;
    const int seg = static_cast<int>(blockIdx.x % S);
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t N = p.N, H = p.H;
    const int64_t t_begin = seg * Lseg;
    const int64_t t_end = t_begin + Lseg < N ? t_begin + Lseg : N;
    const int W = static_cast<int>(p.W);
    const int cbase = w * (D / 4);

    Consts cs;
    zoh_setup<D>(sm, prm, h, p.M, cs);
    load_prologue<D>(sm, prm, q, k, tail_in, b, h, N, H, t_begin, W);
    ST st;
    {
        const float* src = seg == 0 ? (state_in ? state_in + bh * p.M * 2 * D * 2 : nullptr)
                                    : carry + (static_cast<int64_t>(seg - 1) * p.B * p.H + bh) * p.M * 2 * D * 2;
        state_load<D>(st, src);
    }
    RawRegs<D, true> rr;
    prefetch_chunk<D, true>(rr, q, k, v, b, h, N, H, t_begin, static_cast<int>(t_end - t_begin < L ? t_end - t_begin : L));
    int par = 0;
    int n = L;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += L) {
        n = static_cast<int>(t_end - t0 < L ? t_end - t0 : L);
        featmap_chunk<D, true>(sm, rr, prm, h, W, p.eps_feat, p.eps_norm, par, n);
        if (t0 + L < t_end)
            prefetch_chunk<D, true>(rr, q, k, v, b, h, N, H, t0 + L,
                                    static_cast<int>(t_end - t0 - L < L ? t_end - t0 - L : L));
        __syncthreads();

        // ---- key side: G' (skewed Gram), Q^T = U_prev Y_q^T, U update
        half8 aU[2][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                aU[0][kb][jj] = static_cast<_Float16>(st.U[2 * kb][0][jj]);
                aU[0][kb][4 + jj] = static_cast<_Float16>(st.U[2 * kb + 1][0][jj]);
                aU[1][kb][jj] = static_cast<_Float16>(st.U[2 * kb][1][jj]);
                aU[1][kb][4 + jj] = static_cast<_Float16>(st.U[2 * kb + 1][1][jj]);
            }
        {
            f4 accG[4] = {};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const half8 a = ld8(&sm.yq[(16 * w + i) * RL_D + 32 * kb + 8 * g]);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
                    accG[jt] = mfma(a, ld8(&sm.zk[(16 * jt + i) * RL_D + 32 * kb + 8 * g]), accG[jt]);
            }
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int t = 16 * w + 4 * g + jj, j = 16 * jt + i;
                    if (j <= t) sm.gp[t * RL_L + (t - j)] = static_cast<_Float16>(accG[jt][jj]);
                }
        }
        f4 accQ[2][4] = {};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const _Float16* row = &sm.yq[(16 * tt + i) * RL_D + 32 * kb];
                const half8 bq = cat(ld4(row + 4 * g), ld4(row + 16 + 4 * g));
                accQ[0][tt] = mfma(aU[0][kb], bq, accQ[0][tt]);
                accQ[1][tt] = mfma(aU[1][kb], bq, accQ[1][tt]);
            }
        key_state_update<D>(st, sm, cs);
        __syncthreads();

        // ---- S^T = T^T G'^T, then s = sigma (S + abar^{t+1} Q)
        {
            f4 accS[2][4] = {};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    half8 bg = ld8(&sm.gp[(16 * tt + i) * RL_L + 32 * kb + 8 * g]);
                    const int t = 16 * tt + i;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        if (32 * kb + 8 * g + jj > t) bg[jj] = static_cast<_Float16>(0.f);
                    accS[0][tt] = mfma(cs.aT[kb][0], bg, accS[0][tt]);
                    accS[1][tt] = mfma(cs.aT[kb][1], bg, accS[1][tt]);
                }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int t = 16 * tt + i;
                const float sg = sm.sig[t];
                half4 sre, sim, xre, xim;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float qr = accQ[0][tt][jj], qi = accQ[1][tt][jj];
                    const float er = cs.eR[tt][jj], ei = cs.eI[tt][jj];
                    const float sr = sg * (accS[0][tt][jj] + er * qr - ei * qi);
                    const float si = sg * (accS[1][tt][jj] + er * qi + ei * qr);
                    sre[jj] = static_cast<_Float16>(sr);
                    sim[jj] = static_cast<_Float16>(si);
                    xre[jj] = static_cast<_Float16>((sr * er - si * ei) * cs.inv_dt);
                    xim[jj] = static_cast<_Float16>(-(sr * ei + si * er) * cs.inv_dt);
                }
                _Float16* srow = &sm.u.v.s[t * RL_M + 32 * w + 4 * g];
                _Float16* xrow = &sm.u.v.se[t * RL_M + 32 * w + 4 * g];
                *reinterpret_cast<half4*>(srow) = sre;
                *reinterpret_cast<half4*>(srow + 16) = sim;
                *reinterpret_cast<half4*>(xrow) = xre;
                *reinterpret_cast<half4*>(xrow + 16) = xim;
            }
        }
        __syncthreads();

        // ---- value side: P' and P, O_inter = (s abar^{t+1}) Gamma_prev, Gamma update
        half8 bG[4][CW];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int ct = 0; ct < CW; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bG[kb][ct][jj] = static_cast<_Float16>(st.Gam[2 * kb][ct][jj]);
                    bG[kb][ct][4 + jj] = static_cast<_Float16>(st.Gam[2 * kb + 1][ct][jj]);
                }
        {
            f4 accP[4] = {};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const half8 a = ld8(&sm.u.v.s[(16 * w + i) * RL_M + 32 * kb + 8 * g]);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    accP[kt] = mfma(a, ld8(&sm.tpT[(16 * kt + i) * RL_M + 32 * kb + 8 * g]), accP[kt]);
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int t = 16 * w + 4 * g + jj, kc = 16 * kt + i;
                    if (kc <= t) sm.gp[t * RL_L + (t - kc)] = static_cast<_Float16>(accP[kt][jj]);
                }
        }
        f4 accO[4][CW] = {};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const _Float16* row = &sm.u.v.se[(16 * tt + i) * RL_M + 32 * kb];
                const half8 a = cat(ld4(row + 4 * g), ld4(row + 16 + 4 * g));
#pragma unroll
                for (int ct = 0; ct < CW; ++ct) accO[tt][ct] = mfma(a, bG[kb][ct], accO[tt][ct]);
            }
        half8 bZ[2][CW];
        load_bz<D>(bZ, sm);
        value_state_update<D>(st, sm, cs, bZ);
        __syncthreads();

        // ---- O_intra = P Z_v, output
#pragma unroll
        for (int kbj = 0; kbj < 2; ++kbj)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                half8 a = ld8(&sm.gp[(16 * tt + i) * RL_L + 32 * kbj + 8 * g]);
                const int t = 16 * tt + i;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    if (32 * kbj + 8 * g + jj > t) a[jj] = static_cast<_Float16>(0.f);
#pragma unroll
                for (int ct = 0; ct < CW; ++ct) accO[tt][ct] = mfma(a, bZ[kbj][ct], accO[tt][ct]);
            }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int t = 16 * tt + 4 * g + jj;
                if (t < n) {
                    uint16_t* orow = o + ((b * N + t0 + t) * H + h) * D + cbase + i;
#pragma unroll
                    for (int ct = 0; ct < CW; ++ct) orow[16 * ct] = f32_to_bf16(accO[tt][ct][jj] * cs.dt);
                }
            }
        __syncthreads();
        par ^= 1;
    }
    if (seg == S - 1 && state_out != nullptr)
        state_store<D>(st, state_out + bh * p.M * 2 * D * 2, prm, h, p.M, L - n);
}

void plan_segments(const Problem& p, int& S, int64_t& Lseg) {
    const int64_t pairs = p.B * p.H;
    const int64_t chunks = (p.N + L - 1) / L;
    int64_t s = 256 / pairs;  // one workgroup per compute unit
    if (s < 1) s = 1;
    if (s > chunks) s = chunks > 0 ? chunks : 1;
    const int64_t cps = (chunks + s - 1) / s;  // chunks per segment
    Lseg = cps * L;
    S = static_cast<int>((p.N + Lseg - 1) / Lseg);
    if (S < 1) S = 1;
}

}  // namespace

bool chunked_supported(const Problem& p) {
    return p.bf16 && p.M == MM && (p.d == 64 || p.d == 128) && p.W >= 1 && p.W <= kMaxW;
}

size_t chunked_workspace_bytes(const Problem& p) {
    int S;
    int64_t Lseg;
    plan_segments(p, S, Lseg);
    return static_cast<size_t>(S - 1) * p.B * p.H * p.M * 2 * p.d * 2 * sizeof(float);
}

hipError_t launch_forward_chunked(const Problem& p, const idattn_params& prm, const void* q, const void* k,
                                  const void* v, void* o, const float* state_in, const void* tail_in,
                                  float* state_out, void* workspace, hipStream_t stream) {
    int S;
    int64_t Lseg;
    plan_segments(p, S, Lseg);
    const auto* q16 = static_cast<const uint16_t*>(q);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const auto* t16 = static_cast<const uint16_t*>(tail_in);
    float* ws = static_cast<float*>(workspace);
    const int64_t pairs = p.B * p.H;
    if (S > 1) {
        const dim3 g1(static_cast<unsigned>(pairs * (S - 1)));
        if (p.d == 128)
            segment_state_kernel<128><<<g1, NTH, 0, stream>>>(p, prm, k16, v16, t16, ws, Lseg, S);
        else
            segment_state_kernel<64><<<g1, NTH, 0, stream>>>(p, prm, k16, v16, t16, ws, Lseg, S);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t total = pairs * p.M * 2 * p.d;
        segment_carry_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(
            p, prm, state_in, ws, Lseg, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 g3(static_cast<unsigned>(pairs * S));
    if (p.d == 128)
        chunked_forward_kernel<128><<<g3, NTH, 0, stream>>>(p, prm, q16, k16, v16, static_cast<uint16_t*>(o),
                                                            state_in, t16, state_out, ws, Lseg, S);
    else
        chunked_forward_kernel<64><<<g3, NTH, 0, stream>>>(p, prm, q16, k16, v16, static_cast<uint16_t*>(o),
                                                           state_in, t16, state_out, ws, Lseg, S);
    return hipGetLastError();
}

}  // namespace idattn

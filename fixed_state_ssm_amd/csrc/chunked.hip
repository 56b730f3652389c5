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
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // 8 bf16 values

__device__ __forceinline__ f4 mfma(const half8& a, const half8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 ld8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i & 3) of the 4-element read of lane 4j + (i >> 2), for j = 0..3.
typedef short s4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4 ld4_tr(const _Float16* p) {
    const s4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v*)(const_cast<_Float16*>(p)));
    return __builtin_bit_cast(half4, r);
}
// MFMA operand with K along rows of a row-major [k][c] array (row length rl):
// lane (g, i) gets x[k0 + jj][c0 + i], jj = 0..7, with k0 = kbase + 8g.
__device__ __forceinline__ half8 ld8_tr(const _Float16* x, int rl, int kbase, int c0) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    const _Float16* p0 = x + (kbase + 8 * g + (i >> 2)) * rl + c0 + 4 * (i & 3);
    const half4 lo = ld4_tr(p0);
    const half4 hi = ld4_tr(p0 + 4 * rl);
    half8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}
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
    _Float16 zv[L * RL_D];     // z_v [l][c]; holds the raw v rows during the featmap
    float sig[L];              // 1 / (||y_q||^2 + eps_feat)
    // G'[t][k] = G[t][t-k] stored at column L-1-k, and P[t][l]; only the
    // lower-triangular entries are ever written, the rest stay zero
    _Float16 gp[L * RL_L];
    _Float16 pp[L * RL_L];
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
    float2 aL[MM];             // abar^L per mode
    float gain[2 * D], bias[2 * D];  // RMSNorm gain/bias of the head (key half, value half)
    uint16_t halo[2][2][3][D];
    float wq[D * kMaxW], wk[D * kMaxW];
};

// (mode, part) index of row rho of a 32-row block kb: rho < 16 -> re of mode
// 16 kb + rho, else im of mode 16 kb + rho - 16.
__device__ __forceinline__ int blk_mode(int mprime) { return 16 * (mprime >> 5) + (mprime & 15); }
__device__ __forceinline__ int blk_part(int mprime) { return (mprime >> 4) & 1; }

// Complex fp64 power abar^n = exp(n Delta lambda).
__device__ __forceinline__ void cpow(double dt, float lre, float lim, double n, double& pr, double& pi) {
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
    float e0r[4], e0i[4];    // [jj]: abar^{i+1} of mode 16w+4g+jj
    float e16r[4], e16i[4];  // [jj]: abar^{16} of mode 16w+4g+jj; abar^{16tt+i+1} = e0 e16^tt
    float aLUr, aLUi;        // abar^L of mode 16w+i
};

// Per-head tables, computed once per launch by zoh_tables_kernel (fp64
// arithmetic, stored in the shared-memory layouts the chunk kernels use):
//   tpT [L][RL_M] fp16: T'^T[kc][m'] = (T_re | -T_im)[kc][m] / Delta
//   fT  [M2][RL_L] fp16: F^T[m'][j] = (T_re | T_im)[L-1-j][m]
//   pw  [L][MM] float2: abar^{k+1}
//   pwseg[MM], pwback[MM] float2: abar^{Lseg}, abar^{-back}
//   hc: Delta, 1/Delta
// with T[k][m] = bbar_m abar_m^k and m' = 32 (m / 16) + 16 part + m % 16.
constexpr int kTabTpT = 0;
constexpr int kTabFT = kTabTpT + ((L * RL_M * 2 + 255) / 256) * 256;
constexpr int kTabPw = kTabFT + ((M2 * RL_L * 2 + 255) / 256) * 256;
constexpr int kTabPwSeg = kTabPw + L * MM * 8;
constexpr int kTabPwBack = kTabPwSeg + MM * 8;
constexpr int kTabHc = kTabPwBack + MM * 8;
constexpr int kTabBytes = ((kTabHc + 16 + 255) / 256) * 256;

__global__ __launch_bounds__(NTH) void zoh_tables_kernel(Problem p, idattn_params prm, int64_t Lseg, int back,
                                                         uint8_t* __restrict__ tab) {
    const int64_t h = blockIdx.x;
    uint8_t* th = tab + h * kTabBytes;
    _Float16* tpT = reinterpret_cast<_Float16*>(th + kTabTpT);
    _Float16* fT = reinterpret_cast<_Float16*>(th + kTabFT);
    float2* pw = reinterpret_cast<float2*>(th + kTabPw);
    const int tid = threadIdx.x;
    const int m = tid & (MM - 1);
    const int kq = tid >> 6;  // k in [16 kq, 16 kq + 16)
    const int64_t M = p.M;
    const float log_dt = prm.log_dt[h];
    const double dt = exp(static_cast<double>(log_dt));
    const float lre = prm.A[(h * M + m) * 2], lim = prm.A[(h * M + m) * 2 + 1];
    const Zoh z = zoh_mode(log_dt, lre, lim, prm.Bc[(h * M + m) * 2], prm.Bc[(h * M + m) * 2 + 1]);
    const int mre = 32 * (m >> 4) + (m & 15), mim = mre + 16;
    const float inv_dt = static_cast<float>(1.0 / dt);
    double pr, pi;
    cpow(dt, lre, lim, 16.0 * kq, pr, pi);  // abar^k
    for (int k = 16 * kq; k < 16 * kq + 16; ++k) {
        const double tr = z.br * pr - z.bi * pi, ti = z.br * pi + z.bi * pr;  // bbar abar^k
        const double nr = pr * z.ar - pi * z.ai, ni = pr * z.ai + pi * z.ar;  // abar^{k+1}
        pw[k * MM + m] = make_float2(static_cast<float>(nr), static_cast<float>(ni));
        tpT[k * RL_M + mre] = static_cast<_Float16>(static_cast<float>(tr) * inv_dt);
        tpT[k * RL_M + mim] = static_cast<_Float16>(-static_cast<float>(ti) * inv_dt);
        fT[mre * RL_L + (L - 1 - k)] = static_cast<_Float16>(static_cast<float>(tr));
        fT[mim * RL_L + (L - 1 - k)] = static_cast<_Float16>(static_cast<float>(ti));
        pr = nr;
        pi = ni;
    }
    if (tid < MM) {
        double sr, si;
        cpow(dt, lre, lim, static_cast<double>(Lseg), sr, si);
        reinterpret_cast<float2*>(th + kTabPwSeg)[m] = make_float2(static_cast<float>(sr), static_cast<float>(si));
        cpow(dt, lre, lim, -static_cast<double>(back), sr, si);
        reinterpret_cast<float2*>(th + kTabPwBack)[m] = make_float2(static_cast<float>(sr), static_cast<float>(si));
    }
    if (tid == 0) reinterpret_cast<float2*>(th + kTabHc)[0] = make_float2(static_cast<float>(dt), inv_dt);
}

// Copies one head's tables into shared memory and the lane's constants into
// registers; zeroes the triangular G' and P buffers.  Ends with a barrier.
template <int D>
__device__ __forceinline__ void load_tables(Smem<D>& sm, const uint8_t* th, Consts& cs, bool with_tpT) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid >> 6, g = lane >> 4, i = lane & 15;
    typedef uint32_t u4x __attribute__((ext_vector_type(4)));
    if (with_tpT) {
        const u4x* src = reinterpret_cast<const u4x*>(th + kTabTpT);
        u4x* dst = reinterpret_cast<u4x*>(sm.tpT);
        for (int e = tid; e < L * RL_M * 2 / 16; e += NTH) dst[e] = src[e];
    }
    {
        const u4x* src = reinterpret_cast<const u4x*>(th + kTabFT);
        u4x* dst = reinterpret_cast<u4x*>(sm.fT);
        for (int e = tid; e < M2 * RL_L * 2 / 16; e += NTH) dst[e] = src[e];
    }
    {
        u4x* g0 = reinterpret_cast<u4x*>(sm.gp);
        u4x* p0 = reinterpret_cast<u4x*>(sm.pp);
        for (int e = tid; e < L * RL_L * 2 / 16; e += NTH) g0[e] = p0[e] = u4x{0u, 0u, 0u, 0u};
    }
    const float2* pw = reinterpret_cast<const float2*>(th + kTabPw);
    const float2 hc = reinterpret_cast<const float2*>(th + kTabHc)[0];
    cs.dt = hc.x;
    cs.inv_dt = hc.y;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const float2 e = pw[i * MM + 16 * w + 4 * g + jj];
        cs.e0r[jj] = e.x;
        cs.e0i[jj] = e.y;
        const float2 e16 = pw[15 * MM + 16 * w + 4 * g + jj];
        cs.e16r[jj] = e16.x;
        cs.e16i[jj] = e16.y;
    }
    const float2 a = pw[(L - 1) * MM + 16 * w + i];
    cs.aLUr = a.x;
    cs.aLUi = a.y;
    if (tid < MM) sm.aL[tid] = pw[(L - 1) * MM + tid];
    __syncthreads();
}

// ------------------------------------------------------------------ featmap
// Thread mapping: channel group cgi = tid % 32 owns CPT = D/32 consecutive
// channels, token block tb = tid / 32 owns 8 consecutive tokens of the chunk.
// The short conv slides along a register window of 8 + 3 tokens; the three
// tokens before a block come from the neighbouring block through shared
// memory (or from the previous chunk).  Norms over the D channels of a token
// reduce over the 32 lanes of a token block with DPP and one ds_swizzle.
template <int D>
struct FeatMap {
    static constexpr int CPT = D / 32;  // channels per thread
    static constexpr int TPT = 8;       // tokens per thread
};

typedef uint32_t u2 __attribute__((ext_vector_type(2)));
template <int CPT> struct RawVec;
template <> struct RawVec<4> { typedef u2 T; };
template <> struct RawVec<2> { typedef uint32_t T; };

// Raw bf16 values of one chunk held in registers between the prefetch and
// the featmap: CPT channels of 8 tokens per thread, per tensor.
template <int D, bool WITH_Q>
struct RawRegs {
    typedef typename RawVec<FeatMap<D>::CPT>::T T;
    T q[WITH_Q ? 8 : 1];
    T k[8];
    T v[8];
};

template <int D, bool WITH_Q>
__device__ __forceinline__ void prefetch_chunk(RawRegs<D, WITH_Q>& r, const uint16_t* q, const uint16_t* k,
                                               const uint16_t* v, int64_t b, int64_t h, int64_t N, int64_t H,
                                               int64_t t0, int n) {
    typedef typename RawRegs<D, WITH_Q>::T T;
    constexpr int CPT = FeatMap<D>::CPT;
    const int tid = threadIdx.x;
    const int cgi = tid & 31, tb = tid >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int t = 8 * tb + s;
        if (t < n) {
            const int64_t off = ((b * N + t0 + t) * H + h) * D + CPT * cgi;
            if constexpr (WITH_Q) r.q[s] = *reinterpret_cast<const T*>(q + off);
            r.k[s] = *reinterpret_cast<const T*>(k + off);
            r.v[s] = *reinterpret_cast<const T*>(v + off);
        } else {
            if constexpr (WITH_Q) r.q[s] = T{};
            r.k[s] = T{};
            r.v[s] = T{};
        }
    }
}

template <int CPT>
__device__ __forceinline__ void unpack(const typename RawVec<CPT>::T& u, float* x) {
    if constexpr (CPT == 4) {
        x[0] = __uint_as_float(u[0] << 16);
        x[1] = __uint_as_float(u[0] & 0xffff0000u);
        x[2] = __uint_as_float(u[1] << 16);
        x[3] = __uint_as_float(u[1] & 0xffff0000u);
    } else {
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xffff0000u);
    }
}

// v_rcp_f32 (about 1 ulp); the result is rounded to fp16 before any MFMA.
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float silu_fast(float c) { return c * rcp_fast(1.f + __expf(-c)); }

// Sums over the 32 lanes of a half-wave, for 8 values at once (the steps of
// the 8 reductions are interleaved so that DPP read-after-write hazards are
// covered by independent work); every lane gets the totals.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ void sum32x8(float (&x)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] += dpp_mov<0xB1>(x[s]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] += dpp_mov<0x4E>(x[s]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] += dpp_mov<0x141>(x[s]);  // row_half_mirror
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] += dpp_mov<0x140>(x[s]);  // row_mirror
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[s]), 0x401F));  // xor 16
}

template <int CPT>
__device__ __forceinline__ void store_row(_Float16* dst, const _Float16 (&z)[CPT]) {
    if constexpr (CPT == 4) {
        *reinterpret_cast<half4*>(dst) = half4{z[0], z[1], z[2], z[3]};
    } else {
        typedef _Float16 half2v __attribute__((ext_vector_type(2)));
        *reinterpret_cast<half2v*>(dst) = half2v{z[0], z[1]};
    }
}

// Featmap of one chunk (n valid tokens; the rest are zeros).  Uses the union
// region for the neighbour tails.  Reads the halo buffer `par`; writes yq and
// sig (WITH_Q), zk, zv (row-major fp16) and the next halo buffer.  Ends
// without a barrier.
template <int D, bool WITH_Q>
__device__ __forceinline__ void featmap_chunk(Smem<D>& sm, const RawRegs<D, WITH_Q>& r, float eps_feat,
                                              float eps_norm, int par, int n) {
    constexpr int CPT = FeatMap<D>::CPT;
    constexpr int RL_D = Smem<D>::RL_D;
    typedef typename RawRegs<D, WITH_Q>::T T;
    const int tid = threadIdx.x;
    const int cgi = tid & 31, tb = tid >> 5;
    const int c0 = CPT * cgi;
    // tails of this block for the next block (the last block's feed the next chunk)
    T* tails = reinterpret_cast<T*>(sm.u.raw.k);  // [sel][7 blocks][3][D/CPT]
    constexpr int TW = D / CPT;                     // T-elements per row
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        if (tb < 7) {
            if constexpr (WITH_Q) tails[((0 * 7 + tb) * 3 + j) * TW + cgi] = r.q[5 + j];
            tails[((1 * 7 + tb) * 3 + j) * TW + cgi] = r.k[5 + j];
        } else {
            if constexpr (WITH_Q) *reinterpret_cast<T*>(&sm.halo[par ^ 1][0][j][c0]) = r.q[5 + j];
            *reinterpret_cast<T*>(&sm.halo[par ^ 1][1][j][c0]) = r.k[5 + j];
        }
    }
    lds_barrier();
    // One tensor at a time (keys, values, queries) so that only one set of
    // per-token arrays is live.
    // keys: conv window, SiLU, squared norm, RMSNorm
    {
        float yk[8][CPT], sk[8];
        {
            float x[11][CPT], w[CPT][kMaxW];
#pragma unroll
            for (int c = 0; c < CPT; ++c)
#pragma unroll
                for (int j = 0; j < kMaxW; ++j) w[c][j] = sm.wk[(c0 + c) * kMaxW + j];
#pragma unroll
            for (int j = 0; j < 3; ++j)
                unpack<CPT>(tb == 0 ? *reinterpret_cast<const T*>(&sm.halo[par][1][j][c0])
                                    : tails[((1 * 7 + tb - 1) * 3 + j) * TW + cgi], x[j]);
#pragma unroll
            for (int s = 0; s < 8; ++s) unpack<CPT>(r.k[s], x[3 + s]);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                sk[s] = 0.f;
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < kMaxW; ++j) acc = fmaf(w[c][j], x[s + j][c], acc);
                    yk[s][c] = silu_fast(acc);
                    sk[s] = fmaf(yk[s][c], yk[s][c], sk[s]);
                }
            }
        }
        float gk[CPT], bk[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            gk[c] = sm.gain[c0 + c];
            bk[c] = sm.bias[c0 + c];
        }
        sum32x8(sk);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int t = 8 * tb + s;
            const float ssum = sk[s];
            const float inv_k = rcp_fast(ssum + eps_feat);
            // mean over R of xi_k^2 = ssum / (ssum + eps)^2 / R
            const float rk = rsqrtf(ssum * inv_k * inv_k * (1.f / D) + eps_norm) * inv_k;
            _Float16 z[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) z[c] = static_cast<_Float16>(t < n ? fmaf(gk[c] * yk[s][c], rk, bk[c]) : 0.f);
            store_row<CPT>(&sm.zk[t * RL_D + c0], z);
        }
    }
    // values: RMSNorm
    {
        float gv[CPT], bv[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            gv[c] = sm.gain[D + c0 + c];
            bv[c] = sm.bias[D + c0 + c];
        }
        float sv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            float xv[CPT];
            unpack<CPT>(r.v[s], xv);
            sv[s] = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) sv[s] = fmaf(xv[c], xv[c], sv[s]);
        }
        sum32x8(sv);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int t = 8 * tb + s;
            float xv[CPT];
            unpack<CPT>(r.v[s], xv);
            const float rv = rsqrtf(sv[s] * (1.f / D) + eps_norm);
            _Float16 z[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) z[c] = static_cast<_Float16>(t < n ? fmaf(gv[c] * xv[c], rv, bv[c]) : 0.f);
            store_row<CPT>(&sm.zv[t * RL_D + c0], z);
        }
    }
    // queries: conv window, SiLU; y_q stored unscaled, sigma = 1/(||y_q||^2 + eps)
    if constexpr (WITH_Q) {
        float x[11][CPT], w[CPT][kMaxW];
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
            for (int j = 0; j < kMaxW; ++j) w[c][j] = sm.wq[(c0 + c) * kMaxW + j];
#pragma unroll
        for (int j = 0; j < 3; ++j)
            unpack<CPT>(tb == 0 ? *reinterpret_cast<const T*>(&sm.halo[par][0][j][c0])
                                : tails[((0 * 7 + tb - 1) * 3 + j) * TW + cgi], x[j]);
#pragma unroll
        for (int s = 0; s < 8; ++s) unpack<CPT>(r.q[s], x[3 + s]);
        float sq[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int t = 8 * tb + s;
            sq[s] = 0.f;
            _Float16 y[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < kMaxW; ++j) acc = fmaf(w[c][j], x[s + j][c], acc);
                const float yv = silu_fast(acc);
                sq[s] = fmaf(yv, yv, sq[s]);
                y[c] = static_cast<_Float16>(t < n ? yv : 0.f);
            }
            store_row<CPT>(&sm.yq[t * RL_D + c0], y);
        }
        sum32x8(sq);
        if (cgi == 0) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int t = 8 * tb + s;
                sm.sig[t] = t < n ? rcp_fast(sq[s] + eps_feat) : 0.f;
            }
        }
    }
}

// Conv weights of head h (taps beyond W are zero) and the halo of the first
// chunk of a segment starting at t0: raw q, k at t0-3..t0-1 from the input
// (position >= 0), from tail_in (position < 0) or zeros.
template <int D>
__device__ __forceinline__ void load_prologue(Smem<D>& sm, const idattn_params& prm, const uint16_t* q, const uint16_t* k,
                              const uint16_t* tail_in, int64_t b, int64_t h, int64_t N, int64_t H, int64_t t0,
                              int W) {
    for (int e = threadIdx.x; e < 2 * D; e += NTH) {
        sm.gain[e] = prm.gain[h * 2 * D + e];
        sm.bias[e] = prm.bias[h * 2 * D + e];
    }
    for (int e = threadIdx.x; e < D * kMaxW; e += NTH) {
        const int c = e / kMaxW, j = e % kMaxW;  // slot j holds tap j - (kMaxW - W)
        const int tap = j - (kMaxW - W);
        sm.wq[e] = tap >= 0 ? prm.conv_q[(h * D + c) * W + tap] : 0.f;
        sm.wk[e] = tap >= 0 ? prm.conv_k[(h * D + c) * W + tap] : 0.f;
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
__device__ __forceinline__ void state_load(State<D>& st, const float* src) {
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

// Stores the state, first multiplying every mode by corr[m] (abar^{-back},
// which undoes `back` zero-input steps of a zero-padded last chunk) when
// corr is not NULL.
template <int D>
__device__ __forceinline__ void state_store(const State<D>& st, float* dst, const float2* corr) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
    {
        const int m = 16 * w + i;
        const float2 c = corr ? corr[m] : make_float2(1.f, 0.f);
#pragma unroll
        for (int rt = 0; rt < State<D>::RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rt + 4 * g + jj;
                const float ur = st.U[rt][0][jj], ui = st.U[rt][1][jj];
                *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + r) * 2) =
                    make_float2(c.x * ur - c.y * ui, c.x * ui + c.y * ur);
            }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int m = 16 * kb + 4 * g + jj;
            const float2 c = corr ? corr[m] : make_float2(1.f, 0.f);
#pragma unroll
            for (int ct = 0; ct < State<D>::CW; ++ct) {
                const int cc = w * (D / 4) + 16 * ct + i;
                const float gr = st.Gam[2 * kb][ct][jj], gi = st.Gam[2 * kb + 1][ct][jj];
                *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + D + cc) * 2) =
                    make_float2(c.x * gr - c.y * gi, c.x * gi + c.y * gr);
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
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        // F[j][m'] = T_m[L-1-j], j = 32kb+8g+jj, for (re, im) of mode 16w+i
        const half8 bre = ld8(&sm.fT[(32 * w + i) * RL_L + 32 * kb + 8 * g]);
        const half8 bim = ld8(&sm.fT[(32 * w + 16 + i) * RL_L + 32 * kb + 8 * g]);
#pragma unroll
        for (int rt = 0; rt < State<D>::RT; ++rt) {
            const half8 a = ld8_tr(sm.zk, Smem<D>::RL_D, 32 * kb, 16 * rt);  // z_k[j][r], j along K
            st.U[rt][0] = mfma(a, bre, st.U[rt][0]);
            st.U[rt][1] = mfma(a, bim, st.U[rt][1]);
        }
    }
}

template <int D>
__device__ __forceinline__ void value_state_update(State<D>& st, const Smem<D>& sm, const Consts& cs,
                                                   const half8 (&bZ)[2][State<D>::CW]) {
    const int lane = threadIdx.x & (kWave - 1), i = lane & 15;
    const int g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float2 a = sm.aL[16 * kb + 4 * g + jj];
#pragma unroll
            for (int ct = 0; ct < State<D>::CW; ++ct) {
                const float gr = st.Gam[2 * kb][ct][jj], gi = st.Gam[2 * kb + 1][ct][jj];
                st.Gam[2 * kb][ct][jj] = a.x * gr - a.y * gi;
                st.Gam[2 * kb + 1][ct][jj] = a.x * gi + a.y * gr;
            }
        }
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
            bZ[kbj][ct] = ld8_tr(sm.zv, Smem<D>::RL_D, 32 * kbj, w * (D / 4) + 16 * ct);  // z_v[l][c], l along K
}

// ------------------------------------------------------------------ kernels
// Segment end states from a zero start: grid B*H*(S-1), block (bh, seg).
template <int D>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void segment_state_kernel(Problem p, idattn_params prm, const uint16_t* __restrict__ k,
                          const uint16_t* __restrict__ v, const uint16_t* __restrict__ tail_in,
                          const uint8_t* __restrict__ tab, float* __restrict__ ws, int64_t Lseg, int S) {
    __shared__ Smem<D> sm;
    const int64_t bh = blockIdx.x / (S - 1);
    const int seg = static_cast<int>(blockIdx.x % (S - 1));
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t t_begin = seg * Lseg, t_end = t_begin + Lseg;  // segments 0..S-2 are full
    const int W = static_cast<int>(p.W);
    Consts cs;
    load_prologue<D>(sm, prm, k, k, tail_in, b, h, p.N, p.H, t_begin, W);
    load_tables<D>(sm, tab + h * kTabBytes, cs, false);
    State<D> st;
    state_load<D>(st, nullptr);
    RawRegs<D, false> rr;
    prefetch_chunk<D, false>(rr, nullptr, k, v, b, h, p.N, p.H, t_begin, L);
    int par = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += L) {
        featmap_chunk<D, false>(sm, rr, p.eps_feat, p.eps_norm, par, L);
        if (t0 + L < t_end) prefetch_chunk<D, false>(rr, nullptr, k, v, b, h, p.N, p.H, t0 + L, L);
        lds_barrier();
        key_state_update<D>(st, sm, cs);
        half8 bZ[2][State<D>::CW];
        load_bz<D>(bZ, sm);
        value_state_update<D>(st, sm, cs, bZ);
        lds_barrier();
        par ^= 1;
    }
    state_store<D>(st, ws + (static_cast<int64_t>(seg) * p.B * p.H + bh) * p.M * 2 * D * 2, nullptr);
}

// Carry chain over segments, one thread per complex state element:
// ws[seg] <- state entering segment seg+1.
__global__ __launch_bounds__(256) void segment_carry_kernel(Problem p, const float* __restrict__ state_in,
                                                            const uint8_t* __restrict__ tab,
                                                            float* __restrict__ ws, int S) {
    const int64_t total = p.B * p.H * p.M * 2 * p.d;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t m = (e / (2 * p.d)) % p.M;
    const int64_t h = (e / (2 * p.d * p.M)) % p.H;
    const float2 a = reinterpret_cast<const float2*>(tab + h * kTabBytes + kTabPwSeg)[m];  // abar^{Lseg}
    const float ar = a.x, ai = a.y;
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
                            float* state_out, const uint8_t* __restrict__ tab, const float* __restrict__ carry,
                            int64_t Lseg, int S) {
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
    load_prologue<D>(sm, prm, q, k, tail_in, b, h, N, H, t_begin, W);
    load_tables<D>(sm, tab + h * kTabBytes, cs, true);
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
        featmap_chunk<D, true>(sm, rr, p.eps_feat, p.eps_norm, par, n);
        if (t0 + L < t_end)
            prefetch_chunk<D, true>(rr, q, k, v, b, h, N, H, t0 + L,
                                    static_cast<int>(t_end - t0 - L < L ? t_end - t0 - L : L));
        lds_barrier();

        // ---- key side, part 1: G = Y_q Z_k^T (rows 16w..16w+15), stored skewed as G'
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
                    // G'[t][k] = G[t][t-k] stored at column L-1-k
                    if (j <= t) sm.gp[t * RL_L + (L - 1 - t + j)] = static_cast<_Float16>(accG[jt][jj]);
                }
        }
        lds_barrier();

        // ---- key side, part 2, in two halves of 32 tokens: Q^T = U_prev Y_q^T,
        // S^T = T^T G'^T, s = sigma (S + abar^{t+1} Q); then the U update.
        {
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
            float er4[4], ei4[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                er4[jj] = cs.e0r[jj];
                ei4[jj] = cs.e0i[jj];
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f4 accQ[2][2] = {}, accS[2][2] = {};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int tt = 2 * hf + u;
                        const _Float16* row = &sm.yq[(16 * tt + i) * RL_D + 32 * kb];
                        const half8 bq = cat(ld4(row + 4 * g), ld4(row + 16 + 4 * g));
                        accQ[0][u] = mfma(aU[0][kb], bq, accQ[0][u]);
                        accQ[1][u] = mfma(aU[1][kb], bq, accQ[1][u]);
                    }
                // K order of both operands: element jj <-> k = 32kb+8g+7-jj, so
                // that T^T rows come straight from fT (F = T reversed) and G'
                // from its reversed store.
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int col = L - 8 - 32 * kb - 8 * g;
                    const half8 are = ld8(&sm.fT[(32 * w + i) * RL_L + col]);
                    const half8 aim = ld8(&sm.fT[(32 * w + 16 + i) * RL_L + col]);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = 16 * (2 * hf + u) + i;
                        const half8 bg = ld8(&sm.gp[t * RL_L + col]);  // zero where k > t
                        accS[0][u] = mfma(are, bg, accS[0][u]);
                        accS[1][u] = mfma(aim, bg, accS[1][u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int t = 16 * (2 * hf + u) + i;
                    const float sg = sm.sig[t];
                    half4 sre, sim, xre, xim;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float qr = accQ[0][u][jj], qi = accQ[1][u][jj];
                        const float er = er4[jj], ei = ei4[jj];
                        er4[jj] = er * cs.e16r[jj] - ei * cs.e16i[jj];
                        ei4[jj] = er * cs.e16i[jj] + ei * cs.e16r[jj];
                        const float sr = sg * (accS[0][u][jj] + er * qr - ei * qi);
                        const float si = sg * (accS[1][u][jj] + er * qi + ei * qr);
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
        }
        key_state_update<D>(st, sm, cs);
        lds_barrier();

        // ---- value side, part 1: P'[t][k] = Re sum_m s_m(t) T_m[k] / Delta (rows
        // 16w..16w+15), un-skewed into P[t][l] = P'[t][t-l]
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
                    if (kc <= t) sm.pp[t * RL_L + (t - kc)] = static_cast<_Float16>(accP[kt][jj]);
                }
        }
        lds_barrier();

        // ---- value side, part 2, in two halves: o = (s abar^{t+1}) Gamma_prev + P Z_v,
        // then the Gamma update
        {
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
            half8 bZ[2][CW];
            load_bz<D>(bZ, sm);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f4 accO[2][CW] = {};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const _Float16* row = &sm.u.v.se[(16 * (2 * hf + u) + i) * RL_M + 32 * kb];
                        const half8 a = cat(ld4(row + 4 * g), ld4(row + 16 + 4 * g));
#pragma unroll
                        for (int ct = 0; ct < CW; ++ct) accO[u][ct] = mfma(a, bG[kb][ct], accO[u][ct]);
                    }
#pragma unroll
                for (int kbj = 0; kbj < 2; ++kbj)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = 16 * (2 * hf + u) + i;
                        const half8 a = ld8(&sm.pp[t * RL_L + 32 * kbj + 8 * g]);  // zero where l > t
#pragma unroll
                        for (int ct = 0; ct < CW; ++ct) accO[u][ct] = mfma(a, bZ[kbj][ct], accO[u][ct]);
                    }
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int t = 16 * (2 * hf + u) + 4 * g + jj;
                        if (t < n) {
                            uint16_t* orow = o + ((b * N + t0 + t) * H + h) * D + cbase + i;
#pragma unroll
                            for (int ct = 0; ct < CW; ++ct) orow[16 * ct] = f32_to_bf16(accO[u][ct][jj] * cs.dt);
                        }
                    }
            }
            value_state_update<D>(st, sm, cs, bZ);
        }
        lds_barrier();
        par ^= 1;
    }
    if (seg == S - 1 && state_out != nullptr)
        state_store<D>(st, state_out + bh * p.M * 2 * D * 2,
                       n < L ? reinterpret_cast<const float2*>(tab + h * kTabBytes + kTabPwBack) : nullptr);
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
    if (!(p.bf16 && p.M == MM && (p.d == 64 || p.d == 128) && p.W >= 1 && p.W <= kMaxW)) return false;
    // the kernels address one (b, h) sequence with 32-bit byte offsets
    return p.N * p.H * p.d * 2 < (int64_t{1} << 31);
}

static size_t tables_bytes(const Problem& p) { return static_cast<size_t>(p.H) * kTabBytes; }

size_t chunked_workspace_bytes(const Problem& p) {
    return chunked_ws_workspace_bytes(p);
    int S;
    int64_t Lseg;
    plan_segments(p, S, Lseg);
    return tables_bytes(p) + static_cast<size_t>(S - 1) * p.B * p.H * p.M * 2 * p.d * 2 * sizeof(float);
}

hipError_t launch_forward_chunked(const Problem& p, const idattn_params& prm, const void* q, const void* k,
                                  const void* v, void* o, const float* state_in, const void* tail_in,
                                  float* state_out, void* workspace, hipStream_t stream) {
    return launch_forward_chunked_ws(p, prm, q, k, v, o, state_in, tail_in, state_out, workspace, stream);
    int S;
    int64_t Lseg;
    plan_segments(p, S, Lseg);
    const auto* q16 = static_cast<const uint16_t*>(q);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const auto* t16 = static_cast<const uint16_t*>(tail_in);
    uint8_t* tab = static_cast<uint8_t*>(workspace);
    float* ws = reinterpret_cast<float*>(tab + tables_bytes(p));
    const int64_t pairs = p.B * p.H;
    const int64_t last_len = p.N - (S - 1) * Lseg;
    const int back = static_cast<int>((L - last_len % L) % L);
    zoh_tables_kernel<<<dim3(static_cast<unsigned>(p.H)), NTH, 0, stream>>>(p, prm, Lseg, back, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (S > 1) {
        const dim3 g1(static_cast<unsigned>(pairs * (S - 1)));
        if (p.d == 128)
            segment_state_kernel<128><<<g1, NTH, 0, stream>>>(p, prm, k16, v16, t16, tab, ws, Lseg, S);
        else
            segment_state_kernel<64><<<g1, NTH, 0, stream>>>(p, prm, k16, v16, t16, tab, ws, Lseg, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t total = pairs * p.M * 2 * p.d;
        segment_carry_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(
            p, state_in, tab, ws, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 g3(static_cast<unsigned>(pairs * S));
    if (p.d == 128)
        chunked_forward_kernel<128><<<g3, NTH, 0, stream>>>(p, prm, q16, k16, v16, static_cast<uint16_t*>(o),
                                                            state_in, t16, state_out, tab, ws, Lseg, S);
    else
        chunked_forward_kernel<64><<<g3, NTH, 0, stream>>>(p, prm, q16, k16, v16, static_cast<uint16_t*>(o),
                                                           state_in, t16, state_out, tab, ws, Lseg, S);
    return hipGetLastError();
}

}  // namespace idattn

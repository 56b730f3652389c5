// Chunked parallel-in-time forward of the Interdomain Attention mixer with
// wave-specialised workgroups: bf16 I/O, fp16 MFMA operands, fp32
// accumulation and fp32 state, R = d = D in {64, 128}, M = 64 modes.
//
// Chunk algebra (chunks of L = 64 tokens; t, j, l positions in the chunk,
// U_prev / Gamma_prev the states before it, T_m[k] = bbar_m abar_m^k,
// F[j] = T[L-1-j]):
//   s_m(t) = sigma_t [ sum_{j<=t} G[t][j] T_m[t-j] + abar_m^{t+1} (y_q(t) . U_prev,m) ],
//            G = Y_q Z_k^T
//   o(t)   = sum_{l<=t} P[t][l] z_v(l) + Re sum_m s_m(t) abar_m^{t+1} Gamma_prev,m,
//            P[t][l] = Re sum_m s_m(t) T_m[t-l]
//   U      <- abar^L U + Z_k^T F,   Gamma <- abar^L Gamma + F^T Z_v
// The Toeplitz sums become plain products through skewed layouts: the
// stored G'[t][L-1-k] = G[t][t-k] turns the first sum into G' T, and
// P'[t][k] = Re sum_m s_m(t) T_m[k] is un-skewed into P[t][l] = P'[t][t-l].
//
// Scalings that keep fp16 operands in range and save arithmetic:
//  * the conv weights carry a factor -log2(e), so the conv output c' gives
//    SiLU through y' = c' / (1 + 2^c') = -y / ln 2 with no extra multiply;
//  * y' is stored unscaled and the per-token factor
//    sigma~_t = -ln2 / (Delta (ln^2 2 ||y'||^2 + eps)) is applied to s, so
//    that the s~ = s / Delta kept in shared memory, P~ = P / Delta and
//    X = s~ abar^{t+1} = s abar^{t+1} / Delta are all O(1);  o = Delta (P~ Z_v + X Gamma).
//  * T enters every chunk of every sequence, so its fp16 rounding error would
//    add up coherently; it is carried as a pair of fp16 values (about 22
//    bits) and every product with T is two MFMAs.
//
// A workgroup is eight waves, two per SIMD.  Waves 0-3 (one per SIMD) own the
// state and run every MFMA phase of chunk c; waves 4-7 build the features of
// chunk c+1 meanwhile (short conv, SiLU, norms), keep them in registers and
// write them to shared memory once the MFMA waves no longer read the previous
// chunk's tiles.  Each SIMD thus runs one MFMA-bound and one VALU-bound wave.
// All eight waves meet at the same four barriers per chunk:
//   G   (MFMA: G tiles -> G')                       | features: -
//   S   (MFMA: y_q.U, G'T, s~, X; U update; Z_v frag)| features: keys of c+1
//   P   (MFMA: P~ tiles)                             | features: write z_k; values of c+1
//   O   (MFMA: output; Gamma update)                 | features: queries of c+1
//
// Index m' = 2 m + part (part 0 = real, 1 = imaginary) runs over the 2M = 128
// real rows of a complex mode set.  MFMA wave w (0..3) keeps
//   U     : rows r (all D), columns m' in [32w, 32w+32)       -> 2 x D/16 tiles
//   Gamma : rows m' (all 128), columns c in [w D/4, (w+1) D/4) -> 8 x D/64 tiles
// An accumulator tile [X][Y] doubles as an operand with K = X once two of
// them are concatenated (lane (g, i) then supplies K rows 4g..4g+3 and
// 16+4g..16+4g+3 of a 32-row block), so U feeds y_q . U and Gamma feeds the
// readout straight from registers.  z_k and z_v are stored transposed
// ([channel][token]) so that both state updates read them as plain fragments.
#include "common.h"
#include "launch.h"

namespace idattn {
namespace cws {
namespace {

constexpr int L = 64;        // chunk length
constexpr int MM = 64;       // complex modes
constexpr int M2 = 2 * MM;   // m' rows
constexpr int NTH = 512;     // eight waves
constexpr int kMaxW = 4;     // conv widths 1..4
constexpr int RS = M2 + 8;   // padded row length (halfs) of [t][m'] tiles
constexpr int RP = L + 8;    // padded row length of [t][64] tiles
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLn2Sq = 0.4804530139182014f;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Cfg {
    static constexpr int RT = D / 16;   // 16-row tiles over R
    static constexpr int KB = D / 32;   // 32-wide K steps over R
    static constexpr int CW = D / 64;   // 16-column Gamma tiles per MFMA wave
    static constexpr int CPT = D / 32;  // feature channels per thread
    static constexpr int RY = D + 8;    // padded row length of the y' tile
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef short s4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(const half8& a, const half8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ tile layouts
// [rows][64] fp16 tiles keep 128-byte rows with the 16-byte chunk index of
// (row, col) XOR-ed with a function of row % 16, which makes the fragment and
// transposing reads below touch every bank once; [t][*] tiles read as 8-byte
// halves use padded rows instead.
__host__ __device__ constexpr int sw128(int r) { return 2 * (((r >> 1) & 3) ^ (2 * ((r >> 3) & 1))) + ((r >> 3) & 1); }
__host__ __device__ constexpr int o128(int r, int col) { return r * 64 + ((((col >> 3) ^ sw128(r)) & 7) << 3) + (col & 7); }

__device__ __forceinline__ half8 cat(const half4& a, const half4& b) {
    half8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// 32-bit LDS byte addresses.  A per-lane base computed once and passed
// through an empty asm statement stays in one VGPR, and the constant part of
// each access goes into the instruction's 16-bit offset field; the arrays are
// ordered so that every such family of accesses spans less than 64 KiB.
typedef __attribute__((address_space(3))) half8 lds_h8;
typedef __attribute__((address_space(3))) half4 lds_h4;
typedef __attribute__((address_space(3))) half2v lds_h2;
typedef __attribute__((address_space(3))) s4v lds_s4;
typedef __attribute__((address_space(3))) _Float16 lds_h1;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ half8 rd8(uint32_t a) { return *(lds_h8*)(uintptr_t)a; }
__device__ __forceinline__ half4 rd4(uint32_t a) { return *(lds_h4*)(uintptr_t)a; }
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i & 3) of the 4-element read of lane 4j + (i >> 2), for j = 0..3.
__device__ __forceinline__ half4 rd4t(uint32_t a) {
    return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(uintptr_t)a));
}
__device__ __forceinline__ void wr8(uint32_t a, const half8& v) { *(lds_h8*)(uintptr_t)a = v; }
__device__ __forceinline__ void wr4(uint32_t a, float x0, float x1, float x2, float x3) {
    *(lds_h4*)(uintptr_t)a = half4{static_cast<_Float16>(x0), static_cast<_Float16>(x1), static_cast<_Float16>(x2),
                                   static_cast<_Float16>(x3)};
}
__device__ __forceinline__ void wr2(uint32_t a, float x0, float x1) {
    *(lds_h2*)(uintptr_t)a = half2v{static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
}
__device__ __forceinline__ void wr1(uint32_t a, float x) { *(lds_h1*)(uintptr_t)a = static_cast<_Float16>(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sums over the 32 lanes of a half-wave for N values at once; every lane gets the totals.
template <int N>
__device__ __forceinline__ void sum32(float (&x)[N]) {
#pragma unroll
    for (int s = 0; s < N; ++s) x[s] += dpp_mov<0xB1>(x[s]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int s = 0; s < N; ++s) x[s] += dpp_mov<0x4E>(x[s]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int s = 0; s < N; ++s) x[s] += dpp_mov<0x141>(x[s]);  // row_half_mirror
#pragma unroll
    for (int s = 0; s < N; ++s) x[s] += dpp_mov<0x140>(x[s]);  // row_mirror
#pragma unroll
    for (int s = 0; s < N; ++s) x[s] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[s]), 0x401F));
}

// Keeps the compiler from hoisting the next step's operand loads above this
// point: one K-step of fragments is live at a time.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

__device__ __forceinline__ half8 to_half8(const f4& a, const f4& b) {
    half8 r;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        r[jj] = static_cast<_Float16>(a[jj]);
        r[4 + jj] = static_cast<_Float16>(b[jj]);
    }
    return r;
}

// ------------------------------------------------------------------ tables
// Per-head tables, one launch per forward (fp64 arithmetic):
//   ft, ftl [M2][L] fp16, swizzled rows: F^T[m'][j] = T_{m'}[L-1-j] = ft + ftl
//   pw [L][MM] float2: abar^{k+1}
//   pwseg[MM], pwback[MM] float2: abar^{Lseg}, abar^{-back};  hc: Delta, 1/Delta
// with T_{m'}[k] the real (m' even) or imaginary (m' odd) part of bbar_m abar_m^k.
constexpr int kTabFT = 0;
constexpr int kTabFTL = kTabFT + M2 * L * 2;
constexpr int kTabPw = kTabFTL + M2 * L * 2;
constexpr int kTabPwSeg = kTabPw + L * MM * 8;
constexpr int kTabPwBack = kTabPwSeg + MM * 8;
constexpr int kTabHc = kTabPwBack + MM * 8;
constexpr int kTabBytes = ((kTabHc + 16 + 255) / 256) * 256;

// Complex fp64 power abar^n = exp(n Delta lambda).
__device__ __forceinline__ void cpow(double dt, float lre, float lim, double n, double& pr, double& pi) {
    double sy, cy;
    sincos(n * dt * lim, &sy, &cy);
    const double e = exp(n * dt * lre);
    pr = e * cy;
    pi = e * sy;
}

// grid (H, 16), 256 threads: one (k, m) per thread.
__global__ __launch_bounds__(256) void zoh_tables_kernel(Problem p, idattn_params prm, int64_t Lseg, int back,
                                                         uint8_t* __restrict__ tab) {
    const int64_t h = blockIdx.x;
    uint8_t* th = tab + h * kTabBytes;
    const int m = threadIdx.x & (MM - 1);
    const int k = 4 * static_cast<int>(blockIdx.y) + (threadIdx.x >> 6);
    const float log_dt = prm.log_dt[h];
    const float lre = prm.A[(h * MM + m) * 2], lim = prm.A[(h * MM + m) * 2 + 1];
    const Zoh z = zoh_mode(log_dt, lre, lim, prm.Bc[(h * MM + m) * 2], prm.Bc[(h * MM + m) * 2 + 1]);
    const double dt = exp(static_cast<double>(log_dt));
    double pr, pi;
    cpow(dt, lre, lim, static_cast<double>(k), pr, pi);  // abar^k
    const double tv[2] = {z.br * pr - z.bi * pi, z.br * pi + z.bi * pr};
    _Float16* ft = reinterpret_cast<_Float16*>(th + kTabFT);
    _Float16* ftl = reinterpret_cast<_Float16*>(th + kTabFTL);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        const _Float16 hi = static_cast<_Float16>(static_cast<float>(tv[part]));
        ft[o128(2 * m + part, L - 1 - k)] = hi;
        ftl[o128(2 * m + part, L - 1 - k)] = static_cast<_Float16>(static_cast<float>(tv[part] - static_cast<double>(hi)));
    }
    cpow(dt, lre, lim, static_cast<double>(k + 1), pr, pi);
    reinterpret_cast<float2*>(th + kTabPw)[k * MM + m] = make_float2(static_cast<float>(pr), static_cast<float>(pi));
    if (blockIdx.y == 0 && threadIdx.x < MM) {
        cpow(dt, lre, lim, static_cast<double>(Lseg), pr, pi);
        reinterpret_cast<float2*>(th + kTabPwSeg)[m] = make_float2(static_cast<float>(pr), static_cast<float>(pi));
        cpow(dt, lre, lim, -static_cast<double>(back), pr, pi);
        reinterpret_cast<float2*>(th + kTabPwBack)[m] = make_float2(static_cast<float>(pr), static_cast<float>(pi));
        if (threadIdx.x == 0)
            reinterpret_cast<float2*>(th + kTabHc)[0] = make_float2(static_cast<float>(dt), static_cast<float>(1.0 / dt));
    }
}

// ------------------------------------------------------------------ shared memory
template <int D>
struct SmemFwd {
    // window A: [t][*] tiles
    _Float16 yq[L * Cfg<D>::RY];  // y' of the queries [t][r]
    _Float16 sc[L * RS];          // [t][m'] (Re s~, -Im s~)
    _Float16 xc[L * RS];          // [t][m'] (Re X, -Im X)
    // window B: swizzled [rows][64] tiles
    _Float16 zkT[D * L];          // z_k^T [r][j]
    _Float16 zvT[D * L];          // z_v^T [c][l]
    _Float16 ft[M2 * L];          // F^T, high and low fp16 parts
    _Float16 ftl[M2 * L];
    // window C
    _Float16 gp[L * RP];          // G' (zero above the causal band, never rewritten there)
    _Float16 pp[L * RP];          // P~ [t][l] (likewise)
    float sig[L];                 // sigma~_t
    float2 aL[MM];                // abar^L
    float2 pw[17][MM];            // abar^{k+1}, k = 0..16
    float gain[2 * D], bias[2 * D];
    float wq[D * kMaxW], wk[D * kMaxW];  // conv weights times -log2(e), right-aligned taps
    uint16_t halo[2][3][D];              // raw q, k at positions -3..-1 of the sequence
};

template <int D>
struct SmemSeg {
    _Float16 zkT[D * L];
    _Float16 zvT[D * L];
    _Float16 ft[M2 * L];
    _Float16 ftl[M2 * L];
    float2 aL[MM];
    float gain[2 * D], bias[2 * D];
    float wk[D * kMaxW];
    uint16_t halo[2][3][D];
};

// byte distances inside window B (identical in both layouts)
template <int D>
struct WinOff {
    static constexpr uint32_t zv = D * L * 2, ft = 2 * D * L * 2, ftl = 2 * D * L * 2 + M2 * L * 2;
};

// ------------------------------------------------------------------ feature waves
// Thread f = tid - 256 (cgi = f % 32, tb = f / 32) owns channels CPT cgi .. +CPT-1
// of tokens 8tb..8tb+7 of a chunk; the short conv needs the three tokens
// before, which the thread loads itself (positions < 0 read zeros, replaced
// by the stored tail for the first chunk of a sequence).
template <int D>
struct FmT;
template <>
struct FmT<128> {
    typedef u2 T;
};
template <>
struct FmT<64> {
    typedef uint32_t T;
};

// Buffer resources over one (b, h) sequence up to the end of the segment:
// token t, channel c sits at byte 2 (t H D + c) from the sequence's first
// token.  Offsets are whole VGPR operands, which the hardware range-checks;
// loads past the end of a resource return zeros.
struct SeqBuf {
    __amdgpu_buffer_rsrc_t q, k, v;
};
template <int D>
__device__ __forceinline__ SeqBuf seq_buf(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t b,
                                          int64_t h, int64_t N, int64_t H, int64_t t_end) {
    const int64_t first = b * N * H * D + h * D;
    const int nrec = static_cast<int>(t_end * H * D * 2);
    SeqBuf r;
    r.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>((q ? q : k) + first), 0, nrec, 0x00020000);
    r.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + first), 0, nrec, 0x00020000);
    r.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v + first), 0, nrec, 0x00020000);
    return r;
}
template <int D>
__device__ __forceinline__ typename FmT<D>::T bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (D == 128) return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

template <int D>
__device__ __forceinline__ void unpack(const typename FmT<D>::T& u, float* x) {
    if constexpr (D == 128) {
        x[0] = __uint_as_float(u[0] << 16);
        x[1] = __uint_as_float(u[0] & 0xffff0000u);
        x[2] = __uint_as_float(u[1] << 16);
        x[3] = __uint_as_float(u[1] & 0xffff0000u);
    } else {
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xffff0000u);
    }
}

// Raw inputs of one chunk for one thread: 8 tokens and the 3 before (q, k).
template <int D, bool WITH_Q>
struct FmRaw {
    typedef typename FmT<D>::T T;
    T q[WITH_Q ? 11 : 1];
    T k[11];
    T v[8];
};

// tok0 = first token of the chunk; lane_b = 2 (8 tb H D + CPT cgi) bytes, rsb = 2 H D.
template <int D, bool WITH_Q>
__device__ __forceinline__ void load_qk(FmRaw<D, WITH_Q>& r, const SeqBuf& sb, int64_t tok0, int rsb, int lane_b,
                                        bool want_q) {
#pragma unroll
    for (int s = 0; s < 11; ++s) {
        const uint32_t off = static_cast<uint32_t>(lane_b + (tok0 - 3 + s) * rsb);
        if constexpr (WITH_Q)
            if (want_q) r.q[s] = bload<D>(sb.q, off);
        if (!want_q) r.k[s] = bload<D>(sb.k, off);
    }
}
template <int D, bool WITH_Q>
__device__ __forceinline__ void load_v(FmRaw<D, WITH_Q>& r, const SeqBuf& sb, int64_t tok0, int rsb, int lane_b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) r.v[s] = bload<D>(sb.v, static_cast<uint32_t>(lane_b + (tok0 + s) * rsb));
}

// The stored tail replaces the three positions before the sequence start.
template <int D, class SM, class T>
__device__ __forceinline__ void halo_fix(T (&x)[11], const SM& sm, int sel, int64_t tok0) {
    const int cgi = (threadIdx.x - 256) & 31;
    if (tok0 == 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j) x[j] = *reinterpret_cast<const T*>(&sm.halo[sel][j][Cfg<D>::CPT * cgi]);
    }
}

// y' = c' / (1 + 2^c') for 8 tokens x CPT channels; ss = partial ||y'||^2.
template <int D>
__device__ __forceinline__ void conv_silu(const typename FmT<D>::T (&raw)[11], const float* wl, float (&y)[8][Cfg<D>::CPT],
                                          float (&ss)[8]) {
    constexpr int CPT = Cfg<D>::CPT;
    float x[11][CPT];
#pragma unroll
    for (int s = 0; s < 11; ++s) unpack<D>(raw[s], x[s]);
    float w[CPT][kMaxW];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int j = 0; j < kMaxW; ++j) w[c][j] = wl[c * kMaxW + j];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        ss[s] = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            float acc = w[c][0] * x[s][c];
#pragma unroll
            for (int j = 1; j < kMaxW; ++j) acc = fmaf(w[c][j], x[s + j][c], acc);
            y[s][c] = acc * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(acc));
            ss[s] = fmaf(y[s][c], y[s][c], ss[s]);
        }
    }
}

// z_k of the thread's 8 tokens, packed per channel (z masked to 0 at t >= n).
template <int D, bool WITH_Q, class SM>
__device__ __forceinline__ void fm_keys(half8 (&zk)[Cfg<D>::CPT], FmRaw<D, WITH_Q>& r, const SM& sm, int64_t tok0,
                                        int n, float eps_feat, float eps_norm) {
    constexpr int CPT = Cfg<D>::CPT;
    const int f = threadIdx.x - 256, cgi = f & 31, tb = f >> 5, c0 = CPT * cgi;
    if (tb == 0) halo_fix<D>(r.k, sm, 1, tok0);
    float y[8][CPT], ss[8];
    conv_silu<D>(r.k, &sm.wk[c0 * kMaxW], y, ss);
    sum32<8>(ss);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        // xi = -ln2 inv y',  mean xi^2 = ln^2 2 inv^2 ||y'||^2 / D
        const float inv = __builtin_amdgcn_rcpf(fmaf(kLn2Sq, ss[s], eps_feat));
        const float rs = __builtin_amdgcn_rsqf(fmaf(kLn2Sq * (1.f / D) * inv * inv, ss[s], eps_norm));
        ss[s] = (8 * tb + s < n) ? -kLn2 * inv * rs : 0.f;  // rho, 0 past the valid tokens
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const float g = sm.gain[c0 + c], bb = sm.bias[c0 + c];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            zk[c][s] = static_cast<_Float16>(8 * tb + s < n ? fmaf(g * ss[s], y[s][c], bb) : 0.f);
    }
}

// z_v of the thread's 8 tokens, written to z_v^T at column 8tb.
template <int D>
struct FmAddr;
template <int D, bool WITH_Q, class SM>
__device__ __forceinline__ void fm_values(const FmRaw<D, WITH_Q>& r, const SM& sm, const FmAddr<D>& fa, int n,
                                          float eps_norm) {
    constexpr int CPT = Cfg<D>::CPT;
    const int f = threadIdx.x - 256, cgi = f & 31, tb = f >> 5, c0 = CPT * cgi;
    float xv[8][CPT], ss[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        unpack<D>(r.v[s], xv[s]);
        ss[s] = xv[s][0] * xv[s][0];
#pragma unroll
        for (int c = 1; c < CPT; ++c) ss[s] = fmaf(xv[s][c], xv[s][c], ss[s]);
    }
    sum32<8>(ss);
#pragma unroll
    for (int s = 0; s < 8; ++s) ss[s] = __builtin_amdgcn_rsqf(fmaf(1.f / D, ss[s], eps_norm));
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const float g = sm.gain[D + c0 + c], bb = sm.bias[D + c0 + c];
        half8 z;
#pragma unroll
        for (int s = 0; s < 8; ++s) z[s] = static_cast<_Float16>(8 * tb + s < n ? fmaf(g * ss[s], xv[s][c], bb) : 0.f);
        wr8(fa.z[c] + WinOff<D>::zv, z);
    }
}

// y' of the thread's 8 tokens into rows 8tb.. of yq, and sigma~.
template <int D, class SM>
__device__ __forceinline__ void fm_queries(FmRaw<D, true>& r, SM& sm, uint32_t yst, int64_t tok0, float eps_feat,
                                           float inv_dt) {
    constexpr int CPT = Cfg<D>::CPT;
    const int f = threadIdx.x - 256, cgi = f & 31, tb = f >> 5, c0 = CPT * cgi;
    if (tb == 0) halo_fix<D>(r.q, sm, 0, tok0);
    float y[8][CPT], ss[8];
    conv_silu<D>(r.q, &sm.wq[c0 * kMaxW], y, ss);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if constexpr (CPT == 4) wr4(yst + 2 * s * Cfg<D>::RY, y[s][0], y[s][1], y[s][2], y[s][3]);
        else wr2(yst + 2 * s * Cfg<D>::RY, y[s][0], y[s][1]);
    }
    sum32<8>(ss);
    if (cgi == 0) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
            sm.sig[8 * tb + s] = -kLn2 * inv_dt * __builtin_amdgcn_rcpf(fmaf(kLn2Sq, ss[s], eps_feat));
    }
}

// Per-thread store addresses of the feature waves: z_k^T row CPT cgi + c at
// column 8tb (each row has its own swizzle; z_v^T at + WinOff::zv), and y'
// row 8tb at column CPT cgi.
template <int D>
struct FmAddr {
    uint32_t z[Cfg<D>::CPT];
    uint32_t y;
};
template <int D>
__device__ __forceinline__ FmAddr<D> fm_addr(const void* zkT, const void* yq) {
    constexpr int CPT = Cfg<D>::CPT;
    const int f = threadIdx.x - 256, cgi = f & 31, tb = f >> 5;
    FmAddr<D> a;
#pragma unroll
    for (int c = 0; c < CPT; ++c) a.z[c] = opaque(lds_addr(zkT) + 2 * o128(CPT * cgi + c, 8 * tb));
    a.y = yq ? opaque(lds_addr(yq) + 2 * (8 * tb * Cfg<D>::RY + CPT * cgi)) : 0u;
    return a;
}

// Conv weights (times -log2 e, taps right-aligned into 4 slots), gain, bias,
// and the stored tail of the sequence (positions -3..-1; zeros when absent).
template <int D, bool WITH_Q, class SM>
__device__ __forceinline__ void load_prologue(SM& sm, const idattn_params& prm, const uint16_t* tail_in, int64_t b,
                                              int64_t h, int64_t H, int W) {
    for (int e = threadIdx.x; e < 2 * D; e += NTH) {
        sm.gain[e] = prm.gain[h * 2 * D + e];
        sm.bias[e] = prm.bias[h * 2 * D + e];
    }
    for (int e = threadIdx.x; e < D * kMaxW; e += NTH) {
        const int c = e / kMaxW, j = e % kMaxW;
        const int tap = j - (kMaxW - W);
        if constexpr (WITH_Q) sm.wq[e] = tap >= 0 ? -kLog2e * prm.conv_q[(h * D + c) * W + tap] : 0.f;
        sm.wk[e] = tap >= 0 ? -kLog2e * prm.conv_k[(h * D + c) * W + tap] : 0.f;
    }
    for (int e = threadIdx.x; e < 2 * 3 * D; e += NTH) {
        const int sel = e / (3 * D), row = (e / D) % 3, c = e % D;
        const int pos = row - 3;
        uint16_t val = 0;
        if (tail_in != nullptr && pos >= -(W - 1)) {
            const int64_t slot = (W - 1) + pos;
            val = tail_in[(((b * H + h) * 2 + sel) * (W - 1) + slot) * D + c];
        }
        sm.halo[sel][row][c] = val;
    }
}

__device__ __forceinline__ void copy16(void* dst, const void* src, int bytes) {
    for (int e = threadIdx.x; e < bytes / 16; e += NTH)
        reinterpret_cast<u4*>(dst)[e] = reinterpret_cast<const u4*>(src)[e];
}

// ------------------------------------------------------------------ MFMA-wave state
// Lane (g, i) of MFMA wave w:
//   U[mu][rt][jj]  = U_m[r],     r = 16rt + 4g + jj,  m' = 32w + 16mu + i
//   Gm[mt][ct][jj] = Gamma_m[c], m' = 16mt + 4g + jj, c = 16(CW w + ct) + i
// Memory layout: float [M][2D][2] (complex), columns 0..D-1 hold U, D..2D-1 Gamma.
template <int D>
struct State {
    f4 U[2][Cfg<D>::RT];
    f4 Gm[8][Cfg<D>::CW];
};

template <int D>
__device__ __forceinline__ void state_load(State<D>& st, const float* src) {
    constexpr int RT = Cfg<D>::RT, CW = Cfg<D>::CW;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int mu = 0; mu < 2; ++mu)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rt + 4 * g + jj, mp = 32 * w + 16 * mu + i;
                st.U[mu][rt][jj] = src ? src[((mp >> 1) * 2 * D + r) * 2 + (mp & 1)] : 0.f;
            }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int ct = 0; ct < CW; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int mp = 16 * mt + 4 * g + jj, c = 16 * (CW * w + ct) + i;
                st.Gm[mt][ct][jj] = src ? src[((mp >> 1) * 2 * D + D + c) * 2 + (mp & 1)] : 0.f;
            }
}

// Stores the state, first multiplying every mode by corr[m] when corr is not NULL.
template <int D>
__device__ __forceinline__ void state_store(const State<D>& st, float* dst, const float2* corr) {
    constexpr int RT = Cfg<D>::RT, CW = Cfg<D>::CW;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int mu = 0; mu < 2; ++mu) {
        const int mp = 32 * w + 16 * mu + i;
        const float2 c = corr ? corr[mp >> 1] : make_float2(1.f, 0.f);
        const float sc = (mp & 1) ? c.y : -c.y;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rt + 4 * g + jj;
                const float u = st.U[mu][rt][jj];
                const float pu = dpp_mov<0xB1>(u);  // other part of the same mode (lane i ^ 1)
                dst[((mp >> 1) * 2 * D + r) * 2 + (mp & 1)] = fmaf(sc, pu, c.x * u);
            }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int ct = 0; ct < CW; ++ct)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int m = 8 * mt + 2 * g + q, c = 16 * (CW * w + ct) + i;
                const float2 a = corr ? corr[m] : make_float2(1.f, 0.f);
                const float gr = st.Gm[mt][ct][2 * q], gi = st.Gm[mt][ct][2 * q + 1];
                *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + D + c) * 2) =
                    make_float2(a.x * gr - a.y * gi, a.x * gi + a.y * gr);
            }
}

// Window-B lane base (byte address from z_k^T) for fragment reads of rows
// R0 + i at column chunk 4kb + g, R0 = 16 x any tile index of any of the four
// tiles; the wave-uniform offsets of the F^T rows of U's m' block and of the
// z_v^T rows of the wave's Gamma columns are added at use.
template <int D>
struct WinB {
    uint32_t all[2];
    __device__ __forceinline__ uint32_t ownU(int mu, int kb) const {
        return all[kb] + WinOff<D>::ft + 2 * 64 * (32 * (threadIdx.x >> 6) + 16 * mu);
    }
    __device__ __forceinline__ uint32_t ownC(int kb) const {
        return all[kb] + WinOff<D>::zv + 2 * 64 * 16 * Cfg<D>::CW * (threadIdx.x >> 6);
    }
};
template <int D>
__device__ __forceinline__ WinB<D> win_b(const void* zkT) {
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
    WinB<D> b;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) b.all[kb] = opaque(lds_addr(zkT) + 2 * o128(i, 32 * kb + 8 * g));
    return b;
}

// U <- abar^L U + Z_k^T F  (the real and imaginary rows of a mode sit in lanes i, i ^ 1)
template <int D>
__device__ __forceinline__ void key_update(State<D>& st, const WinB<D>& wb, const float (&aLr)[2],
                                           const float (&aLs)[2]) {
    constexpr int RT = Cfg<D>::RT;
    constexpr uint32_t dl = WinOff<D>::ftl - WinOff<D>::ft;
#pragma unroll
    for (int mu = 0; mu < 2; ++mu)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float u = st.U[mu][rt][jj];
                st.U[mu][rt][jj] = fmaf(aLs[mu], dpp_mov<0xB1>(u), aLr[mu] * u);
            }
            if (rt % 2 == 1) step_fence();  // bounds the partner values held at once
        }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        half8 bF[2], bFl[2];
#pragma unroll
        for (int mu = 0; mu < 2; ++mu) {
            bF[mu] = rd8(wb.ownU(mu, kb));  // F[j][m'], j = 32kb + 8g + jj
            bFl[mu] = rd8(wb.ownU(mu, kb) + dl);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const half8 a = rd8(wb.all[kb] + 2048 * rt);  // z_k[j][r = 16rt + i]
#pragma unroll
            for (int mu = 0; mu < 2; ++mu) {
                st.U[mu][rt] = mfma(a, bF[mu], st.U[mu][rt]);
                st.U[mu][rt] = mfma(a, bFl[mu], st.U[mu][rt]);
            }
            if (rt % 4 == 3) step_fence();
        }
    }
}

// Gamma <- abar^L Gamma + F^T Z_v, with bZ[ct][kb] = Z_v[32kb + 8g + jj][16(CW w + ct) + i]
template <int D>
__device__ __forceinline__ void value_update(State<D>& st, const float2* aL, const WinB<D>& wb,
                                             const half8 (&bZ)[Cfg<D>::CW][2]) {
    constexpr int CW = Cfg<D>::CW;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const float4 a = *reinterpret_cast<const float4*>(&aL[8 * mt + 2 * g]);
#pragma unroll
        for (int ct = 0; ct < CW; ++ct) {
            const float r0 = st.Gm[mt][ct][0], i0 = st.Gm[mt][ct][1], r1 = st.Gm[mt][ct][2], i1 = st.Gm[mt][ct][3];
            st.Gm[mt][ct][0] = a.x * r0 - a.y * i0;
            st.Gm[mt][ct][1] = a.x * i0 + a.y * r0;
            st.Gm[mt][ct][2] = a.z * r1 - a.w * i1;
            st.Gm[mt][ct][3] = a.z * i1 + a.w * r1;
        }
        if (mt % 2 == 1) step_fence();
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const half8 a = rd8(wb.all[kb] + WinOff<D>::ft + 2048 * mt);
            const half8 al = rd8(wb.all[kb] + WinOff<D>::ftl + 2048 * mt);
#pragma unroll
            for (int ct = 0; ct < CW; ++ct) {
                st.Gm[mt][ct] = mfma(a, bZ[ct][kb], st.Gm[mt][ct]);
                st.Gm[mt][ct] = mfma(al, bZ[ct][kb], st.Gm[mt][ct]);
            }
            if (mt % 4 == 3) step_fence();
        }
}

template <int D>
__device__ __forceinline__ void load_bz(half8 (&bZ)[Cfg<D>::CW][2], const WinB<D>& wb) {
#pragma unroll
    for (int ct = 0; ct < Cfg<D>::CW; ++ct)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) bZ[ct][kb] = rd8(wb.ownC(kb) + 2048 * ct);
}

// Causal 16 x 16 tiles (tt, kt), kt <= tt, of the G and P~ products, split
// over the four MFMA waves: wave w takes tiles w, w + 4, w + 8 of the list.
__device__ __forceinline__ int tile_tt(int q) { return q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3; }
__device__ __forceinline__ int tile_kt(int q) { return q - (tile_tt(q) * (tile_tt(q) + 1)) / 2; }

// ------------------------------------------------------------------ kernels
// Segment end states from a zero start: grid B*H*(S-1), block (bh, seg).
template <int D>
__global__ __launch_bounds__(NTH) void segment_state_kernel(Problem p, idattn_params prm,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ tail_in,
                                                            const uint8_t* __restrict__ tab, float* __restrict__ ws,
                                                            int64_t Lseg, int S) {
    constexpr int CPT = Cfg<D>::CPT, CW = Cfg<D>::CW;
    __shared__ SmemSeg<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15;
    const bool mw = w < 4;  // MFMA wave
    const int64_t bh = blockIdx.x / (S - 1);
    const int seg = static_cast<int>(blockIdx.x % (S - 1));
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t t_begin = seg * Lseg, t_end = t_begin + Lseg;  // segments 0..S-2 are full
    const int nch = static_cast<int>(Lseg / L);
    const uint8_t* th = tab + h * kTabBytes;
    load_prologue<D, false>(sm, prm, tail_in, b, h, p.H, static_cast<int>(p.W));
    copy16(sm.ft, th + kTabFT, M2 * L * 2);
    copy16(sm.ftl, th + kTabFTL, M2 * L * 2);
    if (tid < MM) sm.aL[tid] = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + tid];
    __syncthreads();
    if (mw) {
        State<D> st;
        state_load<D>(st, nullptr);
        lds_barrier();  // features of chunk 0 are in shared memory
        for (int c = 0; c < nch; ++c) {
            const WinB<D> wb = win_b<D>(sm.zkT);
            float aLr[2], aLs[2];
#pragma unroll
            for (int mu = 0; mu < 2; ++mu) {
                const float2 a = sm.aL[(32 * w + 16 * mu + i) >> 1];
                aLr[mu] = a.x;
                aLs[mu] = (i & 1) ? a.y : -a.y;
            }
            half8 bZ[CW][2];
            key_update<D>(st, wb, aLr, aLs);
            load_bz<D>(bZ, wb);
            lds_barrier();
            value_update<D>(st, sm.aL, wb, bZ);
            lds_barrier();
        }
        state_store<D>(st, ws + (static_cast<int64_t>(seg) * p.B * p.H + bh) * MM * 2 * D * 2, nullptr);
    } else {
        FmRaw<D, false> rr;
        const int rsb = static_cast<int>(p.H * D * 2);
        const int f = tid - 256;
        const int lane_b = 2 * (8 * (f >> 5) * static_cast<int>(p.H * D) + CPT * (f & 31));
        const SeqBuf sq = seq_buf<D>(nullptr, k, v, b, h, p.N, p.H, t_end);
        const FmAddr<D> fa = fm_addr<D>(sm.zkT, nullptr);
        load_qk<D, false>(rr, sq, t_begin, rsb, lane_b, false);
        load_v<D, false>(rr, sq, t_begin, rsb, lane_b);
        {
            half8 zk[CPT];
            fm_keys<D, false>(zk, rr, sm, t_begin, L, p.eps_feat, p.eps_norm);
#pragma unroll
            for (int c = 0; c < CPT; ++c) wr8(fa.z[c], zk[c]);
            fm_values<D, false>(rr, sm, fa, L, p.eps_norm);
            if (nch > 1) {
                load_qk<D, false>(rr, sq, t_begin + L, rsb, lane_b, false);
                load_v<D, false>(rr, sq, t_begin + L, rsb, lane_b);
            }
        }
        lds_barrier();  // features of chunk 0 are in shared memory
        for (int c = 0; c < nch; ++c) {
            const int64_t t0 = t_begin + static_cast<int64_t>(c) * L;
            half8 zk[CPT];
            if (c + 1 < nch) fm_keys<D, false>(zk, rr, sm, t0 + L, L, p.eps_feat, p.eps_norm);
            lds_barrier();
            if (c + 1 < nch) {
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) wr8(fa.z[cc], zk[cc]);
                if (c + 2 < nch) load_qk<D, false>(rr, sq, t0 + 2 * L, rsb, lane_b, false);
                fm_values<D, false>(rr, sm, fa, L, p.eps_norm);
                if (c + 2 < nch) load_v<D, false>(rr, sq, t0 + 2 * L, rsb, lane_b);
            }
            lds_barrier();
        }
    }
}

// Carry chain over segments, one thread per complex state element:
// ws[seg] <- state entering segment seg+1.
__global__ __launch_bounds__(256) void segment_carry_kernel(Problem p, const float* __restrict__ state_in,
                                                            const uint8_t* __restrict__ tab,
                                                            float* __restrict__ ws, int S) {
    const int64_t D2 = 2 * p.d;
    const int64_t total = p.B * p.H * MM * D2;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t m = (e / D2) % MM;
    const int64_t h = (e / (D2 * MM)) % p.H;
    const float2 a = reinterpret_cast<const float2*>(tab + h * kTabBytes + kTabPwSeg)[m];
    float2 c = state_in ? reinterpret_cast<const float2*>(state_in)[e] : make_float2(0.f, 0.f);
    float2* w2 = reinterpret_cast<float2*>(ws);
    for (int seg = 0; seg + 1 < S; ++seg) {
        const float2 loc = w2[seg * total + e];
        c = make_float2(a.x * c.x - a.y * c.y + loc.x, a.x * c.y + a.y * c.x + loc.y);
        w2[seg * total + e] = c;
    }
}

// Full chunk loop of one segment: grid B*H*S, block (bh, seg).
template <int D>
__global__ __launch_bounds__(NTH) void chunked_forward_kernel(Problem p, idattn_params prm,
                                                              const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                              const float* state_in,
                                                              const uint16_t* __restrict__ tail_in, float* state_out,
                                                              const uint8_t* __restrict__ tab,
                                                              const float* __restrict__ carry, int64_t Lseg, int S) {
    constexpr int RT = Cfg<D>::RT, KB = Cfg<D>::KB, CW = Cfg<D>::CW, CPT = Cfg<D>::CPT, RY = Cfg<D>::RY;
    constexpr uint32_t dl = WinOff<D>::ftl - WinOff<D>::ft;
    __shared__ SmemFwd<D> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
    const bool mw = w < 4;  // MFMA wave
    const int64_t bh = blockIdx.x / S;
    const int seg = static_cast<int>(blockIdx.x % S);
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t N = p.N, H = p.H;
    const int64_t t_begin = seg * Lseg;
    const int64_t t_end = t_begin + Lseg < N ? t_begin + Lseg : N;
    const int nch = static_cast<int>((t_end - t_begin + L - 1) / L);
    const int n_last = static_cast<int>(t_end - t_begin - static_cast<int64_t>(nch - 1) * L);
    const uint8_t* th = tab + h * kTabBytes;

    load_prologue<D, true>(sm, prm, tail_in, b, h, H, static_cast<int>(p.W));
    copy16(sm.ft, th + kTabFT, M2 * L * 2);
    copy16(sm.ftl, th + kTabFTL, M2 * L * 2);
    if (tid < MM) sm.aL[tid] = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + tid];
    copy16(sm.pw, th + kTabPw, 16 * MM * 8);
    for (int e = tid; e < L * RP * 2 / 16; e += NTH)
        reinterpret_cast<u4*>(sm.gp)[e] = reinterpret_cast<u4*>(sm.pp)[e] = u4{0u, 0u, 0u, 0u};
    const float2 hc = reinterpret_cast<const float2*>(th + kTabHc)[0];
    const float dt = hc.x, inv_dt = hc.y;

    constexpr uint32_t xc_sc = L * RS * 2;  // xc - sc
    __syncthreads();
    if (mw) {
        // ---------------- MFMA waves: chunk c
        State<D> st;
        state_load<D>(st, seg == 0 ? (state_in ? state_in + bh * MM * 2 * D * 2 : nullptr)
                                   : carry + (static_cast<int64_t>(seg - 1) * p.B * p.H + bh) * MM * 2 * D * 2);
        WinB<D> wb;
        float aLr[2], aLs[2];
        uint32_t a_perm, a_px, c_gp, c_pp, a_st;
        // output: one (b, h) sequence up to the segment end; stores past it are dropped
        const __amdgpu_buffer_rsrc_t ob = __builtin_amdgcn_make_buffer_rsrc(
            o + b * N * H * D + h * D, 0, static_cast<int>(t_end * H * D * 2), 0x00020000);
        const int orsb = static_cast<int>(H * D * 2);
        lds_barrier();  // features of chunk 0 are in shared memory
        for (int c = 0; c < nch; ++c) {
            const int64_t t0 = t_begin + static_cast<int64_t>(c) * L;
            half8 bZ[CW][2];
            // lane bases and per-lane constants, recomputed every chunk (cheaper
            // than holding them in registers across the loop next to the state)
            wb = win_b<D>(sm.zkT);
#pragma unroll
            for (int mu = 0; mu < 2; ++mu) {
                const float2 a = sm.aL[(32 * w + 16 * mu + i) >> 1];
                aLr[mu] = a.x;
                aLs[mu] = (i & 1) ? a.y : -a.y;
            }
            a_perm = opaque(lds_addr(sm.yq) + 2 * (i * RY + 4 * g));  // y' 8-byte halves of rows 16tt + i
            a_px = opaque(lds_addr(sm.xc) + 2 * (i * RS + 4 * g));    // X, likewise
            a_st = opaque(lds_addr(sm.sc) + 2 * (i * RS + 32 * w + 4 * g));
            c_gp = opaque(lds_addr(sm.gp) + 2 * (i * RP + 24 - 8 * g));  // G' fragments at column 56 - 32kb - 8g
            c_pp = opaque(lds_addr(sm.pp) + 2 * (i * RP + 8 * g));

            // ---- G phase: G = Y Z_k^T tiles, stored skewed as G'
#pragma unroll
            for (int slot = 0; slot < 3; ++slot) {
                const int qt = w + 4 * slot;
                if (qt < 10) {
                    const int tt = tile_tt(qt), jt = tile_kt(qt);
                    // (recomputed every chunk: kept out of the registers held across the loop)
                    const uint32_t ar = opaque(lds_addr(sm.yq) + 2 * ((16 * tt + i) * RY + 8 * g));
                    const uint32_t br0 = opaque(lds_addr(sm.zkT) + 2 * o128(8 * g + (i >> 2), 16 * jt + 4 * (i & 3)));
                    const uint32_t br1 = opaque(lds_addr(sm.zkT) + 2 * o128(8 * g + (i >> 2) + 4, 16 * jt + 4 * (i & 3)));
                    f4 accG = {};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        accG = mfma(rd8(ar + 64 * kb), cat(rd4t(br0 + 4096 * kb), rd4t(br1 + 4096 * kb)), accG);
                    const uint32_t gs = opaque(lds_addr(sm.gp) + 2 * ((16 * tt + 4 * g) * (RP - 1) + L - 1 + 16 * jt + i));
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        if (16 * jt + i <= 16 * tt + 4 * g + jj) wr1(gs + 2 * (RP - 1) * jj, accG[jj]);
                }
            }
            lds_barrier();

            // ---- S phase: per U block mu: Q^T = U Y^T, S^T = T^T G'^T (K order reversed:
            // element jj <-> k = 32kb + 8g + 7 - jj), s~ = sigma~ (S + abar^{t+1} Q),
            // X = s~ abar^{t+1}; then the U update and the Z_v fragments
#pragma unroll
            for (int mu = 0; mu < 2; ++mu) {
                // abar^{i+1} and abar^16 of modes 16w + 8mu + 2g + qq
                const float4 e0 = *reinterpret_cast<const float4*>(&sm.pw[i][16 * w + 8 * mu + 2 * g]);
                const float4 e16 = *reinterpret_cast<const float4*>(&sm.pw[15][16 * w + 8 * mu + 2 * g]);
                float er[2] = {e0.x, e0.z}, ei[2] = {e0.y, e0.w};
                const float e16r[2] = {e16.x, e16.z}, e16i[2] = {e16.y, e16.w};
#pragma unroll
                for (int th2 = 0; th2 < 2; ++th2) {  // t-tiles 2 th2, 2 th2 + 1
                    f4 accQ[2], accS[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) accQ[u] = accS[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const half8 aU = to_half8(st.U[mu][2 * kb], st.U[mu][2 * kb + 1]);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const uint32_t row = a_perm + 2 * (16 * (2 * th2 + u) * RY + 32 * kb);
                            accQ[u] = mfma(aU, cat(rd4(row), rd4(row + 32)), accQ[u]);
                        }
                        step_fence();
                    }
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const uint32_t ta =
                            opaque(lds_addr(sm.ft) + 2 * (o128(i, L - 8 - 32 * kb - 8 * g) + 64 * (32 * w + 16 * mu)));
                        const half8 aT = rd8(ta), aTl = rd8(ta + dl);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const half8 bg = rd8(c_gp + 2 * (16 * (2 * th2 + u) * RP + 32 * (1 - kb)));
                            accS[u] = mfma(aT, bg, accS[u]);
                            accS[u] = mfma(aTl, bg, accS[u]);
                        }
                        step_fence();
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int tt = 2 * th2 + u;
                        const float sg = sm.sig[16 * tt + i];
                        float sv[4], xv[4];
#pragma unroll
                        for (int qq = 0; qq < 2; ++qq) {
                            const float qr = accQ[u][2 * qq], qi = accQ[u][2 * qq + 1];
                            const float sr = sg * (accS[u][2 * qq] + er[qq] * qr - ei[qq] * qi);
                            const float si = sg * (accS[u][2 * qq + 1] + er[qq] * qi + ei[qq] * qr);
                            sv[2 * qq] = sr;
                            sv[2 * qq + 1] = -si;
                            xv[2 * qq] = sr * er[qq] - si * ei[qq];
                            xv[2 * qq + 1] = -(sr * ei[qq] + si * er[qq]);
                            const float nr = er[qq] * e16r[qq] - ei[qq] * e16i[qq];
                            ei[qq] = er[qq] * e16i[qq] + ei[qq] * e16r[qq];
                            er[qq] = nr;
                        }
                        wr4(a_st + 2 * (16 * tt * RS + 16 * mu), sv[0], sv[1], sv[2], sv[3]);
                        wr4(a_st + 2 * (16 * tt * RS + 16 * mu) + xc_sc, xv[0], xv[1], xv[2], xv[3]);
                    }
                }
            }
            key_update<D>(st, wb, aLr, aLs);
            load_bz<D>(bZ, wb);
            lds_barrier();

            // ---- P phase: P~'[t][k] = sum_m' sc[t][m'] T[k][m'] tiles (lane (g, i) of the T
            // operand holds k = 16 kt + 15 - i), un-skewed into P~[t][t - k]
#pragma unroll
            for (int slot = 0; slot < 3; ++slot) {
                const int qt = w + 4 * slot;
                if (qt < 10) {
                    const int tt = tile_tt(qt), kt = tile_kt(qt);
                    const uint32_t ar = opaque(lds_addr(sm.sc) + 2 * ((16 * tt + i) * RS + 8 * g));
                    const uint32_t br0 = opaque(lds_addr(sm.ft) + 2 * o128(8 * g + (i >> 2), L - 16 - 16 * kt + 4 * (i & 3)));
                    const uint32_t br1 = opaque(lds_addr(sm.ft) + 2 * o128(8 * g + (i >> 2) + 4, L - 16 - 16 * kt + 4 * (i & 3)));
                    f4 accP = {};
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const half8 a = rd8(ar + 64 * kb);
                        accP = mfma(a, cat(rd4t(br0 + 4096 * kb), rd4t(br1 + 4096 * kb)), accP);
                        accP = mfma(a, cat(rd4t(br0 + 4096 * kb + dl), rd4t(br1 + 4096 * kb + dl)), accP);
                    }
                    const uint32_t ps = opaque(lds_addr(sm.pp) + 2 * ((16 * tt + 4 * g) * (RP + 1) - 16 * kt - 15 + i));
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        if (16 * kt + 15 - i <= 16 * tt + 4 * g + jj) wr1(ps + 2 * (RP + 1) * jj, accP[jj]);
                }
            }
            lds_barrier();

            // ---- O phase: o = Delta (X Gamma_prev + P~ Z_v); Gamma update
#pragma unroll
            for (int ct = 0; ct < CW; ++ct) {
                half8 bG[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) bG[kb] = to_half8(st.Gm[2 * kb][ct], st.Gm[2 * kb + 1][ct]);
                const uint32_t olane = static_cast<uint32_t>(4 * g * orsb + 2 * (16 * (CW * w + ct) + i));
#pragma unroll
                for (int th2 = 0; th2 < 2; ++th2) {  // t-tiles 2 th2, 2 th2 + 1
                    f4 accO[2] = {};
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const uint32_t row = a_px + 2 * (16 * (2 * th2 + u) * RS + 32 * kb);
                            accO[u] = mfma(cat(rd4(row), rd4(row + 32)), bG[kb], accO[u]);
                        }
                        step_fence();
                    }
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            accO[u] = mfma(rd8(c_pp + 2 * (16 * (2 * th2 + u) * RP + 32 * kb)), bZ[ct][kb], accO[u]);
                        step_fence();
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const uint32_t toff = static_cast<uint32_t>((t0 + 16 * (2 * th2 + u) + jj) * orsb);
                            __builtin_amdgcn_raw_buffer_store_b16(to_bf16(accO[u][jj] * dt), ob, olane + toff, 0, 0);
                        }
                }
            }
            value_update<D>(st, sm.aL, wb, bZ);
            lds_barrier();
        }
        if (seg == S - 1 && state_out != nullptr)
            state_store<D>(st, state_out + bh * MM * 2 * D * 2,
                           n_last < L ? reinterpret_cast<const float2*>(th + kTabPwBack) : nullptr);
    } else {
        // ---------------- feature waves: chunk c + 1 while the MFMA waves run chunk c
        FmRaw<D, true> rr;
        const int rsb = static_cast<int>(H * D * 2);
        const int f = tid - 256;
        const int lane_b = 2 * (8 * (f >> 5) * static_cast<int>(H * D) + CPT * (f & 31));
        const SeqBuf sq = seq_buf<D>(q, k, v, b, h, N, H, t_end);
        const FmAddr<D> fa = fm_addr<D>(sm.zkT, sm.yq);
        load_qk<D, true>(rr, sq, t_begin, rsb, lane_b, true);
        load_qk<D, true>(rr, sq, t_begin, rsb, lane_b, false);
        load_v<D, true>(rr, sq, t_begin, rsb, lane_b);
        {
            const int n0 = nch > 1 ? L : n_last;
            half8 zk[CPT];
            fm_keys<D, true>(zk, rr, sm, t_begin, n0, p.eps_feat, p.eps_norm);
#pragma unroll
            for (int c = 0; c < CPT; ++c) wr8(fa.z[c], zk[c]);
            fm_values<D, true>(rr, sm, fa, n0, p.eps_norm);
            fm_queries<D>(rr, sm, fa.y, t_begin, p.eps_feat, inv_dt);
            if (nch > 1) {
                load_qk<D, true>(rr, sq, t_begin + L, rsb, lane_b, true);
                load_qk<D, true>(rr, sq, t_begin + L, rsb, lane_b, false);
                load_v<D, true>(rr, sq, t_begin + L, rsb, lane_b);
            }
        }
        lds_barrier();  // features of chunk 0 are in shared memory
        for (int c = 0; c < nch; ++c) {
            const int64_t t0 = t_begin + static_cast<int64_t>(c) * L;
            const int n1 = c + 2 < nch ? L : (c + 1 < nch ? n_last : 0);  // valid tokens of chunk c + 1
            half8 zk[CPT];
            lds_barrier();  // G phase
            if (c + 1 < nch) fm_keys<D, true>(zk, rr, sm, t0 + L, n1, p.eps_feat, p.eps_norm);
            lds_barrier();  // S phase
            if (c + 1 < nch) {
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) wr8(fa.z[cc], zk[cc]);
                if (c + 2 < nch) load_qk<D, true>(rr, sq, t0 + 2 * L, rsb, lane_b, false);
                fm_values<D, true>(rr, sm, fa, n1, p.eps_norm);
                if (c + 2 < nch) load_v<D, true>(rr, sq, t0 + 2 * L, rsb, lane_b);
            }
            lds_barrier();  // P phase
            if (c + 1 < nch) {
                fm_queries<D>(rr, sm, fa.y, t0 + L, p.eps_feat, inv_dt);
                if (c + 2 < nch) load_qk<D, true>(rr, sq, t0 + 2 * L, rsb, lane_b, true);
            }
            lds_barrier();  // O phase
        }
    }
}

void plan_segments(const Problem& p, int& S, int64_t& Lseg) {
    const int64_t pairs = p.B * p.H;
    const int64_t chunks = (p.N + L - 1) / L;
    int64_t s = 256 / pairs;  // one workgroup per compute unit
    if (s < 1) s = 1;
    if (s > chunks) s = chunks > 0 ? chunks : 1;
    const int64_t cps = (chunks + s - 1) / s;
    Lseg = cps * L;
    S = static_cast<int>((p.N + Lseg - 1) / Lseg);
    if (S < 1) S = 1;
}

template <int D>
hipError_t launch(const Problem& p, const idattn_params& prm, const void* q, const void* k, const void* v, void* o,
                  const float* state_in, const void* tail_in, float* state_out, void* workspace, hipStream_t stream) {
    int S;
    int64_t Lseg;
    plan_segments(p, S, Lseg);
    const auto* q16 = static_cast<const uint16_t*>(q);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const auto* t16 = static_cast<const uint16_t*>(tail_in);
    uint8_t* tab = static_cast<uint8_t*>(workspace);
    float* ws = reinterpret_cast<float*>(tab + static_cast<size_t>(p.H) * kTabBytes);
    const int64_t pairs = p.B * p.H;
    const int64_t last_len = p.N - (S - 1) * Lseg;
    const int back = static_cast<int>((L - last_len % L) % L);
    zoh_tables_kernel<<<dim3(static_cast<unsigned>(p.H), 16), 256, 0, stream>>>(p, prm, Lseg, back, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (S > 1) {
        segment_state_kernel<D><<<dim3(static_cast<unsigned>(pairs * (S - 1))), NTH, 0, stream>>>(p, prm, k16, v16,
                                                                                                 t16, tab, ws, Lseg, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t total = pairs * MM * 2 * p.d;
        segment_carry_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(p, state_in, tab,
                                                                                                  ws, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    chunked_forward_kernel<D><<<dim3(static_cast<unsigned>(pairs * S)), NTH, 0, stream>>>(
        p, prm, q16, k16, v16, static_cast<uint16_t*>(o), state_in, t16, state_out, tab, ws, Lseg, S);
    return hipGetLastError();
}

}  // namespace
}  // namespace cws

size_t chunked_ws_workspace_bytes(const Problem& p) {
    int S;
    int64_t Lseg;
    cws::plan_segments(p, S, Lseg);
    return static_cast<size_t>(p.H) * cws::kTabBytes +
           static_cast<size_t>(S - 1) * p.B * p.H * p.M * 2 * p.d * 2 * sizeof(float);
}

hipError_t launch_forward_chunked_ws(const Problem& p, const idattn_params& prm, const void* q, const void* k,
                                     const void* v, void* o, const float* state_in, const void* tail_in,
                                     float* state_out, void* workspace, hipStream_t stream) {
    if (p.d == 128) return cws::launch<128>(p, prm, q, k, v, o, state_in, tail_in, state_out, workspace, stream);
    return cws::launch<64>(p, prm, q, k, v, o, state_in, tail_in, state_out, workspace, stream);
}

}  // namespace idattn

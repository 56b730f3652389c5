// Chunked parallel-in-time forward of the Interdomain Attention mixer for
// R = d = 128 and M = 64 modes: bf16 I/O, fp16 MFMA operands, fp32
// accumulation and fp32 state.  Eight waves per workgroup, two per SIMD, so
// that one wave's LDS and dependency latency is covered by the other.
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
//
// Index m' = 2 m + part (part 0 = real, 1 = imaginary) runs over the 2M = 128
// real rows of a complex mode set.  Register-resident state, per wave w:
//   U     : rows r (all 128), columns m' in [16w, 16w+16)  -> 8 MFMA tiles
//   Gamma : rows m' (all 128), columns c in [16w, 16w+16)  -> 8 MFMA tiles
// An accumulator tile [X][Y] doubles as an operand with K = X once two of
// them are concatenated (lane (g, i) then supplies K rows 4g..4g+3 and
// 16+4g..16+4g+3 of a 32-row block), so U feeds y_q . U and Gamma feeds the
// readout straight from registers.
//
// z_k and z_v go to shared memory transposed ([channel][token]) so that both
// state updates and the intra-chunk readout read them as plain fragments.
#include "common.h"
#include "launch.h"

namespace idattn {
namespace d128 {
namespace {

constexpr int D = 128;       // R = d
constexpr int L = 64;        // chunk length
constexpr int MM = 64;       // complex modes
constexpr int M2 = 2 * MM;   // m' rows
constexpr int NTH = 512;     // eight waves
constexpr int kMaxW = 4;     // conv widths 1..4
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLn2Sq = 0.4804530139182014f;
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));  // 4 bf16 values
typedef short s4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(const half8& a, const half8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ tile layouts
// Shared-memory tiles are [rows][128] fp16 padded to RQ halfs per row (read
// as 8-byte halves and as 16-byte fragments), [rows][64] fp16 padded to RP,
// and [rows][64] fp16 with the 16-byte chunk index of (row, col) XOR-ed with
// a function of row % 16 (read as 16-byte fragments and with transposing
// reads).  Each layout touches every bank once for the read pattern it serves.
constexpr int RQ = 136;
constexpr int RP = 72;
__host__ __device__ constexpr int sw128(int r) { return 2 * (((r >> 1) & 3) ^ (2 * ((r >> 3) & 1))) + ((r >> 3) & 1); }
__host__ __device__ constexpr int o128(int r, int col) { return r * 64 + ((((col >> 3) ^ sw128(r)) & 7) << 3) + (col & 7); }

__device__ __forceinline__ half8 ld8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ half4 ld4(const _Float16* p) { return *reinterpret_cast<const half4*>(p); }
__device__ __forceinline__ half8 cat(const half4& a, const half4& b) {
    half8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i & 3) of the 4-element read of lane 4j + (i >> 2), for j = 0..3.
__device__ __forceinline__ half4 ld4_tr(const _Float16* p) {
    const s4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v*)(const_cast<_Float16*>(p)));
    return __builtin_bit_cast(half4, r);
}
// MFMA operand with K along the rows of a swizzled [rows][64] tile: lane (g, i)
// gets x[kbase + 8g + jj][c0 + i], jj = 0..7 (kbase a multiple of 16, c0 of 16).
__device__ __forceinline__ half8 ld8_tr128(const _Float16* x, int kbase, int c0) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    const int r0 = kbase + 8 * g + (i >> 2), col = c0 + 4 * (i & 3);
    return cat(ld4_tr(x + o128(r0, col)), ld4_tr(x + o128(r0 + 4, col)));
}

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
// point: one K-step of fragments is live at a time, and the other wave on the
// SIMD covers the load latency.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// ------------------------------------------------------------------ tables
// Per-head tables, one launch per forward (fp64 arithmetic):
//   ft, ftl [M2][L] fp16, swizzled rows: F^T[m'][j] = T_{m'}[L-1-j] = ft + ftl
//   pw [L][MM] float2: abar^{k+1}
//   pwseg[MM], pwback[MM] float2: abar^{Lseg}, abar^{-back};  hc: Delta, 1/Delta
// with T_{m'}[k] the real (m' even) or imaginary (m' odd) part of bbar_m abar_m^k.
// T enters every chunk of every sequence, so its rounding error would add up
// coherently; as the pair (ft, ftl) of fp16 values it carries about 22 bits,
// and every product with T is two MFMAs.
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
// 32-bit LDS byte addresses.  A per-lane base computed once and passed
// through an empty asm statement stays in one VGPR, and the constant part of
// each access goes into the instruction's 16-bit offset field; the arrays are
// ordered so that every such family of accesses spans less than 64 KiB.
typedef __attribute__((address_space(3))) half8 lds_h8;
typedef __attribute__((address_space(3))) half4 lds_h4;
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
__device__ __forceinline__ half4 rd4t(uint32_t a) {
    return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(uintptr_t)a));
}
__device__ __forceinline__ void wr4(uint32_t a, float x0, float x1, float x2, float x3) {
    *(lds_h4*)(uintptr_t)a = half4{static_cast<_Float16>(x0), static_cast<_Float16>(x1), static_cast<_Float16>(x2),
                                   static_cast<_Float16>(x3)};
}
__device__ __forceinline__ void wr1(uint32_t a, float x) { *(lds_h1*)(uintptr_t)a = static_cast<_Float16>(x); }

struct SmemFwd {
    // window A: [t][128] tiles
    _Float16 yq[L * RQ];       // y' of the queries [t][r]
    union {
        struct {
            _Float16 sc[L * RQ];   // [t][m'] (Re s~, -Im s~)
            _Float16 xc[L * RQ];   // [t][m'] (Re X, -Im X)
        } v;
        u2 tails[2 * 16 * 3 * 32]; // featmap neighbour tails [q|k][block][token][lane]
    } u;
    // window B: swizzled [128][64] tiles
    _Float16 zkT[D * L];       // z_k^T [r][j]
    _Float16 zvT[D * L];       // z_v^T [c][l]
    _Float16 ft[M2 * L];       // F^T, high and low fp16 parts
    _Float16 ftl[M2 * L];
    // window C: [t][64] tiles
    _Float16 gp[L * RP];       // G' (zero above the causal band, never rewritten there)
    _Float16 pp[L * RP];       // P~ [t][l] (likewise)
    float sig[L];              // sigma~_t
    float2 aL[MM];             // abar^L
    float gain[2 * D], bias[2 * D];
    float wq[D * kMaxW], wk[D * kMaxW];  // conv weights times -log2(e), right-aligned taps
    uint16_t halo[2][2][3][D];           // raw q, k of the 3 tokens before the chunk, double buffered
};

struct SmemSeg {
    _Float16 zkT[D * L];
    _Float16 zvT[D * L];
    _Float16 ft[M2 * L];
    _Float16 ftl[M2 * L];
    u2 tails[16 * 3 * 32];
    float2 aL[MM];
    float gain[2 * D], bias[2 * D];
    float wk[D * kMaxW];
    uint16_t halo[2][2][3][D];
};
// byte distances inside window B (identical in both layouts)
constexpr uint32_t kZv = D * L * 2, kFt = 2 * D * L * 2, kFtl = 3 * D * L * 2;

// ------------------------------------------------------------------ featmap
// Thread (cgi = tid % 32, tb = tid / 32) owns channels 4cgi..4cgi+3 of tokens
// 4tb..4tb+3; the short conv slides along a 7-token register window whose
// first 3 tokens come from block tb-1 (or, for tb = 0, the previous chunk).
template <bool WITH_Q>
struct Raw {
    u2 q[WITH_Q ? 4 : 1];
    u2 k[4];
    u2 v[4];
};

// Buffer resources over one (b, h) sequence up to the end of the segment:
// token t, channel c sits at byte 2 (t H D + c) from the sequence's first
// token.  Loads past the end of a resource return zeros, which pads a ragged
// last chunk.
struct SeqBuf {
    __amdgpu_buffer_rsrc_t q, k, v;
};
__device__ __forceinline__ SeqBuf seq_buf(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t b,
                                          int64_t h, int64_t N, int64_t H, int64_t t_end) {
    const int64_t first = b * N * H * D + h * D;  // element offset of token 0 of the sequence
    const int nrec = static_cast<int>(t_end * H * D * 2);
    SeqBuf r;
    r.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(q ? q + first : k + first), 0, nrec, 0x00020000);
    r.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + first), 0, nrec, 0x00020000);
    r.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v + first), 0, nrec, 0x00020000);
    return r;
}

// Raw bf16 values of the chunk starting at token t0: lane_off = 2 (4 tb H D +
// 4 cgi) bytes, rsb = 2 H D bytes per token.
template <bool WITH_Q>
__device__ __forceinline__ void prefetch(Raw<WITH_Q>& r, const SeqBuf& sb, int64_t t0, int rsb, uint32_t lane_off) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int soff = static_cast<int>((t0 + s) * rsb);
        if constexpr (WITH_Q)
            r.q[s] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(sb.q, lane_off, soff, 0));
        r.k[s] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(sb.k, lane_off, soff, 0));
        r.v[s] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(sb.v, lane_off, soff, 0));
    }
}

__device__ __forceinline__ void unpack(const u2& u, float* x) {
    x[0] = __uint_as_float(u[0] << 16);
    x[1] = __uint_as_float(u[0] & 0xffff0000u);
    x[2] = __uint_as_float(u[1] << 16);
    x[3] = __uint_as_float(u[1] & 0xffff0000u);
}

// y' = c' / (1 + 2^c') for the 4 x 4 window outputs; ss = partial ||y'||^2.
__device__ __forceinline__ void conv_silu(const float (&x)[7][4], const float (&w)[4][kMaxW], float (&y)[4][4],
                                          float (&ss)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        ss[s] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float acc = w[c][0] * x[s][c];
#pragma unroll
            for (int j = 1; j < kMaxW; ++j) acc = fmaf(w[c][j], x[s + j][c], acc);
            y[s][c] = acc * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(acc));
            ss[s] = fmaf(y[s][c], y[s][c], ss[s]);
        }
    }
}

// Per-lane store addresses of the featmap: z_k^T rows 4cgi + c at column 4tb
// (z_v^T at + kZv), and y' row 4tb at column 4cgi (rows + RQ halfs).
struct FmAddr {
    uint32_t z[4];
    uint32_t y;
};
__device__ __forceinline__ FmAddr fm_addr(const void* zkT, const void* yq) {
    const int cgi = threadIdx.x & 31, tb = threadIdx.x >> 5;
    FmAddr a;
#pragma unroll
    for (int c = 0; c < 4; ++c) a.z[c] = opaque(lds_addr(zkT) + 2 * o128(4 * cgi + c, 4 * tb));
    a.y = yq ? opaque(lds_addr(yq) + 2 * (4 * tb * RQ + 4 * cgi)) : 0u;
    return a;
}

// One chunk (n valid tokens).  Writes zkT, zvT (zero columns past n when
// PARTIAL) and with WITH_Q also yq and sig; reads halo[par], writes
// halo[par ^ 1].  Starts with the neighbour-tail exchange and its barrier,
// ends without one.
template <bool WITH_Q, bool PARTIAL, class SM>
__device__ __forceinline__ void featmap(SM& sm, u2* tails, const Raw<WITH_Q>& r, const FmAddr& fa, float eps_feat,
                                        float eps_norm, float inv_dt, int par, int n) {
    const int cgi = threadIdx.x & 31, tb = threadIdx.x >> 5;
    const int c0 = 4 * cgi;
    constexpr int SELQ = 0, SELK = WITH_Q ? 1 : 0;  // tail slots
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        if (tb < 15) {
            if constexpr (WITH_Q) tails[((SELQ * 16 + tb) * 3 + j) * 32 + cgi] = r.q[1 + j];
            tails[((SELK * 16 + tb) * 3 + j) * 32 + cgi] = r.k[1 + j];
        } else {
            if constexpr (WITH_Q) *reinterpret_cast<u2*>(&sm.halo[par ^ 1][0][j][c0]) = r.q[1 + j];
            *reinterpret_cast<u2*>(&sm.halo[par ^ 1][1][j][c0]) = r.k[1 + j];
        }
    }
    lds_barrier();
    // keys
    {
        float y[4][4], ss[4];
        {
            float x[7][4], w[4][kMaxW];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int j = 0; j < kMaxW; ++j) w[c][j] = sm.wk[(c0 + c) * kMaxW + j];
#pragma unroll
            for (int j = 0; j < 3; ++j)
                unpack(tb == 0 ? *reinterpret_cast<const u2*>(&sm.halo[par][1][j][c0])
                               : tails[((SELK * 16 + tb - 1) * 3 + j) * 32 + cgi], x[j]);
#pragma unroll
            for (int s = 0; s < 4; ++s) unpack(r.k[s], x[3 + s]);
            conv_silu(x, w, y, ss);
        }
        sum32<4>(ss);
        float rho[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // xi = -ln2 inv y',  mean xi^2 = ln^2 2 inv^2 ||y'||^2 / D
            const float inv = __builtin_amdgcn_rcpf(fmaf(kLn2Sq, ss[s], eps_feat));
            const float rs = __builtin_amdgcn_rsqf(fmaf(kLn2Sq * (1.f / D) * inv * inv, ss[s], eps_norm));
            rho[s] = -kLn2 * inv * rs;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float g = sm.gain[c0 + c], bb = sm.bias[c0 + c];
            float z[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                z[s] = fmaf(g * rho[s], y[s][c], bb);
                if (PARTIAL && 4 * tb + s >= n) z[s] = 0.f;
            }
            wr4(fa.z[c], z[0], z[1], z[2], z[3]);
        }
    }
    // values
    {
        float xv[4][4], ss[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            unpack(r.v[s], xv[s]);
            ss[s] = xv[s][0] * xv[s][0];
#pragma unroll
            for (int c = 1; c < 4; ++c) ss[s] = fmaf(xv[s][c], xv[s][c], ss[s]);
        }
        sum32<4>(ss);
        float rs[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) rs[s] = __builtin_amdgcn_rsqf(fmaf(1.f / D, ss[s], eps_norm));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float g = sm.gain[D + c0 + c], bb = sm.bias[D + c0 + c];
            float z[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                z[s] = fmaf(g * rs[s], xv[s][c], bb);
                if (PARTIAL && 4 * tb + s >= n) z[s] = 0.f;
            }
            wr4(fa.z[c] + kZv, z[0], z[1], z[2], z[3]);
        }
    }
    // queries
    if constexpr (WITH_Q) {
        float y[4][4], ss[4];
        {
            float x[7][4], w[4][kMaxW];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int j = 0; j < kMaxW; ++j) w[c][j] = sm.wq[(c0 + c) * kMaxW + j];
#pragma unroll
            for (int j = 0; j < 3; ++j)
                unpack(tb == 0 ? *reinterpret_cast<const u2*>(&sm.halo[par][0][j][c0])
                               : tails[((SELQ * 16 + tb - 1) * 3 + j) * 32 + cgi], x[j]);
#pragma unroll
            for (int s = 0; s < 4; ++s) unpack(r.q[s], x[3 + s]);
            conv_silu(x, w, y, ss);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) wr4(fa.y + 2 * s * RQ, y[s][0], y[s][1], y[s][2], y[s][3]);
        sum32<4>(ss);
        if (cgi == 0) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sm.sig[4 * tb + s] = -kLn2 * inv_dt * __builtin_amdgcn_rcpf(fmaf(kLn2Sq, ss[s], eps_feat));
        }
    }
}

// Conv weights (times -log2 e, taps right-aligned into 4 slots), gain, bias,
// and the halo of the first chunk of a segment starting at t0: raw q, k at
// t0-3..t0-1 from the input (position >= 0), from tail_in (position < 0) or zeros.
template <bool WITH_Q, class SM>
__device__ __forceinline__ void load_prologue(SM& sm, const idattn_params& prm, const uint16_t* q, const uint16_t* k,
                                              const uint16_t* tail_in, int64_t b, int64_t h, int64_t N, int64_t H,
                                              int64_t t0, int W) {
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

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void copy16(void* dst, const void* src, int bytes) {
    for (int e = threadIdx.x; e < bytes / 16; e += NTH)
        reinterpret_cast<u4*>(dst)[e] = reinterpret_cast<const u4*>(src)[e];
}

// ------------------------------------------------------------------ state
// Lane (g, i) of wave w:
//   U[rt][jj]  = U_m[r],     r = 16rt + 4g + jj,  m' = 16w + i
//   Gm[mt][jj] = Gamma_m[c], m' = 16mt + 4g + jj, c = 16w + i
// Memory layout: float [M][2D][2] (complex), columns 0..D-1 hold U, D..2D-1 Gamma.
struct State {
    f4 U[8];
    f4 Gm[8];
};

__device__ __forceinline__ void state_load(State& st, const float* src) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * rt + 4 * g + jj, mp = 16 * w + i;
            st.U[rt][jj] = src ? src[((mp >> 1) * 2 * D + r) * 2 + (mp & 1)] : 0.f;
        }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int mp = 16 * mt + 4 * g + jj, c = 16 * w + i;
            st.Gm[mt][jj] = src ? src[((mp >> 1) * 2 * D + D + c) * 2 + (mp & 1)] : 0.f;
        }
}

// Stores the state, first multiplying every mode by corr[m] when corr is not NULL.
__device__ __forceinline__ void state_store(const State& st, float* dst, const float2* corr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
    {
        const int mp = 16 * w + i;
        const float2 c = corr ? corr[mp >> 1] : make_float2(1.f, 0.f);
        const float sc = (mp & 1) ? c.y : -c.y;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rt + 4 * g + jj;
                const float u = st.U[rt][jj];
                const float pu = dpp_mov<0xB1>(u);  // other part of the same mode (lane i ^ 1)
                dst[((mp >> 1) * 2 * D + r) * 2 + (mp & 1)] = fmaf(sc, pu, c.x * u);
            }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int m = 8 * mt + 2 * g + q, c = 16 * w + i;
            const float2 a = corr ? corr[m] : make_float2(1.f, 0.f);
            const float gr = st.Gm[mt][2 * q], gi = st.Gm[mt][2 * q + 1];
            *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + D + c) * 2) =
                make_float2(a.x * gr - a.y * gi, a.x * gi + a.y * gr);
        }
}

// Lane bases into window B (byte addresses from z_k^T) for fragment reads of
// rows R0 + i at column chunk 4kb + g: all[kb] for R0 = 16 * (0..7) of any of
// the four tiles, own[kb] for R0 = 16w (the wave's m' block or c block).
struct WinB {
    uint32_t all[2];
    uint32_t own[2];
};
__device__ __forceinline__ WinB win_b(const void* zkT) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
    WinB b;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        b.all[kb] = opaque(lds_addr(zkT) + 2 * o128(i, 32 * kb + 8 * g));
        b.own[kb] = opaque(lds_addr(zkT) + 2 * (o128(i, 32 * kb + 8 * g) + 1024 * w));
    }
    return b;
}

// U <- abar^L U + Z_k^T F  (the real and imaginary rows of a mode sit in lanes i, i ^ 1)
__device__ __forceinline__ void key_update(State& st, const WinB& wb, float aLr, float aLs) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float u = st.U[rt][jj];
            st.U[rt][jj] = fmaf(aLs, dpp_mov<0xB1>(u), aLr * u);
        }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const half8 bF = rd8(wb.own[kb] + kFt);   // F[j][m'], j = 32kb + 8g + jj, m' = 16w + i
        const half8 bFl = rd8(wb.own[kb] + kFtl);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const half8 a = rd8(wb.all[kb] + 2048 * rt);  // z_k[j][r = 16rt + i]
            st.U[rt] = mfma(a, bF, st.U[rt]);
            st.U[rt] = mfma(a, bFl, st.U[rt]);
            if (rt == 3) step_fence();
        }
        step_fence();
    }
}

// Gamma <- abar^L Gamma + F^T Z_v, with bZ[kb] = Z_v[32kb + 8g + jj][16w + i]
__device__ __forceinline__ void value_update(State& st, const float2* aL, const WinB& wb, const half8 (&bZ)[2]) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const float4 a = *reinterpret_cast<const float4*>(&aL[8 * mt + 2 * g]);
        const float r0 = st.Gm[mt][0], i0 = st.Gm[mt][1], r1 = st.Gm[mt][2], i1 = st.Gm[mt][3];
        st.Gm[mt][0] = a.x * r0 - a.y * i0;
        st.Gm[mt][1] = a.x * i0 + a.y * r0;
        st.Gm[mt][2] = a.z * r1 - a.w * i1;
        st.Gm[mt][3] = a.z * i1 + a.w * r1;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            st.Gm[mt] = mfma(rd8(wb.all[kb] + kFt + 2048 * mt), bZ[kb], st.Gm[mt]);
            st.Gm[mt] = mfma(rd8(wb.all[kb] + kFtl + 2048 * mt), bZ[kb], st.Gm[mt]);
            if (mt == 3 || mt == 7) step_fence();
        }
}

__device__ __forceinline__ void load_bz(half8 (&bZ)[2], const WinB& wb) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) bZ[kb] = rd8(wb.own[kb] + kZv);
}

__device__ __forceinline__ half8 to_half8(const f4& a, const f4& b) {
    half8 r;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        r[jj] = static_cast<_Float16>(a[jj]);
        r[4 + jj] = static_cast<_Float16>(b[jj]);
    }
    return r;
}

// ------------------------------------------------------------------ kernels
// Segment end states from a zero start: grid B*H*(S-1), block (bh, seg).
__global__ __launch_bounds__(NTH) void segment_state_kernel(Problem p, idattn_params prm,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ tail_in,
                                                            const uint8_t* __restrict__ tab, float* __restrict__ ws,
                                                            int64_t Lseg, int S) {
    __shared__ SmemSeg sm;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, i = lane & 15;
    const int cgi = threadIdx.x & 31, tb = threadIdx.x >> 5;
    const int64_t bh = blockIdx.x / (S - 1);
    const int seg = static_cast<int>(blockIdx.x % (S - 1));
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t t_begin = seg * Lseg, t_end = t_begin + Lseg;  // segments 0..S-2 are full
    const uint8_t* th = tab + h * kTabBytes;
    load_prologue<false>(sm, prm, k, k, tail_in, b, h, p.N, p.H, t_begin, static_cast<int>(p.W));
    copy16(sm.ft, th + kTabFT, M2 * L * 2);
    copy16(sm.ftl, th + kTabFTL, M2 * L * 2);
    if (threadIdx.x < MM) sm.aL[threadIdx.x] = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + threadIdx.x];
    State st;
    state_load(st, nullptr);
    const WinB wb = win_b(sm.zkT);
    const FmAddr fa = fm_addr(sm.zkT, nullptr);
    const int rsb = static_cast<int>(p.H * D * 2);
    const uint32_t lane_off = static_cast<uint32_t>(4 * tb * rsb + 8 * cgi);
    const SeqBuf sq = seq_buf(nullptr, k, v, b, h, p.N, p.H, t_end);
    Raw<false> rr;
    prefetch<false>(rr, sq, t_begin, rsb, lane_off);
    __syncthreads();
    const float2 aLu = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + ((16 * w + i) >> 1)];
    const float aLs = (i & 1) ? aLu.y : -aLu.y;
    int par = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += L) {
        featmap<false, false>(sm, sm.tails, rr, fa, p.eps_feat, p.eps_norm, 0.f, par, L);
        if (t0 + L < t_end) prefetch<false>(rr, sq, t0 + L, rsb, lane_off);
        lds_barrier();
        key_update(st, wb, aLu.x, aLs);
        half8 bZ[2];
        load_bz(bZ, wb);
        value_update(st, sm.aL, wb, bZ);
        par ^= 1;
    }
    state_store(st, ws + (static_cast<int64_t>(seg) * p.B * p.H + bh) * MM * 2 * D * 2, nullptr);
}

// Carry chain over segments, one thread per complex state element:
// ws[seg] <- state entering segment seg+1.
__global__ __launch_bounds__(256) void segment_carry_kernel(Problem p, const float* __restrict__ state_in,
                                                            const uint8_t* __restrict__ tab,
                                                            float* __restrict__ ws, int S) {
    const int64_t total = p.B * p.H * MM * 2 * D;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t m = (e / (2 * D)) % MM;
    const int64_t h = (e / (2 * D * MM)) % p.H;
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
__global__ __launch_bounds__(NTH) void chunked_forward_kernel(Problem p, idattn_params prm,
                                                              const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                              const float* state_in,
                                                              const uint16_t* __restrict__ tail_in, float* state_out,
                                                              const uint8_t* __restrict__ tab,
                                                              const float* __restrict__ carry, int64_t Lseg, int S) {
    __shared__ SmemFwd sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
    const int cgi = tid & 31, tb = tid >> 5;
    const int64_t bh = blockIdx.x / S;
    const int seg = static_cast<int>(blockIdx.x % S);
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t N = p.N, H = p.H;
    const int64_t t_begin = seg * Lseg;
    const int64_t t_end = t_begin + Lseg < N ? t_begin + Lseg : N;
    const uint8_t* th = tab + h * kTabBytes;

    load_prologue<true>(sm, prm, q, k, tail_in, b, h, N, H, t_begin, static_cast<int>(p.W));
    copy16(sm.ft, th + kTabFT, M2 * L * 2);
    copy16(sm.ftl, th + kTabFTL, M2 * L * 2);
    if (tid < MM) sm.aL[tid] = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + tid];
    for (int e = tid; e < L * RP * 2 / 16; e += NTH)
        reinterpret_cast<u4*>(sm.gp)[e] = reinterpret_cast<u4*>(sm.pp)[e] = u4{0u, 0u, 0u, 0u};
    State st;
    state_load(st, seg == 0 ? (state_in ? state_in + bh * MM * 2 * D * 2 : nullptr)
                            : carry + (static_cast<int64_t>(seg - 1) * p.B * p.H + bh) * MM * 2 * D * 2);
    // per-lane constants
    const float2* pw = reinterpret_cast<const float2*>(th + kTabPw);
    const float2 hc = reinterpret_cast<const float2*>(th + kTabHc)[0];
    const float dt = hc.x, inv_dt = hc.y;
    const float2 aLu = pw[(L - 1) * MM + ((16 * w + i) >> 1)];
    const float aLs = (i & 1) ? aLu.y : -aLu.y;
    float e0r[2], e0i[2], e16r[2], e16i[2];  // abar^{i+1}, abar^16 of modes 8w + 2g + q
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        const float2 a = pw[i * MM + 8 * w + 2 * g + qq];
        const float2 a16 = pw[15 * MM + 8 * w + 2 * g + qq];
        e0r[qq] = a.x;
        e0i[qq] = a.y;
        e16r[qq] = a16.x;
        e16i[qq] = a16.y;
    }
    const int tw = w >> 1, jb = 2 * (w & 1);  // G / P~ tiles (tw, jb) and (tw, jb + 1)
    // window A (from yq): 8-byte halves of rows 16tt + i (y' and X), fragments of rows 16tw + i (y', s~),
    // s~ / X stores at rows 16tt + i
    const uint32_t a_perm = opaque(lds_addr(sm.yq) + 2 * (i * RQ + 4 * g));
    const uint32_t a_rowG = opaque(lds_addr(sm.yq) + 2 * ((16 * tw + i) * RQ + 8 * g));
    const uint32_t a_st = opaque(lds_addr(sm.u.v.sc) + 2 * (i * RQ + 16 * w + 4 * g));
    constexpr uint32_t kSc = L * RQ * 2, kXc = 2 * L * RQ * 2;  // from yq
    // window B
    const WinB wb = win_b(sm.zkT);
    uint32_t b_rev[2];   // F^T rows 16w + i at column chunk 7 - 4kb - g (from ft)
    uint32_t b_tr[2][2];  // transposing reads of z_k^T for the G tiles (from zkT)
    uint32_t b_trT[2][2]; // and of F^T for the P~ tiles (from ft)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) b_rev[kb] = opaque(lds_addr(sm.ft) + 2 * (o128(i, L - 8 - 32 * kb - 8 * g) + 1024 * w));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            b_tr[u][hh] = opaque(lds_addr(sm.zkT) + 2 * o128(8 * g + (i >> 2) + 4 * hh, 16 * (jb + u) + 4 * (i & 3)));
            b_trT[u][hh] = opaque(lds_addr(sm.ft) + 2 * o128(8 * g + (i >> 2) + 4 * hh, L - 16 - 16 * (jb + u) + 4 * (i & 3)));
        }
    // window C
    const uint32_t c_gp = opaque(lds_addr(sm.gp) + 2 * (i * RP + 24 - 8 * g));  // G' fragments, column 56 - 32kb - 8g
    const uint32_t c_pp = opaque(lds_addr(sm.pp) + 2 * (i * RP + 8 * g));
    // skewed stores: G'[t][L-1-t+j] and P~[t][t-kc] for t = 16tw + 4g + jj, j = 16(jb+u) + i, kc = 16(jb+u) + 15 - i
    const uint32_t c_gs = opaque(lds_addr(sm.gp) + 2 * ((16 * tw + 4 * g) * (RP - 1) + L - 1 + 16 * jb + i));
    const uint32_t c_ps = opaque(lds_addr(sm.pp) + 2 * ((16 * tw + 4 * g) * (RP + 1) - 16 * jb - 31 + i));
    const FmAddr fa = fm_addr(sm.zkT, sm.yq);
    const int64_t rs = H * D;
    const int rsb = static_cast<int>(rs * 2);
    const uint32_t lane_off = static_cast<uint32_t>(4 * tb * rsb + 8 * cgi);
    const SeqBuf sq = seq_buf(q, k, v, b, h, N, H, t_end);
    Raw<true> rr;
    prefetch<true>(rr, sq, t_begin, rsb, lane_off);
    __syncthreads();

    int par = 0;
    int n = L;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += L) {
        n = static_cast<int>(t_end - t0 < L ? t_end - t0 : L);
        if (n == L)
            featmap<true, false>(sm, sm.u.tails, rr, fa, p.eps_feat, p.eps_norm, inv_dt, par, n);
        else
            featmap<true, true>(sm, sm.u.tails, rr, fa, p.eps_feat, p.eps_norm, inv_dt, par, n);
        if (t0 + L < t_end) prefetch<true>(rr, sq, t0 + L, rsb, lane_off);
        lds_barrier();

        // ---- G = Y Z_k^T (tiles (tw, jb), (tw, jb + 1)) stored skewed; Q^T = U Y^T; U update
        f4 accQ[4];
        {
            if (jb <= tw) {
                f4 accG[2] = {};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const half8 a = rd8(a_rowG + 64 * kb);
                    accG[0] = mfma(a, cat(rd4t(b_tr[0][0] + 4096 * kb), rd4t(b_tr[0][1] + 4096 * kb)), accG[0]);
                    if (jb + 1 <= tw)
                        accG[1] = mfma(a, cat(rd4t(b_tr[1][0] + 4096 * kb), rd4t(b_tr[1][1] + 4096 * kb)), accG[1]);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        if (16 * (jb + u) + i <= 16 * tw + 4 * g + jj)
                            wr1(c_gs + 2 * ((RP - 1) * jj + 16 * u), accG[u][jj]);
            }
            half8 aU[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) aU[kb] = to_half8(st.U[2 * kb], st.U[2 * kb + 1]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) accQ[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const uint32_t row = a_perm + 2 * (16 * tt * RQ + 32 * kb);
                    accQ[tt] = mfma(aU[kb], cat(rd4(row), rd4(row + 32)), accQ[tt]);
                }
                step_fence();
            }
            key_update(st, wb, aLu.x, aLs);
        }
        lds_barrier();

        // ---- S^T = T^T G'^T (K order reversed: element jj <-> k = 32kb + 8g + 7 - jj);
        // s~ = sigma~ (S + abar^{t+1} Q), X = s~ abar^{t+1}
        {
            f4 accS[4] = {};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const half8 aT = rd8(b_rev[kb]);
                const half8 aTl = rd8(b_rev[kb] + (kFtl - kFt));
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const half8 bg = rd8(c_gp + 2 * (16 * tt * RP + 32 * (1 - kb)));
                    accS[tt] = mfma(aT, bg, accS[tt]);
                    accS[tt] = mfma(aTl, bg, accS[tt]);
                }
            }
            float er[2] = {e0r[0], e0r[1]}, ei[2] = {e0i[0], e0i[1]};
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float sg = sm.sig[16 * tt + i];
                float sv[4], xv[4];
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    const float qr = accQ[tt][2 * qq], qi = accQ[tt][2 * qq + 1];
                    const float sr = sg * (accS[tt][2 * qq] + er[qq] * qr - ei[qq] * qi);
                    const float si = sg * (accS[tt][2 * qq + 1] + er[qq] * qi + ei[qq] * qr);
                    sv[2 * qq] = sr;
                    sv[2 * qq + 1] = -si;
                    xv[2 * qq] = sr * er[qq] - si * ei[qq];
                    xv[2 * qq + 1] = -(sr * ei[qq] + si * er[qq]);
                    const float nr = er[qq] * e16r[qq] - ei[qq] * e16i[qq];
                    ei[qq] = er[qq] * e16i[qq] + ei[qq] * e16r[qq];
                    er[qq] = nr;
                }
                wr4(a_st + 2 * 16 * tt * RQ, sv[0], sv[1], sv[2], sv[3]);
                wr4(a_st + 2 * 16 * tt * RQ + (kXc - kSc), xv[0], xv[1], xv[2], xv[3]);
            }
        }
        lds_barrier();

        // ---- P~'[t][k] = sum_m' sc[t][m'] T[k][m'] (tiles (tw, jb), (tw, jb + 1); lane (g, i)
        // of the T operand holds k = 16 kt + 15 - i), un-skewed into P~[t][t - k]
        if (jb <= tw) {
            f4 accP[2] = {};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const half8 a = rd8(a_rowG + kSc + 64 * kb);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (u == 1 && jb + 1 > tw) break;
                    const uint32_t o0 = b_trT[u][0] + 4096 * kb, o1 = b_trT[u][1] + 4096 * kb;
                    accP[u] = mfma(a, cat(rd4t(o0), rd4t(o1)), accP[u]);
                    accP[u] = mfma(a, cat(rd4t(o0 + (kFtl - kFt)), rd4t(o1 + (kFtl - kFt))), accP[u]);
                }
                step_fence();
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (16 * (jb + u) + 15 - i <= 16 * tw + 4 * g + jj)
                        wr1(c_ps + 2 * ((RP + 1) * jj + 16 * (1 - u)), accP[u][jj]);
        }
        lds_barrier();

        // ---- o = Delta (X Gamma_prev + P~ Z_v); Gamma update
        {
            f4 accO[4];
            half8 bG[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) bG[kb] = to_half8(st.Gm[2 * kb], st.Gm[2 * kb + 1]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) accO[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const uint32_t row = a_perm + kXc + 2 * (16 * tt * RQ + 32 * kb);
                    accO[tt] = mfma(cat(rd4(row), rd4(row + 32)), bG[kb], accO[tt]);
                }
                step_fence();
            }
            half8 bZ[2];
            load_bz(bZ, wb);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) accO[tt] = mfma(rd8(c_pp + 2 * (16 * tt * RP + 32 * kb)), bZ[kb], accO[tt]);
                step_fence();
            }
            uint16_t* obase = o + ((b * N + t0) * H + h) * D + 16 * w + i;
            if (n == L) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) obase[(16 * tt + 4 * g + jj) * rs] = to_bf16(accO[tt][jj] * dt);
            } else {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int t = 16 * tt + 4 * g + jj;
                        if (t < n) obase[t * rs] = to_bf16(accO[tt][jj] * dt);
                    }
            }
            value_update(st, sm.aL, wb, bZ);
        }
        par ^= 1;
    }
    if (seg == S - 1 && state_out != nullptr)
        state_store(st, state_out + bh * MM * 2 * D * 2,
                    n < L ? reinterpret_cast<const float2*>(th + kTabPwBack) : nullptr);
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

}  // namespace
}  // namespace d128

size_t chunked_d128_workspace_bytes(const Problem& p) {
    int S;
    int64_t Lseg;
    d128::plan_segments(p, S, Lseg);
    return static_cast<size_t>(p.H) * d128::kTabBytes +
           static_cast<size_t>(S - 1) * p.B * p.H * p.M * 2 * p.d * 2 * sizeof(float);
}

hipError_t launch_forward_chunked_d128(const Problem& p, const idattn_params& prm, const void* q, const void* k,
                                       const void* v, void* o, const float* state_in, const void* tail_in,
                                       float* state_out, void* workspace, hipStream_t stream) {
    using namespace d128;
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
        segment_state_kernel<<<dim3(static_cast<unsigned>(pairs * (S - 1))), NTH, 0, stream>>>(p, prm, k16, v16, t16,
                                                                                              tab, ws, Lseg, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t total = pairs * MM * 2 * D;
        segment_carry_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(p, state_in, tab,
                                                                                                  ws, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    chunked_forward_kernel<<<dim3(static_cast<unsigned>(pairs * S)), NTH, 0, stream>>>(
        p, prm, q16, k16, v16, static_cast<uint16_t*>(o), state_in, t16, state_out, tab, ws, Lseg, S);
    return hipGetLastError();
}

}  // namespace idattn

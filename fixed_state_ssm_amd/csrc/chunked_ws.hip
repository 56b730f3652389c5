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
//  * y' of each token is scaled by a power of two r_t with (r_t ||y'||)^2 in
//    [1, 4), and the mode scores are kept as s~_t = K (S + abar^{t+1} Q) with one
//    constant K = -ln2 / (4 Delta kappa), so that s~, P~ = Re(s~ T^T) and
//    X = s~ abar^{t+1} kept in fp16 are O(1) for queries of any scale; the
//    rest of the true scale, sigma_t = -ln2 / (Delta (ln^2 2 ||y'||^2 + eps)),
//    returns on the output as o_t = omega_t (P~ Z_v + Re X Gamma)_t with
//    omega_t = 4 Delta / (kappa r_t (ln^2 2 ||y'||^2 + eps)) (kappa below).
//  * T enters every chunk of every sequence, so its fp16 rounding error would
//    add up coherently; it is carried as a pair of fp16 values (about 22
//    bits) and every product with T is two MFMAs.
//
// Two kernels run per segment of the sequence.  The feature pass builds z_k
// and z_v of every chunk once (short conv, SiLU, norms), stores them as fp16
// tiles for the forward, and runs the state updates from a zero start to get
// each segment's end state; a carry chain turns those into the state entering
// each segment; the forward then runs the full chunk loop of its segment.
// A workgroup is sixteen waves, four per SIMD, two roles of eight waves:
// key waves own the key state U and run the products that make s~ and X
// (G, y_q . U, G'T) and the U update, and build the queries' features of the
// next chunk; value waves own the value state Gamma and run the P~ tiles, the
// readout (X Gamma, P~ Z_v) and the Gamma update.
//
// Index m' = 2 m + part (part 0 = real, 1 = imaginary) runs over the 2M = 128
// real rows of a complex mode set.  Key wave kw (0..7) keeps U's rows r (all
// D) of columns m' in [16kw, 16kw+16) (D/16 MFMA tiles); value wave vw keeps
// Gamma's rows m' (all 128) of columns c in [16vw, 16vw+16) (8 tiles; value
// waves vw >= D/16 own none).
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
constexpr int NTH = 1024;    // sixteen waves
constexpr int kMaxW = 4;     // conv widths 1..4
constexpr int RP = L + 16;   // padded row length of [t][64] tiles
constexpr int PWS = MM + 4;  // padded row length (float2) of the abar^{k+1} rows
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLn2Sq = 0.4804530139182014f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kFoldMax = 4;  // largest segment count whose carry the forward folds in

// Packed batches.  With C = ceil(H sum_b c_b / 256) chunks per segment
// (c_b chunks in sequence b), sequence b has S_b = max(1, ceil(c_b / C))
// segments, and since ceil(c_b / C) - 1 < c_b / C:
//   blocks       H sum_b S_b       <= 256 + B H
//   end states   H sum_b (S_b - 1) <  256
//   carry list   the b with S_b > kFoldMax have c_b > kFoldMax C, so there
//                are fewer than 256 / (kFoldMax H) of them.
__host__ __device__ constexpr int64_t plan_blocks_max(int64_t B, int64_t H) { return 256 + B * H; }
constexpr int64_t kPlanEndStates = 256;
__host__ __device__ constexpr int64_t carry_cap(int64_t H) { return 256 / (kFoldMax * H) + 1; }
constexpr int kPlanHead = 4;
__host__ __device__ constexpr int64_t plan_ints(int64_t B, int64_t H) {
    return kPlanHead + 6 * B + 1 + carry_cap(H);
}
constexpr int kPlanSortMax = 256;  // batches up to this many sequences get their last segments by size

template <int D>
struct Cfg {
    static constexpr int RT = D / 16;   // 16-row tiles over R
    static constexpr int KB = D / 32;   // 32-wide K steps over R
    static constexpr int CP = D / 2;    // channel pairs = lanes that share a feature token block
    static constexpr int NF = 8 * CP;   // feature threads per role (8 token blocks)
    static constexpr int YR = D;        // row length (halfs) of the y' tile
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
// [rows][128] fp16 tiles: 256-byte rows with the 16-byte chunk index XOR-ed by row % 16.
__host__ __device__ constexpr int x256(int r, int col) { return r * 128 + ((((col >> 3) ^ r) & 15) << 3) + (col & 7); }
// The K-ordered [t][*] tiles (y', X) store their columns in the order in which
// a lane supplies them as an MFMA operand: within each block of 32, column
// 4g + e (e < 4) goes to 8g + e and column 16 + 4g + e to 8g + 4 + e, so that
// lane group g reads its eight K values with one 16-byte access.
__host__ __device__ constexpr int perm32(int c) {
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
// y' [t][r]: 256-byte rows (D = 128) or swizzled 128-byte rows (D = 64), columns in perm32 order.
template <int D>
__host__ __device__ constexpr int yq_off(int t, int c) { return D == 128 ? x256(t, perm32(c)) : o128(t, perm32(c)); }
// Byte offset of y'(8tb + s, c) from y'(8tb, c): s rows on, with the row swizzle
// of token s folded into an XOR of the 16-byte chunk bits only.
template <int D>
__host__ __device__ constexpr uint32_t yq_sx(int s) { return D == 128 ? 16u * s : 32u * (s >> 1); }
template <int D>
constexpr uint32_t kYqRow = 2 * D;
template <int D>
constexpr bool yq_xor_ok() {
    for (int tb = 0; tb < L / 8; ++tb)
        for (int c = 0; c < D; c += 2)
            for (int s = 0; s < 8; ++s) {
                const uint32_t b0 = 2u * yq_off<D>(8 * tb, c);
                if (2u * yq_off<D>(8 * tb + s, c) != (b0 ^ yq_sx<D>(s)) + s * kYqRow<D>) return false;
            }
    return true;
}
static_assert(yq_xor_ok<64>() && yq_xor_ok<128>(), "y' row swizzle must reduce to an XOR of chunk bits");

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
// The thread index passed through an empty asm: what is derived from it is
// recomputed at each use instead of being hoisted out of the chunk loop and
// held in registers beside the state.
__device__ __forceinline__ int tid_now() { return static_cast<int>(opaque(threadIdx.x)); }
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

// DPP lane move (every pattern used here has a valid source for every lane);
// written as an update of 0 with bound_ctrl so that the compiler folds it
// into the consuming VALU instruction.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
// Reduce-scatter of 8 per-token partial sums over an aligned group of NL
// lanes (32 or 64): on return lane l holds the group total of token
// tau(l) = 4 b0 + 2 b1 + b2 (b_k bit k of l), so that the 8 lanes l % NL < 8
// hold all 8 tokens.  Each of the first three steps pairs lanes that differ in
// one of bits 0..2, keeps the half of the tokens that the lane's bit selects
// and adds what the partner sends of that half; the last steps add the one
// remaining value across bit 3 (rotate by 8 within a row), across rows
// (v_permlane16_swap) and across halves (v_permlane32_swap).  For bit 2 the
// partner is the lane 4 apart in rotation within its row of 16, which has the
// other bit 2 and the same bits 0..1; together with the rotation by 8 every
// lane of the group of 4 sharing bits 0..1 contributes once.
template <int NL>
__device__ __forceinline__ float reduce_scatter8(const float (&v)[8]) {
    const int l = tid_now();
    const bool b0 = l & 1, b1 = l & 2, b2 = l & 4;
    float u[4], w[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float send = b0 ? v[k] : v[k + 4], keep = b0 ? v[k + 4] : v[k];
        u[k] = keep + dpp_mov<0xB1>(send);  // quad_perm [1,0,3,2]
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float send = b1 ? u[k] : u[k + 2], keep = b1 ? u[k + 2] : u[k];
        w[k] = keep + dpp_mov<0x4E>(send);  // quad_perm [2,3,0,1]
    }
    float x = (b2 ? w[1] : w[0]) + dpp_mov<0x124>(b2 ? w[0] : w[1]);  // row_ror:4
    x += dpp_mov<0x128>(x);                                           // row_ror:8
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (NL == 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}
__device__ __forceinline__ int scatter_token(int l) { return 4 * (l & 1) + 2 * ((l >> 1) & 1) + ((l >> 2) & 1); }

// Keeps the compiler from hoisting the next step's operand loads above this
// point: one K-step of fragments is live at a time.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }
// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima).  Loads and
// stores share this counter and may complete out of order with respect to
// each other, so once a store is in flight every wait for a load waits for
// the store as well; a wave that stores collects its prefetched loads with
// this wait before it issues the stores.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
// Two floats to a packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, bf16x2));
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

// ------------------------------------------------------------------ tables
// Per-head tables, one launch per forward (fp64 arithmetic):
//   ft, ftl [M2][L] fp16, swizzled rows: F^T[m'][j] = T_{m'}[L-1-j] = ft + ftl
//   pw [L][MM] float2: abar^{k+1}
//   pwseg[MM] float2: abar^{Lseg};  hc float4: Delta, 1/Delta, kappa, 1/kappa
//   hs [L][MM] float2: bbar sum_{j<=k} abar^j, dz [MM] double4: abar, bbar
//   (normalised readout only)
// with kappa a power of two per head such that kappa max_m |bbar_m| is in
// [1/2, 1): F carries kappa (so that a small Delta |B| leaves the fp16 table
// in the normal range), and so do the states derived from it.
// with T_{m'}[k] the real (m' even) or imaginary (m' odd) part of bbar_m abar_m^k.
constexpr int kTabFT = 0;
constexpr int kTabFTL = kTabFT + M2 * L * 2;
constexpr int kTabPw = kTabFTL + M2 * L * 2;
constexpr int kTabPwSeg = kTabPw + L * MM * 8;
constexpr int kTabHc = kTabPwSeg + MM * 8;
constexpr int kTabHs = ((kTabHc + 16 + 255) / 256) * 256;  // [L][MM] float2: bbar sum_{j<=k} abar^j
constexpr int kTabDz = kTabHs + L * MM * 8;                  // [MM] double4: abar, bbar
constexpr int kTabBytes = kTabDz + MM * 32;

// abar^n by repeated squaring in fp64 (n >= 0): about 2 log2(n) complex
// products, so the relative error stays near 1e-14 for any n here, with no
// transcendental function (and no argument reduction of a large n Delta Im
// lambda).
__device__ inline void cpow_int(double ar, double ai, int64_t n, double& pr, double& pi) {
    pr = 1.0;
    pi = 0.0;
    double br = ar, bi = ai;
    while (n > 0) {
        if (n & 1) {
            const double t = pr * br - pi * bi;
            pi = pr * bi + pi * br;
            pr = t;
        }
        const double t = br * br - bi * bi;
        bi = 2.0 * br * bi;
        br = t;
        n >>= 1;
    }
}
// bbar sum_{j<n} abar^j = bbar (abar^n - 1) / (abar - 1), given abar^n (n bbar
// when abar = 1): the response of the S4D system to n steps of a constant
// input of one, which is what the normaliser eta accumulates.  abar - 1 has
// a relative error near 1e-16 / |Delta lambda| in fp64, far below fp32.
__device__ inline void geo_from_pow(double ar, double ai, double br, double bi, double pnr, double pni, double n,
                                    double& sr, double& si) {
    const double dr = ar - 1.0, di = ai;
    const double den = dr * dr + di * di;
    double qr = n, qi = 0.0;
    if (den > 1e-280) {
        const double nr = pnr - 1.0, ni = pni;
        qr = (nr * dr + ni * di) / den;
        qi = (ni * dr - nr * di) / den;
    }
    sr = br * qr - bi * qi;
    si = br * qi + bi * qr;
}

// Complex fp64 power abar^n = exp(n Delta lambda).
__device__ __forceinline__ void cpow(double dt, float lre, float lim, double n, double& pr, double& pi) {
    double sy, cy;
    sincos(n * dt * lim, &sy, &cy);
    const double e = exp(n * dt * lre);
    pr = e * cy;
    pi = e * sy;
}

constexpr int kTabThreads = 320;

// Sum (or max) over the block of the tables kernel; every thread gets it.
__device__ __forceinline__ int64_t block_reduce(int64_t v, bool mx, int64_t* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const int64_t o = __shfl_xor(v, off, kWave);
        v = mx ? (o > v ? o : v) : v + o;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
    for (int j = 1; j < kTabThreads / 64; ++j) v = mx ? (red[j] > v ? red[j] : v) : v + red[j];
    __syncthreads();
    return v;
}

// The plan of a packed batch, built by one block from the sequence table cu
// (device int32 [B + 1]): the segment size C (see plan_blocks_max), the
// offsets of every sequence (exclusive scans over b), the order of the last
// segments and the carry list (abar^{C L} of each head follows in the
// feature pass, from the fp64 abar of the tables).  A table
// that does not rise from 0 to T gives a plan of no blocks: nothing runs and
// no output is written.
__device__ void packed_plan(const Problem& p, const int32_t* __restrict__ cu, int32_t* __restrict__ plan) {
    __shared__ int64_t red[kTabThreads / 64];
    __shared__ int64_t scan[kTabThreads / 64][4];
    __shared__ int32_t key[kPlanSortMax];
    const int tid = threadIdx.x, nt = kTabThreads;
    const int64_t B = p.B, T = p.N, H = p.H;
    auto chunks = [&](int64_t b) -> int64_t {
        const int64_t n = static_cast<int64_t>(cu[b + 1]) - cu[b];
        return n > 0 ? (n + L - 1) / L : 0;
    };
    int64_t tc = 0, bad = 0;
    for (int64_t b = tid; b < B; b += nt) {
        if (cu[b + 1] < cu[b]) bad = 1;
        tc += chunks(b);
    }
    if (tid == 0 && (cu[0] != 0 || cu[B] != T)) bad = 1;
    bad = block_reduce(bad, true, red);
    tc = block_reduce(tc, false, red);
    if (bad) {
        if (tid == 0) {
            plan[0] = 1;
            plan[1] = plan[2] = plan[3] = 0;
        }
        return;
    }
    int64_t cps = (H * tc + 255) / 256;
    cps = cps < 1 ? 1 : cps;
    // exclusive scans over b of c_b, S_b - 1, [S_b > kFoldMax], on contiguous
    // runs of sequences per thread
    const int64_t per = (B + nt - 1) / nt, b0 = tid * per < B ? tid * per : B, b1 = b0 + per < B ? b0 + per : B;
    int64_t v[3] = {0, 0, 0};
    for (int64_t b = b0; b < b1; ++b) {
        const int64_t c = chunks(b), sb = c > cps ? (c + cps - 1) / cps : 1;
        v[0] += c;
        v[1] += sb - 1;
        v[2] += sb > kFoldMax ? 1 : 0;
    }
    int64_t inc[3], tot[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        int64_t x = v[j];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t y = __shfl_up(x, off, kWave);
            if ((tid & 63) >= off) x += y;
        }
        inc[j] = x;
        if ((tid & 63) == 63) scan[tid >> 6][j] = x;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        tot[j] = 0;
        for (int w = 0; w < kTabThreads / 64; ++w) {
            if (w < (tid >> 6)) inc[j] += scan[w][j];
            tot[j] += scan[w][j];
        }
    }
    int64_t ec = inc[0] - v[0], es = inc[1] - v[1], ek = inc[2] - v[2];
    const int64_t cap = carry_cap(H);
    int32_t* soff = plan + kPlanHead + 4 * B;
    int32_t* order = plan + kPlanHead + 5 * B + 1;
    for (int64_t b = b0; b < b1; ++b) {
        const int64_t c = chunks(b), sb = c > cps ? (c + cps - 1) / cps : 1;
        plan[kPlanHead + b] = cu[b];
        plan[kPlanHead + B + b] = cu[b + 1] - cu[b];
        plan[kPlanHead + 2 * B + b] = static_cast<int32_t>(sb);
        plan[kPlanHead + 3 * B + b] = static_cast<int32_t>(ec);
        soff[b] = static_cast<int32_t>(es);
        if (sb > kFoldMax) {
            if (ek < cap) plan[kPlanHead + 6 * B + 1 + ek] = static_cast<int32_t>(b);
            ++ek;
        }
        if (B <= kPlanSortMax) key[b] = static_cast<int32_t>(c - (sb - 1) * cps);  // last segment's chunks
        ec += c;
        es += sb - 1;
    }
    if (tid == 0) {
        plan[0] = static_cast<int32_t>(cps);
        plan[1] = static_cast<int32_t>(H * (tot[1] + B));
        plan[2] = static_cast<int32_t>(tot[2] < cap ? tot[2] : cap);
        plan[3] = static_cast<int32_t>(H * tot[1]);
        soff[B] = static_cast<int32_t>(tot[1]);
    }
    // the order of the last segments: by size, longest first (ties by b), for
    // batches of up to kPlanSortMax sequences; else b itself
    __syncthreads();
    for (int64_t b = tid; b < B; b += nt) {
        int64_t rank = b;
        if (B <= kPlanSortMax) {
            rank = 0;
            const int32_t kb = key[b];
            for (int64_t j = 0; j < B; ++j) rank += (key[j] > kb || (key[j] == kb && j < b)) ? 1 : 0;
        }
        order[rank] = static_cast<int32_t>(b);
    }
}

// grid (H, 17), 320 threads.  Blocks y < 16: threads 0..255 take one (k, m)
// each and evaluate abar^k while threads 256..319 run the ZOH step of mode m
// into shared memory, then T = bbar abar^k and abar^{k+1} = abar^k abar;
// block y = 16: abar^Lseg (threads 0..63), or for a packed batch (plan !=
// nullptr) the plan, built by block (0, 16) alone.  Also abar, bbar in fp64
// (dz), for the closed forms of the normaliser and of packed segment powers.  The ZOH wave of a block
// y < 16 also finds the head's scale kappa.  No thread runs more than one
// fp64 power or ZOH step before the combine.
__global__ __launch_bounds__(kTabThreads) void zoh_tables_kernel(Problem p, idattn_params prm, int64_t Lseg,
                                                                 uint8_t* __restrict__ tab,
                                                                 const int32_t* __restrict__ cu,
                                                                 int32_t* __restrict__ plan) {
    __shared__ Zoh zs[MM];
    __shared__ double kap_s;
    const int64_t h = blockIdx.x;
    if (blockIdx.y == 16 && plan != nullptr) {
        if (h == 0) packed_plan(p, cu, plan);
        return;
    }
    uint8_t* th = tab + h * kTabBytes;
    const int m = threadIdx.x & (MM - 1);
    const float log_dt = prm.log_dt[h];
    const float lre = prm.A[(h * MM + m) * 2], lim = prm.A[(h * MM + m) * 2 + 1];
    const double dt = exp(static_cast<double>(log_dt));
    double pr = 0.0, pi = 0.0;
    if (blockIdx.y == 16) {
        if (threadIdx.x >= MM) return;
        cpow(dt, lre, lim, static_cast<double>(Lseg), pr, pi);
        reinterpret_cast<float2*>(th + kTabPwSeg)[m] = make_float2(static_cast<float>(pr), static_cast<float>(pi));
        return;
    }
    const int k = 4 * static_cast<int>(blockIdx.y) + (threadIdx.x >> 6);
    if (threadIdx.x >= 256) {  // one wave: the ZOH step of mode m, then the head's scale kappa
        const Zoh z = zoh_mode(log_dt, lre, lim, prm.Bc[(h * MM + m) * 2], prm.Bc[(h * MM + m) * 2 + 1]);
        zs[m] = z;
        double b2 = z.br * z.br + z.bi * z.bi;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) b2 = fmax(b2, __shfl_xor(b2, off, kWave));
        if (m == 0) {
            int ex = 0;
            if (b2 > 0.0 && b2 < 1e300) frexp(sqrt(b2), &ex);  // max |bbar| = f 2^ex, f in [1/2, 1)
            ex = ex < -60 ? -60 : ex > 60 ? 60 : ex;
            kap_s = ldexp(1.0, -ex);
        }
    } else
        cpow(dt, lre, lim, static_cast<double>(k), pr, pi);  // abar^k
    __syncthreads();
    if (threadIdx.x >= 256) return;
    const double kap = kap_s;
    if (blockIdx.y == 0 && threadIdx.x == 0)
        reinterpret_cast<float4*>(th + kTabHc)[0] = make_float4(static_cast<float>(dt), static_cast<float>(1.0 / dt),
                                                               static_cast<float>(kap), static_cast<float>(1.0 / kap));
    const Zoh z = zs[m];
    const double tv[2] = {kap * (z.br * pr - z.bi * pi), kap * (z.br * pi + z.bi * pr)};
    _Float16* ft = reinterpret_cast<_Float16*>(th + kTabFT);
    _Float16* ftl = reinterpret_cast<_Float16*>(th + kTabFTL);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        const _Float16 hi = static_cast<_Float16>(static_cast<float>(tv[part]));
        ft[o128(2 * m + part, L - 1 - k)] = hi;
        ftl[o128(2 * m + part, L - 1 - k)] = static_cast<_Float16>(static_cast<float>(tv[part] - static_cast<double>(hi)));
    }
    reinterpret_cast<float2*>(th + kTabPw)[k * MM + m] =
        make_float2(static_cast<float>(pr * z.ar - pi * z.ai), static_cast<float>(pr * z.ai + pi * z.ar));
    if (blockIdx.y == 0 && k == 0) reinterpret_cast<double4*>(th + kTabDz)[m] = make_double4(z.ar, z.ai, z.br, z.bi);
    if (p.eta) {  // Hsum(k) = bbar sum_{j<=k} abar^j, for the normaliser
        double hr, hi;
        geo_from_pow(z.ar, z.ai, z.br, z.bi, pr * z.ar - pi * z.ai, pr * z.ai + pi * z.ar, static_cast<double>(k + 1), hr,
                     hi);
        reinterpret_cast<float2*>(th + kTabHs)[k * MM + m] = make_float2(static_cast<float>(hr), static_cast<float>(hi));
    }
}

// ------------------------------------------------------------------ shared memory
template <int D>
struct SmemFwd {
    // window A: [t][*] tiles
    _Float16 yq[L * D];           // y' of the queries [t][r] (yq_off)
    _Float16 sc[L * M2];          // [t][m'] (Re s~, -Im s~) (x256 of perm32)
    _Float16 xc[L * M2];          // [t][m'] (Re X, -Im X) (x256 of perm32)
    // window B: swizzled [rows][64] tiles
    _Float16 zkT[D * L];          // z_k^T [r][j]
    _Float16 zvT[D * L];          // z_v^T [c][l]
    _Float16 ft[M2 * L];          // F^T, high and low fp16 parts
    _Float16 ftl[M2 * L];
    // window C
    // G' and P~ rows of RP = L + 16 halves, read in columns 0..L-1 only.  The
    // tiles are written whole: the non-causal G'[t][L-1+(j-t)], j > t, land in
    // row t's padding columns L..L+14, and P~[t][t-k], k > t, in row t-1's
    // padding columns RP-15..RP-1 (for t = 0, those of G''s last row, which
    // precedes pp).  The columns below the causal band are zeroed once and
    // never written.
    _Float16 gp[L * RP];          // G'
    _Float16 pp[L * RP];          // P~ [t][l] (must follow gp)
    float om[3][L];               // omega_t, output factor of each token, by chunk mod 3
    float2 aL[MM];                // abar^L
    float2 aH[MM];                // abar^(L/2)
    float2 pw[16][PWS];           // abar^{k+1}, k = 0..15
    float gain[2 * D], bias[2 * D];
    float wq[D * kMaxW], wk[D * kMaxW];  // conv weights times -log2(e), right-aligned taps (layout: wt_index)
    uint16_t halo[2][3][D];              // raw q, k at positions -3..-1 of the sequence
    float fac[16][2][8];                 // per-token feature factors, by wave and token block
    // normalised readout: eta before the chunk, Hsum(15), Hsum(L-1), and the key
    // waves' partial denominators [chunk parity][token][key wave]
    float2 ec0[MM], hs15[MM], hsL[MM];
    float dpart[2][L][8];
};
static_assert(offsetof(SmemFwd<128>, pp) == offsetof(SmemFwd<128>, gp) + sizeof(_Float16) * L * RP &&
                  offsetof(SmemFwd<64>, pp) == offsetof(SmemFwd<64>, gp) + sizeof(_Float16) * L * RP && RP >= L + 15,
              "the P~ tile must follow G' and rows need 15 halves of padding");

template <int D>
struct SmemSeg {
    _Float16 zkT[2][D * L];  // by chunk parity
    _Float16 zvT[2][D * L];
    _Float16 ft[M2 * L];
    _Float16 ftl[M2 * L];
    float2 aL[MM];
    float gain[2 * D], bias[2 * D];
    float wk[D * kMaxW];
    uint16_t halo[2][3][D];
    float fac[16][2][8];
};

// byte distances inside window B (identical in both layouts)
template <int D>
struct WinOff {
    static constexpr uint32_t zv = D * L * 2, ft = 2 * D * L * 2, ftl = 2 * D * L * 2 + M2 * L * 2;
};

// ------------------------------------------------------------------ work of a block
// A block runs one segment of one (b, h) sequence.  Dense batches (plan ==
// nullptr): sequence b at token b N of the token axis, N tokens, S segments
// of Lseg tokens each (the last one shorter or ragged); blocks 0..F-1 run
// the F = B H (S - 1) full segments in ((b, h), seg) order, blocks F.. the
// last segments in (b, h) order, so that the short ones are dispatched last.
// Packed batches: the plan (built on the device from the sequence table)
// gives every sequence its first token, length and segment count S_b, all
// segments of C chunks but each sequence's last.  Blocks 0..F-1 run the F =
// H sum_b (S_b - 1) full segments in (b, h, seg) order; the blocks after them
// run the last segments, in the plan's order of sequences (longest last
// segment first, so that the blocks that do not fit in the first wave of the
// chip are the short ones), heads innermost; blocks past the plan's total
// are idle.  A sequence of no tokens has one block per head, which passes
// its state and tail through.
// Per (b, h) the z_k^T tiles of its chunks are contiguous from tile0, and
// the end states of its segments 0..S_b-2 contiguous from st0 (in units of
// one state).
// Plan layout (int32): [0] C, [1] blocks, [2] sequences in the carry list,
// [3] F, then start[B], len[B], S[B], chunk offset[B], end-state offset[B + 1]
// (exclusive scan of S_b - 1), order[B], carry list[carry_cap(H)].
struct Blk {
    int64_t b, h, bh, t0, n, tile0, st0, Lseg;
    int seg, S;
    bool idle;
};
__device__ __forceinline__ Blk block_work(const Problem& p, const int32_t* plan, int S_dense, int64_t Lseg_dense) {
    Blk k;
    const int64_t x = blockIdx.x;
    if (plan == nullptr) {
        const int64_t F = p.B * p.H * (S_dense - 1);  // full segments, dispatched first
        if (x < F) {
            k.bh = x / (S_dense - 1);
            k.seg = static_cast<int>(x % (S_dense - 1));
        } else {
            k.bh = x - F;
            k.seg = S_dense - 1;
        }
        k.S = S_dense;
        k.b = k.bh / p.H;
        k.h = k.bh % p.H;
        k.t0 = k.b * p.N;
        k.n = p.N;
        k.Lseg = Lseg_dense;
        k.tile0 = k.bh * S_dense * (Lseg_dense / L);
        k.st0 = k.bh * (S_dense - 1);
        k.idle = false;
        return k;
    }
    const int64_t B = p.B, H = p.H, F = plan[3];
    const int32_t* soff = plan + kPlanHead + 4 * B;
    k.idle = x >= plan[1];
    if (k.idle) return k;
    if (x < F) {
        int64_t lo = 0, hi = B - 1;  // the last b with H soff[b] <= x: it has a full segment x
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (H * soff[mid] <= x) lo = mid;
            else hi = mid - 1;
        }
        k.b = lo;
        k.S = plan[kPlanHead + 2 * B + lo];
        const int64_t local = x - H * soff[lo];
        k.h = local / (k.S - 1);
        k.seg = static_cast<int>(local % (k.S - 1));
    } else {
        const int64_t r = x - F;
        k.b = plan[kPlanHead + 5 * B + 1 + r / H];
        k.h = r % H;
        k.S = plan[kPlanHead + 2 * B + k.b];
        k.seg = k.S - 1;
    }
    k.bh = k.b * H + k.h;
    k.t0 = plan[kPlanHead + k.b];
    k.n = plan[kPlanHead + B + k.b];
    k.Lseg = static_cast<int64_t>(plan[0]) * L;
    const int64_t cb = (k.n + L - 1) / L;  // chunks of the sequence
    k.tile0 = H * static_cast<int64_t>(plan[kPlanHead + 3 * B + k.b]) + k.h * cb;
    k.st0 = H * static_cast<int64_t>(soff[k.b]) + k.h * (k.S - 1);
    return k;
}

// A sequence of no tokens: state_out = state_in (or zeros) and tail_out =
// tail_in (or zeros) for this (b, h), by the whole block (each thread reads
// and writes the same elements, so in place is safe).
template <int D>
__device__ __forceinline__ void copy_through_block(const Problem& p, const Blk& k, const float* state_in,
                                                   float* state_out, const uint16_t* tail_in, uint16_t* tail_out) {
    const int64_t sn = MM * 2 * D * 2, tn = 2 * (p.W - 1) * D;
    if (state_out != nullptr)
        for (int64_t e = threadIdx.x; e < sn; e += NTH) state_out[k.bh * sn + e] = state_in ? state_in[k.bh * sn + e] : 0.f;
    if (tail_out != nullptr)
        for (int64_t e = threadIdx.x; e < tn; e += NTH) tail_out[k.bh * tn + e] = tail_in ? tail_in[k.bh * tn + e] : 0;
}

// ------------------------------------------------------------------ features
// Within a role (512 threads), feature thread fi < NF owns channels 2 cgi and
// 2 cgi + 1 (cgi = fi % CP) of tokens 8 tb .. 8 tb + 7 (tb = fi / CP) of a
// chunk, so that the CP lanes of a token block hold all D channels of its
// tokens and the channel norms are lane sums.  The short conv needs the three
// tokens before, which the thread loads itself (positions < 0 read zeros,
// replaced by the stored tail for the first chunk of a sequence).  With
// D = 64 the feature threads are the upper half of the role.
template <int D>
__device__ __forceinline__ int feat_index() {
    return (tid_now() & 511) ^ (Cfg<D>::NF < 512 ? 256 : 0);
}

// Buffer resources over one (b, h) sequence (first token t0 on the token
// axis) up to the end of the segment: token t, channel c sits at byte
// 2 (t H D + c) from the sequence's first token.  Offsets are whole VGPR operands, which the hardware range-checks;
// loads past the end of a resource return zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const uint16_t* x, int64_t t0, int64_t h, int64_t H,
                                                           int64_t t_end) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (t0 * H + h) * D), 0,
                                             static_cast<int>(t_end * H * D * 2), 0x00020000);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The thread's channel pair of 8 tokens at tok0 + 8tb .. (+7) and, with HALO,
// of the 3 before (slots 0..2); rsb = 2 H D is the byte stride of a token.
template <int D, bool HALO>
__device__ __forceinline__ void fm_load(uint32_t (&r)[HALO ? 11 : 8], __amdgpu_buffer_rsrc_t rs, int rsb,
                                        int64_t tok0, int fi = feat_index<D>()) {
    if (fi >= Cfg<D>::NF) return;
    const int cgi = fi % Cfg<D>::CP, tb = fi / Cfg<D>::CP;
    const uint32_t lane_b = static_cast<uint32_t>(8 * tb * rsb + 4 * cgi);
#pragma unroll
    for (int s = 0; s < (HALO ? 11 : 8); ++s)
        r[s] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane_b + static_cast<uint32_t>((tok0 + s - (HALO ? 3 : 0)) * rsb),
                                                    0, 0);
}
// The stored tail replaces the three positions before the sequence start.
template <int D, class SM>
__device__ __forceinline__ void halo_fix(uint32_t (&r)[11], const SM& sm, int sel, int64_t tok0,
                                         int fi = feat_index<D>()) {
    if (tok0 == 0 && fi < Cfg<D>::CP) {
#pragma unroll
        for (int j = 0; j < 3; ++j) r[j] = *reinterpret_cast<const uint32_t*>(&sm.halo[sel][j][2 * fi]);
    }
}
// Conv weight of channel c, tap j (0..3, right-aligned) in shared memory:
// the thread of channel pair cgi reads taps {0,1} and {2,3} of both channels
// as two 16-byte words at consecutive addresses across the lanes.
template <int D>
__host__ __device__ constexpr int wt_index(int c, int j) {
    return (((j >> 1) * Cfg<D>::CP + (c >> 1)) * 2 + (c & 1)) * 2 + (j & 1);
}

// y'[e][s] = c' / (1 + 2^c') for channel 2 cgi + e and token 8 tb + s;
// ss[s] = partial ||y'||^2 over the thread's two channels.
template <int D>
__device__ __forceinline__ void conv_silu(const uint32_t (&r)[11], const float* w, int cgi, float (&y)[2][8],
                                          float (&ss)[8]) {
    const float4 wa = *reinterpret_cast<const float4*>(w + 4 * cgi);                 // taps 0, 1
    const float4 wb = *reinterpret_cast<const float4*>(w + 4 * (Cfg<D>::CP + cgi));  // taps 2, 3
    const float w0[4] = {wa.x, wa.y, wb.x, wb.y}, w1[4] = {wa.z, wa.w, wb.z, wb.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        float a0 = w0[0] * lo_bf16(r[s]), a1 = w1[0] * hi_bf16(r[s]);
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            a0 = fmaf(w0[j], lo_bf16(r[s + j]), a0);
            a1 = fmaf(w1[j], hi_bf16(r[s + j]), a1);
        }
        y[0][s] = a0 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a0));
        y[1][s] = a1 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a1));
        ss[s] = fmaf(y[1][s], y[1][s], y[0][s] * y[0][s]);
    }
}
// Zeroes the features of tokens 8 tb + s >= n (the end of a ragged last chunk).
__device__ __forceinline__ void mask_tokens(float (&z)[2][8], int tb, int n) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const bool ok = 8 * tb + s < n;
        z[0][s] = ok ? z[0][s] : 0.f;
        z[1][s] = ok ? z[1][s] : 0.f;
    }
}
// z^T rows 2 cgi + e, columns 8 tb .. 8 tb + 7: one 16-byte store per channel.
__device__ __forceinline__ void write_zt(const void* zT, int cgi, int tb, const float (&z)[2][8]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        half8 hv;
#pragma unroll
        for (int s = 0; s < 8; ++s) hv[s] = static_cast<_Float16>(z[e][s]);
        wr8(lds_addr(zT) + 2 * o128(2 * cgi + e, 8 * tb), hv);
    }
}

// Per-token factors through shared memory: the lanes l % NL < 8 of each token
// block hold token tau(l); every lane of the block then reads all 8 (the
// accesses of one wave execute in order, so no barrier is needed).
template <int D, class SM>
__device__ __forceinline__ void share_factor(SM& sm, float f, float (&out)[8]) {
    constexpr int NL = Cfg<D>::CP;
    const int l = tid_now(), w = (l >> 6) & 15, blk = NL == 32 ? (l >> 5) & 1 : 0;
    float* slot = const_cast<float*>(&sm.fac[w][blk][0]);
    if ((l & (NL - 1)) < 8) slot[scatter_token(l)] = f;
    const float4 a = *reinterpret_cast<const float4*>(slot), b = *reinterpret_cast<const float4*>(slot + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// z_k of the thread's 8 tokens to z_k^T (zero past n valid tokens).  With
// pre (random Fourier features), slots 3..10 of r hold the features xi_k
// themselves as fp16 pairs (conv and map applied by rff_features_kernel), and
// only the RMSNorm remains.
template <int D, class SM>
__device__ __forceinline__ void fm_keys(const uint32_t (&r)[11], const SM& sm, const void* zT, int n, float eps_feat,
                                        float eps_norm, bool unit, bool pre, int fi = feat_index<D>()) {
    if (fi >= Cfg<D>::NF) return;
    const int cgi = fi % Cfg<D>::CP, tb = fi / Cfg<D>::CP;
    float y[2][8], ss[8], rho[8];
    if (pre) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const half2v x = __builtin_bit_cast(half2v, r[3 + s]);
            y[0][s] = static_cast<float>(x[0]);
            y[1][s] = static_cast<float>(x[1]);
            ss[s] = fmaf(y[1][s], y[1][s], y[0][s] * y[0][s]);
        }
        share_factor<D>(const_cast<SM&>(sm),
                        __builtin_amdgcn_rsqf(fmaf(1.f / D, reduce_scatter8<Cfg<D>::CP>(ss), eps_norm)), rho);
    } else {
        conv_silu<D>(r, sm.wk, cgi, y, ss);
        // xi = -ln2 inv y',  mean xi^2 = ln^2 2 inv^2 ||y'||^2 / D, with inv the
        // reciprocal of ||y||^2 + eps (or of its square root for the unit-norm map)
        const float tot = reduce_scatter8<Cfg<D>::CP>(ss);
        const float den = fmaf(kLn2Sq, tot, eps_feat);
        const float inv = unit ? __builtin_amdgcn_rsqf(den) : __builtin_amdgcn_rcpf(den);
        const float rs = __builtin_amdgcn_rsqf(fmaf(kLn2Sq * (1.f / D) * inv * inv, tot, eps_norm));
        share_factor<D>(const_cast<SM&>(sm), -kLn2 * inv * rs, rho);
    }
    const float g0 = sm.gain[2 * cgi], g1 = sm.gain[2 * cgi + 1], b0 = sm.bias[2 * cgi], b1 = sm.bias[2 * cgi + 1];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        y[0][s] = fmaf(g0 * rho[s], y[0][s], b0);
        y[1][s] = fmaf(g1 * rho[s], y[1][s], b1);
    }
    if (n < L) mask_tokens(y, tb, n);
    write_zt(zT, cgi, tb, y);
}

// z_v of the thread's 8 tokens to z_v^T (zero past n valid tokens).
template <int D, class SM>
__device__ __forceinline__ void fm_values(const uint32_t (&r)[8], const SM& sm, const void* zT, int n, float eps_norm,
                                          int fi = feat_index<D>()) {
    if (fi >= Cfg<D>::NF) return;
    const int cgi = fi % Cfg<D>::CP, tb = fi / Cfg<D>::CP;
    float x[2][8], ss[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        x[0][s] = lo_bf16(r[s]);
        x[1][s] = hi_bf16(r[s]);
        ss[s] = fmaf(x[1][s], x[1][s], x[0][s] * x[0][s]);
    }
    float rs[8];
    share_factor<D>(const_cast<SM&>(sm), __builtin_amdgcn_rsqf(fmaf(1.f / D, reduce_scatter8<Cfg<D>::CP>(ss), eps_norm)),
                    rs);
    const float g0 = sm.gain[D + 2 * cgi], g1 = sm.gain[D + 2 * cgi + 1];
    const float b0 = sm.bias[D + 2 * cgi], b1 = sm.bias[D + 2 * cgi + 1];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        x[0][s] = fmaf(g0 * rs[s], x[0][s], b0);
        x[1][s] = fmaf(g1 * rs[s], x[1][s], b1);
    }
    if (n < L) mask_tokens(x, tb, n);
    write_zt(zT, cgi, tb, x);
}

// y' of the thread's 8 tokens, each token scaled by a power of two r_t with
// (r_t ||y'||)^2 in [1, 4) (so that the fp16 operand neither overflows nor
// loses precision, whatever the scale of q), kept as fp16 pairs until
// fm_write_q; the token's output factor omega_t to om.  With the scaled y'
// the mode scores are s~_t = K (S + abar^{t+1} Q) for one constant K, and
//   o_t = omega_t (P~ Z_v + Re X Gamma)_t,
//   omega_t = 4 Delta / (kappa r_t (ln^2 2 ||y'||^2 + eps))  (the root of the
// bracket for the unit-norm map); odt = 4 Delta / kappa.
// With pre (random Fourier features), slots 3..10 of r hold the features xi_q
// themselves as fp16 pairs, of norm one: they are the operand as they stand
// (r_t = 1), and omega_t = 1 / (K kappa^2) = -odt / ln 2 makes omega_t K xi_q =
// xi_q / kappa^2, what the scaled y' gives the SiLU maps.
template <int D, class SM>
__device__ __forceinline__ void fm_queries(half2v (&yo)[8], const uint32_t (&r)[11], SM& sm, float* om,
                                           float eps_feat, float odt, bool unit, bool pre, int fi = feat_index<D>()) {
    if (fi >= Cfg<D>::NF) return;
    const int cgi = fi % Cfg<D>::CP, tb = fi / Cfg<D>::CP;
    if (pre) {
#pragma unroll
        for (int s = 0; s < 8; ++s) yo[s] = __builtin_bit_cast(half2v, r[3 + s]);
        if (cgi < 8) om[8 * tb + scatter_token(cgi)] = -odt * (1.f / kLn2);
        return;
    }
    float y[2][8], ss[8], rs[8];
    conv_silu<D>(r, sm.wq, cgi, y, ss);
    const float tot = reduce_scatter8<Cfg<D>::CP>(ss);
    // tot in [2^e, 2^(e+1)): r_t = 2^-floor(e/2), 1/r_t = 2^floor(e/2) (tot = 0 gives r_t = 2^64)
    const int e = static_cast<int>((__float_as_uint(tot) >> 23) & 255u) - 127;
    const float rt = __uint_as_float(static_cast<uint32_t>(127 - (e >> 1)) << 23);
    const float inv_rt = __uint_as_float(static_cast<uint32_t>(127 + (e >> 1)) << 23);
    share_factor<D>(sm, rt, rs);
#pragma unroll
    for (int s = 0; s < 8; ++s)
        yo[s] = half2v{static_cast<_Float16>(y[0][s] * rs[s]), static_cast<_Float16>(y[1][s] * rs[s])};
    if (cgi < 8) {
        const float den = fmaf(kLn2Sq, tot, eps_feat);
        om[8 * tb + scatter_token(cgi)] = odt * inv_rt * (unit ? __builtin_amdgcn_rsqf(den) : __builtin_amdgcn_rcpf(den));
    }
}
template <int D>
__device__ __forceinline__ void fm_write_q(const half2v (&yo)[8], const void* yq, int fi = feat_index<D>()) {
    if (fi >= Cfg<D>::NF) return;
    const int cgi = fi % Cfg<D>::CP, tb = fi / Cfg<D>::CP;
    const uint32_t y0 = 2u * yq_off<D>(8 * tb, 2 * cgi);
#pragma unroll
    for (int s = 0; s < 8; ++s) *(lds_h2*)(uintptr_t)(lds_addr(yq) + (y0 ^ yq_sx<D>(s)) + s * kYqRow<D>) = yo[s];
}

// ------------------------------------------------------------------ random Fourier features
// Channel pair cp of the tokens TPT tg - 3 .. TPT tg + TPT - 1 of the 64-token
// tile at t0 of one (b, h) sequence (rs: a buffer resource over it, token
// stride rsb bytes; positions before 0 or past the end read zeros); at the
// start of the sequence the positions before it come from the stored tail
// (tl: that operand's [W-1][D] part of the (b, h) tail, or nullptr).
template <int D, int TPT>
__device__ __forceinline__ void rff_load_raw(uint32_t (&rv)[TPT + 3], __amdgpu_buffer_rsrc_t rs, int rsb,
                                             const uint16_t* __restrict__ tl, int W, int64_t t0, int cp, int tg) {
    const uint32_t lane_b = static_cast<uint32_t>(4 * cp + (TPT * tg - 3) * rsb);
#pragma unroll
    for (int s2 = 0; s2 < TPT + 3; ++s2)
        rv[s2] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane_b + static_cast<uint32_t>((t0 + s2) * rsb), 0, 0);
    if (t0 == 0 && TPT * tg < 3 && tl != nullptr) {
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
            const int pos = TPT * tg + s2 - 3;
            if (pos < 0 && pos >= -(W - 1)) rv[s2] = reinterpret_cast<const uint32_t*>(tl + ((W - 1) + pos) * D)[cp];
        }
    }
}

// xi_w(x) = [cos(w_f^T x), sin(w_f^T x)]_f / sqrt(F) of the conv output x, with
// F = D/2 frequencies per head (the columns of rff_omega[h], d x F), written
// for queries and keys as fp16 [B][N][H][D] (the token layout of q), from
// which the feature pass and the forward read them in place of conv + SiLU.
// Grid (ceil(N / (64 tpb)), B H), one wave per (token tile, frequency tile)
// of a 64-token tile (1024 threads for D = 128, 512 for D = 64); a block takes
// tpb 64-token tiles of one (b, h), one after another, with tpb chosen so
// that the blocks fill the chip about once (the Omega fragments are loaded
// once per block).  The phases are one [F x D] x [D x 64] product
// per operand and 64 tokens on the matrix cores, in fp16 with both factors
// split into high and low parts (three products: hi hi + hi lo + lo hi, fp32
// accumulation), which keeps the phase to about 2^-21 of its terms; cos and
// sin then take the phase in revolutions reduced to [-1/2, 1/2].  Each wave
// keeps the Omega^T fragments of its frequency tile in registers for the
// whole block; the features go through shared memory to 16-byte stores.
template <int D>
constexpr int kRffThreads = 4 * (D / 32) * 64;
template <int D>
__global__ __launch_bounds__(kRffThreads<D>) void rff_features_kernel(Problem p, idattn_params prm,
                                                                   const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ k,
                                                                   const uint16_t* __restrict__ tail_in,
                                                                   _Float16* __restrict__ xq,
                                                                   _Float16* __restrict__ xk, int tpb) {
    constexpr int NT = kRffThreads<D>;
    constexpr int F = D / 2;               // frequencies
    constexpr int KB = D / 32;             // K steps
    constexpr int AP = D + 8;              // row length (halfs) of the [t][channel] tiles: 16-byte
                                           // reads of 16 rows fall on 16 distinct groups of banks
    constexpr int NCP = D / 2;             // channel pairs
    constexpr int TG = NT / NCP;           // token groups
    constexpr int TPT = L / TG;            // tokens per thread
    __shared__ _Float16 ah[2][L * AP], al[2][L * AP];  // conv output [t][c], high and low parts (q, k)
    __shared__ _Float16 xo[2][L * AP];                 // features [t][f] on their way out (q, k)
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, g = ln >> 4, i = ln & 15;
    const int tw = wv & 3, fw = wv >> 2;   // token tile, frequency tile
    const int64_t bhi = blockIdx.y, b = bhi / p.H, h = bhi % p.H, H = p.H, N = p.N;
    const int W = static_cast<int>(p.W);
    // Omega^T fragments, rows f = 16 ft + i, K = 32 kb + 8 g + j
    half8 oh[KB], ol[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = 16 * fw + i, c = 32 * kb + 8 * g + j;
            const float x = prm.rff_omega[(h * D + c) * F + f];
            const _Float16 hi = static_cast<_Float16>(x);
            oh[kb][j] = hi;
            ol[kb][j] = static_cast<_Float16>(x - static_cast<float>(hi));
        }
    // conv taps of the thread's channel pair, right-aligned: tap j multiplies token t - 3 + j
    const int cp = tid % NCP, tg = tid / NCP;
    float wt[2][2][kMaxW];  // [q, k][channel 2 cp + e][tap]
#pragma unroll
    for (int j = 0; j < kMaxW; ++j) {
        const int tap = j - (kMaxW - W);
        const bool on = tap >= 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            wt[0][e][j] = on ? prm.conv_q[(h * D + 2 * cp + e) * W + tap] : 0.f;
            wt[1][e][j] = on ? prm.conv_k[(h * D + 2 * cp + e) * W + tap] : 0.f;
        }
    }
    const float inv_sqrt_f = 1.f / sqrtf(static_cast<float>(F));
    // the (b, h) tail: queries' part, then keys'
    const uint16_t* tlq = tail_in != nullptr ? tail_in + (b * H + h) * 2 * (W - 1) * D : nullptr;
    const uint16_t* tlk = tail_in != nullptr ? tlq + (W - 1) * D : nullptr;
    const int rsb = static_cast<int>(H * D * 2);  // token stride, bytes
    const __amdgpu_buffer_rsrc_t rq = seq_rsrc<D>(q, b * N, h, H, N), rk = seq_rsrc<D>(k, b * N, h, H, N);
    const __amdgpu_buffer_rsrc_t oq = seq_rsrc<D>(reinterpret_cast<const uint16_t*>(xq), b * N, h, H, N);
    const __amdgpu_buffer_rsrc_t ok = seq_rsrc<D>(reinterpret_cast<const uint16_t*>(xk), b * N, h, H, N);
    // tiles of 64 tokens, queries and keys together; the raw values of tile + 1 are
    // loaded while tile runs its products
    const int64_t tb0 = static_cast<int64_t>(blockIdx.x) * tpb * L;
    const int ntl = static_cast<int>(N - tb0 < static_cast<int64_t>(tpb) * L ? (N - tb0 + L - 1) / L : tpb);
    uint32_t rv[2][TPT + 3];
    rff_load_raw<D, TPT>(rv[0], rq, rsb, tlq, W, tb0, cp, tg);
    rff_load_raw<D, TPT>(rv[1], rk, rsb, tlk, W, tb0, cp, tg);
    for (int tl = 0; tl < ntl; ++tl) {
        const int64_t t0 = tb0 + static_cast<int64_t>(tl) * L;
        const int n = static_cast<int>(N - t0 < L ? N - t0 : L);
#pragma unroll
        for (int sel = 0; sel < 2; ++sel)
#pragma unroll
            for (int s2 = 0; s2 < TPT; ++s2) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int j = 0; j < kMaxW; ++j) {
                    a0 = fmaf(wt[sel][0][j], lo_bf16(rv[sel][s2 + j]), a0);
                    a1 = fmaf(wt[sel][1][j], hi_bf16(rv[sel][s2 + j]), a1);
                }
                const int t = TPT * tg + s2;
                const _Float16 h0 = static_cast<_Float16>(a0), h1 = static_cast<_Float16>(a1);
                *reinterpret_cast<half2v*>(&ah[sel][t * AP + 2 * cp]) = half2v{h0, h1};
                *reinterpret_cast<half2v*>(&al[sel][t * AP + 2 * cp]) = half2v{
                    static_cast<_Float16>(a0 - static_cast<float>(h0)), static_cast<_Float16>(a1 - static_cast<float>(h1))};
            }
        if (tl + 1 < ntl) {
            rff_load_raw<D, TPT>(rv[0], rq, rsb, tlq, W, t0 + L, cp, tg);
            rff_load_raw<D, TPT>(rv[1], rk, rsb, tlk, W, t0 + L, cp, tg);
        }
        lds_barrier();  // conv tiles written; the last tile's stores have read xo (the prefetch stays in flight)
        // phases of frequencies 16 fw + 4 g + jj and token 16 tw + i, queries then keys
#pragma unroll
        for (int sel = 0; sel < 2; ++sel) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int bo = (16 * tw + i) * AP + 32 * kb + 8 * g;
                const half8 c_h = rd8(lds_addr(ah[sel]) + 2 * bo), c_l = rd8(lds_addr(al[sel]) + 2 * bo);
                acc = mfma(oh[kb], c_h, acc);
                acc = mfma(oh[kb], c_l, acc);
                acc = mfma(ol[kb], c_h, acc);
            }
            float cs[4], sn[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float r = acc[jj] * 0.15915494309189535f;  // revolutions
                r -= rintf(r);
                cs[jj] = __builtin_amdgcn_cosf(r) * inv_sqrt_f;
                sn[jj] = __builtin_amdgcn_sinf(r) * inv_sqrt_f;
            }
            const int f0 = 16 * fw + 4 * g, row = (16 * tw + i) * AP;
            wr4(lds_addr(xo[sel]) + 2 * (row + f0), cs[0], cs[1], cs[2], cs[3]);
            wr4(lds_addr(xo[sel]) + 2 * (row + F + f0), sn[0], sn[1], sn[2], sn[3]);
        }
        lds_barrier();  // features staged; every wave is past its reads of the conv tiles
#pragma unroll
        for (int sel = 0; sel < 2; ++sel)
            for (int e = tid; e < L * (D / 8); e += NT) {
                const int t = e / (D / 8), ch = e % (D / 8);
                if (t < n)  // (the resource ends at the sequence's last token as well)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u4, rd8(lds_addr(xo[sel]) + 2 * (t * AP + 8 * ch))), sel == 0 ? oq : ok,
                        static_cast<uint32_t>((t0 + t) * rsb + 16 * ch), 0, 0);
            }
    }
}

// Conv weights (times -log2 e, taps right-aligned into 4 slots), gain, bias,
// and the stored tail of the sequence (positions -3..-1; zeros when absent).
template <int D, bool WITH_Q, int NT = NTH, class SM>
__device__ __forceinline__ void load_prologue(SM& sm, const idattn_params& prm, const uint16_t* tail_in, int64_t b,
                                              int64_t h, int64_t H, int W) {
    for (int e = threadIdx.x; e < 2 * D; e += NT) {
        sm.gain[e] = prm.gain[h * 2 * D + e];
        sm.bias[e] = prm.bias[h * 2 * D + e];
    }
    for (int e = threadIdx.x; e < D * kMaxW; e += NT) {
        const int c = e / kMaxW, j = e % kMaxW;
        const int tap = j - (kMaxW - W);
        if constexpr (WITH_Q) sm.wq[wt_index<D>(c, j)] = tap >= 0 ? -kLog2e * prm.conv_q[(h * D + c) * W + tap] : 0.f;
        sm.wk[wt_index<D>(c, j)] = tap >= 0 ? -kLog2e * prm.conv_k[(h * D + c) * W + tap] : 0.f;
    }
    for (int e = threadIdx.x; e < 2 * 3 * D; e += NT) {
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

template <int NT = NTH>
__device__ __forceinline__ void copy16(void* dst, const void* src, int bytes) {
    for (int e = threadIdx.x; e < bytes / 16; e += NT)
        reinterpret_cast<u4*>(dst)[e] = reinterpret_cast<const u4*>(src)[e];
}

// A [D][L] feature tile, global to registers to shared memory: thread x of a
// role (512 threads) moves the 16-byte pieces x, x + 512, ...
template <int D>
constexpr int kTilePieces = D * L * 2 / 16 / 512;
template <int D>
__device__ __forceinline__ void tile_load(u4 (&r)[kTilePieces<D>], const _Float16* src) {
    const int x = tid_now() & 511;
#pragma unroll
    for (int j = 0; j < kTilePieces<D>; ++j) r[j] = reinterpret_cast<const u4*>(src)[512 * j + x];
}
template <int D>
__device__ __forceinline__ void tile_store(const void* dst, const u4 (&r)[kTilePieces<D>]) {
    const int x = tid_now() & 511;
#pragma unroll
    for (int j = 0; j < kTilePieces<D>; ++j)
        *(__attribute__((address_space(3))) u4*)(uintptr_t)(lds_addr(dst) + 16 * (512 * j + x)) = r[j];
}
// ... and shared memory to global, with the same piece mapping.
template <int D>
__device__ __forceinline__ void tile_copy_out(const void* src, _Float16* dst) {
    const int x = tid_now() & 511;
    u4 r[kTilePieces<D>];
#pragma unroll
    for (int j = 0; j < kTilePieces<D>; ++j)
        r[j] = *(__attribute__((address_space(3))) u4*)(uintptr_t)(lds_addr(src) + 16 * (512 * j + x));
#pragma unroll
    for (int j = 0; j < kTilePieces<D>; ++j) reinterpret_cast<u4*>(dst)[512 * j + x] = r[j];
}

// The z^T tile of a ragged last chunk with its n = L - back valid tokens moved
// to columns back .. L-1 (columns 0 .. back-1 zero), from the stored tile in
// the shared-memory layout, by the 512 threads of one role.
template <int D>
__device__ __forceinline__ void shift_tile(const void* dst, const _Float16* src, int back) {
    const int x = tid_now() & 511;
    for (int e = x; e < D * L; e += 512) {
        const int r = e / L, j = e % L;
        const _Float16 val = j >= back ? src[o128(r, j - back)] : static_cast<_Float16>(0.f);
        *(__attribute__((address_space(3))) _Float16*)(uintptr_t)(lds_addr(dst) + 2 * o128(r, j)) = val;
    }
}

// The same for a tile already in shared memory, in two steps around a
// barrier: each of the role's 512 threads reads its elements of the shifted
// tile, then writes them.
template <int D>
__device__ __forceinline__ void shift_tile_read(_Float16 (&r)[D * L / 512], const void* buf, int back) {
    const int x = tid_now() & 511;
#pragma unroll
    for (int u = 0; u < D * L / 512; ++u) {
        const int e = x + 512 * u, row = e / L, j = e % L;
        r[u] = j >= back ? *(__attribute__((address_space(3))) const _Float16*)(uintptr_t)(lds_addr(buf) + 2 * o128(row, j - back))
                         : static_cast<_Float16>(0.f);
    }
}
template <int D>
__device__ __forceinline__ void shift_tile_write(const void* buf, const _Float16 (&r)[D * L / 512]) {
    const int x = tid_now() & 511;
#pragma unroll
    for (int u = 0; u < D * L / 512; ++u) {
        const int e = x + 512 * u, row = e / L, j = e % L;
        *(__attribute__((address_space(3))) _Float16*)(uintptr_t)(lds_addr(buf) + 2 * o128(row, j)) = r[u];
    }
}

// ------------------------------------------------------------------ state
// Key wave kw (0..7), lane (g, i):  U[rt][jj] = U_m[r],  r = 16rt + 4g + jj, m' = 16kw + i
// Value wave vw (0..D/16-1):        G[mt][jj] = Gamma_m[c], m' = 16mt + 4g + jj, c = 16vw + i
// Memory layout: float [M][2D][2] (complex), columns 0..D-1 hold U, D..2D-1 Gamma.
// Loads multiply by `scale` (zeros when src is NULL); stores multiply by `scale`.
template <int D>
__device__ __forceinline__ void u_load(f4 (&U)[Cfg<D>::RT], const float* src, int kw, float scale) {
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15, mp = 16 * kw + i;
#pragma unroll
    for (int rt = 0; rt < Cfg<D>::RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            U[rt][jj] = src ? scale * src[((mp >> 1) * 2 * D + 16 * rt + 4 * g + jj) * 2 + (mp & 1)] : 0.f;
}
template <int D>
__device__ __forceinline__ void g_load(f4 (&G)[8], const float* src, int vw, float scale) {
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15, c = 16 * vw + i;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int mp = 16 * mt + 4 * g + jj;
            G[mt][jj] = src ? scale * src[((mp >> 1) * 2 * D + D + c) * 2 + (mp & 1)] : 0.f;
        }
}
template <int D>
__device__ __forceinline__ void u_store(const f4 (&U)[Cfg<D>::RT], float* dst, int kw, float scale) {
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15, mp = 16 * kw + i;
#pragma unroll
    for (int rt = 0; rt < Cfg<D>::RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            dst[((mp >> 1) * 2 * D + 16 * rt + 4 * g + jj) * 2 + (mp & 1)] = scale * U[rt][jj];
}
template <int D>
__device__ __forceinline__ void g_store(const f4 (&G)[8], float* dst, int vw, float scale) {
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15, c = 16 * vw + i;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int m = 8 * mt + 2 * g + q;
            *reinterpret_cast<float2*>(dst + (static_cast<int64_t>(m) * 2 * D + D + c) * 2) =
                make_float2(scale * G[mt][2 * q], scale * G[mt][2 * q + 1]);
        }
}

// Segment end states and carries in the workspace are kept in lane order:
// each lane's accumulator tiles as consecutive float4s, [key wave][tile][lane]
// for U (D/16 tiles per wave, 128 D floats) followed by [value wave][tile][lane]
// for Gamma (8 tiles per value wave 0..D/16-1, 128 D floats), so that they are
// stored and loaded with coalesced 16-byte accesses.
template <int D>
__device__ __forceinline__ void u_load_lane(f4 (&U)[Cfg<D>::RT], const float* src, int kw) {
    const f4* s4 = reinterpret_cast<const f4*>(src) + (kw * Cfg<D>::RT) * 64 + (threadIdx.x & 63);
#pragma unroll
    for (int rt = 0; rt < Cfg<D>::RT; ++rt) U[rt] = s4[64 * rt];
}
template <int D>
__device__ __forceinline__ void u_store_lane(const f4 (&U)[Cfg<D>::RT], float* dst, int kw) {
    f4* d4 = reinterpret_cast<f4*>(dst) + (kw * Cfg<D>::RT) * 64 + (threadIdx.x & 63);
#pragma unroll
    for (int rt = 0; rt < Cfg<D>::RT; ++rt) d4[64 * rt] = U[rt];
}
template <int D>
__device__ __forceinline__ void g_load_lane(f4 (&G)[8], const float* src, int vw) {
    const f4* s4 = reinterpret_cast<const f4*>(src + 128 * D) + (vw * 8) * 64 + (threadIdx.x & 63);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) G[mt] = s4[64 * mt];
}
template <int D>
__device__ __forceinline__ void g_store_lane(const f4 (&G)[8], float* dst, int vw) {
    f4* d4 = reinterpret_cast<f4*>(dst + 128 * D) + (vw * 8) * 64 + (threadIdx.x & 63);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) d4[64 * mt] = G[mt];
}

// Carry chain folded into the forward (few segments): the state entering
// segment seg is C <- abar^Lseg C + E_j over the end states E_0..E_{seg-1} of
// the segments before it (each from a zero start, in lane order), C =
// state_in (or zero) at first.  A few tiles at a time, every E_j is loaded (address clamped to E_0
// past seg) before any is combined, so that the loads overlap; the combine of
// a j >= seg is discarded.  U: the real and imaginary rows of a mode sit in
// lanes i, i ^ 1; Gamma: in elements 2q, 2q + 1 of a lane.
template <int D, int TG>
__device__ __forceinline__ void u_fold(f4 (&U)[Cfg<D>::RT], const float* e0, int64_t estride, int seg,
                                       const float2* aseg, int kw) {
    constexpr int RT = Cfg<D>::RT;
    const int i = threadIdx.x & 15;
    const float2 a = aseg[(16 * kw + i) >> 1];
    const float as = (i & 1) ? a.y : -a.y;
#pragma unroll
    for (int rt = 0; rt < RT; rt += TG) {
        f4 E[kFoldMax - 1][TG];
#pragma unroll
        for (int j = 0; j < kFoldMax - 1; ++j)
#pragma unroll
            for (int r = 0; r < TG; ++r)
                E[j][r] = reinterpret_cast<const f4*>(e0 + (j < seg ? j : 0) * estride)[(kw * RT + rt + r) * 64 +
                                                                                        (threadIdx.x & 63)];
#pragma unroll
        for (int j = 0; j < kFoldMax - 1; ++j)
#pragma unroll
            for (int r = 0; r < TG; ++r)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float u = U[rt + r][jj];
                    const float n = fmaf(a.x, u, fmaf(dpp_mov<0xB1>(u), as, E[j][r][jj]));
                    U[rt + r][jj] = j < seg ? n : u;
                }
    }
}
template <int D, int TG>
__device__ __forceinline__ void g_fold(f4 (&G)[8], const float* e0, int64_t estride, int seg, const float2* aseg,
                                       int vw) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int mt = 0; mt < 8; mt += TG) {
        f4 E[kFoldMax - 1][TG];
#pragma unroll
        for (int j = 0; j < kFoldMax - 1; ++j)
#pragma unroll
            for (int r = 0; r < TG; ++r)
                E[j][r] = reinterpret_cast<const f4*>(e0 + (j < seg ? j : 0) * estride +
                                                      128 * D)[(vw * 8 + mt + r) * 64 + (threadIdx.x & 63)];
#pragma unroll
        for (int j = 0; j < kFoldMax - 1; ++j)
#pragma unroll
            for (int r = 0; r < TG; ++r)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float2 av = aseg[8 * (mt + r) + 2 * g + q];
                    const float gr = G[mt + r][2 * q], gi = G[mt + r][2 * q + 1];
                    const float nr = fmaf(av.x, gr, fmaf(-av.y, gi, E[j][r][2 * q]));
                    const float ni = fmaf(av.x, gi, fmaf(av.y, gr, E[j][r][2 * q + 1]));
                    G[mt + r][2 * q] = j < seg ? nr : gr;
                    G[mt + r][2 * q + 1] = j < seg ? ni : gi;
                }
    }
}

// Lane byte offset, within a swizzled [rows][64] tile, of the fragment read of
// row R0 + i at column chunk g (R0 any multiple of 16).  Column chunk 4kb + g
// is the same offset with bit 6 flipped: the swizzle XORs the low three chunk
// bits with a function of the row, which leaves bit 2 of the chunk alone.
__device__ __forceinline__ uint32_t frag_off(int ln) { return opaque(2u * o128(ln & 15, 8 * (ln >> 4))); }
__device__ __forceinline__ uint32_t frag_kb(uint32_t off, int kb) { return off ^ (64u * kb); }
// The same holds for the 256-byte rows of x256 (chunk 4kb + g XOR row % 16, kb < 4).
__device__ __forceinline__ uint32_t frag256_off(int ln) { return opaque(2u * x256(ln & 15, 8 * (ln >> 4))); }
constexpr bool frag_xor_ok() {
    for (int r = 0; r < 128; ++r)
        for (int g = 0; g < 4; ++g) {
            for (int kb = 0; kb < 2; ++kb)
                if (o128(r, 32 * kb + 8 * g) != (o128(r % 16, 8 * g) ^ (32 * kb)) + 64 * (r - r % 16)) return false;
            for (int kb = 0; kb < 4; ++kb)
                if (r < 64 && x256(r, 32 * kb + 8 * g) != (x256(r % 16, 8 * g) ^ (32 * kb)) + 128 * (r - r % 16))
                    return false;
        }
    return true;
}
static_assert(frag_xor_ok(), "fragment offsets of K block kb must be an XOR of bit 5 (in halfs)");

// U <- abar^L U + Z_k^T F  (the real and imaginary rows of a mode sit in lanes i, i ^ 1);
// the low parts of F^T follow the high parts at M2 L halfs.
template <int D>
__device__ __forceinline__ void key_update(f4 (&U)[Cfg<D>::RT], const float2* aL, int kw, const void* zkT,
                                           const void* ft, int ln) {
    constexpr int RT = Cfg<D>::RT;
    constexpr uint32_t dl = M2 * L * 2;
    const int i = ln & 15;
    const float2 a = aL[(16 * kw + i) >> 1];
    const float aLs = (i & 1) ? a.y : -a.y;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float u = U[rt][jj];
            U[rt][jj] = fmaf(a.x, u, dpp_mov<0xB1>(u) * aLs);
        }
    }
    const uint32_t off = frag_off(ln);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const uint32_t wb = lds_addr(zkT) + frag_kb(off, kb);
        const uint32_t fo = lds_addr(ft) + frag_kb(off, kb) + 2 * 64 * 16 * kw;  // F^T rows 16kw + i
        const half8 bF = rd8(fo), bFl = rd8(fo + dl);                // F[j][m'], j = 32kb + 8g + jj
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const half8 a8 = rd8(wb + 2048 * rt);  // z_k[j][r = 16rt + i]
            U[rt] = mfma(a8, bF, U[rt]);
            U[rt] = mfma(a8, bFl, U[rt]);
        }
    }
}

// Complex scaling of the two modes (real, imaginary rows) of an accumulator tile.
__device__ __forceinline__ void cscale(f4& x, const float4& a) {
    const float r0 = x[0], i0 = x[1], r1 = x[2], i1 = x[3];
    x[0] = a.x * r0 - a.y * i0;
    x[1] = a.x * i0 + a.y * r0;
    x[2] = a.z * r1 - a.w * i1;
    x[3] = a.z * i1 + a.w * r1;
}

// Gamma <- abar^L Gamma + F^T Z_v, with bZ[kb] = Z_v[32kb + 8g + jj][16vw + i]: one
// complex scaling and every fragment of F (for the feature pass, bound by VALU issue).
template <int D>
__device__ __forceinline__ void value_update_plain(f4 (&G)[8], const float2* aL, const half8 (&bZ)[2],
                                                   const void* ft, int ln) {
    const int g = ln >> 4;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) cscale(G[mt], *reinterpret_cast<const float4*>(&aL[8 * mt + 2 * g]));
    const uint32_t off = frag_off(ln);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const uint32_t wb = lds_addr(ft) + frag_kb(off, kb);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            G[mt] = mfma(rd8(wb + 2048 * mt), bZ[kb], G[mt]);
            G[mt] = mfma(rd8(wb + M2 * L * 2 + 2048 * mt), bZ[kb], G[mt]);
        }
    }
}
// The same for the forward, bound by shared-memory bandwidth there.  The first half of F is abar^(L/2) times the second (F[j] = bbar abar^{L-1-j}),
// so with F1 = F[L/2 .. L-1]:  Gamma <- abar^(L/2) (abar^(L/2) Gamma + F1^T Z_v0) + F1^T Z_v1,
// and each fragment of F1 (high and low parts) is read once for both halves:
// half the shared-memory reads of the plain update for one more complex scaling.
// `off` is the lane's fragment offset frag_off(ln), g = ln >> 4.
template <int D, int GRP = 2>
__device__ __forceinline__ void value_update(f4 (&G)[8], const float2* aH, const half8 (&bZ)[2], const void* ft,
                                             int g, uint32_t off) {
    const uint32_t wb = lds_addr(ft) + frag_kb(off, 1);
#pragma unroll
    for (int m0 = 0; m0 < 8; m0 += GRP) {
        half8 fh[GRP], fl[GRP];
        float4 a[GRP];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            fh[u] = rd8(wb + 2048 * (m0 + u));
            fl[u] = rd8(wb + M2 * L * 2 + 2048 * (m0 + u));
            a[u] = *reinterpret_cast<const float4*>(&aH[8 * (m0 + u) + 2 * g]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < GRP; ++u) {
                cscale(G[m0 + u], a[u]);
                G[m0 + u] = mfma(fh[u], bZ[kb], G[m0 + u]);
                G[m0 + u] = mfma(fl[u], bZ[kb], G[m0 + u]);
            }
    }
}

__device__ __forceinline__ void load_bz(half8 (&bZ)[2], int vw, const void* zvT, uint32_t off) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) bZ[kb] = rd8(lds_addr(zvT) + frag_kb(off, kb) + 2048 * vw);
}

// Causal 16 x 16 tiles (tt, kt), kt <= tt, of the G and P~ products: key wave
// kw takes tile kw of the list, and kw + 8 when that exists.
__device__ __forceinline__ int tile_tt(int q) { return q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3; }
__device__ __forceinline__ int tile_kt(int q) { return q - (tile_tt(q) * (tile_tt(q) + 1)) / 2; }

// ------------------------------------------------------------------ kernels
// Features of every chunk and segment end states from a zero start: grid
// B*H*S, block (bh, seg).  z_k^T and z_v^T of each chunk go to its tile in
// global memory (zt, two [D][L] fp16 tiles per chunk in the shared-memory
// layout, chunks numbered from the sequence start), from which the forward
// copies them; blocks of segments 0..S-2 also run the state updates, the last
// segment's blocks only build features.  z_k and z_v are double-buffered by
// chunk parity, so a chunk needs one barrier: at step c the key waves update U
// with the keys of chunk c and build those of c+1 into the other buffer, the
// value waves do the same for Gamma and the values.
template <int D>
__global__ __launch_bounds__(NTH) void segment_state_kernel(Problem p, idattn_params prm,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ tail_in,
                                                            const float* __restrict__ state_in,
                                                            uint8_t* __restrict__ tab, float* __restrict__ c0,
                                                            float* __restrict__ ws, _Float16* __restrict__ zt,
                                                            int64_t Lseg_dense, int S_dense, const float* eta_in,
                                                            float* eta_out, float2* __restrict__ c0eta,
                                                            const int32_t* __restrict__ plan) {
    __shared__ SmemSeg<D> sm;
    const Blk wk = block_work(p, plan, S_dense, Lseg_dense);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (wk.idle) return;
    if (plan != nullptr && blockIdx.x < plan[3] + p.H && blockIdx.x >= plan[3] && tid < MM) {
        // one block per head (the heads of the first last-segment sequence):
        // abar^{C L} of the head's modes, the carry across segments, by
        // repeated squaring of the fp64 abar (read by the carry kernel and the
        // forward, both later on the stream)
        const double4 z = reinterpret_cast<const double4*>(tab + wk.h * kTabBytes + kTabDz)[tid];
        double pr, pi;
        cpow_int(z.x, z.y, wk.Lseg, pr, pi);
        reinterpret_cast<float2*>(tab + wk.h * kTabBytes + kTabPwSeg)[tid] =
            make_float2(static_cast<float>(pr), static_cast<float>(pi));
    }
    if (wk.n == 0) {  // no tokens: eta passes through (the forward copies state and tail)
        if (p.eta && eta_out != nullptr && tid < MM) {
            const int64_t e = (wk.bh * MM + tid) * 2;
            const float r = eta_in ? eta_in[e] : 0.f, i = eta_in ? eta_in[e + 1] : 0.f;
            eta_out[e] = r;
            eta_out[e + 1] = i;
        }
        return;
    }
    const bool key = w < 8;
    const int64_t bh = wk.bh, b = wk.b, h = wk.h;
    const int seg = wk.seg, S = wk.S;
    const int64_t Lseg = wk.Lseg;
    const bool upd = seg + 1 < S;  // this segment's end state is needed
    const int64_t t_begin = seg * Lseg;
    const int64_t t_end = t_begin + Lseg < wk.n ? t_begin + Lseg : wk.n;
    const int nch = static_cast<int>((t_end - t_begin + L - 1) / L);
    const int n_last = static_cast<int>(t_end - t_begin - static_cast<int64_t>(nch - 1) * L);
    const uint8_t* th = tab + h * kTabBytes;
    load_prologue<D, false>(sm, prm, tail_in, b, h, p.H, static_cast<int>(p.W));
    copy16(sm.ft, th + kTabFT, M2 * L * 2);
    copy16(sm.ftl, th + kTabFTL, M2 * L * 2);
    if (tid < MM) sm.aL[tid] = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + tid];
    __syncthreads();
    float* dst = ws + (wk.st0 + seg) * MM * 2 * D * 2;  // this segment's end state (when upd)
    const int rsb = static_cast<int>(p.H * D * 2);  // token stride, bytes
    // z_k^T tile of chunk c of this segment (the forward builds z_v itself)
    _Float16* zseg = zt + (wk.tile0 + seg * (Lseg / L)) * D * L;
    // The state entering the sequence, times the table scale kappa, staged in
    // lane order for the forward (and the carry chain), which read only this
    // copy: state_in is read here, in a kernel that completes before any block
    // of the forward can write state_out, so the two may be one buffer.
    const bool stage = seg == 0 && state_in != nullptr;
    const float kap = reinterpret_cast<const float4*>(th + kTabHc)[0].z;
    if (p.eta && seg == 0 && tid < MM) {
        // the normaliser: eta_in staged for the forward, and eta_out = abar^N eta_in +
        // bbar sum_{j<N} abar^j in closed form (the same thread reads eta_in and
        // writes eta_out, so the two may be one buffer)
        const int m = tid;
        const double ein_r = eta_in ? eta_in[(bh * MM + m) * 2] : 0.0, ein_i = eta_in ? eta_in[(bh * MM + m) * 2 + 1] : 0.0;
        c0eta[bh * MM + m] = make_float2(static_cast<float>(ein_r), static_cast<float>(ein_i));
        if (eta_out != nullptr) {
            const double4 z = reinterpret_cast<const double4*>(th + kTabDz)[m];  // abar, bbar
            double ar, ai, gr, gi;
            cpow_int(z.x, z.y, wk.n, ar, ai);
            geo_from_pow(z.x, z.y, z.z, z.w, ar, ai, static_cast<double>(wk.n), gr, gi);
            eta_out[(bh * MM + m) * 2] = static_cast<float>(ar * ein_r - ai * ein_i + gr);
            eta_out[(bh * MM + m) * 2 + 1] = static_cast<float>(ar * ein_i + ai * ein_r + gi);
        }
    }
    const float* sin = stage ? state_in + bh * MM * 2 * D * 2 : nullptr;
    float* cst = c0 + bh * MM * 2 * D * 2;
    if (key) {
        const int kw = w;
        f4 U[Cfg<D>::RT];
        if (stage) {
            u_load<D>(U, sin, kw, kap);
            u_store_lane<D>(U, cst, kw);
        }
        u_load<D>(U, nullptr, kw, 1.f);
        const __amdgpu_buffer_rsrc_t rk = seq_rsrc<D>(k, wk.t0, h, p.H, t_end);
        uint32_t rkk[11];
        fm_load<D, true>(rkk, rk, rsb, t_begin);
        halo_fix<D>(rkk, sm, 1, t_begin);
        fm_keys<D>(rkk, sm, sm.zkT[0], nch > 1 ? L : n_last, p.eps_feat, p.eps_norm, p.unit_feat, p.rff_feat);
        if (nch > 1) fm_load<D, true>(rkk, rk, rsb, t_begin + L);
        lds_barrier();  // chunk 0 features
        for (int c = 0; c < nch; ++c) {
            const int64_t t0 = t_begin + static_cast<int64_t>(c) * L;
            tile_copy_out<D>(sm.zkT[c & 1], zseg + c * D * L);
            if (upd) key_update<D>(U, sm.aL, kw, sm.zkT[c & 1], sm.ft, tid_now() & 63);
            if (c + 1 < nch) {
                fm_keys<D>(rkk, sm, sm.zkT[(c + 1) & 1], c + 2 < nch ? L : n_last, p.eps_feat, p.eps_norm,
                           p.unit_feat, p.rff_feat);
                if (c + 2 < nch) {
                    step_fence();
                    fm_load<D, true>(rkk, rk, rsb, t0 + 2 * L);
                }
            }
            lds_barrier();
        }
        if (upd) u_store_lane<D>(U, dst, kw);
    } else {
        const int vw = w - 8;
        const bool own = upd && vw < D / 16;
        f4 G[8];
        if (stage && vw < D / 16) {
            g_load<D>(G, sin, vw, kap);
            g_store_lane<D>(G, cst, vw);
        }
        if (own) g_load<D>(G, nullptr, vw, 1.f);
        // the values' features are needed here only for the end state (upd)
        const __amdgpu_buffer_rsrc_t rv = seq_rsrc<D>(v, wk.t0, h, p.H, t_end);
        uint32_t rvv[8];
        if (upd) {
            fm_load<D, false>(rvv, rv, rsb, t_begin);
            fm_values<D>(rvv, sm, sm.zvT[0], nch > 1 ? L : n_last, p.eps_norm);
            if (nch > 1) fm_load<D, false>(rvv, rv, rsb, t_begin + L);
        }
        lds_barrier();  // chunk 0 features
        for (int c = 0; c < nch; ++c) {
            const int64_t t0 = t_begin + static_cast<int64_t>(c) * L;
            if (own) {
                const int ln = tid_now() & 63;
                half8 bZ[2];
                load_bz(bZ, vw, sm.zvT[c & 1], frag_off(ln));
                value_update_plain<D>(G, sm.aL, bZ, sm.ft, ln);
            }
            if (upd && c + 1 < nch) {
                fm_values<D>(rvv, sm, sm.zvT[(c + 1) & 1], c + 2 < nch ? L : n_last, p.eps_norm);
                if (c + 2 < nch) {
                    step_fence();
                    fm_load<D, false>(rvv, rv, rsb, t0 + 2 * L);
                }
            }
            lds_barrier();
        }
        if (own) g_store_lane<D>(G, dst, vw);
    }
}

// Carry chain over segments (states in lane order): ws[st0 + seg] <- the state
// entering segment seg + 1.  One complex state element per thread (four
// threads share the eight floats of a group: re / im of a U lane pair, or
// two modes of a Gamma lane), walking the segments with the end states of up
// to eight segments loaded before any of them is combined, so that the loads
// overlap instead of forming a chain of dependent round trips.  The state
// entering the sequence comes from the staged copy c0.  Dense batches: every
// (b, h) of S segments.  Packed batches: the (b, h) of the sequences in the
// plan's carry list (those with more segments than the forward folds), S_b
// segments each.  Grid-stride over the elements, so that the grid need not
// match the (device-side) length of the carry list.
constexpr int kCarryBlocks = 2048;
__global__ __launch_bounds__(256) void segment_carry_kernel(Problem p, bool has_state,
                                                            const float* __restrict__ c0,
                                                            const uint8_t* __restrict__ tab,
                                                            float* __restrict__ ws, int S_dense,
                                                            const int32_t* __restrict__ plan) {
    constexpr int kBatch = 8;
    const int D = static_cast<int>(p.d);
    const int64_t per = 128 * D;  // threads per (b, h): one complex element each
    const int64_t npairs = plan == nullptr ? p.B * p.H : static_cast<int64_t>(plan[2]) * p.H;
    const int64_t sst = 256 * D;  // floats per state
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < npairs * per;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t j = e / per;
        int64_t bh, st0;
        int S;
        if (plan == nullptr) {
            bh = j;
            S = S_dense;
            st0 = bh * (S - 1);
        } else {  // pair j of the carry list
            const int64_t B = p.B;
            const int64_t b = plan[kPlanHead + 6 * B + 1 + j / p.H], hh = j % p.H;
            bh = b * p.H + hh;
            S = plan[kPlanHead + 2 * B + b];
            st0 = p.H * static_cast<int64_t>(plan[kPlanHead + 4 * B + b]) + hh * (S - 1);
        }
        const int64_t h = bh % p.H;
        const int o = static_cast<int>((e % per) >> 2) * 8;  // float offset of the group of eight
        const int k = static_cast<int>(e & 3);
        int mode, pre, pim;  // mode, positions of re / im in the eight floats
        if (o < 128 * D) {   // U: [kw][rt][lane][jj], re in lane i, im in lane i + 1
            const int kw = o / (16 * D), ln = (o % 256) / 4;  // (16 D is a multiple of 256)
            mode = 8 * kw + (ln & 15) / 2;
            pre = k;
            pim = 4 + k;
        } else {  // Gamma: [vw][mt][lane][jj], (re, im) of modes m0, m0 + 1 in jj
            const int o2 = o - 128 * D, mt = (o2 % 2048) / 256, ln = (o2 % 256) / 4;
            mode = 8 * mt + 2 * (ln >> 4) + (k & 1);
            pre = 2 * k;
            pim = 2 * k + 1;
        }
        const float2 a = reinterpret_cast<const float2*>(tab + h * kTabBytes + kTabPwSeg)[mode];
        // the staged state_in (lane order, already times kappa) or zero
        float2 c = has_state ? make_float2(c0[bh * sst + o + pre], c0[bh * sst + o + pim]) : make_float2(0.f, 0.f);
        float* base = ws + st0 * sst + o;
        for (int s0 = 0; s0 + 1 < S; s0 += kBatch) {
            const int n = S - 1 - s0 < kBatch ? S - 1 - s0 : kBatch;
            float2 loc[kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj)
                if (jj < n) loc[jj] = make_float2(base[(s0 + jj) * sst + pre], base[(s0 + jj) * sst + pim]);
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj)
                if (jj < n) {
                    c = make_float2(a.x * c.x - a.y * c.y + loc[jj].x, a.x * c.y + a.y * c.x + loc[jj].y);
                    base[(s0 + jj) * sst + pre] = c.x;
                    base[(s0 + jj) * sst + pim] = c.y;
                }
        }
    }
}

// One causal tile (tt, kt) of P~'[t][k] = sum_m' s~[t][m'] T[k][m'] (lane (g, i) of the
// T operand holds k = 16 kt + 15 - i), un-skewed into P~[t][t - k].  K = m' in perm32
// order on both sides: s~ as stored, F^T rows 32kb + 4g + e and 32kb + 16 + 4g + e.
// The lane's shared-memory addresses of tile qt: T fragments (br0, br1), the
// un-skewed P~ row start (ps) and the tile row tt; the same for every chunk.
struct PTile {
    uint32_t br0, br1, ps;
    int tt;
};
template <class SM>
__device__ __forceinline__ PTile p_tile_prep(const SM& sm, int qt, int ln) {
    const int g = ln >> 4, i = ln & 15;
    const int tt = tile_tt(qt), kt = tile_kt(qt);
    return PTile{opaque(lds_addr(sm.ft) + 2 * o128(4 * g + (i >> 2), L - 16 - 16 * kt + 4 * (i & 3))),
                 opaque(lds_addr(sm.ft) + 2 * o128(16 + 4 * g + (i >> 2), L - 16 - 16 * kt + 4 * (i & 3))),
                 opaque(lds_addr(sm.pp) + 2 * ((16 * tt + 4 * g) * (RP + 1) - 16 * kt - 15 + i)), tt};
}
template <class SM>
__device__ __forceinline__ void p_tile_run(const SM& sm, const PTile& pt, uint32_t xoff) {
    constexpr uint32_t dl = M2 * L * 2;
    f4 accP = {};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const half8 a = rd8(lds_addr(sm.sc) + frag_kb(xoff, kb) + 2 * 16 * pt.tt * M2);
        accP = mfma(a, cat(rd4t(pt.br0 + 4096 * kb), rd4t(pt.br1 + 4096 * kb)), accP);
        accP = mfma(a, cat(rd4t(pt.br0 + 4096 * kb + dl), rd4t(pt.br1 + 4096 * kb + dl)), accP);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
        wr1(pt.ps + 2 * (RP + 1) * jj, accP[jj]);  // k > t lands in padding (see SmemFwd)
}
template <class SM>
__device__ __forceinline__ void p_tile(const SM& sm, int qt, int ln, uint32_t xoff) {
    p_tile_run(sm, p_tile_prep(sm, qt, ln), xoff);
}

// Full chunk loop of one segment: grid B*H*S, block (bh, seg).  z_k^T and
// z_v^T of every chunk come ready from the feature pass; the queries' features
// are built here.  The readout of a chunk runs one step behind its s~ and X,
// so that a step c = 0..nch needs two barriers:
//   1  key: queries' features (c+1, held); G tiles, Q^T = U Y^T, U update (c);
//           two P~ tiles (c-1)
//      value: z_v^T (c) to shared memory; the other P~ tiles, X Gamma, Gamma update (c-1)
//   2  key: S^T = T^T G'^T, s~, X (c); y' (c+1) to shared memory
//      value: z_k^T (c+1) to shared memory; P~ Z_v, output (c-1); Z_v fragments (c)
// Every shared tile is written in one phase and read in the next: y', z_k (c)
// read in 1 of step c, rewritten in 2; G' (c) written in 1, read in 2; s~, X
// (c) written in 2 of step c, read in 1 of step c+1; P~ (c-1) written in 1,
// read in 2 of step c; z_v (c) written in 1 and read in 2 of step c into
// registers that the readout of step c+1 uses.
// With ETA (the normalised readout o = Re sum s Gamma / Re sum s eta), the key
// waves also form each token's denominator from the fp32 scores before their
// fp16 rounding: eta_m(t) = abar^{t+1} eta_m(before the chunk) + Hsum_m(t), so
// den_t = Re sum_m s_m(t) eta_m(t) = omega_t kappa Re sum_m s~_m(t) eta_m(t); the
// token factor omega_t cancels in the ratio, so o_t = (P~ Z_v + Re X Gamma)_t /
// (kappa sum_m Re s~ eta).  eta needs no scan: its value at any position is a
// closed form of the staged eta_in (fp64 in the prologue).
template <int D, bool ETA>
__global__ __launch_bounds__(NTH) void chunked_forward_kernel(Problem p, idattn_params prm,
                                                              const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const uint16_t* __restrict__ qf,
                                                              const _Float16* __restrict__ zt, uint16_t* __restrict__ o,
                                                              const float* state_in, const uint16_t* tail_in,
                                                              float* state_out, uint16_t* tail_out,
                                                              const uint8_t* __restrict__ tab,
                                                              const float* __restrict__ c0,
                                                              const float* __restrict__ carry, int64_t Lseg_dense,
                                                              int S_dense, const float2* __restrict__ c0eta,
                                                              bool has_eta, const int32_t* __restrict__ plan) {
    constexpr int RT = Cfg<D>::RT, KB = Cfg<D>::KB, YR = Cfg<D>::YR;
    constexpr uint32_t dl = WinOff<D>::ftl - WinOff<D>::ft;
    __shared__ SmemFwd<D> sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool key = w < 8;
    const Blk wk = block_work(p, plan, S_dense, Lseg_dense);
    if (wk.idle) return;
    if (wk.n == 0) {
        copy_through_block<D>(p, wk, state_in, state_out, tail_in, tail_out);
        return;
    }
    const int64_t bh = wk.bh, b = wk.b, h = wk.h;
    const int seg = wk.seg, S = wk.S;
    const int64_t Lseg = wk.Lseg;
    const int64_t N = wk.n, H = p.H;  // N: tokens of this sequence
    const int64_t t_begin = seg * Lseg;
    const int64_t t_end = t_begin + Lseg < N ? t_begin + Lseg : N;
    const int nch = static_cast<int>((t_end - t_begin + L - 1) / L);
    const int n_last = static_cast<int>(t_end - t_begin - static_cast<int64_t>(nch - 1) * L);
    const uint8_t* th = tab + h * kTabBytes;
    // A ragged last chunk whose end state is stored: the loop skips its state
    // update and the epilogue runs it with the valid tokens at the end of the
    // chunk and the decay abar^n, so that every token keeps its own weight T[n-1-t]
    // (a zero-padded chunk followed by abar^-(L-n) would carry the weights of its
    // first tokens as tiny fp16 values and then amplify their rounding).
    const bool tail_fix = seg == S - 1 && n_last < L && state_out != nullptr;
    const float2* a_n = reinterpret_cast<const float2*>(th + kTabPw) + (n_last - 1) * MM;  // abar^n

    // only the first segment reads the stored tail (and writes the new one at its end)
    load_prologue<D, true>(sm, prm, seg == 0 ? tail_in : nullptr, b, h, H, static_cast<int>(p.W));
    copy16(sm.ft, th + kTabFT, M2 * L * 2);
    copy16(sm.ftl, th + kTabFTL, M2 * L * 2);
    if (tid < MM) sm.aL[tid] = reinterpret_cast<const float2*>(th + kTabPw)[(L - 1) * MM + tid];
    if (tid < MM) sm.aH[tid] = reinterpret_cast<const float2*>(th + kTabPw)[(L / 2 - 1) * MM + tid];
    for (int e = tid; e < 16 * MM; e += NTH) sm.pw[e / MM][e % MM] = reinterpret_cast<const float2*>(th + kTabPw)[e];
    for (int e = tid; e < L * RP * 2 / 16; e += NTH)
        reinterpret_cast<u4*>(sm.gp)[e] = reinterpret_cast<u4*>(sm.pp)[e] = u4{0u, 0u, 0u, 0u};
    // Delta, 1/Delta and the head's table scale kappa, 1/kappa: F and the states
    // carry kappa, undone by K and omega (both carry 1 / kappa) and on
    // the state's way in and out
    const float4 hc = reinterpret_cast<const float4*>(th + kTabHc)[0];
    const float inv_kap = hc.w, kap = hc.z;
    if (ETA && tid < MM) {
        const int m = tid;
        const double4 z = reinterpret_cast<const double4*>(th + kTabDz)[m];  // abar, bbar
        double ar, ai, gr, gi;
        cpow_int(z.x, z.y, t_begin, ar, ai);
        geo_from_pow(z.x, z.y, z.z, z.w, ar, ai, static_cast<double>(t_begin), gr, gi);
        const float2 e = has_eta ? c0eta[bh * MM + m] : make_float2(0.f, 0.f);
        sm.ec0[m] = make_float2(static_cast<float>(ar * e.x - ai * e.y + gr), static_cast<float>(ar * e.y + ai * e.x + gi));
        const float2* hs = reinterpret_cast<const float2*>(th + kTabHs);
        sm.hs15[m] = hs[15 * MM + m];
        sm.hsL[m] = hs[(L - 1) * MM + m];
    }
    (void)kap;
    const float odt = 4.f * hc.x * hc.w;        // 4 Delta / kappa, the output factor's constant part
    const float ks = -0.25f * kLn2 * hc.y * hc.w;  // K = -ln2 / (4 Delta kappa), the mode scores' scale
    const int rsb = static_cast<int>(H * D * 2);  // token stride, bytes
    // state entering the segment: state_in, the carry chain's output, or (fold)
    // state_in followed by the end states of the segments before this one.
    // This kernel never reads state_in itself: the feature pass has staged
    // kappa state_in in lane order (c0), so the last segment's block may write
    // state_out into the same buffer whatever the order in which blocks run.
    const int64_t sstride = MM * 2 * D * 2;  // floats per (b, h) state
    const float* sin = state_in ? c0 + bh * sstride : nullptr;
    const float* src = carry + (wk.st0 + (seg > 0 ? seg - 1 : 0)) * sstride;
    const float* e0 = carry + wk.st0 * sstride;
    const int64_t estride = sstride;
    const bool fold = S <= kFoldMax;  // else the carry kernel has run
    const int nfold = fold ? seg : 0;
    constexpr int kFoldTiles = D == 128 ? 4 : 2;  // tiles per round trip of the fold (register bound)
    const float2* aseg = reinterpret_cast<const float2*>(th + kTabPwSeg);
    constexpr int64_t tile2 = D * L;  // halfs per chunk: z_k^T
    const _Float16* zseg = zt + (wk.tile0 + seg * (Lseg / L)) * tile2;
    __syncthreads();

    if (key) {
        // ---------------- key waves
        const int kw = w;
        float4 hsi = {};  // Hsum(i) of the lane's two modes (normalised readout)
        if constexpr (ETA)
            hsi = reinterpret_cast<const float4*>(th + kTabHs)[((tid & 15) * MM + 8 * kw + 2 * ((tid & 63) >> 4)) / 2];
        f4 U[RT];
        // before the token loads, which are waited for first
        if (seg > 0 && !fold) {
            u_load_lane<D>(U, src, kw);
        } else {
            if (sin != nullptr) u_load_lane<D>(U, sin, kw);
            else u_load<D>(U, nullptr, kw, 1.f);
            if (nfold > 0) u_fold<D, kFoldTiles>(U, e0, estride, nfold, aseg, kw);
        }
        const __amdgpu_buffer_rsrc_t rq = seq_rsrc<D>(qf, wk.t0, h, H, t_end);  // raw q, or its features
        uint32_t rqq[11];  // raw queries of the chunk after the next
        fm_load<D, true>(rqq, rq, rsb, t_begin);
        halo_fix<D>(rqq, sm, 0, t_begin);
        {
            half2v yo[8];
            fm_queries<D>(yo, rqq, sm, sm.om[0], p.eps_feat, odt, p.unit_feat, p.rff_feat);
            fm_write_q<D>(yo, sm.yq);
        }
        if (nch > 1) fm_load<D, true>(rqq, rq, rsb, t_begin + L);
        lds_barrier();  // chunk 0 features
        for (int c = 0; c <= nch; ++c) {
            // ---- phase 1
            f4 accQ[4];
            if (c < nch) {
                // G tiles -> G'; Q^T = U Y^T (rows m' = 16kw + 4g + jj, columns t); U update
                const int ln = tid_now() & 63, g = ln >> 4, i = ln & 15;
                const uint32_t yoff = opaque(2u * yq_off<D>(i, 4 * g));  // y' row i, K block 0
#pragma unroll
                for (int slot = 0; slot < 2; ++slot) {
                    const int qt = kw + 8 * slot;
                    if (qt < 10) {
                        const int tt = tile_tt(qt), jt = tile_kt(qt);
                        // K in perm32 order on both sides: y' fragments as stored, z_k^T rows
                        // 32kb + 4g + e and 32kb + 16 + 4g + e through the transposing reads
                        const uint32_t br0 = opaque(lds_addr(sm.zkT) + 2 * o128(4 * g + (i >> 2), 16 * jt + 4 * (i & 3)));
                        const uint32_t br1 = opaque(lds_addr(sm.zkT) + 2 * o128(16 + 4 * g + (i >> 2), 16 * jt + 4 * (i & 3)));
                        f4 accG = {};
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            const uint32_t ar = lds_addr(sm.yq) + frag_kb(yoff, kb) + 2 * 16 * tt * YR;
                            accG = mfma(rd8(ar), cat(rd4t(br0 + 4096 * kb), rd4t(br1 + 4096 * kb)), accG);
                        }
                        const uint32_t gs = opaque(lds_addr(sm.gp) + 2 * ((16 * tt + 4 * g) * (RP - 1) + L - 1 + 16 * jt + i));
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            wr1(gs + 2 * (RP - 1) * jj, accG[jj]);  // j > t lands in padding
                    }
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) accQ[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const half8 aU = to_half8(U[2 * kb], U[2 * kb + 1]);
                    const uint32_t yb = lds_addr(sm.yq) + frag_kb(yoff, kb);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) accQ[tt] = mfma(aU, rd8(yb + 2 * 16 * tt * YR), accQ[tt]);
                }
                if (!(tail_fix && c == nch - 1)) key_update<D>(U, sm.aL, kw, sm.zkT, sm.ft, ln);
            }
            if (c >= 1 && (kw == 2 || kw == 3)) {
                const int ln = tid_now() & 63;
                p_tile(sm, kw + 6, ln, frag256_off(ln));  // P~ tiles 8, 9 of chunk c-1
            }
            lds_barrier();
            // ---- phase 2
            if (c < nch) {
                const int ln = tid_now() & 63, g = ln >> 4, i = ln & 15;
                // S^T = T^T G'^T (K order reversed: element jj <-> k = 32kb + 8g + 7 - jj),
                // s~ = K (S + abar^{t+1} Q), X = s~ abar^{t+1}
                f4 accS[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) accS[tt] = f4{0.f, 0.f, 0.f, 0.f};
                const uint32_t c_gp = opaque(lds_addr(sm.gp) + 2 * (i * RP + 24 - 8 * g));
                const uint32_t toff = opaque(2u * (o128(i, L - 8 - 8 * g) + 64 * 16 * kw));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint32_t ta = lds_addr(sm.ft) + frag_kb(toff, kb);
                    const half8 aT = rd8(ta), aTl = rd8(ta + dl);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        const half8 bg = rd8(c_gp + 2 * (16 * tt * RP + 32 * (1 - kb)));
                        accS[tt] = mfma(aT, bg, accS[tt]);
                        accS[tt] = mfma(aTl, bg, accS[tt]);
                    }
                }
                // abar^{i+1} and abar^16 of modes 8kw + 2g + qq
                const float4 e0 = *reinterpret_cast<const float4*>(&sm.pw[i][8 * kw + 2 * g]);
                const float4 e16 = *reinterpret_cast<const float4*>(&sm.pw[15][8 * kw + 2 * g]);
                float er[2] = {e0.x, e0.z}, ei[2] = {e0.y, e0.w};
                const float e16r[2] = {e16.x, e16.z}, e16i[2] = {e16.y, e16.w};
                // s~ and X: 8-byte stores at the perm32 position of m' = 16kw + 4g
                const uint32_t pst = opaque(2 * x256(i, perm32(16 * kw + 4 * g)));
                const uint32_t x_st = lds_addr(sm.xc) + pst, s_st = lds_addr(sm.sc) + pst;
                // normalised readout: eta_m(t) of tokens t = i, 16 + i, ..., modes 8kw + 2g + qq
                float etr[2] = {}, eti[2] = {}, h15r[2] = {}, h15i[2] = {}, dp[4] = {};
                if constexpr (ETA) {
                    const float4 c0v = *reinterpret_cast<const float4*>(&sm.ec0[8 * kw + 2 * g]);
                    const float4 h15 = *reinterpret_cast<const float4*>(&sm.hs15[8 * kw + 2 * g]);
                    const float c0r[2] = {c0v.x, c0v.z}, c0i[2] = {c0v.y, c0v.w};
                    const float hr[2] = {hsi.x, hsi.z}, hi[2] = {hsi.y, hsi.w};
                    h15r[0] = h15.x; h15i[0] = h15.y; h15r[1] = h15.z; h15i[1] = h15.w;
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        etr[qq] = er[qq] * c0r[qq] - ei[qq] * c0i[qq] + hr[qq];
                        eti[qq] = er[qq] * c0i[qq] + ei[qq] * c0r[qq] + hi[qq];
                    }
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const float sg = ks;
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
                        if constexpr (ETA) {
                            // Re(s~ eta) of this token, then eta 16 tokens on: abar^16 eta + Hsum(15)
                            dp[tt] = fmaf(sr, etr[qq], fmaf(-si, eti[qq], dp[tt]));
                            const float ar_ = e16r[qq] * etr[qq] - e16i[qq] * eti[qq] + h15r[qq];
                            eti[qq] = e16r[qq] * eti[qq] + e16i[qq] * etr[qq] + h15i[qq];
                            etr[qq] = ar_;
                        }
                    }
                    wr4(x_st + 2 * 16 * tt * M2, xv[0], xv[1], xv[2], xv[3]);
                    wr4(s_st + 2 * 16 * tt * M2, sv[0], sv[1], sv[2], sv[3]);
                }
                if constexpr (ETA) {
                    // sum over the four lane groups (the wave's 8 modes), one partial per
                    // token and key wave; then eta before the next chunk, abar^L eta + Hsum(L-1)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        float x = dp[tt];
                        const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                        x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
                        const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                        x = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
                        if (g == 0) sm.dpart[c & 1][16 * tt + i][kw] = x;
                    }
                    if (i == 0) {
#pragma unroll
                        for (int qq = 0; qq < 2; ++qq) {
                            const int m = 8 * kw + 2 * g + qq;
                            const float2 a = sm.aL[m], e = sm.ec0[m], hl = sm.hsL[m];
                            sm.ec0[m] = make_float2(a.x * e.x - a.y * e.y + hl.x, a.x * e.y + a.y * e.x + hl.y);
                        }
                    }
                }
            }
            if (c + 1 < nch) {
                // queries' features of chunk c+1, after the combine so that no accumulator
                // is live: y' to the tile (read in phase 1 of step c+1), omega to buffer
                // (c+1) mod 3 (last read in phase 2 of step c-1); the raw tokens of c+2 follow
                step_fence();
                half2v yo[8];
                fm_queries<D>(yo, rqq, sm, sm.om[(c + 1) % 3], p.eps_feat, odt, p.unit_feat, p.rff_feat);
                fm_write_q<D>(yo, sm.yq);
                if (c + 2 < nch) {
                    step_fence();
                    fm_load<D, true>(rqq, rq, rsb, t_begin + static_cast<int64_t>(c + 2) * L);
                }
            }
            lds_barrier();
        }
        if (tail_fix) {
            lds_barrier();
            shift_tile<D>(sm.zkT, zseg + (nch - 1) * tile2, L - n_last);
            lds_barrier();
            key_update<D>(U, a_n, kw, sm.zkT, sm.ft, tid_now() & 63);
        }
        if (seg == S - 1 && state_out != nullptr) u_store<D>(U, state_out + bh * MM * 2 * D * 2, kw, inv_kap);
    } else {
        // ---------------- value waves
        const int vw = w - 8;
        const bool own = vw < D / 16;  // owns a 16-column block of Gamma
        f4 G[8];
        if (own) {  // before the tile loads, which are waited for first
            if (seg > 0 && !fold) {
                g_load_lane<D>(G, src, vw);
            } else {
                if (sin != nullptr) g_load_lane<D>(G, sin, vw);
                else g_load<D>(G, nullptr, vw, 1.f);
                if (nfold > 0) g_fold<D, kFoldTiles>(G, e0, estride, nfold, aseg, vw);
            }
        }
        const __amdgpu_buffer_rsrc_t ob = seq_rsrc<D>(o, wk.t0, h, H, t_end);
        const __amdgpu_buffer_rsrc_t rv = seq_rsrc<D>(v, wk.t0, h, H, t_end);
        uint32_t rvv[8];        // raw v of the next chunk to enter
        u4 kr[kTilePieces<D>];  // z_k^T of the chunk after it
        tile_load<D>(kr, zseg);
        fm_load<D, false>(rvv, rv, rsb, t_begin);
        tile_store<D>(sm.zkT, kr);
        if (nch > 1) tile_load<D>(kr, zseg + tile2);
        // lane addresses of this wave's P~ tile and of the s~, X fragment reads, kept
        // across the chunk loop
        const PTile ptv = p_tile_prep(sm, vw, tid_now() & 63);
        const uint32_t xoff = frag256_off(tid_now() & 63);  // s~ and X rows i, K block 0
        const uint32_t foff = frag_off(tid_now() & 63);     // [rows][64] tile fragments (Z_v, F)
        const uint32_t c_pp = opaque(lds_addr(sm.pp) + 2 * ((tid_now() & 15) * RP + 8 * ((tid_now() & 63) >> 4)));
        lds_barrier();  // chunk 0 features
        half8 bZ[2];    // Z_v fragments of the chunk whose readout comes next
        for (int c = 0; c <= nch; ++c) {
            const int64_t t0 = t_begin + static_cast<int64_t>(c) * L;
            f4 accO[4];
            // ---- phase 1: z_v^T (c) from v; P~ tiles, X Gamma, Gamma update (c-1)
            if (c < nch) fm_values<D>(rvv, sm, sm.zvT, c + 1 < nch ? L : n_last, p.eps_norm);
            const int ln = tid_now() & 63;
            if (c >= 1) p_tile_run(sm, ptv, xoff);  // P~ tiles 0..7 of chunk c-1 (8, 9: key waves 2, 3)
            if (c >= 1 && own) {
                // o^T = Gamma_prev^T X^T (c-block vw: lane (g, i) of tile tt holds
                // o[16tt + i][16vw + 4g + jj], four consecutive channels of one token)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) accO[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const half8 bG = to_half8(G[2 * kb], G[2 * kb + 1]);
                    const uint32_t xb = lds_addr(sm.xc) + frag_kb(xoff, kb);  // perm32 positions
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) accO[tt] = mfma(bG, rd8(xb + 2 * 16 * tt * M2), accO[tt]);
                }
                // Gamma update with chunk c-1, once X Gamma has read the state before it
                if (!(tail_fix && c == nch)) value_update<D>(G, sm.aH, bZ, sm.ft, ln >> 4, foff);
            }
            lds_barrier();
            // ---- phase 2: z_k^T (c+1); o^T += Z_v^T P~^T, Delta o (c-1); Z_v fragments (c)
            if (c + 1 < nch) {
                tile_store<D>(sm.zkT, kr);  // read by the key waves in phase 1 of step c+1
                fm_load<D, false>(rvv, rv, rsb, t0 + L);
                if (c + 2 < nch) tile_load<D>(kr, zseg + (c + 2) * tile2);
            }
            const int ln2 = tid_now() & 63;
            if (c >= 1 && own) {
                const int64_t tp = t0 - L;  // first token of chunk c-1
                const int g = ln2 >> 4, i = ln2 & 15;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        accO[tt] = mfma(bZ[kb], rd8(c_pp + 2 * (16 * tt * RP + 32 * kb)), accO[tt]);
                const uint32_t olane = static_cast<uint32_t>(i * rsb + 2 * (16 * vw + 4 * g));
                const float* om = sm.om[(c - 1) % 3];  // chunk c-1, written in phase 1 of step c-2
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const uint32_t toff = static_cast<uint32_t>((tp + 16 * tt) * rsb);
                    float w;
                    if constexpr (ETA) {
                        // 1 / den_t from the key waves' partials of chunk c-1, in a fixed order
                        const float4 a = *reinterpret_cast<const float4*>(&sm.dpart[(c - 1) & 1][16 * tt + i][0]);
                        const float4 bq = *reinterpret_cast<const float4*>(&sm.dpart[(c - 1) & 1][16 * tt + i][4]);
                        w = 1.f / (kap * (((a.x + a.y) + (a.z + a.w)) + ((bq.x + bq.y) + (bq.z + bq.w))));
                    } else {
                        w = om[16 * tt + i];
                    }
                    const u2 pk = {pack_bf16(accO[tt][0] * w, accO[tt][1] * w), pack_bf16(accO[tt][2] * w, accO[tt][3] * w)};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, pk), ob, olane + toff, 0, 0);
                }
            }
            if (c < nch && own) load_bz(bZ, vw, sm.zvT, foff);
            lds_barrier();
        }
        if (tail_fix) {
            // z_v^T of the last chunk is still in shared memory: read it, then
            // write it back with the valid tokens moved to the end
            _Float16 zs[D * L / 512];
            shift_tile_read<D>(zs, sm.zvT, L - n_last);
            lds_barrier();
            shift_tile_write<D>(sm.zvT, zs);
            lds_barrier();
            if (own) {
                const int ln = tid_now() & 63;
                half8 bZl[2];
                load_bz(bZl, vw, sm.zvT, frag_off(ln));
                value_update_plain<D>(G, a_n, bZl, sm.ft, ln);
            }
        }
        if (own && seg == S - 1 && state_out != nullptr) g_store<D>(G, state_out + bh * MM * 2 * D * 2, vw, inv_kap);
    }
    if (seg == 0 && tail_out != nullptr) {
        // New conv tail: positions N-W+1 .. N-1 of q and k, where negative positions
        // come from the stored tail kept in shared memory since the prologue; tail_in
        // is not read again, so tail_out may be the same buffer.
        const int Wm1 = static_cast<int>(p.W) - 1, E = 2 * Wm1 * D;
        for (int e = tid; e < E; e += NTH) {
            const int sel = e / (Wm1 * D), t = (e / D) % Wm1, c = e % D;
            const int64_t pos = N - Wm1 + t;
            tail_out[bh * E + e] = pos < 0 ? sm.halo[sel][3 + pos][c]
                                           : (sel == 0 ? q : k)[((wk.t0 + pos) * H + h) * D + c];
        }
    }
}

// Makespan, in chunk times, of P (b, h) sequences of c chunks each cut into
// segments of C chunks (the last one r = c - (S - 1) C) on kCUs compute units
// with one workgroup each at a time, when the full segments are dispatched
// first and the last segments after them (block_work's order): every
// workgroup costs its chunks plus kBlockCost of fixed work (prologue, state
// load and store).  The dispatcher hands each next workgroup to the unit
// that frees first, so the full segments spread evenly and the last ones
// fill the lowest loads first.
constexpr int kCUs = 256;
constexpr double kBlockCost = 1.5;
double plan_makespan(int64_t P, int64_t c, int64_t C) {
    const int64_t S = (c + C - 1) / C, r = c - (S - 1) * C;
    const double a = static_cast<double>(C) + kBlockCost, b = static_cast<double>(r) + kBlockCost;
    const int64_t nf = P * (S - 1), q = nf / kCUs, rem = nf % kCUs;
    // loads: (kCUs - rem) units at q a, rem units at (q + 1) a; then P last segments
    double lvl[2] = {static_cast<double>(q) * a, static_cast<double>(q + 1) * a};
    int64_t cnt[2] = {kCUs - rem, rem};
    int64_t left = P;
    double top = rem > 0 ? lvl[1] : lvl[0];
    // water-fill: the units at the lowest level take one segment each; a level
    // that rises past the other one swaps roles with it
    while (left > 0) {
        const int lo = (cnt[0] > 0 && (cnt[1] == 0 || lvl[0] <= lvl[1])) ? 0 : 1;
        const int64_t t = cnt[lo] < left ? cnt[lo] : left;
        left -= t;
        const double nv = lvl[lo] + b;
        top = nv > top ? nv : top;
        if (t == cnt[lo]) {
            lvl[lo] = nv;  // the whole level moves up
        } else {           // part of it: those units join a new level above
            const int hi = 1 - lo;
            if (cnt[hi] == 0 || lvl[hi] == nv) {
                lvl[hi] = nv;
                cnt[hi] += t;
                cnt[lo] -= t;
            } else {
                // three distinct levels: the remaining units of lo are the lowest
                // and receive nothing more (left is 0 here, since t < cnt[lo])
                cnt[lo] -= t;
            }
        }
        if (cnt[0] == 0 && cnt[1] == 0) break;
    }
    return top;
}

// Segments of Lseg tokens per (b, h), S of them: the segment size (in chunks)
// that minimises plan_makespan over sizes from half to twice the even split
// P c / kCUs (at most 512 of them, evenly spaced), ties going to fewer
// segments.  Remembered for the last shape asked.
void plan_segments(const Problem& p, int& S, int64_t& Lseg) {
    const int64_t P = p.B * p.H;
    const int64_t c = (p.N + L - 1) / L;
    if (c <= 1) {
        S = 1;
        Lseg = L;
        return;
    }
    static thread_local int64_t memo_P = -1, memo_c = -1, memo_C = 1;
    int64_t best = c;
    if (P == memo_P && c == memo_c) {
        best = memo_C;
    } else {
        const int64_t even = (P * c + kCUs - 1) / kCUs;
        int64_t lo = even / 2 > 1 ? even / 2 : 1, hi = 2 * even < c ? 2 * even : c;
        if (lo > hi) lo = hi;
        const int64_t step = (hi - lo) / 512 + 1;
        double best_t = plan_makespan(P, c, c);
        for (int64_t C = hi; C >= lo; C -= step) {  // larger sizes first: ties keep fewer segments
            const double t = plan_makespan(P, c, C);
            if (t < best_t - 1e-9) {
                best_t = t;
                best = C;
            }
        }
        memo_P = P;
        memo_c = c;
        memo_C = best;
    }
    Lseg = best * L;
    S = static_cast<int>((c + best - 1) / best);
}

// Workspace: the packed plan (packed batches only) | per-head tables | the
// staged kappa state_in, [B H] states in lane order | the staged eta_in,
// [B H][M] complex | segment end states, S_b - 1 per (b, h) | fp16 key-feature
// tiles, one z_k^T per chunk slot | (random Fourier features) xi_q and xi_k,
// fp16 [B][N][H][D] each.
struct WsLayout {
    size_t plan, tab, c0, c0eta, seg, zt, rff, total;
};
WsLayout ws_layout_parts(const Problem& p, size_t plan_bytes, size_t end_states, size_t chunk_slots) {
    const size_t state = static_cast<size_t>(MM) * 2 * p.d * 2 * sizeof(float);
    const size_t pairs = static_cast<size_t>(p.B * p.H);
    WsLayout w;
    w.plan = 0;
    w.tab = ((plan_bytes + 255) / 256) * 256;
    w.c0 = w.tab + static_cast<size_t>(p.H) * kTabBytes;
    w.c0eta = w.c0 + pairs * state;
    w.seg = w.c0eta + ((pairs * MM * 8 + 255) / 256) * 256;
    w.zt = w.seg + end_states * state;
    w.rff = w.zt + chunk_slots * L * p.d * sizeof(_Float16);
    w.total = w.rff + (p.rff_feat ? 2 * static_cast<size_t>(p.B * p.N * p.H * p.d) * sizeof(_Float16) : 0);
    return w;
}
// Dense: S segments of Lseg tokens per (b, h).
WsLayout ws_layout(const Problem& p, int S, int64_t Lseg) {
    const size_t pairs = static_cast<size_t>(p.B * p.H);
    return ws_layout_parts(p, 0, static_cast<size_t>(S - 1) * pairs, pairs * S * static_cast<size_t>(Lseg / L));
}
// Packed (B sequences on p.N = T tokens): the plan's bounds on the end
// states (plan_blocks_max); the chunks, ceil(n_b / L) each, number at most
// min(T, (T + B (L - 1)) / L) per head.
WsLayout ws_layout_packed(const Problem& p) {
    int64_t chunks = (p.N + p.B * (L - 1)) / L;
    chunks = chunks < p.N ? chunks : p.N;
    return ws_layout_parts(p, static_cast<size_t>(plan_ints(p.B, p.H)) * 4, static_cast<size_t>(kPlanEndStates),
                           static_cast<size_t>(p.H * chunks));
}

// Dense (cu == nullptr): B sequences of N tokens, segments planned here.
// Packed (cu != nullptr, device table of p.B + 1 entries on p.N = T tokens):
// the plan is built on the device and the grids cover its largest size.
template <int D>
hipError_t launch(const Problem& p, const idattn_params& prm, const void* q, const void* k, const void* v, void* o,
                  const float* state_in, const void* tail_in, float* state_out, void* tail_out, void* workspace,
                  hipStream_t stream, const float* eta_in, float* eta_out, const int32_t* cu) {
    const bool packed = cu != nullptr;
    int S = 1;
    int64_t Lseg = L;
    const int64_t pairs = p.B * p.H;
    int64_t grid;
    WsLayout lay;
    if (packed) {
        lay = ws_layout_packed(p);
        grid = plan_blocks_max(p.B, p.H);
    } else {
        plan_segments(p, S, Lseg);
        lay = ws_layout(p, S, Lseg);
        grid = pairs * S;
    }
    const auto* q16 = static_cast<const uint16_t*>(q);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const auto* t16 = static_cast<const uint16_t*>(tail_in);
    uint8_t* base = static_cast<uint8_t*>(workspace);
    int32_t* plan = packed ? reinterpret_cast<int32_t*>(base + lay.plan) : nullptr;
    uint8_t* tab = base + lay.tab;
    float* c0 = reinterpret_cast<float*>(base + lay.c0);
    float2* c0eta = reinterpret_cast<float2*>(base + lay.c0eta);
    float* ws = reinterpret_cast<float*>(base + lay.seg);
    _Float16* zt = reinterpret_cast<_Float16*>(base + lay.zt);
    const uint16_t* qf = q16;  // the queries' and keys' feature sources
    const uint16_t* kf = k16;
    if (p.rff_feat) {  // dense batches only (chunked_packed_supported)
        _Float16* xq = reinterpret_cast<_Float16*>(base + lay.rff);
        _Float16* xk = xq + p.B * p.N * p.H * p.d;
        const int64_t tiles = (p.N + L - 1) / L;  // per (b, h)
        int64_t tpb = (tiles * pairs + 255) / 256;  // tiles per block: about one block per compute unit
        tpb = tpb < 1 ? 1 : tpb > tiles ? tiles : tpb;
        rff_features_kernel<D><<<dim3(static_cast<unsigned>((tiles + tpb - 1) / tpb), static_cast<unsigned>(pairs)),
                                 kRffThreads<D>, 0, stream>>>(p, prm, q16, k16, t16, xq, xk, static_cast<int>(tpb));
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
        qf = reinterpret_cast<const uint16_t*>(xq);
        kf = reinterpret_cast<const uint16_t*>(xk);
    }
    zoh_tables_kernel<<<dim3(static_cast<unsigned>(p.H), 17), kTabThreads, 0, stream>>>(p, prm, Lseg, tab, cu, plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    segment_state_kernel<D><<<dim3(static_cast<unsigned>(grid)), NTH, 0, stream>>>(
        p, prm, kf, v16, t16, state_in, tab, c0, ws, zt, Lseg, S, eta_in, eta_out, c0eta, plan);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the carry kernel: dense with more segments than the forward folds; packed
    // when some sequence may have that many (its list says which)
    const int64_t carry_pairs = packed ? (p.N / L >= kFoldMax ? carry_cap(p.H) * p.H : 0)
                                       : (S > kFoldMax ? pairs : 0);
    if (carry_pairs > 0) {
        const int64_t threads = carry_pairs * 128 * p.d;  // one complex element each
        int64_t blocks = (threads + 255) / 256;
        blocks = blocks < kCarryBlocks ? blocks : kCarryBlocks;
        segment_carry_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(p, state_in != nullptr, c0,
                                                                                     tab, ws, S, plan);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.eta)
        chunked_forward_kernel<D, true><<<dim3(static_cast<unsigned>(grid)), NTH, 0, stream>>>(
            p, prm, q16, k16, v16, qf, zt, static_cast<uint16_t*>(o), state_in, t16, state_out,
            static_cast<uint16_t*>(tail_out), tab, c0, ws, Lseg, S, c0eta, eta_in != nullptr, plan);
    else
        chunked_forward_kernel<D, false><<<dim3(static_cast<unsigned>(grid)), NTH, 0, stream>>>(
            p, prm, q16, k16, v16, qf, zt, static_cast<uint16_t*>(o), state_in, t16, state_out,
            static_cast<uint16_t*>(tail_out), tab, c0, ws, Lseg, S, c0eta, false, plan);
    return hipGetLastError();
}

}  // namespace
}  // namespace cws

bool chunked_supported(const Problem& p) {
    // M = 64 modes, d = R in {64, 128}, conv width up to 4; any feature map (random
    // Fourier features through a pre-pass)
    if (!(p.bf16 && p.M == 64 && (p.d == 64 || p.d == 128) && p.W >= 1 && p.W <= 4)) return false;
    // the kernels address one (b, h) sequence with 32-bit byte offsets
    return p.N * p.H * p.d * 2 < (int64_t{1} << 31);
}

size_t chunked_workspace_bytes(const Problem& p) {
    int S;
    int64_t Lseg;
    cws::plan_segments(p, S, Lseg);
    return cws::ws_layout(p, S, Lseg).total;
}

bool chunked_packed_supported(const Problem& p) {
    // the plan's int32 entries: block counts up to 256 + B H and token offsets up to T
    // (random Fourier features: dense batches only, their pre-pass has no plan)
    return chunked_supported(p) && !p.rff_feat && p.B * p.H <= (int64_t{1} << 22) && p.N < (int64_t{1} << 31);
}

size_t chunked_packed_workspace_bytes(const Problem& p) { return cws::ws_layout_packed(p).total; }

hipError_t launch_forward_chunked(const Problem& p, const idattn_params& prm, const void* q, const void* k,
                                  const void* v, void* o, const float* state_in, const void* tail_in,
                                  float* state_out, void* tail_out, void* workspace, hipStream_t stream,
                                  const float* eta_in, float* eta_out) {
    if (p.d == 128)
        return cws::launch<128>(p, prm, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, stream, eta_in,
                                eta_out, nullptr);
    return cws::launch<64>(p, prm, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, stream, eta_in,
                           eta_out, nullptr);
}

hipError_t launch_forward_chunked_packed(const Problem& p, const idattn_params& prm, const int32_t* cu_seqlens,
                                         const void* q, const void* k, const void* v, void* o, const float* state_in,
                                         const void* tail_in, float* state_out, void* tail_out, void* workspace,
                                         hipStream_t stream) {
    if (p.d == 128)
        return cws::launch<128>(p, prm, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, stream,
                                nullptr, nullptr, cu_seqlens);
    return cws::launch<64>(p, prm, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, stream, nullptr,
                           nullptr, cu_seqlens);
}

}  // namespace idattn

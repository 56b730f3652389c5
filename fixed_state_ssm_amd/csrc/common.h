// Device helpers shared by the HIP kernels of libidattn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idattn {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 I/O
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t idx) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    else return static_cast<const float*>(base)[idx];
}

// An element of an I/O tensor as loaded (bf16 bits in the low half, or fp32
// bits) is widened where it is used, so that a batch of loads can all be
// issued before the first wait.
template <bool BF16>
__device__ __forceinline__ float widen(uint32_t raw) {
    return __uint_as_float(BF16 ? raw << 16 : raw);
}

// Buffer loads from a wave-uniform base: a buffer resource over n_bytes at
// base, read at a per-lane byte offset voff plus a uniform byte offset soff, so
// a lane needs no 64-bit address arithmetic.  The hardware checks voff against
// n_bytes (a load past it returns zero); soff is not checked, so callers keep
// voff + soff inside the buffer themselves.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base, uint32_t n_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n_bytes), 0x00020000);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
// n elements of an I/O tensor from element offset off of base as a buffer
// resource, and one element of it, as loaded (see widen), at a per-lane byte
// offset.
template <bool BF16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t io_rsrc(const void* base, int64_t off, int n) {
    constexpr int kEB = BF16 ? 2 : 4;
    return rsrc_at(static_cast<const char*>(base) + off * kEB, static_cast<uint32_t>(n * kEB));
}
template <bool BF16>
__device__ __forceinline__ uint32_t buf_load_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    if constexpr (BF16) return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

// RJ (1, 2 or 4) adjacent floats in one buffer load, and RJ adjacent elements
// of an I/O tensor (bf16 in one 2-, 4- or 8-byte load, or fp32).
template <int RJ>
__device__ __forceinline__ void buf_load_run(float (&x)[RJ], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    static_assert(RJ == 1 || RJ == 2 || RJ == 4, "1, 2 or 4 elements");
    if constexpr (RJ == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(v[j]);
    } else if constexpr (RJ == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        x[0] = __uint_as_float(v[0]);
        x[1] = __uint_as_float(v[1]);
    } else {
        x[0] = buf_load(r, voff, soff);
    }
}
template <int RJ, bool BF16>
__device__ __forceinline__ void buf_load_io_run(float (&x)[RJ], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff) {
    if constexpr (BF16 && RJ == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            x[2 * j] = __uint_as_float(v[j] << 16);
            x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
        }
    } else if constexpr (BF16 && RJ == 2) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        x[0] = __uint_as_float(v << 16);
        x[1] = __uint_as_float(v & 0xffff0000u);
    } else if constexpr (BF16) {
        x[0] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)) << 16);
    } else {
        buf_load_run<RJ>(x, r, voff, soff);
    }
}

// The wave's index in its block, as a value the compiler knows to be uniform
// over the wave (so that what is derived from it stays in scalar registers).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)); }

// ------------------------------------------------------------------ conv rows
constexpr int kConvMax = 8;  // largest conv width W

// Where a conv tap of head h reads its input row: sequence position pos >= 0
// is token tok0 + pos of q and k ([T][H][d]); the W - 1 positions before the
// sequence come from its conv tail ([B H][2][W - 1][d], q rows then k rows)
// when one is given.  A tap that reads nothing (real false, or no row) gets
// the row of token fallback_tok, so that its loads stay in bounds and can be
// issued unconditionally, and ok false, so that the caller zeroes them.  All
// arguments are uniform over the wave, and so is the result.
struct ConvRow {
    const void* bq;
    const void* bk;
    int64_t rq, rk;  // element offsets of the rows in bq, bk
    bool ok;
};
__device__ __forceinline__ ConvRow conv_row(const void* q, const void* k, const void* tail, int64_t tok0,
                                            int64_t pos, int64_t fallback_tok, int64_t b, int64_t h, int64_t H,
                                            int d, int W, bool real) {
    ConvRow r;
    if (real && pos >= 0) {
        r.bq = q;
        r.bk = k;
        r.rq = r.rk = ((tok0 + pos) * H + h) * d;
        r.ok = true;
    } else if (real && tail != nullptr && pos >= -(W - 1)) {
        r.bq = r.bk = tail;
        r.rq = ((b * H + h) * 2 * (W - 1) + (W - 1 + pos)) * d;
        r.rk = r.rq + static_cast<int64_t>(W - 1) * d;
        r.ok = true;
    } else {
        r.bq = q;
        r.bk = k;
        r.rq = r.rk = (fallback_tok * H + h) * d;
        r.ok = false;
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ void store_io(void* base, int64_t idx, float x) {
    if constexpr (BF16) static_cast<uint16_t*>(base)[idx] = f32_to_bf16(x);
    else static_cast<float*>(base)[idx] = x;
}

// ------------------------------------------------------------------ sequences
// Tokens [start, start + len) of sequence b on a token axis of T tokens: b N ..
// b N + N - 1 when cu is NULL, else cu[b] .. cu[b+1] - 1 of a packed batch.
// The packed bounds are clamped into [0, T], so that any contents of cu keep
// every access in bounds (a malformed cu gives wrong results, never a fault).
__device__ __forceinline__ void seq_range(const int32_t* cu, int64_t N, int64_t T, int64_t b, int64_t& start,
                                          int64_t& len) {
    if (cu == nullptr) {
        start = b * N;
        len = N;
        return;
    }
    const int64_t s = min(max(static_cast<int64_t>(cu[b]), int64_t{0}), T);
    const int64_t e = min(max(static_cast<int64_t>(cu[b + 1]), s), T);
    start = s;
    len = e - s;
}

// The sequence of token t: t / N, or the last b in [0, B) with cu[b] <= t
// (binary search; ends in [0, B) whatever cu holds).
__device__ __forceinline__ int64_t seq_of_token(const int32_t* cu, int64_t N, int64_t B, int64_t t) {
    if (cu == nullptr) return t / N;
    int64_t lo = 0, hi = B - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(cu[mid]) <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------------------ barriers
// Workgroup barrier that waits only for this wave's LDS operations.  Unlike
// __syncthreads() it does not wait for outstanding global loads, so loads
// issued ahead of time (prefetch) stay in flight across it.  Use it only
// where no other wave reads global memory this wave wrote before it.
// It is also a scheduling fence: the compiler keeps every instruction on its
// side, which bounds how many registers one phase of a kernel can hold.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------ reductions
// Sums over the 64 lanes of a wave with low latency, for reductions on a
// serial path: lane swaps by DPP within rows of 16 (xor 1, xor 2, rotate by 4
// and 8), then across rows with v_permlane16_swap and v_permlane32_swap, with
// no trip through the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
// Reduce-scatter of 8 values over each half of a wave (lanes 0..31 and
// 32..63 on their own): on return lane l holds its half's total of value
// slot8(l & 31) = 4 b0 + 2 b1 + b2 (b_k bit k of l), so that lanes 0..7 of
// each half hold all eight.  Each of the first three steps pairs lanes that
// differ in one of bits 0..2, keeps the half of the values that the lane's bit
// selects and adds what the partner sends of that half; the last steps add the
// one remaining value across bit 3 (rotate by 8 in a row of 16, whose rotation
// by 4 has already paired bit 2) and across the two rows of the half.  About
// 24 instructions against 8 half_total's 72.
__device__ __forceinline__ int slot8(int lane) { return 4 * (lane & 1) + 2 * ((lane >> 1) & 1) + ((lane >> 2) & 1); }
__device__ __forceinline__ float half_reduce_scatter8(const float (&v)[8], int lane) {
    const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
    float u[4], w[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float send = b0 ? v[k] : v[k + 4], keep = b0 ? v[k + 4] : v[k];
        u[k] = keep + dpp_f<0xB1>(send);  // quad_perm [1,0,3,2]
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float send = b1 ? u[k] : u[k + 2], keep = b1 ? u[k + 2] : u[k];
        w[k] = keep + dpp_f<0x4E>(send);  // quad_perm [2,3,0,1]
    }
    float x = (b2 ? w[1] : w[0]) + dpp_f<0x124>(b2 ? w[0] : w[1]);  // row_ror:4
    x += dpp_f<0x128>(x);                                           // row_ror:8
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
// The total over each half of the wave; every lane gets its half's.
__device__ __forceinline__ float half_total(float x) {
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f<0x124>(x);  // row_ror:4
    x += dpp_f<0x128>(x);  // row_ror:8
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
// The total over the 64 lanes; every lane gets it.
__device__ __forceinline__ float wave_total(float x) {
    x = half_total(x);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ------------------------------------------------------------------ RFF
// Random Fourier features of one token-head held by one wave (Chinese
// rendering of the paper, section 3.1, eq. 6): with D = d/2 frequencies, the
// columns of om = Omega_h (row-major [d][D]),
// xi = [cos(Omega^T c), sin(Omega^T c)] / sqrt(D), cosine half first.
// Lane l holds the conv outputs of channels l + 64 j in cq[j], ck[j] (zero
// past d) and receives the features of the same channels.  Those need only
// the phase of frequency l mod D, so each lane forms one query and one key
// phase: every input is broadcast from its lane with readlane and multiplied
// by that lane's entry of the input's row of Omega (one coalesced row per
// input, shared by queries and keys).
template <int DJ>
__device__ __forceinline__ void rff_features(const float (&cq)[DJ], const float (&ck)[DJ],
                                             const float* __restrict__ om, int d, float (&yq)[DJ],
                                             float (&yk)[DJ]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int D = d >> 1;         // a power of two, at most 64
    const int f = lane & (D - 1);
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int n = min(d - kWave * j, kWave);  // inputs held in slot j: 0, 16, 32 or 64
        for (int l0 = 0; l0 < n; l0 += 16) {
            // sixteen rows of Omega in flight at once
            float w[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) w[u] = om[(kWave * j + l0 + u) * D + f];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                pq = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(cq[j]), l0 + u)), w[u], pq);
                pk = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ck[j]), l0 + u)), w[u], pk);
            }
        }
    }
    float sq, cs_q, sk, cs_k;
    sincosf(pq, &sq, &cs_q);
    sincosf(pk, &sk, &cs_k);
    const float sc = 1.f / sqrtf(static_cast<float>(D));
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int c = lane + kWave * j;
        const bool in = c < d, sn = c >= D;
        yq[j] = in ? (sn ? sq : cs_q) * sc : 0.f;
        yk[j] = in ? (sn ? sk : cs_k) * sc : 0.f;
    }
}

// ------------------------------------------------------------------ ZOH
// Zero-order hold of u' = lambda u + B z over a step Delta = exp(log_dt),
// evaluated in fp64:  abar = exp(Delta lambda),
// bbar = (exp(Delta lambda) - 1) / lambda * B, with exp(z) - 1 written as
// [expm1(x) cos y - 2 sin^2(y/2)] + i exp(x) sin y for z = x + iy so that a
// small |Delta lambda| does not cancel.  lambda == 0 gives bbar = Delta B.
struct Zoh {
    double ar, ai, br, bi;
};

__device__ inline Zoh zoh_mode(float log_dt, float lre, float lim, float bre, float bim) {
    const double dt = exp(static_cast<double>(log_dt));
    const double x = dt * lre, y = dt * lim;
    double sy, cy;
    sincos(y, &sy, &cy);
    const double ex = exp(x);
    const double sh = sin(0.5 * y);
    const double em1_re = expm1(x) * cy - 2.0 * sh * sh;
    const double em1_im = ex * sy;
    double qr, qi;  // (exp(z) - 1) / lambda
    const double l2 = static_cast<double>(lre) * lre + static_cast<double>(lim) * lim;
    if (l2 == 0.0) {
        qr = dt;
        qi = 0.0;
    } else {
        qr = (em1_re * lre + em1_im * lim) / l2;
        qi = (em1_im * lre - em1_re * lim) / l2;
    }
    Zoh z;
    z.ar = ex * cy;
    z.ai = ex * sy;
    z.br = qr * bre - qi * bim;
    z.bi = qr * bim + qi * bre;
    return z;
}

// The sequential scans multiply by abar_f = fl32(abar), which differs from abar by up to
// about 2^-24 relative; a state that is multiplied by it n times carries that
// error n-fold, some 1e-5 in the far terms of a mode with |abar| = 0.998 (a
// memory of about 500 tokens) and more in the n abar^(n-1) weights of the
// abar derivatives.  So every K tokens the scans multiply their states by
// (abar / abar_f)^K, as x + dk x with dk = (abar / abar_f)^K - 1 formed in
// fp64: no term then holds more than K roundings of abar.  K: a power of two.
constexpr int kFixTok = 32;  // the per-mode scans' K: every fourth batch of eight tokens
__device__ __forceinline__ float2 decay_fix(const Zoh& z, int K) {
    const double fr = static_cast<float>(z.ar), fi = static_cast<float>(z.ai);
    const double n = fr * fr + fi * fi;
    double rr = (z.ar * fr + z.ai * fi) / n, ri = (z.ai * fr - z.ar * fi) / n;  // abar / abar_f
    for (int k = 1; k < K; k <<= 1) {
        const double t = rr * rr - ri * ri;
        ri = 2.0 * rr * ri;
        rr = t;
    }
    return make_float2(static_cast<float>(rr - 1.0), static_cast<float>(ri));
}
// (1 + d) x for complex x = (xr, xi)
__device__ __forceinline__ void apply_fix(float2 d, float& xr, float& xi) {
    const float r = fmaf(d.x, xr, fmaf(-d.y, xi, xr));
    xi = fmaf(d.x, xi, fmaf(d.y, xr, xi));
    xr = r;
}

}  // namespace idattn

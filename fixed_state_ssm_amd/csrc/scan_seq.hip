// Sequential fp32 scans: the literal recurrence, one time step after another.
// This is the all-fp32 path (it keeps the per-step rounding of a plain fp32
// recurrence) and the reference the chunked path is compared with.
//
// ssm_key_scan_seq: one half-wave per (b, h, mode m), two modes per wave; lane
// l of a half owns the RJ adjacent channels RJ l .. RJ l + RJ - 1 of U_m.  Each
// step updates U_m(i) = abar U_m(i-1) + bbar z_k(i); the lanes' shares of
// s_m(i) = xi_q(i) . U_m(i) over the R channels are reduced eight tokens at a
// time with one reduce-scatter per quantity over the half, which serves both
// modes of the wave at once.  Each batch of eight tokens issues the next
// batch's loads before it is stepped (two register sets in turn).  With
// the normalised readout (ETA) the wave also carries the mode's normaliser
// eta_m(i) = abar eta_m(i-1) + bbar (over a full batch in closed form, from
// powers of abar formed in fp64) and writes Re(s_m(i) eta_m(i)), the mode's
// share of the denominator; it alone reads and writes eta_m, so eta may be
// updated in place.
//
// ssm_value_scan_readout_seq: one block of sixteen waves per (b, h, 64-channel
// group) and, with M >= 32, per half of the modes; wave w owns a contiguous
// sixteenth of the block's modes, lane l one channel, so Gamma_{m,c} stays in
// registers and o_i,c = Re sum_m s_m(i) Gamma_{m,c}(i) needs only a 16-way
// cross-wave sum through LDS, done once per block of 16 tokens.  The two
// halves' partial sums are added by a small combine kernel: B H d/64 alone
// is fewer blocks than compute units at the model shapes.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace idattn {

namespace {

constexpr int kTok = 8;  // tokens per batch of the key recurrence

// One batch of the key recurrence: the lane's shares of s for each token and,
// for a ragged batch with ETA, the normaliser stepped along (the same in every
// lane of a half); the lane keeps eta after its token ts in etr, eti.  A ragged batch
// steps only its first nt tokens.  A full batch leaves eta to the caller, which
// jumps it over the eight tokens in closed form.
template <int RJ, bool ETA, bool RAGGED>
__device__ __forceinline__ void key_seq_batch(int nt, int ts, float (&ur)[RJ], float (&ui)[RJ],
                                              const float (&xv)[kTok][RJ], const float (&zv)[kTok][RJ], float ar,
                                              float ai, float br, float bi, float (&spr)[kTok], float (&spi)[kTok],
                                              float& er, float& ei, float& etr, float& eti) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        float pr = 0.f, pi = 0.f;
        if (!RAGGED || t < nt) {
#pragma unroll
            for (int j = 0; j < RJ; ++j) {
                const float nr = fmaf(ar, ur[j], fmaf(-ai, ui[j], br * zv[t][j]));
                const float ni = fmaf(ar, ui[j], fmaf(ai, ur[j], bi * zv[t][j]));
                ur[j] = nr;
                ui[j] = ni;
                pr = fmaf(xv[t][j], nr, pr);
                pi = fmaf(xv[t][j], ni, pi);
            }
            if constexpr (ETA && RAGGED) {
                const float nr = fmaf(ar, er, fmaf(-ai, ei, br));
                const float ni = fmaf(ar, ei, fmaf(ai, er, bi));
                er = nr;
                ei = ni;
                etr = t == ts ? nr : etr;
                eti = t == ts ? ni : eti;
            }
        }
        spr[t] = pr;
        spi[t] = pi;
    }
}

template <int RJ, bool ETA>
__global__ __launch_bounds__(256) void key_scan_seq_kernel(Problem p, idattn_params prm,
                                                           const float* __restrict__ xi_q,
                                                           const float* __restrict__ z_k,
                                                           const float* state_in,
                                                           float2* __restrict__ s, float* state_out,
                                                           const float* eta_in, float* eta_out,
                                                           float* __restrict__ pden) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 31;  // the lane in its half
    const int64_t bh = blockIdx.x;
    const int64_t m0 = (static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6)) * 2;  // the wave's first mode
    const int64_t m = m0 + (lane >> 5);
    const int64_t M = p.M;
    const int d = static_cast<int>(p.d);
    if (m0 >= M) return;  // whole wave; no barriers in this kernel
    const bool mok = m < M;  // false for the second half of the last wave when M is odd
    const int64_t mc = mok ? m : M - 1;
    const int64_t h = bh % p.H;
    int64_t start, N;  // this sequence's tokens on the [T] axis
    seq_range(p.cu, p.N, p.T, bh / p.H, start, N);
    const Zoh z = zoh_mode(prm.log_dt[h], prm.A[(h * M + mc) * 2], prm.A[(h * M + mc) * 2 + 1],
                           prm.Bc[(h * M + mc) * 2], prm.Bc[(h * M + mc) * 2 + 1]);
    const float ar = static_cast<float>(z.ar), ai = static_cast<float>(z.ai);
    const float br = static_cast<float>(z.br), bi = static_cast<float>(z.bi);
    const float2 fix = decay_fix(z, kFixTok);

    float ur[RJ], ui[RJ];
    const int64_t st_row = ((bh * M + mc) * 2 * d) * 2;  // complex row m of [M][2d], U half first
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int r = RJ * li + j;
        ur[j] = ui[j] = 0.f;
        if (state_in != nullptr && mok && r < d) {
            ur[j] = state_in[st_row + 2 * r];
            ui[j] = state_in[st_row + 2 * r + 1];
        }
    }
    const int64_t row0 = h * p.T + start;  // workspace rows [H][T]
    float2* srow = s + row0 * M + mc;
    float er = 0.f, ei = 0.f;  // eta_m, the same in every lane of the half
    if (ETA && eta_in != nullptr) {
        er = eta_in[(bh * M + mc) * 2];
        ei = eta_in[(bh * M + mc) * 2 + 1];
    }
    const bool dfull = d == 32 * RJ;
    const int ts = slot8(li);  // the token whose totals this lane ends with
    // eta over a full batch in closed form, eta(i0 + k) = abar^(k+1) eta(i0 - 1)
    // + bbar sum_{j<=k} abar^j: (plr, pli), (qlr, qli) for k = ts (this lane's
    // token), (a8r, a8i), (q8r, q8i) for k = 7 (the next batch's start), in fp64
    float plr = 0.f, pli = 0.f, qlr = 0.f, qli = 0.f, a8r = 0.f, a8i = 0.f, q8r = 0.f, q8i = 0.f;
    if constexpr (ETA) {
        double pr = 1.0, pi = 0.0, sr = 0.0, si = 0.0;  // abar^k and sum_{j<k} abar^j
        for (int k = 0; k < kTok; ++k) {
            sr += pr;
            si += pi;
            const double nr = pr * z.ar - pi * z.ai, ni = pr * z.ai + pi * z.ar;
            pr = nr;
            pi = ni;
            const float br_k = static_cast<float>(z.br * sr - z.bi * si), bi_k = static_cast<float>(z.br * si + z.bi * sr);
            if (k == ts) {
                plr = static_cast<float>(pr);
                pli = static_cast<float>(pi);
                qlr = br_k;
                qli = bi_k;
            }
            if (k == kTok - 1) {
                a8r = static_cast<float>(pr);
                a8i = static_cast<float>(pi);
                q8r = br_k;
                q8i = bi_k;
            }
        }
    }
    const uint32_t coff = 4u * static_cast<uint32_t>(min(RJ * li, d - RJ));  // byte offset of the lane's channels
    // one batch's rows into x, z (tokens clamped below the batch's nt): the
    // lane's RJ adjacent channels in one buffer load per row
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
    auto step = [&](int64_t i0, float (&xv)[kTok][RJ], float (&zv)[kTok][RJ], float (&xn)[kTok][RJ],
                    float (&zn)[kTok][RJ]) {
        const int nt = static_cast<int>(min(N - i0, static_cast<int64_t>(kTok)));
        const int64_t j0 = i0 + kTok < N ? i0 + kTok : i0;
        fetch(j0, static_cast<int>(min(N - j0, static_cast<int64_t>(kTok))), xn, zn);
        float spr[kTok], spi[kTok];
        float etr = 0.f, eti = 0.f;
        if (nt == kTok && dfull) {
            key_seq_batch<RJ, ETA, false>(nt, ts, ur, ui, xv, zv, ar, ai, br, bi, spr, spi, er, ei, etr, eti);
            if constexpr (ETA) {
                etr = fmaf(plr, er, fmaf(-pli, ei, qlr));
                eti = fmaf(plr, ei, fmaf(pli, er, qli));
                const float nr = fmaf(a8r, er, fmaf(-a8i, ei, q8r));
                const float ni = fmaf(a8r, ei, fmaf(a8i, er, q8i));
                er = nr;
                ei = ni;
            }
        } else {  // a ragged batch zeroes what lies out of range
#pragma unroll
            for (int t = 0; t < kTok; ++t)
#pragma unroll
                for (int j = 0; j < RJ; ++j)
                    if (t >= nt || RJ * li + j >= d) xv[t][j] = zv[t][j] = 0.f;
            key_seq_batch<RJ, ETA, true>(nt, ts, ur, ui, xv, zv, ar, ai, br, bi, spr, spi, er, ei, etr, eti);
        }
        static_assert(kFixTok % kTok == 0, "the decay fix at a batch's end");
        if (nt == kTok && i0 % kFixTok == kFixTok - kTok) {  // uniform
#pragma unroll
            for (int j = 0; j < RJ; ++j) apply_fix(fix, ur[j], ui[j]);
        }
        static_assert(kTok == 8, "one reduce-scatter per kTok tokens");
        const float pr = half_reduce_scatter8(spr, lane), pi = half_reduce_scatter8(spi, lane);
        if (li < kTok && ts < nt && mok) {
            srow[(i0 + ts) * M] = make_float2(pr, pi);
            if constexpr (ETA) pden[(row0 + i0 + ts) * M + m] = fmaf(pr, etr, -pi * eti);
        }
    };
    float xa[kTok][RJ], za[kTok][RJ], xb[kTok][RJ], zb[kTok][RJ];  // two batches' rows, in turn
    if (N > 0) fetch(0, static_cast<int>(min(N, static_cast<int64_t>(kTok))), xa, za);
    for (int64_t i0 = 0; i0 < N; i0 += 2 * kTok) {
        step(i0, xa, za, xb, zb);
        if (i0 + kTok >= N) break;
        step(i0 + kTok, xb, zb, xa, za);
    }
    if (state_out != nullptr && mok) {
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int r = RJ * li + j;
            if (r < d) {
                state_out[st_row + 2 * r] = ur[j];
                state_out[st_row + 2 * r + 1] = ui[j];
            }
        }
    }
    if (ETA && eta_out != nullptr && li == 0 && mok) {
        eta_out[(bh * M + m) * 2] = er;
        eta_out[(bh * M + m) * 2 + 1] = ei;
    }
}

constexpr int kBlk = 16;  // tokens per LDS round of the value scan
constexpr int kVW = 16;   // waves per value-scan block: M / 16 modes each, four waves per SIMD

// Sum of x[0..kVW) in a fixed pairwise order (deterministic).
template <int K>
__device__ __forceinline__ float tree_sum(float (&x)[K]) {
#pragma unroll
    for (int step = 1; step < K; step *= 2)
#pragma unroll
        for (int i = 0; i + step < K; i += 2 * step) x[i] += x[i + step];
    return x[0];
}

// The value scan's inputs of one block of tokens go through LDS, one element
// of each per thread: s and, with ETA, the per-mode denominator shares
// (kBlk x M), and z_v (kBlk x 64 channels).  The next block's elements are
// loaded into registers while this block's tokens are stepped; two barriers
// per block.
constexpr int kStage = kVW * kWave;  // threads per block = staged elements per input
static_assert(kBlk * kWave == kStage, "one z_v element per thread");
static_assert(kBlk * 64 <= kStage, "one s element per thread for M <= 64");

struct SeqStage {
    float2 s;
    float z, pd;
};

// Thread e's elements of the block [i0, i0 + nt): s and pden of (token e / M,
// mode e % M), z_v of (token e / 64, channel 64 group + e % 64), at indices
// clamped into the block and below d.
template <bool ETA>
__device__ __forceinline__ SeqStage seq_fetch(int64_t row0, int64_t i0, int nt, int M, int d, int group,
                                              const float2* __restrict__ s, const float* __restrict__ z_v,
                                              const float* __restrict__ pden) {
    const int e = static_cast<int>(threadIdx.x);
    SeqStage r;
    const int64_t im = (row0 + i0 + min(e / M, nt - 1)) * M + e % M;
    r.s = s[im];
    r.pd = ETA ? pden[im] : 0.f;
    r.z = z_v[(row0 + i0 + min(e / kWave, nt - 1)) * d + min(group * kWave + e % kWave, d - 1)];
    return r;
}

// One block of kBlk tokens for the wave's MW modes: Gamma steps forward and
// the wave's share of o goes to red.  A ragged block steps only its first nt
// tokens.
template <int MW, bool RAGGED>
__device__ __forceinline__ void value_seq_block(int nt, const float2* s_row, const float* z_col,
                                                float (*red_t)[kWave], int lane, const float (&ar)[MW],
                                                const float (&ai)[MW], const float (&br)[MW], const float (&bi)[MW],
                                                float (&gr)[MW], float (&gi)[MW], int M) {
#pragma unroll
    for (int t = 0; t < kBlk; ++t) {
        if (RAGGED && t >= nt) continue;
        const float zz = z_col[t * kWave];
        float acc = 0.f;
#pragma unroll
        for (int mm = 0; mm < MW; ++mm) {
            const float2 sv = s_row[t * M + mm];
            const float nr = fmaf(ar[mm], gr[mm], fmaf(-ai[mm], gi[mm], br[mm] * zz));
            const float ni = fmaf(ar[mm], gi[mm], fmaf(ai[mm], gr[mm], bi[mm] * zz));
            gr[mm] = nr;
            gi[mm] = ni;
            acc = fmaf(sv.x, nr, fmaf(-sv.y, ni, acc));
        }
        red_t[t][lane] = acc;
    }
}

// ETA: o = numerator / denominator, the denominator summed over the modes
// from the key scan's per-mode shares pden [H][T][M].
// SPLIT: the modes are split over two blocks (blockIdx.z); split z writes its
// partial numerator to num0 or num1 ([H][T][d] fp32), and combine_seq_kernel
// forms o (and with the normalised readout sums the denominator itself, so a
// split block runs without ETA).
template <bool BF16, int MW, bool ETA, bool SPLIT>
__global__ __launch_bounds__(kStage) void value_scan_seq_kernel(Problem p, idattn_params prm,
                                                                const float2* __restrict__ s,
                                                                const float* __restrict__ z_v,
                                                                const float* state_in, void* __restrict__ o,
                                                                float* state_out, const float* __restrict__ pden,
                                                                float* __restrict__ num0, float* __restrict__ num1) {
    static_assert(!(ETA && SPLIT), "the combine kernel divides when the modes are split");
    __shared__ float2 s_blk[kStage];
    __shared__ float z_blk[kStage];
    __shared__ float p_blk[ETA ? kStage : 1];
    __shared__ float red[kVW][kBlk][kWave];
    __shared__ float den_s[kVW][kBlk];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t H = p.H;
    const int M = static_cast<int>(p.M), d = static_cast<int>(p.d);
    const int group = static_cast<int>(blockIdx.y);
    const int c = group * kWave + lane;
    int64_t start, N;  // this sequence's tokens on the [T] axis
    seq_range(p.cu, p.N, p.T, b, start, N);
    const int64_t row0 = h * p.T + start;  // workspace rows [H][T]
    const bool cok = c < d;
    const int moff = SPLIT ? static_cast<int>(blockIdx.z) * kVW * MW : 0;  // the split's first mode
    float* num = blockIdx.z == 0 ? num0 : num1;

    float ar[MW], ai[MW], br[MW], bi[MW], gr[MW], gi[MW];
    float2 fix[MW];  // the decay fix of a full block (kBlk steps by abar_f)
#pragma unroll
    for (int mm = 0; mm < MW; ++mm) {
        const int64_t m = moff + w * MW + mm;
        const Zoh z = zoh_mode(prm.log_dt[h], prm.A[(h * M + m) * 2], prm.A[(h * M + m) * 2 + 1],
                               prm.Bc[(h * M + m) * 2], prm.Bc[(h * M + m) * 2 + 1]);
        fix[mm] = decay_fix(z, kBlk);
        ar[mm] = static_cast<float>(z.ar);
        ai[mm] = static_cast<float>(z.ai);
        br[mm] = static_cast<float>(z.br);
        bi[mm] = static_cast<float>(z.bi);
        gr[mm] = gi[mm] = 0.f;
        if (state_in != nullptr && cok) {
            const int64_t idx = ((bh * M + m) * 2 * d + d + c) * 2;
            gr[mm] = state_in[idx];
            gi[mm] = state_in[idx + 1];
        }
    }
    if (N > 0) {  // uniform over the block
        const float2* s_row = s_blk + moff + w * MW;
        const float* p_row = p_blk + (ETA ? moff + w * MW : 0);
        int64_t i0 = 0;
        int nt = static_cast<int>(min(N, static_cast<int64_t>(kBlk)));
        SeqStage nx = seq_fetch<ETA>(row0, i0, nt, M, d, group, s, z_v, pden);
        while (i0 < N) {
            {
                const int e = static_cast<int>(threadIdx.x);
                const bool mok = e < nt * M;
                s_blk[e] = mok ? nx.s : make_float2(0.f, 0.f);
                if constexpr (ETA) p_blk[e] = mok ? nx.pd : 0.f;
                z_blk[e] = (e / kWave < nt && group * kWave + e % kWave < d) ? nx.z : 0.f;
            }
            __syncthreads();
            const int64_t j0 = i0 + kBlk;  // the next block, loaded while this one runs
            const int jnt = static_cast<int>(min(N - j0, static_cast<int64_t>(kBlk)));
            if (j0 < N) nx = seq_fetch<ETA>(row0, j0, jnt, M, d, group, s, z_v, pden);
            if constexpr (ETA) {  // the wave's share of the denominator, lane t for token t
                if (lane < nt) {
                    float dn = 0.f;
#pragma unroll
                    for (int mm = 0; mm < MW; ++mm) dn += p_row[lane * M + mm];
                    den_s[w][lane] = dn;
                }
            }
            if (nt == kBlk) {
                value_seq_block<MW, false>(nt, s_row, z_blk + lane, red[w], lane, ar, ai, br, bi, gr, gi, M);
#pragma unroll
                for (int mm = 0; mm < MW; ++mm) apply_fix(fix[mm], gr[mm], gi[mm]);
            } else
                value_seq_block<MW, true>(nt, s_row, z_blk + lane, red[w], lane, ar, ai, br, bi, gr, gi, M);
            __syncthreads();
            for (int e = threadIdx.x; e < nt * kWave; e += kStage) {
                const int t = e / kWave, l = e % kWave;
                const int cc = group * kWave + l;
                if (cc < d) {
                    // fixed pairwise order over the waves' partial sums
                    float part[kVW];
#pragma unroll
                    for (int i = 0; i < kVW; ++i) part[i] = red[i][t][l];
                    float sum = tree_sum(part);
                    if constexpr (SPLIT) {
                        num[(row0 + i0 + t) * d + cc] = sum;
                    } else {
                        if constexpr (ETA) {
#pragma unroll
                            for (int i = 0; i < kVW; ++i) part[i] = den_s[i][t];
                            sum /= tree_sum(part);
                        }
                        store_io<BF16>(o, ((start + i0 + t) * H + h) * d + cc, sum);
                    }
                }
            }
            i0 = j0;
            nt = jnt;
        }
    }
    if (state_out != nullptr && cok) {
#pragma unroll
        for (int mm = 0; mm < MW; ++mm) {
            const int64_t idx = ((bh * M + moff + w * MW + mm) * 2 * d + d + c) * 2;
            state_out[idx] = gr[mm];
            state_out[idx + 1] = gi[mm];
        }
    }
}

// o [T][H][d] from the two splits' partial numerators: o = num0 + num1, or
// with ETA (num0 + num1) / den, den = sum_m pden[h][t][m].  A thread takes four
// adjacent channels (d is 16, 32, 64 or 128: dq_shift = log2(d / 4)), and the
// (token, head) of a row comes from 32-bit index arithmetic when T H fits in
// 32 bits (TH32).  A row's d / 4 threads are adjacent lanes of one wave: each
// sums every (d/4)-th mode share from its own, then the lanes add theirs in a
// fixed butterfly order.
template <bool BF16, bool ETA, bool TH32>
__global__ __launch_bounds__(256) void combine_seq_kernel(Problem p, const float* __restrict__ num0,
                                                          const float* __restrict__ num1,
                                                          const float* __restrict__ pden, void* __restrict__ o,
                                                          int dq_shift) {
    const int64_t H = p.H, T = p.T, d = p.d;
    const int M = static_cast<int>(p.M), dq = 1 << dq_shift;
    const int64_t nq = (T * H) << dq_shift;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < nq;
         q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t th = q >> dq_shift;  // o's row, t H + h
        const int64_t c = (q & ((int64_t{1} << dq_shift) - 1)) * 4;
        int64_t h, t;
        if constexpr (TH32) {
            const uint32_t th32 = static_cast<uint32_t>(th), H32 = static_cast<uint32_t>(H);
            t = th32 / H32;
            h = th32 - static_cast<uint32_t>(t) * H32;
        } else {
            t = th / H;
            h = th - t * H;
        }
        const int64_t w = (h * T + t) * d + c;  // the partials are [H][T][d]
        const float4 a = *reinterpret_cast<const float4*>(num0 + w), b = *reinterpret_cast<const float4*>(num1 + w);
        float x[4] = {a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
        if constexpr (ETA) {
            const float* pr = pden + (h * T + t) * M;
            float den = 0.f;
            for (int m = static_cast<int>(c >> 2); m < M; m += dq) den += pr[m];
            for (int off = 1; off < dq; off <<= 1) den += __shfl_xor(den, off, kWave);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] /= den;
        }
        const int64_t e = th * d + c;
        if constexpr (BF16) {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + e) =
                make_uint2(f32_to_bf16(x[0]) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16),
                           f32_to_bf16(x[2]) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16));
        } else {
            *reinterpret_cast<float4*>(static_cast<float*>(o) + e) = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
}

}  // namespace

hipError_t launch_ssm_key_scan_seq(const Problem& p, const idattn_params& prm, const float* xi_q,
                                   const float* z_k, const float* state_in, float* s,
                                   float* state_out, const float* eta_in, float* eta_out, float* pden,
                                   hipStream_t stream) {
    // two modes per wave, four waves per block
    const dim3 grid(static_cast<unsigned>(p.B * p.H), static_cast<unsigned>((p.M + 7) / 8));
    float2* s2 = reinterpret_cast<float2*>(s);
#define IDATTN_KSCAN(RJ, ETA) \
    key_scan_seq_kernel<RJ, ETA><<<grid, 256, 0, stream>>>(p, prm, xi_q, z_k, state_in, s2, state_out, eta_in, eta_out, pden)
#define IDATTN_KSCAN_D(ETA)                     \
    do {                                        \
        if (p.d > 64) IDATTN_KSCAN(4, ETA);     \
        else if (p.d > 32) IDATTN_KSCAN(2, ETA); \
        else IDATTN_KSCAN(1, ETA);              \
    } while (0)
    if (pden != nullptr) IDATTN_KSCAN_D(true);
    else IDATTN_KSCAN_D(false);
#undef IDATTN_KSCAN_D
#undef IDATTN_KSCAN
    return hipGetLastError();
}

hipError_t launch_ssm_value_scan_readout_seq(const Problem& p, const idattn_params& prm,
                                             const float* s, const float* z_v,
                                             const float* state_in, void* o, float* state_out,
                                             const float* pden, float* num0, float* num1,
                                             hipStream_t stream) {
    // two mode splits when each still gets at least one mode per wave
    const int splits = p.M >= 2 * kVW ? 2 : 1;
    const dim3 grid(static_cast<unsigned>(p.B * p.H), static_cast<unsigned>((p.d + kWave - 1) / kWave),
                    static_cast<unsigned>(splits));
    const float2* s2 = reinterpret_cast<const float2*>(s);
#define IDATTN_VSCAN_K(BF, MW, ETA, SPLIT) \
    value_scan_seq_kernel<BF, MW, ETA, SPLIT><<<grid, kStage, 0, stream>>>(p, prm, s2, z_v, state_in, o, state_out, pden, num0, num1)
#define IDATTN_VSCAN_E(MW, ETA, SPLIT)                  \
    do {                                                \
        if (p.bf16) IDATTN_VSCAN_K(true, MW, ETA, SPLIT); \
        else IDATTN_VSCAN_K(false, MW, ETA, SPLIT);       \
    } while (0)
// split blocks leave the division to the combine kernel
#define IDATTN_VSCAN(MW, SPLIT)                                     \
    do {                                                            \
        if (!(SPLIT) && pden != nullptr) IDATTN_VSCAN_E(MW, true, false); \
        else IDATTN_VSCAN_E(MW, false, SPLIT);                      \
    } while (0)
    switch (p.M / (kVW * splits)) {
        case 1:
            if (splits == 2) IDATTN_VSCAN(1, true);
            else IDATTN_VSCAN(1, false);
            break;
        case 2: IDATTN_VSCAN(2, true); break;
        default: return hipErrorInvalidValue;
    }
#undef IDATTN_VSCAN
#undef IDATTN_VSCAN_E
#undef IDATTN_VSCAN_K
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t nq = p.T * p.H * (p.d / 4);  // d is 16, 32, 64 or 128
    if (nq == 0) return hipSuccess;
    if (p.d % 4 != 0 || (p.d & (p.d - 1)) != 0) return hipErrorInvalidValue;
    const int dq_shift = __builtin_ctzll(static_cast<unsigned long long>(p.d / 4));
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((nq + 255) / 256, 4096));
    const bool th32 = p.T * p.H <= int64_t{0xffffffff};
#define IDATTN_COMB(BF, ETA)                                                                                  \
    do {                                                                                                      \
        if (th32) combine_seq_kernel<BF, ETA, true><<<blocks, 256, 0, stream>>>(p, num0, num1, pden, o, dq_shift); \
        else combine_seq_kernel<BF, ETA, false><<<blocks, 256, 0, stream>>>(p, num0, num1, pden, o, dq_shift);     \
    } while (0)
    if (p.bf16) {
        if (pden != nullptr) IDATTN_COMB(true, true);
        else IDATTN_COMB(true, false);
    } else {
        if (pden != nullptr) IDATTN_COMB(false, true);
        else IDATTN_COMB(false, false);
    }
#undef IDATTN_COMB
    return hipGetLastError();
}

}  // namespace idattn

// Host-side checks of the C ABI, built with AddressSanitizer and UBSan on the
// host code (tests/test_abi_sanitizer.py).  Every call below returns from
// argument validation before any HIP call, so no GPU is needed; the pointers
// are fake, 16-byte aligned device addresses that validation never
// dereferences.  Prints one line per failed expectation and exits non-zero
// if there was any.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "idattn.h"

static int g_fails = 0;
static int g_checks = 0;

static void expect(int got, int want, const char* what) {
    ++g_checks;
    if (got != want) {
        std::printf("FAIL %s: status %d (%s), want %d: %s\n", what, got, idattn_status_string(static_cast<idattn_status>(got)),
                    want, idattn_last_error());
        ++g_fails;
    }
}

// addresses 8 GiB apart, so that no two buffers overlap unless a test asks for it
static void* fake(uint64_t slot, uint64_t byte_offset = 0) {
    return reinterpret_cast<void*>((slot << 33) + byte_offset);
}

static idattn_dims dims(int64_t B, int64_t N, int64_t H, int64_t d, int64_t M, int64_t W, int io, int algo) {
    idattn_dims x;
    std::memset(&x, 0, sizeof(x));
    x.B = B;
    x.N = N;
    x.H = H;
    x.d = d;
    x.M = M;
    x.W = W;
    x.io_dtype = io;
    x.algo = algo;
    x.eps_feat = 1e-6f;
    x.eps_norm = 1e-6f;
    x.feature_norm = IDATTN_FEATURE_SQUARED;
    return x;
}

static idattn_params params() {
    idattn_params p;
    p.conv_q = static_cast<const float*>(fake(20));
    p.conv_k = static_cast<const float*>(fake(21));
    p.gain = static_cast<const float*>(fake(22));
    p.bias = static_cast<const float*>(fake(23));
    p.log_dt = static_cast<const float*>(fake(24));
    p.A = static_cast<const float*>(fake(25));
    p.Bc = static_cast<const float*>(fake(26));
    p.rff_omega = static_cast<const float*>(fake(27));
    return p;
}

static int forward(const idattn_dims& d, const idattn_params& p, size_t ws_bytes, void* o = fake(4),
                   void* state_out = fake(7), const void* q = fake(1)) {
    return idattn_forward(&d, &p, q, fake(2), fake(3), o, static_cast<const float*>(fake(5)), fake(6),
                          static_cast<float*>(state_out), fake(8), fake(9), ws_bytes, nullptr);
}

int main() {
    const idattn_params p = params();

    // the workspace query over every supported shape, both I/O types and every algorithm
    const int64_t ds[] = {16, 32, 64, 128}, ms[] = {16, 32, 64};
    for (int64_t d : ds)
        for (int64_t m : ms)
            for (int64_t w = 1; w <= 8; ++w)
                for (int io = 0; io < 2; ++io)
                    for (int algo = 0; algo < 3; ++algo)
                        for (int64_t n : {int64_t{0}, int64_t{1}, int64_t{63}, int64_t{64}, int64_t{700}}) {
                            const idattn_dims x = dims(3, n, 5, d, m, w, io, algo);
                            size_t bytes = 0;
                            const int st = idattn_forward_workspace_size(&x, &bytes);
                            const bool chunked_ok = io == IDATTN_IO_BF16 && m == 64 && (d == 64 || d == 128) && w <= 4;
                            const int want = (algo == IDATTN_ALGO_CHUNKED && !chunked_ok && n > 0) ? IDATTN_ERR_UNSUPPORTED
                                                                                                  : IDATTN_OK;
                            expect(st, want, "workspace size over the supported shapes");
                        }

    // forward: argument errors, all returned before any HIP call
    idattn_dims x = dims(2, 64, 3, 64, 32, 4, IDATTN_IO_BF16, IDATTN_ALGO_AUTO);
    size_t need = 0;
    expect(idattn_forward_workspace_size(&x, &need), IDATTN_OK, "workspace size");
    expect(forward(x, p, need - 1), IDATTN_ERR_WORKSPACE, "workspace one byte short");
    expect(idattn_forward(nullptr, &p, fake(1), fake(2), fake(3), fake(4), nullptr, nullptr, nullptr, nullptr, fake(9),
                          need, nullptr),
           IDATTN_ERR_NULL, "NULL dims");
    expect(idattn_forward(&x, nullptr, fake(1), fake(2), fake(3), fake(4), nullptr, nullptr, nullptr, nullptr, fake(9),
                          need, nullptr),
           IDATTN_ERR_NULL, "NULL params");
    expect(forward(x, p, need, nullptr), IDATTN_ERR_NULL, "NULL o");
    expect(forward(x, p, need, fake(1, 64)), IDATTN_ERR_ALIAS, "o overlaps q");
    expect(forward(x, p, need, fake(4), fake(4)), IDATTN_ERR_ALIAS, "state_out overlaps o");
    expect(forward(x, p, need, fake(4), fake(7), fake(1, 2)), IDATTN_ERR_ARG, "misaligned q");
    // the allocation-free forward: too large for the scratch array, and argument errors
    {
        const idattn_dims big = dims(64, 4096, 16, 128, 64, 4, IDATTN_IO_BF16, IDATTN_ALGO_CHUNKED);
        expect(idattn_forward_noalloc(&big, &p, fake(1), fake(2), fake(3), fake(4), nullptr, nullptr, nullptr,
                                      nullptr, nullptr),
               IDATTN_ERR_WORKSPACE, "noalloc beyond the scratch array");
        expect(idattn_forward_noalloc(nullptr, &p, fake(1), fake(2), fake(3), fake(4), nullptr, nullptr, nullptr,
                                      nullptr, nullptr),
               IDATTN_ERR_NULL, "noalloc NULL dims");
        expect(idattn_forward_noalloc(&x, &p, fake(1), fake(2), fake(3), fake(1, 64), nullptr, nullptr, nullptr,
                                      nullptr, nullptr),
               IDATTN_ERR_ALIAS, "noalloc o overlaps q");
        expect(idattn_forward_noalloc(&x, &p, fake(1), fake(2), fake(3), nullptr, nullptr, nullptr, nullptr, nullptr,
                                      nullptr),
               IDATTN_ERR_NULL, "noalloc NULL o");
    }
    {
        idattn_dims y = x;
        y.B = 0;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_SHAPE, "B = 0");
        y = x;
        y.d = 48;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_UNSUPPORTED, "d = 48");
        y = x;
        y.M = 128;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_UNSUPPORTED, "M = 128");
        y = x;
        y.W = 9;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_UNSUPPORTED, "W = 9");
        y = x;
        y.io_dtype = 7;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_ARG, "io_dtype");
        y = x;
        y.algo = 9;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_ARG, "algo");
        y = x;
        y.eps_feat = -1.f;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_ARG, "eps_feat < 0");
        y = x;
        y.feature_norm = 3;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_ARG, "feature_norm");
        y = x;
        y.feature_norm = IDATTN_FEATURE_RFF;
        idattn_params r = p;
        r.rff_omega = nullptr;
        expect(forward(y, r, 1ull << 40), IDATTN_ERR_NULL, "NULL rff_omega");
        expect(forward(y, p, 1ull << 40, fake(27, 64)), IDATTN_ERR_ALIAS, "o over rff_omega");
        y = x;
        y.N = int64_t{1} << 50;
        expect(forward(y, p, 1ull << 40), IDATTN_ERR_SHAPE, "N too large");
    }
    {
        idattn_params q = p;
        q.A = nullptr;
        expect(forward(x, q, need), IDATTN_ERR_NULL, "NULL lambda");
    }

    // packed variable-length batches: argument errors
    {
        idattn_dims y = dims(5, 1000, 3, 64, 32, 4, IDATTN_IO_BF16, IDATTN_ALGO_AUTO);
        size_t vneed = 0;
        expect(idattn_forward_varlen_workspace_size(&y, &vneed), IDATTN_OK, "varlen workspace size");
        const int32_t* cu = static_cast<const int32_t*>(fake(30));
        auto var = [&](const idattn_dims& z, const int32_t* c, size_t ws, void* o) {
            return idattn_forward_varlen(&z, &p, c, nullptr, fake(1), fake(2), fake(3), o,
                                         static_cast<const float*>(fake(5)), fake(6), static_cast<float*>(fake(7)),
                                         fake(8), fake(9), ws, nullptr);
        };
        expect(var(y, nullptr, vneed, fake(4)), IDATTN_ERR_NULL, "NULL cu_seqlens");
        expect(var(y, static_cast<const int32_t*>(fake(30, 2)), vneed, fake(4)), IDATTN_ERR_ARG, "misaligned cu_seqlens");
        expect(var(y, cu, vneed - 1, fake(4)), IDATTN_ERR_WORKSPACE, "varlen workspace one byte short");
        expect(var(y, cu, vneed, fake(30, 16)), IDATTN_ERR_ALIAS, "o over cu_seqlens");
        idattn_dims z = y;
        z.algo = IDATTN_ALGO_CHUNKED;
        expect(var(z, cu, vneed, fake(4)), IDATTN_ERR_UNSUPPORTED, "varlen chunked");
        z = y;
        z.N = int64_t{1} << 31;
        expect(var(z, cu, ~size_t{0}, fake(4)), IDATTN_ERR_SHAPE, "varlen T >= 2^31");
        const int32_t bad_host[6] = {0, 100, 50, 600, 900, 1000};
        expect(idattn_forward_varlen(&y, &p, cu, bad_host, fake(1), fake(2), fake(3), fake(4),
                                     static_cast<const float*>(fake(5)), fake(6), static_cast<float*>(fake(7)),
                                     fake(8), fake(9), vneed, nullptr),
               IDATTN_ERR_SHAPE, "decreasing cu_seqlens_host");
    }

    // normalised readout: argument errors
    {
        idattn_dims y = dims(2, 64, 3, 64, 32, 4, IDATTN_IO_BF16, IDATTN_ALGO_AUTO);
        size_t nneed = 0;
        expect(idattn_forward_normalized_workspace_size(&y, &nneed), IDATTN_OK, "normalized workspace size");
        auto nor = [&](const idattn_dims& z, size_t ws, const float* ei, float* eo) {
            return idattn_forward_normalized(&z, &p, fake(1), fake(2), fake(3), fake(4),
                                             static_cast<const float*>(fake(5)), fake(6), ei,
                                             static_cast<float*>(fake(7)), fake(8), eo, fake(9), ws, nullptr);
        };
        const float* ei = static_cast<const float*>(fake(31));
        float* eo = static_cast<float*>(fake(32));
        expect(nor(y, nneed - 1, ei, eo), IDATTN_ERR_WORKSPACE, "normalized workspace one byte short");
        expect(nor(y, nneed, static_cast<const float*>(fake(31, 8)), eo), IDATTN_ERR_ARG, "misaligned eta_in");
        expect(nor(y, nneed, ei, static_cast<float*>(fake(31, 16))), IDATTN_ERR_ALIAS, "eta_out partly over eta_in");
        expect(nor(y, nneed, ei, static_cast<float*>(fake(4, 64))), IDATTN_ERR_ALIAS, "eta_out over o");
        idattn_dims z = y;
        z.algo = IDATTN_ALGO_CHUNKED;
        expect(nor(z, nneed, ei, eo), IDATTN_ERR_UNSUPPORTED, "normalized chunked");
    }

    // decode: 1..8 tokens, argument errors
    {
        idattn_dims y = dims(2, 4, 3, 64, 32, 4, IDATTN_IO_BF16, IDATTN_ALGO_AUTO);
        const uint64_t tok = 2 * 4 * 3 * 64 * 2;  // bytes of q_t for N = 4
        auto dec = [&](const idattn_dims& z, void* o, void* state, void* tail) {
            return idattn_decode_step(&z, &p, fake(1), fake(2), fake(3), o, static_cast<float*>(state), tail, nullptr);
        };
        expect(dec(y, fake(1, tok - 16), fake(5), fake(6)), IDATTN_ERR_ALIAS, "o_t over the end of q_t (N = 4)");
        expect(dec(y, fake(4), nullptr, fake(6)), IDATTN_ERR_NULL, "NULL state");
        expect(dec(y, fake(4), fake(5, 4), fake(6)), IDATTN_ERR_ARG, "misaligned state");
        idattn_dims z = y;
        z.N = 0;
        expect(dec(z, fake(4), fake(5), fake(6)), IDATTN_ERR_SHAPE, "N = 0");
        z.N = 9;
        expect(dec(z, fake(4), fake(5), fake(6)), IDATTN_ERR_UNSUPPORTED, "N = 9");
        z = y;
        z.d = 100;
        expect(dec(z, fake(4), fake(5), fake(6)), IDATTN_ERR_UNSUPPORTED, "d = 100");
    }

    // status strings
    for (int s = 0; s <= 7; ++s) {
        const char* name = idattn_status_string(static_cast<idattn_status>(s));
        expect(name != nullptr && std::strncmp(name, "IDATTN_", 7) == 0, 1, "status string");
    }
    expect(std::strcmp(idattn_status_string(static_cast<idattn_status>(99)), "IDATTN_ERR_UNKNOWN") == 0, 1,
           "unknown status string");

    std::printf("%d checks, %d failed\n", g_checks, g_fails);
    return g_fails == 0 ? 0 : 1;
}

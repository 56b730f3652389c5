// C-ABI layer of libidattn: argument validation (entirely before any HIP
// call), workspace sizing, dispatch to the kernels, error text.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/idattn.h"
#include "launch.h"

static_assert(idattn::kNoallocScratchBytes == IDATTN_NOALLOC_SCRATCH_BYTES, "scratch size must match the header");

namespace {

thread_local char g_last_error[512] = "";

idattn_status fail(idattn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

idattn_status hip_fail(hipError_t e, const char* what) {
    return fail(IDATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* ptr, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    return Range{name, lo, ptr ? lo + bytes : lo};
}

bool overlap(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

bool supported_d(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_m(int64_t m) { return m == 16 || m == 32 || m == 64; }

idattn_status check_dims(const idattn_dims* dims, bool decode) {
    if (dims == nullptr) return fail(IDATTN_ERR_NULL, "dims is NULL");
    const idattn_dims& D = *dims;
    if (D.B < 1 || D.H < 1 || D.d < 1 || D.M < 1 || D.W < 1 || D.N < 0)
        return fail(IDATTN_ERR_SHAPE, "sizes must be positive (N >= 0): B=%lld N=%lld H=%lld d=%lld M=%lld W=%lld",
                    (long long)D.B, (long long)D.N, (long long)D.H, (long long)D.d, (long long)D.M,
                    (long long)D.W);
    if (decode && D.N < 1) return fail(IDATTN_ERR_SHAPE, "decode step needs N >= 1, got %lld", (long long)D.N);
    if (D.io_dtype != IDATTN_IO_F32 && D.io_dtype != IDATTN_IO_BF16)
        return fail(IDATTN_ERR_ARG, "io_dtype %d is not IDATTN_IO_F32 or IDATTN_IO_BF16", D.io_dtype);
    if (D.algo != IDATTN_ALGO_AUTO && D.algo != IDATTN_ALGO_SEQUENTIAL && D.algo != IDATTN_ALGO_CHUNKED)
        return fail(IDATTN_ERR_ARG, "algo %d is not a known idattn_algo", D.algo);
    if (!(D.eps_feat >= 0.f) || !std::isfinite(D.eps_feat))
        return fail(IDATTN_ERR_ARG, "eps_feat must be finite and >= 0");
    if (!(D.eps_norm >= 0.f) || !std::isfinite(D.eps_norm))
        return fail(IDATTN_ERR_ARG, "eps_norm must be finite and >= 0");
    if (D.feature_norm != IDATTN_FEATURE_SQUARED && D.feature_norm != IDATTN_FEATURE_UNIT &&
        D.feature_norm != IDATTN_FEATURE_RFF)
        return fail(IDATTN_ERR_ARG, "feature_norm %d is not a known idattn_feature_norm", D.feature_norm);
    // element counts must stay far from int64 overflow
    const double elems = static_cast<double>(D.B) * D.N * D.H * D.d;
    const double state = static_cast<double>(D.B) * D.H * D.M * D.d * 4.0;
    if (elems > 4.0e15 || state > 4.0e15 || D.H > (1 << 24) || D.B > (1LL << 31) || D.N > (1LL << 40))
        return fail(IDATTN_ERR_SHAPE, "sizes too large");
    if (!supported_d(D.d))
        return fail(IDATTN_ERR_UNSUPPORTED, "d=%lld: supported d (= R) are 16, 32, 64, 128", (long long)D.d);
    if (!supported_m(D.M))
        return fail(IDATTN_ERR_UNSUPPORTED, "M=%lld: supported M are 16, 32, 64", (long long)D.M);
    if (D.W > 8) return fail(IDATTN_ERR_UNSUPPORTED, "W=%lld: supported W are 1..8", (long long)D.W);
    if (D.B * D.H > 0x7fffffffLL)
        return fail(IDATTN_ERR_UNSUPPORTED, "B*H=%lld exceeds one grid dimension", (long long)(D.B * D.H));
    return IDATTN_OK;
}

idattn_status check_params(const idattn_dims& D, const idattn_params* prm) {
    if (prm == nullptr) return fail(IDATTN_ERR_NULL, "params is NULL");
    if (!prm->conv_q || !prm->conv_k || !prm->gain || !prm->bias || !prm->log_dt || !prm->A || !prm->Bc)
        return fail(IDATTN_ERR_NULL, "a parameter pointer is NULL");
    if (D.feature_norm == IDATTN_FEATURE_RFF && !prm->rff_omega)
        return fail(IDATTN_ERR_NULL, "rff_omega is NULL with IDATTN_FEATURE_RFF");
    return IDATTN_OK;
}

// Output buffers must not overlap any parameter the kernels read.
idattn_status check_params_disjoint(const idattn_dims& D, const idattn_params& P, const Range* outs, int n_outs) {
    const size_t conv = static_cast<size_t>(D.H * D.d * D.W) * 4, gb = static_cast<size_t>(D.H * 2 * D.d) * 4;
    const size_t mb = static_cast<size_t>(D.H * D.M * 2) * 4;
    const size_t ob = D.feature_norm == IDATTN_FEATURE_RFF ? static_cast<size_t>(D.H * D.d * (D.d / 2)) * 4 : 0;
    const Range prm[] = {range("conv_q", P.conv_q, conv), range("conv_k", P.conv_k, conv),
                         range("gain", P.gain, gb),        range("bias", P.bias, gb),
                         range("log_dt", P.log_dt, D.H * 4), range("A", P.A, mb),
                         range("Bc", P.Bc, mb),            range("rff_omega", P.rff_omega, ob)};
    for (int i = 0; i < n_outs; ++i)
        for (const Range& b : prm)
            if (overlap(outs[i], b)) return fail(IDATTN_ERR_ALIAS, "%s overlaps parameter %s", outs[i].name, b.name);
    return IDATTN_OK;
}

idattn::Problem problem(const idattn_dims& D) {
    idattn::Problem p;
    p.B = D.B;
    p.N = D.N;
    p.H = D.H;
    p.d = D.d;
    p.M = D.M;
    p.W = D.W;
    p.bf16 = D.io_dtype == IDATTN_IO_BF16;
    p.eps_feat = D.eps_feat;
    p.eps_norm = D.eps_norm;
    p.unit_feat = D.feature_norm == IDATTN_FEATURE_UNIT;
    p.rff_feat = D.feature_norm == IDATTN_FEATURE_RFF;
    p.T = D.B * D.N;
    p.cu = nullptr;
    return p;
}

int resolve_algo(const idattn_dims& D) {
    if (D.algo != IDATTN_ALGO_AUTO) return D.algo;
    return D.io_dtype == IDATTN_IO_BF16 && idattn::chunked_supported(problem(D)) ? IDATTN_ALGO_CHUNKED
                                                                                 : IDATTN_ALGO_SEQUENTIAL;
}

// tokens on the [T] axis: B N for the dense entry points, N for the packed one
size_t seq_workspace_bytes(const idattn_dims& D, int64_t T, bool eta = false) {
    // xi_q, z_k, z_v: float [H][T][d]; s: complex float [H][T][M]; with the
    // normalised readout also the denominator shares, float [H][T][M]
    const size_t tok = static_cast<size_t>(D.H) * T;
    const size_t a = 3 * tok * D.d * sizeof(float);
    const size_t s = tok * D.M * 2 * sizeof(float);
    const size_t e = eta ? tok * D.M * sizeof(float) : 0;
    return ((a + 255) / 256) * 256 + ((s + 255) / 256) * 256 + e;
}

idattn_status workspace_bytes(const idattn_dims& D, int algo, size_t* bytes) {
    if (D.N == 0) {
        *bytes = 0;
        return IDATTN_OK;
    }
    if (algo == IDATTN_ALGO_CHUNKED) {
        const idattn::Problem p = problem(D);
        if (D.io_dtype != IDATTN_IO_BF16)
            return fail(IDATTN_ERR_UNSUPPORTED, "the chunked algorithm needs bf16 I/O");
        if (!idattn::chunked_supported(p))
            return fail(IDATTN_ERR_UNSUPPORTED, "the chunked algorithm has no kernel for d=%lld M=%lld",
                        (long long)D.d, (long long)D.M);
        *bytes = idattn::chunked_workspace_bytes(p);
    } else {
        *bytes = seq_workspace_bytes(D, D.B * D.N);
    }
    return IDATTN_OK;
}

// The sequential path: feature kernel, key scan, value scan with readout, tail.
// With eta (normalised readout) eta_in / eta_out are the normaliser states.
idattn_status run_sequential(const idattn::Problem& p, const idattn_params& prm, const void* q, const void* k,
                             const void* v, void* o, const float* state_in, const void* tail_in, float* state_out,
                             void* tail_out, void* workspace, hipStream_t s, bool eta = false,
                             const float* eta_in = nullptr, float* eta_out = nullptr) {
    const size_t tok = static_cast<size_t>(p.H) * p.T;
    float* xi_q = static_cast<float*>(workspace);
    float* z_k = xi_q + tok * p.d;
    float* z_v = z_k + tok * p.d;
    char* base = static_cast<char*>(workspace);
    const size_t off_s = ((3 * tok * p.d * sizeof(float) + 255) / 256) * 256;
    float* sbuf = reinterpret_cast<float*>(base + off_s);
    float* pden = eta ? reinterpret_cast<float*>(base + off_s + ((tok * p.M * 2 * sizeof(float) + 255) / 256) * 256)
                      : nullptr;
    hipError_t e = idattn::launch_featmap_conv_norm(p, prm, q, k, v, tail_in, xi_q, z_k, z_v, s);
    if (e != hipSuccess) return hip_fail(e, "featmap_conv_norm");
    e = idattn::launch_ssm_key_scan_seq(p, prm, xi_q, z_k, state_in, sbuf, state_out, eta_in, eta_out, pden, s);
    if (e != hipSuccess) return hip_fail(e, "ssm_key_scan");
    // xi_q and z_k are dead once the key scan has run: they take the value scan's partial numerators
    e = idattn::launch_ssm_value_scan_readout_seq(p, prm, sbuf, z_v, state_in, o, state_out, pden, xi_q, z_k, s);
    if (e != hipSuccess) return hip_fail(e, "ssm_value_scan_readout");
    if (tail_out) {
        e = idattn::launch_tail_update(p, q, k, tail_in, tail_out, s);
        if (e != hipSuccess) return hip_fail(e, "tail update");
    }
    return IDATTN_OK;
}

// Buffer checks shared by both forward entry points: alignment, overlaps
// between the outputs and every other buffer (exact in-place state and tail
// allowed), and between the outputs and the parameters.  act = bytes of q
// (and of k, v, o); extra = one more read-only buffer (or an empty range).
idattn_status check_forward_buffers(const idattn_dims& D, const idattn_params& P, const void* q, const void* k,
                                    const void* v, void* o, const float* state_in, const void* tail_in,
                                    float* state_out, void* tail_out, void* workspace, size_t need, size_t act,
                                    const Range& extra) {
    const void* ptrs[] = {q, k, v, o, state_in, tail_in, state_out, tail_out, workspace};
    for (const void* ptr : ptrs)
        if (misaligned(ptr)) return fail(IDATTN_ERR_ARG, "device buffers must be 16-byte aligned");
    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t stb = static_cast<size_t>(D.B) * D.H * D.M * 2 * D.d * 2 * sizeof(float);
    const size_t tlb = static_cast<size_t>(D.B) * D.H * 2 * (D.W - 1) * D.d * io;
    const Range rq = range("q", q, act), rk = range("k", k, act), rv = range("v", v, act);
    const Range ro = range("o", o, act);
    const Range rsi = range("state_in", state_in, stb), rso = range("state_out", state_out, stb);
    const Range rti = range("tail_in", tail_in, tlb), rto = range("tail_out", tail_out, tlb);
    const Range rws = range("workspace", workspace, need);
    const Range outs[] = {ro, rso, rto, rws};
    const Range all[] = {rq, rk, rv, ro, rsi, rso, rti, rto, rws, extra};
    for (const Range& a : outs)
        for (const Range& b : all) {
            if (&a == &b || a.name == b.name) continue;
            if (!overlap(a, b)) continue;
            // exact in-place pairs are allowed
            if ((a.name == rso.name && b.name == rsi.name) || (a.name == rto.name && b.name == rti.name)) {
                if (a.lo == b.lo) continue;
            }
            return fail(IDATTN_ERR_ALIAS, "%s overlaps %s", a.name, b.name);
        }
    return check_params_disjoint(D, P, outs, 4);
}

// N = 0: copy state_in / tail_in to the outputs (zeros when not given).
idattn_status copy_through(const idattn_dims& D, const float* state_in, const void* tail_in, float* state_out,
                           void* tail_out, hipStream_t s) {
    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t stb = static_cast<size_t>(D.B) * D.H * D.M * 2 * D.d * 2 * sizeof(float);
    const size_t tlb = static_cast<size_t>(D.B) * D.H * 2 * (D.W - 1) * D.d * io;
    hipError_t e;
    if (state_out) {
        e = idattn::launch_copy_or_zero(state_in, state_out, static_cast<int64_t>(stb / 4), s);
        if (e != hipSuccess) return hip_fail(e, "state copy");
    }
    if (tail_out && tlb > 0) {
        e = idattn::launch_copy_or_zero(tail_in, tail_out, static_cast<int64_t>(tlb / 4), s);
        if (e != hipSuccess) return hip_fail(e, "tail copy");
    }
    return IDATTN_OK;
}

}  // namespace

extern "C" {

int idattn_version(void) { return 200; }

const char* idattn_status_string(idattn_status st) {
    // A C caller may pass any int; reading it as the C++ enum type would be
    // undefined outside the enumerators' range, so read its bytes as an int.
    static_assert(sizeof(idattn_status) == sizeof(int), "idattn_status must be int-sized");
    int v;
    std::memcpy(&v, &st, sizeof v);
    switch (v) {
        case IDATTN_OK: return "IDATTN_OK";
        case IDATTN_ERR_NULL: return "IDATTN_ERR_NULL";
        case IDATTN_ERR_SHAPE: return "IDATTN_ERR_SHAPE";
        case IDATTN_ERR_UNSUPPORTED: return "IDATTN_ERR_UNSUPPORTED";
        case IDATTN_ERR_WORKSPACE: return "IDATTN_ERR_WORKSPACE";
        case IDATTN_ERR_ALIAS: return "IDATTN_ERR_ALIAS";
        case IDATTN_ERR_ARG: return "IDATTN_ERR_ARG";
        case IDATTN_ERR_HIP: return "IDATTN_ERR_HIP";
    }
    return "IDATTN_ERR_UNKNOWN";
}

const char* idattn_last_error(void) { return g_last_error; }

idattn_status idattn_forward_workspace_size(const idattn_dims* dims, size_t* bytes) {
    if (bytes == nullptr) return fail(IDATTN_ERR_NULL, "bytes is NULL");
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    return workspace_bytes(*dims, resolve_algo(*dims), bytes);
}

}  // extern "C"

namespace {

// Both dense forward entry points.  noalloc: the workspace is the library's
// scratch array (its address looked up after validation), else the caller's.
idattn_status forward_impl(const idattn_dims* dims, const idattn_params* params, const void* q, const void* k,
                           const void* v, void* o, const float* state_in, const void* tail_in, float* state_out,
                           void* tail_out, void* workspace, size_t workspace_bytes_given, void* stream,
                           bool noalloc) {
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    st = check_params(*dims, params);
    if (st != IDATTN_OK) return st;
    const idattn_dims& D = *dims;
    const int algo = resolve_algo(D);
    if (D.N > 0 && (!q || !k || !v || !o)) return fail(IDATTN_ERR_NULL, "q, k, v and o must be non-NULL");
    size_t need = 0;
    st = workspace_bytes(D, algo, &need);
    if (st != IDATTN_OK) return st;
    if (noalloc) {
        if (need > idattn::kNoallocScratchBytes)
            return fail(IDATTN_ERR_WORKSPACE,
                        "these dims need %zu bytes of scratch; idattn_forward_noalloc has %zu "
                        "(IDATTN_NOALLOC_SCRATCH_BYTES); use idattn_forward with a workspace",
                        need, idattn::kNoallocScratchBytes);
    } else {
        if (need > 0 && workspace == nullptr)
            return fail(IDATTN_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
        if (workspace_bytes_given < need)
            return fail(IDATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_given, need);
    }

    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t act = static_cast<size_t>(D.B) * D.N * D.H * D.d * io;
    // the scratch array cannot overlap a caller's buffer: check without it
    st = check_forward_buffers(D, *params, q, k, v, o, state_in, tail_in, state_out, tail_out,
                               noalloc ? nullptr : workspace, noalloc ? 0 : need, act, range("none", nullptr, 0));
    if (st != IDATTN_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (D.N == 0) return copy_through(D, state_in, tail_in, state_out, tail_out, s);
    if (noalloc && need > 0) {
        const hipError_t e = idattn::noalloc_scratch(&workspace);
        if (e != hipSuccess) return hip_fail(e, "scratch address");
    }
    const idattn::Problem p = problem(D);
    if (algo == IDATTN_ALGO_CHUNKED) {
        const hipError_t e = idattn::launch_forward_chunked(p, *params, q, k, v, o, state_in, tail_in, state_out,
                                                            tail_out, workspace, s);
        if (e != hipSuccess) return hip_fail(e, "chunked forward");
        return IDATTN_OK;  // the chunked forward writes tail_out itself
    }
    return run_sequential(p, *params, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, s);
}

}  // namespace

extern "C" {

idattn_status idattn_forward(const idattn_dims* dims, const idattn_params* params, const void* q,
                             const void* k, const void* v, void* o, const float* state_in,
                             const void* tail_in, float* state_out, void* tail_out, void* workspace,
                             size_t workspace_bytes_given, void* stream) {
    return forward_impl(dims, params, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace,
                        workspace_bytes_given, stream, false);
}

idattn_status idattn_forward_noalloc(const idattn_dims* dims, const idattn_params* params, const void* q,
                                     const void* k, const void* v, void* o, const float* state_in,
                                     const void* tail_in, float* state_out, void* tail_out, void* stream) {
    return forward_impl(dims, params, q, k, v, o, state_in, tail_in, state_out, tail_out, nullptr, 0, stream,
                        true);
}

}  // extern "C"

namespace {

// The normalised readout's algorithm and workspace: the chunked one wherever
// the plain readout has it (AUTO picks it there), else the sequential one.
idattn_status normalized_plan(const idattn_dims& D, int* algo, size_t* bytes) {
    *algo = resolve_algo(D);
    if (*algo == IDATTN_ALGO_CHUNKED) {
        idattn_status st = workspace_bytes(D, IDATTN_ALGO_CHUNKED, bytes);
        if (st != IDATTN_OK) return st;
        return IDATTN_OK;
    }
    *bytes = D.N == 0 ? 0 : seq_workspace_bytes(D, D.B * D.N, true);
    return IDATTN_OK;
}

}  // namespace

extern "C" {

idattn_status idattn_forward_normalized_workspace_size(const idattn_dims* dims, size_t* bytes) {
    if (bytes == nullptr) return fail(IDATTN_ERR_NULL, "bytes is NULL");
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    int algo;
    return normalized_plan(*dims, &algo, bytes);
}

idattn_status idattn_forward_normalized(const idattn_dims* dims, const idattn_params* params, const void* q,
                                        const void* k, const void* v, void* o, const float* state_in,
                                        const void* tail_in, const float* eta_in, float* state_out, void* tail_out,
                                        float* eta_out, void* workspace, size_t workspace_bytes_given, void* stream) {
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    st = check_params(*dims, params);
    if (st != IDATTN_OK) return st;
    const idattn_dims& D = *dims;
    int algo;
    size_t need = 0;
    st = normalized_plan(D, &algo, &need);
    if (st != IDATTN_OK) return st;
    if (D.N > 0 && (!q || !k || !v || !o)) return fail(IDATTN_ERR_NULL, "q, k, v and o must be non-NULL");
    if (need > 0 && workspace == nullptr) return fail(IDATTN_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (workspace_bytes_given < need)
        return fail(IDATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_given, need);
    if (misaligned(eta_in) || misaligned(eta_out)) return fail(IDATTN_ERR_ARG, "device buffers must be 16-byte aligned");
    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t act = static_cast<size_t>(D.B) * D.N * D.H * D.d * io;
    const size_t etab = static_cast<size_t>(D.B) * D.H * D.M * 2 * sizeof(float);
    const Range rei = range("eta_in", eta_in, etab), reo = range("eta_out", eta_out, etab);
    // eta_out: an output like the others; it may equal eta_in exactly
    st = check_forward_buffers(D, *params, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, need, act,
                               rei);
    if (st != IDATTN_OK) return st;
    {
        const size_t stb = static_cast<size_t>(D.B) * D.H * D.M * 2 * D.d * 2 * sizeof(float);
        const size_t tlb = static_cast<size_t>(D.B) * D.H * 2 * (D.W - 1) * D.d * io;
        const Range others[] = {range("q", q, act), range("k", k, act), range("v", v, act), range("o", o, act),
                                range("state_in", state_in, stb), range("state_out", state_out, stb),
                                range("tail_in", tail_in, tlb), range("tail_out", tail_out, tlb),
                                range("workspace", workspace, need), rei};
        for (const Range& b : others) {
            if (!overlap(reo, b)) continue;
            if (b.name == rei.name && reo.lo == b.lo) continue;
            return fail(IDATTN_ERR_ALIAS, "eta_out overlaps %s", b.name);
        }
        st = check_params_disjoint(D, *params, &reo, 1);
        if (st != IDATTN_OK) return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (D.N == 0) {
        st = copy_through(D, state_in, tail_in, state_out, tail_out, s);
        if (st != IDATTN_OK || eta_out == nullptr) return st;
        const hipError_t e = idattn::launch_copy_or_zero(eta_in, eta_out, static_cast<int64_t>(etab / 4), s);
        if (e != hipSuccess) return hip_fail(e, "eta copy");
        return IDATTN_OK;
    }
    if (algo == IDATTN_ALGO_CHUNKED) {
        idattn::Problem p = problem(D);
        p.eta = true;
        const hipError_t e = idattn::launch_forward_chunked(p, *params, q, k, v, o, state_in, tail_in, state_out,
                                                            tail_out, workspace, s, eta_in, eta_out);
        if (e != hipSuccess) return hip_fail(e, "chunked forward (normalised readout)");
        return IDATTN_OK;
    }
    return run_sequential(problem(D), *params, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, s, true,
                          eta_in, eta_out);
}

// The chunked algorithm runs a packed batch in one launch sequence whose plan
// (segments per sequence, offsets) is built on the device from cu_seqlens;
// its workspace depends on B, H and T only.
bool varlen_chunked_possible(const idattn_dims& D) {
    return D.io_dtype == IDATTN_IO_BF16 && idattn::chunked_packed_supported(problem(D));
}

size_t varlen_workspace(const idattn_dims& D) {
    if (D.N == 0) return 0;
    size_t bytes = seq_workspace_bytes(D, D.N);
    if (D.algo != IDATTN_ALGO_SEQUENTIAL && varlen_chunked_possible(D)) {
        const size_t c = idattn::chunked_packed_workspace_bytes(problem(D));
        if (c > bytes) bytes = c;
    }
    return bytes;
}

idattn_status idattn_forward_varlen_workspace_size(const idattn_dims* dims, size_t* bytes) {
    if (bytes == nullptr) return fail(IDATTN_ERR_NULL, "bytes is NULL");
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    if (dims->algo == IDATTN_ALGO_CHUNKED && !varlen_chunked_possible(*dims))
        return fail(IDATTN_ERR_UNSUPPORTED, "the chunked algorithm has no kernel for these dims");
    *bytes = varlen_workspace(*dims);
    return IDATTN_OK;
}

idattn_status idattn_forward_varlen(const idattn_dims* dims, const idattn_params* params, const int32_t* cu_seqlens,
                                    const int32_t* cu_seqlens_host, const void* q, const void* k, const void* v,
                                    void* o, const float* state_in, const void* tail_in, float* state_out,
                                    void* tail_out, void* workspace, size_t workspace_bytes_given, void* stream) {
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    st = check_params(*dims, params);
    if (st != IDATTN_OK) return st;
    const idattn_dims& D = *dims;
    if (D.N > 0x7fffffffLL) return fail(IDATTN_ERR_SHAPE, "N=%lld: a packed batch holds < 2^31 tokens", (long long)D.N);
    const bool chunked = D.algo != IDATTN_ALGO_SEQUENTIAL && varlen_chunked_possible(D);
    if (D.algo == IDATTN_ALGO_CHUNKED && !chunked)
        return fail(IDATTN_ERR_UNSUPPORTED, "the chunked algorithm has no kernel for these dims");
    if (cu_seqlens == nullptr) return fail(IDATTN_ERR_NULL, "cu_seqlens is NULL");
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return fail(IDATTN_ERR_ARG, "cu_seqlens must be 4-byte aligned");
    if (cu_seqlens_host != nullptr) {
        if (cu_seqlens_host[0] != 0 || cu_seqlens_host[D.B] != D.N)
            return fail(IDATTN_ERR_SHAPE, "cu_seqlens_host must run from 0 to N=%lld", (long long)D.N);
        for (int64_t b = 0; b < D.B; ++b)
            if (cu_seqlens_host[b + 1] < cu_seqlens_host[b])
                return fail(IDATTN_ERR_SHAPE, "cu_seqlens_host decreases at %lld", (long long)b);
    }
    if (D.N > 0 && (!q || !k || !v || !o)) return fail(IDATTN_ERR_NULL, "q, k, v and o must be non-NULL");
    const size_t need = varlen_workspace(D);
    if (need > 0 && workspace == nullptr) return fail(IDATTN_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (workspace_bytes_given < need)
        return fail(IDATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_given, need);
    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t act = static_cast<size_t>(D.N) * D.H * D.d * io;
    st = check_forward_buffers(D, *params, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, need, act,
                               range("cu_seqlens", cu_seqlens, static_cast<size_t>(D.B + 1) * 4));
    if (st != IDATTN_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (D.N == 0) return copy_through(D, state_in, tail_in, state_out, tail_out, s);
    if (!chunked) {
        idattn::Problem p = problem(D);
        p.T = D.N;
        p.cu = cu_seqlens;
        return run_sequential(p, *params, q, k, v, o, state_in, tail_in, state_out, tail_out, workspace, s);
    }
    const hipError_t e = idattn::launch_forward_chunked_packed(problem(D), *params, cu_seqlens, q, k, v, o, state_in,
                                                               tail_in, state_out, tail_out, workspace, s);
    if (e != hipSuccess) return hip_fail(e, "chunked forward (packed batch)");
    return IDATTN_OK;
}

}  // extern "C"

namespace {

idattn_status check_backward_dims(const idattn_dims* dims) {
    idattn_status st = check_dims(dims, false);
    if (st != IDATTN_OK) return st;
    if (dims->feature_norm == IDATTN_FEATURE_RFF)
        return fail(IDATTN_ERR_UNSUPPORTED, "the backward pass has the SiLU feature maps only (squared, unit)");
    if (dims->algo == IDATTN_ALGO_CHUNKED)
        return fail(IDATTN_ERR_UNSUPPORTED, "the backward pass runs on the sequential algorithm only");
    return IDATTN_OK;
}

}  // namespace

extern "C" {

idattn_status idattn_backward_workspace_size(const idattn_dims* dims, size_t* bytes) {
    if (bytes == nullptr) return fail(IDATTN_ERR_NULL, "bytes is NULL");
    const idattn_status st = check_backward_dims(dims);
    if (st != IDATTN_OK) return st;
    *bytes = dims->N == 0 ? 0 : idattn::backward_workspace_bytes(problem(*dims));
    return IDATTN_OK;
}

idattn_status idattn_backward(const idattn_dims* dims, const idattn_params* params, const void* q, const void* k,
                              const void* v, const float* state_in, const void* tail_in, const void* grad_o,
                              const float* grad_state, void* grad_q, void* grad_k, void* grad_v,
                              const idattn_param_grads* grad_params, float* grad_state_in, void* workspace,
                              size_t workspace_bytes_given, void* stream) {
    idattn_status st = check_backward_dims(dims);
    if (st != IDATTN_OK) return st;
    st = check_params(*dims, params);
    if (st != IDATTN_OK) return st;
    const idattn_dims& D = *dims;
    if (grad_params == nullptr) return fail(IDATTN_ERR_NULL, "grad_params is NULL");
    const idattn_param_grads& G = *grad_params;
    if (!G.conv_q || !G.conv_k || !G.gain || !G.bias || !G.log_dt || !G.A || !G.Bc)
        return fail(IDATTN_ERR_NULL, "a parameter-gradient pointer is NULL");
    if (D.N > 0 && (!q || !k || !v || !grad_o || !grad_q || !grad_k || !grad_v))
        return fail(IDATTN_ERR_NULL, "q, k, v, grad_o, grad_q, grad_k and grad_v must be non-NULL");
    const size_t need = D.N == 0 ? 0 : idattn::backward_workspace_bytes(problem(D));
    if (need > 0 && workspace == nullptr) return fail(IDATTN_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (workspace_bytes_given < need)
        return fail(IDATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_given, need);
    {
        const void* ptrs[] = {q, k, v, state_in, tail_in, grad_o, grad_state, grad_q, grad_k, grad_v, grad_state_in,
                              workspace, G.conv_q, G.conv_k, G.gain, G.bias, G.log_dt, G.A, G.Bc};
        for (const void* ptr : ptrs)
            if (misaligned(ptr)) return fail(IDATTN_ERR_ARG, "device buffers must be 16-byte aligned");
    }
    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t act = static_cast<size_t>(D.B) * D.N * D.H * D.d * io;
    const size_t stb = static_cast<size_t>(D.B) * D.H * D.M * 2 * D.d * 2 * sizeof(float);
    const size_t tlb = static_cast<size_t>(D.B) * D.H * 2 * (D.W - 1) * D.d * io;
    const size_t conv = static_cast<size_t>(D.H * D.d * D.W) * 4, gb = static_cast<size_t>(D.H * 2 * D.d) * 4;
    const size_t mb = static_cast<size_t>(D.H * D.M * 2) * 4;
    const Range outs[] = {range("grad_q", grad_q, act), range("grad_k", grad_k, act), range("grad_v", grad_v, act),
                          range("grad_state_in", grad_state_in, stb), range("workspace", workspace, need),
                          range("grad_conv_q", G.conv_q, conv), range("grad_conv_k", G.conv_k, conv),
                          range("grad_gain", G.gain, gb), range("grad_bias", G.bias, gb),
                          range("grad_log_dt", G.log_dt, D.H * 4), range("grad_A", G.A, mb), range("grad_Bc", G.Bc, mb)};
    const Range ins[] = {range("q", q, act), range("k", k, act), range("v", v, act), range("state_in", state_in, stb),
                         range("tail_in", tail_in, tlb), range("grad_o", grad_o, act),
                         range("grad_state", grad_state, stb)};
    constexpr int n_outs = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < n_outs; ++i) {
        for (int j = 0; j < n_outs; ++j)
            if (i != j && overlap(outs[i], outs[j])) return fail(IDATTN_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range& b : ins)
            if (overlap(outs[i], b)) return fail(IDATTN_ERR_ALIAS, "%s overlaps %s", outs[i].name, b.name);
    }
    st = check_params_disjoint(D, *params, outs, n_outs);
    if (st != IDATTN_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (D.N == 0) {
        hipError_t e = hipSuccess;
        float* const zero_outs[] = {G.conv_q, G.conv_k, G.gain, G.bias, G.log_dt, G.A, G.Bc};
        const size_t zero_bytes[] = {conv, conv, gb, gb, static_cast<size_t>(D.H) * 4, mb, mb};
        for (int i = 0; i < 7 && e == hipSuccess; ++i)
            e = idattn::launch_copy_or_zero(nullptr, zero_outs[i], static_cast<int64_t>(zero_bytes[i] / 4), s);
        if (e == hipSuccess && grad_state_in != nullptr)
            e = idattn::launch_copy_or_zero(grad_state, grad_state_in, static_cast<int64_t>(stb / 4), s);
        if (e != hipSuccess) return hip_fail(e, "backward with no tokens");
        return IDATTN_OK;
    }
    const hipError_t e = idattn::launch_backward(problem(D), *params, q, k, v, state_in, tail_in, grad_o, grad_state,
                                                 grad_q, grad_k, grad_v, G, grad_state_in, workspace, s);
    if (e != hipSuccess) return hip_fail(e, "backward");
    return IDATTN_OK;
}

}  // extern "C"

namespace {

// Both decode entry points; eta (normalised readout) is NULL for the plain one.
idattn_status decode_impl(const idattn_dims* dims, const idattn_params* params, const void* q_t, const void* k_t,
                          const void* v_t, void* o_t, float* state, void* tail, float* eta, bool normalized,
                          void* stream) {
    idattn_status st = check_dims(dims, true);
    if (st != IDATTN_OK) return st;
    st = check_params(*dims, params);
    if (st != IDATTN_OK) return st;
    const idattn_dims& D = *dims;
    if (!q_t || !k_t || !v_t || !o_t || !state) return fail(IDATTN_ERR_NULL, "q_t, k_t, v_t, o_t and state must be non-NULL");
    if (D.W > 1 && !tail) return fail(IDATTN_ERR_NULL, "tail must be non-NULL when W > 1");
    if (normalized && !eta) return fail(IDATTN_ERR_NULL, "eta must be non-NULL");
    {
        const void* ptrs[] = {q_t, k_t, v_t, o_t, state, tail, eta};
        for (const void* ptr : ptrs)
            if (misaligned(ptr)) return fail(IDATTN_ERR_ARG, "device buffers must be 16-byte aligned");
    }
    if (D.N > idattn::kDecodeMaxTokens)
        return fail(IDATTN_ERR_UNSUPPORTED, "decode step takes 1..%d tokens per sequence, got %lld",
                    idattn::kDecodeMaxTokens, (long long)D.N);
    const size_t io = D.io_dtype == IDATTN_IO_BF16 ? 2 : 4;
    const size_t tokb = static_cast<size_t>(D.B) * D.N * D.H * D.d * io;
    const size_t stb = static_cast<size_t>(D.B) * D.H * D.M * 2 * D.d * 2 * sizeof(float);
    const size_t tlb = static_cast<size_t>(D.B) * D.H * 2 * (D.W - 1) * D.d * io;
    const size_t etab = static_cast<size_t>(D.B) * D.H * D.M * 2 * sizeof(float);
    const Range rq = range("q_t", q_t, tokb), rk = range("k_t", k_t, tokb), rv = range("v_t", v_t, tokb);
    const Range ro = range("o_t", o_t, tokb), rs = range("state", state, stb), rt = range("tail", tail, tlb);
    const Range re = range("eta", normalized ? eta : nullptr, etab);
    const Range outs[] = {ro, rs, rt, re};
    const Range all[] = {rq, rk, rv, ro, rs, rt, re};
    for (const Range& a : outs)
        for (const Range& b : all) {
            if (a.name == b.name) continue;
            if (overlap(a, b)) return fail(IDATTN_ERR_ALIAS, "%s overlaps %s", a.name, b.name);
        }
    st = check_params_disjoint(D, *params, outs, 4);
    if (st != IDATTN_OK) return st;
    const hipError_t e = idattn::launch_decode_step(problem(D), *params, q_t, k_t, v_t, o_t, state, tail,
                                                    normalized ? eta : nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode_step");
    return IDATTN_OK;
}

}  // namespace

extern "C" {

idattn_status idattn_decode_step(const idattn_dims* dims, const idattn_params* params, const void* q_t,
                                 const void* k_t, const void* v_t, void* o_t, float* state, void* tail,
                                 void* stream) {
    return decode_impl(dims, params, q_t, k_t, v_t, o_t, state, tail, nullptr, false, stream);
}

idattn_status idattn_decode_step_normalized(const idattn_dims* dims, const idattn_params* params, const void* q_t,
                                            const void* k_t, const void* v_t, void* o_t, float* state, void* tail,
                                            float* eta, void* stream) {
    return decode_impl(dims, params, q_t, k_t, v_t, o_t, state, tail, eta, true, stream);
}

}  // extern "C"

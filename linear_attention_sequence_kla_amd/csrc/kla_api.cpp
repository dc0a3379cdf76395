// kla_api.cpp -- the C ABI of libkla (include/kla.h): argument validation,
// tiling plans, workspace sizing and kernel dispatch.  Every argument error is
// reported before anything is enqueued.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kla.h"
#include "kla_internal.h"

namespace kla {

namespace {

bool mul_ok(int64_t x, int64_t y, int64_t* out) {
    if (x < 0 || y < 0) return false;
    if (x != 0 && y > INT64_MAX / x) return false;
    *out = x * y;
    return true;
}

}  // namespace

bool make_plan(int64_t B, int64_t H, int64_t T, int64_t D, int rows_per_wave, int waves,
               int matrix_words, int state_words, Plan* pl) {
    int64_t BH, C, N;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, D, &C) || !mul_ok(C, T, &N)) return false;
    if (N > INT64_MAX / 16) return false;  // byte offsets of every tensor fit
    const int64_t R = int64_t(rows_per_wave) * waves;
    pl->C = C;
    pl->N = N;
    pl->G = (C + kWave - 1) / kWave;
    pl->n_chunks = (T + R - 1) / R;
    if (!mul_ok(pl->G, pl->n_chunks, &pl->n_tiles)) return false;
    if (pl->n_tiles > int64_t(INT32_MAX)) return false;
    // Each wave addresses its rows with 32-bit byte offsets from one base.
    // When D is a multiple of 64, a column group's 64 channels lie in one
    // slab, so the offsets only span the wave's own rows (plus one row before)
    // whatever T is; otherwise the 64 channels span up to ceil((D + 62) / D)
    // slabs of T*D elements.
    int64_t span_el = 0;
    if (D > 0 && D % kWave == 0)
        span_el = (int64_t(rows_per_wave) + 2) * D + kWave;
    else if (D > 0)
        span_el = ((D + 62) / D) * T * D + 2 * D + int64_t(rows_per_wave) * D;
    pl->offsets_fit = span_el < (int64_t(1) << 30);
    pl->ws = workspace_layout(size_t(pl->n_tiles), matrix_words, state_words);
    return true;
}

namespace {
thread_local char t_detail[512];
}  // namespace

kla_status fail(kla_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_detail, sizeof(t_detail), fmt, ap);
    va_end(ap);
    return s;
}

}  // namespace kla

namespace {

using kla::Plan;
using kla::fail;
using kla::t_detail;

bool overlaps(const void* x, size_t nx, const void* y, size_t ny) {
    if (!x || !y || nx == 0 || ny == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x), b0 = reinterpret_cast<uintptr_t>(y);
    return a0 < b0 + ny && b0 < a0 + nx;
}

bool misaligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }

// dtype and status codes come from C callers (or ctypes) as plain ints.  C++
// may not even read an enum object whose value lies outside the enum's range,
// so an argument is validated through its object representation before it is
// used as the enum.
static_assert(sizeof(kla_dtype) == sizeof(int32_t) && sizeof(kla_status) == sizeof(int32_t),
              "the ABI's enums are int-sized");
template <typename E>
int32_t raw_bits(const E& e) {
    int32_t r;
    memcpy(&r, &e, sizeof(r));
    return r;
}
bool known_dtype(const kla_dtype& d) {
    const int32_t r = raw_bits(d);
    return r == KLA_DTYPE_F32 || r == KLA_DTYPE_BF16;
}
// Rows per wave of the forward kernel for the argument's dtype, in the scan
// or the mixer modes (any value for an unknown dtype, which common_checks
// then rejects).
int fwd_rows(const kla_dtype& d, bool mixer) {
    return known_dtype(d) ? kla::fwd_rows(d, mixer) : kla::kFwdRows;
}
// The forward kernel's tile in the scan modes for this problem (the 4-wave
// float32 tile for an unknown dtype, which common_checks then rejects).
// Waves per tile of the backward kernel from states (4 for an unknown dtype,
// which common_checks then rejects).
int state_bwd_waves(const kla_dtype& d, int64_t T) {
    return known_dtype(d) ? kla::state_bwd_waves(d, T) : 4;
}
kla::FwdTile scan_tile(const kla_dtype& d, int64_t T) {
    return known_dtype(d) ? kla::scan_tile(d, T) : kla::FwdTile{kla::kFwdRows, kla::kFwdWaves};
}

struct Buffer {
    const void* p;
    size_t bytes;
    const char* name;
    bool written;
};

// No written buffer may overlap any other buffer.
kla_status check_overlaps(const Buffer* bufs, int n) {
    for (int i = 0; i < n; ++i) {
        if (!bufs[i].written) continue;
        for (int j = 0; j < n; ++j)
            if (j != i && overlaps(bufs[i].p, bufs[i].bytes, bufs[j].p, bufs[j].bytes))
                return fail(KLA_ERR_INVALID_ARG, "%s overlaps %s", bufs[i].name, bufs[j].name);
    }
    return KLA_OK;
}

// Sizes, dtype and the plan shared by both directions.  Sets *empty when some
// size is 0 (nothing to do).
kla_status common_checks(int64_t B, int64_t H, int64_t T, int64_t D, const kla_dtype& dt,
                         int rows, int waves, int mw, int sw, Plan* pl, bool* empty) {
    t_detail[0] = '\0';
    if (B < 0 || H < 0 || T < 0 || D < 0)
        return fail(KLA_ERR_INVALID_ARG, "negative size B=%lld H=%lld T=%lld D=%lld",
                    (long long)B, (long long)H, (long long)T, (long long)D);
    if (!known_dtype(dt))
        return fail(KLA_ERR_UNSUPPORTED, "unknown input dtype %d", int(raw_bits(dt)));
    if (!kla::make_plan(B, H, T, D, rows, waves, mw, sw, pl))
        return fail(KLA_ERR_INVALID_ARG, "sizes overflow: B=%lld H=%lld T=%lld D=%lld",
                    (long long)B, (long long)H, (long long)T, (long long)D);
    *empty = pl->N == 0;
    if (*empty) return KLA_OK;
    if (!pl->offsets_fit)
        return fail(KLA_ERR_UNSUPPORTED,
                    "one [T, D] slab is too large for D = %lld (T*D = %lld elements; when D is not "
                    "a multiple of 64 the limit is about 2^30 elements per 64 channels)",
                    (long long)D, (long long)(T * D));
    return KLA_OK;
}

kla_status check_workspace(void* workspace, size_t bytes, const Plan& pl) {
    if (!workspace) return fail(KLA_ERR_WORKSPACE, "workspace is NULL");
    if (misaligned(workspace, 256)) return fail(KLA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (bytes < pl.ws.bytes)
        return fail(KLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, pl.ws.bytes);
    return KLA_OK;
}

// Workspace of kla_mixer_bwd: the look-back region (shared in turn by the
// forward recompute and the backward kernel), the recomputed float64 states
// after every kMixBwdRows-th row, the per-tile sums of the channel-gate
// gradients, their per-slice totals (kla::mixer_grad_slices) and the
// reduction's arrival counts.
struct MixerBwdLayout {
    Plan fwd, bwd;
    size_t off_bstate, off_partial, off_slices, off_counts, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Bytes of the mixer's boundary states: the float64 pair (lam, eta) of every
// channel after every kMixBwdRows-th token, [ceil(T / kMixBwdRows)][C][2].
size_t mixer_states_bytes(const Plan& pl, int64_t T) {
    const int64_t blocks = (T + kla::kMixBwdRows - 1) / kla::kMixBwdRows;
    return size_t(blocks) * size_t(pl.C) * 2 * sizeof(double);
}

bool mixer_bwd_layout(int64_t B, int64_t H, int64_t T, int64_t D, const kla_dtype& dt,
                      MixerBwdLayout* l) {
    if (!kla::make_plan(B, H, T, D, fwd_rows(dt, true), kla::kFwdWaves, kla::kFwdMatrixWords,
                        kla::kFwdStateWords, &l->fwd) ||
        !kla::make_plan(B, H, T, D, kla::kMixBwdRows, state_bwd_waves(dt, T), kla::kBwdMatrixWords,
                        kla::kBwdStateWords, &l->bwd))
        return false;
    const size_t states = align256(mixer_states_bytes(l->fwd, T));
    l->off_bstate = align256(l->fwd.ws.bytes > l->bwd.ws.bytes ? l->fwd.ws.bytes : l->bwd.ws.bytes);
    l->off_partial = l->off_bstate + states;
    l->off_slices =
        align256(l->off_partial + size_t(l->bwd.n_tiles) * 2 * kla::kWave * sizeof(double));
    const int64_t slices = kla::mixer_grad_slices(B, H, D, l->bwd.n_chunks);
    l->off_counts = align256(l->off_slices + size_t(slices) * 2 * size_t(H * D) * sizeof(double));
    l->bytes = align256(l->off_counts +
                        size_t((H * D + kla::kWave - 1) / kla::kWave) * sizeof(uint32_t));
    return true;
}

// Workspace of kla_scan_bwd_states: the look-back region (shared in turn by
// the forward recompute and the backward kernel) and the recomputed float64
// states after every kMixBwdRows-th row.
bool scan_bwd_states_layout(int64_t B, int64_t H, int64_t T, int64_t D, const kla_dtype& dt,
                            MixerBwdLayout* l) {
    const kla::FwdTile tile = scan_tile(dt, T);
    if (!kla::make_plan(B, H, T, D, tile.rows, tile.waves, kla::kFwdMatrixWords,
                        kla::kFwdStateWords, &l->fwd) ||
        !kla::make_plan(B, H, T, D, kla::kMixBwdRows, state_bwd_waves(dt, T), kla::kBwdMatrixWords,
                        kla::kBwdStateWords, &l->bwd))
        return false;
    l->off_bstate = align256(l->fwd.ws.bytes > l->bwd.ws.bytes ? l->fwd.ws.bytes : l->bwd.ws.bytes);
    l->off_partial = l->off_bstate + align256(mixer_states_bytes(l->fwd, T));
    l->off_slices = l->off_partial;
    l->off_counts = l->off_partial;
    l->bytes = l->off_partial;
    return true;
}

kla_status scan_fwd_impl(const void* a, const void* p, const void* phi, const void* b,
                         const kla_dtype& in_dtype, const float* lam0, const float* eta0,
                         float* lam, float* eta, double* states, int64_t B, int64_t H, int64_t T,
                         int64_t D, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    bool empty = false;
    const kla::FwdTile tile = scan_tile(in_dtype, T);
    kla_status st = common_checks(B, H, T, D, in_dtype, tile.rows, tile.waves,
                                  kla::kFwdMatrixWords, kla::kFwdStateWords,
                                  &pl, &empty);
    if (st != KLA_OK || empty) return st;

    const void* ins[4] = {a, p, phi, b};
    const char* names[4] = {"a", "p", "phi", "b"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(ins[i], esz))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    if (!lam || !eta) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", lam ? "eta" : "lam");
    if (misaligned(lam, 4) || misaligned(eta, 4))
        return fail(KLA_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
    if ((lam0 && misaligned(lam0, 4)) || (eta0 && misaligned(eta0, 4)))
        return fail(KLA_ERR_UNSUPPORTED, "lam0/eta0 must be 4-byte aligned");
    if (states && misaligned(states, 16))
        return fail(KLA_ERR_UNSUPPORTED, "states is not 16-byte aligned");
    if ((st = check_workspace(workspace, workspace_bytes, pl)) != KLA_OK) return st;

    const size_t in_bytes = size_t(pl.N) * esz, out_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4;
    const Buffer bufs[10] = {{a, in_bytes, "a", false},           {p, in_bytes, "p", false},
                             {phi, in_bytes, "phi", false},       {b, in_bytes, "b", false},
                             {lam0, st_bytes, "lam0", false},     {eta0, st_bytes, "eta0", false},
                             {lam, out_bytes, "lam", true},       {eta, out_bytes, "eta", true},
                             {workspace, pl.ws.bytes, "workspace", true},
                             {states, mixer_states_bytes(pl, T), "states", true}};
    if ((st = check_overlaps(bufs, 10)) != KLA_OK) return st;

    kla::FwdArgs args = {};
    args.in[0] = a;
    args.in[1] = p;
    args.in[2] = phi;
    args.in[3] = b;
    args.lam0 = lam0;
    args.eta0 = eta0;
    args.lam = lam;
    args.eta = eta;
    args.T = T;
    args.D = D;
    args.C = pl.C;
    args.G = pl.G;
    args.n_chunks = pl.n_chunks;
    args.n_tiles = pl.n_tiles;
    args.HD = H * D;
    args.bstate = states;
    args.tall = tile.tall();
    args.ws = kla::workspace_view(workspace, pl.ws);
    const hipError_t err = kla::launch_scan_fwd(
        args, in_dtype, states ? kla::FwdMode::kScanTrain : kla::FwdMode::kScan, stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

}  // namespace

extern "C" {

size_t kla_scan_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                   kla_dtype in_dtype) {
    if (!known_dtype(in_dtype)) return 0;
    Plan pl;
    const kla::FwdTile tile = scan_tile(in_dtype, T);
    if (!kla::make_plan(B, H, T, D, tile.rows, tile.waves, kla::kFwdMatrixWords,
                        kla::kFwdStateWords, &pl) || pl.N == 0)
        return 0;
    return pl.ws.bytes;
}

size_t kla_scan_bwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                   kla_dtype in_dtype) {
    if (!known_dtype(in_dtype)) return 0;
    Plan pl;
    if (!kla::make_plan(B, H, T, D, kla::kBwdRows, kla::kBwdWaves, kla::kBwdMatrixWords,
                        kla::kBwdStateWords, &pl) || pl.N == 0)
        return 0;
    return pl.ws.bytes;
}

kla_status kla_scan_fwd(const void* a, const void* p, const void* phi, const void* b,
                        kla_dtype in_dtype, const float* lam0, const float* eta0,
                        float* lam, float* eta, int64_t B, int64_t H, int64_t T, int64_t D,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return scan_fwd_impl(a, p, phi, b, in_dtype, lam0, eta0, lam, eta, nullptr, B, H, T, D,
                         workspace, workspace_bytes, stream);
}

kla_status kla_scan_fwd_states(const void* a, const void* p, const void* phi, const void* b,
                               kla_dtype in_dtype, const float* lam0, const float* eta0,
                               float* lam, float* eta, double* states, int64_t B, int64_t H,
                               int64_t T, int64_t D, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    t_detail[0] = '\0';
    if (!states && B > 0 && H > 0 && T > 0 && D > 0)
        return fail(KLA_ERR_INVALID_ARG, "states is NULL");
    return scan_fwd_impl(a, p, phi, b, in_dtype, lam0, eta0, lam, eta, states, B, H, T, D,
                         workspace, workspace_bytes, stream);
}

size_t kla_scan_states_size(int64_t B, int64_t H, int64_t T, int64_t D) {
    return kla_mixer_states_size(B, H, T, D);
}

size_t kla_scan_lti_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                       kla_dtype in_dtype) {
    if (!known_dtype(in_dtype)) return 0;
    Plan pl;
    if (!kla::make_plan(B, H, T, D, kla::kLtiRows, kla::kLtiWaves, kla::kFwdMatrixWords,
                        kla::kFwdStateWords, &pl) || pl.N == 0)
        return 0;
    return pl.ws.bytes;
}

kla_status kla_scan_lti_fwd(const float* a, const float* p, const float* phi, const void* b,
                            kla_dtype in_dtype, const float* lam0, const float* eta0,
                            float* lam, float* eta, int64_t B, int64_t H, int64_t T, int64_t D,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    bool empty = false;
    kla_status st = common_checks(B, H, T, D, in_dtype, kla::kLtiRows, kla::kLtiWaves,
                                  kla::kFwdMatrixWords, kla::kFwdStateWords, &pl, &empty);
    if (st != KLA_OK || empty) return st;

    const float* gates[3] = {a, p, phi};
    const char* names[3] = {"a", "p", "phi"};
    for (int i = 0; i < 3; ++i) {
        if (!gates[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(gates[i], 4))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not 4-byte aligned", names[i]);
    }
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    if (!b) return fail(KLA_ERR_INVALID_ARG, "b is NULL");
    if (misaligned(b, esz)) return fail(KLA_ERR_UNSUPPORTED, "b is not %zu-byte aligned", esz);
    if (!lam || !eta) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", lam ? "eta" : "lam");
    if (misaligned(lam, 4) || misaligned(eta, 4))
        return fail(KLA_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
    if ((lam0 && misaligned(lam0, 4)) || (eta0 && misaligned(eta0, 4)))
        return fail(KLA_ERR_UNSUPPORTED, "lam0/eta0 must be 4-byte aligned");
    if ((st = check_workspace(workspace, workspace_bytes, pl)) != KLA_OK) return st;

    const size_t in_bytes = size_t(pl.N) * esz, out_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4, ch_bytes = size_t(H * D) * 4;
    const Buffer bufs[9] = {{a, ch_bytes, "a", false},           {p, ch_bytes, "p", false},
                            {phi, ch_bytes, "phi", false},       {b, in_bytes, "b", false},
                            {lam0, st_bytes, "lam0", false},     {eta0, st_bytes, "eta0", false},
                            {lam, out_bytes, "lam", true},       {eta, out_bytes, "eta", true},
                            {workspace, pl.ws.bytes, "workspace", true}};
    if ((st = check_overlaps(bufs, 9)) != KLA_OK) return st;

    kla::FwdArgs args = {};
    args.in[3] = b;
    args.lam0 = lam0;
    args.eta0 = eta0;
    args.lam = lam;
    args.eta = eta;
    args.a_ch = a;
    args.p_ch = p;
    args.phi_ch = phi;
    args.T = T;
    args.D = D;
    args.C = pl.C;
    args.G = pl.G;
    args.n_chunks = pl.n_chunks;
    args.n_tiles = pl.n_tiles;
    args.HD = H * D;
    args.ws = kla::workspace_view(workspace, pl.ws);
    const hipError_t err = kla::launch_scan_fwd(args, in_dtype, kla::FwdMode::kLti,
                                                stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

size_t kla_mixer_bwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                    kla_dtype in_dtype) {
    if (!known_dtype(in_dtype)) return 0;
    MixerBwdLayout l;
    if (!mixer_bwd_layout(B, H, T, D, in_dtype, &l) || l.fwd.N == 0) return 0;
    return l.bytes;
}

kla_status kla_mixer_bwd(const void* k, const void* v, const void* lam_v, const void* q,
                         kla_dtype in_dtype, const float* a, const float* p, const float* lam0,
                         const float* eta0, const double* states, const float* g_out,
                         const float* g_var, float* g_k,
                         float* g_v, float* g_lam_v, float* g_q, float* g_a, float* g_p,
                         float* g_lam0, float* g_eta0, int64_t B, int64_t H, int64_t T,
                         int64_t D, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    bool empty = false;
    kla_status st = common_checks(B, H, T, D, in_dtype, kla::kMixBwdRows, state_bwd_waves(in_dtype, T),
                                  kla::kBwdMatrixWords, kla::kBwdStateWords, &pl, &empty);
    if (st != KLA_OK || empty) return st;
    MixerBwdLayout lay;
    if (!mixer_bwd_layout(B, H, T, D, in_dtype, &lay) || !lay.fwd.offsets_fit)
        return fail(KLA_ERR_UNSUPPORTED, "sizes not supported: B=%lld H=%lld T=%lld D=%lld",
                    (long long)B, (long long)H, (long long)T, (long long)D);

    const void* ins[4] = {k, v, lam_v, q};
    const char* names[4] = {"k", "v", "lam_v", "q"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(ins[i], esz))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    const void* req[9] = {a, p, g_out, g_k, g_v, g_lam_v, g_q, g_a, g_p};
    const char* rnames[9] = {"a", "p", "g_out", "g_k", "g_v", "g_lam_v", "g_q", "g_a", "g_p"};
    for (int i = 0; i < 9; ++i)
        if (!req[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", rnames[i]);
    const void* f32s[14] = {a, p, lam0, eta0, g_out, g_var, g_k, g_v, g_lam_v, g_q, g_a, g_p,
                            g_lam0, g_eta0};
    for (int i = 0; i < 14; ++i)
        if (f32s[i] && misaligned(f32s[i], 4))
            return fail(KLA_ERR_UNSUPPORTED, "float32 arguments must be 4-byte aligned");
    if (states && misaligned(states, 16))
        return fail(KLA_ERR_UNSUPPORTED, "states is not 16-byte aligned");
    if (!workspace) return fail(KLA_ERR_WORKSPACE, "workspace is NULL");
    if (misaligned(workspace, 256))
        return fail(KLA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < lay.bytes)
        return fail(KLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    lay.bytes);

    const size_t in_bytes = size_t(pl.N) * esz, f_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4, ch_bytes = size_t(H * D) * 4;
    const Buffer bufs[20] = {
        {k, in_bytes, "k", false},            {v, in_bytes, "v", false},
        {lam_v, in_bytes, "lam_v", false},    {q, in_bytes, "q", false},
        {a, ch_bytes, "a", false},            {p, ch_bytes, "p", false},
        {lam0, st_bytes, "lam0", false},      {eta0, st_bytes, "eta0", false},
        {g_out, f_bytes, "g_out", false},     {g_var, f_bytes, "g_var", false},
        {g_k, f_bytes, "g_k", true},          {g_v, f_bytes, "g_v", true},
        {g_lam_v, f_bytes, "g_lam_v", true},  {g_q, f_bytes, "g_q", true},
        {g_a, ch_bytes, "g_a", true},         {g_p, ch_bytes, "g_p", true},
        {g_lam0, st_bytes, "g_lam0", true},   {g_eta0, st_bytes, "g_eta0", true},
        {workspace, lay.bytes, "workspace", true},
        {states, mixer_states_bytes(lay.fwd, T), "states", false}};
    if ((st = check_overlaps(bufs, 20)) != KLA_OK) return st;

    char* ws = static_cast<char*>(workspace);
    const hipStream_t s = stream;
    hipError_t err = hipSuccess;
    const double* bstate = states;
    if (!bstate) {
        // 1. recompute the forward states at every kMixBwdRows-th row (unless
        //    the forward call kept them)
        double* rec = reinterpret_cast<double*>(ws + lay.off_bstate);
        bstate = rec;
        kla::FwdArgs fa = {};
        fa.in[0] = k;
        fa.in[1] = v;
        fa.in[2] = lam_v;
        fa.lam0 = lam0;
        fa.eta0 = eta0;
        fa.bstate = rec;
        fa.a_ch = a;
        fa.p_ch = p;
        fa.T = T;
        fa.D = D;
        fa.C = lay.fwd.C;
        fa.G = lay.fwd.G;
        fa.n_chunks = lay.fwd.n_chunks;
        fa.n_tiles = lay.fwd.n_tiles;
        fa.HD = H * D;
        fa.ws = kla::workspace_view(workspace, lay.fwd.ws);
        err = kla::launch_scan_fwd(fa, in_dtype, kla::FwdMode::kMixerState, s);
        if (err != hipSuccess)
            return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    }

    // 2. the adjoint scan with the mixer's front and back ends
    kla::StateBwdArgs ba = {};
    ba.in[0] = k;
    ba.in[1] = v;
    ba.in[2] = lam_v;
    ba.in[3] = q;
    ba.a_ch = a;
    ba.p_ch = p;
    ba.lam0 = lam0;
    ba.eta0 = eta0;
    ba.bstate = bstate;
    ba.g0 = g_out;
    ba.g1 = g_var;
    ba.out[0] = g_k;
    ba.out[1] = g_v;
    ba.out[2] = g_lam_v;
    ba.out[3] = g_q;
    ba.g_lam0 = g_lam0;
    ba.g_eta0 = g_eta0;
    ba.partial = reinterpret_cast<double*>(ws + lay.off_partial);
    ba.counts = reinterpret_cast<uint32_t*>(ws + lay.off_counts);
    ba.n_counts = (H * D + kla::kWave - 1) / kla::kWave;
    ba.waves = state_bwd_waves(in_dtype, T);
    ba.T = T;
    ba.D = D;
    ba.C = lay.bwd.C;
    ba.G = lay.bwd.G;
    ba.n_chunks = lay.bwd.n_chunks;
    ba.n_tiles = lay.bwd.n_tiles;
    ba.HD = H * D;
    ba.ws = kla::workspace_view(workspace, lay.bwd.ws);
    err = kla::launch_state_bwd(ba, in_dtype, kla::StateBwdMode::kMixer, s);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));

    // 3. channel-gate gradients
    err = kla::launch_mixer_grad_reduce(ba.partial,
                                        reinterpret_cast<double*>(ws + lay.off_slices),
                                        ba.counts, g_a, g_p, B, H, D, lay.bwd.G,
                                        lay.bwd.n_chunks, s);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

size_t kla_mixer_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                    kla_dtype in_dtype) {
    if (!known_dtype(in_dtype)) return 0;
    Plan pl;
    if (!kla::make_plan(B, H, T, D, fwd_rows(in_dtype, true), kla::kFwdWaves,
                        kla::kFwdMatrixWords, kla::kFwdStateWords, &pl) || pl.N == 0)
        return 0;
    return pl.ws.bytes;
}

size_t kla_mixer_states_size(int64_t B, int64_t H, int64_t T, int64_t D) {
    Plan pl;
    if (!kla::make_plan(B, H, T, D, kla::kFwdRows, kla::kFwdWaves, kla::kFwdMatrixWords,
                        kla::kFwdStateWords, &pl) || pl.N == 0)
        return 0;
    return mixer_states_bytes(pl, T);
}

kla_status kla_mixer_fwd(const void* k, const void* v, const void* lam_v, const void* q,
                         kla_dtype in_dtype, const float* a, const float* p, const float* lam0,
                         const float* eta0, float* out, float* var, float* lam_T, float* eta_T,
                         double* states, int64_t B, int64_t H, int64_t T, int64_t D,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    bool empty = false;
    kla_status st = common_checks(B, H, T, D, in_dtype, fwd_rows(in_dtype, true),
                                  kla::kFwdWaves, kla::kFwdMatrixWords, kla::kFwdStateWords,
                                  &pl, &empty);
    if (st != KLA_OK || empty) return st;

    const void* ins[4] = {k, v, lam_v, q};
    const char* names[4] = {"k", "v", "lam_v", "q"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(ins[i], esz))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    if (!a || !p) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", a ? "p" : "a");
    if (!out) return fail(KLA_ERR_INVALID_ARG, "out is NULL");
    if (!lam_T != !eta_T)
        return fail(KLA_ERR_INVALID_ARG, "lam_T and eta_T must both be given or both be NULL");
    const void* f32s[8] = {a, p, lam0, eta0, out, var, lam_T, eta_T};
    for (int i = 0; i < 8; ++i)
        if (f32s[i] && misaligned(f32s[i], 4))
            return fail(KLA_ERR_UNSUPPORTED, "float32 arguments must be 4-byte aligned");
    if (states && misaligned(states, 16))
        return fail(KLA_ERR_UNSUPPORTED, "states is not 16-byte aligned");
    if ((st = check_workspace(workspace, workspace_bytes, pl)) != KLA_OK) return st;

    const size_t in_bytes = size_t(pl.N) * esz, out_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4, ch_bytes = size_t(H * D) * 4;
    const Buffer bufs[14] = {{k, in_bytes, "k", false},           {v, in_bytes, "v", false},
                             {lam_v, in_bytes, "lam_v", false},   {q, in_bytes, "q", false},
                             {a, ch_bytes, "a", false},           {p, ch_bytes, "p", false},
                             {lam0, st_bytes, "lam0", false},     {eta0, st_bytes, "eta0", false},
                             {out, out_bytes, "out", true},       {var, out_bytes, "var", true},
                             {lam_T, st_bytes, "lam_T", true},    {eta_T, st_bytes, "eta_T", true},
                             {workspace, pl.ws.bytes, "workspace", true},
                             {states, mixer_states_bytes(pl, T), "states", true}};
    if ((st = check_overlaps(bufs, 14)) != KLA_OK) return st;

    kla::FwdArgs args = {};
    args.in[0] = k;
    args.in[1] = v;
    args.in[2] = lam_v;
    args.in[3] = q;
    args.lam0 = lam0;
    args.eta0 = eta0;
    args.lam = out;
    args.eta = var;
    args.a_ch = a;
    args.p_ch = p;
    args.lam_T = lam_T;
    args.eta_T = eta_T;
    args.bstate = states;
    args.T = T;
    args.D = D;
    args.C = pl.C;
    args.G = pl.G;
    args.n_chunks = pl.n_chunks;
    args.n_tiles = pl.n_tiles;
    args.HD = H * D;
    args.ws = kla::workspace_view(workspace, pl.ws);
    const hipError_t err = kla::launch_scan_fwd(
        args, in_dtype, states ? kla::FwdMode::kMixerTrain : kla::FwdMode::kMixer,
        stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

kla_status kla_scan_bwd(const void* a, const void* p, kla_dtype in_dtype,
                        const float* lam0, const float* eta0, const float* lam,
                        const float* eta, const float* g_lam, const float* g_eta,
                        float* g_a, float* g_p, float* g_phi, float* g_b, float* g_lam0,
                        float* g_eta0, int64_t B, int64_t H, int64_t T, int64_t D,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    bool empty = false;
    kla_status st = common_checks(B, H, T, D, in_dtype, kla::kBwdRows, kla::kBwdWaves,
                                  kla::kBwdMatrixWords, kla::kBwdStateWords, &pl, &empty);
    if (st != KLA_OK || empty) return st;

    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    if (!a || !p) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", a ? "p" : "a");
    if (misaligned(a, esz) || misaligned(p, esz))
        return fail(KLA_ERR_UNSUPPORTED, "gates must be %zu-byte aligned", esz);
    if (!lam || !eta) return fail(KLA_ERR_INVALID_ARG, "saved %s is NULL", lam ? "eta" : "lam");
    float* outs[4] = {g_a, g_p, g_phi, g_b};
    const char* onames[4] = {"g_a", "g_p", "g_phi", "g_b"};
    for (int i = 0; i < 4; ++i)
        if (!outs[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", onames[i]);
    const void* f32s[12] = {lam0, eta0, lam, eta, g_lam, g_eta, g_a, g_p, g_phi, g_b, g_lam0, g_eta0};
    for (int i = 0; i < 12; ++i)
        if (f32s[i] && misaligned(f32s[i], 4))
            return fail(KLA_ERR_UNSUPPORTED, "float32 arguments must be 4-byte aligned");
    if ((st = check_workspace(workspace, workspace_bytes, pl)) != KLA_OK) return st;

    const size_t in_bytes = size_t(pl.N) * esz, f_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4;
    const Buffer bufs[15] = {
        {a, in_bytes, "a", false},           {p, in_bytes, "p", false},
        {lam0, st_bytes, "lam0", false},     {eta0, st_bytes, "eta0", false},
        {lam, f_bytes, "lam", false},        {eta, f_bytes, "eta", false},
        {g_lam, f_bytes, "g_lam", false},    {g_eta, f_bytes, "g_eta", false},
        {g_a, f_bytes, "g_a", true},         {g_p, f_bytes, "g_p", true},
        {g_phi, f_bytes, "g_phi", true},     {g_b, f_bytes, "g_b", true},
        {g_lam0, st_bytes, "g_lam0", true},  {g_eta0, st_bytes, "g_eta0", true},
        {workspace, pl.ws.bytes, "workspace", true}};
    if ((st = check_overlaps(bufs, 15)) != KLA_OK) return st;

    kla::BwdArgs args;
    args.a = a;
    args.p = p;
    args.lam0 = lam0;
    args.eta0 = eta0;
    args.lam = lam;
    args.eta = eta;
    args.g_lam = g_lam;
    args.g_eta = g_eta;
    args.g_a = g_a;
    args.g_p = g_p;
    args.g_phi = g_phi;
    args.g_b = g_b;
    args.g_lam0 = g_lam0;
    args.g_eta0 = g_eta0;
    args.T = T;
    args.D = D;
    args.C = pl.C;
    args.G = pl.G;
    args.n_chunks = pl.n_chunks;
    args.n_tiles = pl.n_tiles;
    args.ws = kla::workspace_view(workspace, pl.ws);
    const hipError_t err =
        kla::launch_scan_bwd(args, in_dtype, stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

size_t kla_scan_bwd_states_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                          kla_dtype in_dtype) {
    if (!known_dtype(in_dtype)) return 0;
    MixerBwdLayout lay;
    if (!scan_bwd_states_layout(B, H, T, D, in_dtype, &lay) || lay.fwd.N == 0) return 0;
    return lay.bytes;
}

kla_status kla_scan_bwd_states(const void* a, const void* p, const void* phi, const void* b,
                               kla_dtype in_dtype, const float* lam0, const float* eta0,
                               const double* states, const float* g_lam, const float* g_eta,
                               float* g_a, float* g_p, float* g_phi, float* g_b, float* g_lam0,
                               float* g_eta0, int64_t B, int64_t H, int64_t T, int64_t D,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan pl;
    bool empty = false;
    kla_status st = common_checks(B, H, T, D, in_dtype, kla::kMixBwdRows, state_bwd_waves(in_dtype, T),
                                  kla::kBwdMatrixWords, kla::kBwdStateWords, &pl, &empty);
    if (st != KLA_OK || empty) return st;
    MixerBwdLayout lay;
    if (!scan_bwd_states_layout(B, H, T, D, in_dtype, &lay) || !lay.fwd.offsets_fit)
        return fail(KLA_ERR_UNSUPPORTED, "sizes not supported: B=%lld H=%lld T=%lld D=%lld",
                    (long long)B, (long long)H, (long long)T, (long long)D);

    const void* ins[4] = {a, p, phi, b};
    const char* names[4] = {"a", "p", "phi", "b"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(ins[i], esz))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    const void* req[4] = {g_a, g_p, g_phi, g_b};
    const char* rnames[4] = {"g_a", "g_p", "g_phi", "g_b"};
    for (int i = 0; i < 4; ++i)
        if (!req[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", rnames[i]);
    const void* f32s[10] = {lam0, eta0, g_lam, g_eta, g_a, g_p, g_phi, g_b, g_lam0, g_eta0};
    for (int i = 0; i < 10; ++i)
        if (f32s[i] && misaligned(f32s[i], 4))
            return fail(KLA_ERR_UNSUPPORTED, "float32 arguments must be 4-byte aligned");
    if (states && misaligned(states, 16))
        return fail(KLA_ERR_UNSUPPORTED, "states is not 16-byte aligned");
    if (!workspace) return fail(KLA_ERR_WORKSPACE, "workspace is NULL");
    if (misaligned(workspace, 256))
        return fail(KLA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < lay.bytes)
        return fail(KLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    lay.bytes);

    const size_t in_bytes = size_t(pl.N) * esz, f_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4;
    const Buffer bufs[16] = {
        {a, in_bytes, "a", false},           {p, in_bytes, "p", false},
        {phi, in_bytes, "phi", false},       {b, in_bytes, "b", false},
        {lam0, st_bytes, "lam0", false},     {eta0, st_bytes, "eta0", false},
        {g_lam, f_bytes, "g_lam", false},    {g_eta, f_bytes, "g_eta", false},
        {g_a, f_bytes, "g_a", true},         {g_p, f_bytes, "g_p", true},
        {g_phi, f_bytes, "g_phi", true},     {g_b, f_bytes, "g_b", true},
        {g_lam0, st_bytes, "g_lam0", true},  {g_eta0, st_bytes, "g_eta0", true},
        {workspace, lay.bytes, "workspace", true},
        {states, mixer_states_bytes(lay.fwd, T), "states", false}};
    if ((st = check_overlaps(bufs, 16)) != KLA_OK) return st;

    char* ws = static_cast<char*>(workspace);
    hipError_t err = hipSuccess;
    const double* bstate = states;
    if (!bstate) {
        // 1. recompute the forward states at every kMixBwdRows-th row (unless
        //    the forward call kept them)
        double* rec = reinterpret_cast<double*>(ws + lay.off_bstate);
        bstate = rec;
        kla::FwdArgs fa = {};
        fa.in[0] = a;
        fa.in[1] = p;
        fa.in[2] = phi;
        fa.in[3] = b;
        fa.lam0 = lam0;
        fa.eta0 = eta0;
        fa.bstate = rec;
        fa.T = T;
        fa.D = D;
        fa.C = lay.fwd.C;
        fa.G = lay.fwd.G;
        fa.n_chunks = lay.fwd.n_chunks;
        fa.n_tiles = lay.fwd.n_tiles;
        fa.HD = H * D;
        fa.tall = scan_tile(in_dtype, T).tall();
        fa.ws = kla::workspace_view(workspace, lay.fwd.ws);
        err = kla::launch_scan_fwd(fa, in_dtype, kla::FwdMode::kScanState, stream);
        if (err != hipSuccess)
            return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    }

    // 2. the adjoint scan, replaying each wave's rows from the states
    kla::StateBwdArgs ba = {};
    ba.in[0] = a;
    ba.in[1] = p;
    ba.in[2] = phi;
    ba.in[3] = b;
    ba.lam0 = lam0;
    ba.eta0 = eta0;
    ba.bstate = bstate;
    ba.g0 = g_lam;
    ba.g1 = g_eta;
    ba.out[0] = g_a;
    ba.out[1] = g_p;
    ba.out[2] = g_phi;
    ba.out[3] = g_b;
    ba.g_lam0 = g_lam0;
    ba.g_eta0 = g_eta0;
    ba.waves = state_bwd_waves(in_dtype, T);
    ba.T = T;
    ba.D = D;
    ba.C = lay.bwd.C;
    ba.G = lay.bwd.G;
    ba.n_chunks = lay.bwd.n_chunks;
    ba.n_tiles = lay.bwd.n_tiles;
    ba.HD = H * D;
    ba.ws = kla::workspace_view(workspace, lay.bwd.ws);
    err = kla::launch_state_bwd(ba, in_dtype, kla::StateBwdMode::kScan, stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

kla_status kla_decode_step(const void* a, const void* p, const void* phi, const void* b,
                           kla_dtype in_dtype, float* lam, float* eta, int64_t n_channels,
                           hipStream_t stream) {
    t_detail[0] = '\0';
    if (n_channels < 0)
        return fail(KLA_ERR_INVALID_ARG, "negative channel count %lld", (long long)n_channels);
    if (!known_dtype(in_dtype))
        return fail(KLA_ERR_UNSUPPORTED, "unknown input dtype %d", int(raw_bits(in_dtype)));
    if (n_channels == 0) return KLA_OK;
    if (n_channels > INT64_MAX / 8)
        return fail(KLA_ERR_INVALID_ARG, "channel count overflows");
    const void* ins[4] = {a, p, phi, b};
    const char* names[4] = {"a", "p", "phi", "b"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(ins[i], esz))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    if (!lam || !eta) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", lam ? "eta" : "lam");
    if (misaligned(lam, 4) || misaligned(eta, 4))
        return fail(KLA_ERR_UNSUPPORTED, "lam/eta must be 4-byte aligned");
    const size_t in_bytes = size_t(n_channels) * esz, st_bytes = size_t(n_channels) * 4;
    const Buffer bufs[6] = {{a, in_bytes, "a", false},     {p, in_bytes, "p", false},
                            {phi, in_bytes, "phi", false}, {b, in_bytes, "b", false},
                            {lam, st_bytes, "lam", true},  {eta, st_bytes, "eta", true}};
    kla_status st = check_overlaps(bufs, 6);
    if (st != KLA_OK) return st;
    const hipError_t err = kla::launch_decode(a, p, phi, b, in_dtype, lam, eta, n_channels,
                                              stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

kla_status kla_mixer_decode_step(const void* k, const void* v, const void* lam_v, const void* q,
                                 kla_dtype in_dtype, const float* a, const float* p, float* lam,
                                 float* eta, float* out, float* var, int64_t n_channels,
                                 int64_t hd, hipStream_t stream) {
    t_detail[0] = '\0';
    if (n_channels < 0 || hd < 0)
        return fail(KLA_ERR_INVALID_ARG, "negative size n_channels=%lld hd=%lld",
                    (long long)n_channels, (long long)hd);
    if (!known_dtype(in_dtype))
        return fail(KLA_ERR_UNSUPPORTED, "unknown input dtype %d", int(raw_bits(in_dtype)));
    if (n_channels == 0) return KLA_OK;
    if (hd == 0 || n_channels % hd != 0)
        return fail(KLA_ERR_INVALID_ARG, "n_channels=%lld is not a multiple of hd=%lld",
                    (long long)n_channels, (long long)hd);
    if (n_channels > INT64_MAX / 8)
        return fail(KLA_ERR_INVALID_ARG, "channel count overflows");
    const void* ins[4] = {k, v, lam_v, q};
    const char* names[4] = {"k", "v", "lam_v", "q"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (misaligned(ins[i], esz))
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    const void* req[5] = {a, p, lam, eta, out};
    const char* rnames[5] = {"a", "p", "lam", "eta", "out"};
    for (int i = 0; i < 5; ++i)
        if (!req[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", rnames[i]);
    const void* f32s[6] = {a, p, lam, eta, out, var};
    for (int i = 0; i < 6; ++i)
        if (f32s[i] && misaligned(f32s[i], 4))
            return fail(KLA_ERR_UNSUPPORTED, "float32 arguments must be 4-byte aligned");
    const size_t in_bytes = size_t(n_channels) * esz, f_bytes = size_t(n_channels) * 4;
    const size_t ch_bytes = size_t(hd) * 4;
    const Buffer bufs[10] = {{k, in_bytes, "k", false},         {v, in_bytes, "v", false},
                             {lam_v, in_bytes, "lam_v", false}, {q, in_bytes, "q", false},
                             {a, ch_bytes, "a", false},         {p, ch_bytes, "p", false},
                             {lam, f_bytes, "lam", true},       {eta, f_bytes, "eta", true},
                             {out, f_bytes, "out", true},       {var, f_bytes, "var", true}};
    kla_status st = check_overlaps(bufs, 10);
    if (st != KLA_OK) return st;
    const hipError_t err =
        kla::launch_mixer_decode(k, v, lam_v, q, in_dtype, a, p, lam, eta, out, var, n_channels,
                                 hd, stream);
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

kla_status kla_workspace_health(void* workspace, uint32_t* flags_out, hipStream_t stream) {
    t_detail[0] = '\0';
    if (!workspace) return fail(KLA_ERR_WORKSPACE, "workspace is NULL");
    if (!flags_out) return fail(KLA_ERR_INVALID_ARG, "flags_out is NULL");
    hipStream_t s = stream;
    uint32_t* word = static_cast<uint32_t*>(workspace) + 3;
    uint32_t host = 0;
    hipError_t err = hipMemcpyAsync(&host, word, sizeof(host), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err == hipSuccess && host != 0) {
        const uint32_t zero = 0;
        err = hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
        if (err == hipSuccess) err = hipStreamSynchronize(s);
    }
    if (err != hipSuccess) return fail(KLA_ERR_HIP, "health read: %s", hipGetErrorString(err));
    *flags_out = host;
    return KLA_OK;
}

const char* kla_status_string(kla_status s) {
    switch (raw_bits(s)) {
        case KLA_OK: return "KLA_OK";
        case KLA_ERR_INVALID_ARG: return "KLA_ERR_INVALID_ARG";
        case KLA_ERR_UNSUPPORTED: return "KLA_ERR_UNSUPPORTED";
        case KLA_ERR_WORKSPACE: return "KLA_ERR_WORKSPACE";
        case KLA_ERR_HIP: return "KLA_ERR_HIP";
    }
    return "KLA_ERR_UNKNOWN";
}

const char* kla_last_error_detail(void) { return t_detail; }

}  // extern "C"

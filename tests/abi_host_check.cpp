// abi_host_check.cpp -- drives the host side of libkla's C ABI (argument
// validation, plans, workspace sizing, error reporting) under AddressSanitizer
// and UndefinedBehaviorSanitizer, without a GPU.  It is linked against
// kla_api.cpp alone: the kernel launchers below are stand-ins that record the
// launch and report a HIP error, so calls with valid arguments come back as
// KLA_ERR_HIP and every other call must be refused before any launch.  Device
// pointers are fake addresses that are never dereferenced.
//
// Built and run by tests/test_abi_sanitized.py; prints "all checks passed".

#include <stdio.h>
#include <string.h>

#include "kla.h"
#include "kla_internal.h"

namespace kla {

static int g_launches = 0;

hipError_t launch_scan_fwd(const FwdArgs&, kla_dtype, FwdMode, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_scan_bwd(const BwdArgs&, kla_dtype, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_state_bwd(const StateBwdArgs&, kla_dtype, StateBwdMode, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_mixer_grad_reduce(const double*, double*, uint32_t*, float*, float*, int64_t,
                                    int64_t, int64_t, int64_t, int64_t, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_decode(const void*, const void*, const void*, const void*, kla_dtype, float*,
                         float*, int64_t, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_mixer_decode(const void*, const void*, const void*, const void*, kla_dtype,
                               const float*, const float*, float*, float*, float*, float*,
                               int64_t, int64_t, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;
}

}  // namespace kla

static int g_failures = 0;

static void expect(const char* what, int got, int want, int launched, int want_launch) {
    if (got != want || launched != want_launch) {
        printf("FAIL %s: status %d (want %d), launches %d (want %d), detail '%s'\n", what, got,
               want, launched, want_launch, kla_last_error_detail());
        ++g_failures;
    }
}

// This program stands in for a C caller, for which a dtype or status argument
// is a plain int: out-of-range codes are passed through their object
// representation, so the enum checker is off where the program handles them.
#define C_CALLER __attribute__((no_sanitize("enum")))
C_CALLER static kla_dtype dtype_code(int32_t v) {
    kla_dtype d;
    memcpy(&d, &v, sizeof(d));
    return d;
}
C_CALLER static const char* status_text(int32_t v) {
    kla_status s;
    memcpy(&s, &v, sizeof(s));
    return kla_status_string(s);
}

static void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }
static float* F(uintptr_t x) { return reinterpret_cast<float*>(x); }
static double* Dp(uintptr_t x) { return reinterpret_cast<double*>(x); }

// Runs `call` and checks its status and whether it reached a launch.
#define CHECK(what, want, launches, call)            \
    do {                                             \
        const int before = kla::g_launches;          \
        const int st = int(call);                    \
        expect(what, st, want, kla::g_launches - before, launches); \
    } while (0)

C_CALLER int main() {
    const int64_t B = 2, H = 3, T = 300, D = 40;
    const size_t N = size_t(B * H * T * D);
    // fake, disjoint, 256-aligned device ranges
    const uintptr_t base = uintptr_t(1) << 40, step = uintptr_t(1) << 32;
    auto at = [&](int i) { return base + uintptr_t(i) * step; };
    const size_t ws_fwd = kla_scan_fwd_workspace_size(B, H, T, D, KLA_DTYPE_F32);
    const size_t ws_bwd = kla_scan_bwd_workspace_size(B, H, T, D, KLA_DTYPE_F32);
    const size_t ws_lti = kla_scan_lti_fwd_workspace_size(B, H, T, D, KLA_DTYPE_F32);
    const size_t ws_mix = kla_mixer_fwd_workspace_size(B, H, T, D, KLA_DTYPE_BF16);
    const size_t ws_mbw = kla_mixer_bwd_workspace_size(B, H, T, D, KLA_DTYPE_F32);
    if (!ws_fwd || !ws_bwd || !ws_lti || !ws_mix || !ws_mbw) {
        printf("FAIL workspace sizes\n");
        return 1;
    }

    // ---- sizing: empty, negative, overflowing, unknown dtype ----
    if (kla_scan_fwd_workspace_size(0, H, T, D, KLA_DTYPE_F32) != 0 ||
        kla_scan_fwd_workspace_size(-1, H, T, D, KLA_DTYPE_F32) != 0 ||
        kla_scan_fwd_workspace_size(INT64_MAX, INT64_MAX, T, D, KLA_DTYPE_F32) != 0 ||
        kla_scan_fwd_workspace_size(B, H, T, D, dtype_code(7)) != 0 ||
        kla_mixer_states_size(B, H, INT64_MAX / 2, D) != 0 ||
        kla_mixer_bwd_workspace_size(INT64_MAX / 4, 4, T, D, KLA_DTYPE_F32) != 0) {
        printf("FAIL sizing of invalid shapes\n");
        ++g_failures;
    }
    for (int s = -1; s <= 5; ++s)
        if (!status_text(s) || !strlen(status_text(s))) {
            printf("FAIL status string %d\n", s);
            ++g_failures;
        }

    // ---- kla_scan_fwd ----
    auto fwd = [&](uintptr_t a, uintptr_t lam, uintptr_t ws, size_t wsb, int64_t t,
                   kla_dtype dt) C_CALLER {
        return kla_scan_fwd(P(a), P(at(1)), P(at(2)), P(at(3)), dt, F(at(4)), F(at(5)), F(lam),
                            F(at(7)), B, H, t, D, P(ws), wsb, nullptr);
    };
    CHECK("fwd valid (stand-in launch fails)", KLA_ERR_HIP, 1,
          fwd(at(0), at(6), at(8), ws_fwd, T, KLA_DTYPE_F32));
    CHECK("fwd null gate", KLA_ERR_INVALID_ARG, 0, fwd(0, at(6), at(8), ws_fwd, T, KLA_DTYPE_F32));
    CHECK("fwd misaligned gate", KLA_ERR_UNSUPPORTED, 0,
          fwd(at(0) + 2, at(6), at(8), ws_fwd, T, KLA_DTYPE_F32));
    CHECK("fwd output overlaps a gate", KLA_ERR_INVALID_ARG, 0,
          fwd(at(0), at(0) + 64, at(8), ws_fwd, T, KLA_DTYPE_F32));
    CHECK("fwd output overlaps the workspace", KLA_ERR_INVALID_ARG, 0,
          fwd(at(0), at(8) + 256, at(8), ws_fwd, T, KLA_DTYPE_F32));
    CHECK("fwd small workspace", KLA_ERR_WORKSPACE, 0,
          fwd(at(0), at(6), at(8), ws_fwd - 8, T, KLA_DTYPE_F32));
    CHECK("fwd misaligned workspace", KLA_ERR_WORKSPACE, 0,
          fwd(at(0), at(6), at(8) + 16, ws_fwd, T, KLA_DTYPE_F32));
    CHECK("fwd negative T", KLA_ERR_INVALID_ARG, 0, fwd(at(0), at(6), at(8), ws_fwd, -1,
                                                        KLA_DTYPE_F32));
    CHECK("fwd unknown dtype", KLA_ERR_UNSUPPORTED, 0,
          fwd(at(0), at(6), at(8), ws_fwd, T, dtype_code(-3)));
    CHECK("fwd empty", KLA_OK, 0, fwd(0, 0, 0, 0, 0, KLA_DTYPE_F32));
    // (D = 65: a wave's channels straddle two slabs of T * D elements)
    CHECK("fwd slab too large", KLA_ERR_UNSUPPORTED, 0,
          kla_scan_fwd(P(at(0)), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_F32, nullptr, nullptr,
                       F(at(6)), F(at(7)), 1, 1, int64_t(1) << 25, 65, P(at(8)), SIZE_MAX,
                       nullptr));

    // ---- kla_scan_bwd ----
    auto bwd = [&](uintptr_t lam, uintptr_t g_a, size_t wsb) {
        return kla_scan_bwd(P(at(0)), P(at(1)), KLA_DTYPE_F32, F(at(2)), F(at(3)), F(lam),
                            F(at(5)), F(at(6)), F(at(7)), F(g_a), F(at(9)), F(at(10)),
                            F(at(11)), F(at(12)), F(at(13)), B, H, T, D, P(at(14)), wsb,
                            nullptr);
    };
    CHECK("bwd valid", KLA_ERR_HIP, 1, bwd(at(4), at(8), ws_bwd));
    CHECK("bwd null saved state", KLA_ERR_INVALID_ARG, 0, bwd(0, at(8), ws_bwd));
    CHECK("bwd null gradient", KLA_ERR_INVALID_ARG, 0, bwd(at(4), 0, ws_bwd));
    CHECK("bwd gradient overlaps a gate", KLA_ERR_INVALID_ARG, 0, bwd(at(4), at(1) + 4, ws_bwd));
    CHECK("bwd small workspace", KLA_ERR_WORKSPACE, 0, bwd(at(4), at(8), 256));

    // ---- kla_scan_lti_fwd ----
    auto lti = [&](uintptr_t phi, uintptr_t eta) {
        return kla_scan_lti_fwd(F(at(0)), F(at(1)), F(phi), P(at(3)), KLA_DTYPE_F32, nullptr,
                                nullptr, F(at(6)), F(eta), B, H, T, D, P(at(8)), ws_lti,
                                nullptr);
    };
    CHECK("lti valid", KLA_ERR_HIP, 1, lti(at(2), at(7)));
    CHECK("lti null channel gate", KLA_ERR_INVALID_ARG, 0, lti(0, at(7)));
    CHECK("lti outputs overlap", KLA_ERR_INVALID_ARG, 0, lti(at(2), at(6) + 4 * N - 4));

    // ---- kla_mixer_fwd (bf16 token inputs) ----
    auto mix = [&](uintptr_t k, uintptr_t lam_T, uintptr_t eta_T, uintptr_t states) {
        return kla_mixer_fwd(P(k), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_BF16, F(at(4)),
                             F(at(5)), nullptr, nullptr, F(at(6)), F(at(7)), F(lam_T), F(eta_T),
                             Dp(states), B, H, T, D, P(at(8)), ws_mix, nullptr);
    };
    CHECK("mixer valid", KLA_ERR_HIP, 1, mix(at(0), 0, 0, 0));
    CHECK("mixer valid with final state and states", KLA_ERR_HIP, 1,
          mix(at(0), at(9), at(10), at(11)));
    CHECK("mixer one final state", KLA_ERR_INVALID_ARG, 0, mix(at(0), at(9), 0, 0));
    CHECK("mixer misaligned states", KLA_ERR_UNSUPPORTED, 0, mix(at(0), 0, 0, at(11) + 8));
    CHECK("mixer states overlap the readout", KLA_ERR_INVALID_ARG, 0,
          mix(at(0), 0, 0, at(6) + 4 * N - 16));
    CHECK("mixer misaligned bf16 input", KLA_ERR_UNSUPPORTED, 0, mix(at(0) + 1, 0, 0, 0));

    // ---- kla_mixer_bwd (recomputing, and from kept states) ----
    auto mbw = [&](uintptr_t states, uintptr_t g_k, size_t wsb) {
        return kla_mixer_bwd(P(at(0)), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_F32, F(at(4)),
                             F(at(5)), nullptr, nullptr, Dp(states), F(at(6)), F(at(7)), F(g_k),
                             F(at(9)), F(at(10)), F(at(11)), F(at(12)), F(at(13)), nullptr,
                             nullptr, B, H, T, D, P(at(14)), wsb, nullptr);
    };
    CHECK("mixer bwd valid, recomputing", KLA_ERR_HIP, 1, mbw(0, at(8), ws_mbw));
    CHECK("mixer bwd valid, kept states", KLA_ERR_HIP, 1, mbw(at(15), at(8), ws_mbw));
    CHECK("mixer bwd gradient over the states", KLA_ERR_INVALID_ARG, 0,
          mbw(at(15), at(15) + 32, ws_mbw));
    CHECK("mixer bwd null gradient", KLA_ERR_INVALID_ARG, 0, mbw(0, 0, ws_mbw));
    CHECK("mixer bwd small workspace", KLA_ERR_WORKSPACE, 0, mbw(0, at(8), ws_mbw - 256));

    // ---- decode steps ----
    CHECK("decode valid", KLA_ERR_HIP, 1,
          kla_decode_step(P(at(0)), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_F32, F(at(4)),
                          F(at(5)), 1000, nullptr));
    CHECK("decode state overlaps a gate", KLA_ERR_INVALID_ARG, 0,
          kla_decode_step(P(at(0)), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_F32, F(at(3) + 8),
                          F(at(5)), 1000, nullptr));
    CHECK("mixer decode valid", KLA_ERR_HIP, 1,
          kla_mixer_decode_step(P(at(0)), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_BF16,
                                F(at(4)), F(at(5)), F(at(6)), F(at(7)), F(at(8)), nullptr,
                                B * H * D, H * D, nullptr));
    CHECK("mixer decode channels not a multiple of H*D", KLA_ERR_INVALID_ARG, 0,
          kla_mixer_decode_step(P(at(0)), P(at(1)), P(at(2)), P(at(3)), KLA_DTYPE_F32,
                                F(at(4)), F(at(5)), F(at(6)), F(at(7)), F(at(8)), nullptr,
                                B * H * D + 1, H * D, nullptr));

    // ---- diagnostics ----
    uint32_t flags = 0;
    CHECK("health of a NULL workspace", KLA_ERR_WORKSPACE, 0,
          kla_workspace_health(nullptr, &flags, nullptr));
    CHECK("health without an output", KLA_ERR_INVALID_ARG, 0,
          kla_workspace_health(P(at(0)), nullptr, nullptr));
    const char* detail = kla_last_error_detail();
    if (!detail || !strlen(detail)) {
        printf("FAIL last error detail is empty\n");
        ++g_failures;
    }

    if (g_failures) {
        printf("%d checks failed\n", g_failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}

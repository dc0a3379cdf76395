// kla_internal.h -- host-side plumbing shared by the libkla sources (not part
// of the public ABI): tiling plans and the kernel launchers.

#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "kla.h"
#include "kla_lookback.h"

namespace kla {

// Tiling of a [B, H, T, D] problem into tiles of 64 channels by `rows` time
// steps, and the workspace those tiles need.
struct Plan {
    int64_t C;         // channels B*H*D
    int64_t N;         // elements B*H*T*D
    int64_t G;         // 64-channel column groups
    int64_t n_chunks;  // tiles along T
    int64_t n_tiles;
    bool offsets_fit;  // per-wave 32-bit byte offsets cannot overflow
    WorkspaceLayout ws;
};

// Records the calling thread's error text (kla_last_error_detail) and
// returns `s`.
kla_status fail(kla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Returns false on negative or overflowing sizes.
bool make_plan(int64_t B, int64_t H, int64_t T, int64_t D, int rows_per_wave,
               int waves, int matrix_words, int state_words, Plan* pl);

// Forward scan.  Scan mode: the four [B, H, T, D] inputs are the gates a, p,
// phi, b and the outputs lam, eta.  LTI mode: only in[3] (b) is a token
// tensor; a_ch, p_ch, phi_ch hold the time-invariant gates; outputs lam, eta.  Mixer mode: the inputs are the token
// tensors k, v, lam_v, q, the gates are a_ch, p_ch per (h, d) channel and
// phi = k^2 lam_v, b = k lam_v v per token, and the outputs are the readout
// out = q * eta / lam, optionally var = 1 / lam and the final state.
struct FwdArgs {
    const void* in[4];     // a, p, phi, b  |  k, v, lam_v, q
    const float* lam0;     // may be NULL (1)
    const float* eta0;     // may be NULL (0)
    float* lam;            // scan: lam     | mixer: out
    float* eta;            // scan: eta     | mixer: var (may be NULL)
    const float* a_ch;     // mixer, LTI: [H, D]
    const float* p_ch;     // mixer, LTI: [H, D]
    const float* phi_ch;   // LTI: [H, D]
    float* lam_T;          // mixer: final state [B, H, D] (may be NULL)
    float* eta_T;
    double* bstate;        // mixer states: [ceil(T / kMixBwdRows)][C][2] float64
                           // (kMixerState, kMixerTrain)
    bool tall;             // scan modes: the tall tile (scan_tile)
    int64_t T, D, C, G, n_chunks, n_tiles, HD;
    Workspace ws;
};

struct BwdArgs {
    const void* a;
    const void* p;
    const float* lam0;   // may be NULL (1)
    const float* eta0;   // may be NULL (0)
    const float* lam;    // forward outputs
    const float* eta;
    const float* g_lam;  // may be NULL (0)
    const float* g_eta;  // may be NULL (0)
    float* g_a;
    float* g_p;
    float* g_phi;
    float* g_b;
    float* g_lam0;  // may be NULL (not written)
    float* g_eta0;  // may be NULL (not written)
    int64_t T, D, C, G, n_chunks, n_tiles;
    Workspace ws;
};

// Tile shapes (rows per wave, waves per workgroup) and record sizes.
constexpr int kFwdRows = 28, kFwdWaves = 4, kFwdMatrixWords = 7, kFwdStateWords = 2;
// bfloat16 rows take half the registers (two rows to a register), so their
// tiles are sized on their own: 24 rows per wave let the scan run 4 waves per
// SIMD, and the mixer modes, which need more registers per row, take 36.
constexpr int kScanRowsBf16 = 24, kMixerRowsBf16 = 36;
// Rows per wave of the forward kernel for an input type, in the scan and LTI
// modes or in the mixer modes.
inline int fwd_rows(kla_dtype dt, bool mixer) {
    return dt == KLA_DTYPE_F32 ? kFwdRows : mixer ? kMixerRowsBf16 : kScanRowsBf16;
}
// Long float32 sequences take taller tiles in the scan modes: 8 waves of 18
// rows (144-row tiles, two workgroups per CU), which measured 2% faster on
// the long-context shape (1 x 32 x 131072 x 128) and within 1% elsewhere at
// T >= 65536, while shorter sequences are up to 5% faster with the 4-wave
// tiles.
constexpr int kTallRows = 18, kTallWaves = 8;
constexpr int64_t kTallMinT = 65536;
struct FwdTile {
    int rows, waves;
    bool tall() const { return waves == kTallWaves; }
};
// The forward kernel's tile in the scan modes (Scan, ScanState, ScanTrain).
inline FwdTile scan_tile(kla_dtype dt, int64_t T) {
    if (dt == KLA_DTYPE_F32 && T >= kTallMinT) return FwdTile{kTallRows, kTallWaves};
    return FwdTile{fwd_rows(dt, false), kFwdWaves};
}
constexpr int kLtiRows = 64, kLtiWaves = 4;
constexpr int kMixBwdRows = 8;
// Waves per workgroup of the backward kernel from states (kMixBwdRows rows
// each).  float32 inputs: 8 (64-row tiles) from T = 8192 on, 4 (32-row
// tiles, four workgroups per CU) below, which measured 4-10% faster on the
// small-LM layer (T = 2048), level at T = 8192 and 4-7% slower on the long
// context.  bfloat16 inputs: always 4, since their instances fit in 96
// registers and run 5 waves per SIMD, which only workgroups of one wave
// per SIMD can fill (8-13% faster on the 1B-scale layer than 8 waves at 4
// per SIMD).
constexpr int64_t kStateBwdTallT = 8192;
inline int state_bwd_waves(kla_dtype dt, int64_t T) {
    return dt == KLA_DTYPE_F32 && T >= kStateBwdTallT ? 8 : 4;
}
constexpr int kBwdRows = 14, kBwdWaves = 8, kBwdMatrixWords = 6, kBwdStateWords = 2;

// kMixerState: the mixer's gates; writes the float64 states (lam, eta) after
// every kMixBwdRows-th row into FwdArgs::bstate, for the mixer's backward
// pass.  kMixerTrain: kMixer that also writes those states.  kScanState and
// kScanTrain: the same for the scan's gates (states only / lam, eta and the
// states), for the scan's backward pass from states.
enum class FwdMode { kScan, kMixer, kLti, kMixerState, kMixerTrain, kScanState, kScanTrain };
hipError_t launch_scan_fwd(const FwdArgs& args, kla_dtype dtype, FwdMode mode, hipStream_t stream);
hipError_t launch_scan_bwd(const BwdArgs& args, kla_dtype dtype, hipStream_t stream);

// Backward pass from float64 boundary states (the state after every
// kMixBwdRows-th row, written by a forward mode above): each wave replays its
// rows forward from the state before them, then runs the adjoint scan.
//   kMixer: in = k, v, lam_v, q; channel gates a_ch, p_ch; upstream
//           g0 = g_out, g1 = g_var (may be NULL); writes out = g_k, g_v,
//           g_lam_v, g_q and, per tile and lane, the tile's sums of the
//           channel-gate gradients into `partial` ([tile][2][64]).
//   kScan:  in = a, p, phi, b; upstream g0 = g_lam, g1 = g_eta (either may
//           be NULL); writes out = g_a, g_p, g_phi, g_b per token.
// Both write g_lam0, g_eta0 (either may be NULL).
enum class StateBwdMode { kMixer, kScan };
struct StateBwdArgs {
    const void* in[4];
    const float* a_ch;   // kMixer: [H, D]
    const float* p_ch;
    const float* lam0;   // may be NULL (1)
    const float* eta0;   // may be NULL (0)
    const double* bstate;  // forward states after every kMixBwdRows-th row
    const float* g0;
    const float* g1;
    float* out[4];
    float* g_lam0;  // may be NULL
    float* g_eta0;  // may be NULL
    double* partial;  // kMixer only
    uint32_t* counts; // kMixer only: the reduction's arrival counts, zeroed here
    int64_t n_counts;
    int waves;        // state_bwd_waves(dtype, T)
    int64_t T, D, C, G, n_chunks, n_tiles, HD;
    Workspace ws;
};

hipError_t launch_state_bwd(const StateBwdArgs& args, kla_dtype dtype, StateBwdMode mode,
                            hipStream_t stream);
// g_a[h, d], g_p[h, d]: the per-tile sums added over the batch and the chunks
// in a fixed order: in mixer_grad_slices slices of the (b, chunk) pairs
// ([slices][2][H*D] float64 in `slices`), then over the slices by the
// workgroup that finishes its slice last (counts: one uint32 per 64
// channels, zeroed by the backward kernel); with one slice, directly.  A
// slice per kReducePairs pairs (one round of loads per wave of the
// reduction), up to kMaxReduceSlices.
constexpr int64_t kReducePairs = 64;
constexpr int64_t kMaxReduceSlices = 128;
inline int64_t mixer_grad_slices(int64_t B, int64_t H, int64_t D, int64_t n_chunks) {
    (void)H;
    (void)D;
    const int64_t s = (B * n_chunks + kReducePairs - 1) / kReducePairs;
    return s < 1 ? 1 : s > kMaxReduceSlices ? kMaxReduceSlices : s;
}
hipError_t launch_mixer_grad_reduce(const double* partial, double* slices, uint32_t* counts,
                                    float* g_a, float* g_p, int64_t B, int64_t H, int64_t D,
                                    int64_t G, int64_t n_chunks, hipStream_t stream);
hipError_t launch_decode(const void* a, const void* p, const void* phi, const void* b,
                         kla_dtype dtype, float* lam, float* eta, int64_t n, hipStream_t stream);
// One mixer token per channel: k, v, lam_v, q [n] of dtype; a, p [hd] float32
// (channel i uses i % hd); lam, eta updated in place; out (and var unless
// NULL) written.
hipError_t launch_mixer_decode(const void* k, const void* v, const void* lam_v, const void* q,
                               kla_dtype dtype, const float* a, const float* p, float* lam,
                               float* eta, float* out, float* var, int64_t n, int64_t hd,
                               hipStream_t stream);

}  // namespace kla

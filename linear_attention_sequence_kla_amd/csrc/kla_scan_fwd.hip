// kla_scan_fwd.hip -- forward KLA scan kernel for gfx950 (MI355X).
//
// Method (Pith review of arXiv 2602.10743, "What carries the argument" and
// "Circularity check"): per channel, lam_t = M_t(lam_{t-1}) with the Moebius
// matrix M_t = [[1 + p phi, a^2 phi], [p, a^2]], and the information mean
// eta_t = f_t eta_{t-1} + b_t with f_t = a_t / (a_t^2 + p_t lam_{t-1}).
//
// Both maps act linearly on the homogeneous vector (X, Y, Z) with
// lam = X / Z and eta = Y / Z.  One token maps
//     Z' = p X + a^2 Z,   X' = X + phi Z',   Y' = a Y + b Z'
// (so lam' = lam / (a^2 + p lam) + phi and eta' = a eta / (a^2 + p lam) + b).
// As a 3x3 matrix on (X, Y, Z) this is
//     [[1 + p phi, 0, a^2 phi], [b p, a, b a^2], [p, 0, a^2]],
// whose upper-left/corner entries are the Moebius matrix M_t.  Products keep
// the pattern [[A, 0, B], [E, F, G], [C, 0, D]] (7 numbers), and composing
// them is associative (the scan axiom on the same page), so the whole chunk's
// effect is one such matrix and the two recursions of the page become ONE
// scan with ONE carry per chunk.  Matrices and states are projective: any
// positive scale leaves lam and eta unchanged, which the kernel uses to
// renormalise by powers of two.
//
// Kernel structure (single pass; the carry protocol is in kla_lookback.h):
//   * a workgroup of W waves owns one tile: 64 channels (one per lane, so a
//     time row is one coalesced load per wave) by W*L time steps; wave w owns
//     the L rows starting at w*L;
//   * each wave loads its L rows of a, p, phi, b into registers, where they
//     stay until the outputs are written (inputs are read from HBM once);
//   * it folds them into its chunk matrix (float64, renormalised);
//   * wave 0 composes the W chunk matrices, publishes the tile's matrix,
//     looks back over earlier tiles of the same channels for the carry-in
//     state, and publishes the tile's inclusive state;
//   * every wave gets its own carry-in from the tile carry and the chunk
//     matrices of the waves before it, then replays its rows sequentially from
//     on-chip data, writing lam and eta.
//
// The kernel has seven modes (template parameter Mode):
//   * Scan: the four token inputs are the gates a, p, phi, b; writes lam, eta.
//   * Mixer: the fused KLA mixer.  The inputs are the token tensors k, v,
//     lam_v, q and per-channel gates (a, p); phi = k^2 lam_v and b = k lam_v v
//     are formed on the fly (token_gates), and the replay writes the readout
//     q * eta / lam = q * Y / X and the variance 1 / lam = Z / X, so no gate
//     or state tensor crosses HBM.
//   * MixerTrain: Mixer, also writing the boundary states of MixerState
//     (kept by a training caller for the backward pass).  A mode of its own
//     so that the plain mixer's replay carries no extra branch.
//   * MixerState: the mixer's gates, writing the float64 state (lam, eta)
//     after every kMixBwdRows-th row only (the boundary states from which
//     the mixer's backward kernel recomputes its rows' states); q is not
//     read.
//   * Lti: per-channel (a, p, phi) and the token's b only (time-invariant
//     gates; one input row per token, so 64 rows per wave).
//   * ScanState / ScanTrain: the scan's gates, writing the float64 boundary
//     states of MixerState (only them / with lam and eta), from which the
//     scan's backward pass from states recomputes its rows' states.
//
// Arithmetic is float64 for everything carried (chunk matrices, states): the
// exact precision can reach 1e88 and the information mean 1e-51 on hard gates,
// beyond float32's exponent range, and on gfx950 a float64 FMA issues at the
// same rate as an unpacked float32 FMA.  Inputs are float32 or bfloat16 (held
// two rows to a register, with tiles sized for that) and outputs float32.

#include "kla_internal.h"

namespace kla {
namespace {

constexpr int kRenormEvery = 8;  // tokens between renormalisations

// 3x3 projective map [[A, 0, B], [E, F, G], [C, 0, D]] on (lam, eta, 1).
struct Lift {
    double A, B, C, D, E, F, G;
};

// Scales all entries by the power of two that brings the largest to [0.5, 1).
__device__ inline void renorm(Lift& n) {
    const double m = fmax(fmax(fmax(fabs(n.A), fabs(n.B)), fmax(fabs(n.C), fabs(n.D))),
                          fmax(fmax(fabs(n.E), fabs(n.F)), fabs(n.G)));
    const int e = renorm_exponent(m);
    n.A = pow2_scale(n.A, e);
    n.B = pow2_scale(n.B, e);
    n.C = pow2_scale(n.C, e);
    n.D = pow2_scale(n.D, e);
    n.E = pow2_scale(n.E, e);
    n.F = pow2_scale(n.F, e);
    n.G = pow2_scale(n.G, e);
}

// later o earlier: the map that applies `earlier` first.
__device__ inline Lift compose(const Lift& l, const Lift& e) {
    Lift r;
    r.A = fma(l.A, e.A, l.B * e.C);
    r.B = fma(l.A, e.B, l.B * e.D);
    r.C = fma(l.C, e.A, l.D * e.C);
    r.D = fma(l.C, e.B, l.D * e.D);
    r.E = fma(l.E, e.A, fma(l.F, e.E, l.G * e.C));
    r.F = l.F * e.F;
    r.G = fma(l.E, e.B, fma(l.F, e.G, l.G * e.D));
    renorm(r);
    return r;
}

// (lam, eta) <- n(lam, eta).
__device__ inline void apply(const Lift& n, double& lam, double& eta) {
    const double x = fma(n.A, lam, n.B);
    const double y = fma(n.E, lam, fma(n.F, eta, n.G));
    const double r = recip(fma(n.C, lam, n.D));
    lam = x * r;
    eta = y * r;
}

// The chunk matrix of wave j of this workgroup, from LDS.
__device__ inline Lift lds_lift(const double (*s)[7][kWave], int j, int lane) {
    return Lift{s[j][0][lane], s[j][1][lane], s[j][2][lane], s[j][3][lane],
                s[j][4][lane], s[j][5][lane], s[j][6][lane]};
}

// The workgroup's tile matrix: its W chunk matrices composed in time order.
template <int W>
__device__ inline Lift tile_lift(const double (*s)[7][kWave], int lane) {
    Lift t = lds_lift(s, 0, lane);
#pragma unroll 1
    for (int j = 1; j < W; ++j) t = compose(lds_lift(s, j, lane), t);
    return t;
}

__device__ inline void store_lift(double* rec, int lane, const Lift& n) {
    rec_store(rec + 0 * kWave + lane, n.A);
    rec_store(rec + 1 * kWave + lane, n.B);
    rec_store(rec + 2 * kWave + lane, n.C);
    rec_store(rec + 3 * kWave + lane, n.D);
    rec_store(rec + 4 * kWave + lane, n.E);
    rec_store(rec + 5 * kWave + lane, n.F);
    rec_store(rec + 6 * kWave + lane, n.G);
}

__device__ inline Lift load_lift(double* rec, int lane) {
    Lift n;
    n.A = rec_load(rec + 0 * kWave + lane);
    n.B = rec_load(rec + 1 * kWave + lane);
    n.C = rec_load(rec + 2 * kWave + lane);
    n.D = rec_load(rec + 3 * kWave + lane);
    n.E = rec_load(rec + 4 * kWave + lane);
    n.F = rec_load(rec + 5 * kWave + lane);
    n.G = rec_load(rec + 6 * kWave + lane);
    return n;
}

// What the four token inputs are and what the replay writes.
enum class Mode {
    Scan,   // a, p, phi, b per token -> lam, eta
    Mixer,  // k, v, lam_v, q per token, (a, p) per channel -> q eta / lam, 1 / lam
    Lti,    // b per token, (a, p, phi) per channel -> lam, eta
    MixerState,  // k, v, lam_v per token, (a, p) per channel -> boundary (lam, eta)
    MixerTrain,  // Mixer's inputs -> Mixer's outputs and MixerState's
    ScanState,   // Scan's inputs -> boundary (lam, eta) only
    ScanTrain,   // Scan's inputs -> lam, eta and the boundary states
};

// The float64 gates (a, p, phi, b) of one token.  Scan mode reads them from
// the four input rows.  Mixer mode makes them from the token inputs (k, v,
// lam_v, q) and the channel's (a, p): the observation v = k x + noise of
// precision lam_v adds phi = k^2 lam_v to the precision and b = k lam_v v to
// the information mean (the information-form update of the Pith review,
// "Circularity check", with the observation operator k of the ledger).  LTI
// mode takes the channel's time-invariant (a, p, phi) and the token's b.
// Both passes over a row evaluate the same expressions, so they see equal
// gates.
template <Mode M>
__device__ inline void token_gates(float x0, float x1, float x2, float x3, double ac, double pc,
                                   double fc, double& a, double& p, double& ph, double& b) {
    if constexpr (M == Mode::Mixer || M == Mode::MixerState || M == Mode::MixerTrain) {
        const double k = x0, kl = k * double(x2);
        a = ac;
        p = pc;
        ph = kl * k;
        b = kl * double(x1);
    } else if constexpr (M == Mode::Lti) {
        a = ac;
        p = pc;
        ph = fc;
        b = x3;
    } else {
        a = x0;
        p = x1;
        ph = x2;
        b = x3;
    }
}

template <typename In, int L, int W, Mode M>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(3)))
void kla_scan_kernel(FwdArgs g) {
    constexpr bool kMixer = M == Mode::Mixer || M == Mode::MixerTrain;
    constexpr bool kAll = M != Mode::Lti;            // the first three token inputs are read
    constexpr bool kFourth = M != Mode::MixerState;  // the fourth one is read
    __shared__ double s_lift[W][7][kWave];
    __shared__ double s_carry[W][2][kWave];
    static_assert(kFwdMatrixWords == 7 && kFwdStateWords == 2, "record layout");

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t ticket = tile_of_workgroup(blockIdx.x, g.G, g.D, g.n_tiles);
    // This call's tag; only wave 0 (the look-back wave) needs it.  Its load
    // is issued after the tile loads so that it costs no extra latency.
    uint32_t tag = 0;

    if (ticket < g.n_tiles) {
        // ---- tile and lane coordinates ----
        const int64_t c = ticket / g.G;        // chunk along T
        const int64_t grp = ticket - c * g.G;  // 64-channel column group
        const int64_t t0 = (c * W + w) * L;    // first row of this wave
        const int nr = int(min(int64_t(L), g.T - t0));  // rows of this wave (may be <= 0)
        const LaneMap lm = lane_map(grp, t0, lane, g.T, g.D, g.C);
        const uint32_t in_row = uint32_t(g.D * sizeof(In));
        const uint32_t out_row = uint32_t(g.D * sizeof(float));
        // (inputs a mode does not read are NULL and get no address)
        const int64_t in_base = lm.e0 * int64_t(sizeof(In));
        const char* pa = kAll ? static_cast<const char*>(g.in[0]) + in_base : nullptr;
        const char* pp = kAll ? static_cast<const char*>(g.in[1]) + in_base : nullptr;
        const char* pf = kAll ? static_cast<const char*>(g.in[2]) + in_base : nullptr;
        const char* pb = kFourth ? static_cast<const char*>(g.in[3]) + in_base : nullptr;
        // mixer and LTI modes: the channel's time-invariant gates
        double ac = 1.0, pc = 0.0, fc = 0.0;
        if constexpr (M != Mode::Scan) {
            const int64_t hd = lm.qc % g.HD;
            ac = g.a_ch[hd];
            pc = g.p_ch[hd];
            if constexpr (M == Mode::Lti) fc = g.phi_ch[hd];
        }

        // ---- load the wave's rows; rows past T repeat the last row ----
        // (their values only reach chunk matrices that no valid row uses)
        GateRows<In, L> ra, rp, rf, rb;
        if (nr > 0) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const uint32_t off =
                    lm.lane_el * uint32_t(sizeof(In)) + uint32_t(min(i, nr - 1)) * in_row;
                if constexpr (kAll) {
                    ra.load(i, pa, off);
                    rp.load(i, pp, off);
                    rf.load(i, pf, off);
                } else {
                    ra.set(i, 0.0f);
                    rp.set(i, 0.0f);
                    rf.set(i, 0.0f);
                }
                if constexpr (kFourth)
                    rb.load(i, pb, off);
                else
                    rb.set(i, 0.0f);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                ra.set(i, 1.0f);
                rp.set(i, 0.0f);
                rf.set(i, 0.0f);
                rb.set(i, 0.0f);
            }
        }
        if (w == 0) tag = read_tag(g.ws);

        // ---- chunk matrix: the columns (A, E, C) and (B, G, D), and F ----
        Lift m;
        {
            double x1 = 1.0, y1 = 0.0, z1 = 0.0;
            double x3 = 0.0, y3 = 0.0, z3 = 1.0;
            double f = 1.0;
#pragma unroll
            for (int i = 0; i < L; ++i) {
                double a, p, ph, bb;
                token_gates<M>(ra[i], rp[i], rf[i], rb[i], ac, pc, fc, a, p, ph, bb);
                const double a2 = a * a;
                double zn = fma(p, x1, a2 * z1);
                x1 = fma(ph, zn, x1);
                y1 = fma(bb, zn, a * y1);
                z1 = zn;
                zn = fma(p, x3, a2 * z3);
                x3 = fma(ph, zn, x3);
                y3 = fma(bb, zn, a * y3);
                z3 = zn;
                f *= a;
                if ((i % kRenormEvery) == kRenormEvery - 1 || i == L - 1) {
                    m = Lift{x1, x3, z1, z3, y1, f, y3};
                    renorm(m);
                    x1 = m.A; x3 = m.B; z1 = m.C; z3 = m.D; y1 = m.E; f = m.F; y3 = m.G;
                }
            }
        }
        // Keep only the loaded gates (float32, or packed bfloat16) live across
        // the carry exchange: without this barrier the compiler reuses the
        // float64 conversions of the first pass in the second, doubling the
        // registers a tile needs.
        if constexpr (kAll) {
            ra.keep();
            rp.keep();
            rf.keep();
        }
        if constexpr (kFourth) rb.keep();
        s_lift[w][0][lane] = m.A;
        s_lift[w][1][lane] = m.B;
        s_lift[w][2][lane] = m.C;
        s_lift[w][3][lane] = m.D;
        s_lift[w][4][lane] = m.E;
        s_lift[w][5][lane] = m.F;
        s_lift[w][6][lane] = m.G;
        __syncthreads();

        // ---- tile carry (wave 0): publish, look back, publish ----
        if (w == 0) {
            const bool has_next = c + 1 < g.n_chunks;
            double* const matrix = g.ws.matrix;
            double* const state = g.ws.state;
            double lam_in = 1.0, eta_in = 0.0;
            if (c == 0) {
                if (g.lam0) lam_in = g.lam0[lm.qc];
                if (g.eta0) eta_in = g.eta0[lm.qc];
            } else {
                if (has_next) {
                    store_lift(matrix + size_t(ticket) * 7 * kWave, lane,
                               tile_lift<W>(s_lift, lane));
                    publish(&g.ws.flags[ticket], lane, flag_word(tag, kStatusAggregate));
                }
                // Walk back over the flags of this column group to the nearest
                // tile with a published state, then apply the chunk matrices
                // of the tiles after it, oldest first.  (Only one matrix is
                // held at a time, which keeps the registers of the wait low.)
                int64_t j = ticket - g.G;
                uint32_t st;
                while ((st = wait_flag(&g.ws.flags[j], tag, g.ws.header)) == kStatusAggregate)
                    j -= g.G;
                if (st == kStatusInclusive) {
                    lam_in = rec_load(state + size_t(j) * 2 * kWave + lane);
                    eta_in = rec_load(state + size_t(j) * 2 * kWave + kWave + lane);
                    for (int64_t k = j + g.G; k < ticket; k += g.G)
                        apply(load_lift(matrix + size_t(k) * 7 * kWave, lane), lam_in, eta_in);
                }  // else the wait gave up: the health word is set, outputs are wrong
            }
            if (has_next) {
                double l = lam_in, e = eta_in;
                apply(tile_lift<W>(s_lift, lane), l, e);
                rec_store(state + size_t(ticket) * 2 * kWave + lane, l);
                rec_store(state + size_t(ticket) * 2 * kWave + kWave + lane, e);
                publish(&g.ws.flags[ticket], lane, flag_word(tag, kStatusInclusive));
            } else if (g.n_chunks > 1) {
                publish(&g.ws.flags[ticket], lane, flag_word(tag, kStatusFinished));
            }
            // carry-in of every wave: the tile's, then through the earlier
            // waves' chunk matrices (one matrix live at a time)
            s_carry[0][0][lane] = lam_in;
            s_carry[0][1][lane] = eta_in;
#pragma unroll 1
            for (int j = 0; j + 1 < W; ++j) {
                apply(lds_lift(s_lift, j, lane), lam_in, eta_in);
                s_carry[j + 1][0][lane] = lam_in;
                s_carry[j + 1][1][lane] = eta_in;
            }
        }
        __syncthreads();

        // ---- replay the wave's rows from its own carry-in ----
        if (nr > 0) {
            double X = s_carry[w][0][lane], Y = s_carry[w][1][lane], Z = 1.0;
            char* olam = reinterpret_cast<char*>(g.lam) + lm.e0 * int64_t(sizeof(float));
            char* oeta = reinterpret_cast<char*>(g.eta) + lm.e0 * int64_t(sizeof(float));
#pragma unroll
            for (int i = 0; i < L; ++i) {
                if (i >= nr) continue;  // (uniform; keeps the loop fully unrolled)
                double a, p, ph, bb;
                token_gates<M>(ra[i], rp[i], rf[i], rb[i], ac, pc, fc, a, p, ph, bb);
                const double zn = fma(p, X, (a * a) * Z);
                X = fma(ph, zn, X);
                Y = fma(bb, zn, a * Y);
                Z = zn;
                const uint32_t off = lm.lane_el * uint32_t(sizeof(float)) + uint32_t(i) * out_row;
                if constexpr (M == Mode::MixerState || M == Mode::MixerTrain ||
                              M == Mode::ScanState || M == Mode::ScanTrain) {
                    // the state after rows kMixBwdRows * j - 1, j = 1, 2, ...
                    // (the last row's is not needed), as float64 pairs
                    // [j - 1][channel][lam, eta]
                    const int64_t done = t0 + i + 1;
                    if (done % kMixBwdRows == 0 && done < g.T && lm.valid) {
                        const double r = recip(Z);
                        double2* dst = reinterpret_cast<double2*>(
                            g.bstate + ((done / kMixBwdRows - 1) * g.C + lm.q) * 2);
                        *dst = make_double2(X * r, Y * r);
                    }
                }
                if constexpr (kMixer) {
                    // readout: mean eta / lam = Y / X scaled by q, variance 1 / lam = Z / X
                    const double r = recip(X);
                    if (lm.valid) {
                        __builtin_nontemporal_store(float(double(rb[i]) * (Y * r)),
                                                    reinterpret_cast<float*>(olam + off));
                        if (g.eta)
                            __builtin_nontemporal_store(float(Z * r),
                                                        reinterpret_cast<float*>(oeta + off));
                    }
                    if (g.lam_T && t0 + i == g.T - 1 && lm.valid) {
                        const double rz = recip(Z);
                        g.lam_T[lm.q] = float(X * rz);
                        g.eta_T[lm.q] = float(Y * rz);
                    }
                } else if constexpr (M != Mode::MixerState && M != Mode::ScanState) {
                    const double r = recip(Z);
                    if (lm.valid) {
                        __builtin_nontemporal_store(float(X * r), reinterpret_cast<float*>(olam + off));
                        __builtin_nontemporal_store(float(Y * r), reinterpret_cast<float*>(oeta + off));
                    }
                }
                if ((i % kRenormEvery) == kRenormEvery - 1) {
                    const int e = renorm_exponent(fmax(fmax(X, fabs(Y)), Z));
                    X = pow2_scale(X, e);
                    Y = pow2_scale(Y, e);
                    Z = pow2_scale(Z, e);
                }
            }
        }
    }

    // ---- the last workgroup advances the epoch once every tile read it ----
    if (blockIdx.x == gridDim.x - 1 && g.n_chunks > 1 && w == 0)
        advance_epoch(g.ws, tag, (g.n_chunks - 1) * g.G, g.n_tiles, lane);
}

// The scan modes on float32 gates with the tall tile (long sequences).
template <Mode M>
void launch_tall(const FwdArgs& args, hipStream_t stream) {
    const dim3 grid(unsigned(args.n_tiles)), block(kTallWaves * kWave);
    hipLaunchKernelGGL((kla_scan_kernel<float, kTallRows, kTallWaves, M>), grid, block, 0, stream,
                       args);
}

template <int L32, int L16, int W, Mode M>
void launch(const FwdArgs& args, kla_dtype dtype, hipStream_t stream) {
    const dim3 grid(unsigned(args.n_tiles)), block(W * kWave);
    if (dtype == KLA_DTYPE_F32)
        hipLaunchKernelGGL((kla_scan_kernel<float, L32, W, M>), grid, block, 0, stream, args);
    else
        hipLaunchKernelGGL((kla_scan_kernel<uint16_t, L16, W, M>), grid, block, 0, stream, args);
}

}  // namespace

hipError_t launch_scan_fwd(const FwdArgs& args, kla_dtype dtype, FwdMode mode,
                           hipStream_t stream) {
    const bool tall = args.tall && dtype == KLA_DTYPE_F32;
    if (tall && mode == FwdMode::kScan)
        launch_tall<Mode::Scan>(args, stream);
    else if (tall && mode == FwdMode::kScanState)
        launch_tall<Mode::ScanState>(args, stream);
    else if (tall && mode == FwdMode::kScanTrain)
        launch_tall<Mode::ScanTrain>(args, stream);
    else if (mode == FwdMode::kScan)
        launch<kFwdRows, kScanRowsBf16, kFwdWaves, Mode::Scan>(args, dtype, stream);
    else if (mode == FwdMode::kMixer)
        launch<kFwdRows, kMixerRowsBf16, kFwdWaves, Mode::Mixer>(args, dtype, stream);
    else if (mode == FwdMode::kMixerTrain)
        launch<kFwdRows, kMixerRowsBf16, kFwdWaves, Mode::MixerTrain>(args, dtype, stream);
    else if (mode == FwdMode::kMixerState)
        launch<kFwdRows, kMixerRowsBf16, kFwdWaves, Mode::MixerState>(args, dtype, stream);
    else if (mode == FwdMode::kScanState)
        launch<kFwdRows, kScanRowsBf16, kFwdWaves, Mode::ScanState>(args, dtype, stream);
    else if (mode == FwdMode::kScanTrain)
        launch<kFwdRows, kScanRowsBf16, kFwdWaves, Mode::ScanTrain>(args, dtype, stream);
    else
        launch<kLtiRows, kLtiRows, kLtiWaves, Mode::Lti>(args, dtype, stream);
    return hipGetLastError();
}

}  // namespace kla

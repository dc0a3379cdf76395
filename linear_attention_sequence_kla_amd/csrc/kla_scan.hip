// kla_scan.hip -- libkla: forward KLA scan for gfx950 (MI355X).
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
// Kernel structure (single pass, decoupled look-back; Merrill & Garland,
// "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016):
//   * a workgroup of W waves owns one tile: 64 channels (one per lane, so a
//     time row is one coalesced load per wave) by W*L time steps; wave w owns
//     the L rows starting at w*L.  Tiles are numbered (chunk, column group)
//     in workgroup-id order; workgroups are dispatched in increasing id, so
//     every tile a workgroup waits for belongs to one that is already running.
//   * each wave loads its L rows of a, p, phi, b into registers, where they
//     stay until the outputs are written (inputs are read from HBM once);
//   * it folds them into its chunk matrix (float64, renormalised);
//   * wave 0 composes the W chunk matrices, publishes the tile's matrix,
//     looks back over earlier tiles of the same channels for the carry-in
//     state, and publishes the tile's inclusive state;
//   * every wave derives its own carry-in from the tile carry and the chunk
//     matrices of the waves before it, then replays its rows sequentially from
//     on-chip data, writing lam and eta.
//
// Arithmetic is float64 for everything carried (chunk matrices, states): the
// exact precision can reach 1e88 and the information mean 1e-51 on hard gates,
// beyond float32's exponent range, and on gfx950 a float64 FMA issues at the
// same rate as an unpacked float32 FMA.  Inputs and outputs stay 32-bit.
//
// Workspace (caller-owned, zero-filled before first use, self-resetting):
//   [0, 256)         header: u32 reserved[2], u32 epoch, u32 health
//   flags            u64 per tile: (tag << 32) | status, tag = epoch + 1
//   matrix records   per tile: 7 x 64 float64 (A B C D E F G per channel)
//   state records    per tile: 2 x 64 float64 (lam, eta per channel)
// Flags carry the call's tag, so stale flags of earlier calls read as empty
// and nothing needs clearing between calls; the last workgroup advances the
// epoch once every workgroup has read it.  Records and flags are accessed
// only as agent-scope atomics, which stay coherent across XCDs without the
// L2 write-back/invalidate that a release/acquire fence costs.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kla.h"

namespace {

constexpr int kWave = 64;
constexpr uint32_t kStatusAggregate = 1;  // the tile's own matrix is published
constexpr uint32_t kStatusInclusive = 2;  // the tile's inclusive state is published
constexpr uint32_t kStatusFinished = 3;   // a last-chunk tile has its carry-in
constexpr uint32_t kSpinLimit = 1u << 20; // polls before a look-back gives up
constexpr int kRenormEvery = 8;           // tokens between renormalisations

// ---------------------------------------------------------------------------
// Tiling
// ---------------------------------------------------------------------------

struct TileShape {
    int L;  // rows per wave
    int W;  // waves per workgroup
};

// Rows per wave and waves per workgroup of the launched kernels.
constexpr TileShape kTile = {28, 4};

struct Plan {
    int64_t C;          // channels B*H*D
    int64_t N;          // elements B*H*T*D
    int64_t G;          // 64-channel column groups
    int64_t n_chunks;   // tiles along T
    int64_t n_tiles;
    bool offsets_fit;   // per-wave 32-bit byte offsets cannot overflow
    size_t off_flags, off_matrix, off_state, bytes;
};

bool mul_ok(int64_t x, int64_t y, int64_t* out) {
    if (x < 0 || y < 0) return false;
    if (x != 0 && y > INT64_MAX / x) return false;
    *out = x * y;
    return true;
}

// Returns false on negative or overflowing sizes.
bool make_plan(int64_t B, int64_t H, int64_t T, int64_t D, Plan* pl) {
    int64_t BH, C, N;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, D, &C) || !mul_ok(C, T, &N)) return false;
    if (N > INT64_MAX / 16) return false;  // byte offsets of every tensor fit
    const int64_t R = int64_t(kTile.L) * kTile.W;
    pl->C = C;
    pl->N = N;
    pl->G = (C + kWave - 1) / kWave;
    pl->n_chunks = (T + R - 1) / R;
    if (!mul_ok(pl->G, pl->n_chunks, &pl->n_tiles)) return false;
    if (pl->n_tiles > int64_t(UINT32_MAX) - 1 || pl->n_tiles > int64_t(INT32_MAX)) return false;
    // Each wave addresses its rows with 32-bit byte offsets from one base:
    // the 64 channels of a column group span at most ceil((D + 62) / D)
    // slabs of T*D elements, plus the wave's own rows.
    const int64_t span_el = ((D + 62) / (D > 0 ? D : 1)) * T * D + D + int64_t(kTile.L) * D;
    pl->offsets_fit = span_el < (int64_t(1) << 30);
    const size_t nt = size_t(pl->n_tiles);
    pl->off_flags = 256;
    pl->off_matrix = (pl->off_flags + nt * 8 + 255) & ~size_t(255);
    pl->off_state = pl->off_matrix + nt * 7 * kWave * sizeof(double);
    pl->bytes = pl->off_state + nt * 2 * kWave * sizeof(double);
    return true;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// 3x3 projective map [[A, 0, B], [E, F, G], [C, 0, D]] on (lam, eta, 1).
struct Lift {
    double A, B, C, D, E, F, G;
};

// Scales all entries by the power of two that brings the largest to [0.5, 1).
__device__ inline void renorm(Lift& n) {
    const double m = fmax(fmax(fmax(fabs(n.A), fabs(n.B)), fmax(fabs(n.C), fabs(n.D))),
                          fmax(fmax(fabs(n.E), fabs(n.F)), fabs(n.G)));
    const int e = -__builtin_amdgcn_frexp_exp(m);
    n.A = __builtin_amdgcn_ldexp(n.A, e);
    n.B = __builtin_amdgcn_ldexp(n.B, e);
    n.C = __builtin_amdgcn_ldexp(n.C, e);
    n.D = __builtin_amdgcn_ldexp(n.D, e);
    n.E = __builtin_amdgcn_ldexp(n.E, e);
    n.F = __builtin_amdgcn_ldexp(n.F, e);
    n.G = __builtin_amdgcn_ldexp(n.G, e);
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

// 1/z: the hardware float64 reciprocal refined by one Newton step (relative
// error far below float32 resolution; no IEEE division sequence needed).
__device__ inline double recip(double z) {
    const double r = __builtin_amdgcn_rcp(z);
    return fma(fma(-z, r, 1.0), r, r);
}

// (lam, eta) <- n(lam, eta).
__device__ inline void apply(const Lift& n, double& lam, double& eta) {
    const double x = fma(n.A, lam, n.B);
    const double y = fma(n.E, lam, fma(n.F, eta, n.G));
    const double r = recip(fma(n.C, lam, n.D));
    lam = x * r;
    eta = y * r;
}

// Loads one gate from `base + off` (a byte offset) and widens it to float.
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

template <typename In>
__device__ inline float load_gate(const char* base, uint32_t off);

template <>
__device__ inline float load_gate<float>(const char* base, uint32_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const float*>(base + off));
}

template <>
__device__ inline float load_gate<uint16_t>(const char* base, uint32_t off) {
    const uint32_t bits = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(base + off));
    return __uint_as_float(bits << 16);
}

__device__ inline uint64_t flag_word(uint32_t tag, uint32_t status) {
    return (uint64_t(tag) << 32) | status;
}

struct Args {
    const void* a;
    const void* p;
    const void* phi;
    const void* b;
    const float* lam0;
    const float* eta0;
    float* lam;
    float* eta;
    int64_t T, D, C;
    int64_t G, n_chunks, n_tiles;
    uint32_t* header;
    uint64_t* flags;
    double* matrix;  // [tile][7][64]
    double* state;   // [tile][2][64]
};

// Record words are written and read as agent-scope relaxed atomics.  Such
// accesses are coherent across the L2 caches of all XCDs without any cache
// write-back or invalidation, so publishing a record only requires its stores
// to have completed before the flag store is issued.
__device__ inline void rec_store(double* p, double v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), uint64_t(__double_as_longlong(v)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline double rec_load(double* p) {
    return __longlong_as_double(int64_t(__hip_atomic_load(
        reinterpret_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
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

// Publishes a flag once every record store of this wave has completed.  The
// records are agent-coherent atomics, so completion (vmcnt reaching zero) is
// visibility to every other workgroup; no L2 write-back is needed.
__device__ inline void publish(uint64_t* flag, int lane, uint64_t value) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Records `health` bit 0 and tells whether a wait should give up: after
// kSpinLimit polls, or as soon as another wait has given up.
__device__ inline bool give_up(uint32_t spins, uint32_t* header) {
    if ((spins & 255) != 0) return false;
    const uint32_t h = __hip_atomic_load(&header[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(h) != 0 || spins >= kSpinLimit) {
        __hip_atomic_fetch_or(&header[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    return false;
}

// Waits until `flag` carries this call's tag with a non-empty status and
// returns the status (0 if the wait gave up; the health word is then set).
// The caller's record loads are agent-coherent atomics issued after the flag
// was seen, so they observe the records published before it.
__device__ inline uint32_t wait_flag(uint64_t* flag, uint32_t tag, uint32_t* header) {
    for (uint32_t spins = 1;; ++spins) {
        const uint64_t v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
        const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
        if (hi == tag && lo != 0) {
            asm volatile("" ::: "memory");
            return lo;
        }
        if (give_up(spins, header)) return 0;
        __builtin_amdgcn_s_sleep(1);
    }
}

// ---------------------------------------------------------------------------
// The scan kernel
// ---------------------------------------------------------------------------

template <typename In, int L, int W>
__global__ __launch_bounds__(W * kWave) void kla_scan_kernel(Args g) {
    __shared__ double s_lift[W][7][kWave];
    __shared__ double s_carry[W][2][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // Tiles follow the dispatch order of workgroups, which is increasing
    // workgroup id: every tile a workgroup waits for has a lower id, so it
    // was dispatched first and is running or finished.
    const int64_t ticket = blockIdx.x;
    // This call's tag; only wave 0 (the look-back wave) needs it.  Its load
    // is issued after the tile loads so that it costs no extra latency.
    uint32_t tag = 0;

    if (ticket < g.n_tiles) {
        // ---- tile coordinates (wave-uniform) ----
        const int64_t c = ticket / g.G;          // chunk along T
        const int64_t grp = ticket - c * g.G;    // 64-channel column group
        const int64_t q0 = grp * kWave;          // first channel of the group
        const int64_t slab0 = q0 / g.D;
        const int64_t d0 = q0 - slab0 * g.D;
        const int64_t t0 = (c * W + w) * L;      // first row of this wave
        const int nr = int(min(int64_t(L), g.T - t0));  // rows of this wave (may be <= 0)
        const int64_t e0 = (slab0 * g.T + t0) * g.D + d0;  // element of (lane 0, row 0)

        // ---- lane coordinates: channel q, byte offsets from the wave's base ----
        const int64_t q = q0 + lane;
        const bool valid = q < g.C;
        const int64_t qc = valid ? q : q0;       // lanes past C read lane 0's column
        const int64_t slab = qc / g.D;
        const uint32_t lane_el = uint32_t((slab - slab0) * g.T * g.D + (qc - slab * g.D) - d0);
        const uint32_t in_row = uint32_t(g.D * sizeof(In));
        const uint32_t out_row = uint32_t(g.D * sizeof(float));
        const char* pa = static_cast<const char*>(g.a) + e0 * int64_t(sizeof(In));
        const char* pp = static_cast<const char*>(g.p) + e0 * int64_t(sizeof(In));
        const char* pf = static_cast<const char*>(g.phi) + e0 * int64_t(sizeof(In));
        const char* pb = static_cast<const char*>(g.b) + e0 * int64_t(sizeof(In));

        // ---- load the wave's rows; rows past T repeat the last row ----
        // (their values only reach chunk matrices that no valid row uses)
        float ra[L], rp[L], rf[L], rb[L];
        if (nr > 0) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const uint32_t off = lane_el * uint32_t(sizeof(In)) + uint32_t(min(i, nr - 1)) * in_row;
                ra[i] = load_gate<In>(pa, off);
                rp[i] = load_gate<In>(pp, off);
                rf[i] = load_gate<In>(pf, off);
                rb[i] = load_gate<In>(pb, off);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                ra[i] = 1.0f;
                rp[i] = 0.0f;
                rf[i] = 0.0f;
                rb[i] = 0.0f;
            }
        }

        if (w == 0)
            tag = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                      &g.header[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) + 1u;

        // ---- chunk matrix: the columns (A, E, C) and (B, G, D), and F ----
        Lift m;
        {
            double x1 = 1.0, y1 = 0.0, z1 = 0.0;
            double x3 = 0.0, y3 = 0.0, z3 = 1.0;
            double f = 1.0;
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const double a = ra[i], p = rp[i], ph = rf[i], bb = rb[i];
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
        // Keep only the 32-bit gates live across the carry exchange: without
        // this barrier the compiler reuses the float64 conversions of the
        // first pass in the second, doubling the registers a tile needs.
#pragma unroll
        for (int i = 0; i < L; ++i)
            asm volatile("" : "+v"(ra[i]), "+v"(rp[i]), "+v"(rf[i]), "+v"(rb[i]));
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
            double lam_in = 1.0, eta_in = 0.0;
            if (c == 0) {
                if (g.lam0) lam_in = g.lam0[qc];
                if (g.eta0) eta_in = g.eta0[qc];
            } else {
                if (has_next) {
                    store_lift(g.matrix + size_t(ticket) * 7 * kWave, lane,
                               tile_lift<W>(s_lift, lane));
                    publish(&g.flags[ticket], lane, flag_word(tag, kStatusAggregate));
                }
                // Walk back over the flags of this column group to the nearest
                // tile with a published state, then apply the chunk matrices
                // of the tiles after it, oldest first.  (Only one matrix is
                // held at a time, which keeps the registers of the wait low.)
                int64_t j = ticket - g.G;
                uint32_t st;
                while ((st = wait_flag(&g.flags[j], tag, g.header)) == kStatusAggregate) j -= g.G;
                if (st == kStatusInclusive) {
                    lam_in = rec_load(g.state + size_t(j) * 2 * kWave + lane);
                    eta_in = rec_load(g.state + size_t(j) * 2 * kWave + kWave + lane);
                    for (int64_t k = j + g.G; k < ticket; k += g.G)
                        apply(load_lift(g.matrix + size_t(k) * 7 * kWave, lane), lam_in, eta_in);
                }  // else the wait gave up: the health word is set, outputs are wrong
            }
            if (has_next) {
                double l = lam_in, e = eta_in;
                apply(tile_lift<W>(s_lift, lane), l, e);
                rec_store(g.state + size_t(ticket) * 2 * kWave + lane, l);
                rec_store(g.state + size_t(ticket) * 2 * kWave + kWave + lane, e);
                publish(&g.flags[ticket], lane, flag_word(tag, kStatusInclusive));
            } else if (g.n_chunks > 1) {
                publish(&g.flags[ticket], lane, flag_word(tag, kStatusFinished));
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
            char* olam = reinterpret_cast<char*>(g.lam) + e0 * int64_t(sizeof(float));
            char* oeta = reinterpret_cast<char*>(g.eta) + e0 * int64_t(sizeof(float));
#pragma unroll
            for (int i = 0; i < L; ++i) {
                if (i >= nr) continue;  // (uniform; keeps the loop fully unrolled)
                const double a = ra[i], p = rp[i], ph = rf[i], bb = rb[i];
                const double zn = fma(p, X, (a * a) * Z);
                X = fma(ph, zn, X);
                Y = fma(bb, zn, a * Y);
                Z = zn;
                const double r = recip(Z);
                if (valid) {
                    const uint32_t off = lane_el * uint32_t(sizeof(float)) + uint32_t(i) * out_row;
                    __builtin_nontemporal_store(float(X * r), reinterpret_cast<float*>(olam + off));
                    __builtin_nontemporal_store(float(Y * r), reinterpret_cast<float*>(oeta + off));
                }
                if ((i % kRenormEvery) == kRenormEvery - 1) {
                    const double mx = fmax(fmax(X, fabs(Y)), Z);
                    const int e = -__builtin_amdgcn_frexp_exp(mx);
                    X = __builtin_amdgcn_ldexp(X, e);
                    Y = __builtin_amdgcn_ldexp(Y, e);
                    Z = __builtin_amdgcn_ldexp(Z, e);
                }
            }
        }
    }

    // ---- advance the epoch once every workgroup has read it ----
    // Every tile of a column group has read the epoch once the group's last
    // tile has its carry-in (the look-back saw each earlier tile publish with
    // this call's tag).  The last workgroup waits for all last-chunk tiles,
    // then advances the epoch, so the next call's flags carry a new tag.
    if (ticket == int64_t(gridDim.x) - 1 && g.n_chunks > 1 && w == 0) {
        const int64_t first = (g.n_chunks - 1) * g.G;
        for (int64_t k = first + lane; k < g.n_tiles; k += kWave) {
            for (uint32_t spins = 1;; ++spins) {
                const uint64_t v = __hip_atomic_load(&g.flags[k], __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                if (v == flag_word(tag, kStatusFinished)) break;
                if (give_up(spins, g.header)) break;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0)
            __hip_atomic_store(&g.header[2], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

thread_local char t_detail[512];

kla_status fail(kla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kla_status fail(kla_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_detail, sizeof(t_detail), fmt, ap);
    va_end(ap);
    return s;
}

bool overlaps(const void* x, size_t nx, const void* y, size_t ny) {
    if (!x || !y || nx == 0 || ny == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x), b0 = reinterpret_cast<uintptr_t>(y);
    return a0 < b0 + ny && b0 < a0 + nx;
}

template <typename In>
hipError_t launch(const Args& args, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((kla_scan_kernel<In, kTile.L, kTile.W>), dim3(unsigned(grid)),
                       dim3(kTile.W * kWave), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

extern "C" {

size_t kla_scan_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                   kla_dtype in_dtype) {
    if (in_dtype != KLA_DTYPE_F32 && in_dtype != KLA_DTYPE_BF16) return 0;
    Plan pl;
    if (!make_plan(B, H, T, D, &pl) || pl.N == 0) return 0;
    return pl.bytes;
}

kla_status kla_scan_fwd(const void* a, const void* p, const void* phi, const void* b,
                        kla_dtype in_dtype, const float* lam0, const float* eta0,
                        float* lam, float* eta, int64_t B, int64_t H, int64_t T, int64_t D,
                        void* workspace, size_t workspace_bytes, void* stream) {
    t_detail[0] = '\0';
    if (B < 0 || H < 0 || T < 0 || D < 0)
        return fail(KLA_ERR_INVALID_ARG, "negative size B=%lld H=%lld T=%lld D=%lld",
                    (long long)B, (long long)H, (long long)T, (long long)D);
    if (in_dtype != KLA_DTYPE_F32 && in_dtype != KLA_DTYPE_BF16)
        return fail(KLA_ERR_UNSUPPORTED, "unknown input dtype %d", int(in_dtype));
    Plan pl;
    if (!make_plan(B, H, T, D, &pl))
        return fail(KLA_ERR_INVALID_ARG, "sizes overflow: B=%lld H=%lld T=%lld D=%lld",
                    (long long)B, (long long)H, (long long)T, (long long)D);
    if (pl.N == 0) return KLA_OK;
    if (!pl.offsets_fit)
        return fail(KLA_ERR_UNSUPPORTED,
                    "one [T, D] slab is too large (T*D = %lld elements; the limit is about 2^30 "
                    "elements per 64 channels)", (long long)(T * D));

    const void* ins[4] = {a, p, phi, b};
    const char* names[4] = {"a", "p", "phi", "b"};
    const size_t esz = in_dtype == KLA_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i) {
        if (!ins[i]) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (reinterpret_cast<uintptr_t>(ins[i]) % esz)
            return fail(KLA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], esz);
    }
    if (!lam || !eta) return fail(KLA_ERR_INVALID_ARG, "%s is NULL", lam ? "eta" : "lam");
    if (reinterpret_cast<uintptr_t>(lam) % 4 || reinterpret_cast<uintptr_t>(eta) % 4)
        return fail(KLA_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
    if ((lam0 && reinterpret_cast<uintptr_t>(lam0) % 4) ||
        (eta0 && reinterpret_cast<uintptr_t>(eta0) % 4))
        return fail(KLA_ERR_UNSUPPORTED, "lam0/eta0 must be 4-byte aligned");
    if (!workspace) return fail(KLA_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(KLA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.bytes)
        return fail(KLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    pl.bytes);

    // No output may overlap an input, the other output or the workspace.
    const size_t in_bytes = size_t(pl.N) * esz, out_bytes = size_t(pl.N) * 4;
    const size_t st_bytes = size_t(pl.C) * 4;
    struct Range {
        const void* p;
        size_t n;
        const char* name;
    };
    const Range bufs[9] = {{a, in_bytes, "a"},          {p, in_bytes, "p"},
                           {phi, in_bytes, "phi"},      {b, in_bytes, "b"},
                           {lam0, st_bytes, "lam0"},    {eta0, st_bytes, "eta0"},
                           {lam, out_bytes, "lam"},     {eta, out_bytes, "eta"},
                           {workspace, pl.bytes, "workspace"}};
    for (int i = 6; i < 9; ++i)      // lam, eta, workspace (written)
        for (int j = 0; j < 9; ++j)  // against every other buffer
            if (j != i && overlaps(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
                return fail(KLA_ERR_INVALID_ARG, "%s overlaps %s", bufs[i].name, bufs[j].name);

    char* ws = static_cast<char*>(workspace);
    Args args;
    args.a = a;
    args.p = p;
    args.phi = phi;
    args.b = b;
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
    args.header = reinterpret_cast<uint32_t*>(ws);
    args.flags = reinterpret_cast<uint64_t*>(ws + pl.off_flags);
    args.matrix = reinterpret_cast<double*>(ws + pl.off_matrix);
    args.state = reinterpret_cast<double*>(ws + pl.off_state);

    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = in_dtype == KLA_DTYPE_F32 ? launch<float>(args, pl.n_tiles, s)
                                                      : launch<uint16_t>(args, pl.n_tiles, s);
    if (err != hipSuccess)
        return fail(KLA_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
    return KLA_OK;
}

kla_status kla_workspace_health(void* workspace, uint32_t* flags_out, void* stream) {
    t_detail[0] = '\0';
    if (!workspace) return fail(KLA_ERR_WORKSPACE, "workspace is NULL");
    if (!flags_out) return fail(KLA_ERR_INVALID_ARG, "flags_out is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
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
    switch (s) {
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

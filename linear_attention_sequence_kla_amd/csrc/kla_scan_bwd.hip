// kla_scan_bwd.hip -- backward KLA scan kernel (vector-Jacobian product) for
// gfx950 (MI355X).
//
// The forward step (Pith review of arXiv 2602.10743, "Circularity check",
// Theorems 1 and 2), with d_t = a_t^2 + p_t lam_{t-1}:
//     lam_t = lam_{t-1} / d_t + phi_t,     eta_t = (a_t / d_t) eta_{t-1} + b_t.
// Given upstream gradients g_lam[t], g_eta[t] of a loss with respect to the
// outputs, reverse-mode differentiation runs backwards in t.  With
// f = a/d, alpha = f^2 = dlam_t/dlam_{t-1}, beta = -p f eta_{t-1} / d =
// deta_t/dlam_{t-1}, and (cl, ce) the adjoint carried into token t from the
// tokens after it:
//     Lam_t = g_lam[t] + cl,  Eta_t = g_eta[t] + ce        (total adjoints)
//     g_phi[t] = Lam_t,       g_b[t] = Eta_t
//     g_a[t] = Lam_t (-2 a lam_{t-1} / d^2) + Eta_t eta_{t-1} (p lam_{t-1} - a^2) / d^2
//     g_p[t] = Lam_t (-lam_{t-1}^2 / d^2)   + Eta_t (-a lam_{t-1} eta_{t-1} / d^2)
//     carry to t-1: (alpha Lam_t + beta Eta_t, f Eta_t)
// and the carry past the first token is (g_lam0, g_eta0).  The states
// lam_{t-1}, eta_{t-1} are the forward outputs (saved by the caller).
//
// The carry recursion is affine in (cl, ce), so per token it is the 3x3 map
//     [[alpha, beta, alpha g_lam + beta g_eta], [0, f, f g_eta], [0, 0, 1]],
// and a chunk of tokens composes to one map [[u, v, x], [0, w, y], [0, 0, s]]
// (homogeneous: any positive scale of all six entries is the same map, which
// the kernel uses to renormalise by powers of two).  That makes the backward
// pass the same single-pass scan as the forward one, run from the end of the
// sequence: tiles are numbered from the last chunk, each looks back over the
// tiles *after* it in time (kla_lookback.h), and each wave replays its rows
// last to first from its carry, writing the four gradients.

#include "kla_internal.h"

namespace kla {
namespace {

constexpr int kRenormEvery = 8;  // tokens between renormalisations

// Homogeneous affine map on the adjoint carry:
//   (cl, ce) -> ((u cl + v ce + x) / s, (w ce + y) / s).
struct Adj {
    double u, v, x, w, y, s;
};

__device__ inline void renorm(Adj& m) {
    const double mx = fmax(fmax(fmax(fabs(m.u), fabs(m.v)), fmax(fabs(m.x), fabs(m.w))),
                           fmax(fabs(m.y), fabs(m.s)));
    const int e = renorm_exponent(mx);
    m.u = pow2_scale(m.u, e);
    m.v = pow2_scale(m.v, e);
    m.x = pow2_scale(m.x, e);
    m.w = pow2_scale(m.w, e);
    m.y = pow2_scale(m.y, e);
    m.s = pow2_scale(m.s, e);
}

// A.B: the map that applies B first, then A.
__device__ inline Adj mul(const Adj& A, const Adj& B) {
    Adj r;
    r.u = A.u * B.u;
    r.v = fma(A.u, B.v, A.v * B.w);
    r.x = fma(A.u, B.x, fma(A.v, B.y, A.x * B.s));
    r.w = A.w * B.w;
    r.y = fma(A.w, B.y, A.y * B.s);
    r.s = A.s * B.s;
    renorm(r);
    return r;
}

__device__ inline void apply(const Adj& m, double& cl, double& ce) {
    const double r = recip(m.s);
    const double ncl = fma(m.u, cl, fma(m.v, ce, m.x)) * r;
    ce = fma(m.w, ce, m.y) * r;
    cl = ncl;
}

__device__ inline Adj lds_adj(const double (*s)[6][kWave], int j, int lane) {
    return Adj{s[j][0][lane], s[j][1][lane], s[j][2][lane],
               s[j][3][lane], s[j][4][lane], s[j][5][lane]};
}

// The maps of waves w+1..W-1 multiplied (the last wave's applied first;
// waves cover increasing times): the map from the tile's carry to wave w's
// (w < W - 1).
template <int W>
__device__ inline Adj suffix_adj(const double (*s)[6][kWave], int w, int lane) {
    Adj t = lds_adj(s, W - 1, lane);
#pragma unroll 1
    for (int j = W - 2; j > w; --j) t = mul(lds_adj(s, j, lane), t);
    return t;
}

__device__ inline void lds_store_adj(double (*s)[6][kWave], int j, int lane, const Adj& m) {
    s[j][0][lane] = m.u;
    s[j][1][lane] = m.v;
    s[j][2][lane] = m.x;
    s[j][3][lane] = m.w;
    s[j][4][lane] = m.y;
    s[j][5][lane] = m.s;
}

__device__ inline void store_adj(double* rec, int lane, const Adj& m) {
    rec_store(rec + 0 * kWave + lane, m.u);
    rec_store(rec + 1 * kWave + lane, m.v);
    rec_store(rec + 2 * kWave + lane, m.x);
    rec_store(rec + 3 * kWave + lane, m.w);
    rec_store(rec + 4 * kWave + lane, m.y);
    rec_store(rec + 5 * kWave + lane, m.s);
}

__device__ inline Adj load_adj(double* rec, int lane) {
    Adj m;
    m.u = rec_load(rec + 0 * kWave + lane);
    m.v = rec_load(rec + 1 * kWave + lane);
    m.x = rec_load(rec + 2 * kWave + lane);
    m.w = rec_load(rec + 3 * kWave + lane);
    m.y = rec_load(rec + 4 * kWave + lane);
    m.s = rec_load(rec + 5 * kWave + lane);
    return m;
}

__device__ inline float load_f32(const char* base, uint32_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const float*>(base + off));
}

// A row of an optional float32 tensor: always loaded (from a stand-in of the
// same shape when the tensor is absent) and ANDed with `mask` (all ones, or
// zero for an absent tensor).  A load under a branch instead makes the
// compiler wait for every load in flight where the branch rejoins, which
// serialises a wave's row loads one row at a time.
__device__ inline float masked_f32(const char* base, uint32_t off, uint32_t mask) {
    return __uint_as_float(__float_as_uint(load_f32(base, off)) & mask);
}

// The carry exchange of a tile, run after its waves' maps are in s_adj.
// Waves 1..W-2 each store the map from the tile's carry to their own in
// s_suf[w] (the last wave's is the identity).  Wave 0 stores its own such
// map in s_suf[0] and the tile's map in s_suf[W - 1], publishes the tile's
// map, looks back over the tiles later in time for the carry into the
// tile, publishes the tile's inclusive carry and leaves the tile's carry in
// s_tc.  `c` is the tile's chunk along T (tiles are numbered from the
// sequence's end).
template <int W>
__device__ inline void tile_carry(const Workspace& ws, int64_t ticket, int64_t G,
                                  int64_t n_chunks, int64_t c, uint32_t tag,
                                  const double (*s_adj)[6][kWave], double (*s_suf)[6][kWave],
                                  double (*s_tc)[kWave], int w, int lane) {
    static_assert(W >= 2, "the tile's map shares the last wave's slot");
    if (w != 0) {
        if (w + 1 < W) lds_store_adj(s_suf, w, lane, suffix_adj<W>(s_adj, w, lane));
        return;
    }
    const bool has_next = c > 0;  // earlier chunks follow in tile order
    double* const matrix = ws.matrix;
    double* const state = ws.state;
    {
        const Adj s0 = suffix_adj<W>(s_adj, 0, lane);
        if (has_next) {
            // the tile's map, kept in LDS rather than in registers across the
            // wait (written while the record stores drain)
            const Adj t = mul(lds_adj(s_adj, 0, lane), s0);
            const bool agg = c + 1 < n_chunks;
            if (agg) store_adj(matrix + size_t(ticket) * 6 * kWave, lane, t);
            lds_store_adj(s_suf, W - 1, lane, t);
            if (agg) publish(&ws.flags[ticket], lane, flag_word(tag, kStatusAggregate));
        }
        lds_store_adj(s_suf, 0, lane, s0);
    }
    double cl = 0.0, ce = 0.0;  // nothing flows in past the sequence end
    if (c + 1 < n_chunks) {
        int64_t j = ticket - G;
        uint32_t st;
        while ((st = wait_flag(&ws.flags[j], tag, ws.header)) == kStatusAggregate) j -= G;
        if (st == kStatusInclusive) {
            cl = rec_load(state + size_t(j) * 2 * kWave + lane);
            ce = rec_load(state + size_t(j) * 2 * kWave + kWave + lane);
            for (int64_t k = j + G; k < ticket; k += G)
                apply(load_adj(matrix + size_t(k) * 6 * kWave, lane), cl, ce);
        }  // else the wait gave up: the health word is set, outputs are wrong
    }
    if (has_next) {
        double l = cl, e = ce;
        apply(lds_adj(s_suf, W - 1, lane), l, e);
        rec_store(state + size_t(ticket) * 2 * kWave + lane, l);
        rec_store(state + size_t(ticket) * 2 * kWave + kWave + lane, e);
        publish(&ws.flags[ticket], lane, flag_word(tag, kStatusInclusive));
    } else if (n_chunks > 1) {
        publish(&ws.flags[ticket], lane, flag_word(tag, kStatusFinished));
    }
    s_tc[0][lane] = cl;
    s_tc[1][lane] = ce;
}

// The carry into wave w once tile_carry's results are visible: the tile's
// carry through the maps of the waves after it.
template <int W>
__device__ inline void wave_carry(const double (*s_suf)[6][kWave], const double (*s_tc)[kWave],
                                  int w, int lane, double& cl, double& ce) {
    cl = s_tc[0][lane];
    ce = s_tc[1][lane];
    if (w + 1 < W) apply(lds_adj(s_suf, w, lane), cl, ce);
}

template <typename In, int L, int W>
__global__ __launch_bounds__(W * kWave) void kla_scan_bwd_kernel(BwdArgs g) {
    __shared__ double s_adj[W][6][kWave];
    __shared__ double s_suf[W][6][kWave];  // the maps tile_carry leaves
    __shared__ double s_tc[2][kWave];       // the tile's carry
    static_assert(kBwdMatrixWords == 6 && kBwdStateWords == 2, "record layout");

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t ticket = tile_of_workgroup(blockIdx.x, g.G, g.D, g.n_tiles);
    uint32_t tag = 0;

    if (ticket < g.n_tiles) {
        // ---- tile and lane coordinates; tiles run from the sequence's end ----
        const int64_t cc = ticket / g.G;
        const int64_t grp = ticket - cc * g.G;
        const int64_t c = g.n_chunks - 1 - cc;  // chunk along T
        const int64_t t0 = (c * W + w) * L;     // first row of this wave
        const int nr = int(min(int64_t(L), g.T - t0));
        const LaneMap lm = lane_map(grp, t0, lane, g.T, g.D, g.C);
        const uint32_t in_row = uint32_t(g.D * sizeof(In));
        const uint32_t f_row = uint32_t(g.D * sizeof(float));
        const uint32_t in_off = lm.lane_el * uint32_t(sizeof(In));
        const uint32_t f_off = lm.lane_el * uint32_t(sizeof(float));
        const char* pa = static_cast<const char*>(g.a) + lm.e0 * int64_t(sizeof(In));
        const char* pp = static_cast<const char*>(g.p) + lm.e0 * int64_t(sizeof(In));
        // optional upstream gradients: a NULL one is read from a stand-in of
        // the same shape (the g_phi output) and masked to zero (branch-free
        // loads; see masked_f32)
        const char* pgl = reinterpret_cast<const char*>(g.g_lam ? g.g_lam : g.g_phi) + lm.e0 * 4;
        const char* pge = reinterpret_cast<const char*>(g.g_eta ? g.g_eta : g.g_phi) + lm.e0 * 4;
        const uint32_t ml = g.g_lam ? ~0u : 0u, me = g.g_eta ? ~0u : 0u;
        // saved states lam_{t-1}, eta_{t-1}: row t0 + i - 1; sh = 1 when the
        // wave starts the sequence (its row 0 takes lam0, eta0 instead)
        const int sh = t0 > 0 ? 0 : 1;
        const int64_t sb = lm.e0 - (t0 > 0 ? g.D : 0);
        const char* pl = reinterpret_cast<const char*>(g.lam) + sb * 4;
        const char* pe = reinterpret_cast<const char*>(g.eta) + sb * 4;

        // ---- load the wave's rows (rows past T repeat the last one) ----
        float ra[L], rp[L], rl[L], re[L], rgl[L], rge[L];
        if (nr > 0) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int ri = min(i, nr - 1);
                ra[i] = load_gate<In>(pa, in_off + uint32_t(ri) * in_row);
                rp[i] = load_gate<In>(pp, in_off + uint32_t(ri) * in_row);
                if (ri - sh >= 0) {
                    rl[i] = load_f32(pl, f_off + uint32_t(ri - sh) * f_row);
                    re[i] = load_f32(pe, f_off + uint32_t(ri - sh) * f_row);
                } else {
                    rl[i] = g.lam0 ? g.lam0[lm.qc] : 1.0f;
                    re[i] = g.eta0 ? g.eta0[lm.qc] : 0.0f;
                }
                rgl[i] = masked_f32(pgl, f_off + uint32_t(ri) * f_row, ml);
                rge[i] = masked_f32(pge, f_off + uint32_t(ri) * f_row, me);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                ra[i] = 1.0f;
                rp[i] = 0.0f;
                rl[i] = 1.0f;
                re[i] = 0.0f;
                rgl[i] = 0.0f;
                rge[i] = 0.0f;
            }
        }
        if (w == 0) tag = read_tag(g.ws);

        // ---- the wave's map: per-token maps multiplied in time order ----
        Adj m{1.0, 0.0, 0.0, 1.0, 0.0, 1.0};
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if (i < nr) {  // rows past T are the identity
                const double a = ra[i], p = rp[i], lp = rl[i], ep = re[i];
                const double rd = recip(fma(p, lp, a * a));
                const double f = a * rd;
                const double al = f * f;
                const double be = -p * f * ep * rd;
                const double ge = rge[i];
                const double o1 = fma(al, double(rgl[i]), be * ge);
                const double o2 = f * ge;
                const double nx = fma(m.u, o1, fma(m.v, o2, m.x));
                m.v = fma(m.u, be, m.v * f);
                m.u = m.u * al;
                m.y = fma(m.w, o2, m.y);
                m.w = m.w * f;
                m.x = nx;
            }
            if ((i % kRenormEvery) == kRenormEvery - 1 || i == L - 1) renorm(m);
        }
#pragma unroll
        for (int i = 0; i < L; ++i)
            asm volatile("" : "+v"(ra[i]), "+v"(rp[i]), "+v"(rl[i]), "+v"(re[i]), "+v"(rgl[i]),
                         "+v"(rge[i]));
        s_adj[w][0][lane] = m.u;
        s_adj[w][1][lane] = m.v;
        s_adj[w][2][lane] = m.x;
        s_adj[w][3][lane] = m.w;
        s_adj[w][4][lane] = m.y;
        s_adj[w][5][lane] = m.s;
        __syncthreads();

        // ---- tile carry (wave 0: publish, look back over later tiles;
        // the others: their maps from the tile's carry) ----
        tile_carry<W>(g.ws, ticket, g.G, g.n_chunks, c, tag, s_adj, s_suf, s_tc, w, lane);
        __syncthreads();

        // ---- replay the wave's rows last to first, writing the gradients ----
        if (nr > 0) {
            double cl, ce;
            wave_carry<W>(s_suf, s_tc, w, lane, cl, ce);
            char* oa = reinterpret_cast<char*>(g.g_a) + lm.e0 * 4;
            char* op = reinterpret_cast<char*>(g.g_p) + lm.e0 * 4;
            char* of = reinterpret_cast<char*>(g.g_phi) + lm.e0 * 4;
            char* ob = reinterpret_cast<char*>(g.g_b) + lm.e0 * 4;
#pragma unroll
            for (int i = L - 1; i >= 0; --i) {
                if (i >= nr) continue;  // (uniform; keeps the loop fully unrolled)
                const double a = ra[i], p = rp[i], lp = rl[i], ep = re[i];
                const double rd = recip(fma(p, lp, a * a));
                const double rd2 = rd * rd;
                const double Lam = double(rgl[i]) + cl;
                const double Eta = double(rge[i]) + ce;
                // d = a^2 + p lp, rd = 1 / d; the derivatives are listed in
                // kla_state_bwd_kernel below
                const double E = Eta * ep;
                const double ga = rd2 * fma(E, fma(p, lp, -a * a), -2.0 * a * lp * Lam);
                const double gp = -(lp * rd2) * fma(Lam, lp, a * E);
                if (lm.valid) {
                    const uint32_t off = f_off + uint32_t(i) * f_row;
                    __builtin_nontemporal_store(float(ga), reinterpret_cast<float*>(oa + off));
                    __builtin_nontemporal_store(float(gp), reinterpret_cast<float*>(op + off));
                    __builtin_nontemporal_store(float(Lam), reinterpret_cast<float*>(of + off));
                    __builtin_nontemporal_store(float(Eta), reinterpret_cast<float*>(ob + off));
                }
                cl = (a * rd2) * fma(a, Lam, -p * E);
                ce = (a * rd) * Eta;
            }
            if (t0 == 0 && lm.valid) {
                if (g.g_lam0) g.g_lam0[lm.q] = float(cl);
                if (g.g_eta0) g.g_eta0[lm.q] = float(ce);
            }
        }
    }

    // ---- the last workgroup advances the epoch once every tile read it ----
    if (blockIdx.x == gridDim.x - 1 && g.n_chunks > 1 && w == 0)
        advance_epoch(g.ws, tag, (g.n_chunks - 1) * g.G, g.n_tiles, lane);
}

// Backward pass from float64 boundary states: the adjoint scan of the
// kernel above, with the states lam_{t-1}, eta_{t-1} replayed on chip in
// float64 instead of read per row.  The forward pass keeps the float64 state
// after every L-th row (FwdMode::kMixerState/kMixerTrain for the mixer,
// kScanState/kScanTrain for the scan); each wave replays its L rows forward
// from the state before its first row, which gives the states of its rows
// and the wave's adjoint map, and after the tile's carry exchange runs the
// rows last to first.  Float64 states make the gradients exact wherever the
// forward recursion itself is, also where lam or eta leave float32's range
// (lam reaches 1e88 on hard gates).
//
// Mode kScan: the inputs are the gates a, p, phi, b; the upstream gradients
// g_lam, g_eta feed the adjoint scan directly, and each token writes
// g_a, g_p, g_phi = Lam, g_b = Eta (the formulas above).
//
// Mode kMixer (the fused mixer's backward).  Per token the readout
// out = q eta / lam, var = 1 / lam feeds the adjoint scan with
//     g_lam[t] = -(g_out q eta + g_var) / lam^2,   g_eta[t] = g_out q / lam,
// and writes g_q = g_out eta / lam; the gates phi = k^2 lam_v, b = k lam_v v
// send the scan's adjoints Lam (of phi) and Eta (of b) to the token inputs:
//     g_k = 2 Lam k lam_v + Eta lam_v v,  g_lam_v = Lam k^2 + Eta k v,
//     g_v = Eta k lam_v;
// the channel gates a, p collect their per-token adjoints (as g_a, g_p of
// the kernel above) into one sum per tile and lane, added over the batch and
// the chunks by kla_mixer_grad_reduce_kernel.  The mixer's states stay within
// float32's range, so its rows keep float32 copies of them for the reverse
// pass (fewer registers).
//
// Four waves per SIMD (two workgroups of eight waves per CU) are asked for
// explicitly: left to itself the compiler gives the bfloat16 instance a few
// registers more than 128, which halves the workgroups per CU and costs a
// quarter of the bandwidth on bfloat16 inputs.
template <StateBwdMode M> struct StateOf { typedef float T; };
template <> struct StateOf<StateBwdMode::kScan> { typedef double T; };

template <typename In, int L, int W, StateBwdMode M>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(sizeof(In) == 2 ? 5 : 4)))
void kla_state_bwd_kernel(StateBwdArgs g) {
    static_assert(L == kMixBwdRows, "the forward keeps a state every kMixBwdRows rows");
    constexpr bool kMix = M == StateBwdMode::kMixer;
    // float32 instances keep each row's 1 / (a^2 + p lam_{t-1}) from the
    // forward replay for the reverse pass (2% faster); bfloat16 instances
    // recompute it, which with their rows held packed keeps them within 96
    // registers: 5 waves per SIMD instead of 4, 8-13% faster on the
    // 1B-scale layer.
    constexpr bool kKeepRd = sizeof(In) == 4;
    typedef typename StateOf<M>::T S;  // the per-row states kept for the reverse pass
    __shared__ double s_adj[W][6][kWave];
    __shared__ double s_suf[W][6][kWave];  // the maps tile_carry leaves
    __shared__ double s_tc[2][kWave];       // the tile's carry
    __shared__ double s_part[kMix ? W : 1][2][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t ticket = tile_of_workgroup(blockIdx.x, g.G, g.D, g.n_tiles);
    uint32_t tag = 0;

    // the mixer: clear the arrival counts of the channel-gate reduction,
    // which runs after this kernel
    if constexpr (kMix)
        if (blockIdx.x == 0 && w == 0)
            for (int64_t k = lane; k < g.n_counts; k += kWave) g.counts[k] = 0u;

    if (ticket < g.n_tiles) {
        // ---- tile and lane coordinates; tiles run from the sequence's end ----
        const int64_t cc = ticket / g.G;
        const int64_t grp = ticket - cc * g.G;
        const int64_t c = g.n_chunks - 1 - cc;
        const int64_t t0 = (c * W + w) * L;
        const int nr = int(min(int64_t(L), g.T - t0));
        const LaneMap lm = lane_map(grp, t0, lane, g.T, g.D, g.C);
        const uint32_t in_row = uint32_t(g.D * sizeof(In));
        const uint32_t f_row = uint32_t(g.D * sizeof(float));
        const uint32_t in_off = lm.lane_el * uint32_t(sizeof(In));
        const uint32_t f_off = lm.lane_el * uint32_t(sizeof(float));
        const int64_t in_base = lm.e0 * int64_t(sizeof(In));
        const char* p0 = static_cast<const char*>(g.in[0]) + in_base;
        const char* p1 = static_cast<const char*>(g.in[1]) + in_base;
        const char* p2 = static_cast<const char*>(g.in[2]) + in_base;
        const char* p3 = static_cast<const char*>(g.in[3]) + in_base;
        // optional upstream gradients: a NULL one is read from a stand-in of
        // the same shape (the first output) and masked to zero (branch-free
        // loads; see masked_f32)
        const char* pg0 = reinterpret_cast<const char*>(g.g0 ? g.g0 : g.out[0]) + lm.e0 * 4;
        const char* pg1 = reinterpret_cast<const char*>(g.g1 ? g.g1 : g.out[0]) + lm.e0 * 4;
        const uint32_t m0 = g.g0 ? ~0u : 0u, m1 = g.g1 ? ~0u : 0u;
        double ac = 0.0, pc = 0.0;
        if constexpr (kMix) {
            const int64_t hd = lm.qc % g.HD;
            ac = g.a_ch[hd];
            pc = g.p_ch[hd];
        }

        // ---- load the rows and the state before the wave's first row ----
        // (row t0 - 1's boundary state, or the initial state at t0 = 0)
        // mixer: r0..r3 = k, v, lam_v, q; rg0, rg1 = g_out, g_var
        // scan:  r0..r3 = a, p, phi, b;   rg0, rg1 = g_lam, g_eta
        GateRows<In, L> r0, r1, r2, r3;
        float rg0[L], rg1[L];
        double l_in = 1.0, e_in = 0.0;
        if (nr > 0) {
            if (t0 > 0) {
                const double2 st = *reinterpret_cast<const double2*>(
                    g.bstate + ((t0 / L - 1) * g.C + lm.qc) * 2);
                l_in = st.x;
                e_in = st.y;
            } else {
                if (g.lam0) l_in = g.lam0[lm.qc];
                if (g.eta0) e_in = g.eta0[lm.qc];
            }
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int ri = min(i, nr - 1);
                const uint32_t io = in_off + uint32_t(ri) * in_row;
                const uint32_t fo = f_off + uint32_t(ri) * f_row;
                r0.load(i, p0, io);
                r1.load(i, p1, io);
                r2.load(i, p2, io);
                r3.load(i, p3, io);
                rg0[i] = masked_f32(pg0, fo, m0);
                rg1[i] = masked_f32(pg1, fo, m1);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                r0.set(i, 0.0f);
                r1.set(i, 0.0f);
                r2.set(i, 0.0f);
                r3.set(i, 0.0f);
                rg0[i] = rg1[i] = 0.0f;
            }
        }
        if (w == 0) tag = read_tag(g.ws);

        // ---- forward replay of the rows (float64): the states lam_t, eta_t,
        // the adjoints fed in per token (the readout's for the mixer, the
        // upstream gradients for the scan), g_q for the mixer; and the wave's
        // map, the per-token adjoint maps multiplied in time order ----
        // rl[i], re[i]: the state after row i, kept for the reverse pass
        // (which takes the state before row 0 from l_in, e_in); rdv[i]: row
        // i's 1 / (a^2 + p lam_{i-1}) (kKeepRd).
        S rl[L], re[L], rdv[kKeepRd ? L : 1];
        float rgl[L], rge[L];
        Adj m{1.0, 0.0, 0.0, 1.0, 0.0, 1.0};
        {
            double lp = l_in, ep = e_in;
#pragma unroll
            for (int i = 0; i < L; ++i) {
                if (i < nr) {
                    double a, p, ph, bb;
                    if constexpr (kMix) {
                        const double k = r0[i], kl = k * double(r2[i]);
                        a = ac;
                        p = pc;
                        ph = kl * k;
                        bb = kl * double(r1[i]);
                    } else {
                        a = r0[i];
                        p = r1[i];
                        ph = r2[i];
                        bb = r3[i];
                    }
                    const double rd = recip(fma(p, lp, a * a));
                    const double f = a * rd;
                    const double lt = fma(lp, rd, ph);
                    const double et = fma(f, ep, bb);
                    if constexpr (kKeepRd) rdv[i] = S(rd);
                    if constexpr (kMix) {
                        const double rlt = recip(lt);
                        const double go = rg0[i], gq = go * double(r3[i]);
                        rgl[i] = float(-fma(gq, et, double(rg1[i])) * rlt * rlt);
                        rge[i] = float(gq * rlt);
                        if (lm.valid)
                            __builtin_nontemporal_store(
                                float(go * et * rlt),
                                reinterpret_cast<float*>(reinterpret_cast<char*>(g.out[3]) +
                                                         lm.e0 * 4 + f_off + uint32_t(i) * f_row));
                    } else {
                        rgl[i] = rg0[i];
                        rge[i] = rg1[i];
                    }
                    const double al = f * f;
                    const double be = -p * f * ep * rd;
                    const double ge = rge[i];
                    const double o1 = fma(al, double(rgl[i]), be * ge);
                    const double o2 = f * ge;
                    const double nx = fma(m.u, o1, fma(m.v, o2, m.x));
                    m.v = fma(m.u, be, m.v * f);
                    m.u = m.u * al;
                    m.y = fma(m.w, o2, m.y);
                    m.w = m.w * f;
                    m.x = nx;
                    rl[i] = S(lt);
                    re[i] = S(et);
                    lp = lt;
                    ep = et;
                } else {
                    rl[i] = S(1.0);
                    re[i] = S(0.0);
                    if constexpr (kKeepRd) rdv[i] = S(1.0);
                    rgl[i] = rge[i] = 0.0f;
                }
                if ((i % kRenormEvery) == kRenormEvery - 1 || i == L - 1) renorm(m);
            }
        }
        // keep the reverse pass's operands as they are (no recomputation)
#pragma unroll
        for (int i = 0; i < L; ++i) {
            asm volatile("" : "+v"(rl[i]), "+v"(re[i]), "+v"(rgl[i]), "+v"(rge[i]));
            if constexpr (kKeepRd) asm volatile("" : "+v"(rdv[i]));
        }
        r0.keep();
        r1.keep();
        if constexpr (kMix) r2.keep();
        asm volatile("" : "+v"(l_in), "+v"(e_in));
        s_adj[w][0][lane] = m.u;
        s_adj[w][1][lane] = m.v;
        s_adj[w][2][lane] = m.x;
        s_adj[w][3][lane] = m.w;
        s_adj[w][4][lane] = m.y;
        s_adj[w][5][lane] = m.s;
        __syncthreads();

        tile_carry<W>(g.ws, ticket, g.G, g.n_chunks, c, tag, s_adj, s_suf, s_tc, w, lane);
        __syncthreads();

        // ---- replay last to first: input gradients (and the mixer's gate
        // sums) ----
        double sa = 0.0, sp = 0.0;
        if (nr > 0) {
            double cl, ce;
            wave_carry<W>(s_suf, s_tc, w, lane, cl, ce);
            char* o0 = reinterpret_cast<char*>(g.out[0]) + lm.e0 * 4;
            char* o1 = reinterpret_cast<char*>(g.out[1]) + lm.e0 * 4;
            char* o2 = reinterpret_cast<char*>(g.out[2]) + lm.e0 * 4;
            char* o3 = reinterpret_cast<char*>(g.out[3]) + lm.e0 * 4;
#pragma unroll
            for (int i = L - 1; i >= 0; --i) {
                if (i >= nr) continue;
                const double lp = i ? double(rl[i - 1]) : l_in;
                const double ep = i ? double(re[i - 1]) : e_in;
                const double a = kMix ? ac : double(r0[i]);
                const double p = kMix ? pc : double(r1[i]);
                double rd;
                if constexpr (kKeepRd)
                    rd = double(rdv[i]);
                else
                    rd = recip(fma(p, lp, a * a));
                const double rd2 = rd * rd;
                const double Lam = double(rgl[i]) + cl;
                const double Eta = double(rge[i]) + ce;
                // with d = a^2 + p lp (rd = 1 / d): d lam/da = -2 a lp / d^2,
                // d eta/da = ep (p lp - a^2) / d^2, d lam/dp = -lp^2 / d^2,
                // d eta/dp = -a lp ep / d^2; to the state before the row:
                // d lam/d lp = a^2 / d^2, d eta/d lp = -p a ep / d^2,
                // d eta/d ep = a / d
                const double E = Eta * ep;
                const double ga = rd2 * fma(E, fma(p, lp, -a * a), -2.0 * a * lp * Lam);
                const double gp = -(lp * rd2) * fma(Lam, lp, a * E);
                if (lm.valid) {
                    const uint32_t off = f_off + uint32_t(i) * f_row;
                    if constexpr (kMix) {
                        const double k = r0[i], lv = r2[i], ev = Eta * double(r1[i]);
                        __builtin_nontemporal_store(float(lv * fma(Lam + Lam, k, ev)),
                                                    reinterpret_cast<float*>(o0 + off));
                        __builtin_nontemporal_store(float(Eta * k * lv),
                                                    reinterpret_cast<float*>(o1 + off));
                        __builtin_nontemporal_store(float(k * fma(Lam, k, ev)),
                                                    reinterpret_cast<float*>(o2 + off));
                    } else {
                        __builtin_nontemporal_store(float(ga), reinterpret_cast<float*>(o0 + off));
                        __builtin_nontemporal_store(float(gp), reinterpret_cast<float*>(o1 + off));
                        __builtin_nontemporal_store(float(Lam), reinterpret_cast<float*>(o2 + off));
                        __builtin_nontemporal_store(float(Eta), reinterpret_cast<float*>(o3 + off));
                    }
                }
                if constexpr (kMix) {
                    sa += ga;
                    sp += gp;
                }
                cl = (a * rd2) * fma(a, Lam, -p * E);
                ce = (a * rd) * Eta;
            }
            if (t0 == 0 && lm.valid) {
                if (g.g_lam0) g.g_lam0[lm.q] = float(cl);
                if (g.g_eta0) g.g_eta0[lm.q] = float(ce);
            }
        }
        // ---- the mixer: the tile's sums of the channel-gate gradients ----
        if constexpr (kMix) {
            s_part[w][0][lane] = sa;
            s_part[w][1][lane] = sp;
            __syncthreads();
            if (w == 0) {
                double ta = 0.0, tp = 0.0;
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    ta += s_part[j][0][lane];
                    tp += s_part[j][1][lane];
                }
                g.partial[(size_t(ticket) * 2) * kWave + lane] = ta;
                g.partial[(size_t(ticket) * 2 + 1) * kWave + lane] = tp;
            }
        }
    }

    // ---- the last workgroup advances the epoch once every tile read it ----
    if (blockIdx.x == gridDim.x - 1 && g.n_chunks > 1 && w == 0)
        advance_epoch(g.ws, tag, (g.n_chunks - 1) * g.G, g.n_tiles, lane);
}

// g_a[h, d] and g_p[h, d] in fixed-order steps, so the result does not
// depend on timing (deterministic).  Workgroup (x, s) takes 64 channels
// (h, d) and slice s of the (b, chunk) pairs: wave w adds the per-tile sums
// of pairs first + w, first + w + kReduceWaves, ..., and wave 0 adds the
// waves' totals in order.  With one slice that is the result; otherwise it
// goes to slices[s][2][HD], the workgroup counts itself in counts[x] (zeroed
// by the backward kernel before this one runs), and the one that counts
// last adds slices 0, 1, ..., S - 1 in order.  Slices and counts are
// agent-coherent atomics: the count is taken once the slice's stores have
// completed, and the last workgroup loads the slices after its count, as in
// the look-back.  Slices of 64 pairs spread the reduction over many
// workgroups even on short layers: 128 on the small-LM layer (8 x 16 x 2048
// x 64), where one workgroup per 64 channels took 13 us of a 200-us mixer
// backward and the slices take 6.5-7 us.
constexpr int kReduceWaves = 8;

__global__ __launch_bounds__(kReduceWaves * kWave) void kla_mixer_grad_reduce_kernel(
    const double* partial, double* slices, uint32_t* counts, float* g_a, float* g_p,
    int64_t B, int64_t HD, int64_t G, int64_t n_chunks, int64_t per) {
    __shared__ double s_sum[kReduceWaves][2][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t hd = int64_t(blockIdx.x) * kWave + lane;
    const bool in_hd = hd < HD;
    const int64_t hdc = in_hd ? hd : HD - 1;  // (lanes past HD read a channel that exists)
    const int64_t n = B * n_chunks;
    const int64_t first = int64_t(blockIdx.y) * per;
    const int64_t last = min(n, first + per);
    double sa = 0.0, sp = 0.0;
    // pair j = b * n_chunks + cc; (b, cc) advance with j, so the loop
    // divides once; a batch of kBatch pairs' loads is in flight before the
    // first one is added, and pairs past the slice load a valid word and add
    // zero (no branch around a load: the wait for it would serialise them)
    constexpr int kBatch = 8;
    int64_t j = first + w, b = j / n_chunks, cc = j - b * n_chunks;
    while (j < last) {
        size_t off[kBatch];
        bool in[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            in[u] = j < last;
            const uint64_t q = uint64_t(b * HD + hdc);
            off[u] = in[u] ? size_t(cc * G + int64_t(q / kWave)) * 2 * kWave + size_t(q % kWave)
                           : 0;
            j += kReduceWaves;
            cc += kReduceWaves;
            while (cc >= n_chunks) {
                cc -= n_chunks;
                ++b;
            }
        }
        double va[kBatch], vp[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            va[u] = partial[off[u]];
            vp[u] = partial[off[u] + kWave];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            sa += in[u] ? va[u] : 0.0;
            sp += in[u] ? vp[u] : 0.0;
        }
    }
    s_sum[w][0][lane] = sa;
    s_sum[w][1][lane] = sp;
    __syncthreads();
    if (w != 0) return;
    double ta = 0.0, tp = 0.0;
#pragma unroll
    for (int k = 0; k < kReduceWaves; ++k) {
        ta += s_sum[k][0][lane];
        tp += s_sum[k][1][lane];
    }
    const int64_t S = gridDim.y;
    if (S == 1) {
        if (in_hd) {
            g_a[hd] = float(ta);
            g_p[hd] = float(tp);
        }
        return;
    }
    if (in_hd) {
        rec_store(&slices[(int64_t(blockIdx.y) * 2) * HD + hd], ta);
        rec_store(&slices[(int64_t(blockIdx.y) * 2 + 1) * HD + hd], tp);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#ifdef KLA_DEBUG_DELAYS
    // test builds: slices count themselves in a pseudo-random order, so
    // that a different workgroup adds them up
    debug_delay(reinterpret_cast<const uint64_t*>(counts + blockIdx.x),
                uint64_t(blockIdx.y) << 32);
#endif
    uint32_t before = 0;
    if (lane == 0)
        before = __hip_atomic_fetch_add(&counts[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(before) != uint32_t(S - 1)) return;
    asm volatile("" ::: "memory");
    double fa = 0.0, fp = 0.0;
    for (int64_t s0 = 0; s0 < S; s0 += kBatch) {
        double va[kBatch], vp[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t sl = s0 + u < S ? s0 + u : S - 1;
            va[u] = rec_load(&slices[(sl * 2) * HD + hdc]);
            vp[u] = rec_load(&slices[(sl * 2 + 1) * HD + hdc]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            fa += s0 + u < S ? va[u] : 0.0;
            fp += s0 + u < S ? vp[u] : 0.0;
        }
    }
    if (in_hd) {
        g_a[hd] = float(fa);
        g_p[hd] = float(fp);
    }
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs& args, kla_dtype dtype, hipStream_t stream) {
    const dim3 grid(unsigned(args.n_tiles)), block(kBwdWaves * kWave);
    if (dtype == KLA_DTYPE_F32)
        hipLaunchKernelGGL((kla_scan_bwd_kernel<float, kBwdRows, kBwdWaves>), grid, block, 0,
                           stream, args);
    else
        hipLaunchKernelGGL((kla_scan_bwd_kernel<uint16_t, kBwdRows, kBwdWaves>), grid, block, 0,
                           stream, args);
    return hipGetLastError();
}

template <typename In, int W, StateBwdMode M>
void launch_state(const StateBwdArgs& args, hipStream_t stream) {
    const dim3 grid(unsigned(args.n_tiles)), block(W * kWave);
    hipLaunchKernelGGL((kla_state_bwd_kernel<In, kMixBwdRows, W, M>), grid, block, 0, stream, args);
}

hipError_t launch_state_bwd(const StateBwdArgs& args, kla_dtype dtype, StateBwdMode mode,
                            hipStream_t stream) {
    const bool mix = mode == StateBwdMode::kMixer;
    if (dtype != KLA_DTYPE_F32 && args.waves != 4) return hipErrorInvalidValue;
    if (dtype != KLA_DTYPE_F32 && mix)  // bfloat16: 4-wave tiles only (state_bwd_waves)
        launch_state<uint16_t, 4, StateBwdMode::kMixer>(args, stream);
    else if (dtype != KLA_DTYPE_F32)
        launch_state<uint16_t, 4, StateBwdMode::kScan>(args, stream);
    else if (args.waves == 8 && mix)
        launch_state<float, 8, StateBwdMode::kMixer>(args, stream);
    else if (mix)
        launch_state<float, 4, StateBwdMode::kMixer>(args, stream);
    else if (args.waves == 8)
        launch_state<float, 8, StateBwdMode::kScan>(args, stream);
    else
        launch_state<float, 4, StateBwdMode::kScan>(args, stream);
    return hipGetLastError();
}

hipError_t launch_mixer_grad_reduce(const double* partial, double* slices, uint32_t* counts,
                                    float* g_a, float* g_p, int64_t B, int64_t H, int64_t D,
                                    int64_t G, int64_t n_chunks, hipStream_t stream) {
    const int64_t HD = H * D, groups = (HD + kWave - 1) / kWave;
    const int64_t S = mixer_grad_slices(B, H, D, n_chunks);
    const int64_t per = (B * n_chunks + S - 1) / S;
    hipLaunchKernelGGL(kla_mixer_grad_reduce_kernel, dim3(unsigned(groups), unsigned(S)),
                       dim3(kReduceWaves * kWave), 0, stream, partial, slices, counts, g_a, g_p,
                       B, HD, G, n_chunks, per);
    return hipGetLastError();
}

}  // namespace kla

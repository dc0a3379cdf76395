// kla_lookback.h -- the cross-workgroup carry protocol shared by the forward
// and backward scan kernels (single pass, decoupled look-back; Merrill &
// Garland, "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016),
// as it runs on gfx950.
//
// A scan is cut into tiles; tile k's carry depends only on tiles k - G,
// k - 2G, ... (the same column group in earlier chunks; G >= 1 column
// groups).  Workgroups are dispatched in increasing id and run the tile
// tile_of_workgroup() assigns them, which never places a tile a workgroup
// waits for on a higher workgroup id, so every such tile belongs to a
// workgroup already running.
//
// Workspace (caller-owned, zero-filled before first use, self-resetting):
//   [0, 256)        header: u32 reserved, u32 gave_up, u32 epoch, u32 health
//                   (gave_up: the tag of the last call whose waits gave up;
//                   health: sticky bit 0, set by any give-up until it is read)
//   flags           u64 per tile: (tag << 32) | status, tag = epoch + 1
//   matrix records  per tile: kMatrixWords x 64 float64 (the tile's own map)
//   state records   per tile: kStateWords x 64 float64 (its inclusive carry)
// Flags carry the call's tag, so stale flags of earlier calls read as empty
// and nothing needs clearing between calls.  The last workgroup advances the
// epoch once every workgroup has read it (advance_epoch).
//
// Records and flags are accessed only as agent-scope relaxed atomics.  On
// gfx950 these are coherent across the L2 caches of all XCDs without cache
// maintenance, whereas an agent-scope release/acquire fence writes back and
// invalidates the L2.  A flag is stored after `s_waitcnt vmcnt(0)` has seen
// the wave's record stores complete, and record loads are issued after the
// flag was observed.

#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace kla {

constexpr int kWave = 64;
// Status words.  Calls of different shapes or kernels that share a workspace
// lay out flags and records differently, so a flag slot may hold a record
// word (a float64) left by another call; a status is a 32-bit pattern next to
// the 32-bit tag so that such a word is not mistaken for a flag.
constexpr uint32_t kStatusMagic = 0x4b4c4100u;                 // "KLA"
constexpr uint32_t kStatusAggregate = kStatusMagic | 1u;  // the tile's own map is published
constexpr uint32_t kStatusInclusive = kStatusMagic | 2u;  // the tile's inclusive carry is published
constexpr uint32_t kStatusFinished = kStatusMagic | 3u;   // a last tile of its column has its carry-in
constexpr uint32_t kSpinLimit = 1u << 20; // polls before a wait gives up
constexpr size_t kHeaderBytes = 256;

// Device view of a workspace.
struct Workspace {
    uint32_t* header;
    uint64_t* flags;
    double* matrix;  // [tile][matrix words][64]
    double* state;   // [tile][state words][64]
};

// Byte offsets of a workspace for n_tiles tiles.
struct WorkspaceLayout {
    size_t off_flags, off_matrix, off_state, bytes;
};

inline WorkspaceLayout workspace_layout(size_t n_tiles, int matrix_words, int state_words) {
    WorkspaceLayout w;
    w.off_flags = kHeaderBytes;
    w.off_matrix = (w.off_flags + n_tiles * 8 + 255) & ~size_t(255);
    w.off_state = w.off_matrix + n_tiles * size_t(matrix_words) * kWave * sizeof(double);
    w.bytes = w.off_state + n_tiles * size_t(state_words) * kWave * sizeof(double);
    return w;
}

inline Workspace workspace_view(void* base, const WorkspaceLayout& l) {
    char* ws = static_cast<char*>(base);
    return Workspace{reinterpret_cast<uint32_t*>(ws), reinterpret_cast<uint64_t*>(ws + l.off_flags),
                     reinterpret_cast<double*>(ws + l.off_matrix),
                     reinterpret_cast<double*>(ws + l.off_state)};
}

__device__ inline uint64_t flag_word(uint32_t tag, uint32_t status) {
    return (uint64_t(tag) << 32) | status;
}

// This call's tag (the workspace epoch + 1).
__device__ inline uint32_t read_tag(const Workspace& ws) {
    return __builtin_amdgcn_readfirstlane(
               __hip_atomic_load(&ws.header[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) +
           1u;
}

__device__ inline void rec_store(double* p, double v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), uint64_t(__double_as_longlong(v)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline double rec_load(double* p) {
    return __longlong_as_double(int64_t(__hip_atomic_load(
        reinterpret_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
}

#ifdef KLA_DEBUG_DELAYS
// Test builds only (libkla_debug.so): a pause of 0..15 x 127 sleep units,
// pseudo-random per flag and call, before a flag is published, so that
// look-backs meet predecessors in every state (not yet published, aggregate
// only, inclusive late) and walk back over several tiles.
__device__ inline void debug_delay(const uint64_t* flag, uint64_t value) {
    const uint64_t x = (reinterpret_cast<uintptr_t>(flag) >> 3) ^ (value >> 32) * 0x9e3779b9u;
    const uint32_t n = uint32_t((x * 0x9e3779b97f4a7c15ull) >> 60);
    for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
}
#endif

// Publishes a flag once every record store of this wave has completed.  The
// records are agent-coherent atomics, so completion (vmcnt reaching zero) is
// visibility to every other workgroup; no L2 write-back is needed.
__device__ inline void publish(uint64_t* flag, int lane, uint64_t value) {
#ifdef KLA_DEBUG_DELAYS
    debug_delay(flag, value);
#endif
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tells whether a wait of the call tagged `tag` should give up: after
// kSpinLimit polls, or as soon as another wait of the SAME call has given up
// (header[1] holds the tag of the last call that gave up, so a give-up never
// shortens the waits of later calls).  A give-up records the call's tag and
// sets the sticky health bit 0, which stays set until kla_workspace_health
// reads it.
__device__ inline bool give_up(uint32_t spins, uint32_t* header, uint32_t tag) {
    if ((spins & 255) != 0) return false;
    const uint32_t g = __hip_atomic_load(&header[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (uint32_t(__builtin_amdgcn_readfirstlane(g)) == tag || spins >= kSpinLimit) {
        __hip_atomic_store(&header[1], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(&header[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    return false;
}

// Waits until `flag` carries this call's tag with a status and returns the
// status (0 if the wait gave up; the health word is then set).
// The caller's record loads are agent-coherent atomics issued after the flag
// was seen, so they observe the records published before it.
__device__ inline uint32_t wait_flag(uint64_t* flag, uint32_t tag, uint32_t* header) {
    for (uint32_t spins = 1;; ++spins) {
        const uint64_t v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
        const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
        if (hi == tag && (lo == kStatusAggregate || lo == kStatusInclusive ||
                          lo == kStatusFinished)) {
            asm volatile("" ::: "memory");
            return lo;
        }
        if (give_up(spins, header, tag)) return 0;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Run by one wave of the last workgroup once its own work is done.  Tiles
// [first, n_tiles) are the last tile of every column (one per 64-channel
// group); each publishes kStatusFinished after its look-back, which proves
// that every tile of its column read the epoch (it saw each of them publish
// with this call's tag).  Once all have, the epoch advances so that the next
// call's flags carry a new tag.
__device__ inline void advance_epoch(const Workspace& ws, uint32_t tag, int64_t first,
                                     int64_t n_tiles, int lane) {
    for (int64_t k = first + lane; k < n_tiles; k += kWave) {
        for (uint32_t spins = 1;; ++spins) {
            const uint64_t v =
                __hip_atomic_load(&ws.flags[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v == flag_word(tag, kStatusFinished)) break;
            if (give_up(spins, ws.header, tag)) break;
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (lane == 0)
        __hip_atomic_store(&ws.header[2], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 1/z: the hardware float64 reciprocal refined by one Newton step (relative
// error far below float32 resolution; no IEEE division sequence needed).
__device__ inline double recip(double z) {
    const double r = __builtin_amdgcn_rcp(z);
    return fma(fma(-z, r, 1.0), r, r);
}

// Scales x by 2^e (exact unless the result leaves the float64 range).
__device__ inline double pow2_scale(double x, int e) { return __builtin_amdgcn_ldexp(x, e); }

// -e such that max(|values|) * 2^-e lies in [0.5, 1).
__device__ inline int renorm_exponent(double max_abs) {
    return -__builtin_amdgcn_frexp_exp(max_abs);
}

// The tile workgroup `wg` runs.  gfx950 hands workgroups to its eight XCDs
// (each with its own L2) in turn, by workgroup id modulo 8, so tiles k and
// k + 1 land on different XCDs.  When a slab row spans several 64-channel
// groups (D a multiple of 128), column groups 2m and 2m + 1 of a chunk read
// and write the two halves of the same rows; they are given to workgroups
// with ids x and x + 8 of the same aligned block of 16 (x < 8), i.e. to the
// same XCD, which measured 3-4% faster on such shapes.  The map permutes
// each full block of 16 and leaves a partial last block alone; with G >= 16
// a tile's predecessors (G or more tiles earlier) lie in earlier blocks,
// hence on workgroups with lower ids.
__device__ inline int64_t tile_of_workgroup(int64_t wg, int64_t G, int64_t D, int64_t n_tiles) {
    if (D % 128 != 0 || G < 16) return wg;
    const int64_t block = wg >> 4, r = wg & 15;
    if ((block + 1) * 16 > n_tiles) return wg;
    return block * 16 + (r & 7) * 2 + (r >> 3);
}

// Loads one gate from `base + off` (a byte offset) and widens it to float.
template <typename In>
__device__ inline float load_gate(const char* base, uint32_t off);

template <>
__device__ inline float load_gate<float>(const char* base, uint32_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const float*>(base + off));
}

template <>
__device__ inline float load_gate<uint16_t>(const char* base, uint32_t off) {
    const uint32_t bits =
        __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(base + off));
    return __uint_as_float(bits << 16);
}

// One token input of a wave's L rows, held in registers across a kernel's passes.
// float32 values are kept as loaded; bfloat16 values stay packed, two rows
// per register (row 2j in the low half), and widen when read, which halves
// the registers the rows take.
template <typename In, int L>
struct GateRows {
    float v[L];
    __device__ void load(int i, const char* base, uint32_t off) {
        v[i] = __builtin_nontemporal_load(reinterpret_cast<const float*>(base + off));
    }
    __device__ void set(int i, float x) { v[i] = x; }
    __device__ float operator[](int i) const { return v[i]; }
    // pins the values in registers: a later pass reads them there, and the
    // compiler neither reloads nor rematerialises them
    __device__ void keep() {
#pragma unroll
        for (int i = 0; i < L; ++i) asm volatile("" : "+v"(v[i]));
    }
};

template <int L>
struct GateRows<uint16_t, L> {
    uint32_t v[(L + 1) / 2];
    __device__ void put(int i, uint32_t bits) {
        if (i & 1)
            v[i >> 1] |= bits << 16;
        else
            v[i >> 1] = bits;
    }
    __device__ void load(int i, const char* base, uint32_t off) {
        put(i, __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(base + off)));
    }
    // (x exact in bfloat16)
    __device__ void set(int i, float x) { put(i, __float_as_uint(x) >> 16); }
    __device__ float operator[](int i) const {
        const uint32_t x = v[i >> 1];
        return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
    }
    __device__ void keep() {
#pragma unroll
        for (int i = 0; i < (L + 1) / 2; ++i) asm volatile("" : "+v"(v[i]));
    }
};

// Lane coordinates of a tile: 64 consecutive channels q0..q0+63 of the
// flattened (b, h, d) index, starting at time row t0.  Each lane addresses its
// rows with a 32-bit byte offset from the wave's base element e0, so every row
// is one coalesced load per wave and per-row addressing is one add.
struct LaneMap {
    int64_t e0;        // element index of (lane 0's channel, row t0)
    int64_t q;         // this lane's channel (may be >= C)
    int64_t qc;        // q clamped to a valid channel (lane 0's if q >= C)
    bool valid;        // q < C
    uint32_t lane_el;  // element offset of this lane's channel from e0
};

__device__ inline LaneMap lane_map(int64_t grp, int64_t t0, int lane, int64_t T, int64_t D,
                                   int64_t C) {
    LaneMap m;
    const int64_t q0 = grp * kWave;
    const int64_t slab0 = q0 / D;
    const int64_t d0 = q0 - slab0 * D;
    m.e0 = (slab0 * T + t0) * D + d0;
    m.q = q0 + lane;
    m.valid = m.q < C;
    m.qc = m.valid ? m.q : q0;
    const int64_t slab = m.qc / D;
    m.lane_el = uint32_t((slab - slab0) * T * D + (m.qc - slab * D) - d0);
    return m;
}

}  // namespace kla

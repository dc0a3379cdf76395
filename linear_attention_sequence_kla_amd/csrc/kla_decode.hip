// kla_decode.hip -- one-token update of a running KLA filter state (decode).
//
// Linear-time inference ("KLA Part 1" primer, opening: a Kalman recursion
// gives linear-time inference; the running posterior is a sufficient summary,
// §6.2): each generated token applies one predict/update step to the state
// (lam, eta) of every channel, the same step as the scan (Pith review of
// arXiv 2602.10743, "Circularity check"):
//     d = a^2 + p lam,  lam' = lam / d + phi,  eta' = (a / d) eta + b.
// It is computed in float64 as the homogeneous step of the scan kernel
// (Z' = p lam + a^2, lam' = (lam + phi Z') / Z', eta' = (a eta + b Z') / Z')
// and stored back in float32.  Channels are independent: one thread each,
// consecutive threads on consecutive channels (coalesced).  The fused mixer
// has a decode step of its own (kla_mixer_decode_kernel).

#include "kla_internal.h"

namespace kla {
namespace {

template <typename In>
__device__ inline float load_one(const In* x, int64_t i);

template <>
__device__ inline float load_one<float>(const float* x, int64_t i) {
    return __builtin_nontemporal_load(x + i);
}

template <>
__device__ inline float load_one<uint16_t>(const uint16_t* x, int64_t i) {
    return __uint_as_float(uint32_t(__builtin_nontemporal_load(x + i)) << 16);
}

template <typename In>
__global__ __launch_bounds__(256) void kla_decode_kernel(const In* __restrict__ a,
                                                         const In* __restrict__ p,
                                                         const In* __restrict__ phi,
                                                         const In* __restrict__ b,
                                                         float* __restrict__ lam,
                                                         float* __restrict__ eta, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const double av = load_one<In>(a, i), pv = load_one<In>(p, i);
        const double fv = load_one<In>(phi, i), bv = load_one<In>(b, i);
        const double l = lam[i], e = eta[i];
        const double z = fma(pv, l, av * av);
        const double r = recip(z);
        lam[i] = float(fma(fv, z, l) * r);
        eta[i] = float(fma(bv, z, av * e) * r);
    }
}

// One token of the fused mixer (the decode form of the forward kernel's
// mixer mode): gates phi = k^2 lam_v and b = k lam_v v, channel gates a, p
// from the [H*D] arrays (channel i uses i % hd), the same float64 step as
// above, the state stored back in float32, and the readout q eta' / lam'
// and variance 1 / lam' from the float64 state.
template <typename In>
__global__ __launch_bounds__(256) void kla_mixer_decode_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const In* __restrict__ lam_v,
    const In* __restrict__ q, const float* __restrict__ a, const float* __restrict__ p,
    float* __restrict__ lam, float* __restrict__ eta, float* __restrict__ out,
    float* __restrict__ var, int64_t n, int64_t hd) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const double kv = load_one<In>(k, i), vv = load_one<In>(v, i);
        const double lv = load_one<In>(lam_v, i), qv = load_one<In>(q, i);
        const int64_t c = i % hd;
        const double av = a[c], pv = p[c];
        const double l = lam[i], e = eta[i];
        const double z = fma(pv, l, av * av);
        const double r = recip(z);
        const double nl = fma(kv * kv * lv, z, l) * r;
        const double ne = fma(kv * lv * vv, z, av * e) * r;
        const double rl = recip(nl);
        lam[i] = float(nl);
        eta[i] = float(ne);
        out[i] = float(qv * (ne * rl));
        if (var) var[i] = float(rl);
    }
}

}  // namespace

hipError_t launch_mixer_decode(const void* k, const void* v, const void* lam_v, const void* q,
                               kla_dtype dtype, const float* a, const float* p, float* lam,
                               float* eta, float* out, float* var, int64_t n, int64_t hd,
                               hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    const dim3 grid(unsigned(blocks < 65536 ? blocks : 65536)), block(256);
    if (dtype == KLA_DTYPE_F32)
        hipLaunchKernelGGL(kla_mixer_decode_kernel<float>, grid, block, 0, stream,
                           static_cast<const float*>(k), static_cast<const float*>(v),
                           static_cast<const float*>(lam_v), static_cast<const float*>(q), a, p,
                           lam, eta, out, var, n, hd);
    else
        hipLaunchKernelGGL(kla_mixer_decode_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                           static_cast<const uint16_t*>(lam_v), static_cast<const uint16_t*>(q),
                           a, p, lam, eta, out, var, n, hd);
    return hipGetLastError();
}

hipError_t launch_decode(const void* a, const void* p, const void* phi, const void* b,
                         kla_dtype dtype, float* lam, float* eta, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    const dim3 grid(unsigned(blocks < 65536 ? blocks : 65536)), block(256);
    if (dtype == KLA_DTYPE_F32)
        hipLaunchKernelGGL(kla_decode_kernel<float>, grid, block, 0, stream,
                           static_cast<const float*>(a), static_cast<const float*>(p),
                           static_cast<const float*>(phi), static_cast<const float*>(b), lam,
                           eta, n);
    else
        hipLaunchKernelGGL(kla_decode_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(p),
                           static_cast<const uint16_t*>(phi), static_cast<const uint16_t*>(b),
                           lam, eta, n);
    return hipGetLastError();
}

}  // namespace kla

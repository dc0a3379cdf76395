// bench_copy.hip -- copy prototypes of the forward scan's memory structure,
// for the bandwidth ceiling of its tile orders (measurement only, not part of
// the library).
//
// Four input tensors [S, T, D] (float32 or bfloat16) are read and two float32
// outputs written, as by the scan, with no scan arithmetic:
//   stream  one thread per 4 consecutive elements of every tensor;
//   scan    the scan's tiles (64 channels x W waves x L rows, each wave's
//           rows held in registers until written), in the scan's dispatch
//           order: one chunk of every 64-channel column, then the next chunk
//           (the order that keeps a look-back a few tiles deep);
//   addr    the same tiles in address order: every chunk of one column, then
//           the next column;
//   skew    the scan order with column g (column pair g / 2 when pairing)
//           started (g mod K) * M chunks late, arg = K + 1000 M, so that the
//           columns' active chunks sit at different offsets;
//   pol     the scan order, loads and stores with the cache-policy bits
//           arg = 100 * LP + SP (see k_tile_pol; 202 = non-temporal both);
//   colstream  no tiles dispatched at all: one workgroup per arg = 16, 32
//           or 64 channels of a slab walks all T rows itself, tile after
//           tile, with the next tile's loads in flight while the current one
//           is stored (the carry of such a structure would stay on chip, with
//           no look-back); a wave's lanes cover 64 / arg row slices.
// `pair` gives tiles 2m and 2m + 1 of each aligned block of 16 to workgroups
// x and x + 8 (one XCD), as the library does for D a multiple of 128.
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature \
//       -Xclang -packed-fp32-ops bench_copy.hip -o bench_copy
//   ./bench_copy <shape 1..3> <stream|scan|addr|band|super|skew|xcdcol|pol|colstream> <arg> <L> <W> <pair> [sets]
// shape 1: 128 slabs x 2048 x 64 f32, 2: 128 x 8192 x 128 bf16,
// 3: 32 x 131072 x 128 f32.  Prints the mean of 20 launches (`sets` input
// and output sets, default 2, used in turn) as time and fraction of 8 TB/s.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>
#include <vector>
#include <string>
#include <algorithm>

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)

struct Bufs { const void* in[4]; float* out[2]; };

__device__ inline float ld(const float* p) { return __builtin_nontemporal_load(p); }
__device__ inline float ld(const uint16_t* p) { return __uint_as_float(uint32_t(__builtin_nontemporal_load(p)) << 16); }

__device__ inline void pause_ns(uint32_t ns) {
  if (ns == 0) return;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t ticks = ns / 10;
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
}

template <typename In, int L, int W>
__global__ __launch_bounds__(W * 64) void k_tile_reg(Bufs b, int64_t S, int64_t T, int64_t D, uint32_t pause, const int2* table) {
  __shared__ float s_sum[W][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t C = S * D;
  const int2 cg = table[blockIdx.x];
  const int64_t c = cg.x, g = cg.y;
  const int64_t R = int64_t(L) * W;
  const int64_t q = g * 64 + lane;
  const bool valid = q < C;
  const int64_t qc = valid ? q : g * 64;
  const int64_t slab = qc / D, d = qc - slab * D;
  const int64_t t0 = c * R + int64_t(w) * L;
  const int nr = int(min(int64_t(L), T - t0));
  const int64_t base = (slab * T + t0) * D + d;
  const In* a = (const In*)b.in[0] + base; const In* p = (const In*)b.in[1] + base;
  const In* f = (const In*)b.in[2] + base; const In* qq = (const In*)b.in[3] + base;
  float ra[L], rp[L], rf[L], rb[L];
  float s = 0.f;
  if (nr > 0) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t o = int64_t(min(i, nr - 1)) * D;
      ra[i] = ld(a + o); rp[i] = ld(p + o); rf[i] = ld(f + o); rb[i] = ld(qq + o);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) s += ra[i] * rp[i] + rf[i] * rb[i];
  }
  s_sum[w][lane] = s;
  __syncthreads();
  if (w == 0) pause_ns(pause);
  __syncthreads();
  const float tot = s_sum[(w + 1) % W][lane] * 1e-30f;
  if (nr > 0 && valid) {
    float* o0 = b.out[0] + base; float* o1 = b.out[1] + base;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i >= nr) continue;
      __builtin_nontemporal_store(ra[i] + rp[i] + tot, o0 + int64_t(i) * D);
      __builtin_nontemporal_store(rf[i] * rb[i], o1 + int64_t(i) * D);
    }
  }
}

// pol: the scan order's tiles read and written with buffer instructions whose
// cache-policy immediate is LP (loads) and SP (stores): bit 0 sc0, bit 1 nt,
// bit 4 sc1 (sc1:sc0 the coherence scope: wave, group, device, system; nt
// non-temporal).  A wave's buffer descriptors start at its first element.
template <int POL> __device__ inline float bld(__amdgpu_buffer_rsrc_t r, uint32_t off, float*) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL); }
template <int POL> __device__ inline float bld(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t*) { return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, POL)) << 16); }
template <typename In, int L, int W, int LP, int SP>
__global__ __launch_bounds__(W * 64) void k_tile_pol(Bufs b, int64_t S, int64_t T, int64_t D, const int2* table) {
  __shared__ float s_sum[W][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t C = S * D;
  const int2 cg = table[blockIdx.x];
  const int64_t c = cg.x, g = cg.y;
  const int64_t R = int64_t(L) * W;
  const int64_t q0 = g * 64;
  const int64_t slab0 = q0 / D, d0 = q0 - slab0 * D;
  const int64_t q = q0 + lane;
  const bool valid = q < C;
  const int64_t qc = valid ? q : q0;
  const int64_t slab = qc / D, d = qc - slab * D;
  const int64_t t0 = c * R + int64_t(w) * L;
  const int nr = int(min(int64_t(L), T - t0));
  const int64_t e0 = (slab0 * T + t0) * D + d0;
  const uint32_t lane_el = uint32_t((slab - slab0) * T * D + d - d0);
  auto rs = [&](const void* p, int esz) { return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p + e0 * esz), 0, 0x7fffffff, 0x00020000); };
  const auto ra_ = rs(b.in[0], sizeof(In)), rp_ = rs(b.in[1], sizeof(In)), rf_ = rs(b.in[2], sizeof(In)), rb_ = rs(b.in[3], sizeof(In));
  float ra[L], rp[L], rf[L], rb[L];
  float s = 0.f;
  if (nr > 0) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const uint32_t o = (lane_el + uint32_t(min(i, nr - 1)) * uint32_t(D)) * sizeof(In);
      ra[i] = bld<LP>(ra_, o, (In*)0); rp[i] = bld<LP>(rp_, o, (In*)0); rf[i] = bld<LP>(rf_, o, (In*)0); rb[i] = bld<LP>(rb_, o, (In*)0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) s += ra[i] * rp[i] + rf[i] * rb[i];
  }
  s_sum[w][lane] = s;
  __syncthreads();
  const float tot = s_sum[(w + 1) % W][lane] * 1e-30f;
  const auto o0 = rs(b.out[0], 4), o1 = rs(b.out[1], 4);
  if (nr > 0 && valid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i >= nr) continue;
      const uint32_t o = (lane_el + uint32_t(i) * uint32_t(D)) * 4;
      __builtin_amdgcn_raw_buffer_store_b32(ra[i] + rp[i] + tot, o0, o, 0, SP);
      __builtin_amdgcn_raw_buffer_store_b32(rf[i] * rb[i], o1, o, 0, SP);
    }
  }
}

// float4 elementwise stream: each thread 4 consecutive elements of every tensor
template <typename In> struct V4;
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
template <> struct V4<float> { typedef f4v T; };
template <> struct V4<uint16_t> { typedef u2v T; };
__device__ inline void unpack(f4v v, float* o) { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
__device__ inline void unpack(u2v v, float* o) { o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u); o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u); }
template <typename In>
__global__ __launch_bounds__(256) void k_stream(Bufs b, int64_t N) {
  typedef typename V4<In>::T VT;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i * 4 >= N) return;
  float x[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) unpack(__builtin_nontemporal_load((const VT*)b.in[t] + i), x[t]);
  f4v o0 = {x[0][0] + x[1][0], x[0][1] + x[1][1], x[0][2] + x[1][2], x[0][3] + x[1][3]};
  f4v o1 = {x[2][0] * x[3][0], x[2][1] * x[3][1], x[2][2] * x[3][2], x[2][3] * x[3][3]};
  __builtin_nontemporal_store(o0, (f4v*)b.out[0] + i);
  __builtin_nontemporal_store(o1, (f4v*)b.out[1] + i);
}

// colstream: workgroup = NCH channels of one slab for all T; lane = (channel,
// row slice); tile k+1 loaded while tile k is summed, exchanged and stored.
template <typename In, int L>
struct ColBuf {
  float a[L], p[L], f[L], b[L];
  __device__ void load(const In* A, const In* P, const In* F, const In* B, int64_t o, int64_t D, int nr) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t oo = o + int64_t(min(i, nr - 1)) * D;
      a[i] = ld(A + oo); p[i] = ld(P + oo); f[i] = ld(F + oo); b[i] = ld(B + oo);
    }
  }
};

template <typename In, int L, int W, int NCH>
__global__ __launch_bounds__(W * 64) void k_col(Bufs bf, int64_t S, int64_t T, int64_t D) {
  constexpr int SUB = 64 / NCH;
  constexpr int64_t R = int64_t(L) * W * SUB;
  __shared__ float s_sum[2][W][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ch = lane % NCH, sub = lane / NCH;
  const int64_t units = D / NCH;
  const int64_t slab = blockIdx.x / units;
  const int64_t base = slab * T * D + (blockIdx.x - slab * units) * NCH + ch;
  const In* A = (const In*)bf.in[0] + base; const In* P = (const In*)bf.in[1] + base;
  const In* F = (const In*)bf.in[2] + base; const In* B = (const In*)bf.in[3] + base;
  float* o0 = bf.out[0] + base; float* o1 = bf.out[1] + base;
  const int64_t nc = (T + R - 1) / R;
  const int rowoff = (w * SUB + sub) * L;
  ColBuf<In, L> x, y;
  float carry = 0.f;
  auto rows = [&](int64_t k) { return int(min(int64_t(L), T - (k * R + rowoff))); };
  auto process = [&](ColBuf<In, L>& u, int64_t k) {
    const int nr = rows(k);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) s += u.a[i] * u.p[i] + u.f[i] * u.b[i];
    s_sum[k & 1][w][lane] = s;
    __syncthreads();
    carry += s_sum[k & 1][(w + 1) % W][lane] * 1e-30f;
    if (nr > 0) {
      const int64_t o = (k * R + rowoff) * D;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        if (i >= nr) continue;
        __builtin_nontemporal_store(u.a[i] + u.p[i] + carry, o0 + o + int64_t(i) * D);
        __builtin_nontemporal_store(u.f[i] * u.b[i], o1 + o + int64_t(i) * D);
      }
    }
  };
  auto fetch = [&](ColBuf<In, L>& u, int64_t k) {
    const int nr = rows(k);
    if (nr > 0) u.load(A, P, F, B, (k * R + rowoff) * D, D, nr);
  };
  if (nc > 0) fetch(x, 0);
  for (int64_t k = 0; k < nc; k += 2) {
    if (k + 1 < nc) fetch(y, k + 1);
    process(x, k);
    if (k + 1 < nc) {
      if (k + 2 < nc) fetch(x, k + 2);
      process(y, k + 1);
    }
  }
}

struct Shape { const char* name; int64_t S, T, D; int bf16; };

// Orders: tile list as (chunk, group) pairs in dispatch order.
std::vector<std::pair<int,int>> make_order(const std::string& kind, int arg, int64_t G, int64_t nc, int pair) {
  std::vector<std::pair<int,int>> v;
  if (kind == "scan") {
    for (int64_t c = 0; c < nc; ++c) for (int64_t g = 0; g < G; ++g) v.push_back({int(c), int(g)});
  } else if (kind == "addr") {
    for (int64_t g = 0; g < G; ++g) for (int64_t c = 0; c < nc; ++c) v.push_back({int(c), int(g)});
  } else if (kind == "band") {  // bands of arg columns, chunk-major within
    for (int64_t g0 = 0; g0 < G; g0 += arg) {
      const int64_t gb = std::min<int64_t>(arg, G - g0);
      for (int64_t c = 0; c < nc; ++c) for (int64_t j = 0; j < gb; ++j) v.push_back({int(c), int(g0 + j)});
    }
  } else if (kind == "super") {  // arg consecutive chunks per column, then next column
    for (int64_t c0 = 0; c0 < nc; c0 += arg) {
      const int64_t kb = std::min<int64_t>(arg, nc - c0);
      for (int64_t g = 0; g < G; ++g) for (int64_t j = 0; j < kb; ++j) v.push_back({int(c0 + j), int(g)});
    }
  } else if (kind == "skew") {  // scan order with column g started (g % K) * M chunks late (arg = K + 1000 M)
    const int64_t K = std::max(1, arg % 1000), M = std::max(1, arg / 1000), shift = pair ? 1 : 0;
    auto off = [&](int64_t g) { return ((g >> shift) % K) * M; };
    for (int64_t s = 0; s < nc + (K - 1) * M; ++s)
      for (int64_t g = 0; g < G; ++g) {
        const int64_t c = s - off(g);
        if (c >= 0 && c < nc) v.push_back({int(c), int(g)});
      }
  } else if (kind == "xcdcol") {  // scan order, but XCD x (wg mod 8) walks its own contiguous block of columns
    // wg = 8 * m + x ; tile list per XCD: columns [x*G/8, (x+1)*G/8) in scan order
    const int64_t per = G / 8;
    std::vector<std::vector<std::pair<int,int>>> lists(8);
    for (int x = 0; x < 8; ++x)
      for (int64_t c = 0; c < nc; ++c) for (int64_t j = 0; j < per; ++j) lists[x].push_back({int(c), int(x * per + j)});
    for (size_t m = 0; m < lists[0].size(); ++m) for (int x = 0; x < 8; ++x) v.push_back(lists[x][m]);
  }
  if (pair) {  // within each aligned block of 16, ids x and x + 8 get tiles 2m, 2m+1 of the block
    std::vector<std::pair<int,int>> w(v.size());
    for (size_t i = 0; i < v.size(); ++i) {
      const size_t block = i >> 4, r = i & 15;
      size_t t = i;
      if ((block + 1) * 16 <= v.size()) t = block * 16 + (r & 7) * 2 + (r >> 3);
      w[i] = v[t];
    }
    v = w;
  }
  return v;
}

template <typename In>
void run(const char* label, int kind, int arg, int L, int W, int pair, uint32_t pause, const Shape& sh, Bufs* sets, int nsets, hipStream_t st, int2* dtable) {
  const int64_t N = sh.S * sh.T * sh.D, C = sh.S * sh.D, G = (C + 63) / 64;
  const int64_t R = int64_t(L) * W, nc = R > 0 ? (sh.T + R - 1) / R : 0;
  int64_t ntiles = 0;
  if (kind == 2 && (arg <= 0 || 64 % arg != 0 || sh.D % arg != 0)) { printf("bad channel count %d\n", arg); exit(1); }
  if (kind == 1 || kind == 3) {
    auto v = make_order(kind == 3 ? "scan" : label, arg, G, nc, pair);
    ntiles = int64_t(v.size());
    if (ntiles != G * nc) { printf("bad order size\n"); exit(1); }
    std::vector<int2> h(ntiles);
    for (int64_t i = 0; i < ntiles; ++i) h[i] = make_int2(v[i].first, v[i].second);
    CK(hipMemcpy(dtable, h.data(), ntiles * sizeof(int2), hipMemcpyHostToDevice));
  }
  auto launch = [&](const Bufs& b) {
    if (kind == 0) {
      const int64_t blocks = (N / 4 + 255) / 256;
      hipLaunchKernelGGL(k_stream<In>, dim3(blocks), dim3(256), 0, st, b, N);
      return;
    }
    if (kind == 3) {
      const dim3 grid{unsigned(ntiles)}, block{unsigned(W * 64)};
#define TP(LL, WW, LPP, SPP) if (L == LL && W == WW && arg == LPP * 100 + SPP) { hipLaunchKernelGGL((k_tile_pol<In, LL, WW, LPP, SPP>), grid, block, 0, st, b, sh.S, sh.T, sh.D, dtable); return; }
#define TPS(LL, WW) TP(LL, WW, 2, 2) TP(LL, WW, 3, 2) TP(LL, WW, 18, 2) TP(LL, WW, 19, 2) TP(LL, WW, 16, 2) TP(LL, WW, 1, 2) \
      TP(LL, WW, 2, 3) TP(LL, WW, 2, 18) TP(LL, WW, 2, 19) TP(LL, WW, 2, 16) TP(LL, WW, 18, 18) TP(LL, WW, 19, 19) TP(LL, WW, 0, 2) TP(LL, WW, 2, 0)
      TPS(28, 4) TPS(24, 4) TPS(14, 8)
      printf("no pol variant\n"); exit(1);
    }
    if (kind == 2) {
      const dim3 cgrid{unsigned(sh.S * (sh.D / arg))}, cblock{unsigned(W * 64)};
#define TC(LL, WW, NN) if (L == LL && W == WW && arg == NN) { hipLaunchKernelGGL((k_col<In, LL, WW, NN>), cgrid, cblock, 0, st, b, sh.S, sh.T, sh.D); return; }
      TC(4, 16, 64) TC(8, 8, 64) TC(4, 16, 32) TC(8, 8, 32) TC(8, 4, 32) TC(16, 4, 16) TC(8, 8, 16)
      printf("no colstream variant L=%d W=%d arg=%d\n", L, W, arg); exit(1);
    }
    const dim3 grid{unsigned(ntiles)}, block{unsigned(W * 64)};
#define TR(LL, WW) if (L == LL && W == WW) { hipLaunchKernelGGL((k_tile_reg<In, LL, WW>), grid, block, 0, st, b, sh.S, sh.T, sh.D, pause, dtable); return; }
    TR(28, 4) TR(24, 4) TR(16, 4) TR(32, 4) TR(14, 8) TR(20, 4)
    printf("no variant L=%d W=%d\n", L, W); exit(1);
  };
  for (int i = 0; i < 3; ++i) launch(sets[i % nsets]);
  CK(hipGetLastError());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  const int K = 20;
  CK(hipEventRecord(e0, st));
  for (int i = 0; i < K; ++i) launch(sets[i % nsets]);
  CK(hipEventRecord(e1, st));
  CK(hipEventSynchronize(e1));
  float ms; CK(hipEventElapsedTime(&ms, e0, e1));
  const double us = ms * 1000.0 / K;
  const double bytes = double(N) * (4 * sizeof(In) + 8);
  printf("%-5s %-7s arg=%5d L=%2d W=%d pair=%d pause=%5u  %9.1f us  %6.0f GB/s  frac %.3f\n", sh.name, label, arg, L, W, pair, pause, us, bytes / us * 1e-3, bytes / us * 1e-3 / 8000.0);
  fflush(stdout);
  CK(hipEventDestroy(e0)); CK(hipEventDestroy(e1));
}

int main(int argc, char** argv) {
  if (argc < 7) { printf("usage\n"); return 2; }
  const int which = atoi(argv[1]);
  Shape shapes[] = {{"cfg1", 128, 2048, 64, 0}, {"cfg2", 128, 8192, 128, 1}, {"cfg3", 32, 131072, 128, 0}};
  const Shape sh = shapes[which - 1];
  const int64_t N = sh.S * sh.T * sh.D;
  const size_t esz = sh.bf16 ? 2 : 4;
  const int nsets = argc > 7 ? atoi(argv[7]) : 2;
  if (nsets < 1 || nsets > 16) { printf("sets must be 1..16\n"); return 2; }
  Bufs sets[16];
  for (int s = 0; s < nsets; ++s) {
    for (int i = 0; i < 4; ++i) { void* p; CK(hipMalloc(&p, N * esz)); CK(hipMemset(p, 0x3c, N * esz)); sets[s].in[i] = p; }
    for (int i = 0; i < 2; ++i) { CK(hipMalloc(&sets[s].out[i], N * 4)); }
  }
  int2* dtable; CK(hipMalloc(&dtable, sizeof(int2) * (N / 64 / 16 + 1024)));
  hipStream_t st; CK(hipStreamCreate(&st));
  const std::string order = argv[2];
  const int kind = order == "stream" ? 0 : order == "colstream" ? 2 : order == "pol" ? 3 : 1;
  const int arg = atoi(argv[3]), L = atoi(argv[4]), W = atoi(argv[5]), pair = atoi(argv[6]);
  if (sh.bf16) run<uint16_t>(order.c_str(), kind, arg, L, W, pair, 0, sh, sets, nsets, st, dtable);
  else run<float>(order.c_str(), kind, arg, L, W, pair, 0, sh, sets, nsets, st, dtable);
  return 0;
}

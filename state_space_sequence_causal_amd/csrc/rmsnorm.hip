// Group RMSNorm of the gated output of the Mamba-2 layer core: the block's RMSNorm
// (hyper.ai summary of the Nemotron-Nano-2 report, section "方法"), taken after the SiLU(z)
// gate over each of the G groups of d_inner / G contiguous channels:
//     out[k] = g[k] / sqrt(mean over k's group of g^2 + eps) * weight[k].
//
// HBM-bound: every element is read from HBM once and written once. One wave per (row,
// group) unit. For groups of up to 256 16-byte vectors (2048 bf16
// channels; 1280 at the 12B shape) each lane requests all of its K vectors at once and
// keeps them in registers, sums their squares, and after a fixed shuffle tree (so the
// rounding order never changes) scales and stores them. (Waves that walk several units and
// prefetch the next were slower.) Wider groups take two passes, the second re-reading the
// group. out may be g itself: a unit is read completely before any of it is written.
#include "device.h"
#include "launch.h"

namespace m2 {

// 16-byte load and store with the non-temporal hint: each value is read once and written
// once, so neither should displace other data in the caches (71 to 68 us over the 12B 8k
// gated output; the same hint on the conv call's stores made it slower, 78 to 88 us)
template <typename T> __device__ __forceinline__ Vec<T> ld16_stream(const T* p) {
  Vec<T> r;
  r.v = __builtin_nontemporal_load(reinterpret_cast<const decltype(r.v)*>(p));
  return r;
}
template <typename T> __device__ __forceinline__ void st16_stream(T* p, const Vec<T>& r) {
  __builtin_nontemporal_store(r.v, reinterpret_cast<decltype(r.v)*>(p));
}

constexpr int RMS_THREADS = 256;

template <typename T>
__device__ __forceinline__ void rms_weights(const float* weight, int64_t k0, float (&wk)[Vec<T>::VE]) {
#pragma unroll
  for (int i = 0; i < Vec<T>::VE; ++i) wk[i] = weight ? weight[k0 + i] : 1.f;
}

// One (row, group) unit per wave. K > 0: each lane holds K vectors of the unit in
// registers. K == 0: two passes over the group.
template <typename T, int K>
__global__ __launch_bounds__(RMS_THREADS) void group_rmsnorm_kernel(
    const T* g, int64_t g_stride, const float* __restrict__ weight, float eps, T* out,
    int64_t out_stride, int64_t units, int G, int gw) {
  constexpr int VE = Vec<T>::VE;
  const int lane = threadIdx.x & 63;
  const int64_t unit0 = (int64_t)blockIdx.x * (RMS_THREADS / 64) + (threadIdx.x >> 6);
  if (unit0 >= units) return;   // whole waves leave together
  const int nv = gw / VE;
  auto src_of = [&](int64_t u) { return g + (u / G) * g_stride + (int64_t)(u % G) * gw; };
  auto dst_of = [&](int64_t u) { return out + (u / G) * out_stride + (int64_t)(u % G) * gw; };

  if constexpr (K > 0) {
    // past the group's end a lane re-reads the last vector (and counts nothing), so every
    // load is unconditional and all K are in flight together
    const T* src = src_of(unit0);
    Vec<T> a[K];
#pragma unroll
    for (int k = 0; k < K; ++k) a[k] = ld16_stream(src + min(lane + 64 * k, nv - 1) * VE);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VE; ++i) s += a[k].get(i) * a[k].get(i);
      ss += lane + 64 * k < nv ? s : 0.f;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);   // fixed order
    const float scale = 1.f / sqrtf(ss / (float)gw + eps);
    T* dst = dst_of(unit0);
    const int64_t wbase = (int64_t)(unit0 % G) * gw;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int v = lane + 64 * k;
      if (v < nv) {
        float wk[VE];
        rms_weights<T>(weight, wbase + v * VE, wk);
        Vec<T> o;
#pragma unroll
        for (int i = 0; i < VE; ++i) o.set(i, a[k].get(i) * scale * wk[i]);
        st16_stream(dst + v * VE, o);
      }
    }
  } else {
    const T* src = src_of(unit0);
    T* dst = dst_of(unit0);
    const int64_t wbase = (int64_t)(unit0 % G) * gw;
    float ss = 0.f;
    for (int v = lane; v < nv; v += 64) {
      const Vec<T> a = ld16(src + v * VE);
#pragma unroll
      for (int i = 0; i < VE; ++i) ss += a.get(i) * a.get(i);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float scale = 1.f / sqrtf(ss / (float)gw + eps);
    for (int v = lane; v < nv; v += 64) {
      const Vec<T> a = ld16(src + v * VE);
      float wk[VE];
      rms_weights<T>(weight, wbase + v * VE, wk);
      Vec<T> o;
#pragma unroll
      for (int i = 0; i < VE; ++i) o.set(i, a.get(i) * scale * wk[i]);
      st16(dst + v * VE, o);
    }
  }
}

template <typename T, int K>
static hipError_t launch_k(const void* g, int64_t g_stride, const float* weight, float eps, void* out,
                           int64_t out_stride, int64_t rows, int G, int width, hipStream_t stream) {
  const int64_t units = rows * G;
  const int64_t blocks = (units + RMS_THREADS / 64 - 1) / (RMS_THREADS / 64);
  hipLaunchKernelGGL((group_rmsnorm_kernel<T, K>), dim3((unsigned)blocks), dim3(RMS_THREADS), 0, stream,
                     static_cast<const T*>(g), g_stride, weight, eps, static_cast<T*>(out), out_stride,
                     units, G, width / G);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(const void* g, int64_t g_stride, const float* weight, float eps, void* out,
                           int64_t out_stride, int64_t rows, int G, int width, hipStream_t stream) {
  const int nv = width / G / Vec<T>::VE;   // 16-byte vectors per group
  const int K = (nv + 63) / 64;
  switch (K) {
    case 1: return launch_k<T, 1>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
    case 2: return launch_k<T, 2>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
    case 3: return launch_k<T, 3>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
    case 4: return launch_k<T, 4>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
    default: return launch_k<T, 0>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
  }
}

hipError_t launch_group_rmsnorm(int io_bf16, const void* g, int64_t g_stride, const float* weight,
                                float eps, void* out, int64_t out_stride, int64_t rows, int G,
                                int width, hipStream_t stream) {
  if (io_bf16) return launch_t<bf16>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
  return launch_t<float>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
}

}  // namespace m2

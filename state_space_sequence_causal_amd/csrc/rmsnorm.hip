// Group RMSNorm of the gated output of the Mamba-2 layer core: the block's RMSNorm
// (hyper.ai summary of the Nemotron-Nano-2 report, section "方法"), taken after the SiLU(z)
// gate over each of the G groups of d_inner / G contiguous channels:
//     out[k] = g[k] / sqrt(mean over k's group of g^2 + eps) * weight[k].
//
// HBM-bound: every element is read from HBM once and written once. One wave per (row,
// group): a first pass sums the squares of the group's 16-byte vectors (lanes strided by
// the wave width, then a fixed shuffle tree, so the sum's rounding order never changes),
// a second pass re-reads the vectors (2.5 KiB per group at the 12B shape, still in L2),
// scales and stores them. out may be g itself.
#include "device.h"
#include "launch.h"

namespace m2 {

constexpr int RMS_THREADS = 256;

template <typename T>
__global__ __launch_bounds__(RMS_THREADS) void group_rmsnorm_kernel(
    const T* g, int64_t g_stride, const float* __restrict__ weight, float eps, T* out,
    int64_t out_stride, int64_t units, int G, int gw) {
  constexpr int VE = Vec<T>::VE;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * (RMS_THREADS / 64) + (threadIdx.x >> 6);
  if (unit >= units) return;   // whole waves leave together
  const int64_t row = unit / G;
  const int grp = (int)(unit % G);
  const int nv = gw / VE;
  const T* src = g + row * g_stride + (int64_t)grp * gw;
  T* dst = out + row * out_stride + (int64_t)grp * gw;

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
    Vec<T> o;
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      const float wk = weight ? weight[(int64_t)grp * gw + v * VE + i] : 1.f;
      o.set(i, a.get(i) * scale * wk);
    }
    st16(dst + v * VE, o);
  }
}

template <typename T>
static hipError_t launch_t(const void* g, int64_t g_stride, const float* weight, float eps, void* out,
                           int64_t out_stride, int64_t rows, int G, int width, hipStream_t stream) {
  const int64_t units = rows * G;
  const int64_t blocks = (units + RMS_THREADS / 64 - 1) / (RMS_THREADS / 64);
  hipLaunchKernelGGL((group_rmsnorm_kernel<T>), dim3((unsigned)blocks), dim3(RMS_THREADS), 0, stream,
                     static_cast<const T*>(g), g_stride, weight, eps, static_cast<T*>(out), out_stride,
                     units, G, width / G);
  return hipGetLastError();
}

hipError_t launch_group_rmsnorm(int io_bf16, const void* g, int64_t g_stride, const float* weight,
                                float eps, void* out, int64_t out_stride, int64_t rows, int G,
                                int width, hipStream_t stream) {
  if (io_bf16) return launch_t<bf16>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
  return launch_t<float>(g, g_stride, weight, eps, out, out_stride, rows, G, width, stream);
}

}  // namespace m2

// Causal depthwise conv1d (width 4) + bias + SiLU over the xBC channels of the
// Mamba-2 block ("conv window 4": hyper.ai summary of arXiv 2508.14444, section
// "方法"; neurohive article, section "Архитектура").
//
// HBM-bound: each io element is read once (plus a 3-token halo per 128-token
// tile) and written once. SiLU uses the hardware exp2 and reciprocal (a few
// fp32 ulps, far below the bf16 rounding of the output); with the accurate
// library calls the kernel was bound by their instruction count. A thread owns one 16-byte column of channels (8 bf16 or 4 f32)
// over a tile of tokens and slides the 4-tap window along time in registers,
// so loads and stores are whole 16-byte vectors and a wave covers 1 KiB of
// contiguous channels per row.
#include "device.h"
#include "launch.h"

namespace m2 {

constexpr int CONV_THREADS = 256;
constexpr int CONV_W = 4;

template <typename T, int TT>
__global__ __launch_bounds__(CONV_THREADS) void conv1d_kernel(
    const T* __restrict__ u, int64_t u_stride, const float* __restrict__ w,
    const float* __restrict__ bias, T* conv_state, T* __restrict__ out, int64_t out_stride,
    int L, int Cc) {
  constexpr int VE = Vec<T>::VE;
  const int c0 = (blockIdx.x * CONV_THREADS + threadIdx.x) * VE;
  if (c0 >= Cc) return;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int t1 = min(L, t0 + TT);
  const T* ub = u + (int64_t)b * L * u_stride + c0;
  T* ob = out + (int64_t)b * L * out_stride + c0;

  f32x4 wt[VE];
  float bs[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) {
    wt[i] = *reinterpret_cast<const f32x4*>(w + (int64_t)(c0 + i) * CONV_W);
    bs[i] = bias ? bias[c0 + i] : 0.f;
  }

  // window: e0 = u[t-3], e1 = u[t-2], e2 = u[t-1]
  Vec<T> hist[CONV_W - 1];
  T* csb = conv_state ? conv_state + (int64_t)b * (CONV_W - 1) * Cc + c0 : nullptr;
#pragma unroll
  for (int j = 0; j < CONV_W - 1; ++j) {
    int t = t0 - (CONV_W - 1) + j;
    if (t >= 0) hist[j] = ld16(ub + (int64_t)t * u_stride);
    else if (csb) hist[j] = ld16(csb + (int64_t)(t + CONV_W - 1) * Cc);
    else hist[j] = zero16<T>();
  }
  Vec<T> e0 = hist[0], e1 = hist[1], e2 = hist[2];

  constexpr int U = 16;   // loads in flight per thread
  int t = t0;
  for (; t + U <= t1; t += U) {
    Vec<T> cur[U];
#pragma unroll
    for (int k = 0; k < U; ++k) cur[k] = ld16(ub + (int64_t)(t + k) * u_stride);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      Vec<T> o;
#pragma unroll
      for (int i = 0; i < VE; ++i)
        o.set(i, conv4_silu(wt[i], bs[i], e0.get(i), e1.get(i), e2.get(i), cur[k].get(i)));
      st16(ob + (int64_t)(t + k) * out_stride, o);
      e0 = e1; e1 = e2; e2 = cur[k];
    }
  }
  for (; t < t1; ++t) {
    Vec<T> cur = ld16(ub + (int64_t)t * u_stride);
    Vec<T> o;
#pragma unroll
    for (int i = 0; i < VE; ++i)
      o.set(i, conv4_silu(wt[i], bs[i], e0.get(i), e1.get(i), e2.get(i), cur.get(i)));
    st16(ob + (int64_t)t * out_stride, o);
    e0 = e1; e1 = e2; e2 = cur;
  }

  // The tile-0 thread of each channel column is the only reader of the old history
  // (already in registers), so it alone writes the new one: the last W-1 entries of
  // the extended sequence (history, u[0..L-1]).
  if (blockIdx.y == 0 && csb) {
    Vec<T> fin[CONV_W - 1];
#pragma unroll
    for (int j = 0; j < CONV_W - 1; ++j) {
      int i = L + j;  // index into the extended sequence; u[t] sits at t + W - 1
      if (i == 0) fin[j] = hist[0];
      else if (i == 1) fin[j] = hist[1];
      else if (i == 2) fin[j] = hist[2];
      else fin[j] = ld16(ub + (int64_t)(i - (CONV_W - 1)) * u_stride);
    }
#pragma unroll
    for (int j = 0; j < CONV_W - 1; ++j) st16(csb + (int64_t)j * Cc, fin[j]);
  }
}

template <typename T>
static hipError_t launch_t(const void* u, int64_t u_stride, const float* w, const float* bias,
                           void* conv_state, void* out, int64_t out_stride, int B, int L, int Cc,
                           hipStream_t stream) {
  constexpr int TT = 128;
  constexpr int VE = Vec<T>::VE;
  dim3 grid((Cc / VE + CONV_THREADS - 1) / CONV_THREADS, (L + TT - 1) / TT, B);
  hipLaunchKernelGGL((conv1d_kernel<T, TT>), grid, dim3(CONV_THREADS), 0, stream,
                     static_cast<const T*>(u), u_stride, w, bias, static_cast<T*>(conv_state),
                     static_cast<T*>(out), out_stride, L, Cc);
  return hipGetLastError();
}

hipError_t launch_conv1d(int io_bf16, const void* u, int64_t u_stride, const float* w,
                         const float* bias, void* conv_state, void* out, int64_t out_stride,
                         int B, int L, int Cc, hipStream_t stream) {
  if (io_bf16)
    return launch_t<bf16>(u, u_stride, w, bias, conv_state, out, out_stride, B, L, Cc, stream);
  return launch_t<float>(u, u_stride, w, bias, conv_state, out, out_stride, B, L, Cc, stream);
}

}  // namespace m2

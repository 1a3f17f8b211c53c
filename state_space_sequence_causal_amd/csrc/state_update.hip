// One-token decode of the Mamba-2 layer core, both caches updated in place.
//
// The fp32 SSM cache (neurohive article on Nemotron-Nano-2, section
// "Развертывание": the Mamba cache must be kept in float32) dominates the
// traffic: 32 KiB per (sequence, head) read and written once per token, against
// ~0.5 KiB of token inputs. The kernel is therefore a pure HBM stream of the
// state with the conv, dt, gate and output folded into it.
//
// One workgroup per (sequence b, group g): it owns the x channels of the
// group's heads and the group's B and C channels, so every conv-cache column
// has exactly one reader-writer (no cross-workgroup ordering is needed). Each of
// its 16 waves streams one head (two for wider groups) in parts of 8 rows: lane
// (q = l % 16, rg = l / 16) handles p = 4q..4q+3 of rows n = rg + 4k, so one
// wave instruction touches 1 KiB of contiguous state. Two parts are in flight
// while one is updated, and the first two are requested before the conv step,
// which they do not need. y is reduced over the four row groups with cross-lane
// shuffles. Small parts and many waves per CU measured best on MI355X (about
// 5.4 TB/s at batch 64, against about 6.0 TB/s for a plain in-place stream).
#include "device.h"
#include "launch.h"

namespace m2 {

constexpr int DEC_WAVES = 16;
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_P = 64;
constexpr int DEC_N = 128;
constexpr int DEC_W = 4;
constexpr int DEC_K = 2;            // state rows per lane in one work item
constexpr int DEC_IPH = 32 / DEC_K;  // work items per head

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = (f32x4){a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = (bf16x4){(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return (f32x4){(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename T>
__global__ __launch_bounds__(DEC_THREADS) __attribute__((amdgpu_waves_per_eu(4, 8)))
void state_update_kernel(
    const T* __restrict__ u_t, const float* __restrict__ w, const float* __restrict__ bias,
    T* __restrict__ conv_state, const T* __restrict__ dt_raw_t, const float* __restrict__ dt_bias,
    const float* __restrict__ A, const float* __restrict__ D, const T* __restrict__ z_t,
    float* __restrict__ ssm_state, T* __restrict__ y_t, int H, int G) {
  extern __shared__ float smem[];
  constexpr int VE = Vec<T>::VE;
  const int hpg = H / G;
  const int nblk = gridDim.x;
  const int id = xcd_local_order(blockIdx.x, nblk);
  const int b = id / G, g = id % G;
  const int di = H * DEC_P;
  const int Cc = di + 2 * G * DEC_N;
  const int nx = hpg * DEC_P;          // x channels owned
  const int nch = nx + 2 * DEC_N;      // plus B and C of the group
  float* xs = smem;                    // [nx] conv output of the x channels
  float* bsm = smem + nx;              // [N]
  float* csm = bsm + DEC_N;            // [N]
  float* dts = csm + DEC_N;            // [hpg]
  float* das = dts + hpg;              // [hpg] decay a = exp(dt A)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int q = lane & 15, rg = lane >> 4;

  // Work items of this wave: (head j, part) for j = wave, wave + 8, ...; part m holds the
  // 4 DEC_K state rows n = 4 DEC_K m + rg + 4k, k < DEC_K.
  const int nitems = ((hpg - wave + DEC_WAVES - 1) / DEC_WAVES) * DEC_IPH;
  auto item_ptr = [&](int it) {
    const int j = wave + DEC_WAVES * (it / DEC_IPH);
    const int h = g * hpg + j;
    return ssm_state + ((int64_t)b * H + h) * DEC_N * DEC_P + (4 * DEC_K * (it % DEC_IPH) + rg) * DEC_P +
           4 * q;
  };
  f32x4 buf[3][DEC_K];
  auto load_item = [&](int it, f32x4 (&dst)[DEC_K]) {
    const float* st = item_ptr(it);
#pragma unroll
    for (int k = 0; k < DEC_K; ++k)
      dst[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + 4 * k * DEC_P));
  };
  // the state does not depend on the conv: the first two parts are requested first
  if (nitems > 0) load_item(0, buf[0]);
  if (nitems > 1) load_item(1, buf[1]);

  // conv step on the owned channels; the cache shifts by one token
  const T* ub = u_t + (int64_t)b * Cc;
  T* csb = conv_state + (int64_t)b * (DEC_W - 1) * Cc;
  for (int v = tid; v < nch / VE; v += DEC_THREADS) {
    int lc = v * VE;
    int c = lc < nx ? g * nx + lc
                    : (lc < nx + DEC_N ? di + g * DEC_N + (lc - nx) : di + G * DEC_N + g * DEC_N + (lc - nx - DEC_N));
    Vec<T> s0 = ld16(csb + c), s1 = ld16(csb + Cc + c), s2 = ld16(csb + 2 * Cc + c);
    Vec<T> cur = ld16(ub + c);
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      f32x4 wv = *reinterpret_cast<const f32x4*>(w + (int64_t)(c + i) * DEC_W);
      float acc = (bias ? bias[c + i] : 0.f) + wv[0] * s0.get(i) + wv[1] * s1.get(i) +
                  wv[2] * s2.get(i) + wv[3] * cur.get(i);
      smem[lc + i] = silu_fast(acc);
    }
    st16(csb + c, s1);
    st16(csb + Cc + c, s2);
    st16(csb + 2 * Cc + c, cur);
  }
  for (int j = tid; j < hpg; j += DEC_THREADS) {
    int h = g * hpg + j;
    float dt = softplus_f(to_f(dt_raw_t[(int64_t)b * H + h]) + dt_bias[h]);
    dts[j] = dt;
    das[j] = expf(dt * A[h]);
  }
  __syncthreads();

  // stream the items: load item it+1 while item it is updated and stored
  f32x4 yacc = {0.f, 0.f, 0.f, 0.f};
  auto process = [&](int it, const f32x4 (&hv)[DEC_K]) {
    const int j = wave + DEC_WAVES * (it / DEC_IPH);
    const int h = g * hpg + j;
    const float a = das[j], dt = dts[j];
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(xs + j * DEC_P + 4 * q);
    const f32x4 dx = dt * x4;
    float* st = item_ptr(it);
    const int n0 = 4 * DEC_K * (it % DEC_IPH) + rg;
#pragma unroll
    for (int k = 0; k < DEC_K; ++k) {
      const float bn = bsm[n0 + 4 * k], cn = csm[n0 + 4 * k];
      f32x4 nv;
      nv[0] = a * hv[k][0] + bn * dx[0];
      nv[1] = a * hv[k][1] + bn * dx[1];
      nv[2] = a * hv[k][2] + bn * dx[2];
      nv[3] = a * hv[k][3] + bn * dx[3];
      yacc[0] += cn * nv[0];
      yacc[1] += cn * nv[1];
      yacc[2] += cn * nv[2];
      yacc[3] += cn * nv[3];
      __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(st + 4 * k * DEC_P));
    }
    if (it % DEC_IPH == DEC_IPH - 1) {
      // head done: reduce y over the four row groups, add the skip term, gate, store
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        yacc[i] += __shfl_xor(yacc[i], 16);
        yacc[i] += __shfl_xor(yacc[i], 32);
      }
      if (rg == 0) {
        const float dh = D ? D[h] : 0.f;
        f32x4 o = yacc + dh * x4;
        if (z_t) {
          f32x4 zz = load4(z_t + (int64_t)b * di + h * DEC_P + 4 * q);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] *= silu_fast(zz[i]);
        }
        store4(y_t + (int64_t)b * di + h * DEC_P + 4 * q, o[0], o[1], o[2], o[3]);
      }
      yacc = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  // three buffers in rotation: part it+2 is requested while part it is updated
  for (int it = 0; it < nitems; it += 3) {
    if (it + 2 < nitems) load_item(it + 2, buf[2]);
    process(it, buf[0]);
    if (it + 1 < nitems) {
      if (it + 3 < nitems) load_item(it + 3, buf[0]);
      process(it + 1, buf[1]);
    }
    if (it + 2 < nitems) {
      if (it + 4 < nitems) load_item(it + 4, buf[1]);
      process(it + 2, buf[2]);
    }
  }
}

template <typename T>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int hpg = a.H / a.G;
  size_t lds = sizeof(float) * (size_t)(hpg * DEC_P + 2 * DEC_N + 2 * hpg);
  hipLaunchKernelGGL((state_update_kernel<T>), dim3(a.B * a.G), dim3(DEC_THREADS), lds, stream,
                     static_cast<const T*>(a.u_t), a.w, a.bias, static_cast<T*>(a.conv_state),
                     static_cast<const T*>(a.dt_raw_t), a.dt_bias, a.A, a.D,
                     static_cast<const T*>(a.z_t), a.ssm_state, static_cast<T*>(a.y_t), a.H, a.G);
  return hipGetLastError();
}

hipError_t launch_state_update(int io_bf16, const DecodeArgs& a, hipStream_t stream) {
  return io_bf16 ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace m2

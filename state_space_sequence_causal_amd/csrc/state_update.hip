// One-token decode of the Mamba-2 layer core, both caches updated in place.
//
// The fp32 SSM cache (neurohive article on Nemotron-Nano-2, section
// "Развертывание": the Mamba cache must be kept in float32) dominates the
// traffic: 32 KiB per (sequence, head) read and written once per token, against
// ~0.5 KiB of token inputs. The kernel is therefore a pure HBM stream of the
// state with the conv, dt, gate and output folded into it.
//
// With a slot map the caches of token b are an entry of cache pools (continuous
// batching); the rest is unchanged.
//
// One workgroup per (sequence b, group g): it owns the x channels of the
// group's heads and the group's B and C channels, so every conv-cache column
// has exactly one reader-writer (no cross-workgroup ordering is needed). With
// few (sequence, group) pairs, 2 or 4 workgroups share a pair, each with its
// share of the heads and their x channels; the shared B and C columns are then
// shifted by a second, small kernel on the same stream, which the stream starts
// only after every read of the old cache is done (see SPLIT below). When such a
// workgroup holds at most 4 heads, its 16 waves share them: each requests all of
// its 8 parts of one head at once, and y is formed from LDS afterwards (STAGED
// below). Otherwise each of its 16 waves (8 for several tokens a call) streams one head (two or
// more for wider groups, and at 8 waves) in parts of 4 rows: lane
// (q = l % 16, rg = l / 16) handles p = 4q..4q+3 of row n = 4m + rg, so one wave
// instruction touches 1 KiB of contiguous state. Parts rotate through 4 register
// buffers with 3 in flight; every load is unconditional (loads past the wave's
// last part re-read it), so the compiler's count of outstanding memory
// operations is exact and each wait is for the one part it needs. At start-up the
// conv and dt inputs are requested first and the first three state parts right
// after, so the conv that gates the stream does not wait behind the state. A
// head's z is requested when its stream starts and used when it ends. y is
// reduced over the four row groups with cross-lane shuffles. At batch 64 the
// kernel streams about 5.8 TB/s, the rate of a plain in-place stream of the same
// size on this part (an elementwise in-place multiply: 5.87 TB/s). The order in
// which the chip's XCDs take the state blocks matters: with the blocks of each
// XCD contiguous the same kernel streamed 5.45 TB/s; walking a head's parts from
// a start that differs between waves, or letting a workgroup's waves move through
// its heads together, 4.6 to 4.8 TB/s.
#include "device.h"
#include "launch.h"

namespace m2 {

constexpr int DEC_WAVES = 16;
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_P = 64;
constexpr int DEC_N = 128;
constexpr int DEC_W = 4;
constexpr int DEC_K = 1;            // state rows per lane in one work item
constexpr int DEC_NB = 4;           // item buffers
constexpr int DEC_IPH = 32 / DEC_K;  // work items per head
constexpr int DEC_MAX_HPG = 256;     // heads per group the kernel covers (one dt thread each)
static_assert(DEC_MAX_HPG <= DEC_THREADS, "one thread per head for dt");

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

// NT tokens per sequence (1 .. 6; rows b NT + t of u_t, dt_raw_t, z_t, y_t, with row strides us,
// dtrs, zs in elements; y_t is dense), applied in order: the
// conv over the extended sequence (cache, tokens), then for each state part NT updates in
// registers, so the state is read and written once per call. Each token's arithmetic is the
// one-token step's, so NT tokens give the bits of NT one-token calls.
// SPLIT workgroups share a (sequence, group), each with hpg / SPLIT of its heads (small
// batches, so that more CUs stream state). Each convolves B and C from the cache and leaves
// the B and C cache columns alone: conv_shift_bc_kernel, next on the stream, shifts them.
// STAGED (split launches whose share is at most 4 heads, 16 % hpp == 0): every wave of the
// workgroup takes 32 hpp / 16 consecutive parts of one head, all requested at once, updates
// them and stores them, and puts the new parts in LDS; after a barrier the head's first wave
// forms y from LDS in the part order of the one-wave stream, so the bits are the same.
// WAVES: waves per workgroup (16; 8 for several tokens, whose register use lets only one
// 16-wave workgroup per CU: with 8, two heads a wave, the 9B batch-64 grid fits in one round).
template <typename T, int NT, int NB = DEC_NB, int SPLIT = 1, bool STAGED = false, int WAVES = DEC_WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(NT == 1 && NB == DEC_NB ? 8 : 4, 8)))
void state_update_kernel(
    const T* __restrict__ u_t, const float* __restrict__ w, const float* __restrict__ bias,
    T* __restrict__ conv_state, const T* __restrict__ dt_raw_t, const float* __restrict__ dt_bias,
    const float* __restrict__ A, const float* __restrict__ D, const T* __restrict__ z_t,
    float* __restrict__ ssm_state, T* __restrict__ y_t, int H, int G, const int32_t* __restrict__ slots,
    int npool, int64_t us, int64_t zs, int64_t dtrs) {
  static_assert(DEC_IPH % NB == 0, "a head's parts fill whole rounds of the buffers");
  static_assert(SPLIT == 1 || NT == 1, "split launches take one token");
  constexpr int NWAVES = WAVES, NTHREADS = WAVES * 64;
  static_assert(DEC_MAX_HPG <= NTHREADS, "one thread per head for dt");
  static_assert(!STAGED || (SPLIT > 1 && NB >= DEC_IPH / 4), "staged launches: split, one token, up to 8 parts a wave");
  extern __shared__ float smem[];
  constexpr int VE = Vec<T>::VE;
  const int hpg = H / G;
  // Workgroups in launch order, which the dispatcher deals to the XCDs in turn: each XCD then
  // streams every eighth state block rather than one contiguous eighth of the cache (9B batch
  // 64: 93.8 us against 100.5 us with the blocks of an XCD contiguous).
  const int id = blockIdx.x;
  const int part = id % SPLIT;
  const int b = id / SPLIT / G, g = id / SPLIT % G;
  const int hpp = hpg / SPLIT;         // heads of this workgroup
  const int h0w = g * hpg + part * hpp;   // its first head
  const int di = H * DEC_P;
  const int Cc = di + 2 * G * DEC_N;
  const int nx = hpp * DEC_P;          // x channels owned
  const int nch = nx + 2 * DEC_N;      // plus B and C of the group
  // per token t: the conv output of x [nx], B [N], C [N] at smem + t nch; then dt and the decay
  // a = exp(dt A) per (token, head)
  auto xs = [&](int t) { return smem + t * nch; };
  auto bsm = [&](int t) { return smem + t * nch + nx; };
  auto csm = [&](int t) { return smem + t * nch + nx + DEC_N; };
  float* dts = smem + NT * nch;        // [NT][hpp]
  float* das = dts + NT * hpp;         // [NT][hpp]
  // STAGED: the new state parts, [head][part][lane] 16 bytes each, 16-byte aligned
  f32x4* stg = reinterpret_cast<f32x4*>(smem + ((NT * nch + 2 * NT * hpp + 3) & ~3));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the caches of token b are entry sb of the pools (entry b without a slot map); a token
  // whose entry is out of range is skipped: its y is zero and no cache is touched
  int sb = b;
  if (slots) {
    sb = slots[b];
    if (sb < 0 || sb >= npool) {
      for (int i = tid; i < NT * hpp * DEC_P / 4; i += NTHREADS) {
        const int t = i / (hpp * DEC_P / 4), k = i % (hpp * DEC_P / 4);
        store4(y_t + ((int64_t)b * NT + t) * di + h0w * DEC_P + 4 * k, 0.f, 0.f, 0.f, 0.f);
      }
      return;   // the whole workgroup leaves
    }
  }
  const int q = lane & 15, rg = lane >> 4;

  // Work items of this wave: (head j, part) for j = wave, wave + NWAVES, ...; part m holds
  // the 4 DEC_K state rows n = 4 DEC_K m + rg + 4k, k < DEC_K. Item it of the wave is part
  // it % DEC_IPH of its head it / DEC_IPH.
  const int nheads_w = (hpp - wave + NWAVES - 1) / NWAVES;
  const int nitems = nheads_w * DEC_IPH;
  // the wave's state base is uniform; an item is a 32-bit byte offset from it (heads of a
  // wave are NWAVES apart, parts of a head 4 DEC_K rows apart)
  const char* wbase = reinterpret_cast<const char*>(
      ssm_state + ((int64_t)sb * H + h0w + wave) * DEC_N * DEC_P);
  const uint32_t lane_off = (uint32_t)(rg * DEC_P + 4 * q) * 4u;
  auto item_off = [&](int it) -> uint32_t {
    return (uint32_t)((it / DEC_IPH) * NWAVES * DEC_N * DEC_P + (it % DEC_IPH) * 4 * DEC_K * DEC_P) * 4u;
  };
  auto item_ptr = [&](int it) {
    return const_cast<float*>(reinterpret_cast<const float*>(wbase + (item_off(it) + lane_off)));
  };
  // NB buffers, item it in buffer it % NB, NB - 1 items in flight. Loads past the
  // wave's last item re-read the last item (never used): every load is unconditional, so the
  // compiler's count of outstanding memory operations stays exact and each wait is for the
  // one item it needs.
  f32x4 buf[NB][DEC_K];
  auto load_item = [&](int it, f32x4 (&dst)[DEC_K]) {
    const float* st = item_ptr(min(it, nitems - 1));
#pragma unroll
    for (int k = 0; k < DEC_K; ++k)
      dst[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + 4 * k * DEC_P));
  };
  // Start-up. The conv and dt inputs are requested first, then the first state parts: a wait
  // for a load also waits for every load issued before it, so the conv, which gates the
  // stream, must not queue behind the state. Each conv thread owns 4 channels.
  constexpr int CV = 4;
  const T* ub = u_t + (int64_t)b * NT * us;
  T* csb = conv_state + (int64_t)sb * (DEC_W - 1) * Cc;
  const int lc = tid * CV;
  const bool conv_thread = lc < nch;
  const int c = lc < nx ? h0w * DEC_P + lc
                        : (lc < nx + DEC_N ? di + g * DEC_N + (lc - nx) : di + G * DEC_N + g * DEC_N + (lc - nx - DEC_N));
  Raw4<T> e[NT + 3];                   // the extended sequence: 3 cached rows, then the tokens
  f32x4 wv[CV], bv = {0.f, 0.f, 0.f, 0.f};
  if (conv_thread) {
#pragma unroll
    for (int k = 0; k < 3; ++k) e[k] = ld4(csb + k * Cc + c);
#pragma unroll
    for (int t = 0; t < NT; ++t) e[3 + t] = ld4(ub + t * us + c);
#pragma unroll
    for (int i = 0; i < CV; ++i) wv[i] = *reinterpret_cast<const f32x4*>(w + (int64_t)(c + i) * DEC_W);
    if (bias) {
#pragma unroll
      for (int i = 0; i < CV; ++i) bv[i] = bias[c + i];
    }
  }
  float dtr[NT], dtb = 0.f, av = 0.f;
  const bool dt_thread = tid < hpp;
  if (dt_thread) {
    const int h = h0w + tid;
#pragma unroll
    for (int t = 0; t < NT; ++t) dtr[t] = to_f(dt_raw_t[((int64_t)b * NT + t) * dtrs + h]);
    dtb = dt_bias[h];
    av = A[h];
  }
  // STAGED: wave w takes parts sub * ipw .. sub * ipw + ipw - 1 of head jw (hpp divides 16)
  const int wph = STAGED ? NWAVES / hpp : 1, ipw = DEC_IPH / wph;
  const int jw = wave / wph, sub = wave % wph;
  const char* sbase = reinterpret_cast<const char*>(ssm_state + ((int64_t)sb * H + h0w + jw) * DEC_N * DEC_P);
  auto spart = [&](int m) {   // part m of head jw (clamped to the wave's last: never used)
    return const_cast<float*>(reinterpret_cast<const float*>(
        sbase + ((uint32_t)(sub * ipw + min(m, ipw - 1)) * 4 * DEC_P * 4u + lane_off)));
  };
  // the state does not depend on the conv: its first parts are in flight during the conv
  if constexpr (STAGED) {
#pragma unroll
    for (int k = 0; k < NB; ++k) buf[k][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(spart(k)));
  } else if (nitems > 0) {
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) load_item(k, buf[k]);
  }
  // conv steps on the owned channels; the cache shifts by NT tokens
  if (conv_thread) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < CV; ++i)
        smem[t * nch + lc + i] = conv4_silu(wv[i], bv[i], e[t].get(i), e[t + 1].get(i), e[t + 2].get(i),
                                            e[t + 3].get(i));
    if (SPLIT == 1 || lc < nx) {   // split launches: B and C columns after the arrival count
#pragma unroll
      for (int k = 0; k < 3; ++k) *reinterpret_cast<decltype(e[0].v)*>(csb + k * Cc + c) = e[NT + k].v;
    }
  }
  // groups wider than NTHREADS * CV channels: the rest, plainly
  for (int l2 = lc + NTHREADS * CV; l2 < nch; l2 += NTHREADS * CV) {
    const int c2 = l2 < nx ? h0w * DEC_P + l2
                           : (l2 < nx + DEC_N ? di + g * DEC_N + (l2 - nx) : di + G * DEC_N + g * DEC_N + (l2 - nx - DEC_N));
    Raw4<T> a[NT + 3];
#pragma unroll
    for (int k = 0; k < 3; ++k) a[k] = ld4(csb + k * Cc + c2);
#pragma unroll
    for (int t = 0; t < NT; ++t) a[3 + t] = ld4(ub + t * us + c2);
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const f32x4 wq = *reinterpret_cast<const f32x4*>(w + (int64_t)(c2 + i) * DEC_W);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        smem[t * nch + l2 + i] = conv4_silu(wq, bias ? bias[c2 + i] : 0.f, a[t].get(i), a[t + 1].get(i),
                                            a[t + 2].get(i), a[t + 3].get(i));
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) *reinterpret_cast<decltype(a[0].v)*>(csb + k * Cc + c2) = a[NT + k].v;
  }
  // dt and the decay per (token, head), one thread per head: the C ABI allows at most 256 heads
  // per group, fewer than the workgroup's threads
  if (dt_thread) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float dt = softplus_f(dtr[t] + dtb);
      dts[t * hpp + tid] = dt;
      das[t * hpp + tid] = expf(dt * av);
    }
  }
  __syncthreads();

  const T* zsrc = z_t ? z_t : u_t;     // without z a valid row is read and not used
  if constexpr (STAGED) {
    // update the wave's parts, store them, keep them in LDS for the head's y
    {
      const float a0 = das[jw];
      const f32x4 dx0 = dts[jw] * *reinterpret_cast<const f32x4*>(xs(0) + jw * DEC_P + 4 * q);
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (k < ipw) {
          const int m = sub * ipw + k;
          const int n0 = 4 * m + rg;
          const float bn = bsm(0)[n0];
          const f32x4 nv = __builtin_elementwise_fma((f32x4)a0, buf[k][0], bn * dx0);
          __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(spart(k)));
          stg[(jw * DEC_IPH + m) * 64 + lane] = nv;
        }
      }
    }
    __syncthreads();
    if (sub == 0) {
      const int h = h0w + jw;
      const Raw4<T> zz = ld4(zsrc + (int64_t)b * (z_t ? zs : us) + h * DEC_P + 4 * q);
      f32x4 yacc = (f32x4){0.f, 0.f, 0.f, 0.f};
      // the parts in the order of the one-wave stream: the same fma chain, the same bits
#pragma unroll 8
      for (int m = 0; m < DEC_IPH; ++m) {
        const float cn = csm(0)[4 * m + rg];
        yacc = __builtin_elementwise_fma((f32x4)cn, stg[(jw * DEC_IPH + m) * 64 + lane], yacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        yacc[i] += __shfl_xor(yacc[i], 16);
        yacc[i] += __shfl_xor(yacc[i], 32);
      }
      const float dh = D ? D[h] : 0.f;
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(xs(0) + jw * DEC_P + 4 * q);
      f32x4 o = yacc + dh * x4;
      if (z_t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= silu_fast(zz.get(i));
      }
      store4(y_t + (int64_t)b * di + h * DEC_P + 4 * q, o[0], o[1], o[2], o[3]);
    }
    return;
  }
  // stream the heads: per part, request part it + NB - 1, then update part it in place
  // (NT times, one token after the other)
  for (int hj = 0; hj < nheads_w; ++hj) {
    const int j = wave + NWAVES * hj;   // head of this workgroup
    const int h = h0w + j;
    float a[NT];
    f32x4 dx[NT], yacc[NT];
    Raw4<T> zz[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      a[t] = das[t * hpp + j];
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(xs(t) + j * DEC_P + 4 * q);
      dx[t] = dts[t * hpp + j] * x4;
      yacc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
      // the gate's z is requested now and used after the head's stream, so its latency is hidden
      zz[t] = ld4(zsrc + ((int64_t)b * NT + t) * (z_t ? zs : us) + h * DEC_P + 4 * q);
    }
    const float dh = D ? D[h] : 0.f;
#pragma unroll 1
    for (int m0 = 0; m0 < DEC_IPH; m0 += NB) {
#pragma unroll
    for (int mm = 0; mm < NB; ++mm) {
      const int m = m0 + mm;
      const int it = hj * DEC_IPH + m;
      load_item(it + NB - 1, buf[(mm + NB - 1) % NB]);
      // keep the request here: the scheduler would otherwise sink it below the update
      __builtin_amdgcn_sched_barrier(0);
      float* st = item_ptr(it);
      const int n0 = 4 * DEC_K * m + rg;
#pragma unroll
      for (int k = 0; k < DEC_K; ++k) {
        if constexpr (NT == 1) {
          // one token: the update on the loaded part itself. In the loop form below, with one
          // token, the compiler drops the store's non-temporal hint and the stream is ~10%
          // slower; the arithmetic is the same
          const f32x4 (&hv1)[DEC_K] = buf[mm];
          const float bn = bsm(0)[n0 + 4 * k], cn = csm(0)[n0 + 4 * k];
          const f32x4 nv = __builtin_elementwise_fma((f32x4)a[0], hv1[k], bn * dx[0]);
          yacc[0] = __builtin_elementwise_fma((f32x4)cn, nv, yacc[0]);
          __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(st + 4 * k * DEC_P));
          continue;
        }
        f32x4 hv = buf[mm][k];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float bn = bsm(t)[n0 + 4 * k], cn = csm(t)[n0 + 4 * k];
          // the same fma order as the one-token path, so T tokens give the bits of T calls
          const f32x4 nv = __builtin_elementwise_fma((f32x4)a[t], hv, bn * dx[t]);
          yacc[t] = __builtin_elementwise_fma((f32x4)cn, nv, yacc[t]);
          // stored from inside the loop: a store of the loop-carried value after it loses its
          // non-temporal hint in the compiler
          if (t == NT - 1) __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(st + 4 * k * DEC_P));
          hv = nv;
        }
      }
    }
    }
    // head done: per token, reduce y over the four row groups (every lane ends with the sum),
    // add the skip term, gate, store (the four row groups write the same values)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        yacc[t][i] += __shfl_xor(yacc[t][i], 16);
        yacc[t][i] += __shfl_xor(yacc[t][i], 32);
      }
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(xs(t) + j * DEC_P + 4 * q);
      f32x4 o = yacc[t] + dh * x4;
      if (z_t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= silu_fast(zz[t].get(i));
      }
      store4(y_t + ((int64_t)b * NT + t) * di + h * DEC_P + 4 * q, o[0], o[1], o[2], o[3]);
    }
  }
}

// The B and C columns of the conv cache after a split one-token launch: for sequence b
// (entry slots[b] of the pool, skipped when out of range), rows (1, 2, the new token) become
// rows (0, 1, 2). One thread per 16-byte vector of the 2 G N channels reads all three
// before it writes, and the launch before it on the stream has finished every read of the
// old rows, so nothing is overwritten before it is used.
template <typename T>
__global__ __launch_bounds__(256) void conv_shift_bc_kernel(const T* __restrict__ u_t, T* __restrict__ conv_state,
                                                            int B, int H, int G, const int32_t* __restrict__ slots,
                                                            int npool, int64_t us) {
  constexpr int VE = Vec<T>::VE;
  const int di = H * DEC_P, nbc = 2 * G * DEC_N, Cc = di + nbc;
  const int per_seq = nbc / VE;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B * per_seq) return;
  const int b = i / per_seq, c = di + (i % per_seq) * VE;
  int sb = b;
  if (slots) {
    sb = slots[b];
    if (sb < 0 || sb >= npool) return;
  }
  T* cs = conv_state + (int64_t)sb * (DEC_W - 1) * Cc + c;
  const Vec<T> r1 = ld16(cs + Cc), r2 = ld16(cs + 2 * Cc), u = ld16(u_t + (int64_t)b * us + c);
  st16(cs, r1);
  st16(cs + Cc, r2);
  st16(cs + 2 * Cc, u);
}

template <typename T, int NT, int NB = DEC_NB, int SPLIT = 1, bool STAGED = false, int WAVES = DEC_WAVES>
static hipError_t launch_nt(const DecodeArgs& a, hipStream_t stream) {
  const int hpp = a.H / a.G / SPLIT;
  size_t lds = sizeof(float) * ((size_t)NT * (hpp * DEC_P + 2 * DEC_N) + 2 * (size_t)NT * hpp);
  if (STAGED) lds = ((lds + 15) & ~(size_t)15) + (size_t)hpp * DEC_IPH * 64 * sizeof(f32x4);
  // the LDS limit is raised once per instance, and again only for a larger request
  static size_t lds_set = 64 * 1024;
  if (lds > lds_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&state_update_kernel<T, NT, NB, SPLIT, STAGED, WAVES>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set = lds;
  }
  hipLaunchKernelGGL((state_update_kernel<T, NT, NB, SPLIT, STAGED, WAVES>), dim3(a.B * a.G * SPLIT), dim3(WAVES * 64), lds, stream,
                     static_cast<const T*>(a.u_t), a.w, a.bias, static_cast<T*>(a.conv_state),
                     static_cast<const T*>(a.dt_raw_t), a.dt_bias, a.A, a.D,
                     static_cast<const T*>(a.z_t), a.ssm_state, static_cast<T*>(a.y_t), a.H, a.G, a.slots,
                     a.npool, a.u_stride > 0 ? a.u_stride : (int64_t)a.H * DEC_P + 2 * a.G * DEC_N,
                     a.z_stride > 0 ? a.z_stride : (int64_t)a.H * DEC_P, a.dt_stride > 0 ? a.dt_stride : a.H);
  if constexpr (SPLIT > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = a.B * 2 * a.G * DEC_N / Vec<T>::VE;
    hipLaunchKernelGGL((conv_shift_bc_kernel<T>), dim3((n + 255) / 256), dim3(256), 0, stream,
                       static_cast<const T*>(a.u_t), static_cast<T*>(a.conv_state), a.B, a.H, a.G, a.slots, a.npool,
                       a.u_stride > 0 ? a.u_stride : (int64_t)a.H * DEC_P + 2 * a.G * DEC_N);
  }
  return hipGetLastError();
}

static int num_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <typename T>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  switch (a.T) {
    case 1: {
      // few (sequence, group) pairs: split each pair's heads over 4 (or 2) workgroups, whose
      // waves keep 7 parts in flight, so that more CUs stream state. The split keeps to one
      // round of workgroups (one per CU at its register use): an 8-way split at 9B batch 8,
      // two rounds, took 32 us against 18 us. The B and C channels must stay inside the
      // single conv pass (at most 4096 channels).
      const int hpg = a.H / a.G, bg = a.B * a.G, cus = num_cus();
      if (hpg % 4 == 0 && hpg / 4 * DEC_P + 2 * DEC_N <= DEC_THREADS * 4 && bg * 4 <= cus) {
        if (hpg / 4 <= 4 && DEC_WAVES % (hpg / 4) == 0) return launch_nt<T, 1, 2 * DEC_NB, 4, true>(a, stream);
        return launch_nt<T, 1, 2 * DEC_NB, 4>(a, stream);
      }
      if (hpg % 2 == 0 && hpg / 2 * DEC_P + 2 * DEC_N <= DEC_THREADS * 4 && bg * 2 <= cus)
        return launch_nt<T, 1, 2 * DEC_NB, 2>(a, stream);
      return launch_nt<T, 1>(a, stream);
    }
    case 2: return launch_nt<T, 2, DEC_NB, 1, false, 8>(a, stream);
    case 3: return launch_nt<T, 3, DEC_NB, 1, false, 8>(a, stream);
    case 4: return launch_nt<T, 4, DEC_NB, 1, false, 8>(a, stream);
    case 5: return launch_nt<T, 5, DEC_NB, 1, false, 8>(a, stream);
    case 6: return launch_nt<T, 6, DEC_NB, 1, false, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_state_update(int io_bf16, const DecodeArgs& a, hipStream_t stream) {
  return io_bf16 ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace m2

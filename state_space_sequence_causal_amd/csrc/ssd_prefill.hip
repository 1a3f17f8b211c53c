// Chunked selective scan (SSD form) of the Mamba-2 layer core for gfx950.
//
// Computes, per sequence b and head h (group g = h / (H/G)), the recurrence
//   h_t = exp(dt_t A) h_{t-1} + dt_t B_t x_t^T,   y_t = h_t^T C_t + D x_t,  out = y SiLU(z)
// (Mamba-2 block of Nemotron-Nano-2: hyper.ai summary, section "方法"; fp32 state as
// the neurohive section "Развертывание" requires), chunk by chunk. Inside a chunk of
// Q tokens with l_t = sum_{r=c0..t} dt_r A (inclusive, relative to the chunk start):
//   y_t   = exp(l_t) C_t . H_prev                              (state carried in)
//         + sum_{s<=t} (C_t . B_s) exp(l_t - l_s) dt_s x_s      (causal quadratic form)
//         + D x_t,  gated by SiLU(z_t);
//   H_new = exp(l_end) H_prev + sum_s exp(l_end - l_s) dt_s B_s x_s^T.
//
// Design (one workgroup of 4 waves per (b, h), the fp32 state never leaves the chip):
//  * The state H (N x P = 128 x 64 fp32) lives in MFMA accumulators spread over the
//    waves; a copy H^T in LDS feeds the C.H product.
//  * Precision: x, B, C, z, dt enter the MFMAs exactly (they are bf16 inputs). The three
//    computed operands -- the masked decay matrix M, the state H and the decay-weighted
//    x -- are passed as hi + lo bf16 pairs (hi = bf16(v), lo = bf16(v - hi)), i.e. two
//    MFMAs each, which keeps them to ~2^-16 relative instead of bf16's 2^-8. With one
//    bf16 rounding the error of outputs dominated by a single term reaches 4e-2 to
//    2e-1 of rms(y), outside the 2e-2 bar; with the split it stays below 1e-4. The
//    fp32 io mode uses fp32 MFMAs and needs no split.
//  * Per chunk, B, C (Q x 128) and x (Q x 64) are staged in LDS with coalesced 16-byte
//    loads (prefetched one chunk ahead into registers); B and x are also stored
//    transposed so that contractions over tokens read contiguous K runs.
//  * dt and the inclusive log-decay l are built with a wavefront shuffle scan.
//  * Wave w owns token block w (32 tokens) of the chunk: G^T = B C^T tiles for the
//    source blocks s <= w (MFMA), masked and scaled in registers, then used directly
//    as the B operand of Y^T += X^T M^T (no LDS round trip), plus Y^T = H^T C^T for
//    the carried state. Waves with light token blocks take more state tiles
//    (H += (B^T) (w * X)), so the MFMA work per wave is balanced.
//  * The epilogue adds D x, gates with SiLU(z) and stores y with 8/16-byte stores.
//  * Blocks of the same group are dispatched to the same XCD so B and C chunks are
//    shared through one L2.
#include "device.h"
#include "launch.h"

namespace m2 {

constexpr int SP = 64;   // head dim
constexpr int SN = 128;  // state dim
constexpr int SSD_THREADS = 256;
constexpr int MAX_HT = 4;

template <typename T, int Q>
struct SsdCfg {
  static constexpr int VE = Vec<T>::VE;
  static constexpr int PAD = VE;                        // 16 bytes per LDS row
  static constexpr int LDN = SN + PAD;                  // rows with n contiguous
  static constexpr int LDQ = Q + PAD;                   // rows with tokens contiguous
  static constexpr int NTB = Q / 32;
  static constexpr int KS_N = SN / 16;
  static constexpr int KS_Q = Q / 16;
  static constexpr int VPR_N = SN / VE;
  static constexpr int VPR_P = SP / VE;
  static constexpr int NVB = Q * VPR_N / SSD_THREADS;
  static constexpr int NVX = Q * VPR_P / SSD_THREADS;
  static_assert(Q * VPR_N % SSD_THREADS == 0 && Q * VPR_P % SSD_THREADS == 0, "tiling");
  static_assert(Q <= 128, "one 32-token block per wave");
  static constexpr bool SPLIT = sizeof(T) == 2;         // hi/lo operands for bf16 io
};

template <typename T, int Q>
struct SsdSmem {
  using C = SsdCfg<T, Q>;
  T sB[Q][C::LDN];     // B rows (k = n)           : A operand of G^T
  T sC[Q][C::LDN];     // C rows (k = n)           : B operand of G^T and of Y_off
  T sBt[SN][C::LDQ];   // B^T (k = s)              : A operand of the state update
  T sXt[SP][C::LDQ];   // x^T (k = s)              : A operand of Y_diag, B operand of the update
  T sHt[SP][C::LDN];   // H^T of the carried state : A operand of Y_off (hi part)
  T sHtLo[C::SPLIT ? SP : 1][C::LDN];  // lo part of H^T (bf16 io only)
  float sL[Q];         // inclusive log-decay
  float sDt[Q];        // dt
  float sW[Q];         // exp(l_end - l_s) dt_s
  float sPart[Q];      // per-wave partial scans
};

// State tiles (32 x 32 of H[n][p]) each wave updates, balanced against the token-block
// work of wave w. At Q = 128 with split operands, in 32x32x16 MFMA units: token block w
// costs 16 (w+1) + 32 (G^T, Y_diag, Y_off) and a state tile 16, so waves get 4, 3, 1, 0
// tiles: 112, 112, 96, 96.
struct HTiles { int n; int nb[MAX_HT]; int pb[MAX_HT]; };
template <int Q> __device__ __forceinline__ HTiles htiles(int w);
template <> __device__ __forceinline__ HTiles htiles<128>(int w) {
  switch (w) {
    case 0: return {4, {0, 0, 1, 1}, {0, 1, 0, 1}};
    case 1: return {3, {2, 2, 3, 0}, {0, 1, 0, 0}};
    case 2: return {1, {3, 0, 0, 0}, {1, 0, 0, 0}};
    default: return {0, {0, 0, 0, 0}, {0, 0, 0, 0}};
  }
}
template <> __device__ __forceinline__ HTiles htiles<64>(int w) {
  switch (w) {
    case 2: return {4, {0, 0, 1, 1}, {0, 1, 0, 1}};
    case 3: return {4, {2, 2, 3, 3}, {0, 1, 0, 1}};
    default: return {0, {0, 0, 0, 0}, {0, 0, 0, 0}};
  }
}

template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  bf16x4 v;
  __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
};
template <> struct Raw4<float> {
  f32x4 v;
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <typename T> __device__ __forceinline__ Raw4<T> ld4(const T* p) {
  Raw4<T> r;
  r.v = *reinterpret_cast<const decltype(r.v)*>(p);
  return r;
}
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = (bf16x4){(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = (f32x4){a, b, c, d};
}

template <typename T, int Q>
__global__ __launch_bounds__(SSD_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ssd_prefill_kernel(const T* __restrict__ x, int64_t x_stride, const T* __restrict__ Bm,
                        int64_t b_stride, const T* __restrict__ Cm, int64_t c_stride,
                        const T* __restrict__ dt_raw, const float* __restrict__ dt_bias,
                        const float* __restrict__ A, const float* __restrict__ D,
                        const T* __restrict__ z, int64_t z_stride, const float* h0,
                        float* h_final, T* __restrict__ y, int64_t y_stride, int L, int H, int G) {
  using C = SsdCfg<T, Q>;
  constexpr int VE = C::VE;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SsdSmem<T, Q>& S = *reinterpret_cast<SsdSmem<T, Q>*>(smem_raw);

  const int id = xcd_local_order(blockIdx.x, gridDim.x);
  const int b = id / H, h = id % H;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g2 = lane >> 5;

  const int64_t row0 = (int64_t)b * L;
  const T* xb = x + h * SP;
  const T* Bb = Bm + g * SN;
  const T* Cb = Cm + g * SN;
  const float Ah = A[h], dtb = dt_bias[h], Dh = D ? D[h] : 0.f;
  const int nC = (L + Q - 1) / Q;

  // ---------------------------------------------------------------- prefetch registers
  Vec<T> rB[C::NVB], rC[C::NVB], rX[C::NVX];
  float rdt = 0.f;
  bool rdt_ok = false;
  auto load_chunk = [&](int c) {
    const int t0 = c * Q;
#pragma unroll
    for (int i = 0; i < C::NVB; ++i) {
      int v = tid + SSD_THREADS * i, s = v / C::VPR_N, cv = v % C::VPR_N;
      int t = t0 + s;
      if (t < L) {
        rB[i] = ld16(Bb + (row0 + t) * b_stride + cv * VE);
        rC[i] = ld16(Cb + (row0 + t) * c_stride + cv * VE);
      } else {
        rB[i] = zero16<T>();
        rC[i] = zero16<T>();
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVX; ++i) {
      int v = tid + SSD_THREADS * i, s = v / C::VPR_P, cv = v % C::VPR_P;
      int t = t0 + s;
      rX[i] = t < L ? ld16(xb + (row0 + t) * x_stride + cv * VE) : zero16<T>();
    }
    if (tid < Q) {
      int t = t0 + tid;
      rdt_ok = t < L;
      rdt = rdt_ok ? to_f(dt_raw[(row0 + t) * H + h]) : 0.f;
    }
  };

  // ---------------------------------------------------------------- state init
  const HTiles ht = htiles<Q>(wave);
  f32x16 hacc[MAX_HT];
  const int64_t sbase = ((int64_t)b * H + h) * SN * SP;
#pragma unroll
  for (int i = 0; i < MAX_HT; ++i) {
    if (i < ht.n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int n = ht.nb[i] * 32 + acc_row(r, lane), p = ht.pb[i] * 32 + col;
        hacc[i][r] = h0 ? h0[sbase + n * SP + p] : 0.f;
      }
    }
  }
  auto write_state_lds = [&]() {
#pragma unroll
    for (int i = 0; i < MAX_HT; ++i) {
      if (i < ht.n) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          int n = ht.nb[i] * 32 + 8 * r4 + 4 * g2, p = ht.pb[i] * 32 + col;
          float v[4], lo[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[k] = hacc[i][4 * r4 + k];
            lo[k] = v[k] - to_f(from_f<T>(v[k]));
          }
          st4(&S.sHt[p][n], v[0], v[1], v[2], v[3]);
          if constexpr (C::SPLIT) st4(&S.sHtLo[p][n], lo[0], lo[1], lo[2], lo[3]);
        }
      }
    }
  };

  if (nC > 0) load_chunk(0);
  write_state_lds();

  const int tb = wave < C::NTB ? wave : -1;  // token block owned by this wave

  for (int c = 0; c < nC; ++c) {
    const int t0 = c * Q;
    // ------------------------------------------------------------ stage chunk c
#pragma unroll
    for (int i = 0; i < C::NVB; ++i) {
      int v = tid + SSD_THREADS * i, s = v / C::VPR_N, cv = v % C::VPR_N;
      st16(&S.sB[s][cv * VE], rB[i]);
      st16(&S.sC[s][cv * VE], rC[i]);
#pragma unroll
      for (int e = 0; e < VE; ++e) S.sBt[cv * VE + e][s] = rB[i].v[e];
    }
#pragma unroll
    for (int i = 0; i < C::NVX; ++i) {
      int v = tid + SSD_THREADS * i, s = v / C::VPR_P, cv = v % C::VPR_P;
#pragma unroll
      for (int e = 0; e < VE; ++e) S.sXt[cv * VE + e][s] = rX[i].v[e];
    }
    if (tid < Q) {
      float dt = rdt_ok ? softplus_f(rdt + dtb) : 0.f;
      float run = dt * Ah;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        float o = __shfl_up(run, d);
        if (lane >= d) run += o;
      }
      S.sPart[tid] = run;
      S.sDt[tid] = dt;
    }
    if (c + 1 < nC) load_chunk(c + 1);
    __syncthreads();
    if (tid < Q) {
      float off = 0.f, tot = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < (Q + 63) / 64; ++w2) {
        float pw = S.sPart[min(64 * w2 + 63, Q - 1)];
        if (w2 < (tid >> 6)) off += pw;
        tot += pw;
      }
      float l = S.sPart[tid] + off;
      S.sL[tid] = l;
      S.sW[tid] = expf(tot - l) * S.sDt[tid];
    }
    __syncthreads();

    // ------------------------------------------------------------ token block: y
    if (tb >= 0) {
      const int tl = tb * 32 + col;  // lane's token within the chunk
      const int t = t0 + tl;
      const bool tvalid = t < L;
      // epilogue operands, fetched early (L2-resident: x was just staged)
      Raw4<T> xe[2][4], ze[2][4];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          int p0 = pb * 32 + 8 * r4 + 4 * g2;
          if (tvalid) {
            xe[pb][r4] = ld4(xb + (row0 + t) * x_stride + p0);
            if (z) ze[pb][r4] = ld4(z + (row0 + t) * z_stride + h * SP + p0);
          }
        }
      Frag<T> cf[C::KS_N];
#pragma unroll
      for (int j = 0; j < C::KS_N; ++j) cf[j] = frag_contig(&S.sC[tl][16 * j], g2);
      const float lt = S.sL[tl];

      f32x16 yacc[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        yacc[pb] = (f32x16){};
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j) {
          mma(yacc[pb], frag_contig(&S.sHt[pb * 32 + col][16 * j], g2), cf[j]);
          if constexpr (C::SPLIT) mma(yacc[pb], frag_contig(&S.sHtLo[pb * 32 + col][16 * j], g2), cf[j]);
        }
      }
      const float elt = expf(lt);
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r = 0; r < 16; ++r) yacc[pb][r] *= elt;

      for (int si = 0; si <= tb; ++si) {
        f32x16 gacc = (f32x16){};
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j)
          mma(gacc, frag_contig(&S.sB[si * 32 + col][16 * j], g2), cf[j]);
        Frag<T> mf[2], mlo[2];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int s0 = si * 32 + 8 * r4 + 4 * g2;
          const f32x4 ls = *reinterpret_cast<const f32x4*>(&S.sL[s0]);
          const f32x4 ds = *reinterpret_cast<const f32x4*>(&S.sDt[s0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * r4 + i;
            float v = (s0 + i <= tl) ? gacc[r] * expf(lt - ls[i]) * ds[i] : 0.f;
            frag_set<T>(mf[r >> 3], r & 7, v);
            if constexpr (C::SPLIT) frag_set<T>(mlo[r >> 3], r & 7, v - frag_get(mf[r >> 3], r & 7));
          }
        }
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
          for (int pb = 0; pb < 2; ++pb) {
            Frag<T> xa = frag_accrows(&S.sXt[pb * 32 + col][si * 32 + 16 * m2], g2);
            mma(yacc[pb], xa, mf[m2]);
            if constexpr (C::SPLIT) mma(yacc[pb], xa, mlo[m2]);
          }
      }

      if (tvalid) {
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            int p0 = pb * 32 + 8 * r4 + 4 * g2;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float v = yacc[pb][4 * r4 + i] + Dh * xe[pb][r4].get(i);
              if (z) v *= silu_f(ze[pb][r4].get(i));
              o[i] = v;
            }
            st4(y + (row0 + t) * y_stride + h * SP + p0, o[0], o[1], o[2], o[3]);
          }
      }
    }

    // ------------------------------------------------------------ state update
    if (ht.n > 0) {
      const float eend = expf(S.sL[Q - 1]);
#pragma unroll
      for (int i = 0; i < MAX_HT; ++i)
        if (i < ht.n)
#pragma unroll
          for (int r = 0; r < 16; ++r) hacc[i][r] *= eend;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        bool any = false;
#pragma unroll
        for (int i = 0; i < MAX_HT; ++i) any |= (i < ht.n && ht.pb[i] == pb);
        if (!any) continue;
#pragma unroll 2
        for (int j = 0; j < C::KS_Q; ++j) {
          Frag<T> xw = frag_contig(&S.sXt[pb * 32 + col][16 * j], g2), xlo;
          const f32x4 w0 = *reinterpret_cast<const f32x4*>(&S.sW[16 * j + 8 * g2]);
          const f32x4 w1 = *reinterpret_cast<const f32x4*>(&S.sW[16 * j + 8 * g2 + 4]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float v = frag_get(xw, e) * (e < 4 ? w0[e] : w1[e - 4]);
            frag_set<T>(xw, e, v);
            if constexpr (C::SPLIT) frag_set<T>(xlo, e, v - frag_get(xw, e));
          }
#pragma unroll
          for (int i = 0; i < MAX_HT; ++i)
            if (i < ht.n && ht.pb[i] == pb) {
              Frag<T> ba = frag_contig(&S.sBt[ht.nb[i] * 32 + col][16 * j], g2);
              mma(hacc[i], ba, xw);
              if constexpr (C::SPLIT) mma(hacc[i], ba, xlo);
            }
        }
      }
    }
    __syncthreads();
    write_state_lds();
  }

  if (h_final) {
#pragma unroll
    for (int i = 0; i < MAX_HT; ++i) {
      if (i < ht.n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int n = ht.nb[i] * 32 + acc_row(r, lane), p = ht.pb[i] * 32 + col;
          h_final[sbase + n * SP + p] = hacc[i][r];
        }
      }
    }
  }
}

template <typename T, int Q>
static hipError_t launch_tq(const PrefillArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(SsdSmem<T, Q>);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_prefill_kernel<T, Q>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL((ssd_prefill_kernel<T, Q>), dim3(a.B * a.H), dim3(SSD_THREADS), lds, stream,
                     static_cast<const T*>(a.x), a.x_stride, static_cast<const T*>(a.Bm),
                     a.b_stride, static_cast<const T*>(a.Cm), a.c_stride,
                     static_cast<const T*>(a.dt_raw), a.dt_bias, a.A, a.D,
                     static_cast<const T*>(a.z), a.z_stride, a.h0, a.h_final,
                     static_cast<T*>(a.y), a.y_stride, a.L, a.H, a.G);
  return hipGetLastError();
}

size_t ssd_prefill_lds_bytes(int io_bf16, int chunk) {
  if (io_bf16) return chunk == 128 ? sizeof(SsdSmem<bf16, 128>) : sizeof(SsdSmem<bf16, 64>);
  return sizeof(SsdSmem<float, 64>);
}

hipError_t launch_ssd_prefill(int io_bf16, int chunk, const PrefillArgs& a, hipStream_t stream) {
  if (io_bf16) {
    if (chunk == 128) return launch_tq<bf16, 128>(a, stream);
    if (chunk == 64) return launch_tq<bf16, 64>(a, stream);
  } else if (chunk == 64) {
    return launch_tq<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace m2

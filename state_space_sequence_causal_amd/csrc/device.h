// Device helpers for the gfx950 kernels: io element types, 16-byte vectors,
// MFMA fragments and small math. Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }  // RNE

// ---------------------------------------------------------------- 16-byte io vectors
// VE elements of T in 16 bytes.
template <typename T> struct Vec;
template <> struct Vec<bf16> {
  static constexpr int VE = 8;
  bf16x8 v;
  __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
  __device__ __forceinline__ void set(int i, float f) { v[i] = (bf16)f; }
};
template <> struct Vec<float> {
  static constexpr int VE = 4;
  f32x4 v;
  __device__ __forceinline__ float get(int i) const { return v[i]; }
  __device__ __forceinline__ void set(int i, float f) { v[i] = f; }
};

template <typename T> __device__ __forceinline__ Vec<T> ld16(const T* p) {
  Vec<T> r;
  r.v = *reinterpret_cast<const decltype(r.v)*>(p);
  return r;
}
template <typename T> __device__ __forceinline__ void st16(T* p, const Vec<T>& r) {
  *reinterpret_cast<decltype(r.v)*>(p) = r.v;
}
template <typename T> __device__ __forceinline__ Vec<T> zero16() {
  Vec<T> r;
  for (int i = 0; i < Vec<T>::VE; ++i) r.v[i] = from_f<T>(0.f);
  return r;
}

// 4 io elements (8 or 16 bytes)
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  bf16x4 v;
  __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
};
template <> struct Raw4<float> {
  f32x4 v;
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};
// Accesses at a 32-bit byte offset from a base every lane of the wave shares: the compiler
// can then use the scalar-base, 32-bit-offset form and needs no 64-bit address arithmetic.
template <typename V> __device__ __forceinline__ V ld_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename V> __device__ __forceinline__ void st_at(void* base, uint32_t byte_off, const V& v) {
  *reinterpret_cast<V*>(reinterpret_cast<char*>(base) + byte_off) = v;
}
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

// two consecutive io elements as one 32-bit (bf16) or 64-bit (f32) store
__device__ __forceinline__ void st_pair(bf16* p, bf16 a, bf16 b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<bf16x2*>(p) = (bf16x2){a, b};
}
__device__ __forceinline__ void st_pair(float* p, float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<f32x2*>(p) = (f32x2){a, b};
}

// ---------------------------------------------------------------- math
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
__device__ __forceinline__ float softplus_f(float v) { return v > 20.f ? v : log1pf(expf(v)); }
// softplus from the hardware exponential, logarithm and reciprocal (a few ulp, against the
// libm form above): max(v, 0) + log1p(e) with e = exp(-|v|) <= 1, and log1p(e) = e where
// u = 1 + e rounds to 1, else log(u) e / (u - 1), whose quotient cancels the rounding of u
// (Goldberg, "What every computer scientist should know about floating-point arithmetic",
// the log1p example). Above 20 it is v, as softplus_f.
__device__ __forceinline__ float softplus_hw(float v) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.f + e;
  const float l = u == 1.f ? e : __builtin_amdgcn_logf(u) * kLn2 * (e * __builtin_amdgcn_rcpf(u - 1.f));
  return v > 20.f ? v : fmaxf(v, 0.f) + l;
}
// fp64 row moves across lanes (DPP, both 32-bit halves; lanes without a source and rows
// outside ROWS read 0)
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xf, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xf, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Inclusive fp64 sum over each 32-lane half of the wave: doubling shifts inside rows of 16
// lanes (row_shr 1, 2, 4, 8), then the total of row 0 (row 2) added to row 1 (row 3)
// (row_bcast:15 into rows 1 and 3).
__device__ __forceinline__ double scan32_f64(double v) {
  v += dpp_f64<0x111, 0xf>(v);
  v += dpp_f64<0x112, 0xf>(v);
  v += dpp_f64<0x114, 0xf>(v);
  v += dpp_f64<0x118, 0xf>(v);
  v += dpp_f64<0x142, 0xa>(v);
  return v;
}
// lane 31's value in lanes 0..31, lane 63's in lanes 32..63
__device__ __forceinline__ double half_last_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int src = lane < 32 ? 31 : 63;
  const uint32_t lo31 = __builtin_amdgcn_readlane((int)(uint32_t)b, 31), lo63 = __builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi31 = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 31),
                 hi63 = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __builtin_bit_cast(double, src == 31 ? ((uint64_t)hi31 << 32) | lo31 : ((uint64_t)hi63 << 32) | lo63);
}
__device__ __forceinline__ float silu_f(float v) { return v / (1.f + expf(-v)); }
// 2^v with the hardware exponential (v_exp_f32, about 1 ulp); used for decay factors,
// whose arguments are <= 0.
__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
// z * sigmoid(z) from the hardware exponential and reciprocal (each about 1 ulp); for
// z -> -inf the exponential overflows to inf and the result is -0.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e));
}
// One conv output: bias + w[0] u[t-3] + w[1] u[t-2] + w[2] u[t-1] + w[3] u[t] in one fixed
// fma order, then SiLU. Every conv of the library (the conv call, the conv fused into the
// prefill, the decode step) goes through it, so equal inputs give equal values in all three.
__device__ __forceinline__ float conv4_silu(const f32x4& w, float bias, float e0, float e1, float e2,
                                            float e3) {
  return silu_fast(fmaf(w[3], e3, fmaf(w[2], e2, fmaf(w[1], e1, fmaf(w[0], e0, bias)))));
}

// ---------------------------------------------------------------- MFMA 32x32, K in steps of 16
// An operand fragment holds, per lane, 8 values along K for one row (A) or one
// column (B) of a 32-wide tile: lane l covers row/col l % 32 and lane group
// g = l / 32 holds the 8 K-indices kappa(g, e), e = 0..7, of the 16-wide K step.
// Any kappa works as long as A and B use the same one.
// Accumulator (16 fp32 per lane): element r of lane l is D[row][col] with
//   col = l % 32,  row = 8 * (r / 4) + 4 * (l / 32) + (r % 4).
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ void mma(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Fragment with contiguous kappa(g, e) = 8 g + e: p points at K-index 0 of the step;
// 16-byte aligned.
__device__ __forceinline__ Frag<bf16> frag_contig(const bf16* p, int g) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p + 8 * g);
  return f;
}
__device__ __forceinline__ Frag<float> frag_contig(const float* p, int g) {
  Frag<float> f;
  f32x4 a = *reinterpret_cast<const f32x4*>(p + 8 * g);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 8 * g + 4);
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
// Fragment with the accumulator-row kappa(g, e) = 8 (e / 4) + 4 g + (e % 4), which lets
// accumulator registers 8m..8m+7 serve directly as the B operand of K rows 16m..16m+15.
__device__ __forceinline__ Frag<bf16> frag_accrows(const bf16* p, int g) {
  Frag<bf16> f;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p + 4 * g);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 8 + 4 * g);
  f.v = (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
__device__ __forceinline__ Frag<float> frag_accrows(const float* p, int g) {
  Frag<float> f;
  f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 8 + 4 * g);
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}

// frag_accrows with the two 4-element runs at independent (8- or 16-byte aligned) places
__device__ __forceinline__ Frag<bf16> frag_accrows2(const bf16* a, const bf16* b) {
  Frag<bf16> f;
  bf16x4 u = *reinterpret_cast<const bf16x4*>(a);
  bf16x4 v = *reinterpret_cast<const bf16x4*>(b);
  f.v = (bf16x8){u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
  return f;
}
__device__ __forceinline__ Frag<float> frag_accrows2(const float* a, const float* b) {
  Frag<float> f;
  f32x4 u = *reinterpret_cast<const f32x4*>(a);
  f32x4 v = *reinterpret_cast<const f32x4*>(b);
  f.v = (f32x8){u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
  return f;
}

// ---------------------------------------------------------------- hi + lo splits
// A computed fp32 operand v enters a bf16 MFMA as two bf16 values, hi = bf16(v) (RNE) and
// lo = bf16(v - hi), which together hold v to about 2^-16. For a pair of values this costs
// one pair conversion, two exact unpacks, two subtractions and a second pair conversion.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
struct Split2 {
  uint32_t hi, lo;  // packed bf16 pairs, first value in the low half
};
__device__ __forceinline__ Split2 split2(float a, float b) {
  const uint32_t h = pack_bf16(a, b);
  const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xffff0000u);
  return {h, pack_bf16(a - ha, b - hb)};
}
// 8 values into hi and lo operand fragments (element e of the fragment is v[e])
__device__ __forceinline__ void frag_split(const float* v, Frag<bf16>& hi, Frag<bf16>& lo) {
  u32x4 h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const Split2 s = split2(v[2 * k], v[2 * k + 1]);
    h[k] = s.hi;
    l[k] = s.lo;
  }
  hi.v = __builtin_bit_cast(bf16x8, h);
  lo.v = __builtin_bit_cast(bf16x8, l);
}

template <typename T> __device__ __forceinline__ Frag<T> frag_zero() {
  Frag<T> f;
  for (int e = 0; e < 8; ++e) f.v[e] = from_f<T>(0.f);
  return f;
}

template <typename T> __device__ __forceinline__ void frag_set(Frag<T>& f, int e, float v);
template <> __device__ __forceinline__ void frag_set<bf16>(Frag<bf16>& f, int e, float v) { f.v[e] = (bf16)v; }
template <> __device__ __forceinline__ void frag_set<float>(Frag<float>& f, int e, float v) { f.v[e] = v; }
__device__ __forceinline__ float frag_get(const Frag<bf16>& f, int e) { return (float)f.v[e]; }
__device__ __forceinline__ float frag_get(const Frag<float>& f, int e) { return f.v[e]; }

// Blocks are dispatched round-robin over the chip's 8 XCDs (each with its own L2).
// Map dispatch order to a logical order in which consecutive logical ids share an XCD.
__device__ __forceinline__ int xcd_local_order(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

}  // namespace m2

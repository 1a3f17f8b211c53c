// Chunked selective scan (SSD form) of the Mamba-2 layer core for gfx950.
//
// Computes, per sequence b and head h (group g = h / (H/G)), the recurrence
//   h_t = exp(dt_t A) h_{t-1} + dt_t B_t x_t^T,   y_t = h_t^T C_t + D x_t,  out = y SiLU(z)
// (Mamba-2 block of Nemotron-Nano-2: hyper.ai summary, section "方法"; fp32 state as the
// neurohive section "Развертывание" requires), chunk by chunk. Inside a chunk of Q
// tokens, with l_t = sum_{r=c0..t} dt_r A:
//   y_t   = exp(l_t) C_t . H_prev                              (state carried in)
//         + sum_{s<=t} (C_t . B_s) exp(l_t - l_s) dt_s x_s      (causal quadratic form)
//         + D x_t,  gated by SiLU(z_t);
//   H_new = exp(l_end) H_prev + sum_s exp(l_end - l_s) dt_s B_s x_s^T.
//
// Two kernels:
//  * ssd_prep, one workgroup per (sequence, group, chunk). For the group it writes the
//    Gram tiles G^T[s][t] = B_s . C_t of the causal lower triangle in fp32 (MFMA, exact
//    products of the bf16 inputs) in MFMA accumulator order, and B^T and C in MFMA operand
//    order, so that each wave later reads every operand as 1 KiB contiguous per
//    instruction; these are shared by all heads of the group. For each head of the group
//    it writes dt = softplus(dt_raw + dt_bias), the inclusive prefix pi of dt*A*log2(e)
//    inside 32-token blocks, and v_s = exp2(pi_end - pi_s) dt_s (decay from token s to the
//    end of its block, times dt_s).
//  * ssd_scan, one workgroup of 8 waves per (b, h). The fp32 state stays on chip for the
//    whole sequence. Waves 0-3 ("Y waves") own 32-token blocks of the chunk: they build
//    the masked decay matrix M from the Gram tiles and compute Y^T = X^T M^T + H^T C^T
//    and the gated epilogue. Waves 4-7 ("H waves") own 32x32 tiles of the state and run
//    H = exp(l_end) H + B^T (w x). Each SIMD hosts one wave of each kind; the state tiles
//    are dealt so that the MFMA work per SIMD is balanced. Per chunk: stage (x, z, decay
//    vectors) | barrier | compute | barrier | publish the new state.
//
// Decay factors are formed in log2 units from prefix sums taken inside 32-token blocks, so
// no factor is the difference of two large prefix sums: inside a block exp2(pi_t - pi_s);
// across blocks the factor splits into a per-row part F[s] and a per-column part U[t],
// both <= 1, so off-diagonal tiles need no exponentials. D is added to the diagonal of M,
// so the skip term D x_t comes out of the same MFMAs.
//
// Precision: x, B, C, z and dt enter exactly (bf16 inputs). The three computed MFMA
// operands -- M, the state H and the decay-weighted x -- are passed as hi + lo bf16 pairs
// (hi = bf16(v), lo = bf16(v - hi)), i.e. two MFMAs each, which keeps them to ~2^-16
// relative. With a single bf16 rounding the error of outputs dominated by one term reaches
// 4e-2 to 2e-1 of rms(y) on these heavy-tailed outputs, outside the 2e-2 bar; with the
// split it stays below 1e-4. The fp32 io mode uses fp32 MFMAs and needs no split.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace m2 {

constexpr int SP = 64;   // head dim
constexpr int SN = 128;  // state dim
constexpr int PREP_THREADS = 256;
constexpr int SCAN_THREADS = 512;

template <typename T, int Q>
struct Cfg {
  static constexpr int VE = Vec<T>::VE;        // elements per 16 bytes
  static constexpr bool SPLIT = sizeof(T) == 2;
  static constexpr int NTB = Q / 32;           // 32-token blocks per chunk
  static constexpr int NTILES = NTB * (NTB + 1) / 2;
  static constexpr int KS_N = SN / 16;
  static constexpr int KS_Q = Q / 16;
  static constexpr int PAD = VE;
  static constexpr int LDN = SN + PAD;         // LDS rows with n contiguous
  static constexpr int LDQ = Q + PAD;          // LDS rows with tokens contiguous
  static constexpr size_t FB = sizeof(Frag<T>);
  // workspace record per (b, g, chunk): Gram tiles | B^T operand frags | C operand frags
  static constexpr size_t G_BYTES = (size_t)NTILES * 64 * 16 * sizeof(float);
  static constexpr size_t BT_BYTES = (size_t)(SN / 32) * KS_Q * 64 * FB;
  static constexpr size_t CF_BYTES = (size_t)NTB * KS_N * 64 * FB;
  static constexpr size_t REC_BYTES = G_BYTES + BT_BYTES + CF_BYTES;
  // workspace record per (b, h, chunk): dt[Q] | pi[Q] | v[Q]
  static constexpr size_t HREC_BYTES = 3 * Q * sizeof(float);
  static constexpr int XV = Q * SP / VE / SCAN_THREADS;     // 16-byte x vectors per thread
  static constexpr bool PAIRS = XV % 2 == 0;                // two tokens per transposed write
  static constexpr int TPL = Q / 64;                        // decay tokens per lane (lane + 64 k)
  static constexpr int NBD = Q == 128 ? 2 : 1;              // distinct state row blocks per H wave
  static constexpr bool STAGE_Z = Q <= 128;                 // z / y through LDS (LDS budget)
  static_assert(Q * SP % (VE * SCAN_THREADS) == 0, "x staging");
};

// Token position of (row p, token s) in the transposed LDS tiles x^T and (w x)^T. The
// staging writes of a wave cover 8 rows p = 8 cv + e (cv = 0..7) with 8 consecutive token
// pairs each; XOR-ing the token index with 16 (cv mod 8) puts the 8 rows on distinct
// banks. Readers only touch aligned runs of 4 or 8 tokens, which the XOR keeps intact.
template <int Q>
__device__ __forceinline__ int xsw(int p, int s) {
  constexpr int MASK = Q >= 128 ? 7 : Q / 16 - 1;
  return s ^ (16 * ((p >> 3) & MASK));
}

__device__ __forceinline__ int tile_tb(int k) {  // column block of lower-triangle tile k < 36
  int tb = 0;
#pragma unroll
  for (int t = 1; t < 8; ++t) tb += k >= t * (t + 1) / 2;
  return tb;
}

// frag_accrows on a swizzled row: the two 4-token runs are looked up separately.
template <int Q, typename T>
__device__ __forceinline__ Frag<T> frag_accrows_sw(const T* row, int p, int k0, int g) {
  Frag<T> f;
  const int a = xsw<Q>(p, k0 + 4 * g), b = xsw<Q>(p, k0 + 8 + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = row[a + e];
    f.v[4 + e] = row[b + e];
  }
  return f;
}

template <typename T>
__device__ __forceinline__ void st_frag(void* p, const Frag<T>& f) {
  *reinterpret_cast<decltype(f.v)*>(p) = f.v;
}
template <typename T>
__device__ __forceinline__ Frag<T> ld_frag(const void* p) {
  Frag<T> f;
  f.v = *reinterpret_cast<const decltype(f.v)*>(p);
  return f;
}

// Device view of a packed variable-length batch: sanitized row offsets cu[nseq + 1], the
// first global chunk of each sequence cc[nseq + 1] and, per global chunk, info = {first packed
// row, valid rows | 256 if the sequence starts there | 512 if it starts from its entry's state,
// sequence, the sequence's pool entry or -1} (all three in the workspace), and, also in the
// workspace, the x-channel conv history of each sequence at its first chunk (written by the
// prep kernel, read by the scan at a fixed place per chunk),
// the slot map and the initial-state flags, the pools, the chunk capacity of the workspace
// records, and the number of scan workgroups per head (each walks a range of sequences).
struct VarlenDev {
  const int32_t* cu; const int32_t* cc; const int4* info;
  const int32_t* slots; const int32_t* has_init;
  float* ssm_pool; bf16* conv_pool;
  bf16* hist;   // [chunk][3][H * P]: at a sequence's first chunk, the x-channel conv history
  int nseq, npool, maxC, K;
  // pool entry of sequence i, or -1 when it has none (slot out of range)
  __device__ __forceinline__ int slot(int i) const {
    const int s = slots ? slots[i] : i;
    return s >= 0 && s < npool ? s : -1;
  }
  __device__ __forceinline__ bool init(int i) const { return has_init && has_init[i] != 0; }
};

// Offsets of a packed batch, made safe to index with: cu'[i] = min(max(0, cu[0..i]), total),
// so every sequence lies inside the packed rows whatever the caller passed, and the first
// global chunk of each sequence, cc[i] = sum over j < i of ceil((cu'[j+1] - cu'[j]) / 64).
// One workgroup; thread t takes a contiguous run of the nseq + 1 entries.
constexpr int VIDX_THREADS = 1024;
constexpr int INFO_FIRST = 256, INFO_INIT = 512;
__global__ __launch_bounds__(VIDX_THREADS) void varlen_index_kernel(const int32_t* __restrict__ cu_in, int nseq,
                                                                    int total, int32_t* __restrict__ cu_out,
                                                                    int32_t* __restrict__ cc_out,
                                                                    int4* __restrict__ info,
                                                                    const int32_t* __restrict__ slots,
                                                                    const int32_t* __restrict__ has_init,
                                                                    int npool) {
  __shared__ int part[VIDX_THREADS];
  const int t = threadIdx.x, n = nseq + 1;
  const int per = (n + VIDX_THREADS - 1) / VIDX_THREADS;
  const int j0 = min(n, t * per), j1 = min(n, j0 + per);
  // running maximum of the clamped offsets
  int m = 0;
  for (int j = j0; j < j1; ++j) m = max(m, min(max(cu_in[j], 0), total));
  part[t] = m;
  __syncthreads();
  for (int d = 1; d < VIDX_THREADS; d <<= 1) {   // inclusive max scan
    const int o = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] = max(part[t], o);
    __syncthreads();
  }
  m = t > 0 ? part[t - 1] : 0;
  for (int j = j0; j < j1; ++j) {
    m = max(m, min(max(cu_in[j], 0), total));
    cu_out[j] = m;
  }
  __syncthreads();
  // chunk counts and their exclusive sum
  int sum = 0;
  for (int j = j0; j < min(j1, nseq); ++j) sum += (cu_out[j + 1] - cu_out[j] + 63) / 64;
  part[t] = sum;
  __syncthreads();
  for (int d = 1; d < VIDX_THREADS; d <<= 1) {   // inclusive sum scan
    const int o = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += o;
    __syncthreads();
  }
  int run = t > 0 ? part[t - 1] : 0;
  for (int j = j0; j < j1; ++j) {
    cc_out[j] = run;
    if (j < nseq) {
      const int len = cu_out[j + 1] - cu_out[j];
      int sl = slots ? slots[j] : j;
      if (sl < 0 || sl >= npool) sl = -1;
      const int init = sl >= 0 && has_init && has_init[j] != 0 ? INFO_INIT : 0;
      for (int k = 0; k < (len + 63) / 64; ++k)
        info[run + k] = make_int4(cu_out[j] + 64 * k, min(64, len - 64 * k) | (k == 0 ? INFO_FIRST : 0) | init, j, sl);
      run += (len + 63) / 64;
    }
  }
}

// ---------------------------------------------------------------------------- prep kernel
// With CONV, Bm and Cm are the raw xBC columns and the conv (with its 3-token history at the
// sequence start) is applied while the chunk's rows are staged. With VARLEN (CONV only) the
// grid is (group, global chunk) over a packed batch; records are laid out [group][chunk].
template <typename T, int Q, bool CONV, bool VARLEN = false>
__global__ __launch_bounds__(PREP_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void ssd_prep_kernel(
    const T* __restrict__ Bm, int64_t b_stride, const T* __restrict__ Cm, int64_t c_stride,
    const T* __restrict__ dt_raw, const float* __restrict__ dt_bias, const float* __restrict__ A,
    int64_t dt_stride, unsigned char* __restrict__ ws, int L, int H, int G, int nC, ConvArgs cv, VarlenDev vd) {
  static_assert(!VARLEN || CONV, "the packed batch runs with the conv fused");
  using C = Cfg<T, Q>;
  constexpr int VE = C::VE;
  extern __shared__ __align__(16) unsigned char prep_smem[];
  T (*sB)[C::LDN] = reinterpret_cast<T (*)[C::LDN]>(prep_smem);
  T (*sC)[C::LDN] = reinterpret_cast<T (*)[C::LDN]>(prep_smem + sizeof(T) * Q * C::LDN);

  const int rec = blockIdx.x;
  // c: the chunk's record index; t0: its first token inside its sequence
  int c, g, b, t0, len;
  int64_t row0;
  const T* hist0 = nullptr;   // conv history of the chunk's sequence, or none
  if constexpr (VARLEN) {
    g = rec / vd.maxC;
    c = rec % vd.maxC;
    b = 0;
    if (c >= vd.cc[vd.nseq]) return;   // past the batch's chunks: the whole workgroup leaves
    const int4 ci = vd.info[c];
    t0 = ci.x - vd.cu[ci.z];
    len = t0 + (ci.y & 255);           // rows of the sequence up to the chunk's end
    row0 = ci.x;
    if (ci.y & INFO_INIT) hist0 = reinterpret_cast<const T*>(vd.conv_pool) + (int64_t)ci.w * 3 * cv.Cc;
    nC = vd.maxC;
  } else {
    c = rec % nC;
    const int bg = rec / nC;
    g = bg % G;
    b = bg / G;
    t0 = c * Q;
    len = L;
    row0 = (int64_t)b * L + t0;
    if (CONV && cv.state) hist0 = static_cast<const T*>(cv.state) + (int64_t)b * 3 * cv.Cc;
  }
  const T* Bb = Bm + row0 * b_stride + g * SN;
  const T* Cb = Cm + row0 * c_stride + g * SN;
  unsigned char* recp = ws + (size_t)rec * C::REC_BYTES;
  float* gout = reinterpret_cast<float*>(recp);
  unsigned char* btf = recp + C::G_BYTES;
  unsigned char* cff = btf + C::BT_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g2 = lane >> 5;
  const int nvalid = min(Q, len - t0);

  // The B and C rows are requested first; the dt records are formed while they arrive, and
  // then the rows go to LDS (zero past the end of the sequence).
  constexpr int NR = CONV ? 11 : Q * SN / VE / PREP_THREADS;   // 16-byte row vectors per thread
  constexpr bool HOLD = CONV;   // rows held in registers across the dt phase
  Vec<T> rB[HOLD ? NR : 1], rC[CONV || !HOLD ? 1 : NR];
  // CONV: a thread convolves one 16-byte vector of B (vectors 0..15) or C (16..31) over 8
  // consecutive tokens s1 .. s1 + 7, from the 11 raw rows s1 - 3 .. s1 + 7 (chunk-relative;
  // before the sequence start: the history, zeros without one; past the end: the last row,
  // whose outputs are dropped)
  const int vec = tid & 31, s1 = 8 * (tid >> 5);
  const int n0 = (vec & 15) * VE;
  [[maybe_unused]] const bool isC = vec >= 16;
  [[maybe_unused]] const int ch = H * SP + (isC ? G * SN : 0) + g * SN + n0;   // xBC channel
  if constexpr (CONV) {
    static_assert(Q == 64 && SN / VE == 16 && PREP_THREADS == 256, "conv staging layout");
    const T* src = (isC ? Cb : Bb) + n0;
    const int64_t stride = isC ? c_stride : b_stride;
    const T* hist = hist0 ? hist0 + ch : nullptr;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int s = min(s1 - 3 + k, nvalid - 1);
      if (t0 + s < 0) rB[k] = hist ? ld16(hist + (int64_t)(t0 + s + 3) * cv.Cc) : zero16<T>();
      else rB[k] = ld16(src + (int64_t)s * stride);
    }
  } else if constexpr (HOLD) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int v = tid + i * PREP_THREADS;
      const int s = min(v / (SN / VE), nvalid - 1), e0 = v % (SN / VE) * VE;
      rB[i] = ld16(Bb + (int64_t)s * b_stride + e0);
      rC[i] = ld16(Cb + (int64_t)s * c_stride + e0);
    }
  } else {
    for (int v = tid; v < Q * SN / VE; v += PREP_THREADS) {
      const int s = v / (SN / VE), e0 = v % (SN / VE) * VE;
      const bool ok = s < nvalid;
      st16(&sB[s][e0], ok ? ld16(Bb + (int64_t)s * b_stride + e0) : zero16<T>());
      st16(&sC[s][e0], ok ? ld16(Cb + (int64_t)s * c_stride + e0) : zero16<T>());
    }
  }
  // per head of the group: dt and the 32-token block prefix of dt*A*log2(e); a wave takes
  // items wave, wave + 4, ... and requests up to 8 of them at once
  {
    const int hpg = H / G, nitems = hpg * C::TPL;
    const size_t hrec0 = (size_t)b * H * nC;
    unsigned char* hbase = ws + (size_t)gridDim.x * C::REC_BYTES;
    constexpr int DB = 8;
    for (int i0 = wave; i0 < nitems; i0 += DB * (PREP_THREADS / 64)) {
      float raw[DB];
#pragma unroll
      for (int u = 0; u < DB; ++u) {
        const int item = i0 + u * (PREP_THREADS / 64);
        const int j = item / C::TPL, s = 64 * (item % C::TPL) + lane;
        raw[u] = item < nitems && s < nvalid ? to_f(dt_raw[(row0 + s) * dt_stride + g * hpg + j]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < DB; ++u) {
        const int item = i0 + u * (PREP_THREADS / 64);
        if (item >= nitems) break;
        const int j = item / C::TPL, k = item % C::TPL;
        const int h = g * hpg + j;
        const int s = 64 * k + lane;
        const float dt = s < nvalid ? softplus_f(raw[u] + dt_bias[h]) : 0.f;
        float run = dt * A[h] * kLog2e;
#pragma unroll
        for (int d = 1; d < 32; d <<= 1) {
          float o = __shfl_up(run, d, 32);
          if ((lane & 31) >= d) run += o;
        }
        const float tot = __shfl(run, (lane & 32) + 31);   // the block's total
        float* hr = reinterpret_cast<float*>(hbase + (hrec0 + (size_t)h * nC + c) * C::HREC_BYTES);
        hr[s] = dt;
        hr[Q + s] = run;
        hr[2 * Q + s] = exp2_hw(tot - run) * dt;   // decay from s to the end of its block, times dt
      }
    }
  }
  if constexpr (CONV) {
    f32x4 wv[VE];
    float bs[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      wv[i] = *reinterpret_cast<const f32x4*>(cv.w + (int64_t)(ch + i) * 4);
      bs[i] = cv.bias ? cv.bias[ch + i] : 0.f;
    }
    T (*dst)[C::LDN] = isC ? sC : sB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      Vec<T> o = zero16<T>();
      if (s1 + j < nvalid) {
#pragma unroll
        for (int i = 0; i < VE; ++i)
          o.set(i, conv4_silu(wv[i], bs[i], rB[j].get(i), rB[j + 1].get(i), rB[j + 2].get(i),
                              rB[j + 3].get(i)));
      }
      st16(&dst[s1 + j][n0], o);
    }
  } else if constexpr (HOLD) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int v = tid + i * PREP_THREADS;
      const int s = v / (SN / VE), e0 = v % (SN / VE) * VE;
      const bool ok = s < nvalid;
      st16(&sB[s][e0], ok ? rB[i] : zero16<T>());
      st16(&sC[s][e0], ok ? rC[i] : zero16<T>());
    }
  }
  if constexpr (VARLEN) {
    // a sequence's first chunk: the conv history of the group's x channels (zeros without an
    // initial state) goes to the chunk's place in the history area, where the scan reads it
    const int4 ci = vd.info[c];
    if (ci.y & INFO_FIRST) {
      const int nxv = (H / G) * SP / VE;   // 16-byte vectors of the group's x channels per row
      const int HP = H * SP;
      for (int v = tid; v < 3 * nxv; v += PREP_THREADS) {
        const int j = v / nxv, e0 = g * (H / G) * SP + (v % nxv) * VE;
        const Vec<T> hv = hist0 ? ld16(hist0 + (int64_t)j * cv.Cc + e0) : zero16<T>();
        st16(reinterpret_cast<T*>(vd.hist) + ((size_t)c * 3 + j) * HP + e0, hv);
      }
    }
  }
  __syncthreads();
  // Gram tiles: wave w computes lower-triangle tiles k = w, w+4, ...
  for (int k = wave; k < C::NTILES; k += 4) {
    const int tb = tile_tb(k), si = k - tb * (tb + 1) / 2;
    f32x16 acc = (f32x16){};
#pragma unroll
    for (int j = 0; j < C::KS_N; ++j)
      mma(acc, frag_contig(&sB[si * 32 + col][16 * j], g2), frag_contig(&sC[tb * 32 + col][16 * j], g2));
    // stored as [q][lane][4]: accumulator registers 4q .. 4q+3 of every lane, so that each
    // of the reader's four 16-byte loads covers 1 KiB contiguously
    float* dst = gout + (size_t)k * 1024 + 4 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(dst + 256 * q) =
          (f32x4){acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  }
  // B^T operand frags (row n = nb*32 + col, k = s): record (nb, j), lane
  for (int idx = tid; idx < (SN / 32) * C::KS_Q * 64; idx += PREP_THREADS) {
    const int r = idx >> 6, ln = idx & 63;
    const int nb = r / C::KS_Q, j = r % C::KS_Q;
    const int n = nb * 32 + (ln & 31), s0 = 16 * j + 8 * (ln >> 5);
    Frag<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = sB[s0 + e][n];
    st_frag<T>(btf + (size_t)idx * C::FB, f);
  }
  // C operand frags (col t = tb*32 + col, k = n): record (tb, j), lane
  for (int idx = tid; idx < C::NTB * C::KS_N * 64; idx += PREP_THREADS) {
    const int r = idx >> 6, ln = idx & 63;
    const int tb = r / C::KS_N, j = r % C::KS_N;
    st_frag<T>(cff + (size_t)idx * C::FB, frag_contig(&sC[tb * 32 + (ln & 31)][16 * j], ln >> 5));
  }
}

// ---------------------------------------------------------------------------- scan kernel, chunk 256
// One role per wave for the whole chunk: 4 Y waves build the masked decay tiles M^T of their
// token blocks in registers and compute Y^T, 4 H waves update the state (two barriers per
// chunk). z is read straight from HBM (the chunk does not fit LDS alongside the rest).
template <typename T, int Q>
struct WideSmem {
  using C = Cfg<T, Q>;
  T sXt[SP][C::LDQ];                       // x^T (k = s): A operand of Y_diag
  T sXW[SP][C::LDQ];                       // (w x)^T hi: B operand of the state update
  T sXWlo[C::SPLIT ? SP : 1][C::LDQ];      //        lo
  T sHt[SP][C::LDN];                       // H^T hi: A operand of Y_off
  T sHtlo[C::SPLIT ? SP : 1][C::LDN];      //     lo
  float sG[C::STAGE_Z ? Q : 1][SP + 4];    // SiLU(z) of the chunk in fp32, then y (fp32)
  float sPi[Q];                            // inclusive prefix of dt*A*log2e inside 32-token blocks
  float sDt[Q];
  float sE[Q];                             // exp2(lambda_t), lambda from the chunk start
  float sF[C::NTB][Q];                     // sF[tb][s] = exp2(lambda_{32tb-1} - lambda_s) dt_s, s < 32 tb
};

// State tiles (32x32 of H[n][p], nb = n / 32, pb = p / 32) updated by H wave hw, dealt so
// that each SIMD (one Y wave + one H wave) gets about the same number of MFMAs. slot[i]
// indexes the distinct row blocks nbs[] whose B^T operands the wave keeps in registers.
struct HList { int n; int nb[4]; int pb[4]; int slot[4]; int nbs[2]; };
template <int Q> __device__ __forceinline__ HList hlist(int hw);
template <> __device__ __forceinline__ HList hlist<64>(int hw) {
  return {2, {hw, hw, 0, 0}, {0, 1, 0, 0}, {0, 0, 0, 0}, {hw, hw}};
}
template <> __device__ __forceinline__ HList hlist<128>(int hw) {
  switch (hw) {
    case 0: return {3, {0, 0, 1, 0}, {0, 1, 0, 0}, {0, 0, 1, 0}, {0, 1}};
    case 1: return {2, {1, 2, 0, 0}, {1, 0, 0, 0}, {0, 1, 0, 0}, {1, 2}};
    case 2: return {2, {2, 3, 0, 0}, {1, 0, 0, 0}, {0, 1, 0, 0}, {2, 3}};
    default: return {1, {3, 0, 0, 0}, {1, 0, 0, 0}, {0, 0, 0, 0}, {3, 3}};
  }
}
template <> __device__ __forceinline__ HList hlist<256>(int hw) {
  return {2, {hw, hw, 0, 0}, {0, 1, 0, 0}, {0, 0, 0, 0}, {hw, hw}};
}
// Token blocks and p-blocks owned by Y wave y: Q=64: one (tb, pb) each; Q=128: block y,
// both p-blocks; Q=256: blocks y and 7-y (light + heavy), both p-blocks.
template <int Q> struct YPlan;
template <> struct YPlan<64> {
  static constexpr int NT = 1, NPB = 1;
  __device__ static int tb(int y, int) { return y & 1; }
  __device__ static int pb(int y, int) { return y >> 1; }
};
template <> struct YPlan<128> {
  static constexpr int NT = 1, NPB = 2;
  __device__ static int tb(int y, int) { return y; }
  __device__ static int pb(int, int i) { return i; }
};
template <> struct YPlan<256> {
  static constexpr int NT = 2, NPB = 2;
  __device__ static int tb(int y, int k) { return k == 0 ? y : 7 - y; }
  __device__ static int pb(int, int i) { return i; }
};

template <typename T>
__device__ __forceinline__ void split_set(Frag<T>& hi, Frag<T>& lo, int e, float v) {
  frag_set<T>(hi, e, v);
  if constexpr (sizeof(T) == 2) frag_set<T>(lo, e, v - frag_get(hi, e));
}

// one Gram tile (1024 floats, [q][lane][4]) into this lane's accumulator-order registers
__device__ __forceinline__ f32x16 load_tile16(const float* tile, int lane) {
  f32x16 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 v = *reinterpret_cast<const f32x4*>(tile + 256 * q + 4 * lane);
    r[4 * q] = v[0];
    r[4 * q + 1] = v[1];
    r[4 * q + 2] = v[2];
    r[4 * q + 3] = v[3];
  }
  return r;
}

template <typename T, int Q>
__global__ __launch_bounds__(SCAN_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssd_scan_wide_kernel(const T* __restrict__ x, int64_t x_stride, const float* __restrict__ D,
                     const T* __restrict__ z, int64_t z_stride, const float* h0, float* h_final,
                     T* __restrict__ y, int64_t y_stride, const unsigned char* __restrict__ ws,
                     int L, int H, int G) {
  using C = Cfg<T, Q>;
  using YP = YPlan<Q>;
  constexpr int VE = C::VE;
  extern __shared__ __align__(16) unsigned char scan_smem[];
  WideSmem<T, Q>& S = *reinterpret_cast<WideSmem<T, Q>*>(scan_smem);

  const int id = xcd_local_order(blockIdx.x, gridDim.x);
  const int b = id / H, h = id % H;
  const int g = h / (H / G);
  const int nC = (L + Q - 1) / Q;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g2 = lane >> 5;
  const bool ywave = wave < 4;
  const int hw = ywave ? 0 : wave - 4;

  const int64_t row0 = (int64_t)b * L;
  const T* xb = x + h * SP;
  const T* zb = z ? z + h * SP : nullptr;
  T* yb = y + h * SP;
  const float Dh = D ? D[h] : 0.f;
  const unsigned char* wsg = ws + (size_t)(b * G + g) * nC * C::REC_BYTES;
  const float* hrec = reinterpret_cast<const float*>(
      ws + (size_t)G * nC * C::REC_BYTES * (size_t)(gridDim.x / H) +
      ((size_t)b * H + h) * nC * C::HREC_BYTES);

  // ------------------------------------------------------------ staging registers
  // x: XV 16-byte vectors per thread. With PAIRS, vectors 2i and 2i+1 are tokens 2sp and
  // 2sp+1 of one 16-byte column, 8 lanes per token row (coalesced loads), so x^T and
  // (w x)^T go to LDS as 32-bit token pairs. z: the same row-major mapping, 16-byte
  // vectors straight into sZ.
  Vec<T> rX[C::XV], rZ[C::XV];
  float rdt[C::TPL], rpi[C::TPL];
  auto xcoord = [&](int i, int& s, int& cv) {
    constexpr int VPR = SP / VE;  // vectors per token row
    if constexpr (C::PAIRS) {
      const int u = tid + SCAN_THREADS * (i >> 1);
      s = 2 * (u / VPR) + (i & 1);
      cv = u % VPR;
    } else {
      const int v = tid + SCAN_THREADS * i;
      s = v / VPR;
      cv = v % VPR;
    }
  };
  auto load_chunk = [&](int c) {
    const int t0 = c * Q;
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      int s_, cv;
      xcoord(i, s_, cv);
      const int t = t0 + s_;
      const bool ok = t < L;
      rX[i] = ok ? ld16(xb + (row0 + t) * x_stride + cv * VE) : zero16<T>();
      if constexpr (C::STAGE_Z) {
        if (zb) rZ[i] = ok ? ld16(zb + (row0 + t) * z_stride + cv * VE) : zero16<T>();
      }
    }
    const float* hr = hrec + (size_t)c * (3 * Q);
#pragma unroll
    for (int k = 0; k < C::TPL; ++k) {
      rdt[k] = hr[lane + 64 * k];
      rpi[k] = hr[Q + lane + 64 * k];
    }
  };

  // ------------------------------------------------------------ chunk phase S1
  // y of the previous chunk out of sZ (coalesced), z of this chunk in; decay vectors
  // (every wave derives them, so staging threads get w_s by a cross-lane shuffle); x^T and
  // (w x)^T into LDS; prefetch of the next chunk.
  auto phase_s1 = [&](int c) {
    if constexpr (C::STAGE_Z) {
#pragma unroll
      for (int i = 0; i < C::XV; ++i) {
        int s_, cv;
        xcoord(i, s_, cv);
        float* grow = &S.sG[s_][cv * VE];
        if (c > 0) {
          const int t = (c - 1) * Q + s_;
          if (t < L) {
            Vec<T> o;
#pragma unroll
            for (int e = 0; e < VE; ++e) o.set(e, grow[e]);
            st16(yb + (row0 + t) * y_stride + cv * VE, o);
          }
        }
        if (zb) {
#pragma unroll
          for (int e = 0; e < VE; e += 4)
            *reinterpret_cast<f32x4*>(grow + e) =
                (f32x4){silu_fast(rZ[i].get(e)), silu_fast(rZ[i].get(e + 1)),
                        silu_fast(rZ[i].get(e + 2)), silu_fast(rZ[i].get(e + 3))};
        }
      }
    }
    float tot[C::NTB];
#pragma unroll
    for (int k = 0; k < C::TPL; ++k) {
      tot[2 * k] = __shfl(rpi[k], 31);
      tot[2 * k + 1] = __shfl(rpi[k], 63);
    }
    float wv[C::TPL];
#pragma unroll
    for (int k = 0; k < C::TPL; ++k) {
      const int blk = 2 * k + (lane >> 5);
      float before = 0.f, after = 0.f;
#pragma unroll
      for (int bb = 0; bb < C::NTB; ++bb) {
        if (bb < blk) before += tot[bb];
        if (bb > blk) after += tot[bb];
      }
      const float tail = tot[blk] - rpi[k];  // lambda_{end of blk} - lambda_t
      wv[k] = exp2_hw(tail + after) * rdt[k];
      if (wave == 0) {
        const int t = lane + 64 * k;
        S.sPi[t] = rpi[k];
        S.sDt[t] = rdt[k];
        S.sE[t] = exp2_hw(before + rpi[k]);
        float acc = tail;
#pragma unroll
        for (int tb = 1; tb < C::NTB; ++tb) {
          if (tb > blk) {
            S.sF[tb][t] = exp2_hw(acc) * rdt[k];
            acc += tot[tb];
          }
        }
      }
    }
    // w of token s lives in lane s % 64, register s / 64
    auto w_of = [&](int s_) {
      float r = 0.f;
#pragma unroll
      for (int k = 0; k < C::TPL; ++k) {
        const float o = __shfl(wv[k], s_ & 63);
        if ((s_ >> 6) == k) r = o;
      }
      return r;
    };
    if constexpr (C::PAIRS) {
#pragma unroll
      for (int i = 0; i < C::XV; i += 2) {
        int s_, cv;
        xcoord(i, s_, cv);
        const float w0 = w_of(s_), w1 = w_of(s_ + 1);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const T x0 = rX[i].v[e], x1 = rX[i + 1].v[e];
          const float v0 = to_f(x0) * w0, v1 = to_f(x1) * w1;
          const T h0_ = from_f<T>(v0), h1_ = from_f<T>(v1);
          const int p = cv * VE + e, sw = xsw<Q>(p, s_);
          st_pair(&S.sXt[p][sw], x0, x1);
          st_pair(&S.sXW[p][sw], h0_, h1_);
          if constexpr (C::SPLIT)
            st_pair(&S.sXWlo[p][sw], from_f<T>(v0 - to_f(h0_)), from_f<T>(v1 - to_f(h1_)));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::XV; ++i) {
        int s_, cv;
        xcoord(i, s_, cv);
        const float w0 = w_of(s_);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const T x0 = rX[i].v[e];
          const float v0 = to_f(x0) * w0;
          const T h0_ = from_f<T>(v0);
          const int p = cv * VE + e, sw = xsw<Q>(p, s_);
          S.sXt[p][sw] = x0;
          S.sXW[p][sw] = h0_;
          if constexpr (C::SPLIT) S.sXWlo[p][sw] = from_f<T>(v0 - to_f(h0_));
        }
      }
    }
    if (c + 1 < nC) load_chunk(c + 1);
  };

  // The two roles run separate chunk loops with the same barrier sequence (two barriers
  // per chunk), so each role's registers are allocated on their own.
  if (ywave) {
    // ========================================================== Y waves: outputs
    Frag<T> cf[C::KS_N];                // C operand frags of the token block
    f32x16 gq0, gq1;                    // Gram tiles, fetched two ahead
    Raw4<T> ze[YP::NPB][4];             // z when it is not staged through LDS
    auto yfetch = [&](int c, int tb) {
      const unsigned char* rec = wsg + (size_t)c * C::REC_BYTES;
      const unsigned char* cfp = rec + C::G_BYTES + C::BT_BYTES;
#pragma unroll
      for (int j = 0; j < C::KS_N; ++j)
        cf[j] = ld_frag<T>(cfp + ((size_t)(tb * C::KS_N + j) * 64 + lane) * C::FB);
      const float* gt = reinterpret_cast<const float*>(rec);
      const int k0 = tb * (tb + 1) / 2;
      gq0 = load_tile16(gt + (size_t)k0 * 1024, lane);
      if (tb > 0) gq1 = load_tile16(gt + (size_t)(k0 + 1) * 1024, lane);
      if constexpr (!C::STAGE_Z) {
        const int t = c * Q + tb * 32 + col;
        if (zb && t < L) {
#pragma unroll
          for (int i = 0; i < YP::NPB; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              ze[i][r4] = ld4(zb + (row0 + t) * z_stride + YP::pb(wave, i) * 32 + 8 * r4 + 4 * g2);
        }
      }
    };
    if (nC > 0) load_chunk(0);
    for (int c = 0; c < nC; ++c) {
      const int t0 = c * Q;
      const float* gt = reinterpret_cast<const float*>(wsg + (size_t)c * C::REC_BYTES);
      yfetch(c, YP::tb(wave, 0));
      phase_s1(c);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < YP::NT; ++k) {
        const int tb = YP::tb(wave, k);
        if (k > 0) yfetch(c, tb);
        const int tl = tb * 32 + col;
        const int t = t0 + tl;
        f32x16 yoff[YP::NPB], yd[YP::NPB];
        // carried state: Y^T = H^T C^T (scaled by exp2(lambda_t) in the epilogue)
#pragma unroll
        for (int i = 0; i < YP::NPB; ++i) {
          const int prow = YP::pb(wave, i) * 32 + col;
          yoff[i] = (f32x16){};
          yd[i] = (f32x16){};
#pragma unroll
          for (int j = 0; j < C::KS_N; ++j) {
            mma(yoff[i], frag_contig(&S.sHt[prow][16 * j], g2), cf[j]);
            if constexpr (C::SPLIT) mma(yoff[i], frag_contig(&S.sHtlo[prow][16 * j], g2), cf[j]);
          }
        }
        // off-diagonal source blocks si < tb: M = G * F[s]; the column factor U[t] after
        const int k0 = tb * (tb + 1) / 2;
        for (int si = 0; si < tb; ++si) {
          const f32x16 gcur = gq0;
          gq0 = gq1;
          if (si + 2 <= tb) gq1 = load_tile16(gt + (size_t)(k0 + si + 2) * 1024, lane);
          Frag<T> mh[2], ml[2];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 fs = *reinterpret_cast<const f32x4*>(&S.sF[tb][si * 32 + 8 * r4 + 4 * g2]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 4 * r4 + q;
              split_set<T>(mh[r >> 3], ml[r >> 3], r & 7, gcur[r] * fs[q]);
            }
          }
#pragma unroll
          for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < YP::NPB; ++i) {
              const int prow = YP::pb(wave, i) * 32 + col;
              Frag<T> xa = frag_accrows_sw<Q>(S.sXt[prow], prow, si * 32 + 16 * m2, g2);
              mma(yd[i], xa, mh[m2]);
              if constexpr (C::SPLIT) mma(yd[i], xa, ml[m2]);
            }
        }
        const float pit = S.sPi[tl];
        if (tb > 0) {
          const float ut = exp2_hw(pit);  // exp2(lambda_t - lambda_{32tb-1})
#pragma unroll
          for (int i = 0; i < YP::NPB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) yd[i][r] *= ut;
        }
        // diagonal block: exp2(pi_t - pi_s) dt_s for s <= t, plus D on the diagonal (the
        // skip term); its Gram tile is in gq0
        {
          Frag<T> mh[2], ml[2];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int s0 = tb * 32 + 8 * r4 + 4 * g2;
            const f32x4 ps = *reinterpret_cast<const f32x4*>(&S.sPi[s0]);
            const f32x4 ds = *reinterpret_cast<const f32x4*>(&S.sDt[s0]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 4 * r4 + q;
              float v = (s0 + q <= tl) ? gq0[r] * exp2_hw(pit - ps[q]) * ds[q] : 0.f;
              if (s0 + q == tl) v += Dh;
              split_set<T>(mh[r >> 3], ml[r >> 3], r & 7, v);
            }
          }
#pragma unroll
          for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < YP::NPB; ++i) {
              const int prow = YP::pb(wave, i) * 32 + col;
              Frag<T> xa = frag_accrows_sw<Q>(S.sXt[prow], prow, tb * 32 + 16 * m2, g2);
              mma(yd[i], xa, mh[m2]);
              if constexpr (C::SPLIT) mma(yd[i], xa, ml[m2]);
            }
        }
        // epilogue: y = (E_t Y_off + Y_diag) SiLU(z)
        const float et = S.sE[tl];
#pragma unroll
        for (int i = 0; i < YP::NPB; ++i)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int p0 = YP::pb(wave, i) * 32 + 8 * r4 + 4 * g2;
            float o[4];
            if constexpr (C::STAGE_Z) {
              f32x4 gg = {1.f, 1.f, 1.f, 1.f};
              if (zb) gg = *reinterpret_cast<const f32x4*>(&S.sG[tl][p0]);
#pragma unroll
              for (int q = 0; q < 4; ++q) o[q] = (et * yoff[i][4 * r4 + q] + yd[i][4 * r4 + q]) * gg[q];
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float v = et * yoff[i][4 * r4 + q] + yd[i][4 * r4 + q];
                if (zb) v *= silu_fast(ze[i][r4].get(q));
                o[q] = v;
              }
            }
            if constexpr (C::STAGE_Z) {
              *reinterpret_cast<f32x4*>(&S.sG[tl][p0]) = (f32x4){o[0], o[1], o[2], o[3]};
            } else {
              if (t < L) st4(yb + (row0 + t) * y_stride + p0, o[0], o[1], o[2], o[3]);
            }
          }
      }
      __syncthreads();
    }
  } else {
    // ========================================================== H waves: state
    const HList hl = hlist<Q>(hw);
    f32x16 hacc[4];
    Frag<T> af[C::NBD][C::KS_Q];        // B^T operand frags of the chunk
    const int64_t sbase = ((int64_t)b * H + h) * SN * SP;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < hl.n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int n = hl.nb[i] * 32 + acc_row(r, lane), p = hl.pb[i] * 32 + col;
          hacc[i][r] = h0 ? h0[sbase + n * SP + p] : 0.f;
        }
      }
    auto write_state = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < hl.n) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            int n = hl.nb[i] * 32 + 8 * r4 + 4 * g2, p = hl.pb[i] * 32 + col;
            float v[4], lo[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[k] = hacc[i][4 * r4 + k];
              lo[k] = v[k] - to_f(from_f<T>(v[k]));
            }
            st4(&S.sHt[p][n], v[0], v[1], v[2], v[3]);
            if constexpr (C::SPLIT) st4(&S.sHtlo[p][n], lo[0], lo[1], lo[2], lo[3]);
          }
        }
    };
    write_state();
    if (nC > 0) load_chunk(0);
    for (int c = 0; c < nC; ++c) {
      const unsigned char* btf = wsg + (size_t)c * C::REC_BYTES + C::G_BYTES;
#pragma unroll
      for (int d = 0; d < C::NBD; ++d)
#pragma unroll
        for (int j = 0; j < C::KS_Q; ++j)
          af[d][j] = ld_frag<T>(btf + ((size_t)(hl.nbs[d] * C::KS_Q + j) * 64 + lane) * C::FB);
      phase_s1(c);
      __syncthreads();
      const float eend = S.sE[Q - 1];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < hl.n)
#pragma unroll
          for (int r = 0; r < 16; ++r) hacc[i][r] *= eend;
#pragma unroll
      for (int j = 0; j < C::KS_Q; ++j) {
        Frag<T> bh[2], bl[2];
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          const int prow = pb * 32 + col, k0 = xsw<Q>(prow, 16 * j + 8 * g2);
          bh[pb] = frag_contig(&S.sXW[prow][k0], 0);
          if constexpr (C::SPLIT) bl[pb] = frag_contig(&S.sXWlo[prow][k0], 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < hl.n) {
            const Frag<T>& a = (C::NBD > 1 && hl.slot[i]) ? af[C::NBD - 1][j] : af[0][j];
            mma(hacc[i], a, hl.pb[i] ? bh[1] : bh[0]);
            if constexpr (C::SPLIT) mma(hacc[i], a, hl.pb[i] ? bl[1] : bl[0]);
          }
      }
      __syncthreads();
      write_state();
    }
    if (h_final) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < hl.n) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int n = hl.nb[i] * 32 + acc_row(r, lane), p = hl.pb[i] * 32 + col;
            h_final[sbase + n * SP + p] = hacc[i][r];
          }
        }
    }
  }

  // y of the last chunk out of sZ
  if constexpr (C::STAGE_Z) {
    if (nC > 0) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < C::XV; ++i) {
        int s_, cv;
        xcoord(i, s_, cv);
        const int t = (nC - 1) * Q + s_;
        if (t < L) {
          Vec<T> o;
#pragma unroll
          for (int e = 0; e < VE; ++e) o.set(e, S.sG[s_][cv * VE + e]);
          st16(yb + (row0 + t) * y_stride + cv * VE, o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------- scan kernel
// Chunk sizes 64 and 128. Per chunk, three phases separated by barriers:
//  S1 (all waves) stage the chunk: y of the previous chunk out of LDS (coalesced), raw z
//     in, x^T and (w x)^T hi/lo, the chunk's dt / pi / v record; prefetch the next chunk.
//  S2 Y waves: Y^T = H^T C^T for their tiles, scaled by exp2(lambda_t), and SiLU(z) into
//     registers. H waves: the masked decay tiles M^T of the chunk (hi/lo) into LDS, each
//     built once for all Y waves.
//  S3 Y waves: Y^T += X^T M^T and the gated epilogue into LDS. H waves: H = exp2(lambda_end)
//     H + B^T (w x), then the new state (bf16 hi/lo) into LDS for the next chunk.
// Ownership: Y wave y holds two Y^T tiles (token blocks tb, one p-block) whose triangle
// work adds up to the same amount on every wave; H wave w holds two state tiles of one
// p-block. Each SIMD runs one Y wave and one H wave.
//
// Decay bookkeeping (log2 units, lambda_t = sum of dt*A*log2e from the chunk start through
// t, blocks of 32 tokens with totals tot_k and in-block prefixes pi_t):
//   exp2(lambda_t) = exp2(sum_{k<blk(t)} tot_k + pi_t)
//   w_s = exp2(lambda_end - lambda_s) dt_s = v_s exp2(sum_{k>blk(s)} tot_k)
//   decay s -> t across blocks si < tb = v_s exp2(sum_{si<k<tb} tot_k) exp2(pi_t)
template <int Q> struct Own;
template <> struct Own<64> {
  static constexpr int NY = 1;
  static constexpr int NB = 1;   // M tiles built per H wave (at most)
  __device__ static int tb(int y, int) { return y >> 1; }
  __device__ static int build(int w, int) { return w < 3 ? w : -1; }
};
template <> struct Own<128> {
  static constexpr int NY = 2;
  static constexpr int NB = 3;
  __device__ static int tb(int y, int i) { return y < 2 ? (i ? 3 : 0) : (i ? 2 : 1); }
  // lower-triangle tile k = tb (tb + 1) / 2 + si: H wave w builds diagonal tile w and one
  // or two of the off-diagonal tiles 1, 3, 4, 6, 7, 8
  __device__ static int build(int w, int i) {
    if (i == 0) return w * (w + 3) / 2;
    if (i == 1) return w == 0 ? 1 : w == 1 ? 3 : w == 2 ? 4 : 6;
    return w == 0 ? 8 : w == 1 ? 7 : -1;
  }
};

template <typename T, int Q>
struct ScanSmem {
  using C = Cfg<T, Q>;
  T sXt[SP][C::LDQ];                        // x^T (k = s): A operand of Y^T += X^T M^T
  T sXW[SP][C::LDQ];                        // (w x)^T hi: B operand of the state update
  T sXWlo[C::SPLIT ? SP : 1][C::LDQ];       //        lo
  T sHt[SP][C::LDN];                        // H^T hi: A operand of Y^T = H^T C^T
  T sHtlo[C::SPLIT ? SP : 1][C::LDN];       //     lo
  T sZ[Q][SP];                              // z of the chunk, then y (zpos layout)
  Frag<T> sM[C::NTILES][2][64];             // M^T tiles in B-operand order [tile][k step][lane]
  Frag<T> sMlo[C::SPLIT ? C::NTILES : 1][2][64];
  float sRec[3 * Q];                        // dt | pi | v of the chunk
};

// Element (t, p) of the z / y tile sits at column zpos(t, p): 4-element groups XOR-ed with a
// key of the token, so that the epilogue's 4-element accesses (32 tokens x one column group
// per instruction) hit distinct banks. 16-byte staging vectors stay whole; with bf16 the two
// halves of a vector trade places when bit 2 of the key is set.
template <typename T>
__device__ __forceinline__ int zkey(int t) {
  return 4 * ((sizeof(T) == 2 ? t >> 1 : t) & 15);
}
template <typename T>
__device__ __forceinline__ int zpos(int t, int p) { return p ^ zkey<T>(t); }

template <typename T>
__device__ __forceinline__ Vec<T> half_swap(const Vec<T>& v, bool swap) {
  if constexpr (sizeof(T) == 2) {
    Vec<T> r;
    r.v = swap ? __builtin_shufflevector(v.v, v.v, 4, 5, 6, 7, 0, 1, 2, 3) : v.v;
    return r;
  } else {
    return v;
  }
}

template <typename T, int Q>
__global__ __launch_bounds__(SCAN_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssd_scan_kernel(const T* __restrict__ x, int64_t x_stride, const float* __restrict__ D,
                     const T* __restrict__ z, int64_t z_stride, const float* h0, float* h_final,
                     T* __restrict__ y, int64_t y_stride, const unsigned char* __restrict__ ws,
                     int L, int H, int G) {
  using C = Cfg<T, Q>;
  using OW = Own<Q>;
  constexpr int VE = C::VE;
  constexpr int NTB = C::NTB;
  extern __shared__ __align__(16) unsigned char scan_smem[];
  ScanSmem<T, Q>& S = *reinterpret_cast<ScanSmem<T, Q>*>(scan_smem);
  const float* sDt = S.sRec;
  const float* sPi = S.sRec + Q;
  const float* sV = S.sRec + 2 * Q;

  const int id = xcd_local_order(blockIdx.x, gridDim.x);
  const int b = id / H, h = id % H;
  const int g = h / (H / G);
  const int nC = (L + Q - 1) / Q;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g2 = lane >> 5;
  const bool ywave = wave < 4;

  const int64_t row0 = (int64_t)b * L;
  const T* xb = x + h * SP;
  const T* zb = z ? z + h * SP : nullptr;
  T* yb = y + h * SP;
  const float Dh = D ? D[h] : 0.f;
  const unsigned char* wsg = ws + (size_t)(b * G + g) * nC * C::REC_BYTES;
  const float* hrec = reinterpret_cast<const float*>(
      ws + (size_t)G * nC * C::REC_BYTES * (size_t)(gridDim.x / H) +
      ((size_t)b * H + h) * nC * C::HREC_BYTES);

  // ------------------------------------------------------------ staging registers
  // x and z: XV 16-byte vectors per thread. With PAIRS, vectors 2i and 2i+1 are tokens
  // 2sp and 2sp+1 of one 16-byte column, 8 lanes per token row (coalesced loads), so x^T
  // and (w x)^T go to LDS as 32-bit token pairs.
  Vec<T> rX[C::XV], rZ[C::XV];
  float rV[C::XV];                  // v of each staged token
  float rRec;                       // one word of the dt | pi | v record (threads < 3Q)
  float tot[NTB];                   // block totals of the chunk (wave-uniform)
  auto xcoord = [&](int i, int& s, int& cv) {
    constexpr int VPR = SP / VE;  // vectors per token row
    if constexpr (C::PAIRS) {
      const int u = tid + SCAN_THREADS * (i >> 1);
      s = 2 * (u / VPR) + (i & 1);
      cv = u % VPR;
    } else {
      const int v = tid + SCAN_THREADS * i;
      s = v / VPR;
      cv = v % VPR;
    }
  };
  auto load_chunk = [&](int c) {
    const int t0 = c * Q;
    const float* hr = hrec + (size_t)c * (3 * Q);
    // Rows past the end of the sequence load the last row instead (finite values; their
    // dt and v are zero, so they add nothing), which keeps the loads unconditional: a
    // guarded load makes the compiler wait for it on the spot.
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      int s_, cv;
      xcoord(i, s_, cv);
      const int t = min(t0 + s_, L - 1);
      rX[i] = ld16(xb + (row0 + t) * x_stride + cv * VE);
      if (zb) rZ[i] = ld16(zb + (row0 + t) * z_stride + cv * VE);
      rV[i] = hr[2 * Q + s_];
    }
    if (tid < 3 * Q) rRec = hr[tid];
#pragma unroll
    for (int k = 0; k < NTB; ++k) tot[k] = hr[Q + 32 * k + 31];
  };
  // y of chunk c-1 out of sZ, thread by thread over the same vectors it then refills
  auto flush_y = [&](int c, int s_, int cv) {
    const int t = (c - 1) * Q + s_;
    const int key = zkey<T>(s_);
    const Vec<T> v = ld16(&S.sZ[s_][(cv * VE) ^ (key & ~(VE - 1))]);
    if (t < L) st16(yb + (row0 + t) * y_stride + cv * VE, half_swap<T>(v, (key & 4) && VE == 8));
  };

  // ------------------------------------------------------------ phase S1
  // Leaves the chunk's block totals in `ctot` for the rest of the chunk.
  float ctot[NTB];
  auto stage = [&](int c) {
#pragma unroll
    for (int k = 0; k < NTB; ++k) ctot[k] = tot[k];
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      int s_, cv;
      xcoord(i, s_, cv);
      if (c > 0) flush_y(c, s_, cv);
      if (zb) {
        const int key = zkey<T>(s_);
        st16(&S.sZ[s_][(cv * VE) ^ (key & ~(VE - 1))], half_swap<T>(rZ[i], (key & 4) && VE == 8));
      }
    }
    if (tid < 3 * Q) S.sRec[tid] = rRec;
    // w_s = v_s exp2(decay from the end of s's block to the end of the chunk); written as
    // a sum of selects (a table of the per-block factors indexed by the lane's block would
    // go through scratch memory)
    auto w_of = [&](int i, int s_) {
      const int blk = s_ >> 5;
      float after = 0.f;
#pragma unroll
      for (int k = 1; k < NTB; ++k) after += k > blk ? ctot[k] : 0.f;
      return rV[i] * exp2_hw(after);
    };
    if constexpr (C::PAIRS) {
#pragma unroll
      for (int i = 0; i < C::XV; i += 2) {
        int s_, cv;
        xcoord(i, s_, cv);
        const float w0 = w_of(i, s_), w1 = w_of(i + 1, s_ + 1);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const T x0 = rX[i].v[e], x1 = rX[i + 1].v[e];
          const float v0 = to_f(x0) * w0, v1 = to_f(x1) * w1;
          const T h0_ = from_f<T>(v0), h1_ = from_f<T>(v1);
          const int p = cv * VE + e, sw = xsw<Q>(p, s_);
          st_pair(&S.sXt[p][sw], x0, x1);
          st_pair(&S.sXW[p][sw], h0_, h1_);
          if constexpr (C::SPLIT)
            st_pair(&S.sXWlo[p][sw], from_f<T>(v0 - to_f(h0_)), from_f<T>(v1 - to_f(h1_)));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::XV; ++i) {
        int s_, cv;
        xcoord(i, s_, cv);
        const float w0 = w_of(i, s_);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const T x0 = rX[i].v[e];
          const float v0 = to_f(x0) * w0;
          const T h0_ = from_f<T>(v0);
          const int p = cv * VE + e, sw = xsw<Q>(p, s_);
          S.sXt[p][sw] = x0;
          S.sXW[p][sw] = h0_;
          if constexpr (C::SPLIT) S.sXWlo[p][sw] = from_f<T>(v0 - to_f(h0_));
        }
      }
    }
    if (c + 1 < nC) load_chunk(c + 1);
  };

  // The two roles run separate chunk loops with the same barrier sequence (three barriers
  // per chunk), so each role's registers are allocated on their own.
  if (ywave) {
    // ========================================================== Y waves: outputs
    const int pb = wave & 1;
    const int prow = pb * 32 + col;
    Frag<T> cf[OW::NY][C::KS_N];        // C operand frags of the owned token blocks
    auto fetch = [&](int c) {
      const unsigned char* cfp = wsg + (size_t)c * C::REC_BYTES + C::G_BYTES + C::BT_BYTES;
#pragma unroll
      for (int i = 0; i < OW::NY; ++i)
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j)
          cf[i][j] = ld_frag<T>(cfp + ((size_t)(OW::tb(wave, i) * C::KS_N + j) * 64 + lane) * C::FB);
    };
    if (nC > 0) {
      load_chunk(0);
      fetch(0);
    }
    for (int c = 0; c < nC; ++c) {
      stage(c);
      __syncthreads();
      // ---- S2: carried state, scaled by exp2(lambda_t); gate values
      f32x16 acc[OW::NY];
      float gz[OW::NY][16];
#pragma unroll
      for (int i = 0; i < OW::NY; ++i) {
        acc[i] = (f32x16){};
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j) {
          mma(acc[i], frag_contig(&S.sHt[prow][16 * j], g2), cf[i][j]);
          if constexpr (C::SPLIT) mma(acc[i], frag_contig(&S.sHtlo[prow][16 * j], g2), cf[i][j]);
        }
      }
#pragma unroll
      for (int i = 0; i < OW::NY; ++i) {
        const int tb = OW::tb(wave, i);
        const int tl = tb * 32 + col;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          if (zb) {
            const Raw4<T> zz = ld4(&S.sZ[tl][zpos<T>(tl, pb * 32 + 8 * r4 + 4 * g2)]);
#pragma unroll
            for (int q = 0; q < 4; ++q) gz[i][4 * r4 + q] = silu_fast(zz.get(q));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) gz[i][4 * r4 + q] = 1.f;
          }
        }
        float before = 0.f;
#pragma unroll
        for (int k = 0; k < NTB - 1; ++k)
          if (k < tb) before += ctot[k];
        const float et = exp2_hw(before + sPi[tl]);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= et;
      }
      __syncthreads();
      if (c + 1 < nC) fetch(c + 1);
      // ---- S3: intra-chunk part from the M^T tiles, then y = acc * SiLU(z) into sZ
#pragma unroll
      for (int i = 0; i < OW::NY; ++i) {
        const int tb = OW::tb(wave, i);
        const int k0 = tb * (tb + 1) / 2;
        for (int si = 0; si <= tb; ++si) {
#pragma unroll
          for (int m2 = 0; m2 < 2; ++m2) {
            const Frag<T> xa = frag_accrows_sw<Q>(S.sXt[prow], prow, si * 32 + 16 * m2, g2);
            mma(acc[i], xa, S.sM[k0 + si][m2][lane]);
            if constexpr (C::SPLIT) mma(acc[i], xa, S.sMlo[k0 + si][m2][lane]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < OW::NY; ++i) {
        const int tl = OW::tb(wave, i) * 32 + col;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int r = 4 * r4;
          st4(&S.sZ[tl][zpos<T>(tl, pb * 32 + 8 * r4 + 4 * g2)], acc[i][r] * gz[i][r],
              acc[i][r + 1] * gz[i][r + 1], acc[i][r + 2] * gz[i][r + 2], acc[i][r + 3] * gz[i][r + 3]);
        }
      }
      __syncthreads();
    }
  } else {
    // ========================================================== H waves: M^T and state
    const int hw = wave - 4;
    const int pb = hw & 1;
    const int prow = pb * 32 + col;
    const int nb0 = hw >> 1;            // row blocks nb0 and nb0 + 2
    f32x16 hacc[2];
    Frag<T> af[2][C::KS_Q];             // B^T operand frags of the two row blocks
    f32x16 gram[OW::NB];                // Gram tiles of the M^T tiles this wave builds
    const int64_t sbase = ((int64_t)b * H + h) * SN * SP;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = (nb0 + 2 * i) * 32 + acc_row(r, lane);
        hacc[i][r] = h0 ? h0[sbase + n * SP + prow] : 0.f;
      }
    auto fetch_bt = [&](int c) {
      const unsigned char* btf = wsg + (size_t)c * C::REC_BYTES + C::G_BYTES;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < C::KS_Q; ++j)
          af[i][j] = ld_frag<T>(btf + ((size_t)((nb0 + 2 * i) * C::KS_Q + j) * 64 + lane) * C::FB);
    };
    auto fetch_gram = [&](int c) {
      const float* gt = reinterpret_cast<const float*>(wsg + (size_t)c * C::REC_BYTES);
#pragma unroll
      for (int s = 0; s < OW::NB; ++s) {
        const int k = OW::build(hw, s);
        if (k >= 0) gram[s] = load_tile16(gt + (size_t)k * 1024, lane);
      }
    };
    auto write_state = [&]() {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int n = (nb0 + 2 * i) * 32 + 8 * r4 + 4 * g2;
          float v[4], lo[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[k] = hacc[i][4 * r4 + k];
            lo[k] = v[k] - to_f(from_f<T>(v[k]));
          }
          st4(&S.sHt[prow][n], v[0], v[1], v[2], v[3]);
          if constexpr (C::SPLIT) st4(&S.sHtlo[prow][n], lo[0], lo[1], lo[2], lo[3]);
        }
    };
    // M^T tile k = (tb, si) in B-operand order: Gram tile G^T[s][t] times the decay from
    // token s to token t and dt_s, zero above the diagonal, D on the diagonal.
    auto build = [&](int k, const f32x16& gt) {
      const int tb = tile_tb(k), si = k - tb * (tb + 1) / 2;
      const int tl = tb * 32 + col;
      Frag<T> mh[2], ml[2];
      if (si < tb) {
        float mid = 0.f;
#pragma unroll
        for (int kk = 1; kk < NTB - 1; ++kk)
          if (kk > si && kk < tb) mid += ctot[kk];
        const float ut = exp2_hw(mid + sPi[tl]);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 vs = *reinterpret_cast<const f32x4*>(&sV[si * 32 + 8 * r4 + 4 * g2]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * r4 + q;
            split_set<T>(mh[r >> 3], ml[r >> 3], r & 7, gt[r] * (vs[q] * ut));
          }
        }
      } else {
        const float pit = sPi[tl];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int s0 = tb * 32 + 8 * r4 + 4 * g2;
          const f32x4 ps = *reinterpret_cast<const f32x4*>(&sPi[s0]);
          const f32x4 ds = *reinterpret_cast<const f32x4*>(&sDt[s0]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * r4 + q;
            float v = (s0 + q <= tl) ? gt[r] * exp2_hw(pit - ps[q]) * ds[q] : 0.f;
            if (s0 + q == tl) v += Dh;
            split_set<T>(mh[r >> 3], ml[r >> 3], r & 7, v);
          }
        }
      }
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        S.sM[k][m2][lane] = mh[m2];
        if constexpr (C::SPLIT) S.sMlo[k][m2][lane] = ml[m2];
      }
    };
    write_state();
    if (nC > 0) load_chunk(0);
    for (int c = 0; c < nC; ++c) {
      fetch_gram(c);
      stage(c);
      __syncthreads();
      // ---- S2: the chunk's M^T tiles
#pragma unroll
      for (int s = 0; s < OW::NB; ++s) {
        const int k = OW::build(hw, s);
        if (k >= 0) build(k, gram[s]);
      }
      fetch_bt(c);
      __syncthreads();
      // ---- S3: state update, then publish it for the next chunk
      float lam = 0.f;
#pragma unroll
      for (int k = 0; k < NTB; ++k) lam += ctot[k];
      const float eend = exp2_hw(lam);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[i][r] *= eend;
#pragma unroll
      for (int j = 0; j < C::KS_Q; ++j) {
        const int k0 = xsw<Q>(prow, 16 * j + 8 * g2);
        const Frag<T> bh = frag_contig(&S.sXW[prow][k0], 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) mma(hacc[i], af[i][j], bh);
        if constexpr (C::SPLIT) {
          const Frag<T> bl = frag_contig(&S.sXWlo[prow][k0], 0);
#pragma unroll
          for (int i = 0; i < 2; ++i) mma(hacc[i], af[i][j], bl);
        }
      }
      write_state();
      __syncthreads();
    }
    if (h_final) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = (nb0 + 2 * i) * 32 + acc_row(r, lane);
          h_final[sbase + n * SP + prow] = hacc[i][r];
        }
    }
  }

  // y of the last chunk out of sZ
  if (nC > 0) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      int s_, cv;
      xcoord(i, s_, cv);
      flush_y(nC, s_, cv);
    }
  }
}

// ---------------------------------------------------------------------------- pipelined scan, chunk 64
// bf16 io, chunk 64, 16 waves. One barrier per chunk. In iteration c:
//   Y waves 0..3:   chunk c's outputs, Y^T tile (token block y >> 1, p-block y & 1):
//                   H^T C^T scaled by exp2(lambda_t), plus X^T M^T, gated, into sZ.
//   H waves 4..7:   the state to H_c (H wave w: state rows 32 w .. 32 w + 31, both p-blocks),
//                   published into the other half of a double-buffered H^T.
//   helper waves 8..15: chunk c+1's staging (flush of y(c-1), z, x^T, (w x)^T hi/lo), its
//                   masked decay tiles M^T (the diagonal ones in halves by helper waves 0..3,
//                   the other in quarters by helper waves 4..7), the dt / pi / v record of
//                   chunk c+2, and the loads for the chunks after.
// Everything chunk c+1 needs goes to the other half of double-buffered LDS tiles, so the
// barrier that ends the iteration is the only synchronisation; records are staged two chunks
// ahead (three buffers). Four waves per SIMD (one of each kind plus two helpers) hide each
// other's latencies. LDS tiles are unpadded, with XOR swizzles that keep the 16-byte MFMA
// operand reads of H^T and (w x)^T (32 rows per instruction) free of bank conflicts.
constexpr int P64 = 64;
constexpr int P64_THREADS = 1024;
__device__ __forceinline__ int xs64(int p, int s) { return s ^ (8 * ((p ^ (p >> 2)) & 7)); }
__device__ __forceinline__ int hsw(int p, int n) { return n ^ (8 * (p & 15)); }

struct Pipe64Smem {
  bf16 sXt[2][SP][P64];                     // x^T by chunk parity (xs64)
  bf16 sXW[2][SP][P64];                     // (w x)^T hi (xs64)
  bf16 sXWlo[2][SP][P64];                   //         lo
  bf16 sZ[2][P64][SP];                      // z, then y (zpos)
  Frag<bf16> sM[2][3][2][64];               // M^T tiles [parity][tile][k step][lane]
  Frag<bf16> sMlo[2][3][2][64];
  bf16 sHt[2][SP][SN];                      // H^T hi by chunk parity (hsw)
  bf16 sHtlo[2][SP][SN];                    //     lo
  float sRec[3][3 * P64];                   // dt | pi | v, chunk c in slot c % 3
  int4 sInfo[5];                            // packed batch: chunk info, chunk c in slot c % 5
};

// With CONV, x is the raw xBC tensor (x_stride its row stride): the helper waves apply the
// conv to the head's x channels as they stage them, and at the end write the new conv
// history of those channels (and, in the first head of each group, of the group's B and C).
// With VARLEN (CONV only) workgroup (k, h) runs head h over the k-th of K ranges of
// consecutive sequences of a packed batch (ranges balanced by chunk count): it walks their
// chunks as one stream, whose records are contiguous in the workspace. Where a sequence
// ends the H waves store its state to its pool entry and take up the next sequence's
// initial state, which they publish in place of the carried one; the helper waves take
// each chunk's rows from the per-chunk info and, at a sequence start, the conv history
// from the pool. The new conv histories are written at the end.
template <bool CONV, bool VARLEN = false>
__global__ __launch_bounds__(P64_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4)))
void ssd_scan64_kernel(const bf16* __restrict__ x, int64_t x_stride, const float* __restrict__ D,
                       const bf16* __restrict__ z, int64_t z_stride, const float* h0, float* h_final,
                       bf16* __restrict__ y, int64_t y_stride, const unsigned char* __restrict__ ws,
                       int Lrows, int H, int G, ConvArgs cv, VarlenDev vd) {
  static_assert(!VARLEN || CONV, "the packed batch runs with the conv fused");
  using T = bf16;
  using C = Cfg<T, P64>;
  constexpr int Q = P64;
  extern __shared__ __align__(16) unsigned char scan_smem[];
  Pipe64Smem& S = *reinterpret_cast<Pipe64Smem*>(scan_smem);

  const int id = xcd_local_order(blockIdx.x, gridDim.x);
  const int b = id / H, h = id % H;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g2 = lane >> 5;

  // the workgroup's sequence: its L rows from row0, its records, its initial and final state
  // (h0b / hfb: the head's N x P block, or none) and its conv history (read / written).
  // VARLEN: sequences s_begin .. s_end, chunks gc0 + (0 .. nC) with info cinfo[0 .. nC].
  int L;
  int64_t row0;
  [[maybe_unused]] int s_begin = 0, s_end = 0, gc0 = 0;
  [[maybe_unused]] const int4* cinfo = nullptr;
  const unsigned char* wsg;
  const float* hrec;
  const float* h0b;
  float* hfb;
  const T* hist_rd = nullptr;
  T* hist_wr = nullptr;
  if constexpr (VARLEN) {
    const int TC = vd.cc[vd.nseq];
    // first sequence of range kk: the first i with cc[i] >= ceil(kk TC / K)
    auto split = [&](int kk) -> int {
      if (kk <= 0) return 0;
      if (kk >= vd.K) return vd.nseq;
      const int target = (int)(((int64_t)kk * TC + vd.K - 1) / vd.K);
      int lo = 0, hi = vd.nseq;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (vd.cc[mid] < target) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    s_begin = split(b);
    s_end = split(b + 1);
    gc0 = vd.cc[s_begin];
    L = (vd.cc[s_end] - gc0) * Q;   // the stream's chunks, as rows
    row0 = 0;
    cinfo = vd.info + gc0;
    wsg = ws + ((size_t)g * vd.maxC + gc0) * C::REC_BYTES;
    hrec = reinterpret_cast<const float*>(ws + (size_t)G * vd.maxC * C::REC_BYTES +
                                          ((size_t)h * vd.maxC + gc0) * C::HREC_BYTES);
    h0b = nullptr;                  // the initial state of the stream's first sequence
    hfb = nullptr;                  // states are stored per sequence
    if (L > 0) {
      const int4 c0 = cinfo[0];
      if (c0.y & INFO_INIT) h0b = vd.ssm_pool + ((size_t)c0.w * H + h) * SN * SP;
    }
  } else {
    L = Lrows;
    row0 = (int64_t)b * L;
    const int nCw = (L + Q - 1) / Q;
    wsg = ws + (size_t)(b * G + g) * nCw * C::REC_BYTES;
    hrec = reinterpret_cast<const float*>(ws + (size_t)G * nCw * C::REC_BYTES * (size_t)(gridDim.x / H) +
                                          ((size_t)b * H + h) * nCw * C::HREC_BYTES);
    const int64_t sbase = ((int64_t)b * H + h) * SN * SP;
    h0b = h0 ? h0 + sbase : nullptr;
    hfb = h_final ? h_final + sbase : nullptr;
    if (CONV && cv.state) {
      hist_wr = static_cast<T*>(cv.state) + (int64_t)b * 3 * cv.Cc;
      hist_rd = hist_wr;
    }
  }
  const int nC = (L + Q - 1) / Q;
  // block totals of chunk c (pi at the ends of its two 32-token blocks), from LDS
  auto tot_of = [&](int c, int k) { return S.sRec[c % 3][Q + 32 * k + 31]; };
  // packed batch: the info of chunk c, from the workspace (prologue, epilogue) or from the LDS
  // ring, which holds chunks c - 1 .. c + 2 during iteration c (a global read in the loop would
  // be a scalar load, and a pending scalar load makes every LDS wait a full drain)
  [[maybe_unused]] auto info_at = [&](int c, bool ring) -> int4 { return ring ? S.sInfo[c % 5] : cinfo[c]; };

  if (wave < 4) {
    // ========================================================== Y waves
    const int tb = wave >> 1, pb = wave & 1;
    const int prow = pb * 32 + col, tl = tb * 32 + col;
    Frag<T> cf[C::KS_N];
    auto fetch_c = [&](int c) {
      const unsigned char* cfp = wsg + (size_t)c * C::REC_BYTES + C::G_BYTES + C::BT_BYTES;
#pragma unroll
      for (int j = 0; j < C::KS_N; ++j)
        cf[j] = ld_frag<T>(cfp + ((size_t)(tb * C::KS_N + j) * 64 + lane) * C::FB);
    };
    if (nC > 0) fetch_c(0);
    __syncthreads();
    __syncthreads();
    for (int c = 0; c < nC; ++c) {
      const int cur = c & 1, prv = cur ^ 1;
      // ---- carried state, scaled by exp2(lambda_t)
      f32x16 acc = {};
      {
        // four k steps of H^T hi / lo in flight
        Frag<T> ha[4], la[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = hsw(prow, 16 * j + 8 * g2);
          ha[j] = frag_contig(&S.sHt[prv][prow][n], 0);
          la[j] = frag_contig(&S.sHtlo[prv][prow][n], 0);
        }
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j) {
          mma(acc, ha[j & 3], cf[j]);
          mma(acc, la[j & 3], cf[j]);
          if (j + 4 < C::KS_N) {
            const int n = hsw(prow, 16 * (j + 4) + 8 * g2);
            ha[j & 3] = frag_contig(&S.sHt[prv][prow][n], 0);
            la[j & 3] = frag_contig(&S.sHtlo[prv][prow][n], 0);
          }
        }
      }
      const float et = exp2_hw((tb ? tot_of(c, 0) : 0.f) + S.sRec[c % 3][Q + tl]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] *= et;
      fetch_c(min(c + 1, nC - 1));
      // z of this wave's outputs, read ahead of the intra-chunk MFMAs
      Raw4<T> zz[4];
      if (z) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) zz[r4] = ld4(&S.sZ[cur][tl][zpos<T>(tl, pb * 32 + 8 * r4 + 4 * g2)]);
      }
      // ---- intra-chunk part: Y^T += X^T M^T over source blocks si <= tb
#pragma unroll
      for (int si = 0; si < 2; ++si) {
        if (si <= tb) {
          const int k = tb * (tb + 1) / 2 + si;
#pragma unroll
          for (int m2 = 0; m2 < 2; ++m2) {
            const int sa = si * 32 + 16 * m2 + 4 * g2;
            const Frag<T> xa = frag_accrows2(&S.sXt[cur][prow][xs64(prow, sa)],
                                             &S.sXt[cur][prow][xs64(prow, sa + 8)]);
            mma(acc, xa, S.sM[cur][k][m2][lane]);
            mma(acc, xa, S.sMlo[cur][k][m2][lane]);
          }
        }
      }
      // ---- gate and y into sZ[cur] (in place of z)
      if (z) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int r = 4 * r4;
          st4(&S.sZ[cur][tl][zpos<T>(tl, pb * 32 + 8 * r4 + 4 * g2)], acc[r] * silu_fast(zz[r4].get(0)),
              acc[r + 1] * silu_fast(zz[r4].get(1)), acc[r + 2] * silu_fast(zz[r4].get(2)),
              acc[r + 3] * silu_fast(zz[r4].get(3)));
        }
      } else {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int r = 4 * r4;
          st4(&S.sZ[cur][tl][zpos<T>(tl, pb * 32 + 8 * r4 + 4 * g2)], acc[r], acc[r + 1], acc[r + 2],
              acc[r + 3]);
        }
      }
      __syncthreads();
    }
  } else if (wave < 8) {
    // ========================================================== H waves
    // H wave hw owns state rows n = 32 hw .. 32 hw + 31 for both p-blocks, so that no two waves
    // load the same B^T fragments
    const int hw = wave - 4;
    f32x16 hacc[2];                     // [p-block]
    Frag<T> af[C::KS_Q];
    // the head's N x P state block <-> this wave's rows of the accumulators
    auto load_state = [&](const float* src) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = hw * 32 + acc_row(r, lane);
          hacc[i][r] = src ? src[n * SP + i * 32 + col] : 0.f;
        }
    };
    [[maybe_unused]] auto store_state = [&](float* dst) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = hw * 32 + acc_row(r, lane);
          dst[n * SP + i * 32 + col] = hacc[i][r];
        }
    };
    load_state(h0b);
    auto fetch_bt = [&](int c) {
      const unsigned char* btf = wsg + (size_t)c * C::REC_BYTES + C::G_BYTES;
#pragma unroll
      for (int j = 0; j < C::KS_Q; ++j)
        af[j] = ld_frag<T>(btf + ((size_t)(hw * C::KS_Q + j) * 64 + lane) * C::FB);
    };
    auto publish = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int prow = i * 32 + col;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int n = hsw(prow, hw * 32 + 8 * r4 + 4 * g2);
          const Split2 a = split2(hacc[i][4 * r4], hacc[i][4 * r4 + 1]);
          const Split2 d = split2(hacc[i][4 * r4 + 2], hacc[i][4 * r4 + 3]);
          *reinterpret_cast<uint2*>(&S.sHt[buf][prow][n]) = make_uint2(a.hi, d.hi);
          *reinterpret_cast<uint2*>(&S.sHtlo[buf][prow][n]) = make_uint2(a.lo, d.lo);
        }
      }
    };
    publish(1);          // h0 is the state chunk 0 reads
    if (nC > 0) fetch_bt(0);
    __syncthreads();
    __syncthreads();
    for (int c = 0; c < nC; ++c) {
      const int cur = c & 1;
      // ---- state update to H_c, published into sHt[cur]
      const float eend = exp2_hw(tot_of(c, 0) + tot_of(c, 1));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[i][r] *= eend;
#pragma unroll
      for (int j = 0; j < C::KS_Q; ++j) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int prow = i * 32 + col;
          const int k0 = xs64(prow, 16 * j + 8 * g2);
          mma(hacc[i], af[j], frag_contig(&S.sXW[cur][prow][k0], 0));
          mma(hacc[i], af[j], frag_contig(&S.sXWlo[cur][prow][k0], 0));
        }
      }
      if constexpr (VARLEN) {
        // the next chunk starts a sequence: store this sequence's state in its entry, then take
        // up the next one's initial state (zeros without one), which is published below
        if (c + 1 < nC) {
          const int4 cn = info_at(c + 1, true);
          if (cn.y & INFO_FIRST) {
            const int so = info_at(c, true).w;
            if (so >= 0) store_state(vd.ssm_pool + ((size_t)so * H + h) * SN * SP);
            load_state(cn.y & INFO_INIT ? vd.ssm_pool + ((size_t)cn.w * H + h) * SN * SP : nullptr);
          }
        }
      }
      publish(cur);
      fetch_bt(min(c + 1, nC - 1));
      __syncthreads();
    }
    if constexpr (VARLEN) {
      if (nC > 0) {
        const int so = cinfo[nC - 1].w;
        if (so >= 0) store_state(vd.ssm_pool + ((size_t)so * H + h) * SN * SP);
      }
      // an empty sequence without an initial state leaves a zero state in its entry
      for (int i = s_begin; i < s_end; ++i) {
        const int sl = vd.slot(i);
        if (vd.cu[i + 1] == vd.cu[i] && sl >= 0 && !vd.init(i)) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              vd.ssm_pool[((size_t)sl * H + h) * SN * SP + (hw * 32 + acc_row(r, lane)) * SP + ii * 32 + col] = 0.f;
        }
      }
    }
    if (hfb) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = hw * 32 + acc_row(r, lane);
          hfb[n * SP + i * 32 + col] = hacc[i][r];
        }
    }
  } else {
    // ========================================================== helper waves
    // With the conv, the helpers issue ahead of the Y and H waves that share their SIMDs:
    // their chain (loads, the x conv, the tiles of chunk c+1) is then the longest of a chunk,
    // and at equal priority the arbiter often picked the other roles first and the helpers
    // finished last. At 12B 8k the one-call step goes from 320 to 291 us. Raising the H waves
    // instead made it slower (339 us), the Y waves' priority made no difference, and without
    // the conv the same priority slows the scan (240 to 260 us).
    if constexpr (CONV) __builtin_amdgcn_s_setprio(1);
    const int htid = tid - 512, hv = wave - 8;
    const T* xb = x + h * SP;
    const T* zb = z ? z + h * SP : xb;   // without z, x is loaded in its place and not used
    T* yb = y + h * SP;
    const float Dh = D ? D[h] : 0.f;
    // thread: token pair (s0, s0 + 1) = 2 (htid / 16), columns p0 .. p0 + 3 = 4 (htid % 16)
    const int s0 = 2 * (htid >> 4), p0 = 4 * (htid & 15);
    // conv of channels h SP + p0 .. + 3: taps, bias and the history of the sequence start
    f32x4 cw[4];
    float cb[4];
    const T* hist = nullptr;
    if constexpr (CONV) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cw[e] = *reinterpret_cast<const f32x4*>(cv.w + (int64_t)(h * SP + p0 + e) * 4);
        cb[e] = cv.bias ? cv.bias[h * SP + p0 + e] : 0.f;
      }
      if (hist_rd) hist = hist_rd + h * SP + p0;
    }
    // per-thread element offsets inside a chunk's rows fit 32 bits; chunk bases are uniform
    const uint32_t xs = (uint32_t)x_stride, zs = (uint32_t)z_stride, ys = (uint32_t)y_stride;
    // M^T tiles: helper waves 0, 1 build tile 0 (diagonal 0) in halves (k steps hm of 16
    // source tokens), waves 2, 3 tile 2 (diagonal 1); waves 4..7 build tile 1 (block 1 from
    // block 0, no exponentials) in quarters of 8 source tokens. Helper wave v runs on SIMD
    // v % 4, so every SIMD gets half a diagonal tile and a quarter of the other. Waves 0..2
    // also carry the dt / pi / v records (3Q words, a word a thread).
    const int kb = hv < 2 ? 0 : hv < 4 ? 2 : 1;
    const int hm = hv & 1, hq = hv & 3;
    // Each role (records or not, tiles or not) runs its own copy of the loop, so that every
    // copy issues a fixed sequence of memory operations and the compiler's count of
    // outstanding loads stays exact: a merged count would wait for loads just issued.
    auto helpers = [&](auto part_tag, auto rec_tag, auto duty_tag) {
      constexpr int PART = decltype(part_tag)::value;   // 2: a diagonal half, 4: an off quarter
      constexpr bool REC = decltype(rec_tag)::value;
      // VARLEN duties: HIST, helper wave 0 (whose threads hold the first tokens of a chunk),
      // loads each chunk's conv history rows; RING, helper wave 4, keeps the info ring
      constexpr bool HIST = VARLEN && decltype(duty_tag)::value == 1;
      constexpr bool RING = VARLEN && decltype(duty_tag)::value == 2;
      // x rows of the thread's tokens; with the conv, raw rows s0 - 3 .. s0 + 1
      constexpr int NX = CONV ? 5 : 2;
      Raw4<T> rX[NX], rZ[2];
      float rRec = 0.f;
      f32x4 gram[2];                     // Gram tile registers 8 hm .. 8 hm + 7 (4 hq .. 4 hq + 3)
      // the history rows before the sequence that this thread's first tokens read (zeros
      // without a history): for one sequence loaded once in the prologue, for a packed batch
      // by the HIST role with each chunk's rows, from the chunk's place in the history area
      Raw4<T> rH[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) rH[k].v = (bf16x4){};
      // VARLEN: ci is the info of chunk c (from the workspace in the prologue, from the ring in
      // the loop, read at the top of the iteration)
      auto load_set = [&](int c, int4 ci) {   // x and z of this thread's tokens
        // chunk c: its first row, its valid rows and whether a sequence starts there
        int64_t r0;
        int nval;
        bool first;
        if constexpr (VARLEN) {
          r0 = ci.x;
          nval = ci.y & 255;
          first = (ci.y & INFO_FIRST) != 0;
        } else {
          r0 = row0 + (int64_t)c * Q;
          nval = L - c * Q;
          first = c == 0;
        }
        const T* xc = xb + r0 * x_stride;
        const T* zc = zb + r0 * z_stride;
        // Rows past the end of the sequence load the last row instead (finite values; their
        // dt and v are zero, so they add nothing), which keeps the loads unconditional.
        const int lim = nval - 1;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t s = (uint32_t)min(s0 + k, lim);
          if constexpr (!CONV) rX[k] = ld4(xc + (s * xs + p0));
          rZ[k] = ld4(zc + (s * zs + p0));
        }
        if constexpr (CONV) {
          // raw rows s0 - 3 .. s0 + 1 of the chunk, addressed from a base 3 rows back; past the
          // end the last row is read, and in the first chunk the rows before the sequence are
          // read as row 0 and replaced when that chunk is staged
          const T* xh = xc - 3 * x_stride;
          const int lo = first ? 3 : 0;
#pragma unroll
          for (int k = 0; k < NX; ++k) {
            const uint32_t s = (uint32_t)min(max(s0 + k, lo), lim + 3);
            rX[k] = ld4(xh + (s * xs + p0));
          }
          if constexpr (HIST) {
            // every chunk issues the same 3 loads (used only where a sequence starts)
            const T* hp = vd.hist + (size_t)(gc0 + c) * 3 * (H * SP) + h * SP + p0;
#pragma unroll
            for (int k = 0; k < 3; ++k) rH[k] = ld4(hp + min(s0 + k, 2) * (H * SP));
          }
        }
      };
      auto load_rec = [&](int c) {
        if constexpr (REC) rRec = hrec[(size_t)c * (3 * Q) + htid];
      };
      auto put_rec = [&](int c) {
        if constexpr (REC) S.sRec[c % 3][htid] = rRec;
      };
      auto flush_y = [&](int c, bool full, int4 cf) {   // y of chunk c out of sZ[c & 1]
        int64_t r0;
        int nval;
        if constexpr (VARLEN) {
          r0 = cf.x;
          nval = cf.y & 255;
        } else {
          r0 = row0 + (int64_t)c * Q;
          nval = L - c * Q;
        }
        T* yc = yb + r0 * y_stride;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int s = s0 + k;
          const Raw4<T> v = ld4(&S.sZ[c & 1][s][zpos<T>(s, p0)]);
          if (full || s < nval) *reinterpret_cast<bf16x4*>(yc + ((uint32_t)s * ys + p0)) = v.v;
        }
      };
      auto load_hist = [&]() {   // one sequence: the history rows, once
        if constexpr (CONV && !VARLEN) {
#pragma unroll
          for (int k = 0; k < 3; ++k)
            if (hist && s0 + k < 3) rH[k] = ld4(hist + (s0 + k) * cv.Cc);
        }
      };
      // x^T, (w x)^T and z of chunk c (its set in registers) into buffers c & 1; FIRST: chunk 0
      auto stage = [&](int c, auto first_tag, int4 cs) {
        // one sequence: FIRST marks chunk 0 (the prologue's call); a packed batch: the chunk's
        // info cs says whether a sequence starts there
        bool first = decltype(first_tag)::value;
        if constexpr (VARLEN) first = (cs.y & INFO_FIRST) != 0;
        const int buf = c & 1;
        if (z) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
            *reinterpret_cast<bf16x4*>(&S.sZ[buf][s0 + k][zpos<T>(s0 + k, p0)]) = rZ[k].v;
        }
        // w_s = v_s exp2(decay from the end of s's block to the chunk end): block 0 -> tot_1
        const float* rec = S.sRec[c % 3];
        const float2 vs = *reinterpret_cast<const float2*>(&rec[2 * Q + s0]);
        const float wb = s0 < 32 ? exp2_hw(rec[Q + 63]) : 1.f;
        const float w0 = vs.x * wb, w1 = vs.y * wb;
        T xv[2][4];
        if constexpr (CONV) {
          Raw4<T> r[NX];
#pragma unroll
          for (int k = 0; k < NX; ++k) r[k] = rX[k];
          if (first) {
#pragma unroll
            for (int k = 0; k < 3; ++k)
              if (s0 - 3 + k < 0) r[k] = rH[k];   // rH[k] holds history row s0 + k
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int k = 0; k < 2; ++k)
              xv[k][e] = (T)conv4_silu(cw[e], cb[e], r[k].get(e), r[k + 1].get(e), r[k + 2].get(e),
                                       r[k + 3].get(e));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[0][e] = rX[0].v[e];
            xv[1][e] = rX[1].v[e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const T x0 = xv[0][e], x1 = xv[1][e];
          const Split2 v = split2(to_f(x0) * w0, to_f(x1) * w1);
          const int p = p0 + e, sw = xs64(p, s0);
          st_pair(&S.sXt[buf][p][sw], x0, x1);
          *reinterpret_cast<uint32_t*>(&S.sXW[buf][p][sw]) = v.hi;
          *reinterpret_cast<uint32_t*>(&S.sXWlo[buf][p][sw]) = v.lo;
        }
      };
      auto fetch_gram = [&](int c) {   // quads 2 hm, 2 hm + 1 (or quad hq) of the stored tile
        const float* tile = reinterpret_cast<const float*>(wsg + (size_t)c * C::REC_BYTES) +
                            (size_t)kb * 1024 + 4 * lane;
        if constexpr (PART == 2) {
          gram[0] = *reinterpret_cast<const f32x4*>(tile + 512 * hm);
          gram[1] = *reinterpret_cast<const f32x4*>(tile + 512 * hm + 256);
        } else {
          gram[0] = *reinterpret_cast<const f32x4*>(tile + 256 * hq);
        }
      };
      // half hm of tile kb of chunk c into sM[c & 1]: Gram tile times the decay from s to t
      // and dt_s, zero above the diagonal, D on the diagonal. Register 4 j + q of the half is
      // source token 16 hm + 8 j + 4 g2 + q of the tile's source block.
      auto build = [&](int c) {
        if constexpr (PART == 4) {
          // quarter hq of tile 1 (block 1 from block 0): v_s exp2(pi_t); registers 4 hq + q
          // are source tokens 8 hq + 4 g2 + q, elements 4 (hq & 1) + q of k step hq >> 1
          const float* rec = S.sRec[c % 3];
          const float ut = exp2_hw(rec[Q + 32 + col]);
          const f32x4 vq = *reinterpret_cast<const f32x4*>(&rec[2 * Q + 8 * hq + 4 * g2]);
          const Split2 a = split2(gram[0][0] * (vq[0] * ut), gram[0][1] * (vq[1] * ut));
          const Split2 d = split2(gram[0][2] * (vq[2] * ut), gram[0][3] * (vq[3] * ut));
          *reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(&S.sM[c & 1][1][hq >> 1][lane]) +
                                    8 * (hq & 1)) = make_uint2(a.hi, d.hi);
          *reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(&S.sMlo[c & 1][1][hq >> 1][lane]) +
                                    8 * (hq & 1)) = make_uint2(a.lo, d.lo);
        } else {
          const float* rec = S.sRec[c % 3];
          const float* sDt = rec;
          const float* sPi = rec + Q;
          // half hm of a diagonal tile (token block tb onto itself)
          const int tb = kb == 0 ? 0 : 1;
          const int tl = tb * 32 + col;
          float mv[8];
          const float pit = sPi[tl];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int sr = tb * 32 + 16 * hm + 8 * j + 4 * g2;
            const f32x4 ps = *reinterpret_cast<const f32x4*>(&sPi[sr]);
            const f32x4 ds = *reinterpret_cast<const f32x4*>(&sDt[sr]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v = (sr + q <= tl) ? gram[j][q] * exp2_hw(pit - ps[q]) * ds[q] : 0.f;
              if (sr + q == tl) v += Dh;
              mv[4 * j + q] = v;
            }
          }
          Frag<T> mh, ml;
          frag_split(mv, mh, ml);
          S.sM[c & 1][kb][hm][lane] = mh;
          S.sMlo[c & 1][kb][hm][lane] = ml;
        }
      };
      // prologue: records 0 and 1 into LDS; then chunk 0 staged and its tiles built, chunk 1's
      // set in flight
      // packed batch: the HIST role keeps the info ring: chunks 0 .. 2 now, chunk c + 3 in
      // iteration c (requested one iteration earlier). Lane l moves word l % 4 of the info:
      // the per-lane address makes it a vector load (a scalar load in the loop would turn the
      // LDS waits into full drains), and every lane of the wave takes part, so the role's
      // memory operations stay unconditional
      [[maybe_unused]] int rInfo = 0;
      [[maybe_unused]] auto info_word = [&](int c) {
        return reinterpret_cast<const int*>(cinfo + min(c, nC - 1))[lane & 3];
      };
      if constexpr (RING) {
        if (nC > 0) {
#pragma unroll
          for (int k = 0; k < 3; ++k) reinterpret_cast<int*>(&S.sInfo[k])[lane & 3] = info_word(k);
          rInfo = info_word(3);
        }
      }
      // prologue info from the workspace (the ring is filled at the first barrier)
      [[maybe_unused]] const int4 ci0 = VARLEN && nC > 0 ? cinfo[0] : int4{};
      [[maybe_unused]] const int4 ci1 = VARLEN && nC > 0 ? cinfo[min(1, nC - 1)] : int4{};
      if (nC > 0) {
        load_hist();
        load_set(0, ci0);
        load_rec(0);
        put_rec(0);
        load_rec(min(1, nC - 1));
        put_rec(1);
        fetch_gram(0);
        load_rec(min(2, nC - 1));
      }
      __syncthreads();
      if (nC > 0) {
        stage(0, std::true_type{}, ci0);
        load_set(min(1, nC - 1), ci1);
        build(0);
        fetch_gram(min(1, nC - 1));
      }
      __syncthreads();
      for (int c = 0; c < nC; ++c) {
        // packed batch: the infos this iteration uses (chunks c - 1, c + 1, c + 2), read from
        // the ring now so that their latency hides behind the tile build
        int4 im1 = {}, ip1 = {}, ip2 = {};
        if constexpr (VARLEN) {
          im1 = S.sInfo[(c + 4) % 5];
          ip1 = S.sInfo[min(c + 1, nC - 1) % 5];
          ip2 = S.sInfo[min(c + 2, nC - 1) % 5];
        }
        // ---- chunk c + 1: tiles and staging. Chunk indices are clamped, so every iteration
        // issues the same memory operations (the last stages a copy nobody reads).
        build(c + 1);
        fetch_gram(min(c + 2, nC - 1));
        if (c >= 1) flush_y(c - 1, !VARLEN, im1);   // one sequence: chunk c - 1 < nC - 1 is full
        stage(c + 1, std::false_type{}, ip1);
        put_rec(c + 2);
        load_set(min(c + 2, nC - 1), ip2);
        load_rec(min(c + 3, nC - 1));
        if constexpr (RING) {
          reinterpret_cast<int*>(&S.sInfo[(c + 3) % 5])[lane & 3] = rInfo;
          rInfo = info_word(c + 4);
        }
        __syncthreads();
      }
      if (nC > 0) flush_y(nC - 1, false, VARLEN ? S.sInfo[(nC - 1) % 5] : int4{});   // y of the last chunk
      if constexpr (CONV) {
        // the new history: the last 3 raw inputs of (history, sequence). One thread per 4
        // channels reads all 3 before writing any, so an in-place shift (L < 3) is safe; every
        // read of the old history (the staging of chunk 0 here, the prep kernel for B and C)
        // is complete by now.
        const int hpg = H / G;
        int ch = -1;
        if (htid < 16) ch = h * SP + p0;   // the head's x channels
        else if (htid < 80 && h % hpg == 0) {
          const int q = htid - 16;         // the group's B (q < 32) and C channels
          ch = H * SP + (q < 32 ? 0 : G * SN) + g * SN + 4 * (q & 31);
        }
        if constexpr (VARLEN) {
          // every sequence of the workgroup's range that has an entry
          for (int i = s_begin; ch >= 0 && i < s_end; ++i) {
            const int sl = vd.slot(i);
            if (sl < 0) continue;
            T* hs = vd.conv_pool + (int64_t)sl * 3 * cv.Cc + ch;
            const bool init = vd.init(i);
            const int64_t ri = vd.cu[i];
            const int Li = vd.cu[i + 1] - vd.cu[i];
            Raw4<T> f[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
              const int t = Li - 3 + j;
              if (t >= 0) f[j] = ld4(x + (ri + t) * x_stride + ch);
              else if (init) f[j] = ld4(hs + (t + 3) * cv.Cc);
              else f[j].v = (bf16x4){};
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) *reinterpret_cast<bf16x4*>(hs + j * cv.Cc) = f[j].v;
          }
        } else if (hist_wr && ch >= 0) {
          T* hs = hist_wr + ch;
          const T* hr = hist_rd ? hist_rd + ch : nullptr;   // the old history, or zeros
          Raw4<T> f[3];
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const int t = L - 3 + j;
            if (t >= 0) f[j] = ld4(x + (row0 + t) * x_stride + ch);
            else if (hr) f[j] = ld4(hr + (t + 3) * cv.Cc);
            else f[j].v = (bf16x4){};
          }
#pragma unroll
          for (int j = 0; j < 3; ++j) *reinterpret_cast<bf16x4*>(hs + j * cv.Cc) = f[j].v;
        }
      }
    };
    using Half = std::integral_constant<int, 2>;
    using Quarter = std::integral_constant<int, 4>;
    using NoDuty = std::integral_constant<int, 0>;
    using Hist = std::integral_constant<int, 1>;
    using Ring = std::integral_constant<int, 2>;
    if (VARLEN && hv == 0) helpers(Half{}, std::true_type{}, Hist{});
    else if (hv < 3) helpers(Half{}, std::true_type{}, NoDuty{});
    else if (hv < 4) helpers(Half{}, std::false_type{}, NoDuty{});
    else if (VARLEN && hv == 4) helpers(Quarter{}, std::false_type{}, Ring{});
    else helpers(Quarter{}, std::false_type{}, NoDuty{});
  }
}

// ---------------------------------------------------------------------------- host side
// row stride of dt_raw in elements: dense [rows][H] unless the caller gave one
static int64_t dt_stride(const PrefillArgs& a) { return a.dt_stride > 0 ? a.dt_stride : a.H; }

static hipError_t set_lds(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int Q>
static hipError_t launch_tq(const PrefillArgs& a, hipStream_t stream) {
  using C = Cfg<T, Q>;
  const size_t prep_lds = 2 * sizeof(T) * Q * C::LDN;
  constexpr bool WIDE = Q > 128;
  constexpr bool PIPE64 = Q == 64 && sizeof(T) == 2;
  using ScanFn = void (*)(const T*, int64_t, const float*, const T*, int64_t, const float*, float*, T*,
                          int64_t, const unsigned char*, int, int, int);
  size_t scan_lds;
  const void* scan_fn;
  ScanFn scan = nullptr;
  if constexpr (PIPE64) {
    scan_lds = sizeof(Pipe64Smem);
    scan_fn = reinterpret_cast<const void*>(&ssd_scan64_kernel<false>);
  } else {
    if constexpr (WIDE) {
      scan_lds = sizeof(WideSmem<T, Q>);
      scan = &ssd_scan_wide_kernel<T, Q>;
    } else {
      scan_lds = sizeof(ScanSmem<T, Q>);
      scan = &ssd_scan_kernel<T, Q>;
    }
    scan_fn = reinterpret_cast<const void*>(scan);
  }
  static bool configured = false;
  if (!configured) {
    hipError_t e = set_lds(reinterpret_cast<const void*>(&ssd_prep_kernel<T, Q, false>), prep_lds);
    if (e == hipSuccess) e = set_lds(scan_fn, scan_lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int nC = (a.L + Q - 1) / Q;
  if (nC > 0) {
    hipLaunchKernelGGL((ssd_prep_kernel<T, Q, false>), dim3(a.B * a.G * nC), dim3(PREP_THREADS), prep_lds,
                       stream, static_cast<const T*>(a.Bm), a.b_stride, static_cast<const T*>(a.Cm),
                       a.c_stride, static_cast<const T*>(a.dt_raw), a.dt_bias, a.A, dt_stride(a),
                       static_cast<unsigned char*>(a.workspace), a.L, a.H, a.G, nC, ConvArgs{}, VarlenDev{});
  }
  if constexpr (PIPE64) {
    hipLaunchKernelGGL((ssd_scan64_kernel<false>), dim3(a.B * a.H), dim3(P64_THREADS), scan_lds, stream,
                       static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                       a.z_stride, a.h0, a.h_final, static_cast<T*>(a.y), a.y_stride,
                       static_cast<const unsigned char*>(a.workspace), a.L, a.H, a.G, ConvArgs{}, VarlenDev{});
  } else {
    hipLaunchKernelGGL(scan, dim3(a.B * a.H), dim3(SCAN_THREADS), scan_lds, stream,
                       static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                       a.z_stride, a.h0, a.h_final, static_cast<T*>(a.y), a.y_stride,
                       static_cast<const unsigned char*>(a.workspace), a.L, a.H, a.G);
  }
  return hipGetLastError();
}

hipError_t launch_ssd_prefill_conv(const PrefillArgs& a, const ConvArgs& cv, hipStream_t stream) {
  using T = bf16;
  constexpr int Q = P64;
  using C = Cfg<T, Q>;
  const size_t prep_lds = 2 * sizeof(T) * Q * C::LDN;
  static bool configured = false;
  if (!configured) {
    hipError_t e = set_lds(reinterpret_cast<const void*>(&ssd_prep_kernel<T, Q, true>), prep_lds);
    if (e == hipSuccess) e = set_lds(reinterpret_cast<const void*>(&ssd_scan64_kernel<true>), sizeof(Pipe64Smem));
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int nC = (a.L + Q - 1) / Q;
  if (nC > 0) {
    hipLaunchKernelGGL((ssd_prep_kernel<T, Q, true>), dim3(a.B * a.G * nC), dim3(PREP_THREADS), prep_lds,
                       stream, static_cast<const T*>(a.Bm), a.b_stride, static_cast<const T*>(a.Cm),
                       a.c_stride, static_cast<const T*>(a.dt_raw), a.dt_bias, a.A, dt_stride(a),
                       static_cast<unsigned char*>(a.workspace), a.L, a.H, a.G, nC, cv, VarlenDev{});
  }
  hipLaunchKernelGGL((ssd_scan64_kernel<true>), dim3(a.B * a.H), dim3(P64_THREADS), sizeof(Pipe64Smem),
                     stream, static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                     a.z_stride, a.h0, a.h_final, static_cast<T*>(a.y), a.y_stride,
                     static_cast<const unsigned char*>(a.workspace), a.L, a.H, a.G, cv, VarlenDev{});
  return hipGetLastError();
}

// records for up to total / 64 + nseq chunks (the most a packed batch of nseq sequences over
// total rows can have), the per-chunk info, the per-chunk history area, then the sanitized
// offsets and the per-sequence first chunks
static int varlen_max_chunks(int total, int nseq) { return total / P64 + nseq; }

size_t ssd_prefill_varlen_workspace(int total, int nseq, int H, int G) {
  using C = Cfg<bf16, P64>;
  const size_t maxC = (size_t)varlen_max_chunks(total, nseq);
  return maxC * ((size_t)G * C::REC_BYTES + (size_t)H * C::HREC_BYTES + sizeof(int4) +
                 (size_t)3 * H * SP * sizeof(bf16)) +
         2 * ((size_t)nseq + 1) * sizeof(int32_t);
}

// scan workgroups per head: ranges of sequences enough for about two rounds of workgroups on
// the CUs (one workgroup fits a CU), which uses the whole chip while a workgroup's fixed
// start-up and drain stay a small part of its time
static int varlen_ranges(int nseq, int H) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    return n;
  }();
  return max(1, min(nseq, (2 * cus + H / 2) / H));
}

hipError_t launch_ssd_prefill_varlen(const PrefillArgs& a, const ConvArgs& cv, const VarlenArgs& va,
                                     hipStream_t stream) {
  using T = bf16;
  constexpr int Q = P64;
  using C = Cfg<T, Q>;
  const size_t prep_lds = 2 * sizeof(T) * Q * C::LDN;
  static bool configured = false;
  if (!configured) {
    hipError_t e = set_lds(reinterpret_cast<const void*>(&ssd_prep_kernel<T, Q, true, true>), prep_lds);
    if (e == hipSuccess)
      e = set_lds(reinterpret_cast<const void*>(&ssd_scan64_kernel<true, true>), sizeof(Pipe64Smem));
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int maxC = varlen_max_chunks(a.L, va.nseq);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  int4* info = reinterpret_cast<int4*>(ws + (size_t)maxC * ((size_t)a.G * C::REC_BYTES + (size_t)a.H * C::HREC_BYTES));
  bf16* hist = reinterpret_cast<bf16*>(info + maxC);
  int32_t* cu = reinterpret_cast<int32_t*>(hist + (size_t)maxC * 3 * a.H * SP);
  int32_t* cc = cu + va.nseq + 1;
  hipLaunchKernelGGL(varlen_index_kernel, dim3(1), dim3(VIDX_THREADS), 0, stream, va.cu, va.nseq, a.L, cu, cc,
                     info, va.slots, va.has_init, va.npool);
  const int K = varlen_ranges(va.nseq, a.H);
  const VarlenDev vd{cu, cc, info, va.slots, va.has_init, va.ssm_pool, static_cast<bf16*>(va.conv_pool),
                     hist, va.nseq, va.npool, maxC, K};
  hipLaunchKernelGGL((ssd_prep_kernel<T, Q, true, true>), dim3(a.G * maxC), dim3(PREP_THREADS), prep_lds,
                     stream, static_cast<const T*>(a.Bm), a.b_stride, static_cast<const T*>(a.Cm),
                     a.c_stride, static_cast<const T*>(a.dt_raw), a.dt_bias, a.A, dt_stride(a), ws, a.L, a.H, a.G, maxC,
                     cv, vd);
  hipLaunchKernelGGL((ssd_scan64_kernel<true, true>), dim3(K * a.H), dim3(P64_THREADS), sizeof(Pipe64Smem),
                     stream, static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                     a.z_stride, nullptr, nullptr, static_cast<T*>(a.y), a.y_stride, ws, a.L, a.H, a.G, cv, vd);
  return hipGetLastError();
}

template <typename T, int Q>
static size_t ws_bytes(int B, int L, int H, int G) {
  using C = Cfg<T, Q>;
  const size_t nC = ((size_t)L + Q - 1) / Q;
  return nC * ((size_t)B * G * C::REC_BYTES + (size_t)B * H * C::HREC_BYTES);
}

size_t ssd_prefill_workspace(int io_bf16, int chunk, int B, int L, int H, int G) {
  if (io_bf16) {
    if (chunk == 64) return ws_bytes<bf16, 64>(B, L, H, G);
    if (chunk == 128) return ws_bytes<bf16, 128>(B, L, H, G);
    if (chunk == 256) return ws_bytes<bf16, 256>(B, L, H, G);
  } else if (chunk == 64) {
    return ws_bytes<float, 64>(B, L, H, G);
  }
  return 0;
}

hipError_t launch_ssd_prefill(int io_bf16, int chunk, const PrefillArgs& a, hipStream_t stream) {
  if (io_bf16) {
    if (chunk == 64) return launch_tq<bf16, 64>(a, stream);
    if (chunk == 128) return launch_tq<bf16, 128>(a, stream);
    if (chunk == 256) return launch_tq<bf16, 256>(a, stream);
  } else if (chunk == 64) {
    return launch_tq<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace m2

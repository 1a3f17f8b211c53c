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
//    instruction; these are shared by all heads of the group.
//  * ssd_scan64, one workgroup of 16 waves per (b, h), described at its definition. The fp32
//    state stays on chip for the whole sequence. One of its waves forms each chunk's per-token
//    records from dt_raw: dt = softplus(dt_raw + dt_bias), the inclusive prefix pi of
//    dt*A*log2(e) inside 32-token blocks, and v_s = exp2(pi_end - pi_s) dt_s (decay from
//    token s to the end of its block, times dt_s). The prefix is summed in fp64 and kept as
//    an fp32 pair pi = pi_hi + pi_lo: after a token whose decay is very strong the prefix
//    values of a block are large, and the decay between two later tokens, a difference of
//    two of them, would otherwise carry the rounding of their size rather than of its own.
//
// The chunk length a call names (64, 128 or 256) is a tiling choice: the result does not
// depend on it up to rounding, and both kernels always tile at 64 tokens.
//
// Decay factors are formed in log2 units from prefix sums taken inside 32-token blocks, so
// no factor is the difference of two large prefix sums: inside a block exp2(pi_t - pi_s);
// across the two blocks of a chunk the factor splits into a per-source part v_s and a
// per-target part exp2(pi_t), both <= 1, so the off-diagonal tile needs no exponential per
// element. D is added to the diagonal of M, so the skip term D x_t comes out of the same
// MFMAs.
//
// Precision: x, B, C, z and dt enter exactly (bf16 inputs). The three computed MFMA
// operands -- M, the state H and the decay-weighted x -- are passed as hi + lo bf16 pairs
// (hi = bf16(v), lo = bf16(v - hi)), i.e. two MFMAs each, which keeps them to ~2^-16
// relative. With a single bf16 rounding the error of outputs dominated by one term reaches
// 4e-2 to 2e-1 of rms(y) on these heavy-tailed outputs, outside the 2e-2 bar; with the
// split it stays below 1e-4. The fp32 io mode uses fp32 MFMAs and needs no split.
#include <mutex>
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace m2 {

// dt inputs of the scan: dt_raw [rows][stride] (head h at column h), dt_bias [H], A [H]
template <typename T>
struct DtDev {
  const T* raw;
  int64_t stride;
  const float* bias;
  const float* A;
};

constexpr int SP = 64;   // head dim
constexpr int SN = 128;  // state dim
constexpr int PREP_THREADS = 256;

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
  static constexpr size_t FB = sizeof(Frag<T>);
  // workspace record per (b, g, chunk): Gram tiles | B^T operand frags | C operand frags
  static constexpr size_t G_BYTES = (size_t)NTILES * 64 * 16 * sizeof(float);
  static constexpr size_t BT_BYTES = (size_t)(SN / 32) * KS_Q * 64 * FB;
  static constexpr size_t CF_BYTES = (size_t)NTB * KS_N * 64 * FB;
  static constexpr size_t REC_BYTES = G_BYTES + BT_BYTES + CF_BYTES;
};

__device__ __forceinline__ int tile_tb(int k) {  // column block of lower-triangle tile k < 36
  int tb = 0;
#pragma unroll
  for (int t = 1; t < 8; ++t) tb += k >= t * (t + 1) / 2;
  return tb;
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
    unsigned char* __restrict__ ws, int L, int H, int G, int nC, ConvArgs cv, VarlenDev vd) {
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

  // The B and C rows are requested first, then go to LDS (zero past the end of the sequence).
  constexpr int NR = CONV ? 11 : Q * SN / VE / PREP_THREADS;   // 16-byte row vectors per thread
  constexpr bool HOLD = CONV;   // rows held in registers for the conv
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
  // Gram tiles, stored as [q][lane][4]: accumulator registers 4q .. 4q+3 of every lane, so
  // that each of the reader's four 16-byte loads covers 1 KiB contiguously
  if constexpr (C::SPLIT) {
    // bf16 inputs: their products are exact in fp32; MFMA, wave w computes lower-triangle
    // tiles k = w, w+4, ...
    for (int k = wave; k < C::NTILES; k += 4) {
      const int tb = tile_tb(k), si = k - tb * (tb + 1) / 2;
      f32x16 acc = (f32x16){};
#pragma unroll
      for (int j = 0; j < C::KS_N; ++j)
        mma(acc, frag_contig(&sB[si * 32 + col][16 * j], g2), frag_contig(&sC[tb * 32 + col][16 * j], g2));
      float* dst = gout + (size_t)k * 1024 + 4 * lane;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(dst + 256 * q) =
            (f32x4){acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
  } else {
    // fp32 inputs: each entry B_s . C_t is a 128-term dot product in fp64 (the products are
    // exact there), rounded once to fp32, so the all-fp32 mode's Gram carries no summation
    // error. Item (k, q, l) holds accumulator registers 4q .. 4q+3 of lane l of tile k.
    for (int it = tid; it < C::NTILES * 4 * 64; it += PREP_THREADS) {
      const int k = it / 256, q = (it / 64) % 4, l = it % 64;
      const int tb = tile_tb(k), si = k - tb * (tb + 1) / 2;
      const int t = tb * 32 + (l & 31);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int sr = si * 32 + acc_row(4 * q + e, l);
        double dot = 0.0;
        for (int n = 0; n < SN; ++n) dot = fma((double)sB[sr][n], (double)sC[t][n], dot);
        v[e] = (float)dot;
      }
      *reinterpret_cast<f32x4*>(gout + (size_t)k * 1024 + 256 * q + 4 * l) = v;
    }
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

// ---------------------------------------------------------------------------- pipelined scan, chunk 64
// The one scan of the library: bf16 or fp32 io, whatever chunk length the call names (the
// chunk is a tiling choice that does not change the result; the scan tiles at 64 tokens).
// 16 waves, one barrier per chunk. In iteration c:
//   Y waves 0..3:   chunk c's outputs, Y^T tile (token block y >> 1, p-block y & 1):
//                   H^T C^T scaled by exp2(lambda_t), plus X^T M^T, gated, into sZ.
//   H waves 4..7:   the state to H_c (H wave w: state rows 32 w .. 32 w + 31, both p-blocks),
//                   published into the other half of a double-buffered H^T.
//   helper waves 8..15: chunk c+1's staging (flush of y(c-1), z, x^T, (w x)^T hi/lo), its
//                   masked decay tiles M^T (the diagonal ones in halves by helper waves 0..3,
//                   the other in quarters by helper waves 4..7), and the loads for the
//                   chunks after; helper wave 5 also forms chunk c+2's dt / pi / v records
//                   from dt_raw.
// Everything chunk c+1 needs goes to the other half of double-buffered LDS tiles, so the
// barrier that ends the iteration is the only synchronisation; records are staged two chunks
// ahead (three buffers). Four waves per SIMD (one of each kind plus two helpers) hide each
// other's latencies. LDS tiles are unpadded, with XOR swizzles that keep the 16-byte MFMA
// operand reads of H^T and (w x)^T (32 rows per instruction) free of bank conflicts.
// fp32 io runs the same roles with fp32 MFMAs (32x32x2, no hi/lo split). Its z and y move
// between HBM and the Y waves' registers (fp32 z and y tiles would not fit LDS beside the
// rest), and each chunk's contribution to the state is summed in an accumulator of its own
// before it is added to the decayed state, so that the state's rounding error grows with
// the number of chunks rather than with the number of tokens.
constexpr int P64 = 64;
constexpr int P64_THREADS = 1024;
__device__ __forceinline__ int xs64(int p, int s) { return s ^ (8 * ((p ^ (p >> 2)) & 7)); }
__device__ __forceinline__ int hsw(int p, int n) { return n ^ (8 * (p & 15)); }

// Element (t, p) of the bf16 z / y tile sits at column zpos(t, p): 4-element groups XOR-ed
// with a key of the token, so that the epilogue's 4-element accesses (32 tokens x one column
// group per instruction) hit distinct banks; the staging's 4-element groups stay whole.
__device__ __forceinline__ int zpos(int t, int p) { return p ^ (4 * ((t >> 1) & 15)); }

// LDS of the scan; the lo halves and the z / y tile exist only for bf16 io (a token-sized
// placeholder otherwise).
template <typename T>
struct Pipe64Smem {
  static constexpr bool SPLIT = sizeof(T) == 2;
  T sXt[2][SP][P64];                                            // x^T by chunk parity (xs64)
  T sXW[2][SP][P64];                                            // (w x)^T (bf16: hi) (xs64)
  bf16 sXWlo[SPLIT ? 2 : 1][SPLIT ? SP : 1][SPLIT ? P64 : 8];   //         lo
  bf16 sZ[SPLIT ? 2 : 1][SPLIT ? P64 : 1][SPLIT ? SP : 8];      // z, then y (zpos)
  Frag<T> sM[2][3][2][64];                     // M^T tiles [parity][tile][k step][lane]
  Frag<bf16> sMlo[SPLIT ? 2 : 1][3][2][SPLIT ? 64 : 1];
  T sHt[2][SP][SN];                                             // H^T (bf16: hi) by parity (hsw)
  bf16 sHtlo[SPLIT ? 2 : 1][SPLIT ? SP : 1][SPLIT ? SN : 8];    //     lo
  float sRec[3][4 * P64];                      // dt | pi_hi | v | pi_lo, chunk c in slot c % 3
  int4 sInfo[5];                               // packed batch: chunk info, chunk c in slot c % 5
};
static_assert(sizeof(Pipe64Smem<float>) <= 160 * 1024 && sizeof(Pipe64Smem<bf16>) <= 160 * 1024, "LDS");

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
// The phase profile (STAMP): s_memtime at phase boundaries, held in program order by
// scheduling barriers. Per wave, summed over chunks: [0] cycles of the whole chunk loop,
// [1] of the wave's first phase (Y waves: the contraction H^T C^T; H waves: B^T (w x);
// helper waves: building the decay tiles), [2] of its second (Y waves: X^T M^T; helper
// waves: staging the next chunk, the x conv included), [3] a sink that keeps the values
// read to close a phase alive, [4] cycles spent in the chunk's barrier, [5..7] zero. A
// contraction phase runs from before its first operand read to after the first read of
// its accumulator.
__device__ __forceinline__ uint64_t phase_stamp() {
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  return t;
}
constexpr int STAMP_SLOTS = 8;

template <typename T, bool CONV, bool VARLEN = false, bool STAMP = false>
__global__ __launch_bounds__(P64_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4)))
void ssd_scan64_kernel(const T* __restrict__ x, int64_t x_stride, const float* __restrict__ D,
                       const T* __restrict__ z, int64_t z_stride, const float* h0, float* h_final,
                       T* __restrict__ y, int64_t y_stride, const unsigned char* __restrict__ ws,
                       int Lrows, int H, int G, ConvArgs cv, VarlenDev vd, DtDev<T> dd,
                       uint64_t* __restrict__ stamps) {
  static_assert(!VARLEN || CONV, "the packed batch runs with the conv fused");
  static_assert(!CONV || sizeof(T) == 2, "the conv runs inside the scan for bf16 io");
  static_assert(!STAMP || (CONV && !VARLEN), "the phase profile covers the one-call prefill");
  using C = Cfg<T, P64>;
  constexpr int Q = P64;
  constexpr bool SPLIT = C::SPLIT;
  extern __shared__ __align__(16) unsigned char scan_smem[];
  Pipe64Smem<T>& S = *reinterpret_cast<Pipe64Smem<T>*>(scan_smem);

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
  [[maybe_unused]] uint64_t st_loop = 0, st_a = 0, st_b = 0, st_wait = 0;
  [[maybe_unused]] float st_sink = 0.f;
  // the chunk's barrier; with STAMP, the cycles spent in it are counted
  [[maybe_unused]] auto chunk_barrier = [&]() {
    if constexpr (STAMP) {
      const uint64_t w0 = phase_stamp();
      __syncthreads();
      st_wait += phase_stamp() - w0;
    } else {
      __syncthreads();
    }
  };
  [[maybe_unused]] auto stamps_out = [&]() {
    if constexpr (STAMP) {
      if (lane == 0) {
        uint64_t* o = stamps + ((size_t)blockIdx.x * (P64_THREADS / 64) + wave) * STAMP_SLOTS;
        o[0] = st_loop;
        o[1] = st_a;
        o[2] = st_b;
        o[3] = __float_as_uint(st_sink);
        o[4] = st_wait;
        o[5] = o[6] = o[7] = 0;
      }
    }
  };

  if (wave < 4) {
    // ========================================================== Y waves
    const int tb = wave >> 1, pb = wave & 1;
    const int prow = pb * 32 + col, tl = tb * 32 + col;
    // the chunk's C fragments: bf16 holds them in registers, requested a chunk ahead; fp32
    // (twice the registers) loads each k step's fragment where it is used
    using FV = decltype(Frag<T>{}.v);
    const uint32_t cf_lane = (uint32_t)((tb * C::KS_N * 64 + lane) * C::FB);
    auto cf_frag = [&](int c, int j) {
      Frag<T> f;
      f.v = ld_at<FV>(wsg + (size_t)c * C::REC_BYTES + C::G_BYTES + C::BT_BYTES, cf_lane + (uint32_t)(j * 64 * C::FB));
      return f;
    };
    Frag<T> cf[SPLIT ? C::KS_N : 1];
    auto fetch_c = [&](int c) {
      if constexpr (SPLIT) {
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j) cf[j] = cf_frag(c, j);
      }
    };
    if (nC > 0) fetch_c(0);
    __syncthreads();
    __syncthreads();
    if constexpr (STAMP) st_loop = phase_stamp();
    for (int c = 0; c < nC; ++c) {
      const int cur = c & 1, prv = cur ^ 1;
      [[maybe_unused]] uint64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
      if constexpr (STAMP) s0 = phase_stamp();
      // ---- carried state, scaled by exp2(lambda_t)
      f32x16 acc = {};
      {
        // four k steps of H^T (hi / lo) in flight
        Frag<T> ha[4];
        Frag<bf16> la[SPLIT ? 4 : 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = hsw(prow, 16 * j + 8 * g2);
          ha[j] = frag_contig(&S.sHt[prv][prow][n], 0);
          if constexpr (SPLIT) la[j] = frag_contig(&S.sHtlo[prv][prow][n], 0);
        }
#pragma unroll
        for (int j = 0; j < C::KS_N; ++j) {
          if constexpr (SPLIT) {
            mma(acc, ha[j & 3], cf[j]);
            mma(acc, la[j & 3], cf[j]);
          } else {
            mma(acc, ha[j & 3], cf_frag(c, j));
          }
          if (j + 4 < C::KS_N) {
            const int n = hsw(prow, 16 * (j + 4) + 8 * g2);
            ha[j & 3] = frag_contig(&S.sHt[prv][prow][n], 0);
            if constexpr (SPLIT) la[j & 3] = frag_contig(&S.sHtlo[prv][prow][n], 0);
          }
        }
      }
      const float et = exp2_hw((tb ? tot_of(c, 0) : 0.f) + S.sRec[c % 3][Q + tl]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] *= et;
      if constexpr (STAMP) s1 = phase_stamp();
      fetch_c(min(c + 1, nC - 1));
      // z of this wave's outputs, read ahead of the intra-chunk MFMAs (fp32: from HBM, the
      // rows past the end of the sequence clamped to its last)
      Raw4<T> zz[4];
      [[maybe_unused]] const int nval = Lrows - c * Q;
      [[maybe_unused]] const int64_t yrow = row0 + (int64_t)c * Q + min(tl, nval - 1);
      if (z) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          if constexpr (SPLIT) zz[r4] = ld4(&S.sZ[cur][tl][zpos(tl, pb * 32 + 8 * r4 + 4 * g2)]);
          else zz[r4] = ld4(z + yrow * z_stride + h * SP + pb * 32 + 8 * r4 + 4 * g2);
        }
      }
      // ---- intra-chunk part: Y^T += X^T M^T over source blocks si <= tb
      if constexpr (STAMP) s2 = phase_stamp();
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
            if constexpr (SPLIT) mma(acc, xa, S.sMlo[cur][k][m2][lane]);
          }
        }
      }
      if constexpr (STAMP) {
        st_sink += acc[0];
        s3 = phase_stamp();
      }
      // ---- gate; y into sZ[cur] in place of z (bf16), or to HBM (fp32)
      if (z) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] *= silu_fast(zz[r >> 2].get(r & 3));
      }
      if constexpr (SPLIT) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int r = 4 * r4;
          st4(&S.sZ[cur][tl][zpos(tl, pb * 32 + 8 * r4 + 4 * g2)], acc[r], acc[r + 1], acc[r + 2], acc[r + 3]);
        }
      } else if (tl < nval) {
        T* yr = y + yrow * y_stride + h * SP + pb * 32 + 4 * g2;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int r = 4 * r4;
          st4(yr + 8 * r4, acc[r], acc[r + 1], acc[r + 2], acc[r + 3]);
        }
      }
      if constexpr (STAMP) {
        st_a += s1 - s0;
        st_b += s3 - s2;
      }
      chunk_barrier();
    }
    if constexpr (STAMP) {
      st_loop = phase_stamp() - st_loop;
      stamps_out();
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
    const uint32_t bt_lane = (uint32_t)((hw * C::KS_Q * 64 + lane) * C::FB);
    auto fetch_bt = [&](int c) {
      const unsigned char* btf = wsg + (size_t)c * C::REC_BYTES + C::G_BYTES;
#pragma unroll
      for (int j = 0; j < C::KS_Q; ++j)
        af[j].v = ld_at<decltype(af[j].v)>(btf, bt_lane + (uint32_t)(j * 64 * C::FB));
    };
    auto publish = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int prow = i * 32 + col;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int n = hsw(prow, hw * 32 + 8 * r4 + 4 * g2);
          if constexpr (SPLIT) {
            const Split2 a = split2(hacc[i][4 * r4], hacc[i][4 * r4 + 1]);
            const Split2 d = split2(hacc[i][4 * r4 + 2], hacc[i][4 * r4 + 3]);
            *reinterpret_cast<uint2*>(&S.sHt[buf][prow][n]) = make_uint2(a.hi, d.hi);
            *reinterpret_cast<uint2*>(&S.sHtlo[buf][prow][n]) = make_uint2(a.lo, d.lo);
          } else {
            *reinterpret_cast<f32x4*>(&S.sHt[buf][prow][n]) =
                (f32x4){hacc[i][4 * r4], hacc[i][4 * r4 + 1], hacc[i][4 * r4 + 2], hacc[i][4 * r4 + 3]};
          }
        }
      }
    };
    publish(1);          // h0 is the state chunk 0 reads
    if (nC > 0) fetch_bt(0);
    __syncthreads();
    __syncthreads();
    if constexpr (STAMP) st_loop = phase_stamp();
    for (int c = 0; c < nC; ++c) {
      const int cur = c & 1;
      [[maybe_unused]] uint64_t s0 = 0;
      if constexpr (STAMP) s0 = phase_stamp();
      // ---- state update to H_c, published into sHt[cur]
      const float eend = exp2_hw(tot_of(c, 0) + tot_of(c, 1));
      if constexpr (SPLIT) {
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
      } else {
        // the chunk's contribution in its own accumulator, then H = eend H + S_c
        f32x16 sacc[2] = {};
#pragma unroll
        for (int j = 0; j < C::KS_Q; ++j) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int prow = i * 32 + col;
            mma(sacc[i], af[j], frag_contig(&S.sXW[cur][prow][xs64(prow, 16 * j + 8 * g2)], 0));
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) hacc[i][r] = fmaf(hacc[i][r], eend, sacc[i][r]);
      }
      if constexpr (STAMP) {
        st_sink += hacc[0][0] + hacc[1][0];
        st_a += phase_stamp() - s0;
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
      chunk_barrier();
    }
    if constexpr (STAMP) {
      st_loop = phase_stamp() - st_loop;
      stamps_out();
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
    // The helpers issue ahead of the Y and H waves that share their SIMDs: their chain (loads,
    // the x conv, the tiles of chunk c+1, the records of chunk c+2) is the longest of a chunk,
    // and at equal priority the arbiter often picked the other roles first and the helpers
    // finished last. At 12B 8k the one-call step went from 320 to 291 us with it; raising the
    // H waves instead made it slower (339 us), and the Y waves' priority made no difference.
    // Without the conv it helps since the records moved into this loop (the scan of the
    // two-call path: 285 to 281 us per call with its prep).
    __builtin_amdgcn_s_setprio(1);
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
    // v % 4, so every SIMD gets half a diagonal tile and a quarter of the other. Wave 5 also
    // forms the dt / pi_hi / v / pi_lo records (4Q words, a word a thread) from dt_raw.
    const int kb = hv < 2 ? 0 : hv < 4 ? 2 : 1;
    const int hm = hv & 1, hq = hv & 3;
    // Each role (records or not, tiles or not) runs its own copy of the loop, so that every
    // copy issues a fixed sequence of memory operations and the compiler's count of
    // outstanding loads stays exact: a merged count would wait for loads just issued.
    auto helpers = [&](auto part_tag, auto duty_tag) {
      constexpr int PART = decltype(part_tag)::value;   // 2: a diagonal half, 4: an off quarter
      // VARLEN duties: HIST, helper wave 0 (whose threads hold the first tokens of a chunk),
      // loads each chunk's conv history rows; RING, helper wave 4, keeps the info ring.
      // RECS, helper wave 5: the dt / pi_hi / v / pi_lo records of each chunk, two chunks ahead
      constexpr bool HIST = VARLEN && decltype(duty_tag)::value == 1;
      constexpr bool RING = VARLEN && decltype(duty_tag)::value == 2;
      constexpr bool RECS = decltype(duty_tag)::value == 3;
      // x rows of the thread's tokens; with the conv, raw rows s0 - 3 .. s0 + 1
      constexpr int NX = CONV ? 5 : 2;
      Raw4<T> rX[NX], rZ[2];
      // byte offsets of the thread's rows in a full chunk: x rows s0 + k from the x base, z
      // rows s0 + k
      uint32_t oxr[NX], ozr[2];
#pragma unroll
      for (int k = 0; k < NX; ++k) oxr[k] = ((uint32_t)(s0 + k) * xs + p0) * (uint32_t)sizeof(T);
#pragma unroll
      for (int k = 0; k < 2; ++k) ozr[k] = ((uint32_t)(s0 + k) * zs + p0) * (uint32_t)sizeof(T);
      [[maybe_unused]] float rDt = 0.f;   // RECS: dt_raw of token `lane` of the chunk in flight
      [[maybe_unused]] const float dtb = RECS ? dd.bias[h] : 0.f, Ah = RECS ? dd.A[h] : 0.f;
      f32x4 gram[2];                     // Gram tile registers 8 hm .. 8 hm + 7 (4 hq .. 4 hq + 3)
      // the history rows before the sequence that this thread's first tokens read (zeros
      // without a history): for one sequence loaded once in the prologue, for a packed batch
      // by the HIST role with each chunk's rows, from the chunk's place in the history area
      Raw4<T> rH[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) rH[k].v = decltype(rH[k].v){};
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
        // with the conv, x is addressed from a base 3 rows back (raw rows s0 - 3 .. s0 + 1)
        const T* xa = CONV ? xc - 3 * x_stride : xc;
        using XV = decltype(rX[0].v);
        if (nval >= Q && !(CONV && first)) {
          // a full chunk after the first: the loop-invariant offsets
#pragma unroll
          for (int k = 0; k < (CONV ? NX : 2); ++k) rX[k].v = ld_at<XV>(xa, oxr[k]);
          if constexpr (SPLIT) {
#pragma unroll
            for (int k = 0; k < 2; ++k) rZ[k].v = ld_at<XV>(zc, ozr[k]);
          }
        } else {
          // Rows past the end of the sequence load the last row instead (finite values; their
          // dt and v are zero, so they add nothing), which keeps the loads unconditional. In
          // the first chunk the rows before the sequence are read as row 0 and replaced when
          // that chunk is staged.
          const int lim = nval - 1;
          const int lo = CONV && first ? 3 : 0;
#pragma unroll
          for (int k = 0; k < (CONV ? NX : 2); ++k) {
            const uint32_t s = CONV ? (uint32_t)min(max(s0 + k, lo), lim + 3) : (uint32_t)min(s0 + k, lim);
            rX[k].v = ld_at<XV>(xa, (s * xs + p0) * (uint32_t)sizeof(T));
          }
          if constexpr (SPLIT) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const uint32_t s = (uint32_t)min(s0 + k, lim);
              rZ[k].v = ld_at<XV>(zc, (s * zs + p0) * (uint32_t)sizeof(T));
            }
          }
        }
        if constexpr (CONV) {
          if constexpr (HIST) {
            // every chunk issues the same 3 loads (used only where a sequence starts)
            const T* hp = vd.hist + (size_t)(gc0 + c) * 3 * (H * SP) + h * SP + p0;
#pragma unroll
            for (int k = 0; k < 3; ++k) rH[k] = ld4(hp + min(s0 + k, 2) * (H * SP));
          }
        }
      };
      // RECS: chunk c's rows (its first row, its valid rows), then its dt_raw into rDt (past
      // the end of the sequence the last row is read and not used)
      [[maybe_unused]] auto rows_of = [&](int c, int4 ci, int64_t& r0, int& nval) {
        if constexpr (VARLEN) {
          r0 = ci.x;
          nval = ci.y & 255;
        } else {
          r0 = row0 + (int64_t)c * Q;
          nval = L - c * Q;
        }
      };
      auto load_dt = [&](int c, int4 ci) {
        if constexpr (RECS) {
          int64_t r0;
          int nval;
          rows_of(c, ci, r0, nval);
          rDt = to_f(dd.raw[(r0 + min(lane, nval - 1)) * dd.stride + h]);
        }
      };
      // RECS: the records of chunk c (whose dt_raw is in rDt) into slot `slot` % 3: per token
      // dt = softplus(dt_raw + dt_bias) (zero past the end), the prefix pi of dt A log2(e) over
      // its 32-token block summed in fp64 (each term rounded once in fp32) and kept as
      // pi_hi + pi_lo, and v = dt 2^(pi at the block end - pi), the decay from the token to
      // the end of its block
      auto make_rec = [&](int slot, int c, int4 ci) {
        if constexpr (RECS) {
          int64_t r0;
          int nval;
          rows_of(c, ci, r0, nval);
          const float dt = lane < nval ? softplus_hw(rDt + dtb) : 0.f;
          const double run = scan32_f64((double)(dt * Ah * kLog2e));
          const double tot = half_last_f64(run, lane);
          const float hi = (float)run;
          float* r = S.sRec[slot % 3];
          r[lane] = dt;
          r[Q + lane] = hi;
          r[2 * Q + lane] = exp2_hw((float)(tot - run)) * dt;
          r[3 * Q + lane] = (float)(run - (double)hi);
        }
      };
      auto flush_y = [&](int c, bool full, int4 cf) {   // y of chunk c out of sZ[c & 1] (bf16)
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
          const Raw4<bf16> v = ld4(&S.sZ[c & 1][s][zpos(s, p0)]);
          if (full || s < nval) st_at(yc, ((uint32_t)s * ys + p0) * 2u, v.v);
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
        if constexpr (SPLIT) {
          if (z) {
#pragma unroll
            for (int k = 0; k < 2; ++k)
              *reinterpret_cast<bf16x4*>(&S.sZ[buf][s0 + k][zpos(s0 + k, p0)]) = rZ[k].v;
          }
        }
        // w_s = v_s exp2(decay from the end of s's block to the chunk end): block 0 -> tot_1
        const float* rec = S.sRec[c % 3];
        const float2 vs = *reinterpret_cast<const float2*>(&rec[2 * Q + s0]);
        const float wb = s0 < 32 ? exp2_hw(rec[Q + 63]) : 1.f;
        const float w0 = vs.x * wb, w1 = vs.y * wb;
        T xv[2][4];
        [[maybe_unused]] uint32_t xpk[4];   // CONV: the pair (token s0, s0 + 1) of column p0 + e
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
          for (int e = 0; e < 4; ++e) {
            float f[2];
#pragma unroll
            for (int k = 0; k < 2; ++k)
              f[k] = conv4_silu(cw[e], cb[e], r[k].get(e), r[k + 1].get(e), r[k + 2].get(e), r[k + 3].get(e));
            xpk[e] = pack_bf16(f[0], f[1]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[0][e] = rX[0].v[e];
            xv[1][e] = rX[1].v[e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = p0 + e, sw = xs64(p, s0);
          if constexpr (CONV) {
            *reinterpret_cast<uint32_t*>(&S.sXt[buf][p][sw]) = xpk[e];
            const float x0 = __uint_as_float(xpk[e] << 16), x1 = __uint_as_float(xpk[e] & 0xffff0000u);
            const Split2 v = split2(x0 * w0, x1 * w1);
            *reinterpret_cast<uint32_t*>(&S.sXW[buf][p][sw]) = v.hi;
            *reinterpret_cast<uint32_t*>(&S.sXWlo[buf][p][sw]) = v.lo;
            continue;
          }
          const T x0 = xv[0][e], x1 = xv[1][e];
          st_pair(&S.sXt[buf][p][sw], x0, x1);
          if constexpr (SPLIT) {
            const Split2 v = split2(to_f(x0) * w0, to_f(x1) * w1);
            *reinterpret_cast<uint32_t*>(&S.sXW[buf][p][sw]) = v.hi;
            *reinterpret_cast<uint32_t*>(&S.sXWlo[buf][p][sw]) = v.lo;
          } else {
            st_pair(&S.sXW[buf][p][sw], to_f(x0) * w0, to_f(x1) * w1);
          }
        }
      };
      auto fetch_gram = [&](int c) {   // quads 2 hm, 2 hm + 1 (or quad hq) of the stored tile
        const unsigned char* tile = wsg + (size_t)c * C::REC_BYTES + (size_t)kb * 4096;
        const uint32_t lo = 16u * lane;
        if constexpr (PART == 2) {
          gram[0] = ld_at<f32x4>(tile, lo + 2048u * hm);
          gram[1] = ld_at<f32x4>(tile, lo + 2048u * hm + 1024u);
        } else {
          gram[0] = ld_at<f32x4>(tile, lo + 1024u * hq);
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
          if constexpr (SPLIT) {
            const Split2 a = split2(gram[0][0] * (vq[0] * ut), gram[0][1] * (vq[1] * ut));
            const Split2 d = split2(gram[0][2] * (vq[2] * ut), gram[0][3] * (vq[3] * ut));
            *reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(&S.sM[c & 1][1][hq >> 1][lane]) +
                                      8 * (hq & 1)) = make_uint2(a.hi, d.hi);
            *reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(&S.sMlo[c & 1][1][hq >> 1][lane]) +
                                      8 * (hq & 1)) = make_uint2(a.lo, d.lo);
          } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(&S.sM[c & 1][1][hq >> 1][lane]) + 4 * (hq & 1)) =
                (f32x4){gram[0][0] * (vq[0] * ut), gram[0][1] * (vq[1] * ut), gram[0][2] * (vq[2] * ut),
                        gram[0][3] * (vq[3] * ut)};
          }
        } else {
          const float* rec = S.sRec[c % 3];
          const float* sDt = rec;
          const float* sPi = rec + Q;
          const float* sPl = rec + 3 * Q;
          // half hm of a diagonal tile (token block tb onto itself); the decay from s to t is
          // (pi_hi t - pi_hi s) + (pi_lo t - pi_lo s), accurate to the rounding of its own size
          const int tb = kb == 0 ? 0 : 1;
          const int tl = tb * 32 + col;
          float mv[8];
          const float pit = sPi[tl], plt = sPl[tl];
          // Where the block's decay stays above 2^-96 the decay from s to t factors into
          // v_s = dt_s 2^(pi_end - pi_s) (the record) and 2^(pi_t - pi_end) <= 2^96, both
          // normal floats: one exponential per lane instead of one per element.
          const float pe = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(sPi[tb * 32 + 31])));
          const float pel = sPl[tb * 32 + 31];
          if (SPLIT && pe > -96.f) {
            const float at = exp2_hw((pit - pe) + (plt - pel));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int sr = tb * 32 + 16 * hm + 8 * j + 4 * g2;
              const f32x4 vs = *reinterpret_cast<const f32x4*>(&rec[2 * Q + sr]);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float v = (sr + q <= tl) ? gram[j][q] * (vs[q] * at) : 0.f;
                if (sr + q == tl) v += Dh;
                mv[4 * j + q] = v;
              }
            }
          } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int sr = tb * 32 + 16 * hm + 8 * j + 4 * g2;
            const f32x4 ps = *reinterpret_cast<const f32x4*>(&sPi[sr]);
            const f32x4 pl = *reinterpret_cast<const f32x4*>(&sPl[sr]);
            const f32x4 ds = *reinterpret_cast<const f32x4*>(&sDt[sr]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v = (sr + q <= tl) ? gram[j][q] * exp2_hw((pit - ps[q]) + (plt - pl[q])) * ds[q] : 0.f;
              if (sr + q == tl) v += Dh;
              mv[4 * j + q] = v;
            }
          }
          }
          if constexpr (SPLIT) {
            Frag<bf16> mh, ml;
            frag_split(mv, mh, ml);
            S.sM[c & 1][kb][hm][lane] = mh;
            S.sMlo[c & 1][kb][hm][lane] = ml;
          } else {
            Frag<T> mf;
#pragma unroll
            for (int e = 0; e < 8; ++e) mf.v[e] = mv[e];
            S.sM[c & 1][kb][hm][lane] = mf;
          }
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
        load_dt(0, ci0);
        make_rec(0, 0, ci0);
        load_dt(min(1, nC - 1), ci1);
        make_rec(1, min(1, nC - 1), ci1);
        fetch_gram(0);
      }
      __syncthreads();
      if (nC > 0) {
        stage(0, std::true_type{}, ci0);
        load_set(min(1, nC - 1), ci1);
        build(0);
        fetch_gram(min(1, nC - 1));
      }
      __syncthreads();
      if constexpr (STAMP) st_loop = phase_stamp();
      for (int c = 0; c < nC; ++c) {
        // packed batch: the infos this iteration uses (chunks c - 1, c + 1, c + 2), read from
        // the ring now so that their latency hides behind the tile build
        int4 im1 = {}, ip1 = {}, ip2 = {};
        if constexpr (VARLEN) {
          im1 = S.sInfo[(c + 4) % 5];
          ip1 = S.sInfo[min(c + 1, nC - 1) % 5];
          ip2 = S.sInfo[min(c + 2, nC - 1) % 5];
        }
        // RECS: chunk c + 2's dt_raw, used for its records at the end of this iteration
        load_dt(min(c + 2, nC - 1), ip2);
        // ---- chunk c + 1: tiles and staging. Chunk indices are clamped, so every iteration
        // issues the same memory operations (the last stages a copy nobody reads).
        [[maybe_unused]] uint64_t s0 = 0, s1 = 0;
        if constexpr (STAMP) s0 = phase_stamp();
        build(c + 1);
        if constexpr (STAMP) {
          s1 = phase_stamp();
          st_a += s1 - s0;
        }
        fetch_gram(min(c + 2, nC - 1));
        if constexpr (SPLIT) {
          if (c >= 1) flush_y(c - 1, !VARLEN, im1);   // one sequence: chunk c - 1 < nC - 1 is full
        }
        if constexpr (STAMP) s0 = phase_stamp();
        stage(c + 1, std::false_type{}, ip1);
        if constexpr (STAMP) st_b += phase_stamp() - s0;
        make_rec(c + 2, min(c + 2, nC - 1), ip2);
        load_set(min(c + 2, nC - 1), ip2);
        if constexpr (RING) {
          reinterpret_cast<int*>(&S.sInfo[(c + 3) % 5])[lane & 3] = rInfo;
          rInfo = info_word(c + 4);
        }
        chunk_barrier();
      }
      if constexpr (STAMP) {
        st_loop = phase_stamp() - st_loop;
        stamps_out();
      }
      if constexpr (SPLIT) {
        if (nC > 0) flush_y(nC - 1, false, VARLEN ? S.sInfo[(nC - 1) % 5] : int4{});   // y of the last chunk
      }
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
    using Recs = std::integral_constant<int, 3>;
    if (VARLEN && hv == 0) helpers(Half{}, Hist{});
    else if (hv < 4) helpers(Half{}, NoDuty{});
    else if (VARLEN && hv == 4) helpers(Quarter{}, Ring{});
    else if (hv == 5) helpers(Quarter{}, Recs{});
    else helpers(Quarter{}, NoDuty{});
  }
}

// ---------------------------------------------------------------------------- host side
// row stride of dt_raw in elements: dense [rows][H] unless the caller gave one
static int64_t dt_stride(const PrefillArgs& a) { return a.dt_stride > 0 ? a.dt_stride : a.H; }
template <typename T>
static DtDev<T> dt_dev(const PrefillArgs& a) {
  return {static_cast<const T*>(a.dt_raw), dt_stride(a), a.dt_bias, a.A};
}

static hipError_t set_lds(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr int Q = P64;
  using C = Cfg<T, Q>;
  const size_t prep_lds = 2 * sizeof(T) * Q * C::LDN;
  const size_t scan_lds = sizeof(Pipe64Smem<T>);
  static bool configured = false;
  if (!configured) {
    hipError_t e = set_lds(reinterpret_cast<const void*>(&ssd_prep_kernel<T, Q, false>), prep_lds);
    if (e == hipSuccess) e = set_lds(reinterpret_cast<const void*>(&ssd_scan64_kernel<T, false>), scan_lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int nC = (a.L + Q - 1) / Q;
  if (nC > 0) {
    hipLaunchKernelGGL((ssd_prep_kernel<T, Q, false>), dim3(a.B * a.G * nC), dim3(PREP_THREADS), prep_lds,
                       stream, static_cast<const T*>(a.Bm), a.b_stride, static_cast<const T*>(a.Cm),
                       a.c_stride, static_cast<unsigned char*>(a.workspace), a.L, a.H, a.G, nC, ConvArgs{},
                       VarlenDev{});
  }
  hipLaunchKernelGGL((ssd_scan64_kernel<T, false>), dim3(a.B * a.H), dim3(P64_THREADS), scan_lds, stream,
                     static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                     a.z_stride, a.h0, a.h_final, static_cast<T*>(a.y), a.y_stride,
                     static_cast<const unsigned char*>(a.workspace), a.L, a.H, a.G, ConvArgs{}, VarlenDev{},
                     dt_dev<T>(a), nullptr);
  return hipGetLastError();
}

hipError_t launch_ssd_prefill_conv(const PrefillArgs& a, const ConvArgs& cv, hipStream_t stream,
                                   uint64_t* phase_cycles) {
  using T = bf16;
  constexpr int Q = P64;
  using C = Cfg<T, Q>;
  const size_t prep_lds = 2 * sizeof(T) * Q * C::LDN;
  static bool configured = false;
  if (!configured) {
    hipError_t e = set_lds(reinterpret_cast<const void*>(&ssd_prep_kernel<T, Q, true>), prep_lds);
    if (e == hipSuccess)
      e = set_lds(reinterpret_cast<const void*>(&ssd_scan64_kernel<T, true>), sizeof(Pipe64Smem<T>));
    if (e == hipSuccess)
      e = set_lds(reinterpret_cast<const void*>(&ssd_scan64_kernel<T, true, false, true>), sizeof(Pipe64Smem<T>));
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int nC = (a.L + Q - 1) / Q;
  if (nC > 0) {
    hipLaunchKernelGGL((ssd_prep_kernel<T, Q, true>), dim3(a.B * a.G * nC), dim3(PREP_THREADS), prep_lds,
                       stream, static_cast<const T*>(a.Bm), a.b_stride, static_cast<const T*>(a.Cm),
                       a.c_stride, static_cast<unsigned char*>(a.workspace), a.L, a.H, a.G, nC, cv, VarlenDev{});
  }
  if (phase_cycles) {
    hipLaunchKernelGGL((ssd_scan64_kernel<T, true, false, true>), dim3(a.B * a.H), dim3(P64_THREADS),
                       sizeof(Pipe64Smem<T>), stream, static_cast<const T*>(a.x), a.x_stride, a.D,
                       static_cast<const T*>(a.z), a.z_stride, a.h0, a.h_final, static_cast<T*>(a.y), a.y_stride,
                       static_cast<const unsigned char*>(a.workspace), a.L, a.H, a.G, cv, VarlenDev{}, dt_dev<T>(a),
                       phase_cycles);
  } else {
    hipLaunchKernelGGL((ssd_scan64_kernel<T, true>), dim3(a.B * a.H), dim3(P64_THREADS), sizeof(Pipe64Smem<T>),
                       stream, static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                       a.z_stride, a.h0, a.h_final, static_cast<T*>(a.y), a.y_stride,
                       static_cast<const unsigned char*>(a.workspace), a.L, a.H, a.G, cv, VarlenDev{}, dt_dev<T>(a),
                       nullptr);
  }
  return hipGetLastError();
}

// records for up to total / 64 + nseq chunks (the most a packed batch of nseq sequences over
// total rows can have), the per-chunk info, the per-chunk history area, then the sanitized
// offsets and the per-sequence first chunks
static int varlen_max_chunks(int total, int nseq) { return total / P64 + nseq; }

size_t ssd_prefill_varlen_workspace(int total, int nseq, int H, int G) {
  using C = Cfg<bf16, P64>;
  const size_t maxC = (size_t)varlen_max_chunks(total, nseq);
  return maxC * ((size_t)G * C::REC_BYTES + sizeof(int4) + (size_t)3 * H * SP * sizeof(bf16)) +
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
      e = set_lds(reinterpret_cast<const void*>(&ssd_scan64_kernel<T, true, true>), sizeof(Pipe64Smem<T>));
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int maxC = varlen_max_chunks(a.L, va.nseq);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  int4* info = reinterpret_cast<int4*>(ws + (size_t)maxC * (size_t)a.G * C::REC_BYTES);
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
                     a.c_stride, ws, a.L, a.H, a.G, maxC, cv, vd);
  hipLaunchKernelGGL((ssd_scan64_kernel<T, true, true>), dim3(K * a.H), dim3(P64_THREADS), sizeof(Pipe64Smem<T>),
                     stream, static_cast<const T*>(a.x), a.x_stride, a.D, static_cast<const T*>(a.z),
                     a.z_stride, nullptr, nullptr, static_cast<T*>(a.y), a.y_stride, ws, a.L, a.H, a.G, cv, vd,
                     dt_dev<T>(a), nullptr);
  return hipGetLastError();
}

template <typename T, int Q>
static size_t ws_bytes(int B, int L, int H, int G) {
  using C = Cfg<T, Q>;
  const size_t nC = ((size_t)L + Q - 1) / Q;
  return nC * (size_t)B * G * C::REC_BYTES;
}

// The chunk a call names does not change the tiling: every supported chunk runs at 64.
size_t ssd_prefill_workspace(int io_bf16, int, int B, int L, int H, int G) {
  return io_bf16 ? ws_bytes<bf16, P64>(B, L, H, G) : ws_bytes<float, P64>(B, L, H, G);
}

hipError_t launch_ssd_prefill(int io_bf16, int, const PrefillArgs& a, hipStream_t stream) {
  return io_bf16 ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

// ---------------------------------------------------------------------------- static scratch
// Device memory the prefill can use as its workspace without any allocation by the call: a
// file-scope array of PREFILL_SCRATCH_BYTES that every device the library runs on holds
// until the process ends. In host code `prefill_scratch` names a host-side stand-in; its
// device address, different on each device, comes from hipGetSymbolAddress, taken once per
// device with that device current.
__device__ __align__(256) unsigned char prefill_scratch[PREFILL_SCRATCH_BYTES];

hipError_t prefill_scratch_on_current_device(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(prefill_scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace m2

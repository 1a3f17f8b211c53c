// Host-side launchers of the gfx950 kernels (one per .hip source). Called by the
// C-ABI layer after validation; each returns the HIP status of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace m2 {

hipError_t launch_conv1d(int io_bf16, const void* u, int64_t u_stride, const float* w,
                         const float* bias, void* conv_state, void* out, int64_t out_stride,
                         int B, int L, int Cc, hipStream_t stream);

struct PrefillArgs {
  const void* x; int64_t x_stride;
  const void* Bm; int64_t b_stride;
  const void* Cm; int64_t c_stride;
  const void* dt_raw;
  const float* dt_bias; const float* A; const float* D;
  const void* z; int64_t z_stride;
  const float* h0; float* h_final;
  void* y; int64_t y_stride;
  void* workspace;
  int B, L, H, G;
  int64_t dt_stride = 0;   // row stride of dt_raw in elements; 0: dense (H)
};
hipError_t launch_ssd_prefill(int io_bf16, int chunk, const PrefillArgs& a, hipStream_t stream);
// The conv fused into the prefill (bf16 io): x, Bm and Cm of `a` are the raw xBC
// columns; w [Cc][4], bias [Cc] (or NULL) and the [B][3][Cc] history (or NULL; updated to
// the last 3 raw tokens) cover all Cc xBC channels.
struct ConvArgs {
  const float* w; const float* bias;
  void* state;
  int Cc;
};
// phase_cycles: NULL, or [B * H][16 waves][8] uint64 that receive the scan's phase profile
// (cycles of the chunk loop and of each wave's contraction phases, summed over chunks).
hipError_t launch_ssd_prefill_conv(const PrefillArgs& a, const ConvArgs& cv, hipStream_t stream,
                                   uint64_t* phase_cycles = nullptr);
// Packed variable-length sequences with states in slot pools (bf16 io, conv fused):
// sequence i covers packed rows cu[i] .. cu[i+1] of x / Bm / Cm / dt_raw / z / y (a.L is
// the total row count, a.B the sequence count); it starts from ssm_pool / conv_pool entry
// slots[i] when has_init[i] != 0 (else from zeros) and leaves its final state and conv
// history there when 0 <= slots[i] < npool. slots NULL: sequence i uses entry i; has_init
// NULL: every sequence starts from zeros.
struct VarlenArgs {
  const int32_t* cu; const int32_t* slots; const int32_t* has_init;
  float* ssm_pool; void* conv_pool;
  int nseq, npool;
};
hipError_t launch_ssd_prefill_varlen(const PrefillArgs& a, const ConvArgs& cv, const VarlenArgs& va,
                                     hipStream_t stream);
// Workspace of the variable-length prefill: the records of ssd_prefill_workspace for up to
// seqlen / 64 + nseq chunks, then the sanitized offsets and the per-sequence chunk offsets.
size_t ssd_prefill_varlen_workspace(int total, int nseq, int H, int G);
// The prefill's static scratch: a device array of PREFILL_SCRATCH_BYTES per device, for the
// call that allocates nothing. Sets *ptr to its address on the current device (taken once
// per device).
constexpr size_t PREFILL_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t prefill_scratch_on_current_device(void** ptr);
// Workspace bytes the prep/scan pair needs: per (sequence, group, chunk) the causal Gram
// tiles in fp32 and B^T and C in MFMA operand order.
size_t ssd_prefill_workspace(int io_bf16, int chunk, int B, int L, int H, int G);

struct DecodeArgs {
  const void* u_t;
  const float* w; const float* bias;
  void* conv_state;
  const void* dt_raw_t;
  const float* dt_bias; const float* A; const float* D;
  const void* z_t;
  float* ssm_state;
  void* y_t;
  int B, H, G;
  const int32_t* slots = nullptr;   // sequence -> pool entry, or NULL for entry = sequence
  int npool = 0;
  int T = 1;                        // new tokens per sequence (1 .. 6), rows b T + t
  // row strides (elements) of u_t, z_t and dt_raw_t; 0: dense (Cc, H * 64, H)
  int64_t u_stride = 0, z_stride = 0, dt_stride = 0;
};
hipError_t launch_state_update(int io_bf16, const DecodeArgs& a, hipStream_t stream);

// rows x width io elements (row strides in elements), width = G contiguous groups
hipError_t launch_group_rmsnorm(int io_bf16, const void* g, int64_t g_stride, const float* weight,
                                float eps, void* out, int64_t out_stride, int64_t rows, int G,
                                int width, hipStream_t stream);

// Row-major C[M][N] (row stride ldc) = A[M][K] (row stride lda) * W[N][K]^T with W dense,
// io elements, fp32 accumulation, on hipBLASLt. ws / ws_bytes: device workspace the
// library may use. The first call on a device creates that device's hipBLASLt handle and
// each new shape runs the algorithm heuristic once; both are kept until the process ends.
enum { GEMM_OK = 0, GEMM_ERR_LIB = 1, GEMM_ERR_NO_ALGO = 2 };
int gemm_nt(int io_bf16, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* W,
            void* C, int64_t ldc, void* ws, size_t ws_bytes, hipStream_t stream, std::string* err);

}  // namespace m2

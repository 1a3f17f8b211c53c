/*
 * mamba2.h -- C ABI of the MI355X (gfx950) Mamba-2 layer core.
 *
 * The layer is the Mamba-2 mixer of the Nemotron-Nano-2 hybrid model (hyper.ai
 * summary of arXiv 2508.14444, section "方法"; neurohive article, section
 * "Архитектура"): 8 groups, state dimension 128, head dimension 64, expansion 2,
 * conv window 4, no bias in the surrounding linear layers. Its core is
 *
 *   xBC' = SiLU(causal depthwise conv1d(xBC) + bias)       width 4, per channel
 *   dt   = softplus(dt_raw + dt_bias),  a = exp(dt * A)      per token and head
 *   h_t  = a_t h_{t-1} + dt_t B_t x_t^T                      N x P state, fp32
 *   y_t  = h_t^T C_t + D x_t,   out = y * SiLU(z)
 *
 * with B and C shared by the contiguous heads of each group (head h uses group
 * h / (H / G)). The SSM state is always fp32, as the deployment section of the
 * neurohive article ("Развертывание") requires of the Mamba cache.
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA memory).
 *    `dims` is host memory, read during the call only.
 *  - Row-major layouts as commented. "io" means the element type selected by
 *    dims->io_dtype (MAMBA2_BF16 or MAMBA2_F32); parameters (w, bias, dt_bias,
 *    A, D) and SSM states are float32 in every mode.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    null stream). Nothing synchronizes, nothing is allocated, no state is kept
 *    between calls; the exceptions are the mixer calls' hipBLASLt handle and the
 *    algorithm timing of their first call for a shape (see there). The caller
 *    owns every buffer and the stream.
 *  - Validation runs on the host before anything is enqueued. On failure the
 *    call returns a nonzero status, enqueues nothing and leaves every buffer
 *    untouched; mamba2_last_error() describes the failure. Launch failures
 *    return MAMBA2_ERR_HIP. Faults inside kernels surface asynchronously, as
 *    for any stream work.
 *  - Supported shapes: headdim 64, dstate 128, conv_width 4, nheads % ngroups
 *    == 0, batch/seqlen/nheads >= 1 (seqlen 0 is accepted by the prefill calls
 *    and does nothing). io pointers must be 16-byte aligned and io row strides
 *    multiples of 16 bytes; f32 state pointers 16-byte aligned.
 */
#ifndef MAMBA2_H
#define MAMBA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA2_ABI_VERSION 8

enum mamba2_dtype { MAMBA2_F32 = 0, MAMBA2_BF16 = 1 };

enum mamba2_status {
  MAMBA2_OK = 0,
  MAMBA2_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MAMBA2_ERR_SHAPE = 2,       /* a dimension or stride is out of range             */
  MAMBA2_ERR_UNSUPPORTED = 3, /* valid but not implemented (headdim != 64, ...)    */
  MAMBA2_ERR_DTYPE = 4,       /* io_dtype is neither MAMBA2_F32 nor MAMBA2_BF16    */
  MAMBA2_ERR_ALIGN = 5,       /* pointer or stride breaks the 16-byte rule         */
  MAMBA2_ERR_ALIAS = 6,       /* an output overlaps an input it must not overlap   */
  MAMBA2_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required           */
  MAMBA2_ERR_HIP = 8          /* the HIP runtime reported an error at launch       */
};

typedef struct mamba2_dims {
  int32_t batch;      /* B: independent sequences                                  */
  int32_t seqlen;     /* L: tokens per sequence (must be 1 for mamba2_state_update)*/
  int32_t nheads;     /* H: SSM heads; d_inner = H * headdim                       */
  int32_t headdim;    /* P: must be 64                                             */
  int32_t ngroups;    /* G: B/C groups, divides H                                  */
  int32_t dstate;     /* N: must be 128                                            */
  int32_t conv_width; /* W: must be 4                                              */
  int32_t chunk;      /* Q: prefill chunk, 64, 128 or 256: a tiling choice; the    */
                      /*    kernels tile at 64 whichever is named, and the result  */
                      /*    does not depend on it beyond rounding                  */
  int32_t io_dtype;   /* enum mamba2_dtype                                         */
} mamba2_dims;

/*
 * mamba2_conv1d -- causal depthwise conv of width W over `channels` channels,
 * plus bias, then SiLU (the Mamba-2 block's "conv window 4": hyper.ai summary,
 * section "方法"). For token t and channel c:
 *     v = bias[c] + sum_{k=0}^{W-1} w[c*W + k] * u[t-(W-1)+k][c],   out = v / (1 + e^-v)
 * Taps are a cross-correlation: w[c*W + W-1] multiplies the current token.
 * Tokens before t = 0 come from conv_state (zeros if conv_state is NULL).
 *
 *   u          [B][L][channels] io, row stride u_stride elements (>= channels)
 *   w          [channels][W] f32
 *   bias       [channels] f32, or NULL for no bias
 *   conv_state [B][W-1][channels] io, dense, or NULL. In: the W-1 raw inputs
 *              preceding token 0 (slot 0 the oldest). Out: the last W-1 raw
 *              inputs of the extended sequence (history, then u), i.e. the
 *              history a following call or decode step needs. Updated in place.
 *   out        [B][L][channels] io, row stride out_stride; must not overlap u,
 *              w, bias or conv_state.
 * channels must be a multiple of 8 (bf16) or 4 (f32). dims->headdim, dstate,
 * ngroups, nheads and chunk are not used by this call. With seqlen 0 the call
 * does nothing and returns MAMBA2_OK.
 */
int mamba2_conv1d(const mamba2_dims* dims, int32_t channels, const void* u, int64_t u_stride,
                  const float* w, const float* bias, void* conv_state, void* out,
                  int64_t out_stride, void* stream);

/*
 * mamba2_ssd_prefill_workspace_bytes -- device workspace mamba2_ssd_prefill
 * needs for `dims` (0 if `dims` is invalid or the sequence is empty). The scan
 * first computes, once per (sequence, group, chunk), the causal Gram tiles
 * B_s . C_t of the chunk in fp32 and B^T and C laid out as MFMA operands, which
 * every head of the group then reads. The kernels tile at 64 tokens whatever
 * chunk dims names, so with e = sizeof(io):
 *   nchunks * batch * ngroups * (12288 + 16384 * e),   nchunks = ceil(seqlen / 64)
 * The caller owns it; its contents are scratch (nothing is kept between calls).
 */
size_t mamba2_ssd_prefill_workspace_bytes(const mamba2_dims* dims);

/*
 * mamba2_ssd_prefill -- the selective scan over whole sequences (the
 * spec recurrence above, evaluated chunk by chunk: inside a chunk of Q
 * tokens as a causally masked quadratic form on MFMA, across chunks by carrying
 * the fp32 state).
 *
 *   x       [B][L][H*P] io, token row stride x_stride (elements)
 *   Bm, Cm  [B][L][G*N] io, row strides b_stride, c_stride
 *   dt_raw  [B][L][H] io, dense
 *   dt_bias, A [H] f32 (A <= 0 expected, not checked; A > 0 may overflow)
 *   D       [H] f32, or NULL for no skip term
 *   z       [B][L][H*P] io with row stride z_stride, or NULL for no gate
 *   h0      [B][H][N][P] f32 initial state, or NULL for zeros
 *   h_final [B][H][N][P] f32 final state, or NULL; may equal h0 (in place)
 *   y       [B][L][H*P] io, row stride y_stride; must not overlap any input
 *   workspace, workspace_bytes: device scratch of at least
 *           mamba2_ssd_prefill_workspace_bytes(dims) bytes, 16-byte aligned, not
 *           overlapping any other argument (may be NULL when that is 0);
 *           MAMBA2_ERR_WORKSPACE if missing or too small
 * x/B/C may be views into one xBC tensor (row stride = its channel count).
 * With seqlen 0 nothing per-token is read or written (those pointers may be
 * NULL) and h_final receives h0 (or zeros). Row strides above 2^23 elements are
 * rejected (MAMBA2_ERR_SHAPE).
 */
int mamba2_ssd_prefill(const mamba2_dims* dims, const void* x, int64_t x_stride, const void* Bm,
                       int64_t b_stride, const void* Cm, int64_t c_stride, const void* dt_raw,
                       const float* dt_bias, const float* A, const float* D, const void* z,
                       int64_t z_stride, const float* h0, float* h_final, void* y,
                       int64_t y_stride, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mamba2_conv_ssd_prefill_workspace_bytes -- device workspace mamba2_conv_ssd_prefill
 * needs for `dims` (0 if `dims` is invalid). For bf16 io it equals
 * mamba2_ssd_prefill_workspace_bytes(dims); for fp32 io it adds batch * seqlen * Cc
 * fp32 elements (after rounding the former up to 256 bytes), where the conv output is
 * kept between the two steps.
 */
size_t mamba2_conv_ssd_prefill_workspace_bytes(const mamba2_dims* dims);

/*
 * mamba2_conv_ssd_prefill -- the prefill of the layer core from the raw xBC
 * projection: mamba2_conv1d over all Cc = H*P + 2*G*N xBC channels followed by
 * mamba2_ssd_prefill on its x, B and C columns (the conv and the scan of the
 * block: hyper.ai summary, section "方法"). For bf16 io the conv is applied inside
 * the scan's kernels as they stage each chunk, so the conv output never goes through
 * device memory; the results are bitwise those of the two calls in sequence. fp32 io
 * runs the two steps through the workspace.
 *
 *   xBC        [B][L][Cc] io raw (pre-conv) x | B | C, row stride xbc_stride
 *   conv_w     [Cc][4] f32; conv_bias [Cc] f32 or NULL
 *   conv_state [B][3][Cc] io, dense, or NULL: the raw history before token 0
 *              (zeros if NULL), replaced by the last 3 raw inputs of (history,
 *              xBC), as mamba2_conv1d does
 *   dt_raw, dt_bias, A, D, z, h0, h_final, y: as in mamba2_ssd_prefill
 *   workspace, workspace_bytes: at least mamba2_conv_ssd_prefill_workspace_bytes(dims)
 *              bytes, 16-byte aligned, not overlapping any other argument
 * y, conv_state, h_final and the workspace must not overlap each other or any
 * input (h_final may equal h0). With seqlen 0 the history is unchanged and
 * h_final receives h0 (or zeros).
 */
int mamba2_conv_ssd_prefill(const mamba2_dims* dims, const void* xBC, int64_t xbc_stride,
                            const float* conv_w, const float* conv_bias, void* conv_state,
                            const void* dt_raw, const float* dt_bias, const float* A,
                            const float* D, const void* z, int64_t z_stride, const float* h0,
                            float* h_final, void* y, int64_t y_stride, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * mamba2_conv_ssd_prefill_profile -- mamba2_conv_ssd_prefill (bf16 io only; results
 * bitwise those of that call) with a cycle profile of the scan's contraction phases, the
 * measurement behind the per-phase MFMA rates (the MFMA contractions of the SSD scan:
 * hyper.ai summary, section "方法"). For scan workgroup k (k < batch * nheads, one per
 * (sequence, head)) and wave v (16 per workgroup), phase_cycles[(k * 16 + v) * 8 + i] gets
 * shader-clock cycles (s_memtime) summed over the chunk loop:
 *   i = 0  the whole chunk loop;
 *   i = 1  waves 0-3: the carried-state output H^T C^T of their 32x32 output tile;
 *          waves 4-7: the state update B^T (w x) of their 32 state rows;
 *          waves 8-15: building the masked decay tiles of the next chunk;
 *   i = 2  waves 0-3: the intra-chunk product X^T M^T of their tile;
 *          waves 8-15: staging the next chunk (its loads' arrival, the x conv, the hi/lo
 *          splits, the LDS stores);
 *   i = 3  bits of a value the stamps read (kept so that no phase is optimised away);
 *   i = 4  time spent in the chunk's barrier (waiting for the slowest role);
 *   i = 5..7  zero.
 * A contraction phase runs from before its first operand read to after the first read of
 * its result.
 * phase_cycles: device memory of batch * nheads * 128 uint64, 8-byte aligned, not
 * overlapping any other argument (MAMBA2_ERR_NULL / _ALIGN / _ALIAS otherwise); fp32 io
 * is MAMBA2_ERR_UNSUPPORTED. With seqlen 0 it is not written. The stamps slow the scan a
 * little; this call is for measurement, not for production.
 */
int mamba2_conv_ssd_prefill_profile(const mamba2_dims* dims, const void* xBC, int64_t xbc_stride,
                                    const float* conv_w, const float* conv_bias, void* conv_state,
                                    const void* dt_raw, const float* dt_bias, const float* A,
                                    const float* D, const void* z, int64_t z_stride, const float* h0,
                                    float* h_final, void* y, int64_t y_stride, void* workspace,
                                    size_t workspace_bytes, uint64_t* phase_cycles, void* stream);

/*
 * mamba2_conv_ssd_prefill_noalloc -- mamba2_conv_ssd_prefill without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call the allocator). The call itself allocates nothing: its
 * workspace is a static device array of 64 MiB (67108864 bytes) that the library holds on
 * every device it runs on until the process ends. Arguments, results and errors are those
 * of mamba2_conv_ssd_prefill; a setting whose workspace
 * (mamba2_conv_ssd_prefill_workspace_bytes) exceeds 64 MiB is rejected with
 * MAMBA2_ERR_WORKSPACE (at the 12B shape, bf16: up to batch * seqlen = 11904 tokens).
 * Every call on a device uses that device's one array: two calls in flight at once on one
 * device (on different streams) race and give undefined results. Calls on one stream
 * are ordered and safe. Nothing in the array needs to start at zero.
 */
int mamba2_conv_ssd_prefill_noalloc(const mamba2_dims* dims, const void* xBC, int64_t xbc_stride,
                                    const float* conv_w, const float* conv_bias, void* conv_state,
                                    const void* dt_raw, const float* dt_bias, const float* A,
                                    const float* D, const void* z, int64_t z_stride, const float* h0,
                                    float* h_final, void* y, int64_t y_stride, void* stream);

/*
 * mamba2_conv_ssd_prefill_varlen_workspace_bytes -- device workspace of
 * mamba2_conv_ssd_prefill_varlen for `dims` (batch = number of sequences, seqlen =
 * total packed rows; bf16 io, any supported chunk: the kernels tile at 64), 0 if
 * `dims` is invalid or another setting:
 *   M * (ngroups * R + 16 + 384 * nheads) + 8 * (batch + 1),
 *   M = seqlen / 64 + batch
 * with R the per-(group, chunk) record of mamba2_ssd_prefill_workspace_bytes at chunk 64
 * (4096 * 3 + 2 * 128 * 64 * 2 bytes).
 */
size_t mamba2_conv_ssd_prefill_varlen_workspace_bytes(const mamba2_dims* dims);

/*
 * mamba2_conv_ssd_prefill_varlen -- mamba2_conv_ssd_prefill over a packed batch of
 * sequences of different lengths whose states live in slot pools, as an inference engine
 * with continuous batching keeps them (the deployment of the hyper.ai / neurohive pages
 * serves the model through such an engine with an fp32 Mamba cache: neurohive, section
 * "Развертывание"). dims->batch is the number of sequences S, dims->seqlen the number of
 * packed rows; only bf16 io is supported (MAMBA2_ERR_UNSUPPORTED otherwise).
 *
 *   xBC        [seqlen][Cc] io raw rows, row stride xbc_stride; sequence i is rows
 *              cu_seqlens[i] .. cu_seqlens[i+1]
 *   conv_w, conv_bias  as in mamba2_conv1d
 *   cu_seqlens [S+1] int32 (device): 0 = cu[0] <= cu[1] <= ... <= cu[S] <= seqlen.
 *              Offsets that break this are clamped into it (negative to 0, above seqlen
 *              to seqlen, decreasing to the previous one) so that no access leaves
 *              the packed rows; results are then those of the clamped offsets.
 *   slots      [S] int32 (device) or NULL (= 0, 1, ..., S-1): the pool entry of each
 *              sequence. An entry outside [0, npool) means "no entry": the sequence
 *              starts from zeros and its final state and history are not stored.
 *              Two sequences must not share an entry (their writes would race).
 *   has_init   [S] int32 (device) or NULL (= all 0): nonzero when the sequence
 *              continues from the state and conv history in its entry; zero when it
 *              starts from a zero state and a zero history
 *   conv_pool  [npool][3][Cc] io, ssm_pool [npool][H][N][P] f32: the caches. Each
 *              sequence with an entry leaves there its last 3 raw xBC rows (history
 *              included, as mamba2_conv1d) and its final state. May be NULL if npool == 0.
 *   dt_raw     [seqlen][H] io dense; dt_bias, A, D as in mamba2_ssd_prefill
 *   z, y       [seqlen][H*P] io with row strides (z may be NULL)
 *   workspace, workspace_bytes: at least mamba2_conv_ssd_prefill_varlen_workspace_bytes
 * Each sequence's y, final state and history are bitwise those of mamba2_conv_ssd_prefill
 * on that sequence alone (batch 1) started from the same state and history. y, the pools
 * and the workspace must not overlap each other or any input.
 */
int mamba2_conv_ssd_prefill_varlen(const mamba2_dims* dims, const void* xBC, int64_t xbc_stride,
                                   const float* conv_w, const float* conv_bias,
                                   const int32_t* cu_seqlens, const int32_t* slots,
                                   const int32_t* has_init, void* conv_pool, float* ssm_pool,
                                   int32_t npool, const void* dt_raw, const float* dt_bias,
                                   const float* A, const float* D, const void* z, int64_t z_stride,
                                   void* y, int64_t y_stride, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * mamba2_state_update -- decode of T = dims->seqlen new tokens per sequence (1 to 6;
 * several tokens serve e.g. the check of drafted tokens), updating both caches in
 * place: for each token in order, the conv step above on its raw xBC, then one step of
 * the recurrence on the fp32 state. The state is read and written once per call; the
 * results are bitwise those of T one-token calls.
 *
 *   u_t        [B][T][Cc] io raw xBC of the new tokens, Cc = H*P + 2*G*N, dense
 *   w, bias    conv parameters as in mamba2_conv1d ([Cc][W], [Cc] or NULL)
 *   conv_state [B][W-1][Cc] io, updated in place (shifted by one token)
 *   dt_raw_t   [B][T][H] io, dense
 *   dt_bias, A, D as in mamba2_ssd_prefill (D may be NULL)
 *   z_t        [B][T][H*P] io or NULL
 *   ssm_state  [B][H][N][P] f32, updated in place
 *   y_t        [B][T][H*P] io; must not overlap any other argument
 *
 * With one token and fewer than (CU count / 2) (sequence, group) pairs, several
 * workgroups share a pair, and a second small kernel on the same stream shifts the
 * groups' B and C cache columns once they have all read them. The call keeps no device
 * state of its own: calls on different streams (on different caches) are independent.
 */
int mamba2_state_update(const mamba2_dims* dims, const void* u_t, const float* w,
                        const float* bias, void* conv_state, const void* dt_raw_t,
                        const float* dt_bias, const float* A, const float* D, const void* z_t,
                        float* ssm_state, void* y_t, void* stream);

/*
 * mamba2_state_update_slots -- mamba2_state_update for a continuous batch whose caches
 * live in pools (as an inference engine keeps them: neurohive, section
 * "Развертывание"): sequence b (rows b T .. b T + T - 1 of u_t, dt_raw_t, z_t, y_t)
 * updates entry slots[b] of conv_pool [npool][W-1][Cc] and ssm_pool [npool][H][N][P] in
 * place. A sequence whose entry is outside [0, npool) is skipped: its y rows are written
 * as zeros and no cache is touched. Two sequences must not share an entry (their updates
 * would race).
 *
 *   slots  [B] int32 (device), 4-byte aligned; dims->seqlen = T, 1 to 6 tokens
 *   other arguments as in mamba2_state_update (the pools in place of the caches; they may
 *   be NULL when npool == 0)
 * For an entry in range the results are bitwise those of mamba2_state_update on that
 * entry's caches.
 */
int mamba2_state_update_slots(const mamba2_dims* dims, const void* u_t, const float* w,
                              const float* bias, void* conv_pool, const void* dt_raw_t,
                              const float* dt_bias, const float* A, const float* D,
                              const void* z_t, float* ssm_pool, const int32_t* slots,
                              int32_t npool, void* y_t, void* stream);

/*
 * mamba2_group_rmsnorm -- the block's RMSNorm of the gated output (hyper.ai summary,
 * section "方法"), taken after the SiLU(z) gate over each of the G groups of
 * d_inner / G contiguous channels (d_inner = H * P):
 *     out[k] = g[k] / sqrt(mean over k's group of g^2 + eps) * weight[k]
 * It applies to the y of mamba2_ssd_prefill (B * L rows) or of mamba2_state_update
 * (dims->seqlen = 1, B rows).
 *
 *   g       [B][L][H*P] io, row stride g_stride (elements): the gated output
 *   weight  [H*P] f32, or NULL for ones
 *   eps     finite and >= 0 (the Mamba-2 block uses 1e-5)
 *   out     [B][L][H*P] io, row stride out_stride; may be g itself (same stride: in
 *           place), must not otherwise overlap g or weight
 * Each group's sum of squares is formed in fp32 in a fixed order, so results are
 * identical from run to run. d_inner / G must be a multiple of 8 (bf16) or 4 (f32),
 * which headdim 64 guarantees. With seqlen 0 the call does nothing.
 */
int mamba2_group_rmsnorm(const mamba2_dims* dims, const void* g, int64_t g_stride,
                         const float* weight, float eps, void* out, int64_t out_stride,
                         void* stream);

/*
 * The Mamba-2 mixer around the layer core: the pages' layer with its bias-free input and
 * output projections and its RMSNorm (hyper.ai summary, section "方法"; neurohive,
 * section "Архитектура": hidden width 5120 for the 12B model, 4480 after pruning to 9B,
 * expansion 2, no bias in the linear layers, RMSNorm normalisation). Per token row:
 *
 *   [z | xBC | dt_raw] = hidden * w_in^T          E = 2 H P + 2 G N + H features
 *   out_core           = the layer core on (xBC, dt_raw, z), as mamba2_conv_ssd_prefill
 *                        (prefill) or mamba2_state_update (step) computes it
 *   y_n                = mamba2_group_rmsnorm(out_core, norm_w, eps) over ngroups groups
 *   out                = y_n * w_out^T
 *
 *   hidden  [rows][d_model] io, row stride hidden_stride (rows = batch * seqlen; for the
 *           step, row b * seqlen + t is token t of sequence b)
 *   w_in    [E][d_model] io dense: rows 0 .. HP-1 give z, the next Cc give xBC (x, B, C),
 *           the last H give dt_raw (HP = nheads * 64, Cc = HP + 2 * ngroups * 128)
 *   conv_w, conv_bias, dt_bias, A, D: the layer core's parameters
 *   norm_w  [HP] f32 or NULL (= ones); eps >= 0
 *   w_out   [d_model][HP] io dense
 *   out     [rows][d_model] io, row stride out_stride
 * d_model: a positive multiple of 8 (bf16) or 4 (f32) elements, at most 2^20.
 *
 * The projections are hipBLASLt GEMMs with fp32 accumulation. The projected rows
 * [rows][Es] (Es = E rounded up to a multiple of 8), the core's output [rows][HP] and the
 * normalised output [rows][HP] are stored in io precision at the start of the workspace,
 * in that order, each at a 256-byte boundary, and stay there after the call. The first mixer call on a
 * device creates that device's hipBLASLt handle. For each new GEMM shape, the first call
 * times hipBLASLt's first choices for three workspace caps (all of it, 32 MiB, none) on
 * `stream` and keeps the fastest. That call therefore waits for the stream and must not be
 * made under graph capture. The handle and the chosen algorithms are kept until the process
 * ends. No tensor memory is allocated. MAMBA2_ERR_UNSUPPORTED when hipBLASLt has
 * no algorithm for a shape; other hipBLASLt failures return MAMBA2_ERR_HIP.
 * out, the workspace and the updated caches must not overlap each other or an input.
 */

/* mamba2_mixer_prefill_workspace_bytes -- device workspace of mamba2_mixer_prefill for
 * `dims` and d_model, 0 if they are invalid:
 *   a256(rows * Es * e) + 2 * a256(rows * HP * e) + a256(W) + 128 MiB
 * with e the io size, Es = E rounded up to a multiple of 8, W the workspace of
 * mamba2_conv_ssd_prefill for `dims`, a256 rounding up to 256 bytes. */
size_t mamba2_mixer_prefill_workspace_bytes(const mamba2_dims* dims, int32_t d_model);

/* mamba2_mixer_prefill -- the mixer over batch sequences of seqlen tokens: the layer core
 * is mamba2_conv_ssd_prefill (same dims, chunk and io settings; conv_state, h0 and h_final
 * as there). seqlen 0 only carries h0 into h_final. */
int mamba2_mixer_prefill(const mamba2_dims* dims, int32_t d_model, const void* hidden,
                         int64_t hidden_stride, const void* w_in, const float* conv_w,
                         const float* conv_bias, void* conv_state, const float* dt_bias,
                         const float* A, const float* D, const float* h0, float* h_final,
                         const float* norm_w, float eps, const void* w_out, void* out,
                         int64_t out_stride, void* workspace, size_t workspace_bytes,
                         void* stream);

/* mamba2_mixer_step_workspace_bytes -- device workspace of mamba2_mixer_step, 0 if `dims`
 * or d_model is invalid: a256(rows * Es * e) + 2 * a256(rows * HP * e) + 128 MiB. */
size_t mamba2_mixer_step_workspace_bytes(const mamba2_dims* dims, int32_t d_model);

/* mamba2_mixer_step -- the mixer for dims->seqlen = 1 .. 6 new tokens per sequence: the
 * layer core is mamba2_state_update (conv_state and ssm_state updated in place). */
int mamba2_mixer_step(const mamba2_dims* dims, int32_t d_model, const void* hidden,
                      int64_t hidden_stride, const void* w_in, const float* conv_w,
                      const float* conv_bias, void* conv_state, const float* dt_bias,
                      const float* A, const float* D, float* ssm_state, const float* norm_w,
                      float eps, const void* w_out, void* out, int64_t out_stride,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Description of the last failure on the calling thread ("" after success). */
const char* mamba2_last_error(void);

/* MAMBA2_ABI_VERSION of the built library. */
int mamba2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_H */

// C ABI of the Mamba-2 layer core: argument validation (pure host code, run
// before anything touches the device) and dispatch to the gfx950 launchers.
#include "../../include/mamba2.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.h"

#define M2_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int ok() {
  g_err.clear();
  return MAMBA2_OK;
}

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi) in bytes; empty when lo == hi
};
Range span(const void* p, int64_t rows, int64_t stride, int64_t width, int64_t esize) {
  Range r;
  if (!p || rows <= 0 || width <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (uintptr_t)(((rows - 1) * stride + width) * esize);
  return r;
}
bool overlap(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize_of(int io) { return io == MAMBA2_BF16 ? 2 : 4; }

// Checks shared by every call. `need_model` also checks the SSM shape fields.
int check_dims(const mamba2_dims* d, bool need_model) {
  if (!d) return fail(MAMBA2_ERR_NULL, "dims is NULL");
  if (d->io_dtype != MAMBA2_F32 && d->io_dtype != MAMBA2_BF16)
    return fail(MAMBA2_ERR_DTYPE, "io_dtype %d is neither MAMBA2_F32 nor MAMBA2_BF16", d->io_dtype);
  if (d->batch < 1 || d->batch > 65535) return fail(MAMBA2_ERR_SHAPE, "batch %d out of [1, 65535]", d->batch);
  if (d->seqlen < 0) return fail(MAMBA2_ERR_SHAPE, "seqlen %d < 0", d->seqlen);
  if (d->conv_width != 4) return fail(MAMBA2_ERR_UNSUPPORTED, "conv_width %d (only 4)", d->conv_width);
  if (!need_model) return MAMBA2_OK;
  if (d->nheads < 1 || d->ngroups < 1) return fail(MAMBA2_ERR_SHAPE, "nheads %d / ngroups %d < 1", d->nheads, d->ngroups);
  if (d->nheads % d->ngroups) return fail(MAMBA2_ERR_SHAPE, "nheads %d not a multiple of ngroups %d", d->nheads, d->ngroups);
  if (d->headdim != 64) return fail(MAMBA2_ERR_UNSUPPORTED, "headdim %d (only 64)", d->headdim);
  if (d->dstate != 128) return fail(MAMBA2_ERR_UNSUPPORTED, "dstate %d (only 128)", d->dstate);
  if ((int64_t)d->batch * d->nheads > (int64_t)1 << 30)
    return fail(MAMBA2_ERR_SHAPE, "batch * nheads too large");
  return MAMBA2_OK;
}

int check_stride(const char* name, const void* p, int64_t stride, int64_t width, int io) {
  int ve = 16 / esize_of(io);
  if (stride < width) return fail(MAMBA2_ERR_SHAPE, "%s stride %lld < row width %lld", name, (long long)stride, (long long)width);
  if (stride % ve) return fail(MAMBA2_ERR_ALIGN, "%s stride %lld not a multiple of 16 bytes", name, (long long)stride);
  if (!aligned16(p)) return fail(MAMBA2_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MAMBA2_OK;
}

// The prefill kernels form byte offsets inside a chunk's rows in 32 bits.
constexpr int64_t kMaxStride = (int64_t)1 << 23;

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MAMBA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

M2_EXPORT int mamba2_abi_version(void) { return MAMBA2_ABI_VERSION; }

M2_EXPORT const char* mamba2_last_error(void) { return g_err.c_str(); }

M2_EXPORT int mamba2_conv1d(const mamba2_dims* d, int32_t channels, const void* u, int64_t u_stride,
                            const float* w, const float* bias, void* conv_state, void* out,
                            int64_t out_stride, void* stream) {
  int st = check_dims(d, false);
  if (st) return st;
  if (d->seqlen == 0) return ok();  // nothing read or written; the history is unchanged
  if (!u || !w || !out) return fail(MAMBA2_ERR_NULL, "u, w and out must not be NULL");
  const int io = d->io_dtype, es = esize_of(io), ve = 16 / es;
  if (channels < 1 || channels % ve)
    return fail(MAMBA2_ERR_SHAPE, "channels %d must be a positive multiple of %d", channels, ve);
  if ((st = check_stride("u", u, u_stride, channels, io))) return st;
  if ((st = check_stride("out", out, out_stride, channels, io))) return st;
  if (!aligned16(w)) return fail(MAMBA2_ERR_ALIGN, "w is not 16-byte aligned");
  if (conv_state && !aligned16(conv_state)) return fail(MAMBA2_ERR_ALIGN, "conv_state is not 16-byte aligned");
  const int64_t BL = (int64_t)d->batch * d->seqlen;
  Range ro = span(out, BL, out_stride, channels, es);
  Range ins[] = {span(u, BL, u_stride, channels, es), span(w, 1, 0, (int64_t)channels * 4, 4),
                 span(bias, 1, 0, channels, 4),
                 span(conv_state, 1, 0, (int64_t)d->batch * 3 * channels, es)};
  for (const Range& r : ins)
    if (overlap(ro, r)) return fail(MAMBA2_ERR_ALIAS, "out overlaps an input");
  if (overlap(ins[3], ins[0])) return fail(MAMBA2_ERR_ALIAS, "conv_state overlaps u");
  if ((d->seqlen + 63) / 64 > 65535) return fail(MAMBA2_ERR_SHAPE, "seqlen too large");
  return hip_status(m2::launch_conv1d(io == MAMBA2_BF16, u, u_stride, w, bias, conv_state, out,
                                      out_stride, d->batch, d->seqlen, channels,
                                      static_cast<hipStream_t>(stream)),
                    "conv1d launch");
}

namespace {
// The chunk length is a tiling choice that leaves the result unchanged up to rounding; every
// supported value runs the same chunk-64 kernels.
bool chunk_supported(const mamba2_dims* d) { return d->chunk == 64 || d->chunk == 128 || d->chunk == 256; }
}  // namespace

M2_EXPORT size_t mamba2_ssd_prefill_workspace_bytes(const mamba2_dims* d) {
  if (check_dims(d, true) != MAMBA2_OK || !chunk_supported(d)) return 0;
  return m2::ssd_prefill_workspace(d->io_dtype == MAMBA2_BF16, d->chunk, d->batch, d->seqlen,
                                   d->nheads, d->ngroups);
}

M2_EXPORT int mamba2_ssd_prefill(const mamba2_dims* d, const void* x, int64_t x_stride,
                                 const void* Bm, int64_t b_stride, const void* Cm,
                                 int64_t c_stride, const void* dt_raw, const float* dt_bias,
                                 const float* A, const float* D, const void* z, int64_t z_stride,
                                 const float* h0, float* h_final, void* y, int64_t y_stride,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  const int io = d->io_dtype, es = esize_of(io);
  if (!chunk_supported(d))
    return fail(MAMBA2_ERR_UNSUPPORTED, "chunk %d not supported (64, 128, 256)", d->chunk);
  const size_t ws_need = m2::ssd_prefill_workspace(io == MAMBA2_BF16, d->chunk, d->batch,
                                                   d->seqlen, d->nheads, d->ngroups);
  if (!dt_bias || !A) return fail(MAMBA2_ERR_NULL, "dt_bias and A must not be NULL");
  if (d->seqlen > 0 && (!x || !Bm || !Cm || !dt_raw || !y))
    return fail(MAMBA2_ERR_NULL, "x, Bm, Cm, dt_raw and y must not be NULL when seqlen > 0");
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate;
  const int64_t BL = (int64_t)d->batch * d->seqlen;
  if ((st = check_stride("x", x, x_stride, H * P, io))) return st;
  if ((st = check_stride("Bm", Bm, b_stride, G * N, io))) return st;
  if ((st = check_stride("Cm", Cm, c_stride, G * N, io))) return st;
  if ((st = check_stride("y", y, y_stride, H * P, io))) return st;
  if (z && (st = check_stride("z", z, z_stride, H * P, io))) return st;
  if (x_stride > kMaxStride || b_stride > kMaxStride || c_stride > kMaxStride || y_stride > kMaxStride ||
      (z && z_stride > kMaxStride))
    return fail(MAMBA2_ERR_SHAPE, "row strides above 2^23 elements are not supported");
  if ((h0 && !aligned16(h0)) || (h_final && !aligned16(h_final)))
    return fail(MAMBA2_ERR_ALIGN, "h0 / h_final must be 16-byte aligned");
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need))
    return fail(MAMBA2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", ws_need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (ws_need > 0 && !aligned16(workspace))
    return fail(MAMBA2_ERR_ALIGN, "workspace is not 16-byte aligned");
  const int64_t state_elems = (int64_t)d->batch * H * N * P;
  Range ry = span(y, BL, y_stride, H * P, es);
  Range rh0 = span(h0, 1, 0, state_elems, 4), rhf = span(h_final, 1, 0, state_elems, 4);
  Range ins[] = {span(x, BL, x_stride, H * P, es),  span(Bm, BL, b_stride, G * N, es),
                 span(Cm, BL, c_stride, G * N, es), span(dt_raw, BL, H, H, es),
                 span(z, BL, z_stride, H * P, es),  rh0,
                 rhf,                               span(dt_bias, 1, 0, H, 4),
                 span(A, 1, 0, H, 4),               span(D, 1, 0, H, 4)};
  for (const Range& r : ins)
    if (overlap(ry, r)) return fail(MAMBA2_ERR_ALIAS, "y overlaps an input or the state");
  for (int i = 0; i < 5; ++i)
    if (overlap(rhf, ins[i])) return fail(MAMBA2_ERR_ALIAS, "h_final overlaps an input");
  Range rws = span(workspace, 1, 0, (int64_t)ws_need, 1);
  if (overlap(rws, ry)) return fail(MAMBA2_ERR_ALIAS, "workspace overlaps y");
  for (const Range& r : ins)
    if (overlap(rws, r)) return fail(MAMBA2_ERR_ALIAS, "workspace overlaps an input or the state");
  if (h0 && h_final && overlap(rh0, rhf) && rh0.lo != rhf.lo)
    return fail(MAMBA2_ERR_ALIAS, "h_final partially overlaps h0 (only exact in-place is allowed)");
  m2::PrefillArgs a{x, x_stride, Bm, b_stride, Cm, c_stride, dt_raw, dt_bias, A, D,
                    z, z_stride, h0, h_final, y, y_stride, workspace, d->batch, d->seqlen,
                    d->nheads, d->ngroups};
  return hip_status(m2::launch_ssd_prefill(io == MAMBA2_BF16, d->chunk, a, static_cast<hipStream_t>(stream)),
                    "ssd_prefill launch");
}

namespace {
// The conv is fused into the prefill's kernels for bf16 io; fp32 io runs the conv into the
// tail of the workspace first.
bool conv_fused(const mamba2_dims* d) { return d->io_dtype == MAMBA2_BF16; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
size_t conv_prefill_ws(const mamba2_dims* d, size_t* scan_part) {
  const size_t ws = m2::ssd_prefill_workspace(d->io_dtype == MAMBA2_BF16, d->chunk, d->batch,
                                              d->seqlen, d->nheads, d->ngroups);
  if (scan_part) *scan_part = ws;
  if (conv_fused(d) || d->seqlen == 0) return ws;
  const int64_t Cc = (int64_t)d->nheads * d->headdim + 2LL * d->ngroups * d->dstate;
  return align256(ws) + (size_t)d->batch * d->seqlen * Cc * esize_of(d->io_dtype);
}

// The launches of mamba2_conv_ssd_prefill after validation; dt_stride 0 means dense dt_raw.
int run_conv_ssd_prefill(const mamba2_dims* d, const void* xBC, int64_t xbc_stride, const float* conv_w,
                         const float* conv_bias, void* conv_state, const void* dt_raw, int64_t dt_stride,
                         const float* dt_bias, const float* A, const float* D, const void* z, int64_t z_stride,
                         const float* h0, float* h_final, void* y, int64_t y_stride, void* workspace,
                         hipStream_t s, uint64_t* phase_cycles = nullptr) {
  const int io = d->io_dtype, es = esize_of(io);
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate;
  const int64_t HP = H * P, Cc = HP + 2 * G * N;
  size_t ws_scan = 0;
  conv_prefill_ws(d, &ws_scan);
  const char* cx = static_cast<const char*>(xBC);
  if (conv_fused(d) || d->seqlen == 0) {
    m2::PrefillArgs a{xBC, xbc_stride, cx ? cx + HP * es : nullptr, xbc_stride,
                      cx ? cx + (HP + G * N) * es : nullptr, xbc_stride, dt_raw, dt_bias, A, D,
                      z, z_stride, h0, h_final, y, y_stride, workspace, d->batch, d->seqlen,
                      d->nheads, d->ngroups, dt_stride};
    if (d->seqlen == 0)   // nothing to convolve; the history is unchanged, h_final gets h0
      return hip_status(m2::launch_ssd_prefill(io == MAMBA2_BF16, d->chunk, a, s), "conv_ssd_prefill launch");
    m2::ConvArgs cv{conv_w, conv_bias, conv_state, (int)Cc};
    return hip_status(m2::launch_ssd_prefill_conv(a, cv, s, phase_cycles), "conv_ssd_prefill launch");
  }
  // the conv into the workspace's tail, then the prefill from there
  char* tail = static_cast<char*>(workspace) + align256(ws_scan);
  hipError_t e = m2::launch_conv1d(io == MAMBA2_BF16, xBC, xbc_stride, conv_w, conv_bias, conv_state,
                                   tail, Cc, d->batch, d->seqlen, (int)Cc, s);
  if (e != hipSuccess) return hip_status(e, "conv_ssd_prefill conv launch");
  m2::PrefillArgs a{tail, Cc, tail + HP * es, Cc, tail + (HP + G * N) * es, Cc, dt_raw, dt_bias, A, D,
                    z, z_stride, h0, h_final, y, y_stride, workspace, d->batch, d->seqlen,
                    d->nheads, d->ngroups, dt_stride};
  return hip_status(m2::launch_ssd_prefill(io == MAMBA2_BF16, d->chunk, a, s), "conv_ssd_prefill launch");
}
}  // namespace

M2_EXPORT size_t mamba2_conv_ssd_prefill_workspace_bytes(const mamba2_dims* d) {
  if (check_dims(d, true) != MAMBA2_OK || !chunk_supported(d)) return 0;
  return conv_prefill_ws(d, nullptr);
}

namespace {
// mamba2_conv_ssd_prefill, validated; phase_cycles non-NULL runs the scan's phase profile
int conv_ssd_prefill_checked(const mamba2_dims* d, const void* xBC, int64_t xbc_stride, const float* conv_w,
                             const float* conv_bias, void* conv_state, const void* dt_raw, const float* dt_bias,
                             const float* A, const float* D, const void* z, int64_t z_stride, const float* h0,
                             float* h_final, void* y, int64_t y_stride, void* workspace, size_t workspace_bytes,
                             void* stream, uint64_t* phase_cycles) {
  int st = check_dims(d, true);
  if (st) return st;
  const int io = d->io_dtype, es = esize_of(io);
  if (!chunk_supported(d))
    return fail(MAMBA2_ERR_UNSUPPORTED, "chunk %d not supported (64, 128, 256)", d->chunk);
  if (!dt_bias || !A || !conv_w) return fail(MAMBA2_ERR_NULL, "dt_bias, A and conv_w must not be NULL");
  if (d->seqlen > 0 && (!xBC || !dt_raw || !y))
    return fail(MAMBA2_ERR_NULL, "xBC, dt_raw and y must not be NULL when seqlen > 0");
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate;
  const int64_t HP = H * P, Cc = HP + 2 * G * N, BL = (int64_t)d->batch * d->seqlen;
  if (Cc > (int64_t)1 << 24) return fail(MAMBA2_ERR_SHAPE, "too many xBC channels");
  if ((st = check_stride("xBC", xBC, xbc_stride, Cc, io))) return st;
  if ((st = check_stride("y", y, y_stride, HP, io))) return st;
  if (z && (st = check_stride("z", z, z_stride, HP, io))) return st;
  if (xbc_stride > kMaxStride || y_stride > kMaxStride || (z && z_stride > kMaxStride))
    return fail(MAMBA2_ERR_SHAPE, "row strides above 2^23 elements are not supported");
  if (!aligned16(conv_w)) return fail(MAMBA2_ERR_ALIGN, "conv_w is not 16-byte aligned");
  if (conv_state && !aligned16(conv_state)) return fail(MAMBA2_ERR_ALIGN, "conv_state is not 16-byte aligned");
  if ((h0 && !aligned16(h0)) || (h_final && !aligned16(h_final)))
    return fail(MAMBA2_ERR_ALIGN, "h0 / h_final must be 16-byte aligned");
  size_t ws_scan = 0;
  const size_t ws_need = conv_prefill_ws(d, &ws_scan);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need))
    return fail(MAMBA2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", ws_need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (ws_need > 0 && !aligned16(workspace))
    return fail(MAMBA2_ERR_ALIGN, "workspace is not 16-byte aligned");
  const int64_t state_elems = (int64_t)d->batch * H * N * P;
  Range ry = span(y, BL, y_stride, HP, es), rcs = span(conv_state, 1, 0, (int64_t)d->batch * 3 * Cc, es);
  Range rh0 = span(h0, 1, 0, state_elems, 4), rhf = span(h_final, 1, 0, state_elems, 4);
  Range rws = span(workspace, 1, 0, (int64_t)ws_need, 1);
  // inputs read only; the first three are the per-token ones
  Range ins[] = {span(xBC, BL, xbc_stride, Cc, es), span(dt_raw, BL, H, H, es),
                 span(z, BL, z_stride, HP, es),     span(conv_w, 1, 0, Cc * 4, 4),
                 span(conv_bias, 1, 0, Cc, 4),      span(dt_bias, 1, 0, H, 4),
                 span(A, 1, 0, H, 4),               span(D, 1, 0, H, 4)};
  for (const Range& r : ins) {
    if (overlap(ry, r)) return fail(MAMBA2_ERR_ALIAS, "y overlaps an input");
    if (overlap(rcs, r)) return fail(MAMBA2_ERR_ALIAS, "conv_state overlaps an input");
    if (overlap(rws, r)) return fail(MAMBA2_ERR_ALIAS, "workspace overlaps an input");
  }
  for (int i = 0; i < 3; ++i)
    if (overlap(rhf, ins[i])) return fail(MAMBA2_ERR_ALIAS, "h_final overlaps an input");
  const Range outs[] = {ry, rcs, rhf, rws};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(MAMBA2_ERR_ALIAS, "y, conv_state, h_final and workspace must not overlap");
  for (const Range& r : {ry, rcs, rws})
    if (overlap(r, rh0)) return fail(MAMBA2_ERR_ALIAS, "y, conv_state or workspace overlaps h0");
  if (h0 && h_final && overlap(rh0, rhf) && rh0.lo != rhf.lo)
    return fail(MAMBA2_ERR_ALIAS, "h_final partially overlaps h0 (only exact in-place is allowed)");

  if (phase_cycles) {
    if (io != MAMBA2_BF16) return fail(MAMBA2_ERR_UNSUPPORTED, "the phase profile covers bf16 io");
    if (reinterpret_cast<uintptr_t>(phase_cycles) & 7u) return fail(MAMBA2_ERR_ALIGN, "phase_cycles must be 8-byte aligned");
    const Range rpc = span(phase_cycles, 1, 0, (int64_t)d->batch * H * 128, 8);
    for (const Range& r : ins)
      if (overlap(rpc, r)) return fail(MAMBA2_ERR_ALIAS, "phase_cycles overlaps an input");
    for (const Range& r : {ry, rcs, rhf, rws, rh0})
      if (overlap(rpc, r)) return fail(MAMBA2_ERR_ALIAS, "phase_cycles overlaps an output, h0 or the workspace");
  }
  return run_conv_ssd_prefill(d, xBC, xbc_stride, conv_w, conv_bias, conv_state, dt_raw, 0, dt_bias, A, D, z,
                              z_stride, h0, h_final, y, y_stride, workspace, static_cast<hipStream_t>(stream),
                              phase_cycles);
}
}  // namespace

M2_EXPORT int mamba2_conv_ssd_prefill(const mamba2_dims* d, const void* xBC, int64_t xbc_stride,
                                      const float* conv_w, const float* conv_bias, void* conv_state,
                                      const void* dt_raw, const float* dt_bias, const float* A,
                                      const float* D, const void* z, int64_t z_stride,
                                      const float* h0, float* h_final, void* y, int64_t y_stride,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return conv_ssd_prefill_checked(d, xBC, xbc_stride, conv_w, conv_bias, conv_state, dt_raw, dt_bias, A, D, z,
                                  z_stride, h0, h_final, y, y_stride, workspace, workspace_bytes, stream, nullptr);
}

M2_EXPORT int mamba2_conv_ssd_prefill_profile(const mamba2_dims* d, const void* xBC, int64_t xbc_stride,
                                              const float* conv_w, const float* conv_bias, void* conv_state,
                                              const void* dt_raw, const float* dt_bias, const float* A,
                                              const float* D, const void* z, int64_t z_stride,
                                              const float* h0, float* h_final, void* y, int64_t y_stride,
                                              void* workspace, size_t workspace_bytes, uint64_t* phase_cycles,
                                              void* stream) {
  if (!phase_cycles) return fail(MAMBA2_ERR_NULL, "phase_cycles must not be NULL");
  return conv_ssd_prefill_checked(d, xBC, xbc_stride, conv_w, conv_bias, conv_state, dt_raw, dt_bias, A, D, z,
                                  z_stride, h0, h_final, y, y_stride, workspace, workspace_bytes, stream,
                                  phase_cycles);
}

M2_EXPORT int mamba2_conv_ssd_prefill_noalloc(const mamba2_dims* d, const void* xBC, int64_t xbc_stride,
                                              const float* conv_w, const float* conv_bias, void* conv_state,
                                              const void* dt_raw, const float* dt_bias, const float* A,
                                              const float* D, const void* z, int64_t z_stride,
                                              const float* h0, float* h_final, void* y, int64_t y_stride,
                                              void* stream) {
  const int st = check_dims(d, true);
  if (st) return st;
  if (!chunk_supported(d)) return fail(MAMBA2_ERR_UNSUPPORTED, "chunk %d not supported (64, 128, 256)", d->chunk);
  const size_t need = conv_prefill_ws(d, nullptr);
  if (need > m2::PREFILL_SCRATCH_BYTES)
    return fail(MAMBA2_ERR_WORKSPACE, "needs %zu bytes of scratch; the static scratch holds %zu", need,
                m2::PREFILL_SCRATCH_BYTES);
  void* scratch = nullptr;
  const hipError_t e = m2::prefill_scratch_on_current_device(&scratch);
  if (e != hipSuccess) return hip_status(e, "static scratch address");
  return mamba2_conv_ssd_prefill(d, xBC, xbc_stride, conv_w, conv_bias, conv_state, dt_raw, dt_bias, A, D, z,
                                 z_stride, h0, h_final, y, y_stride, scratch, m2::PREFILL_SCRATCH_BYTES, stream);
}

namespace {
bool varlen_supported(const mamba2_dims* d) { return d->io_dtype == MAMBA2_BF16 && chunk_supported(d); }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
}  // namespace

M2_EXPORT size_t mamba2_conv_ssd_prefill_varlen_workspace_bytes(const mamba2_dims* d) {
  if (check_dims(d, true) != MAMBA2_OK || !varlen_supported(d)) return 0;
  return m2::ssd_prefill_varlen_workspace(d->seqlen, d->batch, d->nheads, d->ngroups);
}

M2_EXPORT int mamba2_conv_ssd_prefill_varlen(
    const mamba2_dims* d, const void* xBC, int64_t xbc_stride, const float* conv_w, const float* conv_bias,
    const int32_t* cu_seqlens, const int32_t* slots, const int32_t* has_init, void* conv_pool,
    float* ssm_pool, int32_t npool, const void* dt_raw, const float* dt_bias, const float* A,
    const float* D, const void* z, int64_t z_stride, void* y, int64_t y_stride, void* workspace,
    size_t workspace_bytes, void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  const int io = d->io_dtype, es = esize_of(io);
  if (!varlen_supported(d))
    return fail(MAMBA2_ERR_UNSUPPORTED, "the packed prefill runs with bf16 io, chunk 64, 128 or 256 (got chunk %d, %s)",
                d->chunk, io == MAMBA2_BF16 ? "bf16" : "f32");
  if (!cu_seqlens || !dt_bias || !A || !conv_w)
    return fail(MAMBA2_ERR_NULL, "cu_seqlens, dt_bias, A and conv_w must not be NULL");
  if (d->seqlen > 0 && (!xBC || !dt_raw || !y))
    return fail(MAMBA2_ERR_NULL, "xBC, dt_raw and y must not be NULL when seqlen > 0");
  if (npool < 0) return fail(MAMBA2_ERR_SHAPE, "npool %d < 0", npool);
  if (npool > 0 && (!conv_pool || !ssm_pool))
    return fail(MAMBA2_ERR_NULL, "conv_pool and ssm_pool must not be NULL when npool > 0");
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate;
  const int64_t HP = H * P, Cc = HP + 2 * G * N, T = d->seqlen, S = d->batch;
  if (Cc > (int64_t)1 << 24) return fail(MAMBA2_ERR_SHAPE, "too many xBC channels");
  if ((int64_t)G * (T / 64 + S) > ((int64_t)1 << 31) - 1 || S * H > ((int64_t)1 << 31) - 1)
    return fail(MAMBA2_ERR_SHAPE, "packed batch too large");
  if ((st = check_stride("xBC", xBC, xbc_stride, Cc, io))) return st;
  if ((st = check_stride("y", y, y_stride, HP, io))) return st;
  if (z && (st = check_stride("z", z, z_stride, HP, io))) return st;
  if (xbc_stride > kMaxStride || y_stride > kMaxStride || (z && z_stride > kMaxStride))
    return fail(MAMBA2_ERR_SHAPE, "row strides above 2^23 elements are not supported");
  if (!aligned16(conv_w) || !aligned16(conv_pool) || !aligned16(ssm_pool))
    return fail(MAMBA2_ERR_ALIGN, "conv_w, conv_pool and ssm_pool must be 16-byte aligned");
  if (!aligned4(cu_seqlens) || !aligned4(slots) || !aligned4(has_init))
    return fail(MAMBA2_ERR_ALIGN, "cu_seqlens, slots and has_init must be 4-byte aligned");
  const size_t ws_need = m2::ssd_prefill_varlen_workspace((int)T, (int)S, (int)H, (int)G);
  if (!workspace || workspace_bytes < ws_need)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", ws_need, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned16(workspace)) return fail(MAMBA2_ERR_ALIGN, "workspace is not 16-byte aligned");
  Range ry = span(y, T, y_stride, HP, es), rws = span(workspace, 1, 0, (int64_t)ws_need, 1);
  Range rcp = span(conv_pool, 1, 0, (int64_t)npool * 3 * Cc, es);
  Range rsp = span(ssm_pool, 1, 0, (int64_t)npool * H * N * P, 4);
  Range ins[] = {span(xBC, T, xbc_stride, Cc, es), span(dt_raw, T, H, H, es), span(z, T, z_stride, HP, es),
                 span(conv_w, 1, 0, Cc * 4, 4),        span(conv_bias, 1, 0, Cc, 4),
                 span(dt_bias, 1, 0, H, 4),            span(A, 1, 0, H, 4),
                 span(D, 1, 0, H, 4),                  span(cu_seqlens, 1, 0, S + 1, 4),
                 span(slots, 1, 0, S, 4),              span(has_init, 1, 0, S, 4)};
  const Range outs[] = {ry, rcp, rsp, rws};
  for (const Range& o : outs)
    for (const Range& r : ins)
      if (overlap(o, r)) return fail(MAMBA2_ERR_ALIAS, "y, the pools and the workspace must not overlap an input");
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(MAMBA2_ERR_ALIAS, "y, the pools and the workspace must not overlap");
  const char* cx = static_cast<const char*>(xBC);
  m2::PrefillArgs a{xBC, xbc_stride, cx ? cx + HP * es : nullptr, xbc_stride,
                    cx ? cx + (HP + G * N) * es : nullptr, xbc_stride, dt_raw, dt_bias, A, D,
                    z, z_stride, nullptr, nullptr, y, y_stride, workspace, d->batch, d->seqlen,
                    d->nheads, d->ngroups};
  const m2::ConvArgs cv{conv_w, conv_bias, nullptr, (int)Cc};
  const m2::VarlenArgs va{cu_seqlens, slots, has_init, ssm_pool, conv_pool, d->batch, npool};
  return hip_status(m2::launch_ssd_prefill_varlen(a, cv, va, static_cast<hipStream_t>(stream)),
                    "conv_ssd_prefill_varlen launch");
}

M2_EXPORT int mamba2_state_update(const mamba2_dims* d, const void* u_t, const float* w,
                                  const float* bias, void* conv_state, const void* dt_raw_t,
                                  const float* dt_bias, const float* A, const float* D,
                                  const void* z_t, float* ssm_state, void* y_t, void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if (d->seqlen < 1 || d->seqlen > 6)
    return fail(MAMBA2_ERR_SHAPE, "state_update takes 1 to 6 tokens per sequence (seqlen %d)", d->seqlen);
  if (!u_t || !w || !conv_state || !dt_raw_t || !dt_bias || !A || !ssm_state || !y_t)
    return fail(MAMBA2_ERR_NULL, "u_t, w, conv_state, dt_raw_t, dt_bias, A, ssm_state and y_t must not be NULL");
  const int io = d->io_dtype, es = esize_of(io);
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, B = d->batch;
  if (H / G > 256) return fail(MAMBA2_ERR_UNSUPPORTED, "more than 256 heads per group");
  const int64_t Cc = H * P + 2 * G * N;
  const void* al[] = {u_t, w, conv_state, ssm_state, y_t, z_t};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(MAMBA2_ERR_ALIGN, "u_t, w, conv_state, ssm_state, y_t, z_t must be 16-byte aligned");
  const int64_t BT = B * d->seqlen;   // token rows
  Range ry = span(y_t, BT, H * P, H * P, es);
  Range rcs = span(conv_state, 1, 0, B * 3 * Cc, es), rss = span(ssm_state, 1, 0, B * H * N * P, 4);
  Range ins[] = {span(u_t, BT, Cc, Cc, es),   span(w, 1, 0, Cc * 4, 4),   span(bias, 1, 0, Cc, 4),
                 span(dt_raw_t, BT, H, H, es), span(dt_bias, 1, 0, H, 4), span(A, 1, 0, H, 4),
                 span(D, 1, 0, H, 4),          span(z_t, BT, H * P, H * P, es)};
  for (const Range& r : ins)
    if (overlap(ry, r) || overlap(rcs, r) || overlap(rss, r))
      return fail(MAMBA2_ERR_ALIAS, "y_t, conv_state or ssm_state overlaps an input");
  if (overlap(ry, rcs) || overlap(ry, rss) || overlap(rcs, rss))
    return fail(MAMBA2_ERR_ALIAS, "y_t, conv_state and ssm_state must not overlap");
  m2::DecodeArgs a{u_t, w, bias, conv_state, dt_raw_t, dt_bias, A, D, z_t, ssm_state, y_t,
                   d->batch, d->nheads, d->ngroups, nullptr, 0, d->seqlen};
  return hip_status(m2::launch_state_update(io == MAMBA2_BF16, a, static_cast<hipStream_t>(stream)),
                    "state_update launch");
}

M2_EXPORT int mamba2_state_update_slots(const mamba2_dims* d, const void* u_t, const float* w,
                                        const float* bias, void* conv_pool, const void* dt_raw_t,
                                        const float* dt_bias, const float* A, const float* D,
                                        const void* z_t, float* ssm_pool, const int32_t* slots,
                                        int32_t npool, void* y_t, void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if (d->seqlen < 1 || d->seqlen > 6)
    return fail(MAMBA2_ERR_SHAPE, "state_update_slots takes 1 to 6 tokens per sequence (seqlen %d)", d->seqlen);
  if (!u_t || !w || !dt_raw_t || !dt_bias || !A || !y_t || !slots)
    return fail(MAMBA2_ERR_NULL, "u_t, w, dt_raw_t, dt_bias, A, slots and y_t must not be NULL");
  if (npool < 0) return fail(MAMBA2_ERR_SHAPE, "npool %d < 0", npool);
  if (npool > 0 && (!conv_pool || !ssm_pool))
    return fail(MAMBA2_ERR_NULL, "conv_pool and ssm_pool must not be NULL when npool > 0");
  const int io = d->io_dtype, es = esize_of(io);
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, B = d->batch;
  if (H / G > 256) return fail(MAMBA2_ERR_UNSUPPORTED, "more than 256 heads per group");
  const int64_t Cc = H * P + 2 * G * N;
  const void* al[] = {u_t, w, conv_pool, ssm_pool, y_t, z_t};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(MAMBA2_ERR_ALIGN, "u_t, w, conv_pool, ssm_pool, y_t, z_t must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(slots) & 3u) return fail(MAMBA2_ERR_ALIGN, "slots must be 4-byte aligned");
  const int64_t BT = B * d->seqlen;   // token rows
  Range ry = span(y_t, BT, H * P, H * P, es);
  Range rcs = span(conv_pool, 1, 0, npool * 3 * Cc, es), rss = span(ssm_pool, 1, 0, npool * H * N * P, 4);
  Range ins[] = {span(u_t, BT, Cc, Cc, es),   span(w, 1, 0, Cc * 4, 4),   span(bias, 1, 0, Cc, 4),
                 span(dt_raw_t, BT, H, H, es), span(dt_bias, 1, 0, H, 4), span(A, 1, 0, H, 4),
                 span(D, 1, 0, H, 4),          span(z_t, BT, H * P, H * P, es), span(slots, 1, 0, B, 4)};
  for (const Range& r : ins)
    if (overlap(ry, r) || overlap(rcs, r) || overlap(rss, r))
      return fail(MAMBA2_ERR_ALIAS, "y_t or a pool overlaps an input");
  if (overlap(ry, rcs) || overlap(ry, rss) || overlap(rcs, rss))
    return fail(MAMBA2_ERR_ALIAS, "y_t and the pools must not overlap");
  m2::DecodeArgs a{u_t, w, bias, conv_pool, dt_raw_t, dt_bias, A, D, z_t, ssm_pool, y_t,
                   d->batch, d->nheads, d->ngroups, slots, npool, d->seqlen};
  return hip_status(m2::launch_state_update(io == MAMBA2_BF16, a, static_cast<hipStream_t>(stream)),
                    "state_update_slots launch");
}

M2_EXPORT int mamba2_group_rmsnorm(const mamba2_dims* d, const void* g, int64_t g_stride,
                                   const float* weight, float eps, void* out, int64_t out_stride,
                                   void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if (!(eps >= 0.f) || eps > 3.4e38f) return fail(MAMBA2_ERR_SHAPE, "eps must be finite and >= 0");
  if (d->seqlen == 0) return ok();
  if (!g || !out) return fail(MAMBA2_ERR_NULL, "g and out must not be NULL");
  const int io = d->io_dtype, es = esize_of(io);
  const int64_t width = (int64_t)d->nheads * d->headdim, rows = (int64_t)d->batch * d->seqlen;
  if ((st = check_stride("g", g, g_stride, width, io))) return st;
  if ((st = check_stride("out", out, out_stride, width, io))) return st;
  if (weight && !aligned16(weight)) return fail(MAMBA2_ERR_ALIGN, "weight is not 16-byte aligned");
  Range ro = span(out, rows, out_stride, width, es), rg = span(g, rows, g_stride, width, es);
  Range rw = span(weight, 1, 0, width, 4);
  const bool in_place = out == g && out_stride == g_stride;
  if (overlap(ro, rw) || (!in_place && overlap(ro, rg)))
    return fail(MAMBA2_ERR_ALIAS, "out overlaps g (other than exactly in place) or weight");
  return hip_status(m2::launch_group_rmsnorm(io == MAMBA2_BF16, g, g_stride, weight, eps, out, out_stride,
                                             rows, d->ngroups, (int)width, static_cast<hipStream_t>(stream)),
                    "group_rmsnorm launch");
}

// ------------------------------------------------------------------------------ the mixer
namespace {
constexpr size_t kGemmWs = (size_t)128 << 20;  // hipBLASLt workspace of the mixer calls (stream-K partials)

// Workspace of the mixer calls: the projected rows [z | xBC | dt_raw] (E features, row
// stride Es, a multiple of 8 elements), the layer core's output y, the normalised output,
// the core's own workspace (prefill only) and the GEMM workspace, each at a 256-byte
// boundary. Every stage's result stays in place after the call.
struct MixerLayout {
  int64_t E = 0, Es = 0;
  size_t y_off = 0, n_off = 0, core_off = 0, gemm_off = 0, total = 0;
};
MixerLayout mixer_layout(const mamba2_dims* d, bool prefill) {
  MixerLayout l;
  const int64_t H = d->nheads, HP = H * d->headdim, Cc = HP + 2LL * d->ngroups * d->dstate;
  const int64_t rows = (int64_t)d->batch * d->seqlen;
  const size_t es = esize_of(d->io_dtype);
  l.E = HP + Cc + H;
  l.Es = (l.E + 7) & ~(int64_t)7;
  l.y_off = align256((size_t)rows * l.Es * es);
  l.n_off = l.y_off + align256((size_t)rows * HP * es);
  l.core_off = l.n_off + align256((size_t)rows * HP * es);
  l.gemm_off = l.core_off + align256(prefill ? conv_prefill_ws(d, nullptr) : 0);
  l.total = l.gemm_off + kGemmWs;
  return l;
}

int check_model_width(int32_t d_model, int io) {
  const int ve = 16 / esize_of(io);
  if (d_model < 1 || d_model % ve || d_model > (1 << 20))
    return fail(MAMBA2_ERR_SHAPE, "d_model %d must be a positive multiple of %d up to 2^20", d_model, ve);
  return MAMBA2_OK;
}

int gemm_status(int g, const std::string& msg) {
  if (g == m2::GEMM_OK) return ok();
  return fail(g == m2::GEMM_ERR_NO_ALGO ? MAMBA2_ERR_UNSUPPORTED : MAMBA2_ERR_HIP, "%s", msg.c_str());
}
}  // namespace

M2_EXPORT size_t mamba2_mixer_prefill_workspace_bytes(const mamba2_dims* d, int32_t d_model) {
  if (check_dims(d, true) != MAMBA2_OK || !chunk_supported(d) ||
      check_model_width(d_model, d->io_dtype) != MAMBA2_OK)
    return 0;
  return mixer_layout(d, true).total;
}

M2_EXPORT int mamba2_mixer_prefill(const mamba2_dims* d, int32_t d_model, const void* hidden,
                                   int64_t hidden_stride, const void* w_in, const float* conv_w,
                                   const float* conv_bias, void* conv_state, const float* dt_bias,
                                   const float* A, const float* D, const float* h0, float* h_final,
                                   const float* norm_w, float eps, const void* w_out, void* out,
                                   int64_t out_stride, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  const int io = d->io_dtype, es = esize_of(io);
  if (!chunk_supported(d))
    return fail(MAMBA2_ERR_UNSUPPORTED, "chunk %d not supported (64, 128, 256)", d->chunk);
  if ((st = check_model_width(d_model, io))) return st;
  if (!(eps >= 0.f) || eps > 3.4e38f) return fail(MAMBA2_ERR_SHAPE, "eps must be finite and >= 0");
  if (!w_in || !w_out || !conv_w || !dt_bias || !A)
    return fail(MAMBA2_ERR_NULL, "w_in, w_out, conv_w, dt_bias and A must not be NULL");
  if (d->seqlen > 0 && (!hidden || !out))
    return fail(MAMBA2_ERR_NULL, "hidden and out must not be NULL when seqlen > 0");
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, DM = d_model;
  const int64_t HP = H * P, Cc = HP + 2 * G * N, BL = (int64_t)d->batch * d->seqlen;
  if (Cc > (int64_t)1 << 24) return fail(MAMBA2_ERR_SHAPE, "too many xBC channels");
  if (d->seqlen > 0) {
    if ((st = check_stride("hidden", hidden, hidden_stride, DM, io))) return st;
    if ((st = check_stride("out", out, out_stride, DM, io))) return st;
  }
  if (!aligned16(conv_w) || (conv_state && !aligned16(conv_state)) || (h0 && !aligned16(h0)) ||
      (h_final && !aligned16(h_final)) || (norm_w && !aligned16(norm_w)))
    return fail(MAMBA2_ERR_ALIGN, "conv_w, conv_state, h0, h_final and norm_w must be 16-byte aligned");
  const MixerLayout lay = mixer_layout(d, true);
  if (lay.Es > kMaxStride) return fail(MAMBA2_ERR_SHAPE, "too many projected features");
  if (!workspace || workspace_bytes < lay.total)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", lay.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned16(workspace)) return fail(MAMBA2_ERR_ALIGN, "workspace is not 16-byte aligned");
  const int64_t state_elems = (int64_t)d->batch * H * N * P;
  Range rout = span(out, BL, out_stride, DM, es), rws = span(workspace, 1, 0, (int64_t)lay.total, 1);
  Range rcs = span(conv_state, 1, 0, (int64_t)d->batch * 3 * Cc, es);
  Range rh0 = span(h0, 1, 0, state_elems, 4), rhf = span(h_final, 1, 0, state_elems, 4);
  Range ins[] = {span(hidden, BL, hidden_stride, DM, es), span(w_in, 1, 0, (HP + Cc + H) * DM, es),
                 span(w_out, 1, 0, DM * HP, es),          span(conv_w, 1, 0, Cc * 4, 4),
                 span(conv_bias, 1, 0, Cc, 4),            span(dt_bias, 1, 0, H, 4),
                 span(A, 1, 0, H, 4),                     span(D, 1, 0, H, 4),
                 span(norm_w, 1, 0, HP, 4)};
  for (const Range& r : ins)
    for (const Range& o : {rout, rws, rcs, rhf})
      if (overlap(o, r)) return fail(MAMBA2_ERR_ALIAS, "out, workspace, conv_state or h_final overlaps an input");
  const Range outs[] = {rout, rws, rcs, rhf};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(MAMBA2_ERR_ALIAS, "out, workspace, conv_state and h_final must not overlap");
  for (const Range& r : {rout, rws, rcs})
    if (overlap(r, rh0)) return fail(MAMBA2_ERR_ALIAS, "out, workspace or conv_state overlaps h0");
  if (h0 && h_final && overlap(rh0, rhf) && rh0.lo != rhf.lo)
    return fail(MAMBA2_ERR_ALIAS, "h_final partially overlaps h0 (only exact in-place is allowed)");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  char* zx = ws;                       // [BL][Es]: z | xBC | dt_raw
  char* yb = ws + lay.y_off;           // [BL][HP]: the layer core's gated output
  char* yn = ws + lay.n_off;           // [BL][HP]: its group RMSNorm
  std::string err;
  if (BL > 0) {
    st = gemm_status(m2::gemm_nt(io == MAMBA2_BF16, BL, lay.E, DM, hidden, hidden_stride, w_in, zx, lay.Es,
                                 ws + lay.gemm_off, kGemmWs, s, &err), err);
    if (st) return st;
  }
  st = run_conv_ssd_prefill(d, BL ? zx + HP * es : nullptr, lay.Es, conv_w, conv_bias, conv_state,
                            BL ? zx + (HP + Cc) * es : nullptr, lay.Es, dt_bias, A, D, BL ? zx : nullptr, lay.Es,
                            h0, h_final, BL ? yb : nullptr, HP, ws + lay.core_off, s);
  if (st || BL == 0) return st;
  if ((st = hip_status(m2::launch_group_rmsnorm(io == MAMBA2_BF16, yb, HP, norm_w, eps, yn, HP, BL,
                                                d->ngroups, (int)HP, s),
                       "mixer norm launch")))
    return st;
  return gemm_status(m2::gemm_nt(io == MAMBA2_BF16, BL, DM, HP, yn, HP, w_out, out, out_stride,
                                 ws + lay.gemm_off, kGemmWs, s, &err), err);
}

M2_EXPORT size_t mamba2_mixer_step_workspace_bytes(const mamba2_dims* d, int32_t d_model) {
  if (check_dims(d, true) != MAMBA2_OK || d->seqlen < 1 || d->seqlen > 6 ||
      check_model_width(d_model, d->io_dtype) != MAMBA2_OK)
    return 0;
  return mixer_layout(d, false).total;
}

M2_EXPORT int mamba2_mixer_step(const mamba2_dims* d, int32_t d_model, const void* hidden,
                                int64_t hidden_stride, const void* w_in, const float* conv_w,
                                const float* conv_bias, void* conv_state, const float* dt_bias,
                                const float* A, const float* D, float* ssm_state, const float* norm_w,
                                float eps, const void* w_out, void* out, int64_t out_stride,
                                void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if (d->seqlen < 1 || d->seqlen > 6)
    return fail(MAMBA2_ERR_SHAPE, "mixer_step takes 1 to 6 tokens per sequence (seqlen %d)", d->seqlen);
  const int io = d->io_dtype, es = esize_of(io);
  if ((st = check_model_width(d_model, io))) return st;
  if (!(eps >= 0.f) || eps > 3.4e38f) return fail(MAMBA2_ERR_SHAPE, "eps must be finite and >= 0");
  if (!hidden || !w_in || !w_out || !conv_w || !conv_state || !dt_bias || !A || !ssm_state || !out)
    return fail(MAMBA2_ERR_NULL,
                "hidden, w_in, w_out, conv_w, conv_state, dt_bias, A, ssm_state and out must not be NULL");
  const int64_t H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, DM = d_model;
  if (H / G > 256) return fail(MAMBA2_ERR_UNSUPPORTED, "more than 256 heads per group");
  const int64_t HP = H * P, Cc = HP + 2 * G * N, BT = (int64_t)d->batch * d->seqlen;
  if ((st = check_stride("hidden", hidden, hidden_stride, DM, io))) return st;
  if ((st = check_stride("out", out, out_stride, DM, io))) return st;
  if (!aligned16(conv_w) || !aligned16(conv_state) || !aligned16(ssm_state) || (norm_w && !aligned16(norm_w)))
    return fail(MAMBA2_ERR_ALIGN, "conv_w, conv_state, ssm_state and norm_w must be 16-byte aligned");
  const MixerLayout lay = mixer_layout(d, false);
  if (!workspace || workspace_bytes < lay.total)
    return fail(MAMBA2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", lay.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned16(workspace)) return fail(MAMBA2_ERR_ALIGN, "workspace is not 16-byte aligned");
  Range rout = span(out, BT, out_stride, DM, es), rws = span(workspace, 1, 0, (int64_t)lay.total, 1);
  Range rcs = span(conv_state, 1, 0, (int64_t)d->batch * 3 * Cc, es);
  Range rss = span(ssm_state, 1, 0, (int64_t)d->batch * H * N * P, 4);
  Range ins[] = {span(hidden, BT, hidden_stride, DM, es), span(w_in, 1, 0, (HP + Cc + H) * DM, es),
                 span(w_out, 1, 0, DM * HP, es),          span(conv_w, 1, 0, Cc * 4, 4),
                 span(conv_bias, 1, 0, Cc, 4),            span(dt_bias, 1, 0, H, 4),
                 span(A, 1, 0, H, 4),                     span(D, 1, 0, H, 4),
                 span(norm_w, 1, 0, HP, 4)};
  const Range outs[] = {rout, rws, rcs, rss};
  for (const Range& r : ins)
    for (const Range& o : outs)
      if (overlap(o, r)) return fail(MAMBA2_ERR_ALIAS, "out, workspace, conv_state or ssm_state overlaps an input");
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(MAMBA2_ERR_ALIAS, "out, workspace, conv_state and ssm_state must not overlap");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  char* zx = ws;
  char* yb = ws + lay.y_off;
  char* yn = ws + lay.n_off;
  std::string err;
  st = gemm_status(m2::gemm_nt(io == MAMBA2_BF16, BT, lay.E, DM, hidden, hidden_stride, w_in, zx, lay.Es,
                               ws + lay.gemm_off, kGemmWs, s, &err), err);
  if (st) return st;
  m2::DecodeArgs a{zx + HP * es, conv_w, conv_bias, conv_state, zx + (HP + Cc) * es, dt_bias, A, D, zx,
                   ssm_state, yb, d->batch, d->nheads, d->ngroups, nullptr, 0, d->seqlen};
  a.u_stride = a.z_stride = a.dt_stride = lay.Es;
  if ((st = hip_status(m2::launch_state_update(io == MAMBA2_BF16, a, s), "mixer state_update launch"))) return st;
  if ((st = hip_status(m2::launch_group_rmsnorm(io == MAMBA2_BF16, yb, HP, norm_w, eps, yn, HP, BT,
                                                d->ngroups, (int)HP, s),
                       "mixer norm launch")))
    return st;
  return gemm_status(m2::gemm_nt(io == MAMBA2_BF16, BT, DM, HP, yn, HP, w_out, out, out_stride,
                                 ws + lay.gemm_off, kGemmWs, s, &err), err);
}

"""Python binding of libmamba2.so, the gfx950 Mamba-2 layer core.

Argument marshalling only: every step of the layer runs in the HIP kernels of
the C library (include/mamba2.h). Torch is used for device memory and the
current stream. There is no CPU fallback: if the library is missing, importing
this package raises.

Functions take torch CUDA tensors (bf16 or fp32 io, fp32 parameters and states)
and enqueue on ``torch.cuda.current_stream()``; they return nothing and raise
``Mamba2Error`` on a nonzero status.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "LIB_PATH", "Mamba2Error", "Dims", "lib", "io_dtype_of",
    "mamba2_conv1d", "mamba2_ssd_prefill", "mamba2_state_update",
    "mamba2_ssd_prefill_workspace_bytes", "mamba2_conv_ssd_prefill",
    "mamba2_conv_ssd_prefill_workspace_bytes", "mamba2_conv_ssd_prefill_varlen",
    "mamba2_conv_ssd_prefill_varlen_workspace_bytes", "mamba2_group_rmsnorm",
    "mamba2_state_update_slots", "mamba2_mixer_prefill", "mamba2_mixer_prefill_workspace_bytes",
    "mamba2_mixer_step", "mamba2_mixer_step_workspace_bytes",
    "mamba2_abi_version", "mamba2_last_error",
    "MAMBA2_F32", "MAMBA2_BF16", "STATUS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmamba2.so")

MAMBA2_F32, MAMBA2_BF16 = 0, 1
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_UNSUPPORTED", 4: "ERR_DTYPE",
          5: "ERR_ALIGN", 6: "ERR_ALIAS", 7: "ERR_WORKSPACE", 8: "ERR_HIP"}


class Mamba2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "seqlen", "nheads", "headdim", "ngroups", "dstate", "conv_width",
                 "chunk", "io_dtype")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m state_space_sequence_causal_amd.build`")

# torch first: it loads its own HIP runtime (soname libamdhip64.so.7), and the
# library's dependency of the same soname must bind to that one, so that device
# pointers and streams handed over from torch belong to the runtime that
# launches the kernels.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_dims = ctypes.POINTER(Dims)
lib.mamba2_abi_version.restype = ctypes.c_int
lib.mamba2_last_error.restype = ctypes.c_char_p
lib.mamba2_conv1d.argtypes = [_dims, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp]
lib.mamba2_ssd_prefill_workspace_bytes.argtypes = [_dims]
lib.mamba2_ssd_prefill_workspace_bytes.restype = _sz
lib.mamba2_ssd_prefill.argtypes = [_dims, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                   _i64, _vp, _vp, _vp, _i64, _vp, _sz, _vp]
lib.mamba2_conv_ssd_prefill_workspace_bytes.argtypes = [_dims]
lib.mamba2_conv_ssd_prefill_workspace_bytes.restype = _sz
lib.mamba2_conv_ssd_prefill.argtypes = [_dims, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _i64, _vp, _vp, _vp, _i64, _vp, _sz, _vp]
lib.mamba2_conv_ssd_prefill_profile.argtypes = [_dims, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _i64, _vp, _vp, _vp, _i64, _vp, _sz, _vp, _vp]
lib.mamba2_conv_ssd_prefill_noalloc.argtypes = [_dims, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _i64, _vp, _vp, _vp, _i64, _vp]
lib.mamba2_conv_ssd_prefill_varlen_workspace_bytes.argtypes = [_dims]
lib.mamba2_conv_ssd_prefill_varlen_workspace_bytes.restype = _sz
lib.mamba2_conv_ssd_prefill_varlen.argtypes = [_dims, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                               _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp]
lib.mamba2_state_update.argtypes = [_dims, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.mamba2_state_update_slots.argtypes = [_dims, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _i32, _vp, _vp]
lib.mamba2_group_rmsnorm.argtypes = [_dims, _vp, _i64, _vp, ctypes.c_float, _vp, _i64, _vp]
lib.mamba2_mixer_prefill_workspace_bytes.argtypes = [_dims, _i32]
lib.mamba2_mixer_prefill_workspace_bytes.restype = _sz
lib.mamba2_mixer_prefill.argtypes = [_dims, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_float, _vp, _vp, _i64, _vp, _sz, _vp]
lib.mamba2_mixer_step_workspace_bytes.argtypes = [_dims, _i32]
lib.mamba2_mixer_step_workspace_bytes.restype = _sz
lib.mamba2_mixer_step.argtypes = [_dims, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_float, _vp, _vp, _i64, _vp, _sz, _vp]
for _f in ("mamba2_conv1d", "mamba2_ssd_prefill", "mamba2_conv_ssd_prefill", "mamba2_conv_ssd_prefill_varlen",
           "mamba2_state_update", "mamba2_state_update_slots", "mamba2_group_rmsnorm", "mamba2_mixer_prefill",
           "mamba2_mixer_step"):
    getattr(lib, _f).restype = ctypes.c_int


def mamba2_abi_version() -> int:
    return lib.mamba2_abi_version()


def mamba2_last_error() -> str:
    return lib.mamba2_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise Mamba2Error(status, mamba2_last_error())


def io_dtype_of(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MAMBA2_BF16
    if t.dtype == torch.float32:
        return MAMBA2_F32
    raise Mamba2Error(4, f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _row_stride(t) -> int:
    """Token-row stride (elements) of a [.., L, width] view whose rows are evenly spaced."""
    if t.numel() == 0:
        return t.shape[-1]
    if t.stride(-1) != 1:
        raise Mamba2Error(2, "the last dimension must be contiguous")
    return t.stride(-2)


def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_dims(batch, seqlen, nheads, ngroups, chunk, io, headdim=64, dstate=128, conv_width=4) -> Dims:
    return Dims(batch, seqlen, nheads, headdim, ngroups, dstate, conv_width, chunk, io)


def mamba2_conv1d(u, w, bias, conv_state, out) -> None:
    """out = SiLU(causal depthwise conv1d(u) + bias); conv_state updated in place (or None)."""
    B, L, Cc = u.shape
    d = make_dims(B, L, 1, 1, 64, io_dtype_of(u))
    _check(lib.mamba2_conv1d(ctypes.byref(d), Cc, _ptr(u), _row_stride(u), _ptr(w), _ptr(bias),
                             _ptr(conv_state), _ptr(out), _row_stride(out), _stream()))


def mamba2_ssd_prefill_workspace_bytes(d: Dims) -> int:
    return lib.mamba2_ssd_prefill_workspace_bytes(ctypes.byref(d))


def mamba2_ssd_prefill(x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, h_final, y, *, ngroups: int,
                       chunk: int, workspace=None) -> None:
    """The chunked selective scan; x/Bm/Cm/z/y may be row-strided views (e.g. slices of xBC)."""
    B, L, H = dt_raw.shape
    d = make_dims(B, L, H, ngroups, chunk, io_dtype_of(x))
    if workspace is None:
        need = lib.mamba2_ssd_prefill_workspace_bytes(ctypes.byref(d))
        if need:
            import torch
            workspace = torch.empty(need, dtype=torch.uint8, device=dt_raw.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mamba2_ssd_prefill(
        ctypes.byref(d), _ptr(x), _row_stride(x), _ptr(Bm), _row_stride(Bm), _ptr(Cm),
        _row_stride(Cm), _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(z),
        0 if z is None else _row_stride(z), _ptr(h0), _ptr(h_final), _ptr(y), _row_stride(y),
        _ptr(workspace), ws_bytes, _stream()))


def mamba2_conv_ssd_prefill_workspace_bytes(d: Dims) -> int:
    return lib.mamba2_conv_ssd_prefill_workspace_bytes(ctypes.byref(d))


def mamba2_conv_ssd_prefill(xBC, conv_w, conv_bias, conv_state, dt_raw, dt_bias, A, D, z, h0,
                            h_final, y, *, ngroups: int, chunk: int, workspace=None) -> None:
    """conv1d over the raw xBC ([B, L, Cc], row-strided) then the scan, in one call;
    conv_state ([B, 3, Cc] or None) is updated in place."""
    B, L, H = dt_raw.shape
    d = make_dims(B, L, H, ngroups, chunk, io_dtype_of(xBC))
    if workspace is None:
        need = lib.mamba2_conv_ssd_prefill_workspace_bytes(ctypes.byref(d))
        if need:
            import torch
            workspace = torch.empty(need, dtype=torch.uint8, device=dt_raw.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mamba2_conv_ssd_prefill(
        ctypes.byref(d), _ptr(xBC), _row_stride(xBC), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state),
        _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(z), 0 if z is None else _row_stride(z),
        _ptr(h0), _ptr(h_final), _ptr(y), _row_stride(y), _ptr(workspace), ws_bytes, _stream()))


def mamba2_conv_ssd_prefill_profile(xBC, conv_w, conv_bias, conv_state, dt_raw, dt_bias, A, D, z, h0,
                                    h_final, y, phase_cycles, *, ngroups: int, chunk: int, workspace) -> None:
    """mamba2_conv_ssd_prefill with the scan's phase profile written to phase_cycles (an int64
    device tensor of batch * nheads * 128 elements)."""
    B, L, H = dt_raw.shape
    d = make_dims(B, L, H, ngroups, chunk, io_dtype_of(xBC))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.mamba2_conv_ssd_prefill_profile(
        ctypes.byref(d), _ptr(xBC), _row_stride(xBC), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state),
        _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(z), 0 if z is None else _row_stride(z),
        _ptr(h0), _ptr(h_final), _ptr(y), _row_stride(y), _ptr(workspace), ws_bytes, _ptr(phase_cycles),
        _stream()))


def mamba2_conv_ssd_prefill_noalloc(xBC, conv_w, conv_bias, conv_state, dt_raw, dt_bias, A, D, z, h0,
                                    h_final, y, *, ngroups: int, chunk: int) -> None:
    """mamba2_conv_ssd_prefill with the library's static device scratch as its workspace
    (no allocation by the call)."""
    B, L, H = dt_raw.shape
    d = make_dims(B, L, H, ngroups, chunk, io_dtype_of(xBC))
    _check(lib.mamba2_conv_ssd_prefill_noalloc(
        ctypes.byref(d), _ptr(xBC), _row_stride(xBC), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state),
        _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(z), 0 if z is None else _row_stride(z),
        _ptr(h0), _ptr(h_final), _ptr(y), _row_stride(y), _stream()))


def mamba2_conv_ssd_prefill_varlen_workspace_bytes(d: Dims) -> int:
    return lib.mamba2_conv_ssd_prefill_varlen_workspace_bytes(ctypes.byref(d))


def mamba2_conv_ssd_prefill_varlen(xBC, conv_w, conv_bias, cu_seqlens, slots, has_init, conv_pool,
                                   ssm_pool, dt_raw, dt_bias, A, D, z, y, *, ngroups: int,
                                   workspace=None) -> None:
    """The one-call prefill over packed sequences (xBC [T, Cc] rows, cu_seqlens int32 [S+1]),
    states in slot pools (conv_pool [npool, 3, Cc], ssm_pool [npool, H, N, P]); slots and
    has_init are int32 [S] or None. bf16 io, chunk 64."""
    T, H = dt_raw.shape
    S = cu_seqlens.numel() - 1
    npool = 0 if ssm_pool is None else ssm_pool.shape[0]
    d = make_dims(S, T, H, ngroups, 64, io_dtype_of(xBC))
    if workspace is None:
        import torch
        workspace = torch.empty(lib.mamba2_conv_ssd_prefill_varlen_workspace_bytes(ctypes.byref(d)),
                                dtype=torch.uint8, device=dt_raw.device)
    ws_bytes = workspace.numel() * workspace.element_size()

    def rs(t):
        if t.numel() == 0:
            return t.shape[-1]
        if t.stride(-1) != 1:
            raise Mamba2Error(2, "the last dimension must be contiguous")
        return t.stride(0)
    _check(lib.mamba2_conv_ssd_prefill_varlen(
        ctypes.byref(d), _ptr(xBC), rs(xBC), _ptr(conv_w), _ptr(conv_bias), _ptr(cu_seqlens), _ptr(slots),
        _ptr(has_init), _ptr(conv_pool), _ptr(ssm_pool), npool, _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(D),
        _ptr(z), 0 if z is None else rs(z), _ptr(y), rs(y), _ptr(workspace), ws_bytes, _stream()))


def _decode_shape(dt_raw_t):
    """(B, T, H) of a decode call: dt_raw_t is [B, H] (one token) or [B, T, H]."""
    if dt_raw_t.dim() == 2:
        B, H = dt_raw_t.shape
        return B, 1, H
    return tuple(dt_raw_t.shape)


def mamba2_state_update(u_t, w, bias, conv_state, dt_raw_t, dt_bias, A, D, z_t, ssm_state, y_t,
                        *, ngroups: int) -> None:
    """Decode of one token ([B, ...] rows) or of T tokens per sequence ([B, T, ...] rows, T up
    to 6); conv_state and ssm_state are updated in place."""
    B, T, H = _decode_shape(dt_raw_t)
    d = make_dims(B, T, H, ngroups, 64, io_dtype_of(u_t))
    _check(lib.mamba2_state_update(ctypes.byref(d), _ptr(u_t), _ptr(w), _ptr(bias), _ptr(conv_state),
                                   _ptr(dt_raw_t), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(z_t),
                                   _ptr(ssm_state), _ptr(y_t), _stream()))


def mamba2_state_update_slots(u_t, w, bias, conv_pool, dt_raw_t, dt_bias, A, D, z_t, ssm_pool, slots, y_t,
                              *, ngroups: int) -> None:
    """Decode over cache pools: sequence b (one token, or T tokens with [B, T, ...] rows)
    updates pool entry slots[b] (int32 [B]) of conv_pool [npool, 3, Cc] and
    ssm_pool [npool, H, N, P] in place."""
    B, T, H = _decode_shape(dt_raw_t)
    npool = 0 if ssm_pool is None else ssm_pool.shape[0]
    d = make_dims(B, T, H, ngroups, 64, io_dtype_of(u_t))
    _check(lib.mamba2_state_update_slots(ctypes.byref(d), _ptr(u_t), _ptr(w), _ptr(bias), _ptr(conv_pool),
                                         _ptr(dt_raw_t), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(z_t),
                                         _ptr(ssm_pool), _ptr(slots), npool, _ptr(y_t), _stream()))


def mamba2_group_rmsnorm(g, weight, out, *, ngroups: int, eps: float = 1e-5) -> None:
    """Group RMSNorm of the gated output g ([B, L, H*P] or [B, H*P]) into out (may be g)."""
    if g.dim() == 2:
        B, W = g.shape
        L = 1
        gs, os_ = (g.stride(0) if g.numel() else W), (out.stride(0) if out.numel() else W)
        if g.stride(-1) != 1 or out.stride(-1) != 1:
            raise Mamba2Error(2, "the last dimension must be contiguous")
    else:
        B, L, W = g.shape
        gs, os_ = _row_stride(g), _row_stride(out)
    d = make_dims(B, L, W // 64, ngroups, 64, io_dtype_of(g))
    _check(lib.mamba2_group_rmsnorm(ctypes.byref(d), _ptr(g), gs, _ptr(weight), float(eps), _ptr(out),
                                    os_, _stream()))


def _workspace(need: int, like):
    import torch
    return torch.empty(need, dtype=torch.uint8, device=like.device)


def mamba2_mixer_prefill_workspace_bytes(d: Dims, d_model: int) -> int:
    return lib.mamba2_mixer_prefill_workspace_bytes(ctypes.byref(d), int(d_model))


def mamba2_mixer_prefill(hidden, w_in, conv_w, conv_bias, conv_state, dt_bias, A, D, h0, h_final, norm_w,
                         w_out, out, *, ngroups: int, chunk: int, eps: float = 1e-5, workspace=None) -> None:
    """The Mamba-2 mixer over hidden [B, L, d_model]: in-projection (w_in [E, d_model]),
    the layer core as mamba2_conv_ssd_prefill, group RMSNorm (norm_w [H*P] or None),
    out-projection (w_out [d_model, H*P]) into out [B, L, d_model]."""
    B, L, DM = hidden.shape
    H = dt_bias.shape[0]
    d = make_dims(B, L, H, ngroups, chunk, io_dtype_of(hidden))
    if workspace is None:
        workspace = _workspace(lib.mamba2_mixer_prefill_workspace_bytes(ctypes.byref(d), DM), hidden)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.mamba2_mixer_prefill(
        ctypes.byref(d), DM, _ptr(hidden), _row_stride(hidden), _ptr(w_in), _ptr(conv_w), _ptr(conv_bias),
        _ptr(conv_state), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(h0), _ptr(h_final), _ptr(norm_w), float(eps),
        _ptr(w_out), _ptr(out), _row_stride(out), _ptr(workspace), ws_bytes, _stream()))


def mamba2_mixer_step_workspace_bytes(d: Dims, d_model: int) -> int:
    return lib.mamba2_mixer_step_workspace_bytes(ctypes.byref(d), int(d_model))


def mamba2_mixer_step(hidden, w_in, conv_w, conv_bias, conv_state, dt_bias, A, D, ssm_state, norm_w, w_out,
                      out, *, ngroups: int, eps: float = 1e-5, workspace=None) -> None:
    """The mixer for T = 1 .. 6 new tokens per sequence: hidden and out [B, T, d_model] (or
    [B, d_model] for one token); the layer core is mamba2_state_update, conv_state and
    ssm_state are updated in place."""
    if hidden.dim() == 2:
        hidden, out = hidden.unsqueeze(1), out.unsqueeze(1)
    B, T, DM = hidden.shape
    H = dt_bias.shape[0]
    d = make_dims(B, T, H, ngroups, 64, io_dtype_of(hidden))
    if workspace is None:
        workspace = _workspace(lib.mamba2_mixer_step_workspace_bytes(ctypes.byref(d), DM), hidden)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.mamba2_mixer_step(
        ctypes.byref(d), DM, _ptr(hidden), _row_stride(hidden), _ptr(w_in), _ptr(conv_w), _ptr(conv_bias),
        _ptr(conv_state), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(ssm_state), _ptr(norm_w), float(eps),
        _ptr(w_out), _ptr(out), _row_stride(out), _ptr(workspace), ws_bytes, _stream()))

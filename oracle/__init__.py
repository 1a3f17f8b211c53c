"""fp64 oracle of the Mamba-2 layer core -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never links, calls
or falls back to it.

The arithmetic lives in ``mamba2_oracle.c`` (gcc, double precision) and in
``brute.py`` (numpy, unrolled products); this module only builds and marshals.
Every input is converted to float64 from its exact stored value (bf16 or fp32).

Every function here has pins of its own, listed in the docstrings of the test
modules (tests/test_oracle_*.py); none is "parity unpinned".

Two builds of the same source: ``build`` (gcc -O2, used by the tests and the smoke
check) and ``build_native`` (gcc -O3 -march=native, compiled on the host that runs it,
used only to time the oracle as the CPU baseline). Neither uses fast-math, and both
keep every product and sum a separate rounding (-ffp-contract=off), so the two give
the same bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)
_L = ctypes.c_long


_FLAGS = ["-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-ffp-contract=off"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no fast-math, no -march=native)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", *_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_native(out_dir: str) -> str:
    """Compile the same source with gcc -O3 -march=native (no fast-math, no contraction)
    into ``out_dir`` on this host, for timing the oracle where it runs. The library is
    built fresh each time: the one that ships is built for the machine that built it."""
    lib = os.path.join(out_dir, "liboracle_native.so")
    subprocess.check_call(["gcc", "-O3", "-march=native", *_FLAGS, "-o", lib, _SRC, "-lm"])
    return lib


def load_native(out_dir: str):
    """Builds (build_native) and loads the tuned oracle; returns a handle for ``use``."""
    return _bind(ctypes.CDLL(build_native(out_dir)))


class use:
    """Context manager: the module's functions call ``lib`` (a handle from load_native)
    instead of the default build while inside the block."""

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global _lib
        self.saved, _lib = _load(), self.lib
        return self.lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    lib.oracle_threads.argtypes = [ctypes.c_int]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_conv1d.argtypes = [_L, _L, _L, _L, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
    scan = [_L] * 6 + [_dp] * 11 + [_ip, _L, ctypes.c_int]
    lib.oracle_ssd_scan.argtypes = scan
    lib.oracle_ssd_chunked.argtypes = [_L] * 7 + [_dp] * 11 + [_ip, _L, ctypes.c_int]
    lib.oracle_state_update.argtypes = [_L] * 6 + [_dp] * 3 + [_dp] + [_dp] * 4 + [_dp, _dp, _dp, ctypes.c_int]
    lib.oracle_group_rmsnorm.argtypes = [_L, _L, _L, _dp, _dp, ctypes.c_double, _dp]
    for f in ("oracle_conv1d", "oracle_ssd_scan", "oracle_ssd_chunked", "oracle_state_update",
              "oracle_group_rmsnorm"):
        getattr(lib, f).restype = None
    return lib


def _d(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(_dp)


def threads(requested: int = 0) -> int:
    return _load().oracle_threads(int(requested))


def conv1d(u, w, bias=None, state_in=None, nthreads: int = 0):
    """u [B][L][Cc] -> (out [B][L][Cc], state_out [B][W-1][Cc]); fp64."""
    u, w, bias, state_in = _d(u), _d(w), _d(bias), _d(state_in)
    B, L, Cc = u.shape
    W = w.shape[1]
    out = np.empty_like(u)
    st = np.empty((B, W - 1, Cc), dtype=np.float64)
    _load().oracle_conv1d(B, L, Cc, W, _p(u), _p(w), _p(bias), _p(state_in), _p(out), _p(st),
                          int(nthreads))
    return out, st


def _scan_args(x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, ngroups):
    x, Bm, Cm, dt_raw = _d(x), _d(Bm), _d(Cm), _d(dt_raw)
    dt_bias, A, D, z, h0 = _d(dt_bias), _d(A), _d(D), _d(z), _d(h0)
    B, L, H = dt_raw.shape
    P = x.shape[2] // H
    N = Bm.shape[2] // ngroups
    return x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, B, L, H, P, N


def _heads(heads):
    if heads is None:
        return None, 0, None
    arr = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    return arr, len(arr), arr.ctypes.data_as(_ip)


def ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D=None, z=None, h0=None, *, ngroups: int,
             heads: Optional[Sequence[int]] = None, nthreads: int = 0, y_out=None):
    """O1: the recurrence token by token. Returns (y [B][L][H*P], h_final [B][H][N][P])."""
    x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, B, L, H, P, N = _scan_args(
        x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, ngroups)
    y = np.zeros((B, L, H * P)) if y_out is None else y_out
    hf = np.zeros((B, H, N, P))
    keep, n_sel, hp = _heads(heads)
    _load().oracle_ssd_scan(B, L, H, P, ngroups, N, _p(x), _p(Bm), _p(Cm), _p(dt_raw),
                            _p(dt_bias), _p(A), _p(D), _p(z), _p(h0), _p(y), _p(hf), hp, n_sel,
                            int(nthreads))
    del keep
    return y, hf


def ssd_chunked(x, Bm, Cm, dt_raw, dt_bias, A, D=None, z=None, h0=None, *, ngroups: int,
                chunk: int, heads: Optional[Sequence[int]] = None, nthreads: int = 0):
    """O2: chunk-by-chunk evaluation of the same map."""
    x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, B, L, H, P, N = _scan_args(
        x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, ngroups)
    y = np.zeros((B, L, H * P))
    hf = np.zeros((B, H, N, P))
    keep, n_sel, hp = _heads(heads)
    _load().oracle_ssd_chunked(B, L, H, P, ngroups, N, int(chunk), _p(x), _p(Bm), _p(Cm),
                               _p(dt_raw), _p(dt_bias), _p(A), _p(D), _p(z), _p(h0), _p(y),
                               _p(hf), hp, n_sel, int(nthreads))
    del keep
    return y, hf


def state_update(u_t, w, bias, conv_state, dt_raw_t, dt_bias, A, D, z_t, ssm_state, *,
                 nheads: int, ngroups: int, headdim: int = 64, dstate: int = 128,
                 nthreads: int = 0):
    """One decode token. Returns (y_t [B][H*P], conv_state', ssm_state') as new arrays."""
    u_t, w, bias, dt_raw_t = _d(u_t), _d(w), _d(bias), _d(dt_raw_t)
    dt_bias, A, D, z_t = _d(dt_bias), _d(A), _d(D), _d(z_t)
    cs = np.array(conv_state, dtype=np.float64, copy=True, order="C")
    ss = np.array(ssm_state, dtype=np.float64, copy=True, order="C")
    B = u_t.shape[0]
    y = np.zeros((B, nheads * headdim))
    _load().oracle_state_update(B, nheads, headdim, ngroups, dstate, w.shape[1], _p(u_t), _p(w),
                                _p(bias), _p(cs), _p(dt_raw_t), _p(dt_bias), _p(A), _p(D),
                                _p(z_t), _p(ss), _p(y), int(nthreads))
    return y, cs, ss


def state_update_tokens(u, w, bias, conv_state, dt_raw, dt_bias, A, D, z, ssm_state, *,
                        nheads: int, ngroups: int):
    """T decode tokens per sequence, in order: u [B][T][Cc], dt_raw [B][T][H], z [B][T][H*P]
    or None; state_update applied to one token after the other. Returns
    (y [B][T][H*P], conv_state', ssm_state')."""
    u, dt_raw = _d(u), _d(dt_raw)
    z = None if z is None else _d(z)
    B, T = u.shape[0], u.shape[1]
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    ss = np.array(ssm_state, dtype=np.float64, copy=True)
    y = np.zeros((B, T, nheads * 64))
    for t in range(T):
        y[:, t], cs, ss = state_update(u[:, t], w, bias, cs, dt_raw[:, t], dt_bias, A, D,
                                       None if z is None else z[:, t], ss, nheads=nheads,
                                       ngroups=ngroups)
    return y, cs, ss


def group_rmsnorm(g, weight=None, *, ngroups: int, eps: float = 1e-5):
    """Group RMSNorm of the gated output g [..][width]: each row is cut into ngroups
    contiguous groups, each scaled by 1 / sqrt(mean of squares + eps), then by weight."""
    g = _d(g)
    width = g.shape[-1]
    if width % ngroups:
        raise ValueError("width must be a multiple of ngroups")
    rows = g.size // width
    out = np.empty_like(g)
    _load().oracle_group_rmsnorm(rows, width, ngroups, _p(g), _p(_d(weight)), float(eps), _p(out))
    return out


def split_xbc(xbc, nheads: int, ngroups: int, headdim: int = 64, dstate: int = 128):
    """Views of the x, B and C channel ranges of an xBC tensor [..][Cc]."""
    di, gn = nheads * headdim, ngroups * dstate
    return xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:di + 2 * gn]


def round_bf16(a):
    """Each value stored as bfloat16: rounded to float32, then to 8 significand bits by
    round-to-nearest-even on its bit pattern (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def conv_ssd_prefill_varlen(xbc, cu_seqlens, slots, has_init, conv_pool, ssm_pool, conv_w, conv_b,
                            dt_raw, dt_bias, A, D=None, z=None, *, nheads: int, ngroups: int,
                            io: str = "f32"):
    """The serving form of the prefill: packed sequences of different lengths whose states
    live in slot pools. Sequence i is rows cu_seqlens[i] .. cu_seqlens[i+1] of xbc, dt_raw
    and z; it starts from the history conv_pool[slots[i]] and the state ssm_pool[slots[i]]
    when has_init[i] is nonzero (else from zeros), runs conv1d and then ssd_scan on its own
    rows, and, when 0 <= slots[i] < npool, leaves its last three raw rows (history first)
    and its final state in that entry. slots None means entry i; has_init None means all
    zero. With io "bf16" the conv output is stored as bf16 before the scan reads it, as the
    library stores it in that io type. This is conv1d and ssd_scan applied one sequence at a
    time.

    Returns (y [T][H*P], conv_pool', ssm_pool') with new pool arrays."""
    xbc = _d(xbc)
    dt_raw = _d(dt_raw)
    z = None if z is None else _d(z)
    cu = [int(v) for v in np.asarray(cu_seqlens)]
    S = len(cu) - 1
    conv_pool = np.array(_d(conv_pool), copy=True) if conv_pool is not None else None
    ssm_pool = np.array(_d(ssm_pool), copy=True) if ssm_pool is not None else None
    npool = 0 if ssm_pool is None else ssm_pool.shape[0]
    Cc = xbc.shape[-1]
    N, P = 128, 64
    y = np.zeros((xbc.shape[0], nheads * P))
    for i in range(S):
        a, b = cu[i], cu[i + 1]
        s = i if slots is None else int(slots[i])
        has_slot = 0 <= s < npool
        init = has_slot and has_init is not None and int(has_init[i]) != 0
        hist = conv_pool[s][None] if init else np.zeros((1, 3, Cc))
        h0 = ssm_pool[s][None] if init else np.zeros((1, nheads, N, P))
        if b > a:
            xr, hist_new = conv1d(xbc[None, a:b], conv_w, conv_b, hist)
            if io == "bf16":
                xr = round_bf16(xr)
            x, Bm, Cm = split_xbc(xr, nheads, ngroups)
            yi, hf = ssd_scan(x, Bm, Cm, dt_raw[None, a:b], dt_bias, A, D,
                              None if z is None else z[None, a:b], h0, ngroups=ngroups)
            y[a:b] = yi[0]
        else:   # an empty sequence keeps its history and state
            hist_new, hf = hist, h0
        if has_slot:
            conv_pool[s] = hist_new[0]
            ssm_pool[s] = hf[0]
    return y, conv_pool, ssm_pool


def _project(rows, w):
    """rows [..][K] times w[N][K] transposed, in fp64 (numpy matmul)."""
    rows, w = _d(rows), _d(w)
    return (rows.reshape(-1, rows.shape[-1]) @ w.T).reshape(rows.shape[:-1] + (w.shape[0],))


def _split_projected(zx, nheads: int, ngroups: int):
    """The in-projection's columns in the order z | xBC | dt_raw."""
    di = nheads * 64
    Cc = di + 2 * ngroups * 128
    return zx[..., :di], zx[..., di:di + Cc], zx[..., di + Cc:di + Cc + nheads]


def mixer_prefill(hidden, w_in, conv_w, conv_b, conv_state, dt_bias, A, D, h0, norm_w, w_out, *,
                  nheads: int, ngroups: int, eps: float = 1e-5, io: str = "f32"):
    """The Mamba-2 mixer around the layer core: the Nemotron-Nano-2 layer with its bias-free
    linear layers and RMSNorm (hyper.ai summary, section "方法"; neurohive, section
    "Архитектура"). For hidden [B][L][d_model]:

    1. zx = hidden w_in^T (fp64 matmul), whose columns are z | xBC | dt_raw;
    2. conv1d on xBC from conv_state, then ssd_scan gated by SiLU(z) from h0;
    3. group_rmsnorm of the gated output over ngroups groups with norm_w;
    4. out = (normalised output) w_out^T.

    With io "bf16" every value the library keeps in bf16 between the steps (zx, the conv
    output, the gated output, the normalised output) is rounded with round_bf16 first.
    Returns (out [B][L][d_model], conv_state' [B][3][Cc], h_final [B][H][N][P])."""
    r = round_bf16 if io == "bf16" else (lambda a: a)
    zx = r(_project(hidden, w_in))
    z, xbc, dt_raw = _split_projected(zx, nheads, ngroups)
    xr, hist = conv1d(xbc, conv_w, conv_b, conv_state)
    x, Bm, Cm = split_xbc(r(xr), nheads, ngroups)
    y, hf = ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, z, h0, ngroups=ngroups)
    yn = r(group_rmsnorm(r(y), norm_w, ngroups=ngroups, eps=eps))
    return _project(yn, w_out), hist, hf


def mixer_step(hidden, w_in, conv_w, conv_b, conv_state, dt_bias, A, D, ssm_state, norm_w, w_out, *,
               nheads: int, ngroups: int, eps: float = 1e-5, io: str = "f32"):
    """The mixer for T new tokens per sequence, hidden [B][T][d_model]: as mixer_prefill with
    state_update_tokens as the layer core (its conv output is not stored in between, so with
    io "bf16" only zx, the gated output and the normalised output are rounded).
    Returns (out [B][T][d_model], conv_state', ssm_state')."""
    r = round_bf16 if io == "bf16" else (lambda a: a)
    zx = r(_project(hidden, w_in))
    z, xbc, dt_raw = _split_projected(zx, nheads, ngroups)
    y, cs, ss = state_update_tokens(xbc, conv_w, conv_b, conv_state, dt_raw, dt_bias, A, D, z, ssm_state,
                                    nheads=nheads, ngroups=ngroups)
    yn = r(group_rmsnorm(r(y), norm_w, ngroups=ngroups, eps=eps))
    return _project(yn, w_out), cs, ss

"""Seeded synthetic inputs for the Mamba-2 layer core.

This module is shared by the fp64 oracle, the tests and the benchmark. It draws
random numbers and rounds them to the I/O precision; it contains none of the
layer's arithmetic (no conv, no softplus of dt, no recurrence).

Shapes follow the Mamba-2 hyper-parameters of the Nemotron-Nano-2 report
(hyper.ai summary, section "方法"; neurohive article, section "Архитектура"):
8 groups, state dimension 128, head dimension 64, expansion factor 2, conv
window 4, hidden size 5120 for the 12B base model (so d_inner = 10240 = 160
heads x 64). The 9B shape uses 128 heads (the pages give only the 112-128
search range for pruned Mamba heads; 128 is the value the workloads fix).

Every tensor is drawn from its own ``numpy.random.PCG64`` stream, keyed by
(config seed, tensor id, batch row, token block), so any token block of any
tensor can be regenerated on its own without drawing the rest.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Config", "WORKLOADS", "TINY_F32", "PREFILL_12B_8K", "DECODE_9B_B64", "PREFILL_12B_128K",
    "GENERATE_9B_B8", "config", "bf16_round", "bf16_bits", "bits_to_f32",
    "draw_params", "draw_xbc", "draw_z", "draw_dt_raw", "draw_h0",
    "draw_conv_state", "draw_prefill", "draw_decode_step", "draw_decode_steps", "TOKEN_BLOCK",
    "draw_gated", "draw_norm_weight", "draw_hidden", "draw_mixer_weights", "mixer_features",
]

TOKEN_BLOCK = 256  # tokens per independently seeded block

# tensor ids (part of the stream key; never renumber)
_T_ALOG, _T_DTB, _T_D, _T_CW, _T_CB, _T_XBC, _T_Z, _T_DT, _T_H0, _T_CS = range(10)
_T_GATED, _T_NW = 10, 11
_T_LEN, _T_SLOT, _T_INIT = 12, 13, 14
_T_HID, _T_WIN, _T_WOUT = 15, 16, 17


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    ``dt_mode`` selects how dt_raw is drawn: ``"normal"`` draws dt_raw ~ N(0,1)
    (dt_bias carries the log-uniform time scale); ``"loguniform"`` draws the
    target step u ~ log-uniform[1e-3, 0.1] per (token, head) and stores
    dt_raw = softplus^-1(u) - dt_bias, so the step the layer computes is u up to
    the rounding of dt_raw.
    """
    cid: int
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int = 64
    ngroups: int = 8
    dstate: int = 128
    conv_width: int = 4
    chunk: int = 128
    io: str = "bf16"          # "bf16" or "f32"; parameters and state are always f32
    h0_std: float = 0.0       # 0 => zero initial state
    dt_mode: str = "normal"
    decode_steps: int = 0

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def conv_channels(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.dstate


WORKLOADS: Dict[int, Config] = {
    0: Config(0, "tiny-f32", batch=1, seqlen=256, nheads=4, ngroups=1, chunk=64, io="f32"),
    1: Config(1, "prefill-12b-8k", batch=1, seqlen=8192, nheads=160, chunk=128),
    2: Config(2, "decode-9b-b64", batch=64, seqlen=1, nheads=128, chunk=128, h0_std=0.1),
    3: Config(3, "prefill-12b-128k", batch=1, seqlen=131072, nheads=160, chunk=256,
              dt_mode="loguniform"),
    4: Config(4, "generate-9b-b8", batch=8, seqlen=8192, nheads=128, chunk=128,
              decode_steps=16384),
}


TINY_F32 = WORKLOADS[0]            # small all-fp32 layer, the oracle finishes it in seconds
PREFILL_12B_8K = WORKLOADS[1]      # 12B-shape single-layer prefill, 8192 tokens
DECODE_9B_B64 = WORKLOADS[2]       # 9B-shape decode step, batch 64
PREFILL_12B_128K = WORKLOADS[3]    # 12B-shape 131072-token prefill
GENERATE_9B_B8 = WORKLOADS[4]      # 9B-shape generation run: batch 8, 8192-token prefill, 16384 steps


def config(base, **overrides) -> Config:
    """A workload (a Config, or its id) with some fields replaced."""
    return dataclasses.replace(base if isinstance(base, Config) else WORKLOADS[base], **overrides)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


# ----------------------------------------------------------------------------- rounding
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    return bits_to_f32(bf16_bits(a))


def _io(a: np.ndarray, io: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return bf16_round(a) if io == "bf16" else a


# ----------------------------------------------------------------------------- parameters
def _inv_softplus(u: np.ndarray) -> np.ndarray:
    # distribution recipe only: the value whose softplus is u
    return u + np.log(-np.expm1(-u))


def draw_params(cfg: Config) -> Dict[str, np.ndarray]:
    """Per-layer parameters, always float32.

    A_h = -exp(U[log 1, log 16]); dt_bias_h = softplus^-1(log-uniform[1e-3, 0.1]);
    D_h ~ N(0, 1); conv weight ~ U(-0.5, 0.5) [Cc][W]; conv bias ~ U(-0.1, 0.1).
    """
    H, Cc, W = cfg.nheads, cfg.conv_channels, cfg.conv_width
    A = -np.exp(_rng(cfg.seed, _T_ALOG).uniform(math.log(1.0), math.log(16.0), H))
    dts = np.exp(_rng(cfg.seed, _T_DTB).uniform(math.log(1e-3), math.log(0.1), H))
    dt_bias = _inv_softplus(dts)
    D = _rng(cfg.seed, _T_D).standard_normal(H)
    w = _rng(cfg.seed, _T_CW).uniform(-0.5, 0.5, (Cc, W))
    b = _rng(cfg.seed, _T_CB).uniform(-0.1, 0.1, Cc)
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {"A": f(A), "dt_bias": f(dt_bias), "D": f(D), "conv_w": f(w), "conv_b": f(b)}


# ----------------------------------------------------------------------------- per-token tensors
def _blocks(t0: int, t1: int):
    blk = t0 // TOKEN_BLOCK
    while blk * TOKEN_BLOCK < t1:
        yield blk
        blk += 1


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _tokens(cfg: Config, tid: int, width: int, t0: int, t1: int, fill, stream: int = 0,
            io: str = "f32") -> np.ndarray:
    """Rows [t0, t1) of a [B][T][width] float32 tensor, rounded to ``io``.

    Rows are drawn in 256-row blocks: block k of batch row b comes from the stream
    (seed, tid, b, k, stream), with stream 0 for prefill tokens and 1 for decode steps
    (row = step index). Blocks are independent, so they are filled on a thread pool; the
    result does not depend on the number of threads.
    """
    out = np.empty((cfg.batch, t1 - t0, width), dtype=np.float32)

    def one(job):
        b, blk = job
        b0 = blk * TOKEN_BLOCK
        rows = fill(_rng(cfg.seed, tid, b, blk, stream), TOKEN_BLOCK, width)
        lo, hi = max(t0, b0), min(t1, b0 + TOKEN_BLOCK)
        out[b, lo - t0:hi - t0] = _io(rows[lo - b0:hi - b0], io)

    jobs = [(b, blk) for b in range(cfg.batch) for blk in _blocks(t0, t1)]
    if len(jobs) < 4:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, jobs))
    return out


def _span(cfg: Config, t0: int, t1: Optional[int], step: int):
    """(t0, t1, stream) of a prefill token range or of decode step ``step``."""
    if step >= 0:
        return step, step + 1, 1
    return t0, cfg.seqlen if t1 is None else t1, 0


def _xbc_fill(cfg: Config):
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    s = 1.0 / math.sqrt(cfg.dstate)

    def fill(rng, n, width):
        a = rng.standard_normal((n, width), dtype=np.float32)
        a[:, di:di + 2 * gn] *= np.float32(s)
        return a
    return fill


def _normal_fill(rng, n, width):
    return rng.standard_normal((n, width), dtype=np.float32)


def draw_xbc(cfg: Config, t0: int = 0, t1: Optional[int] = None, step: int = -1) -> np.ndarray:
    """Raw xBC rows [B][t1-t0][Cc]: x channels ~ N(0,1), B and C channels ~ N(0,1)/sqrt(N).

    The same draw serves as the post-conv x/B/C operand of a stand-alone scan.
    Rounded to the config's I/O type.
    """
    t0, t1, stream = _span(cfg, t0, t1, step)
    return _tokens(cfg, _T_XBC, cfg.conv_channels, t0, t1, _xbc_fill(cfg), stream, cfg.io)


def draw_z(cfg: Config, t0: int = 0, t1: Optional[int] = None, step: int = -1) -> np.ndarray:
    t0, t1, stream = _span(cfg, t0, t1, step)
    return _tokens(cfg, _T_Z, cfg.d_inner, t0, t1, _normal_fill, stream, cfg.io)


def _dt_rows(cfg: Config, t0: int, t1: int, stream: int, dt_bias: np.ndarray) -> np.ndarray:
    if cfg.dt_mode == "normal":
        raw = _tokens(cfg, _T_DT, cfg.nheads, t0, t1, _normal_fill, stream)
    else:
        lo, hi = math.log(1e-3), math.log(0.1)
        u = _tokens(cfg, _T_DT, cfg.nheads, t0, t1,
                    lambda rng, n, w: np.exp(rng.uniform(lo, hi, (n, w))).astype(np.float32), stream)
        raw = (_inv_softplus(u.astype(np.float64)) - dt_bias.astype(np.float64)).astype(np.float32)
    return _io(raw, cfg.io)


def draw_dt_raw(cfg: Config, t0: int = 0, t1: Optional[int] = None, step: int = -1,
                dt_bias: Optional[np.ndarray] = None) -> np.ndarray:
    t0, t1, stream = _span(cfg, t0, t1, step)
    bias = draw_params(cfg)["dt_bias"] if dt_bias is None else dt_bias
    return _dt_rows(cfg, t0, t1, stream, bias)


def draw_h0(cfg: Config) -> np.ndarray:
    """Initial SSM state [B][H][N][P], float32; zeros unless ``h0_std`` > 0 (N(0, std^2))."""
    shape = (cfg.batch, cfg.nheads, cfg.dstate, cfg.headdim)
    if cfg.h0_std == 0.0:
        return np.zeros(shape, dtype=np.float32)
    out = np.empty(shape, dtype=np.float32)
    for b in range(cfg.batch):
        out[b] = _rng(cfg.seed, _T_H0, b).standard_normal(shape[1:], dtype=np.float32) * np.float32(cfg.h0_std)
    return out


def draw_conv_state(cfg: Config) -> np.ndarray:
    """Conv history [B][W-1][Cc] (slot 0 oldest), same distributions as the xBC channels."""
    fill = _xbc_fill(cfg)
    out = np.empty((cfg.batch, cfg.conv_width - 1, cfg.conv_channels), dtype=np.float32)
    for b in range(cfg.batch):
        out[b] = fill(_rng(cfg.seed, _T_CS, b), cfg.conv_width - 1, cfg.conv_channels)
    return _io(out, cfg.io)


def draw_prefill(cfg: Config, t0: int = 0, t1: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs of a prefill over tokens [t0, t1): params, xbc, z, dt_raw, h0."""
    p = draw_params(cfg)
    d = dict(p)
    d["xbc"] = draw_xbc(cfg, t0, t1)
    d["z"] = draw_z(cfg, t0, t1)
    d["dt_raw"] = draw_dt_raw(cfg, t0, t1, dt_bias=p["dt_bias"])
    d["h0"] = draw_h0(cfg)
    return d


def draw_decode_steps(cfg: Config, k0: int, k1: int) -> Dict[str, np.ndarray]:
    """Decode steps [k0, k1) at once, step-major ([k][B][...]); entry k equals row 0 of
    what draw_decode_step(cfg, k) returns."""
    bias = draw_params(cfg)["dt_bias"]
    f = lambda a: np.ascontiguousarray(a.transpose(1, 0, 2))
    return {"xbc": f(_tokens(cfg, _T_XBC, cfg.conv_channels, k0, k1, _xbc_fill(cfg), 1, cfg.io)),
            "z": f(_tokens(cfg, _T_Z, cfg.d_inner, k0, k1, _normal_fill, 1, cfg.io)),
            "dt_raw": f(_dt_rows(cfg, k0, k1, 1, bias))}


def draw_decode_step(cfg: Config, step: int) -> Dict[str, np.ndarray]:
    """Fresh one-token inputs for decode step ``step`` ([B][1][...] rows)."""
    return {
        "xbc": draw_xbc(cfg, 0, 1, step=step),
        "z": draw_z(cfg, 0, 1, step=step),
        "dt_raw": draw_dt_raw(cfg, 0, 1, step=step),
    }


def _gated_fill(rng, n, width):
    a = rng.standard_normal((n, width), dtype=np.float32)
    return a * np.exp(np.float32(0.5) * rng.standard_normal((n, width), dtype=np.float32))


def draw_gated(cfg: Config, t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """Stand-in for the gated layer output y * SiLU(z), rows [B][t1-t0][d_inner]: N(0,1) times
    a log-normal scale exp(N(0, 1/4)), which gives the heavy tails the gated output has.
    Rounded to the config's I/O type."""
    t0, t1, stream = _span(cfg, t0, t1, -1)
    return _tokens(cfg, _T_GATED, cfg.d_inner, t0, t1, _gated_fill, stream, cfg.io)


def draw_norm_weight(cfg: Config) -> np.ndarray:
    """Per-channel RMSNorm weight [d_inner] ~ U(0.5, 1.5), fp32."""
    return _rng(cfg.seed, _T_NW).uniform(0.5, 1.5, cfg.d_inner).astype(np.float32)


# ----------------------------------------------------------------------------- packed batches
def draw_lengths(cfg: Config, nseq: int, lo: int, hi: int, total: Optional[int] = None) -> np.ndarray:
    """Sequence lengths for a packed (continuous-batching) prefill: log-uniform in [lo, hi],
    int. With ``total`` the lengths are rescaled (largest remainders) to sum exactly to it."""
    r = _rng(cfg.seed, _T_LEN, nseq)
    lens = np.floor(np.exp(r.uniform(np.log(lo), np.log(hi + 1), nseq))).astype(np.int64)
    lens = np.clip(lens, lo, hi)
    if total is not None:
        w = lens / lens.sum() * total
        base = np.floor(w).astype(np.int64)
        rest = total - int(base.sum())
        order = np.argsort(-(w - base), kind="stable")
        base[order[:rest]] += 1
        lens = base
    return lens.astype(np.int32)


def draw_slots(cfg: Config, nseq: int, npool: int) -> np.ndarray:
    """Distinct pool entries for nseq sequences: a seeded random choice out of npool."""
    return _rng(cfg.seed, _T_SLOT, nseq, npool).permutation(npool)[:nseq].astype(np.int32)


def draw_has_init(cfg: Config, nseq: int, p: float = 0.5) -> np.ndarray:
    """Per-sequence flags (int32 0/1): 1 with probability p (the sequence continues from its
    cached state), else 0 (a new request)."""
    return (_rng(cfg.seed, _T_INIT, nseq).uniform(0, 1, nseq) < p).astype(np.int32)


def draw_pools(cfg: Config, npool: int) -> tuple:
    """Cache pools for npool entries: conv history [npool][3][Cc] drawn like xBC rows (io
    precision) and fp32 states [npool][H][N][P] ~ N(0, 0.1^2)."""
    c = dataclasses.replace(cfg, batch=npool, h0_std=cfg.h0_std or 0.1)
    return draw_conv_state(c), draw_h0(c)


# ----------------------------------------------------------------------------- the mixer
def mixer_features(cfg: Config) -> int:
    """Rows of the in-projection weight: z (d_inner), xBC (Cc), dt_raw (nheads)."""
    return cfg.d_inner + cfg.conv_channels + cfg.nheads


def draw_hidden(cfg: Config, d_model: int, t0: int = 0, t1: Optional[int] = None,
                step: int = -1) -> np.ndarray:
    """Mixer input rows [B][t1-t0][d_model] ~ N(0, 1) (the output of the layer's RMSNorm has
    unit mean square), rounded to the config's I/O type. Decode steps use step >= 0."""
    t0, t1, stream = _span(cfg, t0, t1, step)
    return _tokens(cfg, _T_HID, d_model, t0, t1, _normal_fill, stream, cfg.io)


def _weight_rows(cfg: Config, tid: int, rows: int, cols: int, scale: np.ndarray) -> np.ndarray:
    """A [rows][cols] N(0, 1) matrix, row r scaled by scale[r], drawn in 1024-row blocks with
    their own streams (on a thread pool), rounded to the config's I/O type."""
    out = np.empty((rows, cols), dtype=np.float32)
    blk = 1024

    def one(k):
        r0, r1 = k * blk, min(rows, (k + 1) * blk)
        a = _rng(cfg.seed, tid, cols, k).standard_normal((r1 - r0, cols), dtype=np.float32)
        out[r0:r1] = _io(a * scale[r0:r1, None], cfg.io)

    nb = (rows + blk - 1) // blk
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(nb)))
    return out


def draw_mixer_weights(cfg: Config, d_model: int) -> Dict[str, np.ndarray]:
    """Random-init projection weights of the mixer, in io precision, scaled so that the
    projected features have the distributions the layer core's recipe draws directly:
    w_in [E][d_model] ~ N(0, 1/d_model), with the B and C rows further scaled by
    1/sqrt(d_state) (so z, x and dt_raw come out ~ N(0, 1) and B, C ~ N(0, 1)/sqrt(N));
    w_out [d_model][d_inner] ~ N(0, 1/d_inner); the norm weight as draw_norm_weight."""
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    E = mixer_features(cfg)
    s_in = np.full(E, 1.0 / math.sqrt(d_model), dtype=np.float32)
    s_in[2 * di:2 * di + 2 * gn] /= np.float32(math.sqrt(cfg.dstate))
    w_in = _weight_rows(cfg, _T_WIN, E, d_model, s_in)
    w_out = _weight_rows(cfg, _T_WOUT, d_model, di, np.full(d_model, 1.0 / math.sqrt(di), dtype=np.float32))
    return {"w_in": w_in, "w_out": w_out, "norm_w": draw_norm_weight(cfg)}

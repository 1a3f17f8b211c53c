"""Benchmark of the Mamba-2 layer core on one MI355X.

One step = one pass of the prefill hot path over one batch of synthetic input
already resident in HBM: mamba2_conv_ssd_prefill, the width-4 causal conv + SiLU
over the raw xBC channels and the chunked scan in one call (at chunk 64 the conv
runs inside the scan's kernels), on the 12B-shape single-layer workload: B=1,
L=8192, 160 heads x 64, 8 groups, d_state 128, bf16 io, fp32 state. ``value`` is
prefill tokens/s of that step. The chunk length (--chunk, 64) is the scan's tiling
parameter and does not change what is computed (the GPU tests check chunks 64, 128
and 256 against the oracle). The same run reports under "kernels": the two-call
path (mamba2_conv1d, then mamba2_ssd_prefill) at the same chunk, and the one call at
the workload's listed chunk of 128. The one-token decode state update is measured
in the same run on the 9B-shape batch-64 decode workload and reported under
"decode"; the group RMSNorm of the gated output (not part of the step) under
"kernels" as well.

Per-kernel durations come from HIP events recorded around each launch on the
stream the kernels run on (torch's current stream). Algorithmic bytes count
every input read once, every output written once and the fp32 state read and
written once; they are the roofline numerators.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps K] [--chunk Q]
       [--no-cpu-baseline] [--copy-calibration]
       python bench.py [--chunk Q] --summarize-counters FETCH_CSV WRITE_CSV
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "SSD prefill tokens/s @12B-shape L=8k; decode state-update GB/s % of HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "conv_ssd_prefill": ["ssd_prefill.hip", "device.h"],
    "ssd_prefill": ["ssd_prefill.hip", "device.h"],
    "state_update": ["state_update.hip", "device.h"],
    "conv1d": ["conv1d.hip", "device.h"],
    "group_rmsnorm": ["rmsnorm.hip", "device.h"],
}


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)


def _code_only(src: str) -> str:
    """The source with comments dropped and whitespace runs folded to one space (string and
    character literals kept as written), so that editing a comment keeps the hash."""
    out, pos, gap = [], 0, False
    for m in _CODE_TOKENS.finditer(src):
        if m.start() > pos:
            out.append(" " if gap and out else "")
            out.append(src[pos:m.start()])
            gap = False
        t = m.group(0)
        if t[0] in "\"'":
            out.append(" " if gap and out else "")
            out.append(t)
            gap = False
        else:
            gap = True
        pos = m.end()
    if pos < len(src):
        out.append((" " if gap and out else "") + src[pos:])
    return "".join(out)


def kernel_source_hash(name: str) -> str:
    """Hash of the code (not the comments) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "state_space_sequence_causal_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def run_environment(torch) -> dict:
    """What the line was measured on: the device, the ROCm and torch builds, and a hash of the
    library's sources (the run's working copy need not be a git checkout)."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "state_space_sequence_causal_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "rocm": rocm, "hip": torch.version.hip, "torch": torch.__version__,
            "library_sources_sha256_16": h.hexdigest()[:16]}


def measured_traffic(name: str, chunk: int | None = None):
    """HBM bytes per launch from the committed counter summary, or None when the kernel
    source changed since the counters were taken (or they were taken at another chunk)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[name]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash(name):
        return None
    if chunk is not None and t.get("chunk") != chunk:
        return None
    return t.get("bytes_per_launch")


# ------------------------------------------------------------------------------ clock settle
SETTLE_MS = {}     # workload -> GPU milliseconds spent settling the clocks before its warm-up


def settle(torch, name: str, step, min_ms: float):
    """Runs ``step(k)`` (k = 0, 1, ...) in growing batches until at least ``min_ms`` of GPU
    time has passed between two events on the current stream, so that the clocks have
    ramped up to the workload's steady state before its warm-up and timed steps (the first
    tens of milliseconds after an idle gap run at lower clocks). Records the time spent."""
    if min_ms <= 0:
        SETTLE_MS[name] = 0.0
        return
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    k, batch = 0, 4
    while True:
        for _ in range(batch):
            step(k)
            k += 1
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        if ms >= min_ms:
            break
        batch = min(batch * 2, 256)
    SETTLE_MS[name] = ms


# ------------------------------------------------------------------------------ workloads
def prefill_bytes(cfg) -> dict:
    """Algorithmic HBM bytes of one prefill pass (inputs once, outputs once)."""
    e = 2 if cfg.io == "bf16" else 4
    B, L, H, P, G, N = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    Cc = cfg.conv_channels
    tok = B * L
    ssd = tok * (3 * H * P * e + 2 * G * N * e + H * e)        # x, z, y; B, C; dt
    ssd += B * H * N * P * 4                                     # h_final (h0 = 0 is not read)
    ssd += 3 * H * 4                                             # dt_bias, A, D
    conv = tok * 2 * Cc * e + Cc * 5 * 4 + 2 * B * 3 * Cc * e    # u, out; w, bias; conv cache
    # the one call reads the raw xBC in place of the conv output: the scan's bytes plus the
    # conv parameters and the conv cache in and out
    fused = ssd + Cc * 5 * 4 + 2 * B * 3 * Cc * e
    return {"ssd": ssd, "conv": conv, "fused": fused}


def prefill_flops(cfg) -> float:
    """Algorithmic flops of the chunked scan: per token G(Q+1)N + H(Q+1)P (the causal halves
    of C.B^T and M.X) + 4HNP (chunk state and carried-state output)."""
    H, P, G, N, Q = cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.chunk
    return cfg.batch * cfg.seqlen * (G * (Q + 1) * N + H * (Q + 1) * P + 4 * H * N * P)


def decode_bytes(cfg) -> int:
    e = 2 if cfg.io == "bf16" else 4
    B, H, P, G, N, Cc = cfg.batch, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.conv_channels
    per_seq = 2 * H * N * P * 4 + 2 * 3 * Cc * e + Cc * e + H * P * e + H * e + H * P * e
    params = Cc * 5 * 4 + 3 * H * 4
    return B * per_seq + params


# ------------------------------------------------------------------------------ GPU parts
def run_prefill(args, torch, m2, si, cfg, inp, chunk, fused=True):
    """Times the prefill step at ``chunk``: the one call (fused=True) or mamba2_conv1d then
    mamba2_ssd_prefill. Returns ms per step, wall seconds and the per-call microseconds."""
    dev = lambda a: torch.from_numpy(si.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(a).cuda()
    u, z, dt = dev(inp["xbc"]), dev(inp["z"]), dev(inp["dt_raw"])
    w, bias, dtb, A, D = (f32(inp[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D"))
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    cs = torch.zeros((cfg.batch, 3, cfg.conv_channels), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((cfg.batch, cfg.seqlen, di), dtype=torch.bfloat16, device="cuda")
    hf = torch.empty((cfg.batch, cfg.nheads, cfg.dstate, cfg.headdim), dtype=torch.float32, device="cuda")
    dims = m2.make_dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, chunk, m2.MAMBA2_BF16)
    if fused:
        ws = torch.empty(m2.mamba2_conv_ssd_prefill_workspace_bytes(dims), dtype=torch.uint8, device="cuda")

        def calls():
            m2.mamba2_conv_ssd_prefill(u, w, bias, cs, dt, dtb, A, D, z, None, hf, y,
                                       ngroups=cfg.ngroups, chunk=chunk, workspace=ws)
        calls = [calls]
    else:
        ws = torch.empty(m2.mamba2_ssd_prefill_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
        xbc = torch.empty_like(u)
        x, Bm, Cm = xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:]
        calls = [lambda: m2.mamba2_conv1d(u, w, bias, cs, xbc),
                 lambda: m2.mamba2_ssd_prefill(x, Bm, Cm, dt, dtb, A, D, z, None, hf, y,
                                               ngroups=cfg.ngroups, chunk=chunk, workspace=ws)]

    def step(evs=None):
        for i, f in enumerate(calls):
            if evs:
                evs[i].record()
            f()
        if evs:
            evs[-1].record()

    settle(torch, f"prefill_chunk{chunk}" + ("" if fused else "_two_call"), lambda k: step(), args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: the steps back to back between two events (an event recorded between
    # two launches leaves the GPU idle for a few microseconds, so none is recorded inside it)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t_start.record()
    for k in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_start.elapsed_time(t_end)
    # then the same steps with events around each call, for the per-call durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    per_call = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) * 1e3 / args.steps for i in range(len(calls))]
    return total_ms / args.steps, wall, per_call


CU_PEAK_FLOP_PER_CYCLE = BF16_PEAK_TFLOPS * 1e12 / (256 * 2.4e9)   # dense bf16 MFMA per CU per cycle


def run_phase_profile(args, torch, m2, si, cfg, inp):
    """Per-phase MFMA rates of the step's scan kernel, from its cycle profile
    (mamba2_conv_ssd_prefill_profile: s_memtime around each contraction phase of every wave,
    summed over the chunk loop). For each phase: the algorithmic flops of one (head, chunk),
    the cycles the phase takes per chunk on the CU (the slowest of the four waves that share
    it, one per SIMD, averaged over workgroups), and their ratio against the CU's dense bf16
    MFMA peak. Phases: the carried-state output H^T C^T (2 Q N P flops per chunk), the chunk
    state B^T (w x) (2 Q N P) and the intra-chunk product X^T M^T ((Q + 1) Q P, the causal
    half). The computed operands enter as hi + lo bf16 pairs, so the MFMAs execute twice the
    algorithmic flops of the first two and of the third."""
    dev = lambda a: torch.from_numpy(si.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(a).cuda()
    u, z, dt = dev(inp["xbc"]), dev(inp["z"]), dev(inp["dt_raw"])
    w, bias, dtb, A, D = (f32(inp[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D"))
    B, L, H, Q, N, P = cfg.batch, cfg.seqlen, cfg.nheads, 64, cfg.dstate, cfg.headdim
    cs = torch.zeros((B, 3, cfg.conv_channels), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((B, L, cfg.d_inner), dtype=torch.bfloat16, device="cuda")
    hf = torch.empty((B, H, N, P), dtype=torch.float32, device="cuda")
    dims = m2.make_dims(B, L, H, cfg.ngroups, Q, m2.MAMBA2_BF16)
    ws = torch.empty(m2.mamba2_conv_ssd_prefill_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    cyc = torch.zeros(B * H * 16 * 8, dtype=torch.int64, device="cuda")

    def plain(k=0):
        m2.mamba2_conv_ssd_prefill(u, w, bias, cs, dt, dtb, A, D, z, None, hf, y, ngroups=cfg.ngroups,
                                   chunk=Q, workspace=ws)

    def profiled():
        m2.mamba2_conv_ssd_prefill_profile(u, w, bias, cs, dt, dtb, A, D, z, None, hf, y, cyc,
                                           ngroups=cfg.ngroups, chunk=Q, workspace=ws)

    settle(torch, "phase_profile", plain, args.settle_ms)
    for _ in range(3):
        profiled()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    profiled()
    e1.record()
    torch.cuda.synchronize()
    prof_us = e0.elapsed_time(e1) * 1e3
    c = cyc.view(B * H, 16, 8).cpu().numpy().astype("float64")
    nC = (L + Q - 1) // Q
    loop = float(c[:, 0, 0].mean()) / nC
    phases = {
        "A6_carried_state_output": (c[:, 0:4, 1].max(axis=1).mean() / nC, 2.0 * Q * N * P),
        "A4_chunk_state": (c[:, 4:8, 1].max(axis=1).mean() / nC, 2.0 * Q * N * P),
        "A3_intra_chunk": (c[:, 0:4, 2].max(axis=1).mean() / nC, float((Q + 1) * Q * P)),
    }
    busy = min(B * H, 256) / 256.0
    out = {"method": "cycle stamps around each phase in the scan kernel (mamba2_conv_ssd_prefill_profile), "
                     "12B 8k one-call step",
           "cu_peak_flop_per_cycle": CU_PEAK_FLOP_PER_CYCLE, "chunk_loop_cycles_per_chunk": loop,
           "profiled_call_us": prof_us, "busy_cu_share": busy, "target_frac": 0.5}
    for name, (cycles, flops) in phases.items():
        frac = flops / (cycles * CU_PEAK_FLOP_PER_CYCLE)
        out[name] = {"cycles_per_chunk": float(cycles), "algorithmic_flops_per_chunk": flops,
                     "frac_of_cu_peak": frac, "executed_frac_of_cu_peak": 2 * frac,
                     "frac_of_chip_peak": frac * busy, "share_of_chunk_loop": float(cycles) / loop}
    # per role, cycles per chunk (mean over the role's waves and the workgroups): time in the
    # chunk's barrier, and the helpers' two phases; the role that waits least sets the pace
    roles = {"y_waves": slice(0, 4), "h_waves": slice(4, 8), "helper_waves": slice(8, 16)}
    out["barrier_wait_cycles_per_chunk"] = {k: float(c[:, v, 4].mean()) / nC for k, v in roles.items()}
    out["helper_build_cycles_per_chunk"] = float(c[:, 8:16, 1].mean()) / nC
    out["helper_stage_cycles_per_chunk"] = float(c[:, 8:16, 2].mean()) / nC
    return out


def run_decode(args, torch, m2, si):
    cfg = si.DECODE_9B_B64
    p = si.draw_params(cfg)
    step_inp = si.draw_decode_step(cfg, 0)
    dev = lambda a: torch.from_numpy(si.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(a).cuda()
    u, z, dt = (dev(step_inp[k][:, 0]) for k in ("xbc", "z", "dt_raw"))
    w, bias, dtb, A, D = (f32(p[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D"))
    h0 = f32(si.draw_h0(cfg))
    cs0 = dev(si.draw_conv_state(cfg))
    # two independent (state, cache) sets used in turn: 512 MiB of state, twice the
    # 256 MB Infinity Cache, so each step streams its state from HBM
    states = [h0, h0.clone()]
    caches = [cs0, cs0.clone()]
    y = torch.empty((cfg.batch, cfg.d_inner), dtype=torch.bfloat16, device="cuda")

    def step(k):
        m2.mamba2_state_update(u, w, bias, caches[k & 1], dt, dtb, A, D, z, states[k & 1], y,
                               ngroups=cfg.ngroups)

    settle(torch, "decode", step, args.settle_ms)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    n = args.decode_steps
    # the mean launch duration over back-to-back launches between two events (the timed
    # region), then each launch bracketed by its own events for the median
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(n):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    mean_us = e0.elapsed_time(e1) * 1e3 / n
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for k in range(n):
        evs[k][0].record()
        step(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return cfg, mean_us, times[n // 2]


def run_decode_tokens(args, torch, m2, si, T=4):
    """The 9B-shape batch-64 decode with T new tokens per sequence in one call (the state is
    streamed once for the T tokens), on two alternating state/cache sets like the one-token
    decode."""
    import numpy as np
    cfg = si.DECODE_9B_B64
    p = si.draw_params(cfg)
    steps = si.draw_decode_steps(cfg, 0, T)
    tok = {k: np.ascontiguousarray(v.transpose(1, 0, 2)) for k, v in steps.items()}   # [B][T][...]
    dev = lambda a: torch.from_numpy(si.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(a).cuda()
    u, z, dt = (dev(tok[k]) for k in ("xbc", "z", "dt_raw"))
    w, bias, dtb, A, D = (f32(p[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D"))
    h0 = f32(si.draw_h0(cfg))
    cs0 = dev(si.draw_conv_state(cfg))
    states, caches = [h0, h0.clone()], [cs0, cs0.clone()]
    y = torch.empty((cfg.batch, T, cfg.d_inner), dtype=torch.bfloat16, device="cuda")

    def step(k):
        m2.mamba2_state_update(u, w, bias, caches[k & 1], dt, dtb, A, D, z, states[k & 1], y,
                               ngroups=cfg.ngroups)

    settle(torch, f"decode_tokens{T}", step, args.settle_ms)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    n = args.decode_steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(n):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    e = 2
    B, H, P, G, N, Cc = cfg.batch, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.conv_channels
    nbytes = B * (2 * H * N * P * 4 + 2 * 3 * Cc * e + T * (Cc * e + 2 * H * P * e + H * e)) + Cc * 5 * 4 + 3 * H * 4
    return {"tokens_per_call": T, "us": us, "tokens_per_s": B * T / (us * 1e-6),
            "GB_s": nbytes / (us * 1e-6) / 1e9, "algorithmic_bytes": nbytes,
            "note": f"9B-shape batch 64, {T} new tokens per sequence in one call"}


def run_rmsnorm(args, torch, m2, si, cfg):
    """The group RMSNorm over the prefill's gated output shape (seeded stand-in input). Two
    input/output sets are used in turn (672 MB together), so no step finds its input in the
    256 MB Infinity Cache."""
    g = torch.from_numpy(si.bf16_bits(si.draw_gated(cfg)).view("int16")).view(torch.bfloat16).cuda()
    w = torch.from_numpy(si.draw_norm_weight(cfg)).cuda()
    sets = [(g, torch.empty_like(g)), (g.clone(), torch.empty_like(g))]
    turn = [0]

    def step():
        gi, oi = sets[turn[0]]
        turn[0] ^= 1
        m2.mamba2_group_rmsnorm(gi, w, oi, ngroups=cfg.ngroups)

    settle(torch, "group_rmsnorm", lambda k: step(), args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # launches back to back between two events (an event between two launches would leave
    # the GPU idle for a few microseconds)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    nbytes = 2 * g.numel() * g.element_size() + w.numel() * 4
    return us, nbytes


def _mixer_inputs(torch, si, cfg, d_model, hidden):
    dev = lambda a: torch.from_numpy(si.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(a).cuda()
    p, w = si.draw_params(cfg), si.draw_mixer_weights(cfg, d_model)
    return dict(hid=dev(hidden), w_in=dev(w["w_in"]), w_out=dev(w["w_out"]), norm_w=f32(w["norm_w"]),
                **{k: f32(p[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D")})


def mixer_flops(cfg, d_model: int, rows: int) -> float:
    """The two projections' multiply-adds (2 flops each) per call."""
    E = cfg.d_inner + cfg.conv_channels + cfg.nheads
    return 2.0 * rows * d_model * (E + cfg.d_inner)


def run_mixer_prefill(args, torch, m2, si, cfg, d_model: int = 5120):
    """mamba2_mixer_prefill over the 12B-shape workload: hidden [1][8192][5120] (the 12B
    model's hidden width), in-projection to z | xBC | dt_raw (22,688 features), the layer
    core, the group RMSNorm and the out-projection back to 5120."""
    t = _mixer_inputs(torch, si, cfg, d_model, si.draw_hidden(cfg, d_model))
    cs = torch.zeros((cfg.batch, 3, cfg.conv_channels), dtype=torch.bfloat16, device="cuda")
    hf = torch.empty((cfg.batch, cfg.nheads, cfg.dstate, cfg.headdim), dtype=torch.float32, device="cuda")
    out = torch.empty((cfg.batch, cfg.seqlen, d_model), dtype=torch.bfloat16, device="cuda")
    d = m2.make_dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, 64, m2.MAMBA2_BF16)
    ws = torch.empty(m2.mamba2_mixer_prefill_workspace_bytes(d, d_model), dtype=torch.uint8, device="cuda")

    def step():
        m2.mamba2_mixer_prefill(t["hid"], t["w_in"], t["conv_w"], t["conv_b"], cs, t["dt_bias"], t["A"], t["D"],
                                None, hf, t["norm_w"], t["w_out"], out, ngroups=cfg.ngroups, chunk=64,
                                workspace=ws)

    n = max(1, args.steps // 4)
    settle(torch, "mixer_prefill", lambda k: step(), args.settle_ms)
    for _ in range(max(1, args.warmup // 10)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    rows = cfg.batch * cfg.seqlen
    gf = mixer_flops(cfg, d_model, rows)
    return {"us": us, "tokens_per_s": rows / (us * 1e-6), "d_model": d_model, "calls_timed": n,
            "projection_GFLOP": gf / 1e9, "projection_TFLOP_s_over_whole_call": gf / (us * 1e-6) / 1e12,
            "note": "the mixer around the step: in-projection (hipBLASLt), the step's layer core, "
                    "group RMSNorm, out-projection (hipBLASLt); random-init weights"}


def run_mixer_step(args, torch, m2, si, d_model: int = 4480):
    """mamba2_mixer_step at the 9B decode shape: batch 64, one token, hidden width 4480 (the
    pruned 9B model's), on two alternating cache sets like the decode step."""
    cfg = si.DECODE_9B_B64
    t = _mixer_inputs(torch, si, cfg, d_model, si.draw_hidden(cfg, d_model, step=0))
    h0 = torch.from_numpy(si.draw_h0(cfg)).cuda()
    cs0 = torch.from_numpy(si.bf16_bits(si.draw_conv_state(cfg)).view("int16")).view(torch.bfloat16).cuda()
    states, caches = [h0, h0.clone()], [cs0, cs0.clone()]
    out = torch.empty((cfg.batch, 1, d_model), dtype=torch.bfloat16, device="cuda")
    d = m2.make_dims(cfg.batch, 1, cfg.nheads, cfg.ngroups, 64, m2.MAMBA2_BF16)
    ws = torch.empty(m2.mamba2_mixer_step_workspace_bytes(d, d_model), dtype=torch.uint8, device="cuda")

    def step(k):
        m2.mamba2_mixer_step(t["hid"], t["w_in"], t["conv_w"], t["conv_b"], caches[k & 1], t["dt_bias"], t["A"],
                             t["D"], states[k & 1], t["norm_w"], t["w_out"], out, ngroups=cfg.ngroups,
                             workspace=ws)

    settle(torch, "mixer_step", step, args.settle_ms)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    n = args.decode_steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(n):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    E = cfg.d_inner + cfg.conv_channels + cfg.nheads
    wbytes = 2 * d_model * (E + cfg.d_inner)
    return {"us": us, "tokens_per_s": cfg.batch / (us * 1e-6), "d_model": d_model,
            "weight_bytes": wbytes, "state_bytes": decode_bytes(cfg),
            "GB_s_weights_and_state": (wbytes + decode_bytes(cfg)) / (us * 1e-6) / 1e9,
            "note": "9B-shape batch 64, one token: in-projection, state update, group RMSNorm, "
                    "out-projection; random-init weights"}


def run_generation(args, torch, m2, si):
    """The 9B generation-shaped run on one layer: batch 8, an 8192-token one-call prefill
    (chunk 64), then 16384 sequential decode steps carrying both caches. Inputs are drawn on
    the device from a seeded generator with the recipe's distributions, fresh for every
    decode step (all 16384 steps' inputs, about 5 GB, are drawn before the timed run).
    Reports the prefill time, the mean decode step over all steps launched back to back,
    the median and 99th percentile of 1000 individually timed steps, and tokens/s over the
    whole run."""
    cfg = si.GENERATE_9B_B8
    B, L, H, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    Cc, di = cfg.conv_channels, cfg.d_inner
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed)
    bf = torch.bfloat16

    def xbc(*shape):
        a = torch.randn(*shape, Cc, generator=gen, device="cuda")
        a[..., di:] *= 128 ** -0.5
        return a.to(bf)

    p = {k: torch.from_numpy(v).cuda() for k, v in si.draw_params(cfg).items()}
    u = xbc(B, L)
    z = torch.randn(B, L, di, generator=gen, device="cuda").to(bf)
    dt = torch.randn(B, L, H, generator=gen, device="cuda").to(bf)
    cs = torch.zeros(B, 3, Cc, dtype=bf, device="cuda")
    h = torch.empty(B, H, cfg.dstate, cfg.headdim, dtype=torch.float32, device="cuda")
    y = torch.empty(B, L, di, dtype=bf, device="cuda")
    d = m2.make_dims(B, L, H, G, 64, m2.MAMBA2_BF16)
    ws = torch.empty(m2.mamba2_conv_ssd_prefill_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    K = cfg.decode_steps
    su, sz, sdt = xbc(K, B), torch.randn(K, B, di, generator=gen, device="cuda").to(bf), \
        torch.randn(K, B, H, generator=gen, device="cuda").to(bf)
    yt = torch.empty(B, di, dtype=bf, device="cuda")

    def prefill():
        m2.mamba2_conv_ssd_prefill(u, p["conv_w"], p["conv_b"], cs, dt, p["dt_bias"], p["A"], p["D"], z, None, h,
                                   y, ngroups=G, chunk=64, workspace=ws)

    def step(k):
        i = k % K
        m2.mamba2_state_update(su[i], p["conv_w"], p["conv_b"], cs, sdt[i], p["dt_bias"], p["A"], p["D"], sz[i],
                               h, yt, ngroups=G)

    def pair(k):
        prefill()
        step(k)

    settle(torch, "generation", pair, args.settle_ms)
    for k in range(20):
        pair(k)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    prefill()
    ev[1].record()
    for k in range(cfg.decode_steps):
        step(k)
    ev[2].record()
    torch.cuda.synchronize()
    pre_us = ev[0].elapsed_time(ev[1]) * 1e3
    dec_total_us = ev[1].elapsed_time(ev[2]) * 1e3
    n = 1000
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for k in range(n):
        evs[k][0].record()
        step(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    tokens = B * L + B * cfg.decode_steps
    state_bytes = B * H * cfg.dstate * cfg.headdim * 4 * 2
    return {"workload": "9B shape, batch 8: 8192-token one-call prefill (chunk 64), then 16384 decode steps",
            "prefill_us": pre_us, "decode_steps": cfg.decode_steps,
            "decode_us_per_step": dec_total_us / cfg.decode_steps, "decode_us_p50": t[n // 2],
            "decode_us_p99": t[int(n * 0.99)], "total_ms": (pre_us + dec_total_us) / 1e3,
            "tokens_per_s": tokens / ((pre_us + dec_total_us) * 1e-6),
            "decode_state_GB_s": state_bytes / (dec_total_us / cfg.decode_steps * 1e-6) / 1e9}


def run_other_prefills(args, torch, m2, si):
    """The other prefill workloads, one call each timed over back-to-back launches: the
    128k-token 12B-shape prefill (inputs drawn on the device from a seeded generator with
    the recipe's distributions, dt log-uniform in [1e-3, 0.1] through dt_raw; at chunk 64,
    the fused call, and at the listed chunk 256) and the tiny all-fp32 layer (seeded host
    inputs, chunk 64)."""
    import numpy as np
    out = {}
    cfg = si.PREFILL_12B_128K
    B, L, H, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    Cc, di = cfg.conv_channels, cfg.d_inner
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed)
    bf = torch.bfloat16
    u = torch.randn(B, L, Cc, generator=gen, device="cuda")
    u[..., di:] *= 128 ** -0.5
    u = u.to(bf)
    z = torch.randn(B, L, di, generator=gen, device="cuda").to(bf)
    p = {k: torch.from_numpy(v).cuda() for k, v in si.draw_params(cfg).items()}
    step = torch.exp(torch.empty(B, L, H, device="cuda").uniform_(float(np.log(1e-3)), float(np.log(0.1)),
                                                                    generator=gen))
    dt = (step + torch.log(-torch.expm1(-step)) - p["dt_bias"]).to(bf)   # softplus(dt_raw + dt_bias) = step
    h = torch.empty(B, H, cfg.dstate, cfg.headdim, dtype=torch.float32, device="cuda")
    y = torch.empty(B, L, di, dtype=bf, device="cuda")
    for chunk in (64, 256):
        d = m2.make_dims(B, L, H, G, chunk, m2.MAMBA2_BF16)
        ws = torch.empty(m2.mamba2_conv_ssd_prefill_workspace_bytes(d), dtype=torch.uint8, device="cuda")

        def call():
            m2.mamba2_conv_ssd_prefill(u, p["conv_w"], p["conv_b"], None, dt, p["dt_bias"], p["A"], p["D"], z,
                                       None, h, y, ngroups=G, chunk=chunk, workspace=ws)
        us = _time_calls(torch, call, 2, 5, f"prefill_12b_128k_chunk{chunk}", args.settle_ms)
        out[f"prefill_12b_128k_chunk{chunk}"] = {"us": us, "tokens_per_s": B * L / (us * 1e-6),
                                                  "GB_s": prefill_bytes(cfg)["fused"] / (us * 1e-6) / 1e9}
        del ws
    # one GPU's share of that sequence split 8 ways (context parallelism): 16384 tokens from
    # an incoming state and conv history
    Ls = L // 8
    cs = torch.zeros(B, 3, Cc, dtype=bf, device="cuda")
    h0 = 0.1 * torch.randn(B, H, cfg.dstate, cfg.headdim, generator=gen, device="cuda")
    d = m2.make_dims(B, Ls, H, G, 64, m2.MAMBA2_BF16)
    ws = torch.empty(m2.mamba2_conv_ssd_prefill_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    us_, zs_, dts_, ys_ = u[:, :Ls], z[:, :Ls], dt[:, :Ls], y[:, :Ls]

    def share():
        m2.mamba2_conv_ssd_prefill(us_, p["conv_w"], p["conv_b"], cs, dts_, p["dt_bias"], p["A"], p["D"], zs_, h0,
                                   h, ys_, ngroups=G, chunk=64, workspace=ws)
    us = _time_calls(torch, share, 5, 20, "prefill_12b_16k_share", args.settle_ms)
    out["prefill_12b_16k_share_with_h0"] = {"us": us, "tokens_per_s": B * Ls / (us * 1e-6),
                                             "note": "one GPU's 1/8 share of the 128k sequence, from an "
                                                     "incoming state and history (the history is updated "
                                                     "in place each call)"}
    del ws
    del u, z, dt, y
    cfg = si.TINY_F32
    inp = si.draw_prefill(cfg)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    tu, tz, tdt = f32(inp["xbc"]), f32(inp["z"]), f32(inp["dt_raw"])
    th = torch.empty(1, cfg.nheads, cfg.dstate, cfg.headdim, dtype=torch.float32, device="cuda")
    ty = torch.empty(1, cfg.seqlen, cfg.d_inner, dtype=torch.float32, device="cuda")
    tw = {k: f32(inp[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D")}

    def tiny():
        m2.mamba2_conv_ssd_prefill(tu, tw["conv_w"], tw["conv_b"], None, tdt, tw["dt_bias"], tw["A"], tw["D"], tz,
                                   None, th, ty, ngroups=cfg.ngroups, chunk=64)
    out["prefill_tiny_f32"] = {"us": _time_calls(torch, tiny, 50, 200, "prefill_tiny_f32", args.settle_ms),
                               "note": "batch 1, 256 tokens, 4 heads, 1 group, all fp32, chunk 64 (latency)"}
    return out


def _time_calls(torch, call, warm: int, n: int, name: str = "", settle_ms: float = 0.0) -> float:
    if name:
        settle(torch, name, lambda k: call(), settle_ms)
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def run_varlen(args, torch, m2, si, cfg):
    """The one-call prefill over a packed continuous batch at the 12B shape: 16 sequences of
    seeded log-uniform lengths summing to the workload's 8192 tokens, half of them continuing
    from their entries in a pool of 40 cached states (seeded inputs stand in for requests)."""
    nseq, npool = 16, 40
    lens = si.draw_lengths(cfg, nseq, 16, 2048, cfg.batch * cfg.seqlen)
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(int(v) for v in lens)),
                      dtype=torch.int32, device="cuda")
    slots = torch.from_numpy(si.draw_slots(cfg, nseq, npool)).cuda()
    init = torch.from_numpy(si.draw_has_init(cfg, nseq)).cuda()
    inp = si.draw_prefill(cfg)
    dev = lambda a: torch.from_numpy(si.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(a).cuda()
    u, z, dt = dev(inp["xbc"][0]), dev(inp["z"][0]), dev(inp["dt_raw"][0])
    w, bias, dtb, A, D = (f32(inp[k]) for k in ("conv_w", "conv_b", "dt_bias", "A", "D"))
    cpool_np, spool_np = si.draw_pools(cfg, npool)
    cpool, spool = dev(cpool_np), f32(spool_np)
    y = torch.empty((u.shape[0], cfg.d_inner), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m2.mamba2_conv_ssd_prefill_varlen_workspace_bytes(
        m2.make_dims(nseq, u.shape[0], cfg.nheads, cfg.ngroups, 64, m2.MAMBA2_BF16)), dtype=torch.uint8,
        device="cuda")

    def step():
        m2.mamba2_conv_ssd_prefill_varlen(u, w, bias, cu, slots, init, cpool, spool, dt, dtb, A, D, z, y,
                                          ngroups=cfg.ngroups, workspace=ws)

    settle(torch, "prefill_varlen", lambda k: step(), args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    return us, [int(v) for v in lens]


CALIB_BYTES = 1 << 30


def copy_calibration(torch):
    """One elementwise kernel of known traffic (torch.neg over 2^28 fp32: reads 1 GiB,
    writes 1 GiB), so counter runs can scale FETCH_SIZE and WRITE_SIZE to bytes."""
    a = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


# ------------------------------------------------------------------------------ CPU baseline
def cpu_baseline(cfg, inp, si):
    """The fp64 oracle timed on this host (built here with gcc -O3 -march=native, no
    fast-math), on the same seeded inputs as the GPU step.

    ``value``: the whole 12B-shape 8192-token prefill step (conv1d over all tokens and
    channels, then the sequential scan over all heads) on every thread. Beside it, one
    thread: the tiny all-fp32 layer (whole), the 12B step on one head per group (8 of
    160 heads: the conv of their channels and their scan, scaled to all heads, labelled
    extrapolated), and the 9B batch-64 decode step (whole); the decode step on every
    thread too. About 10-20 s of CPU work in all."""
    import tempfile

    import numpy as np
    import oracle

    d64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    out_dir = tempfile.mkdtemp(prefix="oracle_native_")
    lib = oracle.load_native(out_dir)
    with oracle.use(lib):
        threads = oracle.threads(0)

        def prefill(c, i, heads=None, nthreads=0):
            """conv1d + scan of the prefill inputs ``i`` (heads: a subset, its channels only)"""
            u = d64(i["xbc"])
            w, b = i["conv_w"], i["conv_b"]
            H, G = c.nheads, c.ngroups
            if heads is not None:
                di, gn = c.d_inner, c.ngroups * c.dstate
                cols = np.concatenate([np.arange(h * 64, h * 64 + 64) for h in heads])
                chans = np.concatenate([cols, np.arange(di, di + 2 * gn)])
                u, w, b = np.ascontiguousarray(u[..., chans]), w[chans], b[chans]
                H = len(heads)
            t0 = time.perf_counter()
            xr, _ = oracle.conv1d(u, w, b, None, nthreads=nthreads)
            t1 = time.perf_counter()
            x, Bm, Cm = (np.ascontiguousarray(a) for a in oracle.split_xbc(xr, H, G))
            if heads is None:
                z, dt, dtb, A, D = i["z"], i["dt_raw"], i["dt_bias"], i["A"], i["D"]
            else:
                z, dt = i["z"][..., cols], i["dt_raw"][..., heads]
                dtb, A, D = i["dt_bias"][heads], i["A"][heads], i["D"][heads]
            oracle.ssd_scan(x, Bm, Cm, d64(dt), dtb, A, D, d64(z), None, ngroups=G, nthreads=nthreads)
            return t1 - t0, time.perf_counter() - t1

        t_conv, t_scan = prefill(cfg, inp)
        full = t_conv + t_scan

        tcfg = si.TINY_F32
        c0, s0 = prefill(tcfg, si.draw_prefill(tcfg), nthreads=1)
        hpg = cfg.nheads // cfg.ngroups
        heads = [g * hpg for g in range(cfg.ngroups)]
        c1, s1 = prefill(cfg, inp, heads=heads, nthreads=1)
        # the subset's conv covers its x channels and all B and C channels; scaled per
        # channel and per head to the whole layer
        di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
        sub_ch = len(heads) * 64 + 2 * gn
        one_thread_step = c1 * cfg.conv_channels / sub_ch + s1 * cfg.nheads / len(heads)

        dcfg = si.DECODE_9B_B64
        dp = si.draw_params(dcfg)
        st = si.draw_decode_step(dcfg, 0)
        h0, cs0 = d64(si.draw_h0(dcfg)), d64(si.draw_conv_state(dcfg))

        def decode(nthreads):
            t0 = time.perf_counter()
            oracle.state_update(st["xbc"][:, 0], dp["conv_w"], dp["conv_b"], cs0, st["dt_raw"][:, 0],
                                dp["dt_bias"], dp["A"], dp["D"], st["z"][:, 0], h0, nheads=dcfg.nheads,
                                ngroups=dcfg.ngroups, nthreads=nthreads)
            return time.perf_counter() - t0

        dec_all = min(decode(0) for _ in range(3))
        dec_one = min(decode(1) for _ in range(2))

    tok = cfg.batch * cfg.seqlen
    return {"value": tok / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole 12B 8192-token prefill step once, unscaled, {threads} threads: fp64 "
                      f"conv1d over {cfg.conv_channels} channels ({t_conv:.2f} s) and the sequential "
                      f"scan of all {cfg.nheads} heads ({t_scan:.2f} s); oracle built with gcc -O3 "
                      f"-march=native on this host",
            "build": "gcc -O3 -march=native -ffp-contract=off, no fast-math, OpenMP",
            "single_thread": {
                "tiny_f32_prefill": {"s": c0 + s0, "tokens_per_s": tcfg.batch * tcfg.seqlen / (c0 + s0),
                                     "note": "1 x 256 tokens, 4 heads, whole"},
                "prefill_12b_8k": {"s": one_thread_step, "tokens_per_s": tok / one_thread_step,
                                   "extrapolated": True,
                                   "note": f"heads {heads} (one per group) timed: conv of their "
                                           f"{sub_ch} channels {c1:.2f} s, scan {s1:.2f} s; scaled to "
                                           f"{cfg.conv_channels} channels and {cfg.nheads} heads"},
                "decode_9b_b64": {"us_per_step": dec_one * 1e6,
                                  "tokens_per_s": dcfg.batch / dec_one, "note": "whole step"},
            },
            "decode_9b_b64": {"us_per_step": dec_all * 1e6, "tokens_per_s": dcfg.batch / dec_all,
                              "threads": threads,
                              "note": "whole step, best of 3 (the oracle returns new fp64 copies of the "
                                      "256 MiB state and the conv cache, inside the timing)"}}


# ------------------------------------------------------------------------------ counters
def counter_kernels(chunk: int) -> dict:
    """traffic entry -> (mangled) kernel-name fragments summed per call, for the bf16 prefill
    at chunk length ``chunk``"""
    # every chunk runs the 64-token kernels; rocprofv3 gives a kernel's name mangled, demangled,
    # or cut to its bare name (then numbered in dispatch order where several share it: the
    # one-call step's scan is dispatched first)
    scan = ("ssd_scan64_kernelIDF16bLb0ELb0ELb0E", "ssd_scan64_kernel<__hip_bfloat16, false, false, false>",
            "ssd_scan64_kernel#1")
    return {"conv_ssd_prefill": ["ssd_prep_kernelIDF16bLi64ELb1ELb0E",
                                 ("ssd_scan64_kernelIDF16bLb1ELb0ELb0E",
                                  "ssd_scan64_kernel<__hip_bfloat16, true, false, false>",
                                  "ssd_scan64_kernel#0", "ssd_scan64_kernel")],
            "ssd_prefill": ["ssd_prep_kernelIDF16bLi64ELb0ELb0E", scan],
            "conv1d": ["conv1d_kernel"],
            "state_update": [("state_update_kernelIDF16bLi1E", "state_update_kernel<__hip_bfloat16, 1>",
                              "state_update_kernel")],
            "group_rmsnorm": ["group_rmsnorm_kernel"]}


def _counter_means(path: str, counter: str):
    """Mean counter value per kernel name over its dispatches in a rocprofv3
    counter_collection.csv, and the largest single-dispatch value of torch's elementwise
    kernels (the calibration kernel is by far the largest of those in a bench run)."""
    import csv
    acc, calib = {}, 0.0
    with open(path, newline="") as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    # the mixer runs last and launches some of the same kernels at other strides: only the
    # dispatches before its first GEMM (a hipBLASLt "Cijk" kernel) are counted
    gemm = [int(r["Dispatch_Id"]) for r in rows if "Cijk" in r["Kernel_Name"]]
    cut = min(gemm) if gemm else None
    for row in rows:
        if cut is not None and int(row["Dispatch_Id"]) >= cut:
            continue
        v = float(row["Counter_Value"])
        a = acc.setdefault((row["Kernel_Name"], row["Kernel_Id"]), [0.0, 0, int(row["Dispatch_Id"])])
        a[0] += v
        a[1] += 1
        a[2] = min(a[2], int(row["Dispatch_Id"]))
        if "elementwise_kernel" in row["Kernel_Name"]:
            calib = max(calib, v)
    # Template instantiations can share one (demangled, argument-less) name: such names get
    # "#0", "#1", ... in the order of their first dispatch. In a bench run the one-call step
    # runs first, so "ssd_scan64_kernel#0" is its scan and "#1" the two-call path's.
    names = {}
    for (name, kid), a in acc.items():
        names.setdefault(name, []).append((a[2], kid))
    out = {}
    for (name, kid), a in acc.items():
        ids = sorted(names[name])
        key = name if len(ids) == 1 else f"{name}#{ids.index((a[2], kid))}"
        out[key] = a[0] / a[1]
    return out, calib


def summarize_counters(fetch_csv: str, write_csv: str, chunk: int) -> dict:
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch),
    each scaled by what the same counter reads for the calibration kernel (torch.neg over
    1 GiB in, 1 GiB out). Writes profiles/traffic.json keyed by the kernel source hash."""
    fetch, f_kib = _counter_means(fetch_csv, "FETCH_SIZE")
    write, w_kib = _counter_means(write_csv, "WRITE_SIZE")
    if f_kib <= 0 or w_kib <= 0:
        raise SystemExit("no calibration dispatch found: run the counter passes with --copy-calibration")

    def pick(table, frag):
        alts = frag if isinstance(frag, tuple) else (frag,)   # mangled or demangled name
        hits = [v for k, v in table.items() if k in alts] or \
            [v for k, v in table.items() if any(a in k for a in alts)]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {frag!r}, found {len(hits)}: "
                             f"{sorted(table)}")
        return hits[0]

    f_cal = CALIB_BYTES / (f_kib * 1024.0)
    w_cal = CALIB_BYTES / (w_kib * 1024.0)
    out = {"_calibration": {"kernel": "torch.neg over 2^28 fp32 (1 GiB read, 1 GiB written)",
                            "fetch_factor": f_cal, "write_factor": w_cal}}
    for key, frags in counter_kernels(chunk).items():
        fb = sum(pick(fetch, fr) for fr in frags) * 1024.0 * f_cal
        wb = sum(pick(write, fr) for fr in frags) * 1024.0 * w_cal
        out[key] = {"source_hash": kernel_source_hash(key), "fetch_bytes": fb, "write_bytes": wb,
                    "bytes_per_launch": fb + wb, "kernels": frags}
        if key == "ssd_prefill":
            out[key]["chunk"] = chunk
        if key == "conv_ssd_prefill":
            out[key]["chunk"] = 64
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


# ------------------------------------------------------------------------------ main
def progress(what: str) -> None:
    """One line on stderr as each workload starts (the JSON line goes to stdout)."""
    print(f"[bench] {what}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # a few hundred warm-up steps (~0.1 s): the first tens of milliseconds of GPU work run at
    # lower clocks
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--decode-steps", type=int, default=100)
    # GPU time each workload runs before its warm-up, whatever --warmup is: the clocks ramp
    # up over the first tens of milliseconds after the host has left the GPU idle
    ap.add_argument("--settle-ms", type=float, default=250.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run only what profiles/traffic.json is made from (with --copy-calibration): the "
                         "one-call and two-call prefills, the decode and the group RMSNorm, and print nothing")
    ap.add_argument("--chunk", type=int, default=64, help="scan chunk length of the timed prefill")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs of this script into profiles/traffic.json")
    args = ap.parse_args()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters, args.chunk), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer core runs on a single MI355X with no "
              "collectives, so --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import seeded_inputs as si
    import state_space_sequence_causal_amd as m2

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)
    cfg = si.PREFILL_12B_8K
    inp = si.draw_prefill(cfg)
    progress("12B 8k one-call prefill (the step)")
    ms_step, wall, (step_us,) = run_prefill(args, torch, m2, si, cfg, inp, args.chunk)
    progress("12B 8k two-call prefill")
    _, _, (conv_us, ssd_us) = run_prefill(args, torch, m2, si, cfg, inp, args.chunk, fused=False)
    alt = None
    if args.chunk != cfg.chunk:
        progress(f"12B 8k one-call prefill at chunk {cfg.chunk}")
        alt = run_prefill(args, torch, m2, si, cfg, inp, cfg.chunk)
    by = prefill_bytes(cfg)
    fl = prefill_flops(cfg)
    tokens = cfg.batch * cfg.seqlen
    ssd_gbs = by["ssd"] / (ssd_us * 1e-6) / 1e9
    step_gbs = by["fused"] / (step_us * 1e-6) / 1e9
    fused_kernels = counter_kernels(64)["conv_ssd_prefill"] if args.chunk == 64 else \
        ["conv1d_kernel"] + counter_kernels(args.chunk)["ssd_prefill"]
    if args.counter_pass:
        # the kernels of the traffic table, in the order summarize_counters expects; the rest of
        # the bench (thousands of small dispatches in the generation run) is left out of the
        # counter runs
        progress("9B batch-64 decode")
        run_decode(args, torch, m2, si)
        progress("group RMSNorm")
        run_rmsnorm(args, torch, m2, si, cfg)
        return
    progress("phase profile")
    phases = run_phase_profile(args, torch, m2, si, cfg, inp)
    progress("9B batch-64 decode")
    dcfg, dec_us, dec_p50 = run_decode(args, torch, m2, si)
    progress("group RMSNorm")
    rms_us, rms_bytes = run_rmsnorm(args, torch, m2, si, cfg)
    progress("packed prefill")
    vl_us, vl_lens = run_varlen(args, torch, m2, si, cfg)
    progress("9B batch-64 decode, 4 tokens")
    dec4 = run_decode_tokens(args, torch, m2, si, 4)
    progress("mixer prefill")
    mix_pre = run_mixer_prefill(args, torch, m2, si, cfg)
    progress("mixer step")
    mix_step = run_mixer_step(args, torch, m2, si)
    progress("generation run")
    gen_run = run_generation(args, torch, m2, si)
    progress("other prefills")
    others = run_other_prefills(args, torch, m2, si)
    dby = decode_bytes(dcfg)
    dec_gbs = dby / (dec_us * 1e-6) / 1e9

    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "12B-shape Mamba-2 layer-core prefill: conv1d + chunked SSD scan (one call)",
                   "batch": cfg.batch, "seq_len": cfg.seqlen, "nheads": cfg.nheads,
                   "headdim": cfg.headdim, "ngroups": cfg.ngroups, "dstate": cfg.dstate,
                   "conv_width": cfg.conv_width, "chunk": args.chunk, "io": "bf16",
                   "state": "fp32", "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "mamba2_conv_ssd_prefill (" + (
                         "ssd_prep_kernel<bf16, 64, conv> + ssd_scan64_kernel<conv>" if args.chunk == 64 else
                         " + ".join(k.split("IDF16b")[0] for k in fused_kernels)) + ")",
                     "bound": "hbm", "achieved": step_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": step_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("conv_ssd_prefill", 64) if args.chunk == 64 else None,
                     "algorithmic_bytes": by["fused"], "avg_launch_us": step_us, "phases": phases},
        "kernels": {
            "conv_ssd_prefill": {"us": step_us, "tokens_per_s": tokens / (step_us * 1e-6), "GB_s": step_gbs,
                                 "algorithmic_TFLOP_s": fl / (step_us * 1e-6) / 1e12},
            "ssd_prefill": {"us": ssd_us, "tokens_per_s": tokens / (ssd_us * 1e-6), "GB_s": ssd_gbs,
                            "frac": ssd_gbs / HBM_PEAK_GBS, "algorithmic_bytes": by["ssd"],
                            "algorithmic_TFLOP_s": fl / (ssd_us * 1e-6) / 1e12,
                            "mfma_frac_algorithmic": fl / (ssd_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                            "traffic": measured_traffic("ssd_prefill", args.chunk),
                            "note": "two-call path: the scan after mamba2_conv1d"},
            "conv1d": {"us": conv_us, "GB_s": by["conv"] / (conv_us * 1e-6) / 1e9,
                       "frac": by["conv"] / (conv_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                       "traffic": measured_traffic("conv1d"),
                       "note": "two-call path: the conv over all xBC channels"},
            "two_call_step_us": conv_us + ssd_us,
        },
        "decode": {"workload": "9B-shape decode state update: B=64, 128 heads x 64, 8 groups, "
                               "d_state 128, bf16 io, fp32 state (256 MiB), in place",
                   "us_per_step": dec_us, "us_p50": dec_p50, "GB_s": dec_gbs,
                   "hbm_frac": dec_gbs / HBM_PEAK_GBS, "algorithmic_bytes": dby,
                   "tokens_per_s": dcfg.batch / (dec_us * 1e-6),
                   "traffic": measured_traffic("state_update"),
                   "tokens4": dec4},
        "mixer": {"prefill_12b_8k": mix_pre, "step_9b_b64": mix_step},
        "generation_9b_b8": gen_run,
        "other_prefills": others,
        "wall_s_timed": wall,
        "settle_ms": {k: round(v, 1) for k, v in SETTLE_MS.items()},
        "environment": run_environment(torch),
    }
    out["kernels"]["group_rmsnorm"] = {
        "us": rms_us, "GB_s": rms_bytes / (rms_us * 1e-6) / 1e9,
        "frac": rms_bytes / (rms_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": rms_bytes,
        "traffic": measured_traffic("group_rmsnorm"),
        "note": "block RMSNorm of the gated output over 8 groups of 1280 channels (not in the step)"}
    out["kernels"]["conv_ssd_prefill_varlen"] = {
        "us": vl_us, "tokens_per_s": tokens / (vl_us * 1e-6), "lengths": vl_lens,
        "note": "continuous batch: 16 packed sequences of the 12B shape summing to 8192 tokens, "
                "states in a pool of 40 entries, half continuing from their entry (not the step)"}
    if alt is not None:
        out["kernels"][f"conv_ssd_prefill_chunk{cfg.chunk}"] = {
            "us": alt[2][0], "tokens_per_s": tokens / (alt[2][0] * 1e-6),
            "note": "the one call at the listed chunk (a tiling choice: the same 64-token kernels run)"}
    if not args.no_cpu_baseline:
        progress("CPU baseline (the oracle)")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, si)
    print(json.dumps(out))


if __name__ == "__main__":
    main()

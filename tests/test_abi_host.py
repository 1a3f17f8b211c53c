"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function include/mamba2.h declares, and rejects bad arguments before touching
the device. The fake pointers below are never dereferenced: validation fails
first, so no HIP call is made."""
import ctypes
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "mamba2.h")

m2 = pytest.importorskip("state_space_sequence_causal_amd")

OK, ENULL, ESHAPE, EUNSUP, EDTYPE, EALIGN, EALIAS = 0, 1, 2, 3, 4, 5, 6
BASE = 1 << 40          # fake, 16-byte aligned device addresses far apart
MB = 1 << 30


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(mamba2_\w+)\(", text, re.M)))


def test_header_declares_the_calls():
    names = declared()
    for n in ("mamba2_conv1d", "mamba2_ssd_prefill", "mamba2_state_update", "mamba2_group_rmsnorm",
              "mamba2_conv_ssd_prefill", "mamba2_conv_ssd_prefill_workspace_bytes",
              "mamba2_conv_ssd_prefill_varlen", "mamba2_state_update_slots",
              "mamba2_ssd_prefill_workspace_bytes", "mamba2_mixer_prefill", "mamba2_mixer_step",
              "mamba2_mixer_prefill_workspace_bytes", "mamba2_mixer_step_workspace_bytes",
              "mamba2_last_error", "mamba2_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m2.LIB_PATH)
    for n in declared():
        assert hasattr(lib, n), n


def test_abi_version():
    assert m2.mamba2_abi_version() == 8


def dims(**kw):
    d = dict(batch=1, seqlen=256, nheads=4, ngroups=1, chunk=64, io=m2.MAMBA2_F32)
    d.update(kw)
    return m2.make_dims(**d)


def prefill(d, **kw):
    H, G = d.nheads, d.ngroups
    a = dict(x=BASE, xs=H * 64, Bm=BASE + 4 * MB, bs=G * 128, Cm=BASE + 6 * MB, cs=G * 128,
             dt=BASE + 8 * MB, dtb=BASE + 9 * MB, A=BASE + 10 * MB, D=BASE + 11 * MB,
             z=BASE + 12 * MB, zs=H * 64, h0=BASE + 16 * MB, hf=BASE + 20 * MB, y=BASE + 24 * MB,
             ys=H * 64)
    a.update(kw)
    return m2.lib.mamba2_ssd_prefill(ctypes.byref(d), a["x"], a["xs"], a["Bm"], a["bs"], a["Cm"],
                                     a["cs"], a["dt"], a["dtb"], a["A"], a["D"], a["z"], a["zs"],
                                     a["h0"], a["hf"], a["y"], a["ys"], a.get("ws", BASE + 64 * MB),
                                     a.get("wsb", 1 << 30), None)


def conv(d, channels=512, **kw):
    a = dict(u=BASE, us=channels, w=BASE + 4 * MB, b=BASE + 5 * MB, cs=BASE + 6 * MB,
             out=BASE + 8 * MB, os=channels)
    a.update(kw)
    return m2.lib.mamba2_conv1d(ctypes.byref(d), channels, a["u"], a["us"], a["w"], a["b"], a["cs"],
                                a["out"], a["os"], None)


def decode(d, **kw):
    a = dict(u=BASE, w=BASE + 1 * MB, b=BASE + 2 * MB, cs=BASE + 3 * MB, dt=BASE + 4 * MB,
             dtb=BASE + 5 * MB, A=BASE + 6 * MB, D=BASE + 7 * MB, z=BASE + 8 * MB,
             ss=BASE + 16 * MB, y=BASE + 9 * MB)
    a.update(kw)
    return m2.lib.mamba2_state_update(ctypes.byref(d), a["u"], a["w"], a["b"], a["cs"], a["dt"],
                                      a["dtb"], a["A"], a["D"], a["z"], a["ss"], a["y"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(io=7), EDTYPE), (dict(batch=0), ESHAPE), (dict(seqlen=-1), ESHAPE),
    (dict(nheads=6, ngroups=4), ESHAPE), (dict(nheads=0), ESHAPE),
    (dict(headdim=32), EUNSUP), (dict(dstate=64), EUNSUP), (dict(conv_width=3), EUNSUP),
    (dict(chunk=512), EUNSUP), (dict(chunk=512, io=m2.MAMBA2_BF16), EUNSUP), (dict(chunk=48), EUNSUP),
])
def test_prefill_rejects_dims(kw, code):
    assert prefill(dims(**kw)) == code
    assert m2.mamba2_last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(Bm=None), ENULL), (dict(Cm=None), ENULL), (dict(dt=None), ENULL),
    (dict(dtb=None), ENULL), (dict(A=None), ENULL), (dict(y=None), ENULL),
    (dict(x=BASE + 4), EALIGN), (dict(xs=255), ESHAPE), (dict(xs=258), EALIGN),
    (dict(bs=100), ESHAPE), (dict(ys=250), ESHAPE), (dict(h0=BASE + 16 * MB + 8), EALIGN),
    (dict(y=BASE + 4 * MB), EALIAS), (dict(y=BASE), EALIAS), (dict(hf=BASE + 12 * MB), EALIAS),
    (dict(y=BASE + 20 * MB), EALIAS), (dict(hf=BASE + 16 * MB + 4096), EALIAS),
    (dict(xs=(1 << 23) + 4), ESHAPE), (dict(zs=(1 << 23) + 4), ESHAPE),
])
def test_prefill_rejects_pointers(kw, code):
    assert prefill(dims(), **kw) == code, m2.mamba2_last_error()


def test_dims_null():
    assert m2.lib.mamba2_ssd_prefill(None, BASE, 256, BASE, 128, BASE, 128, BASE, BASE, BASE, None,
                                     None, 0, None, None, BASE, 256, None, 0, None) == ENULL
    assert m2.lib.mamba2_ssd_prefill_workspace_bytes(None) == 0


@pytest.mark.parametrize("kw,chan,code", [
    (dict(u=None), 512, ENULL), (dict(w=None), 512, ENULL), (dict(out=None), 512, ENULL),
    (dict(), 510, ESHAPE), (dict(), 0, ESHAPE), (dict(us=500), 512, ESHAPE),
    (dict(u=BASE + 8), 512, EALIGN), (dict(w=BASE + 4 * MB + 4), 512, EALIGN),
    (dict(out=BASE), 512, EALIAS), (dict(cs=BASE + 8 * MB), 512, EALIAS), (dict(cs=BASE), 512, EALIAS),
])
def test_conv_rejects(kw, chan, code):
    assert conv(dims(), channels=chan, **kw) == code, m2.mamba2_last_error()


def test_conv_bf16_needs_multiple_of_8():
    assert conv(dims(io=m2.MAMBA2_BF16), channels=4, us=8, os=8) == ESHAPE


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), ENULL), (dict(cs=None), ENULL), (dict(ss=None), ENULL), (dict(y=None), ENULL),
    (dict(ss=BASE + 16 * MB + 4), EALIGN), (dict(y=BASE), EALIAS), (dict(cs=BASE + 16 * MB), EALIAS),
])
def test_decode_rejects(kw, code):
    assert decode(dims(seqlen=1), **kw) == code, m2.mamba2_last_error()


def test_decode_token_count():
    """1 to 6 new tokens per sequence."""
    assert decode(dims(seqlen=0)) == ESHAPE
    assert decode(dims(seqlen=7)) == ESHAPE
    assert decode(dims(seqlen=1, nheads=512, ngroups=1)) == EUNSUP
    # the token rows count in the overlap checks: y right after 2 rows of u_t overlaps at T = 3
    d = dims(seqlen=3, batch=1)
    cc = d.nheads * 64 + 2 * d.ngroups * 128
    assert decode(d, y=BASE + 2 * cc * 4) == EALIAS


def test_workspace_size_formula():
    """Per (sequence, group, 64-token chunk): fp32 causal Gram tiles + B^T and C operand
    tiles. The named chunk is a tiling choice: every supported one tiles at 64."""
    for io, es in ((m2.MAMBA2_BF16, 2), (m2.MAMBA2_F32, 4)):
        for chunk in (64, 128, 256):
            d = dims(io=io, chunk=chunk, batch=3, seqlen=1000, nheads=16, ngroups=8)
            rec = 4 * 1024 * 3 + 2 * 128 * 64 * es
            nc = -(-1000 // 64)
            assert m2.mamba2_ssd_prefill_workspace_bytes(d) == nc * 3 * 8 * rec
    assert m2.mamba2_ssd_prefill_workspace_bytes(dims(seqlen=0)) == 0
    assert m2.mamba2_ssd_prefill_workspace_bytes(dims(chunk=100)) == 0
    assert m2.lib.mamba2_ssd_prefill_workspace_bytes(None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(ws=None), 7), (dict(wsb=1000), 7), (dict(ws=BASE + 64 * MB + 8), EALIGN),
    (dict(ws=BASE + 4 * MB), EALIAS), (dict(ws=BASE + 24 * MB), EALIAS),
])
def test_prefill_rejects_workspace(kw, code):
    assert prefill(dims(), **kw) == code, m2.mamba2_last_error()


def rmsnorm(d, **kw):
    a = dict(g=BASE, gs=d.nheads * 64, w=BASE + 8 * MB, eps=1e-5, out=BASE + 16 * MB, os=d.nheads * 64)
    a.update(kw)
    return m2.lib.mamba2_group_rmsnorm(ctypes.byref(d), a["g"], a["gs"], a["w"], a["eps"], a["out"],
                                       a["os"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), ENULL), (dict(out=None), ENULL), (dict(gs=200), ESHAPE), (dict(eps=-1.0), ESHAPE),
    (dict(eps=float("nan")), ESHAPE), (dict(eps=float("inf")), ESHAPE), (dict(gs=258), EALIGN),
    (dict(g=BASE + 4), EALIGN), (dict(w=BASE + 8 * MB + 4), EALIGN),
    (dict(out=BASE + 1024), EALIAS), (dict(out=BASE, os=512), EALIAS), (dict(w=BASE + 16 * MB), EALIAS),
])
def test_rmsnorm_rejects(kw, code):
    assert rmsnorm(dims(), **kw) == code, m2.mamba2_last_error()


def test_rmsnorm_rejects_model_shape():
    assert rmsnorm(dims(nheads=6, ngroups=4)) == ESHAPE
    assert rmsnorm(dims(seqlen=0), g=None, out=None) == OK


# ------------------------------------------------------------------ conv + prefill in one call
def conv_prefill(d, **kw):
    H, G = d.nheads, d.ngroups
    cc = H * 64 + 2 * G * 128
    a = dict(u=BASE, us=cc, w=BASE + 4 * MB, b=BASE + 5 * MB, cs=BASE + 6 * MB, dt=BASE + 8 * MB,
             dtb=BASE + 9 * MB, A=BASE + 10 * MB, D=BASE + 11 * MB, z=BASE + 12 * MB, zs=H * 64,
             h0=BASE + 16 * MB, hf=BASE + 20 * MB, y=BASE + 24 * MB, ys=H * 64, ws=BASE + 64 * MB,
             wsb=1 << 30)
    a.update(kw)
    return m2.lib.mamba2_conv_ssd_prefill(ctypes.byref(d), a["u"], a["us"], a["w"], a["b"], a["cs"],
                                          a["dt"], a["dtb"], a["A"], a["D"], a["z"], a["zs"], a["h0"],
                                          a["hf"], a["y"], a["ys"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), ENULL), (dict(w=None), ENULL), (dict(dt=None), ENULL), (dict(y=None), ENULL),
    (dict(dtb=None), ENULL), (dict(A=None), ENULL),
    (dict(us=500), ESHAPE), (dict(us=1028), EALIGN), (dict(u=BASE + 8), EALIGN),
    (dict(w=BASE + 4 * MB + 4), EALIGN), (dict(cs=BASE + 6 * MB + 8), EALIGN),
    (dict(us=(1 << 23) + 8), ESHAPE), (dict(ys=250), ESHAPE),
    (dict(y=BASE), EALIAS), (dict(y=BASE + 6 * MB), EALIAS), (dict(cs=BASE), EALIAS),
    (dict(cs=BASE + 24 * MB), EALIAS), (dict(hf=BASE), EALIAS), (dict(cs=BASE + 16 * MB), EALIAS),
    (dict(ws=BASE + 6 * MB), EALIAS), (dict(ws=None), 7), (dict(wsb=1000), 7),
])
def test_conv_prefill_rejects(kw, code):
    d = dims(io=m2.MAMBA2_BF16)
    assert conv_prefill(d, **kw) == code, m2.mamba2_last_error()


def test_conv_prefill_rejects_dims():
    assert conv_prefill(dims(chunk=512)) == EUNSUP
    assert conv_prefill(dims(io=m2.MAMBA2_BF16, chunk=48)) == EUNSUP
    assert conv_prefill(dims(nheads=6, ngroups=4)) == ESHAPE


def test_conv_prefill_workspace_size():
    """Fused (bf16, any chunk): the prefill's workspace; fp32: that (rounded up to 256 bytes)
    plus the conv output of all xBC channels."""
    for io, es, chunk in ((m2.MAMBA2_BF16, 2, 64), (m2.MAMBA2_BF16, 2, 128), (m2.MAMBA2_BF16, 2, 256),
                          (m2.MAMBA2_F32, 4, 64), (m2.MAMBA2_F32, 4, 256)):
        d = dims(io=io, chunk=chunk, batch=3, seqlen=1000, nheads=16, ngroups=8)
        base = m2.mamba2_ssd_prefill_workspace_bytes(d)
        want = base if io == m2.MAMBA2_BF16 else \
            -(-base // 256) * 256 + 3 * 1000 * (16 * 64 + 2 * 8 * 128) * es
        assert m2.mamba2_conv_ssd_prefill_workspace_bytes(d) == want
    assert m2.mamba2_conv_ssd_prefill_workspace_bytes(dims(seqlen=0)) == 0
    assert m2.lib.mamba2_conv_ssd_prefill_workspace_bytes(None) == 0


def test_noalloc_prefill_rejects_before_any_launch():
    """mamba2_conv_ssd_prefill_noalloc checks dims and its 64 MiB static scratch on the host:
    a setting whose workspace would not fit is refused (MAMBA2_ERR_WORKSPACE) before anything
    touches a device; at the 12B shape (bf16) 11904 tokens (186 chunks) fit and 11905 do not."""
    fit = dims(io=m2.MAMBA2_BF16, batch=1, seqlen=11904, nheads=160, ngroups=8)
    assert m2.mamba2_conv_ssd_prefill_workspace_bytes(fit) <= 64 << 20
    for d, code in ((dims(io=m2.MAMBA2_BF16, batch=1, seqlen=11905, nheads=160, ngroups=8), 7),
                    (dims(io=m2.MAMBA2_BF16, batch=2, seqlen=8192, nheads=160, ngroups=8), 7),
                    (dims(nheads=6, ngroups=4), ESHAPE), (dims(chunk=48), EUNSUP)):
        H, G = d.nheads, d.ngroups
        cc = H * 64 + 2 * G * 128
        st = m2.lib.mamba2_conv_ssd_prefill_noalloc(
            ctypes.byref(d), BASE, cc, BASE + 4 * MB, BASE + 5 * MB, BASE + 6 * MB, BASE + 8 * MB, BASE + 9 * MB,
            BASE + 10 * MB, BASE + 11 * MB, BASE + 12 * MB, H * 64, BASE + 16 * MB, BASE + 20 * MB, BASE + 24 * MB,
            H * 64, None)
        assert st == code, m2.mamba2_last_error()


# ------------------------------------------------------------------ decode with slot pools
def decode_slots(d, **kw):
    a = dict(u=BASE, w=BASE + 1 * MB, b=BASE + 2 * MB, cs=BASE + 3 * MB, dt=BASE + 4 * MB,
             dtb=BASE + 5 * MB, A=BASE + 6 * MB, D=BASE + 7 * MB, z=BASE + 8 * MB,
             ss=BASE + 64 * MB, sl=BASE + 9 * MB, npool=4, y=BASE + 10 * MB)
    a.update(kw)
    return m2.lib.mamba2_state_update_slots(ctypes.byref(d), a["u"], a["w"], a["b"], a["cs"], a["dt"],
                                            a["dtb"], a["A"], a["D"], a["z"], a["ss"], a["sl"], a["npool"],
                                            a["y"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(sl=None), ENULL), (dict(u=None), ENULL), (dict(y=None), ENULL), (dict(cs=None), ENULL),
    (dict(npool=-1), ESHAPE), (dict(sl=BASE + 9 * MB + 2), EALIGN), (dict(ss=BASE + 64 * MB + 4), EALIGN),
    (dict(y=BASE), EALIAS), (dict(cs=BASE + 64 * MB), EALIAS), (dict(sl=BASE + 10 * MB), EALIAS),
])
def test_decode_slots_rejects(kw, code):
    assert decode_slots(dims(seqlen=1, batch=3), **kw) == code, m2.mamba2_last_error()


def test_decode_slots_token_count():
    assert decode_slots(dims(seqlen=0)) == ESHAPE
    assert decode_slots(dims(seqlen=7)) == ESHAPE


# ------------------------------------------------------------------ packed prefill
def varlen(d, **kw):
    cc = d.nheads * 64 + 2 * d.ngroups * 128
    a = dict(u=BASE, us=cc, w=BASE + 4 * MB, b=BASE + 5 * MB, cu=BASE + 6 * MB, sl=BASE + 7 * MB,
             hi=BASE + 8 * MB, cp=BASE + 9 * MB, sp=BASE + 64 * MB, npool=4, dt=BASE + 10 * MB,
             dtb=BASE + 11 * MB, A=BASE + 12 * MB, D=BASE + 13 * MB, z=BASE + 14 * MB, zs=d.nheads * 64,
             y=BASE + 18 * MB, ys=d.nheads * 64, ws=BASE + 128 * MB, wsb=1 << 30)
    a.update(kw)
    return m2.lib.mamba2_conv_ssd_prefill_varlen(
        ctypes.byref(d), a["u"], a["us"], a["w"], a["b"], a["cu"], a["sl"], a["hi"], a["cp"], a["sp"],
        a["npool"], a["dt"], a["dtb"], a["A"], a["D"], a["z"], a["zs"], a["y"], a["ys"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), ENULL), (dict(u=None), ENULL), (dict(y=None), ENULL), (dict(cp=None), ENULL),
    (dict(npool=-2), ESHAPE), (dict(us=500), ESHAPE), (dict(cu=BASE + 6 * MB + 2), EALIGN),
    (dict(cp=BASE + 9 * MB + 8), EALIGN), (dict(y=BASE), EALIAS), (dict(sp=BASE + 6 * MB), EALIAS),
    (dict(ws=BASE + 18 * MB), EALIAS), (dict(ws=None), 7), (dict(wsb=100), 7),
])
def test_varlen_rejects(kw, code):
    assert varlen(dims(io=m2.MAMBA2_BF16, batch=3, seqlen=300), **kw) == code, m2.mamba2_last_error()


def test_varlen_settings_and_workspace():
    assert varlen(dims(io=m2.MAMBA2_F32, batch=3)) == EUNSUP
    assert varlen(dims(io=m2.MAMBA2_BF16, chunk=512, batch=3)) == EUNSUP
    m = 1000 // 64 + 5
    rec = 4096 * 3 + 2 * 128 * 64 * 2
    for chunk in (64, 128, 256):
        d = dims(io=m2.MAMBA2_BF16, batch=5, seqlen=1000, nheads=16, ngroups=8, chunk=chunk)
        assert m2.mamba2_conv_ssd_prefill_varlen_workspace_bytes(d) == \
            m * (8 * rec + 16 + 384 * 16) + 8 * 6
    assert m2.mamba2_conv_ssd_prefill_varlen_workspace_bytes(dims(io=m2.MAMBA2_F32)) == 0


# ------------------------------------------------------------------ the mixer
def mixer(d, step=False, **kw):
    a = dict(dm=64, h=BASE, hs=64, wi=BASE + 4 * MB, w=BASE + 8 * MB, b=BASE + 9 * MB, cs=BASE + 10 * MB,
             dtb=BASE + 11 * MB, A=BASE + 12 * MB, D=BASE + 13 * MB, h0=BASE + 16 * MB, hf=BASE + 20 * MB,
             ss=BASE + 16 * MB, nw=BASE + 24 * MB, eps=1e-5, wo=BASE + 25 * MB, o=BASE + 32 * MB, os=64,
             ws=BASE + 256 * MB, wsb=1 << 30)
    a.update(kw)
    if step:
        return m2.lib.mamba2_mixer_step(ctypes.byref(d), a["dm"], a["h"], a["hs"], a["wi"], a["w"], a["b"],
                                        a["cs"], a["dtb"], a["A"], a["D"], a["ss"], a["nw"], a["eps"], a["wo"],
                                        a["o"], a["os"], a["ws"], a["wsb"], None)
    return m2.lib.mamba2_mixer_prefill(ctypes.byref(d), a["dm"], a["h"], a["hs"], a["wi"], a["w"], a["b"],
                                       a["cs"], a["dtb"], a["A"], a["D"], a["h0"], a["hf"], a["nw"], a["eps"],
                                       a["wo"], a["o"], a["os"], a["ws"], a["wsb"], None)


MIXER_REJECTS = [
    (dict(wi=None), ENULL), (dict(wo=None), ENULL), (dict(w=None), ENULL), (dict(A=None), ENULL),
    (dict(h=None), ENULL), (dict(o=None), ENULL),
    (dict(dm=0), ESHAPE), (dict(dm=60), ESHAPE), (dict(hs=56), ESHAPE), (dict(os=68), EALIGN),
    (dict(h=BASE + 8), EALIGN), (dict(nw=BASE + 24 * MB + 4), EALIGN), (dict(eps=-1.0), ESHAPE),
    (dict(o=BASE), EALIAS), (dict(o=BASE + 4 * MB), EALIAS), (dict(ws=BASE + 4 * MB), EALIAS),
    (dict(cs=BASE + 4 * MB), EALIAS), (dict(o=BASE + 256 * MB), EALIAS),
    (dict(ws=None), 7), (dict(wsb=1000), 7),
]


@pytest.mark.parametrize("kw,code", MIXER_REJECTS + [(dict(hf=BASE + 25 * MB), EALIAS)])
def test_mixer_prefill_rejects(kw, code):
    assert mixer(dims(io=m2.MAMBA2_BF16), **kw) == code, m2.mamba2_last_error()


@pytest.mark.parametrize("kw,code", MIXER_REJECTS + [(dict(ss=BASE + 25 * MB), EALIAS), (dict(cs=None), ENULL),
                                                     (dict(ss=None), ENULL)])
def test_mixer_step_rejects(kw, code):
    assert mixer(dims(io=m2.MAMBA2_BF16, seqlen=2, batch=3), step=True, **kw) == code, m2.mamba2_last_error()


def test_mixer_settings_and_workspace():
    assert mixer(dims(io=m2.MAMBA2_BF16, chunk=48)) == EUNSUP
    assert mixer(dims(seqlen=7), step=True) == ESHAPE
    assert mixer(dims(seqlen=0), step=True) == ESHAPE
    a256 = lambda v: -(-v // 256) * 256
    for io, es, chunk in ((m2.MAMBA2_BF16, 2, 64), (m2.MAMBA2_BF16, 2, 128), (m2.MAMBA2_F32, 4, 64)):
        d = dims(io=io, chunk=chunk, batch=3, seqlen=1000, nheads=20, ngroups=4)
        E = 2 * 20 * 64 + 2 * 4 * 128 + 20
        Es = -(-E // 8) * 8
        rows = 3 * 1000
        core = m2.mamba2_conv_ssd_prefill_workspace_bytes(d)
        want = a256(rows * Es * es) + 2 * a256(rows * 20 * 64 * es) + a256(core) + (128 << 20)
        assert m2.mamba2_mixer_prefill_workspace_bytes(d, 512) == want
        ds = dims(io=io, batch=5, seqlen=3, nheads=20, ngroups=4)
        assert m2.mamba2_mixer_step_workspace_bytes(ds, 512) == \
            a256(15 * Es * es) + 2 * a256(15 * 20 * 64 * es) + (128 << 20)
    assert m2.mamba2_mixer_prefill_workspace_bytes(dims(), 62) == 0
    assert m2.mamba2_mixer_step_workspace_bytes(dims(seqlen=9), 64) == 0

"""CPU-only checks of the C ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before anything is enqueued (no call here reaches a kernel launch: each one
either fails validation or describes an empty problem)."""
import ctypes
import os
import re

import pytest
import torch

import bit_quantized_decode_amd as bqd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqd.h")

OK, EINVAL, EOVERFLOW, EALIGN, ENULL, EHIP = 0, -1, -2, -3, -4, -5
FAKE = 0x10000  # an aligned, never dereferenced device address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for n in ("cq_prepare", "cq_matvec", "cq_gather_rows", "f8_matvec"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(bqd.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(bqd.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = bqd.lib()
    for code in (OK, EINVAL, EOVERFLOW, EALIGN, ENULL, EHIP):
        assert L.bqd_status_string(code) not in (None, b"", b"unknown status")
    assert L.bqd_status_string(42) == b"unknown status"


def cq(**kw):
    f = dict(output=256, input=200, input_padded=256, group=64, bits=2, row_bytes=64,
             packed=FAKE, norms=FAKE, codebook=FAKE)
    f.update(kw)
    return bqd._CqStruct(**f)


def matvec(m, prepared=FAKE, y=FAKE, batch=1, row_begin=0, row_count=None):
    rc_ = m.output - row_begin if row_count is None else row_count
    return bqd.lib().cq_matvec(ctypes.byref(m), prepared, y, batch, row_begin, rc_, None)


@pytest.mark.parametrize("kw,code", [
    (dict(bits=1), EINVAL), (dict(bits=6), EINVAL), (dict(bits=8), EINVAL),
    (dict(group=3), EINVAL), (dict(group=0), EINVAL), (dict(group=2048, input_padded=2048), EINVAL),
    (dict(input_padded=250), EINVAL), (dict(input_padded=0), EINVAL),
    (dict(input=257), EINVAL), (dict(input=-1), EINVAL),
    (dict(row_bytes=63), EINVAL), (dict(row_bytes=0), EINVAL), (dict(output=-1), EINVAL),
    (dict(output=1 << 30), EINVAL),
    (dict(row_bytes=1 << 62, output=8), EOVERFLOW),
    (dict(packed=0), ENULL), (dict(norms=0), ENULL), (dict(codebook=0), ENULL),
    (dict(norms=FAKE + 1), EALIGN), (dict(codebook=FAKE + 2), EALIGN),
])
def test_cq_matvec_rejects(kw, code):
    assert matvec(cq(**kw)) == code


def test_cq_matvec_argument_errors():
    m = cq()
    assert matvec(m, row_begin=-1, row_count=1) == EINVAL
    assert matvec(m, row_begin=10, row_count=247) == EINVAL
    assert matvec(m, row_begin=257, row_count=0) == EINVAL
    assert matvec(m, batch=-1) == EINVAL
    assert matvec(m, prepared=0) == ENULL
    assert matvec(m, y=0) == ENULL
    assert matvec(m, prepared=FAKE + 2) == EALIGN
    assert matvec(m, y=FAKE + 1) == EALIGN
    # empty problems are valid and enqueue nothing
    assert matvec(m, batch=0) == OK
    assert matvec(m, row_begin=256, row_count=0) == OK
    assert matvec(cq(output=0), prepared=0, y=0) == OK


def test_cq_prepare_argument_errors():
    L = bqd.lib()
    m = cq()
    assert L.cq_prepare(ctypes.byref(m), FAKE, FAKE + 1 << 20, -1, None) == EINVAL
    assert L.cq_prepare(ctypes.byref(m), 0, FAKE, 1, None) == ENULL
    assert L.cq_prepare(ctypes.byref(m), FAKE + 1, FAKE << 4, 1, None) == EALIGN
    assert L.cq_prepare(ctypes.byref(m), FAKE, FAKE + 16, 1, None) == EINVAL  # overlap
    assert L.cq_prepare(ctypes.byref(cq(bits=9)), FAKE, FAKE << 4, 1, None) == EINVAL
    assert L.cq_prepare(ctypes.byref(m), FAKE, FAKE << 4, 0, None) == OK
    assert L.cq_prepare(None, FAKE, FAKE << 4, 1, None) == ENULL


def test_cq_prepare_matvec_argument_errors():
    L = bqd.lib()
    m = cq()
    X, P, Y = FAKE, FAKE << 4, FAKE << 8

    def call(x=X, p=P, y=Y, batch=1, row_begin=0, row_count=256, mm=m):
        return L.cq_prepare_matvec(ctypes.byref(mm), x, p, y, batch, row_begin, row_count, None)

    assert call(batch=-1) == EINVAL
    assert call(x=0) == ENULL
    assert call(p=0) == ENULL
    assert call(y=0) == ENULL
    assert call(x=X + 1) == EALIGN
    assert call(y=Y + 2) == EALIGN
    assert call(p=X + 16) == EINVAL            # prepared overlaps x
    assert call(y=P + 64) == EINVAL            # y overlaps prepared
    assert call(y=X + 4) == EINVAL             # y overlaps x
    assert call(row_begin=10, row_count=247) == EINVAL
    assert call(mm=cq(bits=7)) == EINVAL
    assert call(mm=cq(codebook=0)) == ENULL
    assert call(batch=0) == OK
    assert L.cq_prepare_matvec(None, X, P, Y, 1, 0, 1, None) == ENULL


@pytest.mark.parametrize("args,code", [
    (dict(R=-1), EINVAL), (dict(C=0), EINVAL), (dict(G=0), EINVAL), (dict(G=4097), EINVAL),
    (dict(batch=-1), EINVAL), (dict(R=1 << 30), EINVAL), (dict(C=1 << 28), EINVAL),
    (dict(w=0), ENULL), (dict(scale=0), ENULL), (dict(x=0), ENULL), (dict(y=0), ENULL),
    (dict(x=FAKE + 1), EALIGN), (dict(y=FAKE + 2), EALIGN),
    (dict(batch=0), OK), (dict(R=0), OK),
])
def test_i8_matvec_rejects(args, code):
    a = dict(w=FAKE, R=512, C=4096, scale=FAKE, G=16, x=FAKE, y=FAKE, batch=1)
    a.update(args)
    rc = bqd.lib().i8_matvec(a["w"], a["R"], a["C"], a["scale"], a["G"], a["x"], a["y"],
                             a["batch"], None)
    assert rc == code


def test_kv_int8_argument_errors():
    L = bqd.lib()
    assert L.kv_quantize_int8(FAKE, -1, 128, FAKE, FAKE, None) == EINVAL
    assert L.kv_quantize_int8(FAKE, 4, -1, FAKE, FAKE, None) == EINVAL
    assert L.kv_quantize_int8(0, 4, 128, FAKE, FAKE, None) == ENULL
    assert L.kv_quantize_int8(FAKE, 4, 128, 0, FAKE, None) == ENULL
    assert L.kv_quantize_int8(FAKE, 4, 128, FAKE, 0, None) == ENULL
    assert L.kv_quantize_int8(FAKE + 2, 4, 128, FAKE, FAKE, None) == EALIGN
    assert L.kv_quantize_int8(FAKE, 4, 128, FAKE, FAKE + 1, None) == EALIGN
    assert L.kv_quantize_int8(0, 0, 128, 0, 0, None) == OK
    assert L.kv_int8_dot(FAKE, FAKE, -1, 128, FAKE, FAKE, 1, None) == EINVAL
    assert L.kv_int8_dot(FAKE, FAKE, 4, 0, FAKE, FAKE, 1, None) == EINVAL
    assert L.kv_int8_dot(FAKE, FAKE, 4, 128, FAKE, FAKE, -1, None) == EINVAL
    assert L.kv_int8_dot(0, FAKE, 4, 128, FAKE, FAKE, 1, None) == ENULL
    assert L.kv_int8_dot(FAKE, 0, 4, 128, FAKE, FAKE, 1, None) == ENULL
    assert L.kv_int8_dot(FAKE, FAKE + 1, 4, 128, FAKE, FAKE, 1, None) == EALIGN
    assert L.kv_int8_dot(FAKE, FAKE, 4, 128, FAKE + 2, FAKE, 1, None) == EALIGN
    assert L.kv_int8_dot(FAKE, FAKE, 4, 128, FAKE, FAKE, 0, None) == OK
    assert L.kv_int8_dot(0, 0, 0, 128, 0, 0, 1, None) == OK


def test_hadamard_mlp_argument_errors():
    L = bqd.lib()

    def call(n=FAKE, hidden=512, H=2048, d1=FAKE, d2=FAKE, d3=FAKE, resid=FAKE, u=0, out=FAKE,
             batch=1):
        return L.hadamard_mlp(n, hidden, H, d1, d2, d3, resid, u, out, batch, None)

    assert call(H=3000) == EINVAL
    assert call(H=32768) == EINVAL
    assert call(H=0) == EINVAL
    assert call(hidden=4096) == EINVAL
    assert call(hidden=-1) == EINVAL
    assert call(batch=-1) == EINVAL
    assert call(batch=1 << 31) == EINVAL
    assert call(d2=0) == ENULL
    assert call(n=0) == ENULL
    assert call(out=0) == ENULL
    assert call(resid=FAKE + 2) == EALIGN
    assert call(u=FAKE + 1) == EALIGN
    assert call(batch=0) == OK


def test_cq_matvec_multi_argument_errors():
    L = bqd.lib()
    P = FAKE << 4

    def call(mats, rb=None, rc=None, ys=None, prepared=P, x=None):
        n = len(mats)
        arr = (bqd._CqStruct * max(n, 1))(*mats)
        rbs = None if rb is None else (ctypes.c_int64 * n)(*rb)
        rcs = None if rc is None else (ctypes.c_int64 * n)(*rc)
        yv = (ctypes.c_void_p * max(n, 1))(*(ys or [FAKE << (8 + k) for k in range(n)]))
        if x is None:
            return L.cq_matvec_multi(arr, n, rbs, rcs, prepared, yv, None)
        return L.cq_prepare_matvec_multi(arr, n, rbs, rcs, x, prepared, yv, None)

    m = cq()
    assert call([]) == EINVAL
    assert call([m] * 65) == EINVAL
    assert call([m, cq(group=32)]) == EINVAL                       # unequal groups
    assert call([m, cq(input_padded=512, row_bytes=128)]) == EINVAL  # unequal widths
    assert call([m, m], rb=[0, 10], rc=[256, 247]) == EINVAL        # range past the end
    assert call([m, cq(codebook=0)]) == ENULL
    assert call([m], prepared=0) == ENULL
    assert call([m], prepared=P + 2) == EALIGN
    assert call([m], ys=[P + 64]) == EINVAL                         # output overlaps prepared
    assert call([m], x=FAKE + 1) == EALIGN
    assert call([m, cq(input=100)], x=FAKE) == EINVAL               # unequal inputs, with x
    assert call([m], x=FAKE, ys=[FAKE + 8]) == EINVAL               # output overlaps x
    assert call([m, m], rb=[256, 0], rc=[0, 0]) == OK                # nothing to do
    assert L.cq_matvec_multi(None, 1, None, None, P, (ctypes.c_void_p * 1)(FAKE), None) == ENULL


def test_cq_gather_argument_errors():
    L = bqd.lib()
    m = cq()
    assert L.cq_gather_rows(ctypes.byref(m), FAKE, -1, FAKE << 4, None) == EINVAL
    assert L.cq_gather_rows(ctypes.byref(m), 0, 4, FAKE << 4, None) == ENULL
    assert L.cq_gather_rows(ctypes.byref(m), FAKE + 2, 4, FAKE << 4, None) == EALIGN
    assert L.cq_gather_rows(ctypes.byref(cq(group=6)), FAKE, 4, FAKE << 4, None) == EINVAL
    assert L.cq_gather_rows(ctypes.byref(m), FAKE, 0, FAKE << 4, None) == OK


@pytest.mark.parametrize("args,code", [
    (dict(R=-1), EINVAL), (dict(C=0), EINVAL), (dict(SR=0), EINVAL), (dict(SC=0), EINVAL),
    (dict(SR=513), EINVAL), (dict(SC=4097), EINVAL), (dict(batch=-1), EINVAL),
    (dict(R=1 << 30), EINVAL), (dict(C=1 << 28), EINVAL),
    (dict(w=0), ENULL), (dict(scale=0), ENULL), (dict(x=0), ENULL), (dict(y=0), ENULL),
    (dict(x=FAKE + 1), EALIGN), (dict(y=FAKE + 2), EALIGN),
    (dict(batch=0), OK), (dict(R=0, SR=1), OK),
])
def test_f8_matvec_rejects(args, code):
    a = dict(w=FAKE, R=512, C=4096, scale=FAKE, SR=4, SC=32, x=FAKE, y=FAKE, batch=1)
    a.update(args)
    rc = bqd.lib().f8_matvec(a["w"], a["R"], a["C"], a["scale"], a["SR"], a["SC"], a["x"],
                             a["y"], a["batch"], None)
    assert rc == code


def test_probe_argument_errors():
    L = bqd.lib()
    assert L.bqd_dbg_f16_decode(FAKE + 1, 4, FAKE, None) == EALIGN
    assert L.bqd_dbg_f8_decode(0, 4, FAKE, None) == ENULL
    assert L.bqd_dbg_e8m0_decode(FAKE, -1, FAKE, None) == EINVAL
    assert L.bqd_dbg_f8_decode(FAKE, 0, FAKE, None) == OK
    assert L.bqd_dbg_read_stream(FAKE, 24, FAKE, None) == EINVAL
    assert L.bqd_dbg_read_stream(FAKE, -16, FAKE, None) == EINVAL
    assert L.bqd_dbg_read_stream(FAKE, 1 << 46, FAKE, None) == EINVAL
    assert L.bqd_dbg_read_stream(0, 16, FAKE, None) == ENULL
    assert L.bqd_dbg_read_stream(FAKE, 16, 0, None) == ENULL
    assert L.bqd_dbg_read_stream(FAKE + 8, 16, FAKE, None) == EALIGN
    assert L.bqd_dbg_read_stream(FAKE, 16, FAKE + 2, None) == EALIGN
    assert L.bqd_dbg_read_stream(0, 0, 0, None) == OK
    m = cq()
    assert L.bqd_dbg_cq_unpack(ctypes.byref(m), 256, FAKE, None) == EINVAL
    assert L.bqd_dbg_cq_unpack(ctypes.byref(m), 0, 0, None) == ENULL


SAMPLE_NEED = (246272 + 1023) // 1024 * 64 * 8  # workspace bytes for n = 246272, k = 64


@pytest.mark.parametrize("args,code", [
    (dict(n=0), EINVAL), (dict(n=(1 << 20) + 1), EINVAL), (dict(k=0), EINVAL),
    (dict(k=65), EINVAL), (dict(n=10, k=11), EINVAL), (dict(temperature=-1.0), EINVAL),
    (dict(temperature=float("nan")), EINVAL), (dict(temperature=float("inf")), EINVAL),
    (dict(ws_bytes=SAMPLE_NEED - 1), EINVAL),
    (dict(logits=0), ENULL), (dict(state=0), ENULL), (dict(ws=0), ENULL), (dict(token=0), ENULL),
    (dict(ids=0), ENULL), (dict(vals=0), ENULL),
    (dict(logits=FAKE + 2), EALIGN), (dict(state=FAKE + 1), EALIGN), (dict(ws=FAKE + 2), EALIGN),
    (dict(token=FAKE + 3), EALIGN), (dict(ids=FAKE + 2), EALIGN), (dict(vals=FAKE + 1), EALIGN),
])
def test_logits_sample_rejects(args, code):
    a = dict(logits=FAKE, n=246272, k=64, temperature=0.7, state=FAKE, ws=FAKE,
             ws_bytes=SAMPLE_NEED, token=FAKE, ids=FAKE, vals=FAKE)
    a.update(args)
    rc = bqd.lib().logits_sample(a["logits"], a["n"], a["k"], a["temperature"], a["state"],
                                 a["ws"], a["ws_bytes"], a["token"], a["ids"], a["vals"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(n=0), EINVAL), (dict(n=(1 << 20) + 1), EINVAL), (dict(k=0), EINVAL),
    (dict(k=65), EINVAL), (dict(n=10, k=11), EINVAL), (dict(temperature=-1.0), EINVAL),
    (dict(temperature=float("nan")), EINVAL),
    (dict(logits=0), ENULL), (dict(state=0), ENULL), (dict(token=0), ENULL),
    (dict(ids=0), ENULL), (dict(vals=0), ENULL),
    (dict(logits=FAKE + 2), EALIGN), (dict(token=FAKE + 3), EALIGN), (dict(vals=FAKE + 1), EALIGN),
    (dict(vals=(1 << 32) + 400), EINVAL),   # the values written over the logits
    (dict(token=(3 << 32) + 8), EINVAL),    # the token inside the ids
])
def test_logits_sample_noalloc_rejects(args, code):
    a = dict(logits=1 << 32, n=246272, k=64, temperature=0.7, state=2 << 32, token=4 << 32,
             ids=3 << 32, vals=5 << 32)
    a.update(args)
    rc = bqd.lib().logits_sample_noalloc(a["logits"], a["n"], a["k"], a["temperature"],
                                         a["state"], a["token"], a["ids"], a["vals"], None)
    assert rc == code


def test_logits_sample_workspace_bytes():
    L = bqd.lib()
    assert L.logits_sample_workspace_bytes(246272, 64) == SAMPLE_NEED
    assert L.logits_sample_workspace_bytes(1, 1) == 8
    assert L.logits_sample_workspace_bytes(4097, 3) == 5 * 3 * 8  # blocks of 1024
    assert L.logits_sample_workspace_bytes(256 * 1024, 2) == 256 * 2 * 8
    assert L.logits_sample_workspace_bytes(256 * 1024 + 1, 2) == 129 * 2 * 8  # of 2048
    assert L.logits_sample_workspace_bytes(512 * 1024 + 1, 2) == 129 * 2 * 8  # of 4096
    assert L.logits_sample_workspace_bytes(1 << 20, 64) == 256 * 64 * 8
    for n, k in ((0, 1), (10, 11), (100, 0), (100, 65), ((1 << 20) + 1, 1)):
        assert L.logits_sample_workspace_bytes(n, k) == EINVAL


def test_binding_refuses_host_tensors():
    with pytest.raises(TypeError):
        bqd.f8_matvec(torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(1, 1, dtype=torch.uint8),
                      torch.zeros(16))


# Disjoint fake device buffers, 4 GiB apart; an overlap is made by pointing an
# output into one of them.  Every call below must fail validation (EINVAL)
# before anything is enqueued.
A, B, C_, D, E, F, G_ = ((k + 1) << 32 for k in range(7))


def test_f8_argmax_argument_rules():
    """f8_matvec_argmax: f8_matvec's rules, at least one row, a workspace of
    the stated size and tokens present, aligned and apart from every other
    buffer."""
    L = bqd.lib()
    need = L.f8_matvec_argmax_workspace_bytes(1)
    assert need == 8192 * 8 and L.f8_matvec_argmax_workspace_bytes(3) == 3 * need
    assert L.f8_matvec_argmax_workspace_bytes(-1) == EINVAL
    W, S, X, Y, K, T = FAKE, FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24), \
        FAKE + (4 << 24), FAKE + (5 << 24)
    call = lambda R=512, ws=K, wsb=need, tok=T, y=Y, batch=1: L.f8_matvec_argmax(
        W, R, 4096, S, 4, 32, X, y, batch, ws, wsb, tok, None)
    assert call(R=0) == EINVAL          # no row to take
    assert call(wsb=need - 1) == EINVAL  # workspace too small
    assert call(ws=None) == ENULL
    assert call(tok=None) == ENULL
    assert call(ws=K + 4) == EALIGN     # slots are 8 bytes
    assert call(tok=T + 2) == EALIGN
    assert call(ws=Y + 8) == EINVAL     # workspace over y
    assert call(tok=K + 8) == EINVAL    # token over the workspace
    assert call(tok=X) == EINVAL        # token over x
    assert call(batch=0) == OK          # nothing to do
    assert call(batch=-1) == EINVAL


def test_f8_sample_argument_rules():
    """f8_matvec_sample: f8_matvec's rules, 1 <= R <= 2^20, 1 <= k <= min(64,
    R), a finite temperature >= 0, the argmax workspace, and every output
    (y, workspace, states, tokens, ids, values) present, aligned and apart."""
    L = bqd.lib()
    need = L.f8_matvec_argmax_workspace_bytes(1)
    W, S, X, Y, K, ST, T, I, V = (FAKE + (j << 24) for j in range(9))
    def call(R=512, k=64, temp=0.8, ws=K, wsb=need, st=ST, tok=T, ids=I, vals=V, y=Y, batch=1,
             C=4096):
        return L.f8_matvec_sample(W, R, C, S, 4, 32, X, y, batch, k, temp, st, ws, wsb, tok, ids,
                                  vals, None)
    assert call(R=0, k=1) == EINVAL            # no row to take
    assert call(R=(1 << 20) + 1) == EINVAL     # past the sampler's range
    assert call(k=0) == EINVAL
    assert call(k=65) == EINVAL
    assert call(R=10, k=11) == EINVAL          # k > R
    assert call(temp=-1.0) == EINVAL
    assert call(temp=float("nan")) == EINVAL
    assert call(temp=float("inf")) == EINVAL
    assert call(wsb=need - 1) == EINVAL        # workspace too small
    for kw in ("ws", "st", "tok", "ids", "vals"):
        assert call(**{kw: None}) == ENULL, kw
    assert call(ws=K + 4) == EALIGN            # slots are 8 bytes
    for kw, base in (("st", ST), ("tok", T), ("ids", I), ("vals", V)):
        assert call(**{kw: base + 2}) == EALIGN, kw
    assert call(ws=Y + 8) == EINVAL            # workspace over y
    assert call(st=K + 8) == EINVAL            # state over the workspace
    assert call(tok=ST) == EINVAL              # token on the state
    assert call(ids=T) == EINVAL               # ids over the token
    assert call(vals=I + 64 * 4 - 4) == EINVAL  # values over the last id
    assert call(ids=X + 16) == EINVAL          # ids over x
    assert call(st=W + 100) == EINVAL          # state over the weights
    assert call(batch=2, tok=ST + 4) == EINVAL  # two tokens over two states
    assert call(batch=2) == EINVAL             # a workspace for one vector only
    assert call(batch=0) == OK                 # nothing to do
    assert call(batch=-1) == EINVAL


def test_f8_i8_kv_outputs_overlapping_inputs_are_refused():
    L = bqd.lib()
    f8 = lambda w=A, s=B, x=C_, y=D: L.f8_matvec(w, 512, 4096, s, 4, 32, x, y, 1, None)
    assert f8(y=C_ + 4096) == EINVAL         # y inside x
    assert f8(y=C_ - 64) == EINVAL           # y runs into x
    assert f8(y=A + 1024) == EINVAL          # y inside the weights
    assert f8(y=B) == EINVAL                 # y on the scales
    i8 = lambda w=A, s=B, x=C_, y=D: L.i8_matvec(w, 512, 4096, s, 16, x, y, 1, None)
    assert i8(y=C_ + 16) == EINVAL
    assert i8(y=A + 512 * 4096 - 4) == EINVAL  # the last weight bytes
    assert i8(y=B + 100) == EINVAL
    kd = lambda k=A, s=B, x=C_, y=D: L.kv_int8_dot(k, s, 64, 128, x, y, 1, None)
    assert kd(y=C_ + 4) == EINVAL
    assert kd(y=B) == EINVAL
    assert kd(y=A + 64 * 128 - 4) == EINVAL
    kq = lambda v=A, q=B, s=C_: L.kv_quantize_int8(v, 64, 128, q, s, None)
    assert kq(q=A + 128) == EINVAL           # codes into the vectors
    assert kq(s=A) == EINVAL                 # scales onto the vectors
    assert kq(s=B + 64 * 128 - 4) == EINVAL  # scales onto the codes


def test_cq_outputs_overlapping_inputs_are_refused():
    L = bqd.lib()
    m = cq(packed=A, norms=B, codebook=C_)
    mv = lambda p=D, y=E, mm=m: L.cq_matvec(ctypes.byref(mm), p, y, 1, 0, 256, None)
    assert mv(y=D + 512) == EINVAL           # y inside prepared
    assert mv(y=A + 64) == EINVAL            # y inside the packed rows
    assert mv(y=B + 2044) == EINVAL          # y over the last norms
    assert mv(y=C_ + 12) == EINVAL           # y on the codebook
    pm = lambda x=F, p=D, y=E: L.cq_prepare_matvec(ctypes.byref(m), x, p, y, 1, 0, 256, None)
    assert pm(p=A) == EINVAL                 # prepared written over the packed rows
    assert pm(p=B + 100) == EINVAL
    assert pm(y=D + 8) == EINVAL             # y inside prepared
    g = lambda ids=F, out=G_: L.cq_gather_rows(ctypes.byref(m), ids, 4, out, None)
    assert g(out=F + 12) == EINVAL           # out over the ids
    assert g(out=A) == EINVAL
    assert g(out=C_ - 8) == EINVAL           # out runs into the codebook
    mats = (bqd._CqStruct * 2)(m, cq(packed=F, norms=G_, codebook=C_))
    multi = lambda ys: L.cq_matvec_multi(mats, 2, None, None, D, (ctypes.c_void_p * 2)(*ys), None)
    assert multi([E, E + 512]) == EINVAL     # the two outputs overlap
    assert multi([E, G_ + 40]) == EINVAL     # an output over the second matrix's norms
    assert multi([E, D + 4]) == EINVAL       # an output over prepared


def test_mlp_and_sampler_outputs_overlapping_inputs_are_refused():
    L = bqd.lib()
    mlp = lambda n=A, d1=B, d2=C_, d3=D, r=E, u=0, out=F: L.hadamard_mlp(
        n, 512, 2048, d1, d2, d3, r, u, out, 2, None)
    assert mlp(out=A + 2048) == EINVAL       # out over the second input vector
    assert mlp(out=C_ + 4 * 2047) == EINVAL  # out over the last d2 entry
    assert mlp(out=E) == EINVAL              # out over resid
    assert mlp(u=G_, out=G_ + 4) == EINVAL   # out over u
    smp = lambda logits=A, state=B, ws=C_, tok=D, ids=E, vals=F: L.logits_sample(
        logits, 246272, 64, 0.7, state, ws, SAMPLE_NEED, tok, ids, vals, None)
    assert smp(ws=A + 4096) == EINVAL        # workspace over the logits
    assert smp(tok=E + 8) == EINVAL          # token inside the ids
    assert smp(vals=C_ + SAMPLE_NEED - 4) == EINVAL  # values over the workspace's end
    assert smp(state=A + 4 * 246271) == EINVAL  # state on the last logit

"""CPU oracle for the quantized decode matvec — TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``oracle.c`` (see ``oracle.h`` for the sources each
function follows).  Only the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product library never does.

All arguments are host numpy arrays.  Batched activations are looped here, one
vector at a time, exactly as independent single-vector calls.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Cq(ctypes.Structure):
    _fields_ = [("output", ctypes.c_int64), ("input", ctypes.c_int64),
                ("input_padded", ctypes.c_int64), ("group", ctypes.c_int64),
                ("bits", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                ("packed", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("codebook", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _load(LIB_PATH)
    return _lib


def use_library(path: str = None):
    """Point the wrapper at another build of oracle.c (None: the default one).

    The test suite uses this to run the pins against deliberately broken
    copies of the oracle and confirm that each planted mistake is caught."""
    global _lib
    _lib = None if path is None else _load(path)


def _load(path: str):
    L = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    CQ = ctypes.POINTER(_Cq)
    L.oracle_f16.restype = ctypes.c_float
    L.oracle_f16.argtypes = [ctypes.c_uint16]
    L.oracle_fwht.restype = None
    L.oracle_fwht.argtypes = [P, I64]
    L.oracle_cq_index.restype = ctypes.c_uint32
    L.oracle_cq_index.argtypes = [CQ, I64, I64]
    L.oracle_cq_unpack_row.argtypes = [CQ, I64, P]
    L.oracle_cq_prepare.argtypes = [CQ, P, P]
    L.oracle_cq_matvec.argtypes = [CQ, P, I64, I64, P, P]
    L.oracle_cq_dequantize_row.argtypes = [CQ, I64, P]
    L.oracle_cq_gather.argtypes = [CQ, P, I64, P, P]
    L.oracle_cq_dense_matvec.argtypes = [CQ, P, I64, I64, P]
    L.oracle_e4m3.restype = ctypes.c_float
    L.oracle_e4m3.argtypes = [ctypes.c_uint8]
    L.oracle_e8m0.restype = ctypes.c_float
    L.oracle_e8m0.argtypes = [ctypes.c_uint8]
    L.oracle_f8_matvec.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, P]
    L.oracle_xorshift32.restype = ctypes.c_uint32
    L.oracle_xorshift32.argtypes = [ctypes.c_uint32]
    L.oracle_topk.restype = ctypes.c_int
    L.oracle_topk.argtypes = [P, I64, I64, P, P]
    L.oracle_sample_u.restype = ctypes.c_int32
    L.oracle_sample_u.argtypes = [P, P, I64, ctypes.c_double, ctypes.c_double]
    L.oracle_sample.restype = ctypes.c_int32
    L.oracle_sample.argtypes = [P, P, I64, ctypes.c_double, ctypes.POINTER(ctypes.c_uint32)]
    L.oracle_i8_matvec.argtypes = [P, I64, I64, P, I64, P, I64, I64, P, P]
    L.oracle_store_int8.argtypes = [P, I64, P, P]
    L.oracle_int8_dot.argtypes = [P, P, I64, I64, P, I64, I64, P, P]
    L.oracle_hadamard_mlp.argtypes = [P, I64, I64, P, P, P, P, P, P, P]
    for name in ("oracle_cq_unpack_row", "oracle_cq_prepare", "oracle_cq_matvec",
                 "oracle_cq_dequantize_row", "oracle_cq_gather",
                 "oracle_cq_dense_matvec", "oracle_f8_matvec", "oracle_i8_matvec",
                 "oracle_store_int8", "oracle_int8_dot", "oracle_hadamard_mlp"):
        getattr(L, name).restype = ctypes.c_int
    return L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class CqMatrix:
    """Host-side CQ matrix: shape fields plus the packed, norm and codebook arrays."""

    def __init__(self, output, input, input_padded, group, bits, row_bytes,
                 packed, norms, codebook):
        self.packed = np.ascontiguousarray(packed, dtype=np.uint8)
        self.norms = np.ascontiguousarray(norms).view(np.uint16)
        self.codebook = np.ascontiguousarray(codebook, dtype=np.float32)
        self.output, self.input, self.input_padded = int(output), int(input), int(input_padded)
        self.group, self.bits, self.row_bytes = int(group), int(bits), int(row_bytes)
        self._s = _Cq(self.output, self.input, self.input_padded, self.group, self.bits,
                      self.row_bytes, self.packed.ctypes.data, self.norms.ctypes.data,
                      self.codebook.ctypes.data)

    @classmethod
    def from_case(cls, case):
        s = case.shape
        return cls(s.output, s.input, s.input_padded, s.group, s.bits, s.stride,
                   case.packed, case.norms, case.codebook)

    @property
    def ref(self):
        return ctypes.byref(self._s)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def f16(h: int) -> float:
    return lib().oracle_f16(int(h) & 0xFFFF)


def f16_array(codes: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_f16(int(c)) for c in np.asarray(codes).ravel()],
                    dtype=np.float32).reshape(np.shape(codes))


def fwht(x: np.ndarray) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True)
    lib().oracle_fwht(_ptr(y), y.size)
    return y


def cq_index(m: CqMatrix, row: int, col: int) -> int:
    return lib().oracle_cq_index(m.ref, row, col)


def cq_unpack_row(m: CqMatrix, row: int) -> np.ndarray:
    out = np.zeros(m.input_padded, dtype=np.uint8)
    _check(lib().oracle_cq_unpack_row(m.ref, row, _ptr(out)), "cq_unpack_row")
    return out


def cq_prepare(m: CqMatrix, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    xb = x.reshape(-1, m.input) if m.input else x.reshape(-1, 0)
    out = np.zeros((xb.shape[0], m.input_padded), dtype=np.float32)
    for b in range(xb.shape[0]):
        xv = np.ascontiguousarray(xb[b])
        ov = out[b]
        _check(lib().oracle_cq_prepare(m.ref, _ptr(xv), ov.ctypes.data_as(ctypes.c_void_p)),
               "cq_prepare")
    return out.reshape(x.shape[:-1] + (m.input_padded,)) if x.ndim > 1 else out[0]


def cq_matvec(m: CqMatrix, p: np.ndarray, row_begin: int = 0, row_count=None):
    """Returns (y, mag), each float64 [batch][row_count] (or 1-D for a 1-D p)."""
    if row_count is None:
        row_count = m.output - row_begin
    p = np.ascontiguousarray(p, dtype=np.float32)
    pb = p.reshape(-1, m.input_padded)
    y = np.zeros((pb.shape[0], row_count), dtype=np.float64)
    mag = np.zeros_like(y)
    for b in range(pb.shape[0]):
        pv = np.ascontiguousarray(pb[b])
        _check(lib().oracle_cq_matvec(m.ref, _ptr(pv), row_begin, row_count,
                                      y[b].ctypes.data_as(ctypes.c_void_p),
                                      mag[b].ctypes.data_as(ctypes.c_void_p)), "cq_matvec")
    if p.ndim == 1:
        return y[0], mag[0]
    return y, mag


def cq_dequantize_row(m: CqMatrix, row: int) -> np.ndarray:
    out = np.zeros(m.input, dtype=np.float32)
    _check(lib().oracle_cq_dequantize_row(m.ref, row, _ptr(out)), "cq_dequantize_row")
    return out


def cq_gather(m: CqMatrix, ids: np.ndarray):
    """Returns (out float32 [n][input], gmag float64 [n][input])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = np.zeros((ids.size, m.input), dtype=np.float32)
    gmag = np.zeros((ids.size, m.input), dtype=np.float64)
    _check(lib().oracle_cq_gather(m.ref, _ptr(ids), ids.size, _ptr(out), _ptr(gmag)), "cq_gather")
    return out, gmag


def cq_dense_matvec(m: CqMatrix, x: np.ndarray, row_begin: int = 0, row_count=None):
    if row_count is None:
        row_count = m.output - row_begin
    x = np.ascontiguousarray(x, dtype=np.float32)
    xb = x.reshape(-1, m.input)
    y = np.zeros((xb.shape[0], row_count), dtype=np.float64)
    for b in range(xb.shape[0]):
        xv = np.ascontiguousarray(xb[b])
        _check(lib().oracle_cq_dense_matvec(m.ref, _ptr(xv), row_begin, row_count,
                                            y[b].ctypes.data_as(ctypes.c_void_p)),
               "cq_dense_matvec")
    return y[0] if x.ndim == 1 else y


def e4m3(code: int) -> float:
    return lib().oracle_e4m3(int(code) & 0xFF)


def e4m3_all() -> np.ndarray:
    """Decoded value of every E4M3 code 0..255, as float32."""
    L = lib()
    return np.array([L.oracle_e4m3(c) for c in range(256)], dtype=np.float32)


def e8m0_all() -> np.ndarray:
    L = lib()
    return np.array([L.oracle_e8m0(c) for c in range(256)], dtype=np.float32)


def f8_matvec(w, R, C, s, SR, SC, x, row_begin: int = 0, row_count=None):
    """Returns (y, mag), float64 [batch][row_count] (or 1-D for a 1-D x)."""
    if row_count is None:
        row_count = R - row_begin
    w = np.ascontiguousarray(w, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    xb = x.reshape(-1, C)
    y = np.zeros((xb.shape[0], row_count), dtype=np.float64)
    mag = np.zeros_like(y)
    for b in range(xb.shape[0]):
        xv = np.ascontiguousarray(xb[b])
        _check(lib().oracle_f8_matvec(_ptr(w), R, C, _ptr(s), SR, SC, _ptr(xv), row_begin,
                                      row_count, y[b].ctypes.data_as(ctypes.c_void_p),
                                      mag[b].ctypes.data_as(ctypes.c_void_p)), "f8_matvec")
    if x.ndim == 1:
        return y[0], mag[0]
    return y, mag


def xorshift32(s: int) -> int:
    return lib().oracle_xorshift32(s)


def topk(logits: np.ndarray, k: int):
    """(ids int32 [k], vals float32 [k]) of the k best logits (O12)."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.zeros(k, np.int32)
    vals = np.zeros(k, np.float32)
    _check(lib().oracle_topk(_ptr(x), x.size, k, _ptr(ids), _ptr(vals)), "topk")
    return ids, vals


def sample_u(vals: np.ndarray, ids: np.ndarray, temperature: float, u: float) -> int:
    v = np.ascontiguousarray(vals, dtype=np.float32)
    i = np.ascontiguousarray(ids, dtype=np.int32)
    return lib().oracle_sample_u(_ptr(v), _ptr(i), v.size, temperature, u)


def sample(vals: np.ndarray, ids: np.ndarray, temperature: float, state: int):
    """(token, next state) (O13 with O11)."""
    v = np.ascontiguousarray(vals, dtype=np.float32)
    i = np.ascontiguousarray(ids, dtype=np.int32)
    s = ctypes.c_uint32(state)
    tok = lib().oracle_sample(_ptr(v), _ptr(i), v.size, temperature, ctypes.byref(s))
    return tok, s.value


def i8_matvec(w, R, C, s, G, x, row_begin: int = 0, row_count=None):
    """O14.  w int8 [R][C], s uint8 [R][ceil(C/G)]; returns (y, mag) float64
    [batch][row_count] (or 1-D for a 1-D x)."""
    if row_count is None:
        row_count = R - row_begin
    w = np.ascontiguousarray(w, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    xb = x.reshape(-1, C)
    y = np.zeros((xb.shape[0], row_count), dtype=np.float64)
    mag = np.zeros_like(y)
    for b in range(xb.shape[0]):
        xv = np.ascontiguousarray(xb[b])
        _check(lib().oracle_i8_matvec(_ptr(w), R, C, _ptr(s), G, _ptr(xv), row_begin, row_count,
                                      y[b].ctypes.data_as(ctypes.c_void_p),
                                      mag[b].ctypes.data_as(ctypes.c_void_p)), "i8_matvec")
    if x.ndim == 1:
        return y[0], mag[0]
    return y, mag


def store_int8(v: np.ndarray):
    """O15 on each row of v ([n] or [rows][n]): (q int8, scale float32)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    vb = v.reshape(-1, v.shape[-1]) if v.ndim else v.reshape(1, 1)
    q = np.zeros(vb.shape, dtype=np.int8)
    sc = np.zeros(vb.shape[0], dtype=np.float32)
    for i in range(vb.shape[0]):
        row = np.ascontiguousarray(vb[i])
        qi = q[i]
        si = sc[i:i + 1]
        _check(lib().oracle_store_int8(_ptr(row), row.size, qi.ctypes.data_as(ctypes.c_void_p),
                                       si.ctypes.data_as(ctypes.c_void_p)), "store_int8")
    if v.ndim == 1:
        return q[0], sc[0]
    return q.reshape(v.shape), sc.reshape(v.shape[:-1])


def int8_dot(K, scales, x, row_begin: int = 0, row_count=None):
    """O16.  K int8 [R][d], scales float32 [R], x float32 [d]: (y, mag) float64."""
    K = np.ascontiguousarray(K, dtype=np.int8)
    R, d = K.shape
    if row_count is None:
        row_count = R - row_begin
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.zeros(row_count, dtype=np.float64)
    mag = np.zeros_like(y)
    _check(lib().oracle_int8_dot(_ptr(K), _ptr(scales), R, d, _ptr(x), row_begin, row_count,
                                 _ptr(y), _ptr(mag)), "int8_dot")
    return y, mag


def hadamard_mlp(n, H, d1, d2, d3, resid, u=None):
    """O17.  n, resid, u float32 [hidden]; d1, d2, d3 float32 [H].
    Returns (out float32 [hidden], mag float64 [hidden])."""
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    n, d1, d2, d3, resid = f(n), f(d1), f(d2), f(d3), f(resid)
    hidden = n.size
    out = np.zeros(hidden, dtype=np.float32)
    mag = np.zeros(hidden, dtype=np.float64)
    uu = None if u is None else f(u)
    _check(lib().oracle_hadamard_mlp(_ptr(n), hidden, H, _ptr(d1), _ptr(d2), _ptr(d3), _ptr(resid),
                                     None if uu is None else _ptr(uu), _ptr(out), _ptr(mag)),
           "hadamard_mlp")
    return out, mag

"""Quantized decode matvec on MI355X (gfx950): Python binding of libbqd.so.

Argument marshalling only: every function checks that the torch tensors it is
given live on the GPU with the dtype and layout the C ABI (``include/bqd.h``)
documents, allocates the output tensor when none is passed, and calls the
entry point of the same name on the current torch stream.  All computation
runs in the HIP kernels of ``libbqd.so``; if the library is missing the calls
raise instead of falling back to anything else.

Operations ("Inference engine, part 2: kernels and token step" §1–§3 and
"Row gather"; "attention + tokenizer + sampling: the path to real text",
Step 1):

* ``cq_prepare(m, x)``        zero-pad, per-group FWHT, times 1/sqrt(group)
* ``cq_matvec(m, prepared)``  packed-row codebook dot with fp16 group norms
* ``cq_prepare_matvec(m, x)`` both in one call (the page's cqMatvec(matrix, x))
* ``cq_matvec_multi(ms, prepared)`` / ``cq_prepare_matvec_multi(ms, x)``
  several matrices (row ranges) on one activation, §6
* ``cq_gather_rows(m, rows)`` dense rows: decode x norm, normalized FWHT
* ``f8_matvec(w, scale, x)``  E4M3 weights with E8M0 block scales
* ``i8_matvec(w, scale, x, G)`` int8 weights with E8M0 scales per G columns
  ("attention + tokenizer + sampling", Step 4)
* ``kv_quantize_int8(v)``     storeInt8 per vector ("Inference engine, part 2" §7)
* ``kv_int8_dot(K, scales, x)`` the scaled key dot against an int8 cache
* ``hadamard_mlp(n, H, d1, d2, d3, resid, u)`` the Hadamard MLP (§8)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["BqdError", "CqMatrix", "cq_prepare", "cq_matvec", "cq_prepare_matvec",
           "cq_matvec_multi", "cq_prepare_matvec_multi",
           "cq_gather_rows", "f8_matvec", "i8_matvec", "kv_quantize_int8", "kv_int8_dot", "hadamard_mlp",
           "logits_sample", "logits_sample_workspace_bytes", "logits_sample_noalloc",
           "dbg_cq_unpack", "dbg_f16_decode", "dbg_f8_decode", "dbg_e8m0_decode", "lib",
           "LIB_PATH", "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbqd.so")

# Every symbol include/bqd.h declares.
EXPORTS = ("cq_prepare", "cq_matvec", "cq_prepare_matvec", "cq_matvec_multi",
           "cq_prepare_matvec_multi", "cq_gather_rows", "f8_matvec", "f8_matvec_argmax",
           "f8_matvec_argmax_workspace_bytes", "f8_matvec_sample",
           "i8_matvec", "kv_quantize_int8", "kv_int8_dot", "hadamard_mlp", "logits_sample",
           "logits_sample_workspace_bytes", "logits_sample_noalloc", "bqd_dbg_cq_unpack", "bqd_dbg_f16_decode",
           "bqd_dbg_f8_decode", "bqd_dbg_e8m0_decode", "bqd_dbg_read_stream",
           "bqd_status_string")

READ_STREAM_WORDS = 2048  # BQD_READ_STREAM_WORDS

_lib = None


class BqdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().bqd_status_string(status).decode()
        super().__init__(f"{fn}: {msg} (status {status})")


class _CqStruct(ctypes.Structure):
    _fields_ = [("output", ctypes.c_int64), ("input", ctypes.c_int64),
                ("input_padded", ctypes.c_int64), ("group", ctypes.c_int64),
                ("bits", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                ("packed", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("codebook", ctypes.c_void_p)]


def lib():
    """The loaded libbqd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run bit_quantized_decode_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        S = ctypes.POINTER(_CqStruct)
        for name, args in (
                ("cq_prepare", [S, P, P, I64, P]),
                ("cq_matvec", [S, P, P, I64, I64, I64, P]),
                ("cq_prepare_matvec", [S, P, P, P, I64, I64, I64, P]),
                ("cq_matvec_multi", [S, I64, P, P, P, P, P]),
                ("cq_prepare_matvec_multi", [S, I64, P, P, P, P, P, P]),
                ("cq_gather_rows", [S, P, I64, P, P]),
                ("f8_matvec", [P, I64, I64, P, I64, I64, P, P, I64, P]),
                ("f8_matvec_argmax", [P, I64, I64, P, I64, I64, P, P, I64, P, I64, P, P]),
                ("f8_matvec_sample", [P, I64, I64, P, I64, I64, P, P, I64, I64, ctypes.c_float,
                                      P, P, I64, P, P, P, P]),
                ("i8_matvec", [P, I64, I64, P, I64, P, P, I64, P]),
                ("kv_quantize_int8", [P, I64, I64, P, P, P]),
                ("kv_int8_dot", [P, P, I64, I64, P, P, I64, P]),
                ("hadamard_mlp", [P, I64, I64, P, P, P, P, P, P, I64, P]),
                ("bqd_dbg_cq_unpack", [S, I64, P, P]),
                ("bqd_dbg_f16_decode", [P, I64, P, P]),
                ("bqd_dbg_f8_decode", [P, I64, P, P]),
                ("bqd_dbg_e8m0_decode", [P, I64, P, P]),
                ("bqd_dbg_read_stream", [P, I64, P, P]),
                ("logits_sample", [P, I64, I64, ctypes.c_float, P, P, I64, P, P, P, P]),
                ("logits_sample_noalloc", [P, I64, I64, ctypes.c_float, P, P, P, P, P])):
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I
        L.f8_matvec_argmax_workspace_bytes.argtypes = [I64]
        L.f8_matvec_argmax_workspace_bytes.restype = I64
        L.logits_sample_workspace_bytes.argtypes = [I64, I64]
        L.logits_sample_workspace_bytes.restype = I64
        L.bqd_status_string.argtypes = [I]
        L.bqd_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _call(name: str, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise BqdError(name, rc)


def _stream(t: torch.Tensor, stream):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class CqMatrix:
    """A codebook-quantized matrix resident in GPU memory.

    packed: uint8 [output][row_bytes]; norms: int16 or uint16 holding fp16 bit
    patterns, [output][input_padded // group]; codebook: float32 [2**bits].
    """

    def __init__(self, packed, norms, codebook, *, output, input, input_padded, group, bits,
                 row_bytes=None):
        self.packed = _dev(packed, torch.uint8, "packed")
        self.norms = _dev(norms, (torch.int16, torch.uint16), "norms")
        self.codebook = _dev(codebook, torch.float32, "codebook")
        self.output, self.input, self.input_padded = int(output), int(input), int(input_padded)
        self.group, self.bits = int(group), int(bits)
        self.row_bytes = int(row_bytes if row_bytes is not None else packed.shape[-1])
        # the buffers must hold what the shape fields describe (the C ABI sees
        # only their addresses); the shape rules themselves are checked there
        if self.output > 0 and self.row_bytes > 0 and self.packed.numel() < self.output * self.row_bytes:
            raise ValueError("packed holds fewer than output * row_bytes bytes")
        if self.group > 0 and self.norms.numel() < self.output * (self.input_padded // self.group):
            raise ValueError("norms holds fewer than output * (input_padded / group) entries")
        if 0 <= self.bits <= 16 and self.codebook.numel() < (1 << self.bits):
            raise ValueError("codebook holds fewer than 2**bits entries")
        self._s = _CqStruct(self.output, self.input, self.input_padded, self.group, self.bits,
                            self.row_bytes, self.packed.data_ptr(), self.norms.data_ptr(),
                            self.codebook.data_ptr())

    @classmethod
    def from_arrays(cls, packed, norms, codebook, *, output, input, input_padded, group, bits,
                    row_bytes=None, device="cuda"):
        """Copy host (numpy) arrays to the GPU."""
        import numpy as np
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        return cls(t(packed, np.uint8), t(norms, np.int16), t(codebook, np.float32),
                   output=output, input=input, input_padded=input_padded, group=group,
                   bits=bits, row_bytes=row_bytes)

    @property
    def ref(self):
        return ctypes.byref(self._s)


def cq_prepare(m: CqMatrix, x: torch.Tensor, out: torch.Tensor = None, stream=None):
    """x float32 [batch][input] (or [input]) -> prepared float32 [batch][input_padded]."""
    x = _dev(x, torch.float32, "x")
    if x.shape[-1] != m.input:
        raise ValueError("x must have m.input columns")
    batch = x.numel() // m.input if m.input else (x.shape[0] if x.dim() > 1 else 1)
    shape = x.shape[:-1] + (m.input_padded,)
    out = torch.empty(shape, dtype=torch.float32, device=x.device) if out is None else \
        _dev(out, torch.float32, "out")
    if out.numel() != batch * m.input_padded:
        raise ValueError("out has the wrong size")
    _call("cq_prepare", m.ref, _ptr(x), _ptr(out), batch, _stream(x, stream))
    return out


def cq_matvec(m: CqMatrix, prepared: torch.Tensor, out: torch.Tensor = None, row_begin: int = 0,
              row_count: int = None, stream=None):
    """prepared float32 [batch][input_padded] -> y float32 [batch][row_count]."""
    prepared = _dev(prepared, torch.float32, "prepared")
    if prepared.shape[-1] != m.input_padded:
        raise ValueError("prepared must have m.input_padded columns")
    batch = prepared.numel() // m.input_padded
    row_count = m.output - row_begin if row_count is None else int(row_count)
    shape = prepared.shape[:-1] + (row_count,)
    out = torch.empty(shape, dtype=torch.float32, device=prepared.device) if out is None else \
        _dev(out, torch.float32, "out")
    if out.numel() != batch * row_count:
        raise ValueError("out has the wrong size")
    _call("cq_matvec", m.ref, _ptr(prepared), _ptr(out), batch, int(row_begin), row_count,
          _stream(prepared, stream))
    return out


def cq_prepare_matvec(m: CqMatrix, x: torch.Tensor, prepared: torch.Tensor = None,
                      out: torch.Tensor = None, row_begin: int = 0, row_count: int = None,
                      stream=None):
    """x float32 [batch][input] -> (prepared [batch][input_padded], y [batch][row_count]),
    the results of cq_prepare followed by cq_matvec."""
    x = _dev(x, torch.float32, "x")
    if x.shape[-1] != m.input:
        raise ValueError("x must have m.input columns")
    batch = x.numel() // m.input if m.input else (x.shape[0] if x.dim() > 1 else 1)
    row_count = m.output - row_begin if row_count is None else int(row_count)
    prepared = torch.empty(x.shape[:-1] + (m.input_padded,), dtype=torch.float32,
                           device=x.device) if prepared is None else \
        _dev(prepared, torch.float32, "prepared")
    out = torch.empty(x.shape[:-1] + (row_count,), dtype=torch.float32, device=x.device) \
        if out is None else _dev(out, torch.float32, "out")
    if prepared.numel() != batch * m.input_padded or out.numel() != batch * row_count:
        raise ValueError("prepared or out has the wrong size")
    _call("cq_prepare_matvec", m.ref, _ptr(x), _ptr(prepared), _ptr(out), batch, int(row_begin),
          row_count, _stream(x, stream))
    return prepared, out


def _multi_args(ms, ranges, outs, device):
    n = len(ms)
    ranges = [(0, m.output) for m in ms] if ranges is None else [(int(a), int(b)) for a, b in ranges]
    if len(ranges) != n:
        raise ValueError("one row range per matrix")
    outs = [torch.empty(rc, dtype=torch.float32, device=device) for _, rc in ranges] \
        if outs is None else [_dev(o, torch.float32, "out") for o in outs]
    for o, (_, rc) in zip(outs, ranges):
        if o.numel() != rc:
            raise ValueError("an output has the wrong size")
    descs = (_CqStruct * n)(*[m._s for m in ms])
    rb = (ctypes.c_int64 * n)(*[a for a, _ in ranges])
    rcs = (ctypes.c_int64 * n)(*[b for _, b in ranges])
    ys = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    return n, descs, rb, rcs, ys, outs


def cq_matvec_multi(ms, prepared: torch.Tensor, ranges=None, outs=None, stream=None):
    """Several CqMatrix objects (row ranges [(row_begin, row_count)]) on one
    prepared vector float32 [input_padded] -> list of float32 [row_count]."""
    prepared = _dev(prepared, torch.float32, "prepared")
    if not ms or prepared.numel() != ms[0].input_padded:
        raise ValueError("prepared must have the matrices' input_padded entries")
    n, descs, rb, rcs, ys, outs = _multi_args(ms, ranges, outs, prepared.device)
    _call("cq_matvec_multi", descs, n, rb, rcs, _ptr(prepared), ys, _stream(prepared, stream))
    return outs


def cq_prepare_matvec_multi(ms, x: torch.Tensor, prepared: torch.Tensor = None, ranges=None,
                            outs=None, stream=None):
    """cq_matvec_multi on the raw activation x float32 [input]; returns
    (prepared float32 [input_padded], list of outputs)."""
    x = _dev(x, torch.float32, "x")
    if not ms or x.numel() != ms[0].input:
        raise ValueError("x must have the matrices' input entries")
    prepared = torch.empty(ms[0].input_padded, dtype=torch.float32, device=x.device) \
        if prepared is None else _dev(prepared, torch.float32, "prepared")
    if prepared.numel() != ms[0].input_padded:
        raise ValueError("prepared must have the matrices' input_padded entries")
    n, descs, rb, rcs, ys, outs = _multi_args(ms, ranges, outs, x.device)
    _call("cq_prepare_matvec_multi", descs, n, rb, rcs, _ptr(x), _ptr(prepared), ys,
          _stream(x, stream))
    return prepared, outs


def cq_gather_rows(m: CqMatrix, rows: torch.Tensor, out: torch.Tensor = None, stream=None):
    """rows int32 [n] -> dense rows float32 [n][input]."""
    rows = _dev(rows, torch.int32, "rows")
    n = rows.numel()
    out = torch.empty((n, m.input), dtype=torch.float32, device=rows.device) if out is None else \
        _dev(out, torch.float32, "out")
    if out.numel() != n * m.input:
        raise ValueError("out has the wrong size")
    _call("cq_gather_rows", m.ref, _ptr(rows), n, _ptr(out), _stream(rows, stream))
    return out


def f8_matvec(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor, out: torch.Tensor = None,
              stream=None):
    """w uint8 E4M3 [R][C], scale uint8 E8M0 [SR][SC], x float32 [batch][C] -> [batch][R]."""
    w = _dev(w, torch.uint8, "w")
    scale = _dev(scale, torch.uint8, "scale")
    x = _dev(x, torch.float32, "x")
    R, C = w.shape
    SR, SC = scale.shape
    if x.shape[-1] != C:
        raise ValueError("x must have C columns")
    batch = x.numel() // C
    shape = x.shape[:-1] + (R,)
    out = torch.empty(shape, dtype=torch.float32, device=x.device) if out is None else \
        _dev(out, torch.float32, "out")
    if out.numel() != batch * R:
        raise ValueError("out has the wrong size")
    _call("f8_matvec", _ptr(w), R, C, _ptr(scale), SR, SC, _ptr(x), _ptr(out), batch,
          _stream(x, stream))
    return out


def f8_matvec_argmax_workspace_bytes(batch: int) -> int:
    need = lib().f8_matvec_argmax_workspace_bytes(int(batch))
    if need < 0:
        raise BqdError("f8_matvec_argmax_workspace_bytes", int(need))
    return int(need)


def f8_matvec_argmax(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor,
                     workspace: torch.Tensor = None, out: torch.Tensor = None,
                     token: torch.Tensor = None, stream=None):
    """f8_matvec with the argmax of each vector's outputs fused into the pass:
    (y float32 [batch][R], token int32 [batch]).  workspace: uint8 device
    scratch of f8_matvec_argmax_workspace_bytes(batch) bytes (allocated if
    None; nothing in it needs clearing)."""
    w = _dev(w, torch.uint8, "w")
    scale = _dev(scale, torch.uint8, "scale")
    x = _dev(x, torch.float32, "x")
    R, C = w.shape
    SR, SC = scale.shape
    if x.shape[-1] != C:
        raise ValueError("x must have C columns")
    batch = x.numel() // C
    out = torch.empty(x.shape[:-1] + (R,), dtype=torch.float32, device=x.device) if out is None \
        else _dev(out, torch.float32, "out")
    need = f8_matvec_argmax_workspace_bytes(batch)
    workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if workspace is None else \
        _dev(workspace, torch.uint8, "workspace")
    token = torch.empty(batch, dtype=torch.int32, device=x.device) if token is None else \
        _dev(token, torch.int32, "token")
    if out.numel() != batch * R or token.numel() != batch:
        raise ValueError("out or token has the wrong size")
    _call("f8_matvec_argmax", _ptr(w), R, C, _ptr(scale), SR, SC, _ptr(x), _ptr(out), batch,
          _ptr(workspace), workspace.numel(), _ptr(token), _stream(x, stream))
    return out, token


def f8_matvec_sample(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor, k: int,
                     temperature: float, state: torch.Tensor, workspace: torch.Tensor = None,
                     out: torch.Tensor = None, stream=None):
    """f8_matvec with top-k / temperature sampling of each vector's outputs
    fused onto the pass.  state: int32 or uint32 [batch] on the GPU (the
    xorshift32 states), advanced in place.  Returns (y float32 [batch][R],
    token int32 [batch], topk_ids int32 [batch][k], topk_logits float32
    [batch][k]); workspace as f8_matvec_argmax's (allocated if None)."""
    w = _dev(w, torch.uint8, "w")
    scale = _dev(scale, torch.uint8, "scale")
    x = _dev(x, torch.float32, "x")
    state = _dev(state, (torch.int32, torch.uint32), "state")
    R, C = w.shape
    SR, SC = scale.shape
    if x.shape[-1] != C:
        raise ValueError("x must have C columns")
    batch = x.numel() // C
    if state.numel() != batch:
        raise ValueError("state needs one element per vector")
    out = torch.empty(x.shape[:-1] + (R,), dtype=torch.float32, device=x.device) if out is None \
        else _dev(out, torch.float32, "out")
    if out.numel() != batch * R:
        raise ValueError("out has the wrong size")
    need = f8_matvec_argmax_workspace_bytes(batch)
    workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if workspace is None else \
        _dev(workspace, torch.uint8, "workspace")
    token = torch.empty(batch, dtype=torch.int32, device=x.device)
    ids = torch.empty((batch, k), dtype=torch.int32, device=x.device)
    vals = torch.empty((batch, k), dtype=torch.float32, device=x.device)
    _call("f8_matvec_sample", _ptr(w), R, C, _ptr(scale), SR, SC, _ptr(x), _ptr(out), batch,
          int(k), float(temperature), _ptr(state), _ptr(workspace), workspace.numel(),
          _ptr(token), _ptr(ids), _ptr(vals), _stream(x, stream))
    return out, token, ids, vals


def i8_matvec(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor, G: int = 16,
              out: torch.Tensor = None, stream=None):
    """w int8 [R][C], scale uint8 E8M0 [R][ceil(C/G)], x float32 [batch][C] -> [batch][R]."""
    w = _dev(w, torch.int8, "w")
    scale = _dev(scale, torch.uint8, "scale")
    x = _dev(x, torch.float32, "x")
    R, C = w.shape
    if scale.shape != (R, (C + G - 1) // G):
        raise ValueError("scale must be [R][ceil(C/G)]")
    if x.shape[-1] != C:
        raise ValueError("x must have C columns")
    batch = x.numel() // C
    out = torch.empty(x.shape[:-1] + (R,), dtype=torch.float32, device=x.device) if out is None \
        else _dev(out, torch.float32, "out")
    if out.numel() != batch * R:
        raise ValueError("out has the wrong size")
    _call("i8_matvec", _ptr(w), R, C, _ptr(scale), int(G), _ptr(x), _ptr(out), batch,
          _stream(x, stream))
    return out


def kv_quantize_int8(v: torch.Tensor, q: torch.Tensor = None, scales: torch.Tensor = None,
                     stream=None):
    """v float32 [n][d] -> (q int8 [n][d], scales float32 [n]), storeInt8 per row."""
    v = _dev(v, torch.float32, "v")
    n, d = v.shape
    q = torch.empty((n, d), dtype=torch.int8, device=v.device) if q is None else \
        _dev(q, torch.int8, "q")
    scales = torch.empty(n, dtype=torch.float32, device=v.device) if scales is None else \
        _dev(scales, torch.float32, "scales")
    if q.numel() != n * d or scales.numel() != n:
        raise ValueError("q or scales has the wrong size")
    _call("kv_quantize_int8", _ptr(v), n, d, _ptr(q), _ptr(scales), _stream(v, stream))
    return q, scales


def kv_int8_dot(K: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, out: torch.Tensor = None,
                stream=None):
    """K int8 [R][d], scales float32 [R], x float32 [batch][d] -> [batch][R]."""
    K = _dev(K, torch.int8, "K")
    scales = _dev(scales, torch.float32, "scales")
    x = _dev(x, torch.float32, "x")
    R, d = K.shape
    if scales.numel() != R or x.shape[-1] != d:
        raise ValueError("scales must have R entries and x d columns")
    batch = x.numel() // d
    out = torch.empty(x.shape[:-1] + (R,), dtype=torch.float32, device=x.device) if out is None \
        else _dev(out, torch.float32, "out")
    if out.numel() != batch * R:
        raise ValueError("out has the wrong size")
    _call("kv_int8_dot", _ptr(K), _ptr(scales), R, d, _ptr(x), _ptr(out), batch,
          _stream(x, stream))
    return out


def hadamard_mlp(n: torch.Tensor, H: int, d1: torch.Tensor, d2: torch.Tensor, d3: torch.Tensor,
                 resid: torch.Tensor, u: torch.Tensor = None, out: torch.Tensor = None,
                 stream=None):
    """n, resid, u float32 [batch][hidden]; d1, d2, d3 float32 [H] -> out [batch][hidden]."""
    n = _dev(n, torch.float32, "n")
    d1, d2, d3 = (_dev(t, torch.float32, nm) for t, nm in ((d1, "d1"), (d2, "d2"), (d3, "d3")))
    resid = _dev(resid, torch.float32, "resid")
    hidden = n.shape[-1]
    batch = n.numel() // hidden if hidden else (n.shape[0] if n.dim() > 1 else 1)
    if resid.shape != n.shape or (u is not None and u.shape != n.shape):
        raise ValueError("resid and u must have n's shape")
    if d1.numel() != H or d2.numel() != H or d3.numel() != H:
        raise ValueError("d1, d2, d3 must have H entries")
    if u is not None:
        u = _dev(u, torch.float32, "u")
    out = torch.empty_like(n) if out is None else _dev(out, torch.float32, "out")
    if out.numel() != n.numel():
        raise ValueError("out has the wrong size")
    _call("hadamard_mlp", _ptr(n), hidden, int(H), _ptr(d1), _ptr(d2), _ptr(d3), _ptr(resid),
          None if u is None else _ptr(u), _ptr(out), batch, _stream(n, stream))
    return out


def logits_sample_workspace_bytes(n: int, k: int) -> int:
    need = lib().logits_sample_workspace_bytes(int(n), int(k))
    if need < 0:
        raise BqdError("logits_sample_workspace_bytes", int(need))
    return int(need)


def logits_sample(logits: torch.Tensor, k: int, temperature: float, state: torch.Tensor,
                  workspace: torch.Tensor = None, stream=None):
    """Top-k of float32 logits [n] and one sampled token; `state` (int32 or
    uint32 [1] on the GPU, the xorshift32 state) advances in place.
    Returns (token int32 [1], topk_ids int32 [k], topk_logits float32 [k])."""
    logits = _dev(logits, torch.float32, "logits")
    state = _dev(state, (torch.int32, torch.uint32), "state")
    if state.numel() < 1:
        raise ValueError("state needs one element")
    n = logits.numel()
    need = logits_sample_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    workspace = _dev(workspace, torch.uint8, "workspace")
    token = torch.empty(1, dtype=torch.int32, device=logits.device)
    ids = torch.empty(k, dtype=torch.int32, device=logits.device)
    vals = torch.empty(k, dtype=torch.float32, device=logits.device)
    _call("logits_sample", _ptr(logits), n, int(k), float(temperature), _ptr(state),
          _ptr(workspace), workspace.numel(), _ptr(token), _ptr(ids), _ptr(vals),
          _stream(logits, stream))
    return token, ids, vals


def logits_sample_noalloc(logits: torch.Tensor, k: int, temperature: float, state: torch.Tensor,
                          token: torch.Tensor, topk_ids: torch.Tensor, topk_logits: torch.Tensor,
                          stream=None):
    """logits_sample into caller-given outputs (token int32 [1], topk_ids
    int32 [k], topk_logits float32 [k]), with the library's static scratch as
    the workspace: the call allocates no device memory."""
    logits = _dev(logits, torch.float32, "logits")
    state = _dev(state, (torch.int32, torch.uint32), "state")
    token = _dev(token, torch.int32, "token")
    topk_ids = _dev(topk_ids, torch.int32, "topk_ids")
    topk_logits = _dev(topk_logits, torch.float32, "topk_logits")
    if state.numel() < 1:
        raise ValueError("state needs one element")
    if token.numel() < 1 or topk_ids.numel() < k or topk_logits.numel() < k:
        raise ValueError("token needs 1 element, topk_ids and topk_logits k each")
    _call("logits_sample_noalloc", _ptr(logits), logits.numel(), int(k), float(temperature),
          _ptr(state), _ptr(token), _ptr(topk_ids), _ptr(topk_logits), _stream(logits, stream))
    return token, topk_ids, topk_logits


def dbg_cq_unpack(m: CqMatrix, row: int, stream=None):
    """Codebook indices of one row (uint8 [input_padded]) via the kernels' decoder."""
    out = torch.empty(m.input_padded, dtype=torch.uint8, device=m.packed.device)
    _call("bqd_dbg_cq_unpack", m.ref, int(row), _ptr(out), _stream(out, stream))
    return out


def _decode(name, codes, dtype, stream):
    codes = _dev(codes, dtype, "codes")
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _call(name, _ptr(codes), codes.numel(), _ptr(out), _stream(codes, stream))
    return out


def dbg_f16_decode(codes, stream=None):
    return _decode("bqd_dbg_f16_decode", codes, (torch.int16, torch.uint16), stream)


def dbg_f8_decode(codes, stream=None):
    return _decode("bqd_dbg_f8_decode", codes, torch.uint8, stream)


def dbg_e8m0_decode(codes, stream=None):
    return _decode("bqd_dbg_e8m0_decode", codes, torch.uint8, stream)


def dbg_read_stream(buf, out=None, stream=None):
    """Read every byte of ``buf`` (a contiguous device tensor, 16-byte aligned,
    nbytes a multiple of 16) once; returns ``out`` (int32 [READ_STREAM_WORDS])
    whose XOR is the XOR of the buffer's 32-bit words."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf: a contiguous device tensor")
    if out is None:
        out = torch.empty(READ_STREAM_WORDS, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _call("bqd_dbg_read_stream", _ptr(buf), nbytes, _ptr(out), _stream(buf, stream))
    return out

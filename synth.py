"""Seeded synthetic inputs for the quantized decode matvec workloads.

This module only draws random arrays in the layouts the method reads.  It holds
none of the method's arithmetic (no unpacking, no transform, no decode, no dot
products), so the HIP path and the CPU oracle can both consume its output
without sharing any computation.

Layouts (all host numpy arrays, C-contiguous):

* CQ matrix ("Inference engine, part 1: loader and tokenizer", section 4
  "Retain packed matrices"): ``packed`` uint8 ``[output][row_bytes]`` (a
  little-endian bit stream of ``bits``-wide codebook indices per row, one index
  per padded input column), ``norms`` uint16 fp16 bit patterns
  ``[output][input_padded // group]``, ``codebook`` float32 ``[2**bits]``.
* Activations: float32 ``[batch][input]``.
* FP8 head ("attention + tokenizer + sampling: the path to real text",
  "Step 1 done: F8 kernel"): ``w`` uint8 E4M3 codes ``[R][C]``, ``scale``
  uint8 E8M0 exponents ``[SR][SC]``, activation float32 ``[batch][C]``.
* I8 matvec (same thread, "Step 4 done"): ``w`` int8 ``[R][C]``, ``scale``
  uint8 E8M0 exponents ``[R][ceil(C / G)]``, activation float32 ``[batch][C]``.
* Int8 key cache ("Inference engine, part 2", section 7): key vectors float32
  ``[n][d]`` (to be quantized per vector), queries float32 ``[batch][d]``.
* Hadamard MLP (same page, section 8): normalized input, residual and u
  float32 ``[batch][hidden]``, diagonal scales d1, d2, d3 float32 ``[H]``.

Recipe (per case, a fresh ``numpy.random.default_rng(seed)``; draw order is
fixed): 1. packed bytes or F8 weight bytes, uniform over all 256 byte values;
2. norms (uniform in [0.5, 2] rounded to fp16) or scale exponents (uniform
integers in [120, 130]); 3. activations, standard normal float32; 4. gather row
ids, uniform in [0, output) with replacement.  Uniform random bytes are uniform
random indices because every row's index bits tile its bytes exactly in the
benchmark shapes; bits past the last index in a row (padding) stay random and
must be ignored by a decoder.  The codebook is deterministic: the standard
normal quantiles Phi^-1((i + 0.5) / 2**bits), evaluated in double and rounded
once to float32.
"""
from __future__ import annotations

import dataclasses
import statistics

import numpy as np


def codebook(bits: int) -> np.ndarray:
    """Standard-normal quantile codebook with 2**bits float32 entries."""
    n = 1 << bits
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((i + 0.5) / n) for i in range(n)],
                    dtype=np.float64).astype(np.float32)


def min_row_bytes(input_padded: int, bits: int) -> int:
    """Smallest row stride that holds ``input_padded`` indices of ``bits`` bits."""
    return (input_padded * bits + 7) // 8


@dataclasses.dataclass(frozen=True)
class CqShape:
    output: int
    input: int
    input_padded: int
    group: int
    bits: int
    row_bytes: int = 0          # 0 -> the minimum

    @property
    def stride(self) -> int:
        return self.row_bytes or min_row_bytes(self.input_padded, self.bits)

    @property
    def n_groups(self) -> int:
        return self.input_padded // self.group


@dataclasses.dataclass
class CqCase:
    shape: CqShape
    packed: np.ndarray      # uint8 [output][row_bytes]
    norms: np.ndarray       # uint16 (fp16 bits) [output][n_groups]
    codebook: np.ndarray    # float32 [2**bits]
    x: np.ndarray           # float32 [batch][input]
    ids: np.ndarray         # int32 [n_ids]


@dataclasses.dataclass
class F8Case:
    R: int
    C: int
    SR: int
    SC: int
    w: np.ndarray           # uint8 [R][C]
    scale: np.ndarray       # uint8 [SR][SC]
    x: np.ndarray           # float32 [batch][C]


@dataclasses.dataclass
class I8Case:
    R: int
    C: int
    G: int
    w: np.ndarray           # int8 [R][C]
    scale: np.ndarray       # uint8 [R][ceil(C / G)]
    x: np.ndarray           # float32 [batch][C]


@dataclasses.dataclass
class KvCase:
    v: np.ndarray           # float32 [n][d] key vectors to quantize
    x: np.ndarray           # float32 [batch][d] queries


@dataclasses.dataclass
class HmlpCase:
    n: np.ndarray           # float32 [batch][hidden] normalized block input
    d1: np.ndarray          # float32 [H]
    d2: np.ndarray          # float32 [H]
    d3: np.ndarray          # float32 [H]
    resid: np.ndarray       # float32 [batch][hidden]
    u: np.ndarray           # float32 [batch][hidden]


def _random_bytes(rng: np.random.Generator, shape, wide: bool = False) -> np.ndarray:
    """Uniform bytes; wide: drawn as full-range 64-bit words (a different
    stream, ~3x faster for multi-GiB buffers)."""
    if not wide:
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    n = int(np.prod(shape))
    words = rng.integers(0, 2**64, size=(n + 7) // 8, dtype=np.uint64)
    return words.view(np.uint8)[:n].reshape(shape)


def make_cq(shape: CqShape, seed: int, batch: int = 1, n_ids: int = 0,
            norm_range=(0.5, 2.0), wide_bytes: bool = False) -> CqCase:
    rng = np.random.default_rng(seed)
    packed = _random_bytes(rng, (shape.output, shape.stride), wide_bytes)
    norms = rng.uniform(norm_range[0], norm_range[1],
                        (shape.output, shape.n_groups)).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((batch, shape.input), dtype=np.float32)
    ids = rng.integers(0, shape.output, size=n_ids, dtype=np.int64).astype(np.int32) \
        if n_ids else np.zeros(0, dtype=np.int32)
    return CqCase(shape, packed, np.ascontiguousarray(norms), codebook(shape.bits), x, ids)


def make_f8(R: int, C: int, SR: int, SC: int, seed: int, batch: int = 1,
            exp_range=(120, 130), wide_bytes: bool = False) -> F8Case:
    rng = np.random.default_rng(seed)
    w = _random_bytes(rng, (R, C), wide_bytes)
    scale = rng.integers(exp_range[0], exp_range[1] + 1, size=(SR, SC), dtype=np.int64).astype(np.uint8)
    x = rng.standard_normal((batch, C), dtype=np.float32)
    return F8Case(R, C, SR, SC, w, scale, x)


def make_i8(R: int, C: int, G: int, seed: int, batch: int = 1, exp_range=(120, 130),
            wide_bytes: bool = False) -> I8Case:
    """Weight bytes uniform over all 256 int8 values, E8M0 exponents uniform in
    exp_range, activations N(0, 1); draw order: weights, scales, activations."""
    rng = np.random.default_rng(seed)
    w = _random_bytes(rng, (R, C), wide_bytes).view(np.int8)
    ns = (C + G - 1) // G
    scale = rng.integers(exp_range[0], exp_range[1] + 1, size=(R, ns), dtype=np.int64).astype(np.uint8)
    x = rng.standard_normal((batch, C), dtype=np.float32)
    return I8Case(R, C, G, w, scale, x)


def make_kv(n: int, d: int, seed: int, batch: int = 1) -> KvCase:
    """Key vectors N(0, 1) with a per-vector magnitude spread (each vector
    times 2^k, k uniform in [-4, 4]), then the queries N(0, 1)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, d), dtype=np.float32)
    v *= np.ldexp(np.float32(1), rng.integers(-4, 5, (n, 1))).astype(np.float32)
    x = rng.standard_normal((batch, d), dtype=np.float32)
    return KvCase(v, x)


def make_hmlp(hidden: int, H: int, seed: int, batch: int = 1) -> HmlpCase:
    """Hadamard MLP inputs: the normalized input, then d1, d2, d3, the
    residual and u, all N(0, 1) float32, in that draw order."""
    rng = np.random.default_rng(seed)
    n = rng.standard_normal((batch, hidden), dtype=np.float32)
    d1, d2, d3 = (rng.standard_normal(H, dtype=np.float32) for _ in range(3))
    resid = rng.standard_normal((batch, hidden), dtype=np.float32)
    u = rng.standard_normal((batch, hidden), dtype=np.float32)
    return HmlpCase(n, d1, d2, d3, resid, u)


# The five workloads.  Each is a list of (name, builder) pairs; a builder takes
# no arguments and returns a case.  Seeds restart per case.
C1 = CqShape(output=256, input=200, input_padded=256, group=64, bits=2)
C2_3 = CqShape(output=2048, input=512, input_padded=512, group=128, bits=3)
C2_5 = CqShape(output=2048, input=512, input_padded=512, group=128, bits=5)
C3 = CqShape(output=65536, input=512, input_padded=512, group=128, bits=4)
C4 = CqShape(output=16384, input=4096, input_padded=4096, group=256, bits=4)
HEAD = dict(R=246272, C=4096, SR=1924, SC=32)
WKV = dict(R=512, C=4096, SR=4, SC=32)
C3_GATHER_IDS = 4096
# Beyond the five: an I8 head of the same shape as the F8 one with E8M0 scales
# per 16 columns, and an int8 key cache of 4096 vectors of 128.
I8_HEAD = dict(R=246272, C=4096, G=16)
KV = dict(n=4096, d=128)
# The Hadamard MLP of a 512-wide block ("Inference engine, part 2", sections 7
# and 8) padded to 2048.
HMLP = dict(hidden=512, H=2048)


def make_logits(n: int, seed: int, scale: float = 3.0) -> np.ndarray:
    """float32 logits N(0, scale^2) (a sampler's input of the head's size)."""
    return (scale * np.random.default_rng(seed).standard_normal(n)).astype(np.float32)


# Inputs of many GB drawn on the device by torch's seeded generator (the
# caller passes the torch module); tests copy back the rows they check.
def _device_generator(torch, seed: int, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_normal(torch, shape, seed: int, device, scale: float = 1.0):
    """float32 N(0, scale^2)."""
    g = _device_generator(torch, seed, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale


def device_bytes(torch, n: int, seed: int, device):
    """n uniform bytes."""
    g = _device_generator(torch, seed, device)
    return torch.randint(0, 256, (n,), generator=g, device=device, dtype=torch.uint8)


def device_ids(torch, n: int, high: int, seed: int, device):
    """n int32 ids uniform in [0, high)."""
    g = _device_generator(torch, seed, device)
    return torch.randint(0, high, (n,), generator=g, device=device, dtype=torch.int32)


def device_norms(torch, shape, seed: int, device, lo: float = 0.5, hi: float = 2.0):
    """fp16 norms uniform in [lo, hi), as their int16 bit patterns."""
    g = _device_generator(torch, seed, device)
    return torch.empty(shape, dtype=torch.float16, device=device).uniform_(lo, hi, generator=g) \
        .view(torch.int16)


def config_cases(i: int, batch8: bool = True):
    """Cases of workload ``i`` (1-based), as (name, zero-argument builder)."""
    if i == 1:
        return [("cq2_256x200", lambda: make_cq(C1, seed=0))]
    if i == 2:
        return [("cq3_2048x512", lambda: make_cq(C2_3, seed=1)),
                ("cq5_2048x512", lambda: make_cq(C2_5, seed=1))]
    if i == 3:
        return [("cq4_65536x512_vocab_gather",
                 lambda: make_cq(C3, seed=2, n_ids=C3_GATHER_IDS))]
    if i == 4:
        out = [("cq4_16384x4096_b1", lambda: make_cq(C4, seed=3))]
        if batch8:
            out.append(("cq4_16384x4096_b8", lambda: make_cq(C4, seed=3, batch=8)))
        return out
    if i == 5:
        return [("f8_head_246272x4096", lambda: make_f8(**HEAD, seed=4)),
                ("f8_wkv_512x4096", lambda: make_f8(**WKV, seed=4))]
    raise ValueError(f"no workload {i}")

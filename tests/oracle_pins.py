"""Pins of the CPU oracle to facts the pages and mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
value printed on the pages (golden files, each cited in its header), a closed
form, a textbook or library routine, or exact rational arithmetic on tiny
inputs.  None of them re-types the oracle's own code: the checks go through
numpy/scipy/torch routines or through closed forms.  ``tests/test_oracle_pins``
runs them against the oracle; ``tests/test_oracle_mutants`` runs them against
copies of the oracle with planted mistakes and expects each copy to fail one.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np
import scipy.linalg
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------ test helpers --
def pack_indices(idx: np.ndarray, bits: int, row_bytes: int) -> np.ndarray:
    """Independent packer: numpy's little-endian bit packing of the index bits."""
    idx = np.asarray(idx, dtype=np.uint32)
    R, n = idx.shape
    planes = ((idx[:, :, None] >> np.arange(bits, dtype=np.uint32)) & 1).astype(np.uint8)
    stream = planes.reshape(R, n * bits)
    packed = np.packbits(stream, axis=1, bitorder="little")
    out = np.zeros((R, row_bytes), dtype=np.uint8)
    out[:, :packed.shape[1]] = packed
    return out


def unpack_indices(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Independent unpacker: numpy's little-endian bit unpacking."""
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, :n * bits]
    planes = stream.reshape(packed.shape[0], n, bits).astype(np.uint32)
    return (planes << np.arange(bits, dtype=np.uint32)).sum(axis=2)


def f16_np(norms: np.ndarray) -> np.ndarray:
    return np.asarray(norms, dtype=np.uint16).view(np.float16).astype(np.float64)


def dense_transform_weights(case) -> np.ndarray:
    """norm[r, group(c)] * codebook[idx(r, c)] in float64 (transform domain)."""
    s = case.shape
    idx = unpack_indices(case.packed, s.bits, s.input_padded)
    norm = np.repeat(f16_np(case.norms), s.group, axis=1)
    return norm * case.codebook.astype(np.float64)[idx]


def block_hadamard(n: int, g: int) -> np.ndarray:
    """Block-diagonal Sylvester Hadamard matrix (scipy), normalized by 1/sqrt(g)."""
    H = scipy.linalg.hadamard(g).astype(np.float64) / math.sqrt(g)
    return scipy.linalg.block_diag(*([H] * (n // g)))


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def small_cases():
    """Small CQ shapes spanning every bit width, ragged inputs and padded rows."""
    shapes = [
        synth.CqShape(5, 3, 4, 4, 2),
        synth.CqShape(7, 13, 16, 4, 3),
        synth.CqShape(6, 30, 32, 8, 5),
        synth.CqShape(9, 64, 64, 16, 4, row_bytes=40),
        synth.CqShape(4, 100, 128, 32, 3, row_bytes=53),
        synth.CqShape(3, 200, 256, 64, 2),
        synth.CqShape(4, 250, 256, 128, 5),
        synth.CqShape(3, 256, 256, 256, 4),
    ]
    return [synth.make_cq(s, seed=100 + i, batch=2) for i, s in enumerate(shapes)]


# ------------------------------------------------------------------- pins --
def pin_f16_golden():
    for code, bits, _ in (r[:2] + [r[2:]] for r in _read_table("f16_anchors.txt")):
        v = oracle.f16(int(code, 16))
        if bits == "nan":
            assert math.isnan(v), code
        else:
            got = struct.unpack("<I", struct.pack("<f", v))[0]
            assert got == int(bits, 16), (code, hex(got), bits)


def pin_f16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_array(codes)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def pin_fwht_hadamard4_golden():
    H = np.array([[int(v) for v in r] for r in _read_table("hadamard4.txt")], dtype=np.float32)
    for i in range(4):
        e = np.zeros(4, dtype=np.float32)
        e[i] = 1
        assert np.array_equal(oracle.fwht(e), H[i])


def pin_fwht_sylvester():
    rng = np.random.default_rng(7)
    for n in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        H = scipy.linalg.hadamard(n)
        for j in range(n):
            e = np.zeros(n, dtype=np.float32)
            e[j] = 1
            assert np.array_equal(oracle.fwht(e), H[:, j].astype(np.float32)), (n, j)
        x = rng.integers(-50, 51, n).astype(np.float32)
        assert np.array_equal(oracle.fwht(x), (H @ x.astype(np.int64)).astype(np.float32))


def pin_fwht_involution():
    rng = np.random.default_rng(8)
    for n in (2, 8, 64, 256, 1024):
        x = rng.integers(-100, 101, n).astype(np.float32)
        assert np.array_equal(oracle.fwht(oracle.fwht(x)), (n * x).astype(np.float32))


def pin_fwht_stride_order_rounding():
    """[P1] §1 runs the strides in ascending order and stores every stage in
    fp32; both show in the rounding.  x = [1, 2^-24, -1, 2^-24]: the stride-1
    stage forms 1 + 2^-24 (a tie between 1 and 1 + 2^-23, rounded to the even
    1), 1 - 2^-24 (exact), -1 + 2^-24 (exact) and -1 - 2^-24 (a tie, -1); the
    stride-2 stage then gives [2^-24, -2^-24, 2 - 2^-24 -> 2 (a tie, to the
    even 2), 2].  The strides in the other order, or stages kept exact, give
    the true transform [2^-23, -2^-23, 2, 2]."""
    t = np.float32(2.0 ** -24)
    x = np.array([1, t, -1, t], dtype=np.float32)
    want = np.array([t, -t, 2, 2], dtype=np.float32)
    assert np.array_equal(oracle.fwht(x).view(np.uint32), want.view(np.uint32))
    exact = np.array([2 * t, -2 * t, 2, 2], dtype=np.float32)
    assert not np.array_equal(want, exact)


def pin_crumb_order_golden():
    for row in _read_table("crumb_order.txt"):
        byte = int(row[0], 16)
        m = oracle.CqMatrix(1, 4, 4, 4, 2, 1, np.array([[byte]], np.uint8),
                            np.zeros((1, 1), np.uint16), synth.codebook(2))
        assert [oracle.cq_index(m, 0, c) for c in range(4)] == [int(v) for v in row[1:]], row


def pin_crumb_rule_all_bytes():
    cb = synth.codebook(2)
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    m = oracle.CqMatrix(1, 1024, 1024, 4, 2, 256, packed, np.zeros((1, 256), np.uint16), cb)
    idx = oracle.cq_unpack_row(m, 0)
    for byte in range(256):
        for crumb in range(4):
            assert idx[4 * byte + crumb] == (byte >> (crumb * 2)) & 3


def pin_nibble_order():
    packed = np.array([[0xBA, 0x01]], np.uint8)
    m = oracle.CqMatrix(1, 4, 4, 4, 4, 2, packed, np.zeros((1, 1), np.uint16), synth.codebook(4))
    assert list(oracle.cq_unpack_row(m, 0)) == [0xA, 0xB, 0x1, 0x0]


def pin_index_roundtrip():
    rng = np.random.default_rng(9)
    for bits in (2, 3, 4, 5):
        for n in (1, 3, 8, 13, 24, 40, 64, 100):
            rb = (n * bits + 7) // 8 + int(rng.integers(0, 3))
            idx = rng.integers(0, 1 << bits, (3, n))
            packed = pack_indices(idx, bits, rb)
            # padding bits past the last index hold noise the decoder must ignore
            tail_bits = rb * 8 - n * bits
            if tail_bits:
                noise = pack_indices(rng.integers(0, 2, (3, rb * 8)), 1, rb)
                keep = pack_indices(np.concatenate([np.ones((3, n * bits)), np.zeros((3, tail_bits))], 1), 1, rb)
                packed = (packed & keep) | (noise & ~keep)
            m = oracle.CqMatrix(3, n, n, 1, bits, rb, packed, np.zeros((3, n), np.uint16),
                                synth.codebook(bits))
            for r in range(3):
                assert np.array_equal(oracle.cq_unpack_row(m, r), idx[r]), (bits, n, r)


def pin_prepare_one_hot():
    for g, n_pad, inp in ((4, 8, 6), (64, 256, 200), (128, 512, 512), (256, 512, 300)):
        m = oracle.CqMatrix(1, inp, n_pad, g, 4, n_pad, np.zeros((1, n_pad), np.uint8),
                            np.zeros((1, n_pad // g), np.uint16), synth.codebook(4))
        scale = 1.0 / math.sqrt(g)
        for j in sorted({0, 1, g - 1, inp // 2, inp - 1}):
            x = np.zeros(inp, np.float32)
            x[j] = 1.0
            p = oracle.cq_prepare(m, x)
            g0 = (j // g) * g
            ref = np.zeros(n_pad, np.float32)
            for k in range(g):
                sign = -1.0 if bin((j - g0) & k).count("1") % 2 else 1.0
                ref[g0 + k] = np.float32(sign * scale)
            assert np.array_equal(p, ref), (g, j)


def _round_significand(fr: Fraction, bits: int) -> Fraction:
    """A positive rational rounded to `bits` significant bits, ties to even
    (IEEE round-to-nearest for a normal result)."""
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1  # now 2^e <= fr < 2^(e + 1)
    unit = Fraction(2) ** (e - bits + 1)
    scaled = fr / unit
    q = scaled.numerator // scaled.denominator
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return q * unit


def pin_prepare_scale_rounds_from_fp64():
    """[P1] §2 keeps the scale 1/sqrt(g) as a JavaScript number (a double),
    multiplies in double and stores to a Float32Array: the exact product is
    rounded to 53 bits, then to 24.  Worked exactly in rationals for g = 128
    (where the scale is no power of two): a one-hot v at column 0 transforms to
    v in every column of the group, so every prepared value is v's scaled
    value.  The v below are ones where a plain fp32 product rounds otherwise."""
    g = 128
    s64 = 1.0 / math.sqrt(float(g))  # the library's correctly rounded sqrt and division
    m = oracle.CqMatrix(1, g, g, g, 4, g // 2, np.zeros((1, g // 2), np.uint8),
                        np.zeros((1, 1), np.uint16), synth.codebook(4))
    differs = 0
    for bits in (0x3F800001, 0x3F800006, 0x3F800008, 0x40490FDB, 0x3DCCCCCD, 0x4479C000):
        v = np.array([bits], np.uint32).view(np.float32)[0]
        exact = Fraction(float(v)) * Fraction(s64)
        want = np.float32(float(_round_significand(_round_significand(exact, 53), 24)))
        x = np.zeros(g, np.float32)
        x[0] = v
        p = oracle.cq_prepare(m, x)
        assert np.array_equal(p.view(np.uint32), np.full(g, want).view(np.uint32)), hex(bits)
        differs += np.float32(v) * np.float32(s64) != want
    assert differs >= 3


def pin_prepare_vs_scipy():
    for case in small_cases():
        s = case.shape
        m = oracle.CqMatrix.from_case(case)
        xp = np.zeros((2, s.input_padded))
        xp[:, :s.input] = case.x
        ref = xp @ block_hadamard(s.input_padded, s.group).T
        got = oracle.cq_prepare(m, case.x)
        bound = np.abs(xp).reshape(2, -1, s.group).sum(-1).repeat(s.group, 1) / math.sqrt(s.group)
        assert np.all(np.abs(got - ref) <= 1e-6 * bound + 1e-30), s


def pin_cq_matvec_vs_dense():
    for case in small_cases():
        m = oracle.CqMatrix.from_case(case)
        p = oracle.cq_prepare(m, case.x)
        y, mag = oracle.cq_matvec(m, p)
        D = dense_transform_weights(case)
        ref = p.astype(np.float64) @ D.T
        refmag = np.abs(p.astype(np.float64)) @ np.abs(D).T
        assert np.all(np.abs(y - ref) <= 1e-12 * refmag + 1e-300), case.shape
        assert np.allclose(mag, refmag, rtol=1e-12, atol=0), case.shape


def pin_cq_matvec_row_range():
    case = small_cases()[3]
    m = oracle.CqMatrix.from_case(case)
    p = oracle.cq_prepare(m, case.x[0])
    y_all, _ = oracle.cq_matvec(m, p)
    y_mid, _ = oracle.cq_matvec(m, p, 2, 5)
    assert np.array_equal(y_mid, y_all[2:7])


def pin_matvec_gather_identity():
    """The pages' test: cqMatvec(x)[row] ~ dot(dequantizeRow(row), x), every width."""
    seen_bits = set()
    for case in small_cases():
        m = oracle.CqMatrix.from_case(case)
        p = oracle.cq_prepare(m, case.x)
        y, mag = oracle.cq_matvec(m, p)
        y7 = oracle.cq_dense_matvec(m, case.x)
        assert np.all(np.abs(y - y7) <= 1e-4 * mag + 1e-6), case.shape
        seen_bits.add(case.shape.bits)
    assert seen_bits == {2, 3, 4, 5}


def pin_tiny_exact_rationals():
    """R=3, input 5 -> 8, group 4 (scale 1/2 is exact): exact rational sums."""
    case = synth.make_cq(synth.CqShape(3, 5, 8, 4, 3), seed=11)
    s = case.shape
    m = oracle.CqMatrix.from_case(case)
    x = case.x[0]
    idx = unpack_indices(case.packed, 3, 8)
    H = scipy.linalg.hadamard(4)
    xf = [Fraction(float(v)) for v in x] + [Fraction(0)] * 3
    p_exact = []
    for g0 in (0, 4):
        for k in range(4):
            p_exact.append(sum(int(H[k, j]) * xf[g0 + j] for j in range(4)) / 2)
    p = oracle.cq_prepare(m, x)
    y, mag = oracle.cq_matvec(m, p)
    for r in range(3):
        exact = Fraction(0)
        for g in range(2):
            norm = Fraction(float(np.uint16(case.norms[r, g]).view(np.float16)))
            exact += norm * sum(Fraction(float(case.codebook[idx[r, k]])) * p_exact[k]
                                for k in range(4 * g, 4 * g + 4))
        assert abs(Fraction(y[r]) - exact) <= Fraction(1e-6) * Fraction(mag[r]), r
    _ = s


def pin_dequantize_row_norm_before_transform():
    """[P1] Row gather: each codebook value times the group norm (an fp32
    product), then the transform, then the scale (reading S8); only rounding
    shows the order.  Worked by hand for g = 4, codebook entries 1, 2^-24, -1
    at indices 1, 2, 3, indices [1, 2, 3, 2] and norm 3: the products are
    [3, 3*2^-24, -3, 3*2^-24]; stride 1 gives 3 +- 0.75 ulp(3), which round to
    3 +- 2^-22, so [3 + 2^-22, 3 - 2^-22, -3 + 2^-22, -3 - 2^-22]; stride 2 is
    exact, [2^-21, -2^-21, 6, 6]; times 1/2: [2^-22, -2^-22, 3, 3].  The norm
    applied after the transform would give [3*2^-25, -3*2^-25, 3, 3]."""
    cb = np.zeros(16, np.float32)
    cb[1], cb[2], cb[3] = 1.0, 2.0 ** -24, -1.0
    packed = np.array([[0x21, 0x23]], np.uint8)  # low nibble first: indices 1, 2, 3, 2
    norms = np.array([[0x4200]], np.uint16)      # fp16 3.0
    m = oracle.CqMatrix(1, 4, 4, 4, 4, 2, packed, norms, cb)
    want = np.array([2.0 ** -22, -2.0 ** -22, 3, 3], np.float32)
    assert np.array_equal(oracle.cq_dequantize_row(m, 0).view(np.uint32), want.view(np.uint32))


def pin_dequantize_row_vs_scipy():
    for case in small_cases():
        s = case.shape
        m = oracle.CqMatrix.from_case(case)
        D = dense_transform_weights(case)
        ref = (D @ block_hadamard(s.input_padded, s.group))[:, :s.input]
        for r in range(s.output):
            got = oracle.cq_dequantize_row(m, r)
            bound = (np.abs(D[r]).reshape(-1, s.group).sum(-1).repeat(s.group)
                     / math.sqrt(s.group))[:s.input]
            assert np.all(np.abs(got - ref[r]) <= 2e-6 * bound), (s, r)


def pin_dequantize_inverse_identity():
    """FWHT of the dequantized row (no column drop) gives back sqrt(g)*norm*codebook."""
    case = synth.make_cq(synth.CqShape(4, 64, 64, 16, 4), seed=12)
    s = case.shape
    m = oracle.CqMatrix.from_case(case)
    D = dense_transform_weights(case)
    for r in range(s.output):
        row = oracle.cq_dequantize_row(m, r)
        back = np.concatenate([oracle.fwht(row[g:g + 16]) for g in range(0, 64, 16)])
        assert np.allclose(back, D[r] * math.sqrt(16), rtol=0, atol=1e-5 * np.abs(D[r]).max())


def pin_dense_matvec_accumulates_in_fp64():
    """O7 sums dequantizeRow(r)[c] * x[c] as JavaScript numbers (fp64): against
    numpy's fp64 dot of the same rows, the difference stays at fp64 rounding
    (1e-12 of sum |row * x|), where an fp32 sum would be ~1e-7 off."""
    for case in small_cases():
        m = oracle.CqMatrix.from_case(case)
        x = case.x[0]
        rows = np.stack([oracle.cq_dequantize_row(m, r) for r in range(case.shape.output)])
        ref = rows.astype(np.float64) @ x.astype(np.float64)
        bound = np.abs(rows.astype(np.float64)) @ np.abs(x.astype(np.float64))
        y7 = oracle.cq_dense_matvec(m, x)
        assert np.all(np.abs(y7 - ref) <= 1e-12 * bound), case.shape


def pin_dequantize_scale_rounds_from_fp64():
    """The row gather scales by 1/sqrt(g) as the prepare does (R9): an fp64
    product stored to fp32.  Worked in rationals for g = 128: a row whose only
    nonzero weight is v at column 0 (norm 1) transforms to v in every column,
    so every gathered value is v's scaled value; the v are ones where an fp32
    product rounds otherwise."""
    g = 128
    s64 = 1.0 / math.sqrt(float(g))
    packed = np.zeros((1, g // 2), np.uint8)
    packed[0, 0] = 0x01  # column 0: index 1; every other column: index 0
    norms = np.array([[0x3C00]], np.uint16)  # fp16 1.0
    differs = 0
    for bits in (0x3F800001, 0x3F800006, 0x3F800008, 0x40490FDB, 0x3DCCCCCD, 0x4479C000):
        v = np.array([bits], np.uint32).view(np.float32)[0]
        cb = np.zeros(16, np.float32)
        cb[1] = v
        m = oracle.CqMatrix(1, g, g, g, 4, g // 2, packed, norms, cb)
        want = np.float32(float(_round_significand(_round_significand(
            Fraction(float(v)) * Fraction(s64), 53), 24)))
        row, _ = oracle.cq_gather(m, np.array([0], np.int32))
        assert np.array_equal(row[0].view(np.uint32), np.full(g, want).view(np.uint32)), hex(bits)
        differs += np.float32(v) * np.float32(s64) != want
    assert differs >= 3


def pin_gather():
    case = synth.make_cq(synth.CqShape(11, 100, 128, 32, 5), seed=13, n_ids=9)
    ids = np.concatenate([case.ids, case.ids[:2]])  # duplicates give equal rows
    m = oracle.CqMatrix.from_case(case)
    out, gmag = oracle.cq_gather(m, ids)
    D = dense_transform_weights(case)
    for i, r in enumerate(ids):
        assert np.array_equal(out[i], oracle.cq_dequantize_row(m, int(r)))
        ref = np.abs(D[r]).reshape(-1, 32).sum(-1).repeat(32)[:100] / math.sqrt(32)
        assert np.allclose(gmag[i], ref, rtol=1e-12, atol=0)
    assert np.array_equal(out[-2:], out[:2])


def pin_e4m3_golden():
    for row in _read_table("e4m3_anchors.txt"):
        code, val = int(row[0], 16), float(row[1])
        got = oracle.e4m3(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (row, got)


def pin_e4m3_all_codes():
    got = oracle.e4m3_all()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        if c & 0x7F == 0x7F:           # NaN in the OCP format, the clamp on the pages
            assert got[c] == (-448.0 if c & 0x80 else 448.0)
        else:
            assert got[c].view(np.uint32) == ref[c].view(np.uint32), hex(c)
    # brute force over sign/exponent/mantissa in exact rationals
    for c in range(256):
        s, e, mt = c >> 7, (c >> 3) & 15, c & 7
        v = Fraction(mt, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(mt, 8)) * Fraction(2) ** (e - 7)
        v = min(v, Fraction(448))
        assert Fraction(float(got[c])) == (-v if s else v), hex(c)


def pin_e8m0_all_codes():
    got = oracle.e8m0_all()
    for e in range(256):
        if e == 255:
            assert math.isnan(got[e])
        else:
            assert got[e] == np.float32(math.ldexp(1.0, e - 127)) and got[e] > 0, e


def _f8_dense(case):
    W = torch.from_numpy(case.w.copy()).view(torch.float8_e4m3fn).double().numpy()
    sat = (case.w & 0x7F) == 0x7F
    W[sat] = np.where(case.w[sat] & 0x80, -448.0, 448.0)
    rs = (np.arange(case.R, dtype=np.int64) * case.SR) // case.R
    cs = (np.arange(case.C, dtype=np.int64) * case.SC) // case.C
    S = np.ldexp(1.0, case.scale.astype(np.int64) - 127)[rs][:, cs]
    return W * S


def pin_f8_matvec_vs_dense():
    for (R, C, SR, SC) in ((10, 7, 3, 2), (256, 64, 2, 4), (130, 260, 3, 5), (64, 128, 1, 1)):
        case = synth.make_f8(R, C, SR, SC, seed=R + C, batch=2)
        y, mag = oracle.f8_matvec(case.w, R, C, case.scale, SR, SC, case.x)
        D = _f8_dense(case)
        ref = case.x.astype(np.float64) @ D.T
        refmag = np.abs(case.x.astype(np.float64)) @ np.abs(D).T
        assert np.all(np.abs(y - ref) <= 1e-12 * refmag + 1e-300), (R, C, SR, SC)
        assert np.allclose(mag, refmag, rtol=1e-12, atol=0)


def pin_f8_matvec_one_hot():
    case = synth.make_f8(256, 48, 2, 3, seed=5)
    case.w[:, 17] = np.arange(256, dtype=np.uint8)    # every code through the dot
    x = np.zeros(48, np.float32)
    x[17] = 1.0
    y, _ = oracle.f8_matvec(case.w, 256, 48, case.scale, 2, 3, x)
    for r in range(256):
        s = case.scale[(r * 2) // 256, (17 * 3) // 48]
        v = Fraction(float(oracle.e4m3(r))) * Fraction(2) ** (int(s) - 127)
        assert Fraction(y[r]) == v, r



# ----------------------------------------------------------------- sampling
def _gf2_matrix_of(f):
    """The 32x32 matrix over GF(2) of a linear map on uint32 (column j = f(e_j))."""
    M = np.zeros((32, 32), np.uint8)
    for j in range(32):
        v = f(1 << j)
        for i in range(32):
            M[i, j] = (v >> i) & 1
    return M


def _gf2_pow(M, e):
    R = np.eye(32, dtype=np.int64)
    B = M.astype(np.int64)
    while e:
        if e & 1:
            R = (R @ B) % 2
        B = (B @ B) % 2
        e >>= 1
    return R


def pin_xorshift_full_period():
    """O11 is linear over GF(2) and has the maximal period 2^32 - 1 (the
    property that defines a usable xorshift generator): with T its matrix,
    T^(2^32-1) = I and T^((2^32-1)/p) != I for every prime p dividing
    2^32 - 1 = 3 * 5 * 17 * 257 * 65537."""
    rng = np.random.default_rng(11)
    for _ in range(20):  # linearity: f(a ^ b) = f(a) ^ f(b)
        a, b = (int(v) for v in rng.integers(1, 2**32, 2, dtype=np.uint64))
        assert oracle.xorshift32(a ^ b) == oracle.xorshift32(a) ^ oracle.xorshift32(b)
    T = _gf2_matrix_of(oracle.xorshift32)
    order = 2**32 - 1
    assert np.array_equal(_gf2_pow(T, order), np.eye(32, dtype=np.int64))
    for prime in (3, 5, 17, 257, 65537):
        assert not np.array_equal(_gf2_pow(T, order // prime), np.eye(32, dtype=np.int64)), prime
    # a full-period state sequence never reaches 0 from a nonzero state
    s = 1
    for _ in range(1000):
        s = oracle.xorshift32(s)
        assert s != 0


def _topk_numpy(x, k):
    """Sort key (NaN flag, -value, index); +0 and -0 compare equal."""
    idx = np.arange(x.size)
    nan = np.isnan(x)
    neg = np.where(nan, 0.0, -x.astype(np.float64)) + 0.0  # -0.0 -> +0.0
    order = np.lexsort((idx, neg, nan))
    return order[:k].astype(np.int32)


def pin_topk_vs_numpy_lexsort():
    """O12 against numpy's lexsort on random, tie-heavy and special values."""
    rng = np.random.default_rng(12)
    cases = [rng.standard_normal(5000).astype(np.float32),
             rng.integers(-3, 4, 3000).astype(np.float32),  # many ties
             np.array([1, 3, 3, 2, np.nan, -0.0, 0.0, np.inf, -np.inf, np.inf], np.float32)]
    x = rng.standard_normal(700).astype(np.float32)
    x[rng.integers(0, 700, 60)] = np.nan
    cases.append(x)
    for x in cases:
        for k in (1, 2, 7, 64, min(x.size, 100)):
            k = min(k, x.size)
            ids, vals = oracle.topk(x, k)
            ref = _topk_numpy(x, k)
            assert np.array_equal(ids, ref), (k, ids[:8], ref[:8])
            assert np.array_equal(vals.view(np.uint32), x[ref].view(np.uint32))


def pin_sample_inverse_cdf_grid():
    """O13 inverts the softmax CDF: over the grid u_j = (j + 1/2)/M the
    number of draws that land on candidate i is M * p_i within 1, with p
    from scipy's softmax of vals / temperature."""
    from scipy.special import softmax
    rng = np.random.default_rng(13)
    for k, T in ((5, 1.0), (16, 0.7), (64, 2.5), (3, 0.05)):
        vals = np.sort(rng.standard_normal(k).astype(np.float32))[::-1].copy()
        ids = rng.permutation(10 * k)[:k].astype(np.int32)
        p = softmax(vals.astype(np.float64) / T)
        M = 20000
        counts = {int(i): 0 for i in ids}
        for j in range(M):
            counts[oracle.sample_u(vals, ids, T, (j + 0.5) / M)] += 1
        for i, pi in zip(ids, p):
            assert abs(counts[int(i)] - M * pi) <= 1.0 + 1e-9, (k, T, i, counts[int(i)], M * pi)


def pin_sample_degenerate_cases():
    """Temperature 0 and k = 1 give the top candidate; the generator form
    advances the state exactly once and draws u = state / 2^32."""
    vals = np.array([2.0, 1.0, 0.5], np.float32)
    ids = np.array([40, 10, 30], np.int32)
    for u in (0.0, 0.5, 0.999999):
        assert oracle.sample_u(vals, ids, 0.0, u) == 40
        assert oracle.sample_u(vals[:1], ids[:1], 1.0, u) == 40
    for s in (1, 12345, 0xdeadbeef):
        tok, s2 = oracle.sample(vals, ids, 1.0, s)
        assert s2 == oracle.xorshift32(s)
        assert tok == oracle.sample_u(vals, ids, 1.0, s2 / 2**32)

def _xorshift_preimage(t):
    """The state whose (13, 17, 5) xorshift step gives t: each step
    s ^= s << a (or >> b) is undone by xoring in the shifted partial results
    until the shift runs past 32 bits."""
    mask = 0xFFFFFFFF

    def undo_left(y, a):
        x = y
        for _ in range(32 // a + 1):
            x = y ^ ((x << a) & mask)
        return x

    def undo_right(y, b):
        x = y
        for _ in range(32 // b + 1):
            x = y ^ (x >> b)
        return x

    return undo_left(undo_right(undo_left(t, 5), 17), 13)


def pin_sample_draw_scale():
    """The draw is u = state / 2^32 exactly (R21), checked where it decides
    the token: the state that steps to 2^31 gives u = 1/2; two candidates
    1 and 1 - 2^-24 at T = 1000 weigh 1 and exp(-2^-24 / 1000), so the first
    is drawn iff u < 1 / (1 + exp(-2^-24 / 1000)) = 1/2 + 1.49e-11.  Any
    other scale of the state by ~2^-32 (say 1 / (2^32 - 1), which gives
    1/2 + 1.16e-10) draws the second."""
    pre = _xorshift_preimage(1 << 31)
    vals = np.array([1.0, np.nextafter(np.float32(1), np.float32(0))], np.float32)
    ids = np.array([5, 9], np.int32)
    tok, state = oracle.sample(vals, ids, 1000.0, pre)
    assert state == 1 << 31
    assert tok == 5
    # the boundary itself: just above 1/2 + 1.49e-11 the second candidate wins
    assert oracle.sample_u(vals, ids, 1000.0, 0.5 + 3e-11) == 9


def pin_sample_special_candidates():
    """O13 on special candidates: NaNs (which O12 sorts last) carry no weight,
    so over the u grid they are never drawn and the others keep their softmax
    shares; an infinite top candidate takes every draw; and large logits draw
    exactly as the same logits shifted down by 998 (both exact in fp32, so
    the differences to the top candidate, and every weight, are the same)."""
    from scipy.special import softmax
    vals = np.array([1.5, 0.25, -1.0, np.nan, np.nan], np.float32)
    ids = np.array([7, 3, 9, 1, 2], np.int32)
    p = softmax(vals[:3].astype(np.float64) / 0.8)
    M = 20000
    counts = {int(i): 0 for i in ids}
    for j in range(M):
        counts[oracle.sample_u(vals, ids, 0.8, (j + 0.5) / M)] += 1
    assert counts[1] == 0 and counts[2] == 0, counts
    for i, pi in zip(ids[:3], p):
        assert abs(counts[int(i)] - M * pi) <= 1.0 + 1e-9, (i, counts[int(i)], M * pi)
    top_inf = np.array([np.inf, 2.0, 1.0], np.float32)
    for u in (0.0, 0.3, 0.999):
        assert oracle.sample_u(top_inf, ids[:3], 1.0, u) == 7
    big = np.array([1000.0, 999.5, 999.0, 998.0], np.float32)
    small = big - np.float32(998.0)
    ids4 = np.array([5, 6, 7, 8], np.int32)
    drawn = set()
    for j in range(200):
        u = (j + 0.5) / 200
        t = oracle.sample_u(big, ids4, 0.7, u)
        assert t == oracle.sample_u(small, ids4, 0.7, u), u
        drawn.add(t)
    assert drawn == set(ids4.tolist())


# ------------------------------------------------ I8 matvec (O14) --------
def _i8_case(rng, R, C, G):
    w = rng.integers(-128, 128, (R, C)).astype(np.int8)
    s = rng.integers(118, 133, (R, (C + G - 1) // G)).astype(np.uint8)
    x = rng.standard_normal(C).astype(np.float32)
    return w, s, x


def pin_i8_matvec_dense():
    """numpy dense product with the E8M0 scales expanded by np.repeat
    (groups of G columns, the last one ragged)."""
    rng = np.random.default_rng(31)
    for R, C, G in ((37, 80, 16), (5, 96, 32), (9, 50, 16), (4, 33, 7), (3, 64, 64)):
        w, s, x = _i8_case(rng, R, C, G)
        scale = np.ldexp(1.0, s.astype(np.int64) - 127)
        wf = w.astype(np.float64) * np.repeat(scale, G, axis=1)[:, :C]
        ref = wf @ x.astype(np.float64)
        y, mag = oracle.i8_matvec(w, R, C, s, G, x)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12), (R, C, G)
        assert np.allclose(mag, np.abs(wf) @ np.abs(x.astype(np.float64)), rtol=1e-12)
        y2, _ = oracle.i8_matvec(w, R, C, s, G, x, 2, R - 3)
        assert np.array_equal(y2, y[2:R - 1])


def pin_i8_matvec_one_hot():
    """x = e_c: y[r] = w[r][c] * 2^(s[r][c // G] - 127) exactly, every int8 value."""
    R, C, G = 256, 48, 16
    rng = np.random.default_rng(32)
    w = np.arange(-128, 128, dtype=np.int64).astype(np.int8)[:, None].repeat(C, axis=1)
    w = np.ascontiguousarray(np.roll(w, 5, axis=1))
    s = rng.integers(100, 150, (R, C // G)).astype(np.uint8)
    for c in (0, 15, 16, 47):
        x = np.zeros(C, np.float32)
        x[c] = 1.0
        y, _ = oracle.i8_matvec(w, R, C, s, G, x)
        expect = [math.ldexp(float(w[r, c]), int(s[r, c // G]) - 127) for r in range(R)]
        assert np.array_equal(y, np.array(expect)), c


# ------------------------------------------ storeInt8 (O15) -------------
def pin_store_int8_exact_ties():
    """Largest magnitude 127 makes the scale exactly 1: the codes are the
    inputs rounded half to even (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -63.5 -> -64)."""
    v = np.array([127, 0.5, 1.5, 2.5, -2.5, -63.5, 63.5, -0.5, 3.25, -126.5], np.float32)
    q, sc = oracle.store_int8(v)
    assert sc == np.float32(1.0)
    assert q.tolist() == [127, 0, 2, 2, -2, -64, 64, 0, 3, -126]
    # largest magnitude negative: -127 and scale 1 again
    q, sc = oracle.store_int8(-v)
    assert sc == np.float32(1.0) and q[0] == -127 and q[2] == -2


def pin_store_int8_properties():
    """Codes lie in [-127, 127]; the largest magnitude gets +-127 with its
    sign; every code is within half a step of v / scale; the scale is the
    largest magnitude over 127 rounded to fp32."""
    rng = np.random.default_rng(33)
    vecs = [rng.standard_normal(128), rng.uniform(-1, 1, 64) * 1e-3, -np.abs(rng.standard_normal(33)) * 50,
            rng.standard_cauchy(256), np.r_[rng.standard_normal(63), -400.0]]
    for v in vecs:
        v = v.astype(np.float32)
        q, sc = oracle.store_int8(v)
        a = np.abs(v.astype(np.float64))
        assert sc == np.float32(a.max() / 127.0)
        assert np.all(np.abs(q.astype(np.int64)) <= 127)
        i = int(np.argmax(a))
        assert q[i] == (127 if v[i] > 0 else -127)
        assert np.all(np.abs(v.astype(np.float64) / (a.max() / 127.0) - q) <= 0.5 + 1e-9)


def pin_store_int8_floor_and_specials():
    """The 1e-12 floor: an all-zero vector gets scale 1e-12/127 and zero codes;
    a vector below the floor is coded against it.  A NaN makes the maximum
    NaN (JavaScript's Math.max), hence every code 0 (Int8Array stores NaN as
    0); an infinite element makes every finite code 0."""
    q, sc = oracle.store_int8(np.zeros(8, np.float32))
    assert sc == np.float32(1e-12 / 127) and not q.any()
    q, sc = oracle.store_int8(np.array([2.5e-13, -5e-13], np.float32))
    assert sc == np.float32(1e-12 / 127)
    assert q.tolist() == [round(float(np.float32(2.5e-13)) * 127 / 1e-12),
                          -round(float(np.float32(5e-13)) * 127 / 1e-12)]
    q, sc = oracle.store_int8(np.array([1.0, np.nan, -3.0], np.float32))
    assert math.isnan(sc) and not q.any()
    q, sc = oracle.store_int8(np.array([1.0, np.inf, -3.0], np.float32))
    assert math.isinf(sc) and not q.any()


def pin_store_int8_divides_by_fp64_scale():
    """Codes divide by the scale as a JavaScript number (fp64), not by the
    fp32 value the scale array stores (R26).  With largest magnitude 1 the
    fp64 scale is fl(1/127) and the stored one 3.7e-9 relatively smaller;
    these two inputs put v / scale within 1e-9 of 79.5 and 95.5, on the lower
    side for the fp64 scale and the upper side for the fp32 one, so the codes
    (from exact rational quotients, far from fp64 rounding) are 79 and 95,
    not 80 and 96."""
    from fractions import Fraction
    v = np.array([1.0, 0.625984251499176, 0.751968502998352, -0.625984251499176], np.float32)
    s64 = Fraction(1.0 / 127.0)
    s32 = Fraction(float(np.float32(1.0 / 127.0)))
    for x, code in ((v[1], 79), (v[2], 95)):
        assert math.floor(Fraction(float(x)) / s64 + Fraction(1, 2)) == code
        assert math.floor(Fraction(float(x)) / s32 + Fraction(1, 2)) == code + 1
    q, sc = oracle.store_int8(v)
    assert q.tolist() == [127, 79, 95, -79]
    assert sc == np.float32(1.0 / 127.0)


# ------------------------------------------- scaled int8 dot (O16) --------
def pin_int8_dot_dense():
    rng = np.random.default_rng(34)
    K = rng.integers(-127, 128, (70, 128)).astype(np.int8)
    scales = rng.uniform(1e-3, 2.0, 70).astype(np.float32)
    x = rng.standard_normal(128).astype(np.float32)
    y, mag = oracle.int8_dot(K, scales, x)
    ref = scales.astype(np.float64) * (K.astype(np.float64) @ x.astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    ref_mag = scales.astype(np.float64) * (np.abs(K.astype(np.float64)) @ np.abs(x.astype(np.float64)))
    assert np.allclose(mag, ref_mag, rtol=1e-12)
    y2, _ = oracle.int8_dot(K, scales, x, 10, 20)
    assert np.array_equal(y2, y[10:30])


def pin_int8_quantize_then_dot():
    """storeInt8 then the scaled dot reproduces dot(v, x) within the
    quantization bound sum_j |x_j| * scale / 2."""
    rng = np.random.default_rng(35)
    V = rng.standard_normal((16, 64)).astype(np.float32)
    x = rng.standard_normal(64).astype(np.float32)
    q, sc = oracle.store_int8(V)
    y, _ = oracle.int8_dot(q, sc, x)
    exact = V.astype(np.float64) @ x.astype(np.float64)
    bound = np.abs(x.astype(np.float64)).sum() * sc.astype(np.float64) / 2 * (1 + 1e-6)
    assert np.all(np.abs(y - exact) <= bound)


# ------------------------------------------------ Hadamard MLP (O17) -----
def _hmlp_exact_case(rng, hidden, H):
    n = rng.integers(-3, 4, hidden).astype(np.float32)
    d1 = rng.choice([-1.0, 1.0, 2.0, 0.5], H).astype(np.float32)
    resid = rng.integers(-8, 9, hidden).astype(np.float32)
    z = np.zeros(H)
    z[:hidden] = n
    z1 = (scipy.linalg.hadamard(H) / math.sqrt(H)) @ (d1.astype(np.float64) * z)
    return n, d1, resid, z1


def pin_hadamard_mlp_closed_forms():
    """Inputs whose every fp32 stage is exact (small integers, H = 16 or 64
    so 1/sqrt(H) is a power of two):
      d2 = 0: silu(0) = 0, the block output is the residual;
      d2 = 2^12 * sign(z1): silu(t) = t for t >= 40 in fp64, and with
        d3 = 2^-12 the output is resid + (H_n |H_n (d1 * pad(n))|)[:hidden]
        (H_n the normalized Sylvester matrix from scipy);
      d2 = -2^12 * sign(z1): silu of a large negative argument is -0, the
        block output is the residual again;
      with u: the update is that output minus u."""
    rng = np.random.default_rng(36)
    for hidden, H in ((10, 16), (48, 64)):
        n, d1, resid, z1 = _hmlp_exact_case(rng, hidden, H)
        sign = np.where(z1 >= 0, 1.0, -1.0)
        ones = np.ones(H, np.float32)
        out, _ = oracle.hadamard_mlp(n, H, d1, np.zeros(H, np.float32), ones, resid)
        assert np.array_equal(out, resid)
        nz = np.abs(z1) > 0
        d2 = (sign * 4096.0 * nz).astype(np.float32)
        d3 = np.full(H, 2.0 ** -12, np.float32)
        out, _ = oracle.hadamard_mlp(n, H, d1, d2, d3, resid)
        Hn = scipy.linalg.hadamard(H) / math.sqrt(H)
        expect = resid.astype(np.float64) + (Hn @ (np.abs(z1) * nz))[:hidden]
        assert np.array_equal(out.astype(np.float64), expect), (hidden, H)
        u = rng.integers(-4, 5, hidden).astype(np.float32)
        out_u, _ = oracle.hadamard_mlp(n, H, d1, d2, d3, resid, u)
        assert np.array_equal(out_u.astype(np.float64), expect - u)
        out, _ = oracle.hadamard_mlp(n, H, d1, -d2, d3, resid)
        assert np.array_equal(out, resid)


def pin_hadamard_mlp_magnitude_tight():
    """The MLP's tolerance magnitude |resid| + |u| + |d3| / sqrt(H) * sum|silu|
    is the exact triangle bound of the output: where every silu value is
    positive (d2 = 2^12 sign(z1), silu(t) = t) and the output row is the
    all-ones row of the transform (row 0), the bound is met exactly, so
    magnitude[0] = |resid[0]| + (out[0] - resid[0]) with every stage exact."""
    rng = np.random.default_rng(37)
    for hidden, H in ((10, 16), (48, 64)):
        n, d1, resid, z1 = _hmlp_exact_case(rng, hidden, H)
        nz = np.abs(z1) > 0
        d2 = (np.where(z1 >= 0, 1.0, -1.0) * 4096.0 * nz).astype(np.float32)
        d3 = np.full(H, 2.0 ** -12, np.float32)
        out, mag = oracle.hadamard_mlp(n, H, d1, d2, d3, resid)
        lift = float(out[0]) - float(resid[0])
        assert lift > 0
        assert mag[0] == abs(float(resid[0])) + lift, (hidden, H)


def pin_hadamard_mlp_matrix_form():
    """Random inputs against the float64 matrix form with scipy's Hadamard
    matrix and numpy's exp, within fp32 rounding of the stages."""
    rng = np.random.default_rng(37)
    for hidden, H in ((100, 128), (512, 2048), (64, 64)):
        n = rng.standard_normal(hidden).astype(np.float32)
        d1, d2, d3 = (rng.uniform(-2, 2, H).astype(np.float32) for _ in range(3))
        resid = rng.standard_normal(hidden).astype(np.float32)
        u = rng.standard_normal(hidden).astype(np.float32)
        out, mag = oracle.hadamard_mlp(n, H, d1, d2, d3, resid, u)
        Hn = scipy.linalg.hadamard(H) / math.sqrt(H)
        z = np.zeros(H)
        z[:hidden] = n
        t = d2 * (Hn @ (d1 * z))
        s_ = t / (1 + np.exp(-t))
        ref = resid + (d3 * (Hn @ s_))[:hidden] - u
        assert np.all(np.abs(out - ref) <= 1e-5 * mag + 1e-6), (hidden, H, np.abs(out - ref).max())


def pin_hadamard_mlp_update_rounds_block_first():
    """The block output is stored (fp32) before the update subtracts u (R29:
    every array store rounds).  H = hidden = 1, n = 1.5, d2 = 64 (t = 96, and
    silu(96) = 96 in fp64), d3 = 2^-31 make z = 3 * 2^-26 exactly; resid = 1
    stores the block as 1 (3/8 of an ulp is dropped), and u = -59 * 2^-26
    gives 1 + 59 * 2^-26 = 1 + 7.375 ulp -> 1 + 7 * 2^-23.  One rounding of
    resid + z - u (1 + 7.75 ulp) would give 1 + 2^-20."""
    one = np.ones(1, np.float32)
    f = lambda v: np.array([v], np.float32)
    out, _ = oracle.hadamard_mlp(f(1.5), 1, one, f(64.0), f(2.0 ** -31), f(1.0), f(-59 * 2.0 ** -26))
    assert out[0] == np.float32(1 + 7 * 2.0 ** -23), float(out[0])
    block, _ = oracle.hadamard_mlp(f(1.5), 1, one, f(64.0), f(2.0 ** -31), f(1.0))
    assert block[0] == np.float32(1.0)


def _near_fp32_midpoint(fr: Fraction, rel=Fraction(1, 10 ** 14)) -> bool:
    """True if a positive rational lies within rel of a point halfway between
    two fp32 values, where an fp64 intermediate could round either way."""
    r = _round_significand(fr, 25)  # the nearest 25-bit value: fp32 points and midpoints
    return abs(fr - r) <= rel * fr and r != _round_significand(fr, 24)


def pin_hadamard_mlp_silu_fp64():
    """silu(t) = t / (1 + exp(-t)) is formed as a JavaScript number (fp64) and
    stored to fp32 (R29).  With H = hidden = 1 and d1 = d3 = 1, resid = 0 the
    MLP's output is that stored value for t = d2 * n (exact in fp64), so it
    must equal the exact silu, taken to 40 digits with the decimal module,
    rounded to fp32 (inputs whose exact value lies within 1e-14 of an fp32
    rounding midpoint are skipped: there fp64 may round either way).  An fp32
    silu differs on many of them."""
    from decimal import Decimal, getcontext
    getcontext().prec = 40
    rng = np.random.default_rng(38)
    ones, zero = np.ones(1, np.float32), np.zeros(1, np.float32)
    checked = differs = 0
    for n, d2 in zip(rng.uniform(-6, 6, 300).astype(np.float32), rng.uniform(0.25, 2, 300).astype(np.float32)):
        t = Fraction(float(n)) * Fraction(float(d2))
        dt = Decimal(t.numerator) / Decimal(t.denominator)
        exact = Fraction(dt / (1 + (-dt).exp()))
        if exact == 0 or _near_fp32_midpoint(abs(exact)):
            continue
        mag = _round_significand(abs(exact), 24)
        want = np.float32(float(mag if exact > 0 else -mag))
        out, _ = oracle.hadamard_mlp(np.array([n], np.float32), 1, ones, np.array([d2], np.float32),
                                     ones, zero)
        assert out[0] == want and out.view(np.uint32)[0] == np.array([want]).view(np.uint32)[0], (n, d2)
        t32 = np.float32(n) * np.float32(d2)
        differs += (t32 / (np.float32(1) + np.exp(-t32))) != want
        checked += 1
    assert checked >= 290 and differs >= 10, (checked, differs)


def pin_hadamard_mlp_scale_rounds_from_fp64():
    """normalizedFwht multiplies by 1/sqrt(H) in fp64 and stores to fp32
    (R29), in both transforms.  H = 2, hidden = 1, d1 = 1, d2 = 2^40 (silu(t)
    = t exactly once t > 40), d3 = 2^-40, resid = 0: the first transform of
    [x, 0] is [x, x], scaled to v = fl32(fl64(x s)); the second of [2^40 v,
    2^40 v] is [2^41 v, 0], scaled and brought back by 2^-40, so the output is
    fl32(fl64(2 v s)), worked in rationals.  An fp32 product rounds otherwise
    on some of these x."""
    s64 = 1.0 / math.sqrt(2.0)
    d1, d2, d3 = (np.full(2, v, np.float32) for v in (1.0, 2.0 ** 40, 2.0 ** -40))
    rng = np.random.default_rng(39)
    differs = 0
    for x in rng.uniform(0.01, 100.0, 200).astype(np.float32):
        v = _round_significand(_round_significand(Fraction(float(x)) * Fraction(s64), 53), 24)
        want = np.float32(float(_round_significand(_round_significand(2 * v * Fraction(s64), 53), 24)))
        out, _ = oracle.hadamard_mlp(np.array([x], np.float32), 2, d1, d2, d3, np.zeros(1, np.float32))
        assert out.view(np.uint32)[0] == np.array([want]).view(np.uint32)[0], x
        v32 = np.float32(x) * np.float32(s64)
        differs += np.float32(2 * v32) * np.float32(s64) != want
    assert differs >= 5, differs


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

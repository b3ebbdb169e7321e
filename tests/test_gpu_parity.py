"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: index decode, fp16 / E4M3 / E8M0 value decode, prepare, gather,
and the one-hot cases whose sums are exact.  fp32 dots: per output
|gpu - oracle| <= 1e-4 * sum|w*x| + 1e-6 (sum|w*x| from the oracle).
Sizes: the five workloads at full size (every output, the heads' 246272 rows
included, against the oracle), plus small shapes that cover every
bit width, every fast-kernel lane layout, ragged row counts, padded rows and
the generic (unaligned / odd-width) path.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import bit_quantized_decode_amd as bqd
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def tol_ok(got, ref, mag):
    got = np.asarray(got, dtype=np.float64)
    return np.abs(got - ref) <= 1e-4 * mag + 1e-6


def assert_tol(got, ref, mag, what):
    ratio = np.abs(np.asarray(got, dtype=np.float64) - ref) / (1e-4 * mag + 1e-6)
    print(f"[tol] {what}: max |gpu-oracle| / (1e-4*sum|w*x| + 1e-6) = {ratio.max():.3g}", flush=True)
    ok = tol_ok(got, ref, mag)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs out of tolerance, first at "
                             f"{tuple(i)}: gpu={np.asarray(got)[tuple(i)]} oracle={ref[tuple(i)]} "
                             f"mag={mag[tuple(i)]}")


def dev_matrix(case):
    s = case.shape
    return bqd.CqMatrix.from_arrays(case.packed, case.norms, case.codebook, output=s.output,
                                    input=s.input, input_padded=s.input_padded, group=s.group,
                                    bits=s.bits, row_bytes=s.stride)


def host_matrix(case):
    return oracle.CqMatrix.from_case(case)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits_eq(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------- workloads
WORKLOADS = {name: build for i in range(1, 6) for name, build in synth.config_cases(i)}


@pytest.fixture(scope="module")
def cache():
    return {}


def workload(cache, name):
    if name not in cache:
        print(f"[case] building {name}", flush=True)
        cache[name] = WORKLOADS[name]()
    return cache[name]


CQ_WORKLOADS = [n for n in WORKLOADS if n.startswith("cq")]

# Small CQ shapes: every bit width and every fast lane layout (rows of 8..256
# chunks of 32 columns), ragged row counts, padded rows; then generic-path
# shapes (odd widths, groups under 32, rows not a dword multiple); then shapes
# for the matrix-core batch kernel.
SMALL = [
    synth.CqShape(100, 256, 256, 32, 2), synth.CqShape(77, 500, 512, 64, 3),
    synth.CqShape(45, 1000, 1024, 128, 4), synth.CqShape(33, 2048, 2048, 256, 5),
    synth.CqShape(19, 4096, 4096, 512, 3), synth.CqShape(9, 8192, 8192, 1024, 4),
    synth.CqShape(21, 300, 512, 32, 4, row_bytes=260), synth.CqShape(13, 256, 256, 64, 5, row_bytes=176),
    synth.CqShape(5, 3, 4, 4, 2), synth.CqShape(7, 13, 16, 4, 3), synth.CqShape(6, 30, 32, 8, 5),
    synth.CqShape(9, 64, 64, 16, 4, row_bytes=40), synth.CqShape(4, 100, 128, 32, 3, row_bytes=53),
    synth.CqShape(11, 96, 96, 32, 2), synth.CqShape(3, 250, 256, 128, 5, row_bytes=161),
    # matrix-core batch path: groups >= 256, whole 256-column spans, ragged row tiles
    synth.CqShape(37, 700, 768, 256, 2), synth.CqShape(20, 4096, 4096, 1024, 4, row_bytes=2052),
    # rows wider than every fast layout (16384 columns): the generic kernels
    synth.CqShape(7, 16000, 16384, 1024, 4),
]


def small_case(i, batch=1):
    return synth.make_cq(SMALL[i], seed=1000 + i, batch=batch, n_ids=23)


# ------------------------------------------------------------ decode probes
def test_probe_f8_all_codes():
    for n in (256, 255, 5):
        codes = np.arange(n, dtype=np.uint8)[::-1].copy()
        got = bqd.dbg_f8_decode(to_dev(codes)).cpu().numpy()
        ref = oracle.e4m3_all()[codes]
        assert bits_eq(got, ref), np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))


@pytest.mark.parametrize("nbytes", [16, 1008, 16384, 16384 * 64 + 48, 4096 * 2048 * 16 + 4096 * 5 + 32])
def test_read_stream_reads_every_word(nbytes):
    # The bandwidth probe: the XOR of its per-workgroup words is the XOR of
    # every 32-bit word of the buffer (whole steps, the ragged tail, and a
    # buffer beyond one step per workgroup).
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = to_dev(words.view(np.int32))
    out = torch.full((bqd.READ_STREAM_WORDS,), -1, dtype=torch.int32, device=DEV)
    bqd.dbg_read_stream(buf, out)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_probe_e8m0_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = bqd.dbg_e8m0_decode(to_dev(codes)).cpu().numpy()
    ref = oracle.e8m0_all()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert bits_eq(got[:255], ref[:255])


def test_probe_f16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = bqd.dbg_f16_decode(to_dev(codes.view(np.int16))).cpu().numpy()
    ref = oracle.f16_array(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert bits_eq(got[~nan], ref[~nan])


def check_unpack(case, rows):
    m, h = dev_matrix(case), host_matrix(case)
    for r in rows:
        got = bqd.dbg_cq_unpack(m, int(r)).cpu().numpy()
        assert np.array_equal(got, oracle.cq_unpack_row(h, int(r))), (case.shape, r)


@pytest.mark.parametrize("name", ["cq2_256x200", "cq3_2048x512", "cq5_2048x512",
                                  "cq4_65536x512_vocab_gather", "cq4_16384x4096_b1"])
def test_unpack_workloads(cache, name):
    case = workload(cache, name)
    R = case.shape.output
    rows = range(R) if R <= 256 else np.unique(np.r_[0, 1, R - 1, np.random.default_rng(0).integers(0, R, 40)])
    check_unpack(case, rows)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_unpack_small(i):
    case = small_case(i)
    check_unpack(case, range(case.shape.output))


# ------------------------------------------------------------------ prepare
def check_prepare(case):
    m, h = dev_matrix(case), host_matrix(case)
    got = bqd.cq_prepare(m, to_dev(case.x)).cpu().numpy()
    ref = oracle.cq_prepare(h, case.x)
    assert bits_eq(got, ref), (case.shape, np.argwhere(got.view(np.uint32) != ref.view(np.uint32))[:5])


@pytest.mark.parametrize("name", CQ_WORKLOADS)
def test_prepare_workloads(cache, name):
    check_prepare(workload(cache, name))


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_prepare_small(i):
    check_prepare(small_case(i, batch=3))


# ------------------------------------------------------------------- matvec
def check_matvec(case, row_begin=0, row_count=None):
    """The oracle's reference starts from its own prepared vectors (O3 on the
    raw activations); the GPU's prepared vectors must equal them bit for bit
    for every vector of the batch before they feed the GPU matvec."""
    s = case.shape
    row_count = s.output - row_begin if row_count is None else row_count
    m, h = dev_matrix(case), host_matrix(case)
    p_dev = bqd.cq_prepare(m, to_dev(case.x))
    p_ref = oracle.cq_prepare(h, case.x)
    assert bits_eq(p_dev.cpu().numpy(), p_ref), (s, "prepared vectors differ from the oracle's")
    got = bqd.cq_matvec(m, p_dev, row_begin=row_begin, row_count=row_count).cpu().numpy()
    ref, mag = oracle.cq_matvec(h, p_ref, row_begin, row_count)
    assert_tol(got, ref, mag, f"cq_matvec {s} rows [{row_begin}, +{row_count})")
    return got


@pytest.mark.parametrize("name", CQ_WORKLOADS)
def test_matvec_workloads(cache, name):
    print(f"[case] matvec {name}", flush=True)
    check_matvec(workload(cache, name))


@pytest.mark.parametrize("i", range(len(SMALL)))
@pytest.mark.parametrize("batch", [1, 3, 6])
def test_matvec_small(i, batch):
    check_matvec(small_case(i, batch=batch))


def test_matvec_row_ranges(cache):
    case = workload(cache, "cq4_16384x4096_b1")
    for rb, rc in ((0, 1), (1000, 3001), (16383, 1), (5, 16379)):
        check_matvec(case, rb, rc)
    small = small_case(0, batch=2)
    for rb, rc in ((0, 1), (3, 50), (99, 1)):
        check_matvec(small, rb, rc)


# Matrix-core batch path: eight-vector launches and a remainder launch, row
# ranges, a row count that gives part of the persistent grid a second row
# block (over 256 x 64 rows at 4096 columns), groups of two and four spans,
# and a 15-span row (one span per wavefront, 15 wavefronts).
MFMA_CASES = [
    (synth.CqShape(17084, 4096, 4096, 512, 3), 2, 0, None),
    (synth.CqShape(300, 2048, 2048, 256, 4), 9, 0, None),
    (synth.CqShape(300, 2000, 2048, 256, 5), 16, 7, 250),
    (synth.CqShape(130, 1024, 1024, 1024, 2), 8, 1, 129),
    (synth.CqShape(64, 256, 256, 256, 4), 5, 0, None),
    (synth.CqShape(1000, 3840, 3840, 256, 4), 8, 0, None),
]


@pytest.mark.parametrize("k", range(len(MFMA_CASES)))
def test_matvec_batch_matrix_core(k):
    shape, batch, rb, rc = MFMA_CASES[k]
    print(f"[case] matrix-core {shape} batch {batch} rows [{rb}, +{rc})", flush=True)
    check_matvec(synth.make_cq(shape, seed=500 + k, batch=batch), rb, rc)


def one_hot_inputs(s, cols):
    """x whose prepared vector is exactly e_k for each k in cols: column k of
    the normalized Hadamard block of k's group (every entry +-1/sqrt(g), an
    exact power of two for g = 4^n)."""
    g = s.group
    H = scipy.linalg.hadamard(g)
    x = np.zeros((len(cols), s.input), np.float32)
    for b, k in enumerate(cols):
        g0 = (k // g) * g
        x[b, g0:g0 + g] = H[:, k - g0] / math.sqrt(g)
    return x


@pytest.mark.parametrize("shape,cols", [
    (synth.C4, [0, 31, 32, 255, 256 * 7 + 100, 4095]),
    (synth.C1, [0, 63, 64, 130, 191]),
    (synth.CqShape(64, 1024, 1024, 256, 3), [0, 33, 1023]),
    (synth.CqShape(48, 2048, 2048, 64, 5), [5, 700, 2047]),
    (synth.CqShape(40, 256, 256, 16, 2), [0, 17, 255]),
])
def test_matvec_one_hot_decodes_indices_exactly(shape, cols):
    """codebook[i] = i, norms = 1: y[r] = idx(r, k) exactly, through the fast
    kernels at batch 1 and the shared-weight batch path."""
    case = synth.make_cq(shape, seed=77)
    case.codebook = np.arange(1 << shape.bits, dtype=np.float32)
    case.norms[:] = 0x3C00
    case.x = one_hot_inputs(shape, cols)
    m, h = dev_matrix(case), host_matrix(case)
    p = bqd.cq_prepare(m, to_dev(case.x))
    pe = np.zeros((len(cols), shape.input_padded), np.float32)
    pe[np.arange(len(cols)), cols] = 1.0
    assert bits_eq(p.cpu().numpy(), pe)
    ref = np.stack([[oracle.cq_index(h, r, k) for r in range(shape.output)] for k in cols])
    y1 = np.stack([bqd.cq_matvec(m, p[b:b + 1]).cpu().numpy()[0] for b in range(len(cols))])
    yb = bqd.cq_matvec(m, p).cpu().numpy()
    assert np.array_equal(y1, ref.astype(np.float32))
    assert np.array_equal(yb, ref.astype(np.float32))


# Batch-1 4-bit ring kernel and the fused prepare + matvec entry point: every
# row width the ring kernel covers (512 ... 8192), groups from 8 to 1024 (the
# fused transform runs in the kernel for groups <= 256, two launches above),
# unpadded widths below input_padded, row counts that leave the last
# workgroup partly empty, and row ranges.
RING_CASES = [
    (synth.CqShape(300, 300, 512, 8, 4), 0, None),
    (synth.CqShape(129, 512, 512, 64, 4), 0, None),
    (synth.CqShape(257, 1000, 1024, 16, 4), 3, 200),
    (synth.CqShape(130, 2048, 2048, 128, 4), 0, None),
    (synth.CqShape(200, 4000, 4096, 256, 4), 0, None),
    (synth.CqShape(65, 4096, 4096, 32, 4), 1, 63),
    (synth.CqShape(70, 8192, 8192, 256, 4), 0, None),
    (synth.CqShape(40, 8192, 8192, 1024, 4), 5, 33),
    (synth.CqShape(33, 4096, 4096, 512, 4, row_bytes=2064), 0, None),
]


@pytest.mark.parametrize("k", range(len(RING_CASES)))
def test_prepare_matvec_fused(k):
    shape, rb, rc = RING_CASES[k]
    row_count = shape.output - rb if rc is None else rc
    print(f"[case] prepare+matvec {shape} rows [{rb}, +{row_count})", flush=True)
    case = synth.make_cq(shape, seed=900 + k)
    m, h = dev_matrix(case), host_matrix(case)
    x = to_dev(case.x)
    p, y = bqd.cq_prepare_matvec(m, x, row_begin=rb, row_count=row_count)
    p_ref = oracle.cq_prepare(h, case.x)
    assert bits_eq(p.cpu().numpy(), p_ref)
    ref, mag = oracle.cq_matvec(h, p_ref, rb, row_count)
    assert_tol(y.cpu().numpy(), ref, mag, f"cq_prepare_matvec {shape}")
    # the same bits as the two calls it stands for
    y2 = bqd.cq_matvec(m, bqd.cq_prepare(m, x), row_begin=rb, row_count=row_count)
    assert bits_eq(y.cpu().numpy(), y2.cpu().numpy())


def test_prepare_matvec_workload_and_batches(cache):
    case = workload(cache, "cq4_16384x4096_b1")
    m, h = dev_matrix(case), host_matrix(case)
    p, y = bqd.cq_prepare_matvec(m, to_dev(case.x))
    p_ref = oracle.cq_prepare(h, case.x)
    assert bits_eq(p.cpu().numpy(), p_ref)
    ref, mag = oracle.cq_matvec(h, p_ref)
    assert_tol(y.cpu().numpy(), ref, mag, "cq_prepare_matvec CQ4 16384x4096")
    # batches and other widths take the two-launch path
    small = small_case(0, batch=3)
    ms, hs = dev_matrix(small), host_matrix(small)
    p, y = bqd.cq_prepare_matvec(ms, to_dev(small.x))
    p_ref = oracle.cq_prepare(hs, small.x)
    assert bits_eq(p.cpu().numpy(), p_ref)
    ref, mag = oracle.cq_matvec(hs, p_ref)
    assert_tol(y.cpu().numpy(), ref, mag, "cq_prepare_matvec batch 3")
    # an empty row range still prepares
    p, y = bqd.cq_prepare_matvec(m, to_dev(case.x), row_begin=100, row_count=0)
    assert bits_eq(p.cpu().numpy(), oracle.cq_prepare(h, case.x)) and y.numel() == 0


# cq_prepare_matvec on batches (the prepare, then the matrix-core matvec):
# the workload's eight vectors, a remainder launch, unpadded widths, row
# ranges, a single workgroup over four spans, workgroups of several row
# groups, a single span, and an input that is not a whole number of float4s.
BATCH_PM_CASES = [
    (synth.CqShape(300, 2048, 2048, 256, 4), 9, 0, None),
    (synth.CqShape(1000, 3840, 3840, 256, 4), 8, 0, None),
    (synth.CqShape(77, 4000, 4096, 256, 4), 3, 5, 70),
    (synth.CqShape(20, 1000, 1024, 256, 4), 16, 0, None),
    (synth.CqShape(40000, 512, 512, 256, 4), 8, 3, 39990),
    (synth.CqShape(33, 252, 256, 256, 4), 5, 0, None),
    (synth.CqShape(64, 256, 256, 256, 4), 2, 63, 1),
    (synth.CqShape(21, 1001, 1024, 256, 4), 3, 0, None),
]


def check_prepare_matvec_batch(case, rb=0, rc=None):
    s = case.shape
    rc = s.output - rb if rc is None else rc
    m, h = dev_matrix(case), host_matrix(case)
    x = to_dev(case.x)
    p, y = bqd.cq_prepare_matvec(m, x, row_begin=rb, row_count=rc)
    p_ref = oracle.cq_prepare(h, case.x)
    assert bits_eq(p.cpu().numpy(), p_ref), (s, "prepared vectors differ from the oracle's")
    ref, mag = oracle.cq_matvec(h, p_ref, rb, rc)
    assert_tol(y.cpu().numpy(), ref, mag, f"cq_prepare_matvec {s} batch {len(case.x)}")
    # the same bits as the two calls it stands for
    y2 = bqd.cq_matvec(m, bqd.cq_prepare(m, x), row_begin=rb, row_count=rc)
    assert bits_eq(y.cpu().numpy(), y2.cpu().numpy())


@pytest.mark.parametrize("k", range(len(BATCH_PM_CASES)))
def test_prepare_matvec_batch(k):
    shape, batch, rb, rc = BATCH_PM_CASES[k]
    print(f"[case] batch prepare+matvec {shape} batch {batch} rows [{rb}, +{rc})", flush=True)
    check_prepare_matvec_batch(synth.make_cq(shape, seed=950 + k, batch=batch), rb, rc)


def test_prepare_matvec_batch_workload(cache):
    case = workload(cache, "cq4_16384x4096_b8")
    print(f"[case] batch prepare+matvec {case.shape} batch {len(case.x)}", flush=True)
    check_prepare_matvec_batch(case)


# Several matrices on one activation ([P1] §6): shared launches on the ring
# shapes (up to four matrices a launch: ten take three, 64 take sixteen),
# row ranges, empty ranges, different codebooks, and shapes that fall back
# to one launch each.
MULTI_CASES = [
    ([synth.CqShape(2048, 512, 512, 128, 4), synth.CqShape(300, 512, 512, 128, 4),
      synth.CqShape(65, 512, 512, 128, 4)], [(0, 2048), (10, 200), (64, 1)]),
    ([synth.CqShape(130 + 7 * k, 4000, 4096, 256, 4) for k in range(10)], None),
    ([synth.CqShape(200, 256, 256, 64, 2), synth.CqShape(100, 256, 256, 64, 4),
      synth.CqShape(50, 256, 256, 64, 3)], [(0, 200), (5, 90), (0, 0)]),
    ([synth.CqShape(40, 8192, 8192, 1024, 4), synth.CqShape(33, 8192, 8192, 1024, 4)], None),
    # the most matrices one call takes (64): sixteen shared launches of four
    ([synth.CqShape(20 + 3 * k, 512, 512, 128, 4) for k in range(64)], None),
]


@pytest.mark.parametrize("k", range(len(MULTI_CASES)))
@pytest.mark.parametrize("fused", [False, True])
def test_matvec_multi(k, fused):
    shapes, ranges = MULTI_CASES[k]
    print(f"[case] multi {len(shapes)} matrices {shapes[0]} fused={fused}", flush=True)
    check_multi(shapes, ranges, fused, 950 + 10 * k)


@pytest.mark.parametrize("k", range(16))
def test_matvec_multi_random(k):
    """Random sets of 1-12 matrices on one activation (mostly on the ring
    shapes, some other widths), random row ranges, both entry points."""
    rng = np.random.default_rng(8700 + k)
    if rng.random() < 0.7:
        input_padded, bits_choice = int(rng.choice([512, 1024, 2048, 4096, 8192])), [4]
    else:
        input_padded, bits_choice = int(256 * rng.integers(1, 9)), [2, 3, 4, 5]
    group = int(rng.choice([g for g in (8, 16, 32, 64, 128, 256, 512, 1024) if input_padded % g == 0]))
    input_ = input_padded - (int(rng.integers(0, min(group, 20))) if rng.random() < 0.4 else 0)
    shapes, ranges = [], []
    for _ in range(int(rng.integers(1, 13))):
        bits = int(rng.choice(bits_choice))
        pad = int(rng.choice([0, 0, 16, 4]))
        out = int(rng.integers(1, 1500))
        shapes.append(synth.CqShape(out, input_, input_padded, group, bits,
                                    synth.min_row_bytes(input_padded, bits) + pad))
        rb = int(rng.integers(0, out)) if rng.random() < 0.4 else 0
        ranges.append((rb, int(rng.integers(0, out - rb + 1)) if rng.random() < 0.4 else out - rb))
    for fused in (False, True):
        print(f"[case] random multi {len(shapes)} x {shapes[0]} fused={fused}", flush=True)
        check_multi(shapes, ranges, fused, 8800 + 20 * k)


def check_multi(shapes, ranges, fused, seed0):
    cases = [synth.make_cq(sh, seed=seed0 + j) for j, sh in enumerate(shapes)]
    x = cases[0].x
    ms = [dev_matrix(c) for c in cases]
    ranges = ranges or [(0, sh.output) for sh in shapes]
    p_ref = oracle.cq_prepare(host_matrix(cases[0]), x)
    if fused:
        p, outs = bqd.cq_prepare_matvec_multi(ms, to_dev(x[0]), ranges=ranges)
        assert bits_eq(p.cpu().numpy(), p_ref[0])
    else:
        p = bqd.cq_prepare(ms[0], to_dev(x))[0]
        outs = bqd.cq_matvec_multi(ms, p, ranges=ranges)
    for c, m, (rb, rc), o in zip(cases, ms, ranges, outs):
        got = o.cpu().numpy()
        single = bqd.cq_matvec(m, p[None], row_begin=rb, row_count=rc).cpu().numpy()[0]
        assert bits_eq(got, single)
        if rc:
            ref, mag = oracle.cq_matvec(host_matrix(c), p_ref[0], rb, rc)
            assert_tol(got, ref, mag, f"multi {c.shape} [{rb}, +{rc})")


def test_matvec_unaligned_packed_uses_generic_path():
    case = synth.make_cq(synth.CqShape(50, 512, 512, 128, 4), seed=5)
    s = case.shape
    m = dev_matrix(case)
    buf = torch.zeros(m.packed.numel() + 1, dtype=torch.uint8, device=DEV)
    buf[1:] = m.packed.reshape(-1)
    mo = bqd.CqMatrix(buf[1:], m.norms, m.codebook, output=s.output, input=s.input,
                      input_padded=s.input_padded, group=s.group, bits=s.bits, row_bytes=s.stride)
    p = bqd.cq_prepare(m, to_dev(case.x))
    p_ref = oracle.cq_prepare(host_matrix(case), case.x)
    assert bits_eq(p.cpu().numpy(), p_ref)
    ref, mag = oracle.cq_matvec(host_matrix(case), p_ref)
    assert_tol(bqd.cq_matvec(mo, p).cpu().numpy(), ref, mag, "unaligned packed")
    got = bqd.dbg_cq_unpack(mo, 7).cpu().numpy()
    assert np.array_equal(got, oracle.cq_unpack_row(host_matrix(case), 7))


def test_matvec_deterministic(cache):
    case = workload(cache, "cq4_16384x4096_b8")
    m = dev_matrix(case)
    p = bqd.cq_prepare(m, to_dev(case.x))
    a = bqd.cq_matvec(m, p).cpu().numpy()
    b = bqd.cq_matvec(m, p).cpu().numpy()
    assert bits_eq(a, b)


# ------------------------------------------------------------------- gather
def check_gather(case, ids):
    m, h = dev_matrix(case), host_matrix(case)
    got = bqd.cq_gather_rows(m, to_dev(ids.astype(np.int32))).cpu().numpy()
    ref, _ = oracle.cq_gather(h, ids)
    assert bits_eq(got, ref), (case.shape, np.argwhere(got.view(np.uint32) != ref.view(np.uint32))[:5])


def test_gather_workload(cache):
    case = workload(cache, "cq4_65536x512_vocab_gather")
    check_gather(case, case.ids)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_gather_small(i):
    case = small_case(i)
    check_gather(case, np.concatenate([case.ids, case.ids[:3]]))


def test_gather_identity_with_matvec(cache):
    """The pages' test, end to end on the GPU: matvec[row] ~ dot(gathered row, x)."""
    case = workload(cache, "cq4_65536x512_vocab_gather")
    m = dev_matrix(case)
    rows = case.ids[:512]
    dense = bqd.cq_gather_rows(m, to_dev(rows)).cpu().numpy().astype(np.float64)
    y = bqd.cq_matvec(m, bqd.cq_prepare(m, to_dev(case.x))).cpu().numpy()[0]
    _, mag = oracle.cq_matvec(host_matrix(case), oracle.cq_prepare(host_matrix(case), case.x[0]))
    assert np.all(np.abs(y[rows] - dense @ case.x[0].astype(np.float64)) <= 1e-4 * mag[rows] + 1e-6)


def test_gather_out_of_range_ids_give_nan_rows():
    case = small_case(1)
    m = dev_matrix(case)
    ids = np.array([0, -1, case.shape.output, 2], np.int32)
    got = bqd.cq_gather_rows(m, to_dev(ids)).cpu().numpy()
    ref, _ = oracle.cq_gather(host_matrix(case), ids[[0, 3]])
    assert bits_eq(got[[0, 3]], ref)
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()


# ----------------------------------------------------------------------- F8
def dev_f8(case):
    return to_dev(case.w), to_dev(case.scale), to_dev(case.x)


def check_f8(case, row_blocks=None):
    w, s, x = dev_f8(case)
    got = bqd.f8_matvec(w, s, x).cpu().numpy()
    blocks = row_blocks or [(0, case.R)]
    for rb, rc in blocks:
        ref, mag = oracle.f8_matvec(case.w, case.R, case.C, case.scale, case.SR, case.SC, case.x,
                                    rb, rc)
        assert_tol(got[:, rb:rb + rc], ref, mag, f"f8 {case.R}x{case.C} rows [{rb}, +{rc})")
    return got


# ----------------------------------------------- F8 matvec with fused argmax
def host_argmax(y):
    """Per vector: the row of the largest value, equal values at the lowest row,
    NaN below every number (row 0 if all are NaN), -0 equal to +0."""
    out = []
    for v in np.atleast_2d(y).astype(np.float64):
        ok = ~np.isnan(v)
        out.append(int(np.flatnonzero(v == v[ok].max())[0]) if ok.any() else 0)
    return np.array(out)


def check_f8_argmax(case, workspace=None):
    """y bit-identical to f8_matvec's; the token the argmax of that y (an
    integer decision on the GPU's own values); against the oracle, the chosen
    row is a largest logit within the tolerance of the two rows involved."""
    w, s, x = dev_f8(case)
    y, tok = bqd.f8_matvec_argmax(w, s, x, workspace=workspace)
    y0 = bqd.f8_matvec(w, s, x)
    yn, tokn = y.cpu().numpy().reshape(-1, case.R), tok.cpu().numpy()
    assert bits_eq(yn, y0.cpu().numpy().reshape(-1, case.R))
    assert np.array_equal(tokn, host_argmax(yn)), (tokn, host_argmax(yn))
    ref, mag = oracle.f8_matvec(case.w, case.R, case.C, case.scale, case.SR, case.SC, case.x)
    ref, mag = np.atleast_2d(ref), np.atleast_2d(mag)
    for b, t in enumerate(tokn):
        if np.isnan(ref[b]).all():
            continue
        best = int(np.nanargmax(ref[b]))
        if ref[b][t] == ref[b][best]:  # also where both are +inf
            continue
        tol = 1e-4 * mag[b] + 1e-6
        assert ref[b][t] >= ref[b][best] - tol[t] - tol[best], (b, t, best)
    return tokn


def test_f8_argmax_head(cache):
    case = workload(cache, "f8_head_246272x4096")
    print("[case] f8 head with fused argmax", flush=True)
    ws = torch.full((bqd.f8_matvec_argmax_workspace_bytes(1),), 0xA5, dtype=torch.uint8, device=DEV)
    t1 = check_f8_argmax(case, ws)  # a workspace holding garbage
    assert np.array_equal(check_f8_argmax(case, ws), t1)  # and again, after the first call


@pytest.mark.parametrize("k", range(16))
def test_f8_argmax_random_shapes(k):
    rng = np.random.default_rng(9000 + k)
    R = int(rng.integers(1, 5000))
    C = int(16 * rng.integers(1, 513)) if rng.random() < 0.6 else int(rng.integers(1, 3000))
    SR = int(rng.integers(1, min(R, 64) + 1))
    SC = int(rng.choice([d for d in range(1, min(C, 64) + 1) if C % d == 0]))
    batch = int(rng.choice([1, 1, 2, 3]))
    print(f"[case] f8 argmax {R}x{C} scales {SR}x{SC} batch {batch}", flush=True)
    check_f8_argmax(synth.make_f8(R, C, SR, SC, seed=9100 + k, batch=batch))


@pytest.mark.parametrize("C", [4096, 100])
def test_f8_argmax_ties_nan_and_inf(C):
    """Equal largest logits take the lowest row; a NaN activation makes every
    logit NaN (row 0); +inf in one column makes the lowest +inf row win.
    C = 4096 runs the streaming kernel, C = 100 the generic one."""
    case = synth.make_f8(300, C, 1, 4, seed=91)  # one scale row: equal rows, equal logits
    case.w[:] = 0x00
    for r in (200, 50, 123):
        case.w[r] = 0x38  # 1.0 everywhere: three equal rows
    case.x[:] = np.abs(case.x)
    assert check_f8_argmax(case)[0] == 50
    nan_case = synth.make_f8(300, C, 3, 4, seed=92)
    nan_case.x[0, 7] = np.nan
    assert check_f8_argmax(nan_case)[0] == 0
    inf_case = synth.make_f8(300, C, 3, 4, seed=93)
    inf_case.w[:, 3] = 0x00
    inf_case.w[[40, 17, 250], 3] = 0x38
    inf_case.x[0, 3] = np.inf
    assert check_f8_argmax(inf_case)[0] == 17


# ---------------------------------------- F8 matvec with fused top-k sampling
def host_topk_ids(y, k):
    """Rows of the k best of y: a larger value first, equal values (+0 = -0)
    at the lower row, NaN after every number."""
    v = np.asarray(y, np.float64)
    nan = np.isnan(v)
    order = np.lexsort((np.arange(v.size), -np.where(nan, 0.0, v), nan))
    return order[:k].astype(np.int32)


def _states(seeds):
    return torch.tensor(np.array(seeds, np.uint32).view(np.int32), dtype=torch.int32, device=DEV)


def check_f8_sample(case, k, T, seeds, workspace=None):
    """y bit-identical to f8_matvec's; per vector, the k ids those of y's k
    best (an integer decision on the GPU's own values), the values y's at
    them bit for bit, the state one xorshift32 step on, and ids, values,
    token and state equal to logits_sample's on that y.  Returns
    (y, tokens, ids, vals) as numpy arrays."""
    w, s, x = dev_f8(case)
    st = _states(seeds)
    y, tok, ids, vals = bqd.f8_matvec_sample(w, s, x, k, T, st, workspace=workspace)
    y0 = bqd.f8_matvec(w, s, x)
    yn = y.cpu().numpy().reshape(-1, case.R)
    assert bits_eq(yn, y0.cpu().numpy().reshape(-1, case.R))
    tokn, idsn, valsn = tok.cpu().numpy(), ids.cpu().numpy(), vals.cpu().numpy()
    stn = st.cpu().numpy().view(np.uint32)
    for b in range(yn.shape[0]):
        want = host_topk_ids(yn[b], k)
        assert np.array_equal(idsn[b], want), (b, idsn[b][:8], want[:8])
        assert bits_eq(valsn[b], yn[b][want])
        assert int(stn[b]) == oracle.xorshift32(int(seeds[b]))
        st2 = _states([seeds[b]])
        t2, i2, v2 = bqd.logits_sample(y[b].reshape(-1) if y.dim() > 1 else y, k, T, st2)
        assert np.array_equal(i2.cpu().numpy(), idsn[b])
        assert bits_eq(v2.cpu().numpy(), valsn[b])
        assert int(t2.item()) == int(tokn[b]) and int(st2.cpu().numpy().view(np.uint32)[0]) == stn[b]
        if k == 1 or T == 0.0:
            assert int(tokn[b]) == int(want[0])
        else:
            assert int(tokn[b]) in set(want.tolist())
    return yn, tokn, idsn, valsn


def test_f8_sample_head(cache):
    """The 246272 x 4096 head with top-k sampling fused: the checks of
    check_f8_sample, then against the oracle's logits (every row): the k
    selected values are, in order, the k largest oracle logits within the
    tolerance (the i-th largest moves by at most the largest row error), and
    each selected logit is within tolerance of its own row's oracle value."""
    case = workload(cache, "f8_head_246272x4096")
    print("[case] f8 head with fused top-k sampling", flush=True)
    ws = torch.full((bqd.f8_matvec_argmax_workspace_bytes(1),), 0xA5, dtype=torch.uint8, device=DEV)
    ref, mag = oracle_all_rows(lambda a, c: oracle.f8_matvec(
        case.w, case.R, case.C, case.scale, case.SR, case.SC, case.x[0], a, c), case.R)
    tol = 1e-4 * mag + 1e-6
    for k, T in ((64, 0.8), (1, 1.0), (8, 0.0), (17, 2.5)):
        _, tok, ids, vals = check_f8_sample(case, k, T, [0x9E3779B9 + k], workspace=ws)
        ids, vals = ids[0], vals[0].astype(np.float64)
        assert np.all(np.abs(vals - ref[ids]) <= tol[ids])
        ref_top = np.sort(ref)[::-1][:k]
        assert np.all(np.abs(vals - ref_top) <= tol.max()), k
        print(f"[case] head k={k} T={T}: token {int(tok[0])}, top id {int(ids[0])}", flush=True)


def _exact_f8(R, C, seed, batch=1):
    """F8 weights of exact small values (0, +-0.5, +-1, +-2; scale 2^0) and
    integer activations in [-8, 8]: every product and partial sum is a
    multiple of 0.5 below 2^23 in magnitude, so any summation order gives the
    exact logit and the GPU's y equals the oracle's bit for bit (many equal
    logits, so the order of ties is exercised too)."""
    rng = np.random.default_rng(seed)
    codes = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)
    case = synth.make_f8(R, C, 1, 1, seed=seed, batch=batch)
    case.w[:] = codes[rng.integers(0, codes.size, (R, C), dtype=np.uint8)]
    case.scale[:] = 127
    case.x[:] = rng.integers(-8, 9, case.x.shape).astype(np.float32)
    return case


@pytest.mark.parametrize("R,C,k,T", [(246272, 4096, 64, 0.8), (50000, 4096, 33, 1.5),
                                     (100000, 128, 64, 0.5), (3000, 100, 10, 0.9)])
def test_f8_sample_exact_logits_equal_oracle(R, C, k, T):
    """Where the logits are exact, the fused result equals the oracle's top-k
    and draw on the oracle's own logits, over three chained draws."""
    case = _exact_f8(R, C, seed=R + C)
    print(f"[case] f8 sample exact {R}x{C} k={k} T={T}", flush=True)
    ref, _ = oracle_all_rows(lambda a, c: oracle.f8_matvec(
        case.w, case.R, case.C, case.scale, case.SR, case.SC, case.x[0], a, c), case.R)
    ref = ref.astype(np.float32)
    w, s, x = dev_f8(case)
    seed = 0x12345 + R
    st = _states([seed])
    rid, rval = oracle.topk(ref, k)
    for _ in range(3):
        y, tok, ids, vals = bqd.f8_matvec_sample(w, s, x, k, T, st)
        assert np.array_equal(y.cpu().numpy().reshape(-1), ref)
        assert np.array_equal(ids.cpu().numpy()[0], rid)
        assert np.array_equal(vals.cpu().numpy()[0], rval)
        rtok, seed = oracle.sample(rval, rid, T, seed)
        assert int(st.cpu().numpy().view(np.uint32)[0]) == seed
        if int(tok[0].item()) != rtok:
            assert _near_cdf_boundary(rval, T, seed / 2**32), (int(tok[0].item()), rtok)


@pytest.mark.parametrize("j", range(12))
def test_f8_sample_random_shapes(j):
    """Random shapes through the streaming kernel (C a multiple of 16) and the
    generic one, batches of 1-3 with a state each, k from 1 to min(64, R)."""
    rng = np.random.default_rng(9500 + j)
    R = int(rng.integers(1, 70000)) if j % 3 else int(rng.integers(1, 300))
    C = int(16 * rng.integers(1, 300)) if rng.random() < 0.6 else int(rng.integers(1, 2000))
    SR = int(rng.integers(1, min(R, 64) + 1))
    SC = int(rng.choice([d for d in range(1, min(C, 64) + 1) if C % d == 0]))
    batch = int(rng.choice([1, 1, 2, 3]))
    k = int(rng.integers(1, min(64, R) + 1))
    T = float(rng.choice([0.0, 0.6, 1.0, 3.0]))
    print(f"[case] f8 sample {R}x{C} scales {SR}x{SC} batch {batch} k {k} T {T}", flush=True)
    case = synth.make_f8(R, C, SR, SC, seed=9600 + j, batch=batch)
    check_f8_sample(case, k, T, [int(v) for v in rng.integers(1, 2**32, batch)])


def _grouped_f8(R, C, rows, seed, tied):
    """Weights zero except on `rows` (codes 1.0-1.875 on the first 16 columns,
    the same codes on every such row if tied), activations positive: the
    large logits sit in chosen rows, all other logits are 0."""
    rng = np.random.default_rng(seed)
    case = synth.make_f8(R, C, 1, 1, seed=seed)
    case.w[:] = 0
    case.scale[:] = 127
    if tied:
        case.w[np.ix_(rows, np.arange(16))] = rng.integers(0x38, 0x40, 16).astype(np.uint8)
    else:
        case.w[np.ix_(rows, np.arange(16))] = rng.integers(0x38, 0x40, (rows.size, 16)).astype(np.uint8)
    case.x[:] = np.abs(case.x) + 0.25
    return case


@pytest.mark.parametrize("tied", [False, True])
@pytest.mark.parametrize("k", [64, 5])
def test_f8_sample_top_rows_crowded_in_few_workgroups(tied, k):
    """524288 rows of 128 columns: workgroup w of the streaming kernel stores
    rows [64 w, 64 w + 64); the large logits fill the workgroups whose index
    is below 4k modulo 1024, so the slots that pass the first bound crowd in
    k sets of 32 (thousands of survivors: the sorted path); tied, the top
    workgroups hold thousands of equal candidates (the sorted path again)."""
    R, C = 524288, 128
    wg = np.arange(R // 64)
    sel = wg[(wg % 1024) < 4 * k]
    rows = (64 * sel[:, None] + np.arange(64)[None, :]).reshape(-1)
    case = _grouped_f8(R, C, rows, seed=31 + k, tied=tied)
    print(f"[case] f8 sample crowded k={k} tied={tied}", flush=True)
    check_f8_sample(case, k, 0.7, [4242 + k])


@pytest.mark.parametrize("C", [4096, 100])
def test_f8_sample_ties_nan_and_inf(C):
    """Every logit 0 (the first k rows, in order), every logit NaN (NaN
    values, the first k rows), +inf in three rows (those first, by row, and
    the token the first since the top value is not finite)."""
    case = synth.make_f8(300, C, 1, 4, seed=94)
    case.w[:] = 0x00
    _, _, ids, vals = check_f8_sample(case, 20, 1.0, [5])
    assert np.array_equal(ids[0], np.arange(20))
    nan_case = synth.make_f8(300, C, 3, 4, seed=95)
    nan_case.x[0, 7] = np.nan
    _, tok, ids, vals = check_f8_sample(nan_case, 7, 1.0, [6])
    assert np.array_equal(ids[0], np.arange(7)) and np.isnan(vals[0]).all()
    inf_case = synth.make_f8(300, C, 3, 4, seed=96)
    inf_case.w[:, 3] = 0x00
    inf_case.w[[40, 17, 250], 3] = 0x38
    inf_case.x[0, 3] = np.inf
    _, tok, ids, _ = check_f8_sample(inf_case, 5, 1.0, [7])
    assert list(ids[0][:3]) == [17, 40, 250] and int(tok[0]) == 17


def test_f8_sample_workspace_reuse_and_batch(cache):
    """One workspace holding garbage, reused: a batch of 3 vectors (a state
    each), then a smaller call, then the first again with the same results."""
    case = synth.make_f8(20000, 4096, 157, 32, seed=97, batch=3)
    small = synth.make_f8(700, 512, 7, 8, seed=98)
    ws = torch.full((bqd.f8_matvec_argmax_workspace_bytes(3),), 0x5A, dtype=torch.uint8, device=DEV)
    a = check_f8_sample(case, 64, 0.9, [11, 22, 33], workspace=ws)
    check_f8_sample(small, 9, 0.9, [44], workspace=ws)
    b = check_f8_sample(case, 64, 0.9, [11, 22, 33], workspace=ws)
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint32) if u.dtype == np.float32 else u,
                              np.asarray(v).view(np.uint32) if v.dtype == np.float32 else v)


def test_f8_wkv(cache):
    check_f8(workload(cache, "f8_wkv_512x4096"))


def oracle_all_rows(fn, R):
    """fn(row_begin, row_count) -> (y, mag) over all R rows, the rows split in
    contiguous chunks over host threads (the oracle's ctypes calls release
    the GIL); each chunk is an unmodified oracle call on its row range."""
    import threading
    n = max(1, min(32, len(os.sched_getaffinity(0))))
    per = (R + n - 1) // n
    chunks = [(a, min(per, R - a)) for a in range(0, R, per)]
    res = [None] * len(chunks)

    def run(i, a, c):
        res[i] = fn(a, c)

    ts = [threading.Thread(target=run, args=(i, a, c)) for i, (a, c) in enumerate(chunks)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return (np.concatenate([r[0] for r in res], axis=-1), np.concatenate([r[1] for r in res], axis=-1))


def test_f8_head_all_rows(cache):
    """The head at full size in the benchmark's launch configuration, every one
    of its 246272 rows against the oracle."""
    case = workload(cache, "f8_head_246272x4096")
    print("[case] f8 head full launch, all rows against the oracle", flush=True)
    w, s, x = dev_f8(case)
    got = bqd.f8_matvec(w, s, x).cpu().numpy()
    ref, mag = oracle_all_rows(lambda a, c: oracle.f8_matvec(
        case.w, case.R, case.C, case.scale, case.SR, case.SC, case.x[0], a, c), case.R)
    assert_tol(got[0], ref, mag, f"f8 head {case.R}x{case.C}, all rows")
    again = bqd.f8_matvec(w, s, x).cpu().numpy()
    assert bits_eq(got, again)


@pytest.mark.parametrize("R,C,SR,SC,batch", [
    (10, 7, 3, 2, 1), (130, 260, 3, 5, 2), (64, 128, 1, 1, 1), (257, 4096, 3, 32, 1),
    (300, 1024, 3, 8, 3), (129, 2048, 2, 16, 1), (77, 8192, 1, 64, 1), (40, 768, 4, 3, 1),
    (33, 128, 33, 8, 1),
    # scale blocks of a whole number of rows that is not a power of two (125): the scale row by
    # multiply and shift, up to row 10^6 on a grid-stride launch
    (12000, 2048, 96, 16, 1), (1000000, 256, 8000, 16, 1),
    # rows wider than the fast kernel's widest lane layout (8192 columns): the generic kernel
    (64, 16384, 2, 64, 2),
    # scale blocks of a multiple of an iteration's aligned rows (U * SLOTS = 64, 32, 8 for 8, 16
    # and 64 lanes per row): one scale read per iteration; 12 rows per block (not a multiple of 8)
    (8192, 128, 64, 8, 1), (4096, 256, 64, 16, 2), (24576, 4096, 96, 32, 1),
    (4800, 4096, 400, 32, 1),
])
def test_f8_shapes(R, C, SR, SC, batch):
    check_f8(synth.make_f8(R, C, SR, SC, seed=R * 7 + C, batch=batch))


def test_f8_one_hot_all_codes():
    """Each of the 256 codes through the fast and the generic kernel: with
    x = e_c the row sum is a single exact product."""
    for C, SC, col in ((4096, 32, 1000), (100, 3, 42)):
        case = synth.make_f8(256, C, 2, SC, seed=3)
        case.w[:, col] = np.arange(256, dtype=np.uint8)
        case.x = np.zeros((1, C), np.float32)
        case.x[0, col] = 1.0
        w, s, x = dev_f8(case)
        got = bqd.f8_matvec(w, s, x).cpu().numpy()[0]
        ref = np.array([oracle.e4m3(r) * math.ldexp(1.0, int(case.scale[(r * 2) // 256,
                        (col * SC) // C]) - 127) for r in range(256)], np.float32)
        assert np.array_equal(got, ref), C


def test_f8_unaligned_weight_pointer():
    case = synth.make_f8(64, 1024, 1, 8, seed=9)
    buf = torch.zeros(64 * 1024 + 16, dtype=torch.uint8, device=DEV)
    buf[3:3 + 64 * 1024] = to_dev(case.w).reshape(-1)
    w = buf[3:3 + 64 * 1024].view(64, 1024)
    got = bqd.f8_matvec(w, to_dev(case.scale), to_dev(case.x)).cpu().numpy()
    ref, mag = oracle.f8_matvec(case.w, 64, 1024, case.scale, 1, 8, case.x)
    assert_tol(got, ref, mag, "unaligned f8")


def test_f8_activation_not_16_byte_aligned():
    """x at a 4-byte (not 16-byte) offset: the fast kernel stages it in LDS one
    float at a time; every lane layout, batch 2 (the second vector 4 bytes
    further on as well)."""
    for R, C, SR, SC in ((256, 4096, 2, 32), (96, 1024, 3, 8), (64, 128, 1, 1), (80, 8192, 5, 64)):
        case = synth.make_f8(R, C, SR, SC, seed=R + C, batch=2)
        buf = torch.zeros(2 * C + 4, dtype=torch.float32, device=DEV)
        buf[1:1 + 2 * C] = to_dev(case.x).reshape(-1)
        x = buf[1:1 + 2 * C].view(2, C)
        assert x.data_ptr() % 16 == 4
        got = bqd.f8_matvec(to_dev(case.w), to_dev(case.scale), x).cpu().numpy()
        ref, mag = oracle.f8_matvec(case.w, R, C, case.scale, SR, SC, case.x)
        assert_tol(got, ref, mag, f"f8 x at +4 bytes {R}x{C}")
        aligned = bqd.f8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(case.x)).cpu().numpy()
        assert bits_eq(got, aligned), (R, C)


# -------------------------------------------------------------- empty calls
# ----------------------------------------------------------------------- I8
I8_CASES = [
    (37, 80, 16, 1), (300, 4096, 16, 1), (100, 2048, 32, 3), (65, 128, 16, 2), (33, 16, 16, 1),
    (17, 8192, 64, 1), (10, 100, 7, 2), (513, 1024, 16, 1), (3, 4096, 4096, 1),
    (40, 16384, 16, 2),
]


@pytest.mark.parametrize("R,C,G,batch", I8_CASES)
def test_i8_matvec_shapes(R, C, G, batch):
    case = synth.make_i8(R, C, G, seed=600 + R, batch=batch)
    got = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(case.x), G).cpu().numpy()
    ref, mag = oracle.i8_matvec(case.w, R, C, case.scale, G, case.x)
    assert_tol(got, ref, mag, f"i8_matvec {R}x{C} G{G} batch {batch}")


def test_i8_matvec_one_hot_all_codes():
    """x = e_c: y[r] = w[r][c] * 2^(s - 127) exactly, every int8 value, through
    the streaming kernel (C = 4096) and the generic one (C = 80)."""
    for C, G in ((4096, 16), (80, 16)):
        case = synth.make_i8(256, C, G, seed=7)
        case.w[:, :] = np.arange(-128, 128, dtype=np.int64).astype(np.int8)[:, None]
        for c in (0, 17, C - 1):
            x = np.zeros((1, C), np.float32)
            x[0, c] = 1.0
            got = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(x), G).cpu().numpy()[0]
            ref, _ = oracle.i8_matvec(case.w, 256, C, case.scale, G, x[0])
            assert np.array_equal(got, ref.astype(np.float32)), (C, c)


def test_i8_matvec_unaligned_weights():
    case = synth.make_i8(40, 4096, 16, seed=8)
    buf = torch.zeros(case.w.size + 1, dtype=torch.int8, device=DEV)
    buf[1:] = to_dev(case.w).reshape(-1)
    got = bqd.i8_matvec(buf[1:].reshape(40, 4096), to_dev(case.scale), to_dev(case.x)).cpu().numpy()
    ref, mag = oracle.i8_matvec(case.w, 40, 4096, case.scale, 16, case.x)
    assert_tol(got, ref, mag, "i8_matvec unaligned")


def test_i8_matvec_activation_not_16_byte_aligned():
    """x 4 bytes off 16-byte alignment: the fast kernel stages it in LDS one
    float at a time; the result equals the aligned call's bit for bit."""
    for R, C, G in ((40, 4096, 16), (33, 1024, 32), (20, 128, 16)):
        case = synth.make_i8(R, C, G, seed=R + C)
        xf = np.ascontiguousarray(case.x, np.float32).reshape(-1)
        buf = torch.zeros(xf.size + 4, dtype=torch.float32, device=DEV)
        buf[1:1 + xf.size] = to_dev(xf)
        x = buf[1:1 + xf.size].view(case.x.shape)
        assert x.data_ptr() % 16 == 4
        got = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), x, G).cpu().numpy()
        ref, mag = oracle.i8_matvec(case.w, R, C, case.scale, G, case.x)
        assert_tol(got, ref, mag, f"i8 x at +4 bytes {R}x{C}")
        aligned = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(case.x), G).cpu().numpy()
        assert bits_eq(got, aligned), (R, C)


def test_i8_head_all_rows(cache):
    """The I8 head at full size in the benchmark's launch configuration, every
    row against the oracle."""
    if "i8_head" not in cache:
        print("[case] building i8 head 246272x4096 G16", flush=True)
        cache["i8_head"] = synth.make_i8(**synth.I8_HEAD, seed=5)
    case = cache["i8_head"]
    got = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(case.x), case.G).cpu().numpy()[0]
    ref, mag = oracle_all_rows(lambda a, c: oracle.i8_matvec(
        case.w, case.R, case.C, case.scale, case.G, case.x[0], a, c), case.R)
    assert_tol(got, ref, mag, f"i8 head {case.R}x{case.C}, all rows")


# ------------------------------------------------------------- int8 key cache
def check_kv_quantize(v):
    v = np.ascontiguousarray(v, np.float32)
    q, sc = bqd.kv_quantize_int8(to_dev(v))
    qr, scr = oracle.store_int8(v)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), np.asarray(scr, np.float32).view(np.uint32))
    return q, sc


def test_kv_quantize_workload():
    case = synth.make_kv(**synth.KV, seed=6)
    check_kv_quantize(case.v)


@pytest.mark.parametrize("d", [1, 63, 64, 65, 300, 4096])
def test_kv_quantize_ragged(d):
    rng = np.random.default_rng(d)
    check_kv_quantize(rng.standard_normal((9, d)).astype(np.float32) * 3)


def test_kv_quantize_special_vectors():
    rows = [np.zeros(16), np.r_[127, 0.5, 1.5, 2.5, -2.5, -63.5, 63.5, -0.5, np.zeros(8)],
            np.r_[1.0, np.nan, -3.0, np.zeros(13)], np.r_[1.0, np.inf, -3.0, np.zeros(13)],
            np.r_[-np.inf, 2.0, np.zeros(14)], np.full(16, 3e-13), np.full(16, -1e30),
            np.r_[-400.0, np.linspace(-1, 1, 15)],
            # v / scale within 1e-9 of 79.5 and 95.5: the fp64 scale gives 79 and
            # 95, the fp32 value the scale array stores would give 80 and 96
            np.r_[1.0, 0.625984251499176, 0.751968502998352, -0.625984251499176, np.zeros(12)]]
    q, _ = check_kv_quantize(np.stack(rows).astype(np.float32))
    assert q[-1, :4].tolist() == [127, 79, 95, -79]


@pytest.mark.parametrize("R,d,batch", [(4096, 128, 1), (300, 64, 2), (77, 100, 1), (40, 4096, 3), (5, 1, 1)])
def test_kv_int8_dot(R, d, batch):
    check_kv_dot(synth.make_kv(R, d, seed=700 + d, batch=batch))


def check_kv_dot(case):
    """The GPU's quantized keys (bit-equal to the oracle's) through the GPU key
    dot, against the oracle's dot on the oracle's own keys."""
    R, d = case.v.shape
    batch = case.x.shape[0]
    q, sc = check_kv_quantize(case.v)
    qr, scr = oracle.store_int8(case.v)
    got = bqd.kv_int8_dot(q, sc, to_dev(case.x)).cpu().numpy().reshape(batch, R)
    for b in range(batch):
        ref, mag = oracle.int8_dot(qr, scr, case.x[b])
        assert_tol(got[b], ref, mag, f"kv_int8_dot {R}x{d} vector {b}")


@pytest.mark.parametrize("k", range(24))
def test_kv_random_shapes(k):
    rng = np.random.default_rng(8000 + k)
    R = int(rng.integers(1, 5000))
    d = int(rng.integers(1, 4200)) if rng.random() < 0.5 else int(rng.choice([64, 128, 256]))
    batch = int(rng.choice([1, 1, 2, 3]))
    print(f"[case] random kv {R}x{d} batch {batch}", flush=True)
    check_kv_dot(synth.make_kv(R, d, seed=8100 + k, batch=batch))


# ------------------------------------------------------------- Hadamard MLP
HMLP_CASES = [(512, 2048, 1, True), (10, 16, 3, True), (48, 64, 2, False), (100, 128, 1, True),
              (200, 256, 2, False), (300, 512, 1, True), (1000, 1024, 1, False),
              (4096, 8192, 1, True), (10000, 16384, 2, True), (1, 1, 2, False), (64, 4096, 1, True)]


@pytest.mark.parametrize("hidden,H,batch,with_u", HMLP_CASES)
def test_hadamard_mlp(hidden, H, batch, with_u):
    check_mlp(synth.make_hmlp(hidden, H, seed=800 + H, batch=batch), H, with_u)


@pytest.mark.parametrize("k", range(24))
def test_hadamard_mlp_random_shapes(k):
    rng = np.random.default_rng(8200 + k)
    H = int(2 ** rng.integers(0, 15))
    hidden = int(rng.integers(1, H + 1))
    batch = int(rng.integers(1, 4))
    with_u = bool(rng.random() < 0.5)
    print(f"[case] random mlp {hidden}/{H} batch {batch} u={with_u}", flush=True)
    check_mlp(synth.make_hmlp(hidden, H, seed=8300 + k, batch=batch), H, with_u)


def check_mlp(case, H, with_u):
    batch, hidden = case.n.shape
    u = to_dev(case.u) if with_u else None
    got = bqd.hadamard_mlp(to_dev(case.n), H, to_dev(case.d1), to_dev(case.d2), to_dev(case.d3),
                           to_dev(case.resid), u).cpu().numpy()
    same = 0
    for b in range(batch):
        ref, mag = oracle.hadamard_mlp(case.n[b], H, case.d1, case.d2, case.d3, case.resid[b],
                                       case.u[b] if with_u else None)
        ratio = np.abs(got[b].astype(np.float64) - ref) / (1e-5 * mag + 1e-6)
        assert ratio.max() <= 1.0, (hidden, H, b, ratio.max())
        same += int(np.sum(got[b].view(np.uint32) == ref.view(np.uint32)))
    print(f"[tol] hadamard_mlp {hidden}/{H}: max ratio {ratio.max():.3g}; "
          f"{same} of {batch * hidden} outputs bit-identical", flush=True)


def test_hadamard_mlp_exact_closed_form():
    """The pin's exact construction on the GPU: integer inputs, d2 = 2^12 sign(z1),
    d3 = 2^-12, so every stage is exact and the result is bit-identical."""
    rng = np.random.default_rng(36)
    hidden, H = 48, 64
    n = rng.integers(-3, 4, hidden).astype(np.float32)
    d1 = rng.choice([-1.0, 1.0, 2.0, 0.5], H).astype(np.float32)
    resid = rng.integers(-8, 9, hidden).astype(np.float32)
    z = np.zeros(H)
    z[:hidden] = n
    z1 = (scipy.linalg.hadamard(H) / math.sqrt(H)) @ (d1.astype(np.float64) * z)
    d2 = (np.where(z1 >= 0, 1.0, -1.0) * 4096.0 * (np.abs(z1) > 0)).astype(np.float32)
    d3 = np.full(H, 2.0 ** -12, np.float32)
    got = bqd.hadamard_mlp(to_dev(n[None]), H, to_dev(d1), to_dev(d2), to_dev(d3),
                           to_dev(resid[None])).cpu().numpy()[0]
    ref, _ = oracle.hadamard_mlp(n, H, d1, d2, d3, resid)
    assert bits_eq(got, ref)


def test_hadamard_mlp_update_rounds_block_first():
    """The pin's construction on the GPU: the block output 1 + 3 * 2^-26 is
    stored as 1 before u = -59 * 2^-26 is subtracted, so the update is
    1 + 7 * 2^-23 (one rounding of the whole sum would give 1 + 2^-20)."""
    f = lambda v: to_dev(np.array([v], np.float32))
    one = f(1.0)
    got = bqd.hadamard_mlp(to_dev(np.array([[1.5]], np.float32)), 1, one, f(64.0), f(2.0 ** -31),
                           to_dev(np.array([[1.0]], np.float32)), to_dev(np.array([[-59 * 2.0 ** -26]], np.float32)))
    assert got.cpu().numpy()[0, 0] == np.float32(1 + 7 * 2.0 ** -23)


def test_hadamard_mlp_scale_rounds_from_fp64():
    """The pin's H = 2 construction on the GPU, 200 inputs at once: the output
    is fl32(fl64(2 v / sqrt 2)) with v = fl32(fl64(x / sqrt 2)), so both
    transforms' scales are fp64 products stored to fp32; bit-identical to the
    oracle (pinned to rationals on the same construction)."""
    x = np.random.default_rng(39).uniform(0.01, 100.0, (200, 1)).astype(np.float32)
    d1, d2, d3 = (np.full(2, v, np.float32) for v in (1.0, 2.0 ** 40, 2.0 ** -40))
    resid = np.zeros((200, 1), np.float32)
    got = bqd.hadamard_mlp(to_dev(x), 2, to_dev(d1), to_dev(d2), to_dev(d3), to_dev(resid)).cpu().numpy()
    ref = np.stack([oracle.hadamard_mlp(x[b], 2, d1, d2, d3, resid[b])[0] for b in range(200)])
    assert bits_eq(got, ref)


# Buffers past 2 GiB: every byte offset the kernels form is 64-bit.  Weights
# of more than 2^31 bytes (F8, I8, and CQ4 at batch 1 and 8 plus its row
# gather), a row range that starts past the mark, and a gather whose output
# passes 2 GiB; checked on the first rows, the rows around the 2^31-byte mark
# and the last rows.
BIG = 1 << 31


def ranges_past_2gib(n_rows, row_bytes):
    mark = BIG // row_bytes
    return [(0, 64), (mark - 64, 128), (n_rows - 64, 64)]


def test_f8_weights_past_2gib():
    R, C, SR, SC = 540000, 4096, 1000, 32
    print(f"[case] f8 {R}x{C}, {R * C} weight bytes", flush=True)
    case = synth.make_f8(R, C, SR, SC, seed=61, wide_bytes=True)
    assert case.w.nbytes > BIG
    check_f8(case, ranges_past_2gib(R, C))


def test_i8_weights_past_2gib():
    R, C, G = 540000, 4096, 16
    print(f"[case] i8 {R}x{C} G{G}, {R * C} weight bytes", flush=True)
    case = synth.make_i8(R, C, G, seed=62, wide_bytes=True)
    assert case.w.nbytes > BIG
    got = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(case.x), G).cpu().numpy()[0]
    for a, c in ranges_past_2gib(R, C):
        ref, mag = oracle.i8_matvec(case.w, R, C, case.scale, G, case.x[0], a, c)
        assert_tol(got[a:a + c], ref, mag, f"i8 {R}x{C} rows [{a}, +{c})")


def test_cq_rows_past_2gib():
    shape = synth.CqShape(1100000, 4096, 4096, 256, 4)
    print(f"[case] cq4 {shape.output}x{shape.input}, {shape.output * shape.stride} packed bytes",
          flush=True)
    case = synth.make_cq(shape, seed=63, batch=8, wide_bytes=True)
    assert case.packed.nbytes > BIG
    m, h = dev_matrix(case), host_matrix(case)
    x = to_dev(case.x)
    p_ref = oracle.cq_prepare(h, case.x)
    p1, y1 = bqd.cq_prepare_matvec(m, x[:1])
    p8, y8 = bqd.cq_prepare_matvec(m, x)
    assert bits_eq(p1.cpu().numpy(), p_ref[:1]) and bits_eq(p8.cpu().numpy(), p_ref)
    y1, y8 = y1.cpu().numpy(), y8.cpu().numpy()
    ranges = ranges_past_2gib(shape.output, shape.stride)
    for a, c in ranges:
        ref, mag = oracle.cq_matvec(h, p_ref, a, c)
        assert_tol(y1[:, a:a + c], ref[:1], mag[:1], f"cq4 batch 1 rows [{a}, +{c})")
        assert_tol(y8[:, a:a + c], ref, mag, f"cq4 batch 8 rows [{a}, +{c})")
    # a row range that starts past the mark, at batch 1 and 8
    a, c = ranges[1][0] + 100, 1000
    ref, mag = oracle.cq_matvec(h, p_ref, a, c)
    yr1 = bqd.cq_matvec(m, p1, row_begin=a, row_count=c).cpu().numpy()
    yr8 = bqd.cq_matvec(m, p8, row_begin=a, row_count=c).cpu().numpy()
    assert_tol(yr1, ref[:1], mag[:1], f"cq4 batch 1 row range [{a}, +{c})")
    assert_tol(yr8, ref, mag, f"cq4 batch 8 row range [{a}, +{c})")
    ids = np.concatenate([np.arange(a, a + c) for a, c in ranges]).astype(np.int32)
    g = bqd.cq_gather_rows(m, to_dev(ids)).cpu().numpy()
    assert bits_eq(g, oracle.cq_gather(h, ids)[0])


def test_gather_output_past_2gib():
    case = synth.make_cq(synth.C3, seed=64)
    s = case.shape
    n = BIG // (4 * s.input) + 4096
    print(f"[case] gather of {n} rows of {s.output}x{s.input}, {4 * n * s.input} output bytes",
          flush=True)
    ids = np.random.default_rng(64).integers(0, s.output, n).astype(np.int32)
    m, h = dev_matrix(case), host_matrix(case)
    g = bqd.cq_gather_rows(m, to_dev(ids))
    assert g.numel() * 4 > BIG
    sel = np.concatenate([np.arange(a, a + c) for a, c in ranges_past_2gib(n, 4 * s.input)])
    got = g[torch.from_numpy(sel).to(DEV)].cpu().numpy()
    assert bits_eq(got, oracle.cq_gather(h, ids[sel])[0])


# Seeded random shapes across the dispatch space: every bit width and group,
# widths up to 16384 with ragged unpadded inputs, rows padded past their
# minimum (odd and aligned), batches 1-9 and random row ranges, so the ring,
# batch-1, 4-vector, matrix-core and generic kernels are all chosen by the
# launch rules rather than by hand; each against the oracle, the fused call
# bit-identical to the two it stands for, and a gather of random ids (one out
# of range).  Then F8 and I8 shapes likewise (row widths of whole 16-byte
# chunks and ragged ones, scale blocks that divide the row and ones that
# do not).
def _random_cq_shape(rng):
    group = int(2 ** rng.integers(2, 11))
    n_groups = int(rng.integers(1, max(2, min(16, 16384 // group) + 1)))
    input_padded = group * n_groups
    cut = int(rng.integers(0, min(group, 38))) if rng.random() < 0.5 else 0
    input_ = max(1, input_padded - cut)
    bits = int(rng.integers(2, 6))
    pad = int(rng.choice([0, 0, 0, 1, 3, 4, 16]))
    row_bytes = synth.min_row_bytes(input_padded, bits) + pad
    output = int(rng.integers(1, 2500))
    return synth.CqShape(output, input_, input_padded, group, bits, row_bytes)


@pytest.mark.parametrize("k", range(120))
def test_cq_random_shapes(k):
    rng = np.random.default_rng(7000 + k)
    shape = _random_cq_shape(rng)
    batch = int(rng.choice([1, 1, 2, 3, 8, 9]))
    rb = int(rng.integers(0, shape.output)) if rng.random() < 0.5 else 0
    rc = int(rng.integers(0, shape.output - rb + 1)) if rng.random() < 0.5 else shape.output - rb
    print(f"[case] random cq {shape} batch {batch} rows [{rb}, +{rc})", flush=True)
    case = synth.make_cq(shape, seed=7100 + k, batch=batch, n_ids=16)
    m, h = dev_matrix(case), host_matrix(case)
    x = to_dev(case.x)
    p, y = bqd.cq_prepare_matvec(m, x, row_begin=rb, row_count=rc)
    p_ref = oracle.cq_prepare(h, case.x)
    assert bits_eq(p.cpu().numpy(), p_ref)
    if rc:
        ref, mag = oracle.cq_matvec(h, p_ref, rb, rc)
        assert_tol(y.cpu().numpy(), ref, mag, f"random cq {shape} batch {batch}")
    y2 = bqd.cq_matvec(m, p, row_begin=rb, row_count=rc)
    assert bits_eq(y.cpu().numpy(), y2.cpu().numpy())
    ids = np.r_[case.ids, np.int32(shape.output)].astype(np.int32)
    g = bqd.cq_gather_rows(m, to_dev(ids)).cpu().numpy()
    g_ref, _ = oracle.cq_gather(h, ids[:-1])
    assert bits_eq(g[:-1], g_ref) and np.isnan(g[-1]).all()


@pytest.mark.parametrize("k", range(60))
def test_f8_random_shapes(k):
    rng = np.random.default_rng(7500 + k)
    R = int(rng.integers(1, 3000))
    C = int(16 * rng.integers(1, 513)) if rng.random() < 0.6 else int(rng.integers(1, 3000))
    SR = int(rng.integers(1, min(R, 64) + 1))
    SC = int(rng.choice([d for d in range(1, min(C, 64) + 1) if C % d == 0])) if rng.random() < 0.6 \
        else int(rng.integers(1, min(C, 64) + 1))
    batch = int(rng.choice([1, 1, 2]))
    print(f"[case] random f8 {R}x{C} scales {SR}x{SC} batch {batch}", flush=True)
    check_f8(synth.make_f8(R, C, SR, SC, seed=7600 + k, batch=batch))


@pytest.mark.parametrize("k", range(40))
def test_i8_random_shapes(k):
    rng = np.random.default_rng(7800 + k)
    R = int(rng.integers(1, 3000))
    C = int(16 * rng.integers(1, 513)) if rng.random() < 0.6 else int(rng.integers(1, 3000))
    G = int(16 * rng.integers(1, max(2, min(C // 16, 8) + 1))) if rng.random() < 0.6 and C >= 16 \
        else int(rng.integers(1, min(C, 100) + 1))
    batch = int(rng.choice([1, 1, 2]))
    print(f"[case] random i8 {R}x{C} G{G} batch {batch}", flush=True)
    case = synth.make_i8(R, C, G, seed=7900 + k, batch=batch)
    got = bqd.i8_matvec(to_dev(case.w), to_dev(case.scale), to_dev(case.x), G).cpu().numpy()
    ref, mag = oracle.i8_matvec(case.w, R, C, case.scale, G, case.x)
    assert_tol(got, ref, mag, f"random i8 {R}x{C} G{G} batch {batch}")


# Launches that would pass 2^32 work-items (one dispatch's limit): the kernels
# that take one wavefront or workgroup per unit of work cap their grids and
# loop (the KV quantize, the Hadamard MLP, the prepare and the gather of
# groups under 8, each at 2^26 + 7 units), and the batch-1 ring kernel splits
# a 512-column matrix of 2^29 + 1000 rows (137 GB packed) into launches of at
# most 2^22 - 1 workgroups.  Inputs are drawn on the device; the first,
# middle and last units are checked against the oracle.
HUGE_UNITS = (1 << 26) + 7


def _sampled_units(n):
    sel = np.r_[np.arange(0, 8), np.arange(n // 2 - 4, n // 2 + 4), np.arange(n - 8, n)]
    return sel, torch.from_numpy(sel).to(DEV)


def test_kv_quantize_past_2_32_work_items():
    print(f"[case] kv quantize of {HUGE_UNITS} vectors of 3", flush=True)
    v = synth.device_normal(torch, (HUGE_UNITS, 3), seed=71, device=DEV, scale=3.0)
    q, sc = bqd.kv_quantize_int8(v)
    sel, idx = _sampled_units(HUGE_UNITS)
    qr, scr = oracle.store_int8(v[idx].cpu().numpy())
    assert np.array_equal(q[idx].cpu().numpy(), qr)
    assert bits_eq(sc[idx].cpu().numpy(), scr)


def test_hadamard_mlp_past_2_32_work_items():
    hidden, H = 3, 4
    print(f"[case] hadamard mlp {hidden}/{H} on {HUGE_UNITS} vectors", flush=True)
    rng = np.random.default_rng(72)
    d1, d2, d3 = (rng.standard_normal(H).astype(np.float32) for _ in range(3))
    n = synth.device_normal(torch, (HUGE_UNITS, hidden), seed=73, device=DEV)
    resid = synth.device_normal(torch, (HUGE_UNITS, hidden), seed=74, device=DEV)
    out = bqd.hadamard_mlp(n, H, to_dev(d1), to_dev(d2), to_dev(d3), resid)
    sel, idx = _sampled_units(HUGE_UNITS)
    got, ns, rs = (t[idx].cpu().numpy() for t in (out, n, resid))
    for b in range(len(sel)):
        ref, mag = oracle.hadamard_mlp(ns[b], H, d1, d2, d3, rs[b])
        ratio = np.abs(got[b].astype(np.float64) - ref) / (1e-5 * mag + 1e-6)
        assert ratio.max() <= 1.0, (sel[b], ratio.max())


def test_prepare_past_2_32_work_items():
    case = synth.make_cq(synth.CqShape(4, 32, 32, 32, 4), seed=75)
    print(f"[case] prepare of {HUGE_UNITS} vectors of 32", flush=True)
    m, h = dev_matrix(case), host_matrix(case)
    x = synth.device_normal(torch, (HUGE_UNITS, 32), seed=76, device=DEV)
    p = bqd.cq_prepare(m, x)
    sel, idx = _sampled_units(HUGE_UNITS)
    assert bits_eq(p[idx].cpu().numpy(), oracle.cq_prepare(h, x[idx].cpu().numpy()))


def test_gather_small_groups_past_2_32_work_items():
    case = synth.make_cq(synth.CqShape(1000, 4, 4, 4, 2), seed=77)
    print(f"[case] gather of {HUGE_UNITS} rows of 4 (groups of 4)", flush=True)
    m, h = dev_matrix(case), host_matrix(case)
    ids = synth.device_ids(torch, HUGE_UNITS, 1000, seed=78, device=DEV)
    g = bqd.cq_gather_rows(m, ids)
    sel, idx = _sampled_units(HUGE_UNITS)
    assert bits_eq(g[idx].cpu().numpy(), oracle.cq_gather(h, ids[idx].cpu().numpy())[0])


def test_ring_launch_past_2_32_work_items():
    rows, C = (1 << 29) + 1000, 512
    shape = synth.CqShape(rows, C, C, 128, 4)
    need = rows * (shape.stride + 2 * shape.n_groups + 4)
    if torch.cuda.get_device_properties(0).total_memory < need + (16 << 30):
        pytest.skip(f"needs {need >> 30} GiB of device memory")
    print(f"[case] ring matvec of CQ4 {rows}x{C}, {rows * shape.stride} packed bytes", flush=True)
    packed = synth.device_bytes(torch, rows * shape.stride, seed=79, device=DEV).view(rows, -1)
    norms = synth.device_norms(torch, (rows, shape.n_groups), seed=80, device=DEV)
    cb = synth.codebook(4)
    m = bqd.CqMatrix(packed, norms, to_dev(cb), output=rows, input=C, input_padded=C, group=128,
                     bits=4, row_bytes=shape.stride)
    x = np.random.default_rng(81).standard_normal((1, C)).astype(np.float32)
    p, y = bqd.cq_prepare_matvec(m, to_dev(x))
    y2 = bqd.cq_matvec(m, p)
    chunk = ((1 << 32) // 1024 - 1) * 128  # rows of one launch
    for a, c in ((0, 64), (chunk - 64, 128), (rows - 64, 64)):
        hs = oracle.CqMatrix(c, C, C, 128, 4, shape.stride, packed[a:a + c].cpu().numpy(),
                             norms[a:a + c].cpu().numpy(), cb)
        p_ref = oracle.cq_prepare(hs, x)
        assert bits_eq(p.cpu().numpy(), p_ref)
        ref, mag = oracle.cq_matvec(hs, p_ref)
        assert_tol(y[:, a:a + c].cpu().numpy(), ref, mag, f"ring rows [{a}, +{c})")
        assert bits_eq(y2[:, a:a + c].cpu().numpy(), y[:, a:a + c].cpu().numpy())
    del packed, norms, m, y, y2
    torch.cuda.empty_cache()


def test_binding_rejects_buffers_smaller_than_their_shapes():
    """The C ABI sees addresses only; the binding checks every buffer against
    the shape fields before any launch."""
    case = synth.make_cq(synth.CqShape(10, 512, 512, 128, 4), seed=3)
    m = dev_matrix(case)
    kw = dict(output=10, input=512, input_padded=512, group=128, bits=4, row_bytes=256)
    with pytest.raises(ValueError):
        bqd.CqMatrix(m.packed.reshape(-1)[:-1], m.norms, m.codebook, **kw)
    with pytest.raises(ValueError):
        bqd.CqMatrix(m.packed, m.norms.reshape(-1)[:-1], m.codebook, **kw)
    with pytest.raises(ValueError):
        bqd.CqMatrix(m.packed, m.norms, m.codebook[:15], **kw)
    p = torch.zeros(511, device=DEV)
    with pytest.raises(ValueError):
        bqd.cq_matvec_multi([m, m], p)
    with pytest.raises(ValueError):
        bqd.cq_prepare_matvec_multi([m, m], torch.zeros(500, device=DEV))
    with pytest.raises(ValueError):
        bqd.cq_prepare_matvec_multi([m, m], torch.zeros(512, device=DEV), prepared=p)
    logits = torch.zeros(100, device=DEV)
    no_state = torch.zeros(0, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        bqd.logits_sample(logits, 4, 1.0, no_state)
    with pytest.raises(ValueError):
        bqd.logits_sample_noalloc(logits, 4, 1.0, no_state, torch.zeros(1, dtype=torch.int32, device=DEV),
                                  torch.zeros(4, dtype=torch.int32, device=DEV),
                                  torch.zeros(4, device=DEV))


def test_empty_problems_are_no_ops():
    case = small_case(0)
    m = dev_matrix(case)
    s = case.shape
    y = torch.full((1, 0), 7.0, device=DEV)
    bqd.cq_matvec(m, torch.zeros(1, s.input_padded, device=DEV), row_begin=s.output, row_count=0, out=y)
    out = bqd.cq_gather_rows(m, torch.zeros(0, dtype=torch.int32, device=DEV))
    assert out.shape == (0, s.input)
    p = bqd.cq_prepare(m, torch.zeros(0, s.input, device=DEV))
    assert p.shape == (0, s.input_padded)
    yf = bqd.f8_matvec(torch.zeros(0, 16, dtype=torch.uint8, device=DEV),
                       torch.full((1, 1), 127, dtype=torch.uint8, device=DEV),
                       torch.zeros(1, 16, device=DEV))
    assert yf.shape == (1, 0)
    torch.cuda.synchronize()


# ------------------------------------------------------------- graph replay
def test_graph_replay_matches_eager_beyond_the_path(cache):
    """The entry points beyond the five workloads captured in one HIP graph:
    the fused prepare + matvec, several matrices in one launch, the I8 matvec,
    storeInt8 and the key dot, the Hadamard MLP, the sampler, the F8 matvec
    with its fused argmax and with its fused top-k sampling.  Every replay, with eager fills and
    synchronizations between replays, equals the eager result bitwise; the
    samplers' states are reset before each replay and then hold the eager
    states after one draw; the fused kernels' workspaces are filled with
    garbage before each replay (nothing in them needs clearing)."""
    c4 = workload(cache, "cq4_16384x4096_b8")
    m4 = dev_matrix(c4)
    x1 = to_dev(c4.x[:1])
    shapes = [synth.CqShape(2048, 512, 512, 128, 4), synth.CqShape(300, 512, 512, 128, 4)]
    cases = [synth.make_cq(sh, seed=880 + k) for k, sh in enumerate(shapes)]
    ms = [dev_matrix(c) for c in cases]
    xm = to_dev(cases[0].x[0])
    i8 = synth.make_i8(300, 4096, 16, seed=881)
    w8, s8, x8 = to_dev(i8.w), to_dev(i8.scale), to_dev(i8.x)
    kv = synth.make_kv(1000, 128, seed=882)
    v, xq = to_dev(kv.v), to_dev(kv.x)
    hm = synth.make_hmlp(512, 2048, seed=883)
    hn, d1, d2, d3, hr, hu = (to_dev(a) for a in (hm.n, hm.d1, hm.d2, hm.d3, hm.resid, hm.u))
    logits = to_dev(_logits("normal", 50000, 884))
    fa = synth.make_f8(512, 4096, 4, 32, seed=885)
    wa, sa, xa = dev_f8(fa)
    aws = torch.empty(bqd.f8_matvec_argmax_workspace_bytes(1), dtype=torch.uint8, device=DEV)
    ya = torch.empty(1, fa.R, device=DEV)
    ta = torch.empty(1, dtype=torch.int32, device=DEV)
    seed = 0x1234567
    state = _state_tensor(seed)
    ws = torch.empty(bqd.logits_sample_workspace_bytes(50000, 16), dtype=torch.uint8, device=DEV)
    p1 = torch.empty(1, c4.shape.input_padded, device=DEV)
    y1 = torch.empty(1, c4.shape.output, device=DEV)
    pm = torch.empty(512, device=DEV)
    ym = [torch.empty(sh.output, device=DEV) for sh in shapes]
    yi = torch.empty(1, i8.R, device=DEV)
    q = torch.empty(1000, 128, dtype=torch.int8, device=DEV)
    qs = torch.empty(1000, device=DEV)
    yk = torch.empty(1, 1000, device=DEV)
    ho = torch.empty_like(hn)
    sampled = []
    ff = synth.make_f8(70000, 4096, 70, 32, seed=886)
    wf, sf, xf = dev_f8(ff)
    fws = torch.empty(bqd.f8_matvec_argmax_workspace_bytes(1), dtype=torch.uint8, device=DEV)
    yf = torch.empty(1, ff.R, device=DEV)
    fseed = 0x7654321
    fstate = _state_tensor(fseed)
    fused = []

    def work():
        bqd.cq_prepare_matvec(m4, x1, prepared=p1, out=y1)
        bqd.cq_prepare_matvec_multi(ms, xm, prepared=pm, outs=ym)
        bqd.i8_matvec(w8, s8, x8, G=16, out=yi)
        bqd.kv_quantize_int8(v, q=q, scales=qs)
        bqd.kv_int8_dot(q, qs, xq, out=yk)
        bqd.hadamard_mlp(hn, 2048, d1, d2, d3, hr, hu, out=ho)
        sampled.append(bqd.logits_sample(logits, 16, 0.9, state, ws))
        bqd.f8_matvec_argmax(wa, sa, xa, workspace=aws, out=ya, token=ta)
        fused.append(bqd.f8_matvec_sample(wf, sf, xf, 24, 0.7, fstate, workspace=fws, out=yf)[1:])

    outs = lambda: [p1, y1, pm, *ym, yi, q, qs, yk, ho, ya, ta, yf]
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs()]
    ref_draw = [t.clone() for t in sampled[-1]]
    ref_fused = [t.clone() for t in fused[-1]]
    ref_state = state.clone()
    ref_fstate = fstate.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    draw = sampled[-1]
    fdraw = fused[-1]
    for _ in range(4):
        for t in outs() + list(draw) + list(fdraw):
            t.fill_(-1)
        aws.fill_(0xA5)
        fws.fill_(0x5A)
        state.copy_(_state_tensor(seed))
        fstate.copy_(_state_tensor(fseed))
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs(), ref):
            assert torch.equal(t, r)
        for t, r in zip(draw, ref_draw):
            assert torch.equal(t, r)
        for t, r in zip(fdraw, ref_fused):
            assert torch.equal(t, r)
        assert torch.equal(state, ref_state)
        assert torch.equal(fstate, ref_fstate)


def test_graph_replay_matches_eager(cache):
    """The path captured in a HIP graph: every replay, with eager work and
    synchronizations between replays, equals the eager result bitwise."""
    c4 = workload(cache, "cq4_16384x4096_b8")
    c3 = workload(cache, "cq4_65536x512_vocab_gather")
    f = workload(cache, "f8_wkv_512x4096")
    m4, m3 = dev_matrix(c4), dev_matrix(c3)
    x8, ids = to_dev(c4.x), to_dev(c3.ids)
    w, s, x = dev_f8(f)
    p = torch.empty(8, c4.shape.input_padded, device=DEV)
    y = torch.empty(8, c4.shape.output, device=DEV)
    y1 = torch.empty(1, c4.shape.output, device=DEV)
    g_out = torch.empty(len(c3.ids), c3.shape.input, device=DEV)
    yf = torch.empty(1, f.R, device=DEV)

    def work():
        bqd.cq_prepare(m4, x8, out=p)
        bqd.cq_matvec(m4, p, out=y)
        bqd.cq_matvec(m4, p[:1], out=y1)
        bqd.cq_gather_rows(m3, ids, out=g_out)
        bqd.f8_matvec(w, s, x, out=yf)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (p, y, y1, g_out, yf)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for _ in range(4):
        for t in (p, y, y1, g_out, yf):
            t.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip((p, y, y1, g_out, yf), ref):
            assert torch.equal(t, r)
        work()  # eager work between replays
        torch.cuda.synchronize()



# ------------------------------------------------------------------ sampling
def _state_tensor(seed):
    return torch.tensor([int(np.array([seed], np.uint32).view(np.int32)[0])], dtype=torch.int32,
                        device=DEV)


def _near_cdf_boundary(vals, T, u, tol=1e-12):
    """True if u * S lies within tol * S of a running sum of the softmax
    weights: there two fp64 exp() implementations may pick neighbours."""
    v = vals.astype(np.float64)
    w = np.where(np.isnan(v), 0.0, np.exp((v - v[0]) / T))
    S = w.sum()
    return bool(np.any(np.abs(np.cumsum(w) - u * S) <= tol * S))


def check_sample(logits, k, T, seed, calls=1):
    x = to_dev(np.ascontiguousarray(logits, dtype=np.float32))
    state = _state_tensor(seed)
    s = seed
    ref_ids, ref_vals = oracle.topk(logits, k)
    for _ in range(calls):
        tok, ids, vals = bqd.logits_sample(x, k, T, state)
        ids, vals = ids.cpu().numpy(), vals.cpu().numpy()
        assert np.array_equal(ids, ref_ids), (k, ids[:8], ref_ids[:8])
        assert bits_eq(vals, ref_vals)
        ref_tok, s = oracle.sample(ref_vals, ref_ids, T, s)
        assert int(state.cpu().numpy().view(np.uint32)[0]) == s
        got = int(tok.item())
        if got != ref_tok:  # only where the draw sits on a CDF boundary
            print(f"[boundary] token {got} vs {ref_tok} at u = {s / 2**32!r}", flush=True)
            assert T > 0 and _near_cdf_boundary(ref_vals, T, s / 2**32), (got, ref_tok)


def _logits(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return (3.0 * rng.standard_normal(n)).astype(np.float32)
    if kind == "ties":
        return rng.integers(-3, 4, n).astype(np.float32)
    x = rng.standard_normal(n).astype(np.float32)
    sp = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0], np.float32)
    x[rng.integers(0, n, max(1, n // 50))] = sp[rng.integers(0, 5, max(1, n // 50))]
    return x


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("k,T", [(1, 1.0), (8, 0.0), (8, 0.7), (64, 1.0), (64, 2.5)])
def test_sample_head_sized(kind, k, T):
    """Logits of the F8 head's size (246272): top-k bit-exact, the state and
    the token equal to the oracle's over chained draws."""
    check_sample(_logits(kind, 246272, 90 + k), k, T, seed=0x9E3779B9 + k, calls=4)


# Ragged tails and sizes around the first stage's block counts.
@pytest.mark.parametrize("n,k", [(1, 1), (5, 5), (64, 64), (1023, 5), (1025, 64), (4095, 7),
                                 (4096, 64), (4097, 64), (8191, 3), (32768, 64), (32769, 64),
                                 (65536, 2), (65536 + 17, 33), (131073, 17), (256 * 1024, 64),
                                 (256 * 1024 + 1, 9), (512 * 1024 + 1, 64), (1 << 20, 64)])
def test_sample_ragged_sizes(n, k):
    check_sample(_logits("normal", n, n), k, 0.8, seed=12345 + n)
    check_sample(_logits("ties", n, n + 1), k, 1.3, seed=777 + n)


@pytest.mark.parametrize("n", [246272, 1 << 20])
def test_sample_top_keys_crowded_in_one_block(n):
    """The best 512 logits are the first 512 (a ladder rising with the
    index), so one first-stage block holds all of the top k: the second stage
    finds a list whose first 8 keys all pass its bound and merges every list
    in full."""
    x = _logits("normal", n, n + 5)
    x[:512] = (1000 + np.arange(512)).astype(np.float32)
    check_sample(x, 64, 0.9, seed=31 + n)
    check_sample(x, 40, 0.0, seed=32 + n)


@pytest.mark.parametrize("n,k", [(40, 40), (246272, 64)])
def test_sample_zeros_and_nans_in_top_k(n, k):
    """Zeros of both signs at the top and NaNs (with payloads) inside the k:
    the values whose keys drop the sign or the payload come back bit for bit."""
    rng = np.random.default_rng(n)
    x = -np.abs(rng.standard_normal(n)).astype(np.float32) - np.float32(0.5)
    pos = rng.choice(n, 30 if n > 64 else 12, replace=False)
    x[pos[:len(pos) // 2]] = np.float32(-0.0)
    x[pos[len(pos) // 2:]] = np.float32(0.0)
    if n <= k:  # every logit is a candidate: NaNs with distinct payloads rank last
        nan_bits = np.array([0x7fc00001, 0xffc00002, 0x7f800003, 0x7fffffff], np.uint32)
        x[rng.choice(np.setdiff1d(np.arange(n), pos), 4, replace=False)] = nan_bits.view(np.float32)
    check_sample(x, k, 0.9, seed=4242 + n)
    check_sample(x, k, 0.0, seed=99 + n)


def test_sample_draw_scale_decides():
    """The draw is u = state / 2^32 exactly: state 0x88004000 steps to 2^31
    (u = 1/2), and two logits 1 and 1 - 2^-24 at T = 1000 put the CDF
    boundary at u = 1/2 + 1.49e-11, so the larger logit is drawn; a state
    scaled by 1 / (2^32 - 1) would give 1/2 + 1.16e-10 and the other one."""
    one, below = np.float32(1.0), np.nextafter(np.float32(1.0), np.float32(0.0))
    for logits, want in (([one, below], 0), ([below, one], 1)):
        state = _state_tensor(0x88004000)
        tok, _, _ = bqd.logits_sample(to_dev(np.array(logits, np.float32)), 2, 1000.0, state)
        assert int(state.cpu().numpy().view(np.uint32)[0]) == 1 << 31
        assert int(tok.item()) == want
        ref_ids, ref_vals = oracle.topk(np.array(logits, np.float32), 2)
        assert oracle.sample(ref_vals, ref_ids, 1000.0, 0x88004000) == (want, 1 << 31)


@pytest.mark.parametrize("k", range(30))
def test_sample_random(k):
    rng = np.random.default_rng(8400 + k)
    n = int(rng.integers(1, (1 << 20) + 1)) if rng.random() < 0.7 else int(rng.integers(1, 5000))
    kk = int(rng.integers(1, min(64, n) + 1))
    T = 0.0 if rng.random() < 0.2 else float(rng.uniform(0.05, 3.0))
    kind = str(rng.choice(["normal", "ties", "special"]))
    print(f"[case] random sample n={n} k={kk} T={T:.3f} {kind}", flush=True)
    check_sample(_logits(kind, n, 8500 + k), kk, T, seed=8600 + k, calls=2)


def test_sample_chain_of_twenty():
    """Twenty draws on one device state continue the oracle's sequence."""
    check_sample(_logits("normal", 50000, 5), 16, 1.0, seed=1, calls=20)

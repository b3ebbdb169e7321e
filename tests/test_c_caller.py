"""The C ABI from C.

CPU: include/bqd.h compiles on its own as strict C99 and C11, and a plain C
program (tests/c_abi/caller.c, which includes only bqd.h and the HIP runtime
API) builds and links against libbqd.so.
GPU: that program, run as a child process on seeded inputs, returns what the
oracle computes: the prepared vector, the gathered rows and the top-k bit for
bit, the CQ and F8 matvecs within 1e-4 * sum|w*x| + 1e-6, the sampled
token and advanced state of the oracle's draw, from f8_matvec_argmax the
F8 matvec's y bit for bit with the first of its largest rows as the token,
and from f8_matvec_sample that y again with its k best rows (value, then
row) and their values bit for bit, the state one xorshift step on and a
token among those rows.
"""
import os
import subprocess

import numpy as np
import pytest

import bit_quantized_decode_amd as bqd
import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
STRICT = ["-Wall", "-Wextra", "-Werror", "-pedantic"]


def _build_caller(tmp_path):
    exe = tmp_path / "caller"
    libdir = os.path.dirname(bqd.LIB_PATH)
    cmd = ["gcc", "-std=c11", *STRICT, "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", INCLUDE,
           os.path.join(HERE, "c_abi", "caller.c"), "-o", str(exe),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", libdir, "-lbqd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_is_plain_c(tmp_path, std):
    src = tmp_path / "h.c"
    src.write_text('#include "bqd.h"\nint main(void) { return BQD_OK; }\n')
    r = subprocess.run(["gcc", f"-std={std}", *STRICT, "-I", INCLUDE, str(src), "-o",
                        str(tmp_path / "h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_caller_builds(tmp_path):
    assert os.path.exists(bqd.LIB_PATH), "libbqd.so is not built"
    _build_caller(tmp_path)


@pytest.mark.gpu
def test_c_caller_matches_oracle(tmp_path):
    exe = _build_caller(tmp_path)
    cq = synth.make_cq(synth.CqShape(300, 2000, 2048, 256, 4), seed=91, n_ids=37)
    s = cq.shape
    f8 = synth.make_f8(512, 4096, 4, 32, seed=92)
    logits = synth.make_logits(50000, seed=93)
    k, state0 = 16, 2024
    (tmp_path / "shape.txt").write_text(
        f"{s.output} {s.input} {s.input_padded} {s.group} {s.bits} {s.stride} {cq.ids.size} "
        f"{f8.R} {f8.C} {f8.SR} {f8.SC} {logits.size} {k}\n")
    files = {"packed.bin": cq.packed, "norms.bin": cq.norms.view(np.uint16),
             "codebook.bin": cq.codebook.astype(np.float32), "x.bin": cq.x[0],
             "ids.bin": cq.ids.astype(np.int32), "f8_w.bin": f8.w, "f8_s.bin": f8.scale,
             "f8_x.bin": f8.x[0], "logits.bin": logits, "state.bin": np.array([state0], np.uint32)}
    for name, a in files.items():
        np.ascontiguousarray(a).tofile(tmp_path / name)
    print("[case] C caller: cq_prepare_matvec, cq_gather_rows, f8_matvec, logits_sample, "
          "f8_matvec_argmax, f8_matvec_sample", flush=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = lambda name, dt: np.fromfile(tmp_path / name, dtype=dt)

    h = oracle.CqMatrix.from_case(cq)
    p_ref = oracle.cq_prepare(h, cq.x[0])
    assert np.array_equal(got("prepared.bin", np.uint32), p_ref.view(np.uint32))
    y_ref, mag = oracle.cq_matvec(h, p_ref)
    assert np.all(np.abs(got("y.bin", np.float32) - y_ref) <= 1e-4 * mag + 1e-6)
    g_ref, _ = oracle.cq_gather(h, cq.ids)
    assert np.array_equal(got("gathered.bin", np.uint32), g_ref.reshape(-1).view(np.uint32))
    fy_ref, fmag = oracle.f8_matvec(f8.w, f8.R, f8.C, f8.scale, f8.SR, f8.SC, f8.x[0])
    assert np.all(np.abs(got("f8_y.bin", np.float32) - fy_ref) <= 1e-4 * fmag + 1e-6)
    oid, oval = oracle.topk(logits, k)
    assert np.array_equal(got("topk_ids.bin", np.int32), oid)
    assert np.array_equal(got("topk_logits.bin", np.uint32), oval.view(np.uint32))
    tok, s1 = oracle.sample(oval, oid, 0.8, state0)
    assert int(got("state_out.bin", np.uint32)[0]) == s1
    assert int(got("token.bin", np.int32)[0]) == tok
    fy = got("f8_y.bin", np.float32)
    assert not np.isnan(fy).any()
    assert np.array_equal(got("argmax_y.bin", np.uint32), fy.view(np.uint32))
    assert int(got("argmax_token.bin", np.int32)[0]) == int(np.argmax(fy))
    assert np.array_equal(got("sample_y.bin", np.uint32), fy.view(np.uint32))
    want = np.lexsort((np.arange(fy.size), -fy.astype(np.float64)))[:k]
    sids = got("sample_ids.bin", np.int32)
    assert np.array_equal(sids, want)
    assert np.array_equal(got("sample_logits.bin", np.uint32), fy[want].view(np.uint32))
    assert int(got("sample_state_out.bin", np.uint32)[0]) == s1
    assert int(got("sample_token.bin", np.int32)[0]) in set(want.tolist())

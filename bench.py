#!/usr/bin/env python3
"""Throughput of one decode step over the quantized matvec hot path (1 GPU).

One step runs every stage of the path at the workloads' full sizes:
  1. CQ 4-bit 16384 x 4096 (group 256): prepare + matvec of one vector, one
     launch (cq_prepare_matvec)
  2. the same matrix, 8 activation vectors: prepare, then matvec
  3. CQ 4-bit 65536 x 512 vocabulary table (group 128): the vocabulary
     projection of one vector (cq_prepare_matvec) and a dense gather of 4096
     rows
  4. FP8 E4M3 head 246272 x 4096 with E8M0 128 x 128 block scales: matvec
Inputs are seeded synthetic arrays (synth.py) resident in HBM before timing.
Weights rotate over enough copies that every step reads bytes that are not in
the 256 MB Infinity Cache ("cold").  The value is the step's algorithmic HBM
bytes (weights, activations in, outputs out) over the step time.

Every stage is also timed on its own, with the workloads' small configs and
neighbouring formats as extras; then W warmup steps and exactly K timed steps;
then each stage's outputs from the last timed step are checked against the
CPU oracle (sampled rows; the prepared vector and the gathered rows bit for
bit) and the verdict goes into the JSON line.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
# Host cores granted to a job on one GPU (the affinity mask may show more).
CPU_SHARE = 16
HEAD_STAGE = "f8_head_246272x4096_matvec"
STAGE_LAUNCHES = 16  # back-to-back launches per timed stage graph
METRIC = "weight-stream GB/s & % of HBM peak, CQ/F8 decode matvec; rows/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "f8_head_246272x4096_hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_quantized_decode_amd", "csrc", f) for f in ("f8.hip", "device.h")]


def measured_traffic():
    """HBM bytes per head launch from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE scaled by a plain 1 GiB copy), or None if the kernel sources
    changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()[:16]
    return rec["traffic_bytes"] if rec.get("source_sha256_16") == h else None


# CQ stages with an HBM traffic record: the kernel that runs them (a
# substring of its name in the counter output), the workload, and the bytes
# the method must move per launch (weights, activations and ids in; outputs).
STAGE_TRAFFIC = {
    "cq4_16384x4096_prepare_matvec_b1": dict(
        kernel="cq_matvec_ring", workload="cq4_16384x4096_b1",
        what="CQ4 16384 x 4096 (group 256), one vector, prepare fused",
        reads=16384 * 2048 + 16384 * 16 * 2 + 4 * 4096, writes=4 * 4096 + 4 * 16384),
    "cq4_16384x4096_matvec_b8": dict(
        kernel="cq_matvec_mfma4", workload="cq4_16384x4096_b8",
        what="CQ4 16384 x 4096 (group 256), eight prepared vectors",
        reads=16384 * 2048 + 16384 * 16 * 2 + 8 * 4 * 4096, writes=8 * 4 * 16384),
    "cq4_65536x512_prepare_matvec_b1": dict(
        kernel="cq_matvec_ring", workload="cq4_65536x512_b1",
        what="CQ4 65536 x 512 (group 128) vocabulary projection, one vector, prepare fused",
        reads=65536 * 256 + 65536 * 4 * 2 + 4 * 512, writes=4 * 512 + 4 * 65536),
    "cq4_65536x512_gather_4096": dict(
        kernel="cq_gather_kernel", workload="cq4_65536x512_gather_4096",
        what="4096 rows of CQ4 65536 x 512 (group 128) gathered dense",
        reads=4096 * (256 + 8) + 4 * 4096, writes=4 * 4096 * 512),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="0: the affinity mask, at most the 16 cores of one GPU's share")
    ap.add_argument("--hot", action="store_true", help="one weight copy (cache-resident timing)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two --traffic-probe counter runs into the traffic record "
                         "under profiles/ (no GPU needed); with --stage, a stage's record")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for counter runs: 8 F8 head launches (with --stage: 4 replays of the "
                         "stage's graph of 16 launches), then 8 plain 1 GiB device copies")
    ap.add_argument("--stage", choices=sorted(STAGE_TRAFFIC),
                    help="the CQ stage of --traffic-probe / --traffic-record")
    ap.add_argument("--stage-probe", metavar="STAGE",
                    help="for counter runs: 4 replays of one stage's graph of 16 launches "
                         "(a step stage or an extra, by its name in the JSON line)")
    return ap.parse_args()


class Case:
    """One stage of the step: a callable per weight copy plus its byte count."""

    def __init__(self, name, calls, nbytes, rows):
        self.name, self.calls, self.nbytes, self.rows = name, calls, nbytes, rows
        self.ms = []


def build_cases(torch, bqd, synth, hot, heads=True):
    """The step's stages and the extras; heads=False leaves out the two
    1 GB heads (F8 and I8) and the sampler's logits, for counter probes of
    the CQ stages."""
    dev = "cuda"
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cases = []

    # -- CQ 4-bit 16384 x 4096, batch 1 and batch 8 (one matrix, rotated copies)
    log("generating CQ4 16384x4096 (seed 3)")
    c4 = synth.make_cq(synth.C4, seed=3, batch=8)
    s4 = c4.shape
    k4 = 1 if hot else 16
    packed4, norms4 = T(c4.packed), T(c4.norms.view(np.int16))
    cb4 = T(c4.codebook)
    mats4 = []
    for k in range(k4):
        pk, nm = (packed4, norms4) if k == 0 else (packed4.clone(), norms4.clone())
        mats4.append(bqd.CqMatrix(pk, nm, cb4, output=s4.output, input=s4.input,
                                  input_padded=s4.input_padded, group=s4.group, bits=s4.bits))
    x1, x8 = T(c4.x[:1]), T(c4.x)
    p1 = torch.empty(1, s4.input_padded, device=dev)
    p8 = torch.empty(8, s4.input_padded, device=dev)
    y1 = torch.empty(1, s4.output, device=dev)
    y8 = torch.empty(8, s4.output, device=dev)
    w4 = s4.output * s4.stride + s4.output * s4.n_groups * 2
    # batch 1: x in, the prepared vector and y out, in one launch
    cases.append(Case("cq4_16384x4096_prepare_matvec_b1",
                      [lambda m=m: bqd.cq_prepare_matvec(m, x1, prepared=p1, out=y1) for m in mats4],
                      w4 + 4 * s4.input + 4 * s4.input_padded + 4 * s4.output, s4.output))
    extras = [Case("cq4_16384x4096_matvec_b1",
                   [lambda m=m: bqd.cq_matvec(m, p1, out=y1) for m in mats4],
                   w4 + 4 * s4.input_padded + 4 * s4.output, s4.output),
              Case("cq4_16384x4096_prepare_b1",
                   [lambda m=m: bqd.cq_prepare(m, x1, out=p1) for m in mats4],
                   4 * (s4.input + s4.input_padded), 0)]
    cases.append(Case("cq4_16384x4096_prepare_b8",
                      [lambda m=m: bqd.cq_prepare(m, x8, out=p8) for m in mats4],
                      8 * 4 * (s4.input + s4.input_padded), 0))
    # the 8-vector matvec reads the copy half a rotation away from the one the
    # batch-1 stage of the same step reads, so it is not served from the cache
    half4 = len(mats4) // 2
    cases.append(Case("cq4_16384x4096_matvec_b8",
                      [lambda m=mats4[(k + half4) % len(mats4)]: bqd.cq_matvec(m, p8, out=y8)
                       for k in range(len(mats4))],
                      w4 + 8 * 4 * s4.input_padded + 8 * 4 * s4.output, 8 * s4.output))

    # -- CQ 4-bit 65536 x 512 table: gather 4096 rows
    log("generating CQ4 65536x512 table (seed 2)")
    c3 = synth.make_cq(synth.C3, seed=2, n_ids=synth.C3_GATHER_IDS)
    s3 = c3.shape
    k3 = 1 if hot else 16
    packed3, norms3, cb3 = T(c3.packed), T(c3.norms.view(np.int16)), T(c3.codebook)
    mats3 = [bqd.CqMatrix(packed3 if k == 0 else packed3.clone(), norms3 if k == 0 else norms3.clone(),
                          cb3, output=s3.output, input=s3.input, input_padded=s3.input_padded,
                          group=s3.group, bits=s3.bits) for k in range(k3)]
    x3 = T(c3.x[:1])
    p3 = torch.empty(1, s3.input_padded, device=dev)
    y3 = torch.empty(1, s3.output, device=dev)
    w3 = s3.output * s3.stride + s3.output * s3.n_groups * 2
    cases.append(Case("cq4_65536x512_prepare_matvec_b1",
                      [lambda m=m: bqd.cq_prepare_matvec(m, x3, prepared=p3, out=y3) for m in mats3],
                      w3 + 4 * s3.input + 4 * s3.input_padded + 4 * s3.output, s3.output))
    ids = T(c3.ids)
    g = torch.empty(len(c3.ids), s3.input, device=dev)
    n_ids = len(c3.ids)
    gather_bytes = n_ids * (s3.stride + 2 * s3.n_groups) + 4 * n_ids + 4 * n_ids * s3.input
    # likewise the gather reads a table copy other than the projection's
    half3 = len(mats3) // 2
    cases.append(Case("cq4_65536x512_gather_4096",
                      [lambda m=mats3[(k + half3) % len(mats3)]: bqd.cq_gather_rows(m, ids, out=g)
                       for k in range(len(mats3))],
                      gather_bytes, n_ids))

    hd = yh = None
    if heads:
        # -- FP8 head 246272 x 4096
        log("generating F8 head 246272x4096 (seed 4)")
        hd = synth.make_f8(**synth.HEAD, seed=4)
        kh = 1 if hot else 2
        wh0 = T(hd.w)
        whs = [wh0] + [wh0.clone() for _ in range(kh - 1)]
        sh, xh = T(hd.scale), T(hd.x)
        yh = torch.empty(1, hd.R, device=dev)
        head_bytes = hd.R * hd.C + hd.SR * hd.SC + 4 * hd.C + 4 * hd.R
        cases.append(Case(HEAD_STAGE,
                          [lambda w=w: bqd.f8_matvec(w, sh, xh, out=yh) for w in whs],
                          head_bytes, hd.R))
        # the head with the greedy token (argmax) fused into its pass
        ya = torch.empty(1, hd.R, device=dev)
        aws = torch.empty(bqd.f8_matvec_argmax_workspace_bytes(1), dtype=torch.uint8, device=dev)
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        extras.append(Case("f8_head_246272x4096_matvec_argmax",
                           [lambda w=w: bqd.f8_matvec_argmax(w, sh, xh, workspace=aws, out=ya,
                                                             token=tok)
                            for w in whs], head_bytes + 4, hd.R))
        # the head with top-k (k = 64) / temperature sampling fused onto its
        # pass, and the same work unfused (the head, then logits_sample)
        sst = torch.tensor([12345], dtype=torch.int32, device=dev)
        sws = torch.empty(bqd.logits_sample_workspace_bytes(hd.R, 64), dtype=torch.uint8,
                          device=dev)
        extras.append(Case("f8_head_246272x4096_matvec_sample_k64",
                           [lambda w=w: bqd.f8_matvec_sample(w, sh, xh, 64, 0.8, sst,
                                                             workspace=aws, out=ya)
                            for w in whs], head_bytes + 4 + 8 * 64, hd.R))
        extras.append(Case("f8_head_246272x4096_matvec_then_logits_sample_k64",
                           [lambda w=w: (bqd.f8_matvec(w, sh, xh, out=ya),
                                         bqd.logits_sample(ya.reshape(-1), 64, 0.8, sst, sws))
                            for w in whs], head_bytes + 4 + 8 * 64, hd.R))
        # -- beyond the step: the I8 head (E8M0 scales per 16 columns) and the
        # int8 key cache (quantize 4096 vectors of 128, score one query)
        log("generating I8 head 246272x4096 G16 (seed 5)")
        i8 = synth.make_i8(**synth.I8_HEAD, seed=5)
        wi0 = T(i8.w)
        wis = [wi0] + [wi0.clone() for _ in range(kh - 1)]
        si, xi = T(i8.scale), T(i8.x)
        yi = torch.empty(1, i8.R, device=dev)
        i8_bytes = i8.R * i8.C + i8.scale.size + 4 * i8.C + 4 * i8.R
        extras.append(Case("i8_head_246272x4096_g16_matvec",
                           [lambda w=w: bqd.i8_matvec(w, si, xi, i8.G, out=yi) for w in wis],
                           i8_bytes, i8.R))
    kv = synth.make_kv(**synth.KV, seed=6)
    nkv, dkv = kv.v.shape
    vk, xk = T(kv.v), T(kv.x)
    qk = torch.empty(nkv, dkv, dtype=torch.int8, device=dev)
    sk = torch.empty(nkv, device=dev)
    yk = torch.empty(1, nkv, device=dev)
    extras.append(Case("kv_int8_4096x128_quantize",
                       [lambda: bqd.kv_quantize_int8(vk, q=qk, scales=sk)],
                       4 * nkv * dkv + nkv * dkv + 4 * nkv, nkv))
    extras.append(Case("kv_int8_4096x128_dot",
                       [lambda: bqd.kv_int8_dot(qk, sk, xk, out=yk)],
                       nkv * dkv + 4 * nkv + 4 * dkv + 4 * nkv, nkv))
    # three CQ4 2048 x 512 matrices (group 128) on one activation: one
    # fused launch, against three separate prepare+matvec calls
    tri = [synth.make_cq(synth.C2_3.__class__(2048, 512, 512, 128, 4), seed=20 + j) for j in range(3)]
    tri_m = [bqd.CqMatrix(T(c.packed), T(c.norms.view(np.int16)), T(c.codebook), output=2048,
                          input=512, input_padded=512, group=128, bits=4) for c in tri]
    tri_x = T(tri[0].x[0])
    tri_p = torch.empty(512, device=dev)
    tri_y = [torch.empty(2048, device=dev) for _ in range(3)]
    tri_bytes = 3 * 2048 * (256 + 8) + 4 * 512 + 4 * 512 + 3 * 4 * 2048
    extras.append(Case("cq4_3x2048x512_prepare_matvec_multi",
                       [lambda: bqd.cq_prepare_matvec_multi(tri_m, tri_x, prepared=tri_p, outs=tri_y)],
                       tri_bytes, 3 * 2048))
    extras.append(Case("cq4_3x2048x512_prepare_matvec_separate",
                       [lambda: [bqd.cq_prepare_matvec(m, tri_x[None], prepared=tri_p[None], out=y[None])
                                 for m, y in zip(tri_m, tri_y)]],
                       tri_bytes, 3 * 2048))
    # the workloads' small configs: CQ2 256x200, CQ3 and CQ5 2048x512 (each
    # the page's cqMatvec on one vector: prepare + matvec in one call), and
    # the F8 wkv 512x4096; each whole matrix fits in the L2, so these time
    # cache-resident calls (16 copies still rotate)
    small = {}
    for name, shape, seed in (("cq2_256x200", synth.C1, 0), ("cq3_2048x512", synth.C2_3, 1),
                              ("cq5_2048x512", synth.C2_5, 1)):
        cs = synth.make_cq(shape, seed=seed)
        ss = cs.shape
        base = [T(cs.packed), T(cs.norms.view(np.int16))]
        cbs = T(cs.codebook)
        ms = [bqd.CqMatrix(base[0] if k == 0 else base[0].clone(), base[1] if k == 0 else base[1].clone(),
                           cbs, output=ss.output, input=ss.input, input_padded=ss.input_padded,
                           group=ss.group, bits=ss.bits) for k in range(1 if hot else 16)]
        xs = T(cs.x[:1])
        ps = torch.empty(1, ss.input_padded, device=dev)
        ys = torch.empty(1, ss.output, device=dev)
        wb = ss.output * ss.stride + ss.output * ss.n_groups * 2
        extras.append(Case(f"{name}_prepare_matvec_b1",
                           [lambda m=m, xs=xs, ps=ps, ys=ys: bqd.cq_prepare_matvec(m, xs, prepared=ps, out=ys)
                            for m in ms],
                           wb + 4 * ss.input + 4 * ss.input_padded + 4 * ss.output, ss.output))
        small[name] = (cs, ps, ys)
    wk = synth.make_f8(**synth.WKV, seed=4)
    wkw = [T(wk.w)]
    wkw += [wkw[0].clone() for _ in range(0 if hot else 15)]
    wks, wkx = T(wk.scale), T(wk.x)
    wky = torch.empty(1, wk.R, device=dev)
    extras.append(Case("f8_wkv_512x4096_matvec",
                       [lambda w=w: bqd.f8_matvec(w, wks, wkx, out=wky) for w in wkw],
                       wk.R * wk.C + wk.SR * wk.SC + 4 * wk.C + 4 * wk.R, wk.R))
    small["f8_wkv_512x4096"] = (wk, None, wky)
    hm = synth.make_hmlp(**synth.HMLP, seed=7)
    hn, hd1, hd2, hd3, hr, hu = (T(a) for a in (hm.n, hm.d1, hm.d2, hm.d3, hm.resid, hm.u))
    ho = torch.empty_like(hn)
    H = synth.HMLP["H"]
    extras.append(Case("hadamard_mlp_512_to_2048",
                       [lambda: bqd.hadamard_mlp(hn, H, hd1, hd2, hd3, hr, hu, out=ho)],
                       4 * (3 * H + 4 * hn.numel()), hn.numel()))
    data = dict(c4=c4, c3=c3, head=hd, head_logits=yh, small=small,
                head_dev=(whs[0], sh, xh) if heads else None,
                outputs=dict(p1=p1, y1=y1, p8=p8, y8=y8, p3=p3, y3=y3, g=g, yh=yh))
    return cases, extras, data


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, with its family, model
    and stepping numbers (a virtualized host may report a bare name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                key, val = (t.strip() for t in line.split(":", 1))
                if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                    fields[key] = val
            elif fields:
                break  # the first processor's block is enough
    except OSError:
        return None
    name = fields.get("model name")
    if name is None:
        return None
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(data, threads):
    """The oracle, as it stands, on a bounded sample of the same workload:
    at `threads` threads (rows split over Python threads; ctypes releases the
    GIL) and at one thread on a smaller sample, each the best of 3 timed
    passes after one untimed pass."""
    import oracle

    c4, c3, hd = data["c4"], data["c3"], data["head"]
    h4 = oracle.CqMatrix.from_case(c4)
    h3 = oracle.CqMatrix.from_case(c3)
    p4 = oracle.cq_prepare(h4, c4.x[0])
    p3 = oracle.cq_prepare(h3, c3.x[0])
    s4, s3 = c4.shape, c3.shape

    def split(n, t):
        per = (n + t - 1) // t
        return [(i * per, min(per, n - i * per)) for i in range(t) if i * per < n]

    def run(jobs):
        ts = [threading.Thread(target=f) for f in jobs]
        t0 = time.perf_counter()
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        return time.perf_counter() - t0

    def sample(t, n_head):
        """Seconds per stage, best of 3 after one untimed pass, and the bytes."""
        n_c4, n_ids = s4.output, len(c3.ids)
        stages = {
            "head": lambda: run([lambda a=a, b=b: oracle.f8_matvec(
                hd.w, hd.R, hd.C, hd.scale, hd.SR, hd.SC, hd.x[0], a, b) for a, b in split(n_head, t)]),
            "c4": lambda: run([lambda a=a, b=b: oracle.cq_matvec(h4, p4, a, b)
                               for a, b in split(n_c4, t)]),
            "c3": lambda: run([lambda a=a, b=b: oracle.cq_matvec(h3, p3, a, b)
                               for a, b in split(s3.output, t)]),
            "gather": lambda: run([lambda a=a, b=b: oracle.cq_gather(h3, c3.ids[a:a + b])
                                   for a, b in split(n_ids, t)]),
        }
        secs = {}
        for name, f in stages.items():
            f()
            secs[name] = min(f() for _ in range(3))
        nbytes = (n_head * (hd.C + 4) + n_c4 * (s4.stride + 2 * s4.n_groups + 4)
                  + s3.output * (s3.stride + 2 * s3.n_groups + 4)
                  + n_ids * (s3.stride + 2 * s3.n_groups + 4 + 4 * s3.input))
        return secs, nbytes

    secs, nbytes = sample(threads, hd.R)
    secs1, nbytes1 = sample(1, 16384)
    total, total1 = sum(secs.values()), sum(secs1.values())
    return {
        "value": round(nbytes / total / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"oracle on host cores, best of 3 after one untimed pass, {threads} threads over "
                   f"row chunks: all 246272 F8 head rows ({secs['head']:.3f} s), CQ4 16384x4096 "
                   f"batch 1 ({secs['c4']:.3f} s), CQ4 65536x512 batch 1 ({secs['c3']:.3f} s), "
                   f"gather of {len(c3.ids)} ids ({secs['gather']:.3f} s); value_1_thread: the same "
                   f"with head rows [0,16384) ({secs1['head']:.3f} s) on one thread"),
        "seconds": round(total, 3),
        "value_1_thread": round(nbytes1 / total1 / 1e9, 4),
        "cpu_model": cpu_model(),
    }


def self_check(data, bqd, state):
    """The outputs the last timed step left in each stage's buffers (every
    weight copy holds the same values) against the oracle: the prepared
    vectors and the gathered rows bit for bit; matvec outputs on sampled rows
    within |gpu - oracle| <= 1e-4 * sum|w*x| + 1e-6, reported as the largest
    ratio of the two sides.  The small configs are checked on every row."""
    import torch

    import oracle
    rng = np.random.default_rng(2026)
    out = data["outputs"]
    res = {}

    def ratio(got, ref, mag):
        got = np.asarray(got, np.float64).reshape(-1)
        return float(np.max(np.abs(got - np.asarray(ref).reshape(-1)) /
                            (1e-4 * np.asarray(mag).reshape(-1) + 1e-6)))

    def bits_eq(a, b):
        a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
        return a.shape == b.shape and bool(np.array_equal(a.view(np.uint32), b.view(np.uint32)))

    def tol_rec(name, r, n):
        res[name] = dict(checked=n, max_ratio=round(r, 6), ok=bool(r <= 1.0))

    def rows_ratio(fn, rows):
        worst = 0.0
        for r in rows:
            yr, mr = fn(int(r))
            worst = max(worst, yr)
        return worst

    c4 = data["c4"]
    h4 = oracle.CqMatrix.from_case(c4)
    p1 = oracle.cq_prepare(h4, c4.x[0])
    p8 = oracle.cq_prepare(h4, c4.x)
    res["cq4_16384x4096_prepared_b1"] = dict(bit_exact=bits_eq(out["p1"].cpu().numpy()[0], p1))
    res["cq4_16384x4096_prepared_b8"] = dict(bit_exact=bits_eq(out["p8"].cpu().numpy(), p8))
    rows = rng.choice(c4.shape.output, 256, replace=False)
    y1 = out["y1"].cpu().numpy()[0]
    y8 = out["y8"].cpu().numpy()

    def one(h, p, y, r):
        ref, mag = oracle.cq_matvec(h, p, r, 1)
        return ratio(y[..., r:r + 1], ref, mag), None

    tol_rec("cq4_16384x4096_matvec_b1", rows_ratio(lambda r: one(h4, p1, y1, r), rows), len(rows))
    tol_rec("cq4_16384x4096_matvec_b8", rows_ratio(lambda r: one(h4, p8, y8, r), rows[:64]),
            64 * 8)
    c3 = data["c3"]
    h3 = oracle.CqMatrix.from_case(c3)
    p3 = oracle.cq_prepare(h3, c3.x[0])
    res["cq4_65536x512_prepared_b1"] = dict(bit_exact=bits_eq(out["p3"].cpu().numpy()[0], p3))
    rows = rng.choice(c3.shape.output, 256, replace=False)
    y3 = out["y3"].cpu().numpy()[0]
    tol_rec("cq4_65536x512_matvec_b1", rows_ratio(lambda r: one(h3, p3, y3, r), rows), len(rows))
    sel = np.sort(rng.choice(len(c3.ids), 256, replace=False))
    g_ref, _ = oracle.cq_gather(h3, c3.ids[sel])
    res["cq4_65536x512_gather_4096"] = dict(checked=len(sel),
                                           bit_exact=bits_eq(out["g"].cpu().numpy()[sel], g_ref))
    hd = data["head"]
    yh = out["yh"].cpu().numpy()[0]
    rows = rng.choice(hd.R, 512, replace=False)

    def head_row(r):
        ref, mag = oracle.f8_matvec(hd.w, hd.R, hd.C, hd.scale, hd.SR, hd.SC, hd.x[0], r, 1)
        return ratio(yh[r:r + 1], ref, mag), None

    tol_rec("f8_head_246272x4096_matvec", rows_ratio(head_row, rows), len(rows))
    # the head with its argmax fused: y bit-equal to the head's, the token the
    # argmax of that y (an integer decision on the GPU's values), and that
    # row's logit against the oracle
    w0, s0, x0 = data["head_dev"]
    ya, tok = bqd.f8_matvec_argmax(w0, s0, x0)
    yan, t = ya.cpu().numpy()[0], int(tok.item())
    finite = ~np.isnan(yan)
    t_host = int(np.flatnonzero(yan == yan[finite].max())[0]) if finite.any() else 0
    r_t, ok_t = head_row(t)
    res["f8_head_argmax"] = dict(token=t, max_ratio=round(float(r_t), 6),
                                 ok=bool(bits_eq(yan, yh) and t == t_host and r_t <= 1.0))
    # the head with top-k sampling fused: y bit-equal to the head's; the ids
    # those of that y's 64 best, and ids, values, token and state equal to
    # logits_sample's on that y; each selected logit against the oracle
    st1 = torch.tensor([777], dtype=torch.int32, device=state.device)
    st2 = st1.clone()
    ys, tks, sids, svals = bqd.f8_matvec_sample(w0, s0, x0, 64, 0.8, st1)
    tk2, ids2, vals2 = bqd.logits_sample(ys.reshape(-1), 64, 0.8, st2)
    ysn, sidn = ys.cpu().numpy()[0], sids.cpu().numpy()[0]
    nan = np.isnan(ysn.astype(np.float64))
    want = np.lexsort((np.arange(ysn.size), -np.where(nan, 0.0, ysn.astype(np.float64)), nan))[:64]
    r_s = max(head_row(int(r))[0] for r in sidn)
    res["f8_head_sample_k64"] = dict(
        token=int(tks.item()), max_ratio=round(float(r_s), 6),
        ok=bool(bits_eq(ysn, yh) and np.array_equal(sidn, want) and
                np.array_equal(sidn, ids2.cpu().numpy()) and
                bits_eq(svals.cpu().numpy()[0], vals2.cpu().numpy()) and
                int(tks.item()) == int(tk2.item()) and int(st1.item()) == int(st2.item()) and
                r_s <= 1.0))
    for name, (case, p_dev, y_dev) in data["small"].items():
        y = y_dev.cpu().numpy()[0]
        if name.startswith("f8"):
            ref, mag = oracle.f8_matvec(case.w, case.R, case.C, case.scale, case.SR, case.SC,
                                        case.x[0])
        else:
            h = oracle.CqMatrix.from_case(case)
            pr = oracle.cq_prepare(h, case.x[0])
            res[f"{name}_prepared_b1"] = dict(bit_exact=bits_eq(p_dev.cpu().numpy()[0], pr))
            ref, mag = oracle.cq_matvec(h, pr)
        tol_rec(f"{name}_matvec", ratio(y, ref, mag), len(y))
    # the sampler's top 64 (ids and values bit for bit) on seeded logits of the
    # head's size, an input of its own rather than the head's output
    import synth
    lg = synth.make_logits(data["head_logits"].numel(), seed=8)
    st = state.clone()
    _, ids, vals = bqd.logits_sample(torch.from_numpy(lg).to(state.device), 64, 0.8, st)
    oid, oval = oracle.topk(lg, 64)
    res["logits_top64"] = dict(checked=64, bit_exact=bool(
        np.array_equal(ids.cpu().numpy(), oid) and bits_eq(vals.cpu().numpy(), oval)))
    res["all_ok"] = all(v.get("ok", True) and v.get("bit_exact", True) for v in res.values())
    return res


def capture(torch, fn):
    """A CUDA/HIP graph of fn(): warm up on a side stream, then capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def traffic_probe(torch, bqd, synth, stage=None):
    """A fixed launch sequence for rocprofv3 --pmc runs: the dominant kernel
    (or a CQ stage's graph of 16 launches over its rotated copies, replayed
    4 times), then a plain device copy of known size to calibrate the byte
    counters."""
    if stage:
        cases, extra_cases, _ = build_cases(torch, bqd, synth, False, heads=False)
        c = next(c for c in cases + extra_cases if c.name == stage)
        g = capture(torch, lambda: [c.calls[k % len(c.calls)]() for k in range(STAGE_LAUNCHES)])
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
        del g, cases, extra_cases
    else:
        hd = synth.make_f8(**synth.HEAD, seed=4)
        T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        w, s, x = T(hd.w), T(hd.scale), T(hd.x)
        y = torch.empty(1, hd.R, device="cuda")
        for _ in range(8):
            bqd.f8_matvec(w, s, x, out=y)
        torch.cuda.synchronize()
        del w
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    b = torch.empty_like(a)
    for _ in range(8):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe": stage or HEAD_STAGE, "copy_bytes": n}), flush=True)


def stage_probe(torch, bqd, synth, name, hot):
    """A fixed launch sequence for rocprofv3 --pmc runs on one stage: its
    graph of 16 launches (rotating weight copies), replayed 4 times."""
    cases, extra_cases, _ = build_cases(torch, bqd, synth, hot)
    by_name = {c.name: c for c in cases + extra_cases}
    if name not in by_name:
        raise SystemExit(f"bench.py: no stage {name!r}; stages: {', '.join(sorted(by_name))}")
    c = by_name[name]
    n = STAGE_LAUNCHES
    g = capture(torch, lambda: [c.calls[k % len(c.calls)]() for k in range(n)])
    for _ in range(4):
        g.replay()
    torch.cuda.synchronize()
    print(json.dumps({"stage": name, "launches": 5 * n, "bytes": c.nbytes}), flush=True)


def _dispatch_kib(out_dir, counter, kernel="f8_matvec_fast"):
    """Median per-dispatch value of `counter` for the kernel and for the
    1 GiB copy, from a rocprofv3 --pmc csv directory; also the kernel's full
    name."""
    import csv
    import glob
    import statistics
    vals = {"kernel": [], "copy": []}
    names = set()
    for f in glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = "kernel" if kernel in name else "copy" if "copyBuffer" in name else None
            if key:
                vals[key].append((int(row.get("Dispatch_Id") or 0), float(row["Counter_Value"])))
                if key == "kernel":
                    names.add(name.split("(")[0])
    if len(vals["kernel"]) < 8 or len(vals["copy"]) < 8:
        raise SystemExit(f"{out_dir}: expected 8 {kernel} and 8 copy dispatches for {counter}")
    # the calibration copies are the probe's last 8 copy dispatches (uploads
    # and clones of the inputs come earlier)
    copies = [v for _, v in sorted(vals["copy"])[-8:]]
    return (statistics.median(v for _, v in vals["kernel"]), statistics.median(copies),
            sorted(names))


def stage_traffic_record(stage, fetch_dir, write_dir, out_dir=None):
    """HBM bytes per launch of a CQ stage's kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch, median) each scaled by what the same counter reads for
    a 1 GiB device copy in the same run; written as JSON and markdown under
    profiles/."""
    import hashlib
    st = STAGE_TRAFFIC[stage]
    kf, copy_f, names = _dispatch_kib(fetch_dir, "FETCH_SIZE", st["kernel"])
    kw, copy_w, _ = _dispatch_kib(write_dir, "WRITE_SIZE", st["kernel"])
    gib_kib = float(1 << 20)
    fetch_scale, write_scale = round(gib_kib / copy_f, 2), round(gib_kib / copy_w, 2)
    read_b, write_b = round(kf * 1024 * fetch_scale), round(kw * 1024 * write_scale)
    srcs = [os.path.join(ROOT, "bit_quantized_decode_amd", "csrc", f)
            for f in ("cq.hip", "cq_device.h", "device.h")]
    rec = {
        "stage": stage, "kernel": names, "workload": st["what"],
        "source_sha256_16": hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()[:16],
        "fetch_kib_per_dispatch_raw": kf, "write_kib_per_dispatch_raw": kw,
        "copy_1gib_fetch_kib_raw": copy_f, "copy_1gib_write_kib_raw": copy_w,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "read_bytes": read_b, "write_bytes": write_b, "traffic_bytes": read_b + write_b,
        "algorithmic_read_bytes": st["reads"], "algorithmic_write_bytes": st["writes"],
        "read_over_algorithmic": round(read_b / st["reads"], 4),
        "write_over_algorithmic": round(write_b / st["writes"], 4),
    }
    base = os.path.join(out_dir or os.path.join(ROOT, "profiles"),
                        f"{st['kernel']}_{st['workload']}_hbm_traffic")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    cmd = (f"rocprofv3 --pmc {{FETCH_SIZE|WRITE_SIZE}} --output-format csv -d <dir> -o t -- "
           f"python3 bench.py --traffic-probe --stage {stage}")
    md = [f"# HBM traffic of `{st['kernel']}`: {st['what']}", "",
          "Two counter runs of one fixed launch sequence (the stage's graph of 16 launches over its",
          "16 rotated weight copies, replayed 4 times, then 8 plain 1 GiB device copies), then the",
          "record (no GPU):", "", "```", cmd,
          f"python3 bench.py --traffic-record <fetch dir> <write dir> --stage {stage}", "```", "",
          "Per dispatch (median), KiB as the counters report them:", "",
          "| kernel | FETCH_SIZE | WRITE_SIZE |", "|---|---:|---:|",
          f"| `__amd_rocclr_copyBuffer`, 1 GiB copy | {copy_f:,.1f} | {copy_w:,.1f} |",
          f"| `{', '.join(names)}` | {kf:,.1f} | {kw:,.1f} |", "",
          f"Scales from the copy: FETCH_SIZE x {fetch_scale}, WRITE_SIZE x {write_scale}.", "",
          "| | bytes per launch |", "|---|---:|",
          f"| reads, scaled | {read_b:,} |", f"| algorithmic reads | {st['reads']:,} |",
          f"| reads / algorithmic | {rec['read_over_algorithmic']} |",
          f"| writes, scaled | {write_b:,} |", f"| algorithmic writes | {st['writes']:,} |",
          f"| writes / algorithmic | {rec['write_over_algorithmic']} |", ""]
    with open(base + ".md", "w") as f:
        f.write("\n".join(md))
    print(json.dumps(rec))


def traffic_record(fetch_dir, write_dir):
    """HBM bytes per head launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    each scaled by what the same counter reads for a 1 GiB device copy."""
    import hashlib
    import synth
    hd = synth.HEAD
    head_f, copy_f, _ = _dispatch_kib(fetch_dir, "FETCH_SIZE")
    head_w, copy_w, _ = _dispatch_kib(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    fetch_scale = round(gib_kib / copy_f, 2)
    write_scale = round(gib_kib / copy_w, 2)
    read_b = round(head_f * 1024 * fetch_scale)
    write_b = round(head_w * 1024 * write_scale)
    alg = hd["R"] * hd["C"] + hd["SR"] * hd["SC"]  # weights and scales
    rec = {
        "kernel": "f8_matvec_fast (F8 E4M3 head %dx%d, E8M0 scales %dx%d)" % (hd["R"], hd["C"], hd["SR"], hd["SC"]),
        "source_sha256_16": hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()[:16],
        "fetch_kib_per_dispatch_raw": head_f, "write_kib_per_dispatch_raw": head_w,
        "copy_1gib_fetch_kib_raw": copy_f, "copy_1gib_write_kib_raw": copy_w,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "read_bytes": read_b, "write_bytes": write_b, "traffic_bytes": read_b + write_b,
        "algorithmic_read_bytes": alg, "read_over_algorithmic": round(read_b / alg, 4),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def main():
    args = parse_args()
    if args.traffic_record:
        if args.stage:
            stage_traffic_record(args.stage, *args.traffic_record)
        else:
            traffic_record(*args.traffic_record)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the rows of each matvec shard across GPUs by design only)", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_quantized_decode_amd as bqd
    import synth

    torch.cuda.set_device(0)
    bqd.lib()
    if args.traffic_probe:
        traffic_probe(torch, bqd, synth, args.stage)
        return
    if args.stage_probe:
        stage_probe(torch, bqd, synth, args.stage_probe, args.hot)
        return
    cases, extra_cases, data = build_cases(torch, bqd, synth, args.hot)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    period = max(len(c.calls) for c in cases)  # weight copies rotate with this period

    # One graph per rotation index: the whole step (every stage, in order),
    # and the same step without the head (the head's in-step duration is the
    # difference of the two).
    log(f"capturing {period} step graphs")
    step_graphs = [capture(torch, lambda k=k: [c.calls[k % len(c.calls)]() for c in cases])
                   for k in range(period)]
    head_case = next(c for c in cases if c.name == HEAD_STAGE)
    rest = [c for c in cases if c is not head_case]
    rest_graphs = [capture(torch, lambda k=k: [c.calls[k % len(c.calls)]() for c in rest])
                   for k in range(period)]
    # Per stage (the head aside): one graph of STAGE_LAUNCHES back-to-back
    # launches over the copies.
    stage_graphs = {c.name: capture(torch, lambda c=c: [c.calls[k % len(c.calls)]()
                                                       for k in range(STAGE_LAUNCHES)])
                    for c in rest + extra_cases}

    # Untimed measurements first (they also bring the GPU to its working
    # clock before the timed steps).
    # The head inside the step: HIP events on the launch stream bracket runs
    # of 48 replays of the whole step and of the step without the head,
    # alternated; each difference per step is one sample.
    def replays_ms(graphs, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            graphs[i % period].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    log("timing the head inside the step")
    replays_ms(rest_graphs, period)
    head_samples = []
    for _ in range(8):
        full_ms = replays_ms(step_graphs, 3 * STAGE_LAUNCHES)
        head_samples.append(full_ms - replays_ms(rest_graphs, 3 * STAGE_LAUNCHES))
    head_ms = np.array(head_samples)

    # The other stages: HIP events on the launch stream bracket replays of
    # each stage's graph of STAGE_LAUNCHES back-to-back launches.
    log("timing each stage")
    reps = max(8, args.steps // STAGE_LAUNCHES)
    per_case = {}
    extras = {}
    for c in cases + extra_cases:
        if c is head_case:
            ms = head_ms
        else:
            g = stage_graphs[c.name]
            g.replay()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) / STAGE_LAUNCHES
        c.ms = ms
        gbs = c.nbytes / (ms.mean() * 1e-3) / 1e9
        rec = dict(
            us_mean=round(float(ms.mean() * 1e3), 3), us_median=round(float(np.median(ms) * 1e3), 3),
            us_p10=round(float(np.percentile(ms, 10) * 1e3), 3),
            us_p90=round(float(np.percentile(ms, 90) * 1e3), 3), bytes=c.nbytes,
            gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
            rows_per_s=round(c.rows / (ms.mean() * 1e-3), 1) if c.rows else None)
        if c is head_case:
            per_case[c.name] = dict(rec, timing="in the step: the step minus the step without the "
                                                "head, 8 samples of 3 x 16 replays each")
        elif c in cases:
            per_case[c.name] = dict(rec, timing="16 back-to-back launches per graph replay")
        elif c.name.startswith("cq4_3x"):
            extras[c.name] = dict(rec, note="not part of the step: several matrices on one activation")
        elif c.name.endswith("_sample_k64"):
            extras[c.name] = dict(rec, note="not part of the step: the head with top-k (k = 64, "
                                            "T = 0.8) sampling of its logits" + (
                                                " fused onto the pass (f8_matvec_sample)"
                                                if "then" not in c.name else
                                                ", unfused: f8_matvec, then logits_sample"))
        elif c.name.endswith("_argmax"):
            extras[c.name] = dict(rec, note="not part of the step: the head with its greedy token "
                                            "(argmax) fused into the pass, plus the one-workgroup "
                                            "launch that reduces its slots")
        elif c.name.startswith("cq4_"):
            extras[c.name] = dict(rec, note="not part of the step: the same stage as two calls")
        elif c.name.split("_")[0] in ("cq2", "cq3", "cq5") or c.name.startswith("f8_wkv"):
            extras[c.name] = dict(rec, note="not part of the step: a small workload config, cache-"
                                            "resident (the whole matrix fits in the L2)")
        else:
            extras[c.name] = dict(rec, note="not part of the step: a neighbouring format of the pages")
    # Beyond the step: top-k (k = 64) and a temperature draw over the head's
    # logits, timed the same way (the sampler's state advances on the GPU).
    logits = data["head_logits"].reshape(-1)
    state = torch.tensor([12345], dtype=torch.int32, device="cuda")
    ws = torch.empty(bqd.logits_sample_workspace_bytes(logits.numel(), 64), dtype=torch.uint8,
                     device="cuda")
    g = capture(torch, lambda: [bqd.logits_sample(logits, 64, 0.8, state, ws)
                                for _ in range(STAGE_LAUNCHES)])
    g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) / STAGE_LAUNCHES
    extras["head_logits_sample_k64"] = dict(
        us_mean=round(float(ms.mean() * 1e3), 3), us_median=round(float(np.median(ms) * 1e3), 3),
        logits=logits.numel(), k=64, temperature=0.8, launches=2,
        note="not part of the step: the sampler over the head's logits")
    # The plain read probe at the batch-1 CQ4 stage's size (34,078,720 bytes,
    # 16 rotating copies, graphs of 16 launches as the stages): what one cold
    # launch of that size reads in without any decode.
    nb = 34078720
    bufs = [torch.full((nb // 4,), 0x3C5A96E1 + j, dtype=torch.int32, device="cuda")
            for j in range(16)]
    xo = torch.empty(bqd.READ_STREAM_WORDS, dtype=torch.int32, device="cuda")
    g = capture(torch, lambda: [bqd.dbg_read_stream(bufs[j % 16], xo)
                                for j in range(STAGE_LAUNCHES)])
    g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) / STAGE_LAUNCHES
    extras["read_stream_34078720_bytes"] = dict(
        us_mean=round(float(ms.mean() * 1e3), 3), us_median=round(float(np.median(ms) * 1e3), 3),
        bytes=nb, gbs=round(nb / (ms.mean() * 1e-3) / 1e9, 1),
        frac_hbm=round(nb / (ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        note="not part of the step: the plain read probe (no decode) over the bytes of the "
             "batch-1 CQ4 16384x4096 stage, cold, the reference for one launch of that size")
    del bufs, xo, g
    torch.cuda.synchronize()
    # The achievable-HBM reference: the library's plain read probe over 2 GiB
    # (past the Infinity Cache), median of 8 timed calls.
    buf = torch.full((1 << 29,), 0x5A3C96E1, dtype=torch.int32, device="cuda")
    xor_out = torch.empty(bqd.READ_STREAM_WORDS, dtype=torch.int32, device="cuda")
    bqd.dbg_read_stream(buf, xor_out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(8)]
    for e0, e1 in ev:
        e0.record(stream)
        bqd.dbg_read_stream(buf, xor_out)
        e1.record(stream)
    torch.cuda.synchronize()
    read_ceiling = (1 << 31) / (float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3) / 1e9
    del buf, xor_out
    torch.cuda.synchronize()

    # The steps themselves are launched directly on the stream: the host
    # enqueues a step's six launches in ~50 us, far ahead of the GPU's
    # ~185 us, so the kernels run back to back, without the gap that every
    # graph replay adds at its boundary (~4 us per step measured here).
    def step(i):
        for c in cases:
            c.calls[i % len(c.calls)]()

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed region: exactly K steps, synchronized on both sides.
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # The outputs of the last timed step (every weight copy holds the same
    # values) against the oracle.
    log("checking the last step's outputs against the oracle")
    parity = self_check(data, bqd, state)

    total_bytes = sum(c.nbytes for c in cases)
    total_rows = sum(c.rows for c in cases)
    value = total_bytes / (step_ms * 1e-3) / 1e9
    head = per_case[HEAD_STAGE]
    roofline = dict(bound="hbm", kernel="f8_matvec_fast (F8 head 246272x4096)",
                    achieved=head["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(head["gbs"] / HBM_PEAK_GBS, 4), traffic=measured_traffic(),
                    us_per_launch=head["us_mean"], bytes_per_launch=head["bytes"])
    roofline["frac_of_read_ceiling"] = round(head["gbs"] / read_ceiling, 4)
    for rec in list(per_case.values()) + list(extras.values()):
        if "gbs" in rec:
            rec["frac_read_ceiling"] = round(rec["gbs"] / read_ceiling, 4)
    # 8 vectors: the weights are read once for all 8, and the contraction
    # runs on the matrix cores (bf16 hi/lo operand pairs, all four cross
    # products, fp32 accumulation): 4 x 2 R C B bf16 flops, 1.7 us at the
    # 2.5 PFLOP/s bf16 peak, under the 4.3 us of HBM time, so HBM bounds it.
    b8 = per_case.get("cq4_16384x4096_matvec_b8")
    if b8:
        mfma_flops = 4 * 2 * 16384 * 4096 * 8
        t_hbm = b8["bytes"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = mfma_flops / (BF16_PEAK_TFLOPS * 1e12)
        b8.update(arithmetic="bf16 hi/lo operand pairs on MFMA (all four cross products), fp32 "
                             "accumulation", mfma_flops=mfma_flops, roofline_bound="hbm",
                  roofline_us=round(max(t_hbm, t_mfma) * 1e6, 3),
                  frac_roofline=round(max(t_hbm, t_mfma) / (b8["us_mean"] * 1e-6), 4))
    cpu = None
    if not args.no_cpu_baseline:
        affinity = len(os.sched_getaffinity(0))
        n = args.cpu_threads or min(CPU_SHARE, affinity)
        log(f"cpu baseline: oracle with {n} threads")
        cpu = cpu_baseline(data, n)
        cpu["affinity_cpus"] = affinity
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; synth.py)",
        "config": {"workload": "decode step: CQ4 16384x4096 g256 prepare+matvec at batch 1 and 8; "
                               "CQ4 65536x512 g128 vocabulary projection (batch 1) and gather of "
                               "4096 rows; F8 E4M3 head 246272x4096 with E8M0 [1924x32] scales",
                   "mode": "hot (one weight copy)" if args.hot else
                           "cold (weights rotated past the 256 MB Infinity Cache)",
                   "launch": "the step's six kernel launches enqueued directly on one stream",
                   "parallelism": "single GPU"},
        "rows_per_s": round(total_rows / (step_ms * 1e-3), 1),
        "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
        "read_ceiling": {"kernel": "bqd_dbg_read_stream over 2 GiB (nontemporal 16-byte loads, "
                                   "2048 workgroups of 256)", "gbs": round(read_ceiling, 1),
                         "frac_hbm": round(read_ceiling / HBM_PEAK_GBS, 4)},
        "cases": per_case, "extras": extras, "parity": parity, "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

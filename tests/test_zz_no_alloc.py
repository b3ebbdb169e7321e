"""GPU: the allocation-free sampler (logits_sample_noalloc, its workspace a
static device array inside the library) against logits_sample with a caller
workspace, through the C ABI: top-k ids and values bit for bit, the token and
the advanced generator state equal.  Two calls in a row, the second on fewer
logits (fewer first-stage blocks) than the first, then a third on the first
input again: what an earlier call left in the shared array must not leak into
a later one."""
import numpy as np
import pytest
import torch

import bit_quantized_decode_amd as bqd
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _state(seed):
    return torch.tensor([int(np.array([seed], np.uint32).view(np.int32)[0])], dtype=torch.int32,
                        device=DEV)


def _with_workspace(logits, k, T, seed):
    state = _state(seed)
    tok, ids, vals = bqd.logits_sample(logits, k, T, state)
    return tok.cpu(), ids.cpu(), vals.cpu(), state.cpu()


def _no_alloc(logits, k, T, seed):
    state = _state(seed)
    tok = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ids = torch.full((k,), -1, dtype=torch.int32, device=DEV)
    vals = torch.full((k,), float("nan"), dtype=torch.float32, device=DEV)
    bqd.logits_sample_noalloc(logits, k, T, state, tok, ids, vals)
    return tok.cpu(), ids.cpu(), vals.cpu(), state.cpu()


def _same(a, b):
    tok_a, ids_a, vals_a, st_a = a
    tok_b, ids_b, vals_b, st_b = b
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(vals_a.view(torch.int32), vals_b.view(torch.int32))  # bit for bit
    assert torch.equal(tok_a, tok_b) and torch.equal(st_a, st_b)


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_no_alloc_matches_workspace_entry_point(kind):
    rng = np.random.default_rng(2024)
    big_np = (3.0 * rng.standard_normal(246272) if kind == "normal"
              else rng.integers(-3, 4, 246272)).astype(np.float32)
    small_np = (3.0 * rng.standard_normal(5000) if kind == "normal"
                else rng.integers(-3, 4, 5000)).astype(np.float32)
    big, small = (torch.from_numpy(a).to(DEV) for a in (big_np, small_np))
    for logits, host, k, T, seed in ((big, big_np, 64, 0.8, 0x9E3779B9), (small, small_np, 16, 1.3, 777),
                                     (big, big_np, 7, 0.0, 4242)):
        print(f"[case] no-alloc sampler n={logits.numel()} k={k} T={T} ({kind})", flush=True)
        got = _no_alloc(logits, k, T, seed)
        ref = _with_workspace(logits, k, T, seed)
        torch.cuda.synchronize()
        _same(got, ref)
        # and the oracle's top-k (O12)
        oid, oval = oracle.topk(host, k)
        assert np.array_equal(got[1].numpy(), oid)
        assert np.array_equal(got[2].numpy().view(np.uint32), oval.view(np.uint32))


def test_no_alloc_on_a_stream_of_its_own():
    """The scratch is found on the device that runs the call's stream; on a
    created stream the results still equal logits_sample's on that stream."""
    rng = np.random.default_rng(2025)
    logits = torch.from_numpy((3.0 * rng.standard_normal(100000)).astype(np.float32)).to(DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for fn in (_no_alloc, _with_workspace):
        with torch.cuda.stream(side):
            print(f"[case] {fn.__name__} on a created stream", flush=True)
            outs.append(fn(logits, 32, 0.9, 99))
    torch.cuda.synchronize()
    _same(outs[0], outs[1])


def test_no_alloc_rejects_bad_arguments():
    logits = torch.zeros(100, device=DEV)
    state = _state(1)
    tok = torch.empty(1, dtype=torch.int32, device=DEV)
    ids = torch.empty(65, dtype=torch.int32, device=DEV)
    vals = torch.empty(65, dtype=torch.float32, device=DEV)
    with pytest.raises(bqd.BqdError):
        bqd.logits_sample_noalloc(logits, 65, 1.0, state, tok, ids, vals)  # k above 64
    with pytest.raises(bqd.BqdError):
        bqd.logits_sample_noalloc(logits, 8, -1.0, state, tok, ids, vals)  # negative temperature
    with pytest.raises(bqd.BqdError):  # the values written over the logits
        bqd.logits_sample_noalloc(logits, 8, 1.0, state, tok, ids, logits[:8])

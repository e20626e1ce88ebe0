"""kmr_decode_step_static (the step with the library's static workspace, for callers
that cannot allocate) against kmr_decode_step with a caller workspace, through the
C ABI: two calls in a row, the second with a smaller batch, from identical inputs.
Next ids, logits, the cache and the advanced positions must be the same bits (the
two run the same kernels on the same inputs).  Also: a stalled step poisons the
static array until a call with KMR_CLEAR_WORKSPACE, and a layout too large for the
array is refused before anything runs."""
import numpy as np
import pytest
import torch

from int4_weight_only_gemv_amd import synth
from tests.gpu_util import build_pair, log, make_caches

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kmr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_gemv_amd import kmr as k
    return k


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(kmr, dev, dims, kv_seed, inp, M, flags=0):
    """The same step through the workspace entry point and the static one, each on
    its own copy of the cache and of the position arrays."""
    B = len(inp["ids"])
    outs = []
    for static in (False, True):
        kv, _, _ = make_caches(dims, kv_seed, B, M, "device", host_rows=[])
        pos, cpos, fin = _dev(inp["positions"]), _dev(inp["cache_position"]), _dev(inp["finished"])
        nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        logits = torch.empty((B, dims.vocab), dtype=torch.float32, device="cuda")
        if static:
            dev.decode_step_static(kv, _dev(inp["ids"]), pos, cpos, nxt, finished=fin, logits=logits, advance=True,
                                   flags=flags)
        else:
            ws = kmr.Workspace(dev.cfg, B, M)
            dev.decode_step(kv, _dev(inp["ids"]), pos, cpos, nxt, ws, finished=fin, logits=logits, advance=True,
                            extra_flags=flags)
        torch.cuda.synchronize()
        if not static:
            assert ws.status() == 0
        outs.append((nxt.cpu(), logits.cpu(), kv.k.clone(), kv.v.clone(), pos.cpu(), cpos.cpu(), fin.cpu()))
        del kv
    return outs


def _same(outs, label):
    a, b = outs
    names = ("next", "logits", "k", "v", "positions", "cache_position", "finished")
    eq = [torch.equal(x, y) for x, y in zip(a, b)]
    log(f"  {label}: next {a[0].tolist()} vs {b[0].tolist()}; equal " + ", ".join(f"{n}={e}" for n, e in zip(names, eq)))
    assert all(eq)


def test_static_workspace_step_equals_workspace_step(kmr):
    w4, w1 = synth.WORKLOADS["batch4"], synth.WORKLOADS["step"]
    dims = w4.dims
    seed = synth.base_seed(w1)
    log("static workspace: building the 28-layer model (device draws)")
    layers = [synth.layer_weights(dims, seed, l, where="device", device="cuda") for l in range(dims.n_layers)]
    dev = kmr.DeviceModel(dims, layers, synth.model_globals(dims, seed, where="device", device="cuda"))
    del layers
    log("call 1: batch 4 (row 3 finished), persistent kernel")
    _same(_both(kmr, dev, dims, synth.base_seed(w4), synth.step_inputs(w4), w4.max_len), "batch 4")
    log("call 2: batch 1, the smaller input")
    _same(_both(kmr, dev, dims, synth.base_seed(w1), synth.step_inputs(w1), w1.max_len), "batch 1")


def test_static_workspace_other_layouts_and_recovery(kmr):
    w = synth.WORKLOADS["kv8"]
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)
    dev, dims = pair.dev, w.dims
    inp = synth.step_inputs(w)
    log("kv8: batch 4 persistent, then batch 2 per-phase, through both entry points")
    _same(_both(kmr, dev, dims, 5, inp, w.max_len), "kv8 batch 4")
    inp2 = {k: np.ascontiguousarray(v[..., :2]) for k, v in inp.items()}
    _same(_both(kmr, dev, dims, 6, inp2, w.max_len, flags=kmr.KMR_MULTI_KERNEL), "kv8 batch 2 per-phase")
    # a stalled step poisons the array; KMR_CLEAR_WORKSPACE recovers it
    kv, _, _ = make_caches(dims, 7, 4, w.max_len, "device", host_rows=[])
    args = lambda: (kv, _dev(inp["ids"]), _dev(inp["positions"]), _dev(inp["cache_position"]))
    nxt = torch.zeros(4, dtype=torch.int32, device="cuda")
    dev.decode_step_static(*args(), nxt, flags=kmr.KMR_TEST_STALL)
    torch.cuda.synchronize()
    log(f"  stalled: next {nxt.tolist()}")
    assert torch.all(nxt == -1)
    nxt.zero_()
    dev.decode_step_static(*args(), nxt)
    torch.cuda.synchronize()
    assert torch.all(nxt == -1)
    dev.decode_step_static(*args(), nxt, flags=kmr.KMR_CLEAR_WORKSPACE)
    torch.cuda.synchronize()
    log(f"  after KMR_CLEAR_WORKSPACE: next {nxt.tolist()}")
    assert torch.all(nxt >= 0)
    # too large for the array: refused on the host
    big = kmr.KVCache(dev.cfg, 1, 1, zero=True)
    big.desc.max_len = 1 << 22
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(kmr.KmrError) as e:
        dev.decode_step_static(big, one, torch.zeros((3, 1), dtype=torch.int32, device="cuda"), one.clone(),
                               nxt[:1].clone())
    assert e.value.code == kmr.KMR_ENOMEM

"""Batch invariance of the decode step, bit for bit ("The Ghost in the Batch":
the result of a row must not depend on which other rows share its batch).

A row decoded alone (batch 1) and the same row decoded among three others
(batch 4) must give identical logits, next token and cache writes.  The splits of
the attention depend on the row's own cache position only and every reduction
runs in a fixed order, so the two runs take the same arithmetic steps even though
they use different kernel instantiations.  This holds for the XCD-local
persistent kernel (the default) and for the per-phase kernels; the device-wide
persistent kernel agrees with them within the parity tolerance only.  At the
Qwen3-VL-2B text-decoder size the XCD-local kernel runs its constant-size form,
whose gate/up product goes through the matrix cores at every batch size; that case
is checked on the full 28-layer model.
"""
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
    from int4_weight_only_gemv_amd import kmr as m
    return m


@pytest.fixture(scope="module")
def kv8_pair(kmr):
    w = synth.WORKLOADS["kv8"]
    return build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)


def _run(kmr, pair, kv, ids, pos, cpos, fin, path):
    return _run_model(kmr, pair.dev, pair.dims.vocab, kv, ids, pos, cpos, fin, path)


def _run_model(kmr, dev, vocab, kv, ids, pos, cpos, fin, path):
    B = len(ids)
    ws = kmr.Workspace(dev.cfg, B, kv.k.shape[3])
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, vocab), dtype=torch.float32, device="cuda")
    dev.decode_step(kv, torch.from_numpy(ids).cuda(), torch.from_numpy(pos).cuda(),
                         torch.from_numpy(cpos).cuda(), nxt, ws, finished=torch.from_numpy(fin).cuda(),
                         logits=logits, multi_kernel=(path == "multi_kernel"),
                         device_wide=(path == "device_wide"), cooperative=(path == "cooperative"))
    torch.cuda.synchronize()
    assert ws.status() == 0
    return nxt.cpu().numpy(), logits.cpu()


@pytest.mark.parametrize("path", ["persistent", "multi_kernel"])
def test_row_alone_equals_row_in_batch(kmr, kv8_pair, path):
    w = synth.WORKLOADS["kv8"]
    M = w.max_len
    cpos = np.array([200, 0, 383, 127], np.int32)
    ids = np.array([11, 900, 37, 1500], np.int32)
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    fin = np.zeros(4, np.uint8)
    log(f"batch invariance ({path}): rows decoded in a batch of 4 vs alone, c = {cpos.tolist()}")
    kv4, _, _ = make_caches(w.dims, synth.base_seed(w), 4, M, "host")
    base_k, base_v = kv4.k.clone(), kv4.v.clone()
    next4, logits4 = _run(kmr, kv8_pair, kv4, ids, pos, cpos, fin, path)
    for r in (0, 2, 3):
        kv1, _, _ = make_caches(w.dims, synth.base_seed(w), 1, M, "host")
        kv1.k.copy_(base_k[:, r:r + 1])
        kv1.v.copy_(base_v[:, r:r + 1])
        next1, logits1 = _run(kmr, kv8_pair, kv1, ids[r:r + 1], pos[:, r:r + 1].copy(), cpos[r:r + 1],
                              fin[r:r + 1], path)
        same = torch.equal(logits1[0], logits4[r])
        log(f"  row {r}: next {int(next1[0])} vs {int(next4[r])}, logits bitwise equal: {same}")
        assert same
        assert next1[0] == next4[r]
        assert torch.equal(kv1.k[:, 0], kv4.k[:, r]) and torch.equal(kv1.v[:, 0], kv4.v[:, r])


def test_row_alone_equals_row_in_batch_full_size(kmr):
    w = synth.WORKLOADS["batch4"]
    dims, seed, M = w.dims, synth.base_seed(w), w.max_len
    log("batch invariance at full size: building the 28-layer model (device draws)")
    layers = [synth.layer_weights(dims, seed, l, where="device", device="cuda") for l in range(dims.n_layers)]
    glob = synth.model_globals(dims, seed, where="device", device="cuda")
    dev = kmr.DeviceModel(dims, layers, glob)
    del layers
    cpos = np.array([700, 0, 1023, 64], np.int32)
    ids = np.array([151, 9000, 37, 150000], np.int32)
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    fin = np.zeros(4, np.uint8)
    log(f"  rows decoded in a batch of 4 vs alone, c = {cpos.tolist()}")
    kv4, _, _ = make_caches(dims, seed, 4, M, "device", host_rows=[])
    base_k, base_v = kv4.k.clone(), kv4.v.clone()
    next4, logits4 = _run_model(kmr, dev, dims.vocab, kv4, ids, pos, cpos, fin, "persistent")
    for r in (0, 2, 3):
        kv1 = kmr.KVCache(dev.cfg, 1, M, zero=True)
        kv1.k.copy_(base_k[:, r:r + 1])
        kv1.v.copy_(base_v[:, r:r + 1])
        next1, logits1 = _run_model(kmr, dev, dims.vocab, kv1, ids[r:r + 1], pos[:, r:r + 1].copy(),
                                    cpos[r:r + 1], fin[r:r + 1], "persistent")
        same = torch.equal(logits1[0], logits4[r])
        log(f"  row {r}: next {int(next1[0])} vs {int(next4[r])}, logits bitwise equal: {same}, "
            f"max abs diff {float((logits1[0] - logits4[r]).abs().max()):.3e}, k cache equal "
            f"{torch.equal(kv1.k[:, 0], kv4.k[:, r])}, first differing k layer "
            f"{[l for l in range(dims.n_layers) if not torch.equal(kv1.k[l, 0], kv4.k[l, r])][:1]}")
        assert same
        assert next1[0] == next4[r]
        assert torch.equal(kv1.k[:, 0], kv4.k[:, r]) and torch.equal(kv1.v[:, 0], kv4.v[:, r])
    # the same batch under the runtime's cooperative launch: same kernel, same bits
    kvc = kmr.KVCache(dev.cfg, 4, M, zero=True)
    kvc.k.copy_(base_k)
    kvc.v.copy_(base_v)
    nextc, logitsc = _run_model(kmr, dev, dims.vocab, kvc, ids, pos, cpos, fin, "cooperative")
    log(f"  cooperative launch: logits bitwise equal to the plain launch: {torch.equal(logitsc, logits4)}")
    assert torch.equal(logitsc, logits4) and np.array_equal(nextc, next4)
    assert torch.equal(kvc.k, kv4.k) and torch.equal(kvc.v, kv4.v)

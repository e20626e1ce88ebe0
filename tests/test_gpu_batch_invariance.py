"""Batch invariance of the decode step, bit for bit ("The Ghost in the Batch":
the result of a row must not depend on which other rows share its batch; "The Fork
in the Code" and "The Fix: Three Options": a kernel choice made by batch size
changes a row's bits).

Default path.  A row decoded alone (batch 1) and the same row decoded among three
others (batch 4) give identical logits, next token and cache writes on every
persistent kernel and on the per-phase kernels: attention splits depend on the
row's own cache position only, every reduction runs in a fixed order, and the
device-wide kernel runs one instantiation for every batch of 1..4.  Across 4/5 and
8/9 the default path changes kernels, and rows then agree within the parity
tolerance only.

KMR_BATCH_INVARIANT.  One arithmetic form for every batch size: the same row at
batch 1, 4, 5, 9, 16 and 64 (full size) gives the same bits, and that form matches
the oracle within the parity tolerance.
"""
import numpy as np
import pytest
import torch

import oracle

from int4_weight_only_gemv_amd import synth
from tests.gpu_util import MARGIN, TOL, build_pair, log, make_caches, max_rel

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
                    device_wide=(path == "device_wide"), cooperative=(path == "cooperative"),
                    batch_invariant=(path == "batch_invariant"))
    torch.cuda.synchronize()
    assert ws.status() == 0
    return nxt.cpu().numpy(), logits.cpu()


@pytest.mark.parametrize("path", ["persistent", "device_wide", "multi_kernel", "batch_invariant"])
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


def _row_in_batches(kmr, dev, dims, seed, M, batches, target, place, vocab):
    """Decodes the row `target` (id, (t, h, w), cache position) with
    KMR_BATCH_INVARIANT inside batches of the given sizes, at batch row place(B),
    the other rows drawn at random; returns per batch size (next id, logits row,
    K and V written at the row's cache position)."""
    tid, tpos, tc = target
    base, _, _ = make_caches(dims, seed, 1, M, "device", host_rows=[])
    out = {}
    for B in batches:
        r = place(B)
        rng = np.random.default_rng(31 * B)
        cpos = rng.integers(0, M - 1, B).astype(np.int32)
        ids = rng.integers(0, vocab, B).astype(np.int32)
        pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
        cpos[r], ids[r], pos[:, r] = tc, tid, tpos
        kv, _, _ = make_caches(dims, seed + B, B, M, "device", host_rows=[])
        kv.k[:, r:r + 1].copy_(base.k)
        kv.v[:, r:r + 1].copy_(base.v)
        nxt, logits = _run_model(kmr, dev, vocab, kv, ids, np.ascontiguousarray(pos), cpos,
                                 np.zeros(B, np.uint8), "batch_invariant")
        out[B] = (int(nxt[r]), logits[r].clone(), kv.k[:, r, :, tc].clone(), kv.v[:, r, :, tc].clone())
        del kv
        torch.cuda.empty_cache()
    return out, base


def _assert_same_bits(out, label):
    ref_b = min(out)
    n0, l0, k0, v0 = out[ref_b]
    for B, (n, l, k, v) in out.items():
        same = torch.equal(l, l0) and torch.equal(k, k0) and torch.equal(v, v0) and n == n0
        log(f"  {label}: batch {B}: next {n}, logits/K/V bitwise equal to batch {ref_b}: {same}"
            + ("" if same else f", max logits diff {float((l - l0).abs().max()):.3e}"))
        assert same


def test_batch_invariant_flag_kv8(kmr, kv8_pair):
    """kv8 (group 64, hidden 512): the VALU GEMV and lm_head forms in 8-row tiles."""
    w = synth.WORKLOADS["kv8"]
    log("KMR_BATCH_INVARIANT, kv8: one row at batch 1, 3, 4, 5, 9, 16")
    target = (37, np.array([200, 100, 66], np.int32), 200)
    out, _ = _row_in_batches(kmr, kv8_pair.dev, w.dims, synth.base_seed(w), w.max_len, [1, 3, 4, 5, 9, 16],
                             target, lambda B: B - 1, w.dims.vocab)
    _assert_same_bits(out, "kv8")


def test_batch_invariant_flag_full_size(kmr):
    """The 28-layer model: the matrix-core GEMV and lm_head forms for every tile.
    The row sits at a different batch row each time (first, inside a tile, last);
    the form is checked against the oracle at batch 1."""
    w = synth.WORKLOADS["step"]
    dims, seed, M = w.dims, synth.base_seed(w), w.max_len
    log("KMR_BATCH_INVARIANT at full size: building the 28-layer model and its oracle copy")
    pair = build_pair(dims, seed, "device", with_globals=True)
    target = (151, np.array([700, 350, 233], np.int32), 700)
    places = {1: 0, 4: 3, 5: 2, 9: 8, 16: 9, 64: 37}
    out, base = _row_in_batches(kmr, pair.dev, dims, seed, M, [1, 4, 5, 9, 16, 64], target,
                                lambda B: places[B], dims.vocab)
    _assert_same_bits(out, "full size")
    # the invariant form against the oracle (batch 1, cache row as before the step)
    kh, vh = oracle.as_u16(base.k), oracle.as_u16(base.v)
    ref = pair.ora.decode_step(kh, vh, np.array([target[0]], np.int32), target[1].reshape(3, 1).copy(),
                               np.array([target[2]], np.int32))
    n1, l1, _, _ = out[1]
    err = max_rel(l1.numpy()[None], ref["logits"])
    log(f"  oracle: logits max_rel {err:.3e}, next {n1} vs {int(ref['next'][0])} (margin {float(ref['margin'][0]):.4f})")
    assert err <= TOL
    assert ref["margin"][0] <= MARGIN or n1 == int(ref["next"][0])

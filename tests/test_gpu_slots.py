"""GPU parity of the slot operations (kmr_kv_copy_row, kmr_slot_admit,
kmr_slot_retire) against oracle/slots.py, through the C ABI: the copies are bit
exact, only the copied positions of the destination row change, the slot state
matches, and a row moved into another slot of another cache decodes bit for bit
like the original (kaminari, section 08: continuous batching over per-row cache
slots; copy_row_from)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import slots
from int4_weight_only_gemv_amd import synth
from tests.gpu_util import build_pair, log, make_caches

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kmr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_gemv_amd import kmr as m
    return m


def _noise_kv(kmr, dims, batch, max_len, seed):
    kv = kmr.KVCache(kmr.make_config(dims), batch, max_len, zero=False)
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t in (kv.k, kv.v):
        t.view(torch.int16).copy_(torch.randint(-32768, 32767, t.shape, generator=g, device="cuda",
                                                dtype=torch.int32).to(torch.int16) & 0x7F7F)
    torch.cuda.synchronize()
    return kv


@pytest.mark.parametrize("name,shape", [
    ("kv8", dict(dst=(3, 40), src=(2, 48), n=[1, 37, 40])),
    ("step", dict(dst=(2, 1024), src=(1, 1024), n=[700, 1024])),
])
def test_kv_copy_row_bit_exact(kmr, name, shape):
    dims = synth.WORKLOADS[name].dims
    (bd, md), (bs, ms) = shape["dst"], shape["src"]
    dst = _noise_kv(kmr, dims, bd, md, 1)
    src = _noise_kv(kmr, dims, bs, ms, 2)
    for n in shape["n"]:
        for dr, sr in ((0, bs - 1), (bd - 1, 0)):
            log(f"kv_copy_row {name}: dst row {dr} of {bd}x{md}, src row {sr} of {bs}x{ms}, n={n}")
            kh, vh = oracle.as_u16(dst.k), oracle.as_u16(dst.v)
            slots.kv_copy_row(kh, vh, dr, oracle.as_u16(src.k), oracle.as_u16(src.v), sr, n)
            kmr.kv_copy_row(dst, dr, src, sr, n)
            torch.cuda.synchronize()
            assert np.array_equal(oracle.as_u16(dst.k), kh) and np.array_equal(oracle.as_u16(dst.v), vh)


def test_kv_copy_row_within_one_cache(kmr):
    dims = synth.WORKLOADS["kv8"].dims
    kv = _noise_kv(kmr, dims, 4, 64, 3)
    kh, vh = oracle.as_u16(kv.k), oracle.as_u16(kv.v)
    slots.kv_copy_row(kh, vh, 3, kh.copy(), vh.copy(), 1, 64)
    kmr.kv_copy_row(kv, 3, kv, 1, 64)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.as_u16(kv.k), kh) and np.array_equal(oracle.as_u16(kv.v), vh)


def test_slot_admit_and_retire(kmr):
    B = 4
    ids = torch.tensor([1, 2, 3, 4], dtype=torch.int32, device="cuda")
    pos = torch.arange(12, dtype=torch.int32, device="cuda").view(3, B).contiguous()
    cpos = torch.tensor([10, 11, 12, 13], dtype=torch.int32, device="cuda")
    fin = torch.tensor([0, 1, 0, 0], dtype=torch.uint8, device="cuda")
    h = [t.cpu().numpy().copy() for t in (ids, pos, cpos, fin)]
    slots.slot_admit(*h, 1, 777, (30, 31, 32), 29)
    slots.slot_retire(h[3], 2)
    kmr.slot_admit(ids, pos, cpos, fin, 1, 777, (30, 31, 32), 29)
    kmr.slot_retire(fin, 2)
    torch.cuda.synchronize()
    for t, ref in zip((ids, pos, cpos, fin), h):
        assert np.array_equal(t.cpu().numpy(), ref)


def test_moved_row_decodes_like_the_original(kmr):
    """A row decoded in its own cache (batch 4) and the same row after being copied
    into slot 1 of a batch-2 cache and admitted there: identical logits and token
    (the persistent kernel is batch invariant, so this holds bit for bit)."""
    w = synth.WORKLOADS["kv8"]
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)
    M = w.max_len
    cpos = np.array([200, 0, 383, 127], np.int32)
    ids = np.array([11, 900, 37, 1500], np.int32)
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    kv4, _, _ = make_caches(w.dims, synth.base_seed(w), 4, M, "host")
    kv2, _, _ = make_caches(w.dims, synth.base_seed(w) + 5, 2, M, "host")
    r = 2
    kmr.kv_copy_row(kv2, 1, kv4, r, int(cpos[r]))     # positions [0, c): what the step reads
    ids2 = torch.tensor([5, 0], dtype=torch.int32, device="cuda")
    pos2 = torch.tensor([[40, 0], [20, 0], [13, 0]], dtype=torch.int32, device="cuda")
    cpos2 = torch.tensor([40, 0], dtype=torch.int32, device="cuda")
    fin2 = torch.tensor([0, 1], dtype=torch.uint8, device="cuda")
    kmr.slot_admit(ids2, pos2, cpos2, fin2, 1, int(ids[r]), tuple(int(p) for p in pos[:, r]), int(cpos[r]))

    def run(kv, t_ids, t_pos, t_cpos, t_fin, B):
        ws = kmr.Workspace(pair.dev.cfg, B, M)
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        logits = torch.empty((B, w.dims.vocab), dtype=torch.float32, device="cuda")
        pair.dev.decode_step(kv, t_ids, t_pos, t_cpos, nxt, ws, finished=t_fin, logits=logits)
        torch.cuda.synchronize()
        assert ws.status() == 0
        return nxt.cpu(), logits.cpu()

    n4, l4 = run(kv4, torch.from_numpy(ids).cuda(), torch.from_numpy(pos).cuda(),
                 torch.from_numpy(cpos).cuda(), torch.zeros(4, dtype=torch.uint8, device="cuda"), 4)
    n2, l2 = run(kv2, ids2, pos2, cpos2, fin2, 2)
    log(f"moved row: token {int(n2[1])} vs {int(n4[r])}, logits equal {torch.equal(l2[1], l4[r])}")
    assert torch.equal(l2[1], l4[r]) and int(n2[1]) == int(n4[r])
    assert torch.equal(kv2.k[:, 1, :, : int(cpos[r]) + 1], kv4.k[:, r, :, : int(cpos[r]) + 1])

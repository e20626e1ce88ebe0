"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (set by the arithmetic: bf16 storage, fp16 GEMV inputs, fp32 accumulation
against an fp64 oracle): packed int4 codes and scale/zero bit-exact; cache bytes
outside the written slots bit-identical; next-token ids equal wherever the
oracle's top-2 logit margin exceeds 1e-2; hidden states, logits and written K/V
within max relative error 2e-2 (largest absolute error over the largest
reference magnitude, per row).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_weight_only_gemv_amd import synth
from tests.gpu_util import (MARGIN, TOL, bf16_host, build_pair, log, make_caches, max_rel,
                            to_device_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kmr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_gemv_amd import kmr as k
    return k


# ------------------------------------------------------------------ quantizer

def _crafted_groups(G):
    ties = [0.0, 15 / 64] + [(j + 0.5) / 64 for j in range(15)]
    ties += [0.0] * (G - len(ties))
    scale_tie = list(np.linspace(-15 / 256, 15, G))
    scale_tie[0], scale_tie[-1] = -15 / 256, 15.0
    return np.array([ties, scale_tie, [0.37109375] * G, [0.0] * G, [-2.5] * G], np.float32)


@pytest.mark.parametrize("N,K,G,std", [
    (512, 256, 64, 0.02), (256, 768, 64, 0.02), (37, 384, 128, 1.0),
    (4096, 2048, 128, 0.02), (2048, 6144, 128, 0.02), (64, 512, 128, 300.0), (5, 2, 2, 1.0),
])
def test_quantize_bit_exact(kmr, N, K, G, std):
    log(f"quantize N={N} K={K} G={G} std={std}")
    r = np.random.default_rng(N * 7 + K)
    w = (r.standard_normal((N, K)).astype(np.float32) * np.float32(std))
    if K % G == 0 and G >= 32 and N >= 5:
        c = _crafted_groups(G)
        w[:5, :G] = c
    wb = torch.from_numpy(w).to(torch.bfloat16)
    p_ref, s_ref = oracle.quantize_int4(oracle.as_u16(wb), G)
    p, s = kmr.quantize_int4(wb.cuda(), G)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), p_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref)


# ------------------------------------------------------------------ one layer

def _layer_case(kmr, dims, seed, batch, M, cpos, pos, x0):
    pair = build_pair(dims, seed, "host", with_globals=False)
    kv, kh, vh = make_caches(dims, seed, batch, M, "host")
    k0, v0 = kh.copy(), vh.copy()
    cfg = kmr.make_config(dims)
    ws = kmr.Workspace(cfg, batch, M)
    x_dev = torch.from_numpy(x0.astype(np.float32)).cuda()
    pos_d = torch.from_numpy(pos).cuda()
    cpos_d = torch.from_numpy(cpos).cuda()
    pair.dev.decode_layer(0, kv, x_dev, pos_d, cpos_d, ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    x_ref = x0.astype(np.float32).astype(np.float64).copy()
    pair.ora.decode_layer(0, kh, vh, x_ref, pos, cpos)
    x_got = x_dev.cpu().numpy()
    err = max_rel(x_got, x_ref)
    kg = oracle.as_u16(kv.k)
    vg = oracle.as_u16(kv.v)
    mask = np.zeros(kg.shape, bool)
    for b in range(batch):
        mask[:, b, :, cpos[b], :] = True
    kerr = max_rel(bf16_host(kg[mask]).reshape(-1, dims.head_dim), bf16_host(kh[mask]).reshape(-1, dims.head_dim))
    verr = max_rel(bf16_host(vg[mask]).reshape(-1, dims.head_dim), bf16_host(vh[mask]).reshape(-1, dims.head_dim))
    log(f"  hidden max_rel={err:.3e}  k={kerr:.3e}  v={verr:.3e}")
    assert err <= TOL and kerr <= TOL and verr <= TOL
    assert np.array_equal(kg[~mask], k0[~mask]) and np.array_equal(vg[~mask], v0[~mask])
    return err


@pytest.mark.parametrize("cpos", [0, 1, 16, 63, 64, 65, 127])
def test_decode_layer_tiny(kmr, cpos):
    w = synth.WORKLOADS["tiny"]
    log(f"decode_layer tiny cache_position={cpos}")
    pos = np.array([[cpos], [3], [60]], np.int32)
    x0 = synth.hidden_input(w.dims, 5, 1).numpy()
    _layer_case(kmr, w.dims, synth.base_seed(w), 1, w.max_len, np.array([cpos], np.int32), pos, x0)


def test_decode_layer_tiny_ragged_batch(kmr):
    w = synth.WORKLOADS["tiny"]
    log("decode_layer tiny batch 3 ragged")
    cpos = np.array([0, 77, 127], np.int32)
    pos = np.array([[0, 77, 127], [5, 1, 2], [9, 9, 9]], np.int32)
    x0 = synth.hidden_input(w.dims, 6, 3).numpy()
    _layer_case(kmr, w.dims, synth.base_seed(w), 3, w.max_len, cpos, pos, x0)


def test_decode_layer_full_size(kmr):
    w = synth.WORKLOADS["layer"]
    inp = synth.step_inputs(w)
    log(f"decode_layer full size cache_position={inp['cache_position']}")
    x0 = synth.hidden_input(w.dims, synth.base_seed(w), 1).numpy()
    _layer_case(kmr, w.dims, synth.base_seed(w), 1, w.max_len, inp["cache_position"],
                inp["positions"], x0)


def test_decode_layer_full_size_edges(kmr):
    w = synth.WORKLOADS["layer"]
    log("decode_layer full size, batch 4 at split edges")
    cpos = np.array([0, 63, 64, 1023], np.int32)
    pos = np.array([[0, 63, 64, 1023], [0, 1, 2, 3], [7, 7, 7, 7]], np.int32)
    x0 = synth.hidden_input(w.dims, 9, 4).numpy()
    _layer_case(kmr, w.dims, synth.base_seed(w), 4, w.max_len, cpos, pos, x0)


@pytest.mark.parametrize("batch", [11, 16])
def test_decode_layer_full_size_matrix_core_tiles(kmr, batch):
    """Batch tiles of 9..16 rows with group 128 take the matrix-core GEMV (the QKV and
    gate-up products; O and down run in 8-row tiles on the VALU): a padded tile
    (B = 11, with an 8 + 3-row split of the others) and a full one (B = 16)."""
    w = synth.WORKLOADS["layer"]
    log(f"decode_layer full size, batch {batch} (matrix-core GEMV tiles)")
    rng = np.random.default_rng(500 + batch)
    cpos = rng.integers(0, w.max_len, batch).astype(np.int32)
    cpos[0], cpos[-1] = 0, w.max_len - 1
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    x0 = synth.hidden_input(w.dims, 40 + batch, batch).numpy()
    _layer_case(kmr, w.dims, synth.base_seed(w), batch, w.max_len, cpos, pos, x0)


# ------------------------------------------------------------------ whole step

def _check_step(got_next, got_logits, ref, label):
    lerr = max_rel(got_logits, ref["logits"])
    agree = got_next == ref["next"]
    decisive = ref["margin"] > MARGIN
    log(f"  {label}: logits max_rel={lerr:.3e} tokens={got_next.tolist()} ref={ref['next'].tolist()} "
        f"margins={np.round(ref['margin'], 4).tolist()}")
    assert lerr <= TOL
    assert np.all(agree | ~decisive)


PATHS = ["persistent", "cooperative", "device_wide", "multi_kernel"]


def _path_flags(path):
    return {"multi_kernel": path == "multi_kernel", "device_wide": path == "device_wide",
            "cooperative": path == "cooperative"}


def _step_case(kmr, pair, kv, kh, vh, inp, M, steps=1, advance=False, path="persistent"):
    dims = pair.dims
    B = len(inp["ids"])
    cfg = pair.dev.cfg
    ws = kmr.Workspace(cfg, B, M)
    ids = inp["ids"].copy()
    pos, cpos, fin = inp["positions"].copy(), inp["cache_position"].copy(), inp["finished"].copy()
    pos_d, cpos_d = torch.from_numpy(pos).cuda(), torch.from_numpy(cpos).cuda()
    fin_d = torch.from_numpy(fin).cuda()
    nxt_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits_d = torch.empty((B, dims.vocab), dtype=torch.float32, device="cuda")
    written = set()
    for step in range(steps):
        ids_d = torch.from_numpy(ids).cuda()
        written.update((b, int(c)) for b, c in enumerate(cpos) if 0 <= c < M)
        pair.dev.decode_step(kv, ids_d, pos_d, cpos_d, nxt_d, ws, finished=fin_d, logits=logits_d,
                             advance=advance, **_path_flags(path))
        torch.cuda.synchronize()
        ref = pair.ora.decode_step(kh, vh, ids, pos, cpos, finished=fin, advance=advance)
        _check_step(nxt_d.cpu().numpy(), logits_d.cpu().numpy(), ref, f"step {step}")
        assert np.array_equal(pos_d.cpu().numpy(), pos)
        assert np.array_equal(cpos_d.cpu().numpy(), cpos)
        assert np.array_equal(fin_d.cpu().numpy(), fin)
        ids = ref["next"].astype(np.int32)        # lockstep: both sides take the oracle's token
    assert ws.status() == 0
    if kh.shape[1] == B:
        _check_cache(kv, kh, vh, written)
    return ref


def _check_cache(kv, kh, vh, written):
    """Only the slots the steps wrote may differ from the oracle's cache (bytes);
    those hold the same K/V within tolerance."""
    for dev_t, ref in ((kv.k, kh), (kv.v, vh)):
        got = oracle.as_u16(dev_t)
        diff = np.any(got != ref, axis=-1)                 # [L][B][Hkv][M]
        for l, b, g, m in zip(*np.nonzero(diff)):
            assert (int(b), int(m)) in written, f"slot {(l, b, g, m)} changed but was not written"
        for b, m in written:
            err = max_rel(bf16_host(got[:, b, :, m, :]).reshape(-1, got.shape[-1]),
                          bf16_host(ref[:, b, :, m, :]).reshape(-1, got.shape[-1]))
            assert err <= TOL, f"row {b} slot {m}: K/V max_rel {err:.3e}"


@pytest.mark.parametrize("path", PATHS)
def test_decode_step_tiny(kmr, path):
    w = synth.WORKLOADS["tiny"]
    log(f"decode_step tiny ({path})")
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), 1, w.max_len, "host")
    _step_case(kmr, pair, kv, kh, vh, synth.step_inputs(w), w.max_len, path=path)


@pytest.mark.parametrize("path", PATHS)
def test_decode_step_tiny_batch_advance(kmr, path):
    w = synth.WORKLOADS["tiny"]
    log(f"decode_step tiny batch 3, finished row, advance to the last slot ({path})")
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), 3, w.max_len, "host")
    inp = {"ids": np.array([5, 6, 7], np.int32),
           "positions": np.array([[10, 125, 3], [11, 1, 3], [12, 2, 3]], np.int32),
           "cache_position": np.array([10, 125, 3], np.int32),
           "finished": np.array([0, 0, 1], np.uint8)}
    _step_case(kmr, pair, kv, kh, vh, inp, w.max_len, steps=4, advance=True, path=path)


@pytest.fixture(scope="module")
def kv8_pair(kmr):
    w = synth.WORKLOADS["kv8"]
    return build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)


@pytest.mark.parametrize("path", PATHS)
def test_decode_step_kv8_batch4_advance(kmr, kv8_pair, path):
    """8 kv heads (one per XCD): cache positions on split edges and the last slot."""
    w = synth.WORKLOADS["kv8"]
    log(f"decode_step kv8 batch 4, c = 0/127/128/383, 4 advancing steps ({path})")
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "host")
    _step_case(kmr, kv8_pair, kv, kh, vh, synth.step_inputs(w), w.max_len, steps=4, advance=True,
               path=path)


@pytest.mark.parametrize("batch,cpos", [(1, [255]), (2, [3, 250]), (3, [129, 0, 300])])
def test_decode_step_kv8_small_batches(kmr, kv8_pair, batch, cpos):
    w = synth.WORKLOADS["kv8"]
    log(f"decode_step kv8 batch {batch}, c = {cpos}, 3 advancing steps (persistent)")
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w) + batch, batch, w.max_len, "host")
    c = np.array(cpos, np.int32)
    inp = {"ids": np.arange(batch, dtype=np.int32) * 37 + 5,
           "positions": np.stack([c, c // 2, c // 3]).astype(np.int32),
           "cache_position": c, "finished": np.zeros(batch, np.uint8)}
    _step_case(kmr, kv8_pair, kv, kh, vh, inp, w.max_len, steps=3, advance=True)


@pytest.fixture(scope="module")
def full_pair(kmr):
    w = synth.WORKLOADS["step"]
    log("building the 28-layer model (device draws, oracle quantizes its host copy)")
    return build_pair(w.dims, synth.base_seed(w), "device", with_globals=True)


@pytest.mark.parametrize("path", PATHS)
def test_decode_step_full(kmr, full_pair, path):
    w = synth.WORKLOADS["step"]
    log(f"decode_step 28 layers, batch 1, cache_position 700 ({path})")
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), 1, w.max_len, "device")
    _step_case(kmr, full_pair, kv, kh, vh, synth.step_inputs(w), w.max_len, path=path)


def test_prefill_full_size_matches_oracle_decode(kmr, full_pair):
    """kmr_prefill of 70 tokens at the full model size (one chunk: one ragged 128-token
    tile of each matrix-core GEMM, one ragged attention tile per kv head and 32 tokens)
    against the oracle's decode step run
    token by token over the same cache row (kaminari page, section 04: prefill fills
    the static cache that decode extends): the last token's logits and token, every
    written K/V slot, and no other slot."""
    w = synth.WORKLOADS["step"]
    dims, M, T = w.dims, w.max_len, 70
    rng = np.random.default_rng(T)
    tokens = rng.integers(0, dims.vocab, T).astype(np.int32)
    pos3 = np.ascontiguousarray(np.arange(T, dtype=np.int32)[None].repeat(3, 0))
    log(f"prefill {T} tokens, 28 layers, from position 0 (oracle: {T} decode steps)")
    kv, kh, vh = make_caches(dims, synth.base_seed(w) + T, 1, M, "device")
    ws = kmr.Workspace.for_prefill(full_pair.dev.cfg, T, M)
    nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    logits = torch.empty(dims.vocab, dtype=torch.float32, device="cuda")
    full_pair.dev.prefill(kv, 0, torch.from_numpy(tokens).cuda(), torch.from_numpy(pos3).cuda(), 0, nxt, ws,
                          logits=logits)
    torch.cuda.synchronize()
    assert ws.status() == 0
    kc, vc = kh.copy(), vh.copy()
    for t in range(T):
        ref = full_pair.ora.decode_step(kc, vc, tokens[t:t + 1], np.ascontiguousarray(pos3[:, t:t + 1]),
                                        np.array([t], np.int32))
    err = max_rel(logits.cpu().numpy()[None], ref["logits"])
    got_next = int(nxt.cpu()[0])
    log(f"  logits max_rel={err:.3e} next={got_next} oracle={int(ref['next'][0])} "
        f"margin={float(ref['margin'][0]):.4f}")
    assert err <= TOL
    if ref["margin"][0] > MARGIN:
        assert got_next == int(ref["next"][0])
    D = dims.head_dim
    for dev_t, want, before in ((kv.k, kc, kh), (kv.v, vc, vh)):
        got = oracle.as_u16(dev_t)
        e = max_rel(bf16_host(got[:, 0, :, :T]).reshape(-1, D), bf16_host(want[:, 0, :, :T]).reshape(-1, D))
        log(f"  written K/V max_rel={e:.3e}")
        assert e <= TOL
        assert np.array_equal(got[:, :, :, T:], before[:, :, :, T:])


def test_persistent_and_per_phase_paths_agree(kmr, full_pair):
    w = synth.WORKLOADS["batch4"]
    log("persistent step kernels vs per-phase kernels, batch 4, 3 advancing steps")
    inp = synth.step_inputs(w)
    outs = []
    for path in PATHS:
        kv, _, _ = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "device", host_rows=[0])
        ws = kmr.Workspace(full_pair.dev.cfg, w.batch, w.max_len)
        ids = torch.from_numpy(inp["ids"]).cuda()
        pos, cpos = torch.from_numpy(inp["positions"]).cuda(), torch.from_numpy(inp["cache_position"]).cuda()
        fin = torch.from_numpy(inp["finished"]).cuda()
        nxt = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
        logits = torch.empty((w.batch, w.dims.vocab), dtype=torch.float32, device="cuda")
        seq = []
        for _ in range(3):
            full_pair.dev.decode_step(kv, ids, pos, cpos, nxt, ws, finished=fin, logits=logits,
                                      advance=True, **_path_flags(path))
            seq.append((nxt.clone(), logits.clone()))
            ids = nxt.clone()
        torch.cuda.synchronize()
        assert ws.status() == 0
        outs.append((seq, kv.k.clone(), kv.v.clone(), pos.cpu(), cpos.cpu(), fin.cpu()))
        del kv
    sa, ka, va, pa, ca, fa = outs[-1]          # per-phase kernels as the reference
    for sb, kb, vb, pb, cb, fb in outs[:-1]:
        for (na, la), (nb, lb) in zip(sa, sb):
            err = max_rel(la.cpu().numpy(), lb.cpu().numpy())
            log(f"  logits max_rel between paths {err:.3e}; tokens {na.tolist()} vs {nb.tolist()}")
            assert err <= TOL
        assert torch.equal(pa, pb) and torch.equal(ca, cb) and torch.equal(fa, fb)
        for xa, xb in ((ka, kb), (va, vb)):
            assert max_rel(xa.float().cpu().numpy().reshape(-1, 128),
                           xb.float().cpu().numpy().reshape(-1, 128)) <= TOL


def test_decode_step_batch4_lockstep(kmr, full_pair):
    """The batch-4 workload as specified: 64 consecutive greedy steps with on-device
    advance (row 3 finished throughout; rows whose cache position would reach
    max_len finish by length), both sides fed the oracle's token every step."""
    w = synth.WORKLOADS["batch4"]
    log(f"decode_step 28 layers, batch 4 (row 3 finished), {w.steps} lockstep steps with advance")
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "device")
    _step_case(kmr, full_pair, kv, kh, vh, synth.step_inputs(w), w.max_len, steps=w.steps, advance=True)


def test_decode_step_long16_every_row(kmr, full_pair):
    """The long-context workload (16 rows, 8192-slot cache, cache positions 2048..8000)
    over 4 advancing steps, every row checked: the rows go to the oracle in groups of
    four, each group over all 4 steps on a freshly drawn cache (the oracle holds 4 of
    the 16 rows at a time).  Rows of the group take the oracle's token; the others
    take their own."""
    w = synth.WORKLOADS["long16"]
    B, M, steps = w.batch, w.max_len, 4
    inp = synth.step_inputs(w)
    for g in range(B // 4):
        rows = list(range(4 * g, 4 * g + 4))
        log(f"decode_step 28 layers, batch 16, max_len 8192, {steps} steps; oracle on rows {rows}")
        kv, kh, vh = make_caches(w.dims, synth.base_seed(w), B, M, "device", host_rows=rows)
        ws = kmr.Workspace(full_pair.dev.cfg, B, M)
        ids = inp["ids"].copy()
        pos_d = torch.from_numpy(inp["positions"].copy()).cuda()
        cpos_d = torch.from_numpy(inp["cache_position"].copy()).cuda()
        rpos = np.ascontiguousarray(inp["positions"][:, rows])
        rcpos = inp["cache_position"][rows].copy()
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        logits = torch.empty((B, w.dims.vocab), dtype=torch.float32, device="cuda")
        for s in range(steps):
            full_pair.dev.decode_step(kv, torch.from_numpy(ids).cuda(), pos_d, cpos_d, nxt, ws, logits=logits,
                                      advance=True)
            torch.cuda.synchronize()
            ref = full_pair.ora.decode_step(kh, vh, ids[rows], rpos, rcpos, advance=True)
            got = nxt.cpu().numpy()
            _check_step(got[rows], logits.cpu().numpy()[rows], ref, f"step {s}")
            assert np.array_equal(pos_d.cpu().numpy()[:, rows], rpos)
            assert np.array_equal(cpos_d.cpu().numpy()[rows], rcpos)
            ids = got.astype(np.int32)
            ids[rows] = ref["next"]
        assert ws.status() == 0
        del kv, kh, vh
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ graph capture

def _graph_lockstep(kmr, pair, kv, kh, vh, inp, M, flags, replays=16):
    """One kmr_decode_step with KMR_ADVANCE captured in a HIP graph (through torch's
    graph capture on a side stream) and replayed `replays` times; before each
    replay the oracle's token goes into the captured token buffer (lockstep), and
    after it tokens, logits, positions and cache positions are checked."""
    B = len(inp["ids"])
    ws = kmr.Workspace(pair.dev.cfg, B, M)
    ids = inp["ids"].copy()
    pos, cpos, fin = inp["positions"].copy(), inp["cache_position"].copy(), inp["finished"].copy()
    ids_d = torch.from_numpy(ids.copy()).cuda()
    pos_d, cpos_d = torch.from_numpy(pos.copy()).cuda(), torch.from_numpy(cpos.copy()).cuda()
    fin_d = torch.from_numpy(fin.copy()).cuda()
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, pair.dims.vocab), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pair.dev.decode_step(kv, ids_d, pos_d, cpos_d, nxt, ws, finished=fin_d, logits=logits, advance=True,
                             **flags)
    torch.cuda.synchronize()
    # capture runs nothing: state is as before
    assert np.array_equal(cpos_d.cpu().numpy(), cpos)
    written = set()
    for r in range(replays):
        ids_d.copy_(torch.from_numpy(ids))
        written.update((b, int(c)) for b, c in enumerate(cpos) if 0 <= c < M)
        graph.replay()
        torch.cuda.synchronize()
        ref = pair.ora.decode_step(kh, vh, ids, pos, cpos, finished=fin, advance=True)
        _check_step(nxt.cpu().numpy(), logits.cpu().numpy(), ref, f"replay {r}")
        assert np.array_equal(pos_d.cpu().numpy(), pos)
        assert np.array_equal(cpos_d.cpu().numpy(), cpos)
        assert np.array_equal(fin_d.cpu().numpy(), fin)
        ids = ref["next"].astype(np.int32)
    assert ws.status() == 0
    del graph
    return written


@pytest.mark.parametrize("path", ["persistent", "device_scope_stores"])
def test_decode_step_full_graph_replay(kmr, full_pair, path):
    w = synth.WORKLOADS["step"]
    log(f"decode_step 28 layers, batch 1, captured once, 16 replays in lockstep ({path})")
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), 1, w.max_len, "device")
    flags = {"device_scope_stores": path == "device_scope_stores"}
    written = _graph_lockstep(kmr, full_pair, kv, kh, vh, synth.step_inputs(w), w.max_len, flags)
    _check_cache(kv, kh, vh, written)


@pytest.mark.parametrize("path", ["persistent", "device_scope_stores", "device_wide", "multi_kernel"])
def test_decode_step_kv8_graph_replay(kmr, kv8_pair, path):
    w = synth.WORKLOADS["kv8"]
    log(f"decode_step kv8 batch 4, captured once, 16 replays in lockstep ({path})")
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "host")
    flags = {"device_scope_stores": path == "device_scope_stores", "device_wide": path == "device_wide",
             "multi_kernel": path == "multi_kernel"}
    written = _graph_lockstep(kmr, kv8_pair, kv, kh, vh, synth.step_inputs(w), w.max_len, flags)
    _check_cache(kv, kh, vh, written)


# ------------------------------------------------------------------ full size: failure paths, magnitudes, M-RoPE layout

@pytest.mark.parametrize("wl", ["step", "batch4"])
def test_full_stalled_step_fails_hard_then_recovers(kmr, full_pair, wl):
    """The constant-size persistent kernel (batch 1 and batch 4): a stalled step
    writes -1 and advances nothing, a plain step on the same workspace is refused,
    and a re-initialised workspace decodes like the oracle."""
    from tests.test_gpu_robustness import stall_then_recover
    log(f"decode_step 28 layers, {wl}: stalled step, refusal, re-initialised workspace")
    stall_then_recover(kmr, full_pair, synth.WORKLOADS[wl], {})


def test_full_residual_outliers_1e5(kmr, full_pair):
    """The constant-size kernel at batch 4 with residual-stream channels of 3e4..1.2e5
    (embedding columns set to those values for every token), 2 lockstep steps."""
    w = synth.WORKLOADS["batch4"]
    log("decode_step 28 layers, batch 4, residual outlier channels up to 1.2e5, 2 steps")
    outl = {3: 6.0e4, 1000: -1.0e5, 1025: 3.1e4, 2047: 1.2e5}
    emb_d, emb_h = full_pair.dev.globals["embed"], full_pair.ora.g["embed"]
    saved = {ch: (emb_d[:, ch].clone(), emb_h[:, ch].copy()) for ch in outl}
    try:
        for ch, val in outl.items():
            emb_d[:, ch] = val
            emb_h[:, ch] = oracle.as_u16(torch.tensor([val], dtype=torch.bfloat16))[0]
        kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "device")
        _step_case(kmr, full_pair, kv, kh, vh, synth.step_inputs(w), w.max_len, steps=2, advance=True)
    finally:
        for ch, (d, h) in saved.items():
            emb_d[:, ch] = d
            emb_h[:, ch] = h


def test_full_contiguous_mrope(kmr, full_pair):
    """The constant-size kernel with the contiguous M-RoPE layout (mrope_interleaved = 0)
    on the batch-4 workload, whose rows have distinct t, h, w positions."""
    w = synth.WORKLOADS["batch4"]
    log("decode_step 28 layers, batch 4, contiguous M-RoPE sections, 2 steps")
    full_pair.dev.cfg.mrope_interleaved = 0
    full_pair.ora.cdims.mrope_interleaved = 0
    try:
        inp = synth.step_inputs(w)
        log(f"  positions (t, h, w per row): {inp['positions'].T.tolist()}")
        kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "device")
        _step_case(kmr, full_pair, kv, kh, vh, inp, w.max_len, steps=2, advance=True)
    finally:
        full_pair.dev.cfg.mrope_interleaved = 1
        full_pair.ora.cdims.mrope_interleaved = 1


@pytest.mark.parametrize("B,rows", [(40, [0, 17, 39]), (64, [0, 33, 63])])
def test_decode_step_large_batch_sampled_rows(kmr, full_pair, B, rows):
    """Batches above 16 run in 16-row tiles (40 = 16 + 16 + 8, the last tile on the
    VALU GEMV and a ragged lm_head tile; 64 = KMR_MAX_BATCH, four full tiles); the
    oracle checks rows from different tiles."""
    dims = full_pair.dims
    M = 1024
    log(f"decode_step 28 layers, batch {B}, max_len {M}; oracle on rows {rows}")
    rng = np.random.default_rng(4000 + B)
    cpos = rng.integers(0, M - 1, B).astype(np.int32)
    ids = rng.integers(0, dims.vocab, B).astype(np.int32)
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    kv, kh, vh = make_caches(dims, synth.base_seed(synth.WORKLOADS["step"]), B, M, "device", host_rows=rows)
    ws = kmr.Workspace(full_pair.dev.cfg, B, M)
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, dims.vocab), dtype=torch.float32, device="cuda")
    full_pair.dev.decode_step(kv, torch.from_numpy(ids).cuda(), torch.from_numpy(pos).cuda(),
                              torch.from_numpy(cpos).cuda(), nxt, ws, logits=logits)
    torch.cuda.synchronize()
    assert ws.status() == 0
    ref = full_pair.ora.decode_step(kh, vh, ids[rows], np.ascontiguousarray(pos[:, rows]), cpos[rows].copy())
    _check_step(nxt.cpu().numpy()[rows], logits.cpu().numpy()[rows], ref, "rows")
    del kv


@pytest.mark.parametrize("batch", [1, 4, 16])
def test_decode_step_tokens_without_logits_buffer(kmr, full_pair, batch):
    """Without a logits buffer the lm_head loops take their store-free form; the
    tokens must be those of the run that also writes the logits (same arithmetic)."""
    dims, M = full_pair.dims, 1024
    log(f"decode_step batch {batch}: tokens with and without a logits buffer")
    rng = np.random.default_rng(7000 + batch)
    cpos = rng.integers(0, M - 1, batch).astype(np.int32)
    ids = rng.integers(0, dims.vocab, batch).astype(np.int32)
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    got = []
    for with_logits in (True, False):
        kv, _, _ = make_caches(dims, synth.base_seed(synth.WORKLOADS["step"]), batch, M, "device", host_rows=[])
        ws = kmr.Workspace(full_pair.dev.cfg, batch, M)
        nxt = torch.zeros(batch, dtype=torch.int32, device="cuda")
        logits = torch.empty((batch, dims.vocab), dtype=torch.float32, device="cuda") if with_logits else None
        full_pair.dev.decode_step(kv, torch.from_numpy(ids).cuda(), torch.from_numpy(pos).cuda(),
                                  torch.from_numpy(cpos).cuda(), nxt, ws, logits=logits)
        torch.cuda.synchronize()
        assert ws.status() == 0
        got.append(nxt.cpu().numpy())
        del kv
    log(f"  tokens {got[0].tolist()} vs {got[1].tolist()}")
    assert np.array_equal(got[0], got[1])


@pytest.mark.parametrize("batch", [6, 16])
def test_shared_prefix_step_equals_plain_step(kmr, full_pair, batch):
    """kmr_decode_step_prefix (the prefix's K/V read once for all rows) gives the bits
    of the plain per-phase step when the rows share that K/V: tokens, logits and the
    whole cache.  Row 0 sits exactly at the end of the prefix, row 1 inside it (it
    keeps the plain path), the others past it."""
    dims, M, P = full_pair.dims, 1024, 512
    log(f"decode_step batch {batch}: shared prefix of {P} positions vs the plain per-phase step")
    rng = np.random.default_rng(9000 + batch)
    cpos = rng.integers(P, M - 1, batch).astype(np.int32)
    cpos[0], cpos[1] = P, 100
    ids = rng.integers(0, dims.vocab, batch).astype(np.int32)
    pos = np.stack([cpos, cpos // 2, cpos // 3]).astype(np.int32)
    got = []
    for prefix in (0, P):
        kv, _, _ = make_caches(dims, synth.base_seed(synth.WORKLOADS["step"]), batch, M, "device", host_rows=[])
        kv.k[:, :, :, :P] = kv.k[:, 0:1, :, :P].clone()   # [L][B][Hkv][M][D]: every row holds row 0's prefix
        kv.v[:, :, :, :P] = kv.v[:, 0:1, :, :P].clone()
        ws = kmr.Workspace(full_pair.dev.cfg, batch, M)
        nxt = torch.zeros(batch, dtype=torch.int32, device="cuda")
        logits = torch.empty((batch, dims.vocab), dtype=torch.float32, device="cuda")
        full_pair.dev.decode_step(kv, torch.from_numpy(ids).cuda(), torch.from_numpy(pos).cuda(),
                                  torch.from_numpy(cpos).cuda(), nxt, ws, logits=logits, multi_kernel=True,
                                  shared_prefix=prefix)
        torch.cuda.synchronize()
        assert ws.status() == 0
        got.append((nxt.cpu(), logits.cpu(), kv.k.clone(), kv.v.clone()))
        del kv
    (n0, l0, k0, v0), (n1, l1, k1, v1) = got
    log(f"  tokens {n0.tolist()} vs {n1.tolist()}; logits bitwise equal {torch.equal(l0, l1)}")
    assert torch.equal(n0, n1) and torch.equal(l0, l1)
    assert torch.equal(k0, k1) and torch.equal(v0, v1)


# ------------------------------------------------------------------ error paths

def test_out_of_range_cache_position_sets_status_and_writes_nothing(kmr):
    w = synth.WORKLOADS["tiny"]
    log("decode_layer with cache_position == max_len")
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=False)
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), 2, w.max_len, "host")
    ws = kmr.Workspace(pair.dev.cfg, 2, w.max_len)
    x = torch.ones((2, w.dims.hidden), dtype=torch.float32, device="cuda")
    pos = torch.zeros((3, 2), dtype=torch.int32, device="cuda")
    cpos = torch.tensor([w.max_len, 5], dtype=torch.int32, device="cuda")
    pair.dev.decode_layer(0, kv, x, pos, cpos, ws)
    assert ws.status() == kmr.KMR_STATUS_CACHE_POS
    kg = oracle.as_u16(kv.k)
    assert np.array_equal(kg[:, 0], kh[:, 0])
    assert ws.status() == 0             # cleared by the read


def test_bad_token_sets_status(kmr):
    w = synth.WORKLOADS["tiny"]
    log("decode_step with a token id outside the vocabulary")
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)
    kv, _, _ = make_caches(w.dims, synth.base_seed(w), 1, w.max_len, "host")
    ws = kmr.Workspace(pair.dev.cfg, 1, w.max_len)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    pair.dev.decode_step(kv, torch.tensor([w.dims.vocab], dtype=torch.int32, device="cuda"),
                         torch.zeros((3, 1), dtype=torch.int32, device="cuda"),
                         torch.tensor([3], dtype=torch.int32, device="cuda"), nxt, ws)
    assert ws.status() == kmr.KMR_STATUS_TOKEN

"""Host-side address model of the XCD-local persistent step kernel's weight and
K/V loaders (csrc/kmr_stepx.h), checked for every shape the library accepts.

For each config of a grid, kmr_debug_stepx_fits says whether kmr_decode_step would
run it on that kernel.  For every accepted shape, this test recomputes, from the
kernel's own work split (XCD x, group j of the XCD, wave, lane), the byte range of
every 16-byte code load and the index of every scale/zero load of the q/k/v, o,
gate/up and down projections, and checks that
- every load lies inside its buffer ([rows][K/2] bytes, [rows][K/G] words), and
- every (row, 32-column chunk) of every matrix is loaded exactly once per layer
  (a chunk no lane loads would silently drop columns from a dot product).
The K/V loads of the attention items are checked against the cache layout.  The
shapes the grid holds past the kernel's limits must be refused.  No GPU is needed.
"""
import itertools

import numpy as np
import pytest

from int4_weight_only_gemv_amd import kmr, synth

XCDS, WAVES, LANES = 8, 8, 64
NARROW_CPL = 3           # chunks per lane of an 8-lane group in the split-K loaders
GU_ROWS, GU_K = 24, 2048  # matrix-core gate/up form: act rows per group, columns
FIX = dict(hidden=2048, n_kv_heads=8, n_heads=16, head_dim=128, intermediate=6144, group_size=128, n_groups=256)


def _dims(H, Hq, Hkv, D, I, G):
    q = D // 8
    return synth.Dims(hidden=H, n_heads=Hq, n_kv_heads=Hkv, head_dim=D, intermediate=I, vocab=1024,
                      n_layers=2, group_size=G, mrope_section=(D // 2 - 2 * q, q, q))


class Loads:
    """Collected code loads (row, byte offset in row) and scale/zero loads (row, group)."""

    def __init__(self, rows, K, G):
        self.rows, self.K, self.NG = rows, K, K // G
        self.code = []
        self.sz = []
        self.lgG = G.bit_length() - 1

    def add(self, row, col, with_sz=True):
        """A 16-byte code load of row `row` at column `col` (32 columns), and with_sz:
        the scale/zero word of that column's group."""
        row = np.asarray(row).ravel()
        col = np.asarray(col).ravel()
        self.code.append(np.stack([row, col]))
        if with_sz:
            self.add_sz(row, col)

    def add_sz(self, row, col):
        """A scale/zero load of row `row`, the group of column `col`."""
        self.sz.append(np.stack([np.asarray(row).ravel(), np.asarray(col).ravel() >> self.lgG]))

    def check(self, name, counted=None):
        code = np.concatenate(self.code, axis=1)
        row, col = code
        byte = row.astype(np.int64) * (self.K // 2) + col // 2
        assert np.all(byte >= 0) and np.all(byte + 16 <= self.rows * self.K // 2), f"{name}: code load out of bounds"
        assert np.all(col % 32 == 0) and np.all(col + 32 <= self.K), f"{name}: chunk outside the row"
        sz = np.concatenate(self.sz, axis=1)
        idx = sz[0].astype(np.int64) * self.NG + sz[1]
        assert np.all(sz[1] >= 0) and np.all(sz[1] < self.NG), f"{name}: scale/zero group outside the row"
        assert np.all(idx >= 0) and np.all(idx < self.rows * self.NG), f"{name}: scale/zero load out of bounds"
        # coverage: each (row, chunk) exactly once among the loads whose data is used
        use = np.ones(code.shape[1], bool) if counted is None else np.concatenate(counted)
        key = row[use].astype(np.int64) * (self.K // 32) + col[use] // 32
        counts = np.bincount(key, minlength=self.rows * (self.K // 32))
        assert counts.size == self.rows * (self.K // 32), f"{name}: load past the last chunk"
        missing = int(np.sum(counts == 0))
        twice = int(np.sum(counts > 1))
        assert missing == 0 and twice == 0, f"{name}: {missing} chunks never loaded, {twice} loaded twice"


def model_step_loads(H, Hq, Hkv, D, I, G, nwg):
    WPX, GPX, QPG = nwg // XCDS, Hkv // XCDS, Hq // Hkv
    QX, OX, IX = GPX * (QPG + 2) * D, GPX * QPG * D, I // XCDS
    RPW, RQ, RA = -(-H // WPX), -(-QX // WPX), -(-IX // WPX)
    fixed = (H, Hkv, Hq, D, I, G, nwg) == tuple(FIX[k] for k in
                                                ("hidden", "n_kv_heads", "n_heads", "head_dim", "intermediate",
                                                 "group_size", "n_groups"))
    x, j, wv, ln = np.meshgrid(np.arange(XCDS), np.arange(WPX), np.arange(WAVES), np.arange(LANES), indexing="ij")
    x, j, wv, ln = x.ravel(), j.ravel(), wv.ravel(), ln.ravel()

    def qkv_row(lr):   # weight row of the XCD's local q/k/v row lr
        gl = lr // ((QPG + 2) * D)
        t = lr - gl * (QPG + 2) * D
        g = x * GPX + gl
        return np.where(t < QPG * D, g * QPG * D + t,
                        np.where(t < (QPG + 1) * D, Hq * D + g * D + (t - QPG * D),
                                 Hq * D + Hkv * D + g * D + (t - (QPG + 1) * D)))

    qkv = Loads((Hq + 2 * Hkv) * D, H, G)
    if fixed:
        # matrix-core tile (gate/up layout, T = 1): load i < 2, lane l: local row
        # 8 i + l / 8, chunk 8 wave + ((l % 8) ^ (l / 8)); scale/zero pair l < 32:
        # (row l / 2, group 2 wave + l % 2), lanes past 32 repeat pair 0
        assert RQ == 16
        for i in range(2):
            qkv.add(qkv_row(j * RQ + 8 * i + (ln >> 3)), 32 * (8 * wv + ((ln & 7) ^ (ln >> 3))), with_sz=False)
        qkv.add_sz(qkv_row(j * RQ + np.where(ln < 32, ln >> 1, 0)), 256 * wv + 128 * (ln & 1))
        qkv.check("qkv (matrix-core)")
    else:
        # two rows per wave (one 32-column chunk per lane, lane < H/32)
        used = []
        for i in range(2):
            rr = wv * 2 + i
            lr = j * RQ + rr
            ok = (rr < RQ) & (lr < QX) & (32 * ln < H)
            qkv.add(qkv_row(lr)[ok], 32 * ln[ok])
            used.append(np.ones(int(ok.sum()), bool))
        qkv.check("qkv", used)

    # o and down rows (wnarrow_load): output row j*RPW + 8 wave + lane/8 of the group,
    # the XCD's column slice, chunks (lane % 8) + 8 t
    def narrow(K, KS, name):
        L = Loads(H, K, G)
        orow = j * RPW + wv * 8 + (ln >> 3)
        ok = (wv * 8 + (ln >> 3) < RPW) & (orow < H)
        for t in range(NARROW_CPL):
            c = (ln & 7) + 8 * t
            m = ok & (c < KS // 32)
            L.add(orow[m], x[m] * KS + 32 * c[m])
        L.check(name)

    narrow(Hq * D, OX, "o")
    narrow(I, IX, "down")

    # gate/up rows
    gu = Loads(2 * I, H, G)
    if fixed:
        # matrix-core tiles: load i, lane l: local row 8 i + l / 8 (gate rows, then up
        # rows), chunk 8 wave + ((l % 8) ^ (l / 8)); scale/zero pairs p = 64 u + l < 96:
        # (row p / 2, group 2 wave + p % 2)
        def grow_of(r):
            ar = np.where(r < GU_ROWS, r, r - GU_ROWS)
            return x * IX + j * GU_ROWS + ar + np.where(r < GU_ROWS, 0, I)

        for i in range(6):
            r = 8 * i + (ln >> 3)
            gu.add(grow_of(r), 32 * (8 * wv + ((ln & 7) ^ (ln >> 3))), with_sz=False)
        for u in range(2):
            p = 64 * u + ln
            gu.add_sz(grow_of(np.where(p < 96, p >> 1, 0)), 256 * wv + 128 * (ln & 1))
        gu.check("gate/up (matrix-core)")
    else:
        # three act rows per wave (gate and up rows), one chunk per lane; lanes past the
        # row reload chunk 0 (counted as loads, not as coverage)
        used = []
        for i in range(3):
            la = wv * 3 + i
            gla = j * RA + la
            ok = (la < RA) & (gla < IX)
            cl = np.where(32 * ln < H, ln, 0)
            for half in (0, I):
                gu.add(x[ok] * IX + gla[ok] + half, 32 * cl[ok])
                used.append((32 * ln < H)[ok])
        gu.check("gate/up", used)


def model_kv_loads(D, Hkv, M, B):
    """Attention item loads: row b, kv head g, 128-slot split s, lane (r, i) = (lane / 16,
    lane % 16) of wave w.  K: slot s*128 + 16 w + i (clamped into the cache), 16 bytes at
    dims 32 t + 8 r for t < D/32; V: slots s*128 + 16 w + 4 r + e (clamped), DPL dims from
    DPL i.  Every (slot, dim) of a split's 128 slots must be read exactly once by each of
    the K and V loads (before the clamp), and every load must stay inside the cache."""
    DPL = D // 16
    ns = -(-M // 128)
    w, ln = np.meshgrid(np.arange(WAVES), np.arange(LANES), indexing="ij")
    r, i = (ln >> 4).ravel(), (ln & 15).ravel()
    w = w.ravel()
    head = (np.arange(B)[:, None] * Hkv + np.arange(Hkv)[None]).ravel() * M
    for s in range(ns):
        # K
        pk = s * 128 + 16 * w
        pk = pk + i
        kd = np.stack([32 * t + 8 * r for t in range(D // 32)])            # [t][lane]
        cov = np.zeros((128, D), np.int32)
        for t in range(D // 32):
            for d in range(8):
                np.add.at(cov, (pk - s * 128, kd[t] + d), 1)
        assert np.all(cov == 1), "K: every (slot, dim) of the split once"
        pkc = np.minimum(pk, M - 1)
        assert np.all(kd + 8 <= D) and np.all(kd % 8 == 0)
        # V
        cov[:] = 0
        for e in range(4):
            pv = s * 128 + 16 * w + 4 * r + e
            for d in range(DPL):
                np.add.at(cov, (pv - s * 128, DPL * i + d), 1)
        assert np.all(cov == 1), "V: every (slot, dim) of the split once"
        pvc = np.minimum(s * 128 + 16 * w + 4 * r + 3, M - 1)
        for p in (pkc, pvc):
            assert np.all(p >= 0) and np.all(p < M)
        last = (head.max() + max(pkc.max(), pvc.max())) * D + D
        assert last <= B * Hkv * M * D


GRID = list(itertools.product([512, 1024, 1536, 2048, 2560], [64, 128], [8, 16], [1024, 2048, 3072, 6144, 8192],
                              [32, 128, 256], [64, 128, 256, 512]))


def test_loader_addresses_of_every_accepted_shape():
    accepted = []
    for H, D, Hkv, I, G, nwg in GRID:
        dims = _dims(H, 2 * Hkv, Hkv, D, I, G)
        cfg = kmr.make_config(dims)
        fits = [kmr.debug_stepx_fits(cfg, B, nwg) for B in (1, 4)]
        if fits[0] < 0:
            continue   # not a valid config at all
        assert fits[0] == fits[1], "the batch-1 and batch-4 kernels take the same shapes"
        if fits[0]:
            accepted.append((H, 2 * Hkv, Hkv, D, I, G, nwg))
    assert len(accepted) >= 10
    assert (2048, 16, 8, 128, 6144, 128, 256) in accepted   # the constant-size instantiation's shape
    for shape in accepted:
        model_step_loads(*shape)
    for D in (64, 128):
        for M in (1, 127, 128, 300, 1024):
            model_kv_loads(D, 8, M, 4)


@pytest.mark.parametrize("H,Hq,Hkv,D,I,G,nwg,why", [
    (2560, 16, 8, 128, 6144, 128, 256, "hidden past 64 chunks (one chunk per lane)"),
    (2048, 16, 8, 128, 8192, 128, 256, "intermediate past 6144 (down slice past 24 chunks per 8 lanes)"),
    (2048, 32, 16, 128, 6144, 128, 256, "n_heads*head_dim past 2048"),
    (2048, 16, 8, 128, 6144, 128, 1024, "more than 64 groups per XCD"),
    (2048, 8, 8, 128, 6144, 128, 256, "one q head per kv head"),
    (2048, 16, 8, 128, 6144, 128, 200, "groups not a multiple of the XCD count"),
])
def test_shapes_past_the_loaders_are_refused(H, Hq, Hkv, D, I, G, nwg, why):
    cfg = kmr.make_config(_dims(H, Hq, Hkv, D, I, G))
    assert kmr.debug_stepx_fits(cfg, 1, nwg) == 0, why

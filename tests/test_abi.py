"""Host-only checks of the C ABI: the library loads, exports every function
include/kmr.h declares, the ctypes mirrors match the C struct layouts, and
invalid calls are rejected on the host before anything is launched.  No GPU."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kmr.h")


@pytest.fixture(scope="module")
def kmr():
    from int4_weight_only_gemv_amd import build
    if not os.path.exists(build.OUT):
        build.build(force=False)
    from int4_weight_only_gemv_amd import kmr as k
    return k


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kmr_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("kmr_kv_alloc", "kmr_quantize_int4", "kmr_decode_layer", "kmr_decode_step"):
        assert fn in names


def test_library_exports_every_declared_function(kmr):
    out = subprocess.run(["nm", "-D", "--defined-only", kmr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kmr_[a-z0-9_]+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    assert sorted(kmr.EXPORTED) == declared_functions()


def test_struct_layouts_match_header(kmr, tmp_path):
    import ctypes as C
    prog = tmp_path / "layout.c"
    prog.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "kmr.h"
int main(void) {
  printf("%zu %zu %zu %zu\\n", sizeof(kmr_config), offsetof(kmr_config, rope_theta),
         offsetof(kmr_config, mrope_section), offsetof(kmr_config, eos_id));
  printf("%zu %zu\\n", sizeof(kmr_qweight), offsetof(kmr_qweight, K));
  printf("%zu %zu %zu\\n", sizeof(kmr_layer), offsetof(kmr_layer, qkv), offsetof(kmr_layer, down));
  printf("%zu %zu\\n", sizeof(kmr_model), offsetof(kmr_model, layers));
  printf("%zu %zu %zu\\n", sizeof(kmr_kv), offsetof(kmr_kv, max_len), offsetof(kmr_kv, bytes));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)],
                   check=True)
    got = [list(map(int, line.split())) for line in subprocess.run([str(exe)], capture_output=True,
                                                                    text=True).stdout.splitlines()]
    want = [
        [C.sizeof(kmr.Config), kmr.Config.rope_theta.offset, kmr.Config.mrope_section.offset,
         kmr.Config.eos_id.offset],
        [C.sizeof(kmr.QWeight), kmr.QWeight.K.offset],
        [C.sizeof(kmr.Layer), kmr.Layer.qkv.offset, kmr.Layer.down.offset],
        [C.sizeof(kmr.Model), kmr.Model.layers.offset],
        [C.sizeof(kmr.KV), kmr.KV.max_len.offset, kmr.KV.bytes.offset],
    ]
    assert got == want


def _cfg(kmr, **over):
    from int4_weight_only_gemv_amd import synth
    import dataclasses
    return kmr.make_config(dataclasses.replace(synth.QWEN3VL_2B, **over))


def test_workspace_and_kv_sizes(kmr):
    import ctypes as C
    cfg = _cfg(kmr)
    kv = kmr.KV()
    assert kmr._lib.kmr_kv_alloc(C.byref(cfg), 1, 1024, None, 0, 0, None, C.byref(kv)) == 0
    assert kv.bytes == 2 * 28 * 1 * 8 * 1024 * 128 * 2
    assert kv.k is None and kv.max_len == 1024
    n1 = kmr.workspace_bytes(cfg, 1, 1024)
    n16 = kmr.workspace_bytes(cfg, 16, 8192)
    assert 0 < n1 < n16
    assert kmr.workspace_bytes(cfg, 0, 1024) == 0
    assert kmr.workspace_bytes(cfg, kmr.KMR_MAX_BATCH + 1, 1024) == 0
    pf = kmr._lib.kmr_prefill_workspace_bytes
    assert pf(C.byref(cfg), 0, 1024) == 0 and pf(C.byref(cfg), 8, 0) == 0
    assert pf(C.byref(cfg), 5, 1024) == kmr.workspace_bytes(cfg, 5, 1024)        # one chunk of 5 rows
    assert pf(C.byref(cfg), 1000, 1024) == pf(C.byref(cfg), kmr.KMR_PREFILL_CHUNK, 1024) > n16


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96, mrope_section=(16, 16, 16)), -2),
    (dict(n_kv_heads=3), -2),
    (dict(group_size=48), -2),
    (dict(mrope_section=(24, 20, 19)), -2),
    (dict(hidden=0), -1),
])
def test_bad_configs_are_rejected_on_host(kmr, over, code):
    import ctypes as C
    cfg = _cfg(kmr, **over)
    kv = kmr.KV()
    assert kmr._lib.kmr_kv_alloc(C.byref(cfg), 1, 16, None, 0, 0, None, C.byref(kv)) == code
    assert kmr._lib.kmr_last_error()


def test_bad_calls_are_rejected_before_launch(kmr):
    import ctypes as C
    cfg = _cfg(kmr)
    assert kmr._lib.kmr_quantize_int4(None, 4, 256, 64, None, None, None) == kmr.KMR_EINVAL
    fake = C.c_void_p(0x1000)
    assert kmr._lib.kmr_quantize_int4(fake, 4, 256, 48, fake, fake, None) == kmr.KMR_ESHAPE
    assert kmr._lib.kmr_quantize_int4(fake, 4, 256, 3, fake, fake, None) == kmr.KMR_ESHAPE
    kv = kmr.KV()
    assert kmr._lib.kmr_kv_alloc(C.byref(cfg), 1, 1024, fake, 100, 0, None, C.byref(kv)) == kmr.KMR_ENOMEM
    layer = kmr.Layer()
    rc = kmr._lib.kmr_decode_layer(C.byref(cfg), C.byref(layer), 0, C.byref(kv), fake, fake, fake, 1,
                                   fake, 1 << 30, None)
    assert rc == kmr.KMR_EINVAL and b"norm" in kmr._lib.kmr_last_error()
    assert kmr._lib.kmr_strerror(kmr.KMR_ENOMEM) == b"buffer or workspace too small"


def test_bad_shared_prefix_is_rejected_before_launch(kmr):
    import ctypes as C
    cfg = _cfg(kmr)
    kv = kmr.KV()
    kv.max_len = 1024
    fake = C.c_void_p(0x1000)
    model = kmr.Model()
    for bad in (-1, 1025):
        rc = kmr._lib.kmr_decode_step_prefix(C.byref(cfg), C.byref(model), C.byref(kv), fake, fake, fake, None,
                                             4, fake, None, 0, bad, fake, 1 << 30, None)
        assert rc == kmr.KMR_EINVAL and b"shared_prefix" in kmr._lib.kmr_last_error()
    assert kmr._lib.kmr_decode_step_prefix(C.byref(cfg), C.byref(model), None, fake, fake, fake, None, 4, fake,
                                           None, 0, 0, fake, 1 << 30, None) == kmr.KMR_EINVAL


def test_bad_prefill_calls_are_rejected_before_launch(kmr):
    import ctypes as C
    cfg = _cfg(kmr)
    kv = kmr.KV()
    kv.k, kv.v = 0x1000, 0x2000
    kv.n_layers, kv.batch, kv.n_kv_heads, kv.max_len, kv.head_dim = 28, 2, 8, 64, 128
    fake = C.c_void_p(0x1000)
    model = kmr.Model()
    pf = kmr._lib.kmr_prefill
    for row, start, n, what in ((2, 0, 4, b"cache row"), (-1, 0, 4, b"cache row"), (0, 0, 0, b"outside"),
                                (0, 60, 5, b"outside"), (0, -1, 4, b"outside")):
        rc = pf(C.byref(cfg), C.byref(model), C.byref(kv), row, fake, fake, start, n, fake, None, fake, 1 << 30, None)
        assert rc == kmr.KMR_EINVAL and what in kmr._lib.kmr_last_error(), (row, start, n)
    rc = pf(C.byref(cfg), C.byref(model), C.byref(kv), 1, fake, fake, 60, 4, fake, None, fake, 1 << 30, None)
    assert rc == kmr.KMR_EINVAL and b"model" in kmr._lib.kmr_last_error()   # the range itself is fine


def test_bad_slot_calls_are_rejected_before_launch(kmr):
    import ctypes as C
    fake = C.c_void_p(0x1000)

    def kv(batch, max_len, layers=2, heads=8, dim=128):
        d = kmr.KV()
        d.k, d.v = 0x1000, 0x2000
        d.n_layers, d.batch, d.n_kv_heads, d.max_len, d.head_dim = layers, batch, heads, max_len, dim
        return d

    a, b = kv(4, 64), kv(2, 32)
    copy = kmr._lib.kmr_kv_copy_row
    assert copy(C.byref(a), 4, C.byref(b), 0, 8, None) == kmr.KMR_EINVAL        # dst row
    assert copy(C.byref(a), 0, C.byref(b), 2, 8, None) == kmr.KMR_EINVAL        # src row
    assert copy(C.byref(a), 0, C.byref(b), 1, 33, None) == kmr.KMR_EINVAL       # past src max_len
    assert copy(C.byref(a), 0, C.byref(b), 1, -1, None) == kmr.KMR_EINVAL
    assert copy(C.byref(a), 1, C.byref(a), 1, 8, None) == kmr.KMR_EINVAL        # onto itself
    c = kv(2, 32, heads=4)
    assert copy(C.byref(a), 0, C.byref(c), 1, 8, None) == kmr.KMR_EINVAL        # unequal dims
    assert b"kv heads" in kmr._lib.kmr_last_error()
    assert copy(C.byref(a), 0, C.byref(b), 1, 0, None) == kmr.KMR_OK            # nothing to copy
    p3 = (C.c_int32 * 3)(1, 2, 3)
    admit = kmr._lib.kmr_slot_admit
    assert admit(fake, fake, fake, fake, 4, 4, 7, p3, 5, None) == kmr.KMR_EINVAL
    assert admit(fake, fake, fake, fake, kmr.KMR_MAX_BATCH + 1, 0, 7, p3, 5, None) == kmr.KMR_EINVAL
    assert admit(fake, fake, fake, fake, 4, 0, 7, p3, -1, None) == kmr.KMR_EINVAL
    assert admit(None, fake, fake, fake, 4, 0, 7, p3, 5, None) == kmr.KMR_EINVAL
    assert kmr._lib.kmr_slot_retire(fake, 4, -1, None) == kmr.KMR_EINVAL
    assert kmr._lib.kmr_slot_retire(None, 4, 0, None) == kmr.KMR_EINVAL

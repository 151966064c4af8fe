"""The C-ABI library loads, exports what include/la.h declares, and its host-only
state logic behaves (no device work is launched in this file)."""

import ctypes
import os
import re
import subprocess

import pytest

import streaming_causal_video_amd as L
from streaming_causal_video_amd import _lib
from oracle import Ring

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_exported_dynamic_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in syms, n


def test_struct_layout_matches_c(tmp_path):
    """Compile a probe against include/la.h with gcc and compare the layout with ctypes."""
    src = tmp_path / "probe.c"
    fields = [f[0] for f in _lib.la_kvring._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(la_kvring, {f}));' for f in fields)
    src.write_text(f"""#include <stdio.h>
#include <stddef.h>
#include "la.h"
int main(void) {{
  printf("sizeof %zu\\n", sizeof(la_kvring));
{body}
  return 0;
}}
""")
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                      check=True).stdout.splitlines())
    assert int(out["sizeof"]) == ctypes.sizeof(_lib.la_kvring)
    for f in fields:
        assert int(out[f]) == getattr(_lib.la_kvring, f).offset, f


def make_ring(W=4, dtype=L.LA_BF16, noise=0.75):
    r = L.la_kvring()
    fake = [0x10000, 0x20000, 0x30000, 0x40000]  # never dereferenced by host-only calls
    L.la_kvring_init(r, *fake, W, 48, 16, 2, 128, dtype, noise)
    return r


def test_status_strings_and_version():
    lib = L.lib()
    assert lib.la_status_string(0) == b"ok"
    assert b"noise" in lib.la_status_string(-5)
    assert lib.la_status_string(123) == b"unknown status"
    assert "gfx950" in L.la_version()


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_advance_matches_oracle_window(W):
    """Slot and evicted id of every append agree with the oracle's FIFO window."""
    r = make_ring(W)
    model = Ring(W, 0.75)
    for b in range(1, 40):
        slot, ev = L.la_kvring_advance(r, b)
        assert slot == Ring.slot_of(b, W)
        ev_model = model.append(b, [b], [b], 0.75)
        assert ev == (ev_model or 0)
        r.last_block = b  # the index update an append makes (device copy not exercised here)
        assert L.la_kvring_count(r) == min(b, W)


def test_host_side_refusals_change_nothing():
    lib = L.lib()
    r = make_ring(2)
    before = bytes(r)
    # out-of-order block
    with pytest.raises(L.LAError) as e:
        L.la_kvring_advance(r, 2)
    assert e.value.status == _lib.LA_ERR_STATE
    ev = ctypes.c_int64()
    st = lib.la_kvcache_append_evict(ctypes.byref(r), ctypes.c_void_p(0x50000),
                                     ctypes.c_void_p(0x60000), 3, 0.75, ctypes.byref(ev), None)
    assert st == _lib.LA_ERR_STATE
    # wrong noise level (timestep forcing)
    st = lib.la_kvcache_append_evict(ctypes.byref(r), ctypes.c_void_p(0x50000),
                                     ctypes.c_void_p(0x60000), 1, 0.5, ctypes.byref(ev), None)
    assert st == _lib.LA_ERR_NOISE_LEVEL
    # sink replacement before block 1
    st = lib.la_sink_replace(ctypes.byref(r), ctypes.c_void_p(0x50000), ctypes.c_void_p(0x60000),
                             None)
    assert st == _lib.LA_ERR_STATE
    # a second replacement
    r2 = make_ring(2)
    r2.last_block = 1
    r2.sink_replaced = 1
    st = lib.la_sink_replace(ctypes.byref(r2), ctypes.c_void_p(0x50000), ctypes.c_void_p(0x60000),
                             None)
    assert st == _lib.LA_ERR_STATE
    # NULL and misaligned pointers
    st = lib.la_kvcache_append_evict(ctypes.byref(r), None, ctypes.c_void_p(0x60000), 1, 0.75,
                                     ctypes.byref(ev), None)
    assert st == _lib.LA_ERR_INVALID_ARG
    st = lib.la_kvcache_append_evict(ctypes.byref(r), ctypes.c_void_p(0x50004),
                                     ctypes.c_void_p(0x60000), 1, 0.75, ctypes.byref(ev), None)
    assert st == _lib.LA_ERR_INVALID_ARG
    assert bytes(r) == before


def test_init_validation():
    lib = L.lib()
    r = L.la_kvring()
    p = ctypes.c_void_p(0x10000)
    assert lib.la_kvring_init(ctypes.byref(r), p, p, p, p, 0, 48, 16, 2, 128, 0, 0.5) == _lib.LA_ERR_SHAPE
    assert lib.la_kvring_init(ctypes.byref(r), p, p, p, p, 65, 48, 16, 2, 128, 0, 0.5) == _lib.LA_ERR_SHAPE
    assert lib.la_kvring_init(ctypes.byref(r), p, p, p, p, 4, 48, 16, 2, 100, 0, 0.5) == _lib.LA_ERR_SHAPE
    assert lib.la_kvring_init(ctypes.byref(r), p, p, p, p, 4, 48, 16, 2, 128, 7, 0.5) == _lib.LA_ERR_DTYPE
    assert lib.la_kvring_init(ctypes.byref(r), None, p, p, p, 4, 48, 16, 2, 128, 0, 0.5) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_kvring_init(ctypes.byref(r), p, p, p, p, 4, 48, 16, 2, 128, 0, float("nan")) == _lib.LA_ERR_INVALID_ARG


def test_attention_argument_checks_before_launch():
    lib = L.lib()
    r = make_ring(2)
    p = ctypes.c_void_p(0x70000)
    out = ctypes.c_void_p(0x80000)
    # wrong n_q
    assert lib.la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 47, out, None, 0.1, None) == _lib.LA_ERR_SHAPE
    # non-positive scale
    assert lib.la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 48, out, None, 0.0, None) == _lib.LA_ERR_INVALID_ARG
    # out aliasing q
    assert lib.la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 48, p, None, 0.1, None) == _lib.LA_ERR_INVALID_ARG
    # bf16 path needs head_dim 128
    r64 = L.la_kvring()
    f = [0x10000] * 4
    L.la_kvring_init(r64, *f, 2, 48, 16, 2, 64, L.LA_BF16, 0.5)
    assert lib.la_block_attn_fwd(ctypes.byref(r64), p, p, p, p, 48, out, None, 0.1, None) == _lib.LA_ERR_SHAPE


def test_rope_and_euler_argument_checks():
    lib = L.lib()
    p = ctypes.c_void_p(0x70000)
    assert lib.la_rope_table_bytes(30, 52, 128) == (30 + 52) * 21 * 2 * 4
    assert lib.la_rope_table_bytes(4, 4, 64) == (4 + 4) * 10 * 2 * 4
    assert lib.la_rope3d_rolling(p, p, None, None, 0, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4, None) == _lib.LA_ERR_SHAPE
    assert lib.la_rope3d_rolling(p, p, None, None, 5, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4, None) == _lib.LA_ERR_SHAPE
    assert lib.la_rope3d_rolling(p, None, None, None, 3, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4, None) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_rope3d_rolling(p, p, None, None, 3, 0, None, None, -1, p, 4, 4, 2, 64, 5, 1e4, None) == _lib.LA_ERR_DTYPE
    assert lib.la_fm_euler_step(p, p, 0, -0.25, None) == _lib.LA_OK  # n == 0: nothing to do
    assert lib.la_fm_euler_step(p, p, -1, -0.25, None) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_fm_euler_step(ctypes.c_void_p(0x70000), ctypes.c_void_p(0x70004), 16, -0.25, None) == _lib.LA_ERR_INVALID_ARG


def test_single_hip_runtime_shared_with_torch():
    """The library must run on PyTorch's HIP runtime (it takes PyTorch's pointers,
    streams and events): after loading, exactly one libamdhip64 is mapped."""
    L.lib()
    mapped = _lib._hip_runtimes_mapped()
    assert len(mapped) == 1, mapped

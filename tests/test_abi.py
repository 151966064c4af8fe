"""The C-ABI library loads, exports what include/la.h declares, and its host-only
state logic behaves (no device work is launched in this file)."""

import ctypes
import os
import re
import subprocess

import numpy as np
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


@pytest.mark.parametrize("struct", ["la_kvring", "la_stage"])
def test_struct_layout_matches_c(tmp_path, struct):
    """Compile a probe against include/la.h with gcc and compare the layout with ctypes."""
    src = tmp_path / "probe.c"
    cls = getattr(_lib, struct)
    fields = [f[0] for f in cls._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof({struct}, {f}));' for f in fields)
    src.write_text(f"""#include <stdio.h>
#include <stddef.h>
#include "la.h"
int main(void) {{
  printf("sizeof %zu\\n", sizeof({struct}));
{body}
  return 0;
}}
""")
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                      check=True).stdout.splitlines())
    assert int(out["sizeof"]) == ctypes.sizeof(cls)
    for f in fields:
        assert int(out[f]) == getattr(cls, f).offset, f


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


def test_staged_ring_places_blocks_beyond_the_window():
    """A staged ring (W + 1 slots) keeps the window's rules (the same evictions as the
    oracle's deque) and puts block b in slot (b - 1) mod (W + 1), so the next block's
    slot never holds a block of the window."""
    W, bt, H, d = 3, 48, 2, 128
    slot_bytes = bt * H * d * 2
    r = L.la_kvring()
    L.la_kvring_init_staged(r, 0x100000, 0x800000, 0x30000, 0x40000, W, bt, 16, H, d, L.LA_BF16,
                            0.5)
    assert r.W == W and r.nslots == W + 1
    ref = Ring(W, 0.5)
    lib = L.lib()
    for b in range(1, 3 * W + 3):
        k, v = L.la_kvring_next_slot(r)
        slot, ev = L.la_kvring_advance(r, b)
        assert slot == (b - 1) % (W + 1)
        assert (k, v) == (0x100000 + slot * slot_bytes, 0x800000 + slot * slot_bytes)
        held = [int(r.slot_block[s]) for s in range(W + 1)]
        assert held[slot] == 0 or held[slot] <= b - 1 - W  # free: empty or already evicted
        ref_ev = ref.append(b, None, None, 0.5)
        assert ev == (ref_ev or 0)
        # the host-side index update of an append whose K and V are already in place
        # (no copy is enqueued: both halves are the destination slot itself)
        evo = ctypes.c_int64()
        assert lib.la_kvcache_append_evict(ctypes.byref(r), ctypes.c_void_p(k), ctypes.c_void_p(v),
                                           b, 0.5, ctypes.byref(evo), None) == _lib.LA_OK
        assert evo.value == ev and r.last_block == b
        assert L.la_kvring_count(r) == min(b, W)
        held = [int(r.slot_block[s]) for s in range(W + 1)]
        assert sorted(x for x in held if x > max(b - W, 0)) == ref.ids()
    # W + 1 slots must fit the slot table
    p = ctypes.c_void_p(0x10000)
    assert lib.la_kvring_init_staged(ctypes.byref(L.la_kvring()), p, p, p, p, 64, 48, 16, 2, 128,
                                     0, 0.5) == _lib.LA_ERR_SHAPE
    assert lib.la_kvring_init_staged(ctypes.byref(L.la_kvring()), p, p, p, p, 63, 48, 16, 2, 128,
                                     0, 0.5) == _lib.LA_OK


def test_next_slot_of_a_full_plain_ring_is_refused():
    """A ring of W slots reuses the evicted block's slot, which the next block's
    attention still reads: its next slot is handed out only while the window has room."""
    r = make_ring(2)
    k, v = L.la_kvring_next_slot(r)
    assert (k, v) == (0x10000, 0x20000)
    lib = L.lib()
    evo = ctypes.c_int64()
    for b in (1, 2):
        k, v = L.la_kvring_next_slot(r)
        assert lib.la_kvcache_append_evict(ctypes.byref(r), ctypes.c_void_p(k), ctypes.c_void_p(v),
                                           b, 0.75, ctypes.byref(evo), None) == _lib.LA_OK
    with pytest.raises(L.LAError) as e:
        L.la_kvring_next_slot(r)
    assert e.value.status == _lib.LA_ERR_STATE


def test_corrupt_slot_count_is_refused():
    r = make_ring(4)
    before = bytes(r)
    for bad in (0, 3, 6, 65):
        r.nslots = bad
        with pytest.raises(L.LAError) as e:
            L.la_kvring_advance(r, 1)
        assert e.value.status == _lib.LA_ERR_STATE
        p = ctypes.c_void_p(0x70000)
        assert L.lib().la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 48, ctypes.c_void_p(0x80000),
                                         None, 0.1, 1.0, None, 0, None) == _lib.LA_ERR_STATE
    r.nslots = 4
    assert bytes(r) == before


def test_attention_argument_checks_before_launch():
    lib = L.lib()
    r = make_ring(2)
    p = ctypes.c_void_p(0x70000)
    out = ctypes.c_void_p(0x80000)
    # wrong n_q
    assert lib.la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 47, out, None, 0.1, 1.0, None, 0, None) == _lib.LA_ERR_SHAPE
    # non-positive scale
    assert lib.la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 48, out, None, 0.0, 1.0, None, 0, None) == _lib.LA_ERR_INVALID_ARG
    # out aliasing q
    assert lib.la_block_attn_fwd(ctypes.byref(r), p, p, p, p, 48, p, None, 0.1, 1.0, None, 0, None) == _lib.LA_ERR_INVALID_ARG
    # bf16 path needs head_dim 128
    r64 = L.la_kvring()
    f = [0x10000] * 4
    L.la_kvring_init(r64, *f, 2, 48, 16, 2, 64, L.LA_BF16, 0.5)
    assert lib.la_block_attn_fwd(ctypes.byref(r64), p, p, p, p, 48, out, None, 0.1, 1.0, None, 0, None) == _lib.LA_ERR_SHAPE


def test_rope_and_euler_argument_checks():
    lib = L.lib()
    p = ctypes.c_void_p(0x70000)
    assert lib.la_rope_table_bytes(30, 52, 128) == (30 + 52) * 21 * 2 * 4
    assert lib.la_rope_table_bytes(4, 4, 64) == (4 + 4) * 10 * 2 * 4
    assert lib.la_rope3d_rolling(p, p, None, None, 0, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4, 1.0, None) == _lib.LA_ERR_SHAPE
    assert lib.la_rope3d_rolling(p, p, None, None, 5, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4, 1.0, None) == _lib.LA_ERR_SHAPE
    assert lib.la_rope3d_rolling(p, None, None, None, 3, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4, 1.0, None) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_rope3d_rolling(p, p, None, None, 3, 0, None, None, -1, p, 4, 4, 2, 64, 5, 1e4, 1.0, None) == _lib.LA_ERR_DTYPE
    assert lib.la_fm_euler_step(p, p, 0, -0.25, None) == _lib.LA_OK  # n == 0: nothing to do
    assert lib.la_fm_euler_step(p, p, -1, -0.25, None) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_fm_euler_step(ctypes.c_void_p(0x70000), ctypes.c_void_p(0x70004), 16, -0.25, None) == _lib.LA_ERR_INVALID_ARG


def test_single_hip_runtime_shared_with_torch():
    """The library must run on PyTorch's HIP runtime (it takes PyTorch's pointers,
    streams and events): after loading, exactly one libamdhip64 is mapped."""
    L.lib()
    mapped = _lib._hip_runtimes_mapped()
    assert len(mapped) == 1, mapped


def _fake_stage(rings, dt, base):
    """A la_stage whose device pointers are never dereferenced (refused before launch)."""
    n = len(rings)
    st = _lib.la_stage()
    st.rings = ctypes.cast(rings, ctypes.POINTER(_lib.la_kvring))
    arrs = []
    for i, key in enumerate(("q_raw", "k_raw", "v_raw", "attn_out")):
        a = (ctypes.c_void_p * n)(*[base + 0x100000 * i + 0x1000 * l for l in range(n)])
        arrs.append(a)
        setattr(st, key, ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)))
    st.vel = base + 0x900000
    st.dt = dt
    return st, arrs


def _fake_rings(n, noise, Hl=4, Wl=4, heads=2, d=128):
    rings = (_lib.la_kvring * n)()
    for l in range(n):
        L.la_kvring_init(rings[l], 0x10000, 0x20000, 0x30000, 0x40000, 2, 3 * Hl * Wl, Hl * Wl,
                         heads, d, L.LA_BF16, noise)
    return rings


def test_chain_refusals_change_nothing():
    """la_denoise_chain validates every stage and the noise-level chain before any launch."""
    lib = L.lib()
    p = ctypes.c_void_p(0x7000000)
    x = ctypes.c_void_p(0x8000000)
    # stage noise levels 1.0 -> 0.75 -> 0.5 with dt -0.25 chain correctly ...
    r0, r1, r2 = _fake_rings(2, 1.0), _fake_rings(2, 0.75), _fake_rings(2, 0.4)
    before = [bytes(r) for r in (r0, r1, r2)]
    s0, a0 = _fake_stage(r0, -0.25, 0x1000000)
    s1, a1 = _fake_stage(r1, -0.25, 0x2000000)
    s2, a2 = _fake_stage(r2, -0.25, 0x3000000)
    # ... but 0.75 + (-0.25) != 0.4: refused
    stages = (_lib.la_stage * 3)(s0, s1, s2)
    st = lib.la_denoise_chain(stages, 3, 2, 1, p, p, p, p, 4, 4, 3, -1, 1e4, 0.1, None, 0, x, 64, None)
    assert st == _lib.LA_ERR_NOISE_LEVEL
    # the same rings in two stages: refused
    s1b, a1b = _fake_stage(r0, -0.25, 0x2000000)
    r0b = _fake_rings(2, 0.75)
    stages = (_lib.la_stage * 2)(s0, s1b)
    assert lib.la_denoise_chain(stages, 2, 2, 1, p, p, p, p, 4, 4, 3, -1, 1e4, 0.1, None, 0, x, 64,
                                None) == _lib.LA_ERR_INVALID_ARG
    # out-of-order block: refused
    stages = (_lib.la_stage * 2)(s0, s1)
    assert lib.la_denoise_chain(stages, 2, 2, 2, p, p, p, p, 4, 4, 3, -1, 1e4, 0.1, None, 0, x, 64,
                                None) == _lib.LA_ERR_STATE
    # latent without a velocity: refused
    s1.vel = None
    stages = (_lib.la_stage * 2)(s0, s1)
    assert lib.la_denoise_chain(stages, 2, 2, 1, p, p, p, p, 4, 4, 3, -1, 1e4, 0.1, None, 0, x, 64,
                                None) == _lib.LA_ERR_INVALID_ARG
    # shape mismatch inside a stage
    stages = (_lib.la_stage * 1)(s0)
    assert lib.la_denoise_chain(stages, 1, 2, 1, p, p, p, p, 5, 4, 3, -1, 1e4, 0.1, None, 0, x, 64,
                                None) == _lib.LA_ERR_SHAPE
    assert [bytes(r) for r in (r0, r1, r2)] == before
    del a0, a1, a2, a1b, r0b


def test_fp8_ring_and_entry_point_refusals():
    lib = L.lib()
    p = ctypes.c_void_p(0x70000)
    out = ctypes.c_void_p(0x80000)
    # e4m3 rings initialise; the bf16/f32 attention and the step refuse them
    r8 = L.la_kvring()
    L.la_kvring_init(r8, 0x10000, 0x20000, 0x30000, 0x40000, 2, 48, 16, 2, 128, L.LA_FP8_E4M3, 0.5)
    assert r8.dtype == L.LA_FP8_E4M3
    assert lib.la_block_attn_fwd(ctypes.byref(r8), p, p, p, p, 48, out, None, 0.1, 1.0, None, 0, None) == _lib.LA_ERR_DTYPE
    qarr = (ctypes.c_void_p * 1)(0x50000)
    assert lib.la_denoise_step(ctypes.byref(r8), 1, 1, qarr, qarr, qarr, qarr, p, p, p, None, None,
                               p, 4, 4, 3, -1, 1e4, 0.1, None, 0, None, None, 0, -0.25, 0, None,
                               None) == _lib.LA_ERR_DTYPE
    # la_block_attn_fwd_fp8: wrong ring dtype, head_dim, factors, alignment, aliasing
    rb = make_ring(2)
    args = lambda r, **kw: [ctypes.byref(r), kw.get("q", p), p, p, p, p, kw.get("nq", 48),
                            kw.get("out", out), None, 0.1, kw.get("dq", 0.01), 0.01, 0.01, None]
    assert lib.la_block_attn_fwd_fp8(*args(rb)) == _lib.LA_ERR_DTYPE
    assert lib.la_block_attn_fwd_fp8(*args(r8, nq=47)) == _lib.LA_ERR_SHAPE
    assert lib.la_block_attn_fwd_fp8(*args(r8, dq=0.0)) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_block_attn_fwd_fp8(*args(r8, dq=float("inf"))) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_block_attn_fwd_fp8(*args(r8, q=ctypes.c_void_p(0x70008))) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_block_attn_fwd_fp8(*args(r8, out=p)) == _lib.LA_ERR_INVALID_ARG
    r64 = L.la_kvring()
    L.la_kvring_init(r64, 0x10000, 0x20000, 0x30000, 0x40000, 2, 48, 16, 2, 64, L.LA_FP8_E4M3, 0.5)
    assert lib.la_block_attn_fwd_fp8(*args(r64)) == _lib.LA_ERR_SHAPE
    # la_quantize_fp8
    q = lib.la_quantize_fp8
    assert q(p, L.LA_BF16, out, 0, 1.0, None) == _lib.LA_OK  # n == 0: nothing to do
    assert q(p, L.LA_BF16, out, -1, 1.0, None) == _lib.LA_ERR_INVALID_ARG
    assert q(p, L.LA_FP8_E4M3, out, 16, 1.0, None) == _lib.LA_ERR_DTYPE
    assert q(p, L.LA_BF16, out, 16, 0.0, None) == _lib.LA_ERR_INVALID_ARG
    assert q(p, L.LA_BF16, out, 16, float("nan"), None) == _lib.LA_ERR_INVALID_ARG
    assert q(ctypes.c_void_p(0x70002), L.LA_BF16, out, 16, 1.0, None) == _lib.LA_ERR_INVALID_ARG
    assert q(p, L.LA_F32, ctypes.c_void_p(0x70010), 16, 1.0, None) == _lib.LA_ERR_INVALID_ARG  # overlap
    assert q(None, L.LA_BF16, out, 16, 1.0, None) == _lib.LA_ERR_INVALID_ARG


def test_denoise_step_flag_refusals():
    """Unknown flag bits, and a replacement sink with LA_STEP_ATTEND_ONLY, are refused."""
    lib = L.lib()
    p = ctypes.c_void_p(0x70000)
    rings = (_lib.la_kvring * 1)()
    L.la_kvring_init(rings[0], 0x10000, 0x20000, 0x30000, 0x40000, 2, 48, 16, 2, 128, L.LA_BF16, 0.5)
    arr = (ctypes.c_void_p * 1)(0x50000)
    before = bytes(rings[0])
    call = lambda flags, sink: lib.la_denoise_step(rings, 1, 1, arr, arr, arr, arr, p, p, p, sink,
                                                   sink, p, 4, 4, 3, -1, 1e4, 0.1, None, 0, None, None,
                                                   0, -0.25, flags, None, None)
    assert call(2, None) == _lib.LA_ERR_INVALID_ARG
    assert call(L.LA_STEP_ATTEND_ONLY, arr) == _lib.LA_ERR_INVALID_ARG
    assert bytes(rings[0]) == before


def test_attention_refuses_segments_beyond_32_bit_offsets():
    """Both attention kernels address a key segment with 32-bit byte offsets (the e4m3
    kernel's buffer descriptors hold a 32-bit record count): a segment of
    rows x heads x 128 elements reaching 2^32 bytes is refused before any launch; one that
    fits is not refused for its size."""
    lib = L.lib()
    p = ctypes.c_void_p(0x70000)
    out = ctypes.c_void_p(0x80000)
    fake = [0x10000, 0x20000, 0x30000, 0x40000]

    def ring(block_tokens, dtype):
        r = L.la_kvring()
        L.la_kvring_init(r, *fake, 2, block_tokens, 16, 40, 128, dtype, 0.5)
        return r

    # bf16: (block + 64) x 40 x 128 x 2 B >= 2^32 from block = 419,367
    big = ring(419_400, L.LA_BF16)
    assert lib.la_block_attn_fwd(ctypes.byref(big), p, p, p, p, 419_400, out, None, 0.1, 1.0, None, 0,
                                 None) == _lib.LA_ERR_SHAPE
    # e4m3: (block + 64) x 40 x 128 B >= 2^32 from block = 838,797
    big8 = ring(838_800, L.LA_FP8_E4M3)
    assert lib.la_block_attn_fwd_fp8(ctypes.byref(big8), p, p, p, p, p, 838_800, out, None,
                                     0.1, 1.0, 1.0, 1.0, None) == _lib.LA_ERR_SHAPE
    # just below the limits the size check passes and only the (deliberately) wrong n_q is
    # refused, so the refusal above came from the size
    ok = ring(419_300, L.LA_BF16)
    assert lib.la_block_attn_fwd(ctypes.byref(ok), p, p, p, p, 419_299, out, None, 0.1, 1.0, None, 0,
                                 None) == _lib.LA_ERR_SHAPE
    ok8 = ring(838_700, L.LA_FP8_E4M3)
    assert lib.la_block_attn_fwd_fp8(ctypes.byref(ok8), p, p, p, p, p, 838_699, out, None,
                                     0.1, 1.0, 1.0, 1.0, None) == _lib.LA_ERR_SHAPE


def test_ring_slots_must_be_whole_16_byte_vectors():
    """An e4m3 ring whose slot (block_tokens x heads x head_dim bytes) is not a multiple
    of 16 bytes is refused: its appends could not copy whole vectors and later slots
    would lose their 16-byte alignment.  The same geometry in bf16 is fine."""
    p = [0x10000, 0x20000, 0x30000, 0x40000]
    r = L.la_kvring()
    with pytest.raises(L.LAError) as e:
        L.la_kvring_init(r, *p, 2, 3, 2, 1, 8, L.LA_FP8_E4M3, 0.5)  # 24-byte slots
    assert e.value.status == _lib.LA_ERR_SHAPE
    L.la_kvring_init(r, *p, 2, 4, 2, 1, 8, L.LA_FP8_E4M3, 0.5)  # 32-byte slots
    L.la_kvring_init(r, *p, 2, 3, 2, 1, 8, L.LA_BF16, 0.5)      # 48-byte slots


def test_scale_and_workspace_refusals():
    """q_scale and the softmax scale must be positive and finite; a workspace must be
    256-byte aligned; RoPE refuses a non-positive q_scale.  All before any launch."""
    lib = L.lib()
    r = make_ring(2)
    p = ctypes.c_void_p(0x70000)
    out = ctypes.c_void_p(0x80000)
    call = lambda scale, q_scale, ws, nbytes: lib.la_block_attn_fwd(
        ctypes.byref(r), p, p, p, p, 48, out, None, scale, q_scale, ws, nbytes, None)
    assert call(0.1, 0.0, None, 0) == _lib.LA_ERR_INVALID_ARG
    assert call(0.1, float("inf"), None, 0) == _lib.LA_ERR_INVALID_ARG
    assert call(float("nan"), 1.0, None, 0) == _lib.LA_ERR_INVALID_ARG
    assert call(0.1, 1.0, ctypes.c_void_p(0x90010), 1 << 30) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_rope3d_rolling(p, p, None, None, 3, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4,
                                 0.0, None) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_rope3d_rolling(p, p, None, None, 3, 0, None, None, -1, p, 4, 4, 2, 64, 1, 1e4,
                                 -1.0, None) == _lib.LA_ERR_INVALID_ARG
    assert lib.la_attn_workspace_bytes(0, 40) == 0
    assert lib.la_attn_workspace_bytes(4680, 0) == 0
    # the step: a misaligned workspace, or a non-positive scale, is refused
    rings = _fake_rings(1, 0.5)
    arr = (ctypes.c_void_p * 1)(0x50000)
    before = bytes(rings[0])
    step = lambda scale, ws: lib.la_denoise_step(rings, 1, 1, arr, arr, arr, arr, p, p, p, None,
                                                 None, p, 4, 4, 3, -1, 1e4, scale, ws, 1 << 30,
                                                 None, None, 0, -0.25, 0, None, None)
    assert step(0.1, ctypes.c_void_p(0x90010)) == _lib.LA_ERR_INVALID_ARG
    assert step(0.0, None) == _lib.LA_ERR_INVALID_ARG
    assert bytes(rings[0]) == before


def test_kvringstack_rejects_unsupported_dtypes():
    """KVRingStack maps dtypes as KVRing does and raises before allocating anything."""
    import torch
    for dt in (torch.float16, torch.int8, torch.float64):
        with pytest.raises(TypeError):
            L.KVRingStack(2, 2, 48, 16, 2, 128, dt, 0.5)
        with pytest.raises(TypeError):
            L.KVRing(2, 48, 16, 2, 128, dt, 0.5)


def test_step_wrapper_checks_every_tensor():
    """la_denoise_step / la_denoise_chain (Python) check each per-layer tensor's shape and
    dtype against the rings before anything reaches the library (CPU tensors: a tensor
    that passes every shape and dtype check is then refused as not being on the GPU)."""
    import torch
    Hl, Wl, heads, d = 4, 4, 2, 128
    rings = _fake_rings(2, 0.5, Hl=Hl, Wl=Wl, heads=heads, d=d)
    bt, st = 3 * Hl * Wl, Hl * Wl
    blk = lambda dtype=torch.bfloat16: torch.zeros((bt, heads, d), dtype=dtype)
    snk = lambda: torch.zeros((st, heads, d), dtype=torch.bfloat16)
    table = torch.zeros(L.la_rope_table_bytes(Hl, Wl, d) // 4)
    good = dict(q_raw=[blk(), blk()], k_raw=[blk(), blk()], v_raw=[blk(), blk()],
                attn_out=[blk(), blk()], q_rot_ws=blk(), k_rot_ws=blk(), sink_k_rot_ws=snk())

    def call(**over):
        a = dict(good, **over)
        L.la_denoise_step(rings, 1, a["q_raw"], a["k_raw"], a["v_raw"], a["attn_out"],
                          a["q_rot_ws"], a["k_rot_ws"], a["sink_k_rot_ws"],
                          a.get("table", table), Hl, Wl, scale=0.1, x=a.get("x"),
                          vel=a.get("vel"))

    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call()
    with pytest.raises(ValueError, match="v_raw\\[1\\] has dtype"):
        call(v_raw=[blk(), blk(torch.float32)])
    with pytest.raises(ValueError, match="q_rot_ws has shape"):
        call(q_rot_ws=snk())
    with pytest.raises(ValueError, match="sink_k_rot_ws has shape"):
        call(sink_k_rot_ws=blk())
    with pytest.raises(ValueError, match="attn_out has 1 entries"):
        call(attn_out=[blk()])
    with pytest.raises(ValueError, match="rope_table"):
        call(table=torch.zeros(4))
    with pytest.raises(ValueError, match="float32"):
        call(x=torch.zeros(8, dtype=torch.bfloat16), vel=torch.zeros(8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="vel must match x"):
        call(x=torch.zeros(8), vel=torch.zeros(7))
    stage = dict(rings=rings, q_raw=good["q_raw"], k_raw=good["k_raw"], v_raw=good["v_raw"],
                 attn_out=[blk(), snk()], dt=-0.25)
    with pytest.raises(ValueError, match="stages\\[0\\]\\.attn_out\\[1\\] has shape"):
        L.la_denoise_chain([stage], 1, blk(), blk(), snk(), table, Hl, Wl, scale=0.1)


def test_fp8_step_refusals_change_nothing():
    """la_denoise_step_fp8 validates before any launch: e4m3 rings only (and
    la_denoise_step refuses them), head_dim 128, positive finite scales, the K/V code
    workspaces for plain rings, 16-byte aligned workspaces."""
    lib = L.lib()
    Hl = Wl = 4
    n = 2

    def rings_of(dtype, d=128, staged=False):
        rings = (_lib.la_kvring * n)()
        init = L.la_kvring_init_staged if staged else L.la_kvring_init
        for l in range(n):
            init(rings[l], 0x100000, 0x200000, 0x300000, 0x400000, 2, 3 * Hl * Wl, Hl * Wl, 2, d,
                 dtype, 0.5)
        return rings

    arrs = [(ctypes.c_void_p * n)(*[0x1000000 * (i + 1) + 0x10000 * l for l in range(n)])
            for i in range(4)]
    p = ctypes.c_void_p(0x9000000)

    def call(rings, k8=p, v8=p, q8=p, dq=0.01, flags=0):
        return lib.la_denoise_step_fp8(rings, n, 1, *arrs, p, p, p, q8, k8, v8, p, p, None, None,
                                       p, Hl, Wl, 3, -1, 1e4, 0.1, dq, 0.01, 0.01, None, None, 0,
                                       -0.25, flags, None, None)

    r8 = rings_of(L.LA_FP8_E4M3)
    before = bytes(r8)
    assert call(rings_of(L.LA_BF16)) == _lib.LA_ERR_DTYPE
    assert call(rings_of(L.LA_FP8_E4M3, d=64)) == _lib.LA_ERR_SHAPE
    assert call(r8, dq=0.0) == _lib.LA_ERR_INVALID_ARG
    assert call(r8, dq=float("inf")) == _lib.LA_ERR_INVALID_ARG
    assert call(r8, k8=None) == _lib.LA_ERR_INVALID_ARG          # plain ring: K codes need k8_ws
    assert call(rings_of(L.LA_FP8_E4M3, staged=True), k8=None, v8=None,
                flags=L.LA_STEP_ATTEND_ONLY) == _lib.LA_ERR_INVALID_ARG  # no append: needs them
    assert call(r8, q8=ctypes.c_void_p(0x9000008)) == _lib.LA_ERR_INVALID_ARG  # misaligned
    assert call(r8, flags=4) == _lib.LA_ERR_INVALID_ARG
    assert bytes(r8) == before
    # and the bf16 step refuses e4m3 rings
    assert lib.la_denoise_step(r8, n, 1, *arrs, p, p, p, None, None, p, Hl, Wl, 3, -1, 1e4, 0.1,
                               None, 0, None, None, 0, -0.25, 0, None, None) == _lib.LA_ERR_DTYPE


def _factor64(scale, dq, dk):
    """scale dq dk log2(e) in float64 from the float32 arguments, left to right."""
    f, d = np.float32, np.float64
    return d(f(scale)) * d(f(dq)) * d(f(dk)) * 1.4426950408889634


def _near_pow2(F):
    """Within a relative 2^-24 of a power of two 2^e, -127 <= e <= 127 (elementwise)."""
    m, k = np.frexp(F)
    lo = (m - 0.5 <= 2.0 ** -25) & (k - 1 >= -127) & (k - 1 <= 127)
    hi = (1.0 - m <= 2.0 ** -24) & (k >= -127) & (k <= 127)
    return lo | hi


@pytest.mark.parametrize("scale,dk,dq_min", [(128 ** -0.5, 5 / 448, 5 / 448),
                                              (64 ** -0.5, 3 / 448, 7 / 448),
                                              (0.1, 1.0, 1e-3), (500822.7, 2 / 448, 2 / 448),
                                              (1.0, 0.5, 2.0 / 1.4426950408889634)])
def test_fp8_q_factor_pow2_is_the_least_such_float(scale, dk, dq_min):
    """The helper's dq puts the logit factor within a relative 2^-24 of a power of two, and
    no float in [dq_min, dq) does (every one of them checked)."""
    dq = L.la_fp8_q_factor_pow2(scale, dk, dq_min)
    f32 = np.float32
    assert f32(dq) >= f32(dq_min)
    F = _factor64(scale, dq, dk)
    assert _near_pow2(np.array([F]))[0], F
    assert abs(F / 2.0 ** np.round(np.log2(F)) - 1) <= 2.0 ** -24
    lo = np.array([f32(dq_min)]).view(np.uint32)[0]
    hi = np.array([f32(dq)]).view(np.uint32)[0]
    assert hi - lo < (1 << 24)  # at most one binade apart
    cand = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    assert not _near_pow2(_factor64(scale, cand, dk)).any()


def test_fp8_q_factor_pow2_refusals():
    lib = L.lib()
    out = ctypes.c_float(-1.0)
    for args in [(0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("nan")),
                 (1.0, 1.0, float("inf")), (3e38, 3e38, 1.0)]:
        assert lib.la_fp8_q_factor_pow2(*args, ctypes.byref(out)) == _lib.LA_ERR_INVALID_ARG, args
        assert out.value == -1.0
    assert lib.la_fp8_q_factor_pow2(1.0, 1.0, 1.0, None) == _lib.LA_ERR_INVALID_ARG
    # dq_min already gives a power of two: dq_min itself
    assert L.la_fp8_q_factor_pow2(1.0, 1.0 / 1.4426950408889634, 4.0) == 4.0

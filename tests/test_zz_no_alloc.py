"""la_block_attn_fwd_noalloc (the attention with the library's static workspace, for
callers that cannot allocate) against la_block_attn_fwd with a caller workspace, through
the C ABI: two calls in a row, the second on a smaller input, each compared bit for bit
with the existing entry point and with the float64 oracle."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import StreamOracle

from gpu_helpers import GpuLayerStream, check_attention, say, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import streaming_causal_video_amd as lib
    lib.lib()
    return lib


def _streamed(shape, blocks):
    """A layer streamed through `blocks` blocks (the last one rotated, not yet appended)."""
    gs = GpuLayerStream(shape, keep_lse=True, fused=True, workspace=True)
    for b in range(1, blocks):
        gs.step(b)
    q, k, v = gs.block_dev(blocks)
    L_ = gs.L
    f0 = 3 * (blocks - 1)
    s = shape
    L_.la_rope3d_rolling(q, gs.q_rot, k, gs.k_rot, 3, f0, gs.ring.sink_k_raw, gs.sink_k_rot, -1,
                         gs.table, s.Hl, s.Wl, s.heads, s.head_dim, q_scale=gs.q_scale)
    return gs, v


def test_noalloc_matches_the_workspace_entry_point_on_two_calls(L):
    t = torch()
    # first call: 12 (head, query tile) units, each cut into 32 key ranges (384 records);
    # second call: a smaller layer, 3 units cut into 6 key ranges (18 records)
    for shape, blocks in ((si.MID_BF16, 5), (si.SMALL_BF16, 4)):
        say(f"no-alloc cfg {shape.cfg_id} block {blocks}")
        gs, v = _streamed(shape, blocks)
        gs.attend(v)  # la_block_attn_fwd with an AttnWorkspace
        t.cuda.synchronize()
        want, want_lse = gs.out.clone(), gs.lse.clone()
        gs.out.zero_()
        gs.lse.zero_()
        L.la_block_attn_fwd_noalloc(gs.ring.state, gs.q_rot, gs.sink_k_rot, gs.k_rot, v, gs.out,
                                    gs.lse, scale=gs.scale, q_scale=gs.q_scale)
        t.cuda.synchronize()
        assert t.equal(gs.out.view(t.int16), want.view(t.int16)), "outputs differ"
        assert t.equal(gs.lse, want_lse), "lse differs"
        ref = StreamOracle(shape).block_output(blocks)
        check_attention(to_f64(gs.out), ref, f"no-alloc cfg {shape.cfg_id}")


def test_noalloc_refuses_more_units_than_its_counters(L):
    """More than 16,384 (head, 192-query tile) units: refused before any launch."""
    import ctypes
    lib = L.lib()
    r = L.la_kvring()
    L.la_kvring_init(r, 0x10000, 0x20000, 0x30000, 0x40000, 2, 192 * 410, 16, 40, 128,
                     L.LA_BF16, 0.5)
    p = ctypes.c_void_p(0x70000)
    st = lib.la_block_attn_fwd_noalloc(ctypes.byref(r), p, p, p, p, 192 * 410,
                                       ctypes.c_void_p(0x80000), None, 0.1, 1.0, None)
    assert st == L._lib.LA_ERR_SHAPE

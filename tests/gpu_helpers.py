"""Helpers for GPU parity tests: upload seeded inputs, drive one streamed layer
through the C ABI, compare with tolerances."""

from __future__ import annotations

import functools
import sys

import numpy as np

import seeded_inputs as si

THETA = 10000.0
FRAMES_PER_BLOCK = 3
SINK_DELTA = -1          # sink one latent frame before the block's first frame
NOISE_LEVEL = 0.75       # this stage's t_i (stage t_3 -> t_2 of the 4-step grid)

# Tolerances stated for the path: bf16 attention vs the float64 oracle.
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
F32_MAX_ABS = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def to_dev(st: si.Stored):
    t = torch()
    if st.dtype == "bf16":
        return t.from_numpy(np.array(st.storage).view(np.int16)).cuda().view(t.bfloat16)
    return t.from_numpy(np.array(st.storage)).cuda()


def to_f64(x) -> np.ndarray:
    return x.detach().double().cpu().numpy()


def bf16_bits(x) -> np.ndarray:
    t = torch()
    return x.detach().contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def check_rope_bf16(got_bits: np.ndarray, exact: np.ndarray, raw: np.ndarray, what: str) -> None:
    """bf16 RoPE bound: within 1 bf16 ulp of the oracle's value rounded to nearest even,
    or, where the rotation cancels, within half an ulp plus the float32 arithmetic bound
    2**-21 * |(x, y)| of the pair (cos/sin rounded to float32, one product rounded, one
    fused multiply-add: about 3 * 2**-24 * (|x| + |y|))."""
    d = bf16_ulp_distance(got_bits, si.f64_to_bf16_bits(exact))
    pair = np.sqrt(raw[..., 0::2] ** 2 + raw[..., 1::2] ** 2)
    pair = np.repeat(pair, 2, axis=-1)
    got = si.bf16_bits_to_f64(got_bits)
    mag = np.maximum(np.abs(exact), 1e-300)
    half_ulp = np.ldexp(1.0, np.floor(np.log2(mag)).astype(np.int64) - 8)
    ok = (d <= 1) | (np.abs(got - exact) <= half_ulp + 2.0 ** -21 * pair)
    assert ok.all(), f"{what}: {int((~ok).sum())} elements outside the bound (max {int(d.max())} ulps)"


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def check_attention(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    err = np.abs(got - ref)
    r = rel_l2(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err.max() <= ATTN_MAX_ABS and r <= ATTN_REL_L2, \
        f"{what}: max-abs {err.max():.3e} (<= {ATTN_MAX_ABS}), rel-L2 {r:.3e} (<= {ATTN_REL_L2})"


def block_f0(block: int) -> int:
    return FRAMES_PER_BLOCK * (block - 1)


def softmax_scale(head_dim: int) -> float:
    return head_dim ** -0.5


def q_prescale(head_dim: int) -> float:
    """The factor la_denoise_step has RoPE apply to Q for bf16 rings: the softmax scale
    times log2(e), rounded to float32 (the attention then takes Q as given)."""
    return float(np.float32(softmax_scale(head_dim) * np.log2(np.e)))


def prescaled_q(q: si.Stored, head_dim: int):
    """Given bf16 Q -> (bf16 Q times q_prescale, rounded to nearest even; the float64 Q
    that those bits stand for, i.e. divided by q_prescale again; the factor)."""
    c = q_prescale(head_dim)
    qs = si.make_stored(q.values * c, "bf16")
    return qs, qs.values / c, c


class GpuLayerStream:
    """One layer of the stage streamed block by block through the C ABI.

    Per block b: la_rope3d_rolling (Q, K at f0(b); raw sink K at f0(b)+delta),
    la_block_attn_fwd, la_kvcache_append_evict, and after block 1 la_sink_replace
    with the first latent frame of block 1's raw K and V.
    """

    def __init__(self, shape: si.LayerShape, layer: int = 0, keep_lse: bool = False,
                 fused: bool = True, workspace: bool = True, staged: bool = False):
        """fused: RoPE writes Q times q_prescale and the attention takes it as given (the
        step's form); else the plain rotation and q_scale 1.  workspace: run the
        attention's balanced schedule (bf16 only).  staged: a ring of W + 1 slots whose
        next slot receives the block's rotated K (from RoPE) and its V (a copy) before
        the attention, which reads them there; the append then only records the block
        (the layout of la_denoise_step's staged rings)."""
        import streaming_causal_video_amd as L
        t = torch()
        self.L = L
        self.shape = shape
        self.layer = layer
        self.dtype = t.bfloat16 if shape.dtype == "bf16" else t.float32
        s = shape
        self.staged = staged
        self.ring = L.KVRing(s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, self.dtype,
                             NOISE_LEVEL, staged=staged)
        sk, sv = s.initial_sink(layer)
        self.ring.sink_k_raw.copy_(to_dev(sk))
        self.ring.sink_v.copy_(to_dev(sv))
        nbytes = L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim)
        self.table = t.empty(nbytes // 4, dtype=t.float32, device="cuda")
        L.la_rope_table_fill(self.table, s.Hl, s.Wl, s.head_dim, THETA)
        blk = (s.block_tokens, s.heads, s.head_dim)
        self.q_rot = t.empty(blk, dtype=self.dtype, device="cuda")
        self.k_rot = t.empty_like(self.q_rot)
        self.sink_k_rot = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=self.dtype,
                                  device="cuda")
        self.out = t.empty_like(self.q_rot)
        self.lse = t.empty((s.heads, s.block_tokens), dtype=t.float32, device="cuda") if keep_lse else None
        self._dev = {}
        bf16 = shape.dtype == "bf16"
        self.scale = softmax_scale(s.head_dim)
        self.q_scale = q_prescale(s.head_dim) if fused and bf16 else 1.0
        self.ws = L.AttnWorkspace(s.block_tokens, s.heads) if workspace and bf16 else None

    def block_dev(self, block: int):
        e = self.shape.entry(block)
        if e not in self._dev:
            self._dev[e] = tuple(to_dev(x) for x in self.shape.block_inputs(self.layer, block))
        return self._dev[e]

    def step(self, block: int):
        L, s = self.L, self.shape
        q, k, v = self.block_dev(block)
        f0 = block_f0(block)
        k_dst, v_cur = self.k_rot, v
        if self.staged:
            ka, va = L.la_kvring_next_slot(self.ring.state)
            slot = (ka - self.ring.k_slots.data_ptr()) // self.ring.k_slots[0].nbytes
            k_dst, v_cur = self.ring.k_slots[slot], self.ring.v_slots[slot]
            assert k_dst.data_ptr() == ka and v_cur.data_ptr() == va
            v_cur.copy_(v)
        L.la_rope3d_rolling(q, self.q_rot, k, k_dst, FRAMES_PER_BLOCK, f0,
                            self.ring.sink_k_raw, self.sink_k_rot, SINK_DELTA, self.table, s.Hl,
                            s.Wl, s.heads, s.head_dim, THETA, q_scale=self.q_scale)
        self.attend(v_cur, k_dst)
        ev = L.la_kvcache_append_evict(self.ring.state, k_dst, v_cur, block, NOISE_LEVEL)
        if block == 1:
            n = s.sink_tokens
            L.la_sink_replace(self.ring.state, k[:n], v[:n])
        return ev

    def attend(self, v_cur, k_cur=None):
        """la_block_attn_fwd of the rotated Q/K in place over the ring (before the append);
        k_cur defaults to the rotated-K workspace."""
        self.L.la_block_attn_fwd(self.ring.state, self.q_rot, self.sink_k_rot,
                                 self.k_rot if k_cur is None else k_cur, v_cur,
                                 self.out, self.lse, scale=self.scale, q_scale=self.q_scale,
                                 workspace=self.ws)


@functools.lru_cache(maxsize=None)
def gpu_available() -> bool:
    try:
        t = torch()
        return t.cuda.is_available()
    except Exception:
        return False


def oracle_block_all_heads(shape: si.LayerShape, block: int, rows=None, workers: int = 8,
                           **kw):
    """StreamOracle.block_output(block) for every head, the heads spread over host
    threads (numpy releases the GIL in its products and exponentials).  Returns (out
    [rows, heads, d], lse [heads, rows])."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import StreamOracle

    groups = [list(range(h, shape.heads, workers)) for h in range(min(workers, shape.heads))]

    def one(hs):
        return hs, StreamOracle(shape, heads=hs, **kw).block_output(block, rows=rows, with_lse=True)

    n = shape.block_tokens if rows is None else len(rows)
    out = np.empty((n, shape.heads, shape.head_dim))
    lse = np.empty((shape.heads, n))
    with ThreadPoolExecutor(len(groups)) as ex:
        for hs, (o, l) in ex.map(one, groups):
            out[:, hs, :] = o
            lse[hs, :] = l
    return out, lse

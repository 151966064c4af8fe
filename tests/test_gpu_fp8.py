"""FP8 (e4m3) path on the GPU against the float64 oracle: bit-exact quantisation,
and attention over e4m3 Q/K/V (streamed through an e4m3 ring) against the exact
attention of the decoded tensors.

Tolerance of the FP8 attention (derived in the design doc): the kernel rounds each
probability to e4m3 for the P V product (relative error <= 2^-4), so per
element |out - ref| <= 2^-4 * A + 2^-8 |ref| + 2^-12 max|v|, where A is the
same attention applied to |V| (the bf16 output rounding is the 2^-8 term, the
last term covers probabilities in the e4m3 subnormal range); and over a tensor
the relative L2 error stays near the rms relative rounding error of e4m3
(about 0.026): bar 0.06.  The log-sum-exp is that of the rounded probabilities
(the normaliser of the output).  Each probability's rounding error is a relative
e in [-2^-4, 2^-4] (the kernel lifts P by 2^6 before rounding, so below
p = 2^-12 of the row's reference the e4m3 subnormals give instead an absolute
error of at most 2^-16), so |lse - lse_exact| <= log(1 + 2^-4) plus the
subnormal terms.  With round-to-nearest the errors of different keys do not add
up the same way: with b_i = max(2^-4 p_i, 2^-16) the row sum's relative error
has standard deviation at most sqrt(sum b_i^2 / 3) / sum p (0.036 / sqrt(N_eff)
when no key is subnormal, N_eff = (sum p)^2 / sum p^2 the row's effective number
of keys; p from the exact probabilities).  The per-row bar is 6 of those
standard deviations plus 2^-12 for the float32 arithmetic."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_fp8, dequantize, e4m3_encode, quantize

from gpu_helpers import rel_l2, say, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

FP8_REL_L2 = 0.06
SCALE_QKV = 5.0 / 448.0  # per-tensor scale: |x| = 5 maps to the largest e4m3 value


@pytest.fixture(scope="module")
def L():
    import streaming_causal_video_amd as lib
    lib.lib()
    return lib


def inv32(scale):
    return float(np.float32(1.0) / np.float32(scale))


def gpu_quant(L, x_dev, scale):
    t = torch()
    out = t.empty(x_dev.shape, dtype=t.uint8, device="cuda")
    L.la_quantize_fp8(x_dev, out, inv32(scale))
    return out


# ------------------------------------------------------------------ quantisation
@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 64 * 1024 + 5])
def test_quantize_bf16_bit_exact(L, n):
    t = torch()
    st = si.SMALL_BF16.block_inputs(0, 1)[0]  # bf16, N(0,1)
    vals = st.values.reshape(-1)
    reps = -(-n // vals.size)
    vals = np.tile(vals, reps)[:n] * 1.0
    bits = np.tile(np.array(st.storage).reshape(-1), reps)[:n]
    x = t.from_numpy(bits.view(np.int16).copy()).cuda().view(t.bfloat16)
    for scale in (SCALE_QKV, 1.0 / 448.0, 3.0):  # |x| up to ~5: the 2nd saturates many values
        got = gpu_quant(L, x, scale).cpu().numpy()
        want = quantize(vals.astype(np.float32), scale)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"n={n} scale={scale}: {bad.size} codes differ, e.g. x={vals[bad[0]]} got {got[bad[0]]:#x} want {want[bad[0]]:#x}"


def test_quantize_f32_special_values(L):
    t = torch()
    sp = [0.0, -0.0, 1.0, -1.0, 448.0, -448.0, 449.0, 463.9, 464.0, 465.0, 480.0, 1e30, -1e30,
          2.0 ** -9, -(2.0 ** -9), 2.0 ** -10, -(2.0 ** -10), 1.5 * 2.0 ** -9, 2.0 ** -6,
          1.0625, 1.1875, 1.3125, 3e-45, -3e-45, 240.0, 232.0, 248.0]
    rng = np.random.default_rng(11)
    more = (rng.standard_normal(5000) * np.exp2(rng.integers(-14, 10, 5000))).tolist()
    x = np.array(sp + more, dtype=np.float32)
    xd = t.from_numpy(x).cuda()
    got = gpu_quant(L, xd, 1.0).cpu().numpy()
    want = e4m3_encode(x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_quantize_nan_gives_the_nan_code_of_its_sign(L):
    """NaN inputs (both signs, float32 and bf16, in the 16-element body and in the tail)
    become 0x7F / 0xFF as the oracle encodes them, never a saturated +-448."""
    t = torch()
    x = np.array([1.0, np.nan, -2.0, 3.0] * 5 + [np.copysign(np.nan, -1.0), 0.5, np.nan],
                 dtype=np.float32)  # 23 elements: one 16-element chunk and a tail of 7
    want = e4m3_encode(x.astype(np.float64))
    assert set(want[np.isnan(x)]) == {0x7F, 0xFF}
    got = gpu_quant(L, t.from_numpy(x).cuda(), 1.0).cpu().numpy()
    assert np.array_equal(got, want), (got, want)
    xb = t.from_numpy(x).cuda().to(t.bfloat16)  # NaN stays NaN, sign kept
    got_b = gpu_quant(L, xb, 1.0).cpu().numpy()
    assert np.array_equal(got_b, e4m3_encode(xb.float().cpu().numpy().astype(np.float64)))


def test_e4m3_append_at_an_odd_token_count_is_bit_exact(L):
    """An e4m3 ring of 105-token blocks x 3 heads x 128 (40,320-byte slots, an odd token
    count): appended slots equal the appended codes byte for byte, for more blocks
    than the window (eviction), and the slot index follows (b - 1) mod W."""
    t = torch()
    s = si.SMALL_BF16
    ring = L.KVRing(2, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, t.uint8, 0.75)
    sent = {}
    for b in range(1, 6):
        k = t.randint(0, 256, (s.block_tokens, s.heads, s.head_dim), dtype=t.uint8, device="cuda")
        v = t.randint(0, 256, (s.block_tokens, s.heads, s.head_dim), dtype=t.uint8, device="cuda")
        ev = L.la_kvcache_append_evict(ring.state, k, v, b, 0.75)
        assert ev == (b - 2 if b > 2 else 0)
        sent[b] = (k.clone(), v.clone())
    t.cuda.synchronize()
    for b in (4, 5):
        slot = (b - 1) % 2
        assert t.equal(ring.k_slots[slot], sent[b][0]) and t.equal(ring.v_slots[slot], sent[b][1])
    assert sorted(ring.slot_ids()) == [4, 5]


# ------------------------------------------------------------------ attention
class Fp8Stream:
    """One layer streamed through an e4m3 ring: per block, Q/K/V (bf16 stand-ins for the
    rotated projections) are quantised on the GPU with fixed per-tensor scales, the block
    attends to [sink ; window ; itself], then its K/V codes are appended.  q_pow2: Q's
    factor is the least one >= scale that makes the logit factor a power of two (the
    kernel's folded path), else Q shares K's and V's."""

    def __init__(self, L, shape, layer=0, scale=SCALE_QKV, qk_mult=1.0, q_pow2=False):
        t = torch()
        self.L, self.s, self.layer = L, shape, layer
        self.scale, self.qk_mult = scale, qk_mult
        self.dq = L.la_fp8_q_factor_pow2(shape.head_dim ** -0.5, scale, scale) if q_pow2 else scale
        s = shape
        self.ring = L.KVRing(s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, t.uint8, 0.75)
        sk, sv = s.initial_sink(layer)
        sk = self._mult(sk)
        self.sink_k8 = gpu_quant(L, to_dev(sk), scale)
        self.sink_v8 = gpu_quant(L, to_dev(sv), scale)
        self.codes = {"sink": (quantize(sk.values.astype(np.float32), scale),
                               quantize(sv.values.astype(np.float32), scale))}
        self.out = t.empty((s.block_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
        self.lse = t.empty((s.heads, s.block_tokens), dtype=t.float32, device="cuda")

    def _mult(self, x):
        # Q and K times a power of two (exact in bf16): larger, peakier logits
        return x if self.qk_mult == 1.0 else si.make_stored(x.values * self.qk_mult, "bf16")

    def step(self, b):
        L, s, sc = self.L, self.s, self.scale
        q, k, v = s.block_inputs(self.layer, b)
        q, k = self._mult(q), self._mult(k)
        fs = (self.dq, sc, sc)
        q8, k8, v8 = (gpu_quant(L, to_dev(x), f) for x, f in zip((q, k, v), fs))
        self.codes[b] = tuple(quantize(x.values.astype(np.float32), f) for x, f in zip((q, k, v), fs))
        for dev, ref in zip((q8, k8, v8), self.codes[b]):
            assert np.array_equal(dev.cpu().numpy(), ref), f"block {b}: codes differ"
        L.la_block_attn_fwd_fp8(self.ring.state, q8, self.sink_k8, self.sink_v8, k8, v8, self.out,
                                self.dq, sc, sc, lse=self.lse, scale=s.head_dim ** -0.5)
        L.la_kvcache_append_evict(self.ring.state, k8, v8, b, 0.75)

    def reference(self, b, rows=None, heads=None):
        s = self.s
        ids = list(range(max(1, b - s.W), b))
        ks = [self.codes["sink"][0]] + [self.codes[i][1] for i in ids] + [self.codes[b][1]]
        vs = [self.codes["sink"][1]] + [self.codes[i][2] for i in ids] + [self.codes[b][2]]
        q8 = self.codes[b][0]
        hs = slice(None) if heads is None else heads
        K8, V8 = np.concatenate(ks)[:, hs], np.concatenate(vs)[:, hs]
        Q8 = q8[:, hs] if rows is None else q8[rows][:, hs]
        sc, dq = self.scale, self.dq
        out, lse = attention_fp8(Q8, K8, V8, dq, sc, sc, s.head_dim ** -0.5)
        # the same attention of |V|: bounds the effect of the probability rounding
        absv = np.abs(dequantize(V8, sc))
        from oracle import attention_lse
        Qd, Kd = dequantize(Q8, dq), dequantize(K8, sc)
        bound_a, _ = attention_lse(Qd, Kd, absv, s.head_dim ** -0.5)
        self.lse_bar = lse_bar(Qd, Kd, s.head_dim ** -0.5)
        return out, lse, bound_a, absv.max()


def lse_bar(Qd, Kd, scale):
    """Per-row LSE bar [H, Nq] (module docstring) from the exact probabilities."""
    Nq, H, _ = Qd.shape
    bar = np.empty((H, Nq))
    for h in range(H):
        for r0 in range(0, Nq, 512):
            s = scale * (Qd[r0:r0 + 512, h] @ Kd[:, h].T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            b = np.maximum(2.0 ** -4 * p, 2.0 ** -16)
            sigma = np.sqrt((b * b).sum(axis=1) / 3.0) / p.sum(axis=1)
            bar[h, r0:r0 + 512] = 6 * sigma + 2.0 ** -12
    return bar


def check_lse(got, ref, bar, what):
    err = np.abs(got - ref)
    assert (err <= bar).all(), f"{what}: lse error {err.max():.3e} above its bar"
    say(f"{what}: lse max error {err.max():.3e} (bar {bar.min():.3e} .. {bar.max():.3e})")
    return float(err.max())


def check_fp8(got, ref, bound_a, vmax, what):
    err = np.abs(got - ref)
    lim = 2.0 ** -4 * bound_a + 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * vmax + 1e-6
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    worst = np.argmax(err - lim)
    assert (err <= lim).all(), f"{what}: |err| {err.flat[worst]:.3e} > bound {lim.flat[worst]:.3e}"
    r = rel_l2(got, ref)
    assert r <= FP8_REL_L2, f"{what}: rel-L2 {r:.3e} > {FP8_REL_L2}"
    return r


@pytest.mark.parametrize("q_pow2", [False, True], ids=["dq=dk", "dq-pow2"])
@pytest.mark.parametrize("shape", [si.SMALL_BF16, si.MID_BF16], ids=lambda s: f"cfg{s.cfg_id}")
def test_fp8_attention_stream_small(L, shape, q_pow2):
    t = torch()
    fs = Fp8Stream(L, shape, q_pow2=q_pow2)
    for b in range(1, shape.W + 3):
        fs.step(b)
        t.cuda.synchronize()
        out, lse, a, vmax = fs.reference(b)
        r = check_fp8(to_f64(fs.out), out, a, vmax, f"cfg{shape.cfg_id} block {b}")
        got_lse = fs.lse.cpu().numpy().astype(np.float64)
        check_lse(got_lse, lse, fs.lse_bar, f"fp8 cfg{shape.cfg_id} block {b}")
        say(f"fp8 cfg{shape.cfg_id} block {b}: rel-L2 {r:.4f}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("q_pow2", [False, True], ids=["dq=dk", "dq-pow2"])
def test_fp8_attention_c2_sampled(L, q_pow2):
    """Full C2 shape (40 heads, Nk 24960 in steady state), sampled rows and heads."""
    t = torch()
    shape = si.C2
    fs = Fp8Stream(L, shape, q_pow2=q_pow2)
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, shape.block_tokens - 1],
                                     rng.integers(0, shape.block_tokens, 48)]))
    heads = [0, 17, 39]
    for b in range(1, shape.W + 2):
        fs.step(b)
    t.cuda.synchronize()
    b = shape.W + 1
    out, lse, a, vmax = fs.reference(b, rows=rows, heads=heads)
    got = to_f64(fs.out)[rows][:, heads]
    r = check_fp8(got, out, a, vmax, "C2 fp8")
    got_lse = fs.lse.cpu().numpy().astype(np.float64)[heads][:, rows]
    check_lse(got_lse, lse, fs.lse_bar, f"fp8 C2 block {b}")
    say(f"fp8 C2 block {b}: rel-L2 {r:.4f}")


@pytest.mark.parametrize("q_pow2", [False, True], ids=["dq=dk", "dq-pow2"])
def test_fp8_window_of_one_block(L, q_pow2):
    shape = si.LayerShape(107, "bf16", heads=2, head_dim=128, Hl=6, Wl=11, W=1)
    fs = Fp8Stream(L, shape, q_pow2=q_pow2)
    for b in range(1, 5):
        fs.step(b)
        torch().cuda.synchronize()
        out, lse, a, vmax = fs.reference(b)
        r = check_fp8(to_f64(fs.out), out, a, vmax, f"W=1 block {b}")
        check_lse(fs.lse.cpu().numpy().astype(np.float64), lse, fs.lse_bar, f"fp8 W=1 block {b}")
        say(f"fp8 W=1 block {b}: rel-L2 {r:.4f}")


@pytest.mark.parametrize("q_pow2", [False, True], ids=["dq=dk", "dq-pow2"])
def test_fp8_peaked_logits(L, q_pow2):
    """Q and K times 4 (logit std ~16 after quantisation, scale 20/448 so nothing
    saturates): the row max moves between tiles and segments, so the kernel raises its
    reference max during the stream."""
    shape = si.LayerShape(108, "bf16", heads=3, head_dim=128, Hl=10, Wl=13, W=2)
    fs = Fp8Stream(L, shape, scale=20.0 / 448.0, qk_mult=4.0, q_pow2=q_pow2)
    for b in range(1, shape.W + 3):
        fs.step(b)
        torch().cuda.synchronize()
        out, lse, a, vmax = fs.reference(b)
        r = check_fp8(to_f64(fs.out), out, a, vmax, f"peaked block {b}")
        check_lse(fs.lse.cpu().numpy().astype(np.float64), lse, fs.lse_bar,
                  f"fp8 peaked block {b}")
        say(f"fp8 peaked block {b}: rel-L2 {r:.4f}")


@pytest.mark.parametrize("target_exp", [-60, 4])
def test_fp8_folded_factor_far_from_one(L, target_exp):
    """The folded path with a logit factor of 2^-60 (tiny logits: near-uniform attention)
    and 2^4 (factors near 1, so the codes are the values themselves, and logits of about
    160 in base 2: nearly an argmax), i.e. MFMA operand-scale codes far from 127, against
    the oracle; the attention scale is picked so that the helper's Q factor is near K's."""
    shape = si.LayerShape(109, "bf16", heads=2, head_dim=128, Hl=6, Wl=9, W=2)
    sc = SCALE_QKV if target_exp < 0 else 1.0
    # the attention scale that puts sc * sc * log2(e) * scale at about 2^target_exp
    attn_scale = 2.0 ** target_exp / (sc * sc * 1.4426950408889634) * 0.9
    dq = L.la_fp8_q_factor_pow2(attn_scale, sc, sc)
    f, d = np.float32, np.float64
    F = d(f(attn_scale)) * d(f(dq)) * d(f(sc)) * 1.4426950408889634
    e = np.round(np.log2(F))
    assert abs(F / 2.0 ** e - 1) <= 2.0 ** -24 and abs(e - target_exp) <= 1
    fs = Fp8Stream(L, shape, scale=sc)
    fs.dq = dq
    s = shape
    for b in range(1, s.W + 3):
        q, k, v = s.block_inputs(fs.layer, b)
        fsq = (dq, sc, sc)
        q8, k8, v8 = (gpu_quant(L, to_dev(x), f) for x, f in zip((q, k, v), fsq))
        fs.codes[b] = tuple(quantize(x.values.astype(np.float32), f) for x, f in zip((q, k, v), fsq))
        L.la_block_attn_fwd_fp8(fs.ring.state, q8, fs.sink_k8, fs.sink_v8, k8, v8, fs.out, dq, sc,
                                sc, lse=fs.lse, scale=attn_scale)
        L.la_kvcache_append_evict(fs.ring.state, k8, v8, b, 0.75)
        torch().cuda.synchronize()
        ids = list(range(max(1, b - s.W), b))
        K8 = np.concatenate([fs.codes["sink"][0]] + [fs.codes[i][1] for i in ids] + [fs.codes[b][1]])
        V8 = np.concatenate([fs.codes["sink"][1]] + [fs.codes[i][2] for i in ids] + [fs.codes[b][2]])
        out, lse = attention_fp8(fs.codes[b][0], K8, V8, dq, sc, sc, attn_scale)
        from oracle import attention_lse
        absv = np.abs(dequantize(V8, sc))
        Qd, Kd = dequantize(fs.codes[b][0], dq), dequantize(K8, sc)
        a, _ = attention_lse(Qd, Kd, absv, attn_scale)
        r = check_fp8(to_f64(fs.out), out, a, absv.max(), f"factor 2^{target_exp} block {b}")
        check_lse(fs.lse.cpu().numpy().astype(np.float64), lse, lse_bar(Qd, Kd, attn_scale),
                  f"fp8 factor 2^{target_exp} block {b}")
        say(f"fp8 factor 2^{target_exp} block {b}: rel-L2 {r:.4f}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("q_pow2", [False, True], ids=["dq=dk", "dq-pow2"])
def test_fp8_attention_c5_sampled(L, q_pow2):
    """720p-shaped layer (Nk 56320 at block 5, eviction at 6), sampled rows of two heads."""
    shape = si.C5
    fs = Fp8Stream(L, shape, q_pow2=q_pow2)
    rng = np.random.default_rng(19)
    rows = np.unique(np.concatenate([[0, 255, 256, shape.block_tokens - 1],
                                     rng.integers(0, shape.block_tokens, 40)]))
    heads = [3, 38]
    for b in range(1, shape.W + 3):
        fs.step(b)
        if b >= shape.W + 1:
            torch().cuda.synchronize()
            out, lse, a, vmax = fs.reference(b, rows=rows, heads=heads)
            got = to_f64(fs.out)[rows][:, heads]
            r = check_fp8(got, out, a, vmax, f"C5 fp8 block {b}")
            got_lse = fs.lse.cpu().numpy().astype(np.float64)[heads][:, rows]
            check_lse(got_lse, lse, fs.lse_bar, f"fp8 C5 block {b}")
            say(f"fp8 C5 block {b}: rel-L2 {r:.4f}")


# ------------------------------------------------------------------ the e4m3 step
def _bf16(x):
    """Round float64 values to bf16 (nearest even), as the step's activations are."""
    return si.make_stored(x, "bf16").values


def oracle_fp8_step_block(shape, layer, b, dq, dk, dv):
    """The e4m3 step's attention for block b of one layer, from the definitions: each
    operand rotated exactly (rotations as in StreamOracle), rounded to bf16 like the
    step's activations, quantised with its own scale; the window's blocks the same way
    at their own positions.  Returns (out, lse, bound_a, vmax, codes of K and V of b)."""
    from oracle import StreamOracle, attention_lse
    so = StreamOracle(shape, layer=layer)
    q_raw, k_raw, v = so.raw_block(b)
    f32 = np.float32
    q8 = quantize(_bf16(so.rot_block(q_raw, b)).astype(f32), dq)
    k8 = quantize(_bf16(so.rot_block(k_raw, b)).astype(f32), dk)
    v8 = quantize(v.astype(f32), dv)
    sk_raw, sv = so.sink_for(b)
    keys = [quantize(_bf16(so.rot_sink(sk_raw, b)).astype(f32), dk)]
    vals = [quantize(sv.astype(f32), dv)]
    for b2 in so.window_ids(b):
        _, k2, v2 = so.raw_block(b2)
        keys.append(quantize(_bf16(so.rot_block(k2, b2)).astype(f32), dk))
        vals.append(quantize(v2.astype(f32), dv))
    keys.append(k8)
    vals.append(v8)
    K8, V8 = np.concatenate(keys), np.concatenate(vals)
    scale = shape.head_dim ** -0.5
    out, lse = attention_fp8(q8, K8, V8, dq, dk, dv, scale)
    absv = np.abs(dequantize(V8, dv))
    bound_a, _ = attention_lse(dequantize(q8, dq), dequantize(K8, dk), absv, scale)
    return out, lse, bound_a, absv.max(), (k8, v8)


@pytest.mark.parametrize("q_pow2", [False, True], ids=["dq=dk", "dq-pow2"])
def test_fp8_denoise_step_matches_oracle(L, q_pow2):
    """la_denoise_step_fp8 over 2 layers and W + 2 blocks (sink replacement after block 1,
    evictions, an Euler step per block): each layer's output against the oracle's e4m3
    attention of the rotated, bf16-rounded and quantised operands (the fp8 bars above),
    for staged and for plain rings (staged, the block and the window are one run of
    keys, so the sums are rounded along another order than plain rings'); the latent is
    the same bits; the window's K/V codes equal the oracle's except where RoPE's bf16
    rounding differs by one ulp (then by one code)."""
    t = torch()
    s = si.SMALL_BF16
    n_layers = 2
    dq = dk = dv = SCALE_QKV
    if q_pow2:
        dq = L.la_fp8_q_factor_pow2(s.head_dim ** -0.5, dk, dk)
    stacks = {}
    for mode in ("staged", "plain"):
        st = L.KVRingStack(n_layers, s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim,
                           t.uint8, 0.75, staged=(mode == "staged"))
        for l in range(n_layers):
            sk, sv = s.initial_sink(l)
            st.sink_k_raw[l].copy_(to_dev(sk))
            st.sink_v[l].copy_(to_dev(sv))
        stacks[mode] = st
    blk, snk = (s.block_tokens, s.heads, s.head_dim), (s.sink_tokens, s.heads, s.head_dim)
    bf = lambda shp: t.empty(shp, dtype=t.bfloat16, device="cuda")
    u8 = lambda shp: t.empty(shp, dtype=t.uint8, device="cuda")
    table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                    device="cuda")
    L.la_rope_table_fill(table, s.Hl, s.Wl, s.head_dim, 10000.0)
    outs = {m: [bf(blk) for _ in range(n_layers)] for m in stacks}
    lat = si.latent(s.cfg_id, 0, si.TID_X, (2, 3, 4, 5))
    xs = {m: to_dev(lat) for m in stacks}
    nsink = s.sink_tokens
    for b in range(1, s.W + 3):
        dev = [tuple(to_dev(z) for z in s.block_inputs(l, b)) for l in range(n_layers)]
        vel = to_dev(si.latent(s.cfg_id, b, si.TID_VEL, (2, 3, 4, 5)))
        for m, st in stacks.items():
            L.la_denoise_step_fp8(
                st.states, b, [d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev],
                outs[m], bf(blk), bf(blk), bf(snk), u8(blk),
                None if m == "staged" else u8(blk), None if m == "staged" else u8(blk),
                u8(snk), u8(snk), table, s.Hl, s.Wl, 3, -1, 10000.0,
                scale=s.head_dim ** -0.5, dq=dq, dk=dk, dv=dv,
                sink_k_new=[d[1][:nsink] for d in dev] if b == 1 else None,
                sink_v_new=[d[2][:nsink] for d in dev] if b == 1 else None,
                x=xs[m], vel=vel, dt=-0.25)
        t.cuda.synchronize()
        for l in range(n_layers):
            out, lse, a, vmax, (k8, v8) = oracle_fp8_step_block(s, l, b, dq, dk, dv)
            r = check_fp8(to_f64(outs["staged"][l]), out, a, vmax, f"fp8 step layer {l} block {b}")
            check_fp8(to_f64(outs["plain"][l]), out, a, vmax, f"fp8 step plain {l} block {b}")
            for m, st in stacks.items():
                slot = (b - 1) % st.states[l].nslots
                assert int(st.states[l].slot_block[slot]) == b
                gk = st.k_slots[l, slot].cpu().numpy()
                gv = st.v_slots[l, slot].cpu().numpy()
                assert np.array_equal(gv, v8), f"{m} block {b} layer {l}: V codes differ"
                diff = gk != k8
                assert diff.mean() <= 1e-3, f"{m} block {b} layer {l}: {diff.sum()} K codes differ"
                # a differing code is a neighbour of the oracle's: one bf16 ulp before the
                # quantisation moves a value across at most one e4m3 rounding boundary
                step_ = np.abs(dequantize(gk[diff], dk) - dequantize(k8[diff], dk))
                ref_ = np.abs(dequantize(k8[diff], dk))
                assert (step_ <= ref_ * 2.0 ** -2 + 2.0 ** -9 * dk).all(), m
            say(f"fp8 step layer {l} block {b}: rel-L2 {r:.4f}, K codes differing from the "
                f"oracle's {int(diff.sum())} of {diff.size}")
    assert t.equal(xs["staged"], xs["plain"])
    for m, st in stacks.items():
        for l in range(n_layers):
            assert st.states[l].last_block == s.W + 2 and st.states[l].sink_replaced == 1


@pytest.mark.timeout(900)
def test_fp8_denoise_step_c2_sampled(L):
    """The e4m3 step at the C2 shape (one layer, staged ring, blocks 1..W+1: the ring
    full at the last one, Nk 24960): sampled rows of three heads against the oracle's
    e4m3 attention, and the last block's window V codes bit for bit.  Q's factor is the
    power-of-two one of the e4m3 step benchmark (the kernel's folded path)."""
    t = torch()
    s = si.C2
    dk = dv = SCALE_QKV
    dq = L.la_fp8_q_factor_pow2(s.head_dim ** -0.5, dk, dk)
    st = L.KVRingStack(1, s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, t.uint8, 0.75,
                       staged=True)
    sk, sv = s.initial_sink(0)
    st.sink_k_raw[0].copy_(to_dev(sk))
    st.sink_v[0].copy_(to_dev(sv))
    blk, snk = (s.block_tokens, s.heads, s.head_dim), (s.sink_tokens, s.heads, s.head_dim)
    bf = lambda shp: t.empty(shp, dtype=t.bfloat16, device="cuda")
    u8 = lambda shp: t.empty(shp, dtype=t.uint8, device="cuda")
    table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                    device="cuda")
    L.la_rope_table_fill(table, s.Hl, s.Wl, s.head_dim, 10000.0)
    out = [bf(blk)]
    ws = (bf(blk), bf(blk), bf(snk), u8(blk), None, None, u8(snk), u8(snk))
    last = s.W + 1
    for b in range(1, last + 1):
        q, k, v = (to_dev(z) for z in s.block_inputs(0, b))
        L.la_denoise_step_fp8(st.states, b, [q], [k], [v], out, *ws, table, s.Hl, s.Wl, 3, -1,
                              10000.0, scale=s.head_dim ** -0.5, dq=dq, dk=dk, dv=dv,
                              sink_k_new=[k[:s.sink_tokens]] if b == 1 else None,
                              sink_v_new=[v[:s.sink_tokens]] if b == 1 else None)
    t.cuda.synchronize()
    rng = np.random.default_rng(23)
    rows = np.unique(np.concatenate([[0, s.block_tokens - 1], rng.integers(0, s.block_tokens, 40)]))
    heads = [0, 21, 39]
    from oracle import StreamOracle, attention_lse
    so = StreamOracle(s, layer=0, heads=heads)
    f32 = np.float32
    q_raw, k_raw, v = so.raw_block(last)
    q8 = quantize(_bf16(so.rot_block(q_raw, last)).astype(f32), dq)
    keys = [quantize(_bf16(so.rot_sink(so.sink_for(last)[0], last)).astype(f32), dk)]
    vals = [quantize(so.sink_for(last)[1].astype(f32), dv)]
    for b2 in so.window_ids(last):
        _, k2, v2 = so.raw_block(b2)
        keys.append(quantize(_bf16(so.rot_block(k2, b2)).astype(f32), dk))
        vals.append(quantize(v2.astype(f32), dv))
    keys.append(quantize(_bf16(so.rot_block(k_raw, last)).astype(f32), dk))
    vals.append(quantize(v.astype(f32), dv))
    K8, V8 = np.concatenate(keys), np.concatenate(vals)
    scale = s.head_dim ** -0.5
    ref, _ = attention_fp8(q8[rows], K8, V8, dq, dk, dv, scale)
    absv = np.abs(dequantize(V8, dv))
    bound_a, _ = attention_lse(dequantize(q8[rows], dq), dequantize(K8, dk), absv, scale)
    got = to_f64(out[0])[rows][:, heads]
    r = check_fp8(got, ref, bound_a, absv.max(), "fp8 step C2")
    slot = (last - 1) % (s.W + 1)
    gv = st.v_slots[0, slot].cpu().numpy()[:, heads]
    assert np.array_equal(gv, vals[-1]), "C2 last block: V codes differ"
    say(f"fp8 step C2 block {last}: rel-L2 {r:.4f}")


@pytest.mark.parametrize("block_id", [1, 3])
def test_fp8_step_codes_equal_rope_then_quantise(L, block_id):
    """The e4m3 step's one RoPE + quantisation launch writes, bit for bit, the codes of
    la_rope3d_rolling (bf16 out) followed by la_quantize_fp8: Q, the sink K and the sink V
    in their workspaces, K and V in k8_ws / v8_ws (plain ring, attend-only, so the step
    keeps them there), at block 1 and at a later block (other frame positions)."""
    t = torch()
    s = si.MID_BF16
    dk = dv = SCALE_QKV
    dq = L.la_fp8_q_factor_pow2(s.head_dim ** -0.5, dk, dk)
    st = L.KVRingStack(1, s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, t.uint8,
                       0.75, staged=False)
    sk, sv = s.initial_sink(0)
    st.sink_k_raw[0].copy_(to_dev(sk))
    st.sink_v[0].copy_(to_dev(sv))
    # bring the ring to block_id - 1 (appending zero codes) so the step accepts block_id
    z8 = t.zeros((s.block_tokens, s.heads, s.head_dim), dtype=t.uint8, device="cuda")
    for b in range(1, block_id):
        L.la_kvcache_append_evict(st.states[0], z8, z8, b, 0.75)
    blk, snk = (s.block_tokens, s.heads, s.head_dim), (s.sink_tokens, s.heads, s.head_dim)
    u8 = lambda shp: t.full(shp, 0xAA, dtype=t.uint8, device="cuda")
    bf = lambda shp: t.empty(shp, dtype=t.bfloat16, device="cuda")
    table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                    device="cuda")
    L.la_rope_table_fill(table, s.Hl, s.Wl, s.head_dim, 10000.0)
    q, k, v = (to_dev(z) for z in s.block_inputs(0, block_id))
    q8, k8, v8, sk8, sv8 = u8(blk), u8(blk), u8(blk), u8(snk), u8(snk)
    L.la_denoise_step_fp8(st.states, block_id, [q], [k], [v], [bf(blk)], None, None, None, q8,
                          k8, v8, sk8, sv8, table, s.Hl, s.Wl, 3, -1, 10000.0,
                          scale=s.head_dim ** -0.5, dq=dq, dk=dk, dv=dv,
                          flags=L.LA_STEP_ATTEND_ONLY)
    qr, kr, skr = bf(blk), bf(blk), bf(snk)
    L.la_rope3d_rolling(q, qr, k, kr, 3, 3 * (block_id - 1), st.sink_k_raw[0], skr, -1, table,
                        s.Hl, s.Wl, s.heads, s.head_dim, 10000.0, 1.0)
    want = []
    for x, f in ((qr, dq), (kr, dk), (v, dv), (skr, dk), (st.sink_v[0], dv)):
        o = t.empty(x.shape, dtype=t.uint8, device="cuda")
        L.la_quantize_fp8(x, o, inv32(f))
        want.append(o)
    t.cuda.synchronize()
    for name, got, ref in zip(("Q", "K", "V", "sink K", "sink V"), (q8, k8, v8, sk8, sv8), want):
        assert t.equal(got, ref), f"block {block_id} {name}: {(got != ref).sum().item()} codes differ"
    say(f"fp8 step block {block_id}: the five code tensors equal RoPE then quantisation")

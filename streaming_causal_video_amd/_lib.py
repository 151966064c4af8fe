"""ctypes binding of liblahip (argument marshalling only).

Every function here has the name of the C entry point it calls and does
nothing but check tensors (device, dtype, contiguity, size), pass their
device pointers and the current HIP stream, and turn a non-zero status into
an exception.  All arithmetic runs in the HIP kernels.  There is no fallback:
if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "liblahip.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_STATE, LA_ERR_NOISE_LEVEL, \
    LA_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
LA_BF16, LA_F32, LA_FP8_E4M3 = 0, 1, 2
LA_MAX_WINDOW = 64
LA_STEP_ATTEND_ONLY = 1
LA_MAX_BLOCK_FRAMES = 4

EXPORTED = [
    "la_status_string", "la_last_hip_error", "la_version", "la_kvring_init",
    "la_kvring_init_staged", "la_kvring_advance", "la_kvring_next_slot", "la_kvring_count", "la_rope_table_bytes", "la_rope_table_fill", "la_rope3d_rolling",
    "la_block_attn_fwd", "la_kvcache_append_evict", "la_sink_replace", "la_fm_euler_step",
    "la_denoise_step", "la_denoise_chain", "la_quantize_fp8", "la_block_attn_fwd_fp8",
    "la_attn_workspace_bytes", "la_block_attn_fwd_noalloc", "la_denoise_step_fp8",
    "la_fp8_q_factor_pow2",
]


class la_kvring(ctypes.Structure):
    """Mirror of the C struct la_kvring (include/la.h)."""

    _fields_ = [
        ("k_slots", ctypes.c_void_p),
        ("v_slots", ctypes.c_void_p),
        ("sink_k_raw", ctypes.c_void_p),
        ("sink_v", ctypes.c_void_p),
        ("W", ctypes.c_int32),
        ("nslots", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("noise_level", ctypes.c_float),
        ("sink_replaced", ctypes.c_int32),
        ("last_block", ctypes.c_int64),
        ("slot_block", ctypes.c_int64 * LA_MAX_WINDOW),
    ]


class la_stage(ctypes.Structure):
    """Mirror of the C struct la_stage (include/la.h): one stage of la_denoise_chain."""

    _fields_ = [
        ("rings", ctypes.POINTER(la_kvring)),
        ("q_raw", ctypes.POINTER(ctypes.c_void_p)),
        ("k_raw", ctypes.POINTER(ctypes.c_void_p)),
        ("v_raw", ctypes.POINTER(ctypes.c_void_p)),
        ("attn_out", ctypes.POINTER(ctypes.c_void_p)),
        ("sink_k_new", ctypes.POINTER(ctypes.c_void_p)),
        ("sink_v_new", ctypes.POINTER(ctypes.c_void_p)),
        ("vel", ctypes.c_void_p),
        ("dt", ctypes.c_float),
    ]


class LAError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = _load()
        msg = lib.la_status_string(status).decode()
        if status == LA_ERR_HIP:
            msg += " (" + lib.la_last_hip_error().decode() + ")"
        super().__init__(f"{what}: {msg} [{status}]")
        self.status = status


_LIB = None


def _hip_runtimes_mapped():
    """Paths of the HIP runtime libraries mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split()[-1] if line.strip() else ""
                if "libamdhip64.so" in os.path.basename(p):
                    paths.add(os.path.realpath(p))
    except OSError:
        pass
    return paths


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m streaming_causal_video_amd.build`")
    # The library takes PyTorch's device pointers, streams and events, so it must
    # run on the same HIP runtime as PyTorch.  PyTorch ships its own copy with the
    # same soname: loading torch first makes the dynamic linker bind liblahip's
    # libamdhip64.so.7 dependency to it instead of mapping a second runtime.
    import torch  # noqa: F401
    import torch.cuda  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are mapped into this process "
                          f"({sorted(runtimes)}); import torch before anything loads "
                          "/opt/rocm's libamdhip64")
    P, I32, I64, F, D, VP = (ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_double, ctypes.c_void_p)
    SZ = ctypes.c_size_t
    R = P(la_kvring)
    sig = {
        "la_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "la_last_hip_error": (ctypes.c_char_p, []),
        "la_version": (ctypes.c_char_p, []),
        "la_kvring_init": (ctypes.c_int, [R, VP, VP, VP, VP, I32, I32, I32, I32, I32, ctypes.c_int, F]),
        "la_kvring_init_staged": (ctypes.c_int, [R, VP, VP, VP, VP, I32, I32, I32, I32, I32,
                                                 ctypes.c_int, F]),
        "la_kvring_advance": (ctypes.c_int, [R, I64, P(I32), P(I64)]),
        "la_kvring_next_slot": (ctypes.c_int, [R, P(VP), P(VP)]),
        "la_kvring_count": (I32, [R]),
        "la_rope_table_bytes": (ctypes.c_size_t, [I32, I32, I32]),
        "la_rope_table_fill": (ctypes.c_int, [VP, I32, I32, I32, D, VP]),
        "la_rope3d_rolling": (ctypes.c_int, [VP, VP, VP, VP, I32, I64, VP, VP, I64, VP, I32, I32,
                                             I32, I32, ctypes.c_int, D, F, VP]),
        "la_block_attn_fwd": (ctypes.c_int, [R, VP, VP, VP, VP, I32, VP, VP, F, F, VP, SZ, VP]),
        "la_attn_workspace_bytes": (SZ, [I32, I32]),
        "la_block_attn_fwd_noalloc": (ctypes.c_int, [R, VP, VP, VP, VP, I32, VP, VP, F, F, VP]),
        "la_kvcache_append_evict": (ctypes.c_int, [R, VP, VP, I64, F, P(I64), VP]),
        "la_sink_replace": (ctypes.c_int, [R, VP, VP, VP]),
        "la_fm_euler_step": (ctypes.c_int, [VP, VP, I64, F, VP]),
        "la_denoise_step": (ctypes.c_int, [R, I32, I64, P(VP), P(VP), P(VP), P(VP), VP, VP, VP,
                                           P(VP), P(VP), VP, I32, I32, I32, I64, D, F, VP, SZ,
                                           VP, VP, I64, F, ctypes.c_uint32, P(VP), VP]),
        "la_denoise_step_fp8": (ctypes.c_int, [R, I32, I64, P(VP), P(VP), P(VP), P(VP), VP, VP,
                                               VP, VP, VP, VP, VP, VP, P(VP), P(VP), VP, I32,
                                               I32, I32, I64, D, F, F, F, F, VP, VP, I64, F,
                                               ctypes.c_uint32, P(VP), VP]),
        "la_quantize_fp8": (ctypes.c_int, [VP, ctypes.c_int, VP, I64, F, VP]),
        "la_block_attn_fwd_fp8": (ctypes.c_int, [R, VP, VP, VP, VP, VP, I32, VP, VP, F, F, F, F,
                                                 VP]),
        "la_fp8_q_factor_pow2": (ctypes.c_int, [F, F, F, P(F)]),
        "la_denoise_chain": (ctypes.c_int, [P(la_stage), I32, I32, I64, VP, VP, VP, VP, I32, I32,
                                            I32, I64, D, F, VP, SZ, VP, I64, VP]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def lib():
    """The loaded CDLL (raises ImportError if liblahip.so has not been built)."""
    return _load()


# ---------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_tensor(t, name: str, shape=None, dtype=None):
    """Shape, dtype and contiguity of a tensor argument (not its device)."""
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t, name: str, shape=None, dtype=None):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    _check_tensor(t, name, shape, dtype)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return ctypes.c_void_p(t.data_ptr())


def _check(status: int, what: str):
    if status != LA_OK:
        raise LAError(status, what)


# ---------------------------------------------------------------- C entry points
def la_version() -> str:
    return _load().la_version().decode()


def _addr(x):
    return ctypes.c_void_p(x if isinstance(x, int) else x.data_ptr())


def la_kvring_init(ring: "la_kvring", k_slots, v_slots, sink_k_raw, sink_v, W: int,
                   block_tokens: int, sink_tokens: int, heads: int, head_dim: int,
                   dtype: int, noise_level: float) -> None:
    """Pointers may be tensors or raw integer addresses."""
    _check(_load().la_kvring_init(ctypes.byref(ring), _addr(k_slots), _addr(v_slots),
                                  _addr(sink_k_raw), _addr(sink_v), W, block_tokens, sink_tokens,
                                  heads, head_dim, dtype, noise_level), "la_kvring_init")


def la_kvring_init_staged(ring: "la_kvring", k_slots, v_slots, sink_k_raw, sink_v, W: int,
                          block_tokens: int, sink_tokens: int, heads: int, head_dim: int,
                          dtype: int, noise_level: float) -> None:
    """la_kvring_init with W + 1 slots in k_slots / v_slots."""
    _check(_load().la_kvring_init_staged(ctypes.byref(ring), _addr(k_slots), _addr(v_slots),
                                         _addr(sink_k_raw), _addr(sink_v), W, block_tokens,
                                         sink_tokens, heads, head_dim, dtype, noise_level),
           "la_kvring_init_staged")


def la_kvring_next_slot(ring: "la_kvring"):
    """(k_slot, v_slot) device addresses where block last_block + 1 will be stored."""
    k = ctypes.c_void_p()
    v = ctypes.c_void_p()
    _check(_load().la_kvring_next_slot(ctypes.byref(ring), ctypes.byref(k), ctypes.byref(v)),
           "la_kvring_next_slot")
    return k.value, v.value


def la_kvring_advance(ring: "la_kvring", block_id: int):
    """(slot, evicted) for appending block_id; raises LAError(LA_ERR_STATE) if out of order."""
    slot = ctypes.c_int32()
    ev = ctypes.c_int64()
    _check(_load().la_kvring_advance(ctypes.byref(ring), block_id, ctypes.byref(slot),
                                     ctypes.byref(ev)), "la_kvring_advance")
    return slot.value, ev.value


def la_kvring_count(ring: "la_kvring") -> int:
    return _load().la_kvring_count(ctypes.byref(ring))


def la_rope_table_bytes(Hl: int, Wl: int, head_dim: int) -> int:
    return _load().la_rope_table_bytes(Hl, Wl, head_dim)


def la_rope_table_fill(table, Hl: int, Wl: int, head_dim: int, theta: float = 10000.0) -> None:
    torch = _torch()
    need = la_rope_table_bytes(Hl, Wl, head_dim)
    if table.dtype != torch.float32 or table.numel() * 4 < need:
        raise ValueError("table must be float32 with at least la_rope_table_bytes bytes")
    _check(_load().la_rope_table_fill(_ptr(table, "table"), Hl, Wl, head_dim, theta, _stream()),
           "la_rope_table_fill")


def la_rope3d_rolling(q_in, q_out, k_in, k_out, n_frames: int, f0: int, sink_k_in, sink_k_out,
                      sink_delta: int, table, Hl: int, Wl: int, heads: int, head_dim: int,
                      theta: float = 10000.0, q_scale: float = 1.0) -> None:
    """q_out = q_scale * rotated q_in (q_scale = 1: the plain rotation)."""
    ref = next(t for t in (q_in, k_in, sink_k_in) if t is not None)
    dt = _dtype_code(ref)
    blk = (n_frames * Hl * Wl, heads, head_dim)
    snk = (Hl * Wl, heads, head_dim)
    args = [_ptr(q_in, "q_in", blk, ref.dtype), _ptr(q_out, "q_out", blk, ref.dtype),
            _ptr(k_in, "k_in", blk, ref.dtype), _ptr(k_out, "k_out", blk, ref.dtype)]
    sargs = [_ptr(sink_k_in, "sink_k_in", snk, ref.dtype),
             _ptr(sink_k_out, "sink_k_out", snk, ref.dtype)]
    _check(_load().la_rope3d_rolling(*args, n_frames, f0, *sargs, sink_delta,
                                     _ptr(table, "table"), Hl, Wl, heads, head_dim, dt, theta,
                                     q_scale, _stream()), "la_rope3d_rolling")


def la_attn_workspace_bytes(n_q: int, heads: int) -> int:
    return _load().la_attn_workspace_bytes(n_q, heads)


class AttnWorkspace:
    """Zero-filled device buffer for la_block_attn_fwd's balanced schedule (one per
    stream of attention calls; each call leaves it zero-filled again)."""

    def __init__(self, n_q: int, heads: int, device="cuda"):
        torch = _torch()
        self.nbytes = la_attn_workspace_bytes(n_q, heads)
        if self.nbytes == 0:
            raise ValueError("la_attn_workspace_bytes failed (arguments or device)")
        self.buf = torch.zeros(self.nbytes, dtype=torch.uint8, device=device)
        if self.buf.data_ptr() % 256:
            raise RuntimeError("attention workspace is not 256-byte aligned")


def _ws(ws: Optional[AttnWorkspace]):
    if ws is None:
        return None, 0
    return _ptr(ws.buf, "workspace"), ws.nbytes


def la_block_attn_fwd(ring: "la_kvring", q_rot, sink_k_rot, k_cur_rot, v_cur, out,
                      lse: Optional[object] = None, *, scale: float, q_scale: float = 1.0,
                      workspace: Optional[AttnWorkspace] = None) -> None:
    """scale: the softmax scale of the scores; q_scale: the factor already applied to
    q_rot (la_rope3d_rolling's q_scale); workspace: None or an AttnWorkspace."""
    torch = _torch()
    dtype = torch.bfloat16 if ring.dtype == LA_BF16 else torch.float32
    blk = (ring.block_tokens, ring.heads, ring.head_dim)
    snk = (ring.sink_tokens, ring.heads, ring.head_dim)
    lse_p = None
    if lse is not None:
        lse_p = _ptr(lse, "lse", (ring.heads, ring.block_tokens), torch.float32)
    ws_p, ws_n = _ws(workspace)
    _check(_load().la_block_attn_fwd(
        ctypes.byref(ring), _ptr(q_rot, "q_rot", blk, dtype), _ptr(sink_k_rot, "sink_k_rot", snk, dtype),
        _ptr(k_cur_rot, "k_cur_rot", blk, dtype), _ptr(v_cur, "v_cur", blk, dtype),
        ring.block_tokens, _ptr(out, "out", blk, dtype), lse_p, scale, q_scale, ws_p, ws_n,
        _stream()), "la_block_attn_fwd")


def la_block_attn_fwd_noalloc(ring: "la_kvring", q_rot, sink_k_rot, k_cur_rot, v_cur, out,
                              lse: Optional[object] = None, *, scale: float,
                              q_scale: float = 1.0) -> None:
    """la_block_attn_fwd with the library's static workspace (no allocation)."""
    torch = _torch()
    dtype = torch.bfloat16 if ring.dtype == LA_BF16 else torch.float32
    blk = (ring.block_tokens, ring.heads, ring.head_dim)
    snk = (ring.sink_tokens, ring.heads, ring.head_dim)
    lse_p = None
    if lse is not None:
        lse_p = _ptr(lse, "lse", (ring.heads, ring.block_tokens), torch.float32)
    _check(_load().la_block_attn_fwd_noalloc(
        ctypes.byref(ring), _ptr(q_rot, "q_rot", blk, dtype), _ptr(sink_k_rot, "sink_k_rot", snk, dtype),
        _ptr(k_cur_rot, "k_cur_rot", blk, dtype), _ptr(v_cur, "v_cur", blk, dtype),
        ring.block_tokens, _ptr(out, "out", blk, dtype), lse_p, scale, q_scale, _stream()),
        "la_block_attn_fwd_noalloc")


def _slot_dtype(ring: "la_kvring"):
    torch = _torch()
    return {LA_BF16: torch.bfloat16, LA_F32: torch.float32, LA_FP8_E4M3: torch.uint8}[ring.dtype]


def _sink_dtype(ring: "la_kvring"):
    torch = _torch()
    return torch.bfloat16 if ring.dtype == LA_FP8_E4M3 else _slot_dtype(ring)


def la_quantize_fp8(x, out, inv_scale: float) -> None:
    """out (uint8 tensor of x.numel() codes) = e4m3(x * inv_scale); x bf16 or float32."""
    torch = _torch()
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bf16 or float32")
    if out.dtype != torch.uint8 or out.numel() != x.numel():
        raise ValueError("out must be a uint8 tensor with x.numel() elements")
    _check(_load().la_quantize_fp8(_ptr(x, "x"), LA_BF16 if x.dtype == torch.bfloat16 else LA_F32,
                                   _ptr(out, "out"), x.numel(), inv_scale, _stream()),
           "la_quantize_fp8")


def la_block_attn_fwd_fp8(ring: "la_kvring", q8, sink_k8, sink_v8, k8_cur, v8_cur, out, dq: float,
                          dk: float, dv: float, lse: Optional[object] = None, *,
                          scale: float) -> None:
    """e4m3 attention: q8, sink_k8, sink_v8, k8_cur, v8_cur are uint8 code tensors, out bf16."""
    torch = _torch()
    blk = (ring.block_tokens, ring.heads, ring.head_dim)
    snk = (ring.sink_tokens, ring.heads, ring.head_dim)
    u8 = torch.uint8
    lse_p = None
    if lse is not None:
        lse_p = _ptr(lse, "lse", (ring.heads, ring.block_tokens), torch.float32)
    _check(_load().la_block_attn_fwd_fp8(
        ctypes.byref(ring), _ptr(q8, "q8", blk, u8), _ptr(sink_k8, "sink_k8", snk, u8),
        _ptr(sink_v8, "sink_v8", snk, u8), _ptr(k8_cur, "k8_cur", blk, u8),
        _ptr(v8_cur, "v8_cur", blk, u8), ring.block_tokens, _ptr(out, "out", blk, torch.bfloat16),
        lse_p, scale, dq, dk, dv, _stream()), "la_block_attn_fwd_fp8")


def la_fp8_q_factor_pow2(scale: float, dk: float, dq_min: float) -> float:
    """The least float32 dq >= dq_min whose e4m3 logit factor is a power of two (host only)."""
    dq = ctypes.c_float()
    _check(_load().la_fp8_q_factor_pow2(scale, dk, dq_min, ctypes.byref(dq)), "la_fp8_q_factor_pow2")
    return dq.value


def la_kvcache_append_evict(ring: "la_kvring", k_rot, v, block_id: int, noise_level: float) -> int:
    """Returns the evicted block id (0 if none)."""
    dtype = _slot_dtype(ring)
    blk = (ring.block_tokens, ring.heads, ring.head_dim)
    ev = ctypes.c_int64()
    _check(_load().la_kvcache_append_evict(ctypes.byref(ring), _ptr(k_rot, "k_rot", blk, dtype),
                                           _ptr(v, "v", blk, dtype), block_id, noise_level,
                                           ctypes.byref(ev), _stream()), "la_kvcache_append_evict")
    return ev.value


def la_sink_replace(ring: "la_kvring", k_new_raw, v_new) -> None:
    dtype = _sink_dtype(ring)
    snk = (ring.sink_tokens, ring.heads, ring.head_dim)
    _check(_load().la_sink_replace(ctypes.byref(ring), _ptr(k_new_raw, "k_new_raw", snk, dtype),
                                   _ptr(v_new, "v_new", snk, dtype), _stream()), "la_sink_replace")


def la_fm_euler_step(x, v, dt: float) -> None:
    torch = _torch()
    if x.dtype != torch.float32 or v.dtype != torch.float32 or x.numel() != v.numel():
        raise ValueError("x and v must be float32 tensors of equal size")
    _check(_load().la_fm_euler_step(_ptr(x, "x"), _ptr(v, "v"), x.numel(), dt, _stream()),
           "la_fm_euler_step")


def _check_list(ts, name, shape=None, dtype=None, n=None):
    """_check_tensor on every entry of a per-layer tensor list of length n."""
    if n is not None and len(ts) != n:
        raise ValueError(f"{name} has {len(ts)} entries, expected {n}")
    for i, t in enumerate(ts):
        if t is None:
            raise ValueError(f"{name}[{i}] is None")
        _check_tensor(t, f"{name}[{i}]", shape, dtype)


def _ptr_array(ts, name, shape=None, dtype=None, n=None):
    """Host array of the device pointers of a list of tensors, each checked like _ptr."""
    _check_list(ts, name, shape, dtype, n)
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t, f"{name}[{i}]", shape, dtype).value
    return arr


def _step_dtype(ring: "la_kvring"):
    """Tensor dtype of a step's per-layer activations (the step runs bf16 / f32 rings)."""
    torch = _torch()
    if ring.dtype == LA_BF16:
        return torch.bfloat16
    if ring.dtype == LA_F32:
        return torch.float32
    raise ValueError("la_denoise_step / la_denoise_chain run bf16 or float32 rings only")


def _check_table(table, Hl: int, Wl: int, head_dim: int):
    torch = _torch()
    need = la_rope_table_bytes(Hl, Wl, head_dim)
    if table.dtype != torch.float32 or table.numel() * 4 < need:
        raise ValueError("rope_table must be float32 with at least la_rope_table_bytes bytes")


def la_denoise_step(rings, block_id: int, q_raw, k_raw, v_raw, attn_out, q_rot_ws, k_rot_ws,
                    sink_k_rot_ws, rope_table, Hl: int, Wl: int, frames_per_block: int = 3,
                    sink_delta: int = -1, theta: float = 10000.0, *, scale: float,
                    sink_k_new=None, sink_v_new=None, x=None, vel=None, dt: float = -0.25,
                    timing_events=None, flags: int = 0,
                    attn_ws: Optional[AttnWorkspace] = None) -> None:
    """rings: a ctypes array of la_kvring (see KVRingStack); the other per-layer
    arguments are lists of tensors.  scale: the softmax scale.  timing_events: None or a
    ctypes array of 6*len(rings)+2 raw hipEvent_t handles.  flags: LA_STEP_ATTEND_ONLY
    or 0.  attn_ws: None or an AttnWorkspace for the attention's balanced schedule."""
    torch = _torch()
    n = len(rings)
    if n < 1:
        raise ValueError("rings is empty")
    r0 = rings[0]
    dtype = _step_dtype(r0)
    blk = (r0.block_tokens, r0.heads, r0.head_dim)
    snk = (r0.sink_tokens, r0.heads, r0.head_dim)
    # every shape and dtype first, then the pointers
    lists = [(q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (attn_out, "attn_out")]
    for ts, name in lists:
        _check_list(ts, name, blk, dtype, n)
    for ts, name in ((sink_k_new, "sink_k_new"), (sink_v_new, "sink_v_new")):
        if ts is not None:
            _check_list(ts, name, snk, dtype, n)
    for t, name, shp in ((q_rot_ws, "q_rot_ws", blk), (k_rot_ws, "k_rot_ws", blk),
                         (sink_k_rot_ws, "sink_k_rot_ws", snk)):
        _check_tensor(t, name, shp, dtype)
    n_lat = 0 if x is None else x.numel()
    if x is not None:
        if vel is None or vel.numel() != n_lat:
            raise ValueError("vel must match x")
        if x.dtype != torch.float32 or vel.dtype != torch.float32:
            raise ValueError("x and vel must be float32")
    if timing_events is not None and len(timing_events) != 6 * n + 2:
        raise ValueError(f"timing_events needs {6 * n + 2} events")
    _check_table(rope_table, Hl, Wl, r0.head_dim)
    skn = _ptr_array(sink_k_new, "sink_k_new", snk, dtype, n) if sink_k_new is not None else None
    svn = _ptr_array(sink_v_new, "sink_v_new", snk, dtype, n) if sink_v_new is not None else None
    ws_p, ws_n = _ws(attn_ws)
    _check(_load().la_denoise_step(
        rings, n, block_id, _ptr_array(q_raw, "q_raw", blk, dtype, n),
        _ptr_array(k_raw, "k_raw", blk, dtype, n), _ptr_array(v_raw, "v_raw", blk, dtype, n),
        _ptr_array(attn_out, "attn_out", blk, dtype, n), _ptr(q_rot_ws, "q_rot_ws", blk, dtype),
        _ptr(k_rot_ws, "k_rot_ws", blk, dtype), _ptr(sink_k_rot_ws, "sink_k_rot_ws", snk, dtype),
        skn, svn, _ptr(rope_table, "rope_table"), Hl, Wl, frames_per_block, sink_delta, theta,
        scale, ws_p, ws_n, _ptr(x, "x"), _ptr(vel, "vel"), n_lat, dt, flags, timing_events,
        _stream()), "la_denoise_step")


def la_denoise_step_fp8(rings, block_id: int, q_raw, k_raw, v_raw, attn_out, q_rot_ws, k_rot_ws,
                        sink_k_rot_ws, q8_ws, k8_ws, v8_ws, sink_k8_ws, sink_v8_ws, rope_table,
                        Hl: int, Wl: int, frames_per_block: int = 3, sink_delta: int = -1,
                        theta: float = 10000.0, *, scale: float, dq: float, dk: float,
                        dv: float, sink_k_new=None, sink_v_new=None, x=None, vel=None,
                        dt: float = -0.25, timing_events=None, flags: int = 0) -> None:
    """la_denoise_step for e4m3 rings (KVRingStack(..., torch.uint8)): bf16 activations,
    uint8 code workspaces (k8_ws / v8_ws may be None when the rings are staged and the
    step appends; q_rot_ws, k_rot_ws and sink_k_rot_ws are unused and may be None).
    dq, dk, dv: the per-tensor dequantisation scales."""
    torch = _torch()
    n = len(rings)
    if n < 1:
        raise ValueError("rings is empty")
    r0 = rings[0]
    if r0.dtype != LA_FP8_E4M3:
        raise ValueError("la_denoise_step_fp8 runs e4m3 rings only")
    bf, u8 = torch.bfloat16, torch.uint8
    blk = (r0.block_tokens, r0.heads, r0.head_dim)
    snk = (r0.sink_tokens, r0.heads, r0.head_dim)
    for ts, name in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (attn_out, "attn_out")):
        _check_list(ts, name, blk, bf, n)
    for ts, name in ((sink_k_new, "sink_k_new"), (sink_v_new, "sink_v_new")):
        if ts is not None:
            _check_list(ts, name, snk, bf, n)
    for t, name, shp, dt_ in ((q8_ws, "q8_ws", blk, u8), (sink_k8_ws, "sink_k8_ws", snk, u8),
                              (sink_v8_ws, "sink_v8_ws", snk, u8)):
        _check_tensor(t, name, shp, dt_)
    for t, name in ((k8_ws, "k8_ws"), (v8_ws, "v8_ws")):
        if t is not None:
            _check_tensor(t, name, blk, u8)
    n_lat = 0 if x is None else x.numel()
    if x is not None:
        if vel is None or vel.numel() != n_lat:
            raise ValueError("vel must match x")
        if x.dtype != torch.float32 or vel.dtype != torch.float32:
            raise ValueError("x and vel must be float32")
    if timing_events is not None and len(timing_events) != 6 * n + 2:
        raise ValueError(f"timing_events needs {6 * n + 2} events")
    _check_table(rope_table, Hl, Wl, r0.head_dim)
    skn = _ptr_array(sink_k_new, "sink_k_new", snk, bf, n) if sink_k_new is not None else None
    svn = _ptr_array(sink_v_new, "sink_v_new", snk, bf, n) if sink_v_new is not None else None
    _check(_load().la_denoise_step_fp8(
        rings, n, block_id, _ptr_array(q_raw, "q_raw", blk, bf, n),
        _ptr_array(k_raw, "k_raw", blk, bf, n), _ptr_array(v_raw, "v_raw", blk, bf, n),
        _ptr_array(attn_out, "attn_out", blk, bf, n), None, None, None, _ptr(q8_ws, "q8_ws"),
        _ptr(k8_ws, "k8_ws"), _ptr(v8_ws, "v8_ws"), _ptr(sink_k8_ws, "sink_k8_ws"),
        _ptr(sink_v8_ws, "sink_v8_ws"), skn, svn, _ptr(rope_table, "rope_table"), Hl, Wl,
        frames_per_block, sink_delta, theta, scale, dq, dk, dv, _ptr(x, "x"), _ptr(vel, "vel"),
        n_lat, dt, flags, timing_events, _stream()), "la_denoise_step_fp8")


def la_denoise_chain(stages, block_id: int, q_rot_ws, k_rot_ws, sink_k_rot_ws, rope_table,
                     Hl: int, Wl: int, x=None, frames_per_block: int = 3, sink_delta: int = -1,
                     theta: float = 10000.0, *, scale: float,
                     attn_ws: Optional[AttnWorkspace] = None) -> None:
    """stages: list of dicts, one per stage in order, with keys rings (a KVRingStack's
    .states array), q_raw, k_raw, v_raw, attn_out (lists of per-layer tensors), vel
    (tensor like x, or None when x is None), dt, and optionally sink_k_new,
    sink_v_new (lists, block 1).  scale: the softmax scale."""
    torch = _torch()
    n_layers = len(stages[0]["rings"])
    r0 = stages[0]["rings"][0]
    dtype = _step_dtype(r0)
    blk = (r0.block_tokens, r0.heads, r0.head_dim)
    snk = (r0.sink_tokens, r0.heads, r0.head_dim)
    if x is not None and x.dtype != torch.float32:
        raise ValueError("x must be float32")
    _check_table(rope_table, Hl, Wl, r0.head_dim)
    for t, name, shp in ((q_rot_ws, "q_rot_ws", blk), (k_rot_ws, "k_rot_ws", blk),
                         (sink_k_rot_ws, "sink_k_rot_ws", snk)):
        _check_tensor(t, name, shp, dtype)
    for i, g in enumerate(stages):  # every shape and dtype first, then the pointers
        for key in ("q_raw", "k_raw", "v_raw", "attn_out"):
            _check_list(g[key], f"stages[{i}].{key}", blk, dtype, n_layers)
        for key in ("sink_k_new", "sink_v_new"):
            if g.get(key) is not None:
                _check_list(g[key], f"stages[{i}].{key}", snk, dtype, n_layers)
    arr = (la_stage * len(stages))()
    keep = []  # pointer arrays must outlive the call
    for i, g in enumerate(stages):
        if len(g["rings"]) != n_layers:
            raise ValueError("every stage needs the same number of layers")
        if _step_dtype(g["rings"][0]) != dtype:
            raise ValueError("every stage needs rings of the same dtype")
        st = arr[i]
        st.rings = ctypes.cast(g["rings"], ctypes.POINTER(la_kvring))
        for key in ("q_raw", "k_raw", "v_raw", "attn_out"):
            a = _ptr_array(g[key], f"stages[{i}].{key}", blk, dtype, n_layers)
            keep.append(a)
            setattr(st, key, ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)))
        for key in ("sink_k_new", "sink_v_new"):
            if g.get(key) is not None:
                a = _ptr_array(g[key], f"stages[{i}].{key}", snk, dtype, n_layers)
                keep.append(a)
                setattr(st, key, ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)))
        if x is not None:
            v = g.get("vel")
            if v is None or v.numel() != x.numel() or v.dtype != torch.float32:
                raise ValueError(f"stages[{i}].vel must be float32 like x")
            st.vel = _ptr(v, f"stages[{i}].vel").value
        st.dt = float(g["dt"])
    n_lat = 0 if x is None else x.numel()
    ws_p, ws_n = _ws(attn_ws)
    _check(_load().la_denoise_chain(
        arr, len(stages), n_layers, block_id, _ptr(q_rot_ws, "q_rot_ws", blk, dtype),
        _ptr(k_rot_ws, "k_rot_ws", blk, dtype), _ptr(sink_k_rot_ws, "sink_k_rot_ws", snk, dtype),
        _ptr(rope_table, "rope_table"), Hl, Wl, frames_per_block, sink_delta, theta, scale,
        ws_p, ws_n, _ptr(x, "x"), n_lat, _stream()), "la_denoise_chain")


# ---------------------------------------------------------------- one layer's cache
class KVRing:
    """One layer's ring + sink: device buffers from torch, index state in la_kvring."""

    def __init__(self, W: int, block_tokens: int, sink_tokens: int, heads: int, head_dim: int,
                 dtype, noise_level: float, device="cuda", staged: bool = False):
        """dtype: torch.bfloat16, torch.float32, or torch.uint8 for e4m3 slots (the
        sink of an e4m3 ring is bf16).  staged: W + 1 slots (la_kvring_init_staged)."""
        torch = _torch()
        codes = {torch.bfloat16: LA_BF16, torch.float32: LA_F32, torch.uint8: LA_FP8_E4M3}
        if dtype not in codes:
            raise TypeError(f"unsupported ring dtype {dtype} (bfloat16, float32, or uint8 "
                            "for e4m3 slots)")
        code = codes[dtype]
        sink_dtype = torch.bfloat16 if code == LA_FP8_E4M3 else dtype
        ns = W + 1 if staged else W
        self.k_slots = torch.empty((ns, block_tokens, heads, head_dim), dtype=dtype, device=device)
        self.v_slots = torch.empty_like(self.k_slots)
        self.sink_k_raw = torch.empty((sink_tokens, heads, head_dim), dtype=sink_dtype,
                                      device=device)
        self.sink_v = torch.empty_like(self.sink_k_raw)
        self.state = la_kvring()
        init = la_kvring_init_staged if staged else la_kvring_init
        init(self.state, self.k_slots, self.v_slots, self.sink_k_raw, self.sink_v, W,
             block_tokens, sink_tokens, heads, head_dim, code, noise_level)

    @property
    def count(self) -> int:
        return la_kvring_count(self.state)

    def slot_ids(self):
        return [int(self.state.slot_block[s]) for s in range(self.state.nslots)]


class KVRingStack:
    """Per-layer rings for a whole stage, with the la_kvring structs contiguous so that
    la_denoise_step can take them as one array."""

    def __init__(self, n_layers: int, W: int, block_tokens: int, sink_tokens: int, heads: int,
                 head_dim: int, dtype, noise_level: float, device="cuda", staged: bool = False):
        """staged: W + 1 slots per ring (la_kvring_init_staged; la_denoise_step then
        writes each layer's rotated K straight into its next slot)."""
        torch = _torch()
        codes = {torch.bfloat16: LA_BF16, torch.float32: LA_F32, torch.uint8: LA_FP8_E4M3}
        if dtype not in codes:
            raise TypeError(f"unsupported ring dtype {dtype} (bfloat16, float32, or uint8 "
                            "for e4m3 slots)")
        code = codes[dtype]
        sink_dtype = torch.bfloat16 if code == LA_FP8_E4M3 else dtype
        ns = W + 1 if staged else W
        self.k_slots = torch.empty((n_layers, ns, block_tokens, heads, head_dim), dtype=dtype,
                                   device=device)
        self.v_slots = torch.empty_like(self.k_slots)
        self.sink_k_raw = torch.empty((n_layers, sink_tokens, heads, head_dim), dtype=sink_dtype,
                                      device=device)
        self.sink_v = torch.empty_like(self.sink_k_raw)
        self.states = (la_kvring * n_layers)()
        init = la_kvring_init_staged if staged else la_kvring_init
        for l in range(n_layers):
            init(self.states[l], self.k_slots[l], self.v_slots[l], self.sink_k_raw[l],
                 self.sink_v[l], W, block_tokens, sink_tokens, heads, head_dim, code, noise_level)

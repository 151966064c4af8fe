"""Plain, slow float64 CPU oracle for the streaming denoise step (TEST INFRASTRUCTURE).

This package is test infrastructure only.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The library's product path never calls it, and it shares no code
with the HIP kernels or their host library: the only common code is
``seeded_inputs`` (random draws and rounding to storage types).

Each function follows a passage of the Live Avatar pages (cited by page title
and section) or, where the pages leave a step open, the plainest reading that
the rest supports.  Every step reaches a result with a plain definition
(rotation, softmax attention, a FIFO window, one affine update), so the
oracle *is* that definition written out in float64 numpy with no blocking,
fusion or reordering.

FP8 (``fp8.py``): e4m3 encoding (nearest, ties to even, saturating at 448)
and the attention of decoded tensors; the pages name FP8 quantisation without
its format, so the OCP E4M3 format is the reading taken.

Pinned by the ``-m "not gpu"`` tests against library routines, closed forms,
invariants and brute force (see tests/test_oracle_*.py).  Parity unpinned:
fidelity to the real trained model's choices (RoPE theta and band split, the
sink offset, the replacement sink's K/V, the timestep grid), which the pages
do not print.
"""

from .rope import band_split, band_frequencies, rope3d, token_positions
from .attention import attention, attention_lse
from .cache import Ring, Sink, RingStateError
from .flow import euler_step, linear_path_point, uniform_grid
from .stream import StreamOracle, block_f0, SINK_DELTA, SINK_FIXED_POSITION
from .fp8 import E4M3_MAX, attention_fp8, dequantize, e4m3_decode, e4m3_encode, quantize

__all__ = [
    "band_split", "band_frequencies", "rope3d", "token_positions",
    "attention", "attention_lse",
    "Ring", "Sink", "RingStateError",
    "euler_step", "linear_path_point", "uniform_grid",
    "StreamOracle", "block_f0", "SINK_DELTA", "SINK_FIXED_POSITION",
    "E4M3_MAX", "attention_fp8", "dequantize", "e4m3_decode", "e4m3_encode", "quantize",
]

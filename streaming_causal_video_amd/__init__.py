"""MI355X-native hot path of a streaming timestep-forcing video denoise step.

The product is the C-ABI shared library ``liblahip.so`` (HIP kernels for
gfx950, declared in ``include/la.h``); ``_lib`` is its thin ctypes binding.
Build it with ``python -m streaming_causal_video_amd.build``.
"""

from ._lib import (AttnWorkspace, la_attn_workspace_bytes, la_block_attn_fwd_noalloc, la_denoise_step_fp8, EXPORTED, KVRing, KVRingStack, la_denoise_chain, la_denoise_step, la_stage, la_quantize_fp8, la_block_attn_fwd_fp8, la_fp8_q_factor_pow2, LA_FP8_E4M3, LA_STEP_ATTEND_ONLY, LAError, LA_BF16, LA_F32, la_block_attn_fwd, la_fm_euler_step,
                   la_kvcache_append_evict, la_kvring, la_kvring_advance, la_kvring_count,
                   la_kvring_init, la_kvring_init_staged, la_kvring_next_slot, la_rope3d_rolling,
                   la_rope_table_bytes, la_rope_table_fill,
                   la_sink_replace, la_version, lib)

__all__ = [
    "AttnWorkspace", "la_attn_workspace_bytes", "la_block_attn_fwd_noalloc", "la_denoise_step_fp8", "EXPORTED", "KVRing", "KVRingStack", "la_denoise_chain", "la_denoise_step", "la_stage", "la_quantize_fp8", "la_block_attn_fwd_fp8", "la_fp8_q_factor_pow2", "LA_FP8_E4M3", "LA_STEP_ATTEND_ONLY", "LAError", "LA_BF16", "LA_F32", "la_block_attn_fwd", "la_fm_euler_step",
    "la_kvcache_append_evict", "la_kvring", "la_kvring_advance", "la_kvring_count",
    "la_kvring_init", "la_kvring_init_staged", "la_kvring_next_slot", "la_rope3d_rolling",
    "la_rope_table_bytes", "la_rope_table_fill",
    "la_sink_replace", "la_version", "lib",
]

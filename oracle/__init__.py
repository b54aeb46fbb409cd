"""Plain fp64 CPU oracle for the streaming-video-DiT attention core.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code with the HIP library and
imports nothing from it.

What it computes, each function citing the passage it follows:

  * ``bf16``          exact bf16 <-> fp64 conversion (round to nearest even).
  * ``qknorm_rope3d`` per-(token, head) RMS normalisation of q and k followed
                      by the 3D (t, h, w) rotary embedding, one bf16 rounding
                      at the end ("QK-norm+3D RoPE" fused op,
                      Joy-face_change_optimized README, table of changed
                      files).
  * ``kv_quant``      symmetric int8 K/V cache with one fp32 scale per
                      (token, head) (same README, section 1, int8 K/V bullet).
  * ``attention``     softmax attention of the chunk's queries over the
                      concatenated K/V segments, restricted to the kept
                      (q-block, k-block) tiles of a block mask (FlashVSR
                      deployment notes, Block-Sparse-Attention section: a
                      dense mask must reproduce ordinary SDPA).
  * ``attention_merge`` combination of attention results over disjoint key
                      sets by the log-sum-exp identity (the shard merge of
                      Ulysses / Ring context parallelism, which the Wave
                      Forcing summary compares against).
  * ``norms``         RMSNorm and LayerNorm + modulate over the hidden
                      dimension (the other fused kernels the same README
                      lists, table of changed files).
  * ``window``        window-major token order of windowed sparse attention
                      and its locality mask (FlashVSR deployment notes,
                      spatial tiling section: 8 x 8-token attention blocks,
                      local_range in blocks).

Readings of points the pages leave open are stated in each function.
Parity pinning: every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py``. One part is only partly pinned: the rotary
pairing and axis layout (interleaved adjacent pairs; axis blocks t, h, w in
that order) is a reading the pages do not state. The tests pin the rotary
math against an independent library routine and invariants, but which
layout the original kernel used is parity unpinned.
"""
from .bf16 import bf16_to_f64, f64_to_bf16
from .qknorm_rope3d import rms_norm, rope3d_angles, apply_rope, qknorm_rope3d
from .kv_quant import kv_quant_int8, kv_dequant
from .attention import key_block_index, attention, segment_values, attention_merge
from .window import window_order, window_coords, local_window_mask
from .norms import rmsnorm, layernorm_modulate

__all__ = [
    "bf16_to_f64", "f64_to_bf16",
    "rms_norm", "rope3d_angles", "apply_rope", "qknorm_rope3d",
    "kv_quant_int8", "kv_dequant",
    "key_block_index", "attention", "segment_values", "attention_merge",
    "window_order", "window_coords", "local_window_mask",
    "rmsnorm", "layernorm_modulate",
]

"""MI355X-native prefill attention core: QK RMSNorm -> NeoX RoPE -> causal GQA attention.

The compute lives in ``libpfa.so`` (hand-written HIP kernels for gfx950 behind a
C ABI, declared in ``include/pfa.h``).  :mod:`.ops` is the thin Python binding:
argument marshalling for torch tensors, nothing else.  The library is loaded on
first use; if it has not been built every op raises.
"""
from .ops import (ENTRY_CHUNK, ENTRY_CHUNK_PREP, ENTRY_CHUNK_TILED, ENTRY_PREFILL, ENTRY_PREP,
                  ENTRY_Q8, ENTRY_Q8_PREP, PRECISION_BF16, PRECISION_BF16X3, PRECISION_F16,
                  PRECISION_F32,
                  PfaError, UNIT_FIELDS, attn_plan, attn_units, chunk_workspace_bytes,
                  gqa_attn_q8, gqa_chunk_attn, gqa_prefill_attn, gqa_prefill_attn_noalloc,
                  kv_tiles_bytes, lib, noalloc_scratch_bytes, q8_workspace_bytes, qk_prep_attn,
                  qk_prep_attn_q8, qk_prep_chunk_attn, qk_prep_chunk_attn_tiled, qknorm_rope,
                  quantize_rows, version, workspace_bytes)

__all__ = ["qknorm_rope", "gqa_prefill_attn", "qk_prep_attn", "workspace_bytes",
           "gqa_prefill_attn_noalloc", "noalloc_scratch_bytes",
           "gqa_chunk_attn", "qk_prep_chunk_attn", "chunk_workspace_bytes",
           "qk_prep_chunk_attn_tiled", "kv_tiles_bytes",
           "quantize_rows", "gqa_attn_q8", "qk_prep_attn_q8", "q8_workspace_bytes",
           "attn_plan", "attn_units", "UNIT_FIELDS", "ENTRY_PREFILL", "ENTRY_PREP",
           "ENTRY_CHUNK", "ENTRY_CHUNK_PREP", "ENTRY_Q8", "ENTRY_Q8_PREP", "ENTRY_CHUNK_TILED",
           "lib", "version",
           "PfaError",
           "PRECISION_F32", "PRECISION_BF16", "PRECISION_BF16X3", "PRECISION_F16"]

"""Kimi Delta Attention (KDA) for AMD MI355X (gfx950).

The computation lives in ``libkda.so`` (hand-written HIP kernels behind the C
ABI of ``include/kda.h``); this package is its thin Python binding.  The
library is loaded on first use and every call raises if it is missing.
"""
from ._native import (CHUNK, HEAD_DIM, KDA_BF16, KDA_F32, KdaError, LIB_PATH, chunk_prefill,
                      chunk_prefill_checkpoint, chunk_prefill_checkpoints, chunk_prefill_gated,
                      decode_replay, decode_replay_gated, decode_step, decode_step_gated, load, plan_num_segments, prefill_workspace_size,
                      segment_scan, segment_transition, status_string, version)

__all__ = [
    "CHUNK", "HEAD_DIM", "KDA_BF16", "KDA_F32", "KdaError", "LIB_PATH", "chunk_prefill", "chunk_prefill_checkpoint",
    "chunk_prefill_checkpoints", "chunk_prefill_gated",
    "decode_replay", "decode_replay_gated", "decode_step", "decode_step_gated", "load", "plan_num_segments", "prefill_workspace_size", "segment_scan", "segment_transition",
    "status_string", "version",
]

"""CPU oracle (numpy fp64) for Light Forcing HSA + CAG.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the product path. Shares no code with the HIP library.
"""
from .hsa import (attn_flops, block_budget, block_geometry, block_mask, block_scores, block_tokens,
                  cag_alpha, cag_schedule, uniform_schedule, dense_attn, frame_scores, hsa, pool_blocks, pool_frames,
                  select_blocks, select_blocks_1d, select_frames, sparse_attn)

__all__ = ["attn_flops", "block_budget", "block_geometry", "block_mask", "block_scores", "block_tokens",
           "cag_alpha", "cag_schedule", "uniform_schedule", "dense_attn", "frame_scores", "hsa", "pool_blocks", "pool_frames",
           "select_blocks", "select_blocks_1d", "select_frames", "sparse_attn"]

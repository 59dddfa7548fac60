"""CPU oracle for the Veda tile-sparse self-attention forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package entry point's
smoke check and by the benchmark's CPU-baseline leg, never by the library.
"""

from .veda_oracle import *  # noqa: F401,F403
from .veda_oracle import (bf16_round, bf16_bits_to_float, float_to_bf16_bits, tile_counts,
                          num_tiles, tiled_position, tile_permute, tile_unpermute, trippool,
                          fp32_dot_rows, project, tile_scores, avgpool_scores, topk_row_bruteforce, topk,
                          bitmask, sparse_attention, dense_attention, head_forward,
                          teacher_tile_max, mask_overlap, tile_recall, tile_search_errors,
                          distill_kl, distill_grad, distill_loss, adam_step)

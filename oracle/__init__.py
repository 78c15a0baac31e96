"""CPU oracle for Loki decode-step sparse attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
"""

from .loki_oracle import *  # noqa: F401,F403
from .loki_oracle import (append, attend, attend_indices, bf16_to_f64, calibrate,  # noqa: F401
                          decode, decode_head, dense_attention, dense_decode, f64_to_bf16,
                          from_f64, kv_head, low_rank_scores, rope_embed, rotate, select_topk,
                          softmax,
                          to_f64, topk_gap, valid_in_band)

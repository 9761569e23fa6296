"""CPU oracle of the verify-and-speculate step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it.  The product path (the HIP library and its Python binding) never
does, and shares no code with it.
"""

from .specverify_oracle import (BF16, DRAW_ABS_BAND, F32, FLAG_BAND, BatchResult, ProbVerdict,
                                RowError, SequenceResult,
                                acceptance_probability, argmax_first,
                                cache_hit, cache_hits_batch,
                                first_rejection, forked_topf,
                                forked_topf_batch, inverse_cdf,
                                residual_distribution, residual_weights,
                                sample_at_position, sample_rows, sample_temp,
                                softmax_rows,
                                softmax_temp, verify_batch, verify_from_probs,
                                verify_greedy, verify_sequence, widen)

__all__ = ["BF16", "DRAW_ABS_BAND", "F32", "FLAG_BAND", "BatchResult", "ProbVerdict",
           "RowError", "SequenceResult", "acceptance_probability",
           "argmax_first", "cache_hit", "cache_hits_batch",
           "first_rejection", "forked_topf",
           "forked_topf_batch", "inverse_cdf", "residual_distribution",
           "residual_weights", "sample_at_position", "sample_rows",
           "sample_temp", "softmax_rows",
           "softmax_temp", "verify_batch", "verify_from_probs",
           "verify_greedy", "verify_sequence", "widen"]

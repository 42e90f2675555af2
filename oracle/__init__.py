"""CPU oracle for the speculative-sampling verify step (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  See ``oracle.verify`` for the definitions it follows."""
from .verify import (decode_row, process, inverse_cdf, verify_sequence,  # noqa: F401
                     verify_batch, BatchResult, SeqResult,
                     gumbel_scores, gumbel_target_token, gumbel_verify_sequence,
                     gumbel_verify_batch, GumbelResult, GumbelBatchResult, sample_row, sample_batch,
                     SampleBatchResult)
from . import analytics  # noqa: F401
from . import kseq  # noqa: F401

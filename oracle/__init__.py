"""fp64 CPU oracle of the decode sampling tail (test infrastructure only;
see tail_oracle.py)."""
from .tail_oracle import (BF16, DETERMINISTIC_DRAW, F16, F32, bf16_bits_to_f64,  # noqa: F401
                          bf16_round, logits, mirror, pad_mask, rmsnorm, rmsnorm_page, sample,
                          sample_row, tail, topk, widen)

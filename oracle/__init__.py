"""CPU oracle (test infrastructure only; see nq_oracle's header)."""
from .nq_oracle import (  # noqa: F401
    LRB, WORD_BITS, bits_per_weight_ref, linear_factored_ref, linear_ref, n_words,
    pack_ref, reconstruct_expected_f32, reconstruct_ref, rel_err, sampled_linear_ref,
    sign_bits_ref, sign_product_ref, storage_bits_ref, unpack_ref,
)

"""PBS-Attn CPU oracle -- test infrastructure only (see ``pbs_oracle``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package; the product path never does."""
from .pbs_oracle import *  # noqa: F401,F403
from .pbs_oracle import (KEEP, COVERAGE, bf16_to_f64, descending_order, key_scores,  # noqa: F401
                         segment_permutation, apply_permutation, inverse_permutation,
                         pooled_blocks, block_probabilities, keep_count, select_blocks,
                         visible_keys, attention, dense_causal, prefill, default_scale)

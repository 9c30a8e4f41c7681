"""Plain CPU oracle for the DeepSeek-style MoE feed-forward layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the test suite (``tests/``), the
``smoke()`` entry of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports
nothing from ``mixture_experts_ffn_route_amd``; every input arrives as an
array argument.

Everything is written for clarity, not speed: float64 NumPy, one token and
one expert at a time, following the pages' definitions step by step.

Sources (pages, by title and section):
  * "DeepSeek-V3.2-Exp - Routing weights", excerpts "gate-forward" and
    "moe-forward" -- the learned gate and the per-expert dispatch loop.
  * "From One Giant FFN to 384 Tiny Experts", Ch.1 (SwiGLU definition),
    Ch.4 (DeepSeekMoE gating formula), Ch.6 (selection-only bias),
    Ch.11.2 (Sqrt(Softplus) affinity), 11.4 (SwiGLU clamp), 11.6 (FP4 experts).
  * "DeepSeek V4.1 - Add shared" -- the V4.1 MoE class: routed + shared,
    output cast back to the input dtype.
  * "How was DeepSeek V4's tid2eid derived?" -- eq. (1)/(2), the greedy
    least-loaded construction of the hash-routing table, its randomised
    multi-start variant, and the 2-gram hash of "An extreme case".
  * "From One Giant FFN to 384 Tiny Experts", Ch.6 / 7.1 and the MaxText pull
    request "Load balancing changes for Deepseek v4" -- the bias update and
    the expert-load statistics (balance.py).

Parity status of each function is stated in its module docstring; every
function here is pinned by a test in ``tests/test_oracle_*.py`` against
closed forms, brute force, library routines or hand-derived fixtures.
"""

from .route import (affinity, selection_keys, learned_gate, hash_gate, ngram_hash_gate,
                    smallest_primes_above)
from .balance import load_stats, bias_update
from .mx import (mxfp8_quantize, mxfp8_decode, layer_forward_mx, E4M3_VALUES,
                 fp4_to_fp8_blocks, fp8_blocks_decode)
from .permute import permute
from .ffn import swiglu_expert, layer_forward, dense_map_forward, fp4_decode, E2M1_VALUES
from .tid2eid import (tid2eid_greedy, tid2eid_greedy_order, tid2eid_multistart, tid2eid_objective,
                      tid2eid_bruteforce, balance_violations)

__all__ = [
    "affinity", "selection_keys", "learned_gate", "hash_gate", "ngram_hash_gate",
    "smallest_primes_above", "load_stats", "bias_update",
    "mxfp8_quantize", "mxfp8_decode", "layer_forward_mx", "E4M3_VALUES",
    "fp4_to_fp8_blocks", "fp8_blocks_decode",
    "permute",
    "swiglu_expert", "layer_forward", "dense_map_forward", "fp4_decode", "E2M1_VALUES",
    "tid2eid_greedy", "tid2eid_greedy_order", "tid2eid_multistart", "tid2eid_objective",
    "tid2eid_bruteforce", "balance_violations",
]

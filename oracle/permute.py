"""Oracle: permutation of (token, slot) pairs by expert.

Test infrastructure only (see the package docstring).

Follows the dispatch loop of "DeepSeek-V3.2-Exp - Routing weights", excerpt
"moe-forward" (and the same loop in "DeepSeek V4.1 - Add shared"): the
per-expert counts are a bincount of the flattened indices, and the rows an
expert receives are ``torch.where(indices == e)``, i.e. its (token, slot)
pairs in row-major order of the [T, k] index table.  Packing those row lists
one expert after another gives the permuted order:

  counts[e]   = number of pairs routed to e
  offsets[e]  = exclusive prefix sum of counts (offsets[E] = T*k)
  sorted_tok[r], sorted_slot[r] = the pair at permuted row r
  inverse[t, j] = the permuted row of pair (t, j)

Pins: tests/test_oracle_permute.py (counts sum, exclusive scan, ascending
tokens per segment, sorted[inverse] = identity, agreement with a stable
library argsort, hand-worked fixture tests/golden/permute_small.json).
"""

import numpy as np


def permute(indices, n_experts):
    indices = np.asarray(indices, dtype=np.int64)
    T, k = indices.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    sorted_tok = []
    sorted_slot = []
    for e in range(n_experts):
        rows, slots = np.nonzero(indices == e)   # row-major order, as torch.where
        counts[e] = rows.shape[0]
        sorted_tok.extend(rows.tolist())
        sorted_slot.extend(slots.tolist())
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_tok = np.asarray(sorted_tok, dtype=np.int64)
    sorted_slot = np.asarray(sorted_slot, dtype=np.int64)
    inverse = np.full((T, k), -1, dtype=np.int64)
    for r in range(sorted_tok.shape[0]):
        inverse[sorted_tok[r], sorted_slot[r]] = r
    return counts, offsets, sorted_tok, sorted_slot, inverse

"""Planner oracle: route ids grouped by expert and padded to ``block_m``.

Test infrastructure (see the package docstring).

Definition followed
-------------------
[prime-flash] "Shapes" section: ``sorted_token_ids`` holds the flattened pair
ids ``token * top_k + route``, grouped by expert and padded to ``block_m`` with
-1; ``expert_ids`` names the expert of each ``block_m`` block and
``num_tokens_post_padded`` is the padded row count ("API" section lists the
three outputs of ``moe_align``).  [hpc-ops RFC] "Design" section: the planner
builds the expert histogram, the prefix sums and the row-to-token mapping.

Readings where the pages are silent
-----------------------------------
* experts are laid out in ascending expert id;
* inside one expert, pair ids appear in ascending order (a stable grouping);
* an expert with no routes gets no block;
* a pair whose expert id lies outside [0, E) is not placed anywhere;
* every slot past ``num_tokens_post_padded`` up to the capacity is -1 in
  ``sorted_token_ids``, and every block past the last used one is -1 in
  ``expert_ids``.
"""

import numpy as np


def capacity(num_routes, num_experts, block_m):
    """Upper bound on padded rows and on blocks for any routing.

    Each non-empty expert adds fewer than ``block_m`` padding rows and at most
    min(E, R) experts are non-empty, so R + min(E, R) * (block_m - 1) rows
    always suffice.
    """
    rows = num_routes + min(num_experts, num_routes) * (block_m - 1)
    blocks = -(-rows // block_m)
    return rows, blocks


def align_ref(topk_ids, num_experts, block_m):
    """Return (sorted_token_ids, expert_ids, num_tokens_post_padded).

    ``topk_ids`` is an int array of shape (T, top_k).  The outputs are int32
    arrays of the capacities given by :func:`capacity` and a Python int.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape if ids.ndim == 2 else (0, 1)
    flat = ids.reshape(-1)
    R = flat.size
    rows_cap, blocks_cap = capacity(R, num_experts, block_m)
    sorted_ids = np.full(rows_cap, -1, dtype=np.int32)
    expert_ids = np.full(blocks_cap, -1, dtype=np.int32)
    pos = 0
    for e in range(num_experts):
        members = np.nonzero(flat == e)[0]      # ascending pair ids
        c = members.size
        if c == 0:
            continue
        nblk = -(-c // block_m)
        sorted_ids[pos:pos + c] = members.astype(np.int32)
        expert_ids[pos // block_m: pos // block_m + nblk] = e
        pos += nblk * block_m
    return sorted_ids, expert_ids, pos

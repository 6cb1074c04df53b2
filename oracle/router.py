"""Router oracle: softmax over the experts, top-k, renormalization.

Test infrastructure (see the package docstring).

Definition followed
-------------------
[prime-flash] "Usage" section: the routing comes from the model's gate and
arrives at the planner as ``topk_ids`` (T, top_k) int32, with ``topk_weights``
(T, top_k) the weights of the weighted sum.  [hpc-ops RFC] "Results so far"
section: the weights are the normalized routing weights.  [hpc-ops RFC]
"Design" section: the planner is its own launch because the histogram and the
prefix sums are grid-wide dependencies; the fused router-planner computes this
routing and then that planner in one launch.

Readings where the pages are silent
-----------------------------------
* gate scores are the softmax of the router logits over all E experts;
* the k selected experts are those with the k largest logits (equivalently
  the largest probabilities), listed in descending logit order; equal logits
  go to the lower expert id first;
* the weights are the selected probabilities divided by their sum
  ("normalized"), so the selected weights of a token sum to one;
* logits may be -inf (an expert masked for this token); a masked expert is
  only selected when fewer than k experts are unmasked.

Everything is fp64 from the fp32 logits (exact widening).
"""

import numpy as np


def _select(L, top_k):
    """Indices of the top_k largest entries of each row of L, descending, ties
    to the lower index: a stable sort of -L keeps equal keys in index order."""
    return np.argsort(-L, axis=1, kind="stable")[:, :top_k]


def _softmax(L):
    """Row softmax over all experts, in fp64 (max subtracted first)."""
    m = np.max(L, axis=1, keepdims=True)
    e = np.exp(L - m)
    return e / np.sum(e, axis=1, keepdims=True)


def _weights(L, ids):
    """Selected probabilities renormalized to sum to one per token."""
    p = np.take_along_axis(_softmax(L), ids, axis=1)
    return p / np.sum(p, axis=1, keepdims=True)


def route_ref(logits, top_k):
    """(T, E) float32 router logits -> topk_ids (T, top_k) int32 and
    topk_weights (T, top_k) float64."""
    L = np.asarray(logits, dtype=np.float64)
    if L.ndim != 2:
        raise ValueError("logits must be (T, E)")
    T, E = L.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must lie in [1, E]")
    if T == 0:
        return np.zeros((0, top_k), np.int32), np.zeros((0, top_k), np.float64)
    ids = _select(L, top_k)
    return ids.astype(np.int32), _weights(L, ids)

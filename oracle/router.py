"""Top-k expert selection with softmax route weights: the step that produces the layer's
expert_ids and route_weights from router logits.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages do not define the gate function (how logits are made from x); the layer takes
expert_ids [T, k] and BF16 route_weights [T, k] as given ("Cake SiTU backend", intro).
Readings (the plainest the workload description supports, where the route weights are a
softmax over the k picks of N(0,1) logits):
  * a token's experts are its k largest logits, in decreasing order; equal logits are
    taken in increasing expert id (a stable order, so the result is unique);
  * its weights are the softmax over those k logits only (renormalized), computed here
    in float64 and rounded once to BF16 (round to nearest even).
"""

import numpy as np

from .codecs import f64_to_bf16_bits


def topk_softmax(logits, k):
    """logits float32 [T, E] -> (expert_ids int32 [T, k], route_weights BF16 bits [T, k])."""
    z = np.asarray(logits, dtype=np.float32)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("k out of range")
    # stable descending order: sort by (-logit, expert id)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -z.astype(np.float64)), axis=1)
    ids = order[:, :k]
    sel = np.take_along_axis(z, ids, axis=1).astype(np.float64)
    p = np.exp(sel - sel[:, :1])
    w = p / p.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), f64_to_bf16_bits(w)

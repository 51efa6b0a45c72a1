"""Expert routing: key-value sort, row maps, per-expert histogram, int8 token movement.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows "torch_npu.npu_moe_init_routing_v2" (Ascend API reference), section 计算公式:
  step 1  sortedExpertIdx, sortedRowIdx = keyValueSort(expertIdx, rowIdx)
  step 2  gather map (row_idx_type 0, the default): expandedRowIdx[sortedRowIdx[i]] = i
  step 3  per-expert histogram of sortedExpertIdx; mode 0 (the default) is the prefix
          sum (前缀和)
  step 4  dynamic quant without a smoothing scale:
          scale = row_max(|x|) / 127,  q = round(x / scale)
  step 5  with the full expert range active, tokens move by the scatter index:
          expandedX[i] = quant[sortedRowIdx[i] // K]

rowIdx is the flat index f = t*K + j of expert_idx[t, j].  Readings (R9-R12):
  * keyValueSort is stable: equal experts keep increasing f (the workload asks for a
    stable sort; the page does not say).
  * the histogram output is the inclusive prefix sum with one entry per expert.
  * round is round-half-to-even on the fp32 quotient; |q| is clipped to 127.
  * an all-zero row has scale 0 and all-zero codes.
"""

import numpy as np


def route(expert_ids, num_experts):
    """Steps 1-3 for expert_ids [T, K] int32 with values in [0, E).

    Returns dict with int32 arrays:
      sorted_ids [T*K], sorted_row_idx [T*K], expanded_row_idx [T*K],
      counts [E], cumsum [E] (inclusive).
    """
    ids = np.asarray(expert_ids)
    flat = ids.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("expert id out of range")
    order = np.argsort(flat, kind="stable")               # keyValueSort(expertIdx, rowIdx)
    sorted_ids = flat[order]
    expanded = np.empty_like(order)
    expanded[order] = np.arange(order.size)                # gather map
    counts = np.bincount(flat, minlength=num_experts)
    return {
        "sorted_ids": sorted_ids.astype(np.int32),
        "sorted_row_idx": order.astype(np.int32),
        "expanded_row_idx": expanded.astype(np.int32),
        "counts": counts.astype(np.int32),
        "cumsum": np.cumsum(counts).astype(np.int32),
    }


def int8_row_quant(x_f32):
    """Step 4, dynamic mode without a smoothing scale, per token row (fp32 arithmetic)."""
    x = np.asarray(x_f32, dtype=np.float32)
    row_max = np.max(np.abs(x), axis=1)
    scale = (row_max / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (x / scale[:, None]).astype(np.float32)
    quot = np.where(scale[:, None] == 0, np.float32(0.0), quot)
    q = np.clip(np.rint(quot), -127, 127).astype(np.int8)
    return q, scale


def route_int8(x_f32, expert_ids, num_experts):
    """Steps 1-5 with dynamic int8 quant: the routing outputs of ``route`` plus
    expanded_x int8 [T*K, H] and expanded_scale float32 [T*K]."""
    r = route(expert_ids, num_experts)
    K = np.asarray(expert_ids).shape[1]
    q, scale = int8_row_quant(x_f32)
    src_token = r["sorted_row_idx"].astype(np.int64) // K
    r["expanded_x"] = q[src_token]
    r["expanded_scale"] = scale[src_token]
    r["row_scale"] = scale
    return r

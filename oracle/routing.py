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

rowIdx is the flat index f = t*K + j of expert_idx[t, j].  Readings where the page is silent:
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


# ---------------------------------------------------------------------------------------
# The options of the same page beyond the defaults (section 计算公式 steps 1-6 and the
# parameter list): scatter index type, count and key_value histograms, an active expert
# range with availableIdxNum, static int8 quant, drop/pad to an expert capacity, and
# active_num.  Readings where the page is silent or loose:
#   * ids outside the active range [start, end) take no part: the sort of step 1 keeps
#     the in-range ids in their sorted order and they occupy positions 0..avail-1.
#   * row_idx_type 1: entries past availableIdxNum are left unwritten by the page; here
#     they are -1 (a defined value is one of the allowed contents).
#   * histogram mode 1 is the per-expert count and mode 2 the (expert id, count) pairs of
#     the in-range experts with a nonzero count, in increasing expert id, at the head of
#     an [expert_num, 2] array whose other rows are 0.  The histogram counts every
#     in-range id, also ids that drop/pad or active_num later drop.
#   * static quant: q = round_half_even(fp32(fp32(x * scale) + offset)), saturated to
#     [-128, 127]; scale and offset are fp32 scalars.
#   * drop/pad: expert e's routed rows in sorted order take slots e*C + r, r < C; the
#     gather index of a dropped row is -1; unfilled slots are 0 (scale 0).  Only the
#     gather index type is defined with drop/pad (the scatter index of [E*C] slots has no
#     place in an [N*K] output); active_num does not apply to it.
#   * active_num > 0 keeps expanded rows 0..active_num-1; the index outputs and the
#     histogram are unaffected.  0 and -1 mean no limit.
#   * the non-quant mode with a per-row scale [N] moves that scale like the dynamic
#     quant scale.
# ---------------------------------------------------------------------------------------


def int8_static_quant(x_f32, scale, offset):
    """Step 4, static mode: round(x*scale + offset) per element, in fp32, to int8."""
    x = np.asarray(x_f32, dtype=np.float32)
    y = (x * np.float32(scale)).astype(np.float32)
    y = (y + np.float32(offset)).astype(np.float32)
    return np.clip(np.rint(y), -128, 127).astype(np.int8)


def route_v2(x_f32, expert_ids, expert_num, *, expert_range=None, row_idx_type=0,
             expert_tokens_num_type=0, quant_mode=-1, scale=None, offset=None, drop_pad_mode=0,
             expert_capacity=-1, active_num=-1):
    """All six steps for x [N, H] (fp32 values of the BF16 input; None when only the
    index outputs are wanted) and expert_ids [N, K].

    Returns a dict: sorted_row_idx (the in-range part of the stable sort, [avail]),
    expanded_row_idx [N*K], expert_tokens (mode 0/1: [end-start]; mode 2: [expert_num, 2]),
    available_idx_num, and with x: expanded_x (rows valid: "valid_rows") and, for the
    dynamic mode or a per-row scale in mode -1, expanded_scale.
    """
    ids = np.asarray(expert_ids)
    N, K = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    n = flat.size
    if flat.size and (flat.min() < 0 or flat.max() >= expert_num):
        raise ValueError("expert id out of range")
    start, end = (0, expert_num) if expert_range is None else expert_range
    if not 0 <= start < end <= expert_num:
        raise ValueError("bad active expert range")
    if drop_pad_mode and (start, end) != (0, expert_num):
        raise ValueError("drop/pad needs the full expert range")
    if drop_pad_mode and row_idx_type != 0:
        raise ValueError("drop/pad is defined with the gather index only")
    E_act = end - start

    # step 1: stable key-value sort; the in-range ids stay at the head in sorted order
    order = np.argsort(flat, kind="stable")
    keep = (flat[order] >= start) & (flat[order] < end)
    sorted_row_idx = order[keep]
    avail = sorted_row_idx.size                                # step 6
    sorted_ids = flat[sorted_row_idx]

    # step 3: histogram of the in-range sorted experts
    counts = np.bincount(sorted_ids - start, minlength=E_act).astype(np.int64)
    if expert_tokens_num_type == 0:
        expert_tokens = np.cumsum(counts)
    elif expert_tokens_num_type == 1:
        expert_tokens = counts.copy()
    elif expert_tokens_num_type == 2:
        expert_tokens = np.zeros((expert_num, 2), np.int64)
        nz = np.nonzero(counts)[0]
        expert_tokens[:nz.size, 0] = nz + start
        expert_tokens[:nz.size, 1] = counts[nz]
    else:
        raise ValueError("bad expert_tokens_num_type")

    # rank of each sorted position inside its expert (for drop/pad)
    first = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.arange(avail) - first[sorted_ids - start]

    # step 2: the position map
    gather = np.full(n, -1, np.int64)
    if drop_pad_mode:
        C = expert_capacity
        if C < 1:
            raise ValueError("drop/pad needs expert_capacity >= 1")
        kept = rank < C
        gather[sorted_row_idx[kept]] = (sorted_ids[kept] - start) * C + rank[kept]
    else:
        gather[sorted_row_idx] = np.arange(avail)
    if row_idx_type == 1:
        expanded_row_idx = np.full(n, -1, np.int64)
        expanded_row_idx[:avail] = sorted_row_idx
    else:
        expanded_row_idx = gather

    out = {
        "sorted_row_idx": sorted_row_idx.astype(np.int32),
        "expanded_row_idx": expanded_row_idx.astype(np.int32),
        "expert_tokens": expert_tokens.astype(np.int32),
        "available_idx_num": int(avail),
    }
    if x_f32 is None:
        return out

    # step 4: quantization of the token rows
    x = np.asarray(x_f32, dtype=np.float32)
    H = x.shape[1]
    row_scale = None
    if quant_mode == -1:
        src = x
        if scale is not None:
            row_scale = np.asarray(scale, np.float32).reshape(N)
    elif quant_mode == 0:
        src = int8_static_quant(x, scale, offset)
    elif quant_mode == 1:
        src, row_scale = int8_row_quant(x)
    else:
        raise ValueError("bad quant_mode")

    # step 5: token movement
    if drop_pad_mode:
        rows = end * expert_capacity
        valid_rows = rows
    else:
        rows = n if active_num <= 0 else min(active_num, n)
        valid_rows = min(avail, rows)
    ex = np.zeros((rows, H), src.dtype)
    es = np.zeros(rows, np.float32) if row_scale is not None else None
    if (start, end) == (0, expert_num) and not drop_pad_mode:
        for i in range(valid_rows):                        # by the scatter index
            ex[i] = src[sorted_row_idx[i] // K]
            if es is not None:
                es[i] = row_scale[sorted_row_idx[i] // K]
    else:
        for f in range(n):                                 # by the gather index
            d = gather[f]
            if 0 <= d < rows:
                ex[d] = src[f // K]
                if es is not None:
                    es[d] = row_scale[f // K]
    if drop_pad_mode:
        ex = ex.reshape(end, expert_capacity, H)
        if es is not None:
            es = es.reshape(end, expert_capacity)
    out["expanded_x"] = ex
    out["valid_rows"] = int(valid_rows)
    if es is not None:
        out["expanded_scale"] = es
    return out

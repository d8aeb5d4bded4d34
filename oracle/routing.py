"""Oracle routing: expert histogram, offsets and the stable permutation.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The grouped-experts design (nxmr.cn article on MCoreQAD, section 二.4) runs one
grouped GEMM over all experts, so the routed copies of the tokens are gathered
expert by expert.  The order inside an expert is not stated; the reading taken
is the stable one: experts ascending, and inside an expert the flat routing
index t*k + j ascending (a stable counting sort).
"""
from __future__ import annotations

import numpy as np


def route(topk_ids, num_experts: int):
    """Return counts[E], offsets[E+1], src_of[R] and row_of[R].

    topk_ids is [T, k] int (distinct ids per token, each in [0, E)).
    Routed row r holds flat index src_of[r] = t*k + j; row_of is its inverse.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).ravel()
    counts = np.bincount(ids, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    src_of = np.argsort(ids, kind="stable")
    row_of = np.empty_like(src_of)
    row_of[src_of] = np.arange(ids.size)
    return counts, offsets, src_of, row_of


def route_bruteforce(topk_ids, num_experts: int):
    """The same permutation by an explicit double loop (tiny inputs only)."""
    ids = [int(v) for v in np.asarray(topk_ids).ravel()]
    src_of = []
    for e in range(num_experts):
        for i, v in enumerate(ids):
            if v == e:
                src_of.append(i)
    return np.array(src_of, dtype=np.int64)

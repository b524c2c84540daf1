"""Sparse draft attention and dense block verification over a paged KV cache.

[news], Interpretation: drafting and verification share the policy's
weights; drafting attends to a small selected set of historical KV entries,
verification recomputes the proposed block against the complete history.
[listing], Abstract: sparse attention proposes tokens, full attention
verifies them. [explainer], mechanism paragraph: k sparse draft steps, then
one full-notebook pass checks all k at once.

Conventions (readings, since the pages give no positions or head maps):
* the paged cache is [pages][Hkv][page][D]; position j of sequence b lives
  at page block_table[b][j // page], slot j % page;
* GQA: query head h reads KV head h // G, G = Hq / Hkv;
* a round starts with L committed positions; the pending token sits at
  position L; draft step j (1..k) queries position L + j - 1 and reads the
  selected positions plus this round's positions [L, L + j);
* verification reads the block of k + 1 positions [L, L + k] (pending token
  and k drafts) at the tail of a cache of seq_len = L + k + 1 positions;
  row i (0..k) reads positions [0, L + i] (causal inside the block);
* scores for the next selection: for each KV head and position j, the sum
  over the G query heads of the group and over the k + 1 block rows of the
  row's normalised attention probability at j (rows that cannot see j add
  nothing). The sum (not a max) over heads and rows is the reading adopted.
* logits are scale * q.k with scale passed in by the caller (1/sqrt(D)).

* page scores (the selector variant that keeps whole pages): the score of
  page p of a KV head is the sum of the position scores of its positions
  [16p, 16p + 16) that lie in the cache (the last page may be partial).

Pins: explicit-loop brute force on tiny inputs; torch's fp64 scaled dot
product attention (with the causal block mask and repeated KV heads) as a
library special case; budget = L equals dense decode; k = 0 verification
equals single-token decode; a single kept position returns that V row;
constant keys return the mean of V; scores of each KV head sum to G(k+1);
page scores: an explicit loop over positions, the same G(k+1) total, unit 1
returns the position scores, and a page's score moves only with the
probabilities of its own positions.
"""

import numpy as np


def _wide(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:  # bfloat16 bit patterns
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gather(pages: np.ndarray, bt_row: np.ndarray, kv_head: int, positions) -> np.ndarray:
    """Rows [n][D] (float64) of the given positions of one sequence's KV head."""
    positions = np.asarray(positions, dtype=np.int64)
    P = pages.shape[2]
    phys = np.asarray(bt_row, dtype=np.int64)[positions // P]
    return _wide(pages[phys, kv_head, positions % P, :])


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(scale * K q) V and its log-sum-exp (natural log).

    An empty set (a degenerate budget of zero with no draft positions yet)
    gives a zero output and -inf (reading: the sum over no positions).
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf, np.zeros(0)
    logits = float(scale) * (K @ q)
    m = logits.max()
    e = np.exp(logits - m)
    z = e.sum()
    return (e / z) @ V, m + np.log(z), e / z


def sparse_decode(q, k_pages, v_pages, bt_row, idx, n_sel: int, L: int, cur: int, scale: float):
    """One draft step for one sequence.

    q: [Hq][D]; idx: [Hkv][>= n_sel] kept positions per KV head; the step
    reads idx[kv][:n_sel] and [L, cur). Returns (o [Hq][D], lse [Hq]).
    """
    q = _wide(np.asarray(q))
    Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    o = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    for h in range(Hq):
        kv = h // G
        pos = np.concatenate([np.asarray(idx[kv][:n_sel], dtype=np.int64), np.arange(L, cur, dtype=np.int64)])
        K = gather(k_pages, bt_row, kv, pos)
        V = gather(v_pages, bt_row, kv, pos)
        o[h], lse[h], _ = attend(q[h], K, V, scale)
    return o, lse


def dense_decode(q, k_pages, v_pages, bt_row, length: int, scale: float):
    """Single-query attention of q [Hq][D] over positions [0, length)."""
    q = _wide(np.asarray(q))
    Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    o = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    pos = np.arange(length)
    for h in range(Hq):
        K = gather(k_pages, bt_row, h // G, pos)
        V = gather(v_pages, bt_row, h // G, pos)
        o[h], lse[h], _ = attend(q[h], K, V, scale)
    return o, lse


def verify(q, k_pages, v_pages, bt_row, seq_len: int, k: int, scale: float):
    """Dense block verification for one sequence.

    q: [k+1][Hq][D]. Returns (o [k+1][Hq][D], lse [k+1][Hq],
    scores [Hkv][seq_len]).
    """
    q = _wide(np.asarray(q))
    _, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    o = np.zeros((k + 1, Hq, D))
    lse = np.zeros((k + 1, Hq))
    scores = np.zeros((Hkv, seq_len))
    for kv in range(Hkv):
        K = gather(k_pages, bt_row, kv, np.arange(seq_len))
        V = gather(v_pages, bt_row, kv, np.arange(seq_len))
        for i in range(k + 1):
            last = seq_len - (k + 1) + i  # row i reads [0, last]
            for h in range(kv * G, (kv + 1) * G):
                o[i, h], lse[i, h], p = attend(q[i, h], K[:last + 1], V[:last + 1], scale)
                scores[kv, :last + 1] += p
    return o, lse, scores


def page_scores(scores: np.ndarray, seq_len: int, unit: int = 16) -> np.ndarray:
    """[Hkv][ceil(seq_len / unit)] float64: the sum of each page's position scores (positions
    at and past seq_len are not in the cache and add nothing)."""
    scores = np.asarray(scores, dtype=np.float64)
    npg = -(-int(seq_len) // unit)
    out = np.zeros((scores.shape[0], npg))
    for p in range(npg):
        out[:, p] = scores[:, p * unit:min((p + 1) * unit, int(seq_len))].sum(axis=1)
    return out

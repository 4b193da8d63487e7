"""fp64 CPU oracle for retained-mass block-sparse self-attention (LoSA).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code, tables or constants with it; the two meet only
in the seeded input generator (``synthetic``), which holds no arithmetic of
the method.

Every function restates a definition from page 1, "LoSA: Near-Lossless
Sparse Attention for Training-Free Video Diffusion Acceleration":

* Motivation Summary -- dense attention A = softmax(Q K^T / sqrt(d)) per head;
  block attention mass M(i, j) = sum over the query block's rows and the key
  block's columns of A; Recall and Coverage of a block pattern.
* Methodology Summary, one-time pattern construction -- per head and query
  block, sort key blocks by decreasing mass and keep the shortest prefix whose
  cumulative mass reaches theta times the block's total mass.
* Methodology Summary, sparse attention with a frozen pattern -- softmax over
  the retained keys only (discarded keys leave the denominator), no forced
  local or diagonal blocks.

Readings taken where the page is silent (each is also listed with the design
notes of the repository):

* Tokens at or beyond N (padding up to a whole number of blocks) are not
  tokens: they are masked out of every softmax and mass, rows beyond N are not
  queries (their output is 0) and are excluded from the block average.
* M is stored as the row mean (the page's M divided by the number of valid
  rows of the query block), so each row of blocks sums to 1.  The selection is
  unchanged because the target scales with the total.
* Selection target: p times the *computed* row total.  Ties in mass: lower
  block index first.  p = 1 keeps every block.  Non-finite or negative masses
  count as 0.
* Cumulative-sum arithmetic ("contract rule"): the page's cumulative sum is
  evaluated exactly in integers so any summation order gives one answer:
  e = exponent of the row maximum (max = f * 2^e, f in [1/2, 1)),
  q_j = ceil(m_j * 2^(51 - e)) (an exact power-of-two scaling, so every
  positive mass is at least one unit), P = floor(p * 2^32 + 1/2),
  T = ceil(P * sum_j q_j / 2^32), s = the least prefix length whose integer
  sum is >= T.  A plain fp64 argsort + cumsum is kept beside it as a cross-check.
* Output lists are CSR with ascending block indices per row.  The work order
  ranks each head's n_q rows by kept-block count (descending, ties by row
  index), cuts the ranks into groups of 32, and runs the groups longest
  first (by their first row's count; ties by head, then group).
* Pooled proxy masses (the coarse estimates the page contrasts with exact
  masses -- Motivation Summary, SVG2 / SpargeAttn; the pages give no formula):
  P[i, j] = |B_j| exp(qbar_i . kbar_j * scale) / sum_j' |B_j'| exp(qbar_i .
  kbar_j' * scale), with qbar, kbar the means over the valid tokens of each
  block and |B_j| the valid keys of key block j (each pooled key stands for
  its block's keys).  Rows sum to 1, like M, so the same selector applies.
* Masses within a candidate set (the reduced search of the GSRS card: later
  top-p searches restricted to an earlier candidate set, with exact
  attention weights computed inside the attention pass; the card gives no
  formula): for a row's listed blocks L, the softmax runs over the valid
  tokens of L only (the frozen-pattern attention's softmax) and
  M_L(i, j) = mean over valid rows of block i of the sum over block j's
  tokens of it, for j in L; 0 for blocks outside L.  A row with a non-empty
  list sums to 1; with every block listed M_L = M.
* Online block thresholding (the Sol-Attn page decides which blocks matter
  while its online softmax runs, each block's proxy score tested against a
  threshold, so budgets vary by row; the page gives no rule): visiting a
  row's key blocks in index order, as an online-softmax pass does, block j
  is kept when its mass (exact or proxy, sanitised as for top-p) is at least
  theta times the largest mass seen so far, block j included -- in scores,
  within ln(1/theta) of the running maximum.  theta in (0, 1]; the
  comparison is made in fp64 on the fp32 masses.
* On-the-fly block thresholding inside the attention pass (the Sol-Attn
  page: blocks are chosen while the online softmax runs, by comparing each
  block's proxy score with a threshold, without materialising the proxy map;
  the page gives no formula): the proxy of key block j for query block i is
  the pooled score sbar_ij = scale * qbar_i . kbar_j (block means over valid
  tokens), weighted by the block's valid keys, a_j = sbar_ij + ln|B_j|; in
  index order (the online pass's order) block j is kept when
  a_j >= ln(theta) + max(a_0 .. a_j).  Since the pooled proxy mass is
  P_j = exp(a_j) / Z, this is the online-thresholding rule above applied to P,
  decided in the log domain so that Z (and the map P) is never needed.  The
  decision is taken in fp64 with the interface's fp32 softmax scale widened
  exactly; softmax over the kept blocks' valid tokens follows.  The page's
  correction for the skipped blocks is not part of this reading.
* Drift-triggered refresh (the HASTE page's temporal mask reuse: mask
  prediction is skipped while queries and keys have drifted little since it
  was last made; the page gives no measure): per (batch, head), the drift of
  Q is ||Q - Q_ref||_F / ||Q_ref||_F over the valid tokens, Q_ref being the
  queries of the step at which the head's lists were built, likewise for K
  (0/0 = 0, x/0 = inf for x > 0, NaN stays NaN); a head's lists are rebuilt
  when either drift exceeds a threshold tau, and kept otherwise.

Row numbering: row r = (b * H + h) * n_q + i for batch b, head h, query block i.
Inputs are fp64 arrays [B, H, N_alloc, d] holding the exact values the GPU sees.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "softmax_scale",
    "attention_probs",
    "dense_attention",
    "block_mass",
    "block_mass_rows",
    "pooled_mass",
    "restricted_mass",
    "restricted_mass_rows",
    "sanitize_masses",
    "select_contract",
    "select_contract_row",
    "select_float_row",
    "select_float",
    "p_fixed",
    "sparse_attention",
    "sparse_attention_rows",
    "budget_order",
    "ORDER_GROUP",
    "select_threshold_row",
    "select_threshold",
    "pooled_scores",
    "threshold_inpass_lists",
    "qk_drift",
    "refresh_heads",
    "merge_lists",
    "recall",
    "coverage",
    "row_id",
    "row_split",
]


def softmax_scale(head_dim: int, scale: Optional[float] = None) -> float:
    """1/sqrt(d) (Motivation Summary: A = softmax(Q K^T / sqrt(d)))."""
    return 1.0 / math.sqrt(head_dim) if scale is None or scale <= 0 else float(scale)


def row_id(b: int, h: int, i: int, heads: int, n_q: int) -> int:
    return (b * heads + h) * n_q + i


def row_split(r: int, heads: int, n_q: int) -> Tuple[int, int, int]:
    bh, i = divmod(r, n_q)
    b, h = divmod(bh, heads)
    return b, h, i


def attention_probs(q_rows: np.ndarray, k_keys: np.ndarray, scale: float) -> np.ndarray:
    """Row softmax of q_rows k_keys^T * scale over the given keys (fp64)."""
    s = (q_rows @ k_keys.T) * scale
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_valid: int,
                    scale: Optional[float] = None, chunk: int = 1024) -> np.ndarray:
    """Dense self-attention O = softmax(Q K^T * scale) V over the N valid keys.

    Motivation Summary (definition of A).  Rows >= N are written as 0.
    """
    B, H, Na, d = q.shape
    sc = softmax_scale(d, scale)
    out = np.zeros((B, H, Na, v.shape[-1]), np.float64)
    for b in range(B):
        for h in range(H):
            kk, vv = k[b, h, :n_valid], v[b, h, :n_valid]
            for r0 in range(0, n_valid, chunk):
                r1 = min(n_valid, r0 + chunk)
                a = attention_probs(q[b, h, r0:r1], kk, sc)
                out[b, h, r0:r1] = a @ vv
    return out


def _block_sums(a: np.ndarray, n_valid: int, C: int, n_k: int) -> np.ndarray:
    """Sum columns of a [rows, n_valid] into key blocks of C tokens -> [rows, n_k]."""
    rows = a.shape[0]
    pad = np.zeros((rows, n_k * C), np.float64)
    pad[:, :n_valid] = a
    return pad.reshape(rows, n_k, C).sum(axis=2)


def block_mass_rows(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int,
                    rows: Iterable[Tuple[int, int, int]], scale: Optional[float] = None) -> np.ndarray:
    """Block masses for the listed (b, h, i) query blocks only -> [len(rows), n_k].

    M(i, j) = mean over valid query rows q of block i of the sum over valid
    keys k of block j of A(q, k)  (Motivation Summary, block attention mass;
    row-mean form).
    """
    d = q.shape[-1]
    sc = softmax_scale(d, scale)
    n_k = -(-n_valid // C)
    rows = list(rows)
    out = np.zeros((len(rows), n_k), np.float64)
    for t, (b, h, i) in enumerate(rows):
        r0, r1 = i * R, min((i + 1) * R, n_valid)
        if r1 <= r0:
            continue
        a = attention_probs(q[b, h, r0:r1], k[b, h, :n_valid], sc)
        out[t] = _block_sums(a, n_valid, C, n_k).mean(axis=0)
    return out


def block_mass(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int,
               scale: Optional[float] = None) -> np.ndarray:
    """All block masses M [B, H, n_q, n_k] (fp64, row-mean form)."""
    B, H = q.shape[:2]
    n_q = -(-n_valid // R)
    n_k = -(-n_valid // C)
    M = np.zeros((B, H, n_q, n_k), np.float64)
    for b in range(B):
        for h in range(H):
            M[b, h] = block_mass_rows(q, k, n_valid, R, C, [(b, h, i) for i in range(n_q)], scale)
    return M


def pooled_mass(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int,
                scale: Optional[float] = None) -> np.ndarray:
    """Pooled proxy masses P [B, H, n_q, n_k] (fp64): a block-level softmax of
    the block-mean query against the block-mean keys, each pooled key weighted
    by its block's number of valid keys.  Coarse estimate of M (Motivation
    Summary: coarse mass estimates); equals M exactly when the scores are
    constant within every (query block, key block) pair."""
    B, H, _, d = q.shape
    sc = softmax_scale(d, scale)
    n_q = -(-n_valid // R)
    n_k = -(-n_valid // C)
    qbar = np.stack([q[:, :, i * R:min((i + 1) * R, n_valid)].mean(axis=2) for i in range(n_q)], axis=2)
    kbar = np.stack([k[:, :, j * C:min((j + 1) * C, n_valid)].mean(axis=2) for j in range(n_k)], axis=2)
    size = np.array([min(C, n_valid - j * C) for j in range(n_k)], np.float64)
    s = np.einsum("bhid,bhjd->bhij", qbar, kbar) * sc
    s -= s.max(axis=3, keepdims=True)
    w = size * np.exp(s)
    return w / w.sum(axis=3, keepdims=True)


def sanitize_masses(m: np.ndarray) -> np.ndarray:
    """Non-finite, negative and negative-zero masses count as 0 (fp32 in, fp32 out)."""
    m = np.asarray(m, dtype=np.float32)
    good = np.isfinite(m) & (m > 0)
    return np.where(good, m, np.float32(0.0)).astype(np.float32)


def p_fixed(p: float) -> int:
    """p as a 32-bit fixed-point fraction: floor(p * 2^32 + 1/2), p in (0, 1]."""
    if not (0.0 < p <= 1.0):
        raise ValueError("p must lie in (0, 1]")
    return int(math.floor(p * 4294967296.0 + 0.5))


def _fixed_point_units(m32: np.ndarray) -> np.ndarray:
    """q_j = ceil(m_j * 2^(51 - e)), e = frexp exponent of the row maximum.

    m_j is fp32, so m_j * 2^(51-e) is exact in fp64 (a power-of-two scaling of
    a 24-bit significand) and below 2^51; ceil and the cast to uint64 are exact.
    """
    mx = float(m32.max()) if m32.size else 0.0
    if mx <= 0.0:
        return np.zeros(m32.shape, np.uint64)
    e = math.frexp(mx)[1]
    scaled = np.ldexp(m32.astype(np.float64), 51 - e)
    return np.ceil(scaled).astype(np.uint64)


def select_contract_row(m32: np.ndarray, p: float) -> Tuple[np.ndarray, int]:
    """One row of the one-time pattern construction under the contract rule.

    Methodology Summary (one-time pattern construction): pi sorts key blocks
    by decreasing mass (ties: lower index first), s = min m such that the
    prefix mass reaches the target, omega = pi(1..s).  Returns the kept block
    indices in ascending order and s.
    """
    m32 = sanitize_masses(m32)
    n_k = m32.shape[0]
    pi = np.argsort(-m32, kind="stable")  # mass descending, stable -> index ascending on ties
    P = p_fixed(p)
    if P == 1 << 32:
        s = n_k
    else:
        units = _fixed_point_units(m32)
        prefix = np.cumsum(units[pi], dtype=np.uint64)
        total = int(prefix[-1])
        T = -((-P * total) >> 32)  # ceil(P * total / 2^32), exact Python integers
        s = int(np.argmax(prefix >= np.uint64(T))) + 1
    return np.sort(pi[:s]), s


def select_float_row(m: np.ndarray, p: float) -> Tuple[np.ndarray, int, float]:
    """Plain fp64 cross-check: argsort + cumsum, target p * row total.

    Returns (kept ascending, s, margin) where margin = cum(s) - target is how
    far the deciding prefix lies from the target.
    """
    m64 = sanitize_masses(m).astype(np.float64)
    n_k = m64.shape[0]
    pi = np.argsort(-m64, kind="stable")
    if p >= 1.0:
        return np.sort(pi), n_k, math.inf
    cum = np.cumsum(m64[pi])
    target = p * cum[-1]
    s = int(np.argmax(cum >= target)) + 1
    margin = min(abs(cum[s - 1] - target), abs(cum[s - 2] - target) if s >= 2 else math.inf)
    return np.sort(pi[:s]), s, margin


def select_contract(M32: np.ndarray, p) -> Tuple[np.ndarray, np.ndarray]:
    """CSR lists for every row of M32 [B, H, n_q, n_k] (fp32).

    ``p`` is a scalar or one value per head.  Returns (row_ptr int64 [rows+1],
    col_idx int32 [nnz]).
    """
    B, H, n_q, n_k = M32.shape
    p_h = np.broadcast_to(np.asarray(p, dtype=np.float64), (H,))
    counts = np.zeros(B * H * n_q, np.int64)
    cols: List[np.ndarray] = []
    for b in range(B):
        for h in range(H):
            for i in range(n_q):
                kept, s = select_contract_row(M32[b, h, i], float(p_h[h]))
                counts[row_id(b, h, i, H, n_q)] = s
                cols.append(kept.astype(np.int32))
    row_ptr = np.zeros(B * H * n_q + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    return row_ptr, col_idx


def select_threshold_row(m32: np.ndarray, theta: float) -> np.ndarray:
    """Kept blocks of one row under online thresholding (module header): in
    index order, keep j when m_j >= theta * max(m_0 .. m_j)."""
    m = sanitize_masses(m32).astype(np.float64)
    kept = []
    running = 0.0
    for j in range(m.size):
        running = max(running, float(m[j]))
        if float(m[j]) >= float(theta) * running:
            kept.append(j)
    return np.asarray(kept, np.int64)


def select_threshold(M32: np.ndarray, theta) -> Tuple[np.ndarray, np.ndarray]:
    """CSR lists of online thresholding for every row of M32 [B, H, n_q, n_k];
    ``theta`` is a scalar or one value per head."""
    B, H, n_q, n_k = M32.shape
    t_h = np.broadcast_to(np.asarray(theta, dtype=np.float64), (H,))
    row_ptr = [0]
    cols: List[np.ndarray] = []
    for b in range(B):
        for h in range(H):
            for i in range(n_q):
                kept = select_threshold_row(M32[b, h, i], float(t_h[h]))
                cols.append(kept.astype(np.int32))
                row_ptr.append(row_ptr[-1] + kept.size)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    return np.asarray(row_ptr, np.int64), col_idx


def pooled_scores(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int,
                  scale: Optional[float] = None) -> np.ndarray:
    """sbar[b, h, i, j] = scale * qbar_i . kbar_j (fp64): the mean over the valid
    tokens of query block i against the mean over the valid tokens of key
    block j.  scale defaults to 1/sqrt(d) rounded to fp32 (the interface
    carries the softmax scale as an fp32 number)."""
    B, H, _, d = q.shape
    sc = float(np.float32(softmax_scale(d, scale)))
    n_q = -(-n_valid // R)
    n_k = -(-n_valid // C)
    qbar = np.stack([q[:, :, i * R:min((i + 1) * R, n_valid)].mean(axis=2) for i in range(n_q)], axis=2)
    kbar = np.stack([k[:, :, j * C:min((j + 1) * C, n_valid)].mean(axis=2) for j in range(n_k)], axis=2)
    return np.einsum("bhid,bhjd->bhij", qbar, kbar) * sc


def threshold_inpass_lists(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int, theta,
                           scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray, float]:
    """Kept blocks of on-the-fly block thresholding (module header): per row,
    in index order, a_j = sbar_ij + ln|B_j| and block j is kept when
    a_j >= ln(theta_h) + max(a_0 .. a_j).  ``theta`` is a scalar or one value
    per head, each in (0, 1].  Returns (row_ptr, col_idx ascending, margin).
    With ln(theta) <= 0 a block j > 0 is kept exactly when
    a_j >= ln(theta_h) + max(a_0 .. a_{j-1}); margin is the smallest
    |a_j - ln(theta_h) - max(a_0 .. a_{j-1})| over all rows and blocks j > 0,
    i.e. how far the closest decision lies from a tie (block 0 is always kept)."""
    sbar = pooled_scores(q, k, n_valid, R, C, scale)
    B, H, n_q, n_k = sbar.shape
    t_h = np.broadcast_to(np.asarray(theta, dtype=np.float64), (H,))
    ln_size = np.array([math.log(min(C, n_valid - j * C)) for j in range(n_k)], np.float64)
    row_ptr = [0]
    cols: List[np.ndarray] = []
    margin = math.inf
    for b in range(B):
        for h in range(H):
            ln_t = math.log(float(t_h[h]))
            for i in range(n_q):
                a = sbar[b, h, i] + ln_size
                kept = []
                run = -math.inf
                for j in range(n_k):
                    if j > 0:
                        margin = min(margin, abs(float(a[j]) - (ln_t + run)))
                    run = max(run, float(a[j]))
                    if float(a[j]) >= ln_t + run:
                        kept.append(j)
                cols.append(np.asarray(kept, np.int32))
                row_ptr.append(row_ptr[-1] + len(kept))
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    return np.asarray(row_ptr, np.int64), col_idx, margin


def select_float(M: np.ndarray, p) -> Tuple[np.ndarray, np.ndarray, List[Tuple[int, float]]]:
    """fp64 argsort+cumsum selection of every row; also returns per-row margins."""
    B, H, n_q, n_k = M.shape
    p_h = np.broadcast_to(np.asarray(p, dtype=np.float64), (H,))
    counts = np.zeros(B * H * n_q, np.int64)
    cols, margins = [], []
    for b in range(B):
        for h in range(H):
            for i in range(n_q):
                kept, s, mg = select_float_row(M[b, h, i], float(p_h[h]))
                r = row_id(b, h, i, H, n_q)
                counts[r] = s
                cols.append(kept.astype(np.int32))
                margins.append((r, mg))
    row_ptr = np.zeros(B * H * n_q + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    return row_ptr, np.concatenate(cols), margins


def _kept_tokens(blocks: Sequence[int], C: int, n_valid: int) -> np.ndarray:
    parts = [np.arange(j * C, min((j + 1) * C, n_valid)) for j in blocks]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def sparse_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_valid: int,
                          R: int, C: int, row_ptr: np.ndarray, col_idx: np.ndarray,
                          rows: Iterable[Tuple[int, int, int]],
                          scale: Optional[float] = None) -> List[np.ndarray]:
    """Frozen-pattern sparse attention for the listed (b, h, i) query blocks.

    Methodology Summary (sparse attention with a frozen pattern):
    O(q) = sum over retained keys k of exp(q.k * scale) / (sum over retained
    keys k' of exp(q.k' * scale)) * v_k, the retained keys being the valid
    tokens of the kept blocks of q's query block.  Returns one [rows_i, d]
    array per listed block (valid rows only); an empty list gives zeros.
    """
    B, H, Na, d = q.shape
    sc = softmax_scale(d, scale)
    n_q = -(-n_valid // R)
    out = []
    for (b, h, i) in rows:
        r = row_id(b, h, i, H, n_q)
        blocks = col_idx[int(row_ptr[r]):int(row_ptr[r + 1])]
        r0, r1 = i * R, min((i + 1) * R, n_valid)
        keys = _kept_tokens(blocks, C, n_valid)
        if keys.size == 0 or r1 <= r0:
            out.append(np.zeros((max(r1 - r0, 0), v.shape[-1]), np.float64))
            continue
        # scores against every valid key, the discarded ones set to -inf (they
        # leave the softmax: exp gives exactly 0), then the weights times V
        s = (q[b, h, r0:r1] @ k[b, h, :n_valid].T) * sc
        dropped = np.ones(n_valid, bool)
        dropped[keys] = False
        s[:, dropped] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=1, keepdims=True)
        out.append(a @ v[b, h, :n_valid])
    return out


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_valid: int,
                     R: int, C: int, row_ptr: np.ndarray, col_idx: np.ndarray,
                     scale: Optional[float] = None) -> np.ndarray:
    """Frozen-pattern sparse attention for every row -> O [B, H, N_alloc, d] (0 beyond N)."""
    B, H, Na, d = q.shape
    n_q = -(-n_valid // R)
    O = np.zeros((B, H, Na, v.shape[-1]), np.float64)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(n_q)]
    res = sparse_attention_rows(q, k, v, n_valid, R, C, row_ptr, col_idx, rows, scale)
    for (b, h, i), o in zip(rows, res):
        O[b, h, i * R:i * R + o.shape[0]] = o
    return O


def restricted_mass_rows(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int,
                         row_ptr: np.ndarray, col_idx: np.ndarray, rows: Iterable[Tuple[int, int, int]],
                         scale: Optional[float] = None) -> np.ndarray:
    """Block masses within each listed row's candidate blocks -> [len(rows), n_k].

    GSRS card (reduced search with exact attention weights inside the
    attention pass): the softmax of the frozen-pattern attention, i.e. over
    the valid tokens of the listed blocks only; M_L(i, j) = mean over valid
    rows q of block i of the sum over the valid tokens of block j of it, for
    listed j, and 0 for the rest.
    """
    B, H, Na, d = q.shape
    sc = softmax_scale(d, scale)
    n_q = -(-n_valid // R)
    n_k = -(-n_valid // C)
    rows = list(rows)
    out = np.zeros((len(rows), n_k), np.float64)
    for t, (b, h, i) in enumerate(rows):
        r = row_id(b, h, i, H, n_q)
        blocks = [int(j) for j in col_idx[int(row_ptr[r]):int(row_ptr[r + 1])]]
        r0, r1 = i * R, min((i + 1) * R, n_valid)
        keys = _kept_tokens(blocks, C, n_valid)
        if keys.size == 0 or r1 <= r0:
            continue
        a = attention_probs(q[b, h, r0:r1], k[b, h, keys], sc)  # [rows_i, kept keys]
        owner = keys // C                                         # key block of each kept token
        for j in blocks:
            out[t, j] = a[:, owner == j].sum(axis=1).mean()
    return out


def restricted_mass(q: np.ndarray, k: np.ndarray, n_valid: int, R: int, C: int,
                    row_ptr: np.ndarray, col_idx: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Masses within the candidate lists for every row -> [B, H, n_q, n_k] (fp64)."""
    B, H = q.shape[:2]
    n_q = -(-n_valid // R)
    n_k = -(-n_valid // C)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(n_q)]
    return restricted_mass_rows(q, k, n_valid, R, C, row_ptr, col_idx, rows, scale).reshape(B, H, n_q, n_k)


ORDER_GROUP = 32  # rows per work group in the work order


def budget_order(row_ptr: np.ndarray, n_q: int) -> np.ndarray:
    """Work order.  Within each (batch, head) -- n_q consecutive rows -- rows
    are ranked by kept-block count, descending, ties by row index; the ranks
    are cut into groups of ORDER_GROUP consecutive ranks (the head's last
    group may be shorter); groups run longest first, by the count of their
    first (largest) row, ties by head and then by group; rows within a group
    keep their rank order.

    The pages ask for work ordered by budget because per-head budgets are
    uneven (HASTE page, head-wise adaptive top-p; Sol-Attn page, dynamic but
    imbalanced budgets); a group holds rows of one head, so the workgroups
    that run it side by side share that head's keys and values.
    """
    counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
    rows = np.arange(counts.size, dtype=np.int64)
    head = rows // int(n_q)
    ranked = np.lexsort((rows, -counts, head))          # head-major, count desc, row asc
    rank = np.empty_like(rows)
    rank[ranked] = np.arange(rows.size) - head[ranked] * int(n_q)
    group = rank // ORDER_GROUP
    first = {}
    for r in rows:                                       # each group's first (largest) row
        if rank[r] % ORDER_GROUP == 0:
            first[(int(head[r]), int(group[r]))] = int(counts[r])
    key = np.array([first[(int(head[r]), int(group[r]))] for r in rows], np.int64)
    return np.lexsort((rank, head, -key)).astype(np.int64)


def qk_drift(q: np.ndarray, k: np.ndarray, q_ref: np.ndarray, k_ref: np.ndarray, n_valid: int) -> np.ndarray:
    """Relative Frobenius drift of Q and K per (batch, head) since the reference
    step, over the valid tokens: out[b, h] = (dQ, dK) (HASTE page, temporal
    mask reuse, as read in this module's header)."""
    out = np.zeros(q.shape[:2] + (2,), np.float64)
    for t, (x, xr) in enumerate(((q, q_ref), (k, k_ref))):
        diff = np.asarray(x, np.float64)[:, :, :n_valid] - np.asarray(xr, np.float64)[:, :, :n_valid]
        num = np.sqrt(np.sum(diff * diff, axis=(2, 3)))
        den = np.sqrt(np.sum(np.asarray(xr, np.float64)[:, :, :n_valid] ** 2, axis=(2, 3)))
        for idx in np.ndindex(num.shape):
            n, m = num[idx], den[idx]
            if m > 0:
                out[idx + (t,)] = n / m
            elif m == 0:
                out[idx + (t,)] = math.inf if n > 0 else n  # 0/0 = 0; NaN stays NaN
            else:
                out[idx + (t,)] = m  # NaN
    return out


def refresh_heads(drift: np.ndarray, tau: float) -> np.ndarray:
    """Heads whose lists are rebuilt: either drift exceeds tau (a NaN drift never does)."""
    return np.any(drift > tau, axis=-1)


def merge_lists(rp_a: np.ndarray, ci_a: np.ndarray, rp_b: np.ndarray, ci_b: np.ndarray,
                take_b: np.ndarray, n_q: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row r's list from set b when its head (r // n_q) is refreshed, from set a
    otherwise; CSR in row order."""
    take = np.asarray(take_b).reshape(-1)
    rows = len(rp_a) - 1
    rp, parts = [0], []
    for r in range(rows):
        src_rp, src_ci = (rp_b, ci_b) if take[r // n_q] else (rp_a, ci_a)
        lst = np.asarray(src_ci[int(src_rp[r]):int(src_rp[r + 1])], np.int64)
        parts.append(lst)
        rp.append(rp[-1] + len(lst))
    ci = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return np.asarray(rp, np.int64), ci


def recall(M: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray, n_valid: int, R: int) -> float:
    """Recall(omega) = kept block mass / total block mass (Motivation Summary).

    Uses the page's un-normalised mass, i.e. the row-mean M times the number
    of valid query rows of each block.
    """
    B, H, n_q, n_k = M.shape
    w = np.array([min(R, n_valid - i * R) for i in range(n_q)], np.float64)
    Mw = M * w[None, None, :, None]
    flat = Mw.reshape(B * H * n_q, n_k)
    kept = 0.0
    for r in range(flat.shape[0]):
        kept += flat[r, col_idx[int(row_ptr[r]):int(row_ptr[r + 1])]].sum()
    return float(kept / flat.sum())


def coverage(row_ptr: np.ndarray, batch: int, heads: int, n_q: int, n_k: int) -> float:
    """Coverage(omega) = (1/H) sum_h sum_i |omega_i^h| / (n_q n_k), averaged over batch."""
    nnz = int(np.asarray(row_ptr)[-1])
    return nnz / float(batch * heads * n_q * n_k)

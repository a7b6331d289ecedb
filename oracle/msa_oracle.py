"""CPU oracle for the MiniMax Sparse Attention (MSA) forward pass.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct
definition of what the MSA forward computes, in float64 numpy.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.  The
HIP library never calls it and shares no code with it.

What the method computes (sources: the MSA abstract page "MiniMax 稀疏注意力",
sections 摘要 and 核心贡献; the snilld.dk page "MiniMax lancerer MSA",
section "Hvad er MSA i praksis"; the Hungarian page "MiniMax új eljárása …",
section "Hogyan működik az indexelő és a fő ág?"; the issue write-up
"Substantial numerical differences with Minimax MSA attention vs Minimax's
Reference", sections 原因分析 and 解决步骤):

1. GQA substrate.  G = number of KV heads = number of index-query heads; the
   r = Hq / G query heads h in [g*r, (g+1)*r) use KV head g and share group
   g's block selection (the repeat_interleave fix in 解决步骤).
2. Index branch.  Each group's index-query head is scored against the single
   shared index-key head over the causally visible key tokens; token scores are
   max-pooled over Bk-token blocks (block c = tokens [c*Bk, (c+1)*Bk), counted
   from position 0); a Top-k is taken per query and per group, never pooled
   across index heads (the amax(dim=1) defect described in 原因分析); the
   query's own (local) block is always part of the selection.
3. Main branch.  Exact scaled-dot-product softmax attention of each query head
   over the causally visible tokens of the selected blocks, one softmax over
   their union.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* the index score is the raw dot product q_idx . k_idx (no scale, no
  activation): only two projections are added and softmax preserves order;
* k counts the local block: local block + the best min(k-1, L) of the full
  blocks 0..L-1, where L = floor(t / Bk) and t = q_offset + i;
* only full blocks before the local block are ranked, so the causal mask never
  cuts a ranked block (block c < L ends at (c+1)*Bk - 1 < t);
* ties in block score go to the lower block index;
* a selection row lists the chosen block ids ascending, then -1 padding;
* the main-branch scale is 1/sqrt(d) unless one is given;
* key j is visible to query row i iff j <= q_offset + i.

Index scores are computed in float64; with integer-valued index inputs every
partial sum is an integer far below 2**53, so they are exact.

FP8 caches.  The pages list FP8 among the MSA inference kernel's precisions
(the Hungarian page, section "Elérhetőség") without naming a format; the
reading taken is OCP FP8 E4M3 (e4m3fn) storage for k, v and k_idx with
per-tensor dequantisation scales for k and v.  ``e4m3_to_f64`` decodes such
bytes exactly from the OCP 8-bit floating point specification (OFP8, E4M3
encoding) and ``dequantize_e4m3`` applies a scale; the attention itself is the
same definition applied to the decoded values.

Caches of unequal length.  Serving batches hold caches that differ in length
and grow (the snilld.dk page, sections "POC målinger og miljø" and
"Implementering i produktion").  ``msa_forward_varlen`` applies the same
definition per sequence, with the queries at the last S_q positions of each
cache; a row before the start of its cache (t < 0) sees no key, and the reading
taken is: no selection (-1 only), output 0, lse -inf.  ``page_gather`` reads a
sequence's cache out of a pool of 128-token pages.

KL-alignment teacher (forward only).  Top-k is not differentiable, so a KL loss
trains the index branch to match the main branch; the teacher is the main
distribution over the selected tokens, averaged over the group's heads (the
snilld.dk page, "Træning og stabilisering"; the Hungarian page, "A betanítás és
a kernel-optimalizáció").  Readings taken in ``kl_teacher``: both distributions
are over the tokens the main branch attends to; the index distribution is the
softmax of the raw index scores (times an optional index_scale, 1 by default);
the loss is KL(teacher || index) in natural log.

Backward of the main branch.  The pages name no backward kernel (MSA-PT and
MSA-CPT training needs one).  ``sparse_attention_bwd`` is the gradient of the
main branch with the selection held constant (Top-k is not differentiable):
for each query row, the gradient of exact softmax attention over its token set.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "selection_agreement",
    "sparse_attention_bwd",
    "kl_teacher",
    "page_gather",
    "msa_forward_varlen",
    "e4m3_to_f64",
    "dequantize_e4m3",
    "block_maxima",
    "select_from_maxima",
    "index_select",
    "sparse_attention",
    "msa_forward",
    "dense_causal_attention",
    "token_set",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# FP8 cache values
# ---------------------------------------------------------------------------

def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of each OCP FP8 E4M3 code (uint8).

    Bit layout s eeee mmm, exponent bias 7.  e = 0 encodes the subnormals
    (-1)^s * m * 2^-9; otherwise the value is (-1)^s * (1 + m/8) * 2^(e-7).
    The format has no infinities; the two codes with e = 15 and m = 7 are NaN,
    so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    negative = (c >> 7) == 1
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return np.where(negative, -mag, mag)


def dequantize_e4m3(codes, scale: float = 1.0) -> np.ndarray:
    """scale * value of each E4M3 code, in float64.  The product of a 4-bit
    significand and a float32 scale fits in 53 bits, so it is exact."""
    return e4m3_to_f64(codes) * np.float64(np.float32(scale))


# ---------------------------------------------------------------------------
# Index branch
# ---------------------------------------------------------------------------

def block_maxima(qi: np.ndarray, k_idx_b: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Max-pooled index scores of the full blocks 0..L-1 for one or more query
    vectors of one sequence.

    qi:       [n, D_idx] index-query vectors (one group's head, possibly many rows
              sharing the same local block L)
    k_idx_b:  [S_k, D_idx] the shared index-key head of that sequence
    returns   [n, L] float64, M[:, c] = max_{j in block c} qi . k_idx_b[j]
    """
    qi = _f64(qi)
    if L == 0:
        return np.zeros((qi.shape[0], 0), dtype=np.float64)
    keys = _f64(k_idx_b[: L * block_size])              # [L*Bk, D]
    scores = qi @ keys.T                                 # [n, L*Bk] raw dot products
    return scores.reshape(qi.shape[0], L, block_size).max(axis=2)


def select_from_maxima(M: np.ndarray, L: int, topk: int) -> np.ndarray:
    """Selection rows from block maxima.

    M: [n, L] block maxima of the full blocks before the local block L.
    Returns int32 [n, topk]: the best min(topk-1, L) blocks ordered by
    (score descending, block index ascending), plus L, sorted ascending and
    padded with -1.  No exponential is taken: softmax keeps the order of raw
    scores (the exp-free Top-k of the abstract page, 摘要).
    """
    n = M.shape[0]
    out = np.full((n, topk), -1, dtype=np.int32)
    take = min(topk - 1, L)
    if take > 0:
        # a stable sort of -M keeps equal scores in ascending block order
        order = np.argsort(-M, axis=1, kind="stable")[:, :take]
    else:
        order = np.zeros((n, 0), dtype=np.int64)
    chosen = np.concatenate([order, np.full((n, 1), L, dtype=np.int64)], axis=1)
    chosen.sort(axis=1)
    out[:, : take + 1] = chosen
    return out


def _rows_by_block(q_offset: int, q_len: int, block_size: int, rows: Optional[Iterable[int]]):
    """Group query rows by their local block so rows of one block share a key range."""
    idx = np.arange(q_len) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    L = (q_offset + idx) // block_size
    for Lv in np.unique(L):
        yield int(Lv), idx[L == Lv]


def index_select(q_idx, k_idx, topk: int, q_offset: int = 0, block_size: int = 128,
                 rows: Optional[Sequence[Tuple[int, int]]] = None,
                 chunk: int = 256) -> np.ndarray:
    """Per-group block selection.

    q_idx: [B, S_q, G, D_idx]; k_idx: [B, S_k, D_idx].
    Returns int32 sel [B, G, S_q, topk].  When ``rows`` (pairs (b, i)) is given,
    only those rows are computed and all other entries are left at -2.
    """
    q_idx = np.asarray(q_idx)
    k_idx = np.asarray(k_idx)
    B, S_q, G, _ = q_idx.shape
    if k_idx.shape[1] < q_offset + S_q:
        raise ValueError("kv_len must cover q_offset + q_len")
    sel = np.full((B, G, S_q, topk), -2 if rows is not None else -1, dtype=np.int32)
    per_b = {b: None for b in range(B)} if rows is None else {}
    if rows is not None:
        for b, i in rows:
            per_b.setdefault(int(b), set()).add(int(i))
    for b, rset in per_b.items():
        for L, idx in _rows_by_block(q_offset, S_q, block_size, rset):
            for s0 in range(0, len(idx), chunk):
                part = idx[s0:s0 + chunk]
                for g in range(G):
                    M = block_maxima(q_idx[b, part, g, :], k_idx[b], L, block_size)
                    sel[b, g, part, :] = select_from_maxima(M, L, topk)
    return sel


def selection_agreement(sel, ref) -> dict:
    """How a selection compares with a reference one, in the terms of the check
    the issue write-up runs after its fix (section 验证方法): the number of
    (b, g, i) rows that differ, out of all rows, and the mean number of block ids
    a row shares with its reference row (k of k when nothing diverges).

    sel, ref: int arrays [..., k] of block ids, -1 padded.  A row diverges when
    it is not identical to its reference row (ids, order and padding).  Returns
    {"rows", "diverging", "mean_overlap", "mean_ref_blocks", "k"}.
    """
    a = np.asarray(sel)
    b = np.asarray(ref)
    if a.shape != b.shape:
        raise ValueError(f"shapes differ: {a.shape} vs {b.shape}")
    k = a.shape[-1]
    a2 = a.reshape(-1, k).astype(np.int64)
    b2 = b.reshape(-1, k).astype(np.int64)
    rows = a2.shape[0]
    diverging = int((a2 != b2).any(axis=1).sum())
    # an id of a row counts once if it appears anywhere among the reference row's ids
    shared = ((a2[:, :, None] == b2[:, None, :]) & (b2[:, None, :] >= 0)).any(axis=2) & (a2 >= 0)
    overlap = shared.sum(axis=1)
    return {
        "rows": rows,
        "diverging": diverging,
        "mean_overlap": float(overlap.mean()) if rows else 0.0,
        "mean_ref_blocks": float((b2 >= 0).sum(axis=1).mean()) if rows else 0.0,
        "k": int(k),
    }


# ---------------------------------------------------------------------------
# Main branch
# ---------------------------------------------------------------------------

def token_set(sel_row: np.ndarray, t: int, block_size: int) -> np.ndarray:
    """Key tokens one query at absolute position t attends to: every token of the
    selected blocks that is causally visible (j <= t), in ascending order."""
    toks = []
    for c in sorted(int(c) for c in sel_row if c >= 0):
        lo = c * block_size
        hi = min((c + 1) * block_size, t + 1)
        if hi > lo:
            toks.append(np.arange(lo, hi))
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def _softmax_attend(qh: np.ndarray, kt: np.ndarray, vt: np.ndarray, scale: float):
    """One softmax over the whole token set: qh [r, d], kt/vt [n, d]."""
    s = scale * (qh @ kt.T)                   # [r, n]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ vt) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def sparse_attention(q, k, v, sel, q_offset: int = 0, block_size: int = 128,
                     scale: Optional[float] = None,
                     rows: Optional[Sequence[Tuple[int, int]]] = None):
    """Exact softmax attention over the selected blocks.

    q: [B, S_q, Hq, d]; k, v: [B, G, S_k, d]; sel: int [B, G, S_q, topk].
    Returns (out [B, S_q, Hq, d], lse [B, Hq, S_q]) as float64; rows not listed in
    ``rows`` (when given) are NaN.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    sel = np.asarray(sel)
    B, S_q, Hq, d = q.shape
    G = k.shape[1]
    r = Hq // G
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    out = np.full((B, S_q, Hq, d), np.nan)
    lse = np.full((B, Hq, S_q), np.nan)
    todo = [(b, i) for b in range(B) for i in range(S_q)] if rows is None else rows
    for b, i in todo:
        t = q_offset + i
        for g in range(G):
            T = token_set(sel[b, g, i], t, block_size)
            o, ls = _softmax_attend(_f64(q[b, i, g * r:(g + 1) * r]), _f64(k[b, g, T]),
                                    _f64(v[b, g, T]), scale)
            out[b, i, g * r:(g + 1) * r] = o
            lse[b, g * r:(g + 1) * r, i] = ls
    return out, lse


def msa_forward(q, k, v, q_idx, k_idx, topk: int, q_offset: int = 0, block_size: int = 128,
                scale: Optional[float] = None,
                rows: Optional[Sequence[Tuple[int, int]]] = None):
    """Index branch then main branch.  Returns (out, sel, lse)."""
    sel = index_select(q_idx, k_idx, topk, q_offset, block_size, rows=rows)
    out, lse = sparse_attention(q, k, v, sel, q_offset, block_size, scale, rows=rows)
    return out, sel, lse


def dense_causal_attention(q, k, v, q_offset: int = 0, scale: Optional[float] = None):
    """Plain causal GQA softmax attention (every visible key), float64.

    q: [B, S_q, Hq, d]; k, v: [B, G, S_k, d].  Returns (out, lse)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, S_q, Hq, d = q.shape
    G = k.shape[1]
    r = Hq // G
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((B, S_q, Hq, d))
    lse = np.empty((B, Hq, S_q))
    for b in range(B):
        for i in range(S_q):
            t = q_offset + i
            for g in range(G):
                o, ls = _softmax_attend(_f64(q[b, i, g * r:(g + 1) * r]), _f64(k[b, g, :t + 1]),
                                        _f64(v[b, g, :t + 1]), scale)
                out[b, i, g * r:(g + 1) * r] = o
                lse[b, g * r:(g + 1) * r, i] = ls
    return out, lse


# ---------------------------------------------------------------------------
# Caches of unequal length, paged caches
# ---------------------------------------------------------------------------

def page_gather(pool, pages, n_tokens: int, block_size: int = 128) -> np.ndarray:
    """The first n_tokens tokens of one sequence's cache, read out of a page pool.

    pool:  [P, H, Bk, W] (keys or values) or [P, Bk, W] (index keys)
    pages: the sequence's page ids; logical block c (tokens [c*Bk, (c+1)*Bk)) is
           page pages[c]
    returns [H, n_tokens, W] or [n_tokens, W]
    """
    pool = np.asarray(pool)
    nb = -(-int(n_tokens) // block_size)
    axis = 1 if pool.ndim == 4 else 0
    if nb == 0:
        shape = list(pool.shape[1:])
        shape[axis] = 0
        return np.zeros(shape, dtype=pool.dtype)
    full = np.concatenate([pool[int(pages[c])] for c in range(nb)], axis=axis)
    return full[:, :n_tokens] if axis == 1 else full[:n_tokens]


def msa_forward_varlen(q, k_seqs, v_seqs, q_idx, k_idx_seqs, topk: int, block_size: int = 128,
                       scale: Optional[float] = None):
    """MSA forward over a batch of caches of unequal length.

    q: [B, S_q, Hq, d]; q_idx: [B, S_q, G, D_idx]; for each sequence b,
    k_seqs[b] and v_seqs[b] are [G, n_b, d] and k_idx_seqs[b] is [n_b, D_idx]:
    its n_b cached tokens.  Query row i of sequence b sits at t = n_b - S_q + i.
    Rows with t < 0 precede their cache: selection all -1, output 0, lse -inf.
    Returns (out [B, S_q, Hq, d], sel [B, G, S_q, topk], lse [B, Hq, S_q]).
    """
    q = np.asarray(q)
    q_idx = np.asarray(q_idx)
    B, S_q, Hq, d = q.shape
    G = q_idx.shape[2]
    out = np.zeros((B, S_q, Hq, d))
    sel = np.full((B, G, S_q, topk), -1, dtype=np.int32)
    lse = np.full((B, Hq, S_q), -np.inf)
    for b in range(B):
        n = int(np.asarray(k_idx_seqs[b]).shape[0])
        i0 = max(0, S_q - n)  # the first row at a position >= 0
        if i0 >= S_q:
            continue
        o, sl, ls = msa_forward(q[b:b + 1, i0:], np.asarray(k_seqs[b])[None], np.asarray(v_seqs[b])[None],
                                q_idx[b:b + 1, i0:], np.asarray(k_idx_seqs[b])[None], topk,
                                n - S_q + i0, block_size, scale)
        out[b, i0:] = o[0]
        sel[b, :, i0:] = sl[0]
        lse[b, :, i0:] = ls[0]
    return out, sel, lse


# ---------------------------------------------------------------------------
# KL-alignment teacher (forward)
# ---------------------------------------------------------------------------

def kl_teacher(q, k, q_idx, k_idx, sel, q_offset: int = 0, block_size: int = 128,
               scale: Optional[float] = None, index_scale: float = 1.0,
               rows: Optional[Sequence[Tuple[int, int]]] = None):
    """KL divergence of the index distribution from the group-averaged main one.

    For each (b, g, i) with T the tokens the main branch attends to (token_set):
      teacher  pbar(j) = mean over the r heads h of group g of softmax_T(scale * q_h . k_j)
      index    log qi(j) = log_softmax_T(index_scale * q_idx[b, i, g] . k_idx[b, j])
      kl       = sum_j pbar(j) * (log pbar(j) - log qi(j))     (0 log 0 = 0)
    Returns (kl [B, G, S_q], idx_lse [B, G, S_q]) in float64, idx_lse being the
    log-sum-exp of index_scale * scores over T.  A row with an empty T (before
    the start of its cache) gets kl = 0 and idx_lse = -inf; rows not listed in
    ``rows`` (when given) are NaN.
    """
    q, k, q_idx, k_idx, sel = (np.asarray(a) for a in (q, k, q_idx, k_idx, sel))
    B, S_q, Hq, d = q.shape
    G = k.shape[1]
    r = Hq // G
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    kl = np.full((B, G, S_q), np.nan)
    ilse = np.full((B, G, S_q), np.nan)
    todo = [(b, i) for b in range(B) for i in range(S_q)] if rows is None else rows
    for b, i in todo:
        t = q_offset + i
        for g in range(G):
            T = token_set(sel[b, g, i], t, block_size)
            if T.size == 0:
                kl[b, g, i], ilse[b, g, i] = 0.0, -np.inf
                continue
            s = scale * (_f64(q[b, i, g * r:(g + 1) * r]) @ _f64(k[b, g, T]).T)   # [r, n]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            pbar = p.mean(axis=0)
            si = index_scale * (_f64(k_idx[b, T]) @ _f64(q_idx[b, i, g]))            # [n]
            m = si.max()
            lse = m + math.log(np.exp(si - m).sum())
            plogp = np.where(pbar > 0, pbar * np.log(np.where(pbar > 0, pbar, 1.0)), 0.0)
            kl[b, g, i] = float(plogp.sum() - (pbar * (si - lse)).sum())
            ilse[b, g, i] = lse
    return kl, ilse


# ---------------------------------------------------------------------------
# Backward of the main branch (selection held constant)
# ---------------------------------------------------------------------------

def sparse_attention_bwd(q, k, v, sel, dout, q_offset: int = 0, block_size: int = 128,
                         scale: Optional[float] = None):
    """Gradients of sparse_attention's output with respect to q, k and v.

    For each (b, i, h) with token set T (token_set of its group's selection),
    s_j = scale q.k_j, p = softmax_T(s), o = sum_j p_j v_j.  With the output
    gradient dO = dout[b, i, h]:
      dV[b, g, j] += p_j dO                    (j in T)
      dP_j = dO . v_j,   Dsum = sum_j p_j dP_j  (= dO . o)
      dS_j = p_j (dP_j - Dsum)
      dQ[b, i, h] = scale sum_j dS_j k_j
      dK[b, g, j] += scale dS_j q[b, i, h]
    Returns (dq [B, S_q, Hq, d], dk [B, G, S_k, d], dv [B, G, S_k, d]) in float64.
    """
    q, k, v, sel, dout = (np.asarray(a) for a in (q, k, v, sel, dout))
    B, S_q, Hq, d = q.shape
    G = k.shape[1]
    r = Hq // G
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((B, S_q, Hq, d))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for i in range(S_q):
            t = q_offset + i
            for g in range(G):
                T = token_set(sel[b, g, i], t, block_size)
                if T.size == 0:
                    continue
                qh = _f64(q[b, i, g * r:(g + 1) * r])          # [r, d]
                kt, vt = _f64(k[b, g, T]), _f64(v[b, g, T])      # [n, d]
                do = _f64(dout[b, i, g * r:(g + 1) * r])         # [r, d]
                s = scale * (qh @ kt.T)                          # [r, n]
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = do @ vt.T                                   # [r, n]
                dsum = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - dsum)
                dq[b, i, g * r:(g + 1) * r] = scale * (ds @ kt)
                np.add.at(dk[b, g], T, scale * (ds.T @ qh))
                np.add.at(dv[b, g], T, p.T @ do)
    return dq, dk, dv

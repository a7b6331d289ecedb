"""Helpers of the full-size GPU parity tests.

* ``oracle_selection``: the oracle's selection of every row of a workload,
  computed one sequence at a time from the very values the GPU read (exact
  upcasts; FP8 bytes decoded by the oracle).
* ``check_selection``: the comparison the issue write-up runs after its fix
  (section 验证方法): rows that diverge out of all rows, and the mean overlap of
  each row with its reference row; any diverging row fails.
* ``sparse_kv``: a host copy of one sequence's K or V that holds only the blocks
  a set of selection rows names (the rest stays zero and is never touched, so it
  costs no memory).  The oracle reads exactly those blocks; a block it would
  read outside the set would read zeros and fail the comparison.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import msa_oracle as orc

TOL = 2e-2  # max-abs on bf16 outputs against the fp64 oracle


def seq(t: torch.Tensor, b: int) -> torch.Tensor:
    """Sequence b of a batched tensor as a batch of one (FP8 through its bytes)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)[b:b + 1].view(torch.float8_e4m3fn)
    return t[b:b + 1]


def to_f64(s: synth.Shape, name: str, t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of stored values; FP8 caches decoded and scaled by the oracle."""
    if s.fp8 and name in ("k", "v", "k_idx"):
        scale = {"k": s.k_scale, "v": s.v_scale, "k_idx": 1.0}[name]
        return orc.dequantize_e4m3(synth.codes(t), scale)
    return synth.as_f64(t)


def oracle_selection(s: synth.Shape, q_idx: torch.Tensor, k_idx: torch.Tensor, seqs=None) -> np.ndarray:
    """int32 [len(seqs), G, S_q, k]: the oracle's selection of every row of the given sequences."""
    seqs = list(range(q_idx.shape[0])) if seqs is None else list(seqs)
    ref = np.empty((len(seqs), s.groups, s.q_len, s.topk), dtype=np.int32)
    for j, b in enumerate(seqs):
        qi = to_f64(s, "q_idx", seq(q_idx, b))
        ki = to_f64(s, "k_idx", seq(k_idx, b))
        ref[j] = orc.index_select(qi, ki, s.topk, s.q_offset, s.block_size)[0]
    return ref


def check_selection(name: str, sel_gpu: np.ndarray, ref: np.ndarray) -> dict:
    rep = orc.selection_agreement(sel_gpu, ref)
    print(f"  selection {name}: {rep['diverging']}/{rep['rows']} rows diverge, mean overlap "
          f"{rep['mean_overlap']:.2f} of {rep['mean_ref_blocks']:.2f} blocks (k = {rep['k']})", flush=True)
    if rep["diverging"]:
        bad = np.argwhere((np.asarray(sel_gpu) != np.asarray(ref)).any(axis=-1))
        raise AssertionError(f"{rep['diverging']} selection rows differ, first {bad[:5].tolist()}")
    return rep


def sparse_kv(s: synth.Shape, name: str, t_b: torch.Tensor, blocks_per_group, n_tokens: int) -> np.ndarray:
    """[1, G, n_tokens, d] float64 holding only the listed blocks of each group.

    t_b: the sequence's K or V as stored, [G, n_tokens', d] on the device (n_tokens'
    >= n_tokens); blocks_per_group[g]: block ids of group g to copy."""
    G, _, d = t_b.shape
    out = np.zeros((1, G, n_tokens, d), dtype=np.float64)  # untouched pages are never allocated
    for g in range(G):
        for c in sorted(set(int(c) for c in blocks_per_group[g] if c >= 0)):
            lo, hi = c * s.block_size, min((c + 1) * s.block_size, n_tokens)
            if hi > lo:
                out[0, g, lo:hi] = to_f64(s, name, t_b[g, lo:hi])
    return out


def query_blocks(s: synth.Shape):
    """Row ranges of three whole 128-row query blocks: the first, a middle and the last."""
    nq = -(-s.q_len // s.block_size)
    picks = sorted({0, nq // 2, nq - 1})
    return [(p * s.block_size, min((p + 1) * s.block_size, s.q_len)) for p in picks]


def check_outputs(s: synth.Shape, x: dict, out: torch.Tensor, ref_sel: np.ndarray, seqs, row_ranges) -> float:
    """Max-abs error of the GPU output against the oracle's main branch on the given
    row ranges of the given sequences (selection: the oracle's, already equal to the GPU's)."""
    worst = 0.0
    for j, b in enumerate(seqs):
        for i0, i1 in row_ranges:
            blocks = [ref_sel[j, g, i0:i1].reshape(-1) for g in range(s.groups)]
            kb = sparse_kv(s, "k", seq(x["k"], b)[0], blocks, s.kv_len)
            vb = sparse_kv(s, "v", seq(x["v"], b)[0], blocks, s.kv_len)
            qb = synth.as_f64(x["q"][b:b + 1, i0:i1])
            sub = ref_sel[j:j + 1, :, i0:i1]
            ref_out, _ = orc.sparse_attention(qb, kb, vb, sub, s.q_offset + i0, s.block_size)
            got = out[b:b + 1, i0:i1].float().cpu().numpy()
            worst = max(worst, float(np.abs(got - ref_out).max()))
    return worst

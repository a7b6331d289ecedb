"""Pins for the CPU oracle (no GPU).

Every check here compares the oracle with something other than itself:
hand-worked cases, brute force in pure Python, closed forms, torch's own
scaled-dot-product attention on the CPU in float64, and invariants the MSA
pages state.  A plausible slip in the oracle (a dropped block, an off-by-one in
the causal bound, pooling across index heads, a tie broken the wrong way, a
transposed operand, per-block instead of one softmax) fails at least one test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import msa_oracle as orc
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# hand-worked cases
# ---------------------------------------------------------------------------

def test_hand_index_cases():
    doc = _load("hand_examples.json")
    for case in doc["index_cases"]:
        Bk = case["block_size"]
        kidx = np.array(case["k_idx"], dtype=np.float64)
        for qc in case["queries"]:
            t, k = qc["t"], qc["k"]
            L = t // Bk
            M = orc.block_maxima(np.array([qc["q"]], dtype=np.float64), kidx, L, Bk)
            assert M[0].tolist() == qc["maxima"], qc
            sel = orc.select_from_maxima(M, L, k)
            assert sel[0].tolist() == qc["sel"], qc
            # the same through the full entry point (one sequence, one group, row t)
            q_idx = np.zeros((1, t + 1, 1, kidx.shape[1]))
            q_idx[0, t, 0] = qc["q"]
            full = orc.index_select(q_idx, kidx[None, :], k, 0, Bk, rows=[(0, t)])
            assert full[0, 0, t].tolist() == qc["sel"]


def test_hand_attention_cases():
    doc = _load("hand_examples.json")
    for case in doc["attention_cases"]:
        Bk = case["block_size"]
        for row in case["rows"]:
            keys = np.array(case[row["keys"]])
            S = len(keys)
            t = row["t"]
            q = np.zeros((1, S, 1, 1))
            q[0, t, 0, 0] = 1.0
            k = keys.reshape(1, 1, S, 1)
            v = np.array(case["v"]).reshape(1, 1, S, 1)
            sel = np.full((1, 1, S, len(row["sel"])), -1, dtype=np.int32)
            sel[0, 0, t] = row["sel"]
            out, lse = orc.sparse_attention(q, k, v, sel, 0, Bk, scale=1.0, rows=[(0, t)])
            assert out[0, t, 0, 0] == pytest.approx(row["out"], rel=1e-13, abs=1e-13)
            assert lse[0, 0, t] == pytest.approx(row["lse"], rel=1e-13, abs=1e-13)


# ---------------------------------------------------------------------------
# brute force on tiny inputs (pure Python, no numpy matmul, no sort)
# ---------------------------------------------------------------------------

def _brute_maxima(q, kidx, L, Bk):
    out = []
    for c in range(L):
        best = None
        for j in range(c * Bk, (c + 1) * Bk):
            s = 0
            for e in range(len(q)):
                s += int(q[e]) * int(kidx[j][e])
            best = s if best is None or s > best else best
        out.append(best)
    return out


def _brute_select(M, L, k):
    """The unique (k-1)-subset whose every member precedes every non-member under
    (score desc, index asc), found by enumerating all subsets."""
    take = min(k - 1, L)
    prec = lambda a, b: (M[a] > M[b]) or (M[a] == M[b] and a < b)  # noqa: E731
    winners = []
    for sub in itertools.combinations(range(L), take):
        rest = [c for c in range(L) if c not in sub]
        if all(prec(a, b) for a in sub for b in rest):
            winners.append(sub)
    assert len(winners) == 1
    chosen = sorted(list(winners[0]) + [L])
    return chosen + [-1] * (k - len(chosen))


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.integers(0, 10_000), st.sampled_from([4, 8]), st.integers(1, 4),
       st.integers(1, 3), st.integers(0, 12))
def test_index_select_brute_force(seed, Bk, k, D, q_offset):
    rng = np.random.default_rng(seed)
    S_q = int(rng.integers(1, 40))
    S_k = q_offset + S_q + int(rng.integers(0, 6))
    G = 2
    lo = int(rng.integers(-3, 0))
    hi = int(rng.integers(0, 3))
    q_idx = rng.integers(lo, hi + 1, size=(1, S_q, G, D)).astype(np.float64)
    k_idx = rng.integers(lo, hi + 1, size=(1, S_k, D)).astype(np.float64)
    sel = orc.index_select(q_idx, k_idx, k, q_offset, Bk)
    for i in range(S_q):
        t = q_offset + i
        L = t // Bk
        for g in range(G):
            M = _brute_maxima(q_idx[0, i, g], k_idx[0], L, Bk)
            assert sel[0, g, i].tolist() == _brute_select(M, L, k)


# ---------------------------------------------------------------------------
# closed forms for the selection
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [1, 2, 4, 7])
def test_zero_query_selects_lowest_blocks(k):
    # all scores 0 -> every block ties -> the lowest k-1 ids, plus the local block
    Bk, S = 8, 80
    q_idx = np.zeros((1, S, 2, 4))
    k_idx = np.random.default_rng(0).integers(-4, 5, size=(1, S, 4)).astype(float)
    sel = orc.index_select(q_idx, k_idx, k, 0, Bk)
    for i in range(S):
        L = i // Bk
        want = sorted(set(range(min(k - 1, L))) | {L})
        want += [-1] * (k - len(want))
        assert sel[0, 0, i].tolist() == want
        assert sel[0, 1, i].tolist() == want


@pytest.mark.parametrize("sign", [1, -1])
def test_ramp_selects_nearest_or_farthest(sign):
    # k_idx[j,0] = sign*floor(j/Bk): block maxima are sign*c
    Bk, S, k = 8, 96, 4
    k_idx = np.zeros((1, S, 3))
    k_idx[0, :, 0] = sign * (np.arange(S) // Bk)
    q_idx = np.zeros((1, S, 1, 3))
    q_idx[0, :, 0, 0] = 1
    sel = orc.index_select(q_idx, k_idx, k, 0, Bk)
    for i in range(S):
        L = i // Bk
        if sign > 0:
            pick = list(range(max(0, L - (k - 1)), L))
        else:
            pick = list(range(min(k - 1, L)))
        want = sorted(pick + [L])
        assert sel[0, 0, i].tolist() == want + [-1] * (k - len(want))


# ---------------------------------------------------------------------------
# invariants of the selection
# ---------------------------------------------------------------------------

def _rand_idx(rng, B, S_q, S_k, G, D, lo=-4, hi=4):
    return (rng.integers(lo, hi + 1, size=(B, S_q, G, D)).astype(float),
            rng.integers(lo, hi + 1, size=(B, S_k, D)).astype(float))


@settings(max_examples=25, deadline=None)
@given(st.integers(0, 10_000), st.integers(1, 9), st.integers(0, 40))
def test_selection_invariants(seed, k, q_offset):
    rng = np.random.default_rng(seed)
    Bk, S_q, G, D = 8, 50, 3, 5
    S_k = q_offset + S_q + 3
    q_idx, k_idx = _rand_idx(rng, 2, S_q, S_k, G, D)
    sel = orc.index_select(q_idx, k_idx, k, q_offset, Bk)
    for b in range(2):
        for g in range(G):
            for i in range(S_q):
                t = q_offset + i
                L = t // Bk
                row = sel[b, g, i].tolist()
                ids = [c for c in row if c >= 0]
                assert L in ids                                  # local block always kept
                assert all(0 <= c <= L for c in ids)             # only visible blocks
                assert len(set(ids)) == len(ids)                 # no duplicates
                assert len(ids) == min(k, L + 1)                 # count
                assert ids == sorted(ids)                        # ascending
                assert row[len(ids):] == [-1] * (k - len(ids))   # -1 padding last
                # the token budget never exceeds k*Bk keys
                assert len(orc.token_set(sel[b, g, i], t, Bk)) <= k * Bk


def test_permuting_tokens_within_blocks_keeps_selection():
    rng = np.random.default_rng(3)
    Bk, S, G, D, k = 8, 64, 2, 6, 3
    q_idx, k_idx = _rand_idx(rng, 1, S, S, G, D)
    base = orc.index_select(q_idx, k_idx, k, 0, Bk)
    perm = np.concatenate([c * Bk + rng.permutation(Bk) for c in range(S // Bk)])
    sel = orc.index_select(q_idx, k_idx[:, perm], k, 0, Bk)
    np.testing.assert_array_equal(base, sel)


def test_raw_and_softmax_rankings_agree():
    # ranking max-pooled raw scores == ranking max-pooled softmax probabilities
    # (log-softmax: plain exp would underflow into false ties)
    rng = np.random.default_rng(5)
    Bk, S, G, D, k = 8, 72, 2, 4, 4
    q_idx, k_idx = _rand_idx(rng, 1, S, S, G, D, -8, 8)
    sel = orc.index_select(q_idx, k_idx, k, 0, Bk)
    for i in range(S):
        L = i // Bk
        for g in range(G):
            s = k_idx[0, : i + 1] @ q_idx[0, i, g]
            logp = s - (s.max() + np.log(np.exp(s - s.max()).sum()))
            Mp = logp[: L * Bk].reshape(L, Bk).max(axis=1) if L else np.zeros(0)
            order = sorted(range(L), key=lambda c: (-Mp[c], c))[: min(k - 1, L)]
            want = sorted(order + [L])
            assert sel[0, g, i].tolist() == want + [-1] * (k - len(want))


def _pooled_across_heads(q_idx, k_idx, k, Bk):
    """The defect the issue write-up (原因分析) describes: block scores pooled over
    the index-head axis, one selection broadcast to every group.  Negative control."""
    B, S_q, G, D = q_idx.shape
    sel = np.empty((B, G, S_q, k), dtype=np.int32)
    for b in range(B):
        for i in range(S_q):
            L = i // Bk
            M = np.max(np.stack([orc.block_maxima(q_idx[b, i, g][None], k_idx[b], L, Bk)[0]
                                 for g in range(G)]), axis=0)
            row = orc.select_from_maxima(M[None], L, k)[0]
            sel[b, :, i] = row
    return sel


def _independent(fn, q_idx, k_idx, k, Bk, g_pert, rng):
    """True when perturbing group g_pert's index query changes no other group's rows."""
    a = fn(q_idx, k_idx, k, Bk)
    q2 = q_idx.copy()
    q2[:, :, g_pert] = rng.integers(-4, 5, size=q2[:, :, g_pert].shape)
    b = fn(q2, k_idx, k, Bk)
    others = [g for g in range(q_idx.shape[2]) if g != g_pert]
    return np.array_equal(a[:, others], b[:, others]), not np.array_equal(a[:, g_pert], b[:, g_pert])


def test_per_group_independence_and_pooled_negative_control():
    rng = np.random.default_rng(11)
    Bk, S, G, D, k = 8, 96, 4, 6, 4
    q_idx, k_idx = _rand_idx(rng, 1, S, S, G, D)
    per_group = lambda q, kk, k_, B_: orc.index_select(q, kk, k_, 0, B_)  # noqa: E731
    ok_others, changed = _independent(per_group, q_idx, k_idx, k, Bk, 2, np.random.default_rng(1))
    assert ok_others and changed
    ok_others_pooled, _ = _independent(_pooled_across_heads, q_idx, k_idx, k, Bk, 2,
                                       np.random.default_rng(1))
    assert not ok_others_pooled  # pooling across index heads leaks between groups


def test_pooled_variant_diverges_like_the_issue_reports():
    # 验证方法/报错原文: per-group vs pooled selections differ on most rows
    facts = _load("page_facts.json")
    assert facts["pooled_divergence_after_fix"]["value"] == 0
    rng = np.random.default_rng(2)
    Bk, S, G, D, k = 8, 256, 4, 8, 6
    q_idx, k_idx = _rand_idx(rng, 1, S, S, G, D)
    a = orc.index_select(q_idx, k_idx, k, 0, Bk)
    b = _pooled_across_heads(q_idx, k_idx, k, Bk)
    rows = [(g, i) for g in range(G) for i in range(S) if i // Bk >= k]  # rows with a real choice
    div = sum(not np.array_equal(a[0, g, i], b[0, g, i]) for g, i in rows)
    assert div / len(rows) > 0.5
    # after the fix (one selection per index head), 0 of N rows diverge from a
    # per-group recomputation in pure Python and every row shares all k blocks
    def py_select(M, L):  # Python's own sort on (score desc, id asc), no numpy
        take = sorted(range(L), key=lambda c: (-M[c], c))[:min(k - 1, L)]
        chosen = sorted(take + [L])
        return chosen + [-1] * (k - len(chosen))

    brute = np.array([py_select(_brute_maxima(q_idx[0, i, g], k_idx[0], i // Bk, Bk), i // Bk) for g, i in rows],
                     dtype=np.int32)
    mine = np.array([a[0, g, i] for g, i in rows])
    pooled = np.array([b[0, g, i] for g, i in rows])
    rep = orc.selection_agreement(mine, brute)
    assert rep["rows"] == len(rows) and rep["diverging"] == 0 and rep["mean_overlap"] == k
    rep_pooled = orc.selection_agreement(pooled, brute)
    assert rep_pooled["diverging"] == div and rep_pooled["mean_overlap"] < k


def test_selection_agreement_counts_by_hand():
    ref = np.array([[0, 3, 5, -1], [1, 2, 4, 7], [0, 1, -1, -1]], dtype=np.int32)
    same = orc.selection_agreement(ref, ref)
    assert same == {"rows": 3, "diverging": 0, "mean_overlap": 3.0, "mean_ref_blocks": 3.0, "k": 4}
    sel = np.array([[0, 3, 5, -1],     # identical
                    [1, 2, 6, 7],      # one block swapped: 3 shared
                    [0, 1, 2, -1]],    # an extra block: 2 shared, diverges
                   dtype=np.int32)
    rep = orc.selection_agreement(sel, ref)
    assert rep["diverging"] == 2
    assert rep["mean_overlap"] == pytest.approx((3 + 3 + 2) / 3)
    # padding never counts as a shared block, and shapes must agree
    assert orc.selection_agreement(np.full((1, 4), -1), np.full((1, 4), -1))["mean_overlap"] == 0.0
    with pytest.raises(ValueError):
        orc.selection_agreement(sel[:2], ref)


# ---------------------------------------------------------------------------
# main branch against torch's scaled_dot_product_attention (CPU, float64)
# ---------------------------------------------------------------------------

def _mask_from_sel(sel, S_q, S_k, Hq, q_offset, Bk):
    """Dense [B,Hq,S_q,S_k] boolean mask: selected blocks of head h's group,
    repeat_interleave over the r heads, intersected with causality."""
    B, G, _, _ = sel.shape
    m = np.zeros((B, G, S_q, S_k), dtype=bool)
    for b in range(B):
        for g in range(G):
            for i in range(S_q):
                for c in sel[b, g, i]:
                    if c >= 0:
                        m[b, g, i, c * Bk:(c + 1) * Bk] = True
    causal = np.arange(S_k)[None, :] <= (q_offset + np.arange(S_q))[:, None]
    m &= causal[None, None]
    return torch.from_numpy(m).repeat_interleave(Hq // G, dim=1)


def _torch_sdpa(q, k, v, mask=None, causal=False, scale=None):
    Hq, G = q.shape[2], k.shape[1]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(Hq // G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // G, dim=1)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("q_offset,k", [(0, 2), (0, 3), (13, 2), (40, 5)])
def test_sparse_attention_vs_torch_masked_sdpa(q_offset, k):
    rng = np.random.default_rng(7 + q_offset)
    B, S_q, Hq, G, d, Bk, D = 2, 45, 6, 3, 5, 8, 4
    S_k = q_offset + S_q + 4
    q = rng.standard_normal((B, S_q, Hq, d))
    kk = rng.standard_normal((B, G, S_k, d))
    v = rng.standard_normal((B, G, S_k, d))
    q_idx, k_idx = _rand_idx(rng, B, S_q, S_k, G, D)
    out, sel, lse = orc.msa_forward(q, kk, v, q_idx, k_idx, k, q_offset, Bk)
    mask = _mask_from_sel(sel, S_q, S_k, Hq, q_offset, Bk)
    ref = _torch_sdpa(q, kk, v, mask=mask)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse from the masked logits
    s = np.einsum("bihd,bhjd->bhij", q, np.repeat(kk, Hq // G, axis=1)) / math.sqrt(d)
    s = np.where(mask.numpy(), s, -np.inf)
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_full_budget_equals_dense_causal():
    # when k covers every visible block MSA is dense causal attention
    rng = np.random.default_rng(9)
    B, S, Hq, G, d, Bk, D = 1, 64, 4, 2, 8, 8, 4
    k = S // Bk
    q = rng.standard_normal((B, S, Hq, d))
    kk = rng.standard_normal((B, G, S, d))
    v = rng.standard_normal((B, G, S, d))
    q_idx, k_idx = _rand_idx(rng, B, S, S, G, D)
    out, sel, _ = orc.msa_forward(q, kk, v, q_idx, k_idx, k, 0, Bk)
    ref = _torch_sdpa(q, kk, v, causal=True)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    dense, _ = orc.dense_causal_attention(q, kk, v)
    np.testing.assert_allclose(dense, ref, rtol=1e-12, atol=1e-12)


def test_early_rows_are_dense_at_any_k():
    # rows with t < k*Bk select every visible block
    rng = np.random.default_rng(4)
    B, S, Hq, G, d, Bk, D, k = 1, 80, 4, 2, 8, 8, 4, 3
    q = rng.standard_normal((B, S, Hq, d))
    kk = rng.standard_normal((B, G, S, d))
    v = rng.standard_normal((B, G, S, d))
    q_idx, k_idx = _rand_idx(rng, B, S, S, G, D)
    out, _, _ = orc.msa_forward(q, kk, v, q_idx, k_idx, k, 0, Bk)
    ref = _torch_sdpa(q, kk, v, causal=True)
    np.testing.assert_allclose(out[:, : k * Bk], ref[:, : k * Bk], rtol=1e-12, atol=1e-12)
    assert np.abs(out[:, k * Bk:] - ref[:, k * Bk:]).max() > 1e-3  # later rows are sparse


def test_main_branch_closed_forms():
    rng = np.random.default_rng(12)
    B, S, Hq, G, d, Bk, D, k = 1, 60, 4, 2, 6, 8, 3, 3
    kk = rng.standard_normal((B, G, S, d))
    v = rng.standard_normal((B, G, S, d))
    q_idx, k_idx = _rand_idx(rng, B, S, S, G, D)
    sel = orc.index_select(q_idx, k_idx, k, 0, Bk)
    # q = 0: uniform weights -> mean of v over the token set, lse = ln |T|
    out, lse = orc.sparse_attention(np.zeros((B, S, Hq, d)), kk, v, sel, 0, Bk)
    for i in range(S):
        for h in range(Hq):
            g = h // (Hq // G)
            T = orc.token_set(sel[0, g, i], i, Bk)
            np.testing.assert_allclose(out[0, i, h], v[0, g, T].mean(axis=0), rtol=1e-12, atol=1e-13)
            assert lse[0, h, i] == pytest.approx(math.log(len(T)), abs=1e-12)
    # constant v -> that constant
    q = rng.standard_normal((B, S, Hq, d))
    vc = np.full_like(v, 2.5)
    out, _ = orc.sparse_attention(q, kk, vc, sel, 0, Bk)
    np.testing.assert_allclose(out, 2.5, rtol=1e-13)
    # one key with an overwhelming score -> its value
    k2 = kk.copy()
    i, g = 50, 1
    T = orc.token_set(sel[0, g, i], i, Bk)
    j = int(T[len(T) // 2])
    qv = rng.standard_normal(d)
    k2[0, g, j] = 80.0 * qv / np.linalg.norm(qv)
    q2 = np.zeros((B, S, Hq, d))
    q2[0, i, g * 2:(g + 1) * 2] = 80.0 * qv / np.linalg.norm(qv)
    out, _ = orc.sparse_attention(q2, k2, v, sel, 0, Bk, rows=[(0, i)])
    np.testing.assert_allclose(out[0, i, g * 2], v[0, g, j], rtol=1e-9, atol=1e-9)


def test_k1_is_local_block_causal_attention():
    rng = np.random.default_rng(13)
    B, S, Hq, G, d, Bk, D = 1, 40, 4, 2, 6, 8, 3
    q = rng.standard_normal((B, S, Hq, d))
    kk = rng.standard_normal((B, G, S, d))
    v = rng.standard_normal((B, G, S, d))
    q_idx, k_idx = _rand_idx(rng, B, S, S, G, D)
    out, sel, _ = orc.msa_forward(q, kk, v, q_idx, k_idx, 1, 0, Bk)
    assert (sel[..., 0] == (np.arange(S) // Bk)[None, None]).all()
    blk = np.arange(S) // Bk
    local = (blk[:, None] == blk[None, :]) & (np.arange(S)[None, :] <= np.arange(S)[:, None])
    mask = torch.from_numpy(local)[None, None].expand(B, Hq, S, S)
    np.testing.assert_allclose(out, _torch_sdpa(q, kk, v, mask=mask), rtol=1e-12, atol=1e-12)


def test_group_map_is_contiguous():
    # head h reads KV head floor(h / r) (repeat_interleave of the fix)
    facts = _load("page_facts.json")["qheads_per_kv"]
    Hq, G = facts["num_q_heads"] // 8, facts["num_kv_heads"]
    assert facts["num_q_heads"] // facts["num_kv_heads"] == facts["value"]
    B, S, d, Bk, k = 1, 8, 3, 8, 1
    rng = np.random.default_rng(1)
    q = rng.standard_normal((B, S, Hq, d))
    kk = rng.standard_normal((B, G, S, d))
    v = np.zeros((B, G, S, d))
    for g in range(G):
        v[0, g] = g + 1.0
    sel = np.zeros((B, G, S, k), dtype=np.int32)
    out, _ = orc.sparse_attention(q, kk, v, sel, 0, Bk)
    r = Hq // G
    for h in range(Hq):
        np.testing.assert_allclose(out[0, :, h], h // r + 1.0)


def test_q2k_layout_matches_the_fix():
    # 解决步骤: the kernel-path q2k is [num_kv_heads, bsz*q_len, topk], one list per KV head
    rng = np.random.default_rng(8)
    B, S, G, D, k, Bk = 2, 24, 4, 3, 3, 8
    q_idx, k_idx = _rand_idx(rng, B, S, S, G, D)
    sel = orc.index_select(q_idx, k_idx, k, 0, Bk)
    q2k = torch.from_numpy(sel).permute(1, 0, 2, 3).reshape(G, B * S, k)
    for g in range(G):
        for b in range(B):
            for i in range(S):
                assert q2k[g, b * S + i].tolist() == sel[b, g, i].tolist()


def test_index_scores_exact_integers():
    # fp64 index scores equal int64 ones for the integer workloads
    rng = np.random.default_rng(0)
    s = synth.WORKLOADS[2]
    qi = rng.integers(s.idx_lo, s.idx_hi + 1, size=(16, s.index_dim))
    ki = rng.integers(s.idx_lo, s.idx_hi + 1, size=(4 * 128, s.index_dim))
    M = orc.block_maxima(qi.astype(np.float64), ki.astype(np.float64), 4, 128)
    Mi = (qi @ ki.T).reshape(16, 4, 128).max(axis=2)
    np.testing.assert_array_equal(M, Mi.astype(np.float64))
    assert np.abs(qi @ ki.T).max() <= 16 * s.index_dim < 2 ** 24


def test_page_budget_facts():
    f = _load("page_facts.json")
    assert f["block_size"]["value"] * f["topk"]["value"] == f["token_budget"]["value"]
    for wid in (2, 3, 4, 5):
        s = synth.WORKLOADS[wid]
        assert s.block_size == f["block_size"]["value"] and s.topk == f["topk"]["value"]
        assert s.num_q_heads // s.num_kv_heads == f["qheads_per_kv"]["value"]


def test_synth_inputs_are_exact_and_seeded():
    s = synth.WORKLOADS[1].replace(q_len=64, kv_len=64)
    a = synth.host_inputs(s, 1)
    b = synth.host_inputs(s, 1)
    for n in a:
        assert torch.equal(a[n], b[n])
    assert a["q_idx"].dtype == torch.float32
    qi = a["q_idx"].numpy()
    assert (qi == np.round(qi)).all() and qi.min() >= -8 and qi.max() <= 8
    s2 = synth.WORKLOADS[2].replace(q_len=64, kv_len=64)
    c = synth.host_inputs(s2, 2)
    assert c["q"].dtype == torch.bfloat16
    ki = synth.as_f64(c["k_idx"])
    assert (ki == np.round(ki)).all() and ki.min() >= -4 and ki.max() <= 4


# --- FP8 (OCP E4M3) cache values -------------------------------------------
# The pages list FP8 among the inference kernel's precisions (Hungarian page,
# "Elérhetőség"); the format read into that is OCP FP8 E4M3 (e4m3fn).  The
# decoder is pinned to torch's own float8_e4m3fn conversion and to the special
# values the OCP OFP8 specification fixes for E4M3.

def test_e4m3_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(mine, ref, equal_nan=True)
    assert np.array_equal(np.signbit(mine), np.signbit(ref))


def test_e4m3_special_values():
    v = orc.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite magnitude
    assert v[0x08] == 2.0 ** -6                             # smallest normal
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x01] == 2.0 ** -9  # subnormals
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])          # the only NaNs, no infinities
    assert np.isfinite(v[[c for c in range(256) if c not in (0x7F, 0xFF)]]).all()
    assert v[0x38] == 1.0 and v[0x3C] == 1.5 and v[0xB8] == -1.0
    # sign-magnitude order: positive codes increase strictly, negatives mirror them
    pos = v[0x00:0x7F]
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(v[0x80:0xFF], -pos)


def test_e4m3_dequantize_is_exact():
    from fractions import Fraction
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    for scale in (1.0, 6.0 / 448, 0.0123, 3.0):
        s32 = float(np.float32(scale))
        got = orc.dequantize_e4m3(codes, scale)
        for c, g in zip(codes[::7], got[::7]):
            assert Fraction(g) == Fraction(float(orc.e4m3_to_f64(c))) * Fraction(s32)


def test_synth_fp8_caches():
    s = synth.Shape(2, 5, 700, 300, 8, 2, 64, 32, 4, cache="fp8", k_scale=0.02, v_scale=0.05)
    x = synth.host_inputs(s, 9)
    for n in ("k", "v", "k_idx"):
        assert x[n].dtype == torch.float8_e4m3fn
    for n in ("q", "q_idx"):
        assert x[n].dtype == torch.bfloat16
    ki = orc.e4m3_to_f64(synth.codes(x["k_idx"]))
    assert set(np.unique(ki)) <= set(range(-4, 5))  # integers stored exactly
    # the same seeded draws as the bf16 recipe, divided by the scale before rounding
    ref = synth.host_inputs(s.replace(cache="native", dtype="f32", idx_lo=-4, idx_hi=4), 9)
    kv = orc.e4m3_to_f64(synth.codes(x["k"]))
    assert np.array_equal(ki, synth.as_f64(ref["k_idx"]))
    rel = np.abs(kv * 0.02 - synth.as_f64(ref["k"])) / np.maximum(np.abs(synth.as_f64(ref["k"])), 2.0 ** -6 * 0.02)
    assert rel.max() <= 2.0 ** -4 + 1e-12  # round to nearest with a 3-bit mantissa
    with pytest.raises(TypeError):
        synth.as_f64(x["k"])


# --- caches of unequal length and paged caches --------------------------------

def test_page_gather_inverts_a_scatter():
    rng = np.random.default_rng(3)
    for n in (1, 127, 128, 129, 700):
        nb = -(-n // 128)
        dense_kv = rng.standard_normal((2, nb * 128, 8))
        dense_ki = rng.standard_normal((nb * 128, 4))
        P = nb + 5
        pages = rng.permutation(P)[:nb]
        pool_kv = rng.standard_normal((P, 2, 128, 8))
        pool_ki = rng.standard_normal((P, 128, 4))
        for c in range(nb):  # plain scatter of block c into page pages[c]
            pool_kv[pages[c]] = dense_kv[:, c * 128:(c + 1) * 128]
            pool_ki[pages[c]] = dense_ki[c * 128:(c + 1) * 128]
        assert np.array_equal(orc.page_gather(pool_kv, pages, n), dense_kv[:, :n])
        assert np.array_equal(orc.page_gather(pool_ki, pages, n), dense_ki[:n])
    assert orc.page_gather(np.zeros((3, 2, 128, 8)), [], 0).shape == (2, 0, 8)


def _varlen_case(seed, lens, S_q, G=2, r=2, d=16, D=8, lo=-4, hi=4):
    rng = np.random.default_rng(seed)
    B = len(lens)
    q = rng.standard_normal((B, S_q, G * r, d))
    qi = rng.integers(lo, hi + 1, (B, S_q, G, D)).astype(np.float64)
    ks = [rng.standard_normal((G, n, d)) for n in lens]
    vs = [rng.standard_normal((G, n, d)) for n in lens]
    kis = [rng.integers(lo, hi + 1, (n, D)).astype(np.float64) for n in lens]
    return q, ks, vs, qi, kis


def test_varlen_equal_lengths_is_the_plain_forward():
    lens, S_q, k = [300, 300, 300], 5, 2
    q, ks, vs, qi, kis = _varlen_case(1, lens, S_q)
    out, sel, lse = orc.msa_forward_varlen(q, ks, vs, qi, kis, k, block_size=32)
    ro, rs, rl = orc.msa_forward(q, np.stack(ks), np.stack(vs), qi, np.stack(kis), k, 300 - S_q, 32)
    assert np.array_equal(sel, rs)
    assert np.allclose(out, ro, atol=1e-12) and np.allclose(lse, rl, atol=1e-12)


def test_varlen_rows_before_the_cache():
    # sequence 1 holds 2 tokens but has 5 query rows: rows 0..2 precede it
    lens, S_q, k = [90, 2, 33], 5, 3
    q, ks, vs, qi, kis = _varlen_case(2, lens, S_q)
    out, sel, lse = orc.msa_forward_varlen(q, ks, vs, qi, kis, k, block_size=16)
    assert (sel[1, :, :3] == -1).all() and (out[1, :3] == 0).all() and np.isneginf(lse[1, :, :3]).all()
    ro, rs, rl = orc.msa_forward(q[1:2, 3:], ks[1][None], vs[1][None], qi[1:2, 3:], kis[1][None], k, 0, 16)
    assert np.array_equal(sel[1, :, 3:], rs[0]) and np.allclose(out[1, 3:], ro[0]) and np.allclose(lse[1, :, 3:], rl[0])
    assert sel[1, 0, 3].tolist() == [0, -1, -1]  # position 0: the local block only


def test_varlen_positions_against_torch_sdpa():
    # k at least the number of blocks: every row is dense causal attention over
    # its own cache with the query at position n_b - S_q + i
    lens, S_q, Bk = [40, 7, 64, 3], 4, 16
    q, ks, vs, qi, kis = _varlen_case(5, lens, S_q)
    out, sel, lse = orc.msa_forward_varlen(q, ks, vs, qi, kis, topk=8, block_size=Bk)
    G, r, d = 2, 2, 16
    for b, n in enumerate(lens):
        for i in range(S_q):
            t = n - S_q + i
            if t < 0:
                continue
            for h in range(G * r):
                g = h // r
                qh = torch.from_numpy(q[b, i, h]).view(1, 1, 1, d)
                kk = torch.from_numpy(ks[b][g, :t + 1]).view(1, 1, t + 1, d)
                vv = torch.from_numpy(vs[b][g, :t + 1]).view(1, 1, t + 1, d)
                ref = F.scaled_dot_product_attention(qh, kk, vv).view(d).numpy()
                assert np.allclose(out[b, i, h], ref, atol=1e-12)
                s_ = (ks[b][g, :t + 1] @ q[b, i, h]) / math.sqrt(d)
                assert abs(lse[b, h, i] - (s_.max() + math.log(np.exp(s_ - s_.max()).sum()))) < 1e-12


# --- KL-alignment teacher (forward) --------------------------------------------
# Teacher: the main distribution over the selected tokens averaged over the
# group's heads (snilld page, "Træning og stabilisering"); student: the softmax
# of the index scores over the same tokens; loss KL(teacher || student).

def _kl_case(seed, B=2, S_q=40, S_k=200, qo=160, G=2, r=4, d=16, D=8, k=3, Bk=32):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S_q, G * r, d))
    kk = rng.standard_normal((B, G, S_k, d))
    qi = rng.integers(-3, 4, (B, S_q, G, D)).astype(np.float64)
    ki = rng.integers(-3, 4, (B, S_k, D)).astype(np.float64)
    sel = orc.index_select(qi, ki, k, qo, Bk)
    return q, kk, qi, ki, sel, qo, Bk


def test_kl_teacher_against_torch_kl_div():
    q, kk, qi, ki, sel, qo, Bk = _kl_case(1)
    kl, ilse = orc.kl_teacher(q, kk, qi, ki, sel, qo, Bk, index_scale=0.7)
    B, S_q, Hq, d = q.shape
    G, r = kk.shape[1], Hq // kk.shape[1]
    S_k = kk.shape[2]
    for b in range(B):
        for g in range(G):
            # dense masks from the selection, softmaxes and KL by torch primitives
            mask = torch.zeros(S_q, S_k, dtype=torch.bool)
            for i in range(S_q):
                for c in sel[b, g, i]:
                    if c >= 0:
                        mask[i, c * Bk:min((c + 1) * Bk, qo + i + 1)] = True
            s = torch.einsum("ihd,jd->hij", torch.from_numpy(q[b, :, g * r:(g + 1) * r]),
                             torch.from_numpy(kk[b, g])) / math.sqrt(d)
            pbar = torch.softmax(s.masked_fill(~mask, -math.inf), dim=-1).mean(0)
            si = 0.7 * (torch.from_numpy(qi[b, :, g]) @ torch.from_numpy(ki[b]).T)
            logq = torch.log_softmax(si.masked_fill(~mask, -math.inf), dim=-1)
            ref = F.kl_div(logq.masked_fill(~mask, 0.0), pbar, reduction="none").sum(-1)
            assert np.allclose(kl[b, g], ref.numpy(), atol=1e-12, rtol=1e-10)
            assert np.allclose(ilse[b, g], torch.logsumexp(si.masked_fill(~mask, -math.inf), -1).numpy(), atol=1e-12)


def test_kl_teacher_closed_forms():
    q, kk, qi, ki, sel, qo, Bk = _kl_case(2, r=1, D=16)
    d = q.shape[3]
    # index scores equal to the main scores: the index distribution is the teacher, KL = 0
    qi2 = q[:, :, :, :] / math.sqrt(d)        # r = 1: one head per group, q_idx = scale * q
    ki2 = kk[:, 0]                             # G = 2 groups share the index key: use group 0 only
    kl, _ = orc.kl_teacher(q[:, :, :1], kk[:, :1], qi2[:, :, :1], ki2, sel[:, :1], qo, Bk)
    assert np.abs(kl).max() < 1e-12
    # a uniform teacher (q = 0): KL = lse(s) - mean(s) - log n over the token set
    q0 = np.zeros_like(q)
    kl, ilse = orc.kl_teacher(q0, kk, qi, ki, sel, qo, Bk)
    for b, g, i in [(0, 0, 0), (1, 1, 39), (0, 1, 17)]:
        T = orc.token_set(sel[b, g, i], qo + i, Bk)
        si = ki[b, T] @ qi[b, i, g]
        m = si.max()
        lse = m + math.log(np.exp(si - m).sum())
        assert abs(kl[b, g, i] - (lse - si.mean() - math.log(len(T)))) < 1e-12
        assert abs(ilse[b, g, i] - lse) < 1e-12
    # index_scale -> 0: a uniform student, KL = sum pbar log pbar + log n >= 0
    kl, _ = orc.kl_teacher(q, kk, qi, ki, sel, qo, Bk, index_scale=0.0)
    assert (kl > -1e-12).all()


def test_kl_teacher_invariants():
    q, kk, qi, ki, sel, qo, Bk = _kl_case(3)
    kl, _ = orc.kl_teacher(q, kk, qi, ki, sel, qo, Bk)
    assert (kl >= -1e-12).all()  # Gibbs' inequality
    # identical heads in a group: the teacher is that head's own distribution
    qs = np.repeat(q[:, :, ::4], 4, axis=2)   # r = 4: every head equal to the group's first
    kl_rep, _ = orc.kl_teacher(qs, kk, qi, ki, sel, qo, Bk)
    kl_one, _ = orc.kl_teacher(q[:, :, ::4], kk, qi, ki, sel, qo, Bk)
    assert np.allclose(kl_rep, kl_one, atol=1e-12)
    # rows before their cache (empty token set): 0 and -inf
    sel2 = sel.copy()
    sel2[0, 0, 5] = -1
    kl2, ilse2 = orc.kl_teacher(q, kk, qi, ki, sel2, qo, Bk)
    assert kl2[0, 0, 5] == 0.0 and np.isneginf(ilse2[0, 0, 5])


# --- backward of the main branch --------------------------------------------

def test_sparse_attention_bwd_against_torch_autograd():
    rng = np.random.default_rng(21)
    B, S_q, S_k, qo, G, r, d, D, k, Bk = 2, 30, 160, 130, 2, 3, 8, 4, 3, 32
    q = rng.standard_normal((B, S_q, G * r, d))
    kk = rng.standard_normal((B, G, S_k, d))
    vv = rng.standard_normal((B, G, S_k, d))
    qi = rng.integers(-3, 4, (B, S_q, G, D)).astype(np.float64)
    ki = rng.integers(-3, 4, (B, S_k, D)).astype(np.float64)
    sel = orc.index_select(qi, ki, k, qo, Bk)
    dout = rng.standard_normal((B, S_q, G * r, d))
    dq, dk, dv = orc.sparse_attention_bwd(q, kk, vv, sel, dout, qo, Bk)
    # torch: dense masked SDPA in fp64 with autograd, the mask from the selection
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_(True)       # [B, Hq, S_q, d]
    tk = torch.from_numpy(kk).clone().requires_grad_(True)                            # [B, G, S_k, d]
    tv = torch.from_numpy(vv).clone().requires_grad_(True)
    mask = torch.zeros(B, G * r, S_q, S_k, dtype=torch.bool)
    for b in range(B):
        for g in range(G):
            for i in range(S_q):
                for c in sel[b, g, i]:
                    if c >= 0:
                        mask[b, g * r:(g + 1) * r, i, c * Bk:min((c + 1) * Bk, qo + i + 1)] = True
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(r, dim=1), tv.repeat_interleave(r, dim=1),
                                         attn_mask=mask)
    out.backward(torch.from_numpy(dout).permute(0, 2, 1, 3))
    assert np.allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_sparse_attention_bwd_closed_forms():
    rng = np.random.default_rng(22)
    B, S_q, S_k, G, r, d, Bk = 1, 6, 6, 1, 2, 4, 4
    q = rng.standard_normal((B, S_q, r, d))
    kk = rng.standard_normal((B, G, S_k, d))
    vv = rng.standard_normal((B, G, S_k, d))
    sel = np.full((B, G, S_q, 2), -1, dtype=np.int32)
    sel[0, 0, :, 0] = 0
    sel[0, 0, 4:, 1] = 1
    # a zero output gradient gives zero gradients
    z = orc.sparse_attention_bwd(q, kk, vv, sel, np.zeros_like(q), 0, Bk)
    assert all(np.abs(x).max() == 0 for x in z)
    # row 0 attends to key 0 alone: p = 1, so dq = 0 and dv[0] gets dO of that row
    dout = np.zeros_like(q)
    dout[0, 0] = rng.standard_normal((r, d))
    dq, dk, dv = orc.sparse_attention_bwd(q, kk, vv, sel, dout, 0, Bk)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    assert np.allclose(dv[0, 0, 0], dout[0, 0].sum(axis=0)) and np.abs(dv[0, 0, 1:]).max() == 0
    # the gradients are those of a linear functional: a central difference agrees
    dout = rng.standard_normal(q.shape)
    dq, dk, dv = orc.sparse_attention_bwd(q, kk, vv, sel, dout, 0, Bk)
    f = lambda qq, k_, v_: float((orc.sparse_attention(qq, k_, v_, sel, 0, Bk)[0] * dout).sum())
    eps = 1e-6
    for (arr, grad, idx) in ((q, dq, (0, 5, 1, 2)), (kk, dk, (0, 0, 3, 1)), (vv, dv, (0, 0, 5, 0))):
        a1, a2 = arr.copy(), arr.copy()
        a1[idx] += eps
        a2[idx] -= eps
        args1 = [q, kk, vv]
        args2 = [q, kk, vv]
        which = 0 if arr is q else (1 if arr is kk else 2)
        args1[which], args2[which] = a1, a2
        num = (f(*args1) - f(*args2)) / (2 * eps)
        assert abs(num - grad[idx]) < 1e-7

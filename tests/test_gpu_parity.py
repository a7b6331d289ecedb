"""GPU parity: the HIP library against the fp64 CPU oracle on seeded inputs.

Selections must match bit for bit; outputs within max-abs 1e-5 (fp32 inputs and
outputs) or 2e-2 (bf16) of the fp64 oracle, as stated for the workloads.
Small cases span several tiles and a ragged tail; the workload cases run the
exact shapes the benchmark times and check sampled rows.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import msa_oracle as orc

gpu = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()  # fails loudly when the library is not built
    return msa


def _inputs(s, seed, device="cuda"):
    x = synth.host_inputs(s, seed)
    return {n: t.to(device) for n, t in x.items()}, x


def _check_sel_rows(sel_gpu, sel_ref, rows=None):
    sg = sel_gpu.cpu().numpy()
    if rows is None:
        bad = np.argwhere((sg != sel_ref).any(axis=-1))
        assert bad.size == 0, f"{len(bad)} selection rows differ, first {bad[:5].tolist()}"
    else:
        for b, i in rows:
            np.testing.assert_array_equal(sg[b, :, i], sel_ref[b, :, i], err_msg=f"row b={b} i={i}")


def _max_err(out_gpu, out_ref, rows=None):
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    if rows is None:
        return float(np.abs(o - out_ref).max())
    return max(float(np.abs(o[b, i] - out_ref[b, i]).max()) for b, i in rows)


SMALL_SHAPES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k, dtype)
    (1, 1024, 1024, 0, 8, 2, 64, 32, 4, "f32"),
    (2, 700, 900, 200, 8, 2, 64, 32, 3, "f32"),
    (1, 1000, 1000, 0, 32, 2, 128, 128, 5, "bf16"),
    (2, 513, 1500, 987, 16, 4, 128, 64, 6, "bf16"),
    (1, 300, 4300, 4000, 64, 4, 128, 128, 16, "bf16"),
    (1, 129, 129, 0, 4, 4, 64, 32, 1, "bf16"),
    (3, 1, 2000, 1999, 64, 4, 128, 128, 16, "bf16"),   # decode
    (2, 5, 3000, 2990, 32, 1, 128, 128, 8, "bf16"),    # few queries, one group
    (1, 640, 640, 0, 32, 1, 64, 32, 32, "f32"),        # k above the visible blocks
    (1, 700, 6000, 5300, 16, 2, 128, 128, 24, "bf16"), # k > 16: the longer top lists
    (2, 300, 9000, 8700, 32, 2, 128, 128, 32, "bf16"), # k = 32, several key splits
    # k > 32: every lane half's top list of 63 goes to the merge kernel
    (1, 500, 12000, 11500, 16, 2, 128, 128, 64, "bf16"),  # prefill form, six key splits
    (2, 300, 9000, 8700, 16, 2, 64, 64, 48, "f32"),       # fp32 inputs, k = 48
    (3, 1, 20000, 19999, 64, 4, 128, 128, 64, "bf16"),    # decode (few-row form), 16 key splits
    (1, 900, 900, 0, 8, 2, 64, 32, 64, "bf16"),           # k above the visible blocks
]


@gpu
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_small(shape):
    msa = _msa()
    B, S_q, S_k, qo, Hq, Hkv, d, D, k, dt = shape
    lo, hi = (-8, 8) if dt == "f32" else (-4, 4)
    s = synth.Shape(B, S_q, S_k, qo, Hq, Hkv, d, D, k, dtype=dt, idx_lo=lo, idx_hi=hi)
    x, xh = _inputs(s, 100 + sum(shape[:-1]))
    print(f"case {shape}", flush=True)
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=qo,
                            return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_out, ref_sel, ref_lse = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], k, qo)
    _check_sel_rows(sel, ref_sel)
    err = _max_err(out, ref_out)
    assert err <= TOL[dt], f"max abs err {err}"
    lerr = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    assert lerr <= 1e-3, f"lse err {lerr}"


@gpu
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_sparse_attn_given_selection_and_f32_out(dt):
    # the main branch alone, from the oracle's selection, with an fp32 output
    msa = _msa()
    s = synth.Shape(2, 600, 800, 200, 16, 4, 128, 32, 5, dtype=dt)
    x, xh = _inputs(s, 7)
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_sel = orc.index_select(f["q_idx"], f["k_idx"], s.topk, s.q_offset)
    sel = torch.from_numpy(ref_sel).cuda()
    out, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], sel, q_offset=s.q_offset,
                                   out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = orc.sparse_attention(f["q"], f["k"], f["v"], ref_sel, s.q_offset)
    err = _max_err(out, ref_out)
    assert err <= (1e-5 if dt == "f32" else 1e-2), err
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-3


@gpu
def test_index_select_only_matches_oracle():
    msa = _msa()
    s = synth.Shape(2, 777, 2000, 1000, 8, 4, 64, 128, 16, dtype="bf16")
    x, xh = _inputs(s, 3)
    sel = msa.index_select(x["q_idx"], x["k_idx"], s.topk, q_offset=s.q_offset)
    torch.cuda.synchronize()
    ref = orc.index_select(synth.as_f64(xh["q_idx"]), synth.as_f64(xh["k_idx"]), s.topk, s.q_offset)
    _check_sel_rows(sel, ref)


@gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("topk,cache,offset", [(16, "native", 0), (16, "fp8", 0), (32, "native", 0),
                                               (16, "native", 1)])
def test_index_persistent_grid_ragged_every_row(topk, cache, offset):
    # 8 groups x 32845 rows = 262760 (row, group) pairs: 514 tiles of 512 (k <= 16)
    # or 1027 of 256 (k = 32), the last one holding 104 rows, so each tile is one
    # unit with one key split and the index kernel runs its persistent grid (more
    # tiles than resident workgroups, units handed out in snake order over several
    # rounds); e4m3 keys take the staged path; a selection buffer 4 bytes past a
    # 16-byte boundary (offset 1) takes the per-entry stores instead of 16-byte
    # rows.  Every row is checked.
    msa = _msa()
    n = 32768 + 77
    s = synth.Shape(1, n, n, 0, 32, 8, 64, 128, topk, dtype="bf16", cache=cache)
    x, xh = _inputs(s, 11)
    print(f"persistent-grid shape: {s.batch} x {n} rows, {s.groups} groups, k = {topk}, {cache} keys", flush=True)
    shape = (s.batch, s.groups, n, s.topk)
    buf = torch.full((int(np.prod(shape)) + 4,), -7, dtype=torch.int32, device="cuda")
    out = buf[offset:offset + int(np.prod(shape))].view(shape)
    assert (out.data_ptr() % 16 == 0) == (offset == 0)
    sel = msa.index_select(x["q_idx"], x["k_idx"], s.topk, q_offset=0, sel=out)
    torch.cuda.synchronize()
    assert int(buf[:offset].ne(-7).sum()) == 0 and int(buf[offset + out.numel():].ne(-7).sum()) == 0
    k_idx = orc.dequantize_e4m3(synth.codes(xh["k_idx"]), 1.0) if cache == "fp8" else synth.as_f64(xh["k_idx"])
    ref = orc.index_select(synth.as_f64(xh["q_idx"]), k_idx, s.topk, 0)
    _check_sel_rows(sel, ref)


@gpu
def test_ties_resolve_to_lower_block():
    # all-zero index queries: every block ties, the lowest ids must win
    msa = _msa()
    s = synth.Shape(1, 2048, 2048, 0, 16, 4, 128, 128, 8, dtype="bf16")
    x, _ = _inputs(s, 5)
    q_idx = torch.zeros_like(x["q_idx"])
    sel = msa.index_select(q_idx, x["k_idx"], s.topk).cpu().numpy()
    for i in range(0, 2048, 61):
        L = i // 128
        want = sorted(set(range(min(7, L))) | {L})
        assert sel[0, 0, i].tolist() == want + [-1] * (8 - len(want))


@gpu
def test_deterministic_reruns():
    msa = _msa()
    s = synth.Shape(1, 2048, 2048, 0, 64, 4, 128, 128, 16, dtype="bf16")
    x, _ = _inputs(s, 9)
    a = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], 16, return_sel=True)
    b = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], 16, return_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1])
    assert torch.equal(a[0], b[0])


@gpu
def test_workload_1k_fp32_full():
    msa = _msa()
    s = synth.WORKLOADS[1]
    x, xh = _inputs(s, 1)
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, return_sel=True,
                            return_lse=True)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_out, ref_sel, ref_lse = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], s.topk)
    _check_sel_rows(sel, ref_sel)
    assert _max_err(out, ref_out) <= 1e-5
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-5


@gpu
def test_workload_8k_bf16():
    msa = _msa()
    s = synth.WORKLOADS[2]
    x, xh = _inputs(s, 2)
    out, sel = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, return_sel=True)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_sel = orc.index_select(f["q_idx"], f["k_idx"], s.topk)
    _check_sel_rows(sel, ref_sel)  # every row, bit for bit
    rng = np.random.default_rng(0)
    rows = [(0, int(i)) for i in np.concatenate([rng.integers(0, s.q_len, 120), [0, 1, 127, 128, 8191]])]
    ref_out, _ = orc.sparse_attention(f["q"], f["k"], f["v"], ref_sel, rows=rows)
    assert _max_err(out, ref_out, rows) <= TOL["bf16"]


@gpu
def test_workload_8k_k64_is_dense_causal():
    # With k = 64 every row of the 8K workload (64 blocks) selects all of its
    # visible blocks, so MSA is plain causal attention: the selection is known in
    # closed form and the output must match the dense causal reference.
    msa = _msa()
    s = synth.WORKLOADS[2].replace(topk=64)
    x, xh = _inputs(s, 2)
    print("8K workload, k = 64", flush=True)
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, return_sel=True,
                            return_lse=True)
    torch.cuda.synchronize()
    L = np.arange(s.q_len) // 128
    slot = np.arange(s.topk)
    want = np.where(slot[None, :] <= L[:, None], slot[None, :], -1)
    sg = sel.cpu().numpy()
    assert (sg == want[None, None]).all()
    f = {n: synth.as_f64(xh[n]) for n in ("q", "k", "v")}
    rng = np.random.default_rng(4)
    lg = lse.cpu().numpy()
    for i in [int(v) for v in np.concatenate([rng.integers(0, s.q_len, 24), [0, 127, 128, 8191]])]:
        ro, rl = orc.dense_causal_attention(f["q"][:, i:i + 1], f["k"], f["v"], q_offset=i)
        assert float(np.abs(out[0, i].float().cpu().numpy() - ro[0, 0]).max()) <= TOL["bf16"], i
        assert float(np.abs(lg[0, :, i] - rl[0, :, 0]).max()) <= 1e-3, i


@gpu
@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_match_oracle(seed):
    # seeded sweep over the supported shape space (several tiles, ragged tails)
    msa = _msa()
    rng = np.random.default_rng(1000 + seed)
    dt = "f32" if seed % 4 == 0 else "bf16"
    G = int(rng.choice([1, 2, 4]))
    r = int(rng.choice([1, 2, 4, 8, 16, 32]))
    d = int(rng.choice([64, 128]))
    D = int(rng.choice([32, 64, 128]))
    k = int(rng.integers(1, 33))
    B = int(rng.integers(1, 3))
    S_q = int(rng.integers(1, 600))
    q_offset = int(rng.integers(0, 2500))
    S_k = q_offset + S_q + int(rng.integers(0, 300))
    lo, hi = (-8, 8) if dt == "f32" else (-4, 4)
    s = synth.Shape(B, S_q, S_k, q_offset, G * r, G, d, D, k, dtype=dt, idx_lo=lo, idx_hi=hi)
    print(f"case {s}", flush=True)
    x, xh = _inputs(s, 2000 + seed)
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=q_offset,
                            return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_out, ref_sel, ref_lse = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], k, q_offset)
    _check_sel_rows(sel, ref_sel)
    assert _max_err(out, ref_out) <= TOL[dt]
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-3


@gpu
def test_user_selection_with_invalid_ids_is_safe():
    # ids beyond the cache or after the query's local block are ignored; -1
    # padding anywhere in a row is skipped; the rest is exact attention
    msa = _msa()
    s = synth.Shape(1, 300, 1000, 600, 16, 2, 128, 64, 6, dtype="bf16")
    x, xh = _inputs(s, 11)
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    good = orc.index_select(f["q_idx"], f["k_idx"], s.topk, s.q_offset)
    bad = good.copy()
    nb = (s.kv_len + 127) // 128
    rng = np.random.default_rng(4)
    for g in range(s.groups):
        for i in range(s.q_len):
            row = [c for c in good[0, g, i] if c >= 0]
            L = (s.q_offset + i) // 128
            extra = [nb + 3, 10 ** 6, L + 1] if L + 1 < nb else [nb + 3, 10 ** 6]
            row = row + extra[: s.topk - len(row)]
            rng.shuffle(row)
            bad[0, g, i, :len(row)] = row
            bad[0, g, i, len(row):] = -1
    out = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], torch.from_numpy(bad).cuda(), q_offset=s.q_offset)
    torch.cuda.synchronize()
    ref, _ = orc.sparse_attention(f["q"], f["k"], f["v"], good, s.q_offset)
    assert _max_err(out, ref) <= TOL["bf16"]


@gpu
@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_wide_k(seed):
    # seeded sweep over k = 33..64 with caches long enough that most rows rank
    # more blocks than they keep (the wide top lists and the merge of up to 128)
    msa = _msa()
    rng = np.random.default_rng(3000 + seed)
    dt = "f32" if seed % 3 == 0 else "bf16"
    G = int(rng.choice([1, 2, 4]))
    r = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    D = int(rng.choice([32, 64, 128]))
    k = int(rng.integers(33, 65))
    B = int(rng.integers(1, 3))
    S_q = int(rng.choice([1, 3, int(rng.integers(1, 300))]))
    q_offset = int(rng.integers(4000, 12000))
    S_k = q_offset + S_q + int(rng.integers(0, 300))
    lo, hi = (-8, 8) if dt == "f32" else (-4, 4)
    s = synth.Shape(B, S_q, S_k, q_offset, G * r, G, d, D, k, dtype=dt, idx_lo=lo, idx_hi=hi)
    print(f"case {s}", flush=True)
    x, xh = _inputs(s, 4000 + seed)
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=q_offset,
                            return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_out, ref_sel, ref_lse = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], k, q_offset)
    _check_sel_rows(sel, ref_sel)
    assert _max_err(out, ref_out) <= TOL[dt]
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-3


@gpu
@pytest.mark.parametrize("out_f32", [False, True])
def test_given_selection_with_invalid_ids_r16_d128(out_f32):
    # The prefill shape of the workloads (16 query heads per group, d = 128, bf16)
    # with a caller's selection holding ids past the cache, after the row's own
    # block and -1 padding in any position: those are ignored, the rest is exact
    # attention; fp32 or bf16 output, lse
    msa = _msa()
    s = synth.Shape(2, 333, 1400, 900, 32, 2, 128, 64, 7, dtype="bf16")
    x, xh = _inputs(s, 12)
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    good = orc.index_select(f["q_idx"], f["k_idx"], s.topk, s.q_offset)
    bad = good.copy()
    nb = (s.kv_len + 127) // 128
    rng = np.random.default_rng(5)
    for b in range(s.batch):
        for g in range(s.groups):
            for i in range(s.q_len):
                row = [c for c in good[b, g, i] if c >= 0]
                L = (s.q_offset + i) // 128
                extra = [nb + 3, 10 ** 6, L + 1] if L + 1 < nb else [nb + 3, 10 ** 6]
                row = row + extra[: s.topk - len(row)]
                rng.shuffle(row)
                bad[b, g, i, :len(row)] = row
                bad[b, g, i, len(row):] = -1
    out, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], torch.from_numpy(bad).cuda(), q_offset=s.q_offset,
                                   out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = orc.sparse_attention(f["q"], f["k"], f["v"], good, s.q_offset)
    assert _max_err(out, ref) <= TOL["bf16"]
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-3


@gpu
@pytest.mark.parametrize("case", ["large_logits", "all_scores_very_negative"])
def test_extreme_logit_ranges(case):
    # Scaled scores of several hundred, and rows whose every score is far below
    # zero (exp of the raw scores would overflow or underflow in fp32): the block
    # maxima subtracted inside the kernels keep both exact against the oracle.
    msa = _msa()
    s = synth.Shape(1, 200, 700, 500, 16, 1, 128, 32, 4, dtype="bf16")
    x, xh = _inputs(s, 13)
    q = xh["q"].float()
    k = xh["k"].float()
    if case == "large_logits":
        q = q * 40.0                     # scaled scores of a few hundred (exponents far above 64)
    else:
        k[:] = k[:, :, :1, :]            # every key the same vector k0 ...
        q[:] = -12.0 * k[:, :, :1, :].squeeze(1).unsqueeze(1).expand_as(q)  # ... and q = -12 k0: all scores << 0
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    f["q"], f["k"] = synth.as_f64(qb), synth.as_f64(kb)
    sel = orc.index_select(f["q_idx"], f["k_idx"], s.topk, s.q_offset)
    out, lse = msa.sparse_attn_fwd(qb.cuda(), kb.cuda(), x["v"], torch.from_numpy(sel).cuda(), q_offset=s.q_offset,
                                   return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = orc.sparse_attention(f["q"], f["k"], f["v"], sel, s.q_offset)
    o = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    # Such peaked rows put the whole weight on one or two keys, so an output can be
    # a single value of v (|v| up to ~4.5 here) where one bf16 half-ulp is 2^-9 |v|.
    # The partial state and the output are both rounded to bf16: two half-ulps on
    # top of the bar that holds for the workloads' rows (whose outputs are averages).
    bound = TOL["bf16"] + 2.0 * 2.0 ** -9 * np.abs(ref)
    assert bool((np.abs(o - ref) <= bound).all()), float(np.abs(o - ref).max())
    rel = np.abs(lse.cpu().numpy() - ref_lse) / np.maximum(1.0, np.abs(ref_lse))
    assert float(rel.max()) <= 1e-4

"""GPU parity for caches of unequal length and paged caches (the *_kvcache calls).

Each sequence's cache is read back on the host (dense slices, or
oracle.page_gather over the page pool) and the oracle runs msa_forward_varlen on
it.  Selections must match bit for bit, outputs within the bf16 tolerance
(max-abs 2e-2), lse within 1e-3; rows that precede their cache must give -1
selections, zero output and lse = -inf.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import msa_oracle as orc

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


def _f64(s: synth.Shape, name: str, t: torch.Tensor) -> np.ndarray:
    if s.fp8 and name in ("k", "v", "k_idx"):
        scale = {"k": s.k_scale, "v": s.v_scale, "k_idx": 1.0}[name]
        return orc.dequantize_e4m3(synth.codes(t), scale)
    return synth.as_f64(t)


def _compare(out, sel, lse, ref_out, ref_sel, ref_lse):
    sg = sel.cpu().numpy()
    bad = np.argwhere((sg != ref_sel).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} selection rows differ, first {bad[:5].tolist()}"
    og = out.float().cpu().numpy()
    err = float(np.abs(og - ref_out).max())
    assert err <= TOL, err
    lg = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert float(np.abs(lg[fin] - ref_lse[fin]).max(initial=0.0)) <= 1e-3


def _scales(s):
    return dict(k_scale=s.k_scale, v_scale=s.v_scale) if s.fp8 else {}


DENSE_CASES = [
    # (lens, S_q, Hq, Hkv, d, D, k, cache)
    ([1, 700, 2999, 3000, 1500], 1, 64, 4, 128, 128, 16, "native"),     # decode
    ([2, 130, 2048, 3000], 4, 32, 4, 128, 64, 8, "native"),             # speculative rows; one precedes its cache
    ([1, 700, 2999, 3000, 1500], 1, 64, 4, 128, 128, 32, "fp8"),
    ([1, 9000, 12000, 8190], 1, 64, 4, 128, 128, 64, "native"),        # k = 64 (the wide top lists)
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[6]}-{c[7]}")
def test_dense_varlen(case):
    msa = _msa()
    lens, S_q, Hq, Hkv, d, D, k, cache = case
    alloc = max(lens) + 17
    s = synth.Shape(len(lens), S_q, alloc, 0, Hq, Hkv, d, D, k, cache=cache,
                    k_scale=0.03 if cache == "fp8" else 1.0, v_scale=0.02 if cache == "fp8" else 1.0)
    print(f"dense varlen {case}", flush=True)
    xh = synth.host_inputs(s, 41 + k)
    x = {n: t.cuda() for n, t in xh.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, seq_lens=sl,
                                    return_sel=True, return_lse=True, **_scales(s))
    torch.cuda.synchronize()
    f = {n: _f64(s, n, t) for n, t in xh.items()}
    ks = [f["k"][b, :, :n] for b, n in enumerate(lens)]
    vs = [f["v"][b, :, :n] for b, n in enumerate(lens)]
    kis = [f["k_idx"][b, :n] for b, n in enumerate(lens)]
    ref = orc.msa_forward_varlen(f["q"], ks, vs, f["q_idx"], kis, k)
    _compare(out, sel, lse, *ref)


PAGED_CASES = [
    # (lens, S_q, Hq, Hkv, d, D, k, cache, spare)
    ([130, 4000, 1, 2048, 5000, 777], 1, 64, 4, 128, 128, 16, "native", 7),
    ([130, 4000, 1, 2048, 5000, 777], 1, 64, 4, 128, 128, 16, "fp8", 3),
    ([4096, 129, 3000, 5120], 2, 16, 2, 64, 32, 8, "native", 0),
    ([5000, 333, 4097], 1, 32, 4, 128, 128, 32, "native", 11),
    ([1000, 2600], 300, 32, 2, 128, 128, 8, "native", 5),    # a chunk of 300 rows: the gathered path
    ([2600, 1800, 700], 200, 16, 4, 128, 64, 12, "fp8", 2),
    ([9000, 130, 12000], 1, 32, 4, 128, 128, 48, "fp8", 5),   # k = 48 over pages
    ([9500, 6000], 160, 16, 2, 128, 128, 64, "native", 3),    # k = 64, a chunk of rows
]


def _paged(case, seed):
    lens, S_q, Hq, Hkv, d, D, k, cache, spare = case
    max_pages = -(-max(lens) // 128) + 2
    s = synth.Shape(len(lens), S_q, max_pages * 128, 0, Hq, Hkv, d, D, k, cache=cache,
                    k_scale=0.04 if cache == "fp8" else 1.0, v_scale=0.03 if cache == "fp8" else 1.0)
    table, P = synth.page_table_for(lens, max_pages, spare, seed)
    xh = synth.paged_inputs(s, P, seed)
    return s, table, P, xh


def _paged_oracle(s, lens, table, xh):
    f = {n: _f64(s, n, t) for n, t in xh.items()}
    ks = [orc.page_gather(f["k"], table[b], n) for b, n in enumerate(lens)]
    vs = [orc.page_gather(f["v"], table[b], n) for b, n in enumerate(lens)]
    kis = [orc.page_gather(f["k_idx"], table[b], n) for b, n in enumerate(lens)]
    return orc.msa_forward_varlen(f["q"], ks, vs, f["q_idx"], kis, s.topk)


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: f"{len(c[0])}seq-{c[1]}-{c[6]}-{c[7]}")
def test_paged(case):
    msa = _msa()
    lens = case[0]
    print(f"paged {case}", flush=True)
    s, table, P, xh = _paged(case, 60 + case[1] + case[6])
    x = {n: t.cuda() for n, t in xh.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pt = torch.from_numpy(table).cuda()
    out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, seq_lens=sl,
                                    page_table=pt, return_sel=True, return_lse=True, **_scales(s))
    torch.cuda.synchronize()
    _compare(out, sel, lse, *_paged_oracle(s, lens, table, xh))
    # the two branches on their own give the same
    sel2 = msa.index_select_kvcache(x["q_idx"], x["k_idx"], s.topk, seq_lens=sl, page_table=pt)
    out2 = msa.sparse_attn_fwd_kvcache(x["q"], x["k"], x["v"], sel2, seq_lens=sl, page_table=pt, **_scales(s))
    torch.cuda.synchronize()
    assert torch.equal(sel2, sel) and torch.equal(out2, out)


def test_equal_lengths_match_the_plain_call():
    msa = _msa()
    s = synth.Shape(3, 4, 2000, 1996, 32, 4, 128, 128, 16)
    x = {n: t.cuda() for n, t in synth.host_inputs(s, 8).items()}
    a = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], 16, q_offset=1996, return_sel=True, return_lse=True)
    sl = torch.full((3,), 2000, dtype=torch.int32, device="cuda")
    b = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], 16, seq_lens=sl, return_sel=True,
                        return_lse=True)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_unmapped_pages_are_skipped_safely():
    # sequence 0: a middle block's page id is negative; sequence 1: its local
    # block's page id is past the pool.  Neither is read; the other sequences are
    # unaffected and every output stays finite.
    msa = _msa()
    case = ([4000, 3000, 2500, 900], 1, 64, 4, 128, 128, 16, "native", 4)
    lens = case[0]
    s, table, P, xh = _paged(case, 77)
    ref = _paged_oracle(s, lens, table, xh)
    bad = table.copy()
    bad[0, 5] = -5
    L1 = (lens[1] - 1) // 128
    bad[1, L1] = 10 ** 6
    x = {n: t.cuda() for n, t in xh.items()}
    out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk,
                                    seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                    page_table=torch.from_numpy(bad).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    og, sg, lg = out.float().cpu().numpy(), sel.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert not (sg[0] == 5).any()           # the unmapped block is never ranked
    assert (sg[1, :, 0] == L1).any(axis=-1).all()  # the local block is still listed (it is forced)
    for b in (2, 3):
        assert np.array_equal(sg[b], ref[1][b])
        assert float(np.abs(og[b] - ref[0][b]).max()) <= TOL


@pytest.mark.timeout(900)
def test_paged_decode_workload_every_sequence():
    # every sequence: its selection against the oracle's (ranked over its own cache,
    # read out of the page pool) and its output against the oracle's main branch
    from fullsize import check_selection, sparse_kv
    msa = _msa()
    wid = 7
    s = synth.WORKLOADS[wid]
    print(f"workload {synth.WORKLOAD_NAMES[wid]}: inputs", flush=True)
    x, lens, table, P = synth.paged_workload(wid, device="cuda")
    sl = torch.from_numpy(lens).cuda()
    pt = torch.from_numpy(table).cuda()
    out, sel = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, seq_lens=sl, page_table=pt,
                               kv_len=s.kv_len, return_sel=True)
    torch.cuda.synchronize()
    print("  forward done; oracle on every sequence", flush=True)
    sg = sel.cpu().numpy()
    og = out.float().cpu().numpy()
    ref_sel = np.empty_like(sg)
    worst = 0.0
    for b in range(s.batch):
        n = int(lens[b])
        nb = -(-n // 128)
        pg = torch.from_numpy(table[b, :nb].astype(np.int64)).cuda()
        kib = orc.page_gather(_f64(s, "k_idx", x["k_idx"].index_select(0, pg).cpu()), np.arange(nb), n)
        qi = _f64(s, "q_idx", x["q_idx"][b:b + 1].cpu())
        # query row i of a cache of n tokens sits at n - S_q + i
        ref_sel[b] = orc.index_select(qi, kib[None], s.topk, n - s.q_len, 128)[0]
        # the cache as the oracle reads it: the sequence's pages in logical order, only the selected ones filled
        kseq = x["k"].index_select(0, pg).permute(1, 0, 2, 3).reshape(s.num_kv_heads, nb * 128, s.head_dim)
        vseq = x["v"].index_select(0, pg).permute(1, 0, 2, 3).reshape(s.num_kv_heads, nb * 128, s.head_dim)
        blocks = [ref_sel[b, g].reshape(-1) for g in range(s.groups)]
        kb = sparse_kv(s, "k", kseq, blocks, n)
        vb = sparse_kv(s, "v", vseq, blocks, n)
        ro, _ = orc.sparse_attention(_f64(s, "q", x["q"][b:b + 1].cpu()), kb, vb, ref_sel[b:b + 1], n - s.q_len, 128)
        worst = max(worst, float(np.abs(og[b:b + 1] - ro).max()))
    check_selection(synth.WORKLOAD_NAMES[wid], sg, ref_sel)
    print(f"  outputs of all {s.batch} sequences: max abs err {worst:.3e}", flush=True)
    assert worst <= TOL


@pytest.mark.parametrize("B,paged", [(256, True), (300, True), (256, False), (300, False)])
def test_decode_batch_around_the_in_kernel_unit_limit(B, paged):
    # few-row index form with per-sequence lengths: up to 256 sequences each wave
    # derives its key-split unit from the lengths; beyond that a unit list is built
    msa = _msa()
    rng = np.random.default_rng(B + 7 * paged)
    lens = [int(v) for v in rng.integers(1, 2500, B)]
    lens[:4] = [1, 128, 129, 2499]
    print(f"decode batch B={B} paged={paged}", flush=True)
    if paged:
        case = (lens, 1, 4, 2, 64, 32, 8, "native", 5)
        s, table, P, xh = _paged(case, 900 + B)
        pt = torch.from_numpy(table).cuda()
    else:
        s = synth.Shape(B, 1, max(lens) + 3, 0, 4, 2, 64, 32, 8)
        xh = synth.host_inputs(s, 900 + B)
        pt = None
    x = {n: t.cuda() for n, t in xh.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, seq_lens=sl,
                                    page_table=pt, return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    if paged:
        ref = _paged_oracle(s, lens, table, xh)
    else:
        f = {n: synth.as_f64(t) for n, t in xh.items()}
        ks = [f["k"][b, :, :n] for b, n in enumerate(lens)]
        vs = [f["v"][b, :, :n] for b, n in enumerate(lens)]
        kis = [f["k_idx"][b, :n] for b, n in enumerate(lens)]
        ref = orc.msa_forward_varlen(f["q"], ks, vs, f["q_idx"], kis, s.topk)
    _compare(out, sel, lse, *ref)


@pytest.mark.parametrize("paged", [True, False])
def test_decode_batch_of_short_caches_one_split(paged):
    # every cache under 15 blocks: with contiguous caches one key split per sequence,
    # so every sequence is one unit, also those whose rows rank no block (the paged
    # pool's table is two pages longer than the longest cache: two splits)
    msa = _msa()
    rng = np.random.default_rng(31 + paged)
    lens = [int(v) for v in rng.integers(1, 1900, 64)]
    lens[:3] = [1, 128, 1900]
    print(f"short caches paged={paged}", flush=True)
    if paged:
        s, table, P, xh = _paged((lens, 1, 64, 4, 128, 128, 16, "native", 3), 950)
        pt = torch.from_numpy(table).cuda()
    else:
        s = synth.Shape(64, 1, max(lens) + 5, 0, 64, 4, 128, 128, 16)
        xh = synth.host_inputs(s, 950)
        pt = None
    x = {n: t.cuda() for n, t in xh.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, seq_lens=sl,
                                    page_table=pt, return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    if paged:
        ref = _paged_oracle(s, lens, table, xh)
    else:
        f = {n: synth.as_f64(t) for n, t in xh.items()}
        ref = orc.msa_forward_varlen(f["q"], [f["k"][b, :, :n] for b, n in enumerate(lens)],
                                     [f["v"][b, :, :n] for b, n in enumerate(lens)], f["q_idx"],
                                     [f["k_idx"][b, :n] for b, n in enumerate(lens)], s.topk)
    _compare(out, sel, lse, *ref)

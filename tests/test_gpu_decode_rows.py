"""GPU parity of the decode rows form (one workgroup per (b, i, g) row).

Decode calls with bf16 queries and at least 256 (b, i, g) rows run the whole
main branch in one kernel: the merge of the index kernel's split lists (msa_fwd),
attention over the selected blocks with a running softmax, and the row's output
and lse.  Every case here has at least 256 rows, so that form is the one that
runs.  Against the fp64 oracle: selections bit for bit, outputs within 2e-2
(bf16 outputs) or 1e-2 (fp32 outputs of bf16 inputs), lse within 1e-3.
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


def _f64(s, name, t):
    if s.fp8 and name in ("k", "v", "k_idx"):
        scale = {"k": s.k_scale, "v": s.v_scale, "k_idx": 1.0}[name]
        return orc.dequantize_e4m3(synth.codes(t), scale)
    return synth.as_f64(t)


def _scales(s):
    return dict(k_scale=s.k_scale, v_scale=s.v_scale) if s.fp8 else {}


def _check(out, sel, lse, ref_out, ref_sel, ref_lse, tol=TOL):
    sg = sel.cpu().numpy()
    bad = np.argwhere((sg != ref_sel).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} selection rows differ, first {bad[:5].tolist()}"
    err = float(np.abs(out.float().cpu().numpy() - ref_out).max())
    assert err <= tol, err
    lg = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert float(np.abs(lg[fin] - ref_lse[fin]).max(initial=0.0)) <= 1e-3


ROW_CASES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k, cache)
    (64, 1, 3000, 2999, 64, 4, 128, 128, 16, "native"),   # the decode shape, short caches
    (64, 1, 12000, 11999, 16, 4, 128, 128, 64, "native"),  # k = 64: lists of 63 per lane half
    (64, 1, 5000, 4999, 64, 4, 128, 128, 16, "fp8"),       # FP8 K, V and index keys
    (16, 4, 3000, 2996, 64, 4, 128, 64, 8, "native"),      # four query rows per sequence
    (128, 1, 1500, 1499, 64, 2, 64, 32, 4, "native"),      # d = 64, r = 32
    (64, 1, 900, 899, 4, 4, 128, 32, 32, "native"),        # r = 1, k above the visible blocks
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "x".join(str(v) for v in c))
def test_rows_form_fwd_and_given_selection(case):
    msa = _msa()
    B, S_q, S_k, qo, Hq, Hkv, d, D, k, cache = case
    assert B * S_q * Hkv >= 256
    s = synth.Shape(B, S_q, S_k, qo, Hq, Hkv, d, D, k, cache=cache,
                    k_scale=0.03 if cache == "fp8" else 1.0, v_scale=0.02 if cache == "fp8" else 1.0)
    print(f"rows case {case}", flush=True)
    xh = synth.host_inputs(s, 90 + k + d)
    x = {n: t.cuda() for n, t in xh.items()}
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=qo, return_sel=True,
                            return_lse=True, **_scales(s))
    torch.cuda.synchronize()
    f = {n: _f64(s, n, t) for n, t in xh.items()}
    ref_out, ref_sel, ref_lse = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], k, qo)
    _check(out, sel, lse, ref_out, ref_sel, ref_lse)
    # the main branch alone from the same selection (the selection is read, not merged)
    out2, lse2 = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], sel, q_offset=qo, return_lse=True, **_scales(s))
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


def test_rows_form_fp32_output():
    msa = _msa()
    s = synth.Shape(64, 1, 2500, 2499, 32, 4, 128, 64, 8)
    xh = synth.host_inputs(s, 5)
    x = {n: t.cuda() for n, t in xh.items()}
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, q_offset=s.q_offset,
                            out_dtype=torch.float32, return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], s.topk, s.q_offset)
    # fp32 output of bf16 inputs: P enters the PV product in bf16
    _check(out, sel, lse, *ref, tol=1e-2)


def test_rows_form_varlen_rows_before_the_cache():
    # 64 caches of unequal length, 4 query rows each; two caches are shorter than
    # the rows, whose leading rows precede their cache
    msa = _msa()
    lens = [2, 3] + [int(v) for v in np.random.default_rng(8).integers(4, 3000, 62)]
    alloc = max(lens) + 5
    s = synth.Shape(len(lens), 4, alloc, 0, 32, 4, 128, 128, 8)
    xh = synth.host_inputs(s, 77)
    x = {n: t.cuda() for n, t in xh.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, seq_lens=sl,
                                    return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ks = [f["k"][b, :, :n] for b, n in enumerate(lens)]
    vs = [f["v"][b, :, :n] for b, n in enumerate(lens)]
    kis = [f["k_idx"][b, :n] for b, n in enumerate(lens)]
    ref = orc.msa_forward_varlen(f["q"], ks, vs, f["q_idx"], kis, s.topk)
    _check(out, sel, lse, *ref)
    og = out.float().cpu().numpy()
    assert (og[0, :2] == 0).all() and (og[1, :1] == 0).all()  # rows before the cache give zeros


def test_rows_form_in_a_graph():
    msa = _msa()
    s = synth.Shape(64, 1, 3000, 2999, 64, 4, 128, 128, 16)
    names = ("q", "k", "v", "q_idx", "k_idx")
    static = {n: t.cuda() for n, t in synth.host_inputs(s, 1).items()}

    def call():
        return msa.fwd(*(static[n] for n in names), s.topk, q_offset=s.q_offset, return_sel=True,
                       return_lse=True)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g, sel_g, lse_g = call()
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = synth.host_inputs(s, 200 + rep)
        for n in names:
            static[n].copy_(fresh[n].cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out_g.clone(), sel_g.clone(), lse_g.clone())
        ref = call()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep}"


@pytest.mark.parametrize("seed", range(8))
def test_rows_form_random_shapes(seed):
    # seeded sweep over shapes that take the rows form (>= 256 rows, few queries
    # per (b, g, block)): head layout, dims, k up to 64, FP8 caches, unequal lengths
    msa = _msa()
    rng = np.random.default_rng(5000 + seed)
    G = int(rng.choice([2, 4]))
    r = int(rng.choice([1, 2, 4, 8, 16, 32]))
    d = int(rng.choice([64, 128]))
    D = int(rng.choice([32, 64, 128]))
    k = int(rng.integers(1, 65))
    S_q = int(rng.choice([1, 1, 2]))
    B = 256 // (G * S_q) + int(rng.integers(0, 16))
    cache = "fp8" if seed % 4 == 3 else "native"
    S_k = int(rng.integers(600, 6000)) + 128 * k  # most rows rank more blocks than they keep
    varlen = seed % 3 == 1
    s = synth.Shape(B, S_q, S_k, 0 if varlen else S_k - S_q, G * r, G, d, D, k, cache=cache,
                    k_scale=0.03 if cache == "fp8" else 1.0, v_scale=0.02 if cache == "fp8" else 1.0)
    print(f"rows sweep {s} varlen={varlen}", flush=True)
    xh = synth.host_inputs(s, 6000 + seed)
    x = {n: t.cuda() for n, t in xh.items()}
    f = {n: _f64(s, n, t) for n, t in xh.items()}
    if varlen:
        lens = [int(v) for v in rng.integers(1, S_k + 1, B)]
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, seq_lens=sl,
                                        return_sel=True, return_lse=True, **_scales(s))
        ks = [f["k"][b, :, :n] for b, n in enumerate(lens)]
        vs = [f["v"][b, :, :n] for b, n in enumerate(lens)]
        kis = [f["k_idx"][b, :n] for b, n in enumerate(lens)]
        torch.cuda.synchronize()
        ref = orc.msa_forward_varlen(f["q"], ks, vs, f["q_idx"], kis, k)
    else:
        out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=s.q_offset,
                                return_sel=True, return_lse=True, **_scales(s))
        torch.cuda.synchronize()
        ref = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], k, s.q_offset)
    _check(out, sel, lse, *ref)

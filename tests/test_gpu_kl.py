"""GPU parity of the KL-alignment teacher (msa_kl_teacher_fwd) with the oracle.

The forward runs first (its selection must match the oracle's bit for bit);
its sel and lse then feed the teacher.  The teacher's KL and index lse are
checked against oracle.kl_teacher in fp64 on the same (exact) inputs, within
1e-3 + 1e-4 |ref| (fp32 arithmetic over up to k * 128 tokens; index scores of
the integer inputs reach a few hundred).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import msa_oracle as orc

pytestmark = pytest.mark.gpu


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


def _f64(s, name, t):
    if s.fp8 and name in ("k", "v", "k_idx"):
        scale = {"k": s.k_scale, "v": s.v_scale, "k_idx": 1.0}[name]
        return orc.dequantize_e4m3(synth.codes(t), scale)
    return synth.as_f64(t)


def _close(got, ref, atol=1e-3, rtol=1e-4):
    g = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = np.abs(g[fin] - ref[fin])
    worst = float((err - rtol * np.abs(ref[fin])).max(initial=0.0))
    assert worst <= atol, f"max excess {worst}, max abs err {float(err.max(initial=0.0))}"


KL_SHAPES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k, dtype, cache, index_scale)
    (1, 1000, 1000, 0, 32, 2, 128, 128, 5, "bf16", "native", 1.0),      # gathered path, r = 16
    (2, 513, 1500, 987, 16, 4, 128, 64, 6, "bf16", "native", 0.37),     # r = 4
    (3, 1, 2000, 1999, 64, 4, 128, 128, 16, "bf16", "native", 1.0),     # decode: one item per entry
    (1, 640, 640, 0, 32, 1, 64, 32, 32, "f32", "native", 1.0),          # r = 32, k = 32
    (2, 300, 900, 600, 8, 8, 64, 32, 4, "f32", "native", 0.5),          # r = 1
    (2, 400, 2400, 1700, 16, 4, 128, 128, 12, "bf16", "fp8", 1.0),      # FP8 caches
    (1, 300, 9000, 8700, 16, 2, 128, 128, 64, "bf16", "native", 1.0),   # k = 64
]


@pytest.mark.parametrize("shape", KL_SHAPES, ids=lambda s: "x".join(str(v) for v in s))
def test_kl_teacher_small(shape):
    msa = _msa()
    B, S_q, S_k, qo, Hq, Hkv, d, D, k, dt, cache, isc = shape
    lo, hi = (-8, 8) if dt == "f32" else (-4, 4)
    s = synth.Shape(B, S_q, S_k, qo, Hq, Hkv, d, D, k, dtype=dt, idx_lo=lo, idx_hi=hi, cache=cache,
                    k_scale=0.03 if cache == "fp8" else 1.0, v_scale=0.02 if cache == "fp8" else 1.0)
    print(f"kl case {shape}", flush=True)
    xh = synth.host_inputs(s, 500 + S_q + k)
    x = {n: t.cuda() for n, t in xh.items()}
    sc = dict(k_scale=s.k_scale, v_scale=s.v_scale) if s.fp8 else {}
    _, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=qo, return_sel=True,
                          return_lse=True, **sc)
    kl, ilse = msa.kl_teacher_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], sel, lse, q_offset=qo,
                                  index_scale=isc, k_scale=s.k_scale if s.fp8 else None, return_idx_lse=True)
    torch.cuda.synchronize()
    f = {n: _f64(s, n, t) for n, t in xh.items()}
    ref_sel = orc.index_select(f["q_idx"], f["k_idx"], k, qo)
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    ref_kl, ref_ilse = orc.kl_teacher(f["q"], f["k"], f["q_idx"], f["k_idx"], ref_sel, qo, index_scale=isc)
    _close(kl, ref_kl)
    _close(ilse, ref_ilse)


def test_kl_vanishes_when_the_index_scores_are_the_main_scores():
    # one head per group and one group, q_idx = q, k_idx = k, index_scale = the
    # main scale: the index distribution is the teacher, so KL is 0 up to rounding
    msa = _msa()
    s = synth.Shape(2, 700, 1800, 1100, 1, 1, 128, 128, 8)
    xh = synth.host_inputs(s, 91)
    x = {n: t.cuda() for n, t in xh.items()}
    q_idx = x["q"].clone()                 # [B, S_q, 1, d] doubles as [B, S_q, G, D_idx]
    k_idx = x["k"][:, 0].contiguous()      # [B, S_k, d]
    _, sel, lse = msa.fwd(x["q"], x["k"], x["v"], q_idx, k_idx, 8, q_offset=1100, return_sel=True,
                          return_lse=True)
    kl = msa.kl_teacher_fwd(x["q"], x["k"], q_idx, k_idx, sel, lse, q_offset=1100,
                            index_scale=1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    assert float(kl.abs().max()) < 1e-4


def test_kl_teacher_paged_decode():
    msa = _msa()
    lens = [130, 4000, 1, 2048, 5000, 777]
    max_pages = 42
    s = synth.Shape(len(lens), 1, max_pages * 128, 0, 64, 4, 128, 128, 16)
    table, P = synth.page_table_for(lens, max_pages, 5, 12)
    xh = synth.paged_inputs(s, P, 12)
    x = {n: t.cuda() for n, t in xh.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pt = torch.from_numpy(table).cuda()
    _, sel, lse = msa.fwd_kvcache(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], 16, seq_lens=sl, page_table=pt,
                                  return_sel=True, return_lse=True)
    kl, ilse = msa.kl_teacher_fwd_kvcache(x["q"], x["k"], x["q_idx"], x["k_idx"], sel, lse, seq_lens=sl,
                                          page_table=pt, return_idx_lse=True)
    torch.cuda.synchronize()
    f = {n: _f64(s, n, t) for n, t in xh.items()}
    sg = sel.cpu().numpy()
    for b, n in enumerate(lens):
        kb = orc.page_gather(f["k"], table[b], n)[None]
        kib = orc.page_gather(f["k_idx"], table[b], n)[None]
        ref_kl, ref_ilse = orc.kl_teacher(f["q"][b:b + 1], kb, f["q_idx"][b:b + 1], kib, sg[b:b + 1], n - 1)
        _close(kl[b:b + 1], ref_kl)
        _close(ilse[b:b + 1], ref_ilse)

"""GPU parity of the main branch's backward (msa_sparse_attn_bwd) with the oracle.

The forward runs first; its selection (checked against the oracle's bit for
bit), output and lse feed the backward with a seeded bf16 output gradient.
dq, dk and dv are compared with oracle.sparse_attention_bwd (fp64, exact
inputs); the error bound is 1e-2 of each gradient's largest magnitude: P and dS
enter the MFMA products in bf16, the dQ partials are bf16, and rowsum(dO * O)
uses the forward's bf16 output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import msa_oracle as orc

pytestmark = pytest.mark.gpu
REL = 1e-2


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


def _rel_err(got: torch.Tensor, ref: np.ndarray) -> float:
    g = got.cpu().numpy().astype(np.float64)
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))


BWD_SHAPES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k)
    (1, 700, 700, 0, 32, 2, 128, 64, 5),         # r = 16
    (2, 300, 1500, 1200, 16, 4, 128, 32, 6),     # r = 4, queries at an offset
    (1, 260, 900, 640, 8, 8, 64, 32, 4),         # r = 1, d = 64
    (1, 400, 400, 0, 32, 1, 64, 32, 3),          # r = 32
    (2, 3, 2000, 1997, 64, 4, 128, 128, 16),     # few queries per block
    (1, 1000, 1000, 0, 64, 4, 128, 128, 16),     # the pages' shape, every block of every query
    (1, 300, 9000, 8700, 16, 2, 128, 128, 64),   # k = 64: the dQ combine in two rounds of 32 slots
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(str(v) for v in s))
def test_backward_matches_oracle(shape):
    msa = _msa()
    B, S_q, S_k, qo, Hq, Hkv, d, D, k = shape
    s = synth.Shape(B, S_q, S_k, qo, Hq, Hkv, d, D, k)
    print(f"bwd case {shape}", flush=True)
    xh = synth.host_inputs(s, 700 + S_q + k)
    x = {n: t.cuda() for n, t in xh.items()}
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=qo, return_sel=True,
                            return_lse=True)
    g = torch.Generator().manual_seed(17 + S_q)
    dout_h = torch.randn(out.shape, generator=g).to(torch.bfloat16)
    dq, dk, dv = msa.sparse_attn_bwd(x["q"], x["k"], x["v"], sel, out, lse, dout_h.cuda(), q_offset=qo)
    torch.cuda.synchronize()
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    ref_sel = orc.index_select(f["q_idx"], f["k_idx"], k, qo)
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    rq, rk, rv = orc.sparse_attention_bwd(f["q"], f["k"], f["v"], ref_sel, synth.as_f64(dout_h), qo)
    eq, ek, ev = _rel_err(dq, rq), _rel_err(dk, rk), _rel_err(dv, rv)
    print(f"  relative errors dq {eq:.2e} dk {ek:.2e} dv {ev:.2e}", flush=True)
    assert eq <= REL and ek <= REL and ev <= REL
    # keys that no query attends get exactly zero
    used = np.zeros((B, Hkv, S_k), dtype=bool)
    for b in range(B):
        for g_ in range(Hkv):
            for i in range(S_q):
                used[b, g_, orc.token_set(ref_sel[b, g_, i], qo + i, 128)] = True
    assert float(dk.cpu().numpy()[~used].__abs__().max(initial=0.0)) == 0.0
    assert float(dv.cpu().numpy()[~used].__abs__().max(initial=0.0)) == 0.0

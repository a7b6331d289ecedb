"""GPU parity of the KL teacher and the backward at the 32K x 2 prefill size.

The forward, msa_kl_teacher_fwd and msa_sparse_attn_bwd run exactly as the
benchmark runs them (same shapes, same entry points, a seeded bf16 output
gradient).  The oracle checks what it can compute row by row:

* KL and index lse of sampled (b, i) rows, all groups (1e-3 + 1e-4 |ref|, as
  at small sizes);
* dq of sampled rows: a row's dq depends on its own token set only, so the
  oracle's backward runs on that row alone (relative 1e-2 of the largest
  reference magnitude, as at small sizes);
* dk and dv of the last block of each sequence: no later query exists, so only
  the block's own 128 query rows select it, and the oracle's backward over
  those rows gives the block's exact gradients.

The selections the oracle uses are its own (index_select on the sampled rows),
checked bit for bit against the GPU's first.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import msa_oracle as orc

pytestmark = pytest.mark.gpu
WID = 3
REL = 1e-2


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def fwd_state():
    msa = _msa()
    s = synth.WORKLOADS[WID]
    print(f"workload {synth.WORKLOAD_NAMES[WID]}: inputs", flush=True)
    x = synth.inputs_for(s, WID, device="cuda")
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, q_offset=s.q_offset,
                            return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    print("  forward done", flush=True)
    yield msa, s, x, out, sel, lse
    del x, out, sel, lse
    torch.cuda.empty_cache()


def _row_inputs(x, b, i0, i1):
    """Host fp64 copies of query rows [i0, i1) of sequence b and its whole K, V, k_idx."""
    sl = slice(i0, i1)
    return (_f64(x["q"][b:b + 1, sl]), _f64(x["q_idx"][b:b + 1, sl]))


def _oracle_sel(q_idx_rows, k_idx_b, s, i0):
    return orc.index_select(q_idx_rows, k_idx_b, s.topk, i0)


def test_kl_teacher_32k_b2_sampled(fwd_state):
    msa, s, x, out, sel, lse = fwd_state
    kl, ilse = msa.kl_teacher_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], sel, lse, q_offset=s.q_offset,
                                  return_idx_lse=True)
    torch.cuda.synchronize()
    print("  KL teacher done", flush=True)
    assert bool(torch.isfinite(kl).all()) and float(kl.min()) >= -1e-3  # KL >= 0 up to rounding
    rng = np.random.default_rng(31)
    rows = [(int(b), int(i)) for b, i in zip(rng.integers(0, 2, 12), rng.integers(0, s.q_len, 12))]
    rows += [(0, 0), (1, 2047), (1, s.q_len - 1)]
    for b in (0, 1):
        k_b = _f64(x["k"][b:b + 1])
        ki_b = _f64(x["k_idx"][b:b + 1])
        for bb, i in rows:
            if bb != b:
                continue
            q_r, qi_r = _row_inputs(x, b, i, i + 1)
            ref_sel = _oracle_sel(qi_r, ki_b, s, i)
            assert np.array_equal(sel[b:b + 1, :, i:i + 1].cpu().numpy(), ref_sel), (b, i)
            ref_kl, ref_ilse = orc.kl_teacher(q_r, k_b, qi_r, ki_b, ref_sel, i)
            got_kl = kl[b, :, i].cpu().numpy().astype(np.float64)
            got_il = ilse[b, :, i].cpu().numpy().astype(np.float64)
            for got, ref in ((got_kl, ref_kl[0, :, 0]), (got_il, ref_ilse[0, :, 0])):
                err = np.abs(got - ref) - 1e-4 * np.abs(ref)
                assert float(err.max()) <= 1e-3, (b, i, got, ref)
    print(f"  {len(rows)} rows match", flush=True)


def test_backward_32k_b2_sampled(fwd_state):
    msa, s, x, out, sel, lse = fwd_state
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    dout = torch.randn(out.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = msa.sparse_attn_bwd(x["q"], x["k"], x["v"], sel, out, lse, dout, q_offset=s.q_offset)
    torch.cuda.synchronize()
    print("  backward done", flush=True)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    rng = np.random.default_rng(37)
    rows = [(int(b), int(i)) for b, i in zip(rng.integers(0, 2, 10), rng.integers(0, s.q_len, 10))]
    rows += [(0, 5), (1, s.q_len - 1)]
    S, Bk = s.q_len, s.block_size
    for b in (0, 1):
        k_b, v_b, ki_b = _f64(x["k"][b:b + 1]), _f64(x["v"][b:b + 1]), _f64(x["k_idx"][b:b + 1])
        # dq of sampled rows, one row at a time
        for bb, i in rows:
            if bb != b:
                continue
            q_r, qi_r = _row_inputs(x, b, i, i + 1)
            ref_sel = _oracle_sel(qi_r, ki_b, s, i)
            assert np.array_equal(sel[b:b + 1, :, i:i + 1].cpu().numpy(), ref_sel), (b, i)
            rq, _, _ = orc.sparse_attention_bwd(q_r, k_b, v_b, ref_sel, _f64(dout[b:b + 1, i:i + 1]), i)
            got = dq[b, i].cpu().numpy().astype(np.float64)
            e = float(np.abs(got - rq[0, 0]).max() / max(np.abs(rq).max(), 1e-30))
            assert e <= REL, (b, i, e)
        # dk, dv of the last block: only its own 128 rows select it
        i0 = S - Bk
        q_r, qi_r = _row_inputs(x, b, i0, S)
        ref_sel = _oracle_sel(qi_r, ki_b, s, i0)
        assert np.array_equal(sel[b:b + 1, :, i0:S].cpu().numpy(), ref_sel)
        _, rk, rv = orc.sparse_attention_bwd(q_r, k_b, v_b, ref_sel, _f64(dout[b:b + 1, i0:S]), i0)
        for got_t, ref in ((dk, rk), (dv, rv)):
            got = got_t[b, :, i0:S].cpu().numpy().astype(np.float64)
            r_blk = ref[0, :, i0:S]
            e = float(np.abs(got - r_blk).max() / max(np.abs(r_blk).max(), 1e-30))
            print(f"  b={b} last block relative error {e:.2e}", flush=True)
            assert e <= REL
    print(f"  {len(rows)} dq rows and both last blocks match", flush=True)

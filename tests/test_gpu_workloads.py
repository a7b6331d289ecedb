"""GPU parity at the full workload sizes the benchmark times.

The whole forward runs exactly as in the benchmark (same shapes, same entry
point).  Selections are checked bit for bit against the fp64 oracle on sampled
rows, and on every row against properties that hold at any size (local block
present, ids visible, ascending, count min(k, L+1), -1 padding).  Outputs are
checked on the sampled rows within the bf16 tolerance (max-abs 2e-2).
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


def _selection_properties(sel: torch.Tensor, s: synth.Shape):
    """Every row: ascending ids, local block last, count min(k, L+1), -1 padding."""
    B, G, S_q, k = sel.shape
    t = s.q_offset + torch.arange(S_q, device=sel.device)
    L = (t // s.block_size).view(1, 1, S_q)
    valid = sel >= 0
    count = valid.sum(-1)
    assert torch.equal(count, torch.minimum(torch.full_like(count, k), (L + 1).expand(B, G, S_q)))
    # valid entries first, then padding
    pos = torch.arange(k, device=sel.device).view(1, 1, 1, k)
    assert torch.equal(valid, pos < count.unsqueeze(-1))
    last = sel.gather(-1, (count - 1).clamp(min=0).unsqueeze(-1)).squeeze(-1)
    assert torch.equal(last, L.expand(B, G, S_q).to(sel.dtype))  # the local block, largest id
    d = sel[..., 1:] - sel[..., :-1]
    both = valid[..., 1:] & valid[..., :-1]
    assert bool((d[both] > 0).all())  # strictly ascending, so no duplicates


def _host_f32(t):
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


def _run_and_check(s: synth.Shape, wid: int, rows, sub_batch=None):
    msa = _msa()
    print(f"workload {synth.WORKLOAD_NAMES[wid]}: inputs", flush=True)
    x = synth.inputs_for(s, wid, device="cuda")
    out, sel = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk, q_offset=s.q_offset,
                       return_sel=True)
    torch.cuda.synchronize()
    print("  forward done; properties", flush=True)
    _selection_properties(sel, s)
    bsel = sorted({b for b, _ in rows})
    # host copies of the sampled sequences only, as float64/float32 (exact upcasts)
    idx = torch.tensor(bsel, device="cuda")
    q_idx = x["q_idx"].index_select(0, idx).float().cpu().numpy().astype(np.float64)
    k_idx = x["k_idx"].index_select(0, idx).float().cpu().numpy().astype(np.float64)
    k = _host_f32(x["k"].index_select(0, idx))
    v = _host_f32(x["v"].index_select(0, idx))
    q = _host_f32(x["q"].index_select(0, idx))
    remap = {b: j for j, b in enumerate(bsel)}
    sub_rows = [(remap[b], i) for b, i in rows]
    print(f"  oracle on {len(rows)} rows", flush=True)
    ref_out, ref_sel, _ = orc.msa_forward(q, k, v, q_idx, k_idx, s.topk, s.q_offset, s.block_size, rows=sub_rows)
    sg = sel.index_select(0, idx).cpu().numpy()
    og = _host_f32(out.index_select(0, idx))
    worst = 0.0
    for b, i in sub_rows:
        np.testing.assert_array_equal(sg[b, :, i], ref_sel[b, :, i], err_msg=f"selection row b={b} i={i}")
        worst = max(worst, float(np.abs(og[b, i] - ref_out[b, i]).max()))
    print(f"  max abs err {worst:.3e}", flush=True)
    assert worst <= TOL


def test_workload_32k_b2_sampled():
    s = synth.WORKLOADS[3]
    rng = np.random.default_rng(3)
    rows = [(int(b), int(i)) for b, i in zip(rng.integers(0, 2, 40), rng.integers(0, s.q_len, 40))]
    rows += [(0, 0), (1, 127), (1, 128), (0, s.q_len - 1), (1, s.q_len - 1)]
    _run_and_check(s, 3, rows)


def test_workload_decode_128k_b64_sampled():
    s = synth.WORKLOADS[4]
    rows = [(b, 0) for b in (0, 17, 42, 63)]
    _run_and_check(s, 4, rows)


def test_workload_chunked_prefill_1m_sampled():
    s = synth.WORKLOADS[5]
    rng = np.random.default_rng(5)
    rows = [(0, int(i)) for i in rng.integers(0, s.q_len, 12)] + [(0, 0), (0, s.q_len - 1)]
    _run_and_check(s, 5, rows)

"""The workspace cap (msa_shape.workspace_cap_mib): query rows processed in chunks.

A capped call runs the same kernels on every query row (the gather, the KV-outer
attention and the combine, chunk by chunk over one partial-state region), so its
results must equal those of the uncapped call bit for bit; the uncapped results
are checked against the oracle by the other parity tests, and here also on
sampled rows.  msa_workspace_size must shrink with the cap.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import msa_oracle as orc

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 2e-2}


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


def _fwd(msa, s: synth.Shape, x, cap_mib: int):
    """msa_fwd through the C ABI with the given cap: (out, sel, lse, workspace bytes)."""
    dev = x["q"].device
    sh = msa.make_shape(s.batch, s.q_len, s.kv_len, s.q_offset, s.num_q_heads, s.num_kv_heads, s.head_dim,
                        s.index_dim, s.topk, s.torch_dtype, workspace_cap_mib=cap_mib)
    n = msa.workspace_size(sh, msa.OP_FWD)
    wsr = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    ws = wsr[(-wsr.data_ptr()) % 256:][:n]
    out = torch.empty((s.batch, s.q_len, s.num_q_heads, s.head_dim), dtype=s.torch_dtype, device=dev)
    sel = torch.empty((s.batch, s.groups, s.q_len, s.topk), dtype=torch.int32, device=dev)
    lse = torch.empty((s.batch, s.num_q_heads, s.q_len), dtype=torch.float32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = msa.lib().msa_fwd(ctypes.byref(sh), p(x["q"]), p(x["k"]), p(x["v"]), p(x["q_idx"]), p(x["k_idx"]), p(out),
                           p(sel), p(lse), p(ws), ctypes.c_size_t(n),
                           ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == 0, msa.lib().msa_last_error()
    torch.cuda.synchronize()
    return out, sel, lse, n


CASES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k, dtype, caps in MiB)
    (2, 1000, 1500, 500, 32, 2, 128, 64, 8, "bf16", [1, 2, 40]),    # chunks of 7, 15 and 256 rows
    (1, 1024, 1024, 0, 8, 2, 64, 32, 4, "f32", [1, 3]),             # the fp32 path
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:10])))
def test_capped_calls_equal_the_uncapped_call(case):
    msa = _msa()
    *dims, dt, caps = case
    lo, hi = (-8, 8) if dt == "f32" else (-4, 4)
    s = synth.Shape(*dims, dtype=dt, idx_lo=lo, idx_hi=hi)
    print(f"capped workspace case {case}", flush=True)
    xh = synth.host_inputs(s, 61)
    x = {n: t.cuda() for n, t in xh.items()}
    out0, sel0, lse0, n0 = _fwd(msa, s, x, 0)
    f = {n: synth.as_f64(t) for n, t in xh.items()}
    rows = [(b, i) for b in range(s.batch) for i in (0, 1, s.q_len // 2, s.q_len - 1)]
    ref_out, ref_sel, _ = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], s.topk, s.q_offset,
                                          rows=rows)
    og = out0.float().cpu().numpy()
    for b, i in rows:
        assert np.array_equal(sel0[b, :, i].cpu().numpy(), ref_sel[b, :, i])
        assert float(np.abs(og[b, i] - ref_out[b, i]).max()) <= TOL[dt]
    for cap in caps:
        out, sel, lse, n = _fwd(msa, s, x, cap)
        print(f"  cap {cap} MiB: workspace {n} bytes (uncapped {n0})", flush=True)
        assert n < n0
        assert torch.equal(sel, sel0)
        assert torch.equal(out, out0)
        assert torch.equal(lse, lse0)


def test_capped_call_with_more_blocks_than_the_lds_histogram():
    # a cache of more than 16384 blocks: the gather counts and scatters through
    # global atomics, also chunk by chunk
    msa = _msa()
    s = synth.Shape(1, 4200, 2_200_000, 2_200_000 - 4200, 16, 1, 128, 32, 16)  # about 4 queries per block: gathered
    print("long cache: inputs", flush=True)
    x = synth.inputs_for(s, 62, device="cuda", on_device_limit=0)
    out0, sel0, lse0, n0 = _fwd(msa, s, x, 0)
    out, sel, lse, n = _fwd(msa, s, x, 64)
    print(f"  workspace {n} bytes capped, {n0} uncapped", flush=True)
    assert n < n0
    assert torch.equal(sel, sel0) and torch.equal(out, out0) and torch.equal(lse, lse0)
    # sampled rows against the oracle (selection over the 2.2M-token index cache)
    idx = [0, 2100, 4199]
    qi = synth.as_f64(x["q_idx"][:, idx])
    ki = synth.as_f64(x["k_idx"])
    for j, i in enumerate(idx):
        ref = orc.index_select(qi[:, j:j + 1], ki, s.topk, s.q_offset + i, s.block_size)
        assert np.array_equal(sel0[:, :, i:i + 1].cpu().numpy(), ref)

"""msa_fwd_noalloc (the forward in the library's fixed scratch, for callers that
cannot allocate) against msa_fwd with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the selections must be equal
bit for bit and the outputs and lse within the bf16 tolerance (they are in fact
expected to be identical).  Two calls in a row, the second on a smaller input,
show that nothing left in the shared scratch by one call leaks into the next.
A shape whose workspace exceeds the scratch is refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


def _pair(msa, s: synth.Shape, seed: int):
    print(f"no-alloc case {s}", flush=True)
    x = {n: t.cuda() for n, t in synth.host_inputs(s, seed).items()}
    args = (x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], s.topk)
    ref_out, ref_sel, ref_lse = msa.fwd(*args, q_offset=s.q_offset, return_sel=True, return_lse=True)
    ws_free = msa.workspace_size(msa.make_shape(s.batch, s.q_len, s.kv_len, s.q_offset, s.num_q_heads,
                                                s.num_kv_heads, s.head_dim, s.index_dim, s.topk, s.torch_dtype),
                                 msa.OP_FWD)
    assert 0 < ws_free <= msa.noalloc_scratch_bytes()
    out = torch.full_like(ref_out, float("nan"))
    sel = torch.full_like(ref_sel, -7)
    lse = torch.full_like(ref_lse, float("nan"))
    msa.fwd_noalloc(*args, q_offset=s.q_offset, out=out, sel=sel, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref_sel)
    err = float((out.float() - ref_out.float()).abs().max())
    lerr = float((lse - ref_lse).abs().max())
    print(f"  sel equal, out max diff {err:.3e}, lse max diff {lerr:.3e}, identical "
          f"{bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse))}", flush=True)
    assert err <= TOL and lerr <= 1e-3
    return out, sel


def test_noalloc_matches_workspace_call_twice_second_smaller():
    msa = _msa()
    big = synth.Shape(2, 1024, 1536, 512, 16, 2, 64, 64, 4)      # prefill rows, several tiles, two sequences
    small = synth.Shape(1, 300, 700, 400, 16, 2, 64, 64, 4)      # then a smaller one in the same scratch
    _pair(msa, big, 71)
    _pair(msa, small, 72)


def test_noalloc_decode_then_smaller_decode():
    msa = _msa()
    _pair(msa, synth.Shape(64, 1, 8192, 8191, 64, 4, 128, 128, 16), 73)
    _pair(msa, synth.Shape(8, 1, 3000, 2999, 64, 4, 128, 128, 16), 74)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    msa = _msa()
    L = msa.lib()
    s = msa.make_shape(1, 32768, 32768, 0, 64, 4, 128, 128, 16, torch.bfloat16)
    need = msa.workspace_size(s, msa.OP_FWD)
    assert need > msa.noalloc_scratch_bytes()
    out = torch.full((4,), 3.0, device="cuda")
    p = ctypes.c_void_p(out.data_ptr())  # never read: the call returns before any launch
    st = L.msa_fwd_noalloc(ctypes.byref(s), p, p, p, p, p, p, None, None, None)
    assert st == -3  # MSA_ERR_WORKSPACE
    assert b"msa_fwd_noalloc holds" in L.msa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full((4,), 3.0, device="cuda"))

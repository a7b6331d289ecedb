"""GPU parity with the caches (k, v, k_idx) stored as OCP FP8 E4M3.

The oracle decodes the very bytes the GPU reads (e4m3_to_f64, exact) and
applies the per-tensor scales in float64; the attention it then computes is the
same definition as for bf16 caches.  Every E4M3 value is a bf16 value, so the
tolerances are the bf16 ones: selections bit for bit, outputs max-abs 2e-2,
lse 1e-3.
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


def _rows(t: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    # fp8 tensors are indexed through their bytes
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).index_select(0, idx).view(torch.float8_e4m3fn)
    return t.index_select(0, idx)


def _oracle_inputs(s: synth.Shape, xh):
    return {
        "q": synth.as_f64(xh["q"]),
        "q_idx": synth.as_f64(xh["q_idx"]),
        "k": orc.dequantize_e4m3(synth.codes(xh["k"]), s.k_scale),
        "v": orc.dequantize_e4m3(synth.codes(xh["v"]), s.v_scale),
        "k_idx": orc.e4m3_to_f64(synth.codes(xh["k_idx"])),
    }


FP8_SHAPES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k, k_scale, v_scale)
    (1, 1000, 1000, 0, 32, 2, 128, 128, 5, 1.0, 1.0),            # gathered (KV-outer) path
    (2, 513, 1500, 987, 16, 4, 128, 64, 6, 6.0 / 448, 5.5 / 448),
    (3, 1, 2000, 1999, 64, 4, 128, 128, 16, 6.0 / 448, 5.5 / 448),  # decode path
    (2, 4, 3000, 2990, 32, 1, 64, 32, 8, 0.05, 0.02),             # few queries, d = 64
    (1, 700, 6000, 5300, 16, 2, 64, 32, 24, 0.05, 0.02),          # k > 16
    (2, 300, 9000, 8700, 32, 2, 128, 128, 32, 1.0, 0.5),          # k = 32, several key splits
    (64, 1, 5000, 4999, 64, 4, 128, 128, 16, 6.0 / 448, 5.5 / 448),  # many decode sequences
]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "x".join(f"{v:.3g}" for v in s))
def test_fp8_fwd_small(shape):
    msa = _msa()
    B, S_q, S_k, qo, Hq, Hkv, d, D, k, ks, vs = shape
    s = synth.Shape(B, S_q, S_k, qo, Hq, Hkv, d, D, k, cache="fp8", k_scale=ks, v_scale=vs)
    print(f"fp8 case {shape}", flush=True)
    xh = synth.host_inputs(s, 300 + B + S_q + k)
    x = {n: t.cuda() for n, t in xh.items()}
    out, sel, lse = msa.fwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], k, q_offset=qo,
                            return_sel=True, return_lse=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    f = _oracle_inputs(s, xh)
    ref_out, ref_sel, ref_lse = orc.msa_forward(f["q"], f["k"], f["v"], f["q_idx"], f["k_idx"], k, qo)
    bad = np.argwhere((sel.cpu().numpy() != ref_sel).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} selection rows differ, first {bad[:5].tolist()}"
    err = float(np.abs(out.float().cpu().numpy() - ref_out).max())
    assert err <= TOL, err
    lerr = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    assert lerr <= 1e-3, lerr


def test_fp8_index_select_and_given_selection_f32_out():
    msa = _msa()
    s = synth.Shape(2, 600, 2400, 1700, 16, 4, 128, 128, 12, cache="fp8", k_scale=0.03, v_scale=0.07)
    xh = synth.host_inputs(s, 17)
    x = {n: t.cuda() for n, t in xh.items()}
    f = _oracle_inputs(s, xh)
    sel = msa.index_select(x["q_idx"], x["k_idx"], s.topk, q_offset=s.q_offset)
    torch.cuda.synchronize()
    ref_sel = orc.index_select(f["q_idx"], f["k_idx"], s.topk, s.q_offset)
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    out, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], sel, q_offset=s.q_offset, out_dtype=torch.float32,
                                   return_lse=True, k_scale=s.k_scale, v_scale=s.v_scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = orc.sparse_attention(f["q"], f["k"], f["v"], ref_sel, s.q_offset)
    assert float(np.abs(out.cpu().numpy() - ref_out).max()) <= 1e-2
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-3


def test_fp8_every_code_widens_exactly():
    # One cached token and one query at position 0: the softmax weight is
    # exactly 1, so out = v_scale * v[token 0] and lse = scale * k_scale * q.k[0].
    # With 4 sequences x 2 groups x 128 dims every byte value sits once in v and
    # once in k (the two NaN codes replaced by 0); one-hot queries read each k
    # value back through lse.
    msa = _msa()
    B, G, r, d = 4, 2, 32, 128
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    perm = np.random.default_rng(0).permutation(256).astype(np.uint8)
    kc = codes.reshape(G, d)                                   # group g, dim m: code g*128 + m
    vc = codes[perm].reshape(G, d)
    k8 = np.broadcast_to(kc, (B, G, d)).reshape(B, G, 1, d).copy()
    v8 = np.broadcast_to(vc, (B, G, d)).reshape(B, G, 1, d).copy()
    q = np.zeros((B, 1, G * r, d), np.float32)
    for b in range(B):
        for h in range(G * r):
            q[b, 0, h, b * r + h % r] = 1.0                   # sequence b, head h reads dim b*32 + h%32
    to8 = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
    sel = torch.zeros((B, G, 1, 1), dtype=torch.int32, device="cuda")
    k_scale, v_scale, scale = 0.75, 0.25, 0.5  # v_scale a power of two: out stays exact
    out, lse = msa.sparse_attn_fwd(torch.from_numpy(q).to(torch.bfloat16).cuda(), to8(k8), to8(v8), sel,
                                   scale=scale, out_dtype=torch.float32, return_lse=True,
                                   k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    vals_v = orc.e4m3_to_f64(vc)
    vals_k = orc.e4m3_to_f64(kc)
    for b in range(B):
        for h in range(G * r):
            g = h // r
            assert np.array_equal(out[b, 0, h], v_scale * vals_v[g]), (b, h)  # bit-exact widening of v
            want = scale * k_scale * vals_k[g, b * r + h % r]
            # fp32 rounding of the folded scale and of the log2/ln conversions only
            assert abs(lse[b, h, 0] - want) <= 1e-6 + 2e-6 * abs(want), (b, h, lse[b, h, 0], want)


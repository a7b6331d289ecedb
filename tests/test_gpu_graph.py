"""The forward captured in a HIP graph (torch.cuda.graph over the ctypes call).

The library only enqueues kernels on the caller's stream (no host round trip,
no allocation, no memset), so a whole msa_fwd call can be captured and
replayed.  Each replay runs on new inputs copied into the captured buffers,
with eager work and synchronisations between replays, and must equal an eager
call on the same inputs bit for bit (the forward is deterministic).
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _msa():
    import block_sparse_attention_idx_amd as msa
    msa.lib()
    return msa


CASES = [
    # (B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, k): the gathered prefill path and the decode path
    (1, 700, 700, 0, 32, 2, 128, 64, 8),
    (4, 1, 3000, 2999, 64, 4, 128, 128, 16),
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(str(v) for v in s))
def test_forward_graph_replays_match_eager(shape):
    msa = _msa()
    B, S_q, S_k, qo, Hq, Hkv, d, D, k = shape
    s = synth.Shape(B, S_q, S_k, qo, Hq, Hkv, d, D, k)
    names = ("q", "k", "v", "q_idx", "k_idx")
    static = {n: t.cuda() for n, t in synth.host_inputs(s, 1).items()}

    def call():
        return msa.fwd(*(static[n] for n in names), k, q_offset=qo, return_sel=True, return_lse=True)

    call()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g, sel_g, lse_g = call()
    torch.cuda.synchronize()

    for rep in range(3):
        fresh = synth.host_inputs(s, 100 + rep)
        for n in names:
            static[n].copy_(fresh[n].cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out_g.clone(), sel_g.clone(), lse_g.clone())
        ref = call()  # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep}"

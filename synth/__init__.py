"""Seeded synthetic inputs for the MSA forward pass.

This module only draws random tensors of the right shapes, dtypes and value
distributions.  It holds none of the attention arithmetic: both the CPU oracle
(through the tests and the bench's CPU leg) and the HIP library (through the
Python binding) receive what these functions return.

Workloads (the MSA pages fix Bk = 128 and k = 16 with a GQA layout of 64 query
heads over 4 KV heads; see "Hvad er MSA i praksis" on the snilld.dk MSA page and
the 原因分析 section of the page "Substantial numerical differences with Minimax
MSA attention vs Minimax's Reference"):

* Q, K, V are standard normal; in bf16 workloads they are drawn in fp32 and
  rounded to bf16 (round-to-nearest-even).
* The index query/key tensors hold small integers drawn uniformly from an
  inclusive range (-8..8 for the fp32 workload, -4..4 otherwise), stored exactly
  in the workload dtype, so every index score is an exact integer in fp32.
* FP8 caches (``cache="fp8"``): K and V are the same standard-normal fp32 draws
  divided by the per-tensor dequantisation scale (``k_scale``, ``v_scale``),
  clamped to the E4M3 range +-448 and rounded to OCP FP8 E4M3 by torch's cast;
  the integer index keys are stored exactly in E4M3.  Q and the index queries
  stay bf16.

Two generators exist:

* ``host_inputs``: numpy PCG64 seeded by
  ``SeedSequence([0x4D5341, workload_id, tensor_id, b])`` (tensor ids 0 q, 1 k,
  2 v, 3 q_idx, 4 k_idx; ``b`` the batch/sequence index), drawn per sequence in
  the C order of the tensor's layout.  Used for every workload that fits
  comfortably in host memory.
* ``device_inputs``: torch's device generator (Philox) seeded from the same
  tuple, for the workloads whose inputs are tens of GiB (128K decode cache, 1M
  context) where host generation would dominate the run.  The oracle then reads
  the very same values copied back to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

SEED_ROOT = 0x4D5341  # "MSA"

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "q_idx": 3, "k_idx": 4}
CACHE_TENSORS = ("k", "v", "k_idx")
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Shape:
    """Problem shape.  Layouts: q/out [B,S_q,Hq,d], k/v [B,Hkv,S_k,d],
    q_idx [B,S_q,G,D_idx], k_idx [B,S_k,D_idx], sel int32 [B,G,S_q,k]."""

    batch: int
    q_len: int
    kv_len: int
    q_offset: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    topk: int
    block_size: int = 128
    dtype: str = "bf16"  # "f32" or "bf16"
    idx_lo: int = -4
    idx_hi: int = 4
    cache: str = "native"  # "native" (k, v, k_idx in dtype) or "fp8" (OCP E4M3)
    k_scale: float = 1.0   # dequantisation scales of an fp8 k / v cache
    v_scale: float = 1.0

    @property
    def groups(self) -> int:
        return self.num_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def fp8(self) -> bool:
        return self.cache == "fp8"

    def tensor_dtype(self, name: str) -> torch.dtype:
        if self.fp8 and name in CACHE_TENSORS:
            return torch.float8_e4m3fn
        return self.torch_dtype

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The five workloads.  Names say what they are.
WORKLOADS: Dict[int, Shape] = {
    1: Shape(1, 1024, 1024, 0, 8, 2, 64, 32, 4, dtype="f32", idx_lo=-8, idx_hi=8),
    2: Shape(1, 8192, 8192, 0, 64, 4, 128, 128, 16),
    3: Shape(2, 32768, 32768, 0, 64, 4, 128, 128, 16),
    4: Shape(64, 1, 131072, 131071, 64, 4, 128, 128, 16),
    5: Shape(1, 4096, 1048576, 1044480, 64, 4, 128, 128, 16),
    # the decode workload with its caches in FP8 (scales ~ 6 sigma / 448)
    6: Shape(64, 1, 131072, 131071, 64, 4, 128, 128, 16, cache="fp8", k_scale=6.0 / 448, v_scale=5.5 / 448),
    # decode over 64 caches of unequal length in a shuffled page pool (PAGED below);
    # kv_len is the longest possible cache, positions come from the lengths
    7: Shape(64, 1, 131072, 0, 64, 4, 128, 128, 16),
}

# Paged workloads: cache lengths log-uniform over [lo, hi] (seeded by the
# workload id), pages shuffled in a pool with `spare` pages of no sequence.
PAGED = {7: dict(lo=4096, hi=131072, spare=64)}

WORKLOAD_NAMES = {
    1: "prefill_1k_fp32",
    2: "prefill_8k_bf16",
    3: "prefill_32k_b2_bf16",
    4: "decode_128k_b64_bf16",
    5: "chunked_prefill_1m_q4096_bf16",
    6: "decode_128k_b64_fp8",
    7: "decode_paged_varlen_b64_bf16",
}


def _seed(workload: int, tensor: str, b: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([SEED_ROOT, workload, TENSOR_IDS[tensor], b])


def _per_seq_shape(s: Shape, tensor: str):
    if tensor in ("q",):
        return (s.q_len, s.num_q_heads, s.head_dim)
    if tensor in ("k", "v"):
        return (s.num_kv_heads, s.kv_len, s.head_dim)
    if tensor == "q_idx":
        return (s.q_len, s.groups, s.index_dim)
    if tensor == "k_idx":
        return (s.kv_len, s.index_dim)
    raise KeyError(tensor)


def _to_storage(s: Shape, tensor: str, x: torch.Tensor) -> torch.Tensor:
    """fp32 draws to the tensor's storage dtype (fp8 caches: scaled, clamped)."""
    if s.fp8 and tensor in ("k", "v"):
        scale = s.k_scale if tensor == "k" else s.v_scale
        x = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return x.to(s.tensor_dtype(tensor))


def _host_draw(s: Shape, workload: int, tensor: str, b: int) -> torch.Tensor:
    rng = np.random.Generator(np.random.PCG64(_seed(workload, tensor, b)))
    shp = _per_seq_shape(s, tensor)
    if tensor in ("q", "k", "v"):
        x = rng.standard_normal(size=shp, dtype=np.float32)
    else:
        x = rng.integers(s.idx_lo, s.idx_hi + 1, size=shp, dtype=np.int32).astype(np.float32)
    return _to_storage(s, tensor, torch.from_numpy(x))


def host_inputs(s: Shape, workload: int = 0) -> Dict[str, torch.Tensor]:
    """All five inputs as CPU tensors in the workload dtype (PCG64 recipe)."""
    out = {}
    for name in ("q", "k", "v", "q_idx", "k_idx"):
        out[name] = torch.stack([_host_draw(s, workload, name, b) for b in range(s.batch)])
    return out


def _device_seed(workload: int, tensor: str, b: int) -> int:
    ss = _seed(workload, tensor, b)
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def device_inputs(s: Shape, workload: int, device="cuda", names=("q", "k", "v", "q_idx", "k_idx")
                  ) -> Dict[str, torch.Tensor]:
    """The inputs (all five by default) generated on the device (Philox), per sequence."""
    out = {}
    for name in names:
        shp = _per_seq_shape(s, name)
        t = torch.empty((s.batch,) + shp, dtype=s.tensor_dtype(name), device=device)
        for b in range(s.batch):
            g = torch.Generator(device=device)
            g.manual_seed(_device_seed(workload, name, b))
            if name in ("q", "k", "v"):
                # draw in fp32, round to the storage dtype; chunk to bound scratch
                flat = t[b].view(-1)
                n = flat.numel()
                step = 1 << 28
                for o in range(0, n, step):
                    m = min(step, n - o)
                    flat[o:o + m].copy_(_to_storage(s, name, torch.randn(m, generator=g, device=device,
                                                                         dtype=torch.float32)))
            else:
                t[b].copy_(_to_storage(s, name, torch.randint(s.idx_lo, s.idx_hi + 1, shp, generator=g,
                                                              device=device, dtype=torch.int32).float()))
        out[name] = t
    return out


def host_bytes(s: Shape) -> int:
    e = 4 if s.dtype == "f32" else 2
    ec = 1 if s.fp8 else e
    return (e * (2 * s.batch * s.q_len * s.num_q_heads * s.head_dim + s.batch * s.q_len * s.groups * s.index_dim)
            + ec * (2 * s.batch * s.num_kv_heads * s.kv_len * s.head_dim + s.batch * s.kv_len * s.index_dim))


def inputs_for(s: Shape, workload: int = 0, device: Optional[str] = None,
               on_device_limit: int = 1 << 30) -> Dict[str, torch.Tensor]:
    """Host recipe when the inputs are small, device recipe above ``on_device_limit``
    bytes (only when a device is given)."""
    if device is not None and host_bytes(s) > on_device_limit:
        return device_inputs(s, workload, device)
    x = host_inputs(s, workload)
    if device is not None:
        x = {n: t.to(device) for n, t in x.items()}
    return x


def as_f64(t) -> np.ndarray:
    """Exact upcast of a stored fp32/bf16 tensor (or array) to a float64 array.
    FP8 tensors are refused: their bytes go to the oracle's decoder (codes())."""
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu")
        if t.dtype == torch.float8_e4m3fn:
            raise TypeError("fp8 tensor: pass codes(t) to the oracle's e4m3 decoder")
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


# ---- caches of unequal length, paged caches ---------------------------------

POOL_MARK = 0x504F4F4C  # "POOL": seed word of a whole page pool


def varlen_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded cache lengths, log-uniform over [lo, hi] (int32 [batch])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 0x4C454E, seed])))
    x = np.exp(rng.uniform(np.log(lo), np.log(hi + 1), size=batch)).astype(np.int64)
    return np.clip(x, lo, hi).astype(np.int32)


def page_table_for(seq_lens, max_pages: int, spare: int = 0, seed: int = 0, block_size: int = 128):
    """A shuffled page pool: the logical blocks of every sequence get distinct
    pages in random order; entries past a sequence's blocks are -1.  ``spare``
    pages belong to no sequence.  Returns (table int32 [B, max_pages], num_pages)."""
    need = [-(-int(n) // block_size) for n in seq_lens]
    if max(need, default=0) > max_pages:
        raise ValueError("a sequence needs more than max_pages pages")
    P = sum(need) + spare
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 0x504147, seed])))
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((len(need), max_pages), -1, dtype=np.int32)
    o = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[o:o + nb]
        o += nb
    return table, P


def _pool_shape(s: Shape, tensor: str, num_pages: int):
    if tensor in ("k", "v"):
        return (num_pages, s.num_kv_heads, s.block_size, s.head_dim)
    return (num_pages, s.block_size, s.index_dim)


def paged_inputs(s: Shape, num_pages: int, workload: int = 0, device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """q and q_idx per sequence as in host_inputs; k, v [P, Hkv, 128, d] and
    k_idx [P, 128, D_idx] page pools, each drawn whole from one generator seeded
    by (workload, tensor, POOL_MARK), with the value recipes of the dense caches.
    On the host (PCG64) without a device, on the device (Philox) with one."""
    out = {}
    for name in ("q", "q_idx"):
        if device is None:
            out[name] = torch.stack([_host_draw(s, workload, name, b) for b in range(s.batch)])
        else:
            out[name] = device_inputs_one(s, workload, name, device)
    for name in ("k", "v", "k_idx"):
        shp = _pool_shape(s, name, num_pages)
        ss = np.random.SeedSequence([SEED_ROOT, workload, TENSOR_IDS[name], POOL_MARK])
        if device is None:
            rng = np.random.Generator(np.random.PCG64(ss))
            if name == "k_idx":
                x = rng.integers(s.idx_lo, s.idx_hi + 1, size=shp, dtype=np.int32).astype(np.float32)
            else:
                x = rng.standard_normal(size=shp, dtype=np.float32)
            out[name] = _to_storage(s, name, torch.from_numpy(x))
        else:
            g = torch.Generator(device=device)
            g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
            t = torch.empty(shp, dtype=s.tensor_dtype(name), device=device)
            flat = t.view(-1)
            step = 1 << 28
            for o in range(0, flat.numel(), step):
                m = min(step, flat.numel() - o)
                if name == "k_idx":
                    x = torch.randint(s.idx_lo, s.idx_hi + 1, (m,), generator=g, device=device,
                                      dtype=torch.int32).float()
                else:
                    x = torch.randn(m, generator=g, device=device, dtype=torch.float32)
                flat[o:o + m].copy_(_to_storage(s, name, x))
            out[name] = t
    return out


def paged_workload(workload: int, device: Optional[str] = None):
    """Inputs of a paged workload: (inputs, seq_lens int32 [B], page_table int32
    [B, kv_len / 128], num_pages)."""
    s = WORKLOADS[workload]
    cfg = PAGED[workload]
    lens = varlen_lengths(s.batch, cfg["lo"], cfg["hi"], seed=workload)
    table, P = page_table_for(lens, s.kv_len // s.block_size, cfg["spare"], seed=workload)
    return paged_inputs(s, P, workload, device), lens, table, P


def device_inputs_one(s: Shape, workload: int, name: str, device) -> torch.Tensor:
    """One per-sequence input (q or q_idx) drawn on the device as in device_inputs."""
    return device_inputs(s, workload, device, names=(name,))[name]


def codes(t: torch.Tensor) -> np.ndarray:
    """The raw bytes of an fp8 tensor as a uint8 array of the same shape."""
    return t.detach().to("cpu").view(torch.uint8).numpy()


def n_blocks(kv_len: int, block_size: int = 128) -> int:
    return int(math.ceil(kv_len / block_size))

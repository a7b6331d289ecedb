"""Benchmark of the MSA forward on one MI355X.

Prints ONE JSON line.  A step is one msa_fwd call (index branch: scores,
block max-pool, per-group Top-k; main branch: query gather, KV-outer sparse
attention, combine) over one batch of the prefill workload (B=2, S=32768,
Hq=64, Hkv=4, d=128, D_idx=128, Bk=128, k=16, bf16), inputs resident in HBM.
``value`` is the algorithmic TFLOP/s of the whole step (main + index branch
FLOPs, the masked half of the local block and the skipped blocks excluded).

``roofline`` is for the dominant kernel (the KV-outer attention kernel): its
algorithmic FLOPs per launch over its own average duration, timed with HIP
events recorded around that kernel on the stream it runs on.  The decode
workload (64 sequences x 128K cache) is reported beside it in GB/s of
algorithmic HBM bytes, with bf16 caches (``decode``), with FP8 E4M3 caches
(``decode_fp8``) and over 64 caches of unequal length (4K-128K tokens) in a
shuffled page pool (``decode_paged``).  ``kl_teacher`` and ``backward`` time the KL-alignment
teacher forward and the main branch's backward on the prefill workload, and ``extra`` the 8K and
1M-context prefill workloads (all skipped with --no-extra).  ``cpu_baseline`` times the fp64 CPU
oracle on a bounded sample of query rows of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--decode-steps 100]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MSA fwd TFLOP/s (prefill 32K/128K) + decode KV GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNELS = {"index_score": 1, "topk_merge": 2, "gather": 3, "attention": 4, "combine": 5}
KL_KERNELS = {"kl_teacher": 6, "kl_combine": 7}
BWD_KERNELS = {"bwd": 8, "bwd_combine": 9}


def main_branch_bytes(s: synth.Shape, sel: torch.Tensor) -> dict:
    """HBM bytes of one msa_sparse_attn_fwd call in the KV-outer form (gather,
    attention, combine), from the selection it runs on.  An edge is one
    selection entry (b, g, i, slot) that names a block; per edge the attention
    reads the query rows of the group (r*d*e) and writes a partial state
    (r*(d*e + 4)), which the combine reads back; per used (b, g, block) bucket
    the attention reads K and V once (2*Bk*d*c); the gather reads the selection
    twice and writes and reads one 4-byte entry per edge; the combine writes the
    output and the log-sum-exp."""
    e = 2 if s.dtype == "bf16" else 4
    c = 1 if s.fp8 else e
    r = s.num_q_heads // s.num_kv_heads
    valid = sel >= 0
    edges = int(valid.sum().item())
    nb = (s.kv_len + s.block_size - 1) // s.block_size
    used = torch.zeros((s.batch * s.groups * nb,), dtype=torch.bool, device=sel.device)
    bg = torch.arange(s.batch * s.groups, device=sel.device).view(s.batch, s.groups, 1, 1) * nb
    used[(sel.long() + bg)[valid]] = True
    buckets = int(used.sum().item())
    sel_entries = s.batch * s.groups * s.q_len * s.topk
    parts = {
        "query_gather": edges * r * s.head_dim * e,
        "partial_write": edges * r * (s.head_dim * e + 4),
        "partial_read": edges * r * (s.head_dim * e + 4),
        "kv_blocks": buckets * 2 * s.block_size * s.head_dim * c,
        "gather": 2 * sel_entries * 4 + 2 * edges * 4,
        "output": s.batch * s.q_len * s.num_q_heads * (s.head_dim * e + 4),
    }
    return {"edges": edges, "buckets": buckets, "bytes_per_edge": round(sum(parts.values()) / max(edges, 1), 1),
            "total": float(sum(parts.values())), "parts": parts}


def sparse_attn_leg(run, s: synth.Shape, flop_main: float, steps=10) -> dict:
    """msa_sparse_attn_fwd (gather + attention + combine) on a workload's selection,
    against the MFMA peak and against the HBM roofline of its modelled bytes."""
    ms = run.sparse_attn(steps)
    bm = main_branch_bytes(s, run.sel)
    tfl = flop_main / (ms * 1e-3) / 1e12
    gbs = bm["total"] / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "tflops": round(tfl, 2), "frac_of_mfma_peak": round(tfl / PEAK_BF16_TFLOPS, 4),
            "bytes": bm["total"], "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "hbm_floor_ms": round(bm["total"] / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
            "edges": bm["edges"], "buckets": bm["buckets"], "bytes_per_edge": bm["bytes_per_edge"],
            "bytes_by_part": bm["parts"]}


def index_select_leg(run, flop_index: float, steps=20) -> dict:
    """msa_index_select alone, called back to back (its inputs stay in the
    Infinity Cache between calls), against the MFMA peak; beside the in-step
    index kernel time, which follows the main branch's HBM-bound kernels."""
    ms = run.index_select(steps)
    tfl = flop_index / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "tflops": round(tfl, 2), "frac_of_mfma_peak": round(tfl / PEAK_BF16_TFLOPS, 4)}


class HipEvents:
    """Raw hipEvent_t pairs (the library records them around one kernel)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        """Elapsed time, or None when the events were never recorded (the kernel did not run)."""
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            self.hip.hipGetLastError()  # clear the error this query left behind
            return None
        return float(ms.value)

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def recorded_traffic(profile: str, source: str, key: str = "traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed counter summary under profiles/, or None when
    the kernel source has changed since those counters were taken (hash mismatch)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    src = os.path.join(ROOT, "block_sparse_attention_idx_amd", "csrc", source)
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines() if ": " in line)
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    if fields.get("source_sha256_16", "").strip() != digest or key not in fields:
        return None
    return float(fields[key])


def algorithmic_work(s: synth.Shape):
    """(main-branch FLOP, index-branch FLOP, decode HBM bytes) of one msa_fwd call.

    main:  4*d*Hq*B * sum_i [(n_sel(t)-1)*Bk + (t mod Bk) + 1], n_sel = min(k, L+1)
    index: 2*D_idx*G*B * sum_i L(t)*Bk           (only full blocks before L are scored)
    bytes: B*[S_k*D_idx*c + G*n_sel*Bk*d*c*2 + 2*Hq*d*e + G*D_idx*e + 4*G*k]
           (e bytes per query/output element, c per cache element: 1 for FP8 caches)
    """
    t = s.q_offset + np.arange(s.q_len, dtype=np.int64)
    L = t // s.block_size
    n_sel = np.minimum(s.topk, L + 1)
    toks = (n_sel - 1) * s.block_size + (t % s.block_size) + 1
    flop_main = 4.0 * s.head_dim * s.num_q_heads * s.batch * float(toks.sum())
    flop_index = 2.0 * s.index_dim * s.groups * s.batch * float((L * s.block_size).sum())
    e = 2 if s.dtype == "bf16" else 4
    c = 1 if s.fp8 else e
    nsel_last = int(n_sel[-1])
    bytes_dec = s.batch * (s.kv_len * s.index_dim * c + s.groups * nsel_last * s.block_size * s.head_dim * c * 2
                           + 2 * s.num_q_heads * s.head_dim * e + s.groups * s.index_dim * e + 4 * s.groups * s.topk)
    return flop_main, flop_index, float(bytes_dec)


def paged_decode_bytes(s: synth.Shape, lens) -> float:
    """Algorithmic bytes of one decode step over caches of lengths ``lens``: the
    decode formula with S_k replaced by each sequence's own length."""
    e = 2 if s.dtype == "bf16" else 4
    c = 1 if s.fp8 else e
    total = 0
    for n in np.asarray(lens, dtype=np.int64):
        n_sel = min(s.topk, (int(n) - 1) // s.block_size + 1)
        total += (int(n) * s.index_dim * c + s.groups * n_sel * s.block_size * s.head_dim * c * 2
                  + 2 * s.num_q_heads * s.head_dim * e + s.groups * s.index_dim * e + 4 * s.groups * s.topk)
    return float(total)


class Runner:
    """One workload on the GPU: inputs, outputs and workspace allocated once.
    Paged workloads run msa_fwd_kvcache over their page pool."""

    def __init__(self, msa, s: synth.Shape, wid: int):
        self.msa, self.s = msa, s
        self.cache = None
        if wid in synth.PAGED:
            self.x, self.lens, table, P = synth.paged_workload(wid, device="cuda")
            self.seq_lens = torch.from_numpy(self.lens).cuda()
            self.table = torch.from_numpy(table).cuda()
            self.cache = msa.MsaKvCache()
            self.cache.seq_lens = self.seq_lens.data_ptr()
            self.cache.page_table = self.table.data_ptr()
            self.cache.max_pages, self.cache.num_pages = table.shape[1], P
        else:
            self.x = synth.inputs_for(s, wid, device="cuda")
        dev = self.x["q"].device
        self.out = torch.empty((s.batch, s.q_len, s.num_q_heads, s.head_dim), dtype=s.torch_dtype, device=dev)
        self.sel = torch.empty((s.batch, s.groups, s.q_len, s.topk), dtype=torch.int32, device=dev)
        self.shape = msa.make_shape(s.batch, s.q_len, s.kv_len, s.q_offset, s.num_q_heads, s.num_kv_heads,
                                    s.head_dim, s.index_dim, s.topk, s.torch_dtype,
                                    cache_format=msa.CACHE_FP8_E4M3 if s.fp8 else msa.CACHE_NATIVE,
                                    k_scale=s.k_scale if s.fp8 else None, v_scale=s.v_scale if s.fp8 else None)
        self.L = msa.lib()
        cref = ctypes.byref(self.cache) if self.cache is not None else None
        n = self.L.msa_workspace_size_kvcache(ctypes.byref(self.shape), cref, msa.OP_FWD)
        self.ws_raw = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        off = (-self.ws_raw.data_ptr()) % 256
        self.ws = self.ws_raw[off:off + n]
        self.stream = torch.cuda.current_stream(dev)
        self.args = [ctypes.byref(self.shape), cref] + [ctypes.c_void_p(self.x[n_].data_ptr())
                                                         for n_ in ("q", "k", "v", "q_idx", "k_idx")]
        self.args += [ctypes.c_void_p(self.out.data_ptr()), ctypes.c_void_p(self.sel.data_ptr()), None,
                      ctypes.c_void_p(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel()),
                      ctypes.c_void_p(self.stream.cuda_stream)]

    def step(self):
        st = self.L.msa_fwd_kvcache(*self.args)
        if st != 0:
            raise RuntimeError(self.L.msa_last_error().decode())

    def layer_copies(self, n):
        """Argument lists of n more calls over copies of this workload's inputs (the
        same values in other buffers), as the same step of other layers would be."""
        copies = []
        for _ in range(n):
            xc = {k: t.clone() for k, t in self.x.items()}
            a = list(self.args)
            for j, name in enumerate(("q", "k", "v", "q_idx", "k_idx")):
                a[2 + j] = ctypes.c_void_p(xc[name].data_ptr())
            copies.append((xc, a))
        return copies

    def clean_time(self, steps, warmup, layers=()):
        """ms per step over exactly `steps` calls with nothing recorded between them:
        one event pair around the whole timed region, synchronised on both sides.
        (An event recorded between steps or around a kernel adds a few microseconds
        of its own, which would be charged to short decode steps.)  With `layers`
        (from layer_copies) consecutive calls take this workload's inputs and the
        copies in turn, so no call finds the previous call's K/V in the caches."""
        arglists = [self.args] + [a for _, a in layers]
        fn = self.L.msa_fwd_kvcache

        def call(n):
            if fn(*arglists[n % len(arglists)]) != 0:
                raise RuntimeError(self.L.msa_last_error().decode())

        for n in range(warmup):
            call(n)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for n in range(steps):
            call(n)
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def time_steps(self, steps, warmup, timed_kernel=None):
        """Returns (ms per step, list of per-step ms of timed_kernel or None).  The
        per-step times of the last call are kept in self.step_ms."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = HipEvents() if timed_kernel else None
        kev = [(ev.create(), ev.create()) for _ in range(steps)] if timed_kernel else None
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        marks[0].record(self.stream)
        for i in range(steps):
            if kev:
                self.L.msa_set_kernel_timer(KERNELS[timed_kernel], kev[i][0], kev[i][1])
            self.step()
            marks[i + 1].record(self.stream)
        torch.cuda.synchronize()
        self.L.msa_set_kernel_timer(0, None, None)
        total = marks[0].elapsed_time(marks[-1])
        self.step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
        per_kernel = None
        if kev:
            per_kernel = [ev.elapsed_ms(a, b) for a, b in kev]
            for a, b in kev:
                ev.destroy(a)
                ev.destroy(b)
        return total / steps, per_kernel

    def graph_time(self, steps, warmup=3):
        """ms per step when one msa_fwd call is captured in a HIP graph (on a
        stream of its own, default priority) and the graph is replayed."""
        gs = torch.cuda.Stream()
        args = list(self.args)
        args[-1] = ctypes.c_void_p(gs.cuda_stream)
        fn = self.L.msa_fwd_kvcache
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            for _ in range(warmup):
                if fn(*args) != 0:
                    raise RuntimeError(self.L.msa_last_error().decode())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            if fn(*args) != 0:
                raise RuntimeError(self.L.msa_last_error().decode())
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def kl_teacher(self, steps=10, warmup=2):
        """Time msa_kl_teacher_fwd on this workload's selection and lse: (ms per call,
        per-kernel ms).  One forward with lse first provides them."""
        s, msa = self.s, self.msa
        dev = self.x["q"].device
        lse = torch.empty((s.batch, s.num_q_heads, s.q_len), dtype=torch.float32, device=dev)
        fa = list(self.args)
        fa[9] = ctypes.c_void_p(lse.data_ptr())
        if self.L.msa_fwd_kvcache(*fa) != 0:
            raise RuntimeError(self.L.msa_last_error().decode())
        kl = torch.empty((s.batch, s.groups, s.q_len), dtype=torch.float32, device=dev)
        cref = ctypes.byref(self.cache) if self.cache is not None else None
        ka = [ctypes.byref(self.shape), cref] + [ctypes.c_void_p(self.x[n].data_ptr()) for n in ("q", "k", "q_idx", "k_idx")]
        ka += [ctypes.c_void_p(self.sel.data_ptr()), ctypes.c_void_p(lse.data_ptr()), ctypes.c_float(1.0),
               ctypes.c_void_p(kl.data_ptr()), None, ctypes.c_void_p(self.ws.data_ptr()),
               ctypes.c_size_t(self.ws.numel()), ctypes.c_void_p(self.stream.cuda_stream)]

        def call():
            if self.L.msa_kl_teacher_fwd_kvcache(*ka) != 0:
                raise RuntimeError(self.L.msa_last_error().decode())
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = HipEvents()
        per = {}
        for name, kid in KL_KERNELS.items():
            a, b = ev.create(), ev.create()
            self.L.msa_set_kernel_timer(kid, a, b)
            call()
            torch.cuda.synchronize()
            self.L.msa_set_kernel_timer(0, None, None)
            per[name] = ev.elapsed_ms(a, b)
            ev.destroy(a)
            ev.destroy(b)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(steps):
            call()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps, per

    def backward(self, steps=5, warmup=1):
        """Time msa_sparse_attn_bwd on this workload (selection, output and lse
        from one forward; a seeded bf16 output gradient): (ms per call, per-kernel ms)."""
        s, msa = self.s, self.msa
        dev = self.x["q"].device
        lse = torch.empty((s.batch, s.num_q_heads, s.q_len), dtype=torch.float32, device=dev)
        fa = list(self.args)
        fa[9] = ctypes.c_void_p(lse.data_ptr())
        if self.L.msa_fwd_kvcache(*fa) != 0:
            raise RuntimeError(self.L.msa_last_error().decode())
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        dout = torch.randn(self.out.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dq = torch.empty(self.out.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(self.x["k"].shape, dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)
        n = msa.workspace_size(self.shape, msa.OP_SPARSE_ATTN_BWD)
        wsr = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        ws = wsr[(-wsr.data_ptr()) % 256:][:n]
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        ba = [ctypes.byref(self.shape), ptr(self.x["q"]), ptr(self.x["k"]), ptr(self.x["v"]), ptr(self.sel),
              ptr(self.out), ptr(lse), ptr(dout), ptr(dq), ptr(dk), ptr(dv), ptr(ws), ctypes.c_size_t(n),
              ctypes.c_void_p(self.stream.cuda_stream)]

        def call():
            if self.L.msa_sparse_attn_bwd(*ba) != 0:
                raise RuntimeError(self.L.msa_last_error().decode())
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = HipEvents()
        per = {}
        for name, kid in BWD_KERNELS.items():
            a, b = ev.create(), ev.create()
            self.L.msa_set_kernel_timer(kid, a, b)
            call()
            torch.cuda.synchronize()
            self.L.msa_set_kernel_timer(0, None, None)
            per[name] = ev.elapsed_ms(a, b)
            ev.destroy(a)
            ev.destroy(b)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(steps):
            call()
        t1.record(self.stream)
        torch.cuda.synchronize()
        del ws, wsr, dq, dk, dv, dout
        return t0.elapsed_time(t1) / steps, per

    def index_select(self, steps=20, warmup=3):
        """ms per msa_index_select call on this workload's index queries and keys."""
        cref = ctypes.byref(self.cache) if self.cache is not None else None
        ia = [ctypes.byref(self.shape), cref] + [ctypes.c_void_p(self.x[n].data_ptr()) for n in ("q_idx", "k_idx")]
        ia += [ctypes.c_void_p(self.sel.data_ptr()), ctypes.c_void_p(self.ws.data_ptr()),
               ctypes.c_size_t(self.ws.numel()), ctypes.c_void_p(self.stream.cuda_stream)]

        def call():
            if self.L.msa_index_select_kvcache(*ia) != 0:
                raise RuntimeError(self.L.msa_last_error().decode())
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(steps):
            call()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def sparse_attn(self, steps=10, warmup=2):
        """ms per msa_sparse_attn_fwd call (gather + attention + combine) on this
        workload's selection, which one msa_fwd call first provides."""
        self.step()
        cref = ctypes.byref(self.cache) if self.cache is not None else None
        sa = [ctypes.byref(self.shape), cref] + [ctypes.c_void_p(self.x[n].data_ptr()) for n in ("q", "k", "v")]
        sa += [ctypes.c_void_p(self.sel.data_ptr()), ctypes.c_void_p(self.out.data_ptr()), None,
               ctypes.c_void_p(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel()),
               ctypes.c_void_p(self.stream.cuda_stream)]

        def call():
            if self.L.msa_sparse_attn_fwd_kvcache(*sa) != 0:
                raise RuntimeError(self.L.msa_last_error().decode())
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(steps):
            call()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def kernel_breakdown(self, steps=3):
        res = {}
        for name in KERNELS:
            _, ks = self.time_steps(steps, 0, name)
            if all(k is not None for k in ks):  # kernels this shape does not launch are left out
                res[name] = float(np.median(ks))
        return res


def step_stats(step_ms):
    return {"ms_p50": round(float(np.median(step_ms)), 4), "ms_p99": round(float(np.percentile(step_ms, 99)), 4)}


DECODE_WORKLOADS = (4, 6, 7)
DECODE_LAYERS = 4  # input copies the decode step rotates through


def decode_leg(msa, wid: int, args, steps=None, graph=True):
    """One decode workload: GB/s of algorithmic bytes, and the k_idx scan kernel
    (the index kernel) against the HBM roofline.  steps defaults to --decode-steps;
    graph=False skips the HIP-graph replays."""
    steps = args.decode_steps if steps is None else steps
    sd = synth.WORKLOADS[wid]
    name = synth.WORKLOAD_NAMES[wid]
    print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
    drun = Runner(msa, sd, wid)
    paged = drun.cache is not None
    dec_bytes = paged_decode_bytes(sd, drun.lens) if paged else algorithmic_work(sd)[2]
    # decode steps of four layers in turn: a 128K x 64 step reads 0.3 GB of K/V that
    # the 256 MB Infinity Cache could otherwise keep from one repeat of it to the next
    layers = drun.layer_copies(DECODE_LAYERS - 1)
    dms = drun.clean_time(steps, args.warmup, layers)
    del layers
    _, idx_ms = drun.time_steps(steps, 0, "index_score")  # per-step and per-kernel events
    stats = step_stats(drun.step_ms)
    dk = {} if args.no_breakdown else drun.kernel_breakdown()
    gbs = dec_bytes / (dms * 1e-3) / 1e9
    idx_avg = float(np.mean(idx_ms))
    kidx_tokens = int(np.sum(drun.lens, dtype=np.int64)) if paged else sd.batch * sd.kv_len
    kidx_bytes = float(kidx_tokens * sd.index_dim * (1 if sd.fp8 else 2))
    profile = {4: "index_topk_decode_128k_b64_hbm.md", 6: "index_topk_decode_128k_b64_fp8_hbm.md",
               7: "index_topk_decode_paged_varlen_b64_hbm.md"}[wid]
    res = {
        "workload": name, "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_step": round(dms, 4), **stats, "steps": steps, "bytes_per_step": dec_bytes,
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "index_topk", "achieved": round(kidx_bytes / (idx_avg * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(kidx_bytes / (idx_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "bytes_per_launch": kidx_bytes, "avg_launch_ms": round(idx_avg, 4),
                     "traffic": recorded_traffic(profile, "index_topk.hip", "traffic_read_bytes_per_launch")},
        "kernels_ms": {k: round(v, 4) for k, v in dk.items()},
    }
    if paged:
        res["cache_tokens"] = {"total": kidx_tokens, "min": int(drun.lens.min()), "max": int(drun.lens.max())}
    if graph:
        # the same call replayed from a HIP graph (launch gaps between its kernels removed)
        gms = drun.graph_time(steps, args.warmup)
        res["graph"] = {"ms_per_step": round(gms, 4), "value": round(dec_bytes / (gms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(dec_bytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del drun
    torch.cuda.empty_cache()
    return res


def cpu_baseline(s: synth.Shape, x, out_gpu, sel_gpu, budget_s: float):
    """Time the fp64 oracle on growing samples of query rows until ~budget_s."""
    from oracle import msa_oracle as orc
    import threadpoolctl

    def host(t):
        t = t.detach().cpu()
        return (t.float() if t.dtype == torch.bfloat16 else t).numpy()

    q, k, v = host(x["q"]), host(x["k"]), host(x["v"])
    q_idx, k_idx = host(x["q_idx"]), host(x["k_idx"])
    rng = np.random.default_rng(1234)
    flop_per_row = []
    rows_done = []
    elapsed = 0.0
    sel_ok, max_err = True, 0.0
    out_np = host(out_gpu)
    sel_np = sel_gpu.cpu().numpy()
    batch = 16
    while elapsed < budget_s and len(rows_done) < s.batch * s.q_len:
        rows = [(int(rng.integers(0, s.batch)), int(rng.integers(0, s.q_len))) for _ in range(batch)]
        t0 = time.perf_counter()
        o, sel, _ = orc.msa_forward(q, k, v, q_idx, k_idx, s.topk, s.q_offset, s.block_size, rows=rows)
        elapsed += time.perf_counter() - t0
        for b, i in rows:
            t = s.q_offset + i
            L = t // s.block_size
            n_sel = min(s.topk, L + 1)
            flop_per_row.append(4.0 * s.head_dim * s.num_q_heads * ((n_sel - 1) * s.block_size + t % s.block_size + 1)
                                + 2.0 * s.index_dim * s.groups * L * s.block_size)
            sel_ok &= bool(np.array_equal(sel_np[b, :, i], sel[b, :, i]))
            max_err = max(max_err, float(np.abs(out_np[b, i] - o[b, i]).max()))
        rows_done += rows
    info = threadpoolctl.threadpool_info()
    blas = [d for d in info if d.get("user_api") == "blas"]
    threads = max([d.get("num_threads", 1) for d in blas] or [1])
    return {
        "value": sum(flop_per_row) / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(rows_done)} random query rows (all {s.groups} groups, both branches) of "
                  f"the {synth.WORKLOAD_NAMES.get(3)} workload, {elapsed:.1f} s of fp64 numpy",
        "host_cpus": os.cpu_count(),
        "host": host_info(),
        "blas": [{k: d.get(k) for k in ("internal_api", "version", "num_threads")} for d in blas],
        "gpu_rows_match": {"selection_equal": sel_ok, "max_abs_err": max_err},
    }


WORKSPACE_CAP_MIB = 3500  # keeps the 32K x 2 workspace under 4 GB


def bounded_leg(msa, run, s: synth.Shape, args) -> dict:
    """ms per msa_fwd step of this workload with workspace_cap_mib = WORKSPACE_CAP_MIB,
    next to the uncapped workspace; outputs must equal the uncapped call's."""
    sh = msa.make_shape(s.batch, s.q_len, s.kv_len, s.q_offset, s.num_q_heads, s.num_kv_heads, s.head_dim,
                        s.index_dim, s.topk, s.torch_dtype, workspace_cap_mib=WORKSPACE_CAP_MIB)
    n = msa.workspace_size(sh, msa.OP_FWD)
    dev = run.x["q"].device
    wsr = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    ws = wsr[(-wsr.data_ptr()) % 256:][:n]
    out = torch.empty_like(run.out)
    a = list(run.args)
    a[0] = ctypes.byref(sh)
    a[7] = ctypes.c_void_p(out.data_ptr())
    a[-3], a[-2] = ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(n)
    fn = run.L.msa_fwd_kvcache
    for _ in range(args.warmup):
        if fn(*a) != 0:
            raise RuntimeError(run.L.msa_last_error().decode())
    run.step()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, run.out))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(run.stream)
    for _ in range(args.steps):
        fn(*a)
    t1.record(run.stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    del ws, wsr, out
    return {"workspace_cap_mib": WORKSPACE_CAP_MIB, "workspace_bytes": n, "uncapped_workspace_bytes": run.ws.numel(),
            "ms_per_step": round(ms, 4), "equal_to_uncapped": same}


def selection_check(s: synth.Shape, wid: int, x, sel_gpu) -> dict:
    """Every selection row of the timed workload against the fp64 oracle's, reported
    as the issue write-up's check after its fix reports it (section 验证方法):
    diverging rows out of all (b, g, i) rows, and the mean overlap of each row's
    blocks with the oracle's."""
    from oracle import msa_oracle as orc
    t0 = time.perf_counter()
    ref = np.empty((s.batch, s.groups, s.q_len, s.topk), dtype=np.int32)
    for b in range(s.batch):
        qi = x["q_idx"][b:b + 1].float().numpy().astype(np.float64)  # exact upcasts of the stored values
        ki = x["k_idx"][b:b + 1].float().numpy().astype(np.float64)
        ref[b] = orc.index_select(qi, ki, s.topk, s.q_offset, s.block_size)[0]
    rep = orc.selection_agreement(sel_gpu.numpy(), ref)
    rep["workload"] = synth.WORKLOAD_NAMES[wid]
    rep["oracle_s"] = round(time.perf_counter() - t0, 1)
    return rep


def work_rates(flop_main, flop_index, step_tflops, kern):
    """Each timed part's TFLOP/s and its fraction of the bf16 MFMA peak: the
    index kernel (msa_index_select's work), the main branch alone (what
    msa_sparse_attn_fwd runs: gather + attention + combine) and the whole step."""
    out = {"flop_main": flop_main, "flop_index": flop_index,
           "step_frac_of_mfma_peak": round(step_tflops / PEAK_BF16_TFLOPS, 4)}
    if kern:
        idx = flop_index / (kern["index_score"] * 1e-3) / 1e12
        sa = flop_main / (sum(kern.get(k, 0.0) for k in ("gather", "attention", "combine")) * 1e-3) / 1e12
        out.update({"index_tflops": round(idx, 2), "index_frac_of_mfma_peak": round(idx / PEAK_BF16_TFLOPS, 4),
                    "sparse_attn_tflops": round(sa, 2),
                    "sparse_attn_frac_of_mfma_peak": round(sa / PEAK_BF16_TFLOPS, 4)})
    else:
        out.update({"index_tflops": None, "sparse_attn_tflops": None})
    return out


def host_info():
    """CPU model and memory of the machine the oracle ran on."""
    model, mem_gb = None, None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        with open("/proc/meminfo") as f:
            kb = next((int(ln.split()[1]) for ln in f if ln.startswith("MemTotal")), None)
        mem_gb = round(kb / 2 ** 20, 1) if kb else None
    except OSError:
        pass
    return {"cpu_model": model, "mem_gib": mem_gb}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the KL teacher, the backward and the 8K and 1M-context prefill workloads")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel timing passes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 4 plain device copies of 1 GiB (known bytes, for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the MSA library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    import block_sparse_attention_idx_amd as msa
    msa.lib()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copy calibration: 4 copies of 1073741824 bytes", file=sys.stderr, flush=True)
    wid = args.workload
    s = synth.WORKLOADS[wid]
    if wid in DECODE_WORKLOADS:
        # a decode workload on its own: its GB/s line (the k_idx scan's HBM roofline)
        leg = decode_leg(msa, wid, args, steps=args.steps, graph=not args.no_breakdown)
        result = {"metric": METRIC, "value": leg["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                  "warmup": args.warmup, "ms_per_step": leg["ms_per_step"],
                  **{k: leg[k] for k in ("ms_p50", "ms_p99") if k in leg},
                  "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                  "data": "synthetic",
                  "config": {"workload": leg["workload"], "batch": s.batch, "q_len": s.q_len, "kv_len": s.kv_len,
                             "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads, "head_dim": s.head_dim,
                             "index_dim": s.index_dim, "block_size": s.block_size, "topk": s.topk,
                             "cache": "e4m3" if s.fp8 else "bf16"},
                  "roofline": leg["roofline"], "frac_of_hbm_peak": leg["frac_of_hbm_peak"],
                  "kernels_ms": leg["kernels_ms"], "cpu_baseline": None}
        for k in ("cache_tokens", "graph"):
            if k in leg:
                result[k] = leg[k]
        print(json.dumps(result))
        return
    flop_main, flop_index, _ = algorithmic_work(s)
    print(f"[bench] {synth.WORKLOAD_NAMES[wid]}: generating inputs", file=sys.stderr, flush=True)
    run = Runner(msa, s, wid)
    print("[bench] timing msa_fwd", file=sys.stderr, flush=True)
    ms = run.clean_time(args.steps, args.warmup)
    _, attn_ms = run.time_steps(args.steps, 0, "attention")  # per-step and per-kernel events
    stats = step_stats(run.step_ms)
    kern = {} if args.no_breakdown else run.kernel_breakdown()
    attn_avg = float(np.mean(attn_ms))
    value = (flop_main + flop_index) / (ms * 1e-3) / 1e12
    achieved = flop_main / (attn_avg * 1e-3) / 1e12
    traffic = recorded_traffic("attn_kvouter_prefill_32k_b2_hbm.md", "attn.hip") if wid == 3 else None
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        **stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": synth.WORKLOAD_NAMES[wid], "batch": s.batch, "q_len": s.q_len,
                   "kv_len": s.kv_len, "q_offset": s.q_offset, "num_q_heads": s.num_q_heads,
                   "num_kv_heads": s.num_kv_heads, "head_dim": s.head_dim, "index_dim": s.index_dim,
                   "block_size": s.block_size, "topk": s.topk},
        "roofline": {"bound": "mfma", "kernel": "attn_kvouter", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_unit": "bytes",
                     # the counted HBM bytes per launch over this run's launch time, against 8 TB/s
                     "traffic_frac_of_hbm_peak": (round(traffic / (attn_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                                                  if traffic else None),
                     "flop_per_launch": flop_main, "avg_launch_ms": round(attn_avg, 4)},
        "work": work_rates(flop_main, flop_index, value, kern),
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
    }
    print(f"[bench] {ms:.3f} ms/step, attention {attn_avg:.3f} ms", file=sys.stderr, flush=True)
    if not args.no_extra:
        # the KL-alignment teacher on the same workload: QK^T again (half the main
        # FLOPs) plus the index scores over the same tokens
        flop_kl = flop_main * (0.5 + s.index_dim * s.groups / (2.0 * s.head_dim * s.num_q_heads))
        kms, kper = run.kl_teacher()
        result["kl_teacher"] = {"ms": round(kms, 4), "tflops": round(flop_kl / (kms * 1e-3) / 1e12, 2),
                                "frac_of_mfma_peak": round(flop_kl / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                "flop": flop_kl, "kernels_ms": {k: round(v, 4) for k, v in kper.items() if v}}
        # the main branch's backward: S, dP, dV, dK and dQ products, 10 d FLOP per (row, key)
        flop_bwd = 2.5 * flop_main
        bms, bper = run.backward()
        result["backward"] = {"ms": round(bms, 4), "tflops": round(flop_bwd / (bms * 1e-3) / 1e12, 2),
                              "frac_of_mfma_peak": round(flop_bwd / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "flop": flop_bwd, "kernels_ms": {k: round(v, 4) for k, v in bper.items() if v}}

    if not args.no_extra:
        result["sparse_attn"] = sparse_attn_leg(run, s, flop_main)
        result["index_select"] = index_select_leg(run, flop_index)
    if not args.no_extra and wid == 3:
        # the same step with the workspace capped (msa_shape.workspace_cap_mib): the main
        # branch runs over query-row chunks whose partial states fit the cap
        result["bounded_workspace"] = bounded_leg(msa, run, s, args)
    # the CPU legs run after every GPU leg (so GPU-busy samples land on GPU work):
    # keep host copies of this workload's inputs and results for them
    host = None
    if not args.no_cpu:
        host = ({n: t.cpu() for n, t in run.x.items()}, run.out.cpu(), run.sel.cpu())
    del run
    torch.cuda.empty_cache()

    if not args.no_extra:
        # the other prefill workloads, reported beside the headline one
        result["extra"] = {}
        for ew in (2, 5):
            se = synth.WORKLOADS[ew]
            fm, fi, _ = algorithmic_work(se)
            print(f"[bench] {synth.WORKLOAD_NAMES[ew]}: generating inputs", file=sys.stderr, flush=True)
            er = Runner(msa, se, ew)
            ems = er.clean_time(10, 2)
            eatt = er.time_steps(10, 0, "attention")[1]
            eidx = er.time_steps(5, 0, "index_score")[1]
            eatt_ms, eidx_ms = float(np.mean(eatt)), float(np.median(eidx))
            result["extra"][synth.WORKLOAD_NAMES[ew]] = {
                "ms_per_step": round(ems, 4), "tflops": round((fm + fi) / (ems * 1e-3) / 1e12, 2),
                "attention_ms": round(eatt_ms, 4), "attention_frac_of_mfma_peak": round(fm / (eatt_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "index_ms": round(eidx_ms, 4), "index_frac_of_mfma_peak": round(fi / (eidx_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "flop_main": fm, "flop_index": fi, "sparse_attn": sparse_attn_leg(er, se, fm),
                "index_select": index_select_leg(er, fi)}
            del er
            torch.cuda.empty_cache()

    if not args.no_decode:
        result["decode"] = decode_leg(msa, 4, args)
        result["decode_fp8"] = decode_leg(msa, 6, args)
        result["decode_paged"] = decode_leg(msa, 7, args)

    if host is not None:
        hx, hout, hsel = host
        print("[bench] selection check (oracle on every row)", file=sys.stderr, flush=True)
        result["selection_check"] = selection_check(s, wid, hx, hsel)
        print("[bench] cpu baseline (oracle on sampled rows)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(s, hx, hout, hsel, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()

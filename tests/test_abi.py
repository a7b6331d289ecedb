"""The C ABI without a GPU: the library loads, exports what include/msa.h
declares, and rejects bad arguments before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_idx_amd as msa
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = msa.lib()
    names = _declared()
    assert {"msa_index_select", "msa_sparse_attn_fwd", "msa_fwd", "msa_workspace_size",
            "msa_status_string", "msa_last_error", "msa_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", msa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (msa_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_header():
    assert ctypes.sizeof(msa.MsaShape) == 72
    assert msa.MsaShape.cache_format.offset == 12
    assert msa.MsaShape.q_offset.offset == 16
    assert msa.MsaShape.softmax_scale.offset == 48
    assert msa.MsaShape.k_scale.offset == 60
    assert msa.MsaShape.v_scale.offset == 64
    assert msa.MsaShape.workspace_cap_mib.offset == 68
    text = open(HEADER).read()
    assert "MSA_CACHE_NATIVE = 0" in text and "MSA_CACHE_FP8_E4M3 = 1" in text


def _shape(wid=2, **kw):
    s = synth.WORKLOADS[wid]
    import torch
    sh = msa.make_shape(s.batch, s.q_len, s.kv_len, s.q_offset, s.num_q_heads, s.num_kv_heads, s.head_dim,
                        s.index_dim, s.topk, torch.float32 if s.dtype == "f32" else torch.bfloat16)
    for k, v in kw.items():
        setattr(sh, k, v)
    return sh


def _fwd(sh, ws=None, ws_bytes=0, **ptrs):
    L = msa.lib()
    p = {n: FAKE for n in ("q", "k", "v", "q_idx", "k_idx", "out")}
    p.update(ptrs)
    return L.msa_fwd(ctypes.byref(sh) if sh is not None else None, p["q"], p["k"], p["v"], p["q_idx"],
                     p["k_idx"], p["out"], None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, -1), ("q_len", -1, -1), ("kv_len", 0, -1), ("q_offset", -5, -1), ("kv_len", 100, -1),
    ("num_q_heads", 62, -1), ("num_kv_heads", 0, -1), ("topk", 0, -1), ("block_size", 0, -1),
    ("dtype", 7, -1), ("out_dtype", 9, -1), ("cache_format", 2, -1), ("cache_format", -1, -1), ("workspace_cap_mib", -3, -1),
    ("head_dim", 0, -1),
    ("block_size", 64, -2), ("topk", 65, -2), ("head_dim", 96, -2), ("index_dim", 48, -2),
    ("num_q_heads", 12, -2),
])
def test_invalid_and_unsupported_shapes(field, value, status):
    sh = _shape(**{field: value})
    assert _fwd(sh) == status
    assert msa.lib().msa_last_error().decode() != ""
    assert msa.workspace_size(sh, msa.OP_FWD) == 0


def test_null_pointers_rejected():
    L = msa.lib()
    sh = _shape()
    assert _fwd(None) == -1
    for name in ("q", "k", "v", "q_idx", "k_idx", "out"):
        assert _fwd(sh, **{name: None}) == -1, name
    assert L.msa_index_select(ctypes.byref(sh), FAKE, None, FAKE, None, 0, None) == -1
    assert L.msa_sparse_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == -1


@pytest.mark.parametrize("field", ["softmax_scale", "k_scale", "v_scale"])
@pytest.mark.parametrize("scale", [float("nan"), float("inf"), -0.5])
def test_bad_scale_rejected(field, scale):
    sh = _shape()
    setattr(sh, field, scale)
    assert _fwd(sh) == -1


def test_fp8_caches_need_bf16_queries():
    sh = _shape(1, cache_format=1)  # the fp32 workload
    assert _fwd(sh) == -2
    assert "FP8" in msa.lib().msa_last_error().decode()
    sh = _shape(2, cache_format=1)
    assert msa.workspace_size(sh, msa.OP_FWD) == msa.workspace_size(_shape(2), msa.OP_FWD)


def test_workspace_checks():
    sh = _shape()
    need = msa.workspace_size(sh, msa.OP_FWD)
    assert need > 0
    assert _fwd(sh) == -3  # NULL workspace
    assert _fwd(sh, ctypes.c_void_p(0x10010), need) == -3  # not 256-byte aligned
    assert _fwd(sh, ctypes.c_void_p(0x10000), need - 1) == -3  # too small
    assert "workspace" in msa.lib().msa_last_error().decode()


def test_empty_query_is_a_no_op():
    sh = _shape(q_len=0)
    assert _fwd(sh) == 0
    assert msa.workspace_size(sh, msa.OP_FWD) == 0


def test_status_strings_and_version():
    L = msa.lib()
    for st, name in ((0, "MSA_OK"), (-1, "MSA_ERR_INVALID"), (-2, "MSA_ERR_UNSUPPORTED"),
                     (-3, "MSA_ERR_WORKSPACE"), (-4, "MSA_ERR_HIP")):
        assert L.msa_status_string(st).decode() == name
    assert re.match(r"\d+\.\d+\.\d+", L.msa_version().decode())


def test_workspace_sizes_for_the_workloads():
    # deterministic, and large enough for the partial states the main branch keeps
    for wid, s in synth.WORKLOADS.items():
        sh = _shape(wid)
        a = msa.workspace_size(sh, msa.OP_FWD)
        assert a == msa.workspace_size(sh, msa.OP_FWD) and a % 256 == 0
        e = 4 if s.dtype == "f32" else 2
        partials = s.batch * s.q_len * s.num_q_heads * s.topk * s.head_dim * e
        assert a >= partials
        assert msa.workspace_size(sh, msa.OP_INDEX_SELECT) >= 0  # 0 when one key split needs no lists
        assert msa.workspace_size(sh, msa.OP_SPARSE_ATTN) <= a
    # a bad op code gives 0
    assert msa.lib().msa_workspace_size(ctypes.byref(_shape()), 7) == 0


def test_python_layer_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        msa.sparse_attn_fwd(q, q, q, torch.zeros(1, 2, 4, 1, dtype=torch.int32))


def test_python_cache_format_rules():
    import torch
    bf, f8 = torch.bfloat16, torch.float8_e4m3fn
    t = lambda dt: torch.zeros(1, dtype=dt)
    assert msa._cache_format(bf, [("k", t(bf)), ("v", t(bf))]) == msa.CACHE_NATIVE
    assert msa._cache_format(bf, [("k", t(f8)), ("v", t(f8)), ("k_idx", t(f8))]) == msa.CACHE_FP8_E4M3
    with pytest.raises(ValueError):  # mixed caches
        msa._cache_format(bf, [("k", t(f8)), ("v", t(bf))])
    with pytest.raises(ValueError):  # fp8 next to fp32 queries
        msa._cache_format(torch.float32, [("k", t(f8)), ("v", t(f8))])


def test_kvcache_descriptor_checks():
    L = msa.lib()
    sh = _shape(4)  # the 128K decode shape: q_offset 131071
    c = msa.MsaKvCache()
    c.seq_lens = 0x2000  # never dereferenced: validation fails or nothing is launched
    args = lambda cache: (ctypes.byref(sh), ctypes.byref(cache), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                          None, 0, None)
    assert L.msa_fwd_kvcache(*args(c)) == -1  # lengths given but q_offset != 0
    assert "q_offset" in L.msa_last_error().decode()
    sh.q_offset = 0
    c.page_table = 0x3000
    c.max_pages, c.num_pages = 0, 10
    assert L.msa_fwd_kvcache(*args(c)) == -1  # a page table needs max_pages >= 1
    c.max_pages = 1023  # 1023 * 128 < kv_len 131072
    assert L.msa_fwd_kvcache(*args(c)) == -1
    assert "max_pages" in L.msa_last_error().decode()
    c.max_pages = 1024
    assert L.msa_fwd_kvcache(*args(c)) == -3  # valid: now only the workspace is missing
    # with lengths, the plan bounds positions by kv_len, not by q_offset + q_len
    # (q_offset 0 and one query row: without lengths there is no block to rank)
    need_var = L.msa_workspace_size_kvcache(ctypes.byref(sh), ctypes.byref(c), msa.OP_INDEX_SELECT)
    need_fixed = L.msa_workspace_size_kvcache(ctypes.byref(sh), None, msa.OP_INDEX_SELECT)
    assert need_var > 0 and need_fixed == 0
    assert L.msa_workspace_size_kvcache(ctypes.byref(sh), None, msa.OP_FWD) == msa.workspace_size(sh, msa.OP_FWD)


def test_kl_teacher_checks():
    L = msa.lib()
    sh = _shape(2)
    args = lambda **kw: [ctypes.byref(sh)] + [kw.get(n, FAKE) for n in ("q", "k", "q_idx", "k_idx", "sel", "lse")] + \
        [ctypes.c_float(kw.get("isc", 1.0)), kw.get("kl", FAKE), None, kw.get("ws", None), kw.get("wsb", 0), None]
    for name in ("q", "k", "q_idx", "k_idx", "sel", "lse", "kl"):
        assert L.msa_kl_teacher_fwd(*args(**{name: None})) == -1, name
    assert L.msa_kl_teacher_fwd(*args(isc=float("nan"))) == -1
    assert "index_scale" in L.msa_last_error().decode()
    assert L.msa_kl_teacher_fwd(*args()) == -3  # valid: only the workspace is missing
    need = msa.workspace_size(sh, msa.OP_KL_TEACHER)
    # the main branch's gather and partial regions, cut into smaller work items
    assert need >= msa.workspace_size(sh, msa.OP_SPARSE_ATTN) > 0
    assert msa.lib().msa_set_kernel_timer(9, None, None) == 0 and msa.lib().msa_set_kernel_timer(10, None, None) == -1


def test_backward_checks():
    L = msa.lib()
    sh = _shape(2)  # bf16
    args = lambda **kw: [ctypes.byref(sh)] + [kw.get(n, FAKE) for n in ("q", "k", "v", "sel", "out", "lse", "dout",
                                                                      "dq", "dk", "dv")] + [None, 0, None]
    for name in ("q", "k", "v", "sel", "out", "lse", "dout", "dq", "dk", "dv"):
        assert L.msa_sparse_attn_bwd(*args(**{name: None})) == -1, name
    assert L.msa_sparse_attn_bwd(*args()) == -3  # valid: only the workspace is missing
    assert msa.workspace_size(sh, msa.OP_SPARSE_ATTN_BWD) > msa.workspace_size(sh, msa.OP_SPARSE_ATTN)
    for field, value in (("dtype", 0), ("out_dtype", 0), ("cache_format", 1), ("k_scale", 0.5)):
        bad = _shape(2, **{field: value})
        assert L.msa_sparse_attn_bwd(ctypes.byref(bad), *args()[1:]) == -2, field


def test_noalloc_validates_before_touching_a_device():
    L = msa.lib()
    sh = _shape(2)
    # a NULL input: refused by the argument checks msa_fwd runs
    st = L.msa_fwd_noalloc(ctypes.byref(sh), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None)
    assert st == -1 and b"non-NULL" in L.msa_last_error()
    # the 8K prefill needs ~2 GiB of workspace: more than the fixed scratch holds
    assert msa.workspace_size(sh, msa.OP_FWD) > msa.noalloc_scratch_bytes()
    st = L.msa_fwd_noalloc(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None)
    assert st == -3 and b"msa_fwd_noalloc holds" in L.msa_last_error()
    # a bad shape is reported as such
    bad = _shape(2, topk=0)
    assert L.msa_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1
    assert msa.noalloc_scratch_bytes() == 64 << 20

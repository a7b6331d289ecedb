// Host side of the MSA C ABI: argument checks, workspace layout, launch plans.
// Every check runs before anything is enqueued, so an error leaves all outputs
// untouched and needs no GPU.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/msa.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;
thread_local msa::KernelTimer g_timer = {0, nullptr, nullptr};

const msa::KernelTimer* timer() { return g_timer.which ? &g_timer : nullptr; }

msa_status fail(msa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
msa_status fail(msa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr size_t kAlign = 256;
constexpr int kTokensPerItem = 128;
constexpr int kAttnGrid = 512;      // persistent attention grid: 2 workgroups per CU
// Units the key splits aim for: 4 per CU for the row-tile kernel (each unit
// pays a fixed ~20 us for its queries, last ranking and list write), 8 per CU
// for the few-row form, whose units stream keys from HBM.
constexpr int kIndexTargetUnits = 1024;
constexpr int kIndexTargetUnitsFewRows = 2048;
constexpr int64_t kIndexVarlenChunk = 16;  // key blocks per unit when sequences have their own lengths
constexpr int kIndexMinTiles = 512;  // row tiles that fill 256 CUs without key splits

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2_upto32(int r) { return r == 1 || r == 2 || r == 4 || r == 8 || r == 16 || r == 32; }

int elem_bytes(int dtype) { return dtype == MSA_F32 ? 4 : 2; }

bool fp8_cache(const msa_shape* s) { return s->cache_format == MSA_CACHE_FP8_E4M3; }

bool scale_ok(float x) { return std::isfinite(x) && x >= 0.0f; }

// Shape checks shared by every op.  'op' selects the op-specific ones.
msa_status check_shape(const msa_shape* s, int op) {
  if (!s) return fail(MSA_ERR_INVALID, "shape is NULL");
  static_assert(sizeof(msa_shape) == 72, "msa_shape layout");
  if (s->workspace_cap_mib < 0) return fail(MSA_ERR_INVALID, "workspace_cap_mib must be >= 0");
  if (s->cache_format != MSA_CACHE_NATIVE && s->cache_format != MSA_CACHE_FP8_E4M3)
    return fail(MSA_ERR_INVALID, "unknown cache_format %d", s->cache_format);
  if (s->batch < 1) return fail(MSA_ERR_INVALID, "batch must be >= 1 (got %d)", s->batch);
  if (s->q_len < 0) return fail(MSA_ERR_INVALID, "q_len must be >= 0 (got %d)", s->q_len);
  if (s->kv_len < 1) return fail(MSA_ERR_INVALID, "kv_len must be >= 1 (got %d)", s->kv_len);
  if (s->q_offset < 0) return fail(MSA_ERR_INVALID, "q_offset must be >= 0");
  if (s->q_offset + (int64_t)s->q_len > (int64_t)s->kv_len)
    return fail(MSA_ERR_INVALID, "kv_len (%d) must be >= q_offset + q_len (%lld)", s->kv_len,
                (long long)(s->q_offset + s->q_len));
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(MSA_ERR_INVALID, "head counts must be >= 1");
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(MSA_ERR_INVALID, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", s->num_q_heads,
                s->num_kv_heads);
  if (s->head_dim < 1 || s->index_dim < 1) return fail(MSA_ERR_INVALID, "head_dim and index_dim must be >= 1");
  if (s->block_size < 1) return fail(MSA_ERR_INVALID, "block_size must be >= 1");
  if (s->topk < 1) return fail(MSA_ERR_INVALID, "topk must be >= 1 (got %d)", s->topk);
  if (s->dtype != MSA_F32 && s->dtype != MSA_BF16) return fail(MSA_ERR_INVALID, "unknown dtype %d", s->dtype);
  if (s->out_dtype != MSA_F32 && s->out_dtype != MSA_BF16)
    return fail(MSA_ERR_INVALID, "unknown out_dtype %d", s->out_dtype);
  if (!scale_ok(s->softmax_scale))
    return fail(MSA_ERR_INVALID, "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  if (!scale_ok(s->k_scale) || !scale_ok(s->v_scale))
    return fail(MSA_ERR_INVALID, "k_scale and v_scale must be finite and >= 0 (0 means 1)");

  if (s->block_size != msa::kBlock)
    return fail(MSA_ERR_UNSUPPORTED, "block_size %d: only 128 is built", s->block_size);
  if (fp8_cache(s) && s->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "FP8 caches are built for bf16 queries only");
  if (s->topk > 64) return fail(MSA_ERR_UNSUPPORTED, "topk %d: at most 64 is built", s->topk);
  if (s->q_len >= (1 << 25)) return fail(MSA_ERR_UNSUPPORTED, "q_len must be < 2^25");
  if ((int64_t)s->batch * s->num_kv_heads * ceil_div(s->kv_len, msa::kBlock) >= (1LL << 31))
    return fail(MSA_ERR_UNSUPPORTED, "batch * kv heads * blocks exceeds 2^31");
  const bool index_op = op == MSA_OP_INDEX_SELECT || op == MSA_OP_FWD || op == MSA_OP_KL_TEACHER;
  const bool attn_op = op == MSA_OP_SPARSE_ATTN || op == MSA_OP_FWD || op == MSA_OP_KL_TEACHER ||
                       op == MSA_OP_SPARSE_ATTN_BWD;
  if (op == MSA_OP_SPARSE_ATTN_BWD) {
    if (s->dtype != MSA_BF16 || s->out_dtype != MSA_BF16 || fp8_cache(s))
      return fail(MSA_ERR_UNSUPPORTED, "the backward is built for bf16 q, k, v, out and dout");
    if ((s->k_scale != 0.0f && s->k_scale != 1.0f) || (s->v_scale != 0.0f && s->v_scale != 1.0f))
      return fail(MSA_ERR_UNSUPPORTED, "the backward takes unscaled caches (k_scale, v_scale 0 or 1)");
  }
  if (index_op) {
    if (s->index_dim != 32 && s->index_dim != 64 && s->index_dim != 128)
      return fail(MSA_ERR_UNSUPPORTED, "index_dim %d: built for 32, 64, 128", s->index_dim);
    if ((int64_t)s->q_len * s->num_kv_heads * s->batch >= (1LL << 31))
      return fail(MSA_ERR_UNSUPPORTED, "batch * q_len * groups exceeds 2^31");
  }
  if (attn_op) {
    if (s->head_dim != 64 && s->head_dim != 128)
      return fail(MSA_ERR_UNSUPPORTED, "head_dim %d: built for 64 and 128", s->head_dim);
    const int r = s->num_q_heads / s->num_kv_heads;
    if (!is_pow2_upto32(r))
      return fail(MSA_ERR_UNSUPPORTED, "query heads per group %d: built for 1, 2, 4, 8, 16, 32", r);
    if (s->out_dtype != MSA_F32 && s->out_dtype != s->dtype)
      return fail(MSA_ERR_UNSUPPORTED, "out_dtype must be MSA_F32 or the input dtype");
    if ((int64_t)s->batch * s->num_kv_heads * s->q_len * s->topk >= (1LL << 31))
      return fail(MSA_ERR_UNSUPPORTED, "batch * groups * q_len * topk exceeds 2^31");
  }
  return MSA_OK;
}

// ---- caches ---------------------------------------------------------------

msa_status check_cache(const msa_shape* s, const msa_kv_cache* c) {
  if (!c) return MSA_OK;
  if (c->seq_lens && s->q_offset != 0)
    return fail(MSA_ERR_INVALID, "q_offset must be 0 when seq_lens is given (positions come from the lengths)");
  if (c->page_table) {
    if (c->max_pages < 1 || c->num_pages < 1)
      return fail(MSA_ERR_INVALID, "max_pages and num_pages must be >= 1 with a page table");
    if ((int64_t)s->kv_len > (int64_t)c->max_pages * msa::kBlock)
      return fail(MSA_ERR_INVALID, "kv_len (%d) exceeds max_pages * 128 (%lld)", s->kv_len,
                  (long long)c->max_pages * msa::kBlock);
    if ((int64_t)s->batch * c->max_pages >= (1LL << 31))
      return fail(MSA_ERR_UNSUPPORTED, "batch * max_pages exceeds 2^31");
  }
  if (c->seq_lens && (int64_t)s->batch * ((int64_t)s->q_len * s->num_kv_heads / 128 + 1) >= (1LL << 24))
    return fail(MSA_ERR_UNSUPPORTED, "batch * row tiles exceeds 2^24 with seq_lens");
  return MSA_OK;
}

msa::CacheMap cache_map(const msa_kv_cache* c) {
  msa::CacheMap m{};
  if (c) {
    m.seq_lens = c->seq_lens;
    m.pages = c->page_table;
    if (c->page_table) {
      m.max_pages = c->max_pages;
      m.num_pages = c->num_pages;
    }
  }
  return m;
}

// The largest position a query row can have: the bound the launch plans use.
int64_t max_pos(const msa_shape* s, const msa_kv_cache* c) {
  if (c && c->seq_lens) return (int64_t)s->kv_len - 1;
  return s->q_offset + s->q_len - 1;
}

// ---- index plan -----------------------------------------------------------

struct IndexPlan {
  msa::IndexParams p;
  int cap;
  size_t off_s, off_i, off_units, off_count;  // partial lists, unit list (0 when unused)
  bool lists, unit_list;
  size_t bytes;
};

IndexPlan plan_index(const msa_shape* s, const msa_kv_cache* cache) {
  IndexPlan ip{};
  msa::IndexParams& p = ip.p;
  p.cm = cache_map(cache);
  p.B = s->batch;
  p.S_q = s->q_len;
  p.S_k = s->kv_len;
  p.G = s->num_kv_heads;
  p.topk = s->topk;
  p.q_offset = s->q_offset;
  p.rows_per_b = s->q_len * s->num_kv_heads;
  p.small = p.rows_per_b <= msa::kIndexSmallRows && s->dtype == MSA_BF16 ? 1 : 0;
  p.rows_wg = p.small ? p.rows_per_b : msa::index_rows_per_wg(s->topk, s->dtype == MSA_BF16);
  p.ntile = (int)ceil_div(p.rows_per_b, p.rows_wg);
  p.ntile_total = p.B * p.ntile;
  const int64_t Lmax = s->q_len > 0 ? max_pos(s, cache) / msa::kBlock : 0;
  // Enough row tiles to fill the GPU: one unit per tile, no merge.  Otherwise
  // split the key blocks so that about kIndexTargetUnits units exist (at least
  // 16 blocks per unit, 8 in the few-row form where 4 waves share a unit's
  // blocks, and no more lists per row than the merge takes).
  // With per-sequence lengths the work per sequence is unknown here: a fixed,
  // small chunk keeps short caches from leaving most units idle, and a unit
  // list built on the device packs the units that hold work first.
  ip.cap = msa::index_cap(s->topk);
  const bool wide = ip.cap == msa::kIndexWideCap;  // every lane half's list goes to the merge
  p.lps = wide ? (p.small ? 8 : 2) : 1;
  const int64_t max_split = msa::merge_max_lists(ip.cap) / p.lps;
  int64_t chunk = std::max<int64_t>(1, Lmax), nsplit = 1;
  if (Lmax > 0 && p.ntile_total < kIndexMinTiles) {
    const int64_t min_chunk = p.small ? 8 : 16;
    const int target = p.small ? kIndexTargetUnitsFewRows : kIndexTargetUnits;
    const int64_t want = std::max<int64_t>(1, ceil_div(target, std::max(1, p.ntile_total)));
    const bool varlen = cache && cache->seq_lens;
    chunk = std::max<int64_t>({min_chunk, varlen ? kIndexVarlenChunk : ceil_div(Lmax, want), ceil_div(Lmax, max_split)});
    nsplit = ceil_div(Lmax, chunk);
  }
  p.chunk = (int)chunk;
  p.nsplit = (int)nsplit;
  p.nunits = p.ntile_total * p.nsplit;
  p.grid_per_xcd = (int)ceil_div(p.nunits, 8);
  const size_t entries = (size_t)p.B * p.rows_per_b * p.nsplit * p.lps * ip.cap;
  size_t off = 0;
  ip.lists = p.nsplit > 1 || wide;
  if (ip.lists) {
    ip.off_s = off;
    off += align_up(entries * 4);
    ip.off_i = off;
    off += align_up(entries * 4);
  }
  ip.unit_list = cache && cache->seq_lens;  // work per sequence known only on the device
  // the few-row form (one row tile per sequence) derives its units in the kernel
  p.units_inline = ip.unit_list && p.small && p.ntile == 1 && p.B <= 64 * msa::kInlineUnitsPerLane ? 1 : 0;
  if (p.units_inline) ip.unit_list = false;
  if (ip.unit_list) {
    ip.off_units = off;
    off += align_up((size_t)p.nunits * 4);
    ip.off_count = off;
    off += align_up(4);
  }
  p.persist = p.nsplit == 1 && !p.small && !ip.unit_list && !p.units_inline ? 1 : 0;
  ip.bytes = off;
  return ip;
}

void bind_index(IndexPlan& ip, char* ws, const void* q_idx, const void* k_idx, int32_t* sel) {
  ip.p.part_s = ip.lists ? (float*)(ws + ip.off_s) : nullptr;
  ip.p.part_i = ip.lists ? (int32_t*)(ws + ip.off_i) : nullptr;
  ip.p.units = ip.unit_list ? (int32_t*)(ws + ip.off_units) : nullptr;
  ip.p.unit_count = ip.unit_list ? (int32_t*)(ws + ip.off_count) : nullptr;
  ip.p.q_idx = q_idx;
  ip.p.k_idx = k_idx;
  ip.p.sel = sel;
}

// ---- attention plan -------------------------------------------------------

struct AttnPlan {
  msa::AttnParams p;
  size_t off_counts, off_offsets, off_cursor, off_item_off, off_nitems, off_entries, off_items, off_po, off_pl;
  size_t bytes;
};

// tpi: query tokens per work item of the gather; fwd_main: the forward's main
// branch (msa_sparse_attn_fwd, msa_fwd), whose partial states the shape's
// workspace_cap_mib may bound
AttnPlan plan_attn(const msa_shape* s, const msa_kv_cache* cache, int tpi = kTokensPerItem, bool fwd_main = false) {
  AttnPlan ap{};
  msa::AttnParams& p = ap.p;
  p.cm = cache_map(cache);
  p.B = s->batch;
  p.S_q = s->q_len;
  p.S_k = s->kv_len;
  p.Hq = s->num_q_heads;
  p.G = s->num_kv_heads;
  p.r = s->num_q_heads / s->num_kv_heads;
  p.d = s->head_dim;
  p.topk = s->topk;
  p.q_offset = s->q_offset;
  p.nb = (int)ceil_div(s->kv_len, msa::kBlock);
  p.nbuckets = p.B * p.G * p.nb;
  p.tpi = tpi;
  const int64_t Lmax = s->q_len > 0 ? max_pos(s, cache) / msa::kBlock : 0;
  // queries per (b, g, block) on average; below 2 the gather buys nothing
  const double per_bucket = (double)s->q_len * std::min<int64_t>(s->topk, Lmax + 1) / (double)(Lmax + 1);
  p.direct = per_bucket < 2.0 ? 1 : 0;
  // decode with enough (b, i, g) rows to give every CU one: a workgroup per row
  // runs the whole main branch (bf16 queries; the fp32 form's LDS does not fit)
  p.rows_mode = p.direct && s->dtype == MSA_BF16 &&
                (int64_t)s->batch * s->q_len * s->num_kv_heads >= msa::kDecodeRowsMin ? 1 : 0;
  p.n_direct = (int64_t)p.B * p.G * p.S_q * p.topk;
  p.grid = kAttnGrid;
  // 6 workgroups per CU, twice what fits at once (44 KiB of LDS each): measured
  // faster than one resident round for bf16 and paged caches, as fast for e4m3
  p.grid_decode = 1536;
  const float scale = s->softmax_scale != 0.0f ? s->softmax_scale : 1.0f / std::sqrt((float)s->head_dim);
  const float kscale = s->k_scale != 0.0f ? s->k_scale : 1.0f;
  p.scale_log2 = scale * kscale * 1.4426950408889634f;
  p.v_scale = s->v_scale != 0.0f ? s->v_scale : 1.0f;
  p.out_f32 = s->out_dtype == MSA_F32 ? 1 : 0;

  p.row0 = 0;
  p.nrows = p.chunk_rows = p.S_q;
  if (fwd_main && !p.direct && s->workspace_cap_mib > 0) {
    // rows per chunk: the partial states (and gather entries) of that many rows of
    // every sequence fit the cap; full gather tiles when the cap allows them
    const size_t per_row = (size_t)p.B * p.G * p.topk * ((size_t)p.r * (p.d * elem_bytes(s->dtype) + 4) + 4);
    const size_t cap = (size_t)s->workspace_cap_mib << 20;
    int64_t rows = std::max<int64_t>(1, (int64_t)(cap / per_row));
    if (rows >= 256) rows = rows / 256 * 256;
    p.chunk_rows = (int)std::min<int64_t>(rows, p.S_q);
  }
  const size_t nbk = (size_t)p.nbuckets + 1;
  const size_t entries = (size_t)p.B * p.G * p.chunk_rows * p.topk;  // the partial states one pass holds
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  if (!p.direct) {
    ap.off_counts = take(nbk * 4);
    ap.off_offsets = take(nbk * 4);
    ap.off_cursor = take(nbk * 4);
    ap.off_item_off = take(nbk * 4);
    ap.off_nitems = take(4);
    ap.off_entries = take(entries * 4);
    // items: at most one partial item per bucket plus entries / tpi full ones
    ap.off_items = take(((size_t)p.nbuckets + entries / p.tpi + 1) * 4);
  }
  const size_t prow = entries * (size_t)p.r;  // (b, i, g, slot, head)
  ap.off_po = take(prow * p.d * elem_bytes(s->dtype));
  ap.off_pl = take(prow * 4);
  ap.bytes = off;
  return ap;
}

// Backward: the main branch's gather (never direct) with work items of
// msa::kBwdTokensPerItem tokens and one workgroup per possible item, dispatched as
// slots free; plus rowsum(dO * O).
AttnPlan plan_bwd(const msa_shape* s, size_t* off_dsum) {
  msa_shape s2 = *s;
  AttnPlan ap = plan_attn(&s2, nullptr);
  msa::AttnParams& p = ap.p;
  if (p.direct) {  // redo the layout with the gather regions
    p.direct = 0;
    const size_t nbk = (size_t)p.nbuckets + 1;
    const size_t entries = (size_t)p.B * p.G * p.S_q * p.topk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
      const size_t o = off;
      off += align_up(bytes);
      return o;
    };
    ap.off_counts = take(nbk * 4);
    ap.off_offsets = take(nbk * 4);
    ap.off_cursor = take(nbk * 4);
    ap.off_item_off = take(nbk * 4);
    ap.off_nitems = take(4);
    ap.off_entries = take(entries * 4);
    ap.off_items = take(((size_t)p.nbuckets + entries / msa::kBwdTokensPerItem + 1) * 4);
    ap.off_po = take(entries * (size_t)p.r * p.d * 2);
    ap.off_pl = take(entries * (size_t)p.r * 4);
    ap.bytes = off;
  }
  p.tpi = msa::kBwdTokensPerItem;
  // items: at most one partial item per bucket plus entries / tpi full ones
  p.grid = (int)std::min<int64_t>((int64_t)p.nbuckets + (int64_t)p.B * p.G * p.S_q * p.topk / p.tpi + 1, 1 << 30);
  *off_dsum = ap.bytes;
  ap.bytes += align_up((size_t)s->batch * s->num_q_heads * s->q_len * 4);
  return ap;
}

void bind_attn(AttnPlan& ap, char* ws) {
  msa::AttnParams& p = ap.p;
  if (!p.direct) {
    p.counts = (int32_t*)(ws + ap.off_counts);
    p.offsets = (int32_t*)(ws + ap.off_offsets);
    p.cursor = (int32_t*)(ws + ap.off_cursor);
    p.item_off = (int32_t*)(ws + ap.off_item_off);
    p.n_items = (int32_t*)(ws + ap.off_nitems);
    p.entries = (int32_t*)(ws + ap.off_entries);
    p.item_bucket = (int32_t*)(ws + ap.off_items);
  }
  p.part_o = ws + ap.off_po;
  p.part_lse = (float*)(ws + ap.off_pl);
}

size_t sel_bytes(const msa_shape* s) {
  return align_up((size_t)s->batch * s->num_kv_heads * s->q_len * s->topk * 4);
}

msa_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MSA_OK;
  if (!ws) return fail(MSA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (((uintptr_t)ws) % kAlign != 0) return fail(MSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return MSA_OK;
}

// An error left by an earlier, unrelated HIP call on this thread would be read
// back by hipGetLastError after our launches; drop it first so a status names
// only this call's failures.
void clear_stale_hip_error() { (void)hipGetLastError(); }

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- the allocation-free entry point's scratch ---------------------------
//
// msa_fwd_noalloc takes its workspace from this array (each GPU the library runs
// on holds its own copy until the process ends).  In host code the name is only
// a stand-in: kernels get the device address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept below.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

msa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

const char* msa_version(void) { return "0.2.0"; }

msa_status msa_set_kernel_timer(int kernel, void* start_event, void* stop_event) {
  if (kernel < MSA_KERNEL_NONE || kernel > MSA_KERNEL_BWD_COMBINE)
    return fail(MSA_ERR_INVALID, "unknown kernel id %d", kernel);
  if (kernel == MSA_KERNEL_NONE || !start_event || !stop_event) {
    g_timer = {0, nullptr, nullptr};
    return MSA_OK;
  }
  g_timer = {kernel, (hipEvent_t)start_event, (hipEvent_t)stop_event};
  return MSA_OK;
}

const char* msa_status_string(msa_status st) {
  switch (st) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID: return "MSA_ERR_INVALID";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

size_t msa_workspace_size_kvcache(const msa_shape* s, const msa_kv_cache* cache, int op) {
  const std::string saved = g_last_error;
  size_t r = 0;
  if (op >= MSA_OP_INDEX_SELECT && op <= MSA_OP_SPARSE_ATTN_BWD && check_shape(s, op) == MSA_OK &&
      check_cache(s, cache) == MSA_OK && s->q_len > 0) {
    if (op == MSA_OP_INDEX_SELECT) r = plan_index(s, cache).bytes;
    else if (op == MSA_OP_SPARSE_ATTN) r = plan_attn(s, cache, kTokensPerItem, true).bytes;
    else if (op == MSA_OP_KL_TEACHER) r = plan_attn(s, cache, msa::kKlTokensPerItem).bytes;
    else if (op == MSA_OP_SPARSE_ATTN_BWD) {
      size_t od = 0;
      r = cache ? 0 : plan_bwd(s, &od).bytes;
    }
    else r = sel_bytes(s) + std::max(plan_index(s, cache).bytes, plan_attn(s, cache, kTokensPerItem, true).bytes);
  }
  g_last_error = saved;
  return r;
}

size_t msa_workspace_size(const msa_shape* s, int op) { return msa_workspace_size_kvcache(s, nullptr, op); }

msa_status msa_index_select_kvcache(const msa_shape* s, const msa_kv_cache* cache, const void* q_idx,
                                    const void* k_idx, int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_shape(s, MSA_OP_INDEX_SELECT);
  if (st != MSA_OK || (st = check_cache(s, cache)) != MSA_OK) return st;
  if (!q_idx || !k_idx || !sel) return fail(MSA_ERR_INVALID, "q_idx, k_idx and sel must be non-NULL");
  if (s->q_len == 0) return MSA_OK;
  IndexPlan ip = plan_index(s, cache);
  if ((st = check_ws(ws, ws_bytes, ip.bytes)) != MSA_OK) return st;
  bind_index(ip, (char*)ws, q_idx, k_idx, sel);
  clear_stale_hip_error();
  return hip_status(msa::launch_index_select(ip.p, s->dtype == MSA_BF16, fp8_cache(s), s->index_dim,
                                             (hipStream_t)stream, timer()),
                    "index select launch");
}

msa_status msa_index_select(const msa_shape* s, const void* q_idx, const void* k_idx, int32_t* sel, void* ws,
                            size_t ws_bytes, void* stream) {
  return msa_index_select_kvcache(s, nullptr, q_idx, k_idx, sel, ws, ws_bytes, stream);
}

msa_status msa_sparse_attn_fwd_kvcache(const msa_shape* s, const msa_kv_cache* cache, const void* q, const void* k,
                                       const void* v, const int32_t* sel, void* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream) {
  msa_status st = check_shape(s, MSA_OP_SPARSE_ATTN);
  if (st != MSA_OK || (st = check_cache(s, cache)) != MSA_OK) return st;
  if (!q || !k || !v || !sel || !out) return fail(MSA_ERR_INVALID, "q, k, v, sel and out must be non-NULL");
  if (s->q_len == 0) return MSA_OK;
  AttnPlan ap = plan_attn(s, cache, kTokensPerItem, true);
  if ((st = check_ws(ws, ws_bytes, ap.bytes)) != MSA_OK) return st;
  bind_attn(ap, (char*)ws);
  ap.p.q = q;
  ap.p.k = k;
  ap.p.v = v;
  ap.p.sel = sel;
  ap.p.out = out;
  ap.p.lse = lse;
  clear_stale_hip_error();
  return hip_status(msa::launch_sparse_attention(ap.p, s->dtype == MSA_BF16, fp8_cache(s), (hipStream_t)stream,
                                                 timer()),
                    "sparse attention launch");
}

msa_status msa_sparse_attn_fwd(const msa_shape* s, const void* q, const void* k, const void* v, const int32_t* sel,
                               void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return msa_sparse_attn_fwd_kvcache(s, nullptr, q, k, v, sel, out, lse, ws, ws_bytes, stream);
}

msa_status msa_fwd_kvcache(const msa_shape* s, const msa_kv_cache* cache, const void* q, const void* k,
                           const void* v, const void* q_idx, const void* k_idx, void* out, int32_t* sel_out,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_shape(s, MSA_OP_FWD);
  if (st != MSA_OK || (st = check_cache(s, cache)) != MSA_OK) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !out)
    return fail(MSA_ERR_INVALID, "q, k, v, q_idx, k_idx and out must be non-NULL");
  if (s->q_len == 0) return MSA_OK;
  IndexPlan ip = plan_index(s, cache);
  AttnPlan ap = plan_attn(s, cache, kTokensPerItem, true);
  const size_t need = sel_bytes(s) + std::max(ip.bytes, ap.bytes);
  if ((st = check_ws(ws, ws_bytes, need)) != MSA_OK) return st;
  char* w = (char*)ws;
  int32_t* sel = sel_out ? sel_out : (int32_t*)w;
  char* scratch = w + sel_bytes(s);  // index lists and attention state reuse one region
  bind_index(ip, scratch, q_idx, k_idx, sel);
  // the decode rows kernel merges the split lists itself (it writes no partial
  // state, so the lists stay intact in the shared region)
  const bool merge_in_rows = ap.p.rows_mode && ip.lists;
  ip.p.merge_in_consumer = merge_in_rows ? 1 : 0;
  hipStream_t hs = (hipStream_t)stream;
  clear_stale_hip_error();
  st = hip_status(msa::launch_index_select(ip.p, s->dtype == MSA_BF16, fp8_cache(s), s->index_dim, hs, timer()),
                  "index select launch");
  if (st != MSA_OK) return st;
  bind_attn(ap, scratch);
  ap.p.q = q;
  ap.p.k = k;
  ap.p.v = v;
  ap.p.sel = sel;
  ap.p.out = out;
  ap.p.lse = lse;
  if (merge_in_rows) {
    ap.p.lists_s = ip.p.part_s;
    ap.p.lists_i = ip.p.part_i;
    ap.p.list_cap = ip.cap;
    ap.p.list_stride = ip.p.nsplit * ip.p.lps;
    ap.p.list_chunk = ip.p.chunk;
    ap.p.list_lps = ip.p.lps;
    ap.p.sel_w = sel;
  }
  return hip_status(msa::launch_sparse_attention(ap.p, s->dtype == MSA_BF16, fp8_cache(s), hs, timer()),
                    "sparse attention launch");
}

msa_status msa_kl_teacher_fwd_kvcache(const msa_shape* s, const msa_kv_cache* cache, const void* q, const void* k,
                                      const void* q_idx, const void* k_idx, const int32_t* sel, const float* lse,
                                      float index_scale, float* kl, float* idx_lse, void* ws, size_t ws_bytes,
                                      void* stream) {
  msa_status st = check_shape(s, MSA_OP_KL_TEACHER);
  if (st != MSA_OK || (st = check_cache(s, cache)) != MSA_OK) return st;
  if (!q || !k || !q_idx || !k_idx || !sel || !lse || !kl)
    return fail(MSA_ERR_INVALID, "q, k, q_idx, k_idx, sel, lse and kl must be non-NULL");
  if (!std::isfinite(index_scale)) return fail(MSA_ERR_INVALID, "index_scale must be finite");
  if (s->q_len == 0) return MSA_OK;
  AttnPlan ap = plan_attn(s, cache, msa::kKlTokensPerItem);
  if ((st = check_ws(ws, ws_bytes, ap.bytes)) != MSA_OK) return st;
  bind_attn(ap, (char*)ws);
  ap.p.q = q;
  ap.p.k = k;
  ap.p.sel = sel;
  // the per-block terms take the place of the partial outputs (3 floats per
  // (token, group, slot) against r * d values)
  msa::KlParams kp{q_idx, k_idx, lse, index_scale, s->index_dim, (float*)ap.p.part_o, kl, idx_lse};
  clear_stale_hip_error();
  return hip_status(msa::launch_kl_teacher(ap.p, kp, s->dtype == MSA_BF16, fp8_cache(s), (hipStream_t)stream, timer()),
                    "KL teacher launch");
}

msa_status msa_kl_teacher_fwd(const msa_shape* s, const void* q, const void* k, const void* q_idx, const void* k_idx,
                              const int32_t* sel, const float* lse, float index_scale, float* kl, float* idx_lse,
                              void* ws, size_t ws_bytes, void* stream) {
  return msa_kl_teacher_fwd_kvcache(s, nullptr, q, k, q_idx, k_idx, sel, lse, index_scale, kl, idx_lse, ws, ws_bytes,
                                    stream);
}

msa_status msa_sparse_attn_bwd(const msa_shape* s, const void* q, const void* k, const void* v, const int32_t* sel,
                               const void* out, const float* lse, const void* dout, float* dq, float* dk, float* dv,
                               void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_shape(s, MSA_OP_SPARSE_ATTN_BWD);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !sel || !out || !lse || !dout || !dq || !dk || !dv)
    return fail(MSA_ERR_INVALID, "q, k, v, sel, out, lse, dout, dq, dk and dv must be non-NULL");
  if (s->q_len == 0) return MSA_OK;
  size_t off_dsum = 0;
  AttnPlan ap = plan_bwd(s, &off_dsum);
  if ((st = check_ws(ws, ws_bytes, ap.bytes)) != MSA_OK) return st;
  bind_attn(ap, (char*)ws);
  ap.p.q = q;
  ap.p.k = k;
  ap.p.v = v;
  ap.p.sel = sel;
  const float scale = s->softmax_scale != 0.0f ? s->softmax_scale : 1.0f / std::sqrt((float)s->head_dim);
  msa::BwdParams bp{out, dout, lse, (float*)((char*)ws + off_dsum), dq, dk, dv, scale};
  clear_stale_hip_error();
  return hip_status(msa::launch_sparse_attention_bwd(ap.p, bp, (hipStream_t)stream, timer()), "backward launch");
}

msa_status msa_fwd(const msa_shape* s, const void* q, const void* k, const void* v, const void* q_idx,
                   const void* k_idx, void* out, int32_t* sel_out, float* lse, void* ws, size_t ws_bytes,
                   void* stream) {
  return msa_fwd_kvcache(s, nullptr, q, k, v, q_idx, k_idx, out, sel_out, lse, ws, ws_bytes, stream);
}

size_t msa_noalloc_scratch_bytes(void) { return kScratchBytes; }

msa_status msa_fwd_noalloc(const msa_shape* s, const void* q, const void* k, const void* v, const void* q_idx,
                           const void* k_idx, void* out, int32_t* sel_out, float* lse, void* stream) {
  // the checks msa_fwd runs, first, so that errors name the arguments, not the scratch
  msa_status st = check_shape(s, MSA_OP_FWD);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !out)
    return fail(MSA_ERR_INVALID, "q, k, v, q_idx, k_idx and out must be non-NULL");
  if (s->q_len == 0) return MSA_OK;
  const size_t need =
      sel_bytes(s) + std::max(plan_index(s, nullptr).bytes, plan_attn(s, nullptr, kTokensPerItem, true).bytes);
  if (need > kScratchBytes)
    return fail(MSA_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; msa_fwd_noalloc holds %zu (use msa_fwd)",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != MSA_OK) return st;
  return msa_fwd_kvcache(s, nullptr, q, k, v, q_idx, k_idx, out, sel_out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"

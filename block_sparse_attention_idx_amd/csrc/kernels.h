// Kernel parameter blocks and launchers shared by the host API and the .hip
// translation units.  Host-only code includes this; device code lives in the
// .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;  // Bk: tokens per KV block, fixed on the GPU path
constexpr int kBwdTokensPerItem = 512;  // query tokens per backward work item (dK, dV meet in fp32 atomics)
constexpr int kKlTokensPerItem = 64;    // query tokens per KL-teacher work item (their index scores fit in LDS)
constexpr int kMaxItemTokens = 256;     // most query tokens per KV-outer attention item (its LDS entry list)

// Optional events recorded around one kernel (see msa_set_kernel_timer).
struct KernelTimer {
  int which;  // msa_kernel id, 0 = off
  hipEvent_t start, stop;
};

inline void timer_start(const KernelTimer* t, int which, hipStream_t s) {
  if (t && t->which == which) (void)hipEventRecord(t->start, s);
}
inline void timer_stop(const KernelTimer* t, int which, hipStream_t s) {
  if (t && t->which == which) (void)hipEventRecord(t->stop, s);
}

enum { kKernIndexScore = 1, kKernTopkMerge = 2, kKernGather = 3, kKernAttention = 4, kKernCombine = 5,
       kKernKlTeacher = 6, kKernKlCombine = 7, kKernBwd = 8, kKernBwdCombine = 9 };

// Where the caches (k, v, k_idx) of each sequence live.  Without a length
// table every sequence holds S_k tokens and its query row 0 sits at q_offset;
// with one, sequence b holds seq_lens[b] tokens (clamped to [0, S_k]) and its
// query row i sits at seq_lens[b] - S_q + i.  Without a page table a cache is
// a dense [B, H, S_k, W] tensor; with one it is a pool [num_pages, H, 128, W]
// and logical block c of sequence b is page pages[b * max_pages + c].
struct CacheMap {
  const int32_t* seq_lens;  // [B] or null
  const int32_t* pages;     // [B, max_pages] or null
  int max_pages, num_pages;
};

__device__ __forceinline__ int cache_len(const CacheMap& m, int S_k, int b) {
  return m.seq_lens ? min(max(m.seq_lens[b], 0), S_k) : S_k;
}

// Absolute position of query row 0 of sequence b (negative: leading rows see no key).
__device__ __forceinline__ int64_t first_pos(const CacheMap& m, int64_t q_offset, int S_q, int S_k, int b) {
  return m.seq_lens ? (int64_t)cache_len(m, S_k, b) - S_q : q_offset;
}

// Local block of position t; -1 for a row before the cache start.
__device__ __forceinline__ int local_block(int64_t t) { return t >= 0 ? (int)(t / kBlock) : -1; }

// Element offset of token 0 of logical block c, head hidx, of sequence b in a
// cache of H heads and W elements per token; -1 when its page id is out of range.
__device__ __forceinline__ int64_t block_offset(const CacheMap& m, int S_k, int H, int W, int b, int hidx, int c) {
  if (!m.pages) return (((int64_t)b * H + hidx) * S_k + (int64_t)c * kBlock) * W;
  const int pg = m.pages[(int64_t)b * m.max_pages + c];
  if (pg < 0 || pg >= m.num_pages) return -1;
  return (((int64_t)pg * H + hidx) * kBlock) * W;
}

// Whether block c of sequence b can be read (always, without a page table).
__device__ __forceinline__ bool block_mapped(const CacheMap& m, int b, int c) {
  if (!m.pages) return true;
  const int pg = m.pages[(int64_t)b * m.max_pages + c];
  return pg >= 0 && pg < m.num_pages;
}

// Index branch (index_topk.hip).
struct IndexParams {
  const void* q_idx;   // [B, S_q, G, D]
  const void* k_idx;   // [B, S_k, D]
  float* part_s;       // [B*S_q*G, nsplit * lps, CAP] partial top-list scores
  int32_t* part_i;     // same shape: block ids (-1 = empty)
  int32_t* sel;        // [B, G, S_q, topk]
  CacheMap cm;
  int64_t q_offset;
  int B, S_q, S_k, G, topk;
  int rows_per_b;      // S_q * G
  int ntile;           // row tiles per sequence
  int ntile_total;     // B * ntile
  int nsplit, chunk;   // key-block splits and blocks per split
  int lps;             // partial lists per (row, split): 1, or 2 / 8 in the wide form (one per lane half)
  int nunits;          // ntile_total * nsplit
  int grid_per_xcd;    // ceil(nunits / 8)
  int small;           // 1: bf16 queries and rows_per_b <= kIndexSmallRows, one unit per (sequence, split)
  int rows_wg;         // (row, group) pairs per row tile
  // With per-sequence lengths: the units that hold work, packed as
  // (row tile << 7) | split by index_units_kernel, and their number.  Null otherwise.
  int32_t* units;
  int32_t* unit_count;
  // With per-sequence lengths in the few-row form and B <= 64 * kInlineUnitsPerLane:
  // each wave finds its unit from the lengths itself (units and unit_count null).
  int units_inline;
  int merge_in_consumer;  // host only: the lists are merged by the decode rows kernel, not topk_merge_kernel
  // One key split and one unit per row tile, heaviest first (no unit list):
  // the launch may run the units on a persistent grid (index_topk_kernel).
  int persist;
};

// At most this many (row, group) pairs per sequence: the index kernel's
// few-row form (each wave ranks whole blocks on its own).
constexpr int kIndexSmallRows = 32;
// Sequences per lane when a wave derives its unit from the lengths (B <= 256).
constexpr int kInlineUnitsPerLane = 4;

// Top lists hold up to k - 1 entries: 15 (k <= 16), 31 (k <= 32) or 63
// (k <= 64).  Lists of 63 (the wide form) are not merged inside the index
// kernels: every lane half writes its own list (2 per split in the prefill form,
// 8 in the few-row form) and topk_merge_kernel merges them, at most
// kMergeMaxLists per row.
constexpr int kIndexWideCap = 63;
constexpr int kMergeMaxLists = 128;
constexpr int index_cap(int topk) { return topk <= 16 ? 15 : topk <= 32 ? 31 : kIndexWideCap; }
// Rows per topk_merge_kernel workgroup, and the most lists per row whose
// scores and ids fit 64 KiB of LDS for all of them.
constexpr int merge_rows_per_wg(int cap) { return cap == kIndexWideCap ? 1 : 4; }
constexpr int merge_max_lists(int cap) {
  return 65536 / (2 * merge_rows_per_wg(cap) * cap * 4) < kMergeMaxLists ? 65536 / (2 * merge_rows_per_wg(cap) * cap * 4)
                                                                           : kMergeMaxLists;
}

// Index rows per workgroup: waves x 32 rows x RT row tiles, RT = 2 for lists
// of up to 15 entries (k <= 16), 1 for the longer lists.  bf16 queries with
// lists of up to 31 entries run 8 waves (one workgroup per CU, two waves per
// SIMD); fp32 queries and lists of 63 fill a SIMD's registers with one wave,
// so they run 4.
constexpr int index_row_tiles(int topk) { return topk <= 16 ? 2 : 1; }
constexpr int index_waves(int topk, bool bf16) { return bf16 && index_cap(topk) != kIndexWideCap ? 8 : 4; }
constexpr int index_rows_per_wg(int topk, bool bf16) { return index_waves(topk, bf16) * 32 * index_row_tiles(topk); }

// fp8_keys: k_idx holds OCP FP8 E4M3 values (q_idx bf16).
hipError_t launch_index_select(const IndexParams& p, bool bf16_inputs, bool fp8_keys, int index_dim, hipStream_t s,
                               const KernelTimer* timer);

// Main branch (attn.hip).
struct AttnParams {
  const void* q;       // [B, S_q, Hq, d]
  const void* k;       // [B, G, S_k, d]
  const void* v;       // [B, G, S_k, d]
  const int32_t* sel;  // [B, G, S_q, topk]
  void* out;           // [B, S_q, Hq, d]
  float* lse;          // [B, Hq, S_q] or null
  CacheMap cm;
  // query gather (bucket = (b, g, c))
  int32_t* counts;     // [nbuckets]
  int32_t* offsets;    // [nbuckets + 1]
  int32_t* cursor;     // [nbuckets]
  int32_t* item_off;   // [nbuckets + 1]: first work item of each bucket
  int32_t* entries;    // [B*G*S_q*topk]: (query row << 6) | slot, grouped by bucket
  int32_t* item_bucket;  // [max items]: bucket of each work item
  int32_t* n_items;    // device scalar
  // partial softmax states per (b, i, g, slot, head)
  void* part_o;        // o / l in the partial dtype, [.., d]
  float* part_lse;     // log2 of sum_j 2^(s'_j), s' = scale * log2(e) * q.k
  int64_t q_offset;
  int B, S_q, S_k, Hq, G, r, d, topk;
  // Query rows [row0, row0 + nrows) of every sequence are gathered, attended and
  // combined by one pass; the partial states hold those rows only, indexed
  // ((b * nrows + i - row0) * G + g) * topk + slot.  One pass covers all rows
  // unless the caller capped the workspace (chunk_rows < S_q).
  int row0, nrows, chunk_rows;
  int nb;              // key blocks per sequence, ceil(S_k / 128)
  int nbuckets;        // B * G * nb
  int tpi;             // query tokens per work item
  int direct;          // 1: one item per selection entry, no gather
  int64_t n_direct;    // B * G * S_q * topk when direct
  int grid;            // persistent grid size of the attention kernel
  int grid_decode;     // persistent grid size of the decode-form attention kernel
  float scale_log2;    // softmax scale * key scale * log2(e)
  float v_scale;       // dequantisation scale of the value cache (1 if none)
  int out_f32;         // output dtype: 1 fp32, 0 input dtype
  // Decode rows form (direct, bf16 queries, enough rows): one workgroup per
  // (b, i, g) row runs the whole main branch, no partial states or combine.
  int rows_mode;
  // with it, the index kernel's partial lists when it left them unmerged
  // (lists_s null: sel holds the selection); the rows kernel then writes sel
  const float* lists_s;    // [rows, list_stride, list_cap]
  const int32_t* lists_i;
  int list_cap, list_stride, list_chunk, list_lps;
  int32_t* sel_w;          // the selection buffer the merged rows are written to
};

// Rows (B * S_q * G) from which decode uses the rows form: one workgroup per
// row fills the 256 CUs.
constexpr int kDecodeRowsMin = 256;

// fp8_cache: k and v hold OCP FP8 E4M3 values (q and the partial states bf16).
hipError_t launch_sparse_attention(const AttnParams& p, bool bf16_inputs, bool fp8_cache, hipStream_t s,
                                   const KernelTimer* timer);

// Query gather of the KV-outer kernels (nothing when p.direct).
void launch_gather(const AttnParams& p, hipStream_t s, const KernelTimer* timer);

// KL-alignment teacher (kl.hip): the main branch's token sets and work items,
// plus the index tensors, the main branch's lse and the outputs.
struct KlParams {
  const void* q_idx;   // [B, S_q, G, D_idx]
  const void* k_idx;   // [B, S_k, D_idx] (or a page pool)
  const float* lse;    // [B, Hq, S_q] main-branch log-sum-exp (natural log)
  float index_scale;   // multiplies the raw index scores before their softmax
  int index_dim;
  float* part;         // [B, S_q, G, topk, 3]: per block sum pbar (log pbar - s), max s, sum exp(s - max)
  float* kl;           // [B, G, S_q]
  float* idx_lse;      // [B, G, S_q] or null
};

hipError_t launch_kl_teacher(const AttnParams& p, const KlParams& kp, bool bf16_inputs, bool fp8_cache,
                             hipStream_t s, const KernelTimer* timer);

// Backward of the main branch (bwd.hip): bf16 q, k, v, out and dout; fp32
// gradients.  The gather cuts buckets into work items of p.tpi tokens and
// p.part_o holds the bf16 dQ partials.
struct BwdParams {
  const void* out;     // [B, S_q, Hq, d] forward output
  const void* dout;    // [B, S_q, Hq, d] its gradient
  const float* lse;    // [B, Hq, S_q] forward log-sum-exp (natural log)
  float* dsum;         // [B, Hq, S_q] workspace: rowsum(dout * out)
  float* dq;           // [B, S_q, Hq, d]
  float* dk;           // [B, G, S_k, d]
  float* dv;           // [B, G, S_k, d]
  float scale;         // softmax scale (key scale included)
};

hipError_t launch_sparse_attention_bwd(const AttnParams& p, const BwdParams& bp, hipStream_t s,
                                       const KernelTimer* timer);

}  // namespace msa

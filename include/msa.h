/*
 * msa.h - C ABI of the MiniMax Sparse Attention (MSA) forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  MSA is block-sparse grouped-query attention with two
 * branches (abstract page "MiniMax 稀疏注意力", sections 摘要 and 核心贡献;
 * snilld.dk page "MiniMax lancerer MSA", section "Hvad er MSA i praksis"):
 *
 *  - Index branch.  For every GQA group g (G = num_kv_heads groups, one
 *    index-query head each) and every query row i at absolute position
 *    t = q_offset + i, the raw dot products of q_idx[b,i,g,:] with the single
 *    shared index-key head k_idx[b,j,:] are max-pooled over absolute blocks of
 *    Bk tokens (block c = tokens [c*Bk, (c+1)*Bk)).  With L = floor(t / Bk)
 *    the query's local block, the selection is L plus the best min(k-1, L) of
 *    the full blocks 0..L-1, ranked by block score descending and, on equal
 *    scores, block index ascending.  Ranking is done on raw scores: softmax is
 *    monotone, so no exponential is needed (the exp-free Top-k of the
 *    abstract).  Selections are per group and are never pooled across index
 *    heads (issue write-up "Substantial numerical differences with Minimax MSA
 *    attention vs Minimax's Reference", sections 原因分析 and 解决步骤).
 *  - Main branch.  Query head h belongs to group g = floor(h / r), r = Hq/G.
 *    It attends with exact scaled-dot-product softmax to the causally visible
 *    tokens (j <= t) of its group's selected blocks: one softmax over their
 *    union, keys and values of KV head g.
 *
 * Layouts (all dense, contiguous, row-major; e = 4 bytes for MSA_F32, 2 for
 * MSA_BF16, 1 for FP8 caches):
 *    q, out   [B, S_q, Hq, d]
 *    k, v     [B, Hkv, S_k, d]       one (head, block) is a contiguous span
 *    q_idx    [B, S_q, G, D_idx]     G = Hkv index-query heads
 *    k_idx    [B, S_k, D_idx]        the one shared index-key head
 *    sel      int32 [B, G, S_q, k]   ascending block ids, then -1 padding
 *    lse      fp32 [B, Hq, S_q]      natural-log log-sum-exp of the scaled
 *                                    scores over the attended tokens
 *
 * Ownership and threading.  Every data pointer is a device pointer owned by
 * the caller.  The library allocates no device memory; scratch memory is the
 * caller's workspace (256-byte aligned, at least msa_workspace_size() bytes),
 * except for msa_fwd_noalloc, which works in a fixed scratch array of the
 * library's own (see there).  Work is enqueued on the given HIP stream
 * (hipStream_t passed as void*, NULL = the null stream) and the calls return
 * without synchronising.  Different threads may call concurrently on
 * different streams with different workspaces.  Three things persist between
 * calls: the profiling hook of msa_set_kernel_timer (thread-local, off unless
 * set), msa_fwd_noalloc's scratch with its per-device address, and, per
 * device, the number of index-kernel workgroups the GPU holds at once (CU
 * count x occupancy, queried once; it sizes the index kernel's persistent
 * grid and changes no result).
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; on
 * an error nothing is launched and outputs are untouched.  A failed launch
 * returns MSA_ERR_HIP.  msa_last_error() gives a thread-local message for the
 * last failing call of the calling thread.  Device faults surface at the
 * caller's synchronisation.
 *
 * Caches in FP8.  The pages list FP8 among the precisions of the MSA
 * inference kernel (aiforradalom.online page "MiniMax új eljárása
 * 28-szorosára csökkenti az AI-figyelem számítási igényét", section
 * "Elérhetőség"), without fixing a format.  Here, with cache_format =
 * MSA_CACHE_FP8_E4M3, k, v and k_idx hold OCP FP8 E4M3 (e4m3fn) bytes while
 * q, q_idx and the output stay in dtype (which must be MSA_BF16).  The keys
 * and values attended to are k_scale * k and v_scale * v (per-tensor
 * dequantisation scales).  Index keys are used as stored: a positive common
 * scale would not change any ranking, so none is taken.
 *
 * Supported on the GPU: block_size == 128; 1 <= topk <= 64; head_dim in
 * {64, 128}; index_dim in {32, 64, 128}; r = Hq / Hkv in {1, 2, 4, 8, 16,
 * 32}; dtype MSA_F32 or MSA_BF16 (the same for q, k, v, q_idx, k_idx unless
 * the caches are FP8); out_dtype MSA_F32 or the input dtype.  Other values
 * give MSA_ERR_UNSUPPORTED.  Selections are exact when the index inputs make
 * every index score exactly representable in fp32 (for example small
 * integers).
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID = -1,      /* a null pointer, a negative or inconsistent size */
  MSA_ERR_UNSUPPORTED = -2,  /* a valid shape the library has no kernel for    */
  MSA_ERR_WORKSPACE = -3,    /* workspace missing, too small or misaligned      */
  MSA_ERR_HIP = -4           /* a HIP launch or runtime call failed             */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

/* Element format of the caches k, v and k_idx. */
typedef enum {
  MSA_CACHE_NATIVE = 0,   /* the same dtype as q                                */
  MSA_CACHE_FP8_E4M3 = 1  /* OCP FP8 E4M3 bytes; requires dtype == MSA_BF16      */
} msa_cache_format;

typedef struct {
  int32_t batch;        /* B: sequences                                         */
  int32_t q_len;        /* S_q: query rows per sequence (0 = nothing to do)     */
  int32_t kv_len;       /* S_k: cached tokens per sequence, >= q_offset + S_q   */
  int32_t cache_format; /* msa_cache_format of k, v and k_idx                   */
  int64_t q_offset;     /* absolute position of query row 0 (every sequence)    */
  int32_t num_q_heads;  /* Hq                                                   */
  int32_t num_kv_heads; /* Hkv = G, also the number of index-query heads        */
  int32_t head_dim;     /* d                                                    */
  int32_t index_dim;    /* D_idx                                                */
  int32_t block_size;   /* Bk                                                   */
  int32_t topk;         /* k: blocks per (query, group), local block included   */
  float softmax_scale;  /* main-branch scale; 0 means 1/sqrt(d)                 */
  int32_t dtype;        /* msa_dtype of q and q_idx (and of the native caches)  */
  int32_t out_dtype;    /* msa_dtype of out                                     */
  float k_scale;        /* keys attended to are k_scale * k; 0 means 1          */
  float v_scale;        /* values attended to are v_scale * v; 0 means 1        */
  int32_t workspace_cap_mib; /* 0, or a bound on the main branch's partial states */
} msa_shape;            /* 72 bytes                                             */

/* workspace_cap_mib.  The KV-outer main branch keeps one partial softmax state
 * per selection entry (about r * d * e bytes per (query row, group, slot); 16 GiB
 * for B = 2, S_q = 32768, Hq = 64, d = 128, k = 16 in bf16).  With a cap > 0, a
 * call that gathers queries (prefill; decode-sized calls never do) processes the
 * query rows in chunks of as many rows of every sequence as keep the partial
 * states within that many MiB (at least one row per chunk), reusing one region;
 * msa_workspace_size reports the smaller workspace that results.  The results do
 * not depend on the cap.  Negative values are invalid. */

enum { MSA_OP_INDEX_SELECT = 0, MSA_OP_SPARSE_ATTN = 1, MSA_OP_FWD = 2, MSA_OP_KL_TEACHER = 3,
       MSA_OP_SPARSE_ATTN_BWD = 4 };

/* Bytes of workspace the given op needs for this shape (0 when the shape is
 * invalid or unsupported; the call itself then reports why).  The same shape
 * always gives the same size. */
size_t msa_workspace_size(const msa_shape* shape, int op);

/* Index branch: block max-pooled index scores and the per-group exp-free
 * Top-k with the forced local block (snilld.dk page, "Hvad er MSA i praksis";
 * the issue write-up, 解决步骤, for the per-index-head [B, H_idx, S_q, topk]
 * result).  Reads q_idx and k_idx, writes sel [B, G, S_q, k].  The token score
 * matrix is never stored: block maxima stream through a running Top-k. */
msa_status msa_index_select(const msa_shape* shape, const void* q_idx, const void* k_idx,
                            int32_t* sel, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Main branch for a given selection: exact softmax attention of every query
 * head over the visible tokens of its group's selected blocks (snilld.dk page,
 * "Hvad er MSA i praksis"), computed KV-block-outer with the queries that chose
 * each block gathered together (snilld.dk page, "Teknisk forklaring …"; the
 * abstract page, 引言, on the swapped FlashAttention loop order).  sel rows must
 * hold distinct block ids <= the row's local block, ascending, -1 padded, and
 * must contain the local block.  lse may be NULL. */
msa_status msa_sparse_attn_fwd(const msa_shape* shape, const void* q, const void* k,
                               const void* v, const int32_t* sel, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Both branches.  sel_out (may be NULL) receives the selection; lse may be NULL. */
msa_status msa_fwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                   const void* q_idx, const void* k_idx, void* out, int32_t* sel_out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Without a workspace --------------------------------------------------
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): msa_fwd with
 * the library's own scratch instead of a caller workspace.  Arguments, results
 * and errors are those of msa_fwd.  The scratch is a static device array of
 * msa_noalloc_scratch_bytes() bytes (64 MiB) that each GPU the library runs on
 * holds until the process ends; its device address is looked up on the first
 * call on each device (with that device current).  Shapes whose workspace
 * (msa_workspace_size(shape, MSA_OP_FWD)) exceeds it are refused with
 * MSA_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * the same array: calls that overlap on one GPU (different streams, or other
 * threads) race and give undefined results; calls ordered on one stream are
 * fine.  Nothing is allocated or freed by the call. */
msa_status msa_fwd_noalloc(const msa_shape* shape, const void* q, const void* k, const void* v,
                           const void* q_idx, const void* k_idx, void* out, int32_t* sel_out, float* lse,
                           void* stream);

/* Bytes of the scratch msa_fwd_noalloc works in. */
size_t msa_noalloc_scratch_bytes(void);

/* ---- Caches of unequal length, optionally paged -------------------------
 *
 * Serving batches hold KV caches that grow and differ in length (snilld.dk
 * page, sections "POC målinger og miljø" and "Implementering i produktion":
 * batches of 1-4 sequences at 4k-128k contexts, growing KV caches in long
 * conversations).  The *_kvcache calls take the same shape plus this
 * descriptor:
 *
 *  - seq_lens (device int32 [B], or NULL): sequence b holds seq_lens[b] tokens
 *    (values are clamped to [0, kv_len]) and its query row i sits at
 *    t = seq_lens[b] - q_len + i; shape->q_offset must then be 0.  Rows with
 *    t < 0 precede their cache: their selection is all -1, their output 0 and
 *    their lse -inf.  NULL: every sequence holds kv_len tokens and row i sits
 *    at q_offset + i, as in the plain calls.
 *  - page_table (device int32 [B, max_pages], or NULL): the caches are pools of
 *    128-token pages, k and v [num_pages, Hkv, 128, d] and k_idx
 *    [num_pages, 128, D_idx]; logical block c (tokens [128c, 128c + 128)) of
 *    sequence b is page page_table[b * max_pages + c].  kv_len, the longest
 *    cache, must be <= max_pages * 128.  Page ids outside [0, num_pages) are
 *    never read: such a block is neither ranked nor attended.  NULL: the caches
 *    are dense, k and v [B, Hkv, kv_len, d] and k_idx [B, kv_len, D_idx].
 *
 * Selections hold logical block ids.  Everything else (dtypes, FP8 caches,
 * scales, workspace rules, errors) is as for the plain calls, which are the
 * *_kvcache calls with cache == NULL. */
typedef struct {
  const int32_t* seq_lens;   /* [B] device, or NULL                               */
  const int32_t* page_table; /* [B, max_pages] device, or NULL                    */
  int32_t max_pages;         /* columns of page_table (ignored without one)       */
  int32_t num_pages;         /* pages in each pool (ignored without a page table) */
} msa_kv_cache;

/* Workspace for the *_kvcache calls (it depends on whether lengths are given). */
size_t msa_workspace_size_kvcache(const msa_shape* shape, const msa_kv_cache* cache, int op);

msa_status msa_index_select_kvcache(const msa_shape* shape, const msa_kv_cache* cache, const void* q_idx,
                                    const void* k_idx, int32_t* sel, void* workspace, size_t workspace_bytes,
                                    void* stream);

msa_status msa_sparse_attn_fwd_kvcache(const msa_shape* shape, const msa_kv_cache* cache, const void* q,
                                       const void* k, const void* v, const int32_t* sel, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream);

msa_status msa_fwd_kvcache(const msa_shape* shape, const msa_kv_cache* cache, const void* q, const void* k,
                           const void* v, const void* q_idx, const void* k_idx, void* out, int32_t* sel_out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---- KL-alignment teacher (forward only) ---------------------------------
 *
 * Top-k is not differentiable, so MSA trains the index branch with a KL loss
 * towards the main branch; the teacher is the main distribution over the
 * selected tokens averaged over the heads of the GQA group (snilld.dk page,
 * section "Træning og stabilisering"; Hungarian page, section "A betanítás és
 * a kernel-optimalizáció").  For each (b, g, i), with T the tokens the main
 * branch attends to (the visible tokens of the selected blocks):
 *    pbar(j)  = mean over the r heads h of group g of softmax_T(scale * q_h . k_j)
 *    log q(j) = log_softmax_T(index_scale * q_idx[b,i,g,:] . k_idx[b,j,:])
 *    kl[b,g,i]      = sum_{j in T} pbar(j) * (log pbar(j) - log q(j))   (natural log)
 *    idx_lse[b,g,i] = log sum_{j in T} exp(index_scale * q_idx . k_idx_j)
 * sel and lse are those of the forward (msa_fwd's sel_out and lse, or any
 * selection with the main branch's lse for it); the teacher then needs no
 * second softmax pass.  kl and idx_lse are fp32 [B, G, S_q]; idx_lse may be
 * NULL.  A row that sees no token gets kl = 0 and idx_lse = -inf.
 * index_scale must be finite (1 keeps the raw scores the selection ranks).
 * The shape, caches, FP8 format and k_scale are as for the main branch
 * (v_scale is not used); workspace: msa_workspace_size(shape,
 * MSA_OP_KL_TEACHER). */
msa_status msa_kl_teacher_fwd(const msa_shape* shape, const void* q, const void* k, const void* q_idx,
                              const void* k_idx, const int32_t* sel, const float* lse, float index_scale,
                              float* kl, float* idx_lse, void* workspace, size_t workspace_bytes, void* stream);

msa_status msa_kl_teacher_fwd_kvcache(const msa_shape* shape, const msa_kv_cache* cache, const void* q,
                                      const void* k, const void* q_idx, const void* k_idx, const int32_t* sel,
                                      const float* lse, float index_scale, float* kl, float* idx_lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- Backward of the main branch ------------------------------------------
 *
 * MSA-PT and MSA-CPT train the model with sparse attention (snilld.dk page,
 * section "Træning og stabilisering"); the pages name no backward kernel.
 * Top-k is not differentiable, so the selection is held constant and each
 * query row gets the gradient of exact softmax attention over its token set T
 * (as in msa_sparse_attn_fwd): with p = softmax_T(scale q.k), o = sum p v and
 * the output gradient dO,
 *    dV[b,g,j] += p_j dO,   dS_j = p_j (dO.v_j - dO.o),
 *    dQ[b,i,h] = scale sum_j dS_j k_j,   dK[b,g,j] += scale dS_j q[b,i,h].
 * Inputs: q, k, v, sel and the forward's out and lse (natural log), dout like
 * out; all bf16 except lse.  Outputs dq [B, S_q, Hq, d], dk and dv
 * [B, Hkv, S_k, d], fp32; keys no query attends get zero.  dk and dv sum the
 * contributions of a block's query groups with fp32 atomics, so their last
 * bits may differ between calls; dq is summed in a fixed order.  Built for
 * dtype == out_dtype == MSA_BF16, native caches and k_scale, v_scale in
 * {0, 1}; workspace: msa_workspace_size(shape, MSA_OP_SPARSE_ATTN_BWD). */
msa_status msa_sparse_attn_bwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                               const int32_t* sel, const void* out, const float* lse, const void* dout,
                               float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Kernels of the forward path, for msa_set_kernel_timer. */
typedef enum {
  MSA_KERNEL_NONE = 0,
  MSA_KERNEL_INDEX_SCORE = 1, /* index scores, block max-pool, partial top lists */
  MSA_KERNEL_TOPK_MERGE = 2,  /* merge of the partial lists, local block, -1 pad   */
  MSA_KERNEL_GATHER = 3,      /* query gather: histogram, scan, scatter (4 launches) */
  MSA_KERNEL_ATTENTION = 4,   /* KV-outer sparse attention (partial states)         */
  MSA_KERNEL_COMBINE = 5,     /* merge of the partial states into out and lse       */
  MSA_KERNEL_KL_TEACHER = 6,  /* KL teacher: per-block terms                        */
  MSA_KERNEL_KL_COMBINE = 7,  /* KL teacher: per-row totals                         */
  MSA_KERNEL_BWD = 8,         /* backward: block gradients and dQ partials          */
  MSA_KERNEL_BWD_COMBINE = 9  /* backward: dQ partials summed                        */
} msa_kernel;

/* Profiling hook (thread-local state: the one exception to calls being
 * independent of each other).  For the calling thread, every later msa_* call
 * records start_event (a hipEvent_t) on its stream right before launching
 * `kernel` and stop_event right after it, so hipEventElapsedTime gives that
 * kernel's own duration.  kernel = MSA_KERNEL_NONE (or NULL events) turns the
 * hook off; it is off until set.  The events stay owned by the caller.  A call
 * captured into a HIP graph while the hook is set records the two event nodes
 * into the graph, and every replay records them again: turn the hook off
 * before capturing.  A kernel a call does not launch
 * records nothing: decode calls with bf16 queries and at least 256
 * (batch, query row, group) rows run the merge of the split lists, the
 * attention and the combine as one kernel, timed as MSA_KERNEL_ATTENTION. */
msa_status msa_set_kernel_timer(int kernel, void* start_event, void* stop_event);

/* Static string naming a status code. */
const char* msa_status_string(msa_status status);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* msa_last_error(void);

/* Library version, e.g. "0.2.0". */
const char* msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */

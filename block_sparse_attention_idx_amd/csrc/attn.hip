// Main branch of MSA on gfx950: exact softmax attention over the selected
// blocks, computed KV-block-outer.
//
// Method (snilld.dk page "MiniMax lancerer MSA", sections "Hvad er MSA i
// praksis" and "Teknisk forklaring hvorfor kompleksiteten skifter"; abstract
// page "MiniMax 稀疏注意力", 摘要 and 引言): each query head attends with one
// exact softmax to the causally visible tokens of its group's selected blocks.
// The sparse path iterates over KV blocks and gathers, for each block, the
// queries that selected it, which keeps reads of the KV cache contiguous and
// raises arithmetic intensity; this is the FlashAttention skeleton with its
// two loops swapped.
//
// Pipeline (all on the caller's stream, no host round trip):
//   1. gather_hist / gather_scan / item_table: bucket every selection entry
//      (b, g, i, slot) by its block (b, g, c): LDS histograms with one global
//      atomic per bin, exclusive scan, scatter.  A bucket is cut into work items
//      of up to tpi query tokens.
//   2. attn_kvouter: a persistent grid walks the work items.  An item stages
//      K (128 x d) and V^T (d x 128) of its block in LDS once, then runs passes
//      of 4 waves x 32 rows; a row is one (token, head) and the r heads of a
//      token are adjacent rows, so the whole group shares the staged tile.
//      S^T = K Q^T and O^T = V^T P^T are 32x32 MFMA tiles; every lane owns one
//      row, so the block-local softmax needs one cross-half exchange.  The
//      result is a partial state per (token, slot, head): o / l in the input
//      dtype plus the fp32 log2-sum-exp of the block's scaled scores.
//   3. combine: per (token, head) the partial states of its slots are merged
//      (weights 2^(lse_s - max)) into the output and the log-sum-exp.
// With S_q small (decode) the gather is skipped: one item per selection entry,
// or, with bf16 queries and enough (b, i, g) rows to give every CU one, the
// rows form: one workgroup per row merges the index kernel's split lists,
// attends over the row's blocks with a running softmax and writes the row, so
// neither partial states nor the merge and combine launches are needed.
//
// K and V may be stored as OCP FP8 E4M3 (storage type S = e4m3, compute type
// T = bf16): staging widens them exactly to bf16, the per-tensor key scale is
// folded into the softmax scale and the value scale is applied by the combine.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace msa {

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Query gather.  A workgroup takes kGatherRows query rows of one (b, g),
// histograms their selection entries in LDS, and adds each non-zero bin to the
// global bucket count with one atomic.  The scatter pass redoes the histogram,
// reserves one contiguous range per bin with one atomic on the bucket cursor,
// and places entries with LDS atomics.  The order of entries inside a bucket is
// arbitrary; every entry's result is computed independently of its neighbours.
constexpr int kGatherRows = 256;
constexpr int kMaxHistBins = 16384;  // 64 KiB of LDS counters

template <bool SCATTER>
__global__ __launch_bounds__(256) void gather_hist_kernel(AttnParams p) {
  extern __shared__ int32_t hist[];
  const int bg = blockIdx.y;
  const int i0 = p.row0 + blockIdx.x * kGatherRows;
  const int rows = min(kGatherRows, p.row0 + p.nrows - i0);
  for (int c = threadIdx.x; c < p.nb; c += 256) hist[c] = 0;
  __syncthreads();
  const int32_t* sbase = p.sel + ((int64_t)bg * p.S_q + i0) * p.topk;
  const int n = rows * p.topk;
  for (int e = threadIdx.x; e < n; e += 256) {
    const int c = sbase[e];
    if (c >= 0 && c < p.nb) atomicAdd(&hist[c], 1);  // ids outside the cache are ignored
  }
  __syncthreads();
  int32_t* gcount = (SCATTER ? p.cursor : p.counts) + (int64_t)bg * p.nb;
  for (int c = threadIdx.x; c < p.nb; c += 256) {
    const int h = hist[c];
    if (h) {
      const int base = atomicAdd(&gcount[c], h);
      if (SCATTER) hist[c] = base;
    }
  }
  if (!SCATTER) return;
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += 256) {
    const int c = sbase[e];
    if (c >= 0 && c < p.nb) {
      const int pos = atomicAdd(&hist[c], 1);
      const int i = i0 + e / p.topk, slot = e - (e / p.topk) * p.topk;
      p.entries[pos] = (i << 6) | slot;
    }
  }
}

// Same result for caches too long for an LDS histogram: one global atomic per entry.
__global__ __launch_bounds__(256) void gather_count_kernel(AttnParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over the pass's rows
  const int64_t total = (int64_t)p.B * p.G * p.nrows * p.topk;
  if (e >= total) return;
  const int64_t per_bg = (int64_t)p.nrows * p.topk;
  const int64_t bg = e / per_bg;  // b * G + g
  const int c = p.sel[(bg * p.S_q + p.row0) * p.topk + (e - bg * per_bg)];
  if (c < 0 || c >= p.nb) return;
  atomicAdd(&p.counts[bg * p.nb + c], 1);
}

// item -> bucket table: one thread per bucket writes the ids of its items.
__global__ __launch_bounds__(256) void item_table_kernel(AttnParams p) {
  const int bk = blockIdx.x * 256 + threadIdx.x;
  if (bk >= p.nbuckets) return;
  const int a = p.item_off[bk], e = p.item_off[bk + 1];
  for (int it = a; it < e; ++it) p.item_bucket[it] = bk;
}

__global__ __launch_bounds__(256) void gather_scatter_kernel(AttnParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over the pass's rows
  const int64_t total = (int64_t)p.B * p.G * p.nrows * p.topk;
  if (e >= total) return;
  const int slot = (int)(e % p.topk);
  const int64_t rest = e / p.topk;
  const int i = p.row0 + (int)(rest % p.nrows);
  const int64_t bg = rest / p.nrows;
  const int c = p.sel[(bg * p.S_q + i) * p.topk + slot];
  if (c < 0 || c >= p.nb) return;
  const int pos = atomicAdd(&p.cursor[bg * p.nb + c], 1);
  p.entries[pos] = (i << 6) | slot;
}

// Single workgroup: exclusive scans of the bucket sizes (entries and items).
__global__ __launch_bounds__(1024) void gather_scan_kernel(AttnParams p) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_itm[1024];
  const int n = p.nbuckets;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int32_t cs = 0, is = 0;
  for (int j = lo; j < hi; ++j) {
    const int32_t c = p.counts[j];
    cs += c;
    is += (c + p.tpi - 1) / p.tpi;
  }
  s_cnt[threadIdx.x] = cs;
  s_itm[threadIdx.x] = is;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t a = 0, b2 = 0;
    if ((int)threadIdx.x >= off) {
      a = s_cnt[threadIdx.x - off];
      b2 = s_itm[threadIdx.x - off];
    }
    __syncthreads();
    s_cnt[threadIdx.x] += a;
    s_itm[threadIdx.x] += b2;
    __syncthreads();
  }
  int32_t co = s_cnt[threadIdx.x] - cs, io = s_itm[threadIdx.x] - is;  // exclusive
  for (int j = lo; j < hi; ++j) {
    const int32_t c = p.counts[j];
    p.offsets[j] = co;
    p.cursor[j] = co;
    p.item_off[j] = io;
    co += c;
    io += (c + p.tpi - 1) / p.tpi;
  }
  if (threadIdx.x == 1023) {
    p.offsets[n] = s_cnt[1023];
    p.item_off[n] = s_itm[1023];
    *p.n_items = s_itm[1023];
  }
}

template <typename T, typename S, int D, int R>
// two workgroups per CU for bf16; the fp32 form (correctness path) takes the registers of one
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void attn_kvouter_kernel(AttnParams p) {
  using M = Mma<T>;
  using IO = ChunkIO<T, S>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
  constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int LDK = D + E;              // K row pitch (elements)
  // V^T row pitch: 8 bytes beyond a multiple of 256 B, so the 32 rows one
  // 8-byte read instruction touches fall in distinct LDS banks
  constexpr int LDV = kBlock + 8 / (int)sizeof(T);
  constexpr int TPW = 32 / R;             // query tokens per wave per pass
  constexpr int TPP = 4 * TPW;            // query tokens per pass
  constexpr int NDT = D / 32;             // 32-wide output tiles along d
  constexpr int NPV = kBlock / KSTEP;     // PV instructions per d tile
  __shared__ __align__(16) T Ks[kBlock * LDK];
  __shared__ __align__(16) T Vt[D * LDV];
  __shared__ int32_t tok_s[kMaxItemTokens];  // the item's (row << 6) | slot entries

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t total = p.direct ? p.n_direct : (int64_t)*p.n_items;

  for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
    int b, g, c, ntok;
    const int32_t* toks;
    int32_t direct_tok = 0;
    if (p.direct) {
      c = p.sel[item];
      if (c < 0 || c >= p.nb) continue;  // uniform across the workgroup
      const int slot = (int)(item % p.topk);
      const int64_t rest = item / p.topk;
      const int i = (int)(rest % p.S_q);
      const int64_t bg = rest / p.S_q;
      g = (int)(bg % p.G);
      b = (int)(bg / p.G);
      direct_tok = (i << 6) | slot;
      toks = nullptr;
      ntok = 1;
    } else {
      const int bk = p.item_bucket[item];
      const int start = (int)(item - p.item_off[bk]) * p.tpi;
      ntok = min(p.tpi, p.counts[bk] - start);
      toks = p.entries + p.offsets[bk] + start;
      c = bk % p.nb;
      const int bg = bk / p.nb;
      g = bg % p.G;
      b = bg / p.G;
    }

    // an unmapped page, or a block past the end of the cache: nothing to attend (uniform)
    const int slen = cache_len(p.cm, p.S_k, b);
    const int64_t kv0 = block_offset(p.cm, p.S_k, p.G, D, b, g, c);
    if (kv0 < 0 || (int64_t)c * kBlock >= slen) continue;
    const int64_t qo = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b);

    __syncthreads();  // the previous item is done with the LDS tiles
    {
      const int rows_ok = (int)min((int64_t)kBlock, (int64_t)slen - (int64_t)c * kBlock);
      // Every load below is unconditional (rows past the cache end re-read its
      // last row and are zeroed afterwards), so all of them are in flight at once.
      constexpr int KCH = kBlock * D / E;
      static_assert(KCH % 256 == 0, "K staging covers the block exactly");
      constexpr int KU = KCH / 256;
      constexpr int VT = (D / E) * (kBlock / E);
      constexpr int VU = (VT + 255) / 256;
      const S* ksrc = (const S*)p.k + kv0;
      const S* vsrc = (const S*)p.v + kv0;
      typename IO::raw kx[KU];
      typename IO::raw vin[VU][E];
      // the item's entries go to LDS with the staging, so no pass waits on a global read for its rows
      const int32_t ent = toks ? toks[min((int)threadIdx.x, ntok - 1)] : direct_tok;
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int ch = threadIdx.x + u * 256;
        const int row = ch / (D / E), col = ch - row * (D / E);
        kx[u] = IO::load(ksrc + (int64_t)min(row, rows_ok - 1) * D + col * E);
      }
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int tl = min((int)threadIdx.x + u * 256, VT - 1);
        const int dg = tl % (D / E), kg = tl / (D / E);
#pragma unroll
        for (int r = 0; r < E; ++r)
          vin[u][r] = IO::load(vsrc + (int64_t)min(kg * E + r, rows_ok - 1) * D + dg * E);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep every staging load ahead of the first use
      if ((int)threadIdx.x < ntok) tok_s[threadIdx.x] = ent;
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int ch = threadIdx.x + u * 256;
        const int row = ch / (D / E), col = ch - row * (D / E);
        i32x4 x = IO::widen(kx[u]);
        if (row >= rows_ok) x = i32x4{};
        *(i32x4*)&Ks[row * LDK + col * E] = x;
      }
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int tl = threadIdx.x + u * 256;
        if (VT % 256 != 0 && tl >= VT) break;
        const int dg = tl % (D / E), kg = tl / (D / E);
        i32x4 vw[E];
#pragma unroll
        for (int r = 0; r < E; ++r) vw[r] = kg * E + r < rows_ok ? IO::widen(vin[u][r]) : i32x4{};
        i32x4 outc[E];
        transpose_tile<T, E>(vw, outc);
#pragma unroll
        for (int r = 0; r < E; ++r) {  // rows are 8-byte aligned: two 8-byte stores
          uint2* dst = (uint2*)&Vt[(dg * E + r) * LDV + kg * E];
          dst[0] = make_uint2((uint32_t)outc[r][0], (uint32_t)outc[r][1]);
          dst[1] = make_uint2((uint32_t)outc[r][2], (uint32_t)outc[r][3]);
        }
      }
    }
    __syncthreads();

    const int64_t key0 = (int64_t)c * kBlock;
    for (int p0 = 0; p0 < ntok; p0 += TPP) {
      if (p0 + wave * TPW >= ntok) continue;  // this wave has no rows in this pass
      const int tslot = p0 + wave * TPW + l32 / R;
      const bool in_list = tslot < ntok;
      const int32_t entry = in_list ? tok_s[tslot] : 0;
      const int i = entry >> 6, slot = entry & 63;
      // keys of this block visible to the row: index within block <= lim
      const int64_t rel = qo + i - key0;  // query position relative to the block
      const bool rv = in_list && rel >= 0;        // a block after the query is skipped
      const int lim = (!rv || rel >= kBlock) ? kBlock : (int)rel;
      const int hh = l32 % R;
      const int head = g * R + hh;

      // rows that are skipped still read a valid Q row (entry 0) and are never stored
      frag qf[NKS];
      {
        const T* qrow = (const T*)p.q + (((int64_t)b * p.S_q + i) * p.Hq + head) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const frag*)(qrow + ks * KSTEP + h * KPL);
      }
      __builtin_amdgcn_sched_barrier(0);  // all Q loads in flight before the first MFMA
      f32x16 sacc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const frag a = *(const frag*)&Ks[(kt * 32 + l32) * LDK + ks * KSTEP + h * KPL];
          sacc[kt] = M::mma(a, qf[ks], sacc[kt]);
        }
      }
      // the causal mask only bites in a row's local block
      if (__any(lim < kBlock - 1)) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (kt * 32 + c_row(j, h) > lim) sacc[kt][j] = kNegInf;
      }
      // block-local softmax in log2 units: p = 2^(s * scale*log2(e) - m), scale > 0
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kt][j]);
      mx = wave_max_xor32(mx);
      const float sl2 = p.scale_log2;
      const float moff = -mx * sl2;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][j], sl2, moff));
          sacc[kt][j] = e;
          lsum += e;
        }
      lsum = xor_sum<32>(lsum);

      // O^T = V^T P^T.  Instruction ks2 consumes registers j0..j0+KPL-1 of key
      // tile kt; the A operand supplies V^T for exactly those keys.
      f32x16 oacc[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
      for (int ks2 = 0; ks2 < NPV; ++ks2) {
        const int kt = (ks2 * KPL) / 16, j0 = (ks2 * KPL) % 16;
        frag pb;
        if constexpr (KPL == 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = from_f32<T>(sacc[kt][j0 + e]);
        } else {
          pb = sacc[kt][j0];
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* vrow = &Vt[(dt * 32 + l32) * LDV + kt * 32];
          frag va;
          if constexpr (KPL == 8) {
            // keys c_row(j0 + e, h): two runs of four
            const bf16x4 lo4 = *(const bf16x4*)(vrow + c_row(j0, h));
            const bf16x4 hi4 = *(const bf16x4*)(vrow + c_row(j0 + 4, h));
            va = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          } else {
            va = vrow[c_row(j0, h)];
          }
          oacc[dt] = M::mma(va, pb, oacc[dt]);
        }
      }

      // Partial state of this (token, slot): o / l in the lane-native order of the
      // O^T tile (chunk q of lane (head, h) at ((q * 2 + h) * R + head) * 16 bytes),
      // so one store instruction writes 2 * R * 16 contiguous bytes per token.
      if (rv) {
        const float inv = 1.0f / lsum;
        const int64_t ptok = (((int64_t)b * p.nrows + i - p.row0) * p.G + g) * p.topk + slot;
        T* po = (T*)p.part_o + ptok * (R * D);
        constexpr int NQ = NDT * 16 / E;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          Chunk16 w;
          if constexpr (sizeof(T) == 2) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(oacc[(q * 8 + e) / 16][(q * 8 + e) % 16] * inv);
            w = __builtin_bit_cast(Chunk16, v);
          } else {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = oacc[(q * 4 + e) / 16][(q * 4 + e) % 16] * inv;
            w = __builtin_bit_cast(Chunk16, v);
          }
          // streamed out and read once by the combine: keep it out of the caches' way
          __builtin_nontemporal_store(__builtin_bit_cast(i32x4, w), (i32x4*)(po + ((q * 2 + h) * R + hh) * E));
        }
        if (h == 0) __builtin_nontemporal_store(mx * sl2 + __builtin_amdgcn_logf(lsum), &p.part_lse[ptok * R + hh]);
      }
    }
  }
}

// Decode form of the main branch: one work item = one selection entry
// (b, g, i, slot), i.e. the r rows of one token against one block.  All four
// waves work on the item: wave w scores keys [32w, 32w + 32) (S^T = K Q^T with K
// read straight from global memory as the A operand), the block-local softmax
// is combined across waves through LDS, P^T goes to LDS, and wave w then forms
// the d-slice [32w, 32w + 32) of O^T = V^T P^T from the LDS copies of V^T and
// P^T.  The partial state is written in the same lane-native layout as the
// KV-outer kernel, so the combine is shared.
template <typename T, typename S, int D, int R>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnParams p) {
  using M = Mma<T>;
  using IO = ChunkIO<T, S>;
  // K fragments come straight from global memory: KPL elements of S per lane
  constexpr bool kNative = std::is_same<S, T>::value;
  typedef typename std::conditional<kNative, typename Mma<T>::frag, uint2>::type kraw;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
  constexpr int E = 16 / (int)sizeof(T);
  constexpr int LDV = kBlock + E;  // V^T pitch (elements), 16-byte aligned rows
  constexpr int LDP = kBlock + E;  // P^T pitch
  constexpr int NDT = D / 32;
  constexpr int NPV = kBlock / KSTEP;
  static_assert(R <= 32, "one 32-row tile holds the token's heads");
  __shared__ __align__(16) T Vt[D * LDV];
  __shared__ __align__(16) T Ps[32 * LDP];
  __shared__ float red_m[4][32];
  __shared__ float red_l[4][32];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const float sl2 = p.scale_log2;

  for (int64_t item = blockIdx.x; item < p.n_direct; item += gridDim.x) {
    const int c = p.sel[item];
    if (c < 0 || c >= p.nb) continue;  // uniform across the workgroup
    const int slot = (int)(item % p.topk);
    const int64_t rest = item / p.topk;
    const int i = (int)(rest % p.S_q);
    const int64_t bg = rest / p.S_q;
    const int g = (int)(bg % p.G);
    const int b = (int)(bg / p.G);
    const int64_t key0 = (int64_t)c * kBlock;
    const int slen = cache_len(p.cm, p.S_k, b);
    const int64_t rel = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + i - key0;
    if (rel < 0 || key0 >= slen) continue;  // a block after the query: nothing visible (uniform)
    const int64_t kv0 = block_offset(p.cm, p.S_k, p.G, D, b, g, c);
    if (kv0 < 0) continue;  // an unmapped page is never read; the combine skips it too
    const int lim = rel >= kBlock ? kBlock : (int)rel;
    const int rows_ok = (int)min((int64_t)kBlock, (int64_t)slen - key0);

    // loads: this wave's 32 K rows (A operand), the token's Q rows (B operand), and
    // this thread's share of V; all issued before any is used
    const int krow = min(wave * 32 + l32, rows_ok - 1);
    const S* kp = (const S*)p.k + kv0 + (int64_t)krow * D;
    const int qh = l32 < R ? l32 : 0;  // rows past r repeat head 0 and are never stored
    const T* qp = (const T*)p.q + (((int64_t)b * p.S_q + i) * p.Hq + g * R + qh) * D;
    kraw ka[NKS];
    frag qb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      ka[ks] = *(const kraw*)(kp + ks * KSTEP + h * KPL);
      qb[ks] = *(const frag*)(qp + ks * KSTEP + h * KPL);
    }
    constexpr int VT = (D / E) * (kBlock / E);
    constexpr int VU = (VT + 255) / 256;
    typename IO::raw vin[VU][E];
    const S* vsrc = (const S*)p.v + kv0;
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int tl = min((int)threadIdx.x + u * 256, VT - 1);
      const int dg = tl % (D / E), kg = tl / (D / E);
#pragma unroll
      for (int r = 0; r < E; ++r)
        vin[u][r] = IO::load(vsrc + (int64_t)min(kg * E + r, rows_ok - 1) * D + dg * E);
    }
    __builtin_amdgcn_sched_barrier(0);

    __syncthreads();  // the previous item is done with the LDS tiles
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int tl = threadIdx.x + u * 256;
      if (VT % 256 != 0 && tl >= VT) break;
      const int dg = tl % (D / E), kg = tl / (D / E);
      i32x4 vw[E];
#pragma unroll
      for (int r = 0; r < E; ++r) vw[r] = kg * E + r < rows_ok ? IO::widen(vin[u][r]) : i32x4{};
      i32x4 outc[E];
      transpose_tile<T, E>(vw, outc);
#pragma unroll
      for (int r = 0; r < E; ++r) *(i32x4*)&Vt[(dg * E + r) * LDV + kg * E] = outc[r];
    }

    // S^T for keys [32w, 32w + 32): lane (row l32, half h) holds keys 32w + c_row(j, h)
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      frag a;
      if constexpr (kNative) a = ka[ks];
      else a = __builtin_bit_cast(frag, IO::widen(ka[ks]));
      sacc = M::mma(a, qb[ks], sacc);
    }
    if (lim < kBlock - 1) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (wave * 32 + c_row(j, h) > lim) sacc[j] = kNegInf;
    }
    float mw = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; ++j) mw = fmaxf(mw, sacc[j]);
    mw = wave_max_xor32(mw);
    if (h == 0) red_m[wave][l32] = mw;
    __syncthreads();
    const float mx = fmaxf(fmaxf(red_m[0][l32], red_m[1][l32]), fmaxf(red_m[2][l32], red_m[3][l32]));
    const float moff = -mx * sl2;
    float lw = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], sl2, moff));
      sacc[j] = e;
      lw += e;
    }
    lw = xor_sum<32>(lw);
    if (h == 0) red_l[wave][l32] = lw;
    // P^T row l32: keys 32w + c_row(j, h) come in runs of four
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      T* dst = &Ps[l32 * LDP + wave * 32 + q4 * 8 + h * 4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(sacc[q4 * 4 + e]);
    }
    __syncthreads();

    if (wave < NDT) {
      // O^T slice d in [32w, 32w + 32) over all 128 keys, natural key order
      f32x16 oacc = f32x16{};
#pragma unroll
      for (int ks2 = 0; ks2 < NPV; ++ks2) {
        const frag va = *(const frag*)&Vt[(wave * 32 + l32) * LDV + ks2 * KSTEP + h * KPL];
        const frag pb = *(const frag*)&Ps[l32 * LDP + ks2 * KSTEP + h * KPL];
        oacc = M::mma(va, pb, oacc);
      }
      const float lsum = red_l[0][l32] + red_l[1][l32] + red_l[2][l32] + red_l[3][l32];
      if (l32 < R) {
        const float inv = 1.0f / lsum;
        const int64_t ptok = (((int64_t)b * p.nrows + i - p.row0) * p.G + g) * p.topk + slot;
        T* po = (T*)p.part_o + ptok * (R * D);
        // lane-native chunks q = (wave * 16 + j) / E of this lane's registers
#pragma unroll
        for (int qq = 0; qq < 16 / E; ++qq) {
          const int q = wave * (16 / E) + qq;
          Chunk16 w;
          T* wv = (T*)&w;
#pragma unroll
          for (int e = 0; e < E; ++e) wv[e] = from_f32<T>(oacc[qq * E + e] * inv);
          __builtin_nontemporal_store(__builtin_bit_cast(i32x4, w), (i32x4*)(po + ((q * 2 + h) * R + l32) * E));
        }
        if (wave == 0 && h == 0)
          __builtin_nontemporal_store(mx * sl2 + __builtin_amdgcn_logf(lsum), &p.part_lse[ptok * R + l32]);
      }
    }
  }
}

// Decode rows form: one workgroup per (b, i, g) row runs the row's whole main
// branch -- the merge of the index kernel's split lists when it left them,
// attention over the selected blocks with a running softmax, and the row's
// output and log-sum-exp -- so no partial state goes through HBM and no merge
// or combine kernel runs.  8 waves in two teams of 4: team u takes the row's
// visible selected blocks u, u + 2, ... (ascending ids).  Per block, each wave
// of the team scores 32 of the block's keys (K read straight from HBM as the A
// operand), the block's row maxima and sums meet in the team's LDS, P^T and V^T
// go to the team's LDS, and wave w accumulates the d-slice [32w, 32w + 32) of
// O^T, rescaled by 2^(m_old - m_new) when the running maximum grows.  The next
// block's K and V are loaded while the current one is computed.  At the end the
// two teams' (m, l, O) are merged and the row is written.
template <typename S, int D, int R>
__global__ __launch_bounds__(512) void attn_decode_rows_kernel(AttnParams p) {
  using T = bf16;
  using M = Mma<T>;
  using IO = ChunkIO<T, S>;
  constexpr bool kNative = std::is_same<S, T>::value;
  typedef typename std::conditional<kNative, typename Mma<T>::frag, uint2>::type kraw;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
  constexpr int E = 8;             // bf16 per 16-byte chunk
  constexpr int LDV = kBlock + E;  // V^T pitch (elements), 16-byte aligned rows
  constexpr int LDP = kBlock + E;  // P^T pitch
  constexpr int NDT = D / 32;      // waves of a team that own a d-slice of O^T
  constexpr int NPV = kBlock / KSTEP;
  constexpr int VT = (D / E) * (kBlock / E);  // 8x8 transpose tiles of a V block
  constexpr int VU = (VT + 255) / 256;        // per thread of a team
  static_assert(R <= 32, "one 32-row tile holds the token's heads");
  constexpr int TEAM_BYTES = (D * LDV + 32 * LDP) * (int)sizeof(T);
  constexpr int MERGE_BYTES = kMergeMaxLists * kIndexWideCap * 8;  // the largest list set of a row
  constexpr int XBYTES = 4 * 16 * 64 * 4 + 64 * 4;                 // team 1's O^T, m and l at the end
  constexpr int RAW = 2 * TEAM_BYTES > MERGE_BYTES ? 2 * TEAM_BYTES : MERGE_BYTES;
  static_assert(RAW >= XBYTES, "the final exchange fits");
  __shared__ __align__(16) char raw[RAW];
  __shared__ float red_m[2][4][32];
  __shared__ float red_l[2][4][32];
  __shared__ int pos_s[64];  // the row's selection by position
  __shared__ int blk_s[64];  // its visible blocks, ascending
  __shared__ int64_t off_s[64];  // and their element offsets in k and v (pages resolved here, once)
  __shared__ int nv_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int team = wave >> 2, wt = wave & 3, ttid = tid & 255;
  const int h = lane >> 5, l32 = lane & 31;
  const float sl2 = p.scale_log2;
  const int64_t row = blockIdx.x;  // (b * S_q + i) * G + g
  const int g = (int)(row % p.G);
  const int64_t bi = row / p.G;  // b * S_q + i
  const int i = (int)(bi % p.S_q);
  const int b = (int)(bi / p.S_q);
  const int64_t t = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + i;
  const int L = local_block(t);
  const int slen = cache_len(p.cm, p.S_k, b);

  // the token's query rows (rows past r repeat head 0 and are never stored)
  frag qb[NKS];
  {
    const int qh = l32 < R ? l32 : 0;
    const T* qp = (const T*)p.q + (bi * p.Hq + g * R + qh) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qb[ks] = *(const frag*)(qp + ks * KSTEP + h * KPL);
  }

  // the row's selection (merged here from the split lists, or read) and its
  // visible, mapped blocks in ascending order
  if (wave == 0) {
    const int64_t srow = (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
    pos_s[lane] = -1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (p.lists_s) {  // merge the split lists; the selection goes to sel_w
      if (L >= 0) {
        const int nl = L > 0 ? (L + p.list_chunk - 1) / p.list_chunk * p.list_lps : 0;
        const int64_t base = row * p.list_stride * p.list_cap;
        float* ss = (float*)raw;
        int* si = (int*)(raw + MERGE_BYTES / 2);
        const MergedSlot m =
            merge_row_lists(p.lists_s + base, p.lists_i + base, nl, p.list_cap, min(p.topk - 1, L), L, ss, si, lane);
        if (m.pos >= 0) {
          p.sel_w[srow + m.pos] = m.id;
          pos_s[m.pos] = m.id;
        } else if (lane < p.topk) {
          p.sel_w[srow + lane] = -1;
        }
      } else if (lane < p.topk) {
        p.sel_w[srow + lane] = -1;  // a row before the start of its cache selects nothing
      }
    } else if (L >= 0 && lane < p.topk) {
      pos_s[lane] = p.sel[srow + lane];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int c = lane < p.topk ? pos_s[lane] : -1;
    const int64_t key0 = (int64_t)c * kBlock;
    const bool ok = c >= 0 && c < p.nb && key0 <= t && key0 < slen && block_mapped(p.cm, b, c);
    const uint64_t bal = __ballot(ok);
    if (ok) {
      const int ci = __popcll(bal & ((1ull << lane) - 1));
      blk_s[ci] = c;
      off_s[ci] = block_offset(p.cm, p.S_k, p.G, D, b, g, c);
    }
    if (lane == 0) nv_s = __popcll(bal);
  }
  __syncthreads();
  const int nv = nv_s;

  // one block of the team: this wave's 32 K rows and this thread's share of V
  struct Blk {
    kraw ka[NKS];
    typename IO::raw vin[VU][E];
    int lim, rows_ok;
    bool has;
  };
  // A team without a block still issues its loads (row 0 at the start of the
  // pool, always valid memory; the values are not used), so that every path
  // leaves the same loads in flight and no wait covers the next block's.
  auto load_blk = [&](int j, Blk& x) {
    const int ci = 2 * j + team;
    x.has = ci < nv;  // uniform across the team
    int64_t kv0 = 0;
    x.lim = 0;
    x.rows_ok = 1;
    if (x.has) {
      const int c = blk_s[ci];
      const int64_t key0 = (int64_t)c * kBlock;
      const int64_t rel = t - key0;
      x.lim = rel >= kBlock ? kBlock : (int)rel;
      x.rows_ok = (int)min((int64_t)kBlock, (int64_t)slen - key0);
      kv0 = off_s[ci];
    }
    const int krow = min(wt * 32 + l32, x.rows_ok - 1);
    const S* kp = (const S*)p.k + kv0 + (int64_t)krow * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) x.ka[ks] = *(const kraw*)(kp + ks * KSTEP + h * KPL);
    const S* vsrc = (const S*)p.v + kv0;
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int tl = min(ttid + u * 256, VT - 1);
      const int dg = tl % (D / E), kg = tl / (D / E);
#pragma unroll
      for (int r = 0; r < E; ++r)
        x.vin[u][r] = IO::load(vsrc + (int64_t)min(kg * E + r, x.rows_ok - 1) * D + dg * E);
    }
  };

  T* Vt = (T*)(raw + team * TEAM_BYTES);
  T* Ps = Vt + D * LDV;
  float m_run = kNegInf, l_run = 0.f;  // of row l32, the same in every lane of the row
  f32x16 oacc = f32x16{};
  auto step = [&](const Blk& x) {
    __syncthreads();  // the previous block's V^T and P^T reads are done (and the list merge)
    f32x16 sacc;  // defined (and used) only when the team has a block
    if (x.has) {
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int tl = ttid + u * 256;
        if (VT % 256 != 0 && tl >= VT) break;
        const int dg = tl % (D / E), kg = tl / (D / E);
        i32x4 vw[E];
#pragma unroll
        for (int r = 0; r < E; ++r) vw[r] = kg * E + r < x.rows_ok ? IO::widen(x.vin[u][r]) : i32x4{};
        i32x4 outc[E];
        transpose_tile<T, E>(vw, outc);
#pragma unroll
        for (int r = 0; r < E; ++r) *(i32x4*)&Vt[(dg * E + r) * LDV + kg * E] = outc[r];
      }
      // S^T for keys [32 wt, 32 wt + 32): lane (row l32, half h) holds keys 32 wt + c_row(j, h)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        frag a;
        if constexpr (kNative) a = x.ka[ks];
        else a = __builtin_bit_cast(frag, IO::widen(x.ka[ks]));
        sacc = M::mma(a, qb[ks], ks == 0 ? f32x16{} : sacc);
      }
      if (x.lim < kBlock - 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (wt * 32 + c_row(j, h) > x.lim) sacc[j] = kNegInf;
      }
      float mw = kNegInf;
#pragma unroll
      for (int j = 0; j < 16; ++j) mw = fmaxf(mw, sacc[j]);
      mw = wave_max_xor32(mw);
      if (h == 0) red_m[team][wt][l32] = mw;
    }
    __syncthreads();
    float alpha = 1.f, m_new = m_run;
    if (x.has) {
      // key 0 of a visible block is visible, so the block maximum is finite
      const float mb = fmaxf(fmaxf(red_m[team][0][l32], red_m[team][1][l32]),
                             fmaxf(red_m[team][2][l32], red_m[team][3][l32]));
      m_new = fmaxf(m_run, mb);
      alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);  // 0 for the first block
      const float moff = -m_new * sl2;
      float lw = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], sl2, moff));
        sacc[j] = e;
        lw += e;
      }
      lw = xor_sum<32>(lw);
      if (h == 0) red_l[team][wt][l32] = lw;
      // P^T row l32: keys 32 wt + c_row(j, h) come in runs of four
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        T* dst = &Ps[l32 * LDP + wt * 32 + q4 * 8 + h * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(sacc[q4 * 4 + e]);
      }
    }
    __syncthreads();
    if (x.has) {
      l_run = l_run * alpha + (red_l[team][0][l32] + red_l[team][1][l32] + red_l[team][2][l32] + red_l[team][3][l32]);
      m_run = m_new;
      if (wt < NDT) {
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[j] *= alpha;
#pragma unroll
        for (int ks2 = 0; ks2 < NPV; ++ks2) {
          const frag va = *(const frag*)&Vt[(wt * 32 + l32) * LDV + ks2 * KSTEP + h * KPL];
          const frag pb = *(const frag*)&Ps[l32 * LDP + ks2 * KSTEP + h * KPL];
          oacc = M::mma(va, pb, oacc);
        }
      }
    }
  };

  // rounds of two blocks (one per team), the next round's loads in flight
  const int rounds = (nv + 1) / 2;
  Blk xa, xb;
  load_blk(0, xa);
  for (int j = 0; j < rounds; j += 2) {
    load_blk(j + 1, xb);
    step(xa);
    if (j + 1 >= rounds) break;
    load_blk(j + 2, xa);
    step(xb);
  }

  // merge the teams: team 1 hands (m, l, O^T slices) to team 0 through LDS
  __syncthreads();
  float* xo = (float*)raw;  // [4 waves][16][64 lanes]
  float* xm = xo + 4 * 16 * 64;
  if (team == 1) {
    if (wt < NDT) {
#pragma unroll
      for (int j = 0; j < 16; ++j) xo[(wt * 16 + j) * 64 + lane] = oacc[j];
    }
    if (wt == 0 && h == 0) {
      xm[l32] = m_run;
      xm[32 + l32] = l_run;
    }
  }
  __syncthreads();
  if (team == 0 && wt < NDT && l32 < R) {
    const float m1 = xm[l32], l1 = xm[32 + l32];
    const float mt = fmaxf(m_run, m1);
    const bool any = mt != kNegInf;  // false only for a row that sees no key
    const float a0 = any ? __builtin_amdgcn_exp2f((m_run - mt) * sl2) : 0.f;
    const float a1 = any ? __builtin_amdgcn_exp2f((m1 - mt) * sl2) : 0.f;
    const float W = l_run * a0 + l1 * a1;
    const float inv = any ? p.v_scale / W : 0.f;
    const int64_t orow = (bi * p.Hq + g * R + l32) * D;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = wt * 32 + q4 * 8 + h * 4;
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o4[e] = (oacc[q4 * 4 + e] * a0 + xo[(wt * 16 + q4 * 4 + e) * 64 + lane] * a1) * inv;
      if (p.out_f32) {
        *(f32x4*)((float*)p.out + orow + d0) = f32x4{o4[0], o4[1], o4[2], o4[3]};
      } else {
        *(bf16x4*)((T*)p.out + orow + d0) =
            bf16x4{from_f32<T>(o4[0]), from_f32<T>(o4[1]), from_f32<T>(o4[2]), from_f32<T>(o4[3])};
      }
    }
    if (wt == 0 && h == 0 && p.lse)
      p.lse[((int64_t)b * p.Hq + g * R + l32) * p.S_q + i] =
          any ? (mt * sl2 + __builtin_amdgcn_logf(W)) * 0.69314718055994531f : kNegInf;
  }
}

// s_waitcnt immediate that waits until at most vm vector-memory operations
// are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Transposing LDS read of four bf16 (gfx950): in each 16-lane group, lane i
// gets column c0 + i of rows r0 .. r0 + 3 when lane s points at row r0 + s / 4,
// column c0 + 4 (s % 4).
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* ptr) {
  return __builtin_bit_cast(bf16x4,
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(ptr)));
}

// Workgroup barrier for LDS data: this wave's LDS writes complete, then the
// barrier; the memory clobber keeps the compiler from moving memory accesses
// across it.  A fence (as in __syncthreads) would, in a kernel that moves
// data into LDS by DMA, make every barrier wait for all vector-memory
// operations in flight; the block loop below waits for exactly the DMA it
// needs before its first barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Decode rows form for r <= 16: one workgroup per (b, i, g) row, as
// attn_decode_rows_kernel, but all 8 waves work on one block at a time so that
// a row keeps NBUF blocks in flight.  Each wave scores 16 of the block's keys
// with 16x16x32 MFMA tiles (K read straight from HBM as the A operand: 16
// VGPRs per block, 8 for e4m3), V goes from HBM into a ring of NBUF LDS tiles
// by DMA (no registers), and wave w accumulates the d-slice [16w, 16w + 16) of
// O^T, its V^T operand read from a row-major bf16 V tile with transposing LDS
// reads (native keys: the ring slot itself; e4m3: a tile the block's bytes are
// widened into first).  Row maxima and sums meet in LDS; O^T is rescaled by
// 2^(m_old - m_new) as the running maximum grows.
template <typename S, int D, int R>
__global__ __launch_bounds__(512) void attn_decode_rows16_kernel(AttnParams p) {
  using T = bf16;
  typedef bf16x8 frag;
  constexpr bool kNative = std::is_same<S, T>::value;
  typedef typename std::conditional<kNative, frag, uint2>::type kraw;  // 8 elements of S
  constexpr int SB = (int)sizeof(S);
  constexpr int NW = 8;                   // waves
  constexpr int KPW = kBlock / NW;        // keys per wave (16)
  constexpr int NKS = D / 32;             // k-steps of S^T = K Q^T
  constexpr int CPR = D / 8;              // 16-byte chunks per row of the bf16 V tile
  constexpr int SCPR = D * SB / 16;       // 16-byte chunks per row of a stored V block
  constexpr int RPP = 1024 / (D * SB);    // stored rows per 1 KiB DMA piece
  constexpr int PPW = kBlock / RPP / NW;  // DMA pieces per wave per block
  constexpr int VMB = NKS + PPW;          // vector-memory instructions per lane per block
  constexpr int NBUF = 4;                 // blocks in flight
  constexpr int VBYTES = kBlock * D * SB; // one stored V block
  constexpr int TBYTES = kBlock * D * 2;  // the bf16 V tile
  constexpr int LDP = kBlock + 8;         // P^T pitch [row][key]
  constexpr int NDW = D / 16;             // waves that own a d-slice of O^T
  constexpr int MERGE_BYTES = kMergeMaxLists * kIndexWideCap * 8;  // the largest list set of a row
  constexpr int HALF = MERGE_BYTES / 2;
  static_assert(R <= 16, "16 rows per tile");
  static_assert(PPW * RPP * NW == kBlock && SCPR * RPP == 64, "the DMA pieces cover a block");
  // the V ring: one array per slot, so that reading one slot is visibly
  // independent of the DMA into the others.  The list merge (scores, block
  // ids) runs before the ring starts, in slot 0 and slot 1 (native) or the
  // bf16 tile (e4m3).
  constexpr int S0 = VBYTES > HALF ? VBYTES : HALF;
  constexpr int S1 = kNative ? S0 : VBYTES;
  constexpr int STB = kNative ? 16 : (TBYTES > HALF ? TBYTES : HALF);
  __shared__ __align__(16) char vr0[S0];
  __shared__ __align__(16) char vr1[S1];
  __shared__ __align__(16) char vr2[VBYTES];
  __shared__ __align__(16) char vr3[VBYTES];
  __shared__ __align__(16) char vtb[STB];
  __shared__ __align__(16) T Ps[16 * LDP];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];
  __shared__ int pos_s[64];
  __shared__ int blk_s[64];
  __shared__ int64_t off_s[64];
  __shared__ int nv_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const float sl2 = p.scale_log2;
  const int64_t row = blockIdx.x;  // (b * S_q + i) * G + g
  const int g = (int)(row % p.G);
  const int64_t bi = row / p.G;  // b * S_q + i
  const int i = (int)(bi % p.S_q);
  const int b = (int)(bi / p.S_q);
  const int64_t t = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + i;
  const int L = local_block(t);
  const int slen = cache_len(p.cm, p.S_k, b);

  // Q^T operand: Q[row l16][d 32 ks + 8 g4 ..] (rows past r repeat head 0, never stored)
  frag qb[NKS];
  {
    const int qh = l16 < R ? l16 : 0;
    const T* qp = (const T*)p.q + (bi * p.Hq + g * R + qh) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qb[ks] = *(const frag*)(qp + ks * 32 + g4 * 8);
  }

  // the row's selection (merged here from the split lists, or read) and its
  // visible, mapped blocks in ascending order with their offsets
  if (wave == 0) {
    const int64_t srow = (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
    pos_s[lane] = -1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (p.lists_s) {
      if (L >= 0) {
        const int nl = L > 0 ? (L + p.list_chunk - 1) / p.list_chunk * p.list_lps : 0;
        const int64_t base = row * p.list_stride * p.list_cap;
        float* ss = (float*)vr0;
        int* si = (int*)(kNative ? vr1 : vtb);
        const MergedSlot m =
            merge_row_lists(p.lists_s + base, p.lists_i + base, nl, p.list_cap, min(p.topk - 1, L), L, ss, si, lane);
        if (m.pos >= 0) {
          p.sel_w[srow + m.pos] = m.id;
          pos_s[m.pos] = m.id;
        } else if (lane < p.topk) {
          p.sel_w[srow + lane] = -1;
        }
      } else if (lane < p.topk) {
        p.sel_w[srow + lane] = -1;
      }
    } else if (L >= 0 && lane < p.topk) {
      pos_s[lane] = p.sel[srow + lane];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int c = lane < p.topk ? pos_s[lane] : -1;
    const int64_t key0 = (int64_t)c * kBlock;
    const bool ok = c >= 0 && c < p.nb && key0 <= t && key0 < slen && block_mapped(p.cm, b, c);
    const uint64_t bal = __ballot(ok);
    if (ok) {
      const int ci = __popcll(bal & ((1ull << lane) - 1));
      blk_s[ci] = c;
      off_s[ci] = block_offset(p.cm, p.S_k, p.G, D, b, g, c);
    }
    if (lane == 0) nv_s = __popcll(bal);
  }
  __syncthreads();  // the selection is in LDS and the merge is done with the ring
  const int nv = nv_s;

  // 16-byte chunk c of row r of a V tile sits at chunk c ^ sw(r) (the swizzle of
  // the backward's [row][d] tiles: the rows of one transposing read fall in
  // distinct banks)
  auto sw = [](int r) { return CPR == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 3) << 1) | ((r >> 2) & 1)); };
  auto vat = [&](int r, int col) { return r * D + ((((col >> 3) ^ sw(r))) << 3) + (col & 7); };

  // Issue block n: this wave's 16 K rows into kf and its PPW pieces of V into
  // ring slot n % NBUF (native keys in the bf16 tile's swizzled layout, e4m3
  // as stored).  Past the row's blocks the loads read row 0 of the pool (valid
  // memory, never used), so every block issues the same VMB instructions and
  // the explicit waits below count them exactly.
  // lane j holds block j's element offset and rows (past the row's blocks:
  // offset 0 and one row), read by block index with readlane, so issuing a
  // block needs no LDS read
  const int64_t lane_off = lane < nv ? off_s[lane] : 0;
  const int lane_rows = lane < nv ? (int)min((int64_t)kBlock, (int64_t)slen - (int64_t)blk_s[lane] * kBlock) : 1;
  auto issue = [&](int n, kraw (&kf)[NKS], char* slot) {
    // n >= nv reads lane 63: offset 0 and one row, or with 64 blocks the last
    // block (valid memory either way; the slot is never read)
    const int nl = n < nv ? n : 63;
    const int64_t kv0 = ((int64_t)__builtin_amdgcn_readlane((int)(lane_off >> 32), nl) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)lane_off, nl);
    const int rows_ok = __builtin_amdgcn_readlane(lane_rows, nl);
    const int krow = min(wave * KPW + l16, rows_ok - 1);
    const S* kp = (const S*)p.k + kv0 + (int64_t)krow * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = *(const kraw*)(kp + ks * 32 + g4 * 8);
    const char* vb = (const char*)((const S*)p.v + kv0);
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
      const int piece = wave * PPW + u;
      const int r = piece * RPP + lane / SCPR;
      const int cq = kNative ? (lane % SCPR) ^ sw(r) : lane % SCPR;
      const int rs = min(r, rows_ok - 1);  // rows past the cache end re-read its last row (masked)
      __builtin_amdgcn_global_load_lds((const void*)(vb + ((int64_t)rs * D * SB + cq * 16)),
                                       (__attribute__((address_space(3))) void*)(slot + piece * 1024), 16, 0, 0);
    }
  };

  float m_run = kNegInf, l_run = 0.f;  // of row l16, the same in every lane of the row
  f32x4 oacc = f32x4{};
  auto step = [&](int n, const kraw (&kf)[NKS], kraw (&knext)[NKS], const char* cur, char* nxt) {
    // block n's own loads are done (the two after it may still be in flight) ...
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * VMB));
    // ... and every wave's: block n's V tile is in LDS, block n - 1 is done with its slot
    lds_barrier();
    issue(n + NBUF - 1, knext, nxt);  // into the slot and registers block n - 1 used
    __builtin_amdgcn_sched_barrier(0);
    const T* V = (const T*)(kNative ? cur : vtb);
    if constexpr (!kNative) {
      // widen the block's e4m3 values (exact) into the bf16 tile; its readers
      // come after the next barrier, its previous readers were before the last
      constexpr int NCV = kBlock * SCPR / 512;
#pragma unroll
      for (int u = 0; u < NCV; ++u) {
        const int q = tid + u * 512;
        const int r = q / SCPR, c = q % SCPR;
        const i32x4 x = *(const i32x4*)(cur + r * (D * SB) + c * 16);
        const uint2 w0 = e4m3x4_to_bf16((uint32_t)x[0]), w1 = e4m3x4_to_bf16((uint32_t)x[1]);
        const uint2 w2 = e4m3x4_to_bf16((uint32_t)x[2]), w3 = e4m3x4_to_bf16((uint32_t)x[3]);
        *(i32x4*)((T*)vtb + vat(r, c * 16)) = i32x4{(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y};
        *(i32x4*)((T*)vtb + vat(r, c * 16 + 8)) = i32x4{(int)w2.x, (int)w2.y, (int)w3.x, (int)w3.y};
      }
    }
    const int64_t rel = t - (int64_t)blk_s[n] * kBlock;
    const int lim = rel >= kBlock ? kBlock : (int)rel;
    // S^T for keys [16 wave, 16 wave + 16): lane (row l16, group g4) holds keys 16 wave + 4 g4 + j
    auto kfrag = [&](int ks) -> frag {
      if constexpr (kNative) return kf[ks];
      else return __builtin_bit_cast(frag, ChunkIO<T, S>::widen(kf[ks]));
    };
    f32x4 sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(0), qb[0], f32x4{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < NKS; ++ks) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(ks), qb[ks], sacc, 0, 0, 0);
    if (lim < kBlock - 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (wave * KPW + g4 * 4 + j > lim) sacc[j] = kNegInf;
    }
    float mw = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    mw = xor_max<16>(mw);
    mw = xor_max<32>(mw);
    if (g4 == 0) red_m[wave][l16] = mw;
    lds_barrier();
    // key 0 of a visible block is visible, so the block maximum is finite
    float mb = red_m[0][l16];
#pragma unroll
    for (int w = 1; w < NW; ++w) mb = fmaxf(mb, red_m[w][l16]);
    const float m_new = fmaxf(m_run, mb);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);  // 0 for the first block
    const float moff = -m_new * sl2;
    float lw = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], sl2, moff));
      sacc[j] = e;
      lw += e;
    }
    lw = xor_sum<16>(lw);
    lw = xor_sum<32>(lw);
    if (g4 == 0) red_l[wave][l16] = lw;
    *(bf16x4*)&Ps[l16 * LDP + wave * KPW + g4 * 4] =
        bf16x4{from_f32<T>(sacc[0]), from_f32<T>(sacc[1]), from_f32<T>(sacc[2]), from_f32<T>(sacc[3])};
    lds_barrier();
    float lb = red_l[0][l16];
#pragma unroll
    for (int w = 1; w < NW; ++w) lb += red_l[w][l16];
    l_run = l_run * alpha + lb;
    m_run = m_new;
    if (wave < NDW) {
      oacc *= alpha;
      // O^T slice d in [16 wave, 16 wave + 16): V^T rows read transposed from the
      // row-major tile (keys 32 kk + 8 g4 + (0..7) at d 16 wave + l16), P^T rows
      // straight from Ps
#pragma unroll
      for (int kk = 0; kk < kBlock / 32; ++kk) {
        const int r0 = kk * 32 + g4 * 8 + (l16 >> 2), c0 = wave * 16 + 4 * (l16 & 3);
        const frag va = __builtin_shufflevector(lds_read_tr(V + vat(r0, c0)), lds_read_tr(V + vat(r0 + 4, c0)), 0, 1,
                                                2, 3, 4, 5, 6, 7);
        const frag pb = *(const frag*)&Ps[l16 * LDP + kk * 32 + g4 * 8];
        oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc, 0, 0, 0);
      }
    }
  };

  kraw k0[NKS], k1[NKS], k2[NKS], k3[NKS];
  static_assert(NBUF == 4, "four slots below");
  issue(0, k0, vr0);
  issue(1, k1, vr1);
  issue(2, k2, vr2);
  for (int n = 0; n < nv; n += 4) {
    step(n, k0, k3, vr0, vr3);
    if (n + 1 >= nv) break;
    step(n + 1, k1, k0, vr1, vr0);
    if (n + 2 >= nv) break;
    step(n + 2, k2, k1, vr2, vr1);
    if (n + 3 >= nv) break;
    step(n + 3, k3, k2, vr3, vr2);
  }
  // no DMA may still be writing this workgroup's LDS when it ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  if (wave < NDW && l16 < R) {
    const bool any = m_run != kNegInf;  // false only for a row that sees no key
    const float inv = any ? p.v_scale / l_run : 0.f;
    const int64_t o = (bi * p.Hq + g * R + l16) * D + wave * 16 + g4 * 4;
    if (p.out_f32) {
      *(f32x4*)((float*)p.out + o) = f32x4{oacc[0] * inv, oacc[1] * inv, oacc[2] * inv, oacc[3] * inv};
    } else {
      *(bf16x4*)((T*)p.out + o) = bf16x4{from_f32<T>(oacc[0] * inv), from_f32<T>(oacc[1] * inv),
                                         from_f32<T>(oacc[2] * inv), from_f32<T>(oacc[3] * inv)};
    }
    if (wave == 0 && g4 == 0 && p.lse)
      p.lse[((int64_t)b * p.Hq + g * R + l16) * p.S_q + i] =
          any ? (m_run * sl2 + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : kNegInf;
  }
}

// Merge the partial states of one (token, group) over its selected slots:
// out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s.
// A thread owns one 16-byte chunk of the lane-native partial layout (E values
// of one head: runs of four consecutive d).  Every load is unconditional, from a
// clamped address, so all of a thread's loads are in flight together; unused
// slots are removed by selects.  When a workgroup covers whole (token, group)
// rows, the result goes through LDS so the output is written in full lines.
constexpr int kCombineThreads = 512;  // two (token, group) rows per workgroup at r = 16, d = 128: half the launches

template <typename T, typename TO, int D, int R, int KMAX>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(AttnParams p) {
  constexpr int E = 16 / (int)sizeof(T);
  constexpr int NCHT = D * R / E;  // chunks per (token, slot) partial
  constexpr bool STAGED = NCHT <= kCombineThreads && kCombineThreads % NCHT == 0;
  constexpr int RPW = STAGED ? kCombineThreads / NCHT : 1;  // (token, group) rows per workgroup
  __shared__ __align__(16) TO ostage[STAGED ? RPW * R * D : 1];
  const int64_t u = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  const int64_t rows_total = (int64_t)p.B * p.nrows * p.G;  // the pass's (b, i, g) rows
  const int64_t total = rows_total * NCHT;
  const bool live = u < total;
  const int64_t uc = live ? u : total - 1;
  const int ch = (int)(uc % NCHT);
  const int64_t rowg = uc / NCHT;  // (b * nrows + i - row0) * G + g: its partial states
  const int g = (int)(rowg % p.G);
  const int64_t bic = rowg / p.G;
  const int i = p.row0 + (int)(bic % p.nrows);
  const int b = (int)(bic / p.nrows);
  const int64_t bi = (int64_t)b * p.S_q + i;
  const int hh = ch % R, h = (ch / R) & 1, q = ch / (2 * R);
  const int64_t t = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + i;
  const int32_t* srow = p.sel + (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
  const int64_t pbase = rowg * p.topk;

  // The slots' partial chunks are held in registers KC at a time: all of them
  // for k <= 32, two rounds of 32 for larger k (the weights come first, from
  // every slot's log-sum-exp).
  constexpr int KC = KMAX < 32 ? KMAX : 32;
  float ls[KMAX];
  i32x4 x[KC];
  auto load_chunks = [&](int s0) {
#pragma unroll
    for (int s2 = 0; s2 < KC; ++s2) {
      const int sc = min(s0 + s2, p.topk - 1);
      x[s2] = __builtin_nontemporal_load((const i32x4*)((const T*)p.part_o + (pbase + sc) * (R * D) + ch * E));
    }
  };
  float mx = kNegInf;
  if constexpr (STAGED) {
    // A workgroup's rows share their selection rows and log-sum-exps: load those
    // once into LDS instead of once per thread.
    __shared__ int sel_s[RPW][KMAX];
    __shared__ float lse_s[RPW][KMAX][R];
    const int64_t row0 = (int64_t)blockIdx.x * RPW;
    for (int e = threadIdx.x; e < RPW * KMAX; e += kCombineThreads) {
      const int lr = e / KMAX, s2 = e - lr * KMAX;
      const int64_t rg = min(row0 + lr, rows_total - 1);
      const int64_t rbi = rg / p.G;
      const int rgg = (int)(rg - rbi * p.G);
      const int ri = p.row0 + (int)(rbi % p.nrows), rb = (int)(rbi / p.nrows);
      int c = -1;
      if (s2 < p.topk) {
        c = p.sel[(((int64_t)rb * p.G + rgg) * p.S_q + ri) * p.topk + s2];
        const int64_t rt = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, rb) + ri;
        if (!(c >= 0 && c < p.nb && (int64_t)c * kBlock <= rt && block_mapped(p.cm, rb, c))) c = -1;
      }
      sel_s[lr][s2] = c;
    }
    for (int e = threadIdx.x; e < RPW * KMAX * R; e += kCombineThreads) {
      const int lr = e / (KMAX * R), rem = e - lr * (KMAX * R);
      const int s2 = rem / R, hd = rem - s2 * R;
      const int64_t rg = min(row0 + lr, rows_total - 1);
      lse_s[lr][s2][hd] = s2 < p.topk ? p.part_lse[(rg * p.topk + s2) * R + hd] : 0.f;
    }
    __syncthreads();
    const int lr = (int)(threadIdx.x / NCHT);
    load_chunks(0);
#pragma unroll
    for (int s2 = 0; s2 < KMAX; ++s2) {
      ls[s2] = sel_s[lr][s2] >= 0 ? lse_s[lr][s2][hh] : kNegInf;
      mx = fmaxf(mx, ls[s2]);
    }
  } else {
    int cs[KMAX];
#pragma unroll
    for (int s2 = 0; s2 < KMAX; ++s2) {
      const int sc = min(s2, p.topk - 1);
      cs[s2] = srow[sc];
      ls[s2] = p.part_lse[(pbase + sc) * R + hh];
    }
    load_chunks(0);
#pragma unroll
    for (int s2 = 0; s2 < KMAX; ++s2) {
      const int c = cs[s2];
      const bool used = s2 < p.topk && c >= 0 && c < p.nb && (int64_t)c * kBlock <= t && block_mapped(p.cm, b, c);
      ls[s2] = used ? ls[s2] : kNegInf;
      mx = fmaxf(mx, ls[s2]);
    }
  }
  float W = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s0 = 0; s0 < KMAX; s0 += KC) {
    if (s0 > 0) load_chunks(s0);
#pragma unroll
    for (int s2 = 0; s2 < KC; ++s2) {
      const int s = s0 + s2;
      const bool used = ls[s] != kNegInf;
      const float w = used ? exp2f(ls[s] - mx) : 0.f;
      W += w;
      const typename Vec16<T>::type xv = __builtin_bit_cast(typename Vec16<T>::type, x[s2]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += used ? w * to_f32(xv[e]) : 0.f;
    }
  }
  // the value cache's dequantisation scale (1 if none); a row that sees no key
  // (it precedes its cache) gets zeros and lse = -inf
  const float inv = W > 0.f ? p.v_scale / W : 0.f;
  const int r0 = (q * E) % 16, dt = (q * E) / 16;
  if constexpr (STAGED) {
    TO* srow_o = ostage + (int)(threadIdx.x / NCHT) * (R * D) + hh * D;
#pragma unroll
    for (int m = 0; m < E / 4; ++m) {
      const int d0 = dt * 32 + (r0 / 4 + m) * 8 + 4 * h;
#pragma unroll
      for (int e = 0; e < 4; ++e) srow_o[d0 + e] = from_f32<TO>(acc[4 * m + e] * inv);
    }
    __syncthreads();
    // each staged (b, i, g) row is one contiguous R * D run of out, written in full lines
    const int64_t wrow0 = (int64_t)blockIdx.x * RPW;
    const int64_t wrows = rows_total - wrow0 < RPW ? rows_total - wrow0 : RPW;
    constexpr int ROW_CHUNKS = R * D * (int)sizeof(TO) / 16;
    constexpr int CHUNKS = RPW * ROW_CHUNKS;
    const Chunk16* src = (const Chunk16*)ostage;
#pragma unroll
    for (int k = 0; k < (CHUNKS + kCombineThreads - 1) / kCombineThreads; ++k) {
      const int c = (int)threadIdx.x + k * kCombineThreads;
      const int lr = c / ROW_CHUNKS;
      if (lr < wrows) {
        const int64_t rg = wrow0 + lr;
        const int64_t rbi = rg / p.G;
        const int rgg = (int)(rg - rbi * p.G);
        const int64_t orow = ((rbi / p.nrows) * p.S_q + p.row0 + rbi % p.nrows) * p.G + rgg;
        ((Chunk16*)((TO*)p.out + orow * R * D))[c - lr * ROW_CHUNKS] = src[c];
      }
    }
  } else if (live) {
    TO* orow = (TO*)p.out + (bi * p.Hq + g * R + hh) * D;
#pragma unroll
    for (int m = 0; m < E / 4; ++m) {
      const int d0 = dt * 32 + (r0 / 4 + m) * 8 + 4 * h;
#pragma unroll
      for (int e = 0; e < 4; ++e) orow[d0 + e] = from_f32<TO>(acc[4 * m + e] * inv);
    }
  }
  if (live && q == 0 && h == 0 && p.lse)
    p.lse[((int64_t)b * p.Hq + g * R + hh) * p.S_q + i] = (mx + log2f(W)) * 0.69314718055994531f;
}

void launch_gather(const AttnParams& p, hipStream_t s, const KernelTimer* tm) {
  const int64_t entries = (int64_t)p.B * p.G * p.nrows * p.topk;  // this pass's rows
  if (!p.direct) {
    timer_start(tm, kKernGather, s);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((p.nbuckets + 255) / 256)), dim3(256), 0, s,
                       p.counts, (int64_t)p.nbuckets);
    const bool lds_hist = p.nb <= kMaxHistBins;
    const dim3 hgrid((unsigned)((p.nrows + kGatherRows - 1) / kGatherRows), (unsigned)(p.B * p.G));
    if (lds_hist)
      hipLaunchKernelGGL(gather_hist_kernel<false>, hgrid, dim3(256), p.nb * 4, s, p);
    else
      hipLaunchKernelGGL(gather_count_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, p);
    hipLaunchKernelGGL(gather_scan_kernel, dim3(1), dim3(1024), 0, s, p);
    hipLaunchKernelGGL(item_table_kernel, dim3((unsigned)((p.nbuckets + 255) / 256)), dim3(256), 0, s, p);
    if (lds_hist)
      hipLaunchKernelGGL(gather_hist_kernel<true>, hgrid, dim3(256), p.nb * 4, s, p);
    else
      hipLaunchKernelGGL(gather_scatter_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, p);
    timer_stop(tm, kKernGather, s);
  }
}

template <typename T, typename S, int D, int R>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t s, const KernelTimer* tm) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (p.rows_mode) {  // the whole main branch in one launch, no combine
      timer_start(tm, kKernAttention, s);
      const dim3 rgrid((unsigned)((int64_t)p.B * p.S_q * p.G));
      if constexpr (R <= 16)
        hipLaunchKernelGGL((attn_decode_rows16_kernel<S, D, R>), rgrid, dim3(512), 0, s, p);
      else
        hipLaunchKernelGGL((attn_decode_rows_kernel<S, D, R>), rgrid, dim3(512), 0, s, p);
      timer_stop(tm, kKernAttention, s);
      return hipGetLastError();
    }
  }
  if (!p.direct && p.tpi > kMaxItemTokens) return hipErrorInvalidValue;  // the item's entries must fit its LDS list
  // One pass over all query rows, or (workspace capped) passes over chunks of
  // chunk_rows rows that share the gather buckets and the partial-state region.
  const int step = p.direct || p.chunk_rows <= 0 ? p.S_q : p.chunk_rows;
  for (int r0 = 0; r0 < p.S_q; r0 += step) {
    AttnParams pc = p;
    pc.row0 = r0;
    pc.nrows = min(step, p.S_q - r0);
    launch_gather(pc, s, tm);
    timer_start(tm, kKernAttention, s);
    if (pc.direct)
      hipLaunchKernelGGL((attn_decode_kernel<T, S, D, R>), dim3(pc.grid_decode), dim3(256), 0, s, pc);
    else
      hipLaunchKernelGGL((attn_kvouter_kernel<T, S, D, R>), dim3(pc.grid), dim3(256), 0, s, pc);
    timer_stop(tm, kKernAttention, s);
    timer_start(tm, kKernCombine, s);
    constexpr int E = 16 / (int)sizeof(T);
    const int64_t units = (int64_t)pc.B * pc.nrows * pc.G * (D * R / E);
    const dim3 cgrid((unsigned)((units + kCombineThreads - 1) / kCombineThreads));
    if (pc.topk <= 16) {
      if (pc.out_f32) hipLaunchKernelGGL((combine_kernel<T, float, D, R, 16>), cgrid, dim3(kCombineThreads), 0, s, pc);
      else hipLaunchKernelGGL((combine_kernel<T, T, D, R, 16>), cgrid, dim3(kCombineThreads), 0, s, pc);
    } else if (pc.topk <= 32) {
      if (pc.out_f32) hipLaunchKernelGGL((combine_kernel<T, float, D, R, 32>), cgrid, dim3(kCombineThreads), 0, s, pc);
      else hipLaunchKernelGGL((combine_kernel<T, T, D, R, 32>), cgrid, dim3(kCombineThreads), 0, s, pc);
    } else {
      if (pc.out_f32) hipLaunchKernelGGL((combine_kernel<T, float, D, R, 64>), cgrid, dim3(kCombineThreads), 0, s, pc);
      else hipLaunchKernelGGL((combine_kernel<T, T, D, R, 64>), cgrid, dim3(kCombineThreads), 0, s, pc);
    }
    timer_stop(tm, kKernCombine, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, typename S, int D>
static hipError_t launch_attn_d(const AttnParams& p, hipStream_t s, const KernelTimer* tm) {
  switch (p.r) {
    case 1: return launch_attn_t<T, S, D, 1>(p, s, tm);
    case 2: return launch_attn_t<T, S, D, 2>(p, s, tm);
    case 4: return launch_attn_t<T, S, D, 4>(p, s, tm);
    case 8: return launch_attn_t<T, S, D, 8>(p, s, tm);
    case 16: return launch_attn_t<T, S, D, 16>(p, s, tm);
    case 32: return launch_attn_t<T, S, D, 32>(p, s, tm);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename S>
static hipError_t launch_attn_s(const AttnParams& p, hipStream_t s, const KernelTimer* tm) {
  if (p.d == 64) return launch_attn_d<T, S, 64>(p, s, tm);
  if (p.d == 128) return launch_attn_d<T, S, 128>(p, s, tm);
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_attention(const AttnParams& p, bool bf16_inputs, bool fp8_cache, hipStream_t s,
                                   const KernelTimer* tm) {
  if (fp8_cache) return bf16_inputs ? launch_attn_s<bf16, e4m3>(p, s, tm) : hipErrorInvalidValue;
  if (bf16_inputs) return launch_attn_s<bf16, bf16>(p, s, tm);
  return launch_attn_s<float, float>(p, s, tm);
}

}  // namespace msa

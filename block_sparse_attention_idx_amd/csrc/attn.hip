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
//   1. gather_count / gather_scan / gather_scatter: bucket every selection
//      entry (b, g, i, slot) by its block (b, g, c): histogram, exclusive scan,
//      scatter.  A bucket is cut into work items of up to tpi query tokens.
//   2. attn_kvouter: a persistent grid walks the work items.  An item stages
//      K (128 x d) and V^T (d x 128) of its block in LDS once, then runs passes
//      of 4 waves x 32 rows; a row is one (token, head) and the r heads of a
//      token are adjacent rows, so the whole group shares the staged tile.
//      S^T = K Q^T and O^T = V^T P^T are 32x32 MFMA tiles; every lane owns one
//      row, so the block-local softmax needs one cross-half exchange.  The
//      result is a partial state per (token, slot, head): o / l in the input
//      dtype plus m and l in fp32.
//   3. combine: per (token, head) the partial states of its slots are merged
//      (max of m, rescaled sums) into the output and the log-sum-exp.
// With S_q small (decode) the gather is skipped: one item per selection entry.
#include "common.h"
#include "kernels.h"

namespace msa {

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void gather_count_kernel(AttnParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.G * p.S_q * p.topk;
  if (e >= total) return;
  const int c = p.sel[e];
  if (c < 0 || c >= p.nb) return;  // ids outside the cache are ignored, never dereferenced
  const int64_t bg = e / ((int64_t)p.S_q * p.topk);  // b * G + g
  atomicAdd(&p.counts[bg * p.nb + c], 1);
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

__global__ __launch_bounds__(256) void gather_scatter_kernel(AttnParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.G * p.S_q * p.topk;
  if (e >= total) return;
  const int c = p.sel[e];
  if (c < 0 || c >= p.nb) return;
  const int slot = (int)(e % p.topk);
  const int64_t rest = e / p.topk;
  const int i = (int)(rest % p.S_q);
  const int64_t bg = rest / p.S_q;
  const int pos = atomicAdd(&p.cursor[bg * p.nb + c], 1);
  p.entries[pos] = (i << 6) | slot;
}

// E x E transpose of 16-byte rows (E = 16 / sizeof(T)).
template <typename T, int E>
__device__ __forceinline__ void transpose_tile(const Chunk16 (&in)[E], Chunk16 (&out)[E]) {
  const T* a = (const T*)in;
  T* o = (T*)out;
#pragma unroll
  for (int r = 0; r < E; ++r)
#pragma unroll
    for (int c = 0; c < E; ++c) o[c * E + r] = a[r * E + c];
}

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void attn_kvouter_kernel(AttnParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
  constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int LDK = D + E;              // K row pitch (elements)
  constexpr int LDV = kBlock + E;         // V^T row pitch (elements)
  constexpr int TPW = 32 / R;             // query tokens per wave per pass
  constexpr int TPP = 4 * TPW;            // query tokens per pass
  constexpr int NDT = D / 32;             // 32-wide output tiles along d
  constexpr int NPV = kBlock / KSTEP;     // PV instructions per d tile
  __shared__ __align__(16) T Ks[kBlock * LDK];
  __shared__ __align__(16) T Vt[D * LDV];

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
      // bucket = last one whose first item is <= item
      int lo = 0, hi = p.nbuckets;  // item_off[lo] <= item < item_off[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.item_off[mid] <= item) lo = mid;
        else hi = mid;
      }
      const int bk = lo;
      const int start = (int)(item - p.item_off[bk]) * p.tpi;
      ntok = min(p.tpi, p.counts[bk] - start);
      toks = p.entries + p.offsets[bk] + start;
      c = bk % p.nb;
      const int bg = bk / p.nb;
      g = bg % p.G;
      b = bg / p.G;
    }

    __syncthreads();  // the previous item is done with the LDS tiles
    {
      const int64_t kv0 = (((int64_t)b * p.G + g) * p.S_k + (int64_t)c * kBlock) * D;
      const int rows_ok = (int)min((int64_t)kBlock, (int64_t)p.S_k - (int64_t)c * kBlock);
      // K: 128 rows of D, row-major
      constexpr int KCH = kBlock * D / E;
      const Chunk16* ksrc = (const Chunk16*)((const T*)p.k + kv0);
      for (int ch = threadIdx.x; ch < KCH; ch += 256) {
        const int row = ch / (D / E), col = ch - row * (D / E);
        Chunk16 x = {};
        if (row < rows_ok) x = ksrc[ch];
        *(Chunk16*)&Ks[row * LDK + col * E] = x;
      }
      // V^T: E x E tiles, transposed in registers
      constexpr int VT = (D / E) * (kBlock / E);
      const T* vsrc = (const T*)p.v + kv0;
      for (int tl = threadIdx.x; tl < VT; tl += 256) {
        const int dg = tl % (D / E), kg = tl / (D / E);
        Chunk16 in[E], outc[E];
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int key = kg * E + r;
          Chunk16 x = {};
          if (key < rows_ok) x = *(const Chunk16*)(vsrc + (int64_t)key * D + dg * E);
          in[r] = x;
        }
        transpose_tile<T, E>(in, outc);
#pragma unroll
        for (int r = 0; r < E; ++r) *(Chunk16*)&Vt[(dg * E + r) * LDV + kg * E] = outc[r];
      }
    }
    __syncthreads();

    for (int p0 = 0; p0 < ntok; p0 += TPP) {
      if (p0 + wave * TPW >= ntok) continue;  // this wave has no rows in this pass
      const int tslot = p0 + wave * TPW + l32 / R;
      const bool in_list = tslot < ntok;
      const int32_t entry = in_list ? (toks ? toks[tslot] : direct_tok) : 0;
      const int i = entry >> 6, slot = entry & 63;
      // a block entirely after the query has no visible key: the row is skipped
      const bool rv = in_list && (int64_t)c * kBlock <= p.q_offset + i;
      const int64_t t = rv ? p.q_offset + i : (int64_t)1 << 62;
      const int hh = l32 % R;
      const int head = g * R + hh;

      frag qf[NKS];
      {
        const T* qrow = (const T*)p.q + (((int64_t)b * p.S_q + i) * p.Hq + head) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          qf[ks] = rv ? *(const frag*)(qrow + ks * KSTEP + h * KPL) : M::zero();
      }
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
      // scale into log2 units, causal mask inside the block, block-local softmax
      const int64_t key0 = (int64_t)c * kBlock;
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float s = sacc[kt][j] * p.scale_log2;
          if (key0 + kt * 32 + c_row(j, h) > t) s = kNegInf;
          sacc[kt][j] = s;
          mx = fmaxf(mx, s);
        }
      mx = wave_max_xor32(mx);
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = exp2f(sacc[kt][j] - mx);
          sacc[kt][j] = e;
          lsum += e;
        }
      lsum += __shfl_xor(lsum, 32);

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

      if (rv) {
        const float inv = 1.0f / lsum;
        const int64_t prow = (((((int64_t)b * p.S_q + i) * p.G + g) * p.topk + slot) * R + hh);
        T* po = (T*)p.part_o + prow * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = dt * 32 + q4 * 8 + h * 4;
            if constexpr (sizeof(T) == 2) {
              bf16x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = from_f32<T>(oacc[dt][q4 * 4 + e] * inv);
              *(bf16x4*)(po + d0) = w;
            } else {
              f32x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = oacc[dt][q4 * 4 + e] * inv;
              *(f32x4*)(po + d0) = w;
            }
          }
        if (h == 0) {
          p.part_m[prow] = mx;
          p.part_l[prow] = lsum;
        }
      }
    }
  }
}

// Merge the partial states of one (token, head) over its selected slots.
template <typename T, typename TO, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnParams p) {
  constexpr int CE = 16 / (int)sizeof(T);
  constexpr int NCH = D / CE;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.S_q * p.Hq * NCH;
  if (u >= total) return;
  const int dc = (int)(u % NCH);
  const int64_t rowq = u / NCH;
  const int hq = (int)(rowq % p.Hq);
  const int64_t bi = rowq / p.Hq;  // b * S_q + i
  const int i = (int)(bi % p.S_q);
  const int b = (int)(bi / p.S_q);
  const int g = hq / p.r, hh = hq - g * p.r;
  const int32_t* srow = p.sel + (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
  const int64_t pbase = (bi * p.G + g) * p.topk;
  const int64_t t = p.q_offset + i;
  auto used = [&](int s) {
    const int c = srow[s];
    return c >= 0 && c < p.nb && (int64_t)c * kBlock <= t;
  };
  float mx = kNegInf;
  for (int s = 0; s < p.topk; ++s)
    if (used(s)) mx = fmaxf(mx, p.part_m[(pbase + s) * p.r + hh]);
  float W = 0.f;
  float acc[CE];
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  for (int s = 0; s < p.topk; ++s) {
    if (!used(s)) continue;
    const int64_t pr = (pbase + s) * p.r + hh;
    const float w = p.part_l[pr] * exp2f(p.part_m[pr] - mx);
    W += w;
    const Chunk16 x = *(const Chunk16*)((const T*)p.part_o + pr * D + dc * CE);
    const T* xv = (const T*)&x;
#pragma unroll
    for (int e = 0; e < CE; ++e) acc[e] += w * to_f32(xv[e]);
  }
  const float inv = 1.0f / W;
  TO* o = (TO*)p.out + rowq * D + dc * CE;
#pragma unroll
  for (int e = 0; e < CE; ++e) o[e] = from_f32<TO>(acc[e] * inv);
  if (dc == 0 && p.lse) p.lse[((int64_t)b * p.Hq + hq) * p.S_q + i] = (mx + log2f(W)) * 0.69314718055994531f;
}

template <typename T, int D, int R>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t s, const KernelTimer* tm) {
  const int64_t entries = (int64_t)p.B * p.G * p.S_q * p.topk;
  if (!p.direct) {
    timer_start(tm, kKernGather, s);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((p.nbuckets + 255) / 256)), dim3(256), 0, s,
                       p.counts, (int64_t)p.nbuckets);
    hipLaunchKernelGGL(gather_count_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, p);
    hipLaunchKernelGGL(gather_scan_kernel, dim3(1), dim3(1024), 0, s, p);
    hipLaunchKernelGGL(gather_scatter_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, p);
    timer_stop(tm, kKernGather, s);
  }
  timer_start(tm, kKernAttention, s);
  hipLaunchKernelGGL((attn_kvouter_kernel<T, D, R>), dim3(p.grid), dim3(256), 0, s, p);
  timer_stop(tm, kKernAttention, s);
  timer_start(tm, kKernCombine, s);
  constexpr int CE = 16 / (int)sizeof(T);
  const int64_t units = (int64_t)p.B * p.S_q * p.Hq * (D / CE);
  if (p.out_f32)
    hipLaunchKernelGGL((combine_kernel<T, float, D>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((combine_kernel<T, T, D>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, p);
  timer_stop(tm, kKernCombine, s);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(const AttnParams& p, hipStream_t s, const KernelTimer* tm) {
  switch (p.r) {
    case 1: return launch_attn_t<T, D, 1>(p, s, tm);
    case 2: return launch_attn_t<T, D, 2>(p, s, tm);
    case 4: return launch_attn_t<T, D, 4>(p, s, tm);
    case 8: return launch_attn_t<T, D, 8>(p, s, tm);
    case 16: return launch_attn_t<T, D, 16>(p, s, tm);
    case 32: return launch_attn_t<T, D, 32>(p, s, tm);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_attention(const AttnParams& p, bool bf16_inputs, hipStream_t s, const KernelTimer* tm) {
  if (bf16_inputs) {
    if (p.d == 64) return launch_attn_d<bf16, 64>(p, s, tm);
    if (p.d == 128) return launch_attn_d<bf16, 128>(p, s, tm);
  } else {
    if (p.d == 64) return launch_attn_d<float, 64>(p, s, tm);
    if (p.d == 128) return launch_attn_d<float, 128>(p, s, tm);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa

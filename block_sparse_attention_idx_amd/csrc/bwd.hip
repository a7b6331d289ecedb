// Backward of the MSA main branch on gfx950 (the selection held constant).
//
// The pages name no backward kernel; MSA-PT / MSA-CPT training needs one
// (snilld.dk page "MiniMax lancerer MSA", section "Træning og stabilisering").
// Top-k is not differentiable, so the selection is a constant and each query
// row gets the gradient of exact softmax attention over its token set:
//   P = exp(scale S - lse), dP = dO V^T, Dsum = rowsum(dO o O),
//   dS = P o (dP - Dsum), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// KV-outer, like the forward: a work item is a block with up to 512 of the
// queries that selected it (the buckets of early blocks, visible to most
// queries, are many times the mean); the block's dK and dV accumulate over the
// item's queries in registers and are added to the (zeroed) outputs with fp32
// atomics, so their summation order between items is not fixed.  Wave w owns the
// block's keys [32w, 32w + 32) and keeps their K and V rows in registers as
// MFMA B operands (8 waves: waves w and w + 4 own the same keys and split d
// between their dK / dV accumulators, so two waves fit on each SIMD).  Passes of 32 rows ((token, head) pairs; the r heads of a
// token adjacent) are shared by the 4 waves; a pass's Q and dO rows are
// fetched one pass ahead (the bucket's token entries sit in LDS) and written to
// LDS both row-major and transposed:
//   S = Q K_w^T and dP = dO V_w^T put the wave's key in the lane and the rows in
//   the registers -- directly the A operand of dV_w += P^T dO and
//   dK_w += dS^T Q, whose B operands (dO, Q with rows as the reduction index)
//   come from transposed tiles in LDS;
//   dS goes to LDS ([row][key]) and wave w forms the d-slice [32w, 32w + 32) of
//   dQ^T = K^T dS^T over all 128 keys (K^T staged once per item), stored as a
//   bf16 partial per (token, slot) in the forward's lane-native layout and
//   summed over the slots by bwd_dq_combine_kernel.
#include "common.h"
#include "kernels.h"

namespace msa {

constexpr float kLog2eB = 1.4426950408889634f;

__global__ void bwd_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

// Dsum[b, h, i] = dO[b, i, h, :] . O[b, i, h, :] in fp32, one thread per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(AttnParams p, BwdParams bp) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b * S_q + i) * Hq + h
  if (row >= (int64_t)p.B * p.S_q * p.Hq) return;
  const bf16x8* o = (const bf16x8*)((const bf16*)bp.out + row * D);
  const bf16x8* g = (const bf16x8*)((const bf16*)bp.dout + row * D);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const bf16x8 a = o[c], b = g[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
  }
  const int h = (int)(row % p.Hq);
  const int64_t bi = row / p.Hq;
  const int i = (int)(bi % p.S_q);
  const int b = (int)(bi / p.S_q);
  bp.dsum[((int64_t)b * p.Hq + h) * p.S_q + i] = acc;
}

template <int D, int R>
__global__ __launch_bounds__(512, 1) void attn_bwd_kernel(AttnParams p, BwdParams bp) {
  using T = bf16;
  using M = Mma<T>;
  using frag = M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
  constexpr int E = 8;               // bf16 elements per 16-byte chunk
  constexpr int NDT = D / 32;        // 32-wide d tiles
  constexpr int TPW = 32 / R;        // tokens per pass of 32 rows
  constexpr int CH = D / E;          // 16-byte chunks per row
  constexpr int NT = 512;            // 8 waves: wave w owns keys [32 (w % 4), +32) and half of d
  constexpr int CPT = (32 * CH + NT - 1) / NT;  // chunks of a pass's Q (and dO) rows per thread
  constexpr bool kAllStage = (32 * CH) % NT == 0;  // false (d = 64): threads past 32 * CH idle
  constexpr int NDH = NDT / 2;       // d tiles of a wave's dK / dV
  constexpr int ECH = 1024;          // token entries staged in LDS at a time
  constexpr int LDT = kBlock + 8;    // K^T pitch: [d][key]
  constexpr int LDQ = D + 8;         // Q, dO pitch: [row][d]
  constexpr int LDR = 32 + 8;        // Q^T, dO^T pitch: [d][row], rows swizzled by d (tsw)
  constexpr int LDS2 = kBlock + 8;   // dS pitch: [row][key]
  __shared__ __align__(16) T Kt[D * LDT];
  __shared__ __align__(16) T Qr[32 * LDQ];
  __shared__ __align__(16) T Or[32 * LDQ];
  __shared__ __align__(16) T Qt[D * LDR];
  __shared__ __align__(16) T Ot[D * LDR];
  __shared__ __align__(16) T dSs[32 * LDS2];
  __shared__ float lse_s[32], dsum_s[32];
  __shared__ int lim_s[32];
  __shared__ int32_t ent_s[32];
  __shared__ int32_t tok_s[ECH];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int kgrp = wave & 3, dh = wave >> 2;  // key group and d half
  // Row position of row `row` in line d of the transposed tiles.  XOR with a
  // multiple of 4 keeps the aligned runs of four rows the MFMA operands read
  // contiguous, and spreads the 8-d column chunks written together over the
  // LDS banks (with a plain layout all of them map to one bank).
  auto tsw = [](int d, int row) { return row ^ (4 * ((d >> 3) & 7)); };
  const float sl2 = p.scale_log2;

  for (int64_t item = blockIdx.x; item < (int64_t)*p.n_items; item += gridDim.x) {
    const int bk = p.item_bucket[item];
    const int start = (int)(item - p.item_off[bk]) * p.tpi;
    const int ntok = min(p.tpi, p.counts[bk] - start);
    const int32_t* toks = p.entries + p.offsets[bk] + start;
    const int c = bk % p.nb;
    const int bg = bk / p.nb;
    const int g = bg % p.G, b = bg / p.G;
    const int64_t key0 = (int64_t)c * kBlock;
    if (key0 >= p.S_k) continue;  // uniform
    const int64_t kv0 = (((int64_t)b * p.G + g) * p.S_k + key0) * D;
    const int rows_ok = (int)min((int64_t)kBlock, (int64_t)p.S_k - key0);
    const int64_t qo = p.q_offset;

    // this wave's 32 keys: K and V rows as B operands (lane = key), for the whole item
    const int kw = kgrp * 32 + l32;
    frag kf[NKS], vf[NKS];
    {
      const T* kr = (const T*)p.k + kv0 + (int64_t)min(kw, rows_ok - 1) * D;
      const T* vr = (const T*)p.v + kv0 + (int64_t)min(kw, rows_ok - 1) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kf[ks] = *(const frag*)(kr + ks * KSTEP + h * KPL);
        vf[ks] = *(const frag*)(vr + ks * KSTEP + h * KPL);
      }
    }
    __syncthreads();  // the previous item is done with the LDS tiles
    {
      // K^T [d][key] by 8 x 8 transposes; rows past the cache end are zero
      constexpr int VT = (D / E) * (kBlock / E);
      for (int tl = threadIdx.x; tl < VT; tl += NT) {
        const int dg = tl % (D / E), kg = tl / (D / E);
        i32x4 in[E], outc[E];
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int kr = kg * E + r;
          in[r] = kr < rows_ok ? *(const i32x4*)((const T*)p.k + kv0 + (int64_t)kr * D + dg * E) : i32x4{};
        }
        transpose_tile<T, E>(in, outc);
#pragma unroll
        for (int r = 0; r < E; ++r) *(i32x4*)&Kt[(dg * E + r) * LDT + kg * E] = outc[r];
      }
    }
    // the bucket's token entries, ECH at a time from ent_base
    int ent_base = 0;
    auto stage_entries = [&](int base) {
      for (int t = threadIdx.x; t < ECH; t += NT) tok_s[t] = base + t < ntok ? toks[base + t] : 0;
    };
    stage_entries(0);
    __syncthreads();

    // A pass's rows, fetched into registers one pass ahead: chunks of its Q and
    // dO rows (row = token (p0 + row / R), head row % R) and, in wave 0, row
    // (lane % 32)'s entry with its raw lse and rowsum.  Nothing here consumes a
    // loaded value, so no wait is placed before the pass's compute.
    i32x4 qx[CPT], ox[CPT];
    float lse_n = 0.f, dsum_n = 0.f;
    int32_t ent_n = 0, pslot_n = 0;
    auto fetch = [&](int p0) {
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int ch = min((int)threadIdx.x + u * NT, 32 * CH - 1);  // idle threads re-read the last chunk
        const int row = ch / CH, col = ch - row * CH;
        const int tslot = min(p0 + row / R, ntok - 1);  // rows past the list reuse a valid row
        const int i = tok_s[tslot - ent_base] >> 6;
        const int64_t roff = (((int64_t)b * p.S_q + i) * p.Hq + g * R + row % R) * D + col * E;
        qx[u] = *(const i32x4*)((const T*)p.q + roff);
        ox[u] = *(const i32x4*)((const T*)bp.dout + roff);
      }
      if (wave == 0) {
        const int rr = lane & 31;
        pslot_n = p0 + rr / R;
        ent_n = tok_s[min(pslot_n, ntok - 1) - ent_base];
        const int64_t hrow = ((int64_t)b * p.Hq + g * R + rr % R) * p.S_q + (ent_n >> 6);
        lse_n = bp.lse[hrow];
        dsum_n = bp.dsum[hrow];
      }
    };

    f32x16 dk_acc[NDH], dv_acc[NDH];  // d tiles dh * NDH + t
#pragma unroll
    for (int t = 0; t < NDH; ++t) {
      dk_acc[t] = f32x16{};
      dv_acc[t] = f32x16{};
    }

    fetch(0);
    for (int p0 = 0; p0 < ntok; p0 += TPW) {
      __syncthreads();  // the previous pass is done with the pass tiles
      // this pass's rows into LDS: row-major (A operands of S and dP) and
      // transposed (B operands of dV and dK)
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int ch = threadIdx.x + u * NT;
        if (!kAllStage && ch >= 32 * CH) break;
        const int row = ch / CH, col = ch - row * CH;
        *(i32x4*)&Qr[row * LDQ + col * E] = qx[u];
        *(i32x4*)&Or[row * LDQ + col * E] = ox[u];
        const bf16x8 qv = __builtin_bit_cast(bf16x8, qx[u]), ov = __builtin_bit_cast(bf16x8, ox[u]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int d = col * E + e;
          Qt[d * LDR + tsw(d, row)] = qv[e];
          Ot[d * LDR + tsw(d, row)] = ov[e];
        }
      }
      if (threadIdx.x < 32) {
        const bool valid = pslot_n < ntok;
        const int64_t rel = qo + (ent_n >> 6) - key0;
        // lim: the last visible key of the block, -1 when the row sees none of it
        lim_s[threadIdx.x] = (!valid || rel < 0) ? -1 : (rel >= kBlock ? kBlock - 1 : (int)rel);
        ent_s[threadIdx.x] = valid ? ent_n : -1;
        lse_s[threadIdx.x] = valid ? lse_n * kLog2eB : 0.f;
        dsum_s[threadIdx.x] = valid ? dsum_n : 0.f;
      }
      const bool has_next = p0 + TPW < ntok;
      if (has_next && p0 + 2 * TPW > ent_base + ECH) {  // the next pass needs the next entries
        ent_base = p0 + TPW;
        stage_entries(ent_base);
      }
      __syncthreads();
      if (has_next) fetch(p0 + TPW);  // in flight during this pass
      __builtin_amdgcn_sched_barrier(0);

      // S = Q K_w^T and dP = dO V_w^T: lane = key kw, register j = row c_row(j, h)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const frag qa = *(const frag*)&Qr[l32 * LDQ + ks * KSTEP + h * KPL];
        const frag oa = *(const frag*)&Or[l32 * LDQ + ks * KSTEP + h * KPL];
        s = M::mma(qa, kf[ks], s);
        dp = M::mma(oa, vf[ks], dp);
      }
      float pj[16], dsj[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = c_row(j, h);
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], sl2, -lse_s[row]));
        pj[j] = kw <= lim_s[row] ? e : 0.f;
        dsj[j] = pj[j] * (dp[j] - dsum_s[row]);
      }

      // dV_w += P^T dO and dK_w += dS^T Q; step ks2 pairs reduction index h*8+e
      // with row c_row(8 ks2 + e, h): two runs of four rows of the [d][row] tiles
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        frag pa, da;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pa[e] = (bf16)pj[ks2 * 8 + e];
          da[e] = (bf16)dsj[ks2 * 8 + e];
        }
#pragma unroll
        for (int t = 0; t < NDH; ++t) {
          const int dt = dh * NDH + t;
          const int d = dt * 32 + l32;
          const int lo = tsw(d, ks2 * 16 + h * 4), hi = tsw(d, ks2 * 16 + 8 + h * 4);
          const frag ob = __builtin_shufflevector(*(const bf16x4*)&Ot[d * LDR + lo], *(const bf16x4*)&Ot[d * LDR + hi],
                                                  0, 1, 2, 3, 4, 5, 6, 7);
          const frag qb = __builtin_shufflevector(*(const bf16x4*)&Qt[d * LDR + lo], *(const bf16x4*)&Qt[d * LDR + hi],
                                                  0, 1, 2, 3, 4, 5, 6, 7);
          dv_acc[t] = M::mma(pa, ob, dv_acc[t]);
          dk_acc[t] = M::mma(da, qb, dk_acc[t]);
        }
      }

      // dQ: dS to LDS [row][key] (one copy per key group), then wave w < NDT
      // forms d-slice w of dQ^T = K^T dS^T
      if (dh == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) dSs[c_row(j, h) * LDS2 + kw] = (bf16)dsj[j];
      }
      __syncthreads();
      if (wave < NDT) {
        f32x16 dq = f32x16{};
#pragma unroll
        for (int ks = 0; ks < kBlock / KSTEP; ++ks) {
          const frag a = *(const frag*)&Kt[(wave * 32 + l32) * LDT + ks * KSTEP + h * KPL];
          const frag bb = *(const frag*)&dSs[l32 * LDS2 + ks * KSTEP + h * KPL];
          dq = M::mma(a, bb, dq);
        }
        // lane = row l32 (its token and head), registers = d wave * 32 + c_row(j, h)
        const int32_t entry = ent_s[l32];
        if (entry >= 0 && lim_s[l32] >= 0) {
          const int i = entry >> 6, slot = entry & 63, hh = l32 % R;
          const int64_t ptok = (((int64_t)b * p.S_q + i) * p.G + g) * p.topk + slot;
          T* po = (T*)p.part_o + ptok * (R * D);
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {  // chunks q = 2 wave + qq of the lane-native layout
            const int q = wave * 2 + qq;
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (bf16)dq[qq * 8 + e];
            __builtin_nontemporal_store(__builtin_bit_cast(i32x4, v), (i32x4*)(po + ((q * 2 + h) * R + hh) * E));
          }
        }
      }
    }

    // the block's dK (times the scale) and dV: lane = d, register j = key c_row(j, h)
#pragma unroll
    for (int t = 0; t < NDH; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kr = kgrp * 32 + c_row(j, h);
        if (kr < rows_ok) {
          const int64_t o = kv0 + (int64_t)kr * D + (dh * NDH + t) * 32 + l32;
          atomicAdd(&bp.dk[o], dk_acc[t][j] * bp.scale);
          atomicAdd(&bp.dv[o], dv_acc[t][j]);
        }
      }
  }
}

// dq[b, i, h, :] = scale * (sum over the row's visible selected blocks of the
// partials); a thread per 16-byte chunk of the lane-native partial layout.
template <int D, int R>
__global__ __launch_bounds__(256) void bwd_dq_combine_kernel(AttnParams p, BwdParams bp) {
  constexpr int E = 8;
  constexpr int NCHT = D * R / E;  // chunks per (token, slot) partial
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= (int64_t)p.B * p.S_q * p.G * NCHT) return;
  const int ch = (int)(u % NCHT);
  const int64_t rowg = u / NCHT;  // (b * S_q + i) * G + g
  const int g = (int)(rowg % p.G);
  const int64_t bi = rowg / p.G;
  const int i = (int)(bi % p.S_q);
  const int b = (int)(bi / p.S_q);
  const int hh = ch % R, h = (ch / R) & 1, q = ch / (2 * R);
  const int64_t t = p.q_offset + i;
  const int32_t* srow = p.sel + (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s2 = 0; s2 < p.topk; ++s2) {
    const int c = srow[s2];
    if (c < 0 || c >= p.nb || (int64_t)c * kBlock > t) continue;
    const bf16x8 x = __builtin_bit_cast(
        bf16x8, __builtin_nontemporal_load((const i32x4*)((const bf16*)p.part_o + (rowg * p.topk + s2) * (R * D) + ch * E)));
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += (float)x[e];
  }
  const int r0 = (q * E) % 16, dt = (q * E) / 16;
  float* orow = bp.dq + (bi * p.Hq + g * R + hh) * D;
#pragma unroll
  for (int m = 0; m < E / 4; ++m) {
    const int d0 = dt * 32 + (r0 / 4 + m) * 8 + 4 * h;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[d0 + e] = acc[4 * m + e] * bp.scale;
  }
}

template <int D, int R>
static hipError_t launch_bwd_t(const AttnParams& p, const BwdParams& bp, hipStream_t s, const KernelTimer* tm) {
  const int64_t rows = (int64_t)p.B * p.S_q * p.Hq;
  const int64_t kvn = (int64_t)p.B * p.G * p.S_k * D;
  timer_start(tm, kKernBwd, s);
  hipLaunchKernelGGL((bwd_dsum_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p, bp);
  // blocks no query selected get zero gradients
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((kvn + 255) / 256)), dim3(256), 0, s, bp.dk, kvn);
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((kvn + 255) / 256)), dim3(256), 0, s, bp.dv, kvn);
  timer_stop(tm, kKernBwd, s);
  launch_gather(p, s, tm);
  timer_start(tm, kKernBwd, s);
  hipLaunchKernelGGL((attn_bwd_kernel<D, R>), dim3(p.grid), dim3(512), 0, s, p, bp);
  timer_stop(tm, kKernBwd, s);
  timer_start(tm, kKernBwdCombine, s);
  const int64_t units = (int64_t)p.B * p.S_q * p.G * (D * R / 8);
  hipLaunchKernelGGL((bwd_dq_combine_kernel<D, R>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, p, bp);
  timer_stop(tm, kKernBwdCombine, s);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const AttnParams& p, const BwdParams& bp, hipStream_t s, const KernelTimer* tm) {
  switch (p.r) {
    case 1: return launch_bwd_t<D, 1>(p, bp, s, tm);
    case 2: return launch_bwd_t<D, 2>(p, bp, s, tm);
    case 4: return launch_bwd_t<D, 4>(p, bp, s, tm);
    case 8: return launch_bwd_t<D, 8>(p, bp, s, tm);
    case 16: return launch_bwd_t<D, 16>(p, bp, s, tm);
    case 32: return launch_bwd_t<D, 32>(p, bp, s, tm);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_attention_bwd(const AttnParams& p, const BwdParams& bp, hipStream_t s,
                                       const KernelTimer* tm) {
  if (p.d == 64) return launch_bwd_d<64>(p, bp, s, tm);
  if (p.d == 128) return launch_bwd_d<128>(p, bp, s, tm);
  return hipErrorInvalidValue;
}

}  // namespace msa

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
// atomics, so their summation order between items is not fixed.
//
// Eight waves.  Waves 0-3 ("S waves") own the block's keys [32w, 32w + 32),
// keep their K rows in registers as MFMA B operands and form S = Q K_w^T, P and
// dV_w += P^T dO; waves 4-7 ("dS waves") own the same keys, keep their V rows
// and form dP = dO V_w^T, dS = P o (dP - Dsum) (P handed over in fp32 through
// LDS) and dK_w += dS^T Q.  S and dP put the key in the lane and the rows in the
// registers, which is directly the A operand of the dV / dK products; their B
// operands (dO and Q with the rows as the reduction index) come from the
// row-major Q and dO tiles through gfx950's transposing LDS read.  A pass holds
// 32 rows ((token, head) pairs, the r heads of a token adjacent); its Q and dO
// rows are fetched three passes ahead into two register sets and written to a
// double-buffered LDS tile one pass ahead.  dS^T goes to LDS and all 8 waves
// form 16 x 16 tiles of dQ^T = K^T dS^T for the previous pass between the next
// pass's products and its barrier; the tile is staged in LDS and stored as a
// bf16 partial [head][d] per (token, slot), summed over the slots by
// bwd_dq_combine_kernel.
#include "common.h"
#include "kernels.h"

namespace msa {

constexpr float kLog2eB = 1.4426950408889634f;

__global__ void bwd_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

// Dsum[b, h, i] = dO[b, i, h, :] . O[b, i, h, :] in fp32: a lane per 16-byte
// chunk (consecutive lanes read consecutive chunks), D / 8 lanes per row summed
// by butterfly.
template <int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(AttnParams p, BwdParams bp) {
  constexpr int L = D / 8;  // lanes per row (16 or 8), a power of two within a wave
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.B * p.S_q * p.Hq;
  const int64_t row = u / L;  // (b * S_q + i) * Hq + h
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *((const bf16x8*)bp.out + u), b8 = *((const bf16x8*)bp.dout + u);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b8[e], acc);
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && (u % L) == 0) {
    const int h = (int)(row % p.Hq);
    const int64_t bi = row / p.Hq;
    const int i = (int)(bi % p.S_q);
    const int b = (int)(bi / p.S_q);
    bp.dsum[((int64_t)b * p.Hq + h) * p.S_q + i] = acc;
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950): within each group of 16 lanes, lane i receives,
// as element e, element i % 4 of the 8 bytes addressed by lane 4 e + i / 4 of
// the group.  Pointing lane s of a group at 4 consecutive elements of row
// r0 + s / 4, column c0 + 4 (s % 4) of a row-major tile hands lane i the column
// c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 read_tr(const bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

template <int D, int R>
__global__ __launch_bounds__(512, 1) void attn_bwd_kernel(AttnParams p, BwdParams bp) {
  using T = bf16;
  using M = Mma<T>;
  using frag = M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
  constexpr int E = 8;               // bf16 elements per 16-byte chunk
  constexpr int NDT = D / 32;        // 32-wide d tiles of dK / dV
  constexpr int TPW = 32 / R;        // tokens per pass of 32 rows
  constexpr int CH = D / E;          // 16-byte chunks per row
  constexpr int NT = 512;            // 8 waves
  constexpr int CPT = (32 * CH + NT - 1) / NT;  // chunks of a pass's Q (and dO) rows per thread
  constexpr bool kAllStage = (32 * CH) % NT == 0;  // false (d = 64): threads past 32 * CH idle
  constexpr int ECH = kBwdTokensPerItem;  // an item's token entries, all staged in LDS
  constexpr int NQT = D / 64;        // 16 x 16 dQ tiles per wave
  constexpr int LDST = 32;           // dS^T pitch: [key][row]
  __shared__ __align__(16) T Ks[kBlock * D];      // K [key][d]
  __shared__ __align__(16) T Qr[2][32 * D];       // the pass's Q and dO rows [row][d], two passes
  __shared__ __align__(16) T Or[2][32 * D];
  __shared__ __align__(16) float Ps[4 * 4 * 64 * 4];  // P handed from S waves to dS waves
  __shared__ __align__(16) T dSt[kBlock * LDST];  // dS^T [key][row]
  constexpr int LDQS = D + 8;                      // dQ tile pitch: [row][d]
  __shared__ __align__(16) T dQs[32 * LDQS];       // a pass's dQ in bf16, stored to the partials in full rows
  __shared__ float lse_s[2][32], dsum_s[2][32];
  __shared__ int lim_s[2][32];
  __shared__ int32_t ent_s[2][32];
  __shared__ int32_t tok_s[ECH];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, gl = lane & 15;  // 16-lane group and lane in it (transposing reads)
  // Waves 0-3 (S waves) own keys [32 w, 32 w + 32): S = Q K_w^T, P, dV_w += P^T dO.
  // Waves 4-7 (dS waves) own the same keys: dP = dO V_w^T, dS = P o (dP - Dsum),
  // dK_w += dS^T Q.  All 8 form 16 x 16 tiles of dQ^T = K^T dS^T.
  const bool sw_wave = wave < 4;
  const int kgrp = wave & 3;
  const int kw = kgrp * 32 + l32;
  // 16-byte chunk c of row r of the [row][d] tiles (Q, dO, K) sits at chunk
  // c ^ sw(r): 16 consecutive rows put one chunk in 16 distinct bank groups (the
  // MFMA A-operand reads) and 4 consecutive rows put a run of 4 (2 for d = 64)
  // chunks in distinct banks (the transposing reads).
  auto sw = [](int r) { return CH == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 3) << 1) | ((r >> 2) & 1)); };
  auto at = [&](int r, int col) { return r * D + ((((col >> 3) ^ sw(r))) << 3) + (col & 7); };
  // dS^T: chunk c of key row k at c ^ 2 ((k >> 3) & 1), so rows k and k + 8 differ
  auto at_ds = [](int k, int row) { return k * LDST + ((((row >> 3) ^ (((k >> 3) & 1) << 1))) << 3) + (row & 7); };
  const float sl2 = p.scale_log2;
  // Per-lane element offsets of the transposing reads; the swizzles repeat every
  // 16 rows of the [row][d] tiles and every 16 key rows of dS^T, so each read of
  // a loop below is one of these plus a constant.
  //  dV / dK B operands: row 4 (grp / 2) + gl / 4 (+ 8), d 32 t + 16 (grp % 2) + 4 (gl % 4)
  int boff[NDT][2];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      boff[t][hf] = at(4 * (grp >> 1) + (gl >> 2) + 8 * hf, 32 * t + 16 * (grp & 1) + 4 * (gl & 3));
  //  dQ: K^T from key rows 8 grp + gl / 4 (+ 4), d 16 d16 + 4 (gl % 4); dS^T from
  //  the same key rows, rows 16 rt + 4 (gl % 4)
  const int d16 = wave % (D / 16);
  const int koff0 = at(8 * grp + (gl >> 2), 16 * d16 + 4 * (gl & 3));
  const int koff4 = at(8 * grp + 4 + (gl >> 2), 16 * d16 + 4 * (gl & 3));
  int doff[NQT];
#pragma unroll
  for (int u = 0; u < NQT; ++u) doff[u] = at_ds(8 * grp + (gl >> 2), 16 * ((wave + 8 * u) / (D / 16)) + 4 * (gl & 3));

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

    // B operands of S (K rows) or dP (V rows) for the wave's keys, lane = key kw
    frag kvf[NKS];
    {
      const T* src = (const T*)(sw_wave ? p.k : p.v) + kv0 + (int64_t)min(kw, rows_ok - 1) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) kvf[ks] = *(const frag*)(src + ks * KSTEP + h * KPL);
    }
    __syncthreads();  // the previous item is done with every LDS tile
    for (int ch = threadIdx.x; ch < kBlock * CH; ch += NT) {  // K, rows past the cache end zero
      const int r = ch / CH, cc = ch - r * CH;
      const i32x4 x = r < rows_ok ? *(const i32x4*)((const T*)p.k + kv0 + (int64_t)r * D + cc * E) : i32x4{};
      *(i32x4*)&Ks[r * D + ((cc ^ sw(r)) << 3)] = x;
    }
    for (int t = threadIdx.x; t < ECH; t += NT) tok_s[t] = t < ntok ? toks[t] : 0;
    __syncthreads();

    // A pass's rows, fetched into one of two register sets three passes before
    // use and written to LDS one pass before: chunks of its Q and dO rows
    // (row = token (p0 + row / R), head row % R) and, in wave 0, row (lane % 32)'s
    // entry with its raw lse and rowsum.
    struct Rows {
      i32x4 qx[CPT], ox[CPT];
      float lse_n, dsum_n;
      int32_t ent_n, pslot_n;
    };
    Rows rw[2];
    auto fetch = [&](int p0, Rows& r) {
      i32x4* qx = r.qx;
      i32x4* ox = r.ox;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int ch = min((int)threadIdx.x + u * NT, 32 * CH - 1);  // idle threads re-read the last chunk
        const int row = ch / CH, col = ch - row * CH;
        const int i = tok_s[min(p0 + row / R, ntok - 1)] >> 6;  // rows past the list reuse a valid row
        const int64_t roff = (((int64_t)b * p.S_q + i) * p.Hq + g * R + row % R) * D + col * E;
        qx[u] = *(const i32x4*)((const T*)p.q + roff);
        ox[u] = *(const i32x4*)((const T*)bp.dout + roff);
      }
      if (wave == 0) {
        const int rr = lane & 31;
        r.pslot_n = p0 + rr / R;
        r.ent_n = tok_s[min(r.pslot_n, ntok - 1)];
        const int64_t hrow = ((int64_t)b * p.Hq + g * R + rr % R) * p.S_q + (r.ent_n >> 6);
        r.lse_n = bp.lse[hrow];
        r.dsum_n = bp.dsum[hrow];
      }
    };
    // registers -> LDS buffer nb_
    auto stage = [&](int nb_, const Rows& r) {
      const i32x4* qx = r.qx;
      const i32x4* ox = r.ox;
      const float lse_n = r.lse_n, dsum_n = r.dsum_n;
      const int32_t ent_n = r.ent_n, pslot_n = r.pslot_n;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int ch = threadIdx.x + u * NT;
        if (!kAllStage && ch >= 32 * CH) break;
        const int row = ch / CH, col = ch - row * CH;
        *(i32x4*)&Qr[nb_][row * D + ((col ^ sw(row)) << 3)] = qx[u];
        *(i32x4*)&Or[nb_][row * D + ((col ^ sw(row)) << 3)] = ox[u];
      }
      if (threadIdx.x < 32) {
        const bool valid = pslot_n < ntok;
        const int64_t rel = qo + (ent_n >> 6) - key0;
        // lim: the last visible key of the block, -1 when the row sees none of it
        lim_s[nb_][threadIdx.x] = (!valid || rel < 0) ? -1 : (rel >= kBlock ? kBlock - 1 : (int)rel);
        ent_s[nb_][threadIdx.x] = valid ? ent_n : -1;
        lse_s[nb_][threadIdx.x] = valid ? lse_n * kLog2eB : 0.f;
        dsum_s[nb_][threadIdx.x] = valid ? dsum_n : 0.f;
      }
    };

    f32x16 acc[NDT];  // dV_w (S waves) or dK_w (dS waves): lane = d, register j = key c_row(j, h)
#pragma unroll
    for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};

    // dQ^T = K^T dS^T of the previous pass in 16 x 16 x 32 tiles, issued between
    // the next pass's S / dP products and its barrier (dS^T is rewritten only
    // after that barrier): wave w takes d rows 16 (w % (D / 16)) and row tiles
    // (w + 8 u) / (D / 16); lane = row 16 rt + gl, registers = d 4 grp + j.  The
    // tile goes to LDS; after the barrier every thread stores 16 bytes of it.
    constexpr int QCH = D / 8;  // 16-byte chunks per dQ row
    const int srow = (int)threadIdx.x / QCH, schunk = (int)threadIdx.x % QCH;  // this thread's chunk to store
    int32_t st_ent = -1;  // the stored pass's entry and visibility of row srow
    int st_lim = -1;
    auto dq_pass = [&]() {
      f32x4 dq[NQT];
#pragma unroll
      for (int u = 0; u < NQT; ++u) dq[u] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < kBlock / 32; ++ks) {
        const frag a = __builtin_shufflevector(read_tr(Ks + koff0 + 32 * ks * D), read_tr(Ks + koff4 + 32 * ks * D), 0,
                                               1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int u = 0; u < NQT; ++u) {
          const frag bb = __builtin_shufflevector(read_tr(dSt + doff[u] + 32 * ks * LDST),
                                                  read_tr(dSt + doff[u] + (32 * ks + 4) * LDST), 0, 1, 2, 3, 4, 5, 6, 7);
          dq[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, dq[u], 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < NQT; ++u) {
        const int rt = (wave + 8 * u) / (D / 16);
        *(bf16x4*)&dQs[(16 * rt + gl) * LDQS + 16 * d16 + 4 * grp] =
            bf16x4{(bf16)dq[u][0], (bf16)dq[u][1], (bf16)dq[u][2], (bf16)dq[u][3]};
      }
    };
    // partial per (token, slot): [head][d] bf16; thread srow, schunk writes 16 bytes
    auto dq_store = [&]() {
      if (srow < 32 && st_ent >= 0 && st_lim >= 0) {
        const int i = st_ent >> 6, slot = st_ent & 63;
        const int64_t ptok = (((int64_t)b * p.S_q + i) * p.G + g) * p.topk + slot;
        *(i32x4*)((T*)p.part_o + (ptok * R + srow % R) * D + schunk * 8) = *(const i32x4*)&dQs[srow * LDQS + schunk * 8];
      }
    };

    fetch(0, rw[0]);
    stage(0, rw[0]);
    if (TPW < ntok) fetch(TPW, rw[1]);
    if (2 * TPW < ntok) fetch(2 * TPW, rw[0]);
    __syncthreads();
    for (int p00 = 0; p00 < ntok; p00 += 2 * TPW)
#pragma unroll
    for (int buf = 0; buf < 2; ++buf) {  // pass p0 uses row buffer buf and refills register set buf ^ 1
      const int p0 = p00 + buf * TPW;
      if (p0 >= ntok) break;
      // the next pass's rows into the other buffer (its readers, the previous
      // pass, finished before that pass's last barrier); the register set
      // freed refetches three passes ahead
      if (p0 + TPW < ntok) {
        stage(buf ^ 1, rw[buf ^ 1]);
        if (p0 + 3 * TPW < ntok) fetch(p0 + 3 * TPW, rw[buf ^ 1]);
      }
      const T* Qb = Qr[buf];
      const T* Ob = Or[buf];

      // S = Q K_w^T (S waves) or dP = dO V_w^T (dS waves): lane = key kw, register j = row c_row(j, h)
      f32x16 s = f32x16{};
      {
        const T* A = sw_wave ? Qb : Ob;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const frag a = *(const frag*)&A[at(l32, ks * KSTEP + h * KPL)];
          s = M::mma(a, kvf[ks], s);
        }
      }
      if (p0 > 0) dq_pass();  // the previous pass's dQ, overlapping this pass's products
      frag pa[2];  // P or dS in bf16: A operands of dV / dK, step ks2 pairs index h*8+e with row c_row(8 ks2 + e, h)
      if (sw_wave) {
        float pj[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = c_row(j, h);
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], sl2, -lse_s[buf][row]));
          pj[j] = kw <= lim_s[buf][row] ? e : 0.f;
        }
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
          *(f32x4*)&Ps[((kgrp * 4 + j4) * 64 + lane) * 4] = f32x4{pj[4 * j4], pj[4 * j4 + 1], pj[4 * j4 + 2], pj[4 * j4 + 3]};
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pa[ks2][e] = (bf16)pj[ks2 * 8 + e];
      }
      __syncthreads();  // P is in LDS (and the previous pass's dQ tile)
      if (p0 > 0) dq_store();
      if (!sw_wave) {
        float dsj[16];
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const f32x4 pv = *(const f32x4*)&Ps[((kgrp * 4 + j4) * 64 + lane) * 4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * j4 + e;
            dsj[j] = pv[e] * (s[j] - dsum_s[buf][c_row(j, h)]);
          }
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pa[ks2][e] = (bf16)dsj[ks2 * 8 + e];
        // dS^T [key][row]: registers 4m .. 4m + 3 are rows 8m + 4h .. + 3
#pragma unroll
        for (int m = 0; m < 4; ++m)
          *(bf16x4*)&dSt[at_ds(kw, 8 * m + 4 * h)] =
              bf16x4{(bf16)dsj[4 * m], (bf16)dsj[4 * m + 1], (bf16)dsj[4 * m + 2], (bf16)dsj[4 * m + 3]};
      }
      // dV_w += P^T dO or dK_w += dS^T Q; B operands (rows as the reduction
      // index) by transposing reads: rows 16 ks2 + 4 h' + 0..3 and + 8, with h'
      // the half of the 16-lane group
      {
        const T* Bt = sw_wave ? Ob : Qb;
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
          for (int t = 0; t < NDT; ++t) {
            const frag bb = __builtin_shufflevector(read_tr(Bt + boff[t][0] + 16 * ks2 * D),
                                                    read_tr(Bt + boff[t][1] + 16 * ks2 * D), 0, 1, 2, 3, 4, 5, 6, 7);
            acc[t] = M::mma(pa[ks2], bb, acc[t]);
          }
      }
      // this pass's dQ row for the store, read before the metadata buffer turns over
      if (srow < 32) {
        st_ent = ent_s[buf][srow];
        st_lim = lim_s[buf][srow];
      }
      __syncthreads();  // dS^T is in LDS; the pass's row buffers are free
    }
    dq_pass();  // the item's last pass
    __syncthreads();
    dq_store();

    // the block's dV (S waves) or dK times the scale (dS waves): lane = d, register j = key c_row(j, h)
    // (key kgrp * 32 + 4 h + c_row(j, 0), d 32 t + l32): one base per lane plus constants
    float* dst = (sw_wave ? bp.dv : bp.dk) + kv0 + (int64_t)(kgrp * 32 + 4 * h) * D + l32;
    const int lim_k = rows_ok - (kgrp * 32 + 4 * h);
    const float f = sw_wave ? 1.f : bp.scale;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (c_row(j, 0) < lim_k) atomicAdd(dst + c_row(j, 0) * D + t * 32, acc[t][j] * f);
  }
}

// dq[b, i, h, :] = scale * (sum over the row's visible selected blocks of the
// partials [head][d]); a thread per 16-byte chunk.  The slots' chunks are
// loaded from clamped addresses, up to 32 of them before any is used, and the
// slots that are not visible selected blocks are dropped by selects; the sum
// runs in slot order.
template <int D, int R, int KMAX>
__global__ __launch_bounds__(512) void bwd_dq_combine_kernel(AttnParams p, BwdParams bp) {
  constexpr int E = 8;
  constexpr int CPR = D / E;  // chunks per head row
  const int64_t u = (int64_t)blockIdx.x * 512 + threadIdx.x;
  if (u >= (int64_t)p.B * p.S_q * p.G * R * CPR) return;
  const int ch = (int)(u % CPR);
  const int64_t rest = u / CPR;
  const int hh = (int)(rest % R);
  const int64_t rowg = rest / R;  // (b * S_q + i) * G + g
  const int g = (int)(rowg % p.G);
  const int64_t bi = rowg / p.G;
  const int i = (int)(bi % p.S_q);
  const int b = (int)(bi / p.S_q);
  const int64_t t = p.q_offset + i;
  const int32_t* srow = p.sel + (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
  constexpr int KC = KMAX < 32 ? KMAX : 32;  // slots held in registers at once
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s0 = 0; s0 < KMAX; s0 += KC) {
    i32x4 x[KC];
    int cs[KC];
#pragma unroll
    for (int s2 = 0; s2 < KC; ++s2) {
      const int sc = min(s0 + s2, p.topk - 1);
      cs[s2] = srow[sc];
      x[s2] = __builtin_nontemporal_load(
          (const i32x4*)((const bf16*)p.part_o + ((rowg * p.topk + sc) * R + hh) * D + ch * E));
    }
#pragma unroll
    for (int s2 = 0; s2 < KC; ++s2) {
      const int c = cs[s2];
      const bool used = s0 + s2 < p.topk && c >= 0 && c < p.nb && (int64_t)c * kBlock <= t;
      const bf16x8 xv = __builtin_bit_cast(bf16x8, x[s2]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += used ? (float)xv[e] : 0.f;
    }
  }
  f32x4* orow = (f32x4*)(bp.dq + (bi * p.Hq + g * R + hh) * D + ch * E);
  orow[0] = f32x4{acc[0], acc[1], acc[2], acc[3]} * bp.scale;
  orow[1] = f32x4{acc[4], acc[5], acc[6], acc[7]} * bp.scale;
}

template <int D, int R>
static hipError_t launch_bwd_t(const AttnParams& p, const BwdParams& bp, hipStream_t s, const KernelTimer* tm) {
  const int64_t rows = (int64_t)p.B * p.S_q * p.Hq;
  const int64_t kvn = (int64_t)p.B * p.G * p.S_k * D;
  timer_start(tm, kKernBwd, s);
  hipLaunchKernelGGL((bwd_dsum_kernel<D>), dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, s, p, bp);
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
  const dim3 cgrid((unsigned)((units + 511) / 512));
  if (p.topk <= 16) hipLaunchKernelGGL((bwd_dq_combine_kernel<D, R, 16>), cgrid, dim3(512), 0, s, p, bp);
  else if (p.topk <= 32) hipLaunchKernelGGL((bwd_dq_combine_kernel<D, R, 32>), cgrid, dim3(512), 0, s, p, bp);
  else hipLaunchKernelGGL((bwd_dq_combine_kernel<D, R, 64>), cgrid, dim3(512), 0, s, p, bp);
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

// KL-alignment teacher of MSA on gfx950, forward only.
//
// Method (snilld.dk page "MiniMax lancerer MSA", section "Træning og
// stabilisering"; Hungarian page "MiniMax új eljárása …", section "A
// betanítás és a kernel-optimalizáció"): Top-k cannot be differentiated, so a
// KL loss trains the index branch to follow the main branch.  The teacher is
// the main branch's attention distribution over the selected tokens, averaged
// over the heads of the GQA group; the student is the softmax of the index
// scores over the same tokens.  Per (b, g, i), with s_j the index scores times
// index_scale:
//   KL = sum_j pbar(j) (log pbar(j) - log q(j)),   q = softmax(s)
//      = sum_j pbar(j) (log pbar(j) - s_j) + lse(s).
// With the main branch's log-sum-exp given, pbar(j) needs no second softmax
// pass, so every selected block contributes additive terms: its sum of
// pbar (log pbar - s), plus the max and the exp-sum of its index scores.
//
// Work items and token lists are those of the main branch's gather (items of
// kKlTokensPerItem tokens).  Per item the block's K and index keys are staged
// in LDS; the index scores S_idx^T = K_idx Q_idx^T of all the item's tokens are
// formed first, 32 tokens per MFMA tile (the r heads of a token share its index
// query, so they are computed once per token), and kept in LDS in place of the
// index keys.  Passes of 4 waves x 32 (token, head) rows then recompute the
// main scores on 32x32 MFMA tiles.  For r >= 8 a pass forms S = Q K^T: a lane
// holds one key of each key tile and 16 (token, head) rows in its registers,
// so a token's head sum is in-lane adds plus one swap between the lane halves.
// For r < 8 it forms S^T = K Q^T: the r heads of a token sit in r adjacent
// lanes, and their probabilities are summed by a butterfly that leaves lane hh
// of the group owning 64 / r of its half's keys.  Either way each logarithm is
// taken once per key, not once per head, and each lane reads just its keys'
// index scores.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace msa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// The 64 scores of a lane (4 key tiles x 16 registers) as one vector value:
// selecting between its elements by a lane-dependent condition then stays a
// register select (an array indexed that way would be placed in memory).
typedef float f32x64 __attribute__((ext_vector_type(64)));

// The partner of a lane at butterfly step O (lanes of a token are R aligned,
// consecutive lanes): lanes differing in bit 0 or bit 1 (quad permutes), lanes
// i and 7 - i of each 8 (half-row mirror) and i and 15 - i of each 16 (row
// mirror) -- all DPP moves, full-rate VALU with no LDS round trip -- and lanes
// 16 apart (a lane permute).  Each pairs lanes whose bit O differs and whose
// higher bits agree, which is all a butterfly needs.
template <int O>
__device__ __forceinline__ float partner(float x) {
  const int v = __builtin_bit_cast(int, x);
  if constexpr (O == 1) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  else if constexpr (O == 2) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  else if constexpr (O == 4) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
  else if constexpr (O == 8) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
  else return __shfl_xor(x, O);
}

// Butterfly over the R lanes of a token (steps O = R/2, R/4, ..., 1): at each
// step a lane keeps the upper or lower half of its N values by bit O of hh and
// adds the partner's copy of that half.  Afterwards lane hh holds the sums of
// slots hh * (64 / R) + k in x[k], k < 64 / R.
template <int O, int N>
struct Butterfly {
  __device__ static __forceinline__ void sum(f32x64& x, int hh) {
    const bool up = (hh & O) != 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      const float lo = x[k], hi = x[k + N / 2];
      const float slo = lo + partner<O>(lo), shi = hi + partner<O>(hi);
      x[k] = up ? shi : slo;
    }
    Butterfly<O / 2, N / 2>::sum(x, hh);
  }
};

template <int N>
struct Butterfly<0, N> {
  __device__ static __forceinline__ void sum(f32x64&, int) {}
};

// Reductions over all lanes of one token: its R lanes (steps 1, 2, 4, ...: each
// step joins two groups already reduced) in both halves.
template <int R, int O = 1>
__device__ __forceinline__ float token_sum(float x) {
  if constexpr (O < R) return token_sum<R, 2 * O>(x + partner<O>(x));
  else return x + __shfl_xor(x, 32);
}

// Sum / max over the 32 lanes of a lane half.
__device__ __forceinline__ float half_sum(float x) {
  x += partner<1>(x);
  x += partner<2>(x);
  x += partner<4>(x);
  x += partner<8>(x);
  return x + __shfl_xor(x, 16);
}
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, partner<1>(x));
  x = fmaxf(x, partner<2>(x));
  x = fmaxf(x, partner<4>(x));
  x = fmaxf(x, partner<8>(x));
  return fmaxf(x, __shfl_xor(x, 16));
}

template <int R, int O = 1>
__device__ __forceinline__ float token_max(float x) {
  if constexpr (O < R) return token_max<R, 2 * O>(fmaxf(x, partner<O>(x)));
  else return fmaxf(x, __shfl_xor(x, 32));
}

template <typename T, typename S, int D, int R, int DI>
// two workgroups per CU for bf16; the fp32 form (correctness path) takes the registers of one
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void kl_teacher_kernel(AttnParams p, KlParams kp) {
  using M = Mma<T>;
  using IO = ChunkIO<T, S>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP, NKI = DI / KSTEP;
  constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk of T
  constexpr int LDK = D + E, LDI = DI + E;
  constexpr int TPW = 32 / R, TPP = 4 * TPW;
  constexpr int NV = 64;      // score registers per lane: 4 key tiles x 16
  constexpr int NK = NV / R;  // keys a lane owns after the head butterfly
  // index scores of the item's tokens, fp32 [token][h][register slot]: the C
  // layout of the 32x32 tiles (lane = token, slot kt * 16 + j = key
  // kt * 32 + c_row(j, h)); the token pitch is 4 floats past 128, so the 32
  // tokens a store instruction writes fall in distinct banks
  constexpr int LDSC = 2 * NV + 4;
  static_assert(kKlTokensPerItem <= 64, "two 32-token index tiles per item");
  constexpr int KI_BYTES = kBlock * LDI * (int)sizeof(T), SC_BYTES = kKlTokensPerItem * LDSC * 4;
  __shared__ __align__(16) T Ks[kBlock * LDK];
  __shared__ __align__(16) char kis_raw[KI_BYTES > SC_BYTES ? KI_BYTES : SC_BYTES];  // index keys, then scores
  __shared__ int32_t ent_s[kBlock];  // the item's token entries ((row << 6) | slot)
  // r >= 8: the transposed pass (S = Q K^T, a lane holds one key per key tile
  // and 16 rows); the log2-domain lse of each wave's 32 rows goes through LDS
  // to the lanes whose registers hold those rows
  constexpr bool kT = R >= 8;
  __shared__ float lse_s[4][32];
  T* KIs = (T*)kis_raw;
  float* sc = (float*)kis_raw;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int hh = l32 % R;
  const int64_t total = p.direct ? p.n_direct : (int64_t)*p.n_items;
  const float sl2 = p.scale_log2;  // main scale (key scale included) in log2 units

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
    // an unmapped page, or a block past the end of the cache: nothing to score (uniform)
    const int slen = cache_len(p.cm, p.S_k, b);
    const int64_t kv0 = block_offset(p.cm, p.S_k, p.G, D, b, g, c);
    const int64_t ki0 = block_offset(p.cm, p.S_k, 1, DI, b, 0, c);
    if (kv0 < 0 || ki0 < 0 || (int64_t)c * kBlock >= slen) continue;
    const int64_t qo = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b);

    __syncthreads();  // the previous item is done with the LDS tiles
    if ((int)threadIdx.x < ntok) ent_s[threadIdx.x] = toks ? toks[threadIdx.x] : direct_tok;
    {
      // K and the index keys of the block; rows past the cache end re-read its
      // last row and are zeroed; every load is issued before any is stored
      const int rows_ok = (int)min((int64_t)kBlock, (int64_t)slen - (int64_t)c * kBlock);
      constexpr int KU = kBlock * D / E / 256, IU = kBlock * DI / E / 256;
      static_assert(KU >= 1 && IU >= 1 && (kBlock * DI / E) % 256 == 0, "staging covers the block");
      const S* ksrc = (const S*)p.k + kv0;
      const S* isrc = (const S*)kp.k_idx + ki0;
      typename IO::raw kx[KU], ix[IU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int ch = threadIdx.x + u * 256;
        const int row = ch / (D / E), col = ch - row * (D / E);
        kx[u] = IO::load(ksrc + (int64_t)min(row, rows_ok - 1) * D + col * E);
      }
#pragma unroll
      for (int u = 0; u < IU; ++u) {
        const int ch = threadIdx.x + u * 256;
        const int row = ch / (DI / E), col = ch - row * (DI / E);
        ix[u] = IO::load(isrc + (int64_t)min(row, rows_ok - 1) * DI + col * E);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int ch = threadIdx.x + u * 256;
        const int row = ch / (D / E), col = ch - row * (D / E);
        *(i32x4*)&Ks[row * LDK + col * E] = row < rows_ok ? IO::widen(kx[u]) : i32x4{};
      }
#pragma unroll
      for (int u = 0; u < IU; ++u) {
        const int ch = threadIdx.x + u * 256;
        const int row = ch / (DI / E), col = ch - row * (DI / E);
        *(i32x4*)&KIs[row * LDI + col * E] = row < rows_ok ? IO::widen(ix[u]) : i32x4{};
      }
    }
    __syncthreads();

    // index scores of the item's tokens: wave w forms key tiles 2 (w / 2) and
    // 2 (w / 2) + 1 of token tile w % 2 (tokens past the list use the first
    // entry's row and are never read)
    {
      const int tt = wave & 1;
      const bool active = tt * 32 < ntok;  // uniform
      f32x16 siacc[2];
      siacc[0] = f32x16{};
      siacc[1] = f32x16{};
      if (active) {
        const int32_t e0 = ent_s[min(tt * 32 + l32, ntok - 1)];
        const T* qirow = (const T*)kp.q_idx + (((int64_t)b * p.S_q + (e0 >> 6)) * p.G + g) * DI;
        frag qif[NKI];
#pragma unroll
        for (int ks = 0; ks < NKI; ++ks) qif[ks] = *(const frag*)(qirow + ks * KSTEP + h * KPL);
#pragma unroll
        for (int ks = 0; ks < NKI; ++ks)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int kt = 2 * (wave >> 1) + u;
            const frag a = *(const frag*)&KIs[(kt * 32 + l32) * LDI + ks * KSTEP + h * KPL];
            siacc[u] = M::mma(a, qif[ks], siacc[u]);
          }
      }
      __syncthreads();  // every wave is done with the index keys
      if (active) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kt = 2 * (wave >> 1) + u;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v4 = f32x4{siacc[u][q4 * 4], siacc[u][q4 * 4 + 1], siacc[u][q4 * 4 + 2], siacc[u][q4 * 4 + 3]};
            if constexpr (kT)  // [token][key]: registers 4 q4 .. 4 q4 + 3 are keys kt * 32 + c_row(4 q4, h) + 0 .. 3
              *(f32x4*)(sc + (tt * 32 + l32) * LDSC + kt * 32 + c_row(q4 * 4, h)) = v4;
            else
              *(f32x4*)(sc + (tt * 32 + l32) * LDSC + h * NV + kt * 16 + q4 * 4) = v4;
          }
        }
      }
      __syncthreads();
    }

    const int64_t key0 = (int64_t)c * kBlock;
    const int head = g * R + hh;
    // A wave's rows of pass ps: the token entry (from LDS), its Q row, index
    // query row and main lse; loaded one pass ahead of their use.  Rows past
    // the token list read token 0's (valid) rows and are never stored.
    auto load_rows = [&](int ps, frag (&qf)[NKS], float& lse2, int32_t& entry) {
      const int tslot = ps * TPP + wave * TPW + l32 / R;
      entry = tslot < ntok ? ent_s[tslot] : -1;
      const int i = entry >= 0 ? entry >> 6 : 0;
      const T* qrow = (const T*)p.q + (((int64_t)b * p.S_q + i) * p.Hq + head) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const frag*)(qrow + ks * KSTEP + h * KPL);
      lse2 = kp.lse[((int64_t)b * p.Hq + head) * p.S_q + i] * kLog2e;
    };
    auto pass = [&](int ps, const frag (&qf)[NKS], float lse2, int32_t entry) {
      const int i = entry >= 0 ? entry >> 6 : 0, slot = entry & 63;
      const int64_t rel = qo + i - key0;  // query position relative to the block
      const bool rv = entry >= 0 && rel >= 0;
      const int lim = (!rv || rel >= kBlock) ? kBlock - 1 : (int)rel;  // last visible key
      const bool masked = __any(lim < kBlock - 1);  // the causal mask only bites in a local block

      // teacher: this head's probabilities exp(scale q.k - lse)
      f32x64 pv;
      {
        f32x16 sacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const frag a = *(const frag*)&Ks[(kt * 32 + l32) * LDK + ks * KSTEP + h * KPL];
            sacc[kt] = M::mma(a, qf[ks], sacc[kt]);
          }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 16; ++j) pv[kt * 16 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][j], sl2, -lse2));
      }
      Butterfly<R / 2, NV>::sum(pv, hh);  // pv[0, NK): sums over the token's heads

      // student: this lane's slots of the token's index scores times index_scale
      float sv[NK];
      {
        const int tslot = min(ps * TPP + wave * TPW + l32 / R, ntok - 1);
        const float* src = sc + tslot * LDSC + h * NV + hh * NK;
#pragma unroll
        for (int k = 0; k < NK; ++k) sv[k] = src[k] * kp.index_scale;
      }
      // Lane hh holds register slots hh * NK + k (slot s: key tile s / 16,
      // register s % 16).  The heads of a token share its visibility limit, so
      // the causal mask of a local block applies here, after the head sums.
      if (masked) {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const int sl = hh * NK + k;
          const int key = (sl >> 4) * 32 + c_row(sl & 15, h);
          if (key > lim) {
            pv[k] = 0.f;
            sv[k] = kNegInf;
          }
        }
      }

      // this lane's keys, then the token's totals over its lanes
      float ent = 0.f, smax = kNegInf;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const float pb = pv[k] * (1.0f / R);
        ent += pb > 0.f ? pb * (__builtin_amdgcn_logf(pb) * kLn2 - sv[k]) : 0.f;
        smax = fmaxf(smax, sv[k]);
      }
      ent = token_sum<R>(ent);
      smax = token_max<R>(smax);
      float sexp = 0.f;
      if (smax != kNegInf) {
#pragma unroll
        for (int k = 0; k < NK; ++k) sexp += __builtin_amdgcn_exp2f((sv[k] - smax) * kLog2e);
      }
      sexp = token_sum<R>(sexp);
      if (rv && hh == 0 && h == 0) {
        const int64_t ptok = (((int64_t)b * p.S_q + i) * p.G + g) * p.topk + slot;
        kp.part[ptok * 3 + 0] = ent;
        kp.part[ptok * 3 + 1] = smax;
        kp.part[ptok * 3 + 2] = sexp;
      }
    };

    // The transposed pass (r >= 8): the Q rows are the A operand, so lane l
    // holds key kt * 32 + l % 32 of each key tile and rows c_row(j, h) of the
    // wave's 32 (token, head) rows in register j -- token j / JPT, the same in
    // both lane halves.  A token's head sum is then JPT in-lane adds and one
    // swap between the halves, after which half h carries tokens 2 u + h (one
    // token per pass: both halves carry it and half 0 reports), and the key
    // reductions run over the 32 lanes of a half.
    constexpr int JPT = 16 / TPW;            // registers per token
    constexpr int TPL = TPW >= 2 ? TPW / 2 : 1;  // tokens a lane carries after the swap
    auto pass_t = [&](int ps, const frag (&qf)[NKS], float lse2, int32_t entry) {
      // the per-row lse into the registers that hold the rows
      if (h == 0) lse_s[wave][l32] = lse2;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float lr[16];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 v4 = *(const f32x4*)&lse_s[wave][a * 8 + h * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) lr[a * 4 + e] = v4[e];
      }
      (void)entry;
      // the pass's tokens (uniform): entry, query index, visibility limit
      int ti[TPW], tslot_c[TPW], tlim[TPW], tptok_slot[TPW];
      bool trv[TPW];
      bool masked = false;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tslot = ps * TPP + wave * TPW + t;
        const int e = tslot < ntok ? ent_s[tslot] : -1;
        ti[t] = e >= 0 ? e >> 6 : 0;
        tptok_slot[t] = e & 63;
        tslot_c[t] = min(tslot, ntok - 1);
        const int64_t rel = qo + ti[t] - key0;
        trv[t] = e >= 0 && rel >= 0;
        tlim[t] = (!trv[t] || rel >= kBlock) ? kBlock - 1 : (int)rel;
        masked |= tlim[t] < kBlock - 1;
      }

      f32x16 sacc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const frag a = *(const frag*)&Ks[(kt * 32 + l32) * LDK + ks * KSTEP + h * KPL];
          sacc[kt] = M::mma(qf[ks], a, sacc[kt]);
        }
      // this half's head sums of each token's probabilities, key kt * 32 + l32
      float hs[TPW][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          float acc = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][t * JPT], sl2, -lr[t * JPT]));
#pragma unroll
          for (int j = t * JPT + 1; j < (t + 1) * JPT; ++j)
            acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][j], sl2, -lr[j]));
          hs[t][kt] = acc;
        }
      // both halves' heads: token 2 u + h (u < TPL) in half h, or the one token in both
      float pb[TPL][4], sv[TPL][4];
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const int t0 = TPW >= 2 ? 2 * u : 0, t1 = TPW >= 2 ? 2 * u + 1 : 0;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(hs[t0][kt]), __float_as_uint(hs[t1][kt]),
                                                          false, false);
          pb[u][kt] = (__uint_as_float(x[0]) + __uint_as_float(x[1])) * (1.0f / R);
        }
        const int tsl = h && TPW >= 2 ? tslot_c[t1] : tslot_c[t0];
        const float* src = sc + tsl * LDSC + l32;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sv[u][kt] = src[kt * 32] * kp.index_scale;
        if (masked) {  // the heads of a token share its limit: mask after the sums
          const int lim = h && TPW >= 2 ? tlim[t1] : tlim[t0];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            if (kt * 32 + l32 > lim) {
              pb[u][kt] = 0.f;
              sv[u][kt] = kNegInf;
            }
        }
      }
      // per token: the entropy terms and the index scores' max and exp-sum over its 128 keys
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        float ent = 0.f, smax = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const float q = pb[u][kt];
          ent += q > 0.f ? q * (__builtin_amdgcn_logf(q) * kLn2 - sv[u][kt]) : 0.f;
          smax = fmaxf(smax, sv[u][kt]);
        }
        ent = half_sum(ent);
        smax = half_max(smax);
        float sexp = 0.f;
        if (smax != kNegInf) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) sexp += __builtin_amdgcn_exp2f((sv[u][kt] - smax) * kLog2e);
        }
        sexp = half_sum(sexp);
        const int t0 = TPW >= 2 ? 2 * u : 0, t1 = TPW >= 2 ? 2 * u + 1 : 0;
        const bool rv = h && TPW >= 2 ? trv[t1] : trv[t0];
        if (rv && l32 == 0 && (TPW >= 2 || h == 0)) {
          const int i = h && TPW >= 2 ? ti[t1] : ti[t0];
          const int slot = h && TPW >= 2 ? tptok_slot[t1] : tptok_slot[t0];
          const int64_t ptok = (((int64_t)b * p.S_q + i) * p.G + g) * p.topk + slot;
          kp.part[ptok * 3 + 0] = ent;
          kp.part[ptok * 3 + 1] = smax;
          kp.part[ptok * 3 + 2] = sexp;
        }
      }
    };
    auto run_pass = [&](int ps, const frag (&qf)[NKS], float lse2, int32_t entry) {
      if constexpr (kT) pass_t(ps, qf, lse2, entry);
      else pass(ps, qf, lse2, entry);
    };

    const int npass = wave * TPW < ntok ? (ntok - wave * TPW + TPP - 1) / TPP : 0;
    if (npass > 0) {
      frag qfA[NKS], qfB[NKS];
      float lseA, lseB;
      int32_t entA, entB;
      load_rows(0, qfA, lseA, entA);
      for (int ps = 0; ps < npass; ps += 2) {
        load_rows(ps + 1, qfB, lseB, entB);
        __builtin_amdgcn_sched_barrier(0);
        run_pass(ps, qfA, lseA, entA);
        if (ps + 1 < npass) {
          load_rows(ps + 2, qfA, lseA, entA);
          __builtin_amdgcn_sched_barrier(0);
          run_pass(ps + 1, qfB, lseB, entB);
        }
      }
    }
  }
}

// One thread per (b, g, i): the block terms of the row's visible selected
// blocks give KL = sum ent + lse_idx, lse_idx = m + log sum_s l_s e^(m_s - m).
// A row that sees no block gets KL = 0 and lse_idx = -inf.
__global__ __launch_bounds__(256) void kl_combine_kernel(AttnParams p, KlParams kp) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b * G + g) * S_q + i
  if (row >= (int64_t)p.B * p.G * p.S_q) return;
  const int i = (int)(row % p.S_q);
  const int64_t bg = row / p.S_q;
  const int g = (int)(bg % p.G);
  const int b = (int)(bg / p.G);
  const int64_t t = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + i;
  const int32_t* srow = p.sel + row * p.topk;
  const float* part = kp.part + ((((int64_t)b * p.S_q + i) * p.G + g) * p.topk) * 3;
  float ent = 0.f, m = kNegInf;
  for (int s = 0; s < p.topk; ++s) {
    const int c = srow[s];
    if (c < 0 || c >= p.nb || (int64_t)c * kBlock > t || !block_mapped(p.cm, b, c)) continue;
    ent += part[s * 3 + 0];
    m = fmaxf(m, part[s * 3 + 1]);
  }
  float l = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < p.topk; ++s) {
      const int c = srow[s];
      if (c < 0 || c >= p.nb || (int64_t)c * kBlock > t || !block_mapped(p.cm, b, c)) continue;
      l += part[s * 3 + 2] * __builtin_amdgcn_exp2f((part[s * 3 + 1] - m) * kLog2e);
    }
  }
  const float lse = m != kNegInf ? m + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
  kp.kl[row] = m != kNegInf ? ent + lse : 0.f;
  if (kp.idx_lse) kp.idx_lse[row] = lse;
}

template <typename T, typename S, int D, int R, int DI>
static hipError_t launch_kl_t(const AttnParams& p, const KlParams& kp, hipStream_t s, const KernelTimer* tm) {
  launch_gather(p, s, tm);
  timer_start(tm, kKernKlTeacher, s);
  hipLaunchKernelGGL((kl_teacher_kernel<T, S, D, R, DI>), dim3(p.grid), dim3(256), 0, s, p, kp);
  timer_stop(tm, kKernKlTeacher, s);
  timer_start(tm, kKernKlCombine, s);
  const int64_t rows = (int64_t)p.B * p.G * p.S_q;
  hipLaunchKernelGGL(kl_combine_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p, kp);
  timer_stop(tm, kKernKlCombine, s);
  return hipGetLastError();
}

template <typename T, typename S, int D, int R>
static hipError_t launch_kl_r(const AttnParams& p, const KlParams& kp, hipStream_t s, const KernelTimer* tm) {
  switch (kp.index_dim) {
    case 32: return launch_kl_t<T, S, D, R, 32>(p, kp, s, tm);
    case 64: return launch_kl_t<T, S, D, R, 64>(p, kp, s, tm);
    case 128: return launch_kl_t<T, S, D, R, 128>(p, kp, s, tm);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename S, int D>
static hipError_t launch_kl_d(const AttnParams& p, const KlParams& kp, hipStream_t s, const KernelTimer* tm) {
  switch (p.r) {
    case 1: return launch_kl_r<T, S, D, 1>(p, kp, s, tm);
    case 2: return launch_kl_r<T, S, D, 2>(p, kp, s, tm);
    case 4: return launch_kl_r<T, S, D, 4>(p, kp, s, tm);
    case 8: return launch_kl_r<T, S, D, 8>(p, kp, s, tm);
    case 16: return launch_kl_r<T, S, D, 16>(p, kp, s, tm);
    case 32: return launch_kl_r<T, S, D, 32>(p, kp, s, tm);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename S>
static hipError_t launch_kl_s(const AttnParams& p, const KlParams& kp, hipStream_t s, const KernelTimer* tm) {
  if (p.d == 64) return launch_kl_d<T, S, 64>(p, kp, s, tm);
  if (p.d == 128) return launch_kl_d<T, S, 128>(p, kp, s, tm);
  return hipErrorInvalidValue;
}

hipError_t launch_kl_teacher(const AttnParams& p, const KlParams& kp, bool bf16_inputs, bool fp8_cache,
                             hipStream_t s, const KernelTimer* tm) {
  if (fp8_cache) return bf16_inputs ? launch_kl_s<bf16, e4m3>(p, kp, s, tm) : hipErrorInvalidValue;
  if (bf16_inputs) return launch_kl_s<bf16, bf16>(p, kp, s, tm);
  return launch_kl_s<float, float>(p, kp, s, tm);
}

}  // namespace msa

// Index branch of MSA on gfx950: block max-pooled index scores and the
// per-group exp-free Top-k with the forced local block.
//
// Method (snilld.dk page "MiniMax lancerer MSA", section "Hvad er MSA i
// praksis"; abstract page "MiniMax 稀疏注意力", 摘要): every GQA group's
// index-query head is scored against the single shared index-key head, the
// token scores are max-pooled over 128-token blocks, and each (query, group)
// keeps the Top-k blocks, always including the query's local block.  Softmax
// preserves order, so raw scores are ranked (no exp).
//
// Design.  A unit is a tile of (query row, group) pairs of one sequence (the
// rows of q_idx [B,S_q,G,D] are contiguous per (i, g)) and a contiguous range of
// key blocks; a workgroup of 8 waves (bf16 queries; 4 otherwise) takes 512
// pairs (256 for k > 16), 64 per wave.  Per block, the shared k_idx tile (128
// keys x D) reaches LDS -- by DMA into a ring of four tiles for native bf16
// keys, through registers into two tiles otherwise -- and is multiplied
// against the rows' index queries held in registers: S^T = K_idx * Q_idx^T with
// 32x32 MFMA tiles, so each lane owns one query row and 64 of the block's 128
// keys (the other 64 sit in lane ^ 32).  With one key split per tile the
// units run on a persistent grid in snake order (index_topk_kernel).
// The block max is a register reduction plus one cross-half exchange; it goes
// straight into a running top list in registers and is never stored.  The two
// lane halves take alternate blocks, so each keeps its own list; at the end the
// two are merged through LDS into one list per (row, key split).  The lists of
// a row's splits are merged by topk_merge_kernel, which also adds the local
// block, sorts ascending and pads with -1; with a single split the index kernel
// does that itself.  For k > 32 (lists of 63) each lane half writes its own
// list and topk_merge_kernel always merges them.
//
// Index keys stored as OCP FP8 E4M3 (S = e4m3) are widened exactly to bf16 as
// they are staged, so the scores are the same as for the bf16 values they hold.
//
// Exactness: with integer-valued inputs every score is an integer of
// magnitude <= D * max|q| * max|k| < 2^24, so fp32 MFMA accumulation is exact in
// any order, and ties are broken by block index exactly as the definition says.
// Only full blocks before the local block are ranked (block c < L ends at or
// before t), so no causal mask is needed inside the ranked blocks.
#include <atomic>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace msa {

template <int CAP>
__device__ __forceinline__ void list_insert(float (&s)[CAP], int (&id)[CAP], float x, int c) {
  // s is sorted descending; every index already present is smaller than c, so
  // an equal score keeps the earlier (lower-index) entry first.  Slot j takes
  // s[j - 1] when x > s[j - 1], x when s[j] < x <= s[j - 1], else keeps s[j]:
  // the median of the three.  The ids follow through bit masks, which keeps
  // the update free of branches.
  unsigned m_hi = x > s[CAP - 1] ? ~0u : 0u;  // x > s[j], for the slot j being updated
#pragma unroll
  for (int j = CAP - 1; j >= 1; --j) {
    const unsigned m_lo = x > s[j - 1] ? ~0u : 0u;
    s[j] = __builtin_amdgcn_fmed3f(s[j - 1], x, s[j]);
    const unsigned t = (m_lo & (unsigned)id[j - 1]) | (~m_lo & (unsigned)c);
    id[j] = (int)((m_hi & t) | (~m_hi & (unsigned)id[j]));
    m_hi = m_lo;
  }
  s[0] = m_hi ? x : s[0];
  id[0] = m_hi ? c : id[0];
}

// Slots HI down to LO of list_insert.  Called for descending ranges in turn
// (CAP - 1 first), it finds the slots above HI already updated and those from
// LO - 1 down still as they were, which is all a slot's update reads.
template <int CAP, int HI, int LO>
__device__ __forceinline__ void list_insert_range(float (&s)[CAP], int (&id)[CAP], float x, int c) {
  unsigned m_hi = x > s[HI] ? ~0u : 0u;
#pragma unroll
  for (int j = HI; j >= (LO > 1 ? LO : 1); --j) {
    const unsigned m_lo = x > s[j - 1] ? ~0u : 0u;
    s[j] = __builtin_amdgcn_fmed3f(s[j - 1], x, s[j]);
    const unsigned t = (m_lo & (unsigned)id[j - 1]) | (~m_lo & (unsigned)c);
    id[j] = (int)((m_hi & t) | (~m_hi & (unsigned)id[j]));
    m_hi = m_lo;
  }
  if constexpr (LO == 0) {
    s[0] = m_hi ? x : s[0];
    id[0] = m_hi ? c : id[0];
  }
}

// f(std::integral_constant<int, I>) for I = B .. E - 1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }

// v in ascending order: Batcher's bitonic sorting network (NP a power of two),
// min / max pairs with every index known at compile time.
template <int NP>
__device__ __forceinline__ void sort_ascending(int (&v)[NP]) {
  static_assert((NP & (NP - 1)) == 0, "power of two");
#pragma unroll
  for (int lk = 1; (1 << lk) <= NP; ++lk)
#pragma unroll
    for (int lj = lk - 1; lj >= 0; --lj)
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int l = i ^ (1 << lj);
        if (l > i) {
          const int lo = min(v[i], v[l]), hi = max(v[i], v[l]);
          const bool up = (i & (1 << lk)) == 0;  // direction of this bitonic run
          v[i] = up ? lo : hi;
          v[l] = up ? hi : lo;
        }
      }
}

// One (row, key split) result: with several splits the merged list goes to
// the partial lists for topk_merge_kernel; with one split the first min(k-1, L)
// entries are the selection, and the local block and -1 padding are added
// with the ids in ascending order.
template <int CAP>
__device__ __forceinline__ void emit_row(const IndexParams& p, int b, int n, int split, int L, const float (&ms)[CAP],
                                         const int (&mi)[CAP]) {
  if (p.nsplit > 1) {
    const int64_t rowg = (int64_t)b * p.rows_per_b + n;
    float* ds = p.part_s + (rowg * p.nsplit + split) * CAP;
    int32_t* di = p.part_i + (rowg * p.nsplit + split) * CAP;
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
      ds[j] = ms[j];
      di[j] = mi[j];
    }
    return;
  }
  const int i = n / p.G, g = n - (n / p.G) * p.G;
  int32_t* out = p.sel + (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
  if (L < 0) {  // a row before the start of its cache selects nothing
    for (int j = 0; j < p.topk; ++j) out[j] = -1;
    return;
  }
  const int take = min(p.topk - 1, L);
  // the ids of the first `take` entries in ascending order; the other slots
  // hold INT_MAX and sort last
  constexpr int NP = pow2_at_least(CAP + 1);
  int v[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) v[j] = j < CAP && j < take ? mi[j] : INT_MAX;
  sort_ascending(v);
  auto val = [&](int j) { return j < take ? v[j] : j == take ? L : -1; };
  if (p.topk == NP && (reinterpret_cast<uintptr_t>(p.sel) & 15) == 0) {  // whole 16-byte rows
#pragma unroll
    for (int j = 0; j < NP; j += 4) *(i32x4*)(out + j) = i32x4{val(j), val(j + 1), val(j + 2), val(j + 3)};
  } else {
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (j < p.topk) out[j] = val(j);
  }
}

// The wide form (lists of 63): a lane half's own list for row rowg, written as
// partial list `list` of the row for topk_merge_kernel.
template <int CAP>
__device__ __forceinline__ void emit_half_list(const IndexParams& p, int64_t rowg, int list, const float (&ls)[CAP],
                                               const int (&li)[CAP]) {
  float* ds = p.part_s + (rowg * p.nsplit * p.lps + list) * CAP;
  int32_t* di = p.part_i + (rowg * p.nsplit * p.lps + list) * CAP;
#pragma unroll
  for (int j = 0; j < CAP; ++j) {
    ds[j] = ls[j];
    di[j] = li[j];
  }
}

// The unit (row tile tg = b * ntile + tile, key split) of workgroup lin, or
// false when it has none.  With a unit list (sequences of their own lengths)
// the units holding work come first.  Otherwise, with key splits, hardware
// hands consecutive workgroup ids to the 8 XCDs in turn, so the order gives
// each XCD a contiguous run of units (one key range, many row tiles) whose
// k_idx range stays in its L2; without splits, heavy_first puts the tiles with
// the most causal blocks first.
// Unit lin of the packed unit list, derived by the calling wave from the
// sequence lengths (the few-row form, one row tile per sequence): lane j counts
// the busy splits of sequences PER j .. PER j + PER - 1, loaded together; a
// wave-wide inclusive scan orders the counts by sequence, a ballot finds the
// lane whose range holds lin, and that lane walks its own sequences.  The same
// units in the same order as index_units_kernel writes, without its launch and
// the two dependent loads of its list.
__device__ __forceinline__ bool inline_unit(const IndexParams& p, int lin, int& b, int& split) {
  constexpr int PER = kInlineUnitsPerLane;
  const int lane = threadIdx.x & 63;
  int cnt[PER];
  int sum = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int bb = lane * PER + u;
    int c = 0;
    if (bb < p.B) {
      if (p.nsplit == 1) {
        c = 1;
      } else {
        const int L = local_block(first_pos(p.cm, p.q_offset, p.S_q, p.S_k, bb) + (p.rows_per_b - 1) / p.G);
        c = L > 0 ? (L + p.chunk - 1) / p.chunk : 0;
      }
    }
    cnt[u] = c;
    sum += c;
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lin >= __shfl(incl, 63)) return false;
  const int owner = __popcll(__ballot(incl <= lin));  // lanes whose units all precede lin
  int r = lin - (incl - sum), sb = 0, ss = 0;
  bool found = false;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (!found && r < cnt[u]) {
      found = true;
      sb = lane * PER + u;
      ss = r;
    }
    r -= cnt[u];
  }
  b = __shfl(sb, owner);
  split = __shfl(ss, owner);
  return true;
}

__device__ __forceinline__ bool unit_of(const IndexParams& p, int lin, bool heavy_first, int& tg, int& split) {
  if (p.units_inline) return inline_unit(p, lin, tg, split);  // one row tile per sequence: tg = b
  if (p.units) {
    if (lin >= *p.unit_count) return false;
    const int u = p.units[lin];
    split = u & 127;
    tg = u >> 7;
    return true;
  }
  if (p.nsplit == 1 && heavy_first) {
    // heaviest row tiles first, the sequences interleaved: workgroup lin goes
    // to XCD lin % 8, so each XCD gets the tiles of as few sequences as possible
    // (one when B divides 8), whose k_idx blocks its running tiles share in L2
    if (lin >= p.nunits) return false;
    split = 0;
    tg = (lin % p.B) * p.ntile + p.ntile - 1 - lin / p.B;
    return true;
  }
  const int logical = (lin & 7) * p.grid_per_xcd + (lin >> 3);
  if (logical < 0 || logical >= p.nunits) return false;
  split = logical / p.ntile_total;
  tg = logical - split * p.ntile_total;
  return true;
}

// Unit list for sequences of their own lengths: per row tile, one unit per key
// split that holds blocks before the tile's last local block (one unit when
// there is a single split, which also writes rows without blocks), packed in
// tile order by one workgroup (a scan over per-thread counts).
__global__ __launch_bounds__(1024) void index_units_kernel(IndexParams p) {
  __shared__ int32_t s_cnt[1024];
  const int n = p.ntile_total;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  auto count = [&](int tg) {
    if (p.nsplit == 1) return 1;
    const int b = tg / p.ntile, tile = tg - b * p.ntile;
    const int n_last = min((tile + 1) * p.rows_wg, p.rows_per_b) - 1;
    const int L = local_block(first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + n_last / p.G);
    return L > 0 ? (L + p.chunk - 1) / p.chunk : 0;
  };
  int mine = 0;
  for (int tg = lo; tg < hi; ++tg) mine += count(tg);
  s_cnt[threadIdx.x] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = (int)threadIdx.x >= off ? s_cnt[threadIdx.x - off] : 0;
    __syncthreads();
    s_cnt[threadIdx.x] += a;
    __syncthreads();
  }
  int o = s_cnt[threadIdx.x] - mine;
  for (int tg = lo; tg < hi; ++tg) {
    const int k = count(tg);
    for (int sp = 0; sp < k; ++sp) p.units[o++] = (tg << 7) | sp;
  }
  if (threadIdx.x == 1023) *p.unit_count = s_cnt[1023];
}

// Issue order of one accumulator chain of index_topk_kernel: each of its N
// products is followed by up to V VALU instructions and, when DS, one LDS read.
template <int N, int V, bool DS>
__device__ __forceinline__ void chain_schedule() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if constexpr (DS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    chain_schedule<N - 1, V, DS>();
  }
}

// Keeps the work producing x where it stands in program order: the empty asm
// takes x in a VGPR and counts as a side effect, so the optimisers cannot sink
// that work past the scheduling fences that follow.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(int& x) { asm volatile("" : "+v"(x)); }

// Row tile tg, key split `split` (both uniform over the workgroup); tid is
// threadIdx.x.
template <typename T, typename S, int DI, int CAP, int RT>
__device__ __forceinline__ void index_topk_unit(const IndexParams& p, int tg, int split, int tid) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = DI / KSTEP;
  // LDS tile of a block: 128 rows of DI elements of T, unpadded; 16-byte chunk c
  // of row r sits at chunk c ^ sw(r), so the 16 rows an A-operand read touches
  // at one column fall in distinct banks
  constexpr int RB = DI * (int)sizeof(T);  // bytes per LDS row
  constexpr int CPR = RB / 16;             // 16-byte chunks per LDS row
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  constexpr int SWS = CPR >= 16 ? 0 : CPR == 8 ? 1 : CPR == 4 ? 2 : 3;
  constexpr int TILE_BYTES = kBlock * RB;
  auto sw = [](int r) { return (r >> SWS) & (CPR - 1); };
  auto at = [&](int r, int col) { return r * DI + (((col / EPC) ^ sw(r)) * EPC) + col % EPC; };
  constexpr int kWaves = index_waves(CAP + 1, sizeof(T) == 2);
  constexpr int NT = 64 * kWaves;
  // native bf16 keys go straight from HBM into the tile (no registers); e4m3
  // and fp32 keys are staged through registers
  constexpr bool kDma = std::is_same<S, T>::value && sizeof(T) == 2 && TILE_BYTES % (kWaves * 1024) == 0;
  constexpr int ROWS_WAVE = 32 * RT;
  constexpr int ROWS_WG = kWaves * ROWS_WAVE;
  // staging: 16-byte chunks of k_idx in its storage type S; a chunk holds SE
  // keys' elements and widens to SE / (16 / sizeof(T)) chunks of T in LDS
  constexpr int SE = 16 / (int)sizeof(S);
  constexpr int CH_PER_ROW = DI / SE;
  constexpr int CH_TOTAL = kBlock * CH_PER_ROW;  // staged chunks per block: chunk threadIdx.x + u NT, u < CH_PER_THREAD
  constexpr int CH_PER_THREAD = kDma ? 1 : (CH_TOTAL + NT - 1) / NT;
  static_assert(kDma || CH_TOTAL % NT == 0 || CH_TOTAL < NT, "staging split");
  // LDS tiles: a ring of NBUF with native keys (DMA runs NBUF - 1 blocks
  // ahead; the workgroup has the CU's LDS to itself), two with staged keys
  constexpr int NBUF = kDma ? 4 : 2;
  constexpr int KS_BYTES = NBUF * TILE_BYTES;
  constexpr bool kWide = CAP == kIndexWideCap;      // lane halves write their own lists
  constexpr int LIST_BYTES = kWide ? 0 : RT * kWaves * 2 * CAP * 32 * 8;  // every list of the workgroup
  constexpr int SMEM = KS_BYTES > LIST_BYTES ? KS_BYTES : LIST_BYTES;
  static_assert(SMEM <= 160 * 1024, "LDS of one CU");
  __shared__ __align__(16) char smem[SMEM];
  T* Ks = (T*)smem;  // [NBUF][kBlock * DI]

  const int b = tg / p.ntile;
  const int tile = tg - b * p.ntile;
  const int n_first = tile * ROWS_WG;
  const int n_last = min(n_first + ROWS_WG, p.rows_per_b) - 1;
  const int64_t qo = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b);
  const int Lmax = max(local_block(qo + n_last / p.G), 0);
  const int c_begin = split * p.chunk;
  const int c_end = min(c_begin + p.chunk, Lmax);
  const bool has_blocks = c_begin < c_end;
  if (!has_blocks && p.nsplit > 1) return;  // a single split still writes rows with L = 0

  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  int rowL[RT];
  bool rvalid[RT];
  frag qf[RT][NKS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n_first + wave * ROWS_WAVE + rt * 32 + l32;
    rvalid[rt] = n < p.rows_per_b;
    const int nc = rvalid[rt] ? n : p.rows_per_b - 1;  // invalid rows read a valid row
    rowL[rt] = local_block(qo + nc / p.G);
    const T* qrow = (const T*)p.q_idx + ((int64_t)b * p.rows_per_b + nc) * DI;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[rt][ks] = *(const frag*)(qrow + ks * KSTEP + h * KPL);
  }

  float ls[RT][CAP];
  int li[RT][CAP];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
      ls[rt][j] = kNegInf;
      li[rt][j] = -1;
    }

  const S* kpool = (const S*)p.k_idx;
  // Keys arrive ahead of the blocks being scored.  Native bf16 keys go by DMA
  // into a ring of four LDS tiles a pair of blocks at a time: while one pair is
  // scored from two tiles the next lands in the other two, and the workgroup
  // meets at a barrier once per pair.  Staged keys are loaded two blocks ahead
  // into registers (`pre` holds block c + 1, stored to the other of two tiles
  // after block c is scored, `pre2` is in flight for block c + 2).  Past the
  // range's end the last block is fetched again and its scores are dropped, so
  // every block runs the same straight-line code.
  i32x4 pre[CH_PER_THREAD], pre2[CH_PER_THREAD];
  // Element offset of block c in the key pool and whether its page is mapped
  // (an unmapped page is read from the pool start and scored -inf).  The page
  // id is a scalar load (the constant address space), so it does not count
  // against the vector loads in flight that the ring's waits count.
  typedef const int32_t __attribute__((address_space(4))) cint32;
  auto lookup = [&](int c, int64_t& off, bool& mapped) {
    if (!p.cm.pages) {
      mapped = true;
      off = ((int64_t)b * p.S_k + (int64_t)c * kBlock) * DI;
      return;
    }
    const int pg = ((cint32*)p.cm.pages)[(int64_t)b * p.cm.max_pages + c];
    mapped = pg >= 0 && pg < p.cm.num_pages;
    off = mapped ? (int64_t)pg * kBlock * DI : 0;
  };
  // one staged chunk into the LDS tile: SE elements from column col of a row
  auto stage = [&](T* tile, int ch, i32x4 x) {
    const int row = ch / CH_PER_ROW, col = (ch - row * CH_PER_ROW) * SE;
    if constexpr (std::is_same<S, T>::value) {
      *(i32x4*)&tile[at(row, col)] = x;
    } else {  // 16 e4m3 keys widen to two chunks of bf16
      const uint2 a = e4m3x4_to_bf16((uint32_t)x[0]), b2 = e4m3x4_to_bf16((uint32_t)x[1]);
      const uint2 c2 = e4m3x4_to_bf16((uint32_t)x[2]), d2 = e4m3x4_to_bf16((uint32_t)x[3]);
      *(i32x4*)&tile[at(row, col)] = i32x4{(int)a.x, (int)a.y, (int)b2.x, (int)b2.y};
      *(i32x4*)&tile[at(row, col + 8)] = i32x4{(int)c2.x, (int)c2.y, (int)d2.x, (int)d2.y};
    }
  };
  auto load_staged = [&](i32x4(&dst)[CH_PER_THREAD], int64_t off) {
    const i32x4* src = (const i32x4*)(kpool + off);
#pragma unroll
    for (int u = 0; u < CH_PER_THREAD; ++u)
      if (tid + u * NT < CH_TOTAL) dst[u] = src[tid + u * NT];
  };
  auto stage_all = [&](T* tile, const i32x4(&src)[CH_PER_THREAD]) {
#pragma unroll
    for (int u = 0; u < CH_PER_THREAD; ++u)
      if (tid + u * NT < CH_TOTAL) stage(tile, tid + u * NT, src[u]);
  };
  // native keys: a block straight into tile bi.  Wave w fills 1 KiB pieces
  // (w * NU + u) of the tile; the hardware puts lane L's 16 bytes at byte 16 L
  // of a piece, so lane L reads the chunk the swizzle assigns to that slot.
  constexpr int NU = kDma ? TILE_BYTES / (kWaves * 1024) : 1;
  uint32_t dma_src[NU];  // byte offset within the block of lane L's chunk of piece u
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int kb = (wave * NU + u) * 1024 + lane * 16;
    const int r = kb / RB, pc = (kb % RB) / 16;
    dma_src[u] = (uint32_t)(r * RB + (pc ^ sw(r)) * 16);
  }
  auto dma_block = [&](int64_t off, int bi) {
    const char* src = (const char*)(kpool + off);
    char* tile = smem + bi * TILE_BYTES;
#pragma unroll
    for (int u = 0; u < NU; ++u)
      __builtin_amdgcn_global_load_lds((const void*)(src + dma_src[u]),
                                       (__attribute__((address_space(3))) void*)(tile + (wave * NU + u) * 1024), 16,
                                       0, 0);
  };
  // Wait until at most n of this wave's vector loads are in flight (s_waitcnt
  // vmcnt(n); the export and LDS counters are left alone).
  auto wait_vm = [](auto n_tag) {
    constexpr int n = decltype(n_tag)::value;
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };
  // Workgroup barrier of the block loop.  With DMA it leaves out the release
  // fence of __syncthreads(), which waits for every load in flight: this
  // wave's LDS accesses are complete (lgkmcnt 0), its DMA of the next pair has
  // landed (wait_vm before it), and the asm's memory clobber keeps the compiler
  // from moving memory operations across it.
  auto block_barrier = [] {
    if constexpr (kDma) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else __syncthreads();
  };

  // mq: bit j = block c + j is mapped, for the block (staged) or pair (DMA) c
  // about to be scored; off_n: offsets of the blocks its code fetches (c + 2 and,
  // with DMA, c + 3)
  int mq = 0;
  int64_t off_n[2] = {0, 0};
  if (has_blocks) {
    int64_t o[4];
    bool m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lookup(min(c_begin + j, c_end - 1), o[j], m[j]);
      mq |= (int)m[j] << j;
    }
    off_n[0] = o[2];
    off_n[1] = o[3];
    if constexpr (kDma) {
      dma_block(o[0], 0);
      dma_block(o[1], 1);
      wait_vm(std::integral_constant<int, 0>{});  // this wave's pieces of the first pair are in LDS
    } else {
      load_staged(pre, o[0]);
      load_staged(pre2, o[1]);
      stage_all(Ks, pre);
#pragma unroll
      for (int u = 0; u < CH_PER_THREAD; ++u) pre[u] = pre2[u];
    }
  }
  block_barrier();

  // Software pipeline of one wave.  A block is 4 key tiles x RT row tiles =
  // 4 RT accumulator chains of NKS products; chain q accumulates into acc[q & 1].
  // While chain q runs on the matrix core the lanes fold chain q - 1's finished
  // tile into the running block max, and after a key tile's last chain the
  // next key tile's A operands are loaded into the registers that chain has
  // finished with.  Blocks pair up: lanes of half 0 rank the first block of a
  // pair for their row, lanes of half 1 the second (one exchange of the half
  // maxima); a pair's ranking is spread over the next pair's 8 RT chains, a
  // quarter of one row tile's list after every other chain.  (bf16 operands;
  // fp32 ones have too few registers left for the overlap, so their chains are
  // folded as they finish and their operands load per key tile.)
  constexpr bool kPipe = sizeof(T) == 2;
  float pm[RT], pmA[RT], pmB[RT], full[RT];
  int fullc = 0;  // block of this lane half's entry in the pair being ranked
  f32x16 acc[2];
  frag a[NKS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) pm[rt] = pmA[rt] = pmB[rt] = full[rt] = kNegInf;
  auto fold = [&](float& m, const f32x16& t) {
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, t[j]);
  };
  // the full block maxima of the pair c0, c0 + 1 from pmA / pmB: lanes 0-31 get
  // block c0's, lanes 32-63 block c0 + 1's
  auto pair_full = [&](int c0) {
    fullc = c0 + h;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(pmA[rt]), __float_as_uint(pmB[rt]), false,
                                                      false);
      const bool keep = rvalid[rt] & (fullc < rowL[rt]);
      full[rt] = keep ? fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1])) : kNegInf;
    }
  };
  // chunk k (0 .. 4 RT - 1) of ranking a pair: row tile k / 4, the k % 4-th
  // quarter of its list's slots from the bottom
  auto rank_chunk = [&](auto k_tag) {
    constexpr int k = decltype(k_tag)::value, rt = k / 4, W = (CAP + 3) / 4;
    constexpr int HI = CAP - 1 - (k % 4) * W, LO = HI - W + 1 > 0 ? HI - W + 1 : 0;
    if constexpr (HI >= 0) {
      list_insert_range<CAP, HI, LO>(ls[rt], li[rt], full[rt], fullc);
#pragma unroll
      for (int j = LO; j <= HI; ++j) {
        pin(ls[rt][j]);
        pin(li[rt][j]);
      }
    }
  };
  // block c from `tile`, the blk-th (0, 1) of its pair; valid: its max counts
  auto score_block = [&](int c, auto blk_tag, const T* tile, bool valid) {
    constexpr int blk = decltype(blk_tag)::value;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const frag*)&tile[at(l32, ks * KSTEP + h * KPL)];
    if constexpr (blk == 0) pair_full(c - 2);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) pm[rt] = kNegInf;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 4 * RT>([&](auto q_tag) {
      // stage q: chain q's products; between them chain q - 1's fold, every
      // other stage a chunk of the previous pair's ranking, and after a key
      // tile's last row tile the next key tile's operands
      constexpr int q = decltype(q_tag)::value, kt = q / RT, rt = q % RT;
      constexpr int sp = blk * 4 * RT + q;  // stage within the pair
      constexpr bool ranks = sp % 2 == 1;
      constexpr bool loads = kPipe && rt == RT - 1 && kt < 3;
      if constexpr (!kPipe && rt == 0 && kt > 0) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const frag*)&tile[at(kt * 32 + l32, ks * KSTEP + h * KPL)];
        __builtin_amdgcn_sched_barrier(0);
      }
      f32x16 t = M::mma(a[0], qf[rt][0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < NKS; ++ks) t = M::mma(a[ks], qf[rt][ks], t);
      if constexpr (loads) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const frag*)&tile[at((kt + 1) * 32 + l32, ks * KSTEP + h * KPL)];
      }
      if constexpr (!kPipe) {
        fold(pm[rt], t);
        pin(pm[rt]);
      } else if constexpr (q > 0) {
        fold(pm[(q - 1) % RT], acc[(q - 1) & 1]);
        pin(pm[(q - 1) % RT]);
      }
      if constexpr (ranks) rank_chunk(std::integral_constant<int, (sp - 1) / 2>{});
      if constexpr (kPipe) chain_schedule<NKS, ranks ? 4 : 2, loads>();
      __builtin_amdgcn_sched_barrier(0);
      acc[q & 1] = t;
    });
    if constexpr (kPipe) fold(pm[RT - 1], acc[1]);  // the last chain (4 RT is even)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float v = valid ? pm[rt] : kNegInf;
      if constexpr (blk == 0) pmA[rt] = v;
      else pmB[rt] = v;
    }
  };
  int buf = 0;  // the tile of block c (DMA: of the pair's first block)
  if constexpr (kDma) {
    for (int c = c_begin; c < c_end; c += 2) {
      // the next pair into the other two tiles (their readers passed the barrier)
      dma_block(off_n[0], buf ^ 2);
      dma_block(off_n[1], (buf ^ 2) + 1);
      score_block(c, std::integral_constant<int, 0>{}, Ks + buf * (kBlock * DI), (mq & 1) != 0);
      score_block(c + 1, std::integral_constant<int, 1>{}, Ks + (buf + 1) * (kBlock * DI),
                  (mq & 2) != 0 && c + 1 < c_end);
      {  // the pair after next (page lookups stay out of the code above)
        bool m0, m1;
        lookup(min(c + 4, c_end - 1), off_n[0], m0);
        lookup(min(c + 5, c_end - 1), off_n[1], m1);
        mq = (mq | ((int)m0 << 4) | ((int)m1 << 5)) >> 2;
      }
      wait_vm(std::integral_constant<int, 0>{});  // this wave's pieces of the next pair are in LDS
      block_barrier();
      buf ^= 2;
    }
  } else {
    auto staged_block = [&](int c, auto blk_tag) {
      load_staged(pre2, off_n[0]);  // block c + 2
      score_block(c, blk_tag, Ks + buf * (kBlock * DI), (mq & 1) != 0);
      stage_all(Ks + (buf ^ 1) * (kBlock * DI), pre);  // block c + 1 into the other tile
#pragma unroll
      for (int u = 0; u < CH_PER_THREAD; ++u) pre[u] = pre2[u];
      {
        bool m;
        lookup(min(c + 3, c_end - 1), off_n[0], m);
        mq = (mq | ((int)m << 3)) >> 1;
      }
      block_barrier();
      buf ^= 1;
    };
    for (int c = c_begin; c < c_end; c += 2) {
      staged_block(c, std::integral_constant<int, 0>{});
      if (c + 1 < c_end) {
        staged_block(c + 1, std::integral_constant<int, 1>{});
      } else {  // no second block: its share of the previous pair's ranking, and an empty max
        static_for<2 * RT, 4 * RT>([&](auto k_tag) { rank_chunk(k_tag); });
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) pmB[rt] = kNegInf;
      }
    }
  }
  // the ring's last fetches (blocks past the range, into tiles nobody reads)
  // land before the tiles are reused below or the workgroup's LDS is released
  if constexpr (kDma) wait_vm(std::integral_constant<int, 0>{});
  if (has_blocks) {  // the last pair
    pair_full(c_begin + ((c_end - c_begin - 1) & ~1));
    static_for<0, 4 * RT>([&](auto k_tag) { rank_chunk(k_tag); });
  }

  if constexpr (kWide) {  // list split * 2 + h of each row
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = n_first + wave * ROWS_WAVE + rt * 32 + l32;
      if (rvalid[rt]) emit_half_list<CAP>(p, (int64_t)b * p.rows_per_b + n, split * 2 + h, ls[rt], li[rt]);
    }
    return;
  }
  // Merge the two half lists of each row through LDS (the K tiles are free
  // now), then write one list per (row, split).  Every list goes to LDS at
  // once; with two row tiles the lanes of half h merge row tile h, with one
  // the lanes of half 0.
  float* xs = (float*)smem;  // [RT][kWaves][2 halves][CAP][32 rows]
  int* xi = (int*)(smem + LIST_BYTES / 2);
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
      const int o = (((rt * kWaves + wave) * 2 + h) * CAP + j) * 32 + l32;
      xs[o] = ls[rt][j];
      xi[o] = li[rt][j];
    }
  __syncthreads();
  static_assert(RT == 1 || RT == 2, "one row tile per lane half");
  const int mt = RT == 2 ? h : 0;  // the row tile this lane merges
  const bool mvalid = (RT == 2 || h == 0) && (mt ? rvalid[RT - 1] : rvalid[0]);
  if (mvalid) {
    const int n = n_first + wave * ROWS_WAVE + mt * 32 + l32;
    const int oa = (((mt * kWaves + wave) * 2 + 0) * CAP) * 32 + l32;
    const int ob = oa + CAP * 32;
    float ms[CAP];
    int mi[CAP];
    int ia = 0, ib = 0;
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
      const float sa = ia < CAP ? xs[oa + ia * 32] : kNegInf;
      const int ida = ia < CAP ? xi[oa + ia * 32] : -1;
      const float sb = ib < CAP ? xs[ob + ib * 32] : kNegInf;
      const int idb = ib < CAP ? xi[ob + ib * 32] : -1;
      // empty entries (id -1) rank last
      const bool take_a = idb < 0 || (ida >= 0 && ranks_before(sa, ida, sb, idb));
      ms[j] = take_a ? sa : sb;
      mi[j] = take_a ? ida : idb;
      ia += take_a ? 1 : 0;
      ib += take_a ? 0 : 1;
    }
    if constexpr (!kWide) emit_row<CAP>(p, b, n, split, mt ? rowL[RT - 1] : rowL[0], ms, mi);
  }
}

// The units of a launch: one per workgroup, or with p.persist a grid of at
// most as many workgroups as the GPU holds at once, each taking one unit per
// round q = 0, 1, ... in snake order (workgroup w: unit q G + w in even
// rounds, q G + G - 1 - w in odd ones).  With the heaviest row tiles first the
// rounds of every workgroup add up to about the same number of blocks, and a
// CU goes on to its next unit without waiting for the dispatcher.
// Each round reads the parameters and the thread id anew through an empty asm,
// so what a unit derives from them is computed inside the round rather than
// hoisted out of the loop and kept live across the block loop.
template <typename T, typename S, int DI, int CAP, int RT>
__global__ __launch_bounds__(64 * index_waves(CAP + 1, sizeof(T) == 2), 1) void index_topk_kernel(IndexParams p) {
  typedef const IndexParams __attribute__((address_space(4))) kparams;
  const int G = (int)gridDim.x, w = (int)blockIdx.x;
  for (int q = 0;; ++q) {
    kparams* kp = (kparams*)__builtin_amdgcn_kernarg_segment_ptr();  // p: the only argument
    int tid = (int)threadIdx.x;
    asm volatile("" : "+s"(kp), "+v"(tid));
    const IndexParams pu = *(const IndexParams*)kp;  // loads of the constant address space
    const int lin = (q & 1) ? (q + 1) * G - 1 - w : q * G + w;
    int tg, split;
    if (!unit_of(pu, lin, true, tg, split)) return;
    // uniform: block and page indices stay in scalar registers
    index_topk_unit<T, S, DI, CAP, RT>(pu, __builtin_amdgcn_readfirstlane(tg), __builtin_amdgcn_readfirstlane(split),
                                       tid);
    if (!pu.persist) return;
    __syncthreads();  // the next unit's keys overwrite the LDS this one's lists used
  }
}

// Few rows per sequence (S_q * G <= 32, e.g. decode).  One 32-row tile holds
// all of a sequence's (row, group) pairs, so rather than four waves sharing a
// staged block, each wave takes whole blocks of the unit's key range (wave w:
// blocks c_begin + w, c_begin + w + 4, ...), with no barrier in the block loop.
// A 32-key tile is read with linear non-temporal 16-byte loads one tile ahead of
// its use (the pattern that streams fastest from HBM) and rearranged into the
// MFMA A-operand layout through the wave's own LDS tile.  A lane's operand is 16
// bytes of one key row: for e4m3 keys that is two k-steps, so the reduction
// dimension is taken in the order d = 32 p + 16 h + 8 (ks % 2) + e (p = ks / 2)
// for both operands; any order common to K and Q gives the same dot products.
// As in the kernel above the two lane halves of a wave rank alternate blocks of
// its sequence; the 4 x 2 lists of a row are merged through LDS at the end.
template <typename T, typename S, int DI, int CAP>
__global__ __launch_bounds__(256, CAP == kIndexWideCap ? 1 : 2) void index_topk_small_kernel(IndexParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = DI / KSTEP;
  constexpr bool kNative = std::is_same<S, T>::value;
  // one lane's 16-byte share of a K tile per load: one k-step of native keys,
  // two k-steps of e4m3 keys
  typedef typename std::conditional<kNative, frag, i32x4>::type kraw;
  static_assert(kNative || (sizeof(S) == 1 && KPL == 8 && NKS % 2 == 0), "e4m3 keys come as 16-byte runs");
  constexpr int NKR = kNative ? NKS : NKS / 2;  // 16-byte loads per lane per tile
  // A 32-key tile (32 rows of RB bytes, contiguous in memory) is read with
  // linear non-temporal 16-byte loads (lane L, load u: byte 1024 u + 16 L), put
  // in the wave's LDS tile and read back in the MFMA layout: lane l takes
  // 16-byte chunk 2 u + h of row l % 32 (k-step u of native keys; k-steps 2u,
  // 2u + 1 of e4m3 keys, whose dims the query fragments take in the same order).
  // Chunk c of row r sits at chunk c ^ sw(r), which puts the 16 rows of a read
  // and the 16 chunks of a write in distinct LDS banks.
  constexpr int RB = DI * (int)sizeof(S);  // bytes per key row
  constexpr int CPR = RB / 16;             // 16-byte chunks per row
  static_assert(NKR * 1024 == 32 * RB, "a tile is NKR loads of 1 KiB per wave");
  constexpr int SWS = CPR == 16 ? 0 : CPR == 8 ? 1 : CPR == 4 ? 2 : 3;
  auto sw = [](int r) { return (r >> SWS) & (CPR - 1); };
  // element offset of k-step ks, lane half h in the query row (16 elements per 16 bytes of e4m3)
  auto koff = [](int ks, int hh) { return kNative ? ks * KSTEP + hh * KPL : (ks / 2) * 32 + hh * 16 + (ks % 2) * 8; };
  constexpr int NL = 8;  // lists per row: 4 waves x 2 lane halves
  constexpr bool kWide = CAP == kIndexWideCap;  // the 8 lists go to topk_merge_kernel unmerged
  constexpr int MERGE_BYTES = kWide ? 0 : NL * CAP * 32 * 8, TILE_BYTES = 4 * 32 * RB;
  static_assert(MERGE_BYTES <= 65536, "list merge fits the static LDS");
  // the waves' key tiles during the block loop, the list merge afterwards
  __shared__ __align__(16) char lds_raw[MERGE_BYTES > TILE_BYTES ? MERGE_BYTES : TILE_BYTES];
  float* xs = (float*)lds_raw;
  int* xi = (int*)(lds_raw + NL * CAP * 32 * 4);

  int b, split;  // one row tile per sequence: the tile is the sequence
  if (!unit_of(p, blockIdx.x, false, b, split)) return;
  const int64_t qo = first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b);
  const int Lmax = max(local_block(qo + (p.rows_per_b - 1) / p.G), 0);
  const int c_begin = split * p.chunk;
  const int c_end = min(c_begin + p.chunk, Lmax);
  if (c_begin >= c_end && p.nsplit > 1) return;  // a single split still writes rows with L = 0

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const bool rvalid = l32 < p.rows_per_b;
  const int nc = rvalid ? l32 : p.rows_per_b - 1;  // invalid rows read a valid row
  const int rowL = local_block(qo + nc / p.G);
  frag qf[NKS];
  {
    const T* qrow = (const T*)p.q_idx + ((int64_t)b * p.rows_per_b + nc) * DI;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const frag*)(qrow + koff(ks, h));
  }
  float ls[CAP];
  int li[CAP];
#pragma unroll
  for (int j = 0; j < CAP; ++j) {
    ls[j] = kNegInf;
    li[j] = -1;
  }

  // this wave's blocks: c_begin + wave + 4 j for j < nbw, read as 4 nbw tiles of 32 keys
  const int nbw = c_end - c_begin > wave ? (c_end - c_begin - wave + 3) / 4 : 0;
  const int ntl = 4 * nbw;
  const S* kpool = (const S*)p.k_idx;
  // Paged caches: lane j holds the page id of the wave's block j, read before
  // the block loop so that no tile load waits on a page-table read (blocks past
  // the 64th of a wave, in caches beyond 4M tokens, read the table directly).
  const bool paged = p.cm.pages != nullptr;
  const int pg_lane = paged && lane < nbw ? p.cm.pages[(int64_t)b * p.cm.max_pages + c_begin + wave + 4 * lane] : 0;
  // element offset of the wave's block j, or -1 when its page is unmapped
  // `far` (a compile-time flag): the wave has more than 64 blocks, and those past
  // the 64th read the page table directly.  The block loop is built once with and
  // once without that read: a load whose result the next tile's address needs
  // makes the compiler wait for every load in flight, the prefetch included.
  auto blk_off = [&](int j, auto far) -> int64_t {
    const int c = c_begin + wave + 4 * j;
    if (!paged) return ((int64_t)b * p.S_k + (int64_t)c * kBlock) * DI;
    int pg;
    if constexpr (decltype(far)::value)
      pg = j < 64 ? __builtin_amdgcn_readlane(pg_lane, j) : p.cm.pages[(int64_t)b * p.cm.max_pages + c];
    else
      pg = __builtin_amdgcn_readlane(pg_lane, j);  // j < nbw <= 64
    return pg >= 0 && pg < p.cm.num_pages ? (int64_t)pg * kBlock * DI : -1;
  };
  // tile tl of the wave; tl past the end re-reads the last one (just read, so from
  // L2); an unmapped page is read from the pool start and scored -inf
  auto load_tile = [&](i32x4 (&a)[NKR], int tl, auto far) {
    const int tc = min(tl, ntl - 1);
    const int64_t o = blk_off(tc / 4, far);
    const char* src = (const char*)(kpool + (o < 0 ? 0 : o) + (tc % 4) * 32 * DI) + lane * 16;
#pragma unroll
    for (int u = 0; u < NKR; ++u) a[u] = __builtin_nontemporal_load((const i32x4*)(src + u * 1024));
  };
  char* wtile = lds_raw + wave * 32 * RB;
  // this lane's max over its 16 keys of the tile
  auto tile_max = [&](const i32x4 (&ld)[NKR]) {
#pragma unroll
    for (int u = 0; u < NKR; ++u) {  // linear chunk 64 u + lane: row (64 u + lane) / CPR
      const int r = (64 * u + lane) / CPR, c = (64 * u + lane) % CPR;
      *(i32x4*)(wtile + (r * CPR + (c ^ sw(r))) * 16) = ld[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    kraw a[NKR];
#pragma unroll
    for (int u = 0; u < NKR; ++u) a[u] = *(const kraw*)(wtile + (l32 * CPR + ((2 * u + h) ^ sw(l32))) * 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x16 acc = f32x16{};
#pragma unroll
    for (int u = 0; u < NKR; ++u) {
      if constexpr (kNative) {
        acc = M::mma(a[u], qf[u], acc);
      } else {
        const uint2 w0 = e4m3x4_to_bf16((uint32_t)a[u][0]), w1 = e4m3x4_to_bf16((uint32_t)a[u][1]);
        const uint2 w2 = e4m3x4_to_bf16((uint32_t)a[u][2]), w3 = e4m3x4_to_bf16((uint32_t)a[u][3]);
        acc = M::mma(__builtin_bit_cast(frag, i32x4{(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y}), qf[2 * u], acc);
        acc = M::mma(__builtin_bit_cast(frag, i32x4{(int)w2.x, (int)w2.y, (int)w3.x, (int)w3.y}), qf[2 * u + 1], acc);
      }
    }
    float m = acc[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) m = fmaxf(m, acc[j]);
    return m;
  };

  float pm = kNegInf, pmA = kNegInf;
  auto process = [&](const i32x4 (&a)[NKR], int tl, auto far) {
    pm = fmaxf(pm, tile_max(a));
    if (tl % 4 != 3) return;  // the block continues in the next tile
    const int j = tl / 4;
    float full = xor_max<32>(pm);
    pm = kNegInf;
    if (blk_off(j, far) < 0) full = kNegInf;
    // blocks pair up: half 0 ranks the wave's even blocks, half 1 the odd ones
    const bool second = (j & 1) != 0;
    if (!second) pmA = full;
    if (second || j + 1 == nbw) {
      const int c = c_begin + wave + 4 * j;
      const float mine = h ? (second ? full : kNegInf) : pmA;
      const int cc = (h || !second) ? c : c - 4;
      const float x = (rvalid && cc < rowL) ? mine : kNegInf;
      list_insert<CAP>(ls, li, x, cc);
    }
  };
  // ntl is a multiple of 4.  Native tiles: one in flight ahead of the one
  // processed; e4m3 tiles, half the bytes, three (the same bytes in flight).
  auto scan = [&](auto far) {
    if constexpr (kNative) {
      i32x4 ta[NKR], tb[NKR];
      load_tile(ta, 0, far);
      for (int tl = 0; tl < ntl; tl += 2) {
        load_tile(tb, tl + 1, far);
        __builtin_amdgcn_sched_barrier(0);
        process(ta, tl, far);
        load_tile(ta, tl + 2, far);
        __builtin_amdgcn_sched_barrier(0);
        process(tb, tl + 1, far);
      }
    } else {
      i32x4 ta[NKR], tb[NKR], tc[NKR], td[NKR];
      load_tile(ta, 0, far);
      load_tile(tb, 1, far);
      load_tile(tc, 2, far);
      for (int tl = 0; tl < ntl; tl += 4) {
        load_tile(td, tl + 3, far);
        __builtin_amdgcn_sched_barrier(0);
        process(ta, tl, far);
        load_tile(ta, tl + 4, far);
        __builtin_amdgcn_sched_barrier(0);
        process(tb, tl + 1, far);
        load_tile(tb, tl + 5, far);
        __builtin_amdgcn_sched_barrier(0);
        process(tc, tl + 2, far);
        load_tile(tc, tl + 6, far);
        __builtin_amdgcn_sched_barrier(0);
        process(td, tl + 3, far);
      }
    }
  };
  if (nbw > 0) {
    if (paged && nbw > 64) scan(std::true_type{});
    else scan(std::false_type{});
  }

  if constexpr (kWide) {  // list split * 8 + wave * 2 + h of the row
    if (rvalid) emit_half_list<CAP>(p, (int64_t)b * p.rows_per_b + l32, split * NL + wave * 2 + h, ls, li);
    return;
  }
  // merge the 8 lists of each row through LDS: [list][CAP][32 rows]
  __syncthreads();  // every wave is done with its key tile (the same LDS)
#pragma unroll
  for (int j = 0; j < CAP; ++j) {
    const int o = ((wave * 2 + h) * CAP + j) * 32 + l32;
    xs[o] = ls[j];
    xi[o] = li[j];
  }
  __syncthreads();
  if (wave == 0 && h == 0 && rvalid) {
    int pos[NL];
#pragma unroll
    for (int w = 0; w < NL; ++w) pos[w] = 0;
    float ms[CAP];
    int mi[CAP];
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
      float bs = kNegInf;
      int bi = -1, bw = -1;
#pragma unroll
      for (int w = 0; w < NL; ++w) {
        const int o = (w * CAP + min(pos[w], CAP - 1)) * 32 + l32;
        const float s2 = xs[o];
        const int i2 = pos[w] < CAP ? xi[o] : -1;
        // empty entries (id -1) rank last; block ids are unique across the lists
        if (i2 >= 0 && (bi < 0 || ranks_before(s2, i2, bs, bi))) {
          bs = s2;
          bi = i2;
          bw = w;
        }
      }
      ms[j] = bs;
      mi[j] = bi;
#pragma unroll
      for (int w = 0; w < NL; ++w) pos[w] += (w == bw) ? 1 : 0;
    }
    if constexpr (!kWide) emit_row<CAP>(p, b, l32, split, rowL, ms, mi);
  }
}

// One wave per (b, i, g) row: the row's lists (lps per key split, each sorted
// by score desc then block asc; at most kMergeMaxLists) are loaded into LDS,
// then k-1 rounds of a wave-wide argmax over the list heads pick the
// Top-(k-1); the local block is added, ids are sorted ascending and padded
// with -1.  WPB waves (rows) per workgroup.
template <int CAP, int WPB>
__global__ __launch_bounds__(64 * WPB) void topk_merge_kernel(IndexParams p) {
  // dynamic LDS: [WPB waves][nsplit * lps * CAP] scores, then the same for block ids
  extern __shared__ __align__(16) char msmem[];
  const int per_wave = p.nsplit * p.lps * CAP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * WPB + wave;
  if (row >= (int64_t)p.B * p.rows_per_b) return;
  const int b = (int)(row / p.rows_per_b);
  const int n = (int)(row - (int64_t)b * p.rows_per_b);
  const int i = n / p.G, g = n - (n / p.G) * p.G;
  const int L = local_block(first_pos(p.cm, p.q_offset, p.S_q, p.S_k, b) + i);
  int32_t* out = p.sel + (((int64_t)b * p.G + g) * p.S_q + i) * p.topk;
  if (L < 0) {  // a row before the start of its cache selects nothing
    if (lane < p.topk) out[lane] = -1;
    return;
  }
  const int nl = L > 0 ? (L + p.chunk - 1) / p.chunk * p.lps : 0;  // lists of the splits before L
  const int take = min(p.topk - 1, L);

  const float* gs = p.part_s + row * per_wave;
  const int32_t* gi = p.part_i + row * per_wave;
  float* ss = (float*)msmem + wave * per_wave;
  int* si = (int*)msmem + WPB * per_wave + wave * per_wave;
  const MergedSlot m = merge_row_lists(gs, gi, nl, CAP, take, L, ss, si, lane);
  if (m.pos >= 0) out[m.pos] = m.id;
  else if (lane < p.topk) out[lane] = -1;
}

constexpr int kMaxIndexDevices = 64;  // devices whose resident workgroup counts are kept

template <typename T, typename S, int DI, int CAP>
static hipError_t launch_index_t(const IndexParams& p, hipStream_t s, const KernelTimer* tm) {
  timer_start(tm, kKernIndexScore, s);
  if (p.units) hipLaunchKernelGGL(index_units_kernel, dim3(1), dim3(1024), 0, s, p);
  constexpr int RT = index_row_tiles(CAP + 1);
  constexpr int NT = 64 * index_waves(CAP + 1, sizeof(T) == 2);
  static_assert(NT / 2 * RT == index_rows_per_wg(CAP + 1, sizeof(T) == 2), "host and kernel agree on the row tile");
  static_assert(index_cap(CAP + 1) == CAP, "host and kernel agree on the list length");
  bool small_done = false;
  if constexpr (sizeof(T) == 2) {  // the few-row form is built for bf16 queries
    if (p.small) {
      hipLaunchKernelGGL((index_topk_small_kernel<T, S, DI, CAP>), dim3(p.grid_per_xcd * 8), dim3(256), 0, s, p);
      small_done = true;
    }
  }
  if (!small_done) {
    // the persistent grid: the workgroups resident at once, counted once per device
    static std::atomic<int> resident[kMaxIndexDevices];
    IndexParams pl = p;
    unsigned grid = (unsigned)p.grid_per_xcd * 8;
    if (p.persist) {
      int dev = -1;
      pl.persist = 0;
      if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxIndexDevices) {
        int r = resident[dev].load(std::memory_order_relaxed);
        if (r == 0) {
          int cus = 0, per_cu = 0;
          if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
              hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, index_topk_kernel<T, S, DI, CAP, RT>, NT, 0) ==
                  hipSuccess)
            r = cus * per_cu;
          (void)hipGetLastError();  // a failed query leaves the one-unit grid and no error behind
          if (r > 0) resident[dev].store(r, std::memory_order_relaxed);
        }
        if (r > 0 && r < p.nunits) {
          pl.persist = 1;
          grid = (unsigned)r;
        }
      }
    }
    hipLaunchKernelGGL((index_topk_kernel<T, S, DI, CAP, RT>), dim3(grid), dim3(NT), 0, s, pl);
  }
  timer_stop(tm, kKernIndexScore, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.nsplit == 1 && CAP != kIndexWideCap) return hipGetLastError();  // the index kernel wrote the selection
  if (p.merge_in_consumer) return hipGetLastError();  // the decode rows kernel merges the lists
  const int64_t rows = (int64_t)p.B * p.rows_per_b;
  timer_start(tm, kKernTopkMerge, s);
  constexpr int WPB = merge_rows_per_wg(CAP);  // the host keeps nsplit * lps <= merge_max_lists(CAP)
  const size_t lds = (size_t)2 * WPB * p.nsplit * p.lps * CAP * 4;
  hipLaunchKernelGGL((topk_merge_kernel<CAP, WPB>), dim3((unsigned)((rows + WPB - 1) / WPB)), dim3(64 * WPB), lds, s,
                     p);
  timer_stop(tm, kKernTopkMerge, s);
  return hipGetLastError();
}

template <typename T, typename S, int DI>
static hipError_t launch_index_d(const IndexParams& p, hipStream_t s, const KernelTimer* tm) {
  if (p.topk <= 16) return launch_index_t<T, S, DI, 15>(p, s, tm);
  if (p.topk <= 32) return launch_index_t<T, S, DI, 31>(p, s, tm);
  return launch_index_t<T, S, DI, kIndexWideCap>(p, s, tm);
}

template <typename T, typename S>
static hipError_t launch_index_s(const IndexParams& p, int index_dim, hipStream_t s, const KernelTimer* tm) {
  switch (index_dim) {
    case 32: return launch_index_d<T, S, 32>(p, s, tm);
    case 64: return launch_index_d<T, S, 64>(p, s, tm);
    case 128: return launch_index_d<T, S, 128>(p, s, tm);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_index_select(const IndexParams& p, bool bf16_inputs, bool fp8_keys, int index_dim, hipStream_t s,
                               const KernelTimer* tm) {
  if (fp8_keys) return bf16_inputs ? launch_index_s<bf16, e4m3>(p, index_dim, s, tm) : hipErrorInvalidValue;
  if (bf16_inputs) return launch_index_s<bf16, bf16>(p, index_dim, s, tm);
  return launch_index_s<float, float>(p, index_dim, s, tm);
}

}  // namespace msa

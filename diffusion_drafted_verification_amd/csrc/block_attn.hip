// Block attention of one Orthrus decode step on gfx950.
//
// What is computed (Orthrus explainer, gist.science arXiv 2605.12825,
// technical summary §2.1-§2.3): K block rows of every query head attend to the
// L cached AR keys/values of their KV head (always visible) and to the K block
// keys, bidirectionally in the diffusion view (M_diff, §2.2 rule 2) or
// causally in the AR verify view (§2.3).
//
// How (MI355X-first; the flash-attention dependency the pages name is prior
// art for other hardware, not the blueprint):
//   * one work-group per (sequence b, KV head g, context split s) with 2G
//     waves: the G query heads sharing KV head g times the two 32-position
//     halves of each 64-position stage, so each KV byte is read from HBM once
//     and feeds a (G x 32)-row tile;
//   * bf16 with G <= 4 (attn_stream): context stages go HBM -> LDS by LDS-DMA
//     (no staging registers) through a ring of kRing stages; K and V both stay
//     token-major with XOR chunk swizzles, V is read back transposed by
//     ds_read_b64_tr_b16.  fp32 and G = 8 (attn_main): a register-staged
//     double buffer, V transposed when it is written to LDS;
//   * S^T = K Q^T and O^T = V^T P^T on MFMA 32x32 tiles with fp32
//     accumulation: the score tile's accumulator layout is directly the B
//     operand of the PV product (no shuffles), and every lane owns one query
//     row, so row rescales are per-lane multiplies;
//   * online softmax in the log2 domain with a lazy (threshold) rescale;
//     only the row max needs one cross-lane exchange per 32 keys;
//   * the block tile and the ragged context tail are the only masked tiles;
//     the mask mode is a template parameter;
//   * when a sequence is split over several work-groups each writes a
//     partial (bf16 O / l on the streaming path, fp32 O otherwise, plus the
//     row's max and sum) and a combine kernel merges them; the work-group
//     order puts all splits of one (b, g) on one XCD so the partials stay in
//     that XCD's L2;
//   * the split length is fixed by the host from max_ctx_len, or, for a
//     ragged batch that asks for it, chosen on the device from ctx_lens so
//     that one round of about 256 work-groups covers the batch evenly, or
//     two rounds of shorter ones where one round would be poorly balanced (a
//     separate instantiation of the streaming kernel and its combine);
//   * a prompt prefill runs its 32-row chunks as virtual sequences of this
//     layout; attn_prefill_pair serves two consecutive chunks per work-group
//     so that each streamed key feeds twice the query rows.
#include <type_traits>

#include "orthrus_device.h"
#include "orthrus_host.h"

namespace orthrus {

constexpr int kTile = 64;          // context positions per LDS stage
constexpr int kMaxSplit = 8192;    // positions per work-group (sizes the page-id table)
constexpr int kRows = 32;          // block rows per wave (one query head)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;  // rescale O only when the max grows by > 2^8

struct AttnArgs {
  const char* q;
  const char* k_cache;
  const char* v_cache;
  const char* k_blk;
  const char* v_blk;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  char* out;
  // split partials for attn_combine, one slot per (b, h, split, row):
  float* ws_o;      // [B, Hq, s_max, 32, D]  register-staged kernel: unnormalised O (fp32)
  bf16* ws_p;       // [B, Hq, s_max, 32, D]  streaming kernel: normalised O / l (bf16)
  float2* ws_ml;    // [B, Hq, s_max, 32]     (running max in log2 units, row sum)
  int B, K, Hq, Hkv, max_pages, num_pages, max_ctx, split, s_max;
  float c;          // softmax scale * log2(e)
  int kv_once;      // the call reads each context K/V byte once: nontemporal stream
  // balanced split (streaming path): the split length is chosen per call from
  // ctx_lens so that one round of Q work-groups per KV head covers the batch;
  // the partial of unit (b, s) sits in slot P_b + s of its KV head's U slots;
  // Q2 > Q allows a second round of units (Q2 per KV head) when one round
  // leaves the batch poorly balanced
  int bal, Q, U, Q2;
  int2* ws_rec;     // balanced split: (splits, first slot) per sequence, for attn_combine
  int s_hint;       // split count that sizes the combine's lane groups (a
                    // batch with every length at max_ctx has this many)
};

constexpr int kBalMinTiles = 320 / kTile;        // shortest automatic or balanced split: 320 positions
constexpr int kBalMaxTiles = kMaxSplit / kTile;  // longest: kMaxSplit
constexpr float kBalRoundEff = 0.85f;            // balanced split: below this average / longest unit
                                                 // in one round, use two

// Inclusive prefix sum over the 64 lanes of a wave on the DPP paths (no LDS
// round trip): shifts by 1, 2, 4, 8 within each 16-lane row, then the row
// totals through the broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ __forceinline__ int wave_total(int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), kWave - 1); }

// ceil(T / t) for 0 <= T < 2^18 and 4 <= t <= 128 with rt ~ 1 / t (within a
// few ulp): the float estimate is floor(T / t) or one less, and two exact
// integer tests raise it to the ceiling.
__device__ __forceinline__ int ceil_div_small(int T, int t, float rt) {
  int q = (int)((float)T * rt);
  q += q * t < T;
  q += q * t < T;
  return q;
}

// Splits of a sequence of T 64-position tiles at t tiles per split (an empty
// context still makes one unit: the block keys).
__device__ __forceinline__ int bal_splits(int T, int t, float rt) { return T > 0 ? ceil_div_small(T, t, rt) : 1; }

// The balanced split of one call, computed identically by every wave that
// needs it (lane l holds sequence B - 1 - l, so B <= 64): the smallest t in
// [kBalMinTiles, kBalMaxTiles] with sum_b ceil(T_b / t) <= Q, or kBalMaxTiles
// when none is.  t_guess (the split of a batch with every length at max_ctx)
// is tested first: with equal lengths it is the answer.  Returns t; n and P
// are this lane's split count and the exclusive prefix of the counts.
struct BalSplit {
  int t, n, P, L;
};

__device__ BalSplit balanced_split(const AttnArgs& a, int lane, int t_guess) {
  const bool act = lane < a.B;
  int L = act ? a.ctx_lens[a.B - 1 - lane] : 0;
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int T = (L + kTile - 1) / kTile;
  auto count = [&](int t) { return wave_total(act ? bal_splits(T, t, __builtin_amdgcn_rcpf((float)t)) : 0); };
  // Every length is at most max_ctx, so count(t_guess) <= Q unless t_guess
  // is kBalMaxTiles, and the answer is at most t_guess.
  int lo = kBalMinTiles, hi = t_guess;
  if (hi == kBalMaxTiles && count(hi) > a.Q) {
    lo = hi;
  } else {
    if (hi > lo) {
      if (count(hi - 1) > a.Q) lo = hi;
      else --hi;
    }
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (count(mid) <= a.Q) hi = mid;
      else lo = mid + 1;
    }
  }
  // One round (at most Q units per KV head) is poorly balanced when its
  // average unit is below kBalRoundEff of the longest, t: then up to Q2
  // shorter units (two rounds), numbered longest first within each sequence
  // and dispatched as work-groups free up, shorten the critical path (an
  // equal-length batch stays at one round: its average is t)
  if (a.Q2 > a.Q && lo > kBalMinTiles) {
    const int tiles = wave_total(act ? (T > 0 ? T : 1) : 0);
    if ((float)tiles < kBalRoundEff * (float)a.Q * (float)lo) {
      int lo2 = kBalMinTiles, hi2 = lo;
      while (lo2 < hi2) {
        const int mid = (lo2 + hi2) >> 1;
        if (count(mid) <= a.Q2) hi2 = mid;
        else lo2 = mid + 1;
      }
      lo = lo2;
    }
  }
  BalSplit r;
  r.t = lo;
  r.n = act ? bal_splits(T, lo, __builtin_amdgcn_rcpf((float)lo)) : 0;
  r.P = wave_incl_scan(r.n) - r.n;
  r.L = L;
  return r;
}

// Unit j of one KV head under the balanced split.  Units are numbered split
// index first, then sequence (B - 1 down to 0): with equal lengths this is
// the fixed split's work-group order.
struct BalUnit {
  int b, s, n, L, split, slot;
  bool live;
};

__device__ BalUnit balanced_unit(const AttnArgs& a, int j, int lane) {
  const BalSplit q = balanced_split(a, lane, a.split / kTile);
  BalUnit u;
  u.live = false;
  int C = 0, s = 0;
  uint64_t mask = 0;
  for (;;) {
    mask = __ballot(q.n > s);
    const int c = __popcll(mask);
    if (c == 0) return u;  // j is past the last unit
    if (j < C + c) break;
    C += c;
    ++s;
  }
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  const uint64_t sel = __ballot(q.n > s && rank == j - C);
  const int ls = __ffsll((unsigned long long)sel) - 1;
  u.b = a.B - 1 - ls;
  u.s = s;
  u.n = __builtin_amdgcn_readlane(q.n, ls);
  u.L = __builtin_amdgcn_readlane(q.L, ls);
  u.slot = __builtin_amdgcn_readlane(q.P, ls) + s;
  u.split = q.t * kTile;
  // a unit outside the batch or its partial slots would be an arithmetic
  // slip: drop it rather than write out of range
  u.live = ls >= 0 && ls < a.B && u.slot < a.U && u.s < u.n;
  return u;
}

__device__ __forceinline__ int swap_bits23(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

template <typename T, int D>
struct AttnLayout {
  static constexpr int ESZ = sizeof(T);
  static constexpr int KROW = D * ESZ;            // bytes of one K row
  static constexpr int KCH = KROW / 16;           // 16-byte chunks per K row
  static constexpr int KSW = (KCH < 16 ? KCH : 16) - 1;
  static constexpr int VROW = kTile * ESZ;        // bytes of one V^T row (64 tokens)
  static constexpr int VCH = VROW / 16;
  static constexpr int KBYTES = kTile * KROW;
  static constexpr int STAGE = KBYTES + D * VROW;
  static constexpr int UNITS = (kTile / 4) * KCH;  // (token quad, chunk) load units per stage
  static constexpr int EPC = 16 / ESZ;            // elements per 16-byte chunk
  static constexpr int VCHUNKS = Vec8<T>::bytes / 16;  // chunks per 8-element operand

  __device__ static int kslot(int row, int chunk) { return row * KROW + ((chunk ^ (row & KSW)) << 4); }
  __device__ static int vswz(int d) { return ((d >> 3) ^ d) & (VCH - 1); }
  __device__ static int vslot(int d, int chunk) { return d * VROW + ((chunk ^ vswz(d)) << 4); }
};

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type lds_vec8(const char* base, int off0, int off1) {
  typedef typename Vec8<T>::type V;
  if constexpr (sizeof(T) == 2) {
    u32x4 x = ld16(base + off0);
    return __builtin_bit_cast(V, x);
  } else {
    u32x4 x0 = ld16(base + off0), x1 = ld16(base + off1);
    struct P { u32x4 a, b; } pr{x0, x1};
    return __builtin_bit_cast(V, pr);
  }
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type pack_p(const f32x16& s, int j) {
  typename Vec8<T>::type r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)s[8 * j + e];
  return r;
}

// Global -> register staging of one 64-position stage.  Half of the
// work-group's waves stage K, the other half V.  Unit u covers four
// consecutive positions (one token quad, never crossing a page) and one
// 16-byte chunk of the head dimension.
template <typename T, int D, int NT>
struct Stage {
  typedef AttnLayout<T, D> Lay;
  static constexpr int LT = NT / 2;                          // loader threads per tensor
  static constexpr int UPT = (Lay::UNITS + LT - 1) / LT;     // units per loader thread
  u32x4 r[UPT][4];
  uint32_t valid;  // bit 4j+t: r[j][t] holds data (else it is stored as zeros)

  // Issue the loads of one stage without consuming them: every load reads a
  // valid address (the block K/V base stands in for unused positions) and the
  // zeroing of unused positions waits until store time, so the loads of
  // several stages stay in flight together.  cache / blk: the tensor this
  // thread stages (K or V).
  // Positions at or past p_end (the split's end, <= N) are never read: the
  // page-id table only covers the split.
  __device__ void load(const char* cache, const char* blk, const AttnArgs& a, const int* pages, int page_base,
                       int b, int g, int L, int p_end, int p0, int ltid) {
    valid = 0;
    // a stage entirely inside the cached context (the common case): one page
    // id per thread and four loads at fixed offsets from one address
    const bool all_cached = p0 + kTile <= L && p0 + kTile <= p_end;
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = ltid + j * LT;
      if (Lay::UNITS % LT != 0 && u >= Lay::UNITS) break;
      const int tq = u / Lay::KCH, c = u % Lay::KCH;
      const int pos0 = p0 + 4 * tq;  // four positions of one page
      const int pidx = (pos0 >> 4) - page_base;  // padded stages run past the split: clamp
      const int page = pages[pidx < kMaxSplit / kPage ? pidx : kMaxSplit / kPage - 1];
      const size_t coff =
          ((size_t)((page > 0 ? page : 0) * a.Hkv + g) * kPage + (pos0 & 15)) * Lay::KROW + c * 16;
      if (all_cached) {
        const bool ok = page >= 0;
        const char* src = ok ? cache + coff : blk;
#pragma unroll
        for (int t = 0; t < 4; ++t) r[j][t] = ld16(src + (ok ? t * Lay::KROW : 0));
        valid |= (ok ? 15u : 0u) << (4 * j);
        continue;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pos = pos0 + t;
        const bool in_cache = pos < L && pos < p_end && page >= 0;
        const bool in_blk = pos >= L && pos < p_end;
        const size_t boff = ((size_t)(b * a.K + (in_blk ? pos - L : 0)) * a.Hkv + g) * Lay::KROW + c * 16;
        const char* src = in_cache ? cache + coff + t * Lay::KROW : blk + boff;
        r[j][t] = ld16(src);
        valid |= (uint32_t)(in_cache || in_blk) << (4 * j + t);
      }
    }
  }

  __device__ u32x4 get(int j, int t) const {
    return ((valid >> (4 * j + t)) & 1) ? r[j][t] : u32x4{0, 0, 0, 0};
  }

  // K rows go to LDS row swap_bits23(token) (so the score accumulator holds
  // eight consecutive tokens per lane half), XOR-swizzled by 16-byte chunk.
  __device__ void store_k(char* ks, int ltid) const {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = ltid + j * LT;
      if (Lay::UNITS % LT != 0 && u >= Lay::UNITS) break;
      const int tq = u / Lay::KCH, c = u % Lay::KCH;
#pragma unroll
      for (int t = 0; t < 4; ++t) st16(ks + Lay::kslot(swap_bits23(4 * tq + t), c), get(j, t));
    }
  }

  // V is written transposed: row d holds the 64 positions of element d.
  __device__ void store_v(char* vs, int ltid) const {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = ltid + j * LT;
      if (Lay::UNITS % LT != 0 && u >= Lay::UNITS) break;
      const int tq = u / Lay::KCH, c = u % Lay::KCH;
      const u32x4 x0 = get(j, 0), x1 = get(j, 1), x2 = get(j, 2), x3 = get(j, 3);
      if constexpr (sizeof(T) == 2) {
        // element e of the chunk is d = c*8 + e; four positions -> 8 bytes of row d
        const int tch = tq >> 1, half = (tq & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x2 pk;
          if (e & 1) {
            pk[0] = (x0[w] >> 16) | (x1[w] & 0xffff0000u);
            pk[1] = (x2[w] >> 16) | (x3[w] & 0xffff0000u);
          } else {
            pk[0] = (x0[w] & 0xffffu) | (x1[w] << 16);
            pk[1] = (x2[w] & 0xffffu) | (x3[w] << 16);
          }
          *reinterpret_cast<u32x2*>(vs + Lay::vslot(c * 8 + e, tch) + half) = pk;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) st16(vs + Lay::vslot(c * 4 + e, tq), u32x4{x0[e], x1[e], x2[e], x3[e]});
      }
    }
  }
};

// One work-group per (sequence b, KV head g, context split s); 2G waves:
// wave w serves query head g*G + w%G on the 32-position half w/G of every
// 64-position stage.  The two halves of a head keep separate softmax states
// and are merged through LDS at the end.
template <typename T, int D, int G, int MODE>
__global__ void __launch_bounds__(2 * kWave * G) attn_main(AttnArgs a) {
  typedef AttnLayout<T, D> Lay;
  typedef typename Vec8<T>::type V8;
  constexpr int NT = 2 * kWave * G;
  constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int MB = D / 32;   // 32-wide blocks of the head dimension in O^T
  typedef Stage<T, D, NT> St;
  // stages kept in flight in registers (about 64 staging registers at most)
  constexpr int PD = (St::UPT * 16 <= 16) ? 3 : ((St::UPT * 16 <= 32) ? 2 : 1);
  constexpr int MERGE = G * (MB * 16 + 2) * kWave * 4;
  constexpr int SMEM = (2 * Lay::STAGE > MERGE) ? 2 * Lay::STAGE : MERGE;

  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int pages[kMaxSplit / kPage];

  const int BH = a.B * a.Hkv;
  const int bg = blockIdx.x % BH;
  const int s = blockIdx.x / BH;
  // sequences in reverse order: where later sequences carry longer contexts
  // (the chunks of a prompt prefill) the longest work-groups start first
  const int b = a.B - 1 - bg / a.Hkv, g = bg % a.Hkv;
  const int tid = threadIdx.x;
  const int p_begin = s * a.split;
  const int page_base = p_begin >> 4;
  // page ids of this split (loaded before the context length is known, so
  // the two loads overlap); ids outside [0, num_pages) become -1
  int pg[(kMaxSplit / kPage + NT - 1) / NT];
#pragma unroll
  for (int k = 0; k < (kMaxSplit / kPage + NT - 1) / NT; ++k) {
    const int x = tid + k * NT, lp = page_base + x;
    pg[k] = (x < a.split / kPage && lp < a.max_pages) ? a.page_table[(size_t)b * a.max_pages + lp] : -1;
  }
  int L = a.ctx_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int N = L + a.K;
  // splits partition the cached context; the last one also takes the K block keys
  const int S_b = L > 0 ? (L + a.split - 1) / a.split : 1;
  if (s >= S_b) return;
  const int p_end = s == S_b - 1 ? N : p_begin + a.split;
  const int ntiles = (p_end - p_begin + kTile - 1) / kTile;
  const int wave = tid / kWave, lane = tid % kWave;
  const int i = lane & 31, hi = lane >> 5;
  const int hw = wave % G, sub = wave / G;
  const int h = g * G + hw;
  // loader role: the first half of the threads stages V, the second K
  const bool v_loader = tid < NT / 2;
  const int ltid = v_loader ? tid : tid - NT / 2;
  const char* src_cache = v_loader ? a.v_cache : a.k_cache;
  const char* src_blk = v_loader ? a.v_blk : a.k_blk;

#pragma unroll
  for (int k = 0; k < (kMaxSplit / kPage + NT - 1) / NT; ++k) {
    const int x = tid + k * NT;
    if (x < kMaxSplit / kPage) pages[x] = (pg[k] >= 0 && pg[k] < a.num_pages) ? pg[k] : -1;
  }

  // this wave's query rows as the B operand of S^T = K Q^T (one 16-wide k-step each)
  V8 qf[KS];
  {
    const char* qrow = a.q + ((size_t)(b * a.K + (i < a.K ? i : 0)) * a.Hq + h) * D * sizeof(T);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = (16 * ks + 8 * hi) * sizeof(T);
      if constexpr (sizeof(T) == 2) {
        qf[ks] = __builtin_bit_cast(V8, ld16(qrow + off));
      } else {
        struct P { u32x4 x, y; } pr{ld16(qrow + off), ld16(qrow + off + 16)};
        qf[ks] = __builtin_bit_cast(V8, pr);
      }
      if (i >= a.K) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (T)0.f;
      }
    }
  }
  __syncthreads();  // page ids visible

  f32x16 o[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[m][r] = 0.f;
  float m_c = -INFINITY;  // running max of this lane's row, log2 units
  float l = 0.f;          // this lane's share of the row sum
  const float c = a.c;

  // Register ring of PD stages.  The stage count is padded to a multiple of
  // PD and every load is issued unconditionally (stages past the split read
  // valid addresses and are masked), so the ring body is straight-line code
  // and the compiler's wait counts keep PD stages in flight.
  St st[PD];
#pragma unroll
  for (int p = 0; p < PD; ++p)
    st[p].load(src_cache, src_blk, a, pages, page_base, b, g, L, p_end, p_begin + p * kTile, ltid);

  const int nt_pad = ((ntiles + PD - 1) / PD) * PD;
  for (int t0 = 0; t0 < nt_pad; t0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int t = t0 + p;
      char* buf = smem + (t & 1) * Lay::STAGE;
      if (v_loader) st[p].store_v(buf + Lay::KBYTES, ltid);
      else st[p].store_k(buf, ltid);
      __syncthreads();
      st[p].load(src_cache, src_blk, a, pages, page_base, b, g, L, p_end, p_begin + (t + PD) * kTile, ltid);

      const int pbase = p_begin + t * kTile + 32 * sub;
      if (pbase < p_end) {
        const char* ks_lds = buf;
        const char* vs_lds = buf + Lay::KBYTES;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int row = 32 * sub + i;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int e0 = (16 * ks + 8 * hi) * sizeof(T) / 16;  // first chunk of the operand
          const V8 av = lds_vec8<T>(ks_lds, Lay::kslot(row, e0), Lay::kslot(row, e0 + 1));
          acc = mfma_step(av, qf[ks], acc);
        }
        // acc[r] is the score of position pbase + 16*(r/8) + 8*hi + r%8 for row i
        if (pbase + 32 > L) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pos = pbase + 16 * (r >> 3) + 8 * hi + (r & 7);
            bool vis;
            if (MODE == ORTHRUS_DIFF_BIDIR) vis = pos < N;
            else vis = pos < L || (pos < N && pos - L <= i);
            if (!vis) acc[r] = -INFINITY;
          }
        }
        float mx = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
        mx = wave_max_xor32(mx);
        const bool need = mx * c > m_c + kRescaleLog2;
        if (__any(need)) {
          const float new_mc = need ? mx * c : m_c;
          const float sc = (new_mc == m_c) ? 1.f : __builtin_amdgcn_exp2f(m_c - new_mc);
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[m][r] *= sc;
          l *= sc;
          m_c = new_mc;
        }
        const float mref = (m_c == -INFINITY) ? 0.f : m_c;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], c, -mref));
          l += acc[r];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const V8 pv = pack_p<T>(acc, j);
          const int e0 = (32 * sub + 16 * j + 8 * hi) * sizeof(T) / 16;
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const int d = 32 * m + i;
            const V8 vv = lds_vec8<T>(vs_lds, Lay::vslot(d, e0), Lay::vslot(d, e0 + 1));
            o[m] = mfma_step(vv, pv, o[m]);
          }
        }
      }
    }
  }

  // merge the two position halves of each head: the second-half wave hands
  // its (max, sum, O) to the first-half wave through LDS
  __syncthreads();  // every wave is done with the stage buffers
  float* mo = reinterpret_cast<float*>(smem) + hw * (MB * 16 + 2) * kWave;
  if (sub == 1) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) mo[(m * 16 + r) * kWave + lane] = o[m][r];
    mo[(MB * 16) * kWave + lane] = m_c;
    mo[(MB * 16 + 1) * kWave + lane] = l;
  }
  __syncthreads();
  if (sub == 1) return;
  {
    const float m1 = mo[(MB * 16) * kWave + lane];
    const float l1 = mo[(MB * 16 + 1) * kWave + lane];
    const float mm = fmaxf(m_c, m1);
    const float w0 = (m_c == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_c - mm);
    const float w1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[m][r] = w0 * o[m][r] + w1 * mo[(m * 16 + r) * kWave + lane];
    l = w0 * l + w1 * l1;
    m_c = mm;
  }

  const float l_row = l + __shfl_xor(l, 32, kWave);
  if (i >= a.K) return;
  // o[m][r] holds d = 32m + 8*(r/4) + 4*hi + r%4 of row i
  if (S_b == 1) {
    const float inv = 1.f / l_row;
    char* orow = a.out + ((size_t)(b * a.K + i) * a.Hq + h) * D * sizeof(T);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * m + 8 * rg + 4 * hi;
        if constexpr (sizeof(T) == 2) {
          bf16x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (bf16)(o[m][4 * rg + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + d0 * 2) = y;
        } else {
          f32x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = o[m][4 * rg + e] * inv;
          *reinterpret_cast<f32x4*>(orow + d0 * 4) = y;
        }
      }
  } else {
    const size_t prow = ((size_t)(b * a.Hq + h) * a.s_max + s) * kRows + i;
    float* po = a.ws_o + prow * D;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * m + 8 * rg + 4 * hi;
        *reinterpret_cast<f32x4*>(po + d0) =
            f32x4{o[m][4 * rg], o[m][4 * rg + 1], o[m][4 * rg + 2], o[m][4 * rg + 3]};
      }
    if (hi == 0) a.ws_ml[prow] = make_float2(m_c, l_row);
  }
}

// Merge the split partials of sequences whose context spans several
// work-groups: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, where
// O_s is stored unnormalised (fp32) or as O_s / l_s (bf16, NORM).
// A row (b, i, h) is served by SG groups of D/4 lanes (4 outputs per lane);
// group q takes splits q, q+SG, ... and issues all of its loads before
// reducing; the groups of a row then merge (shuffles within a wave, LDS
// otherwise).  A work-group covers 256 / (SG D/4) consecutive rows of one
// (b, g); block id = chunk * (B Hkv) + b Hkv + g, so the rows of one (b, g)
// run on the XCD that wrote its partials (when B Hkv % 8 == 0).
template <typename T, int D, int SG, bool NORM>
__global__ void __launch_bounds__(256) attn_combine(AttnArgs a) {
  constexpr int TPR = D / 4;          // lanes per group
  constexpr int LPR = TPR * SG;       // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per work-group
  constexpr int PER = 4;              // splits per group in flight at once
  __shared__ float red_m[256 / kWave];
  __shared__ f32x4 red_o[SG > 2 ? SG : 1][TPR];
  __shared__ float red_l[SG > 2 ? SG : 1];

  const int BH = a.B * a.Hkv, G = a.Hq / a.Hkv;
  const int bg = blockIdx.x % BH, chunk = blockIdx.x / BH;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int tid = threadIdx.x;
  const int rl = chunk * RPB + tid / LPR;         // row within (b, g): w * K + i
  const bool live = rl < G * a.K;
  const int w = rl / a.K, i = rl % a.K;
  const int h = g * G + w;
  int L = a.ctx_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int S_b = L > 0 ? (L + a.split - 1) / a.split : 1;
  if (S_b <= 1) return;                             // uniform over the work-group
  const int x = tid % LPR, sg = x / TPR, d0 = 4 * (x % TPR);
  const size_t base = (size_t)(b * a.Hq + (live ? h : 0)) * a.s_max * kRows + (live ? i : 0);

  float M = -INFINITY;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s0 = sg; s0 < S_b; s0 += SG * PER) {
    float2 ml[PER];
    f32x4 xo[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int s = s0 + k * SG;
      const size_t r = base + (size_t)(s < S_b ? s : 0) * kRows;
      ml[k] = a.ws_ml[r];
      if constexpr (NORM) {  // bf16 O / l: weight by the split's row sum
        const bf16x4 y = *reinterpret_cast<const bf16x4*>(a.ws_p + r * D + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) xo[k][e] = (float)y[e] * ml[k].y;
      } else {
        xo[k] = *reinterpret_cast<const f32x4*>(a.ws_o + r * D + d0);
      }
      if (s >= S_b) ml[k].x = -INFINITY;
    }
    float mnew = M;
#pragma unroll
    for (int k = 0; k < PER; ++k) mnew = fmaxf(mnew, ml[k].x);
    if (mnew != -INFINITY) {
      const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mnew);
      acc *= sc;
      den *= sc;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float w8 = (ml[k].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - mnew);
        acc += w8 * xo[k];
        den += w8 * ml[k].y;
      }
      M = mnew;
    }
  }
  if constexpr (SG == 2) {
    // the two groups of a row are adjacent TPR-lane blocks of one wave
    const float Mo = __shfl_xor(M, TPR, kWave);
    const float Mall = fmaxf(M, Mo);
    const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mall);
    acc *= sc;
    den *= sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], TPR, kWave);
    den += __shfl_xor(den, TPR, kWave);
  } else if constexpr (SG > 2) {
    // one row per work-group: merge the groups through LDS
    float Mw = M;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) Mw = fmaxf(Mw, __shfl_xor(Mw, off, kWave));
    if (tid % kWave == 0) red_m[tid / kWave] = Mw;
    __syncthreads();
    float Mall = red_m[0];
#pragma unroll
    for (int k = 1; k < 256 / kWave; ++k) Mall = fmaxf(Mall, red_m[k]);
    const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mall);
    red_o[sg][x % TPR] = acc * sc;
    if (x % TPR == 0) red_l[sg] = den * sc;
    __syncthreads();
    if (sg != 0) return;
    acc = red_o[0][x];
    den = red_l[0];
#pragma unroll
    for (int q = 1; q < SG; ++q) {
      acc += red_o[q][x];
      den += red_l[q];
    }
  }
  if (!live || sg != 0) return;
  const float inv = 1.f / den;
  char* orow = a.out + ((size_t)(b * a.K + i) * a.Hq + h) * D * sizeof(T);
  if constexpr (sizeof(T) == 2) {
    bf16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x4*>(orow + d0 * 2) = y;
  } else {
    *reinterpret_cast<f32x4*>(orow + d0 * 4) = acc * inv;
  }
}

// Merge of bf16 normalised partials (streaming path).  A row (b, i, h) is
// served by SG lane groups of D/8 lanes; a lane owns 8 consecutive outputs
// and the splits sg, sg + SG, ... (at most SPL of them: every load is issued
// before any is used), and the SG groups of a row (adjacent within one wave)
// merge with xor shuffles: no LDS, no barrier.  A work-group covers 4 waves x
// 64 / (SG D/8) consecutive rows of one (b, g); block id = chunk * (B Hkv) +
// b Hkv + g as for attn_combine.
template <int D, int SG, int SPL, bool BAL>
__global__ void __launch_bounds__(256)
    attn_combine_bf16(const int32_t* pre_ctx, const float2* pre_ml, const char* pre_p, int pre_B, int pre_Hkv,
                      int pre_Hq, int pre_K, int pre_maxctx, int pre_split, int pre_smax, AttnArgs a) {
  // the leading scalar arguments repeat the fields the first loads depend
  // on, preloaded into SGPRs when the wave starts (as for attn_stream)
  constexpr int C = D / 8;               // lanes per row and split group
  constexpr int RPW = kWave / (C * SG);  // rows per wave
  constexpr int RPB = 4 * RPW;           // rows per work-group
  static_assert(RPW >= 1, "a row fits one wave");
  const int BH = pre_B * pre_Hkv, G = pre_Hq / pre_Hkv;
  const int bg = blockIdx.x % BH, chunk = blockIdx.x / BH;
  const int b = bg / pre_Hkv, g = bg % pre_Hkv;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int rl = chunk * RPB + wave * RPW + lane / (C * SG);  // row within (b, g): w * K + i
  const int sg = (lane / C) % SG, c = lane % C;
  const bool live = rl < G * pre_K;
  const int w = live ? rl / pre_K : 0, i = live ? rl % pre_K : 0;
  const int h = g * G + w;
  int S_b;
  size_t base, sstride;  // row of split 0, rows between splits
  if constexpr (BAL) {
    const int2 rec = a.ws_rec[b];  // written by the attention kernel
    S_b = rec.x;
    const int P = rec.y;
    if (P < 0 || P + S_b > a.U) return;  // an arithmetic slip: never read past the slots
    base = ((size_t)(g * a.U + P) * G + w) * kRows + i;
    sstride = (size_t)G * kRows;
  } else {
    int L = pre_ctx[b];
    L = L < 0 ? 0 : (L > pre_maxctx ? pre_maxctx : L);
    S_b = L > 0 ? (L + pre_split - 1) / pre_split : 1;
    base = (size_t)(b * pre_Hq + h) * pre_smax * kRows + i;
    sstride = kRows;
  }
  if (S_b <= 1) return;  // uniform over the work-group

  float M = -INFINITY, den = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = sg; s0 < S_b; s0 += SG * SPL) {
    float2 ml[SPL];
    u32x4 x[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int sp = s0 + SG * j;
      const size_t r = base + (size_t)(sp < S_b ? sp : 0) * sstride;
      ml[j] = pre_ml[r];
      x[j] = *reinterpret_cast<const u32x4*>(pre_p + r * D * 2 + c * 16);
      if (sp >= S_b) ml[j].x = -INFINITY;
    }
    float mnew = M;
#pragma unroll
    for (int j = 0; j < SPL; ++j) mnew = fmaxf(mnew, ml[j].x);
    if (mnew != -INFINITY) {
      const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mnew);
      den *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float wj = (ml[j].x == -INFINITY) ? 0.f : ml[j].y * __builtin_amdgcn_exp2f(ml[j].x - mnew);
        den += wj;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += wj * __uint_as_float(x[j][k] << 16);
          acc[2 * k + 1] += wj * __uint_as_float(x[j][k] & 0xffff0000u);
        }
      }
      M = mnew;
    }
  }
  // merge the SG split groups of the row (lanes c + C q, q < SG)
#pragma unroll
  for (int off = C; off < C * SG; off <<= 1) {
    const float Mo = __shfl_xor(M, off, kWave);
    const float Mall = fmaxf(M, Mo);
    const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mall);
    den *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
    den += __shfl_xor(den, off, kWave);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
    M = Mall;
  }
  if (!live || sg != 0) return;
  const float inv = 1.f / den;
  u32x4 y;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16 lo = (bf16)(acc[2 * k] * inv), hi2 = (bf16)(acc[2 * k + 1] * inv);
    y[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi2) << 16);
  }
  *reinterpret_cast<u32x4*>(a.out + ((size_t)(b * pre_K + i) * pre_Hq + h) * D * 2 + c * 16) = y;
}

template <typename T, int D, bool NORM>
static hipError_t launch_combine(const AttnArgs& a, hipStream_t stream) {
  const int rows = (a.Hq / a.Hkv) * a.K;  // per (b, g)
  if constexpr (NORM) {
    // split groups per row so that a lane holds at most 8 splits in flight
    auto go2 = [&](auto sg_tag) {
      constexpr int SG = decltype(sg_tag)::value;
      constexpr int RPB = 4 * (kWave / ((D / 8) * SG));
      const int chunks = (rows + RPB - 1) / RPB;
      const char* p = reinterpret_cast<const char*>(a.ws_p);
      if (a.bal)
        hipLaunchKernelGGL((attn_combine_bf16<D, SG, 8, true>), dim3(chunks * a.B * a.Hkv), dim3(256), 0, stream,
                           a.ctx_lens, a.ws_ml, p, a.B, a.Hkv, a.Hq, a.K, a.max_ctx, a.split, a.s_max, a);
      else
        hipLaunchKernelGGL((attn_combine_bf16<D, SG, 8, false>), dim3(chunks * a.B * a.Hkv), dim3(256), 0, stream,
                           a.ctx_lens, a.ws_ml, p, a.B, a.Hkv, a.Hq, a.K, a.max_ctx, a.split, a.s_max, a);
    };
    if (a.s_hint > 16) go2(std::integral_constant<int, 4>());
    else if (a.s_hint > 8) go2(std::integral_constant<int, 2>());
    else go2(std::integral_constant<int, 1>());
    return hipGetLastError();
  }
  auto go = [&](auto sg_tag) {
    constexpr int SG = decltype(sg_tag)::value;
    constexpr int RPB = 256 / ((D / 4) * SG);
    const int chunks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((attn_combine<T, D, SG, NORM>), dim3(chunks * a.B * a.Hkv), dim3(256), 0, stream, a);
  };
  if (a.s_max >= 16) go(std::integral_constant<int, 256 / (D / 4)>());
  else if (a.s_max >= 3) go(std::integral_constant<int, 2>());
  else go(std::integral_constant<int, 1>());
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 streaming kernel.  Same work decomposition, masks and softmax as
// attn_main, but the K/V stages go HBM -> LDS through the LDS-DMA path
// (global_load_lds_dwordx4: no staging registers, no LDS store instructions)
// and V stays token-major in LDS, read back transposed by ds_read_b64_tr_b16.
// A ring of kRing 64-position stages (distinct LDS arrays) keeps kRing - 1
// stages of DMA in flight: at stage t every wave waits for its own loads of
// stage t + 1 (vmcnt), one barrier publishes it, then the DMA of stage
// t + kRing - 1 is issued into the buffer stage t - 1 just released.
// Work-group = 2G waves; wave w serves query head g*G + w%G on the
// 32-position half w/G of each stage.
constexpr int kRing = 4;

template <int D>
struct StreamLayout {
  static constexpr int ROWB = D * 2;         // bytes per K/V row
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row (16 or 8)
  static constexpr int TILEB = kTile * ROWB; // one tensor's 64-row tile
  static constexpr int STAGE = 2 * TILEB;    // K tile then V tile
  static constexpr int RPI = 1024 / ROWB;    // rows per wave DMA instruction (4 or 8)
  static constexpr int IPT = kTile / RPI;    // DMA instructions per tensor tile
  static constexpr int KSW = CPR - 1;        // K: chunk ^= row & KSW
  __device__ static int kswz(int row) { return row & KSW; }
  // V: a 32-lane transposed read covers 4 consecutive rows x 64 bytes; the
  // XOR puts those 4 x 4 chunks on 16 distinct chunk positions (all 64
  // banks).  D = 128 rows are 256 B (every row starts at bank 0): chunk ^=
  // 4 (row & 3).  D = 64 rows are 128 B (odd rows start at bank 32): chunk ^=
  // 4 ((row >> 1) & 1).
  __device__ static int vswz(int row) { return D == 128 ? (row & 3) << 2 : ((row >> 1) & 1) << 2; }
};

// a page id as used: ids outside [0, num_pages) read page 0 instead (results
// for such positions are unspecified, but every access stays in bounds)
__device__ __forceinline__ int valid_page(int p, int num_pages) {
  return (unsigned)p < (unsigned)num_pages ? p : 0;
}

// DMA of one stage (positions p0 .. p0 + 63).  Lane l of a wave instruction
// writes 16 bytes at the instruction's LDS base + 16 l, i.e. row (base row +
// l / CPR), chunk slot l % CPR, and therefore loads the chunk the slot's
// swizzle assigns there.  The stage's instructions are dealt round-robin to
// the waves (wave w owns q = w + NW k).  A lane's offset inside its (page,
// head) block depends only on (lane, slot): loop invariant.
template <int D, int NW>
struct DmaPlan {
  typedef StreamLayout<D> Lay;
  static constexpr int NI = 2 * Lay::IPT;       // instructions per stage
  static constexpr int NS = (NI + NW - 1) / NW; // per wave

  __device__ static int voff(int wave, int lane, int k) {
    const int q = wave + NW * k;
    const int ten = q / Lay::IPT, ii = q % Lay::IPT;
    const int row = ii * Lay::RPI + lane / Lay::CPR;
    const int tok = ten == 0 ? swap_bits23(row) : row;
    const int chunk = (lane % Lay::CPR) ^ (ten == 0 ? Lay::kswz(row) : Lay::vswz(row));
    return (tok & 15) * Lay::ROWB + chunk * 16;
  }

  // the whole stage lies in the cached context, in the (valid) pages pid0..3
  __device__ static void issue_ids(char* st, const AttnArgs& a, int g, int pid0, int pid1, int pid2, int pid3,
                                   int wave, int lane) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int q = wave + NW * k;
      if (NI % NW != 0 && q >= NI) break;
      const int ten = q / Lay::IPT, ii = q % Lay::IPT;
      const int slot = (ii * Lay::RPI) >> 4;  // the instruction's rows share one page
      const int page = slot == 0 ? pid0 : slot == 1 ? pid1 : slot == 2 ? pid2 : pid3;
      const char* base = (ten == 0 ? a.k_cache : a.v_cache) + (size_t)(page * a.Hkv + g) * (kPage * Lay::ROWB);
      char* dst = st + ten * Lay::TILEB + ii * 1024;
      dma16_kv(base + voff(wave, lane, k), dst, a.kv_once);
    }
  }

  // the whole stage lies in the cached context; the stage is page aligned,
  // so its four page ids are one 16-byte LDS read
  __device__ static void issue_cached(char* st, const AttnArgs& a, const int* pages, int page_base, int g, int p0,
                                      int wave, int lane) {
    const int4 pq = *reinterpret_cast<const int4*>(pages + ((p0 >> 4) - page_base));
    const int n = a.num_pages;
    issue_ids(st, a, g, valid_page(__builtin_amdgcn_readfirstlane(pq.x), n),
              valid_page(__builtin_amdgcn_readfirstlane(pq.y), n), valid_page(__builtin_amdgcn_readfirstlane(pq.z), n),
              valid_page(__builtin_amdgcn_readfirstlane(pq.w), n), wave, lane);
  }

  // the stage reaches the context tail, the block rows or the split end:
  // per-lane source selection (positions past the split end read a valid
  // block K/V address; their scores are masked)
  __device__ static void issue_tail(char* st, const AttnArgs& a, const int* pages, int page_base, int b, int g,
                                    int L, int p_end, int p0, int wave, int lane) {
    const int lrow = lane / Lay::CPR, cs = lane % Lay::CPR;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int q = wave + NW * k;
      if (NI % NW != 0 && q >= NI) break;
      const int ten = q / Lay::IPT, ii = q % Lay::IPT;
      const int row = ii * Lay::RPI + lrow;
      const int tok = ten == 0 ? swap_bits23(row) : row;
      const int chunk = cs ^ (ten == 0 ? Lay::kswz(row) : Lay::vswz(row));
      const char* cache = ten == 0 ? a.k_cache : a.v_cache;
      const char* blk = ten == 0 ? a.k_blk : a.v_blk;
      const int pos = p0 + tok;
      const char* src = blk + chunk * 16;
      if (pos < L && pos < p_end)
        src = cache + ((size_t)(valid_page(pages[(pos >> 4) - page_base], a.num_pages) * a.Hkv + g) * kPage +
                       (pos & 15)) * Lay::ROWB + chunk * 16;
      else if (pos >= L && pos < p_end)
        src = blk + ((size_t)(b * a.K + (pos - L)) * a.Hkv + g) * Lay::ROWB + chunk * 16;
      char* dst = st + ten * Lay::TILEB + ii * 1024;
      dma16_kv(src, dst, a.kv_once);
    }
  }

  __device__ static void issue(char* st, const AttnArgs& a, const int* pages, int page_base, int b, int g, int L,
                               int p_end, int p0, int wave, int lane) {
    if (p0 >= p_end) return;
    if (p0 + kTile <= L && p0 + kTile <= p_end)
      issue_cached(st, a, pages, page_base, g, p0, wave, lane);
    else
      issue_tail(st, a, pages, page_base, b, g, L, p_end, p0, wave, lane);
  }
};

// The leading scalar arguments repeat the fields the prologue's first loads
// depend on (context lengths, page table and the work-group decomposition).
// Scalar kernel arguments can be preloaded into SGPRs when the wave starts
// (the build asks for the first six), so the first context-length and
// page-id loads do not wait for a kernel-argument load.
template <int D, int G, int MODE, bool BAL>
__global__ void __launch_bounds__(2 * kWave * G)
    attn_stream(const int32_t* pre_ctx, const int32_t* pre_pt, int pre_B, int pre_Hkv, int pre_split,
                int pre_maxpages, AttnArgs a) {
  typedef StreamLayout<D> Lay;
  typedef DmaPlan<D, 2 * G> Plan;
  constexpr int NW = 2 * G;
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;
  static_assert(4 * (MB / 2) * 16 * kWave * 4 <= Lay::STAGE, "exchange area: four waves per stage buffer");
  static_assert(G <= 4, "exchange areas cover eight waves");

  __shared__ __attribute__((aligned(1024))) char st0[Lay::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Lay::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[Lay::STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[Lay::STAGE];
  __shared__ __attribute__((aligned(16))) int pages[kMaxSplit / kPage];

  // G = 2 measured faster reading these from the argument struct
  const int arg_B = G == 4 ? pre_B : a.B, arg_Hkv = G == 4 ? pre_Hkv : a.Hkv;
  const int BH = arg_B * arg_Hkv;
  const int bg = blockIdx.x % BH;
  const int g = bg % arg_Hkv;
  // the fixed split's unit: sequences in reverse order, so where later
  // sequences carry longer contexts (the chunks of a prompt prefill) the
  // longest work-groups start first.  Under the balanced split it is the unit
  // of a batch whose lengths all equal max_ctx: its page ids are loaded
  // before the lengths are known and kept when the guess holds.
  int s = blockIdx.x / BH;
  int b = arg_B - 1 - bg / arg_Hkv;
  int split = G == 4 ? pre_split : a.split;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int i = lane & 31, hi = lane >> 5;
  const int hw = wave % G, sub = wave / G;
  const int h = g * G + hw;

  // ---- prologue.  The context length and the page ids of the first three
  // stages are scalar loads (constant address space: counted by lgkmcnt, not
  // by vmcnt), so the K/V DMA of those stages starts after one load latency.
  // The split's page table and the query rows reach LDS by DMA as well: no
  // load the compiler tracks with vmcnt is in flight behind the K/V stream,
  // so the hand-placed vmcnt waits below stay exact (the balanced split's
  // length loads are consumed before the first DMA).
  typedef const __attribute__((address_space(4))) int cint;
  constexpr int NPRO = (kRing - 1) * kTile / kPage;  // page ids of the prologue stages
  int L = BAL ? 0 : ((cint*)(G == 4 ? pre_ctx : a.ctx_lens))[b];  // balanced: every length is read below
  int page_base = (s * split) >> 4;
  bool ids_ok;
  int pid[NPRO];  // raw; checked where used
  auto load_ids = [&]() {
    const int arg_maxpages = G == 4 ? pre_maxpages : a.max_pages;
    ids_ok = page_base + NPRO <= arg_maxpages;
    if (ids_ok) {
      cint* row = (cint*)((G == 4 ? pre_pt : a.page_table) + (size_t)b * arg_maxpages + page_base);
#pragma unroll
      for (int j = 0; j < NPRO; ++j) pid[j] = row[j];
    } else {
#pragma unroll
      for (int j = 0; j < NPRO; ++j) pid[j] = 0;
    }
  };
  load_ids();
  int S_b;
  size_t part;        // this wave's partial slot (rows part * kRows ...)
  int first_slot = 0;  // balanced split: slot of the sequence's split 0
  if constexpr (BAL) {
    const BalUnit u = balanced_unit(a, blockIdx.x / a.Hkv, lane);
    if (!u.live) return;  // uniform over the work-group
    const bool same = u.b == b && u.s * u.split == s * split;
    b = u.b;
    s = u.s;
    split = u.split;
    page_base = (s * split) >> 4;
    if (!same) load_ids();
    L = u.L;
    S_b = u.n;
    part = (size_t)(g * a.U + u.slot) * G + hw;
    first_slot = u.slot - u.s;
  } else {
    L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
    S_b = L > 0 ? (L + split - 1) / split : 1;
    if (s >= S_b) return;
    part = (size_t)(b * a.Hq + h) * a.s_max + s;
  }
  const int p_begin = s * split;
  const int N = L + a.K;
  const int p_end = s == S_b - 1 ? N : p_begin + split;
  const int ntiles = (p_end - p_begin + kTile - 1) / kTile;

  // the split's page ids -> LDS (raw; checked where they are used); ids past
  // the table row are never used
  {
    const int npt = min(split / kPage, a.max_pages - page_base);
    const int* prow = a.page_table + (size_t)b * a.max_pages + page_base;
    for (int k = wave; k * kWave < npt; k += NW) {
      const int x = k * kWave + lane;
      dma4(prow + (x < npt ? x : 0), reinterpret_cast<char*>(pages) + k * kWave * 4);
    }
  }
  // the G query heads of every block row -> st3 (free until stage 3 is
  // issued): row i holds QR bytes, its 16-byte chunks XOR-swizzled by the row
  // (i & QSW) so the per-lane reads below hit distinct banks; rows >= K read
  // row 0 and are zeroed after the read
  constexpr int QR = G * D * 2;
  constexpr int QCH = QR / 16;
  constexpr int QSW = (QCH < 16 ? QCH : 16) - 1;
  constexpr int RQ = 1024 / QR;  // rows per DMA instruction
  static_assert(kRows * QR <= Lay::STAGE, "query rows fit one stage buffer");
  for (int k = wave; k < kRows / RQ; k += NW) {
    const int row = k * RQ + lane / QCH, slot = lane % QCH;
    const char* src = a.q + ((size_t)(b * a.K + (row < a.K ? row : 0)) * a.Hq + g * G) * D * 2 +
                      ((slot ^ (row & QSW)) << 4);
    dma16(src, st3 + k * 1024);
  }
  typedef bf16x8 V8;
  V8 qf[KS];  // this wave's query rows (B operand of QK), read from st3 below

  f32x16 o[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[m][r] = 0.f;
  float m_c = -INFINITY;
  float l = 0.f;
  const float c = a.c;

  // lane constants of the LDS reads
  // K, this wave's score tile, k-step ks: row 32 sub + i, chunk (2 ks + hi) ^ (row & KSW)
  //   = ((32 sub + i) * ROWB + ((hi ^ (i & KSW)) << 4)) ^ (ks << 5)
  const int kofs = (32 * sub + i) * Lay::ROWB + ((hi ^ (i & Lay::KSW)) << 4);
  // V^T operand, 16-position step j, d block m, half hh: the lane supplies
  // row 32 sub + 16 j + 8 hi + 4 hh + s16/4 and the 8 bytes at element
  // 32 m + 16 ((lane/16) & 1) + 4 (s16 & 3); with the V swizzle this is
  //   (32 sub + 16 j + 4 hh) * ROWB + (vofs ^ (m << 6))
  const int s16 = lane & 15, g2 = (lane >> 4) & 1;
  const int vrow = s16 >> 2;
  const int vchunk = (2 * g2 + ((s16 >> 1) & 1)) ^ Lay::vswz(vrow);
  const int vofs = (8 * hi + vrow) * Lay::ROWB + (vchunk << 4) + 8 * (s16 & 1);

  // One stage = QK (scores of this wave's 32 positions), softmax, PV.  The
  // scores of stage t+1 are computed during iteration t (software
  // pipelining), so their MFMAs can overlap this stage's softmax VALU work.
  // A tile's MFMA operands are all read from LDS before its first MFMA (one
  // read issued before each MFMA made every MFMA wait for its own read).
  auto qk = [&](const char* stage, f32x16& sc) {
    V8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = __builtin_bit_cast(V8, ld16(stage + (kofs ^ (ks << 5))));
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma_step(kf[ks], qf[ks], sc);
  };
  // softmax, first half: mask the tail, row max, lazy rescale of the
  // running state; returns the reference max for the exponentials
  auto sm_max = [&](f32x16& sc, int pbase) {
    // sc[r]: score of position pbase + 16(r/8) + 8hi + r%8 for row i
    if (pbase + 32 > L) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = pbase + 16 * (r >> 3) + 8 * hi + (r & 7);
        bool vis;
        if (MODE == ORTHRUS_DIFF_BIDIR) vis = pos < N;
        else vis = pos < L || (pos < N && pos - L <= i);
        if (!vis) sc[r] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = wave_max_xor32(mx);
    const bool need = mx * c > m_c + kRescaleLog2;
    if (__any(need)) {
      const float new_mc = need ? mx * c : m_c;
      const float f = (new_mc == m_c) ? 1.f : __builtin_amdgcn_exp2f(m_c - new_mc);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[m][r] *= f;
      l *= f;
      m_c = new_mc;
    }
    return (m_c == -INFINITY) ? 0.f : m_c;
  };
  // softmax, second half: probabilities (the two 16-position B operands of
  // PV) and the row sum
  auto sm_exp = [&](f32x16& sc, float mref, V8& p0, V8& p1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mref));
      l += sc[r];
    }
    p0 = pack_p<bf16>(sc, 0);
    p1 = pack_p<bf16>(sc, 1);
  };
  auto pv = [&](const char* stage, const V8& p0, const V8& p1) {
    const char* vt = stage + Lay::TILEB + 32 * sub * Lay::ROWB;
    V8 vf[2][MB];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const char* vb = vt + 16 * j * Lay::ROWB;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int off = vofs ^ (m << 6);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ORTHRUS_LDS bf16x4*)(vb + off));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ORTHRUS_LDS bf16x4*)(vb + 4 * Lay::ROWB + off));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[j][m][e] = lo[e];
          vf[j][m][4 + e] = hi4[e];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < MB; ++m) o[m] = mfma_step(vf[j][m], j == 0 ? p0 : p1, o[m]);
  };

  char* const ring[kRing] = {st0, st1, st2, st3};
  // stages 0 .. kRing-2 in flight: straight from the scalar page ids when all
  // of them are whole cached stages, else through the LDS page table
  if (ids_ok && p_begin + (kRing - 1) * kTile <= L && p_begin + (kRing - 1) * kTile <= p_end) {
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u)
      Plan::issue_ids(ring[u], a, g, valid_page(pid[4 * u], a.num_pages), valid_page(pid[4 * u + 1], a.num_pages),
                      valid_page(pid[4 * u + 2], a.num_pages), valid_page(pid[4 * u + 3], a.num_pages), wave, lane);
  } else {
    wait_vmcnt<0>();  // this wave's page-table (and query) DMA
    __syncthreads();  // the split's page ids are in LDS
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u)
      Plan::issue(ring[u], a, pages, page_base, b, g, L, p_end, p_begin + u * kTile, wave, lane);
  }
  // stage 0 (and, issued before it, the page table and query rows) landed
  if (ntiles > 2) wait_vmcnt<2 * Plan::NS>();
  else wait_vmcnt<0>();
  barrier_no_fence();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int chunk = (hw * (D * 2 / 16) + 2 * ks + hi) ^ (i & QSW);
    qf[ks] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(st3 + i * QR + chunk * 16));
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[ks][e] = i < a.K ? qf[ks][e] : (bf16)0.f;
  }
  // scores of stage t live in scores[t & 1] (kRing is even, so the parity is
  // a compile-time constant in the unrolled body)
  static_assert(kRing % 2 == 0, "score double buffer alternates with the ring");
  f32x16 scores[2];
  qk(ring[0], scores[0]);
#pragma unroll
  for (int r = 0; r < 16; ++r) scores[1][r] = 0.f;
  const int my_lo = p_begin + 32 * sub;  // this wave's first position in a stage
  for (int t0 = 0; t0 < ntiles; t0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int t = t0 + u;
      if (t >= ntiles) break;
      // stage t+1 must have landed (the loads of stage t+2 may still fly)
      if (t + 2 < ntiles) wait_vmcnt<Plan::NS>();
      else wait_vmcnt<0>();
      barrier_no_fence();
      Plan::issue(ring[(u + kRing - 1) % kRing], a, pages, page_base, b, g, L, p_end,
                  p_begin + (t + kRing - 1) * kTile, wave, lane);
      const char* cur = ring[u];
      const char* nxt = ring[(u + 1) % kRing];
      const int pbase = my_lo + t * kTile;
      // One basic block for the scheduler: the next stage's QK MFMAs are
      // independent of this stage's exponentials and can issue beside them.
      // Both run unconditionally: past the last stage the QK reads a stale
      // buffer whose scores are never used, and a wave half wholly past the
      // end of the last split has every position masked (zero weight).
      V8 p0, p1;
      const float mref = sm_max(scores[u & 1], pbase);
      qk(nxt, scores[(u + 1) & 1]);
      sm_exp(scores[u & 1], mref, p0, p1);
      pv(cur, p0, p1);
    }
  }

  // ---- epilogue.  The two 32-position halves of each head (sub 0, sub 1)
  // are merged through LDS; afterwards sub 0 owns d blocks [0, MB/2) of the
  // head and sub 1 owns [MB/2, MB).  Both evaluate the row statistics with
  // the same expression (sub 0's values first), so they agree bit for bit.
  wait_vmcnt<0>();
  __syncthreads();  // the ring is free
  if constexpr (BAL) {
    // sequence b's split count and first partial slot, for the combine
    if (s == 0 && g == 0 && tid == 0) a.ws_rec[b] = make_int2(S_b, first_slot);
  }
  constexpr int MH = MB / 2;
  constexpr int NC = MH * 4;                 // 16-byte chunks a lane hands over
  constexpr int XSH = NC == 8 ? 1 : 2;       // chunk swizzle: 16 lanes of a
  // 16-byte access cover all 64 banks (lane stride 16 NC bytes)
  // exchange areas: wave slot k = 2 hw + sub; slots 0-3 in st0, 4-7 in st1;
  // lane l's chunk c at (c ^ ((l >> XSH) & (NC - 1)))
  auto xslot = [&](int k) { return (k < 4 ? st0 : st1) + (k & 3) * (NC * 16) * kWave + lane * (NC * 16); };
  const int xsw = (lane >> XSH) & (NC - 1);
  {
    char* xo = xslot(hw * 2 + sub);
    float* xm = reinterpret_cast<float*>(st2) + (hw * 2 + sub) * 2 * kWave;
    // the half the partner keeps (selects, not a runtime index, keep o in
    // registers)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int mm = c / 4, r0 = 4 * (c % 4);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sub == 0 ? o[MH + mm][r0 + e] : o[mm][r0 + e];
      *reinterpret_cast<f32x4*>(xo + ((c ^ xsw) << 4)) = v;
    }
    xm[lane] = m_c;
    xm[kWave + lane] = l;
  }
  __syncthreads();
  f32x16 oh[MH];
  float row_m, row_l;
  {
    const int other = 1 - sub;
    const char* yo = xslot(hw * 2 + other);
    const float* ym = reinterpret_cast<const float*>(st2) + (hw * 2 + other) * 2 * kWave;
    const float m1 = ym[lane], l1 = ym[kWave + lane];
    const float mA = sub == 0 ? m_c : m1, mB = sub == 0 ? m1 : m_c;
    const float lA = sub == 0 ? l : l1, lB = sub == 0 ? l1 : l;
    const float mm_ = fmaxf(mA, mB);
    const float wA = (mA == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mA - mm_);
    const float wB = (mB == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mB - mm_);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int mm = c / 4, r0 = 4 * (c % 4);
      const f32x4 oth = *reinterpret_cast<const f32x4*>(yo + ((c ^ xsw) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float own = sub == 0 ? o[mm][r0 + e] : o[MH + mm][r0 + e];
        oh[mm][r0 + e] = sub == 0 ? wA * own + wB * oth[e] : wA * oth[e] + wB * own;
      }
    }
    const float lh = wA * lA + wB * lB;  // this lane's half of the row sum
    row_l = lh + __shfl_xor(lh, 32, kWave);
    row_m = mm_;
  }
  if (i >= a.K) return;  // both lanes of a swap pair share i
  const float inv = 1.f / row_l;
  // Lane (i, hi) holds, for d block m = sub MH + mm, the elements
  // d = 32 m + 8 rg + 4 hi + e at oh[mm][4 rg + e].  One permlane32 swap per
  // packed register pair hands rg = 2, 3 of lane (i, 0) to lane (i, 1) and
  // rg = 0, 1 of lane (i, 1) to lane (i, 0): each lane then owns the 8
  // consecutive elements d = 32 m + 16 hi + 8 j + (0..7), j = 0, 1, and
  // writes them as one 16-byte store.
  auto pack2 = [](float x, float y) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)y) << 16);
  };
  char* const row_out = S_b == 1 ? a.out + ((size_t)(b * a.K + i) * a.Hq + h) * D * 2
                                 : reinterpret_cast<char*>(a.ws_p) + (part * kRows + i) * D * 2;
#pragma unroll
  for (int mm = 0; mm < MH; ++mm) {
    uint32_t pk[4][2];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      pk[rg][0] = pack2(oh[mm][4 * rg] * inv, oh[mm][4 * rg + 1] * inv);
      pk[rg][1] = pack2(oh[mm][4 * rg + 2] * inv, oh[mm][4 * rg + 3] * inv);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(pk[j][0], pk[j + 2][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pk[j][1], pk[j + 2][1], false, false);
      const int d0 = 32 * (sub * MH + mm) + 16 * hi + 8 * j;
      *reinterpret_cast<u32x4*>(row_out + d0 * 2) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
  }
  // ---- split context: the row statistics (max in log2 units, sum) go with
  // the normalised partial (bf16, O / l) to slot s; attn_combine merges.
  if (S_b > 1 && sub == 0 && hi == 0)
    a.ws_ml[part * kRows + i] = make_float2(row_m, row_l);
}

// Prompt prefill tile (AR_CAUSAL, bf16, G <= 4).  A prefill runs the
// prompt's 32-row chunks as virtual sequences of this layout (chunk j of
// sequence b: a causal block after L_b + 32 j cached tokens), C chunks per
// sequence.  One work-group serves a PAIR of consecutive chunks (2j', 2j'+1)
// of one sequence for KV head g and context split s.  Wave w owns query head
// g G + w % G on the 32 rows of chunk 2j' + w / G and computes every position
// of each 64-position stage (two 32-position score tiles), so each K/V byte
// the work-group streams serves 64 G query rows instead of the 32 G of
// attn_stream: the re-reads of a long prompt's prefix, which bound the
// chunked prefill, halve.
//
// The stream covers the first chunk's context (L0 cached positions, read
// through the page table) and then the pair's 64 prompt rows (read from the
// prompt's own k/v, as block keys).  For the second chunk the first chunk's
// rows are cached context; they are the same values.  Each chunk keeps its
// own split partition, the one the combine derives from its context length:
// in the first chunk's last split the second chunk's waves mask positions
// past their own split end, and where only the second chunk has a split left
// the first chunk's waves run with every position masked and write nothing.
// Outputs and partials use the per-chunk rows of the virtual batch, so the
// combine kernel is shared with attn_stream.
template <int D, int G>
__global__ void __launch_bounds__(2 * kWave * G) attn_prefill_pair(AttnArgs a, int C) {
  typedef StreamLayout<D> Lay;
  typedef DmaPlan<D, 2 * G> Plan;
  constexpr int NW = 2 * G;
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;
  constexpr int QR = G * D * 2;                            // bytes of one row's G query heads
  constexpr int QB = 2 * kRows * QR;                       // the pair's 64 query rows
  constexpr int NQB = (QB + Lay::STAGE - 1) / Lay::STAGE;  // stage buffers they occupy
  static_assert(NQB == 1 || NQB == 2, "the pair's query rows fit two stage buffers");
  static_assert(QR <= 1024 && 1024 % QR == 0, "whole rows per DMA instruction");

  __shared__ __attribute__((aligned(1024))) char st0[Lay::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Lay::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[Lay::STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[Lay::STAGE];
  __shared__ __attribute__((aligned(16))) int pages[kMaxSplit / kPage];

  // block id = s * (pairs * Hkv) + pair * Hkv + g: the work-groups of one KV
  // head share an XCD; pairs in reverse order (the longest, latest chunks
  // first)
  const int PC = (C + 1) / 2;
  const int NP = (a.B / C) * PC;
  const int BH = NP * a.Hkv;
  const int bg = blockIdx.x % BH;
  const int g = bg % a.Hkv;
  const int s = blockIdx.x / BH;
  const int pb = NP - 1 - bg / a.Hkv;
  const int jp = pb % PC;
  const int vb0 = (pb / PC) * C + 2 * jp;  // the pair's first chunk
  const bool has1 = 2 * jp + 1 < C;        // a second chunk exists
  const int split = a.split;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int i = lane & 31, hi = lane >> 5;
  const int hw = wave % G, rb = wave / G;
  const int h = g * G + hw;

  int L0 = a.ctx_lens[vb0];
  L0 = L0 < 0 ? 0 : (L0 > a.max_ctx ? a.max_ctx : L0);
  // each chunk's split count and the end of its range in split s
  auto splits_of = [&](int Lc) { return Lc > 0 ? (Lc + split - 1) / split : 1; };
  const int L1 = L0 + kRows;
  const int S0 = splits_of(L0), S1 = splits_of(L1);
  const int p_begin = s * split;
  const int e0 = s < S0 ? (s == S0 - 1 ? L0 + kRows : p_begin + split) : p_begin;
  const int e1 = has1 && s < S1 ? (s == S1 - 1 ? L1 + kRows : p_begin + split) : p_begin;
  const int p_end = e0 > e1 ? e0 : e1;  // the stream: both chunks' ranges in split s
  if (p_end <= p_begin) return;         // uniform over the work-group
  const int ntiles = (p_end - p_begin + kTile - 1) / kTile;
  // this wave's chunk: context Lw, its range ends at pew (p_begin: no split s)
  const int Lw = rb == 0 ? L0 : L1;
  const int pew = rb == 0 ? e0 : e1;
  const int Sw = rb == 0 ? S0 : S1;
  const int vbw = vb0 + rb;
  const int page_base = p_begin >> 4;

  // ---- prologue: the split's page ids and the pair's query rows reach LDS
  // by DMA before the first stages, so the hand-placed vmcnt waits stay exact
  {
    const int npt = min(split / kPage, a.max_pages - page_base);
    const int* prow = a.page_table + (size_t)vb0 * a.max_pages + page_base;
    for (int k = wave; k * kWave < npt; k += NW) {
      const int x = k * kWave + lane;
      dma4(prow + (x < npt ? x : 0), reinterpret_cast<char*>(pages) + k * kWave * 4);
    }
  }
  // query row r (0..63) of the pair: QR bytes at byte r QR of the query
  // area (st3, or st2 then st3), its 16-byte chunks XOR-swizzled by (r & QSW);
  // rows of a missing second chunk read row 0 (never used)
  constexpr int QCH = QR / 16;
  constexpr int QSW = (QCH < 16 ? QCH : 16) - 1;
  constexpr int RQ = 1024 / QR;
  char* const qarea0 = NQB == 2 ? st2 : st3;
  auto qaddr = [&](int off) -> char* { return off < Lay::STAGE ? qarea0 + off : st3 + (off - Lay::STAGE); };
  for (int k = wave; k < 2 * kRows / RQ; k += NW) {
    const int row = k * RQ + lane / QCH, slot = lane % QCH;
    const int src_row = row < kRows || has1 ? vb0 * kRows + row : vb0 * kRows;
    const char* src = a.q + ((size_t)src_row * a.Hq + g * G) * D * 2 + ((slot ^ (row & QSW)) << 4);
    dma16(src, qaddr(k * 1024));
  }
  // K/V stages 0 .. NPRO_ST - 1 (the ring's other buffers hold the queries)
  constexpr int NPRO_ST = kRing - NQB;
  char* const ring[kRing] = {st0, st1, st2, st3};
  wait_vmcnt<0>();  // this wave's page-table and query DMA
  __syncthreads();  // the split's page ids are in LDS
#pragma unroll
  for (int u = 0; u < NPRO_ST; ++u)
    Plan::issue(ring[u], a, pages, page_base, vb0, g, L0, p_end, p_begin + u * kTile, wave, lane);
  // stage 0 landed (the later prologue stages may still fly when all of
  // them were issued)
  if (ntiles >= NPRO_ST) wait_vmcnt<(NPRO_ST - 1) * Plan::NS>();
  else wait_vmcnt<0>();
  barrier_no_fence();
  typedef bf16x8 V8;
  V8 qf[KS];
  {
    const int r = kRows * rb + i;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int chunk = (hw * (D * 2 / 16) + 2 * ks + hi) ^ (r & QSW);
      qf[ks] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(qaddr(r * QR + chunk * 16)));
    }
  }

  f32x16 o[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[m][r] = 0.f;
  float m_c = -INFINITY;
  float l = 0.f;
  const float c = a.c;
  const int kofs = i * Lay::ROWB + ((hi ^ (i & Lay::KSW)) << 4);
  const int s16 = lane & 15, g2 = (lane >> 4) & 1;
  const int vrow = s16 >> 2;
  const int vchunk = (2 * g2 + ((s16 >> 1) & 1)) ^ Lay::vswz(vrow);
  const int vofs = (8 * hi + vrow) * Lay::ROWB + (vchunk << 4) + 8 * (s16 & 1);

  // One 32-position tile (positions 32 q .. 32 q + 31 of a stage) at a time,
  // with online softmax per tile: the scores of the next tile (the stage's
  // second tile, or the next stage's first) are computed before this tile's
  // softmax, so their MFMAs can issue beside its exponentials, and only two
  // score tiles are live (the register budget of two waves per SIMD).
  // The operands of a tile's MFMAs are all read from LDS before the first of
  // them: issued one before each MFMA, every MFMA waited for its own read
  // (measured 5 % slower on the 8192-token prompt).
  auto qk = [&](const char* stage, int q, f32x16& sc) {
    V8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = __builtin_bit_cast(V8, ld16(stage + q * kRows * Lay::ROWB + (kofs ^ (ks << 5))));
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma_step(kf[ks], qf[ks], sc);
  };
  // mask (this wave's causal rows and range), row max, lazy rescale
  const int vis_end = Lw < pew ? Lw : pew;  // below it every position is visible
  auto sm_max = [&](f32x16& sc, int pbase) {
    // sc[r]: position pbase + 16 (r / 8) + 8 hi + r % 8, row i
    if (pbase + 32 > vis_end) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = pbase + 16 * (r >> 3) + 8 * hi + (r & 7);
        const bool vis = pos < pew && (pos < Lw || pos - Lw <= i);
        if (!vis) sc[r] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = wave_max_xor32(mx);
    const bool need = mx * c > m_c + kRescaleLog2;
    if (__any(need)) {
      const float new_mc = need ? mx * c : m_c;
      const float f = (new_mc == m_c) ? 1.f : __builtin_amdgcn_exp2f(m_c - new_mc);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[m][r] *= f;
      l *= f;
      m_c = new_mc;
    }
    return (m_c == -INFINITY) ? 0.f : m_c;
  };
  auto sm_exp = [&](f32x16& sc, float mref, V8& p0, V8& p1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mref));
      l += sc[r];
    }
    p0 = pack_p<bf16>(sc, 0);
    p1 = pack_p<bf16>(sc, 1);
  };
  auto pv = [&](const char* stage, int q, const V8& p0, const V8& p1) {
    const char* vt = stage + Lay::TILEB + q * kRows * Lay::ROWB;
    V8 vf[2][MB];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const char* vb = vt + 16 * j * Lay::ROWB;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int off = vofs ^ (m << 6);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ORTHRUS_LDS bf16x4*)(vb + off));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ORTHRUS_LDS bf16x4*)(vb + 4 * Lay::ROWB + off));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[j][m][e] = lo[e];
          vf[j][m][4 + e] = hi4[e];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < MB; ++m) o[m] = mfma_step(vf[j][m], j == 0 ? p0 : p1, o[m]);
  };

  // scores[q] holds the scores of tile q of the current stage
  f32x16 scores[2];
  qk(ring[0], 0, scores[0]);
  for (int t0 = 0; t0 < ntiles; t0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int t = t0 + u;
      if (t >= ntiles) break;
      // stage t+1 must have landed (the loads of stage t+2 may still fly;
      // with two query buffers, stage 2 is issued only below, at t = 0)
      if (NQB == 2 && t == 0) wait_vmcnt<0>();
      else if (t + 2 < ntiles) wait_vmcnt<Plan::NS>();
      else wait_vmcnt<0>();
      barrier_no_fence();
      if (NQB == 2 && t == 0)  // st2 held query rows until this barrier
        Plan::issue(ring[2], a, pages, page_base, vb0, g, L0, p_end, p_begin + 2 * kTile, wave, lane);
      Plan::issue(ring[(u + kRing - 1) % kRing], a, pages, page_base, vb0, g, L0, p_end,
                  p_begin + (t + kRing - 1) * kTile, wave, lane);
      const char* cur = ring[u];
      const char* nxt = ring[(u + 1) % kRing];
      const int pbase = p_begin + t * kTile;
      // Past the last stage the next tile's QK reads a stale buffer whose
      // scores are never used.
      V8 p0, p1;
      float mref = sm_max(scores[0], pbase);
      qk(cur, 1, scores[1]);
      sm_exp(scores[0], mref, p0, p1);
      pv(cur, 0, p0, p1);
      mref = sm_max(scores[1], pbase + kRows);
      qk(nxt, 0, scores[0]);
      sm_exp(scores[1], mref, p0, p1);
      pv(cur, 1, p0, p1);
    }
  }
  wait_vmcnt<0>();  // no DMA outlives the loop
  if (pew <= p_begin) return;  // this chunk has no split s (or does not exist)

  // ---- epilogue: every wave holds whole rows; the two lanes of a row
  // (hi = 0, 1) add their halves of the row sum
  const float row_l = l + __shfl_xor(l, 32, kWave);
  const float inv = 1.f / row_l;
  const size_t part = (size_t)(vbw * a.Hq + h) * a.s_max + s;
  auto pack2 = [](float x, float y) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)y) << 16);
  };
  char* const row_out = Sw == 1 ? a.out + ((size_t)(vbw * a.K + i) * a.Hq + h) * D * 2
                                : reinterpret_cast<char*>(a.ws_p) + (part * kRows + i) * D * 2;
  // lane (i, hi) holds d = 32 m + 8 rg + 4 hi + e at o[m][4 rg + e]; one
  // permlane32 swap per register pair gives each lane 8 consecutive
  // elements d = 32 m + 16 hi + 8 j + (0..7) for one 16-byte store
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    uint32_t pk[4][2];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      pk[rg][0] = pack2(o[m][4 * rg] * inv, o[m][4 * rg + 1] * inv);
      pk[rg][1] = pack2(o[m][4 * rg + 2] * inv, o[m][4 * rg + 3] * inv);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(pk[j][0], pk[j + 2][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pk[j][1], pk[j + 2][1], false, false);
      const int d0 = 32 * m + 16 * hi + 8 * j;
      *reinterpret_cast<u32x4*>(row_out + d0 * 2) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
  }
  if (Sw > 1 && hi == 0) a.ws_ml[part * kRows + i] = make_float2(m_c, row_l);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Work-groups per KV head of one round on 256 CUs.
static int attn_round_slots(const orthrus_attn_desc& d) { return ceil_div(256, d.n_kv_heads); }

int attn_split_tokens(const orthrus_attn_desc& d) {
  // splits partition the cached context (the last split also takes the K
  // block keys)
  const long Lm = d.max_ctx_len > 0 ? d.max_ctx_len : 1;
  const long l64 = ((Lm + kTile - 1) / kTile) * kTile;
  if (d.split_tokens > 0) return (int)(d.split_tokens < l64 ? d.split_tokens : l64);
  // Automatic: the shortest split (in 64-position tiles, kBalMinTiles ..
  // kBalMaxTiles) that keeps a batch of max_ctx_len contexts within one round
  // of about 256 work-groups, B ceil(L / split) <= ceil(256 / Hkv) per KV
  // head; the longest split when even that needs more.  Measured on MI355X
  // (Qwen3-8B heads, 8192 tokens): at B1 320-position splits (208
  // work-groups of 5 stages) beat 256 (256 of 4) by 6-9 %, and a second,
  // partial round costs 25-35 % (B3, B6); from B8 up the full round is best.
  const long Tm = (Lm + kTile - 1) / kTile;
  const int Q = attn_round_slots(d);
  auto count = [&](int t) { return (long)d.batch * ceil_div(Tm, t); };
  // One short sequence (each work-group has at most 8 stages): the call is
  // bound by per-work-group latency, and the best measured fill is about
  // 80 % of a round with at least 3 stages per work-group (B1: 192-position
  // splits ran 6-9 % faster than 320 at 2048 and 4096 tokens with Qwen3-8B
  // heads and at 2048 with Qwen3-1.7B heads; at 8192 tokens this picks 320,
  // which beat 256 and 192).
  if (d.batch == 1) {
    const int Q80 = (Q * 13) / 16;
    int t = 3;
    while (t <= 8 && count(t) > Q80) ++t;
    if (t <= 8) {
      const long split = (long)t * kTile;
      return (int)(split < l64 ? split : l64);
    }
  }
  int lo = kBalMinTiles, hi = kBalMaxTiles;
  if (count(hi) > Q) {
    lo = hi;
  } else {
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (count(mid) <= Q) hi = mid;
      else lo = mid + 1;
    }
  }
  const long split = (long)lo * kTile;
  return (int)(split < l64 ? split : l64);
}

static int attn_s_max(const orthrus_attn_desc& d, int split) {
  return d.max_ctx_len > 0 ? ceil_div(d.max_ctx_len, split) : 1;
}

// bf16 with up to 4 query heads per KV head runs the LDS-DMA streaming
// kernel plus attn_combine_bf16; everything else the register-staged kernel
// plus attn_combine
static bool attn_stream_path(const orthrus_attn_desc& d) {
  return d.dtype == ORTHRUS_BF16 && d.n_q_heads / d.n_kv_heads <= 4;
}

// How one call divides the cached context among work-groups.  With the
// balanced split requested, several sequences (at most 64, fewer than 256
// (b, KV head) pairs) and the streaming kernel, the split length is chosen on the device
// from ctx_lens (balanced_split): the smallest multiple of 64 positions in
// [320, kMaxSplit] that makes at most Q = ceil(256 / Hkv) units per KV head,
// so one round of about 256 work-groups covers a ragged batch as evenly as
// the 64-position tiles allow; where that round's average unit is below
// kBalRoundEff of its longest, the smallest split with at most Q2 = 2 Q units
// (two rounds) instead.  The host knows only max_ctx_len: its split
// is the one a batch of that length everywhere gets, the partial slots are
// sized for the worst case, and the grid has U slots per KV head (units past
// the batch's last one exit at once).  Otherwise the split is fixed by the
// host (attn_split_tokens).
struct SplitPlan {
  bool bal;
  int split, s_max, s_hint, Q, U, Q2;
};

static SplitPlan attn_plan(const orthrus_attn_desc& d) {
  SplitPlan p{false, attn_split_tokens(d), 0, 0, 0, 0, 0};
  p.s_max = attn_s_max(d, p.split);
  p.s_hint = p.s_max;
  if (d.split_tokens != ORTHRUS_SPLIT_BALANCED || !attn_stream_path(d) || d.batch < 2 || d.batch > 64 ||
      d.batch * d.n_kv_heads >= 256 || d.max_ctx_len >= (1 << 24))  // tile counts stay exact in fp32
    return p;
  const long Tm = ((long)d.max_ctx_len + kTile - 1) / kTile;
  if (ceil_div(Tm, kBalMinTiles) <= 1) return p;  // no sequence can be split
  // the automatic split is the balanced one of a batch whose lengths all
  // equal max_ctx_len: the device's search starts from it
  p.bal = true;
  p.Q = attn_round_slots(d);
  p.Q2 = 2 * p.Q;
  const long most_units = (long)d.batch * ceil_div(Tm, kBalMaxTiles);
  p.U = (int)(most_units > p.Q2 ? most_units : p.Q2);
  const int most = ceil_div(Tm, kBalMinTiles);
  p.s_max = most < p.U - d.batch + 1 ? most : p.U - d.batch + 1;
  p.s_hint = ceil_div(Tm, p.split / kTile);
  return p;
}

struct WsLayout {
  size_t bytes, off_ml, off_rec;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// partial outputs (bf16 on the streaming path, fp32 otherwise), then the row
// statistics: [B, Hq, s_max, 32] rows under a fixed split, [Hkv, U, G, 32]
// under the balanced one, which adds one (splits, first slot) pair per
// sequence
static WsLayout attn_ws_layout(const orthrus_attn_desc& d) {
  WsLayout w{0, 0, 0};
  const SplitPlan p = attn_plan(d);
  if (p.s_max <= 1) return w;
  const size_t rows = p.bal ? (size_t)d.n_q_heads * p.U * kRows : (size_t)d.batch * d.n_q_heads * p.s_max * kRows;
  w.off_ml = align256(rows * d.head_dim * (attn_stream_path(d) ? 2 : 4));
  w.bytes = w.off_ml + rows * sizeof(float2);
  if (p.bal) {
    w.off_rec = align256(w.bytes);
    w.bytes = w.off_rec + (size_t)d.batch * sizeof(int2);
  }
  return w;
}

size_t attn_workspace_bytes(const orthrus_attn_desc& d) { return attn_ws_layout(d).bytes; }

template <typename T, int D, int G>
static hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t stream) {
  const int grid = a.bal ? a.U * a.Hkv : a.s_max * a.B * a.Hkv;
  // bf16 with up to 4 query heads per KV head: the LDS-DMA streaming kernel;
  // otherwise the register-staged kernel
  constexpr bool stream_path = sizeof(T) == 2 && G <= 4;
  if constexpr (stream_path) {
    const dim3 blk(2 * kWave * G);
    if (mode == ORTHRUS_DIFF_BIDIR) {
      if (a.bal) hipLaunchKernelGGL((attn_stream<D, G, ORTHRUS_DIFF_BIDIR, true>), dim3(grid), blk, 0, stream, a.ctx_lens,
                           a.page_table, a.B, a.Hkv, a.split, a.max_pages, a);
      else hipLaunchKernelGGL((attn_stream<D, G, ORTHRUS_DIFF_BIDIR, false>), dim3(grid), blk, 0, stream, a.ctx_lens,
                           a.page_table, a.B, a.Hkv, a.split, a.max_pages, a);
    } else {
      if (a.bal) hipLaunchKernelGGL((attn_stream<D, G, ORTHRUS_AR_CAUSAL, true>), dim3(grid), blk, 0, stream, a.ctx_lens,
                           a.page_table, a.B, a.Hkv, a.split, a.max_pages, a);
      else hipLaunchKernelGGL((attn_stream<D, G, ORTHRUS_AR_CAUSAL, false>), dim3(grid), blk, 0, stream, a.ctx_lens,
                           a.page_table, a.B, a.Hkv, a.split, a.max_pages, a);
    }
  } else {
    if (mode == ORTHRUS_DIFF_BIDIR)
      hipLaunchKernelGGL((attn_main<T, D, G, ORTHRUS_DIFF_BIDIR>), dim3(grid), dim3(2 * kWave * G), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_main<T, D, G, ORTHRUS_AR_CAUSAL>), dim3(grid), dim3(2 * kWave * G), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.s_max <= 1) return e;
  return launch_combine<T, D, stream_path>(a, stream);
}

// a prefill's virtual batch (C chunks per sequence) on the pair kernel,
// then the combine of its split partials
template <int D, int G>
static hipError_t launch_prefill_pair(const AttnArgs& a, int C, hipStream_t stream) {
  const int pairs = (a.B / C) * ((C + 1) / 2);
  hipLaunchKernelGGL((attn_prefill_pair<D, G>), dim3(a.s_max * pairs * a.Hkv), dim3(2 * kWave * G), 0, stream, a,
                     C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.s_max <= 1) return e;
  return launch_combine<bf16, D, true>(a, stream);
}

template <int D>
static hipError_t dispatch_prefill_pair(const AttnArgs& a, int G, int C, hipStream_t s) {
  switch (G) {
    case 1: return launch_prefill_pair<D, 1>(a, C, s);
    case 2: return launch_prefill_pair<D, 2>(a, C, s);
    default: return launch_prefill_pair<D, 4>(a, C, s);
  }
}

template <typename T, int D>
static hipError_t dispatch_g(const AttnArgs& a, int G, int mode, hipStream_t s) {
  switch (G) {
    case 1: return launch_attn<T, D, 1>(a, mode, s);
    case 2: return launch_attn<T, D, 2>(a, mode, s);
    case 4: return launch_attn<T, D, 4>(a, mode, s);
    default: return launch_attn<T, D, 8>(a, mode, s);
  }
}

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_block_attn_workspace_bytes(const orthrus_attn_desc* desc) {
  if (validate_desc(desc) != ORTHRUS_OK) return 0;
  return attn_workspace_bytes(*desc);
}

extern "C" int32_t orthrus_block_attn_split_tokens(const orthrus_attn_desc* desc) {
  if (validate_desc(desc) != ORTHRUS_OK) return 0;
  return attn_plan(*desc).split;
}

orthrus_status orthrus::block_attn_run(const void* q, const void* k_cache, const void* v_cache, const void* k_blk,
                                       const void* v_blk, const int32_t* page_table, const int32_t* ctx_lens,
                                       int32_t mode, void* out, const orthrus_attn_desc* desc, void* workspace,
                                       size_t workspace_bytes, void* stream, bool kv_read_once, int pair_chunks) {
  orthrus_status st = validate_desc(desc);
  if (st != ORTHRUS_OK) return st;
  if (!q || !k_cache || !v_cache || !k_blk || !v_blk || !page_table || !ctx_lens || !out)
    return ORTHRUS_ERR_NULL;
  if (mode != ORTHRUS_DIFF_BIDIR && mode != ORTHRUS_AR_CAUSAL) return ORTHRUS_ERR_SHAPE;
  if (!aligned16(q, k_cache, v_cache, k_blk, v_blk, out) || !aligned4(page_table, ctx_lens)) return ORTHRUS_ERR_SHAPE;
  const orthrus_attn_desc& d = *desc;
  const size_t need = attn_workspace_bytes(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ORTHRUS_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15)) return ORTHRUS_ERR_WORKSPACE;

  AttnArgs a;
  a.q = (const char*)q;
  a.k_cache = (const char*)k_cache;
  a.v_cache = (const char*)v_cache;
  a.k_blk = (const char*)k_blk;
  a.v_blk = (const char*)v_blk;
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.out = (char*)out;
  a.B = d.batch;
  a.K = d.block_k;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.max_ctx = d.max_ctx_len;
  const SplitPlan plan = attn_plan(d);
  a.split = plan.split;
  a.s_max = plan.s_max;
  a.bal = plan.bal ? 1 : 0;
  a.Q = plan.Q;
  a.Q2 = plan.Q2;
  a.U = plan.U;
  a.s_hint = plan.s_hint;
  a.ws_o = nullptr;
  a.ws_p = nullptr;
  a.ws_ml = nullptr;
  a.ws_rec = nullptr;
  if (need > 0) {
    const WsLayout wl = attn_ws_layout(d);
    if (attn_stream_path(d)) a.ws_p = (bf16*)workspace;
    else a.ws_o = (float*)workspace;
    a.ws_ml = (float2*)((char*)workspace + wl.off_ml);
    if (plan.bal) a.ws_rec = (int2*)((char*)workspace + wl.off_rec);
  }
  const float scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.f / sqrtf((float)d.head_dim);
  a.c = scale * kLog2e;
  a.kv_once = kv_read_once ? 1 : 0;
  const int G = d.n_q_heads / d.n_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (pair_chunks > 0 && attn_stream_path(d) && mode == ORTHRUS_AR_CAUSAL && !plan.bal && d.block_k == kRows &&
      d.batch % pair_chunks == 0)
    e = d.head_dim == 128 ? dispatch_prefill_pair<128>(a, G, pair_chunks, s)
                          : dispatch_prefill_pair<64>(a, G, pair_chunks, s);
  else if (d.dtype == ORTHRUS_BF16)
    e = d.head_dim == 128 ? dispatch_g<bf16, 128>(a, G, mode, s) : dispatch_g<bf16, 64>(a, G, mode, s);
  else
    e = d.head_dim == 128 ? dispatch_g<float, 128>(a, G, mode, s) : dispatch_g<float, 64>(a, G, mode, s);
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

extern "C" orthrus_status orthrus_block_attn(const void* q, const void* k_cache, const void* v_cache,
                                             const void* k_blk, const void* v_blk,
                                             const int32_t* page_table, const int32_t* ctx_lens,
                                             int32_t mode, void* out, const orthrus_attn_desc* desc,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  // a decode call reads every cached K/V byte once
  return block_attn_run(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, mode, out, desc, workspace,
                        workspace_bytes, stream, true);
}

// ---------------------------------------------------------------------------
// block attention without a caller workspace: the split partials live in a
// fixed device array of the library (one copy per GPU, for the life of the
// process), for callers that cannot allocate.
// ---------------------------------------------------------------------------

#include <mutex>

static __device__ __align__(256) char scratch[ORTHRUS_STATIC_SCRATCH_BYTES];

namespace orthrus {

constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU (host-side cache)
static std::mutex g_scratch_mu;

// Address of this library's scratch array on device `dev`, looked up once per
// device with that device current (the host-side name `scratch` is only a
// stand-in: each GPU holds its own copy at its own address).
static void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return g_scratch[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !p) return nullptr;
  g_scratch[dev] = p;
  return p;
}

}  // namespace orthrus

extern "C" orthrus_status orthrus_block_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                     const void* k_blk, const void* v_blk,
                                                     const int32_t* page_table, const int32_t* ctx_lens,
                                                     int32_t mode, void* out, const orthrus_attn_desc* desc,
                                                     void* stream) {
  orthrus_status st = validate_desc(desc);
  if (st != ORTHRUS_OK) return st;
  if (!q || !k_cache || !v_cache || !k_blk || !v_blk || !page_table || !ctx_lens || !out)
    return ORTHRUS_ERR_NULL;
  if (mode != ORTHRUS_DIFF_BIDIR && mode != ORTHRUS_AR_CAUSAL) return ORTHRUS_ERR_SHAPE;
  if (!aligned16(q, k_cache, v_cache, k_blk, v_blk, out) || !aligned4(page_table, ctx_lens)) return ORTHRUS_ERR_SHAPE;
  const size_t need = attn_workspace_bytes(*desc);
  if (need > ORTHRUS_STATIC_SCRATCH_BYTES) return ORTHRUS_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return ORTHRUS_ERR_LAUNCH;
    ws = scratch_on(dev);
    if (!ws) return ORTHRUS_ERR_LAUNCH;
  }
  return block_attn_run(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, mode, out, desc, ws,
                        need > 0 ? ORTHRUS_STATIC_SCRATCH_BYTES : 0, stream, true);
}

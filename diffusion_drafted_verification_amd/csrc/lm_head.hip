// Language-model head with a fused greedy argmax on gfx950: the projection
// that turns each view's final hidden states into the tokens the consensus
// step compares (Orthrus explainer, gist.science arXiv 2605.12825, technical
// summary §2.3: the diffusion head's drafts and the frozen AR head's exact
// targets both come out of the model's vocabulary projection).
//
//   logits[m, v] = sum_k hidden[m, k] * weight[v, k]   (bf16 in, fp32 accumulate)
//   token[m]     = lowest v attaining max_v logits[m, v]
//
// The logits never reach memory.  At decode sizes (rows = B * K = 32 .. 128)
// the weight [V, H] is read once per call and every byte of it feeds `rows`
// multiply-adds, so the kernel is bound by the weight stream from HBM.
//
// The weight is used in a packed layout (lm_head_pack, once per weight):
// 32-row tiles, and within a tile the A-operand fragment of every MFMA
// k-step (64 lanes x 16 bytes) stored contiguously in lane order, so a wave
// reads its tile as one sequential stream of whole 1 KiB loads (nontemporal
// when the weight is read once).  Measured on this GPU, that streams the
// weight at ~6.4 TB/s where the row-major layout (32 rows x 32 bytes per load
// instruction) tops out near 5.0 TB/s.
//
// lm_head_tiles: one work-group of 4 waves per (128-row vocabulary tile,
// group of MT x 32 hidden rows: 32 for up to 32 rows, else 64).  Each wave streams its 32-row packed
// tile straight from HBM into MFMA A-operand registers (no reuse, so no
// LDS), double-buffered by phase of KP hidden elements.  The hidden rows of
// the phase are staged once per work-group in LDS (XOR chunk swizzle,
// conflict-free 16-byte reads) as the B operand.  Products run
// on v_mfma_f32_32x32x16_bf16 with D[n][m] in the accumulators, so each lane
// owns one hidden row m and 16 vocabulary rows: the tile's argmax is a
// per-lane max, one exchange between the lane halves and one merge of the
// four waves in LDS, stored as a 64-bit key (order-preserving value bits << 32
// | ~index: a larger key is a larger value, then a lower index).  Blocks of
// one tile (its row groups) are placed on one XCD so that, when the rows need
// several groups, the later groups find the weight tile in that XCD's L2.
//
// lm_head_dma (more than 64 hidden rows): both operands reach LDS by
// LDS-DMA, the weight issued by half of the eight waves and the hidden rows by
// the other half, and the work-group multiplies a tile of 128 weight rows by
// 128 hidden rows, or 256 by 256 (each wave a block of weight slices by
// accumulator tiles).  The two 256-row groups of 512 rows run on one XCD.
//
// lm_head_finish: one work-group per group of rows reduces each row's tile
// keys (32 threads per row, all loads issued before the reduction), writes the tokens
// and, for the accept entry point, compares them with the drafts (wave
// ballot: first mismatch) exactly as the greedy consensus does.
#include "orthrus_device.h"
#include "orthrus_host.h"

namespace orthrus {

typedef float lm_f32x2 __attribute__((ext_vector_type(2)));

constexpr int kLmWaves = 4;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kLmTileN = kLmWaves * 32;  // vocabulary rows per tile
constexpr int kLmFinThreads = 1024;  // 32 rows x 32 threads
constexpr int kFinBatch = 40;         // tile keys per thread in flight
constexpr int kFinPairs = 20;         // (max, sum) pairs per thread in flight
constexpr float kLog2e = 1.4426950408889634f;

struct LmArgs {
  const bf16* h;               // [M, H]
  lm_f32x2* ms;                   // [M, ntiles] (tile max, sum of exp(logit - max)) or nullptr
  const uint8_t* masked;       // denoise: [M] 1 = position still masked
  const int32_t* n_unmask;     // denoise: [M / R]
  float* conf;                 // denoise: [M] greedy token's softmax probability
  uint8_t* masked_out;         // denoise: [M]
  const u32x4* w;              // packed weight: [ceil(V / 32)][H / 16][64 lanes] 16-byte fragments
  unsigned long long* part;    // [M, ntiles] tile keys
  const int32_t* drafts;       // [M] (accept) or nullptr
  int32_t* tokens;             // [M] or nullptr
  float* maxv;                 // [M] or nullptr
  int32_t* accept_len;         // [M / R]
  int32_t* next_token;         // [M / R]
  int M, H, V, ntiles, mgroups, R;
};

__device__ __forceinline__ uint32_t lm_order_bits(float v) {
  if (v == 0.f) v = 0.f;  // -0.0 and +0.0 are equal: one encoding
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float lm_from_order_bits(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}

__device__ __forceinline__ void lm_keep(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

template <int MT, int KP, bool NT>
__global__ void __launch_bounds__(kLmThreads) lm_head_tiles(LmArgs a) {
  constexpr int CH = KP / 8;     // 16-byte chunks of one hidden row per phase
  constexpr int NW = KP / 16;    // weight chunks per lane per phase = MFMA steps
  constexpr int ROWS = MT * 32;  // hidden rows per work-group
  constexpr int NA = ROWS * CH / kLmThreads;
  static_assert(CH >= 16 && (ROWS * CH) % kLmThreads == 0, "phase shape");
  __shared__ u32x4 hs[2][ROWS * CH];
  __shared__ float rv[kLmWaves][32];
  __shared__ int ri[kLmWaves][32];
  __shared__ float rs[kLmWaves][32];

  // block -> (tile, row group): the row groups of one tile share an XCD
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int tile = (local / a.mgroups) * 8 + xcd, mg = local % a.mgroups;
  if (tile >= a.ntiles) return;  // uniform: padding of the tile count to 8

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane >> 5, c32 = lane & 31;
  const int m0 = mg * ROWS;
  const int nbase = tile * kLmTileN + wave * 32;
  // a 32-row tile past the padded vocabulary reads the last tile (in
  // bounds); its rows are past V and are dropped below
  const int t32 = min(nbase / 32, (a.V - 1) / 32);
  const int steps = a.H / 16;
  const u32x4* wtile = a.w + (size_t)t32 * steps * kWave + lane;
  const int P = a.H / KP;

  auto load_w = [&](int p, u32x4(&wv)[NW]) {
    const u32x4* src = wtile + (size_t)p * NW * kWave;
#pragma unroll
    for (int i = 0; i < NW; ++i) wv[i] = NT ? __builtin_nontemporal_load(src + i * kWave) : src[i * kWave];
  };
  auto load_h = [&](int p, u32x4(&hv)[NA]) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + kLmThreads * i, r = q / CH, c = q % CH;
      const int m = min(m0 + r, a.M - 1);  // rows past M repeat the last row and are dropped
      hv[i] = ld16(a.h + (size_t)m * a.H + (size_t)p * KP + 8 * c);
    }
  };
  auto store_h = [&](int buf, const u32x4(&hv)[NA]) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + kLmThreads * i, r = q / CH, c = q % CH;
      hs[buf][r * CH + (c ^ (r & 15))] = hv[i];
    }
  };
  // lane (c32, g) holds weight elements k0 + 16 s + 8 g + e of step s; the
  // B operand of the same step is hidden row c32 at the same k: chunk 2 s + g
  auto compute = [&](int buf, const u32x4(&wv)[NW], f32x16(&acc)[MT]) {
#pragma unroll
    for (int s = 0; s < NW; ++s) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, wv[s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 32 + c32, c = 2 * s + g;
        const bf16x8 bv = __builtin_bit_cast(bf16x8, hs[buf][r * CH + (c ^ (r & 15))]);
        acc[mt] = mfma_step(av, bv, acc[mt]);
      }
    }
  };

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mt][e] = 0.f;

  u32x4 hv[NA], w0[NW], w1[NW];
  load_h(0, hv);
  load_w(0, w0);
  store_h(0, hv);
  __syncthreads();
  for (int p = 0; p < P; p += 2) {
    // phase p: weights w0, hidden buffer 0; the hidden rows of phase p + 1
    // are loaded first so that their wait does not cover the weight loads
    if (p + 1 < P) {
      load_h(p + 1, hv);
      load_w(p + 1, w1);
    }
    compute(0, w0, acc);
    if (p + 1 < P) store_h(1, hv);
    __syncthreads();
    if (p + 1 >= P) break;
    // phase p + 1: weights w1, hidden buffer 1
    if (p + 2 < P) {
      load_h(p + 2, hv);
      load_w(p + 2, w0);
    }
    compute(1, w1, acc);
    if (p + 2 < P) store_h(0, hv);
    __syncthreads();
  }

  // argmax of the tile per hidden row.  Accumulator register e of lane
  // (c32, g) holds vocabulary row nbase + 8 (e / 4) + 4 g + e % 4 and hidden
  // row m0 + 32 mt + c32; the rows grow with e, so a strict compare keeps
  // the lowest index.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int nn = nbase + 8 * (e >> 2) + 4 * g + (e & 3);
      if (nn < a.V && acc[mt][e] > bv) {
        bv = acc[mt][e];
        bi = nn;
      }
    }
    lm_keep(bv, bi, __shfl_xor(bv, 32, kWave), __shfl_xor(bi, 32, kWave));
    // softmax statistics of the tile (denoise): the sum of exp(logit - max)
    // over the wave's 32 rows, then merged over the four waves
    float se = 0.f;
    if (a.ms) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int nn = nbase + 8 * (e >> 2) + 4 * g + (e & 3);
        se += nn < a.V ? __builtin_amdgcn_exp2f((acc[mt][e] - bv) * kLog2e) : 0.f;
      }
      se += __shfl_xor(se, 32, kWave);
    }
    if (g == 0) {
      rv[wave][c32] = bv;
      ri[wave][c32] = bi;
      rs[wave][c32] = se;
    }
    __syncthreads();
    if (wave == 0 && g == 0) {
      const float wmax0 = bv;
#pragma unroll
      for (int w = 1; w < kLmWaves; ++w) lm_keep(bv, bi, rv[w][c32], ri[w][c32]);
      const int m = m0 + mt * 32 + c32;
      if (m < a.M) {
        a.part[(size_t)m * a.ntiles + tile] =
            ((unsigned long long)lm_order_bits(bv) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)bi);
        if (a.ms) {
          // waves whose rows are all past V hold (-inf, 0) and add nothing
          float tot = se * __builtin_amdgcn_exp2f((wmax0 - bv) * kLog2e);
#pragma unroll
          for (int w = 1; w < kLmWaves; ++w)
            tot += rv[w][c32] == -INFINITY ? 0.f : rs[w][c32] * __builtin_amdgcn_exp2f((rv[w][c32] - bv) * kLog2e);
          a.ms[(size_t)m * a.ntiles + tile] = lm_f32x2{bv, tot};
        }
      }
    }
    __syncthreads();
  }
}

// Many hidden rows (more than 64): both operands reach LDS by LDS-DMA in
// stages of 32 or 64 hidden elements, and the work-group multiplies a tile of
// NSL 32-row weight slices by MT 32-row accumulator tiles.  Eight waves, two
// per SIMD (which hides LDS latency and the per-stage barrier better than one
// wave per SIMD): wave w computes a block of VW weight slices (vocabulary part
// w % (NSL / VW)) by RW accumulator tiles (row part w / (NSL / VW)).  Per
// k-step a wave reads VW + RW operand fragments from LDS for VW RW products.
// Moving the operands into LDS is what bounds this kernel: with its MFMAs
// taken out it ran nearly as long (670 against 720 us at 512 rows), and each
// CU moved about 40 GB/s whatever the mix of HBM and L2 bytes.  So the tile
// is chosen for bytes per product: 256 x 256 (65,536 accumulators, 128
// registers per lane) moves (256 + 256) rows per k for the products that
// 128 x 512 serves with (128 + 512).  The weight stream comes from HBM and
// the hidden rows from L2.  Loads complete in
// issue order per wave, so one wave that issued both would wait for the deep
// weight prefetch whenever it needs the next hidden stage.  Hence the issue
// is split by wave: the first half of the waves issue only the weight DMA
// (NWR stage slots, NWR - 1 ahead), the second half only the hidden-row DMA
// (NHR slots, NHR - 1 ahead); each waits on its own count, one barrier per
// stage publishes both, and all waves compute.
//   weight stage j: weight slice t, step s (16 elements) at (NS t + s) KiB,
//     lane l's 16 bytes at + 16 l (the packed fragment order)
//   hidden stage j: row r at r * 2 KS bytes, its 16-byte chunks XOR-swizzled
//     (lm_dma_hofs) so that the 16 rows of a 16-lane read group land on 16
//     distinct bank groups
// hidden row r's 16-byte chunk c in a stage of CH chunks per row: an XOR of
// the chunk index that puts the 16 rows of a 16-lane read group on 16
// distinct bank groups (CH = 4: 64-byte rows; CH = 8: 128-byte rows)
template <int CH>
__device__ __forceinline__ int lm_dma_hofs(int r, int c) {
  if constexpr (CH == 4) return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
  else return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

// wait until the stages issued after the awaited one, at most K of them with
// STEP loads each, are the only ones in flight (k = how many exist)
template <int STEP, int K>
__device__ __forceinline__ void lm_wait_stages(int k) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (k >= K) wait_vmcnt<K * STEP>();
    else lm_wait_stages<STEP, K - 1>(k);
  }
}

template <int NSL, int MT, int KS, int NWR, int NHR, int VW, int RW, bool NT>
__global__ void __launch_bounds__(kWave * (NSL / VW) * (MT / RW), 1) lm_head_dma(LmArgs a) {
  constexpr int NVP = NSL / VW;                 // vocabulary parts (VW 32-row weight slices each)
  constexpr int NRP = MT / RW;                  // row parts (RW accumulator tiles of 32 rows each)
  constexpr int NWV = NVP * NRP;                // waves
  constexpr int ROWS = MT * 32;
  constexpr int NS = KS / 16;                   // MFMA k-steps per stage
  constexpr int CH = KS / 8;                    // 16-byte chunks of a hidden row per stage
  constexpr int WSTAGE = NSL * NS * 1024;       // weight bytes per stage
  constexpr int HSTAGE = ROWS * KS * 2;         // hidden bytes per stage
  constexpr int NIW = NWV / 2;                  // waves issuing each operand
  constexpr int NWI = NSL * NS / NIW;           // weight DMA instructions per issuing wave and stage
  constexpr int NHI = HSTAGE / 1024 / NIW;      // hidden DMA instructions per issuing wave and stage
  static_assert(KS == 32 || KS == 64, "stage of 32 or 64 hidden elements");
  static_assert(NSL % VW == 0 && MT % RW == 0, "wave tiling");
  static_assert(NWI * NIW == NSL * NS && NHI * NIW * 1024 == HSTAGE, "issue shape");
  constexpr int DW = NWR - 1, DH = NHR - 1;    // stages in flight ahead of the one in use
  static_assert(DW >= 1 && DH >= 1, "at least one stage ahead");
  static_assert((DW - 1) * NWI <= 63 && (DH - 1) * NHI <= 63, "wait counts fit vmcnt");
  __shared__ __attribute__((aligned(1024))) char wring[NWR][WSTAGE];
  __shared__ __attribute__((aligned(1024))) char hring[NHR][HSTAGE];
  // the epilogue's merge of the vocabulary parts reuses the weight ring
  // (dead once every wave is past the loop), so the rings may take all of LDS
  static_assert(3 * NRP * NVP * 32 * 4 <= NWR * WSTAGE, "merge arrays fit the weight ring");
  float(*rv)[NVP][32] = reinterpret_cast<float(*)[NVP][32]>(&wring[0][0]);
  int(*ri)[NVP][32] = reinterpret_cast<int(*)[NVP][32]>(&wring[0][0] + NRP * NVP * 32 * 4);
  float(*rs)[NVP][32] = reinterpret_cast<float(*)[NVP][32]>(&wring[0][0] + 2 * NRP * NVP * 32 * 4);

  // block -> (tile, row group): the row groups of one tile share an XCD
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int tile = (local / a.mgroups) * 8 + xcd, mg = local % a.mgroups;
  if (tile >= a.ntiles) return;  // uniform: padding of the tile count to 8

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int vp = wave % NVP, rp = wave / NVP;  // vocabulary part, row part
  const int g = lane >> 5, c32 = lane & 31;
  const int m0 = mg * ROWS;
  const int steps = a.H / 16;
  const int P = a.H / KS;
  const int last32 = (a.V - 1) / 32;

  // weight issue (waves 0 .. NIW - 1): instruction q = NWI w + i covers
  // slice q / NS, step q % NS of the stage; 32-row slices past the padded
  // vocabulary read the last slice (in bounds), their rows are dropped below
  auto issue_w = [&](int j) {
    if (j >= P) return;
    char* dst = wring[j % NWR];
#pragma unroll
    for (int i = 0; i < NWI; ++i) {
      const int q = NWI * wave + i, t = q / NS, s = q % NS;
      const int t32 = min(tile * NSL + t, last32);
      const u32x4* src = a.w + ((size_t)t32 * steps + NS * j + s) * kWave + lane;
      if (NT) dma16_nt(src, dst + q * 1024);
      else dma16(src, dst + q * 1024);
    }
  };
  // hidden issue (waves NIW .. NWV - 1): instruction q = (w - NIW) + NIW k
  // covers rows (64 / CH) q .. + 64 / CH - 1; lane l fills row
  // (64 / CH) q + l / CH, slot l % CH with the chunk the swizzle puts there;
  // rows past M repeat row M - 1 (dropped)
  auto issue_h = [&](int j) {
    if (j >= P) return;
    char* dst = hring[j % NHR];
    const int slot = lane % CH;
#pragma unroll
    for (int k = 0; k < NHI; ++k) {
      const int q = (wave - NIW) + NIW * k;
      const int r = (kWave / CH) * q + lane / CH;
      const int c = (lm_dma_hofs<CH>(r, slot) - r * CH * 16) >> 4;  // the swizzle is an involution
      const int m = min(m0 + r, a.M - 1);
      dma16(a.h + (size_t)m * a.H + (size_t)j * KS + 8 * c, dst + q * 1024);
    }
  };

  f32x16 acc[VW][RW];
#pragma unroll
  for (int v = 0; v < VW; ++v)
#pragma unroll
    for (int k = 0; k < RW; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[v][k][e] = 0.f;

  const bool wissue = wave < NIW;
  if (wissue) {
    for (int u = 0; u < DW; ++u) issue_w(u);
  } else {
    for (int u = 0; u < DH; ++u) issue_h(u);
  }
  for (int j = 0; j < P; ++j) {
    // stage j has landed: the issuing waves wait on their own loads (only
    // later stages may still fly), then one barrier publishes the stage and
    // frees the slots of stage j - 1
    if (wissue) lm_wait_stages<NWI, DW - 1>(min(DW - 1, P - 1 - j));
    else lm_wait_stages<NHI, DH - 1>(min(DH - 1, P - 1 - j));
    barrier_no_fence();
    if (wissue) issue_w(j + DW);
    else issue_h(j + DH);
    // every operand of the stage is read from LDS before the first MFMA:
    // the reads return in issue order, so the MFMAs follow them down the queue
    const char* ws = wring[j % NWR] + vp * VW * NS * 1024 + lane * 16;
    const char* hs = hring[j % NHR];
    u32x4 af[NS][VW], bf[NS][RW];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int v = 0; v < VW; ++v) af[s][v] = *reinterpret_cast<const u32x4*>(ws + (v * NS + s) * 1024);
#pragma unroll
      for (int k = 0; k < RW; ++k)
        bf[s][k] = *reinterpret_cast<const u32x4*>(hs + lm_dma_hofs<CH>((rp * RW + k) * 32 + c32, 2 * s + g));
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int v = 0; v < VW; ++v)
#pragma unroll
        for (int k = 0; k < RW; ++k)
          acc[v][k] = mfma_step(__builtin_bit_cast(bf16x8, af[s][v]), __builtin_bit_cast(bf16x8, bf[s][k]),
                                acc[v][k]);
    __builtin_amdgcn_sched_group_barrier(0x100, NS * (VW + RW), 0);  // the LDS reads first
    __builtin_amdgcn_sched_group_barrier(0x008, NS * VW * RW, 0);    // then the MFMAs
  }
  wait_vmcnt<0>();  // nothing in flight past the loop (the last stages issue nothing)
  if constexpr (NVP > 1) __syncthreads();  // every wave's last ring reads are done

  // argmax of the tile per hidden row, as in lm_head_tiles: accumulator e of
  // acc[v][k] in lane (c32, g) holds vocabulary row nbase_v + 8 (e / 4) +
  // 4 g + e % 4 (nbase_v = first row of the wave's slice v) and hidden row
  // m0 + 32 (rp RW + k) + c32; slices are visited in vocabulary order, so a
  // strict compare keeps the lowest index; the NVP vocabulary parts of a row
  // part merge in LDS
  const int nbase = tile * NSL * 32 + vp * VW * 32;
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < VW; ++v)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int nn = nbase + 32 * v + 8 * (e >> 2) + 4 * g + (e & 3);
        if (nn < a.V && acc[v][k][e] > bv) {
          bv = acc[v][k][e];
          bi = nn;
        }
      }
    lm_keep(bv, bi, __shfl_xor(bv, 32, kWave), __shfl_xor(bi, 32, kWave));
    float se = 0.f;
    if (a.ms) {
#pragma unroll
      for (int v = 0; v < VW; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int nn = nbase + 32 * v + 8 * (e >> 2) + 4 * g + (e & 3);
          se += nn < a.V ? __builtin_amdgcn_exp2f((acc[v][k][e] - bv) * kLog2e) : 0.f;
        }
      se += __shfl_xor(se, 32, kWave);
    }
    if constexpr (NVP > 1) {
      if (g == 0) {
        rv[rp][vp][c32] = bv;
        ri[rp][vp][c32] = bi;
        rs[rp][vp][c32] = se;
      }
      __syncthreads();
    }
    if (vp == 0 && g == 0) {
      const float wmax0 = bv;
#pragma unroll
      for (int w = 1; w < NVP; ++w) lm_keep(bv, bi, rv[rp][w][c32], ri[rp][w][c32]);
      const int m = m0 + (rp * RW + k) * 32 + c32;
      if (m < a.M) {
        a.part[(size_t)m * a.ntiles + tile] =
            ((unsigned long long)lm_order_bits(bv) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)bi);
        if (a.ms) {
          // parts whose rows are all past V hold (-inf, 0) and add nothing
          float tot = se * __builtin_amdgcn_exp2f((wmax0 - bv) * kLog2e);
#pragma unroll
          for (int w = 1; w < NVP; ++w)
            tot += rv[rp][w][c32] == -INFINITY
                       ? 0.f
                       : rs[rp][w][c32] * __builtin_amdgcn_exp2f((rv[rp][w][c32] - bv) * kLog2e);
          a.ms[(size_t)m * a.ntiles + tile] = lm_f32x2{bv, tot};
        }
      }
    }
    if constexpr (NVP > 1) __syncthreads();
  }
}

template <int NSL, int MT, int KS, int NWR, int NHR, int VW, int RW, bool NT>
static orthrus_status lm_launch_dma(LmArgs& a, hipStream_t s) {
  a.ntiles = (a.V + 32 * NSL - 1) / (32 * NSL);
  const long tiles8 = ((long)a.ntiles + 7) / 8 * 8;
  hipLaunchKernelGGL((lm_head_dma<NSL, MT, KS, NWR, NHR, VW, RW, NT>), dim3((unsigned)(tiles8 * a.mgroups)),
                     dim3(kWave * (NSL / VW) * (MT / RW)), 0, s, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

__device__ __forceinline__ unsigned long long lm_max_u64(unsigned long long x, unsigned long long y) {
  return x > y ? x : y;
}

// one work-group per group of R <= 32 rows (one sequence's K rows for the
// accept entry point): 32 threads per row, each loading up to kFinBatch of
// the row's tile keys at once (one memory round trip for the Qwen3 head's
// 1187 tiles), then a max over the row's 32 threads
__global__ void __launch_bounds__(kLmFinThreads) lm_head_finish(LmArgs a) {
  __shared__ int32_t gtok[32];
  __shared__ float gconf[32];
  const int grp = blockIdx.x, tid = threadIdx.x;
  const int i = tid / 32, sub = tid % 32;
  const int m = grp * a.R + i;
  const bool live = i < a.R && m < a.M;
  unsigned long long best = 0;
  if (live) {
    const unsigned long long* keys = a.part + (size_t)m * a.ntiles;
    for (int q0 = 0; q0 < a.ntiles; q0 += 32 * kFinBatch) {
      unsigned long long x[kFinBatch];
#pragma unroll
      for (int j = 0; j < kFinBatch; ++j)  // past the end: the last key again (a max ignores repeats)
        x[j] = keys[min(q0 + sub + 32 * j, a.ntiles - 1)];
#pragma unroll
      for (int j = 0; j < kFinBatch; ++j) best = lm_max_u64(best, x[j]);
    }
  }
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)best, off, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), off, kWave);
    best = lm_max_u64(best, ((unsigned long long)hi << 32) | lo);
  }
  const float vmax = lm_from_order_bits((uint32_t)(best >> 32));
  // denoise: the token's probability 1 / sum_t s_t exp(m_t - M) from the
  // tiles' (max m_t, sum s_t) pairs, merged online (M, the largest m_t, is
  // the greedy token's logit), independently of the keys above
  float conf = 0.f;
  if (a.ms) {
    float pm = -INFINITY, ps = 0.f;
    if (live) {
      const lm_f32x2* pairs = a.ms + (size_t)m * a.ntiles;
      for (int q0 = 0; q0 < a.ntiles; q0 += 32 * kFinPairs) {
        lm_f32x2 y[kFinPairs];
#pragma unroll
        for (int j = 0; j < kFinPairs; ++j) y[j] = pairs[min(q0 + sub + 32 * j, a.ntiles - 1)];
        float bm = pm;
#pragma unroll
        for (int j = 0; j < kFinPairs; ++j) bm = fmaxf(bm, y[j][0]);
        float bs = ps * __builtin_amdgcn_exp2f((pm - bm) * kLog2e);
#pragma unroll
        for (int j = 0; j < kFinPairs; ++j)  // the clamped repeats are dropped here
          bs += q0 + sub + 32 * j < a.ntiles ? y[j][1] * __builtin_amdgcn_exp2f((y[j][0] - bm) * kLog2e) : 0.f;
        pm = bm;
        ps = bs;
      }
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      const float om = __shfl_xor(pm, off, kWave), os = __shfl_xor(ps, off, kWave);
      const float mm = fmaxf(pm, om);
      ps = (pm == -INFINITY ? 0.f : ps * __builtin_amdgcn_exp2f((pm - mm) * kLog2e)) +
           (om == -INFINITY ? 0.f : os * __builtin_amdgcn_exp2f((om - mm) * kLog2e));
      pm = mm;
    }
    conf = 1.f / ps;
  }
  if (live && sub == 0) {
    const int32_t tok = (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
    gtok[i] = tok;
    gconf[i] = conf;
    if (a.tokens) a.tokens[m] = tok;
    if (a.maxv) a.maxv[m] = vmax;
    if (a.conf) a.conf[m] = conf;
  }
  if (!a.drafts && !a.masked) return;
  __syncthreads();
  if (tid >= kWave) return;
  const int lane = tid, K = a.R, b = grp;
  if (a.masked) {
    // low-confidence remasking: the n most confident masked positions are
    // unmasked; rank = masked positions ahead in (confidence desc, position)
    const bool mk = lane < K && a.masked[b * K + lane] != 0;
    const unsigned long long mbits = __ballot(mk);
    int rank = 0;
    const float ci = lane < K ? gconf[lane] : 0.f;
    for (int j = 0; j < K; ++j) {
      const float cj = gconf[j];
      rank += ((mbits >> j) & 1) && (cj > ci || (cj == ci && j < lane));
    }
    if (lane < K) a.masked_out[b * K + lane] = mk && rank >= a.n_unmask[b] ? 1 : 0;
    return;
  }
  bool miss = false;
  int32_t gt = 0;
  if (lane < K) {
    gt = gtok[lane];
    miss = a.drafts[b * K + lane] != gt;
  }
  const unsigned long long mask = __ballot(miss);
  const int acc = mask ? (__ffsll((long long)mask) - 1) : K;
  const int last = acc < K ? acc : K - 1;
  const int nxt = __shfl(gt, last, kWave);
  if (lane == 0) {
    a.accept_len[b] = acc;
    a.next_token[b] = nxt;
  }
}

// packed[t][s][l] = weight[32 t + l % 32][16 s + 8 (l / 32) .. + 8] (zero
// past the vocabulary): one thread per 16-byte fragment
__global__ void __launch_bounds__(256) lm_head_pack(const bf16* w, u32x4* packed, int H, int V, long total) {
  const long f = (long)blockIdx.x * 256 + threadIdx.x;
  if (f >= total) return;
  const int steps = H / 16;
  const int l = (int)(f % kWave);
  const long ts = f / kWave;
  const int s = (int)(ts % steps);
  const long t = ts / steps;
  const long n = 32 * t + l % 32;
  packed[f] = n < V ? ld16(w + n * H + 16 * s + 8 * (l / 32)) : u32x4{0, 0, 0, 0};
}

static size_t lm_packed_bytes(int hidden, int vocab) {
  return (size_t)((vocab + 31) / 32) * 32 * hidden * sizeof(bf16);
}

static bool lm_shape_ok(long rows, int hidden, int vocab) {
  if (rows < 1 || vocab < 1 || hidden < 256 || hidden > 65536 || hidden % 256 != 0) return false;
  const long ntiles = (vocab + (long)kLmTileN - 1) / kLmTileN;
  const long tiles8 = (ntiles + 7) / 8 * 8;
  const long mgroups = (rows + 63) / 64;
  return tiles8 * mgroups * 4 <= 0x7fffffffL && rows <= (1L << 24);
}

static size_t lm_workspace(long rows, int vocab) {
  const long ntiles = (vocab + (long)kLmTileN - 1) / kLmTileN;
  return (size_t)rows * ntiles * sizeof(unsigned long long);
}

// denoise: the keys, then the (max, sum) pairs
static size_t lm_denoise_workspace(long rows, int vocab) { return 2 * lm_workspace(rows, vocab); }

template <int MT, int KP, bool NT>
static orthrus_status lm_launch_tiles(const LmArgs& a, hipStream_t s) {
  const long tiles8 = ((long)a.ntiles + 7) / 8 * 8;
  hipLaunchKernelGGL((lm_head_tiles<MT, KP, NT>), dim3((unsigned)(tiles8 * a.mgroups)), dim3(kLmThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

static orthrus_status lm_run(LmArgs a, hipStream_t s, int finish_groups) {
  a.ntiles = (a.V + kLmTileN - 1) / kLmTileN;
  orthrus_status st;
  // 32 rows: one group, deep phases.  64 rows: one 64-row group with shallow
  // phases (two waves per SIMD fit).  One row group reads every weight byte
  // once: nontemporal loads (measured about 15 % faster at 32 and 64 rows).
  // More rows: the DMA kernel, eight waves (two per SIMD).  128 rows: 128 x
  // 128 tiles in 64-element stages.  256 rows: 256 x 256 tiles.  512 rows:
  // the two 256-row groups of each 256-row weight tile on one XCD; the
  // nontemporal hint measured slightly faster there than ordinary loads
  // (638-643 against 647-650 us), though each group reads the tile.  Measured
  // at the Qwen3-8B head (alternating runs on one box, us per call): 128 x 512
  // tiles with 4 x 2 wave blocks took 697-711 us at 512 rows, 256 x 256 tiles
  // 628-634; at 256 rows 128 x 256 tiles with 2 x 2 blocks took 400-416 us,
  // 256 x 256 tiles 386-390.  128 x 128 tiles at 128 rows measured the same
  // as 256 x 128 (594 work-groups, three rounds).  Earlier: eight waves
  // beat four (275 against 286 us at 128 rows), and squarer wave blocks beat
  // 1 x MT / 2 ones by about 5 %.  Above 512 rows, 256-row groups of one
  // weight tile run on one XCD with ordinary loads, so after the first group
  // the tile mostly comes from L2.
  if (a.M <= 32) {
    a.mgroups = 1;
    st = lm_launch_tiles<1, 256, true>(a, s);
  } else if (a.M <= 64) {
    a.mgroups = 1;
    st = lm_launch_tiles<2, 128, true>(a, s);
  } else if (a.M <= 128) {
    a.mgroups = 1;
    st = lm_launch_dma<4, 4, 64, 6, 3, 1, 2, true>(a, s);
  } else if (a.M <= 256) {
    a.mgroups = 1;
    st = lm_launch_dma<8, 8, 32, 6, 4, 2, 4, true>(a, s);
  } else if (a.M <= 512) {
    a.mgroups = 2;
    st = lm_launch_dma<8, 8, 32, 4, 6, 4, 2, true>(a, s);
  } else {
    a.mgroups = (a.M + 255) / 256;
    st = lm_launch_dma<8, 8, 32, 4, 6, 4, 2, false>(a, s);
  }
  if (st != ORTHRUS_OK) return st;
  hipLaunchKernelGGL(lm_head_finish, dim3((unsigned)finish_groups), dim3(kLmFinThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

static bool lm_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_lm_head_packed_bytes(int32_t hidden_size, int32_t vocab) {
  if (!lm_shape_ok(1, hidden_size, vocab)) return 0;
  return lm_packed_bytes(hidden_size, vocab);
}

extern "C" orthrus_status orthrus_lm_head_pack_weight(const void* weight, void* packed, int32_t hidden_size,
                                                      int32_t vocab, void* stream) {
  if (!weight || !packed) return ORTHRUS_ERR_NULL;
  if (!lm_shape_ok(1, hidden_size, vocab)) return ORTHRUS_ERR_SHAPE;
  if (!lm_aligned(weight) || !lm_aligned(packed)) return ORTHRUS_ERR_SHAPE;
  const long total = (long)lm_packed_bytes(hidden_size, vocab) / 16;
  const long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffL) return ORTHRUS_ERR_SHAPE;
  hipLaunchKernelGGL(lm_head_pack, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const bf16*)weight,
                     (u32x4*)packed, hidden_size, vocab, total);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

extern "C" size_t orthrus_lm_head_workspace_bytes(int32_t rows, int32_t hidden_size, int32_t vocab) {
  if (!lm_shape_ok(rows, hidden_size, vocab)) return 0;
  return lm_workspace(rows, vocab);
}

extern "C" orthrus_status orthrus_lm_head_argmax(const void* hidden, const void* weight, int32_t* tokens,
                                                 float* max_logits, int32_t rows, int32_t hidden_size,
                                                 int32_t vocab, void* workspace, size_t workspace_bytes,
                                                 void* stream) {
  if (!hidden || !weight || !tokens) return ORTHRUS_ERR_NULL;
  if (!lm_shape_ok(rows, hidden_size, vocab)) return ORTHRUS_ERR_SHAPE;
  if (!lm_aligned(hidden) || !lm_aligned(weight)) return ORTHRUS_ERR_SHAPE;
  if (!workspace || workspace_bytes < lm_workspace(rows, vocab) || (reinterpret_cast<uintptr_t>(workspace) & 7))
    return ORTHRUS_ERR_WORKSPACE;
  LmArgs a = {};
  a.h = (const bf16*)hidden;
  a.w = (const u32x4*)weight;
  a.part = (unsigned long long*)workspace;
  a.tokens = tokens;
  a.maxv = max_logits;
  a.M = rows;
  a.H = hidden_size;
  a.V = vocab;
  a.R = 32;
  return lm_run(a, (hipStream_t)stream, (rows + 31) / 32);
}

extern "C" orthrus_status orthrus_lm_head_greedy_accept(const void* hidden, const void* weight,
                                                        const int32_t* draft_tokens, int32_t* accept_len,
                                                        int32_t* next_token, int32_t* ar_tokens, int32_t batch,
                                                        int32_t block_k, int32_t hidden_size, int32_t vocab,
                                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!hidden || !weight || !draft_tokens || !accept_len || !next_token) return ORTHRUS_ERR_NULL;
  if (batch < 1 || block_k < 1 || block_k > 32) return ORTHRUS_ERR_SHAPE;
  const long rows = (long)batch * block_k;
  if (!lm_shape_ok(rows, hidden_size, vocab)) return ORTHRUS_ERR_SHAPE;
  if (!lm_aligned(hidden) || !lm_aligned(weight)) return ORTHRUS_ERR_SHAPE;
  if (!workspace || workspace_bytes < lm_workspace(rows, vocab) || (reinterpret_cast<uintptr_t>(workspace) & 7))
    return ORTHRUS_ERR_WORKSPACE;
  LmArgs a = {};
  a.h = (const bf16*)hidden;
  a.w = (const u32x4*)weight;
  a.part = (unsigned long long*)workspace;
  a.drafts = draft_tokens;
  a.tokens = ar_tokens;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.M = (int)rows;
  a.H = hidden_size;
  a.V = vocab;
  a.R = block_k;
  return lm_run(a, (hipStream_t)stream, batch);
}

extern "C" size_t orthrus_lm_head_denoise_workspace_bytes(int32_t rows, int32_t hidden_size, int32_t vocab) {
  if (!lm_shape_ok(rows, hidden_size, vocab)) return 0;
  return lm_denoise_workspace(rows, vocab);
}

extern "C" orthrus_status orthrus_lm_head_denoise_step(const void* hidden, const void* packed_weight,
                                                       const uint8_t* masked, const int32_t* n_unmask,
                                                       int32_t* tokens, float* confidence, uint8_t* new_masked,
                                                       int32_t batch, int32_t block_k, int32_t hidden_size,
                                                       int32_t vocab, void* workspace, size_t workspace_bytes,
                                                       void* stream) {
  if (!hidden || !packed_weight || !masked || !n_unmask || !tokens || !new_masked) return ORTHRUS_ERR_NULL;
  if (batch < 1 || block_k < 1 || block_k > 32) return ORTHRUS_ERR_SHAPE;
  const long rows = (long)batch * block_k;
  if (!lm_shape_ok(rows, hidden_size, vocab)) return ORTHRUS_ERR_SHAPE;
  if (!lm_aligned(hidden) || !lm_aligned(packed_weight)) return ORTHRUS_ERR_SHAPE;
  if (!workspace || workspace_bytes < lm_denoise_workspace(rows, vocab) ||
      (reinterpret_cast<uintptr_t>(workspace) & 7))
    return ORTHRUS_ERR_WORKSPACE;
  LmArgs a = {};
  a.h = (const bf16*)hidden;
  a.w = (const u32x4*)packed_weight;
  a.part = (unsigned long long*)workspace;
  a.ms = (lm_f32x2*)((char*)workspace + lm_workspace(rows, vocab));
  a.masked = masked;
  a.n_unmask = n_unmask;
  a.tokens = tokens;
  a.conf = confidence;
  a.masked_out = new_masked;
  a.M = (int)rows;
  a.H = hidden_size;
  a.V = vocab;
  a.R = block_k;
  return lm_run(a, (hipStream_t)stream, batch);
}

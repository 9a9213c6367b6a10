// Lossless acceptance of sampled drafts at temperature T > 0 on gfx950: the
// stochastic form of the consensus step of one Orthrus decode step (Orthrus
// explainer, gist.science arXiv 2605.12825, technical summary §2.3; §4 names
// the temperature settings).  For each sequence, rows in order, with
// p = softmax(ar_logits / T) and q = softmax(draft_logits / T) of the row and
// x the draft token: x is accepted when u_accept * q[x] < p[x]; at the first
// rejection the correction token is drawn from max(p - q, 0) by inverse CDF
// with u_resample (from p itself when that residual is zero everywhere).
// The uniforms are inputs.
//
// Three launches, no atomics, every reduction in a fixed order (run-to-run
// bit-identical):
//   sample_stats  one work-group per (row, chunk of 4096 or 8192 logits):
//                 the chunk's max and sum of 2^((x - max) log2e / T) for both
//                 heads, 16-byte nontemporal loads (HBM-bound: 8 bytes per
//                 logit pair);
//   sample_resid  one work-group per (sequence, chunk): all 256 threads first
//                 decide the sequence's rows (8 threads per row merge the
//                 chunk pairs into the row normalisers; a wave ballot finds
//                 the first rejection), then sum max(p - q, 0) over the
//                 chunk of the rejected row; chunk 0 stores the decision;
//   sample_pick   one work-group per sequence: wave scan of the chunk sums
//                 finds the chunk where the running sum passes
//                 u_resample * total, a work-group scan of 16- or 32-logit runs
//                 finds the run, one thread walks the run in index order.
// The kernel boundaries order the passes; the workspace needs no
// initialisation.
#include "orthrus_device.h"
#include "orthrus_host.h"

namespace orthrus {

constexpr int kSampleThreads = 256;
constexpr int kSampleWaves = kSampleThreads / kWave;
// Logits per work-group (a chunk).  A few rows (one or two sequences) take
// 4096: twice the work-groups of 8192 on the chip, measured 24.1 -> 20.2 us
// per call for one sequence of Qwen3 rows.  More rows take 8192, which fills
// the chip already (16 sequences: 4096 measured the same or up to 5 %
// slower).
constexpr int kSmallChunk = 4096, kLargeChunk = 8192;
static int sample_chunk(long rows) { return rows <= 64 ? kSmallChunk : kLargeChunk; }
constexpr int kRowThreads = kSampleThreads / 32;  // threads per block row in the decision

struct SampleArgs {
  const float* ar;      // [B, K, V]
  const float* dr;      // [B, K, V]
  const int32_t* drafts;
  const float* u_acc;   // [B, K]
  const float* u_res;   // [B]
  int32_t* accept_len;
  int32_t* next_token;
  f32x4* stats;         // [B*K, nchunks] (max_p, sum_p, max_q, sum_q)
  f32x4* rowstat;       // [B] (M_p, 1 / Z_p, M_q, 1 / Z_q) of the rejected row
  int32_t* rej;         // [B] rejected row, K when every draft was accepted
  float* rsum;          // [B, nchunks] residual sums of the rejected row
  float c;              // log2(e) / T
  int B, K, V, chunk, nchunks;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// (max m, sum s of 2^((x - m) c)) pairs; -inf logits carry no mass
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2, float c) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * ex2((m - mm) * c) + s2 * ex2((m2 - mm) * c);
  m = mm;
}

__device__ __forceinline__ void ms_add4(float& m, float& s, f32x4 v, float c) {
  const float mm = fmaxf(m, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  if (mm == -INFINITY) return;
  s = s * ex2((m - mm) * c) + ((ex2((v[0] - mm) * c) + ex2((v[1] - mm) * c)) +
                               (ex2((v[2] - mm) * c) + ex2((v[3] - mm) * c)));
  m = mm;
}

// merge the (m, s) pair of the lane that a DPP control selects into this
// lane's; where it selects none (a row outside ROW_MASK) the pair merged is
// (-inf, 0), which leaves this lane's unchanged.  Data movement on the VALU,
// no LDS round trip.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_merge(float& m, float& s, float c) {
  const float m2 = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -INFINITY), __builtin_bit_cast(int, m), CTRL,
                                         ROW_MASK, 0xf, false));
  const float s2 = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), CTRL, ROW_MASK, 0xf, false));
  ms_merge(m, s, m2, s2, c);
}

// both pairs reduced over each aligned group of 8 lanes, the result in every
// lane of the group: partners at lane ^ 1, lane ^ 2, then the mirror image in
// the group
__device__ __forceinline__ void merge8(float& mp, float& sp, float& mq, float& sq, float c) {
  dpp_merge<0xb1, 0xf>(mp, sp, c);   // quad_perm [1, 0, 3, 2]
  dpp_merge<0xb1, 0xf>(mq, sq, c);
  dpp_merge<0x4e, 0xf>(mp, sp, c);   // quad_perm [2, 3, 0, 1]
  dpp_merge<0x4e, 0xf>(mq, sq, c);
  dpp_merge<0x141, 0xf>(mp, sp, c);  // row_half_mirror
  dpp_merge<0x141, 0xf>(mq, sq, c);
}

// both pairs reduced over the wave, the result in lane 63: groups of 8, the
// 16-lane rows through their mirror image, then the row results through the
// broadcasts of lanes 15 and 31
__device__ __forceinline__ void merge_wave(float& mp, float& sp, float& mq, float& sq, float c) {
  merge8(mp, sp, mq, sq, c);
  dpp_merge<0x140, 0xf>(mp, sp, c);  // row_mirror
  dpp_merge<0x140, 0xf>(mq, sq, c);
  dpp_merge<0x142, 0xa>(mp, sp, c);  // row_bcast:15 -> rows 1, 3
  dpp_merge<0x142, 0xa>(mq, sq, c);
  dpp_merge<0x143, 0xc>(mp, sp, c);  // row_bcast:31 -> rows 2, 3
  dpp_merge<0x143, 0xc>(mq, sq, c);
}

// [begin, end) of one row as a scalar head up to 16-byte alignment (< 4
// logits), whole 16-byte vectors (at most CH / 4 / kSampleThreads per
// thread for a chunk of CH logits) and a scalar tail (< 4 logits)
struct Split16 {
  int head_end, nvec, tail;
};

__device__ __forceinline__ Split16 split16(const float* x, int begin, int end) {
  const int mis = (int)((reinterpret_cast<uintptr_t>(x + begin) >> 2) & 3);
  Split16 sp;
  sp.head_end = min(end, begin + ((4 - mis) & 3));
  sp.nvec = (end - sp.head_end) >> 2;
  sp.tail = sp.head_end + 4 * sp.nvec;
  return sp;
}

// Each kernel's leading scalar arguments repeat the fields its first loads
// depend on; they are preloaded into SGPRs when a wave starts, so the loads
// do not wait for a kernel-argument load.
template <int CH>
__global__ void __launch_bounds__(kSampleThreads)
    sample_stats(const float* pre_ar, const float* pre_dr, int pre_V, int pre_nchunks, SampleArgs a) {
  constexpr int kVecPerThread = CH / 4 / kSampleThreads;
  __shared__ f32x4 red[kSampleWaves];
  const int row = blockIdx.x / pre_nchunks, ck = blockIdx.x % pre_nchunks;
  const int tid = threadIdx.x;
  const int begin = ck * a.chunk, end = min(begin + a.chunk, pre_V);
  const float* xp = pre_ar + (size_t)row * pre_V;
  const float* xq = pre_dr + (size_t)row * pre_V;
  const Split16 sp = split16(xp, begin, end), sq_ = split16(xq, begin, end);
  const f32x4* pv = reinterpret_cast<const f32x4*>(xp + sp.head_end);
  const f32x4* qv = reinterpret_cast<const f32x4*>(xq + sq_.head_end);
  const f32x4 none = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  // every load of both heads is issued before any is consumed
  f32x4 vp[kVecPerThread], vq[kVecPerThread];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    const int k = tid + kSampleThreads * j;
    vp[j] = k < sp.nvec ? __builtin_nontemporal_load(pv + k) : none;
    vq[j] = k < sq_.nvec ? __builtin_nontemporal_load(qv + k) : none;
  }
  const int hi_ = begin + tid, ti = sp.tail + tid, tq = sq_.tail + tid, hq = begin + tid;
  const float ph = hi_ < sp.head_end ? xp[hi_] : -INFINITY, pt = ti < end ? xp[ti] : -INFINITY;
  const float qh = hq < sq_.head_end ? xq[hq] : -INFINITY, qt = tq < end ? xq[tq] : -INFINITY;
  float mp = -INFINITY, sp_ = 0.f, mq = -INFINITY, sq = 0.f;
  ms_add4(mp, sp_, f32x4{ph, pt, -INFINITY, -INFINITY}, a.c);
  ms_add4(mq, sq, f32x4{qh, qt, -INFINITY, -INFINITY}, a.c);
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    ms_add4(mp, sp_, vp[j], a.c);
    ms_add4(mq, sq, vq[j], a.c);
  }
  merge_wave(mp, sp_, mq, sq, a.c);
  if (tid % kWave == kWave - 1) red[tid / kWave] = f32x4{mp, sp_, mq, sq};
  __syncthreads();
  if (tid == 0) {
    mp = red[0][0], sp_ = red[0][1], mq = red[0][2], sq = red[0][3];
#pragma unroll
    for (int w = 1; w < kSampleWaves; ++w) {
      ms_merge(mp, sp_, red[w][0], red[w][1], a.c);
      ms_merge(mq, sq, red[w][2], red[w][3], a.c);
    }
    a.stats[(size_t)row * pre_nchunks + ck] = f32x4{mp, sp_, mq, sq};
  }
}

// probability of logit x from the row's (max m, reciprocal of the sum rz).
// The product is rounded on its own (never contracted into a later p - q),
// so equal heads give p - q == 0 exactly and a zero residual.
__device__ __forceinline__ float prob(float x, float m, float rz, float c) {
#pragma clang fp contract(off)
  return ex2((x - m) * c) * rz;
}

// row normalisers (M_p, Z_p, M_q, Z_q) -> (M_p, 1 / Z_p, M_q, 1 / Z_q)
__device__ __forceinline__ f32x4 recip_sums(f32x4 n) { return f32x4{n[0], 1.f / n[1], n[2], 1.f / n[3]}; }

__device__ __forceinline__ float resid(const float* xp, const float* xq, const f32x4& n, float c, bool use_p,
                                       int v) {
  const float p = prob(xp[v], n[0], n[1], c);
  return use_p ? p : fmaxf(p - prob(xq[v], n[2], n[3], c), 0.f);
}

__device__ __forceinline__ float resid4(f32x4 xp, f32x4 xq, const f32x4& n, float c) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += fmaxf(prob(xp[j], n[0], n[1], c) - prob(xq[j], n[2], n[3], c), 0.f);
  return s;
}

// x plus the value of the lane that a DPP control selects (0 where it
// selects none): data movement on the VALU, no LDS round trip
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, BOUND_ZERO);
  return x + __builtin_bit_cast(float, y);
}

// inclusive prefix sum over the wave in a fixed order: shifts by 1, 2, 4, 8
// within each 16-lane row, then the row totals through the broadcasts of
// lanes 15 and 31
__device__ __forceinline__ float wave_scan(float x, int) {
  x = dpp_add<0x111, 0xf, true>(x);   // row_shr:1
  x = dpp_add<0x112, 0xf, true>(x);   // row_shr:2
  x = dpp_add<0x114, 0xf, true>(x);   // row_shr:4
  x = dpp_add<0x118, 0xf, true>(x);   // row_shr:8
  x = dpp_add<0x142, 0xa, false>(x);  // row_bcast:15 -> rows 1, 3
  x = dpp_add<0x143, 0xc, false>(x);  // row_bcast:31 -> rows 2, 3
  return x;
}

// the wave's total in every lane
__device__ __forceinline__ float wave_sum(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_scan(x, 0)), kWave - 1));
}

__global__ void __launch_bounds__(kSampleThreads)
    sample_resid(const f32x4* pre_stats, const int32_t* pre_drafts, const float* pre_ar, const float* pre_dr,
                 int pre_K, int pre_nchunks, int pre_V, SampleArgs a) {
  __shared__ f32x4 nrm[32];
  __shared__ int ok[32];
  __shared__ int rej_s;
  __shared__ float red[kSampleWaves];
  const int b = blockIdx.x / pre_nchunks, ck = blockIdx.x % pre_nchunks;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // decision: kRowThreads threads per row merge its chunk pairs (chunks
  // sub, sub + 8, ...), a DPP merge over the 8 gives the normalisers
  {
    const int i = tid / kRowThreads, sub = tid % kRowThreads;
    const bool live = i < pre_K;
    const int row = b * pre_K + i;
    int x = 0;
    float xa = 0.f, xd = 0.f;
    bool in = false;
    if (live && sub == 0) {
      x = pre_drafts[row];
      in = x >= 0 && x < pre_V;  // a draft outside the vocabulary is rejected
      if (in) {
        xa = pre_ar[(size_t)row * pre_V + x];
        xd = pre_dr[(size_t)row * pre_V + x];
      }
    }
    float mp = -INFINITY, sp = 0.f, mq = -INFINITY, sq = 0.f;
    if (live)
      for (int q = sub; q < pre_nchunks; q += kRowThreads) {
        const f32x4 t = pre_stats[(size_t)row * pre_nchunks + q];
        ms_merge(mp, sp, t[0], t[1], a.c);
        ms_merge(mq, sq, t[2], t[3], a.c);
      }
    static_assert(kRowThreads == 8, "the decision merges groups of 8 lanes");
    merge8(mp, sp, mq, sq, a.c);
    if (live && sub == 0) {
      const f32x4 nr = recip_sums(f32x4{mp, sp, mq, sq});
      const float px = in ? prob(xa, nr[0], nr[1], a.c) : 0.f;
      const float qx = in ? prob(xd, nr[2], nr[3], a.c) : 0.f;
      ok[i] = a.u_acc[row] * qx < px;
      nrm[i] = nr;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const unsigned long long mask = __ballot(lane < pre_K && !ok[lane]);
    if (lane == 0) rej_s = mask ? (__ffsll((long long)mask) - 1) : pre_K;
  }
  __syncthreads();
  const int r = rej_s;
  if (ck == 0 && tid == 0) {
    a.accept_len[b] = r;
    a.rej[b] = r;
    if (r == pre_K) a.next_token[b] = pre_drafts[b * pre_K + pre_K - 1];
    else a.rowstat[b] = nrm[r];
  }
  if (r == pre_K) return;  // uniform: every draft accepted

  const f32x4 n = nrm[r];
  const size_t off = (size_t)(b * pre_K + r) * pre_V;
  const float* xp = pre_ar + off;
  const float* xq = pre_dr + off;
  const int begin = ck * a.chunk, end = min(begin + a.chunk, pre_V);
  float s = 0.f;
  if (((reinterpret_cast<uintptr_t>(xp) ^ reinterpret_cast<uintptr_t>(xq)) & 15) == 0) {
    const int mis = (int)((reinterpret_cast<uintptr_t>(xp + begin) >> 2) & 3);
    const int head_end = min(end, begin + ((4 - mis) & 3));
    for (int v = begin + tid; v < head_end; v += kSampleThreads) s += resid(xp, xq, n, a.c, false, v);
    const int nvec = (end - head_end) >> 2;
    const f32x4* pv = reinterpret_cast<const f32x4*>(xp + head_end);
    const f32x4* qv = reinterpret_cast<const f32x4*>(xq + head_end);
#pragma unroll 4
    for (int k = tid; k < nvec; k += kSampleThreads) s += resid4(pv[k], qv[k], n, a.c);
    for (int v = head_end + 4 * nvec + tid; v < end; v += kSampleThreads) s += resid(xp, xq, n, a.c, false, v);
  } else {
    for (int v = begin + tid; v < end; v += kSampleThreads) s += resid(xp, xq, n, a.c, false, v);
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    float t = red[0];
#pragma unroll
    for (int w = 1; w < kSampleWaves; ++w) t += red[w];
    a.rsum[(size_t)b * pre_nchunks + ck] = t;
  }
}


// mass of chunk k of the rejected row: the residual sum, or (when the
// residual is zero everywhere) p's mass from the chunk pair
__device__ __forceinline__ float chunk_mass(const SampleArgs& a, int b, int r, const f32x4& n, bool use_p, int k) {
  if (!use_p) return a.rsum[(size_t)b * a.nchunks + k];
  const f32x4 t = a.stats[(size_t)(b * a.K + r) * a.nchunks + k];
  return t[0] == -INFINITY ? 0.f : t[1] * ex2((t[0] - n[0]) * a.c) * n[1];
}

template <int CH>
__global__ void __launch_bounds__(kSampleThreads)
    sample_pick(const int32_t* pre_rej, const f32x4* pre_rowstat, const float* pre_rsum, const float* pre_ures,
                int pre_nchunks, SampleArgs a) {
  constexpr int kRun = CH / kSampleThreads;  // logits per thread
  __shared__ float wtot[kSampleWaves];
  __shared__ int wpick[kSampleWaves];
  __shared__ int chosen_s;
  __shared__ float target_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  // the decision, the normalisers and the first 64 chunk sums are loaded
  // together (rowstat is only used when a row was rejected)
  const int r = pre_rej[b];
  const f32x4 n = pre_rowstat[b];
  float cs0 = (wave == 0 && lane < pre_nchunks) ? pre_rsum[(size_t)b * pre_nchunks + lane] : 0.f;
  const float u = pre_ures[b];
  if (r >= a.K) return;  // every draft accepted: next_token is already written

  if (wave == 0) {
    // total residual mass (lane-strided, then a wave sum)
    float t = cs0;
    for (int k = lane + kWave; k < pre_nchunks; k += kWave) t += pre_rsum[(size_t)b * pre_nchunks + k];
    t = wave_sum(t);
    const bool use_p = !(t > 0.f);
    if (use_p) {
      cs0 = lane < pre_nchunks ? chunk_mass(a, b, r, n, true, lane) : 0.f;
      t = cs0;
      for (int k = lane + kWave; k < pre_nchunks; k += kWave) t += chunk_mass(a, b, r, n, true, k);
      t = wave_sum(t);
    }
    const float target = u * t;
    // first chunk whose running sum passes the target; the last chunk with
    // mass if rounding leaves the target at or past the end
    float carry = 0.f;
    int ck = -1, last = -1;
    float run_ck = 0.f, run_last = 0.f;
    for (int k0 = 0; k0 < pre_nchunks && ck < 0; k0 += kWave) {
      const int k = k0 + lane;
      const float cs = k0 == 0 ? cs0 : (k < pre_nchunks ? chunk_mass(a, b, r, n, use_p, k) : 0.f);
      const float incl = carry + wave_scan(cs, lane);
      const unsigned long long hit = __ballot(cs > 0.f && incl > target);
      const unsigned long long mass = __ballot(cs > 0.f);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        ck = k0 + l;
        run_ck = __shfl(incl - cs, l, kWave);
      } else if (mass) {
        const int l = 63 - __clzll((long long)mass);
        last = k0 + l;
        run_last = __shfl(incl - cs, l, kWave);
      }
      carry = __shfl(incl, kWave - 1, kWave);
    }
    if (ck < 0) {
      ck = last < 0 ? 0 : last;
      run_ck = run_last;
    }
    if (lane == 0) {
      chosen_s = use_p ? -1 - ck : ck;  // sign carries the mode
      target_s = target - run_ck;       // mass still to pass inside the chunk
    }
  }
  __syncthreads();
  const bool use_p = chosen_s < 0;
  const int ck = use_p ? -1 - chosen_s : chosen_s;
  const float base = target_s;
  const size_t off = (size_t)(b * a.K + r) * a.V;
  const float* xp = a.ar + off;
  const float* xq = a.dr + off;
  const int begin = ck * a.chunk, end = min(begin + a.chunk, a.V);
  const int lo = min(begin + tid * kRun, end), hi = min(lo + kRun, end);
  // the thread's run of logits, all loads in flight, then its masses kept
  // in registers for the walk
  float xa[kRun], xd[kRun], rv[kRun];
  if (hi - lo == kRun && ((reinterpret_cast<uintptr_t>(xp + lo) | reinterpret_cast<uintptr_t>(xq + lo)) & 15) == 0) {
    // a whole, 16-byte aligned run (any vocabulary divisible by 4): 16-byte loads
    const f32x4* pv = reinterpret_cast<const f32x4*>(xp + lo);
    const f32x4* qv = reinterpret_cast<const f32x4*>(xq + lo);
    f32x4 va[kRun / 4], vd[kRun / 4];
#pragma unroll
    for (int k = 0; k < kRun / 4; ++k) {
      va[k] = pv[k];
      vd[k] = qv[k];
    }
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      xa[j] = va[j / 4][j % 4];
      xd[j] = vd[j / 4][j % 4];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      xa[j] = lo + j < hi ? xp[lo + j] : -INFINITY;
      xd[j] = lo + j < hi ? xq[lo + j] : -INFINITY;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    const float p = prob(xa[j], n[0], n[1], a.c);
    rv[j] = lo + j >= hi ? 0.f : (use_p ? p : fmaxf(p - prob(xd[j], n[2], n[3], a.c), 0.f));
    s += rv[j];
  }
  // exclusive start of each thread's run: wave scan plus the earlier waves
  const float incl_w = wave_scan(s, lane);
  if (lane == kWave - 1) wtot[wave] = incl_w;
  __syncthreads();
  float before = 0.f;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  const float start = before + (incl_w - s);
  const unsigned long long hit = __ballot(s > 0.f && start + s > base);
  const unsigned long long mass = __ballot(s > 0.f);
  if (lane == 0)
    wpick[wave] = hit ? wave * kWave + (__ffsll((long long)hit) - 1)
                      : (mass ? -2 - (wave * kWave + 63 - __clzll((long long)mass)) : -1);
  __syncthreads();
  int pick = -1, last = -1;
  for (int w = 0; w < kSampleWaves; ++w) {
    const int p = wpick[w];
    if (p >= 0) {
      pick = p;
      break;
    }
    if (p <= -2) last = -2 - p;
  }
  const bool past_end = pick < 0;
  if (past_end) pick = last;
  if (pick < 0) {  // no mass in the chunk (cannot happen for a chosen chunk)
    if (tid == 0) a.next_token[b] = begin;
    return;
  }
  if (tid != pick) return;
  // walk the run in index order: the first logit whose running sum passes
  // the target, else (rounding left the target at or past the run's mass)
  // the last logit with mass
  float run = start;
  int found = -1, v_last = lo;
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    if (found < 0 && rv[j] > 0.f) {
      v_last = lo + j;
      if (!past_end && run + rv[j] > base) found = lo + j;
    }
    run += rv[j];
  }
  a.next_token[b] = found >= 0 ? found : v_last;
}

static size_t sample_workspace(int batch, int block_k, int vocab, int* nchunks, size_t* off) {
  const int chunk = sample_chunk((long)batch * block_k);
  *nchunks = (vocab + chunk - 1) / chunk;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)batch * block_k;
  off[0] = 0;                                             // stats
  off[1] = up(rows * *nchunks * sizeof(f32x4));           // rowstat
  off[2] = off[1] + up((size_t)batch * sizeof(f32x4));    // rej
  off[3] = off[2] + up((size_t)batch * sizeof(int32_t));  // rsum
  return off[3] + up((size_t)batch * *nchunks * sizeof(float));
}

static bool sample_shape_ok(int batch, int block_k, int vocab) {
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return false;
  const long nchunks = (vocab + (long)kSmallChunk - 1) / kSmallChunk;  // at most
  return (long)batch * block_k * nchunks <= 0x7fffffffL;
}

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_sample_accept_workspace_bytes(int32_t batch, int32_t block_k, int32_t vocab) {
  if (!sample_shape_ok(batch, block_k, vocab)) return 0;
  int nchunks;
  size_t off[4];
  return sample_workspace(batch, block_k, vocab, &nchunks, off);
}

extern "C" orthrus_status orthrus_sample_accept(const float* ar_logits, const float* draft_logits,
                                                const int32_t* draft_tokens, const float* u_accept,
                                                const float* u_resample, float temperature, int32_t* accept_len,
                                                int32_t* next_token, int32_t batch, int32_t block_k, int32_t vocab,
                                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!ar_logits || !draft_logits || !draft_tokens || !u_accept || !u_resample || !accept_len || !next_token)
    return ORTHRUS_ERR_NULL;
  if (!sample_shape_ok(batch, block_k, vocab)) return ORTHRUS_ERR_SHAPE;
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return ORTHRUS_ERR_SHAPE;
  const float c = 1.4426950408889634f / temperature;
  if (!(c < INFINITY)) return ORTHRUS_ERR_SHAPE;  // T so small that log2(e) / T overflows
  int nchunks;
  size_t off[4];
  const size_t need = sample_workspace(batch, block_k, vocab, &nchunks, off);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15))
    return ORTHRUS_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  SampleArgs a;
  a.ar = ar_logits;
  a.dr = draft_logits;
  a.drafts = draft_tokens;
  a.u_acc = u_accept;
  a.u_res = u_resample;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.stats = (f32x4*)(ws + off[0]);
  a.rowstat = (f32x4*)(ws + off[1]);
  a.rej = (int32_t*)(ws + off[2]);
  a.rsum = (float*)(ws + off[3]);
  a.c = c;
  a.B = batch;
  a.K = block_k;
  a.V = vocab;
  a.chunk = sample_chunk((long)batch * block_k);
  a.nchunks = nchunks;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid_stats((unsigned)((long)batch * block_k * nchunks));
  if (a.chunk == kSmallChunk)
    hipLaunchKernelGGL(sample_stats<kSmallChunk>, grid_stats, dim3(kSampleThreads), 0, s, a.ar, a.dr, a.V,
                       a.nchunks, a);
  else
    hipLaunchKernelGGL(sample_stats<kLargeChunk>, grid_stats, dim3(kSampleThreads), 0, s, a.ar, a.dr, a.V,
                       a.nchunks, a);
  if (hipGetLastError() != hipSuccess) return ORTHRUS_ERR_LAUNCH;
  hipLaunchKernelGGL(sample_resid, dim3((unsigned)((long)batch * nchunks)), dim3(kSampleThreads), 0, s, a.stats,
                     a.drafts, a.ar, a.dr, a.K, a.nchunks, a.V, a);
  if (hipGetLastError() != hipSuccess) return ORTHRUS_ERR_LAUNCH;
  if (a.chunk == kSmallChunk)
    hipLaunchKernelGGL(sample_pick<kSmallChunk>, dim3((unsigned)batch), dim3(kSampleThreads), 0, s, a.rej, a.rowstat,
                       a.rsum, a.u_res, a.nchunks, a);
  else
    hipLaunchKernelGGL(sample_pick<kLargeChunk>, dim3((unsigned)batch), dim3(kSampleThreads), 0, s, a.rej, a.rowstat,
                       a.rsum, a.u_res, a.nchunks, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

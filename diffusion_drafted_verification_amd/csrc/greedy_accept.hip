// Greedy consensus of one Orthrus decode step on gfx950 (Orthrus explainer,
// gist.science arXiv 2605.12825, technical summary §2.3): per block row the
// AR head's greedy token (argmax over the vocabulary, lowest index on ties),
// then the longest prefix of drafts that equals those tokens.
//
// Two launches.  argmax_chunks: each work-group scans one contiguous chunk
// (4096 or 8192 logits) of one logits row with 16-byte nontemporal loads
// (the scan is HBM-bound: 4 bytes per logit) and reduces its (value,
// index) candidates, as 64-bit keys (order-preserving value bits << 32 |
// ~index: the larger key is the larger value, then the lower index), with a
// DPP max-scan across the wave and a max over the waves in LDS; the chunk's
// key goes to the workspace.  accept_rows: one work-group per
// sequence reduces each row's chunk keys to the greedy token, then compares
// the K tokens with the drafts (wave ballot: first mismatch) and writes
// accept_len / next_token / ar_tokens.  The kernel boundary orders the two
// passes: no atomics, no fences, and the workspace needs no initialisation.
#include "orthrus_device.h"
#include "orthrus_host.h"

namespace orthrus {

constexpr int kArgmaxThreads = 256;

struct AcceptArgs {
  const float* logits;
  const int32_t* drafts;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t* ar_tokens;
  unsigned long long* part;   // [B*K, nchunks] chunk keys
  int B, K, V, chunk, nchunks;
};

__device__ __forceinline__ uint32_t order_bits(float v) {
  if (v == 0.f) v = 0.f;  // -0.0 and +0.0 are equal: give them one encoding
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void keep_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// max of k and the key of the lane that a DPP control selects (key 0,
// below every real key, where it selects none)
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ unsigned long long dpp_max_u64(unsigned long long k) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)k, CTRL, ROW_MASK, 0xf, BOUND_ZERO);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(k >> 32), CTRL, ROW_MASK, 0xf, BOUND_ZERO);
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o > k ? o : k;
}

// the wave's largest key, in every lane: a max-scan on the DPP paths (shifts
// by 1, 2, 4, 8 within each 16-lane row, then the row maxima through the
// broadcasts of lanes 15 and 31), read from the last lane
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k) {
  k = dpp_max_u64<0x111, 0xf, true>(k);   // row_shr:1
  k = dpp_max_u64<0x112, 0xf, true>(k);   // row_shr:2
  k = dpp_max_u64<0x114, 0xf, true>(k);   // row_shr:4
  k = dpp_max_u64<0x118, 0xf, true>(k);   // row_shr:8
  k = dpp_max_u64<0x142, 0xa, false>(k);  // row_bcast:15 -> rows 1, 3
  k = dpp_max_u64<0x143, 0xc, false>(k);  // row_bcast:31 -> rows 2, 3
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, kWave - 1);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), kWave - 1);
  return ((unsigned long long)hi << 32) | lo;
}

// the key of a (value, index) candidate: a larger key is a larger value, then
// a lower index (the empty candidate, -inf at index 2^31 - 1, stays above 0)
__device__ __forceinline__ unsigned long long cand_key(float v, int i) {
  return ((unsigned long long)order_bits(v) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

// The leading scalar arguments repeat the fields the first loads depend on;
// they are preloaded into SGPRs when a wave starts (the build asks for the
// first four), so the scan does not wait for a kernel-argument load.
__global__ void __launch_bounds__(kArgmaxThreads)
    argmax_chunks(const float* pre_logits, int pre_V, int pre_chunk, int pre_nchunks, AcceptArgs a) {
  __shared__ unsigned long long wkey[kArgmaxThreads / kWave];

  const int row = blockIdx.x / pre_nchunks;  // b * K + i
  const int ck = blockIdx.x % pre_nchunks;
  const int tid = threadIdx.x;
  const int begin = ck * pre_chunk;
  const int end = min(begin + pre_chunk, pre_V);
  const float* x = pre_logits + (size_t)row * pre_V;

  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // scalar head up to 16-byte alignment, vector body, scalar tail; every
  // thread visits its indices in increasing order
  const int mis = (int)((reinterpret_cast<uintptr_t>(x + begin) >> 2) & 3);
  const int head_end = min(end, begin + ((4 - mis) & 3));
  for (int idx = begin + tid; idx < head_end; idx += kArgmaxThreads) keep_better(bv, bi, x[idx], idx);
  const int nvec = (end - head_end) >> 2;
  const f32x4* xv = reinterpret_cast<const f32x4*>(x + head_end);
#pragma unroll 8
  for (int k = tid; k < nvec; k += kArgmaxThreads) {
    const f32x4 v = __builtin_nontemporal_load(xv + k);
    const int idx = head_end + 4 * k;
    keep_better(bv, bi, v[0], idx);
    keep_better(bv, bi, v[1], idx + 1);
    keep_better(bv, bi, v[2], idx + 2);
    keep_better(bv, bi, v[3], idx + 3);
  }
  for (int idx = head_end + 4 * nvec + tid; idx < end; idx += kArgmaxThreads) keep_better(bv, bi, x[idx], idx);

  const unsigned long long wk = wave_max_u64(cand_key(bv, bi));
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane == 0) wkey[wave] = wk;
  __syncthreads();
  if (tid == 0) {
    unsigned long long k = wkey[0];
#pragma unroll
    for (int w = 1; w < kArgmaxThreads / kWave; ++w) k = wkey[w] > k ? wkey[w] : k;
    a.part[(size_t)row * pre_nchunks + ck] = k;
  }
}

// One work-group per sequence: wave w reduces rows w, w + 4, ... (each row's
// chunk keys, one per lane; the first 64 keys of all its rows are loaded
// before any is reduced), then wave 0 scans the K greedy tokens.
constexpr int kAcceptThreads = 256;
constexpr int kAcceptWaves = kAcceptThreads / kWave;
constexpr int kRowsPerWave = (32 + kAcceptWaves - 1) / kAcceptWaves;

__global__ void __launch_bounds__(kAcceptThreads)
    accept_rows(const unsigned long long* pre_part, int pre_K, int pre_nchunks, AcceptArgs a) {
  __shared__ int32_t gtok[32];
  const int b = blockIdx.x;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  unsigned long long best[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int i = wave + kAcceptWaves * j;
    best[j] = (i < pre_K && lane < pre_nchunks) ? pre_part[(size_t)(b * pre_K + i) * pre_nchunks + lane] : 0ull;
  }
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int i = wave + kAcceptWaves * j;
    if (i >= pre_K) break;
    const unsigned long long* keys = pre_part + (size_t)(b * pre_K + i) * pre_nchunks;
    for (int q = lane + kWave; q < pre_nchunks; q += kWave) best[j] = keys[q] > best[j] ? keys[q] : best[j];
    const unsigned long long m = wave_max_u64(best[j]);
    if (lane == 0) gtok[i] = (int32_t)(0xffffffffu - (uint32_t)(m & 0xffffffffu));
  }
  __syncthreads();
  if (wave != 0) return;
  int32_t gt = 0;
  bool miss = false;
  if (lane < pre_K) {
    gt = gtok[lane];
    miss = a.drafts[b * pre_K + lane] != gt;
    if (a.ar_tokens) a.ar_tokens[b * pre_K + lane] = gt;
  }
  const unsigned long long mask = __ballot(miss);
  const int acc = mask ? (__ffsll((long long)mask) - 1) : pre_K;
  const int last = acc < pre_K ? acc : pre_K - 1;
  const int nxt = __shfl(gt, last, kWave);
  if (lane == 0) {
    a.accept_len[b] = acc;
    a.next_token[b] = nxt;
  }
}

// Logits per work-group.  A few rows (one or two sequences) take 4096 (16
// KiB, 16 values per thread in flight): twice the work-groups on the chip,
// measured 10.2 -> 8.4 us for one sequence of Qwen3 rows (32 x 151,936).
// More rows take 8192, which fills the chip already (16 sequences: 52 us
// against 55 us with 4096).
static int accept_chunk(long rows, int vocab) {
  const int c = rows <= 64 ? 4096 : 8192;
  return vocab < c ? vocab : c;
}

static size_t accept_workspace(int batch, int block_k, int vocab, int* chunk, int* nchunks) {
  *chunk = accept_chunk((long)batch * block_k, vocab);
  *nchunks = (vocab + *chunk - 1) / *chunk;
  return (size_t)batch * block_k * *nchunks * sizeof(unsigned long long);
}

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_greedy_accept_workspace_bytes(int32_t batch, int32_t block_k, int32_t vocab) {
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return 0;
  int chunk, nchunks;
  return accept_workspace(batch, block_k, vocab, &chunk, &nchunks);
}

extern "C" orthrus_status orthrus_greedy_accept(const float* ar_logits, const int32_t* draft_tokens,
                                                int32_t* accept_len, int32_t* next_token, int32_t* ar_tokens,
                                                int32_t batch, int32_t block_k, int32_t vocab, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  if (!ar_logits || !draft_tokens || !accept_len || !next_token) return ORTHRUS_ERR_NULL;
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return ORTHRUS_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(ar_logits) & 3) return ORTHRUS_ERR_SHAPE;
  int chunk, nchunks;
  const size_t need = accept_workspace(batch, block_k, vocab, &chunk, &nchunks);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7))
    return ORTHRUS_ERR_WORKSPACE;
  const long grid = (long)batch * block_k * nchunks;
  if (grid > 0x7fffffffL) return ORTHRUS_ERR_SHAPE;
  AcceptArgs a;
  a.logits = ar_logits;
  a.drafts = draft_tokens;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.ar_tokens = ar_tokens;
  a.part = (unsigned long long*)workspace;
  a.B = batch;
  a.K = block_k;
  a.V = vocab;
  a.chunk = chunk;
  a.nchunks = nchunks;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(argmax_chunks, dim3((unsigned)grid), dim3(kArgmaxThreads), 0, s, a.logits, a.V, a.chunk,
                     a.nchunks, a);
  if (hipGetLastError() != hipSuccess) return ORTHRUS_ERR_LAUNCH;
  hipLaunchKernelGGL(accept_rows, dim3((unsigned)batch), dim3(kAcceptThreads), 0, s, a.part, a.K, a.nchunks, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

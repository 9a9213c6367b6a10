// Greedy consensus of one Orthrus decode step on gfx950 (Orthrus explainer,
// gist.science arXiv 2605.12825, technical summary §2.3): per block row the
// AR head's greedy token (argmax over the vocabulary, lowest index on ties),
// then the longest prefix of drafts that equals those tokens.
//
// One launch.  Each work-group scans one contiguous chunk of one logits row
// with 16-byte loads (the scan is HBM-bound: 4 bytes per logit), reduces
// (value, index) pairs across the wave with xor shuffles and across waves in
// LDS, and folds its winner into the row's 64-bit slot with one atomic max on
// (order-preserving value bits << 32 | ~index), which makes ties resolve to the
// lowest index.  The last work-group to finish a sequence (ticket counter)
// reads the K slots, takes the first draft mismatch with a wave ballot, writes
// accept_len / next_token / ar_tokens and clears the slots and the counter, so
// the workspace is zero again for the next call.
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
  unsigned long long* slots;  // [B*K]
  unsigned int* counters;     // [B]
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

__global__ void __launch_bounds__(kArgmaxThreads) argmax_accept(AcceptArgs a) {
  __shared__ float wv[kArgmaxThreads / kWave];
  __shared__ int wi[kArgmaxThreads / kWave];
  __shared__ unsigned int ticket;

  const int row = blockIdx.x / a.nchunks;  // b * K + i
  const int ck = blockIdx.x % a.nchunks;
  const int b = row / a.K;
  const int tid = threadIdx.x;
  const int begin = ck * a.chunk;
  const int end = min(begin + a.chunk, a.V);
  const size_t gbase = (size_t)row * a.V;
  const float* x = a.logits + gbase;

  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // scalar head up to 16-byte alignment, vector body, scalar tail; every
  // thread visits its indices in increasing order
  const int mis = (int)((reinterpret_cast<uintptr_t>(x + begin) >> 2) & 3);
  const int head_end = min(end, begin + ((4 - mis) & 3));
  for (int idx = begin + tid; idx < head_end; idx += kArgmaxThreads) keep_better(bv, bi, x[idx], idx);
  const int nvec = (end - head_end) >> 2;
  const f32x4* xv = reinterpret_cast<const f32x4*>(x + head_end);
#pragma unroll 4
  for (int k = tid; k < nvec; k += kArgmaxThreads) {
    const f32x4 v = __builtin_nontemporal_load(xv + k);
    const int idx = head_end + 4 * k;
    keep_better(bv, bi, v[0], idx);
    keep_better(bv, bi, v[1], idx + 1);
    keep_better(bv, bi, v[2], idx + 2);
    keep_better(bv, bi, v[3], idx + 3);
  }
  for (int idx = head_end + 4 * nvec + tid; idx < end; idx += kArgmaxThreads) keep_better(bv, bi, x[idx], idx);

#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bi, off, kWave);
    keep_better(bv, bi, ov, oi);
  }
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane == 0) {
    wv[wave] = bv;
    wi[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kArgmaxThreads / kWave; ++w) keep_better(bv, bi, wv[w], wi[w]);
    const unsigned long long key =
        ((unsigned long long)order_bits(bv) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)bi);
    atomicMax(&a.slots[row], key);
    __threadfence();
    ticket = atomicAdd(&a.counters[b], 1u);
  }
  __syncthreads();
  if (ticket != (unsigned int)(a.K * a.nchunks - 1) || wave != 0) return;

  // last work-group of sequence b: consensus over the K rows
  __threadfence();
  uint32_t gtok = 0;
  bool miss = false;
  if (lane < a.K) {
    unsigned long long* slot = &a.slots[b * a.K + lane];
    const unsigned long long key = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    gtok = 0xffffffffu - (uint32_t)(key & 0xffffffffu);
    miss = a.drafts[b * a.K + lane] != (int32_t)gtok;
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.ar_tokens) a.ar_tokens[b * a.K + lane] = (int32_t)gtok;
  }
  const unsigned long long mask = __ballot(miss);
  const int acc = mask ? (__ffsll((long long)mask) - 1) : a.K;
  const int last = acc < a.K ? acc : a.K - 1;
  const int nxt = __shfl((int)gtok, last, kWave);
  if (lane == 0) {
    a.accept_len[b] = acc;
    a.next_token[b] = nxt;
    __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

static int accept_chunk(int batch, int block_k, int vocab) {
  // about 2048 work-groups in total, 2K..16K logits (8..64 KiB) each
  const long total = (long)batch * block_k * vocab;
  long c = (total + 2047) / 2048;
  c = (c + 3) & ~3L;
  if (c < 2048) c = 2048;
  if (c > 16384) c = 16384;
  if (c > vocab) c = vocab;
  return (int)c;
}

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_greedy_accept_workspace_bytes(int32_t batch, int32_t block_k, int32_t vocab) {
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return 0;
  return (size_t)batch * block_k * 8 + (((size_t)batch * 4 + 15) & ~(size_t)15);
}

extern "C" orthrus_status orthrus_greedy_accept(const float* ar_logits, const int32_t* draft_tokens,
                                                int32_t* accept_len, int32_t* next_token, int32_t* ar_tokens,
                                                int32_t batch, int32_t block_k, int32_t vocab, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  if (!ar_logits || !draft_tokens || !accept_len || !next_token) return ORTHRUS_ERR_NULL;
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return ORTHRUS_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(ar_logits) & 3) return ORTHRUS_ERR_SHAPE;
  const size_t need = orthrus_greedy_accept_workspace_bytes(batch, block_k, vocab);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7))
    return ORTHRUS_ERR_WORKSPACE;
  const long rows = (long)batch * block_k;
  AcceptArgs a;
  a.logits = ar_logits;
  a.drafts = draft_tokens;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.ar_tokens = ar_tokens;
  a.slots = (unsigned long long*)workspace;
  a.counters = (unsigned int*)((char*)workspace + (size_t)rows * 8);
  a.B = batch;
  a.K = block_k;
  a.V = vocab;
  a.chunk = accept_chunk(batch, block_k, vocab);
  a.nchunks = (vocab + a.chunk - 1) / a.chunk;
  const long grid = rows * a.nchunks;
  if (grid > 0x7fffffffL) return ORTHRUS_ERR_SHAPE;
  hipLaunchKernelGGL(argmax_accept, dim3((unsigned)grid), dim3(kArgmaxThreads), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

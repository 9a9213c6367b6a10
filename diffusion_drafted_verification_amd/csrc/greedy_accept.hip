// Greedy consensus of one Orthrus decode step on gfx950 (Orthrus explainer,
// gist.science arXiv 2605.12825, technical summary §2.3): per block row the
// AR head's greedy token (argmax over the vocabulary, lowest index on ties),
// then the longest prefix of drafts that equals those tokens.
//
// One launch, three levels.  Each work-group scans one contiguous chunk of
// one logits row with 16-byte loads (the scan is HBM-bound: 4 bytes per
// logit) and reduces (value, index) pairs across the wave with xor shuffles
// and across waves in LDS into one 64-bit key (order-preserving value bits
// << 32 | ~index: the larger key is the larger value, then the lower index).
// It stores the key and takes a ticket on its row; the last chunk of a row
// reduces the row's keys to the greedy token and takes a ticket on its
// sequence; the last row of a sequence compares the K tokens with the drafts
// (wave ballot: first mismatch) and writes accept_len / next_token /
// ar_tokens.  Every workspace word is cleared by the work-group that consumes
// it (keys by the row's last chunk, tokens and tickets by their last reader),
// so the whole workspace is zero again after every call, whatever shape the
// next call has.  No address is hit by more than max(chunks, K)
// atomics.
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
  int32_t* gtok;              // [B*K] greedy tokens
  unsigned int* row_cnt;      // [B*K] tickets
  unsigned int* seq_cnt;      // [B] tickets
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

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)k, off, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, kWave);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}

__global__ void __launch_bounds__(kArgmaxThreads) argmax_accept(AcceptArgs a) {
  __shared__ float wv[kArgmaxThreads / kWave];
  __shared__ int wi[kArgmaxThreads / kWave];
  __shared__ int row_last;

  const int row = blockIdx.x / a.nchunks;  // b * K + i
  const int ck = blockIdx.x % a.nchunks;
  const int b = row / a.K;
  const int tid = threadIdx.x;
  const int begin = ck * a.chunk;
  const int end = min(begin + a.chunk, a.V);
  const float* x = a.logits + (size_t)row * a.V;

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
    __hip_atomic_store(&a.part[(size_t)row * a.nchunks + ck], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    row_last = atomicAdd(&a.row_cnt[row], 1u) == (unsigned int)(a.nchunks - 1);
  }
  __syncthreads();
  if (!row_last || wave != 0) return;

  // last chunk of this row: the row's greedy token
  __threadfence();
  unsigned long long best = 0;
  for (int q = lane; q < a.nchunks; q += kWave) {
    unsigned long long* slot = &a.part[(size_t)row * a.nchunks + q];
    const unsigned long long k = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // leave the workspace zeroed
    best = k > best ? k : best;
  }
  best = wave_max_u64(best);
  int seq_last = 0;
  if (lane == 0) {
    const int32_t tok = (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
    __hip_atomic_store(&a.gtok[row], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.row_cnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    seq_last = atomicAdd(&a.seq_cnt[b], 1u) == (unsigned int)(a.K - 1);
  }
  seq_last = __shfl(seq_last, 0, kWave);
  if (!seq_last) return;

  // last row of sequence b: consensus over its K rows
  __threadfence();
  int32_t gt = 0;
  bool miss = false;
  if (lane < a.K) {
    gt = __hip_atomic_load(&a.gtok[b * a.K + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.gtok[b * a.K + lane], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    miss = a.drafts[b * a.K + lane] != gt;
    if (a.ar_tokens) a.ar_tokens[b * a.K + lane] = gt;
  }
  const unsigned long long mask = __ballot(miss);
  const int acc = mask ? (__ffsll((long long)mask) - 1) : a.K;
  const int last = acc < a.K ? acc : a.K - 1;
  const int nxt = __shfl(gt, last, kWave);
  if (lane == 0) {
    a.accept_len[b] = acc;
    a.next_token[b] = nxt;
    __hip_atomic_store(&a.seq_cnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

static int accept_chunk(int vocab) {
  // 8192 logits (32 KiB) per work-group: 32 values per thread in flight
  return vocab < 8192 ? vocab : 8192;
}

struct AcceptLayout {
  size_t part, gtok, row_cnt, seq_cnt, total;
  int chunk, nchunks;
};

static AcceptLayout accept_layout(int batch, int block_k, int vocab) {
  AcceptLayout L;
  const size_t rows = (size_t)batch * block_k;
  L.chunk = accept_chunk(vocab);
  L.nchunks = (vocab + L.chunk - 1) / L.chunk;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.part = 0;
  L.gtok = up(rows * L.nchunks * 8);
  L.row_cnt = L.gtok + up(rows * 4);
  L.seq_cnt = L.row_cnt + up(rows * 4);
  L.total = L.seq_cnt + up((size_t)batch * 4);
  return L;
}

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_greedy_accept_workspace_bytes(int32_t batch, int32_t block_k, int32_t vocab) {
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return 0;
  return accept_layout(batch, block_k, vocab).total;
}

extern "C" orthrus_status orthrus_greedy_accept(const float* ar_logits, const int32_t* draft_tokens,
                                                int32_t* accept_len, int32_t* next_token, int32_t* ar_tokens,
                                                int32_t batch, int32_t block_k, int32_t vocab, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  if (!ar_logits || !draft_tokens || !accept_len || !next_token) return ORTHRUS_ERR_NULL;
  if (batch < 1 || block_k < 1 || block_k > 32 || vocab < 1) return ORTHRUS_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(ar_logits) & 3) return ORTHRUS_ERR_SHAPE;
  const AcceptLayout lay = accept_layout(batch, block_k, vocab);
  if (!workspace || workspace_bytes < lay.total || (reinterpret_cast<uintptr_t>(workspace) & 7))
    return ORTHRUS_ERR_WORKSPACE;
  const long grid = (long)batch * block_k * lay.nchunks;
  if (grid > 0x7fffffffL) return ORTHRUS_ERR_SHAPE;
  char* ws = (char*)workspace;
  AcceptArgs a;
  a.logits = ar_logits;
  a.drafts = draft_tokens;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.ar_tokens = ar_tokens;
  a.part = (unsigned long long*)(ws + lay.part);
  a.gtok = (int32_t*)(ws + lay.gtok);
  a.row_cnt = (unsigned int*)(ws + lay.row_cnt);
  a.seq_cnt = (unsigned int*)(ws + lay.seq_cnt);
  a.B = batch;
  a.K = block_k;
  a.V = vocab;
  a.chunk = lay.chunk;
  a.nchunks = lay.nchunks;
  hipLaunchKernelGGL(argmax_accept, dim3((unsigned)grid), dim3(kArgmaxThreads), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

// Commit of one Orthrus decode step on gfx950 (Orthrus explainer,
// gist.science arXiv 2605.12825, technical summary §2.3: the cache keeps only
// the committed positions).  The AR verify pass's block K/V rows
// 0 .. n-1, n = min(accept_len + 1, K), are scattered into the paged cache at
// logical positions ctx_len .. ctx_len + n - 1.  One work-group per
// (sequence, block row); 16-byte copies of the Hkv x D row of K and of V.
//
// Also the library's plain streaming copy and read, used as measurement
// probes.
#include "orthrus_device.h"
#include "orthrus_host.h"

namespace orthrus {

struct AppendArgs {
  char* k_cache;            // single layer: the tensors themselves
  char* v_cache;
  const char* k_blk;
  const char* v_blk;
  const uint64_t* k_cache_list;  // several layers: device arrays of per-layer pointers
  const uint64_t* v_cache_list;
  const uint64_t* k_blk_list;
  const uint64_t* v_blk_list;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  const int32_t* accept_len;
  int32_t* new_ctx_lens;
  int32_t* slots;
  int B, K, Hkv, max_pages, num_pages, max_ctx, row_bytes, head_bytes;
};

__global__ void __launch_bounds__(256) kv_append_kernel(AppendArgs a) {
  const int layer = blockIdx.x / (a.B * a.K);
  const int br = blockIdx.x % (a.B * a.K);
  const int b = br / a.K, r = br % a.K;
  // a context length outside [0, max_ctx] breaks the call's contract: such a
  // sequence is skipped (nothing written, new length and slots -1) rather
  // than clamped, which would overwrite committed rows
  const int L = a.ctx_lens[b];
  const bool seq_ok = L >= 0 && L <= a.max_ctx;
  int acc = a.accept_len[b];
  acc = acc < 0 ? 0 : (acc > a.K ? a.K : acc);
  const int n = acc + 1 < a.K ? acc + 1 : a.K;
  const int pos = L + r;
  bool write = seq_ok && r < n;
  int page = -1;
  if (write) {
    const int lp = pos / kPage;
    page = lp < a.max_pages ? a.page_table[(size_t)b * a.max_pages + lp] : -1;
    if (page < 0 || page >= a.num_pages) write = false;
  }
  if (threadIdx.x == 0 && layer == 0) {
    if (a.slots) a.slots[b * a.K + r] = write ? page * kPage + pos % kPage : -1;
    if (r == 0 && a.new_ctx_lens) a.new_ctx_lens[b] = seq_ok ? L + n : -1;
  }
  if (!write) return;
  char* k_cache = a.k_cache_list ? reinterpret_cast<char*>(a.k_cache_list[layer]) : a.k_cache;
  char* v_cache = a.v_cache_list ? reinterpret_cast<char*>(a.v_cache_list[layer]) : a.v_cache;
  const char* k_blk = a.k_blk_list ? reinterpret_cast<const char*>(a.k_blk_list[layer]) : a.k_blk;
  const char* v_blk = a.v_blk_list ? reinterpret_cast<const char*>(a.v_blk_list[layer]) : a.v_blk;
  const int units = a.row_bytes / 16;  // per tensor: Hkv heads x D elements
  const size_t src_row = (size_t)(b * a.K + r) * a.row_bytes;
  for (int u = threadIdx.x; u < 2 * units; u += blockDim.x) {
    const int tensor = u / units, uu = u % units;
    const int g = uu / (a.head_bytes / 16), cc = uu % (a.head_bytes / 16);
    const size_t dst = ((size_t)(page * a.Hkv + g) * kPage + pos % kPage) * a.head_bytes + cc * 16;
    if (tensor == 0)
      st16(k_cache + dst, ld16(k_blk + src_row + uu * 16));
    else
      st16(v_cache + dst, ld16(v_blk + src_row + uu * 16));
  }
}

__global__ void __launch_bounds__(256) copy_probe_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                         size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) dst[k] = src[k];
}

// read-only stream: every 16-byte unit of src once with nontemporal loads (16
// in flight per thread; measured about 15 % faster than ordinary loads on this
// GPU), folded by XOR into one 16-byte value per thread of sink
constexpr int kReadBlocks = 1024;

__global__ void __launch_bounds__(256) read_probe_kernel(const u32x4* __restrict__ src, size_t n,
                                                         u32x4* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 16;
  u32x4 acc = {0, 0, 0, 0};
  for (size_t b = (size_t)blockIdx.x * blockDim.x * 16 + threadIdx.x; b < n; b += stride) {
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = b + (size_t)blockDim.x * i < n ? __builtin_nontemporal_load(src + b + (size_t)blockDim.x * i)
                                             : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= v[i];
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

static orthrus_status append_launch(AppendArgs& a, const orthrus_attn_desc& d, int n_layers,
                                     const int32_t* page_table, const int32_t* ctx_lens, const int32_t* accept_len,
                                     int32_t* new_ctx_lens, int32_t* slots, void* stream) {
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.accept_len = accept_len;
  a.new_ctx_lens = new_ctx_lens;
  a.slots = slots;
  a.B = d.batch;
  a.K = d.block_k;
  a.Hkv = d.n_kv_heads;
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.max_ctx = d.max_ctx_len;
  const int esz = d.dtype == ORTHRUS_BF16 ? 2 : 4;
  a.head_bytes = d.head_dim * esz;
  a.row_bytes = d.n_kv_heads * a.head_bytes;
  const long grid = (long)n_layers * d.batch * d.block_k;
  if (grid > 0x7fffffffL) return ORTHRUS_ERR_SHAPE;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

}  // namespace orthrus

using namespace orthrus;

extern "C" orthrus_status orthrus_kv_append(void* k_cache, void* v_cache, const void* k_blk, const void* v_blk,
                                            const int32_t* page_table, const int32_t* ctx_lens,
                                            const int32_t* accept_len, int32_t* new_ctx_lens, int32_t* slots,
                                            const orthrus_attn_desc* desc, void* stream) {
  orthrus_status st = validate_desc(desc);
  if (st != ORTHRUS_OK) return st;
  if (!k_cache || !v_cache || !k_blk || !v_blk || !page_table || !ctx_lens || !accept_len) return ORTHRUS_ERR_NULL;
  if (!aligned16(k_cache, v_cache, k_blk, v_blk) ||
      !aligned4(page_table, ctx_lens, accept_len, new_ctx_lens, slots))
    return ORTHRUS_ERR_SHAPE;
  AppendArgs a = {};
  a.k_cache = (char*)k_cache;
  a.v_cache = (char*)v_cache;
  a.k_blk = (const char*)k_blk;
  a.v_blk = (const char*)v_blk;
  return append_launch(a, *desc, 1, page_table, ctx_lens, accept_len, new_ctx_lens, slots, stream);
}

extern "C" orthrus_status orthrus_kv_append_layers(const uint64_t* k_cache_ptrs, const uint64_t* v_cache_ptrs,
                                                   const uint64_t* k_blk_ptrs, const uint64_t* v_blk_ptrs,
                                                   int32_t n_layers, const int32_t* page_table,
                                                   const int32_t* ctx_lens, const int32_t* accept_len,
                                                   int32_t* new_ctx_lens, int32_t* slots,
                                                   const orthrus_attn_desc* desc, void* stream) {
  orthrus_status st = validate_desc(desc);
  if (st != ORTHRUS_OK) return st;
  if (!k_cache_ptrs || !v_cache_ptrs || !k_blk_ptrs || !v_blk_ptrs || !page_table || !ctx_lens || !accept_len)
    return ORTHRUS_ERR_NULL;
  if (n_layers < 1 || n_layers > 4096) return ORTHRUS_ERR_SHAPE;
  if (!aligned_to<8>(k_cache_ptrs, v_cache_ptrs, k_blk_ptrs, v_blk_ptrs) ||
      !aligned4(page_table, ctx_lens, accept_len, new_ctx_lens, slots))
    return ORTHRUS_ERR_SHAPE;
  AppendArgs a = {};
  a.k_cache_list = k_cache_ptrs;
  a.v_cache_list = v_cache_ptrs;
  a.k_blk_list = k_blk_ptrs;
  a.v_blk_list = v_blk_ptrs;
  return append_launch(a, *desc, n_layers, page_table, ctx_lens, accept_len, new_ctx_lens, slots, stream);
}

extern "C" orthrus_status orthrus_copy_probe(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return ORTHRUS_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return ORTHRUS_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15) return ORTHRUS_ERR_SHAPE;
  const size_t n = bytes / 16;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (u32x4*)dst,
                     (const u32x4*)src, n);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

extern "C" int32_t orthrus_abi_version(void) { return ORTHRUS_ABI_VERSION; }

extern "C" const char* orthrus_status_str(int32_t s) {
  switch (s) {
    case ORTHRUS_OK: return "ok";
    case ORTHRUS_ERR_NULL: return "a required pointer is NULL";
    case ORTHRUS_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case ORTHRUS_ERR_UNSUPPORTED: return "dtype, head_dim, group size or page size not supported";
    case ORTHRUS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ORTHRUS_ERR_LAUNCH: return "the HIP runtime reported a launch error";
  }
  return "unknown status";
}

extern "C" orthrus_status orthrus_read_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                                             void* stream) {
  if (!src || !sink) return ORTHRUS_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return ORTHRUS_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) & 15) return ORTHRUS_ERR_SHAPE;
  if (sink_bytes < (size_t)kReadBlocks * 256 * 16) return ORTHRUS_ERR_WORKSPACE;
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadBlocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                     bytes / 16, (u32x4*)sink);
  return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

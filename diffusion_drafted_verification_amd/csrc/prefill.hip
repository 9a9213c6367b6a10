// Prompt prefill on gfx950: the frozen AR head's causal attention over a
// prompt placed after L_b already-cached tokens, and the write of the
// prompt's keys and values into the shared paged cache (Orthrus explainer,
// gist.science arXiv 2605.12825, technical summary §2.1: the one shared
// cache holds the AR head's keys and values; the prompt is what first fills
// it, processed causally like any AR prefill).
//
// The prompt is cut into 32-row chunks.  Chunk j of sequence b is exactly a
// causal block of the AR verify pass (AR_CAUSAL, K = 32) placed after
// L_b + 32 j cached tokens: its rows see the cached context, the earlier
// chunks (which are in the cache by then) and the rows of the chunk up to
// their own.  So once every prompt row's key and value is in the cache, the
// prefill is one call of the block-attention kernels over B x C "virtual"
// sequences (C = chunks per sequence), each reading its sequence's page
// table row:
//   prefill_prepare   one launch: the virtual page-table rows and context
//                     lengths and the sequences' new lengths L_b +
//                     prompt_len_b (prefill_setup), and the prompt rows
//                     r < prompt_len_b of k and v at logical positions
//                     L_b + r (prefill_kv_write: one work-group per row,
//                     16-byte copies);
//   orthrus_block_attn(AR_CAUSAL) on the virtual batch, with the prompt's
//                     own k/v as the block keys/values.
// Each chunk's group of G query heads shares one (G x 32)-row MFMA tile per
// KV head, so every key read serves 32 G query rows (64 G where the pair
// kernel serves two chunks per work-group).
#include "orthrus_device.h"
#include "orthrus_host.h"

namespace orthrus {

constexpr int kChunk = 32;

struct PrefillArgs {
  const int32_t* page_table;  // [B, max_pages]
  const int32_t* ctx_lens;    // [B]
  const int32_t* prompt_lens; // [B]
  int32_t* vtable;            // [B * C, max_pages]
  int32_t* vctx;              // [B * C]
  int32_t* new_ctx_lens;      // [B] or nullptr
  char* k_cache;
  char* v_cache;
  const char* k;              // [B, S, Hkv, D]
  const char* v;
  int B, C, S, max_pages, num_pages, max_ctx, row_bytes, head_bytes, Hkv;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// virtual sequence bc = (b, j): its page-table row and context length
__device__ void prefill_setup(const PrefillArgs& a, int bc) {
  const int b = bc / a.C, j = bc % a.C;
  const int L = clampi(a.ctx_lens[b], 0, a.max_ctx);
  const int n = clampi(a.prompt_lens[b], 0, a.S);
  for (int p = threadIdx.x; p < a.max_pages; p += blockDim.x)
    a.vtable[(size_t)bc * a.max_pages + p] = a.page_table[(size_t)b * a.max_pages + p];
  if (threadIdx.x == 0) {
    // chunks past the prompt compute unused rows over an empty context
    a.vctx[bc] = kChunk * j < n ? L + kChunk * j : 0;
    if (j == 0 && a.new_ctx_lens) a.new_ctx_lens[b] = L + n;
  }
}

// prompt row (b, r) into the cache
__device__ void prefill_kv_write(const PrefillArgs& a, int row) {
  const int b = row / a.S, r = row % a.S;
  const int n = clampi(a.prompt_lens[b], 0, a.S);
  if (r >= n) return;
  const int pos = clampi(a.ctx_lens[b], 0, a.max_ctx) + r;
  const int lp = pos / kPage;
  const int page = lp < a.max_pages ? a.page_table[(size_t)b * a.max_pages + lp] : -1;
  if (page < 0 || page >= a.num_pages) return;  // an invalid page id is never written through
  const int units = a.row_bytes / 16;
  const size_t src_row = ((size_t)b * a.S + r) * a.row_bytes;
  for (int u = threadIdx.x; u < 2 * units; u += blockDim.x) {
    const int tensor = u / units, uu = u % units;
    const int g = uu / (a.head_bytes / 16), cc = uu % (a.head_bytes / 16);
    const size_t dst = ((size_t)(page * a.Hkv + g) * kPage + pos % kPage) * a.head_bytes + cc * 16;
    if (tensor == 0)
      st16(a.k_cache + dst, ld16(a.k + src_row + uu * 16));
    else
      st16(a.v_cache + dst, ld16(a.v + src_row + uu * 16));
  }
}

// One launch for both preparations (they write disjoint outputs and the
// attention launch after it orders them): work-groups 0 .. B C - 1 set up the
// virtual sequences, the next B S write one prompt row each.  Two launches
// cost a launch and a kernel boundary more on every prefill call.
__global__ void __launch_bounds__(256) prefill_prepare(PrefillArgs a) {
  const long nv = (long)a.B * a.C;
  if ((long)blockIdx.x < nv) prefill_setup(a, (int)blockIdx.x);
  else prefill_kv_write(a, (int)((long)blockIdx.x - nv));
}

// the block-attention descriptor of the virtual batch, validated
static orthrus_status prefill_desc(const orthrus_attn_desc* d, int32_t max_prompt, orthrus_attn_desc* vd, int* C,
                                   int* S) {
  if (!d) return ORTHRUS_ERR_NULL;
  if (max_prompt < 1 || max_prompt > (1 << 24)) return ORTHRUS_ERR_SHAPE;
  *S = (max_prompt + kChunk - 1) / kChunk * kChunk;
  *C = *S / kChunk;
  if ((long)d->batch * *C > 0x7fffffffL / 64) return ORTHRUS_ERR_SHAPE;
  *vd = *d;
  // automatic split: the longest allowed (the virtual batch of chunks already
  // fills the GPU, and measured on the Qwen3-8B shape, fewer splits beat the
  // extra combine pass: 2k prompt after 8k cached, 412 -> 371 us)
  if (vd->split_tokens == 0) vd->split_tokens = 8192;
  vd->block_k = kChunk;
  vd->batch = d->batch * *C;
  const long vmax = (long)d->max_ctx_len + *S - kChunk;
  if (d->max_ctx_len < 0 || vmax > 0x7fffffffL) return ORTHRUS_ERR_SHAPE;
  vd->max_ctx_len = (int32_t)vmax;
  return validate_desc(vd);
}

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunks per attention work-group for the virtual batch vd of B sequences
// with C chunks each: 2 (the pair kernel: bf16 with G <= 4) when that grid
// still fills two rounds of 256 work-groups, else 1.  A pair does twice the
// work of a chunk, so with fewer work-groups the longest pair sets the time.
// Measured on the Qwen3-8B shape (one layer): an 8192-token prompt 750 ->
// 689 us and a 2048-token prompt after 8192 cached tokens 461 -> 424 us with
// pairs, but a 2048-token prompt on an empty cache (one round of pairs)
// 76.5 -> 95 us.
static int prefill_chunks_per_wg(const orthrus_attn_desc& vd, int B, int C) {
  // the pair kernel serves fixed splits of the streaming path only
  if (vd.dtype != ORTHRUS_BF16 || vd.n_q_heads / vd.n_kv_heads > 4 || vd.split_tokens <= 0) return 1;
  const long splits = vd.max_ctx_len > 0 ? ((long)vd.max_ctx_len + vd.split_tokens - 1) / vd.split_tokens : 1;
  const long grid = splits * B * ((C + 1) / 2) * vd.n_kv_heads;
  return grid >= 2 * 256 ? 2 : 1;
}

struct PrefillWs {
  size_t off_ctx, off_attn, attn_bytes, total;
};

static PrefillWs prefill_ws(const orthrus_attn_desc& vd) {
  PrefillWs w;
  w.off_ctx = up256((size_t)vd.batch * vd.max_pages_per_seq * sizeof(int32_t));
  w.off_attn = w.off_ctx + up256((size_t)vd.batch * sizeof(int32_t));
  w.attn_bytes = orthrus_block_attn_workspace_bytes(&vd);
  w.total = w.off_attn + w.attn_bytes;
  return w;
}

}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_prefill_workspace_bytes(const orthrus_attn_desc* desc, int32_t max_prompt) {
  orthrus_attn_desc vd;
  int C, S;
  if (prefill_desc(desc, max_prompt, &vd, &C, &S) != ORTHRUS_OK) return 0;
  return prefill_ws(vd).total;
}

extern "C" int32_t orthrus_prefill_chunks_per_workgroup(const orthrus_attn_desc* desc, int32_t max_prompt) {
  orthrus_attn_desc vd;
  int C, S;
  if (prefill_desc(desc, max_prompt, &vd, &C, &S) != ORTHRUS_OK) return 0;
  return prefill_chunks_per_wg(vd, desc->batch, C);
}

extern "C" orthrus_status orthrus_prefill(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                                          const int32_t* page_table, const int32_t* ctx_lens,
                                          const int32_t* prompt_lens, int32_t max_prompt, void* out,
                                          int32_t* new_ctx_lens, const orthrus_attn_desc* desc, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !k_cache || !v_cache || !page_table || !ctx_lens || !prompt_lens || !out)
    return ORTHRUS_ERR_NULL;
  if (!aligned16(q, k, v, k_cache, v_cache, out) || !aligned4(page_table, ctx_lens, prompt_lens, new_ctx_lens))
    return ORTHRUS_ERR_SHAPE;
  orthrus_attn_desc vd;
  int C, S;
  const orthrus_status vs = prefill_desc(desc, max_prompt, &vd, &C, &S);
  if (vs != ORTHRUS_OK) return vs;
  const PrefillWs w = prefill_ws(vd);
  if (!workspace || workspace_bytes < w.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return ORTHRUS_ERR_WORKSPACE;
  const int elem = vd.dtype == ORTHRUS_BF16 ? 2 : 4;
  char* ws = (char*)workspace;
  PrefillArgs a;
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.prompt_lens = prompt_lens;
  a.vtable = (int32_t*)ws;
  a.vctx = (int32_t*)(ws + w.off_ctx);
  a.new_ctx_lens = new_ctx_lens;
  a.k_cache = (char*)k_cache;
  a.v_cache = (char*)v_cache;
  a.k = (const char*)k;
  a.v = (const char*)v;
  a.B = desc->batch;
  a.C = C;
  a.S = S;
  a.max_pages = vd.max_pages_per_seq;
  a.num_pages = vd.num_pages;
  a.max_ctx = desc->max_ctx_len;
  a.head_bytes = vd.head_dim * elem;
  a.row_bytes = vd.n_kv_heads * a.head_bytes;
  a.Hkv = vd.n_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(prefill_prepare, dim3((unsigned)((long)a.B * C + (long)a.B * S)), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return ORTHRUS_ERR_LAUNCH;
  // the chunks re-read the prompt's K/V through the caches: ordinary loads
  return block_attn_run(q, k_cache, v_cache, k, v, a.vtable, a.vctx, ORTHRUS_AR_CAUSAL, out, &vd,
                        w.attn_bytes ? ws + w.off_attn : nullptr, w.attn_bytes, stream, false,
                        prefill_chunks_per_wg(vd, desc->batch, C) == 2 ? C : 0);
}

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
//   * one work-group per (sequence b, KV head g, context split s); its G waves
//     are the G query heads sharing KV head g, so each KV byte is read from HBM
//     once and feeds a (G x 32)-row tile;
//   * context positions stream through LDS in 64-token stages (double
//     buffered, register-staged prefetch of the next stage); K is kept
//     token-major with an XOR chunk swizzle, V is stored transposed so both
//     MFMA operands are single 16-byte LDS reads;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 with fp32
//     accumulation: the score tile's accumulator layout is directly the B
//     operand of the PV product (no shuffles), and every lane owns one query
//     row, so row rescales are per-lane multiplies;
//   * online softmax in the log2 domain with a lazy (threshold) rescale;
//     only the row max needs one cross-lane exchange per 32 keys;
//   * the block tile and the ragged context tail are the only masked tiles;
//     the mask mode is a template parameter;
//   * when a sequence is split over several work-groups each writes fp32
//     partials (unnormalised O, running max, sum) and a combine kernel merges
//     them; the work-group order puts all splits of one (b, g) on one XCD so
//     the partials stay in that XCD's L2.
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
  float* ws_o;      // [B, Hq, s_max, 32, D]  unnormalised partial outputs
  float2* ws_ml;    // [B, Hq, s_max, 32]     (running max in log2 units, row sum)
  int B, K, Hq, Hkv, max_pages, num_pages, max_ctx, split, s_max;
  float c;          // softmax scale * log2(e)
};

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

// Global -> register staging of one 64-position stage.  Unit u covers four
// consecutive positions (one token quad, never crossing a page) and one
// 16-byte chunk of the head dimension, for both K and V.
template <typename T, int D, int NT>
struct Stage {
  typedef AttnLayout<T, D> Lay;
  static constexpr int UPT = (Lay::UNITS + NT - 1) / NT;
  u32x4 k[UPT][4];
  u32x4 v[UPT][4];

  __device__ void load(const AttnArgs& a, const int* pages, int page_base, int b, int g, int L, int N,
                       int p0, int tid) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + j * NT;
      if (Lay::UNITS % NT != 0 && u >= Lay::UNITS) break;
      const int tq = u / Lay::KCH, c = u % Lay::KCH;
      const int pos0 = p0 + 4 * tq;
      if (pos0 + 4 <= L) {  // four cached positions of one page
        const int page = pages[(pos0 >> 4) - page_base];
        if (page >= 0) {
          const size_t off = ((size_t)(page * a.Hkv + g) * kPage + (pos0 & 15)) * Lay::KROW + c * 16;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            k[j][t] = ld16(a.k_cache + off + t * Lay::KROW);
            v[j][t] = ld16(a.v_cache + off + t * Lay::KROW);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            k[j][t] = u32x4{0, 0, 0, 0};
            v[j][t] = u32x4{0, 0, 0, 0};
          }
        }
      } else {
        // tail of the context, the block rows, or past the end: every load is
        // issued from a valid address and zeroed afterwards when unused
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int pos = pos0 + t;
          const char* kp = a.k_blk;
          const char* vp = a.v_blk;
          bool ok = false;
          if (pos < L) {
            const int page = pages[(pos >> 4) - page_base];
            if (page >= 0) {
              const size_t off = ((size_t)(page * a.Hkv + g) * kPage + (pos & 15)) * Lay::KROW + c * 16;
              kp = a.k_cache + off;
              vp = a.v_cache + off;
              ok = true;
            }
          } else if (pos < N) {
            const size_t off = ((size_t)(b * a.K + (pos - L)) * a.Hkv + g) * Lay::KROW + c * 16;
            kp = a.k_blk + off;
            vp = a.v_blk + off;
            ok = true;
          }
          const u32x4 kk = ld16(kp), vv = ld16(vp);
          const u32x4 z{0, 0, 0, 0};
          k[j][t] = ok ? kk : z;
          v[j][t] = ok ? vv : z;
        }
      }
    }
  }

  // K rows go to LDS row swap_bits23(token) (so the score accumulator holds
  // eight consecutive tokens per lane half); V is written transposed.
  __device__ void store(char* stage, int tid) const {
    char* ks = stage;
    char* vs = stage + Lay::KBYTES;
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + j * NT;
      if (Lay::UNITS % NT != 0 && u >= Lay::UNITS) break;
      const int tq = u / Lay::KCH, c = u % Lay::KCH;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = swap_bits23(4 * tq + t);
        st16(ks + Lay::kslot(row, c), k[j][t]);
      }
      if constexpr (sizeof(T) == 2) {
        // element e of the chunk is d = c*8 + e; four tokens -> 8 bytes of row d
        const int tch = tq >> 1, half = (tq & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x2 pk;
          if (e & 1) {
            pk[0] = (v[j][0][w] >> 16) | (v[j][1][w] & 0xffff0000u);
            pk[1] = (v[j][2][w] >> 16) | (v[j][3][w] & 0xffff0000u);
          } else {
            pk[0] = (v[j][0][w] & 0xffffu) | (v[j][1][w] << 16);
            pk[1] = (v[j][2][w] & 0xffffu) | (v[j][3][w] << 16);
          }
          const int d = c * 8 + e;
          *reinterpret_cast<u32x2*>(vs + Lay::vslot(d, tch) + half) = pk;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = c * 4 + e;
          st16(vs + Lay::vslot(d, tq), u32x4{v[j][0][e], v[j][1][e], v[j][2][e], v[j][3][e]});
        }
      }
    }
  }
};

template <typename T, int D, int G, int MODE>
__global__ void __launch_bounds__(kWave * G) attn_main(AttnArgs a) {
  typedef AttnLayout<T, D> Lay;
  typedef typename Vec8<T>::type V8;
  constexpr int NT = kWave * G;
  constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int MB = D / 32;   // 32-wide blocks of the head dimension in O^T

  __shared__ __attribute__((aligned(16))) char smem[2 * Lay::STAGE];
  __shared__ int pages[kMaxSplit / kPage];

  const int BH = a.B * a.Hkv;
  const int bg = blockIdx.x % BH;
  const int s = blockIdx.x / BH;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  int L = a.ctx_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int N = L + a.K;
  const int S_b = (N + a.split - 1) / a.split;
  if (s >= S_b) return;
  const int p_begin = s * a.split;
  const int p_end = min(p_begin + a.split, N);
  const int ntiles = (p_end - p_begin + kTile - 1) / kTile;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int i = lane & 31, hi = lane >> 5;
  const int h = g * G + wave;

  // page ids of this split's cached positions (invalid ids become -1)
  const int page_base = p_begin >> 4;
  for (int x = tid; x < a.split / kPage; x += NT) {
    const int lp = page_base + x;
    int id = -1;
    if (lp * kPage < L && lp < a.max_pages) {
      id = a.page_table[(size_t)b * a.max_pages + lp];
      if (id < 0 || id >= a.num_pages) id = -1;
    }
    pages[x] = id;
  }

  // this wave's query rows as the B operand of S^T = K Q^T (one 16-wide k-step each)
  V8 qf[KS];
  {
    const char* qrow = a.q + ((size_t)(b * a.K + i) * a.Hq + h) * D * sizeof(T);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (i < a.K) {
        const int off = (16 * ks + 8 * hi) * sizeof(T);
        if constexpr (sizeof(T) == 2) {
          qf[ks] = __builtin_bit_cast(V8, ld16(qrow + off));
        } else {
          struct P { u32x4 x, y; } pr{ld16(qrow + off), ld16(qrow + off + 16)};
          qf[ks] = __builtin_bit_cast(V8, pr);
        }
      } else {
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
  float l = 0.f;          // this lane half's share of the row sum
  const float c = a.c;

  Stage<T, D, NT> st;
  st.load(a, pages, page_base, b, g, L, N, p_begin, tid);

  for (int t = 0; t < ntiles; ++t) {
    char* buf = smem + (t & 1) * Lay::STAGE;
    st.store(buf, tid);
    __syncthreads();
    const int p0 = p_begin + t * kTile;
    if (t + 1 < ntiles) st.load(a, pages, page_base, b, g, L, N, p0 + kTile, tid);

    const char* ks_lds = buf;
    const char* vs_lds = buf + Lay::KBYTES;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int pbase = p0 + 32 * sub;
      if (pbase >= p_end) break;
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
// work-groups: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_combine(AttnArgs a, int G) {
  constexpr int TPR = D / 4;          // threads per row (4 outputs each)
  constexpr int RPW = 256 / TPR;      // rows per work-group
  const int id = blockIdx.x;
  const int g = id % a.Hkv;
  const int b = (id / a.Hkv) % a.B;
  const int rest = id / (a.Hkv * a.B);  // = rg * G + w
  const int w = rest % G, rg = rest / G;
  const int h = g * G + w;
  const int i = rg * RPW + threadIdx.x / TPR;
  if (i >= a.K) return;
  int L = a.ctx_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int S_b = (L + a.K + a.split - 1) / a.split;
  if (S_b <= 1) return;
  const int d0 = 4 * (threadIdx.x % TPR);
  const size_t base = (size_t)(b * a.Hq + h) * a.s_max * kRows + i;
  float M = -INFINITY;
  for (int s = 0; s < S_b; ++s) M = fmaxf(M, a.ws_ml[base + (size_t)s * kRows].x);
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < S_b; ++s) {
    const float2 ml = a.ws_ml[base + (size_t)s * kRows];
    const float w8 = (ml.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.ws_o + (base + (size_t)s * kRows) * D + d0);
    acc += w8 * x;
    den += w8 * ml.y;
  }
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

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

int attn_split_tokens(const orthrus_attn_desc& d) {
  const long N = (long)d.max_ctx_len + d.block_k;
  const long n64 = ((N + kTile - 1) / kTile) * kTile;
  if (d.split_tokens > 0) return (int)(d.split_tokens < n64 ? d.split_tokens : n64);
  // aim for ~1024 work-groups at the longest context; keep splits >= 256
  // positions so partial results stay small next to the KV bytes they cover
  const int units = d.batch * d.n_kv_heads;
  const int s_target = units >= 1024 ? 1 : ceil_div(1024, units);
  long split = ((ceil_div(N, s_target) + kTile - 1) / kTile) * kTile;
  if (split < 256) split = 256;
  if (split > kMaxSplit) split = kMaxSplit;
  if (split > n64) split = n64;
  return (int)split;
}

size_t attn_workspace_bytes(const orthrus_attn_desc& d) {
  const int split = attn_split_tokens(d);
  const int s_max = ceil_div((long)d.max_ctx_len + d.block_k, split);
  if (s_max <= 1) return 0;
  const size_t rows = (size_t)d.batch * d.n_q_heads * s_max * kRows;
  return rows * d.head_dim * sizeof(float) + rows * sizeof(float2);
}

template <typename T, int D, int G>
static hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t stream) {
  const int grid = a.s_max * a.B * a.Hkv;
  if (mode == ORTHRUS_DIFF_BIDIR)
    hipLaunchKernelGGL((attn_main<T, D, G, ORTHRUS_DIFF_BIDIR>), dim3(grid), dim3(kWave * G), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_main<T, D, G, ORTHRUS_AR_CAUSAL>), dim3(grid), dim3(kWave * G), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.s_max <= 1) return e;
  constexpr int RPW = 256 / (D / 4);
  const int cgrid = ((a.K + RPW - 1) / RPW) * G * a.B * a.Hkv;
  hipLaunchKernelGGL((attn_combine<T, D>), dim3(cgrid), dim3(256), 0, stream, a, G);
  return hipGetLastError();
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
  return attn_split_tokens(*desc);
}

extern "C" orthrus_status orthrus_block_attn(const void* q, const void* k_cache, const void* v_cache,
                                             const void* k_blk, const void* v_blk,
                                             const int32_t* page_table, const int32_t* ctx_lens,
                                             orthrus_mode mode, void* out, const orthrus_attn_desc* desc,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  orthrus_status st = validate_desc(desc);
  if (st != ORTHRUS_OK) return st;
  if (!q || !k_cache || !v_cache || !k_blk || !v_blk || !page_table || !ctx_lens || !out)
    return ORTHRUS_ERR_NULL;
  if (mode != ORTHRUS_DIFF_BIDIR && mode != ORTHRUS_AR_CAUSAL) return ORTHRUS_ERR_SHAPE;
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
  a.split = attn_split_tokens(d);
  a.s_max = ceil_div((long)d.max_ctx_len + d.block_k, a.split);
  const size_t rows = (size_t)d.batch * d.n_q_heads * a.s_max * kRows;
  a.ws_o = need ? (float*)workspace : nullptr;
  a.ws_ml = need ? (float2*)((char*)workspace + rows * d.head_dim * sizeof(float)) : nullptr;
  const float scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.f / sqrtf((float)d.head_dim);
  a.c = scale * kLog2e;
  const int G = d.n_q_heads / d.n_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d.dtype == ORTHRUS_BF16)
    e = d.head_dim == 128 ? dispatch_g<bf16, 128>(a, G, mode, s) : dispatch_g<bf16, 64>(a, G, mode, s);
  else
    e = d.head_dim == 128 ? dispatch_g<float, 128>(a, G, mode, s) : dispatch_g<float, 64>(a, G, mode, s);
  return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

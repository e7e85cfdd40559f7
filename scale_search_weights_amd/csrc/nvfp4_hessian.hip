// Block-diagonal calibration Gram matrices H_b = sum_t x_t,b x_t,b^T (Local-Hessian
// write-up, "Change the objective": XX^T weighs the output error and only its 16x16
// diagonal blocks are kept) and the per-expert token lists that feed the grouped form.
//
// H is bandwidth-bound (16 flop per byte of bf16 X against a bf16-MFMA ridge near 300), so
// the bf16 kernel is organised to stream X once at full width:
//  * a workgroup owns 64 W channels (W 16-channel blocks per wave; W = 4 for a dense X, so
//    every token row is read in 512-byte pieces, 1 for the gathered rows of the grouped
//    form) and a chunk of tokens; each step stages a [32 tokens x 64 W channels] tile in
//    LDS with W coalesced 16-byte loads per lane, and the next step's loads (for the
//    grouped form also its row ids) are issued before this step's MFMAs;
//  * each wave reads a block's 16 channels x 32 tokens out of LDS as the MFMA operand
//    (lane = channel, eight tokens per lane; the row pitch is padded so the four lane
//    groups hit disjoint banks) and issues one v_mfma_f32_16x16x32_bf16 with the same
//    register as both A and B: A = X_b^T and B = X_b hold identical fragments, so any
//    K ordering the hardware uses pairs the same token on both sides;
//  * partial sums per (token chunk, block) go to the workspace and a second kernel adds
//    them in ascending chunk order, so results are deterministic without atomics.
// bf16 x bf16 products are exact in fp32; only the accumulation rounds.
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

constexpr int HT = 32;        // tokens per step
constexpr int HC = 64;        // channels per workgroup
constexpr int PITCH16 = 66;   // bf16 LDS row pitch in elements (132 B)
constexpr int PITCH32 = 68;   // fp32 LDS row pitch in elements (272 B)

constexpr int HW_DENSE = 4;      // bf16 dense: blocks per wave (512-byte row segments)
constexpr int HW_GROUPED = 1;    // bf16 grouped: blocks per wave
constexpr int64_t TC_DENSE = 4096;  // tokens per workgroup (dense, large n)

// tokens (dense) or list positions (grouped) per workgroup
static inline int64_t hess_chunk(int64_t n, bool grouped) {
  if (n < 65536) return 512;
  return grouped ? 2048 : TC_DENSE;
}

static inline int64_t hess_items_max(int64_t tokens, int64_t groups, int64_t n_ids, bool grouped) {
  if (!grouped) {
    const int64_t tc = hess_chunk(tokens, false);
    return (tokens + tc - 1) / tc;
  }
  const int64_t tc = hess_chunk(n_ids, true);
  return n_ids / tc + groups;
}

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t hessian_workspace_size(int64_t tokens, int64_t cols, int64_t groups, int64_t n_ids) {
  const bool grouped = n_ids >= 0;
  const int64_t items = hess_items_max(tokens, groups, n_ids, grouped);
  const int64_t nb = cols / 16;
  return align256(sizeof(int32_t) * (size_t)(groups + 1)) +
         sizeof(float) * (size_t)items * (size_t)nb * 256;
}

// item_off[g] = number of token chunks in groups < g (chunks of tc ids), capped at cap.
__global__ void k_hess_items(const int32_t *__restrict__ offsets, int64_t groups, int64_t n_ids,
                             int64_t tc, int64_t cap, int32_t *__restrict__ item_off) {
  __shared__ int64_t part[256];
  const int64_t per = (groups + 255) / 256;
  const int64_t g0 = threadIdx.x * per, g1 = min(groups, g0 + per);
  int64_t s = 0;
  for (int64_t g = g0; g < g1; ++g) {
    int64_t a = offsets[g], b = offsets[g + 1];
    a = a < 0 ? 0 : (a > n_ids ? n_ids : a);
    b = b < a ? a : (b > n_ids ? n_ids : b);
    s += (b - a + tc - 1) / tc;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t run = 0;
    for (int i = 0; i < 256; ++i) {
      const int64_t c = part[i];
      part[i] = run;
      run += c;
    }
  }
  __syncthreads();
  int64_t run = part[threadIdx.x];
  for (int64_t g = g0; g < g1; ++g) {
    item_off[g] = (int32_t)(run < cap ? run : cap);
    int64_t a = offsets[g], b = offsets[g + 1];
    a = a < 0 ? 0 : (a > n_ids ? n_ids : a);
    b = b < a ? a : (b > n_ids ? n_ids : b);
    run += (b - a + tc - 1) / tc;
  }
  if (g1 == groups && g0 < g1) item_off[groups] = (int32_t)(run < cap ? run : cap);
  if (groups == 0 && threadIdx.x == 0) item_off[0] = 0;
}

// Resolve this workgroup's token range [p0, p1) (positions in the id list, or token
// indices in the dense form). Returns false if the item index is past the real count.
template <bool GROUPED>
__device__ __forceinline__ bool hess_range(int64_t it, int64_t tokens, int64_t groups,
                                           const int32_t *offsets, int64_t n_ids,
                                           const int32_t *item_off, int64_t tc, int64_t &p0,
                                           int64_t &p1) {
  if (!GROUPED) {
    p0 = it * tc;
    p1 = min(p0 + tc, tokens);
    return p0 < p1;
  }
  if (it >= item_off[groups]) return false;
  int64_t lo = 0, hi = groups;  // largest g with item_off[g] <= it
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (item_off[mid] <= it) lo = mid;
    else hi = mid;
  }
  int64_t a = offsets[lo], b = offsets[lo + 1];
  a = a < 0 ? 0 : (a > n_ids ? n_ids : a);
  b = b < a ? a : (b > n_ids ? n_ids : b);
  p0 = a + (it - item_off[lo]) * tc;
  p1 = min(p0 + tc, b);
  return p0 < p1;
}

template <bool GROUPED, int W>
__global__ void __launch_bounds__(256)
    k_hess_bf16(const uint16_t *__restrict__ x, int64_t tokens, int64_t cols, int64_t groups,
                const int32_t *__restrict__ offsets, const int32_t *__restrict__ ids, int64_t n_ids,
                const int32_t *__restrict__ item_off, int64_t tc, float *__restrict__ partial,
                int64_t nb) {
  constexpr int C = HC * W;          // channels per workgroup: W blocks per wave
  constexpr int PITCH = C + 2;       // u16; the 8-row stride of the MFMA reads shifts banks by 8
  constexpr int SEGS = C / 8;        // 16-byte segments per token row
  constexpr int ROWS = 256 / SEGS;   // token rows per load instruction
  constexpr int NLD = HT / ROWS;     // 16-byte loads per lane per step (= W)
  __shared__ __attribute__((aligned(16))) uint16_t tile[HT * PITCH];
  // grid x = (token item, channel chunk), chunks fastest: one dimension, so long inputs with
  // more items than a y dimension holds still launch
  const int64_t nch = (cols + C - 1) / C;
  const int64_t it = (int64_t)blockIdx.x / nch;
  int64_t p0, p1;
  if (!hess_range<GROUPED>(it, tokens, groups, offsets, n_ids, item_off, tc, p0, p1)) return;
  const int64_t ch0 = ((int64_t)blockIdx.x % nch) * C;
  const int r = threadIdx.x / SEGS, q = threadIdx.x % SEGS;
  const int64_t ch = ch0 + q * 8;
  const bool ch_ok = ch < cols;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int fk = (lane >> 4) * 8;

  auto token_at = [&](int64_t pp) -> int64_t {
    if (pp >= p1) return -1;
    const int64_t tok = GROUPED ? (int64_t)ids[pp] : pp;
    return (tok >= 0 && tok < tokens) ? tok : -1;
  };
  auto tokens_of = [&](int64_t pos, int64_t tok[NLD]) {
#pragma unroll
    for (int s = 0; s < NLD; ++s) tok[s] = token_at(pos + r + ROWS * s);
  };
  auto load = [&](const int64_t tok[NLD], uint4 out[NLD]) {
#pragma unroll
    for (int s = 0; s < NLD; ++s)
      out[s] = (tok[s] >= 0 && ch_ok) ? *reinterpret_cast<const uint4 *>(x + tok[s] * cols + ch)
                                      : make_uint4(0u, 0u, 0u, 0u);
  };

  // software pipeline: this step's rows are in cur, the next step's token rows are known,
  // and the next step's loads are issued before this step's MFMAs
  v4f acc[W];
#pragma unroll
  for (int w = 0; w < W; ++w) acc[w] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  int64_t tk[NLD];
  uint4 cur[NLD];
  tokens_of(p0, tk);
  load(tk, cur);
  tokens_of(p0 + HT, tk);
  for (int64_t pos = p0; pos < p1; pos += HT) {
#pragma unroll
    for (int s = 0; s < NLD; ++s) {
      unsigned *dst = reinterpret_cast<unsigned *>(tile + (r + ROWS * s) * PITCH + q * 8);
      dst[0] = cur[s].x;
      dst[1] = cur[s].y;
      dst[2] = cur[s].z;
      dst[3] = cur[s].w;
    }
    __syncthreads();
    if (pos + HT < p1) {
      load(tk, cur);
      tokens_of(pos + 2 * HT, tk);
    }
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int fch = (wave * W + w) * 16 + (lane & 15);
      v8u16 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = tile[(fk + j) * PITCH + fch];
      const v8bf a = __builtin_bit_cast(v8bf, f);
      acc[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[w], 0, 0, 0);
    }
    __syncthreads();
  }
  const int col = lane & 15, row0 = (lane >> 4) * 4;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int64_t b = ch0 / 16 + wave * W + w;
    if (b < nb) {
      float *P = partial + (it * nb + b) * 256;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) P[(row0 + rr) * 16 + col] = acc[w][rr];
    }
  }
}

template <bool GROUPED>
__global__ void __launch_bounds__(256)
    k_hess_f32(const float *__restrict__ x, int64_t tokens, int64_t cols, int64_t groups,
               const int32_t *__restrict__ offsets, const int32_t *__restrict__ ids, int64_t n_ids,
               const int32_t *__restrict__ item_off, int64_t tc, float *__restrict__ partial,
               int64_t nb) {
  __shared__ __attribute__((aligned(16))) float tile[HT * PITCH32];
  // grid x = (token item, channel chunk), chunks fastest
  const int64_t nch = (cols + HC - 1) / HC;
  const int64_t it = (int64_t)blockIdx.x / nch;
  int64_t p0, p1;
  if (!hess_range<GROUPED>(it, tokens, groups, offsets, n_ids, item_off, tc, p0, p1)) return;
  const int64_t ch0 = ((int64_t)blockIdx.x % nch) * HC;
  const int r = threadIdx.x >> 3, q = threadIdx.x & 7;
  const int64_t ch = ch0 + q * 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int fch = wave * 16 + (lane & 15), fk = lane >> 4;

  auto load = [&](int64_t pos, float4 &u, float4 &v) {
    const int64_t pp = pos + r;
    u = v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pp < p1 && ch < cols) {
      const int64_t tok = GROUPED ? (int64_t)ids[pp] : pp;
      if (tok >= 0 && tok < tokens) {
        const float4 *s = reinterpret_cast<const float4 *>(x + tok * cols + ch);
        u = s[0];
        v = s[1];
      }
    }
  };

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float4 c0, c1;
  load(p0, c0, c1);
  for (int64_t pos = p0; pos < p1; pos += HT) {
    float4 *dst = reinterpret_cast<float4 *>(tile + r * PITCH32 + q * 8);
    dst[0] = c0;
    dst[1] = c1;
    __syncthreads();
    if (pos + HT < p1) load(pos + HT, c0, c1);
#pragma unroll
    for (int k0 = 0; k0 < HT; k0 += 4) {
      const float a = tile[(k0 + fk) * PITCH32 + fch];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, a, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int64_t b = ch0 / 16 + wave;
  if (b < nb) {
    float *P = partial + (it * nb + b) * 256;
    const int col = lane & 15, row0 = (lane >> 4) * 4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) P[(row0 + rr) * 16 + col] = acc[rr];
  }
}

// H[g][b][e] (+)= sum of partial[it][b][e] over the group's items, ascending.
__global__ void __launch_bounds__(256)
    k_hess_reduce(const float *__restrict__ partial, const int32_t *__restrict__ item_off,
                  int64_t n_items_dense, int64_t nb, float *__restrict__ H, int accumulate) {
  const int64_t b = blockIdx.x, g = blockIdx.y, e = threadIdx.x;
  const int64_t i0 = item_off ? item_off[g] : 0;
  const int64_t i1 = item_off ? item_off[g + 1] : n_items_dense;
  // loads in batches of eight (independent, in flight together); the sum stays ascending
  const float *src = partial + b * 256 + e;
  const int64_t stride = nb * 256;
  float s = 0.0f;
  int64_t it = i0;
  for (; it + 8 <= i1; it += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[(it + k) * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; it < i1; ++it) s += src[it * stride];
  float *out = H + (g * nb + b) * 256 + e;
  *out = accumulate ? *out + s : s;
}

int launch_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                         const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                         float *H, int accumulate, void *workspace, hipStream_t st) {
  const bool grouped = group_offsets != nullptr;
  const int64_t nb = cols / 16;
  const int64_t items = hess_items_max(tokens, groups, grouped ? n_ids : -1, grouped);
  const int64_t tc = hess_chunk(grouped ? n_ids : tokens, grouped);
  int32_t *item_off = nullptr;
  char *ws = static_cast<char *>(workspace);
  if (grouped) item_off = reinterpret_cast<int32_t *>(ws);
  float *partial = reinterpret_cast<float *>(ws + align256(sizeof(int32_t) * (size_t)(groups + 1)));
  if (grouped)
    hipLaunchKernelGGL(k_hess_items, dim3(1), dim3(256), 0, st, group_offsets, groups, n_ids, tc,
                       items, item_off);
  if (items > 0) {
    const dim3 g((unsigned)(items * ((cols + HC - 1) / HC))), b(256);
    const int64_t cw = HC * (grouped ? HW_GROUPED : HW_DENSE);
    const dim3 gb((unsigned)(items * ((cols + cw - 1) / cw)));
    if (dtype == NVFP4_DTYPE_BF16) {
      const uint16_t *xb = static_cast<const uint16_t *>(x);
      if (grouped)
        hipLaunchKernelGGL((k_hess_bf16<true, HW_GROUPED>), gb, b, 0, st, xb, tokens, cols, groups,
                           group_offsets, token_ids, n_ids, item_off, tc, partial, nb);
      else
        hipLaunchKernelGGL((k_hess_bf16<false, HW_DENSE>), gb, b, 0, st, xb, tokens, cols, groups, nullptr,
                           nullptr, n_ids, nullptr, tc, partial, nb);
    } else {
      const float *xf = static_cast<const float *>(x);
      if (grouped)
        hipLaunchKernelGGL(k_hess_f32<true>, g, b, 0, st, xf, tokens, cols, groups, group_offsets,
                           token_ids, n_ids, item_off, tc, partial, nb);
      else
        hipLaunchKernelGGL(k_hess_f32<false>, g, b, 0, st, xf, tokens, cols, groups, nullptr,
                           nullptr, n_ids, nullptr, tc, partial, nb);
    }
  }
  hipLaunchKernelGGL(k_hess_reduce, dim3((unsigned)nb, (unsigned)groups), dim3(256), 0, st,
                     partial, item_off, items, nb, H, accumulate);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ routing groups
//
// A stable counting sort of the (token, slot) pairs of the routing table by expert: pair
// i = t * topk + k keeps its flattened order within its expert, so each expert lists its
// tokens in ascending order (a token routed twice to one expert appears twice). Pairs are
// cut into chunks of 32 W; per chunk, an LDS bitmap per expert marks the chunk's pairs routed
// there, and a pair's rank among them is a popcount of the bits below it.
//  1. k_route_count: per (chunk, expert) counts, from LDS counters;
//  2. k_route_scan: one workgroup turns them into per-expert offsets and per-(chunk,
//     expert) bases (experts in blocks of up to 1024, chunks split into segments);
//  3. k_route_scatter: every pair writes its token at base + rank.

static inline int route_words(int64_t experts) {
  int64_t w = 16384 / (experts > 0 ? experts : 1);
  return (int)(w > 64 ? 64 : (w < 1 ? 1 : w));
}

static inline int64_t route_chunks(int64_t pairs, int64_t experts) {
  const int64_t cp = 32 * (int64_t)route_words(experts);
  return (pairs + cp - 1) / cp;
}

size_t route_workspace_size(int64_t tokens, int64_t topk, int64_t experts) {
  const int64_t chunks = route_chunks(tokens * topk, experts);
  return sizeof(int32_t) * (size_t)(chunks > 0 ? chunks : 1) * (size_t)(experts > 0 ? experts : 1);
}

__global__ void __launch_bounds__(256)
    k_route_count(const int32_t *__restrict__ ids, int64_t pairs, int E, int64_t cp,
                  int32_t *__restrict__ counts) {
  extern __shared__ unsigned cnt[];
  const int64_t chunk = blockIdx.x, i0 = chunk * cp;
  const int64_t n = min(cp, pairs - i0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0u;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i0 + i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1u);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[chunk * E + e] = (int32_t)cnt[e];
}

// One workgroup of 1024 threads. For a block of EB experts, thread (e, s) owns expert e and
// segment s of the chunks; counts are replaced by the base of each (chunk, expert) in
// token_ids and offsets[e] gets the start of expert e.
__global__ void __launch_bounds__(1024)
    k_route_scan(int32_t *__restrict__ counts, int64_t chunks, int E, int32_t *__restrict__ offsets) {
  __shared__ int32_t part[1024];
  __shared__ int32_t tot[1024];
  __shared__ int32_t carry;
  const int t = threadIdx.x;
  const int EB = E < 1024 ? E : 1024;
  const int SEG = 1024 / EB;
  const int64_t L = (chunks + SEG - 1) / SEG;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += EB) {
    const int el = t % EB, sg = t / EB, e = e0 + el;
    const bool on = sg < SEG && e < E;
    const int64_t c0 = sg * L, c1 = min(chunks, c0 + L);
    int32_t sum = 0;
    if (on) {
      int64_t c = c0;
      for (; c + 8 <= c1; c += 8) {
        int32_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = counts[(c + k) * E + e];
#pragma unroll
        for (int k = 0; k < 8; ++k) sum += v[k];
      }
      for (; c < c1; ++c) sum += counts[c * E + e];
    }
    part[t] = sum;
    __syncthreads();
    // per-expert totals and the exclusive prefix of this thread's segment
    int32_t pre = 0, all = 0;
    if (on) {
      for (int k = 0; k < SEG; ++k) {
        const int32_t v = part[k * EB + el];
        if (k < sg) pre += v;
        all += v;
      }
    }
    if (sg == 0) tot[el] = on ? all : 0;
    __syncthreads();
    // inclusive scan of the block's expert totals (Hillis-Steele over EB entries)
    for (int off = 1; off < EB; off <<= 1) {
      const int32_t v = (t < EB && t >= off) ? tot[t - off] : 0;
      __syncthreads();
      if (t < EB) tot[t] += v;
      __syncthreads();
    }
    if (on) {
      const int32_t ebase = carry + (el > 0 ? tot[el - 1] : 0);
      if (sg == 0) offsets[e] = ebase;
      int32_t run = ebase + pre;
      for (int64_t c = c0; c < c1; ++c) {
        const int32_t v = counts[c * E + e];
        counts[c * E + e] = run;
        run += v;
      }
    }
    __syncthreads();
    if (t == 0) carry += tot[EB - 1];
    __syncthreads();
  }
  if (t == 0) offsets[E] = carry;
}

__global__ void __launch_bounds__(256)
    k_route_scatter(const int32_t *__restrict__ ids, int64_t pairs, int topk, int E, int W,
                    const int32_t *__restrict__ base, int32_t *__restrict__ token_ids) {
  extern __shared__ unsigned bm[];
  const int64_t chunk = blockIdx.x, cp = 32 * (int64_t)W, i0 = chunk * cp;
  const int n = (int)min(cp, pairs - i0);
  for (int i = threadIdx.x; i < E * W; i += blockDim.x) bm[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i0 + i];
    if (e >= 0 && e < E) atomicOr(&bm[e * W + (i >> 5)], 1u << (i & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i0 + i];
    if (e < 0 || e >= E) continue;
    const int wd = i >> 5;
    const unsigned *row = bm + e * W;
    int rank = __popc(row[wd] & ((1u << (i & 31)) - 1u));
    for (int w = 0; w < wd; ++w) rank += __popc(row[w]);
    token_ids[base[chunk * E + e] + rank] = (int32_t)((i0 + i) / topk);
  }
}

int launch_route_groups(const int32_t *expert_ids, int64_t tokens, int64_t topk, int64_t experts,
                        int32_t *offsets, int32_t *token_ids, void *workspace, hipStream_t st) {
  const int E = (int)experts, W = route_words(experts);
  const int64_t pairs = tokens * topk, cp = 32 * (int64_t)W;
  const int64_t chunks = route_chunks(pairs, experts);
  int32_t *counts = static_cast<int32_t *>(workspace);
  if (chunks > 0)
    hipLaunchKernelGGL(k_route_count, dim3((unsigned)chunks), dim3(256), sizeof(unsigned) * E, st,
                       expert_ids, pairs, E, cp, counts);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, st, counts, chunks, E, offsets);
  if (chunks > 0)
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)chunks), dim3(256),
                       sizeof(unsigned) * (size_t)E * (size_t)W, st, expert_ids, pairs, (int)topk,
                       E, W, counts, token_ids);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

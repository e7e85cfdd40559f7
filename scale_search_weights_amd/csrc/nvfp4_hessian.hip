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
// The grouped form in bf16 (per-expert H from routed token lists) normally runs its own
// kernels, k_hess_plan and k_hess_grouped (below), which serve the rows the experts share
// from L2; k_hess_bf16's gathered form remains for inputs too large for their 32-bit
// offsets. bf16 x bf16 products are exact in fp32; only the accumulation rounds.
#include <utility>

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

// Grouped form, bf16 (k_hess_plan + k_hess_grouped): each group's token list is cut into
// interleaved pieces of at most P positions (positions k, k + m, k + 2m, ... for m pieces),
// so every piece spans the whole token range evenly; the pieces are dealt to GV_G piece
// groups, longest first, in rounds of GV_G (at most GV_NV pieces per group).
constexpr int GV_G = 32;       // piece groups per channel chunk
constexpr int GV_NV = 8;       // pieces per group (accumulators per wave)
constexpr int GV_SLOTS = GV_G * GV_NV;
constexpr int GV_NW = 4;       // windows each piece is walked in
constexpr int GV_NWMAX = 16;   // (segment table: windows x pieces per group)
constexpr int GV_DEPTH = 2;    // steps whose rows are in flight

// positions per piece for the grouped plan: at least 2048, and few enough pieces to fit
static inline int64_t gv_piece(int64_t groups, int64_t n_ids) {
  const int64_t room = GV_SLOTS - groups;  // pieces beyond one per group
  int64_t p = room > 0 ? (n_ids + room - 1) / room : n_ids + 1;
  const int64_t even = (n_ids + 2 * GV_G - 1) / (2 * GV_G);  // about half a group's share
  p = p > even ? p : even;
  return p > 2048 ? p : 2048;
}

// the grouped kernel addresses X and the id list through 32-bit buffer offsets
static inline bool gv_usable(int64_t tokens, int64_t cols, int64_t groups, int64_t n_ids) {
  return groups > 0 && groups < GV_SLOTS && n_ids > 0 && tokens * cols * 2 < 0xFFFFFF00ll &&
         n_ids * 4 < 0xFFFFFF00ll;
}

static inline size_t gv_plan_bytes() { return align256(sizeof(int32_t) * GV_SLOTS * 5); }

size_t hessian_workspace_size(int64_t tokens, int64_t cols, int64_t groups, int64_t n_ids) {
  const bool grouped = n_ids >= 0;
  const int64_t items = hess_items_max(tokens, groups, n_ids, grouped);  // >= the plan's pieces
  const int64_t nb = cols / 16;
  return align256(sizeof(int32_t) * (size_t)(groups + 1)) + (grouped ? gv_plan_bytes() : 0) +
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

// ------------------------------------------------------------------ grouped form, bf16
//
// The grouped Hessian gathers every routed row, 8x the rows of X at top-8 routing; this form
// makes the experts that share a token row read it from the same L2 at about the same time.
// k_hess_plan (one workgroup) cuts each group's list into interleaved pieces, so a piece's
// positions spread evenly over the token range, and deals them to GV_G piece groups, longest
// first, in rounds (balanced within ~1% at the MoE configuration, as close as a piece-by-piece
// longest-processing-time deal there). item_off[g] is the first piece of group g (the
// reduce adds a group's pieces in order; a group of one piece is written straight into H).
// plan[slot] = (group, k, m, n_pieces_positions, piece index), slot = piece_group * GV_NV + j;
// n = -1 marks an empty slot.
__global__ void __launch_bounds__(256)
    k_hess_plan(const int32_t *__restrict__ offsets, int64_t groups, int64_t n_ids, int64_t P,
                int32_t *__restrict__ item_off, int32_t *__restrict__ plan) {
  __shared__ int32_t n_g[GV_SLOTS], m_g[GV_SLOTS], first[GV_SLOTS + 1];
  __shared__ __attribute__((aligned(16))) int32_t vsize[GV_SLOTS];
  __shared__ int32_t vgrp[GV_SLOTS], vorder[GV_SLOTS], slot_of[GV_SLOTS];
  __shared__ __attribute__((aligned(16))) int32_t gload[GV_G];
  const int t = threadIdx.x;
  for (int g = t; g < groups; g += blockDim.x) {
    int64_t a = offsets[g], b = offsets[g + 1];
    a = a < 0 ? 0 : (a > n_ids ? n_ids : a);
    b = b < a ? a : (b > n_ids ? n_ids : b);
    n_g[g] = (int32_t)(b - a);
    m_g[g] = (int32_t)((b - a + P - 1) / P);
  }
  for (int i = t; i < GV_SLOTS * 5; i += blockDim.x) plan[i] = (i % 5 == 3) ? -1 : 0;
  __syncthreads();
  if (t < 64) {  // first[g]: pieces of the groups before g (a scan over 64 groups at a time)
    int carry = 0;
    for (int c0 = 0; c0 < groups; c0 += 64) {
      const int g = c0 + t, mine = g < groups ? m_g[g] : 0;
      int inc = mine;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        inc += t >= d ? o : 0;
      }
      if (g < groups) first[g] = carry + inc - mine;
      carry += __shfl(inc, 63, 64);
    }
    if (t == 0) first[groups] = carry;  // <= GV_SLOTS by the choice of P
  }
  __syncthreads();
  const int V = first[groups];
  for (int g = t; g <= groups; g += blockDim.x) item_off[g] = first[g];
  for (int v = t; v < V; v += blockDim.x) {
    int lo = 0, hi = (int)groups;  // last group with first[g] <= v
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (first[mid] <= v) lo = mid;
      else hi = mid;
    }
    while (lo + 1 < groups && first[lo + 1] <= v) ++lo;  // skip groups with no pieces
    const int k = v - first[lo], m = m_g[lo];
    vgrp[v] = lo;
    vsize[v] = (n_g[lo] - k + m - 1) / m;  // >= 1
  }
  for (int v = V + t; v < GV_SLOTS; v += blockDim.x) vsize[v] = -1;
  __syncthreads();
  for (int v = t; v < V; v += blockDim.x) {  // rank: longest first, then piece order
    const int sv = vsize[v];
    int r = 0;
#pragma unroll 4
    for (int u = 0; u < V; u += 4) {  // u + 3 < GV_SLOTS; sizes past V are -1, never counted
      const int4 q = *reinterpret_cast<const int4 *>(vsize + u);
      r += (q.x > sv) | ((q.x == sv) & (u < v));
      r += (q.y > sv) | ((q.y == sv) & (u + 1 < v));
      r += (q.z > sv) | ((q.z == sv) & (u + 2 < v));
      r += (q.w > sv) | ((q.w == sv) & (u + 3 < v));
    }
    vorder[r] = v;
  }
  __syncthreads();
  // Deal in rounds of GV_G pieces: round r gives the pieces ranked GV_G r .. GV_G r + GV_G - 1
  // (longest first) to the piece groups in increasing order of load (ties to the lower
  // group), so a group takes at most one piece a round, GV_NV in all (V <= GV_SLOTS).
  int load = 0;  // thread q < GV_G: piece group q's load (<= n_ids < 2^30)
  for (int r0 = 0, rnd = 0; r0 < V; r0 += GV_G, ++rnd) {
    if (t < GV_G) gload[t] = load;
    __syncthreads();
    if (t < GV_G) {
      int rank = 0;
#pragma unroll
      for (int q = 0; q < GV_G; q += 4) {
        const int4 l4 = *reinterpret_cast<const int4 *>(gload + q);
        rank += (l4.x < load || (l4.x == load && q < t)) ? 1 : 0;
        rank += (l4.y < load || (l4.y == load && q + 1 < t)) ? 1 : 0;
        rank += (l4.z < load || (l4.z == load && q + 2 < t)) ? 1 : 0;
        rank += (l4.w < load || (l4.w == load && q + 3 < t)) ? 1 : 0;
      }
      const int i = r0 + rank;
      if (i < V) {
        slot_of[i] = t * GV_NV + rnd;
        load += vsize[vorder[i]];
      }
    }
    __syncthreads();
  }
  for (int i = t; i < V; i += blockDim.x) {
    const int v = vorder[i], g = vgrp[v];
    int32_t *e = plan + slot_of[i] * 5;
    e[0] = g;
    e[1] = v - first[g];
    e[2] = m_g[g];
    e[3] = vsize[v];
    e[4] = v;
  }
}

// One workgroup per (64-channel chunk, piece group): wave w owns block w of the chunk and one
// 16x16 accumulator per piece of the group (one live, swapped in registers when the piece
// changes). The workgroup walks window after window; in each window it takes, piece by
// piece, the piece's positions that fall in the window (its next 1/NW, rounded to whole
// 32-token steps; a segment table in LDS holds each window's share of each piece).
// Workgroups are numbered so that one XCD runs all the piece groups of its chunks: they walk
// the token range in step, so a token row's chunk segment is read from memory once and
// served to its other experts from that XCD's L2.
//
// Loads go straight into LDS (raw buffer loads with an LDS destination, no registers), so
// several steps are in flight without the register moves that would make the compiler wait
// for each load: the 32 rows' 128-byte segments of step i + 2 go into stage (i + 2) % 4 (wave
// w loads rows 8w..8w+7, lane l row 8w + l/8, segment (l % 8) ^ 2(row % 4), a swizzle that
// lets each 16-lane transposed read hit distinct banks), and each wave's list ids of step
// i + 4 into its own id slot i % 4. Waits are explicit vector-memory counts. A row past the
// step's end, or with an id outside [0, tokens), gets an out-of-range offset and reads as
// zeros. Each wave reads its block's operand transposed (ds_read_tr16_b64: lane i of a
// 16-lane group gets 4 consecutive tokens of channel i) for one v_mfma_f32_16x16x32_bf16
// with the same register as A and B.
#define HESS_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))

template <int D>
__global__ void __launch_bounds__(256)
    k_hess_grouped(const uint16_t *__restrict__ x, int64_t tokens, int64_t cols,
                   const int32_t *__restrict__ offsets, const int32_t *__restrict__ ids,
                   int64_t n_ids, const int32_t *__restrict__ plan, int NW,
                   float *__restrict__ partial, int64_t nb, float *__restrict__ H, int accumulate) {
  constexpr int SB = HT * 2 * HC;  // stage bytes: 32 rows x 128 bytes
  constexpr int NR = D + 2;        // ring slots: stages and id slots
  static_assert(NR <= 6, "ring of at most six slots");
  // one array per ring slot, so the compiler sees that loads into one slot never alias reads
  // of another and inserts no waits of its own
  __shared__ __attribute__((aligned(16))) unsigned char st0[SB], st1[SB], st2[SB], st3[SB],
      st4[NR > 4 ? SB : 16], st5[NR > 5 ? SB : 16];
  __shared__ __attribute__((aligned(16))) int32_t id0[256], id1[256], id2[256], id3[256],
      id4[NR > 4 ? 256 : 4], id5[NR > 5 ? 256 : 4];
  __shared__ int32_t sp[GV_NV][5];
  __shared__ long long sbase[GV_NV];
  const int64_t nch = (cols + HC - 1) / HC, n_wg = nch * GV_G;
  int64_t wid = blockIdx.x;
  if ((n_wg & 7) == 0) wid = (wid & 7) * (n_wg >> 3) + (wid >> 3);
  const int64_t c = wid / GV_G;
  const int pg = (int)(wid % GV_G);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  if (t < GV_NV * 5) sp[t / 5][t % 5] = plan[pg * GV_NV * 5 + t];
  __syncthreads();
  if (t < GV_NV && sp[t][3] >= 0) {
    int64_t a = offsets[sp[t][0]];
    a = a < 0 ? 0 : (a > n_ids ? n_ids : a);
    sbase[t] = a + sp[t][1];
  }
  int ns = 0;
#pragma unroll
  for (int j = 0; j < GV_NV; ++j) ns += sp[j][3] >= 0 ? 1 : 0;
  ns = __builtin_amdgcn_readfirstlane(ns);
  if (ns == 0) return;
  __syncthreads();

  // Segment table: segment g = w * ns + j holds the positions of piece j that fall in window
  // w, its share of the first w + 1 windows rounded down to whole steps (the last window
  // takes the rest, so every step of a piece but its last is full): the list index of its
  // first position, its stride (the piece count m of its group) and its length. Built once,
  // it makes each step a cursor increment.
  __shared__ int32_t seg_pos[GV_NWMAX * GV_NV], seg_len[GV_NWMAX * GV_NV], seg_mj[GV_NWMAX * GV_NV];
  const int nseg = NW * ns;
  if (t < nseg) {
    const int w = t / ns, j = t % ns;
    const int64_t n = sp[j][3];
    auto bound = [&](int ww) -> int64_t {
      if (ww < 0) return 0;
      if (ww >= NW - 1) return n;
      return (int64_t)HT * (((int64_t)(ww + 1) * n / NW) / HT);
    };
    const int64_t lo = bound(w - 1), hi = bound(w);
    seg_pos[t] = (int32_t)(sbase[j] + (int64_t)sp[j][2] * lo);  // < n_ids
    seg_len[t] = (int32_t)(hi - lo);
    seg_mj[t] = sp[j][2] * 8 + j;
  }
  __syncthreads();
  // a step: slot j, rows cnt (0 after the last step), list index pos of its first row, stride m
  struct Step {
    int j, cnt, pos, m;
  };
  // cursor: segment sg, its rows left and the list index of its next step (uniform)
  int sg = -1, left = 0, pos = 0, mj = 0;
  auto next = [&]() -> Step {
    while (left <= 0) {
      if (sg + 1 >= nseg) return Step{0, 0, 0, 0};
      ++sg;
      left = __builtin_amdgcn_readfirstlane(seg_len[sg]);
      pos = __builtin_amdgcn_readfirstlane(seg_pos[sg]);
      mj = __builtin_amdgcn_readfirstlane(seg_mj[sg]);
    }
    const int m = mj >> 3;
    const Step st{mj & 7, left < HT ? left : HT, pos, m};
    left -= HT;
    pos += m * HT;
    return st;
  };

  const int r = 8 * wave + (lane >> 3);              // this lane's token row in a step
  const int q = (lane & 7) ^ (2 * (r & 3));           // the row segment it loads (swizzled)
  const int64_t ch = c * HC + q * 8;
  const uint32_t OOR = 0xFFFFFFF0u;                   // an offset past both buffers' ranges
  const int64_t xbytes = tokens * cols * 2;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), (short)0, (int)(uint32_t)xbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(ids), (short)0, (int)(uint32_t)(n_ids * 4), 0x00020000);
  typedef __attribute__((address_space(3))) void lds_void;
  // the list ids of step s for this wave's rows (each lane: its row's id) -> id slot
  auto load_ids = [&](const Step &s, int32_t *slot) {
    const uint32_t off = r < s.cnt ? (uint32_t)(s.pos + s.m * r) * 4u : OOR;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ir, (lds_void *)(slot + 64 * wave), 4, off, 0, 0, 0);
  };
  // the rows of step s (ids already in the slot) -> stage
  auto load_rows = [&](const Step &s, const int32_t *slot, unsigned char *stage) {
    const int32_t tok = slot[64 * wave + lane];
    const bool ok = r < s.cnt && tok >= 0 && tok < tokens && ch < cols;
    const uint32_t off = ok ? ((uint32_t)tok * (uint32_t)cols + (uint32_t)ch) * 2u : OOR;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(stage + 1024 * wave), 16, off, 0, 0, 0);
  };
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  // operand read: lane (group G, r16) reads row 8G + r16/4 (+4) at channel group r16 % 4 of
  // block `wave`, i.e. segment 2 wave + (r16 % 4)/2, byte 8 ((r16 % 4) & 1)
  const int rrow = 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int m4 = lane & 3;
  const int seg = 2 * wave + (m4 >> 1);
  const int rd0 = rrow * 128 + ((seg ^ (2 * (rrow & 3))) * 16) + (m4 & 1) * 8;
  const int rd1 = (rrow + 4) * 128 + ((seg ^ (2 * ((rrow + 4) & 3))) * 16) + (m4 & 1) * 8;

  // one accumulator per piece; the current piece's is `cur`, swapped when the piece changes
  // (once per segment, every few steps)
  v4f acc[GV_NV];
#pragma unroll
  for (int j = 0; j < GV_NV; ++j) acc[j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  v4f cur = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  int curj = 0;
  auto mfma_step = [&](const Step &s, const unsigned char *stage) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(stage + rd0));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(stage + rd1));
    const v4s pr[2] = {lo, hi};
    const v8bf a = __builtin_bit_cast(v8bf, pr);
    const int j = __builtin_amdgcn_readfirstlane(s.j);
    if (j != curj) {
#pragma unroll
      for (int jj = 0; jj < GV_NV; ++jj)
        if (jj == curj) acc[jj] = cur;
#pragma unroll
      for (int jj = 0; jj < GV_NV; ++jj)
        if (jj == j) cur = acc[jj];
      curj = j;
    }
    cur = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, cur, 0, 0, 0);
  };

  // ring slot k of stages and id slots (compile-time k)
  auto stage_at = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) return st0;
    else if constexpr (k == 1) return st1;
    else if constexpr (k == 2) return st2;
    else if constexpr (k == 3) return st3;
    else if constexpr (k == 4) return st4;
    else return st5;
  };
  auto idslot_at = [&](auto kc) -> int32_t * {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) return id0;
    else if constexpr (k == 1) return id1;
    else if constexpr (k == 2) return id2;
    else if constexpr (k == 3) return id3;
    else if constexpr (k == 4) return id4;
    else return id5;
  };
  // steps i .. i + 2D (uniform): S[0] is multiplied; S[1..D-1] have rows in flight or
  // landed; S[D..2D-1] have ids in flight or landed; S[2D] is next. The rows of step j go
  // to ring slot j % NR, its ids to id slot j % NR, loaded D steps before its rows.
  Step S[2 * D + 1];
#pragma unroll
  for (int i = 0; i < 2 * D + 1; ++i) S[i] = next();
  // prologue, leaving the loop's order in flight: ids of steps 0..D-1 (landed), then
  // rows k, ids D + k for k = 0..D-1
  [&]<int... k>(std::integer_sequence<int, k...>) {
    (load_ids(S[k], idslot_at(std::integral_constant<int, k % NR>{})), ...);
  }(std::make_integer_sequence<int, D>{});
  HESS_WAIT_VM(0);
  [&]<int... k>(std::integer_sequence<int, k...>) {
    ((load_rows(S[k], idslot_at(std::integral_constant<int, k % NR>{}),
                stage_at(std::integral_constant<int, k % NR>{})),
      load_ids(S[D + k], idslot_at(std::integral_constant<int, (D + k) % NR>{}))), ...);
  }(std::make_integer_sequence<int, D>{});
  // one step i (ring position u = i % NR): the ids of step i + D have landed when at most
  // 2D - 2 vector-memory ops are younger (the rows and ids of steps i + 1 .. i + D - 1 and
  // i + D + 1 .. i + 2D - 1), which also completes this wave's rows of step i; issue the rows
  // of step i + D and the ids of step i + 2D; barrier; multiply step i
  bool done = false;
  auto one = [&](auto uc) {
    constexpr int u = decltype(uc)::value;
    if (done) return;
    HESS_WAIT_VM(2 * D - 2);
    load_rows(S[D], idslot_at(std::integral_constant<int, (u + D) % NR>{}),
              stage_at(std::integral_constant<int, (u + D) % NR>{}));
    load_ids(S[2 * D], idslot_at(std::integral_constant<int, (u + 2 * D) % NR>{}));
    __builtin_amdgcn_s_barrier();
    mfma_step(S[0], stage_at(std::integral_constant<int, u>{}));
    const Step sn = next();
#pragma unroll
    for (int i = 0; i < 2 * D; ++i) S[i] = S[i + 1];
    S[2 * D] = sn;
    done = S[0].cnt == 0;
  };
  while (S[0].cnt > 0 && !done) {
    [&]<int... u>(std::integer_sequence<int, u...>) {
      (one(std::integral_constant<int, u>{}), ...);
    }(std::make_integer_sequence<int, NR>{});
  }
  HESS_WAIT_VM(0);  // no load may land in LDS after the workgroup ends
#pragma unroll
  for (int jj = 0; jj < GV_NV; ++jj)
    if (jj == curj) acc[jj] = cur;
  const int64_t b = c * (HC / 16) + wave;
  if (b < nb) {
    const int col = lane & 15, row0 = (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < GV_NV; ++j) {
      if (j < ns) {
        if (sp[j][2] == 1) {  // the group's only piece: its H block directly
          float *P = H + ((int64_t)sp[j][0] * nb + b) * 256;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float *o = P + (row0 + k) * 16 + col;
            *o = accumulate ? *o + acc[j][k] : acc[j][k];
          }
        } else {
          float *P = partial + ((int64_t)sp[j][4] * nb + b) * 256;
#pragma unroll
          for (int k = 0; k < 4; ++k) P[(row0 + k) * 16 + col] = acc[j][k];
        }
      }
    }
  }
}
#undef HESS_WAIT_VM

// H[g][b][e] (+)= sum of partial[it][b][e] over the group's items, ascending. With
// skip_single, a group of one item is left alone: the grouped kernel wrote its H directly.
__global__ void __launch_bounds__(256)
    k_hess_reduce(const float *__restrict__ partial, const int32_t *__restrict__ item_off,
                  int64_t n_items_dense, int64_t nb, float *__restrict__ H, int accumulate,
                  int skip_single) {
  const int64_t b = blockIdx.x, g = blockIdx.y, e = threadIdx.x;
  const int64_t i0 = item_off ? item_off[g] : 0;
  const int64_t i1 = item_off ? item_off[g + 1] : n_items_dense;
  if (skip_single && i1 - i0 == 1) return;  // written by the product kernel
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
  int32_t *plan = reinterpret_cast<int32_t *>(ws + align256(sizeof(int32_t) * (size_t)(groups + 1)));
  float *partial = reinterpret_cast<float *>(reinterpret_cast<char *>(plan) +
                                             (grouped ? gv_plan_bytes() : 0));
  if (grouped && dtype == NVFP4_DTYPE_BF16 && gv_usable(tokens, cols, groups, n_ids)) {
    const int64_t P = gv_piece(groups, n_ids);
    const int NW = GV_NW;
    hipLaunchKernelGGL(k_hess_plan, dim3(1), dim3(256), 0, st, group_offsets, groups, n_ids, P,
                       item_off, plan);
    const int64_t nch = (cols + HC - 1) / HC;
    hipLaunchKernelGGL(k_hess_grouped<GV_DEPTH>, dim3((unsigned)(nch * GV_G)), dim3(256), 0, st,
                       static_cast<const uint16_t *>(x), tokens, cols, group_offsets, token_ids,
                       n_ids, plan, NW, partial, nb, H, accumulate);
    hipLaunchKernelGGL(k_hess_reduce, dim3((unsigned)nb, (unsigned)groups), dim3(256), 0, st,
                       partial, item_off, items, nb, H, accumulate, 1);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
  }
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
                     partial, item_off, items, nb, H, accumulate, 0);
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
//  3. k_route_scatter: every pair writes its token at base + rank (rank: a per-expert
//     prefix of the chunk's word popcounts plus one popcount).

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
    // the segment's first RK counts stay in registers for the write pass below (all read at
    // once; read again there they were a chain of dependent round trips)
    constexpr int RK = 32;
    int32_t keep[RK];
    int32_t *const seg = counts + (on ? c0 * E + e : 0);  // count c0 + k at seg[k * E]
    const int nk = on ? (int)min((int64_t)RK, c1 - c0) : 0;
#pragma unroll
    for (int k = 0; k < RK; ++k) keep[k] = k < nk ? seg[k * E] : 0;
#pragma unroll
    for (int k = 0; k < RK; ++k) sum += keep[k];
    if (on) {
      int64_t c = c0 + RK;
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
#pragma unroll
      for (int k = 0; k < RK; ++k) {
        if (k < nk) seg[k * E] = run;
        run += keep[k];
      }
      for (int64_t c = c0 + RK; c < c1; ++c) {
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
  // pre[e][w]: the expert's pairs in words 0 .. w - 1 (an exclusive scan of the words'
  // popcounts), so a pair's rank is one lookup and one popcount; a wave scans floor(64 / W)
  // experts' rows at a time, lane l holding word l % W of row l / W
  unsigned *pre = bm + E * W;
  {
    const int lane = threadIdx.x & 63, rows = 64 / W, r = lane / W, wl = lane % W;
    for (int e0 = (threadIdx.x >> 6) * rows; e0 < E; e0 += (blockDim.x >> 6) * rows) {
      const int e = e0 + r;
      const bool on = r < rows && e < E;
      const int c = on ? __popc(bm[e * W + wl]) : 0;
      int v = c;
      for (int d = 1; d < W; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        v += wl >= d ? o : 0;
      }
      if (on) pre[e * W + wl] = (unsigned)(v - c);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i0 + i];
    if (e < 0 || e >= E) continue;
    const int wd = i >> 5;
    const int rank = (int)pre[e * W + wd] + __popc(bm[e * W + wd] & ((1u << (i & 31)) - 1u));
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
                       2 * sizeof(unsigned) * (size_t)E * (size_t)W, st, expert_ids, pairs,
                       (int)topk, E, W, counts, token_ids);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

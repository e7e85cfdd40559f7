// Full Gram matrix H = X^T X of the layer input X [tokens, cols] (fp32 result).
//
// The Local-Hessian search needs only the 16x16 diagonal blocks of X X^T ([LH] "Change the
// objective"); GPTQ rounding, which the same page says combines with it, needs all of it.
// This is a dense contraction over tokens (2 T C^2 flops), so it runs on the matrix cores:
//  * only tiles on or above the diagonal are computed (256 x 256 channels each, eight
//    waves of 64 x 128); the reduction mirrors them, so H comes out exactly symmetric;
//  * tokens are split into chunks (8 to 16 for long inputs: the count whose workgroups fill
//    whole rounds best); each (chunk, tile) writes a partial tile, and k_gram_reduce adds
//    the partials in chunk order (deterministic);
//  * each XCD (with its own L2) takes a contiguous range of (chunk, tile) units and walks
//    the tiles row by row, so the workgroups running together on it share their row panel
//    and stream the same token rows (spreading every chunk over all XCDs fetched X twelve
//    times over; this fetches it about four times).
//
// bf16: v_mfma_f32_32x32x16_bf16. A lane's operand is 8 consecutive tokens of one channel,
// while a token row is contiguous in memory. The token rows go into LDS as they are (raw
// buffer loads that write LDS directly: no registers, so four 32-token stages can be in
// flight, and rows past the chunk read as zero through the descriptor's range), and the
// operands come out transposed through ds_read_b64_tr_b16 (gfx950), two reads of four
// tokens per operand. Any order of tokens inside a K slice is valid as long as both
// operands use the same one, which holds because A and B come from the same rows.
// fp32: v_mfma_f32_32x32x2_f32 straight from a [token][channel] tile (no transpose needed).
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef __bf16 gram_v8bf __attribute__((ext_vector_type(8)));
typedef float gram_v16f __attribute__((ext_vector_type(16)));

constexpr int GT = 256;   // output tile edge (channels)
constexpr int GC = 2 * GT;  // channels staged per step: the tile's row and column channels
constexpr int GK = 64;    // token granularity of the chunks (bf16)
constexpr int GKF = 32;   // tokens per step, fp32
constexpr int GTHREADS = 512;  // 8 waves: 4 x 2 quarters of 64 x 128

struct GramGeom {
  int64_t nt, tiles, nc, tc;
};

static int gram_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

constexpr int GXCD = 8;  // XCDs; workgroups are dispatched to them round-robin

// Token chunks per tile: for long inputs (chunks of at least 2048 tokens possible) the count
// in 8..16 whose workgroups fill whole rounds of one per CU best (the time is about the
// rounds times a round's length, which falls as 1/chunks; 15 chunks of 136 tiles make 8
// full rounds where 16 made 8.5); else as many as fill whole rounds of one workgroup per CU
// best; one when the tiles alone number four per CU.
static GramGeom gram_geom(int64_t tokens, int64_t cols, int cus) {
  GramGeom g;
  g.nt = (cols + GT - 1) / GT;
  g.tiles = g.nt * (g.nt + 1) / 2;
  const int64_t steps = (tokens + GK - 1) / GK;
  int64_t max_nc = steps / 32;
  if (max_nc > 16) max_nc = 16;
  // with at least four tiles per CU the tiles alone fill the device: no token split (which
  // would multiply the partial-tile workspace without adding useful parallelism)
  if (g.tiles >= 4 * (int64_t)cus) max_nc = 1;
  if (max_nc < 1) max_nc = 1;
  int64_t best = 1;
  double best_t = -1.0;
  if (max_nc >= 8) {
    for (int64_t nc = 8; nc <= max_nc; ++nc) {
      const double t = (double)((g.tiles * nc + cus - 1) / cus) / (double)nc;
      if (best_t < 0.0 || t < best_t - 1e-12) {
        best_t = t;
        best = nc;
      }
    }
  } else {
    double best_eff = -1.0;
    for (int64_t nc = 1; nc <= max_nc; ++nc) {
      const int64_t wgs = g.tiles * nc;
      const int64_t rounds = (wgs + cus - 1) / cus;
      const double eff = (double)wgs / (double)(rounds * cus);
      if (eff > best_eff + 1e-9) {
        best_eff = eff;
        best = nc;
      }
    }
  }
  const int64_t spc = (steps + best - 1) / best > 0 ? (steps + best - 1) / best : 1;
  g.tc = spc * GK;
  g.nc = tokens > 0 ? (tokens + g.tc - 1) / g.tc : 1;
  return g;
}

// workgroup -> (token chunk, tile): the (chunk, tile) units in chunk-major order, tiles row
// by row, are cut into GXCD contiguous ranges, and XCD x (= wid % GXCD) walks range x, so
// the workgroups running together on an XCD share their row panel and stream the same token
// rows. A workgroup past the last unit gets chunk >= nc and returns.
__device__ __forceinline__ void gram_work(int64_t wid, int64_t tiles, int64_t nc, int64_t &chunk,
                                          int64_t &tile) {
  const int64_t per = (nc * tiles + GXCD - 1) / GXCD;
  const int64_t u = (wid % GXCD) * per + wid / GXCD;
  chunk = u / tiles;
  tile = u % tiles;
}

static int64_t gram_grid(const GramGeom &g) {
  return GXCD * ((g.nc * g.tiles + GXCD - 1) / GXCD);
}

size_t gram_workspace_size(int64_t tokens, int64_t cols) {
  const GramGeom g = gram_geom(tokens, cols, gram_cus());
  return sizeof(float) * (size_t)g.nc * (size_t)g.tiles * GT * GT;
}

// upper-triangle tile index -> (ti, tj), ti <= tj, row by row
__device__ __forceinline__ void gram_tile(int64_t t, int64_t nt, int64_t &ti, int64_t &tj) {
  int64_t i = 0;
  while (t >= nt - i) {
    t -= nt - i;
    ++i;
  }
  ti = i;
  tj = i + t;
}

// bf16 staging: 32-token stages in four LDS buffers, three stages in flight. A stage holds
// its token rows as they lie in memory (the tile's 256 row channels, then its 256 column
// channels: 1 KiB) at a pitch of GROWB bytes; the 64-byte pad puts the four token rows a
// transposing read touches at bank offsets 0, 16, 32, 48, so the two 16-lane groups of a
// read pass (channels 16 apart) use disjoint banks.
constexpr int GK2 = 32;                  // tokens per stage
constexpr int GNST = 4;                  // stages in LDS
constexpr int GROWB = 2 * GC + 64;       // bytes per staged token row
constexpr int GSTAGE = GK2 * GROWB;      // bytes per stage

// s_waitcnt with only the vector-memory count N (expcnt and lgkmcnt left at their maxima)
#define GRAM_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))

__global__ void __launch_bounds__(GTHREADS)
    k_gram_bf16(const uint16_t *__restrict__ x, int64_t tokens, int64_t cols, int64_t nt,
                int64_t tiles, int64_t nc, int64_t tc, float *__restrict__ partial) {
  // four separate arrays, so that each stage's reads wait only for the loads into it
  __shared__ __attribute__((aligned(16))) char st0[GSTAGE], st1[GSTAGE], st2[GSTAGE], st3[GSTAGE];
  int64_t chunk, tile, ti, tj;
  gram_work(blockIdx.x, tiles, nc, chunk, tile);
  if (chunk >= nc) return;
  gram_tile(tile, nt, ti, tj);
  const int64_t p0 = chunk * tc;
  const int64_t p1 = p0 + tc < tokens ? p0 + tc : tokens;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Loading: wave w stages token rows w, w + 8, w + 16, w + 24 of each stage, one row per
  // instruction (64 lanes x 16 bytes, written by the load straight into LDS at lane * 16):
  // lanes 0-31 the row tile's channels, 32-63 the column tile's. Channel groups past cols
  // load channels 0..7 (they only reach partial-tile rows and columns the reduction drops);
  // token rows past p1 have an empty descriptor range and read as zero.
  const int64_t chg = lane < 32 ? ti * GT + lane * 8 : tj * GT + (lane - 32) * 8;
  const int ch_bytes = (int)((chg < cols ? chg : 0) * 2);
  const int nst = (int)((p1 - p0 + GK2 - 1) / GK2);
  auto issue = [&](int st, char *lb) {
    const int64_t pos = p0 + (int64_t)st * GK2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = wave + 8 * i;
      const int nrec = pos + t < p1 ? (int)(cols * 2) : 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(x + (pos + t) * cols), (short)0, nrec, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(lb + t * GROWB), 16, ch_bytes, 0, 0, 0);
    }
  };

  // Operands: v_mfma_f32_32x32x16_bf16 wants, in lane l, tokens 8 (l >> 5) .. +7 of channel
  // l & 31 of the fragment. ds_read_b64_tr_b16 gives lane i of a 16-lane group element
  // i % 4 of the 8 bytes read by lanes 4k + i / 4 (k = 0..3) of the group; so lane r of
  // group G reads token row 8 (G >> 1) + r / 4 (+ 4 for the second half) at channel
  // 16 (G & 1) + 4 (r % 4) of the fragment, and receives 4 consecutive tokens of channel
  // 16 (G & 1) + r.
  const int G = lane >> 4, r = lane & 15;
  const int lane_off = (8 * (G >> 1) + (r >> 2)) * GROWB + (16 * (G & 1) + 4 * (r & 3)) * 2;
  const int wr = wave >> 1, wc = wave & 1;  // wave's 64 x 128 part of the tile
  typedef short gram_v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) gram_v4s lds_v4s;
  auto frag = [&](const char *buf, int kk, int cb) {
    const char *p = buf + lane_off + kk * 16 * GROWB + cb * 2;
    const gram_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)p);
    const gram_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p + 4 * GROWB));
    const gram_v4s v[2] = {lo, hi};
    return __builtin_bit_cast(gram_v8bf, v);
  };

  gram_v16f acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // a stage's products: all 24 operand reads first, then the 16 products
  auto compute = [&](const char *buf) {
    gram_v8bf A[GK2 / 16][2], B[GK2 / 16][4];
#pragma unroll
    for (int kk = 0; kk < GK2 / 16; ++kk) {
#pragma unroll
      for (int a = 0; a < 2; ++a) A[kk][a] = frag(buf, kk, wr * 64 + a * 32);
#pragma unroll
      for (int b = 0; b < 4; ++b) B[kk][b] = frag(buf, kk, GT + wc * 128 + b * 32);
    }
#pragma unroll
    for (int kk = 0; kk < GK2 / 16; ++kk)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[kk][a], B[kk][b], acc[a][b], 0, 0, 0);
  };
  // one stage: wait for this wave's loads of it (those of the next two may stay in flight),
  // then a bare barrier (a memory fence here would also wait for the loads still in flight;
  // the empty asm statements keep the compiler from moving memory accesses across it): every
  // wave's rows of the stage are in LDS, and every wave's reads of the previous stage have
  // completed, since its products consumed them. Then refill the previous stage's buffer
  // three stages ahead and compute.
  auto stage = [&](int st, const char *cur, char *refill) {
    const int later = nst - 1 - st;
    if (later >= 2) GRAM_WAIT_VM(8);
    else if (later == 1) GRAM_WAIT_VM(4);
    else GRAM_WAIT_VM(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + GNST - 1 < nst) issue(st + GNST - 1, refill);
    compute(cur);
  };
  if (nst > 0) issue(0, st0);
  if (nst > 1) issue(1, st1);
  if (nst > 2) issue(2, st2);
  for (int st = 0; st < nst; st += GNST) {
    stage(st, st0, st3);
    if (st + 1 < nst) stage(st + 1, st1, st0);
    if (st + 2 < nst) stage(st + 2, st2, st1);
    if (st + 3 < nst) stage(st + 3, st3, st2);
  }

  // D layout of a 32x32 MFMA: lane l, register e -> row (e & 3) + 4 (l >> 5) + 8 (e >> 2),
  // column l & 31
  float *P = partial + (chunk * tiles + tile) * (int64_t)(GT * GT);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wr * 64 + a * 32 + (e & 3) + 4 * (lane >> 5) + 8 * (e >> 2);
        const int col = wc * 128 + b * 32 + (lane & 31);
        P[row * GT + col] = acc[a][b][e];
      }
}

__global__ void __launch_bounds__(GTHREADS)
    k_gram_f32(const float *__restrict__ x, int64_t tokens, int64_t cols, int64_t nt,
               int64_t tiles, int64_t nc, int64_t tc, float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float lds[2][GKF * GC];
  int64_t chunk, tile, ti, tj;
  gram_work(blockIdx.x, tiles, nc, chunk, tile);
  if (chunk >= nc) return;
  gram_tile(tile, nt, ti, tj);
  const int64_t p0 = chunk * tc;
  const int64_t p1 = p0 + tc < tokens ? p0 + tc : tokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int q = tid & 127, r0 = tid >> 7;  // 4 channels (128 groups), token rows r0 + 4 s
  const int64_t chg = q < 64 ? ti * GT + q * 4 : tj * GT + (q - 64) * 4;
  const bool ch_ok = chg < cols;
  float4 in[8];
  auto load = [&](int64_t pos) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t tok = pos + r0 + 4 * s;
      in[s] = (ch_ok && tok < p1) ? *reinterpret_cast<const float4 *>(x + tok * cols + chg)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](float *buf) {
#pragma unroll
    for (int s = 0; s < 8; ++s) *reinterpret_cast<float4 *>(buf + (r0 + 4 * s) * GC + q * 4) = in[s];
  };

  const int wr = wave >> 1, wc = wave & 1;
  gram_v16f acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  int cur = 0;
  if (p0 < p1) {
    load(p0);
    store(lds[0]);
  }
  __syncthreads();
  for (int64_t pos = p0; pos < p1; pos += GKF) {
    const bool more = pos + GKF < p1;
    if (more) load(pos + GKF);
    const float *buf = lds[cur];
#pragma unroll 4
    for (int kk = 0; kk < GKF / 2; ++kk) {
      const float *rowp = buf + (kk * 2 + (lane >> 5)) * GC;
      float A[2], B[4];
#pragma unroll
      for (int a = 0; a < 2; ++a) A[a] = rowp[wr * 64 + a * 32 + (lane & 31)];
#pragma unroll
      for (int b = 0; b < 4; ++b) B[b] = rowp[GT + wc * 128 + b * 32 + (lane & 31)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(A[a], B[b], acc[a][b], 0, 0, 0);
    }
    if (more) store(lds[cur ^ 1]);
    lds_barrier();
    cur ^= 1;
  }

  float *P = partial + (chunk * tiles + tile) * (int64_t)(GT * GT);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * 64 + a * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        const int col = wc * 128 + b * 32 + (lane & 31);
        P[row * GT + col] = acc[a][b][r];
      }
}

// One workgroup per 32x32 piece of an upper tile: sums the chunk partials in order and
// writes the piece and its mirror image (diagonal pieces: the upper triangle, mirrored).
__global__ void __launch_bounds__(256)
    k_gram_reduce(const float *__restrict__ partial, int64_t nt, int64_t tiles, int64_t nc,
                  int64_t cols, float *__restrict__ H, int accumulate) {
  __shared__ float sm[32][33];
  const int64_t tile = blockIdx.x;
  const int pr = blockIdx.y / (GT / 32), pc = blockIdx.y % (GT / 32);  // piece within the tile
  int64_t ti, tj;
  gram_tile(tile, nt, ti, tj);
  if (ti == tj && pr > pc) return;  // covered by the mirror of (pc, pr)
  const int t = threadIdx.x;
  const int rr = t >> 3, cc = (t & 7) * 4;
  const int64_t off = (int64_t)(pr * 32 + rr) * GT + pc * 32 + cc;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t c = 0; c < nc; ++c) {
    const float4 v = *reinterpret_cast<const float4 *>(partial + (c * tiles + tile) * GT * GT + off);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  sm[rr][cc] = s.x;
  sm[rr][cc + 1] = s.y;
  sm[rr][cc + 2] = s.z;
  sm[rr][cc + 3] = s.w;
  __syncthreads();
  const int64_t I0 = ti * GT + pr * 32, J0 = tj * GT + pc * 32;
  const bool diag = (ti == tj && pr == pc);
  // direct: H[I0 + rr][J0 + cc + k]
  if (I0 + rr < cols) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = cc + k;
      if (J0 + j >= cols) continue;
      const float v = (diag && j < rr) ? sm[j][rr] : sm[rr][j];
      float *h = H + (I0 + rr) * cols + J0 + j;
      *h = accumulate ? *h + v : v;
    }
  }
  if (diag) return;
  // mirror: H[J0 + rr][I0 + cc + k] = sum[cc + k][rr]
  if (J0 + rr < cols) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = cc + k;
      if (I0 + i >= cols) continue;
      float *h = H + (J0 + rr) * cols + I0 + i;
      const float v = sm[i][rr];
      *h = accumulate ? *h + v : v;
    }
  }
}

int launch_full_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, float *H,
                        int accumulate, void *workspace, hipStream_t st) {
  const GramGeom g = gram_geom(tokens, cols, gram_cus());
  float *partial = static_cast<float *>(workspace);
  const dim3 grid((unsigned)gram_grid(g));
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_gram_bf16, grid, dim3(GTHREADS), 0, st, static_cast<const uint16_t *>(x),
                       tokens, cols, g.nt, g.tiles, g.nc, g.tc, partial);
  else
    hipLaunchKernelGGL(k_gram_f32, grid, dim3(GTHREADS), 0, st, static_cast<const float *>(x),
                       tokens, cols, g.nt, g.tiles, g.nc, g.tc, partial);
  hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)g.tiles, (GT / 32) * (GT / 32)), dim3(256), 0,
                     st, partial, g.nt, g.tiles, g.nc, cols, H, accumulate);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

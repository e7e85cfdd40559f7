// Full Gram matrix H = X^T X of the layer input X [tokens, cols] (fp32 result).
//
// The Local-Hessian search needs only the 16x16 diagonal blocks of X X^T ([LH] "Change the
// objective"); GPTQ rounding, which the same page says combines with it, needs all of it.
// This is a dense contraction over tokens (2 T C^2 flops), so it runs on the matrix cores:
//  * only tiles on or above the diagonal are computed (256 x 256 channels each, eight
//    waves of 64 x 128); the reduction mirrors them, so H comes out exactly symmetric;
//  * tokens are split into chunks (16 or 8 for long inputs); each (chunk, tile) writes a
//    partial tile, and k_gram_reduce adds the partials in chunk order (deterministic);
//  * each XCD (with its own L2) takes whole chunks and walks their tiles row by row, so
//    the workgroups running together on it share their row panel and stream the same
//    token rows (spreading every chunk over all XCDs fetched X twelve times over; this
//    fetches it about four times).
//
// bf16: v_mfma_f32_32x32x16_bf16. A lane's operand is 8 consecutive tokens of one channel,
// while a token row is contiguous in memory, so each step (64 tokens x 512 channels: the
// tile's row and column channels) is transposed on the way into LDS: a lane loads 8 token
// rows x 8 channels (eight 16-byte raw buffer loads from scalar descriptors, no address
// arithmetic per load, rows past the chunk zero-filled by the range check), transposes the
// 8x8 block of 16-bit values in registers (32 byte permutes) and writes eight 16-byte
// channel rows. LDS rows are 128 bytes (64 tokens); the
// 16-byte token groups are XOR-swizzled by (c ^ c >> 3) & 7 so that both the transposing
// writes (8 lanes = 8 channels 8 apart) and the MFMA reads (8 lanes = 8 adjacent channels)
// touch 8 distinct bank groups. Any order of tokens inside a K slice is valid as long as
// both operands use the same one, which holds because A and B come from the same rows.
// fp32: v_mfma_f32_32x32x2_f32 straight from a [token][channel] tile (no transpose needed).
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef __bf16 gram_v8bf __attribute__((ext_vector_type(8)));
typedef float gram_v16f __attribute__((ext_vector_type(16)));
typedef unsigned gram_v4u __attribute__((ext_vector_type(4)));

constexpr int GT = 256;   // output tile edge (channels)
constexpr int GC = 2 * GT;  // channels staged per step: the tile's row and column channels
constexpr int GK = 64;    // tokens per step, bf16
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

// Token chunks per tile: 16 or 8 when the tokens allow chunks of at least 2048 (then each
// XCD takes whole chunks, so its L2 streams only those rows), else as many as fill whole
// rounds of one workgroup per CU best.
static GramGeom gram_geom(int64_t tokens, int64_t cols, int cus) {
  GramGeom g;
  g.nt = (cols + GT - 1) / GT;
  g.tiles = g.nt * (g.nt + 1) / 2;
  const int64_t steps = (tokens + GK - 1) / GK;
  int64_t max_nc = steps / 32;
  if (max_nc > 16) max_nc = 16;
  if (max_nc < 1) max_nc = 1;
  const bool by_xcd = max_nc >= 8;
  int64_t best = max_nc >= 16 ? 16 : (max_nc >= 8 ? 8 : 1);
  double best_eff = -1.0;
  for (int64_t nc = 1; nc <= max_nc && !by_xcd; ++nc) {
    const int64_t wgs = g.tiles * nc;
    const int64_t rounds = (wgs + cus - 1) / cus;
    const double eff = (double)wgs / (double)(rounds * cus);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = nc;
    }
  }
  const int64_t spc = (steps + best - 1) / best > 0 ? (steps + best - 1) / best : 1;
  g.tc = spc * GK;
  g.nc = tokens > 0 ? (tokens + g.tc - 1) / g.tc : 1;
  if (by_xcd && g.nc % GXCD != 0) g.nc = (g.nc + GXCD - 1) / GXCD * GXCD;  // empty tail chunks
  return g;
}

// workgroup -> (token chunk, tile). With nc % 8 == 0, XCD x (= wid % 8) takes chunks
// x, x + 8, ...; its workgroups walk the tiles row by row, so the ones running together
// share their row panel. Otherwise chunk-major.
__device__ __forceinline__ void gram_work(int64_t wid, int64_t tiles, int64_t nc, int64_t &chunk,
                                          int64_t &tile) {
  if (nc % GXCD == 0) {
    const int64_t x = wid % GXCD, slot = wid / GXCD;
    chunk = x + GXCD * (slot / tiles);
    tile = slot % tiles;
  } else {
    chunk = wid / tiles;
    tile = wid % tiles;
  }
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

__device__ __forceinline__ int gram_swz(int c) { return (c ^ (c >> 3)) & 7; }

__global__ void __launch_bounds__(GTHREADS)
    k_gram_bf16(const uint16_t *__restrict__ x, int64_t tokens, int64_t cols, int64_t nt,
                int64_t tiles, int64_t nc, int64_t tc, float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][GC * GK];
  int64_t chunk, tile, ti, tj;
  gram_work(blockIdx.x, tiles, nc, chunk, tile);
  gram_tile(tile, nt, ti, tj);
  const int64_t p0 = chunk * tc;
  const int64_t p1 = p0 + tc < tokens ? p0 + tc : tokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // staging role: 8 channels (group q of 64: 32 row-tile, 32 column-tile) x 8 tokens
  // (group g of the step's 8)
  const int q = tid & 63, g = tid >> 6;
  const int64_t chg = q < 32 ? ti * GT + q * 8 : tj * GT + (q - 32) * 8;
  // cols % 16 == 0: a group of 8 channels is all in or all out. Groups past the last
  // channel load channels 0..7 instead: they only feed rows and columns of the partial
  // tile at or beyond cols, which the reduction drops.
  const int64_t chl = chg < cols ? chg : 0;
  // Raw buffer loads: token row pos + s + 8 g of the step is row 8 g of a buffer that
  // starts at token pos + s (a scalar descriptor) and holds only the rows below p1, so
  // rows past the chunk read as zero; the lane's byte offset (below 2^23) never changes.
  const int lo_bytes = (int)(((int64_t)(g * 8) * cols + chl) * 2);
  uint4 in[8];
  auto load = [&](int64_t pos) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      int64_t rows = p1 - pos - s;
      rows = rows < 0 ? 0 : (rows > GK ? GK : rows);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(x + (pos + s) * cols), (short)0, (int)(rows * cols * 2),
          0x00020000);
      const gram_v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, lo_bytes, 0, 0);
      in[s] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  // 8x8 transpose of 16-bit values: output channel i of token pair (2e, 2e + 1) takes the
  // low (even i) or high (odd i) halves of dword i / 2 of both rows (v_perm_b32 byte select)
  auto store = [&](uint16_t *buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
      unsigned o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint4 a4 = in[2 * e], b4 = in[2 * e + 1];
        const unsigned a = (i >> 1) == 0 ? a4.x : (i >> 1) == 1 ? a4.y : (i >> 1) == 2 ? a4.z : a4.w;
        const unsigned b = (i >> 1) == 0 ? b4.x : (i >> 1) == 1 ? b4.y : (i >> 1) == 2 ? b4.z : b4.w;
        o[e] = __builtin_amdgcn_perm(b, a, sel);  // bytes 0-3 from a, 4-7 from b
      }
      const int c = q * 8 + i;
      *reinterpret_cast<uint4 *>(buf + c * GK + ((g ^ gram_swz(c)) << 3)) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  const int wr = wave >> 1, wc = wave & 1;  // wave's 64 x 128 part of the tile
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
  for (int64_t pos = p0; pos < p1; pos += GK) {
    const bool more = pos + GK < p1;
    if (more) load(pos + GK);
    const uint16_t *buf = lds[cur];
#pragma unroll
    for (int s4 = 0; s4 < GK / 16; ++s4) {
      const int gg = 2 * s4 + (lane >> 5);
      gram_v8bf A[2], B[4];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c = wr * 64 + a * 32 + (lane & 31);
        A[a] = __builtin_bit_cast(gram_v8bf, *reinterpret_cast<const uint4 *>(
                                                 buf + c * GK + ((gg ^ gram_swz(c)) << 3)));
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c = GT + wc * 128 + b * 32 + (lane & 31);
        B[b] = __builtin_bit_cast(gram_v8bf, *reinterpret_cast<const uint4 *>(
                                                 buf + c * GK + ((gg ^ gram_swz(c)) << 3)));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a], B[b], acc[a][b], 0, 0, 0);
    }
    if (more) store(lds[cur ^ 1]);
    lds_barrier();
    cur ^= 1;
  }

  // D layout of a 32x32 MFMA: lane l, register r -> row (r & 3) + 4 (l >> 5) + 8 (r >> 2),
  // column l & 31
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

__global__ void __launch_bounds__(GTHREADS)
    k_gram_f32(const float *__restrict__ x, int64_t tokens, int64_t cols, int64_t nt,
               int64_t tiles, int64_t nc, int64_t tc, float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float lds[2][GKF * GC];
  int64_t chunk, tile, ti, tj;
  gram_work(blockIdx.x, tiles, nc, chunk, tile);
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
  const dim3 grid((unsigned)(g.nc * g.tiles));
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

// prefill.hip -- batched prompt prefill: the n prompt positions of a call go
// through every layer together, so each linear is a GEMM of n rows against the
// weights (read once per layer instead of once per position), run on the
// matrix cores, and attention is a causal tile loop on the matrix cores too.
//
// Per layer (rows t = 0..n-1 at positions p0 + t; x_n = the rows after the
// LayerNorm that comes next, written by the kernel that last changed x):
//   gemm  x_n W_qkv^T + b; the new key and value rows also go into the cache
//   attn  per (16 rows, head): causal softmax over cache rows 0..p0+t and the
//         weighted sum of values, 64 keys a step with a running maximum and sum
//   gemm  attn W_ap^T in K-split partials; row pass: x += sum + b, x_n = LN2(x)
//   gemm  act = gelu_new(x_n W_fc^T + b)
//   gemm  act W_pr^T in K-split partials; row pass: x += sum + b, x_n = the
//         next layer's LN1 (after the last layer the final LayerNorm)
// then the head (the last row's logits) and the argmax.
//
// Matrix-core layout (v_mfma_f32_16x16x4f32, 64 lanes, lane l = 16 g + r):
// lane l supplies A[r][slot g] and B[slot g][r] and holds C[4 g + e][r] in
// result element e.  A contraction is cut into four runs, slot g taking the
// g-th run one input per step, so a lane reads its operands as float4 runs.
//
// GEMM: C[n][N] = A[n][K] W[N][K]^T with output-major weights, tiles of
// BM x 64 (or 48) outputs per workgroup of four waves, K in stages of 32 or 64
// through LDS (double-buffered: the next stage's loads are in flight while the
// current one is multiplied).  fp16 weights are widened exactly and int4
// weights become zero + code * scale with one rounding (the quantised model's
// values) as a stage is written to LDS; products and sums are fp32.  Tiles are
// numbered so that the workgroups on one XCD share weight columns (its L2
// holds them).  The two projections (N = E) have few column tiles, so their K
// is split in up to four parts that run as separate tiles (at 1,024 rows: 768
// tiles, three per CU); a short prompt's linears all split K further, so that
// the weights stream on every CU.  The parts are added in a fixed order, so
// results do not depend on scheduling.
#include <hip/hip_fp16.h>

#include <type_traits>
#include <utility>

#include "lib_internal.h"

namespace gpt2dec {
namespace {

typedef float pf_f4 __attribute__((ext_vector_type(4)));

enum { PF_QKV = 0, PF_PART = 1, PF_GELU = 2 };

constexpr int HEAD_XCH = 8;   // float4 chunks of a row a lane keeps (row passes, head): E <= 2048

__device__ __forceinline__ float pf_wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float pf_gelu_new(float x) {
  // x * logistic(2 * sqrt(2/pi) * (x + 0.044715 x^3))
  const float z2 = 1.5957691216057308f * __builtin_fmaf(0.044715f * x, x * x, x);
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-z2));
}

__device__ __forceinline__ float pf_half(unsigned bits) { return __half2float(__ushort_as_half((unsigned short)bits)); }

// GEMM stages sit in LDS as rows of BK floats with no padding; the 16-byte
// quads of row r are stored in the order q ^ s(r), so that the same quad of
// 16 consecutive rows (a read) and the quads of one row (a write) fall in
// distinct banks.  Returns the float offset of quad q in row r.
template <int BK>
__device__ __forceinline__ int pf_swz(int r, int q) {
  constexpr int QR = BK / 4;  // quads per row: 8 or 16
  return (q ^ ((r / (16 / QR)) & (QR - 1))) * 4;
}

// ---------------------------------------------------------------- row passes
// One wave per row; lane l holds the row's float4 chunks l, l + 64, ... (at most
// HEAD_XCH of them: E <= 2048) in registers.

// xn = (x - mean) / sqrt(var + eps) * gamma + beta for the row held in xv
// (mean first, then the mean squared deviation).
__device__ __forceinline__ void pf_layernorm_row(const float4 (&xv)[HEAD_XCH], int E, const float *gamma,
                                                 const float *beta, float eps, float *o, int l) {
  const int nch = E / 4;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++)
    if (l + 64 * j < nch) s += (xv[j].x + xv[j].y) + (xv[j].z + xv[j].w);
  const float mean = pf_wave_sum(s) / (float)E;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++)
    if (l + 64 * j < nch) {
      const float a = xv[j].x - mean, b = xv[j].y - mean, c = xv[j].z - mean, d = xv[j].w - mean;
      q = __builtin_fmaf(a, a, q);
      q = __builtin_fmaf(b, b, q);
      q = __builtin_fmaf(c, c, q);
      q = __builtin_fmaf(d, d, q);
    }
  const float rstd = __builtin_amdgcn_rsqf(pf_wave_sum(q) / (float)E + eps);
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++) {
    const int c = l + 64 * j;
    if (c >= nch) break;
    const float4 g = *reinterpret_cast<const float4 *>(gamma + 4 * c);
    const float4 b = *reinterpret_cast<const float4 *>(beta + 4 * c);
    *reinterpret_cast<float4 *>(o + 4 * c) =
        make_float4((xv[j].x - mean) * rstd * g.x + b.x, (xv[j].y - mean) * rstd * g.y + b.y,
                    (xv[j].z - mean) * rstd * g.z + b.z, (xv[j].w - mean) * rstd * g.w + b.w);
  }
}

// x[t] = wte[token t] + wpe[p0 + t], and xn[t] = LN(x[t]).
__global__ void __launch_bounds__(256) prefill_embed_ln(const int *tok, const float *wte, const float *wpe, int E,
                                                        int p0, int n, const float *gamma, const float *beta,
                                                        float eps, float *x, float *xn) {
  const int t = blockIdx.x * 4 + threadIdx.x / 64, l = threadIdx.x % 64;
  if (t >= n) return;
  const int nch = E / 4;
  float *xr = x + (size_t)t * E;
  const float *we = wte + (size_t)tok[t] * E, *pe = wpe + (size_t)(p0 + t) * E;
  float4 xv[HEAD_XCH];
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++) {
    const int c = l + 64 * j;
    xv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nch) {
      const float4 a = *reinterpret_cast<const float4 *>(we + 4 * c);
      const float4 b = *reinterpret_cast<const float4 *>(pe + 4 * c);
      xv[j] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
      *reinterpret_cast<float4 *>(xr + 4 * c) = xv[j];
    }
  }
  pf_layernorm_row(xv, E, gamma, beta, eps, xn + (size_t)t * E, l);
}

// x[t] += (part_0[t] + part_1[t] + ...) + bias, then xn[t] = LN(x[t]).  The
// parts are a projection's K-split partial sums [S][n][E], added in order.
template <int S>
__global__ void __launch_bounds__(256) prefill_resid_ln(const float *part, int n, int E, const float *bias,
                                                        const float *gamma, const float *beta, float eps, float *x,
                                                        float *xn) {
  const int t = blockIdx.x * 4 + threadIdx.x / 64, l = threadIdx.x % 64;
  if (t >= n) return;
  const int nch = E / 4;
  float *xr = x + (size_t)t * E;
  const size_t ps = (size_t)n * E;
  const float *pr = part + (size_t)t * E;
  float4 xv[HEAD_XCH];
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++) {
    const int c = l + 64 * j;
    xv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nch) {
      float4 v = *reinterpret_cast<const float4 *>(pr + 4 * c);
#pragma unroll
      for (int sp = 1; sp < S; sp++) {
        const float4 w = *reinterpret_cast<const float4 *>(pr + sp * ps + 4 * c);
        v = make_float4(v.x + w.x, v.y + w.y, v.z + w.z, v.w + w.w);
      }
      const float4 b = *reinterpret_cast<const float4 *>(bias + 4 * c);
      const float4 x0 = *reinterpret_cast<const float4 *>(xr + 4 * c);
      xv[j] = make_float4(x0.x + (v.x + b.x), x0.y + (v.y + b.y), x0.z + (v.z + b.z), x0.w + (v.w + b.w));
      *reinterpret_cast<float4 *>(xr + 4 * c) = xv[j];
    }
  }
  pf_layernorm_row(xv, E, gamma, beta, eps, xn + (size_t)t * E, l);
}

// The same for many parts (a short prompt's projections, ns of them): one
// workgroup per row, a thread per float4 chunk (two at most: E <= 2048), the
// parts' loads eight at a time and their sums in order; the LayerNorm's two
// sums are combined over the four waves through LDS.
__global__ void __launch_bounds__(256) prefill_resid_ln_wg(const float *part, int ns, int n, int E,
                                                           const float *bias, const float *gamma, const float *beta,
                                                           float eps, float *x, float *xn) {
  __shared__ float red[2][4];
  const int t = blockIdx.x, tid = threadIdx.x, wv = tid / 64, l = tid % 64, nch = E / 4;
  float *xr = x + (size_t)t * E;
  const size_t ps = (size_t)n * E;
  const float *pr = part + (size_t)t * E;
  pf_f4 xv[2];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int c = tid + 256 * j;
    xv[j] = pf_f4{0.f, 0.f, 0.f, 0.f};
    if (c >= nch) continue;
    pf_f4 v = *reinterpret_cast<const pf_f4 *>(pr + 4 * c);
    for (int s0 = 1; s0 < ns; s0 += 8) {
      pf_f4 w[8];
#pragma unroll
      for (int u = 0; u < 8; u++) w[u] = *reinterpret_cast<const pf_f4 *>(pr + (size_t)min(s0 + u, ns - 1) * ps + 4 * c);
#pragma unroll
      for (int u = 0; u < 8; u++)
        if (s0 + u < ns) v += w[u];
    }
    const pf_f4 b = *reinterpret_cast<const pf_f4 *>(bias + 4 * c);
    const pf_f4 x0 = *reinterpret_cast<const pf_f4 *>(xr + 4 * c);
    xv[j] = x0 + (v + b);
    *reinterpret_cast<pf_f4 *>(xr + 4 * c) = xv[j];
    sum += (xv[j][0] + xv[j][1]) + (xv[j][2] + xv[j][3]);
  }
  sum = pf_wave_sum(sum);
  if (l == 0) red[0][wv] = sum;
  __syncthreads();
  const float mean = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) / (float)E;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < 2; j++)
    if (tid + 256 * j < nch)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float d = xv[j][e] - mean;
        q = __builtin_fmaf(d, d, q);
      }
  q = pf_wave_sum(q);
  if (l == 0) red[1][wv] = q;
  __syncthreads();
  const float rstd = __builtin_amdgcn_rsqf(((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) / (float)E + eps);
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int c = tid + 256 * j;
    if (c >= nch) continue;
    const pf_f4 g = *reinterpret_cast<const pf_f4 *>(gamma + 4 * c);
    const pf_f4 b = *reinterpret_cast<const pf_f4 *>(beta + 4 * c);
    pf_f4 o;
#pragma unroll
    for (int e = 0; e < 4; e++) o[e] = (xv[j][e] - mean) * rstd * g[e] + b[e];
    *reinterpret_cast<pf_f4 *>(xn + (size_t)t * E + 4 * c) = o;
  }
}

// A K-split QKV or fc: y = (part_0 + part_1 + ...) + bias over [n][N], then
// QKV: the row, and its key / value part into the cache rows p0 + t;
// fc: gelu_new of it.
template <bool QKV>
__global__ void __launch_bounds__(256) prefill_finish(const float *part, int S, int n, int N, const float *bias,
                                                      float *out, float *kc, float *vc, int E, int D, int P, int p0) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x, total = (size_t)n * N;
  if (idx >= total) return;
  const int t = (int)(idx / N), o = (int)(idx % N);
  float v = part[idx];
  // eight parts' loads at a time, then their sums in order
  for (int s0 = 1; s0 < S; s0 += 8) {
    float w[8];
#pragma unroll
    for (int u = 0; u < 8; u++) w[u] = part[(size_t)min(s0 + u, S - 1) * total + idx];
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (s0 + u < S) v += w[u];
  }
  const float y = v + bias[o];
  if constexpr (QKV) {
    out[idx] = y;
    if (o >= E) {
      const int ev = (o - E) % E, hh = ev / D, d = ev % D;
      float *cache = (o < 2 * E) ? kc : vc;
      cache[((size_t)hh * P + p0 + t) * D + d] = y;
    }
  } else {
    out[idx] = pf_gelu_new(y);
  }
}

// ---------------------------------------------------------------- GEMM
struct GemmArgs {
  const float *a;        // [n_rows][K] input rows
  int n_rows;
  const void *w;         // [N][K] output-major weights of this layer
  const float2 *sz;      // int4: (scale, zero) per group of 32
  const float *bias;     // [N]
  int N, K;
  float *out;            // [n_rows][N] (QKV, GELU) or partial sums [splits][n_rows][N] (PART)
  float *kc, *vc;        // QKV: this layer's cache blocks [H][P][D]
  int E, D, P, p0;
  int splits;            // K parts (PART only; else 1)
  int tiles_m, tiles_n, n_tiles;  // M tiles, N tiles, all tiles (x splits)
};

// One stage of weights (ROWS = 64 or 48 rows x BK = 32 or 64 inputs) in flight,
// in its storage type, as PIECES loads spread over the 256 threads; store()
// writes it to LDS as fp32 rows (quads swizzled).  Where the pieces do not
// divide among the threads, the extra threads load a piece again (no load is
// conditional) and only the first PIECES store.
template <int WD, int BK, int ROWS>
struct WStage;
template <int BK, int ROWS>
struct WStage<WD_F32, BK, ROWS> {
  static constexpr int C4 = BK / 4, PIECES = ROWS * C4;  // float4 per row; per stage
  static constexpr int N = (PIECES + 255) / 256;
  pf_f4 v[N];
  __device__ void load(const GemmArgs &g, int n0, int k0, int tid) {
    const float *w = static_cast<const float *>(g.w);
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int f = (tid + i * 256) % PIECES, row = f / C4, c4 = f % C4;
      v[i] = *reinterpret_cast<const pf_f4 *>(w + (size_t)(n0 + row) * g.K + k0 + c4 * 4);
    }
  }
  __device__ void store(float (*ws)[BK], int tid) const {
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int f = tid + i * 256, row = f / C4, c4 = f % C4;
      if (PIECES % 256 == 0 || f < PIECES) *reinterpret_cast<pf_f4 *>(&ws[row][pf_swz<BK>(row, c4)]) = v[i];
    }
  }
};
template <int BK, int ROWS>
struct WStage<WD_F16, BK, ROWS> {
  static constexpr int C8 = BK / 8, PIECES = ROWS * C8;  // 8-half pieces per row; per stage
  static constexpr int N = (PIECES + 255) / 256;
  uint4 v[N];
  __device__ void load(const GemmArgs &g, int n0, int k0, int tid) {
    const __half *w = static_cast<const __half *>(g.w);
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int f = (tid + i * 256) % PIECES;
      v[i] = *reinterpret_cast<const uint4 *>(w + (size_t)(n0 + f / C8) * g.K + k0 + (f % C8) * 8);
    }
  }
  __device__ void store(float (*ws)[BK], int tid) const {
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int f = tid + i * 256, row = f / C8, q = (f % C8) * 2;
      if (PIECES % 256 != 0 && f >= PIECES) continue;
      *reinterpret_cast<pf_f4 *>(&ws[row][pf_swz<BK>(row, q)]) =
          pf_f4{pf_half(v[i].x & 0xffffu), pf_half(v[i].x >> 16), pf_half(v[i].y & 0xffffu), pf_half(v[i].y >> 16)};
      *reinterpret_cast<pf_f4 *>(&ws[row][pf_swz<BK>(row, q + 1)]) =
          pf_f4{pf_half(v[i].z & 0xffffu), pf_half(v[i].z >> 16), pf_half(v[i].w & 0xffffu), pf_half(v[i].w >> 16)};
    }
  }
};
template <int BK, int ROWS>
struct WStage<WD_Q4, BK, ROWS> {
  // four pieces per row, each BK/4 codes (even input in the low nibble) of
  // one group of 32, with that group's (scale, zero)
  static constexpr int NW = BK / 32, PIECES = ROWS * 4;  // 32-bit words of codes per piece
  static_assert(PIECES <= 256, "one piece per thread");
  uint32_t q[NW];
  float2 s;
  __device__ void load(const GemmArgs &g, int n0, int k0, int tid) {
    const int f = tid % PIECES;
    const size_t e0 = (size_t)(n0 + (f >> 2)) * g.K + k0 + (f & 3) * (BK / 4);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(g.w) + e0 / 2);
#pragma unroll
    for (int i = 0; i < NW; i++) q[i] = src[i];
    s = g.sz[e0 / 32];
  }
  __device__ void store(float (*ws)[BK], int tid) const {
    if (PIECES < 256 && tid >= PIECES) return;
    const int row = tid >> 2, q0 = (tid & 3) * (BK / 16);  // this thread's first quad of the row
#pragma unroll
    for (int i = 0; i < NW; i++) {
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; j++) f[j] = __builtin_fmaf((float)((q[i] >> (4 * j)) & 15u), s.x, s.y);
      *reinterpret_cast<pf_f4 *>(&ws[row][pf_swz<BK>(row, q0 + 2 * i)]) = pf_f4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<pf_f4 *>(&ws[row][pf_swz<BK>(row, q0 + 2 * i + 1)]) = pf_f4{f[4], f[5], f[6], f[7]};
    }
  }
};

template <int WD, int MODE, int BM, int BK, int BN>
__global__ void __launch_bounds__(256) prefill_gemm(GemmArgs g) {
  // waves WM x WN over the tile; each wave owns TM x TN blocks of 16 x 16
  // (48-column tiles: the four waves stacked, 16 x 48 each)
  constexpr int WM = BN == 48 ? 4 : BM >= 32 ? 2 : 1, WN = 4 / WM;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  static_assert(TM >= 1 && TN >= 1 && TM * WM * 16 == BM && TN * WN * 16 == BN, "whole 16 x 16 blocks");
  constexpr int AF4 = BM * BK / 4;                  // float4 of an A stage
  constexpr int AI = AF4 / 256;                     // per thread
  __shared__ float as[2][BM][BK];
  __shared__ float ws[2][BN][BK];
  // XCD-aware tile order: workgroup id -> XCD id % 8; each XCD takes a run of
  // consecutive tiles, which walk the M tiles of one weight column block first
  const int per = gridDim.x / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= g.n_tiles) return;
  const int m0 = (t % g.tiles_m) * BM, rest = t / g.tiles_m;
  const int n0 = (rest % g.tiles_n) * BN, sp = rest / g.tiles_n;
  const int tid = threadIdx.x, wv = tid / 64, l = tid % 64, r = l & 15, gs = l >> 4;
  const int mw = (wv / WN) * (BM / WM), nw = (wv % WN) * (BN / WN);
  const int KT = g.K / BK / g.splits, kbase = sp * KT * BK;  // this tile's part of K

  constexpr int AC4 = BK / 4;                       // float4 per A row
  pf_f4 av[AI];
  WStage<WD, BK, BN> wst;
  // Rows past the last (a ragged last tile) load the last row again: they only
  // feed output rows that are never written.  The loads are unconditional so
  // that nothing waits for them before the stage's products.  (Staging values
  // are native vectors: arrays of the float4 struct were kept in scratch.)
  static_assert(AF4 % 256 == 0, "an A stage is whole float4 per thread");
  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AI; i++) {
      const int f = tid + i * 256, row = min(m0 + f / AC4, g.n_rows - 1), c4 = f % AC4;
      av[i] = *reinterpret_cast<const pf_f4 *>(g.a + (size_t)row * g.K + k0 + c4 * 4);
    }
  };
  auto store_a = [&](int b) {
#pragma unroll
    for (int i = 0; i < AI; i++) {
      const int f = tid + i * 256, row = f / AC4, c4 = f % AC4;
      *reinterpret_cast<pf_f4 *>(&as[b][row][pf_swz<BK>(row, c4)]) = av[i];
    }
  };

  pf_f4 c[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) c[i][j] = pf_f4{0.f, 0.f, 0.f, 0.f};

  load_a(kbase);
  wst.load(g, n0, kbase, tid);
  store_a(0);
  wst.store(ws[0], tid);
  __syncthreads();
  for (int kt = 0; kt < KT; kt++) {
    const int b = kt & 1;
    if (kt + 1 < KT) {
      load_a(kbase + (kt + 1) * BK);
      wst.load(g, n0, kbase + (kt + 1) * BK, tid);
    }
    // slot gs of the stage: inputs gs*BK/4 .. (gs+1)*BK/4 - 1, one per step
    constexpr int RUN = BK / 16;  // float4 per run
    pf_f4 ar[TM][RUN], wr[TN][RUN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int h = 0; h < RUN; h++)
        ar[i][h] = *reinterpret_cast<const pf_f4 *>(&as[b][mw + i * 16 + r][pf_swz<BK>(mw + i * 16 + r, gs * (BK / 16) + h)]);
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int h = 0; h < RUN; h++)
        wr[j][h] = *reinterpret_cast<const pf_f4 *>(&ws[b][nw + j * 16 + r][pf_swz<BK>(nw + j * 16 + r, gs * (BK / 16) + h)]);
#pragma unroll
    for (int h = 0; h < RUN; h++) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
          c[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[i][h][0], wr[j][h][0], c[i][j], 0, 0, 0);
          c[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[i][h][1], wr[j][h][1], c[i][j], 0, 0, 0);
          c[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[i][h][2], wr[j][h][2], c[i][j], 0, 0, 0);
          c[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[i][h][3], wr[j][h][3], c[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < KT) {
      store_a(b ^ 1);
      wst.store(ws[b ^ 1], tid);
    }
    __syncthreads();
  }

  // epilogue: block (i, j), element e is row m0 + mw + 16 i + 4 gs + e, column n0 + nw + 16 j + r
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int o = n0 + nw + j * 16 + r;
      const float bo = MODE == PF_PART ? 0.f : g.bias[o];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = m0 + mw + i * 16 + gs * 4 + e;
        if (row >= g.n_rows) continue;
        const float y = c[i][j][e] + bo;
        if constexpr (MODE == PF_PART) {
          g.out[((size_t)sp * g.n_rows + row) * g.N + o] = c[i][j][e];
        } else if constexpr (MODE == PF_GELU) {
          g.out[(size_t)row * g.N + o] = pf_gelu_new(y);
        } else {  // QKV: the row, and its key / value part into the cache at position p0 + row
          g.out[(size_t)row * g.N + o] = y;
          if (o >= g.E) {
            const int ev = (o - g.E) % g.E, hh = ev / g.D, d = ev % g.D;
            float *cache = (o < 2 * g.E) ? g.kc : g.vc;
            cache[((size_t)hh * g.P + g.p0 + row) * g.D + d] = y;
          }
        }
      }
    }
}

// ---------------------------------------------------------------- attention
// One workgroup of four waves per (16 rows, head); wave w takes the 64-key
// steps w, w + 4, ... and the four partial results (running maximum, sum and
// weighted values per row) are merged through LDS in wave order.
//
// Scores are formed transposed, S^T = K Q^T (keys as the A rows, the rows'
// queries as the B columns), so each lane holds the scores of one row (r) for
// four keys per 16-key block, which is exactly the B operand of O^T = V^T P^T:
// the weights never leave the registers.  Slot g of the score contraction
// takes dims 16 i + 4 g + c (step 4 i + c), so the four lanes of a key row read
// 64 contiguous bytes per load.  The queries are scaled by log2(e)/sqrt(D) as
// they are read, so scores are in base-2 units and each weight is one exp2.
// The running maximum and sum belong to row r in every lane that holds it; the
// row's maximum over a step is combined over the four lanes of the row (lanes
// r, r+16, r+32, r+48).  Output dims are spread as d = (D/16) r' + db over the
// D/16 result blocks db, so a lane reads each value row as one run.  A step
// wholly below every row's position (all but the last one or two of a block)
// needs no masking and no clamping of row indices.
//
// Balance: a block's work grows with its position.  All workgroups are
// resident at once, and workgroups i, i + C, i + 2C, ... share a CU (one per
// CU in each round of C = the CU count), so the blocks are taken longest
// first and every other round in reverse order: each CU gets long and short
// blocks.
template <int D>
__global__ void __launch_bounds__(256) prefill_attention(const float *qkv, const float *kc, const float *vc, int E,
                                                         int P, int p0, int n, int cus, float *out) {
  constexpr int RQ = D / 4;   // a lane's dims in the score contraction
  constexpr int DV = D / 16;  // value dims a lane reads per key (result blocks)
  __shared__ float sm[4][16], sl[4][16];
  __shared__ float so[4][D][17];
  const int wv = threadIdx.x / 64, l = threadIdx.x % 64, r = l & 15, gs = l >> 4;
  const int H = E / D, nqb = (n + 15) / 16, total = nqb * H;
  const int wg = (int)blockIdx.x, round = wg / cus, pos = wg % cus, size = min(cus, total - round * cus);
  const int k = (round & 1) ? round * cus + size - 1 - pos : wg;  // rank of this workgroup's block by length
  const int qb = nqb - 1 - k / H, h = k % H;
  const int t0 = qb * 16, t = t0 + r;
  const int jmax = p0 + min(t0 + 15, n - 1);  // last cache row the block may read
  const int pq = min(p0 + t, jmax);           // last key of row r
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  float q[RQ];
  {
    const float *qr = qkv + (size_t)min(t, n - 1) * 3 * E + h * D + 4 * gs;
#pragma unroll
    for (int i = 0; i < RQ / 4; i++) {
      const float4 v = *reinterpret_cast<const float4 *>(qr + 16 * i);
      q[4 * i] = v.x * qscale;
      q[4 * i + 1] = v.y * qscale;
      q[4 * i + 2] = v.z * qscale;
      q[4 * i + 3] = v.w * qscale;
    }
  }
  const float *Kh = kc + (size_t)h * P * D, *Vh = vc + (size_t)h * P * D;
  float m = -INFINITY, lsum = 0.f;
  pf_f4 o[DV];
#pragma unroll
  for (int db = 0; db < DV; db++) o[db] = pf_f4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int j0, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    // scores: block kb, element e is key j0 + 16 kb + 4 gs + e of row r
    pf_f4 s[4];
    float kr[4][RQ];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int row = MASKED ? min(j0 + kb * 16 + r, jmax) : j0 + kb * 16 + r;
      const float *kp = Kh + (size_t)row * D + 4 * gs;
#pragma unroll
      for (int i = 0; i < RQ / 4; i++) {
        const float4 v = *reinterpret_cast<const float4 *>(kp + 16 * i);
        kr[kb][4 * i] = v.x;
        kr[kb][4 * i + 1] = v.y;
        kr[kb][4 * i + 2] = v.z;
        kr[kb][4 * i + 3] = v.w;
      }
      s[kb] = pf_f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < RQ; i++)
#pragma unroll
      for (int kb = 0; kb < 4; kb++) s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[kb][i], q[i], s[kb], 0, 0, 0);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        if constexpr (MASKED) s[kb][e] = (j0 + kb * 16 + gs * 4 + e <= pq) ? s[kb][e] : -INFINITY;
        mx = fmaxf(mx, s[kb][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // (masked: a row with no key in this step keeps its maximum, mx = -inf;
    // one whose first key this is starts from m = -inf, where alpha is 0)
    const float mn = fmaxf(m, mx);
    const float alpha = (MASKED && mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float p;
        if constexpr (MASKED) p = (j0 + kb * 16 + gs * 4 + e <= pq) ? __builtin_amdgcn_exp2f(s[kb][e] - mn) : 0.f;
        else p = __builtin_amdgcn_exp2f(s[kb][e] - mn);
        s[kb][e] = p;
        ps += p;
      }
    lsum = __builtin_fmaf(lsum, alpha, ps);
#pragma unroll
    for (int db = 0; db < DV; db++) o[db] *= alpha;
    // O^T += V^T P^T: step e of block kb takes key j0 + 16 kb + 4 gs + e
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int key = j0 + kb * 16 + gs * 4 + e;
        const float *vp = Vh + (size_t)(MASKED ? min(key, jmax) : key) * D + r * DV;
        float vv[DV];
        if constexpr (DV == 4) {
          const float4 v = *reinterpret_cast<const float4 *>(vp);
          vv[0] = v.x; vv[1] = v.y; vv[2] = v.z; vv[3] = v.w;
        } else {
#pragma unroll
          for (int db = 0; db < DV; db++) vv[db] = vp[db];
        }
#pragma unroll
        for (int db = 0; db < DV; db++) o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[db], s[kb][e], o[db], 0, 0, 0);
      }
  };
  for (int j0 = 64 * wv; j0 <= jmax; j0 += 256) {
    if (j0 + 63 <= p0 + t0) step(j0, std::false_type{});
    else step(j0, std::true_type{});
  }
  // this wave's partials: row maximum and sum, and O^T (block db, element e:
  // dim DV (4 gs + e) + db of row r)
  float tot = lsum + __shfl_xor(lsum, 16);
  tot += __shfl_xor(tot, 32);
  if (gs == 0) {
    sm[wv][r] = m;
    sl[wv][r] = tot;
  }
#pragma unroll
  for (int db = 0; db < DV; db++)
#pragma unroll
    for (int e = 0; e < 4; e++) so[wv][DV * (4 * gs + e) + db][r] = o[db][e];
  __syncthreads();
  // merge: thread i takes outputs i, i + 256, ... of the 16 x D block (row-major)
  for (int i = threadIdx.x; i < 16 * D; i += 256) {
    const int rr = i / D, d = i % D;
    if (t0 + rr >= n) break;
    float mm = sm[0][rr];
#pragma unroll
    for (int w = 1; w < 4; w++) mm = fmaxf(mm, sm[w][rr]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float f = sm[w][rr] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[w][rr] - mm);  // waves with no keys add nothing
      num = __builtin_fmaf(f, so[w][d][rr], num);
      den = __builtin_fmaf(f, sl[w][rr], den);
    }
    out[(size_t)(t0 + rr) * E + h * D + d] = num / den;
  }
}

// ---------------------------------------------------------------- head
// The better of two (logit, id) candidates for the argmax: a larger value, or
// the lower id of equal values; NaN never wins and id -1 is no candidate.
__device__ __forceinline__ void pf_better(float &v, int &i, float v2, int i2) {
  if (i2 >= 0 && !__builtin_isnan(v2) && (i < 0 || v2 > v || (v2 == v && i2 < i))) {
    v = v2;
    i = i2;
  }
}

// logits[v] = head row v . xn for the one normalised row xn; each wave takes
// four rows at a time, a lane the float4 chunks l, l + 64, ...  Each
// workgroup (16 rows) also leaves its best (logit, id) in best[blockIdx.x].
template <int HWD>
__global__ void __launch_bounds__(256) prefill_head(const void *head, const float *xn, int E, int V,
                                                    float *logits, float2 *best) {
  __shared__ float bv[4];
  __shared__ int bi[4];
  const int l = threadIdx.x % 64, wv = threadIdx.x / 64, nch = E / 4;
  const int row0 = (blockIdx.x * 4 + wv) * 4;
  float4 xv[HEAD_XCH];
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++) {
    const int c = l + 64 * j;
    xv[j] = c < nch ? *reinterpret_cast<const float4 *>(xn + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < HEAD_XCH; j++) {
    const int c = l + 64 * j;
    if (c >= nch) break;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = min(row0 + i, V - 1);
      float4 w;
      if constexpr (HWD == WD_F32) {
        w = *reinterpret_cast<const float4 *>(static_cast<const float *>(head) + (size_t)row * E + 4 * c);
      } else {
        const uint2 hb = *reinterpret_cast<const uint2 *>(static_cast<const __half *>(head) + (size_t)row * E + 4 * c);
        w = make_float4(pf_half(hb.x & 0xffffu), pf_half(hb.x >> 16), pf_half(hb.y & 0xffffu), pf_half(hb.y >> 16));
      }
      acc[i] = __builtin_fmaf(w.x, xv[j].x, acc[i]);
      acc[i] = __builtin_fmaf(w.y, xv[j].y, acc[i]);
      acc[i] = __builtin_fmaf(w.z, xv[j].z, acc[i]);
      acc[i] = __builtin_fmaf(w.w, xv[j].w, acc[i]);
    }
  }
  float mv = -INFINITY;
  int mi = -1;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float v = pf_wave_sum(acc[i]);
    if (row0 + i < V) {
      if (l == 0) logits[row0 + i] = v;
      pf_better(mv, mi, v, row0 + i);
    }
  }
  if (l == 0) {
    bv[wv] = mv;
    bi[wv] = mi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = bv[0];
    int i = bi[0];
    for (int w = 1; w < 4; w++) pf_better(v, i, bv[w], bi[w]);
    best[blockIdx.x] = make_float2(v, __int_as_float(i));
  }
}

// The id of the largest logit, the lowest among equal ones (NaN never wins;
// -1 when every logit is NaN), from the head workgroups' candidates, by one
// workgroup.
__global__ void __launch_bounds__(1024) prefill_argmax(const float2 *best, int nb, int *out) {
  __shared__ float bv[1024];
  __shared__ int bi[1024];
  float v = -INFINITY;
  int idx = -1;
  for (int i = threadIdx.x; i < nb; i += 1024) {
    const float2 c = best[i];
    pf_better(v, idx, c.x, __float_as_int(c.y));
  }
  bv[threadIdx.x] = v;
  bi[threadIdx.x] = idx;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      float v1 = bv[threadIdx.x];
      int i1 = bi[threadIdx.x];
      pf_better(v1, i1, bv[threadIdx.x + s], bi[threadIdx.x + s]);
      bv[threadIdx.x] = v1;
      bi[threadIdx.x] = i1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = bi[0];
}

// Rows per tile: the largest of 64, 32, 16 that still gives about one tile per
// CU.  64-row tiles take K in stages of 32 (32 KB of LDS), the shorter ones
// in stages of 64 (half the barriers per input).
int pick_bm(int n, int N, int splits, int cus) {
  const int tn = N / 64 * splits, enough = cus - cus / 16;
  if (n > 32 && tn * ((n + 63) / 64) >= enough) return 64;
  if (n > 16 && tn * ((n + 31) / 32) >= enough) return 32;
  return 16;
}

template <int WD, int MODE>
hipError_t gemm_bm(GemmArgs g, int cus, hipStream_t s) {
  const int bm = pick_bm(g.n_rows, g.N, g.splits, cus);
  g.tiles_m = (g.n_rows + bm - 1) / bm;
  // 64-row tiles: 48 columns instead of 64 where that leaves the busiest CU
  // less work (tiles per CU rounded up, times the tile's width)
  int bn = 64;
  if (bm == 64 && g.N % 48 == 0) {
    const long t64 = (long)g.tiles_m * (g.N / 64) * g.splits, t48 = (long)g.tiles_m * (g.N / 48) * g.splits;
    if ((t48 + cus - 1) / cus * 48 < (t64 + cus - 1) / cus * 64) bn = 48;
  }
  g.tiles_n = g.N / bn;
  g.n_tiles = g.tiles_m * g.tiles_n * g.splits;
  const dim3 grid((unsigned)((g.n_tiles + 7) / 8 * 8));
  if (bm == 64 && bn == 48) prefill_gemm<WD, MODE, 64, 32, 48><<<grid, 256, 0, s>>>(g);
  else if (bm == 64) prefill_gemm<WD, MODE, 64, 32, 64><<<grid, 256, 0, s>>>(g);
  else if (bm == 32) prefill_gemm<WD, MODE, 32, 64, 64><<<grid, 256, 0, s>>>(g);
  else prefill_gemm<WD, MODE, 16, 64, 64><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

template <int MODE>
hipError_t gemm_wd(int wd, const GemmArgs &g, int cus, hipStream_t s) {
  if (wd == WD_F32) return gemm_bm<WD_F32, MODE>(g, cus, s);
  if (wd == WD_F16) return gemm_bm<WD_F16, MODE>(g, cus, s);
  return gemm_bm<WD_Q4, MODE>(g, cus, s);
}

// K parts of a linear [n][K] x [K][N].  With few tiles (a short prompt): as
// many as keep the tiles within two per CU, so that the weights stream on
// every CU (their partial sums [d][n][N] must fit the partials buffer of
// cap floats).  Otherwise a projection (N = E) takes up to four (the most
// that divide K's stages of 64), the other linears none.
int pick_splits(int n, int N, int K, bool projection, int cus, size_t cap) {
  const int bm = pick_bm(n, N, 1, cus), st = K / 64;
  const long tiles = (long)((n + bm - 1) / bm) * (N / 64);
  if (tiles < cus / 2) {
    int best = 1;
    for (int d = 2; d <= st; d++)
      if (st % d == 0 && tiles * d <= 2L * cus && (size_t)d * n * N <= cap) best = d;
    return best;
  }
  if (!projection) return 1;
  return st % 4 == 0 ? 4 : st % 3 == 0 ? 3 : st % 2 == 0 ? 2 : 1;
}

// x += (the S partial sums in order) + bias; xn = LN(x): one wave per row for
// up to four parts, one workgroup per row for more.
hipError_t resid_ln(const float *part, int S, int n, int E, const float *bias, const float *gamma, const float *beta,
                    float eps, float *x, float *xn, hipStream_t s) {
  const dim3 grid((unsigned)((n + 3) / 4));
  switch (S) {
  case 1: prefill_resid_ln<1><<<grid, 256, 0, s>>>(part, n, E, bias, gamma, beta, eps, x, xn); break;
  case 2: prefill_resid_ln<2><<<grid, 256, 0, s>>>(part, n, E, bias, gamma, beta, eps, x, xn); break;
  case 3: prefill_resid_ln<3><<<grid, 256, 0, s>>>(part, n, E, bias, gamma, beta, eps, x, xn); break;
  case 4: prefill_resid_ln<4><<<grid, 256, 0, s>>>(part, n, E, bias, gamma, beta, eps, x, xn); break;
  default:
    prefill_resid_ln_wg<<<dim3((unsigned)n), 256, 0, s>>>(part, S, n, E, bias, gamma, beta, eps, x, xn);
    break;
  }
  return hipGetLastError();
}

template <bool QKV>
hipError_t finish(const float *part, int S, int n, int N, const float *bias, float *out, float *kc, float *vc, int E,
                  int D, int P, int p0, hipStream_t s) {
  const size_t total = (size_t)n * N;
  prefill_finish<QKV><<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(part, S, n, N, bias, out, kc, vc, E, D,
                                                                             P, p0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &p, hipStream_t s) {
  const int E = p.E, F = 4 * p.E, D = p.D, H = p.E / p.D, n = p.n;
  // E % 64: whole GEMM column tiles (N = 3E, E, 4E) and stages of 64 (K = E, 4E);
  // E <= 2048: the head's input chunks fit its registers; D of 32 or 64
  // the head's argmax candidates ((V + 15) / 16 pairs) reuse the partials buffer
  if (n < 1 || p.cus < 1 || E % 64 != 0 || E > 4 * 64 * HEAD_XCH || (D != 32 && D != 64) ||
      (size_t)(p.V + 15) / 16 * sizeof(float2) > (size_t)4 * p.P * E * sizeof(float))
    return hipErrorInvalidValue;
  const DecodeArgs &a = *p.dec;
  const dim3 rows((unsigned)((n + 3) / 4));
  const size_t cap = (size_t)4 * p.P * E;  // floats of the partials buffer
  // x_n lives in p.att (the attention output's buffer) whenever attention is not
  // using it; the projections' partial sums in p.part
  float *xn = p.att;
  prefill_embed_ln<<<rows, 256, 0, s>>>(p.tok, a.wte, a.wpe, E, p.p0, n, a.ln1w, a.ln1b, a.eps, p.x, xn);
  hipError_t e = hipGetLastError();
  const size_t wq = (size_t)3 * E * E, wa = (size_t)E * E, wf = (size_t)F * E;
  auto wptr = [&](const MatW &m, size_t elems_per_layer, int l) {
    const size_t o = (size_t)l * elems_per_layer;
    const void *w = p.wd == WD_F32 ? (const void *)(static_cast<const float *>(m.w) + o)
                    : p.wd == WD_F16 ? (const void *)(static_cast<const __half *>(m.w) + o)
                                     : (const void *)(static_cast<const uint8_t *>(m.w) + o / 2);
    return std::make_pair(w, m.sz ? m.sz + o / 32 : nullptr);
  };
  for (int l = 0; l < p.L && e == hipSuccess; l++) {
    GemmArgs g{};
    g.n_rows = n;
    g.E = E;
    g.D = D;
    g.P = p.P;
    g.p0 = p.p0;
    g.splits = 1;
    // QKV with the new cache rows (x_n = LN1 of the rows)
    auto q = wptr(a.qkv, wq, l);
    g.a = xn; g.w = q.first; g.sz = q.second; g.bias = a.bqkv + (size_t)l * 3 * E;
    g.N = 3 * E; g.K = E; g.out = p.qkv;
    g.kc = a.kc + (size_t)l * H * p.P * D; g.vc = a.vc + (size_t)l * H * p.P * D;
    g.splits = pick_splits(n, g.N, g.K, false, p.cus, cap);
    if (g.splits == 1) {
      e = gemm_wd<PF_QKV>(p.wd, g, p.cus, s);
    } else {
      g.out = p.part;
      e = gemm_wd<PF_PART>(p.wd, g, p.cus, s);
      if (e == hipSuccess) e = finish<true>(p.part, g.splits, n, g.N, g.bias, p.qkv, g.kc, g.vc, E, D, p.P, p.p0, s);
    }
    if (e != hipSuccess) break;
    const dim3 ag((unsigned)((n + 15) / 16 * H));
    if (D == 64) prefill_attention<64><<<ag, 256, 0, s>>>(p.qkv, g.kc, g.vc, E, p.P, p.p0, n, p.cus, p.att);
    else prefill_attention<32><<<ag, 256, 0, s>>>(p.qkv, g.kc, g.vc, E, p.P, p.p0, n, p.cus, p.att);
    e = hipGetLastError();
    if (e != hipSuccess) break;
    // attention projection (partials), then x += sum + b and x_n = LN2(x)
    auto ap = wptr(a.ap, wa, l);
    g.a = p.att; g.w = ap.first; g.sz = ap.second; g.bias = nullptr;
    g.N = E; g.K = E; g.out = p.part; g.splits = pick_splits(n, E, E, true, p.cus, cap);
    e = gemm_wd<PF_PART>(p.wd, g, p.cus, s);
    if (e != hipSuccess) break;
    e = resid_ln(p.part, g.splits, n, E, a.bap + (size_t)l * E, a.ln2w + (size_t)l * E, a.ln2b + (size_t)l * E,
                 a.eps, p.x, xn, s);
    if (e != hipSuccess) break;
    // fc + gelu_new
    auto fc = wptr(a.fc, wf, l);
    g.a = xn; g.w = fc.first; g.sz = fc.second; g.bias = a.bfc + (size_t)l * F;
    g.N = F; g.K = E; g.out = p.act; g.splits = pick_splits(n, F, E, false, p.cus, cap);
    if (g.splits == 1) {
      e = gemm_wd<PF_GELU>(p.wd, g, p.cus, s);
    } else {
      g.out = p.part;
      e = gemm_wd<PF_PART>(p.wd, g, p.cus, s);
      if (e == hipSuccess) e = finish<false>(p.part, g.splits, n, F, g.bias, p.act, nullptr, nullptr, E, D, p.P, p.p0, s);
    }
    if (e != hipSuccess) break;
    // MLP projection (partials), then x += sum + b and x_n = the next LayerNorm
    auto pr = wptr(a.pr, wf, l);
    g.a = p.act; g.w = pr.first; g.sz = pr.second; g.bias = nullptr;
    g.N = E; g.K = F; g.out = p.part; g.splits = pick_splits(n, E, F, true, p.cus, cap);
    e = gemm_wd<PF_PART>(p.wd, g, p.cus, s);
    if (e != hipSuccess) break;
    const bool last = l + 1 == p.L;
    const float *gam = last ? a.lnfw : a.ln1w + (size_t)(l + 1) * E;
    const float *bet = last ? a.lnfb : a.ln1b + (size_t)(l + 1) * E;
    e = resid_ln(p.part, g.splits, n, E, a.bpr + (size_t)l * E, gam, bet, a.eps, p.x, xn, s);
  }
  if (e != hipSuccess) return e;
  // the head on the last row of x_n (the final LayerNorm), the argmax
  const float *xl = xn + (size_t)(n - 1) * E;
  // the head workgroups' argmax candidates go to the (now free) partials buffer
  const int hb = (p.V + 15) / 16;
  float2 *best = reinterpret_cast<float2 *>(p.part);
  if (p.head_wd == WD_F16) prefill_head<WD_F16><<<hb, 256, 0, s>>>(a.head, xl, E, p.V, a.logits, best);
  else prefill_head<WD_F32><<<hb, 256, 0, s>>>(a.head, xl, E, p.V, a.logits, best);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_argmax<<<1, 1024, 0, s>>>(best, hb, p.argmax);
  return hipGetLastError();
}

}  // namespace gpt2dec

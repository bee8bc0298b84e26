// prefill.hip -- batched prompt prefill: the n prompt positions of a call go
// through every layer together, so each linear is a GEMM of n rows against the
// weights (read once per layer instead of once per position), run on the
// matrix cores.
//
// Per layer (n rows at positions p0 .. p0+n-1):
//   gemm  LN1 of the rows (in the prologue), x W_qkv^T + b, and the new key and
//         value rows written into the cache (in the epilogue)
//   attn  per (row, head): causal softmax over the cached positions 0..p, the
//         weighted sum of values (running maximum and sum, 64 positions a step)
//   gemm  x += attn W_ap^T + b
//   gemm  gelu_new(LN2 of the rows W_fc^T + b)
//   gemm  x += act W_pr^T + b
// then the last row's final LayerNorm, the head (its logits) and the argmax.
//
// GEMM tile: a workgroup of four waves computes 16 rows x 16 output columns
// with v_mfma_f32_16x16x4f32 (lane l holds A[l%16][l/16] and B[l/16][l%16];
// result element i of lane l is C[4*(l/16)+i][l%16]).  Wave w contracts the
// quarter w of K; inside it the MFMA's four k slots take four contiguous runs
// of S = K/16 inputs (slot g: kq + g*S + s for step s), so each lane reads its
// A and W values as float4 runs.  The four partial tiles are summed in LDS in
// wave order.  fp16 weights are widened exactly; int4 weights become
// zero + code * scale with one rounding, the values the quantised model
// defines; the products and sums are fp32 throughout.
#include <hip/hip_fp16.h>

#include <utility>

#include "dec_internal.h"

namespace gpt2dec {
namespace {

typedef float pf_f4 __attribute__((ext_vector_type(4)));

enum { PF_QKV = 0, PF_RESID = 1, PF_GELU = 2, PF_HEAD = 3 };

__device__ __forceinline__ float pf_wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float pf_wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Four consecutive weights of output row `row` from input k (a multiple of 4),
// as fp32.
template <int WD>
__device__ __forceinline__ float4 pf_w4(const void *w, const float2 *sz, size_t row, int K, int k) {
  if constexpr (WD == WD_F32) {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(w) + row * K + k);
  } else if constexpr (WD == WD_F16) {
    const uint2 h = *reinterpret_cast<const uint2 *>(static_cast<const __half *>(w) + row * K + k);
    return make_float4(__half2float(__ushort_as_half((unsigned short)(h.x & 0xffffu))),
                       __half2float(__ushort_as_half((unsigned short)(h.x >> 16))),
                       __half2float(__ushort_as_half((unsigned short)(h.y & 0xffffu))),
                       __half2float(__ushort_as_half((unsigned short)(h.y >> 16))));
  } else {
    const uint32_t q = *reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(w) + (row * K + k) / 2);
    const float2 p = sz[(row * K + k) / 32];
    return make_float4(__builtin_fmaf((float)(q & 15u), p.x, p.y), __builtin_fmaf((float)((q >> 4) & 15u), p.x, p.y),
                       __builtin_fmaf((float)((q >> 8) & 15u), p.x, p.y),
                       __builtin_fmaf((float)((q >> 12) & 15u), p.x, p.y));
  }
}

__device__ __forceinline__ float pf_gelu_new(float x) {
  // x * logistic(2 * sqrt(2/pi) * (x + 0.044715 x^3))
  const float z2 = 1.5957691216057308f * __builtin_fmaf(0.044715f * x, x * x, x);
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-z2));
}

struct GemmArgs {
  const float *a;        // [rows][K] input rows (the residual stream for the LayerNorm modes)
  int a_row0;            // first input row of the call (the head: the last row)
  int n_rows;            // rows of the call
  const void *w;         // [N][K] output-major weights of this layer
  const float2 *sz;      // int4: (scale, zero) per group of 32
  const float *bias;     // [N] or null
  const float *gamma, *beta;  // LayerNorm modes
  float eps;
  int N, K;
  float *out;            // [rows][N] (QKV, gelu), the residual [rows][N] (RESID), [N] logits (HEAD)
  float *kc, *vc;        // QKV: this layer's cache blocks [H][P][D]
  int E, D, P, p0;
};

template <int WD, int MODE>
__global__ void __launch_bounds__(256) prefill_gemm(GemmArgs g) {
  constexpr bool LN = (MODE == PF_QKV || MODE == PF_GELU || MODE == PF_HEAD);
  __shared__ float red[4][16][17];
  extern __shared__ float as[];  // LayerNorm modes: [16][K + 4] normalised rows
  const int tid = threadIdx.x, wv = tid / 64, l = tid % 64;
  const int o0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int nv = min(16, g.n_rows - t0);  // valid rows of this tile
  const int K = g.K, AS = K + 4;
  if constexpr (LN) {
    // wave wv normalises rows wv, wv+4, ... of the tile (zeros past the valid rows)
    for (int r = wv; r < 16; r += 4) {
      float *dst = as + r * AS;
      if (r < nv) {
        const float *x = g.a + (size_t)(g.a_row0 + t0 + r) * K;
        float s = 0.f;
        for (int k = l; k < K; k += 64) s += x[k];
        const float mean = pf_wave_sum(s) / (float)K;
        float q = 0.f;
        for (int k = l; k < K; k += 64) {
          const float d = x[k] - mean;
          q = __builtin_fmaf(d, d, q);
        }
        const float rstd = __builtin_amdgcn_rsqf(pf_wave_sum(q) / (float)K + g.eps);
        for (int k = l; k < K; k += 64) dst[k] = (x[k] - mean) * rstd * g.gamma[k] + g.beta[k];
      } else {
        for (int k = l; k < K; k += 64) dst[k] = 0.f;
      }
    }
    __syncthreads();
  }
  // this wave's quarter of K, the lane's k slot and row/column
  const int KQ = K / 4, S = K / 16, kq = wv * KQ;
  const int gs = l / 16, r = l % 16;
  const int kb = kq + gs * S;  // the lane's run of S inputs
  const size_t wrow = (size_t)min(o0 + r, g.N - 1);
  const int arow = min(r, max(nv - 1, 0));
  const float *ag = g.a + (size_t)(g.a_row0 + t0 + arow) * K;
  pf_f4 c = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; s += 4) {
    const float4 wq = pf_w4<WD>(g.w, g.sz, wrow, K, kb + s);
    float4 av;
    if constexpr (LN) av = *reinterpret_cast<const float4 *>(as + r * AS + kb + s);
    else av = (r < nv) ? *reinterpret_cast<const float4 *>(ag + kb + s) : make_float4(0.f, 0.f, 0.f, 0.f);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, wq.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, wq.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, wq.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, wq.w, c, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; i++) red[wv][4 * gs + i][r] = c[i];
  __syncthreads();
  // epilogue: thread (row i, column cc) sums the four waves' partials in order
  const int i = tid / 16, cc = tid % 16;
  const int t = t0 + i, o = o0 + cc;
  if (i >= nv || o >= g.N) return;
  const float v = ((red[0][i][cc] + red[1][i][cc]) + red[2][i][cc]) + red[3][i][cc];
  if constexpr (MODE == PF_HEAD) {
    g.out[o] = v;
  } else if constexpr (MODE == PF_RESID) {
    float *x = g.out + (size_t)t * g.N + o;
    *x = *x + (v + g.bias[o]);
  } else if constexpr (MODE == PF_GELU) {
    g.out[(size_t)t * g.N + o] = pf_gelu_new(v + g.bias[o]);
  } else {  // QKV: the row, and its key / value part into the cache at position p0 + t
    const float y = v + g.bias[o];
    g.out[(size_t)t * g.N + o] = y;
    if (o >= g.E) {
      const int e = (o - g.E) % g.E, h = e / g.D, d = e % g.D;
      float *cache = (o < 2 * g.E) ? g.kc : g.vc;
      cache[((size_t)h * g.P + g.p0 + t) * g.D + d] = y;
    }
  }
}

// x[t] = wte[token t] + wpe[p0 + t]
__global__ void __launch_bounds__(256) prefill_embed(const int *tok, const float *wte, const float *wpe, int E,
                                                     int p0, float *x) {
  const int t = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i < E) x[(size_t)t * E + i] = wte[(size_t)tok[t] * E + i] + wpe[(size_t)(p0 + t) * E + i];
}

// One wave per (row t, head h): causal attention of position p0 + t over the
// cache rows 0 .. p0 + t of this layer, 64 positions a step (lane = position
// for the scores, lane = dimension for the values), with a running maximum and
// sum.  out[t][h*D ..] = the weighted sum of values.
__global__ void __launch_bounds__(64) prefill_attention(const float *qkv, const float *kc, const float *vc, int E,
                                                        int D, int P, int p0, float *out) {
  __shared__ float q[64];
  __shared__ float e[64];
  const int t = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int p = p0 + t;
  const float scale = 1.0f / sqrtf((float)D);
  if (l < D) q[l] = qkv[(size_t)t * 3 * E + h * D + l];
  __syncthreads();
  const float *K = kc + (size_t)h * P * D, *V = vc + (size_t)h * P * D;
  float m = -INFINITY, ssum = 0.f, acc = 0.f;
  for (int j0 = 0; j0 <= p; j0 += 64) {
    const int j = j0 + l;
    float sc = -INFINITY;
    if (j <= p) {
      const float *kr = K + (size_t)j * D;
      float d0 = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 kk = *reinterpret_cast<const float4 *>(kr + d);
        d0 = __builtin_fmaf(kk.x, q[d], d0);
        d0 = __builtin_fmaf(kk.y, q[d + 1], d0);
        d0 = __builtin_fmaf(kk.z, q[d + 2], d0);
        d0 = __builtin_fmaf(kk.w, q[d + 3], d0);
      }
      sc = d0 * scale;
    }
    const float mn = fmaxf(m, pf_wave_max(sc));
    const float w = (j <= p) ? __expf(sc - mn) : 0.f;
    const float alpha = __expf(m - mn);  // 0 on the first step (m = -inf)
    ssum = ssum * alpha + pf_wave_sum(w);
    e[l] = w;
    __syncthreads();
    if (l < D) {
      float a = acc * alpha;
      const int jn = min(64, p + 1 - j0);
      for (int jj = 0; jj < jn; jj++) a = __builtin_fmaf(e[jj], V[(size_t)(j0 + jj) * D + l], a);
      acc = a;
    }
    m = mn;
    __syncthreads();
  }
  if (l < D) out[(size_t)t * E + h * D + l] = acc / ssum;
}

// The id of the largest logit, the lowest among equal ones (NaN never wins;
// -1 when every logit is NaN), by one workgroup.
__global__ void __launch_bounds__(1024) prefill_argmax(const float *logits, int V, int *out) {
  __shared__ float bv[1024];
  __shared__ int bi[1024];
  float v = -INFINITY;
  int idx = -1;
  for (int i = threadIdx.x; i < V; i += 1024) {
    const float x = logits[i];
    if (x > v || (idx < 0 && x == v)) {
      v = x;
      idx = i;
    }
  }
  bv[threadIdx.x] = v;
  bi[threadIdx.x] = idx;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      const float v2 = bv[threadIdx.x + s];
      const int i2 = bi[threadIdx.x + s];
      const float v1 = bv[threadIdx.x];
      const int i1 = bi[threadIdx.x];
      if (i2 >= 0 && (i1 < 0 || v2 > v1 || (v2 == v1 && i2 < i1))) {
        bv[threadIdx.x] = v2;
        bi[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = bi[0];
}

template <int WD, int MODE>
hipError_t gemm_launch(const GemmArgs &g, int m_tiles, hipStream_t s) {
  const dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)m_tiles);
  const size_t lds = (MODE == PF_RESID) ? 0 : (size_t)16 * (g.K + 4) * sizeof(float);
  if (lds > 64 * 1024) {  // wide models: the normalised rows take more than the default 64 KiB
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_gemm<WD, MODE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  prefill_gemm<WD, MODE><<<grid, 256, lds, s>>>(g);
  return hipGetLastError();
}

template <int MODE>
hipError_t gemm_wd(int wd, const GemmArgs &g, int m_tiles, hipStream_t s) {
  if (wd == WD_F32) return gemm_launch<WD_F32, MODE>(g, m_tiles, s);
  if (wd == WD_F16) return gemm_launch<WD_F16, MODE>(g, m_tiles, s);
  return gemm_launch<WD_Q4, MODE>(g, m_tiles, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &p, hipStream_t s) {
  const int E = p.E, F = 4 * p.E, D = p.D, H = p.E / p.D, n = p.n;
  // (K = E or 4E: a multiple of 64 makes each lane's run of K/16 inputs whole float4 steps)
  // (the LayerNorm tiles hold 16 rows of E + 4 floats in LDS: at most 160 KiB)
  if (n < 1 || E % 64 != 0 || D % 4 != 0 || D > 64 || (size_t)16 * (E + 4) * 4 > 160 * 1024)
    return hipErrorInvalidValue;
  const int mt = (n + 15) / 16;
  const DecodeArgs &a = *p.dec;
  prefill_embed<<<dim3((unsigned)((E + 255) / 256), (unsigned)n), 256, 0, s>>>(p.tok, a.wte, a.wpe, E, p.p0, p.x);
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
    g.eps = a.eps;
    g.E = E;
    g.D = D;
    g.P = p.P;
    g.p0 = p.p0;
    // LN1 + QKV, with the new cache rows
    auto q = wptr(a.qkv, wq, l);
    g.a = p.x; g.w = q.first; g.sz = q.second; g.bias = a.bqkv + (size_t)l * 3 * E;
    g.gamma = a.ln1w + (size_t)l * E; g.beta = a.ln1b + (size_t)l * E;
    g.N = 3 * E; g.K = E; g.out = p.qkv;
    g.kc = a.kc + (size_t)l * H * p.P * D; g.vc = a.vc + (size_t)l * H * p.P * D;
    e = gemm_wd<PF_QKV>(p.wd, g, mt, s);
    if (e != hipSuccess) break;
    prefill_attention<<<dim3((unsigned)n, (unsigned)H), 64, 0, s>>>(p.qkv, g.kc, g.vc, E, D, p.P, p.p0, p.att);
    e = hipGetLastError();
    if (e != hipSuccess) break;
    // attention projection + residual
    auto ap = wptr(a.ap, wa, l);
    g.a = p.att; g.w = ap.first; g.sz = ap.second; g.bias = a.bap + (size_t)l * E;
    g.N = E; g.K = E; g.out = p.x;
    e = gemm_wd<PF_RESID>(p.wd, g, mt, s);
    if (e != hipSuccess) break;
    // LN2 + fc + gelu_new
    auto fc = wptr(a.fc, wf, l);
    g.a = p.x; g.w = fc.first; g.sz = fc.second; g.bias = a.bfc + (size_t)l * F;
    g.gamma = a.ln2w + (size_t)l * E; g.beta = a.ln2b + (size_t)l * E;
    g.N = F; g.K = E; g.out = p.act;
    e = gemm_wd<PF_GELU>(p.wd, g, mt, s);
    if (e != hipSuccess) break;
    // MLP projection + residual
    auto pr = wptr(a.pr, wf, l);
    g.a = p.act; g.w = pr.first; g.sz = pr.second; g.bias = a.bpr + (size_t)l * E;
    g.N = E; g.K = F; g.out = p.x;
    e = gemm_wd<PF_RESID>(p.wd, g, mt, s);
  }
  if (e != hipSuccess) return e;
  // final LayerNorm of the last row, the head, the argmax
  GemmArgs g{};
  g.a = p.x; g.a_row0 = n - 1; g.n_rows = 1;
  g.w = a.head; g.sz = nullptr; g.bias = nullptr; g.gamma = a.lnfw; g.beta = a.lnfb; g.eps = a.eps;
  g.N = p.V; g.K = E; g.out = a.logits;
  e = gemm_wd<PF_HEAD>(p.head_wd, g, 1, s);
  if (e != hipSuccess) return e;
  prefill_argmax<<<1, 1024, 0, s>>>(a.logits, p.V, p.argmax);
  return hipGetLastError();
}

}  // namespace gpt2dec

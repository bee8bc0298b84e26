// relayout.hip -- one-time weight re-layout at load (gfx950).
//
// The checkpoint stores the four block matrices as Conv1D [input][output]; the
// decode kernel streams them output-major, each output row contiguous (gpt2.s
// README, "Inner Workings"; blog Step 1: the transposed layout is what makes
// the matrix-vector product read memory in order).  These kernels transpose
// through LDS tiles so that both the read of a source row and the write of a
// destination row are coalesced, and optionally convert on the way:
//   fp16 : round to nearest even (v_cvt_f16_f32 in the default mode), subnormals kept;
//   int4 : after the transpose, groups of 32 inputs of one output row are
//          quantised asymmetrically: lo/hi = group min/max, scale = (hi-lo)/15,
//          zero = lo, code = clamp(rint((w-lo)/scale), 0, 15) (0 if scale is 0);
//          two codes per byte, the even input in the low nibble.
#include <hip/hip_fp16.h>

#include "dec_internal.h"

namespace gpt2dec {
namespace {

constexpr int TT = 32;  // transpose tile

// dst[n][k] = src[k][n]; src is K x N row-major.
template <typename Out>
__global__ void __launch_bounds__(256) transpose_kernel(const float *__restrict__ src, Out *__restrict__ dst,
                                                        int K, int N) {
  __shared__ float tile[TT][TT + 1];
  const int n0 = blockIdx.x * TT, k0 = blockIdx.y * TT;
  const int tx = threadIdx.x % TT, ty = threadIdx.x / TT;  // 32 x 8
  for (int r = ty; r < TT; r += 8) {
    const int k = k0 + r, n = n0 + tx;
    tile[r][tx] = (k < K && n < N) ? src[(size_t)k * N + n] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < TT; r += 8) {
    const int n = n0 + r, k = k0 + tx;
    if (n < N && k < K) {
      const float v = tile[tx][r];
      if constexpr (sizeof(Out) == 4) dst[(size_t)n * K + k] = v;
      else dst[(size_t)n * K + k] = __float2half_rn(v);
    }
  }
}

// One thread per (row, group of 32): quantise tmp[N][K] into nibbles + (scale, zero).
__global__ void __launch_bounds__(256) quantise_q4_kernel(const float *__restrict__ tmp, uint8_t *__restrict__ nib,
                                                          float2 *__restrict__ sz, int K, int N) {
#pragma clang fp contract(off)
  const int groups = K / 32;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (size_t)N * groups) return;
  const size_t row = gid / groups, g = gid % groups;
  const float *w = tmp + row * K + g * 32;
  float lo = w[0], hi = w[0];
  for (int i = 1; i < 32; i++) {
    if (w[i] < lo) lo = w[i];
    if (w[i] > hi) hi = w[i];
  }
  const float scale = (hi - lo) / 15.0f;
  uint8_t *out = nib + (row * K + g * 32) / 2;
  for (int i = 0; i < 32; i += 2) {
    int c[2];
    for (int j = 0; j < 2; j++) {
      int q = 0;
      if (scale != 0.0f) {
        float r = rintf((w[i + j] - lo) / scale);
        if (r < 0.0f) r = 0.0f;
        if (r > 15.0f) r = 15.0f;
        q = (int)r;
      }
      c[j] = q;
    }
    out[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
  }
  sz[gid] = make_float2(scale, lo);
}

__global__ void __launch_bounds__(256) convert_f16_kernel(const float *__restrict__ src, __half *__restrict__ dst,
                                                          size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __float2half_rn(src[i]);
}

__global__ void __launch_bounds__(256) fill_kernel(float *dst, size_t n, float v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = v;
}

// Chunk c (4 consecutive elements) of an output-major matrix from element
// offset lofs, as the weights the stored data stand for: fp32 as is, fp16
// widened (exact), int4 as zero + code * scale with one rounding.  This reads
// the same stored codes, scales and zeros as the GEMV, but the int4 GEMV does
// not form these values: it sums scale * sum(code * x) + zero * sum(x) over a
// group's inputs.  So a bitwise comparison of this decode pins the stored
// data; the int4 dot products are pinned through the logits only.
__device__ __forceinline__ float4 chunk_f4(int wd, const void *w, const float2 *szp, size_t lofs, size_t c) {
  if (wd == WD_F32) return reinterpret_cast<const float4 *>(w)[lofs / 4 + c];
  if (wd == WD_F16) {
    const uint2 h = reinterpret_cast<const uint2 *>(w)[lofs / 4 + c];
    return make_float4(__half2float(__ushort_as_half((unsigned short)(h.x & 0xffffu))),
                       __half2float(__ushort_as_half((unsigned short)(h.x >> 16))),
                       __half2float(__ushort_as_half((unsigned short)(h.y & 0xffffu))),
                       __half2float(__ushort_as_half((unsigned short)(h.y >> 16))));
  }
  const uint32_t q = reinterpret_cast<const uint16_t *>(w)[lofs / 4 + c];
  const float2 p = szp[lofs / 32 + c / 8];
  return make_float4(__builtin_fmaf((float)(q & 15u), p.x, p.y), __builtin_fmaf((float)((q >> 4) & 15u), p.x, p.y),
                     __builtin_fmaf((float)((q >> 8) & 15u), p.x, p.y),
                     __builtin_fmaf((float)((q >> 12) & 15u), p.x, p.y));
}

__global__ void __launch_bounds__(256) dequant_kernel(int wd, const void *w, const float2 *szp, size_t lofs,
                                                      size_t nchunks, float *__restrict__ dst) {
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  reinterpret_cast<float4 *>(dst)[c] = chunk_f4(wd, w, szp, lofs, c);
}

// One thread per output row n of W (the weights as the GEMV decodes them):
// gsum[n] = sum_k W[n][k] * gain[k] and bsum[n] = sum_k W[n][k] * shift[k] + bias[n],
// accumulated in double and rounded once.
__global__ void __launch_bounds__(256) fold_ln_kernel(int wd, const void *w, const float2 *szp, size_t lofs, int N,
                                                      int K, const float *__restrict__ gain,
                                                      const float *__restrict__ shift,
                                                      const float *__restrict__ bias, float *__restrict__ gsum,
                                                      float *__restrict__ bsum) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  double sg = 0.0, sb = 0.0;
  for (int c = 0; c < K / 4; c++) {
    const float4 v = chunk_f4(wd, w, szp, lofs, (size_t)n * (K / 4) + c);
    const float wv[4] = {v.x, v.y, v.z, v.w};
    for (int i = 0; i < 4; i++) {
      sg += (double)wv[i] * (double)gain[4 * c + i];
      sb += (double)wv[i] * (double)shift[4 * c + i];
    }
  }
  gsum[n] = (float)sg;
  bsum[n] = (float)(sb + (bias ? (double)bias[n] : 0.0));
}

inline unsigned blocks_for(size_t n, unsigned t) { return (unsigned)((n + t - 1) / t); }

}  // namespace

hipError_t relayout_f32(const float *src, float *dst, int K, int N, hipStream_t s) {
  dim3 grid((N + TT - 1) / TT, (K + TT - 1) / TT);
  transpose_kernel<float><<<grid, 256, 0, s>>>(src, dst, K, N);
  return hipGetLastError();
}

hipError_t relayout_f16(const float *src, void *dst, int K, int N, hipStream_t s) {
  dim3 grid((N + TT - 1) / TT, (K + TT - 1) / TT);
  transpose_kernel<__half><<<grid, 256, 0, s>>>(src, reinterpret_cast<__half *>(dst), K, N);
  return hipGetLastError();
}

hipError_t relayout_q4(const float *src, float *tmp, uint8_t *nib, float2 *sz, int K, int N, hipStream_t s) {
  hipError_t e = relayout_f32(src, tmp, K, N, s);
  if (e != hipSuccess) return e;
  const size_t groups = (size_t)N * (K / 32);
  quantise_q4_kernel<<<blocks_for(groups, 256), 256, 0, s>>>(tmp, nib, sz, K, N);
  return hipGetLastError();
}

hipError_t convert_f16(const float *src, void *dst, size_t n, hipStream_t s) {
  convert_f16_kernel<<<blocks_for(n, 256), 256, 0, s>>>(src, reinterpret_cast<__half *>(dst), n);
  return hipGetLastError();
}

hipError_t fold_ln(int wd, const MatW &m, size_t lofs, int N, int K, const float *gain, const float *shift,
                   const float *bias, float *gsum, float *bsum, hipStream_t s) {
  if (N <= 0 || K % 4 != 0) return hipErrorInvalidValue;
  fold_ln_kernel<<<blocks_for((size_t)N, 256), 256, 0, s>>>(wd, m.w, m.sz, lofs, N, K, gain, shift, bias, gsum,
                                                           bsum);
  return hipGetLastError();
}

hipError_t fill_f32(float *dst, size_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_kernel<<<blocks_for(n, 256), 256, 0, s>>>(dst, n, v);
  return hipGetLastError();
}

hipError_t debug_dequant(int wd, const MatW &m, size_t lofs, int N, int K, float *dst, hipStream_t s) {
  const size_t nch = (size_t)N * K / 4;
  dequant_kernel<<<blocks_for(nch, 256), 256, 0, s>>>(wd, m.w, m.sz, lofs, nch, dst);
  return hipGetLastError();
}

}  // namespace gpt2dec

// decode_kernel.hip -- the persistent batch-1 GPT-2 decode kernel for gfx950.
//
// One cooperative launch runs `nsteps` whole forward passes (one token each).
// The per-token work follows the node order of the gpt2-125m "model.fir" file:
// embedding add, then per layer
//   A: LayerNorm 1 + QKV linear + bias          (K/V of this position kept for attention)
//   B: attn_decode over positions 0..position   (split over position chunks)
//   C: chunk merge + attention linear + bias + residual
//   D: LayerNorm 2 + fc linear + bias + gelu_new
//   E: projection linear + bias + residual
// and finally H: final LayerNorm + tied output head + argmax.
//
// Work split.  Every workgroup owns RAP consecutive rows of each E-output
// matrix (3*RAP of QKV, 4*RAP of fc), so the 256 workgroups of the 124M shape
// each stream an equal 1/256 of every matrix, and a contiguous 1/256 of the
// head.  A workgroup is one control wave plus NCW compute waves:
//   * compute waves hold the workgroup's weight slices of a whole layer in
//     registers and re-issue the loads for the next layer as soon as a slice
//     has been used, so the HBM stream runs a full layer ahead of the
//     dependency chain;
//   * the control wave waits for the inputs of each phase, normalises them
//     into LDS, and publishes the phase's outputs.
// Batch 1 makes every linear a matrix-vector product (0.5 flop per fp32 byte),
// so there is no MFMA here: the kernel is bound by weight bytes and by the
// latency of the 5L+1 dependent phases of a token.
//
// Synchronisation.  There is no grid barrier.  Each output element is written
// as one 64-bit agent-scope atomic word (float bits | epoch << 32), where the
// epoch numbers the producing phase uniquely within and across launches; a
// consumer polls the words it needs until all carry the expected epoch.  Per-
// location atomic coherence is all this needs: no cache write-back/invalidate
// fences are executed in the loop.  KV-cache rows are written with
// agent-scope stores one step before any other workgroup reads them.
#include <hip/hip_fp16.h>

#include "dec_internal.h"

namespace gpt2dec {
namespace {

constexpr int CHMIN = 16;      // positions per attention chunk before a head is split further
constexpr int PSTRIDE = 256;   // LDS stride of per-wave partial sums (>= rows per workgroup)

template <int E_, int D_, int NCW_, int RAP_, int MAXCH_>
struct Shape {
  static constexpr int E = E_, D = D_, H = E_ / D_, F = 4 * E_;
  static constexpr int NCW = NCW_;        // compute waves
  static constexpr int NL = 64 * NCW_;    // compute lanes
  static constexpr int NT = NL + 64;      // threads: compute waves + control wave
  static constexpr int RAP = RAP_;        // rows of an E-output matrix per workgroup
  static constexpr int G = E_ / RAP_;     // workgroups
  static constexpr int MAXCH = MAXCH_;    // attention chunks per head at most
  static_assert(E_ % D_ == 0 && E_ % 64 == 0, "shape");
  static_assert(H * MAXCH <= G, "one attention chunk per workgroup at most");
  // LDS layout (floats)
  static constexpr int L_XS = 0;                         // [F] phase input vector
  static constexpr int L_PART = L_XS + F;                // [NCW][PSTRIDE] partial row sums
  static constexpr int L_Q = L_PART + NCW * PSTRIDE;     // [D] query of the attention item
  static constexpr int L_KP = L_Q + D;                   // [D] key of this position
  static constexpr int L_VP = L_KP + D;                  // [D] value of this position
  static constexpr int L_SC = L_VP + D;                  // [64] chunk scores / weights
  static constexpr int L_SLOT = L_SC + 64;               // [D+2] chunk output (o, m, l)
  static constexpr int L_FLAG = L_SLOT + D + 2;          // [4] control flags
  static constexpr int L_TOTAL = L_FLAG + 4;
};

// 124M shape: 256 workgroups x (3 compute + 1 control) waves.
using ShapeS = Shape<768, 64, 3, 3, 16>;
// tiny shape: 32 workgroups x (2 compute + 1 control) waves.
using ShapeT = Shape<128, 32, 2, 4, 8>;

// Rows of length K split in 4-element chunks over the NL compute lanes: either
// a row spans whole passes of all lanes (ROWWIDE, PPR passes per row) or one
// pass covers RPP rows of KC lanes each.
template <class S, int K>
struct RowGeo {
  static constexpr int KC = K / 4;
  static constexpr bool ROWWIDE = (KC % S::NL) == 0;
  static_assert(ROWWIDE || (S::NL % KC == 0 && KC <= 64), "unsupported row geometry");
  static constexpr int PPR = ROWWIDE ? KC / S::NL : 1;
  static constexpr int RPP = ROWWIDE ? 1 : S::NL / KC;
};

// Geometry of one workgroup slice: R rows of length K.
template <class S, int R, int K>
struct Geo : RowGeo<S, K> {
  static constexpr int NCH = R * RowGeo<S, K>::KC;
  static_assert(NCH % S::NL == 0, "slice must split evenly over compute lanes");
  static constexpr int NPASS = NCH / S::NL;
};

// ---- weight chunks: 4 consecutive inputs of one output row ----------------
template <int WD> struct Chunk;
template <> struct Chunk<WD_F32> { float4 v; };
template <> struct Chunk<WD_F16> { uint2 v; };
template <> struct Chunk<WD_Q4> { uint32_t q; float2 sz; };

// gc: chunk index inside the layer's [N][K] matrix (= row*K/4 + k/4);
// lofs: element offset of the layer (= layer*N*K).
template <int WD>
__device__ __forceinline__ Chunk<WD> ld_chunk(const MatW &m, size_t lofs, size_t gc) {
  Chunk<WD> c;
  if constexpr (WD == WD_F32) {
    c.v = reinterpret_cast<const float4 *>(m.w)[lofs / 4 + gc];
  } else if constexpr (WD == WD_F16) {
    c.v = reinterpret_cast<const uint2 *>(m.w)[lofs / 4 + gc];
  } else {
    c.q = reinterpret_cast<const uint16_t *>(m.w)[lofs / 4 + gc];
    c.sz = m.sz[lofs / 32 + gc / 8];
  }
  return c;
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

// The weights a chunk stands for, as fp32.  fp16 widening is exact; int4 is
// dequantised with one fused multiply-add per weight: fma(code, scale, zero).
template <int WD>
__device__ __forceinline__ float4 deq(const Chunk<WD> &c) {
  if constexpr (WD == WD_F32) {
    return c.v;
  } else if constexpr (WD == WD_F16) {
    return make_float4(h2f(c.v.x), h2f(c.v.x >> 16), h2f(c.v.y), h2f(c.v.y >> 16));
  } else {
    const float s = c.sz.x, z = c.sz.y;
    return make_float4(__builtin_fmaf((float)(c.q & 15u), s, z),
                       __builtin_fmaf((float)((c.q >> 4) & 15u), s, z),
                       __builtin_fmaf((float)((c.q >> 8) & 15u), s, z),
                       __builtin_fmaf((float)((c.q >> 12) & 15u), s, z));
  }
}

__device__ __forceinline__ float dot4(float4 w, float4 x, float acc) {
  acc = __builtin_fmaf(w.x, x.x, acc);
  acc = __builtin_fmaf(w.y, x.y, acc);
  acc = __builtin_fmaf(w.z, x.z, acc);
  acc = __builtin_fmaf(w.w, x.w, acc);
  return acc;
}

// Butterfly reductions: every lane of the group ends with the same bits.
template <int W>
__device__ __forceinline__ float seg_sum(float a) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) a += __shfl_xor(a, m, 64);
  return a;
}
__device__ __forceinline__ float wave_sum(float a) { return seg_sum<64>(a); }
__device__ __forceinline__ float wave_max(float a) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
  return a;
}

__device__ __forceinline__ void wg_barrier() {
  // LDS writes of this wave are complete, then the workgroup barrier; vector
  // memory loads in flight (weight prefetch) are deliberately not waited for.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- tagged cross-workgroup words -----------------------------------------
__device__ __forceinline__ uint64_t tld(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tst(uint64_t *p, float v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tst_u(uint64_t *p, uint32_t v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | (uint64_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded waiting: a wait that outlives the time limit, or sees another
// workgroup's abort, sets the error word and makes the caller stop.
struct Waiter {
  const DecodeArgs *a;
  long long t0;
  int phase;
  __device__ bool expired() {
    if (__hip_atomic_load(a->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    if ((long long)wall_clock64() - t0 > a->timeout_ticks) {
      int zero = 0;
      if (__hip_atomic_compare_exchange_strong(a->err, &zero, 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        __hip_atomic_store(a->err + 1, (int)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a->err + 2, phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return true;
    }
    return false;
  }
};

// Poll PER*64 tagged floats (element lane + 64*j) into v until all carry ep.
template <int PER>
__device__ bool poll_vec(const uint64_t *src, uint32_t ep, float (&v)[PER], int lane, Waiter &wt) {
  while (true) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PER; j++) {
      const uint64_t x = tld(src + lane + 64 * j);
      v[j] = __uint_as_float((uint32_t)x);
      ok &= ((uint32_t)(x >> 32) == ep);
    }
    if (__all(ok)) return true;
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// LayerNorm of E values held lane-strided (element lane + 64*j) into LDS,
// following the model file's layernorm kernel: mean, biased variance,
// ((x - mean) * rsqrt(var + eps)) * gamma + beta.
template <int E>
__device__ __forceinline__ void layernorm_to_lds(const float (&x)[E / 64], const float (&g)[E / 64],
                                                 const float (&b)[E / 64], float eps, float *dst,
                                                 int lane) {
  constexpr int PER = E / 64;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < PER; j++) s += x[j];
  const float mean = wave_sum(s) * (1.0f / (float)E);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const float d = x[j] - mean;
    q = __builtin_fmaf(d, d, q);
  }
  const float var = wave_sum(q) * (1.0f / (float)E);
  const float r = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < PER; j++) dst[lane + 64 * j] = __builtin_fmaf((x[j] - mean) * r, g[j], b[j]);
}

__device__ __forceinline__ float gelu_new(float f) {
  // x * sigmoid(2*sqrt(2/pi) * (x + 0.044715 x^3)), the model file's gelu_new
  float t = f * f;
  t = t * f;
  t = t * 0.044715f;
  t = t + f;
  t = t * 1.5957691216057308f;
  t = 1.0f / (1.0f + expf(-t));
  return f * t;
}

// Attention chunking of positions 0..p: nch chunks of ch positions (last one shorter).
template <class S>
__device__ __forceinline__ void att_chunks(int p, int &nch, int &ch) {
  const int n = p + 1;
  nch = (n + CHMIN - 1) / CHMIN;
  if (nch > S::MAXCH) nch = S::MAXCH;
  ch = (n + nch - 1) / nch;
}

template <class S>
__device__ __forceinline__ uint32_t epoch_of(const DecodeArgs &a, int step, int ph) {
  return a.epoch0 + (uint32_t)step * (uint32_t)(5 * a.L + 1) + (uint32_t)ph + 1u;
}

// ---- compute waves ---------------------------------------------------------
template <class S, int R, int K, int WD, int NP>
__device__ __forceinline__ void load_slice(Chunk<WD> (&w)[NP], const MatW &m, int layer, int lane) {
  using Gm = Geo<S, R, K>;
  static_assert(NP == Gm::NPASS, "register slice size");
  const size_t lofs = (size_t)layer * (size_t)(R * S::G) * K;
  const size_t c0 = (size_t)blockIdx.x * Gm::NCH + lane;
#pragma unroll
  for (int i = 0; i < Gm::NPASS; i++) w[i] = ld_chunk<WD>(m, lofs, c0 + (size_t)i * S::NL);
}

template <class S, int R, int K, int WD, int NP>
__device__ __forceinline__ void slice_dot(const Chunk<WD> (&w)[NP], const float *xs, float *part, int lane) {
  using Gm = Geo<S, R, K>;
  static_assert(NP == Gm::NPASS, "register slice size");
  if constexpr (Gm::ROWWIDE) {
    const int wave = lane >> 6;
#pragma unroll
    for (int r = 0; r < R; r++) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < Gm::PPR; j++) {
        const float4 x = reinterpret_cast<const float4 *>(xs)[j * S::NL + lane];
        a = dot4(deq<WD>(w[r * Gm::PPR + j]), x, a);
      }
      a = wave_sum(a);
      if ((lane & 63) == 0) part[wave * PSTRIDE + r] = a;
    }
  } else {
    const int kc = lane % Gm::KC;
    const float4 x = reinterpret_cast<const float4 *>(xs)[kc];
#pragma unroll
    for (int i = 0; i < Gm::NPASS; i++) {
      float a = dot4(deq<WD>(w[i]), x, 0.f);
      a = seg_sum<Gm::KC>(a);
      if (kc == 0) part[i * Gm::RPP + lane / Gm::KC] = a;
    }
  }
}

// Row total from the partials (read by the control wave).
template <class S, int K>
__device__ __forceinline__ float row_total(const float *part, int r) {
  using Gm = RowGeo<S, K>;
  if constexpr (Gm::ROWWIDE) {
    float t = part[r];
#pragma unroll
    for (int w = 1; w < S::NCW; w++) t += part[w * PSTRIDE + r];
    return t;
  } else {
    return part[r];
  }
}

// One attention chunk (head h, positions t0..t1-1) on the control wave.  Scores and
// softmax weights follow the attn_decode kernel (q.k * 1/sqrt(D), subtract the
// maximum, exp); the chunk leaves (o = sum e_t v_t, m = max, l = sum e_t) for
// the merge.
template <class S>
__device__ void attention_chunk(const DecodeArgs &a, float *lds, int l, int h, int p, int t0, int t1,
                                int lane) {
  constexpr int D = S::D, D4 = D / 4, RPL = 64 / D4;
  const float *K = a.kc + ((size_t)(l * S::H + h) * a.P) * D;
  const float *V = a.vc + ((size_t)(l * S::H + h) * a.P) * D;
  const float scale = 1.0f / sqrtf((float)D);
  const float4 q4 = reinterpret_cast<const float4 *>(lds + S::L_Q)[lane % D4];
  const int n = t1 - t0;
  const bool last = (t1 == p + 1);      // this chunk ends at the current position
  const int tg = last ? p : t1;         // rows t0..tg-1 come from the cache
  // (global and LDS reads stay in separate statements so that neither turns
  // into a generic-address load)
  for (int it = 0; it * RPL < tg - t0; it++) {
    const int t = t0 + it * RPL + lane / D4;
    float4 k4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < tg) k4 = reinterpret_cast<const float4 *>(K + (size_t)t * D)[lane % D4];
    float s = dot4(k4, q4, 0.f);
    s = seg_sum<D4>(s) * scale;
    if ((lane % D4) == 0 && t < tg) lds[S::L_SC + (t - t0)] = s;
  }
  if (last) {
    const float4 k4 = reinterpret_cast<const float4 *>(lds + S::L_KP)[lane % D4];
    float s = dot4(k4, q4, 0.f);
    s = seg_sum<D4>(s) * scale;
    if (lane == 0) lds[S::L_SC + (p - t0)] = s;
  }
  const float s = lane < n ? lds[S::L_SC + lane] : -INFINITY;
  const float m = wave_max(s);
  const float e = lane < n ? expf(s - m) : 0.f;
  const float lsum = wave_sum(e);
  lds[S::L_SC + lane] = e;
  // o[d] = sum_t e_t * v_t[d] in ascending t; lanes cover d (and, for D < 64,
  // alternate rows)
  constexpr int RG = 64 / D;
  const int d = lane % D, g = lane / D;
  float o = 0.f;
  for (int t = t0 + g; t < tg; t += RG) o = __builtin_fmaf(lds[S::L_SC + (t - t0)], V[(size_t)t * D + d], o);
  if (last && ((p - t0) % RG) == g) o = __builtin_fmaf(lds[S::L_SC + (p - t0)], lds[S::L_VP + d], o);
#pragma unroll
  for (int m2 = 32; m2 >= D; m2 >>= 1) o += __shfl_xor(o, m2, 64);
  if (lane < D) lds[S::L_SLOT + lane] = o;
  if (lane == 0) {
    lds[S::L_SLOT + D] = m;
    lds[S::L_SLOT + D + 1] = lsum;
  }
}

template <class S, int WD>
__device__ void compute_main(const DecodeArgs &a, float *lds, int lane) {
  constexpr int E = S::E, F = S::F, RAP = S::RAP;
  Chunk<WD> wq[Geo<S, 3 * RAP, E>::NPASS];
  Chunk<WD> wa[Geo<S, RAP, E>::NPASS];
  Chunk<WD> wf[Geo<S, 4 * RAP, E>::NPASS];
  Chunk<WD> wp[Geo<S, RAP, F>::NPASS];
  load_slice<S, 3 * RAP, E, WD>(wq, a.qkv, 0, lane);
  load_slice<S, RAP, E, WD>(wa, a.ap, 0, lane);
  load_slice<S, 4 * RAP, E, WD>(wf, a.fc, 0, lane);
  load_slice<S, RAP, F, WD>(wp, a.pr, 0, lane);
  // plain LDS accesses: the barrier's memory clobber orders them
  const int *flag = reinterpret_cast<const int *>(lds + S::L_FLAG);
  float *part = lds + S::L_PART;
  const float *xs = lds + S::L_XS;
  for (int step = 0; step < a.nsteps; step++) {
    for (int l = 0; l < a.L; l++) {
      const int ln = (l + 1 == a.L) ? 0 : l + 1;
      // A: QKV
      wg_barrier();
      if (flag[0]) return;
      slice_dot<S, 3 * RAP, E, WD>(wq, xs, part, lane);
      wg_barrier();
      load_slice<S, 3 * RAP, E, WD>(wq, a.qkv, ln, lane);
      // B: attention runs on the control wave alone
      // C: attention projection
      wg_barrier();
      if (flag[0]) return;
      slice_dot<S, RAP, E, WD>(wa, xs, part, lane);
      wg_barrier();
      load_slice<S, RAP, E, WD>(wa, a.ap, ln, lane);
      // D: fc
      wg_barrier();
      if (flag[0]) return;
      slice_dot<S, 4 * RAP, E, WD>(wf, xs, part, lane);
      wg_barrier();
      load_slice<S, 4 * RAP, E, WD>(wf, a.fc, ln, lane);
      // E: MLP projection
      wg_barrier();
      if (flag[0]) return;
      slice_dot<S, RAP, F, WD>(wp, xs, part, lane);
      wg_barrier();
      load_slice<S, RAP, F, WD>(wp, a.pr, ln, lane);
    }
    // H: output head over this workgroup's vocabulary rows
    wg_barrier();
    if (flag[0]) return;
    {
      using Gm = RowGeo<S, E>;
      constexpr int KC = Gm::KC;
      const int hr0 = (int)(((long long)blockIdx.x * a.V) / S::G);
      const int hr1 = (int)(((long long)(blockIdx.x + 1) * a.V) / S::G);
      const int nr = hr1 - hr0;
      const MatW hm{a.head, nullptr};
      constexpr int HWD = (WD == WD_F16) ? WD_F16 : WD_F32;
      if constexpr (Gm::ROWWIDE) {
        constexpr int PPR = Gm::PPR;
        constexpr int NB = 8;
        const int wave = lane >> 6;
        float4 xv[PPR];
#pragma unroll
        for (int j = 0; j < PPR; j++) xv[j] = reinterpret_cast<const float4 *>(xs)[j * S::NL + lane];
        for (int r0 = 0; r0 < nr; r0 += NB) {
          Chunk<HWD> hc[NB][PPR];
#pragma unroll
          for (int b = 0; b < NB; b++) {
            const int r = min(r0 + b, nr - 1);
#pragma unroll
            for (int j = 0; j < PPR; j++)
              hc[b][j] = ld_chunk<HWD>(hm, 0, (size_t)(hr0 + r) * KC + j * S::NL + lane);
          }
#pragma unroll
          for (int b = 0; b < NB; b++) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < PPR; j++) acc = dot4(deq<HWD>(hc[b][j]), xv[j], acc);
            acc = wave_sum(acc);
            if ((lane & 63) == 0 && r0 + b < nr) part[wave * PSTRIDE + r0 + b] = acc;
          }
        }
      } else {
        constexpr int RPP = Gm::RPP;
        const int kc = lane % KC;
        const float4 x = reinterpret_cast<const float4 *>(xs)[kc];
        for (int r0 = 0; r0 < nr; r0 += RPP) {
          const int r = r0 + lane / KC;
          const int rr = min(r, nr - 1);
          const Chunk<HWD> hc = ld_chunk<HWD>(hm, 0, (size_t)(hr0 + rr) * KC + kc);
          float acc = dot4(deq<HWD>(hc), x, 0.f);
          acc = seg_sum<KC>(acc);
          if (kc == 0 && r < nr) part[r] = acc;
        }
      }
    }
    wg_barrier();
  }
}

// ---- control wave ----------------------------------------------------------
template <class S, int WD>
__device__ void control_main(const DecodeArgs &a, float *lds, int lane) {
  constexpr int E = S::E, F = S::F, D = S::D, H = S::H, RAP = S::RAP, G = S::G;
  constexpr int PE = E / 64, PF = F / 64;
  const int w = blockIdx.x;
  int *flag = reinterpret_cast<int *>(lds + S::L_FLAG);
  float *xs = lds + S::L_XS;
  const float *part = lds + S::L_PART;
  float res = 0.f;   // residual stream value of row w*RAP + lane (lanes < RAP)
  int tok = 0;
  Waiter wt{&a, 0, 0};
  auto abort_all = [&]() {
    if (lane == 0) flag[0] = 1;
    wg_barrier();
  };
  for (int step = 0; step < a.nsteps; step++) {
    const int p = a.pos0 + step;
    // token of this step: fed, or the argmax of the previous step
    if (step < a.n_feed) {
      tok = a.feed[step];
    }
    if (step > 0) {
      const uint32_t ep = epoch_of<S>(a, step - 1, 5 * a.L);
      wt.t0 = wall_clock64();
      wt.phase = 5 * a.L;
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      while (true) {
        bool ok = true;
        float v = -INFINITY;
        uint32_t idx = 0xffffffffu;
        for (int g0 = lane; g0 < G; g0 += 64) {
          const uint64_t xv = tld(a.amax_t + g0), xi = tld(a.amax_t + G + g0);
          ok &= ((uint32_t)(xv >> 32) == ep) && ((uint32_t)(xi >> 32) == ep);
          const float cv = __uint_as_float((uint32_t)xv);
          const uint32_t ci = (uint32_t)xi;
          if (cv > v || (cv == v && ci < idx)) { v = cv; idx = ci; }
        }
        if (__all(ok)) { bv = v; bi = idx; break; }
        if (wt.expired()) { abort_all(); return; }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const uint32_t oi = (uint32_t)__shfl_xor((int)bi, m, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (w == 0 && lane == 0 && step - 1 >= a.out_from) a.out_ids[step - 1 - a.out_from] = (int)bi;
      // (an all-NaN head cannot name a row; keep the index in range)
      if (step >= a.n_feed) tok = bi < (uint32_t)a.V ? (int)bi : 0;
    }
    for (int l = 0; l < a.L; l++) {
      const uint32_t epA = epoch_of<S>(a, step, 5 * l + 0), epB = epA + 1, epC = epA + 2,
                     epD = epA + 3, epE = epA + 4;
      // ---------------- A: LayerNorm 1 + QKV
      {
        float x[PE], g[PE], b[PE];
#pragma unroll
        for (int j = 0; j < PE; j++) {
          g[j] = a.ln1w[l * E + lane + 64 * j];
          b[j] = a.ln1b[l * E + lane + 64 * j];
        }
        if (l == 0) {
#pragma unroll
          for (int j = 0; j < PE; j++)
            x[j] = a.wte[(size_t)tok * E + lane + 64 * j] + a.wpe[(size_t)p * E + lane + 64 * j];
          if (lane < RAP) {
            const int o = w * RAP + lane;
            res = a.wte[(size_t)tok * E + o] + a.wpe[(size_t)p * E + o];
          }
        } else {
          wt.t0 = wall_clock64();
          wt.phase = 5 * (l - 1) + 4;
          if (!poll_vec<PE>(a.xb_t + (size_t)(l - 1) * E, epA - 1, x, lane, wt)) { abort_all(); return; }
        }
        layernorm_to_lds<E>(x, g, b, a.eps, xs, lane);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        wg_barrier();
        constexpr int R = 3 * RAP;
        if (lane < R) {
          const int o = w * R + lane;
          const float y = row_total<S, E>(part, lane) + a.bqkv[l * 3 * E + o];
          tst(a.qkv_t + (size_t)l * 3 * E + o, y, epA);
        }
      }
      // ---------------- B: attention chunk
      {
        int nch, ch;
        att_chunks<S>(p, nch, ch);
        const int item = w;
        const bool has = item < H * nch;
        int h = 0, c = 0, t0 = 0, t1 = 0;
        if (has) {
          h = item / nch;
          c = item % nch;
          t0 = c * ch;
          t1 = min(t0 + ch, p + 1);
          const bool last = (t1 == p + 1);
          wt.t0 = wall_clock64();
          wt.phase = 5 * l + 0;
          const uint64_t *qk = a.qkv_t + (size_t)l * 3 * E + h * D + (lane % D);
          while (true) {
            const uint64_t xq = tld(qk);
            uint64_t xk = ((uint64_t)epA << 32), xv = ((uint64_t)epA << 32);
            if (last) {
              xk = tld(qk + E);
              xv = tld(qk + 2 * E);
            }
            const bool ok = ((uint32_t)(xq >> 32) == epA) && ((uint32_t)(xk >> 32) == epA) &&
                            ((uint32_t)(xv >> 32) == epA);
            if (__all(ok)) {
              if (lane < D) {
                lds[S::L_Q + lane] = __uint_as_float((uint32_t)xq);
                lds[S::L_KP + lane] = __uint_as_float((uint32_t)xk);
                lds[S::L_VP + lane] = __uint_as_float((uint32_t)xv);
                if (last) {
                  const size_t row = ((size_t)(l * H + h) * a.P + p) * D + lane;
                  st_agent(a.kc + row, __uint_as_float((uint32_t)xk));
                  st_agent(a.vc + row, __uint_as_float((uint32_t)xv));
                }
              }
              break;
            }
            if (wt.expired()) { abort_all(); return; }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        if (has) {
          attention_chunk<S>(a, lds, l, h, p, t0, t1, lane);
          // cache row stores complete before the chunk result is published
          __builtin_amdgcn_s_waitcnt(0);
          uint64_t *dst = a.att_t + ((size_t)(l * H + h) * S::MAXCH + c) * (D + 2);
          if (lane < D) tst(dst + lane, lds[S::L_SLOT + lane], epB);
          if (lane == 0) {
            tst(dst + D, lds[S::L_SLOT + D], epB);
            tst(dst + D + 1, lds[S::L_SLOT + D + 1], epB);
          }
        }
      }
      // ---------------- C: merge chunks, attention projection + residual
      {
        int nch, ch;
        att_chunks<S>(p, nch, ch);
        wt.t0 = wall_clock64();
        wt.phase = 5 * l + 1;
        const int d = lane % D;
        for (int h = 0; h < H; h++) {
          const uint64_t *src = a.att_t + ((size_t)(l * H + h) * S::MAXCH) * (D + 2);
          while (true) {
            bool ok = true;
            float mc[S::MAXCH], lc[S::MAXCH], oc[S::MAXCH];
#pragma unroll
            for (int c = 0; c < S::MAXCH; c++) {
              if (c < nch) {
                const uint64_t *s = src + (size_t)c * (D + 2);
                const uint64_t xo = tld(s + d), xm = tld(s + D), xl = tld(s + D + 1);
                ok &= ((uint32_t)(xo >> 32) == epB) && ((uint32_t)(xm >> 32) == epB) &&
                      ((uint32_t)(xl >> 32) == epB);
                oc[c] = __uint_as_float((uint32_t)xo);
                mc[c] = __uint_as_float((uint32_t)xm);
                lc[c] = __uint_as_float((uint32_t)xl);
              }
            }
            if (__all(ok)) {
              float M = mc[0];
#pragma unroll
              for (int c = 1; c < S::MAXCH; c++)
                if (c < nch) M = fmaxf(M, mc[c]);
              float Ls = 0.f, O = 0.f;
#pragma unroll
              for (int c = 0; c < S::MAXCH; c++) {
                if (c < nch) {
                  const float f = expf(mc[c] - M);
                  Ls = __builtin_fmaf(lc[c], f, Ls);
                  O = __builtin_fmaf(oc[c], f, O);
                }
              }
              if (lane < D) xs[h * D + d] = O / Ls;
              break;
            }
            if (wt.expired()) { abort_all(); return; }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        wg_barrier();
        if (lane < RAP) {
          const int o = w * RAP + lane;
          const float mix = row_total<S, E>(part, lane) + a.bap[l * E + o];
          res = res + mix;
          tst(a.xa_t + (size_t)l * E + o, res, epC);
        }
      }
      // ---------------- D: LayerNorm 2 + fc + gelu_new
      {
        float x[PE], g[PE], b[PE];
#pragma unroll
        for (int j = 0; j < PE; j++) {
          g[j] = a.ln2w[l * E + lane + 64 * j];
          b[j] = a.ln2b[l * E + lane + 64 * j];
        }
        wt.t0 = wall_clock64();
        wt.phase = 5 * l + 2;
        if (!poll_vec<PE>(a.xa_t + (size_t)l * E, epC, x, lane, wt)) { abort_all(); return; }
        layernorm_to_lds<E>(x, g, b, a.eps, xs, lane);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        wg_barrier();
        constexpr int R = 4 * RAP;
        if (lane < R) {
          const int o = w * R + lane;
          const float f = row_total<S, E>(part, lane) + a.bfc[l * F + o];
          tst(a.act_t + (size_t)l * F + o, gelu_new(f), epD);
        }
      }
      // ---------------- E: MLP projection + residual
      {
        float x[PF];
        wt.t0 = wall_clock64();
        wt.phase = 5 * l + 3;
        if (!poll_vec<PF>(a.act_t + (size_t)l * F, epD, x, lane, wt)) { abort_all(); return; }
#pragma unroll
        for (int j = 0; j < PF; j++) xs[lane + 64 * j] = x[j];
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        wg_barrier();
        if (lane < RAP) {
          const int o = w * RAP + lane;
          const float mix = row_total<S, F>(part, lane) + a.bpr[l * E + o];
          res = res + mix;
          tst(a.xb_t + (size_t)l * E + o, res, epE);
        }
      }
    }
    // ---------------- H: final LayerNorm + head + local argmax
    {
      const uint32_t epH = epoch_of<S>(a, step, 5 * a.L);
      float x[PE], g[PE], b[PE];
#pragma unroll
      for (int j = 0; j < PE; j++) {
        g[j] = a.lnfw[lane + 64 * j];
        b[j] = a.lnfb[lane + 64 * j];
      }
      wt.t0 = wall_clock64();
      wt.phase = 5 * a.L - 1;
      if (!poll_vec<PE>(a.xb_t + (size_t)(a.L - 1) * E, epH - 1, x, lane, wt)) { abort_all(); return; }
      layernorm_to_lds<E>(x, g, b, a.eps, xs, lane);
      if (lane == 0) flag[0] = 0;
      wg_barrier();
      wg_barrier();
      const int hr0 = (int)(((long long)w * a.V) / G);
      const int hr1 = (int)(((long long)(w + 1) * a.V) / G);
      const int nr = hr1 - hr0;
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      for (int r = lane; r < nr; r += 64) {
        const float v = row_total<S, E>(part, r);
        a.logits[hr0 + r] = v;
        if (v > bv || (v == bv && (uint32_t)(hr0 + r) < bi)) { bv = v; bi = (uint32_t)(hr0 + r); }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const uint32_t oi = (uint32_t)__shfl_xor((int)bi, m, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) {
        tst(a.amax_t + w, bv, epH);
        tst_u(a.amax_t + G + w, bi, epH);
      }
    }
  }
  // the last step's greedy id
  if (w == 0) {
    const uint32_t ep = epoch_of<S>(a, a.nsteps - 1, 5 * a.L);
    wt.t0 = wall_clock64();
    wt.phase = 5 * a.L;
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    while (true) {
      bool ok = true;
      float v = -INFINITY;
      uint32_t idx = 0xffffffffu;
      for (int g0 = lane; g0 < G; g0 += 64) {
        const uint64_t xv = tld(a.amax_t + g0), xi = tld(a.amax_t + G + g0);
        ok &= ((uint32_t)(xv >> 32) == ep) && ((uint32_t)(xi >> 32) == ep);
        const float cv = __uint_as_float((uint32_t)xv);
        const uint32_t ci = (uint32_t)xi;
        if (cv > v || (cv == v && ci < idx)) { v = cv; idx = ci; }
      }
      if (__all(ok)) { bv = v; bi = idx; break; }
      if (wt.expired()) return;
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const uint32_t oi = (uint32_t)__shfl_xor((int)bi, m, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0 && a.nsteps - 1 >= a.out_from) a.out_ids[a.nsteps - 1 - a.out_from] = (int)bi;
  }
}

template <class S, int WD>
__global__ void __launch_bounds__(S::NT, 1) decode_kernel(DecodeArgs a) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  if (tid >= S::NL) control_main<S, WD>(a, lds, tid - S::NL);
  else compute_main<S, WD>(a, lds, tid);
}

template <class S>
constexpr size_t lds_bytes() {
  // the layout needs S::L_TOTAL floats; ask for more than half of the CU's
  // 160 KB so that exactly one workgroup lands on each CU
  return 96 * 1024;
}

template <class S>
const void *kernel_for(int wd) {
  switch (wd) {
  case WD_F32: return reinterpret_cast<const void *>(&decode_kernel<S, WD_F32>);
  case WD_F16: return reinterpret_cast<const void *>(&decode_kernel<S, WD_F16>);
  case WD_Q4: return reinterpret_cast<const void *>(&decode_kernel<S, WD_Q4>);
  }
  return nullptr;
}

template <class S>
hipError_t launch_t(int wd, const DecodeArgs &a, hipStream_t s) {
  static_assert(S::L_TOTAL * sizeof(float) <= 96 * 1024, "LDS layout too large");
  const void *k = kernel_for<S>(wd);
  if (!k) return hipErrorInvalidValue;
  DecodeArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchCooperativeKernel(k, dim3(S::G), dim3(S::NT), args, lds_bytes<S>(), s);
}

template <class S>
hipError_t occupancy_t(int wd, int *blocks) {
  const void *k = kernel_for<S>(wd);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes<S>());
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, S::NT, lds_bytes<S>());
}

template <class S>
void info_t(ShapeInfo *o) {
  o->E = S::E;
  o->D = S::D;
  o->G = S::G;
  o->threads = S::NT;
  o->lds_bytes = lds_bytes<S>();
  o->maxch = S::MAXCH;
}

}  // namespace

bool shape_info(int E, int D, ShapeInfo *out) {
  if (E == ShapeS::E && D == ShapeS::D) { info_t<ShapeS>(out); return true; }
  if (E == ShapeT::E && D == ShapeT::D) { info_t<ShapeT>(out); return true; }
  return false;
}

hipError_t launch_decode(int E, int D, int wd, const DecodeArgs &a, hipStream_t s) {
  if (E == ShapeS::E && D == ShapeS::D) return launch_t<ShapeS>(wd, a, s);
  if (E == ShapeT::E && D == ShapeT::D) return launch_t<ShapeT>(wd, a, s);
  return hipErrorInvalidValue;
}

hipError_t decode_occupancy(int E, int D, int wd, int *blocks) {
  if (E == ShapeS::E && D == ShapeS::D) return occupancy_t<ShapeS>(wd, blocks);
  if (E == ShapeT::E && D == ShapeT::D) return occupancy_t<ShapeT>(wd, blocks);
  return hipErrorInvalidValue;
}

}  // namespace gpt2dec

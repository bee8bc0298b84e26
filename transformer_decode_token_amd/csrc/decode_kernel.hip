// decode_kernel.hip -- the persistent batch-1 GPT-2 decode kernel for gfx950.
//
// One cooperative launch runs `nsteps` whole forward passes (one token each).
// The per-token work follows the node order of the gpt2-125m "model.fir" file:
// embedding add, then per layer
//   A: LayerNorm 1 + QKV linear + bias
//   B: attn_decode: this position's K/V are appended, causal softmax over
//      positions 0..position, weighted sum of values (split in position chunks
//      of at most 64; the first chunk of a head merges the others)
//   C: attention linear + bias + residual
//   D: LayerNorm 2 + fc linear + bias + gelu_new
//   E: projection linear + bias + residual
// and finally H: final LayerNorm + tied output head + argmax.
//
// Work split.  Every workgroup owns RAP consecutive output rows of each
// E-output matrix (3*RAP of QKV, 4*RAP of fc), so the 256 workgroups of the
// 124M shape each stream an equal 1/256 of every matrix, and a contiguous
// 1/256 of the head.  Inside a workgroup each output row is owned by a segment
// of LPR lanes (16 or 64), so a row's dot product ends in one short DPP
// reduction and all rows reduce at once.  A workgroup is one control wave plus
// NCW compute waves:
//   * compute waves stream the workgroup's weight slices through two register
//     buffers, requesting each slice one phase before it is used;
//   * the control wave waits for the inputs of each phase, normalises them
//     into LDS, runs the attention chunk, and publishes the phase's outputs.
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

#ifndef G2_HEAD_NT
#define G2_HEAD_NT 0
#endif
constexpr bool HEAD_NT = G2_HEAD_NT != 0;  // head rows: temporal loads (may stay in the memory-side cache)
constexpr int CHMIN = 64;      // positions per attention chunk before a head is split
constexpr int PSTRIDE = 256;   // LDS room for row results (>= rows per workgroup)

template <int E_, int D_, int NCW_, int RAP_, int MAXCH_, int LPRH_>
struct Shape {
  static constexpr int E = E_, D = D_, H = E_ / D_, F = 4 * E_;
  static constexpr int NCW = NCW_;        // compute waves
  static constexpr int NL = 64 * NCW_;    // compute lanes
  static constexpr int NT = NL + 64;      // threads: compute waves + control wave
  static constexpr int RAP = RAP_;        // rows of an E-output matrix per workgroup
  static constexpr int G = E_ / RAP_;     // workgroups
  static constexpr int MAXCH = MAXCH_;    // attention chunks per head at most
  static constexpr int LPRH = LPRH_;      // lanes per head row
  static_assert(E_ % D_ == 0 && E_ % 64 == 0 && D_ <= 64 && 64 % (D_ / 4) == 0, "shape");
  static_assert(H * MAXCH <= G, "one attention chunk per workgroup at most");
  // LDS layout (floats)
  static constexpr int L_XS = 0;                         // [F] phase input vector
  static constexpr int L_PART = L_XS + F;                // [PSTRIDE] row results
  static constexpr int L_Q = L_PART + PSTRIDE;           // [D] query of the attention item
  static constexpr int L_KP = L_Q + D;                   // [D] key of this position
  static constexpr int L_VP = L_KP + D;                  // [D] value of this position
  static constexpr int L_SC = L_VP + D;                  // [64] chunk scores / weights
  static constexpr int L_FLAG = L_SC + 64;               // [4] control flags
  static constexpr int L_TOTAL = L_FLAG + 4;
};

// 124M shape: 256 workgroups x (3 compute + 1 control) waves.
using ShapeS = Shape<768, 64, 3, 3, 16, 16>;
// tiny shape: 32 workgroups x (2 compute + 1 control) waves.
using ShapeT = Shape<128, 32, 2, 4, 8, 8>;

constexpr int lpr_for(int R, int KC, int NL) {
  int l = 64;
  while (l > 1 && (R * l > NL || KC % l != 0)) l >>= 1;
  return l;
}

// Geometry of one workgroup slice: R rows of length K in 4-element chunks.
// Lane l < R*LPR owns row l/LPR and the chunks (l%LPR) + LPR*i, i < NPASS.
template <class S, int R, int K>
struct Geo {
  static constexpr int KC = K / 4;
  static constexpr int LPR = lpr_for(R, KC, S::NL);
  static constexpr int NPASS = KC / LPR;
  static constexpr int ACTIVE = R * LPR;
  static_assert(ACTIVE <= S::NL && KC % LPR == 0 && LPR >= 4, "row geometry");
};

// ---- weight chunks: 4 consecutive inputs of one output row ----------------
template <int WD> struct Chunk;
template <> struct Chunk<WD_F32> { float4 v; };
template <> struct Chunk<WD_F16> { uint2 v; };
template <> struct Chunk<WD_Q4> { uint32_t q; float2 sz; };

// gc: chunk index inside the layer's [N][K] matrix (= row*K/4 + k/4);
// lofs: element offset of the layer (= layer*N*K).
// Weights are read once per token: non-temporal loads keep them from
// displacing the small, reused data (LayerNorm parameters, biases,
// activations) in the caches.
typedef float g2_v4f __attribute__((ext_vector_type(4)));
typedef float g2_v2f __attribute__((ext_vector_type(2)));
typedef unsigned int g2_v2u __attribute__((ext_vector_type(2)));

template <int WD, bool NT = true>
__device__ __forceinline__ Chunk<WD> ld_chunk(const MatW &m, size_t lofs, size_t gc) {
  Chunk<WD> c;
  if constexpr (WD == WD_F32) {
    if constexpr (NT) {
      const g2_v4f v = __builtin_nontemporal_load(reinterpret_cast<const g2_v4f *>(m.w) + lofs / 4 + gc);
      c.v = make_float4(v.x, v.y, v.z, v.w);
    } else {
      c.v = reinterpret_cast<const float4 *>(m.w)[lofs / 4 + gc];
    }
  } else if constexpr (WD == WD_F16) {
    if constexpr (NT) {
      const g2_v2u v = __builtin_nontemporal_load(reinterpret_cast<const g2_v2u *>(m.w) + lofs / 4 + gc);
      c.v = make_uint2(v.x, v.y);
    } else {
      c.v = reinterpret_cast<const uint2 *>(m.w)[lofs / 4 + gc];
    }
  } else {
    c.q = __builtin_nontemporal_load(reinterpret_cast<const unsigned short *>(m.w) + lofs / 4 + gc);
    const g2_v2f z = __builtin_nontemporal_load(reinterpret_cast<const g2_v2f *>(m.sz) + lofs / 32 + gc / 8);
    c.sz = make_float2(z.x, z.y);
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

// ---- DPP reductions ----------------------------------------------------------
// Inclusive scans with row_shr 1,2,4,8 (within 16-lane rows), then
// row_bcast:15 / row_bcast:31 across rows: the total of each W-lane segment
// ends in the segment's last lane.  Lanes whose DPP source is out of range,
// or whose row is masked off, take the identity.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or(float v, float ident) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(v), CTRL, ROWMASK,
                                                    0xF, false));
}
template <int W>
__device__ __forceinline__ float seg_sum_last(float v) {
  static_assert(W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "segment");
  v += dpp_or<0x111, 0xF>(v, 0.f);
  v += dpp_or<0x112, 0xF>(v, 0.f);
  if constexpr (W >= 8) v += dpp_or<0x114, 0xF>(v, 0.f);
  if constexpr (W >= 16) v += dpp_or<0x118, 0xF>(v, 0.f);
  if constexpr (W >= 32) v += dpp_or<0x142, 0xA>(v, 0.f);
  if constexpr (W >= 64) v += dpp_or<0x143, 0xC>(v, 0.f);
  return v;
}
// Whole-wave sum / max, the same bits in every lane.
__device__ __forceinline__ float wave_sum_all(float v) {
  const float t = seg_sum_last<64>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 63));
}
__device__ __forceinline__ float wave_max_all(float v) {
  const float ninf = -INFINITY;
  v = fmaxf(v, dpp_or<0x111, 0xF>(v, ninf));
  v = fmaxf(v, dpp_or<0x112, 0xF>(v, ninf));
  v = fmaxf(v, dpp_or<0x114, 0xF>(v, ninf));
  v = fmaxf(v, dpp_or<0x118, 0xF>(v, ninf));
  v = fmaxf(v, dpp_or<0x142, 0xA>(v, ninf));
  v = fmaxf(v, dpp_or<0x143, 0xC>(v, ninf));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ uint32_t wave_min_u32_all(uint32_t v) {
  auto step = [](uint32_t x, uint32_t y) { return x < y ? x : y; };
#define G2_MIN_STEP(CTRL, ROWMASK) \
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffffu, (int)v, CTRL, ROWMASK, 0xF, false))
  G2_MIN_STEP(0x111, 0xF);
  G2_MIN_STEP(0x112, 0xF);
  G2_MIN_STEP(0x114, 0xF);
  G2_MIN_STEP(0x118, 0xF);
  G2_MIN_STEP(0x142, 0xA);
  G2_MIN_STEP(0x143, 0xC);
#undef G2_MIN_STEP
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Greedy pick over the wave: the largest value, and the lowest index among
// the lanes that hold it (each lane passes its own best value and index).
__device__ __forceinline__ uint32_t wave_argmax(float v, uint32_t idx, float *best = nullptr) {
  const float m = wave_max_all(v);
  if (best) *best = m;
  return wave_min_u32_all(v == m ? idx : 0xffffffffu);
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
__device__ __forceinline__ bool tag_is(uint64_t x, uint32_t ep) { return (uint32_t)(x >> 32) == ep; }
// Every published vector exists in NCOPY copies, one per XCD (workgroup w is
// taken to run on XCD w % 8): a producer writes all copies, a consumer polls
// the copy of its own XCD, which spreads the polling over 8x the lines.
constexpr int NCOPY = 8;
__device__ __forceinline__ int my_copy() { return (int)(blockIdx.x % NCOPY); }
__device__ __forceinline__ void tst_all(uint64_t *base, size_t stride, size_t idx, float v, uint32_t ep) {
#pragma unroll
  for (int c = 0; c < NCOPY; c++) tst(base + c * stride + idx, v, ep);
}
__device__ __forceinline__ float payload(uint64_t x) { return __uint_as_float((uint32_t)x); }

// Bounded waiting: a wait that outlives the time limit, or sees another
// workgroup's abort, sets the error word and makes the caller stop.
struct Waiter {
  const DecodeArgs *a;
  long long t0;
  int phase;
  __device__ void start(int ph) {
    t0 = (long long)wall_clock64();
    phase = ph;
  }
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
      v[j] = payload(x);
      ok &= tag_is(x, ep);
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
  const float mean = wave_sum_all(s) * (1.0f / (float)E);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const float d = x[j] - mean;
    q = __builtin_fmaf(d, d, q);
  }
  const float var = wave_sum_all(q) * (1.0f / (float)E);
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

// Optional timeline of one workgroup's control wave (lane 0): inputs ready, first and
// second workgroup barrier passed, outputs published.
__device__ __forceinline__ void stamp(const DecodeArgs &a, int step, int ph, int which, int G) {
  if (a.trace && step < a.trace_steps)
    a.trace[(((size_t)step * (5 * a.L + 1) + ph) * G + blockIdx.x) * 4 + which] = (long long)wall_clock64();
}

__device__ __forceinline__ uint32_t epoch_of(const DecodeArgs &a, int step, int ph) {
  return a.epoch0 + (uint32_t)step * (uint32_t)(5 * a.L + 1) + (uint32_t)ph + 1u;
}

// ---- compute waves ---------------------------------------------------------
template <class S, int R, int K, int WD, int NB>
__device__ __forceinline__ void load_slice(Chunk<WD> (&w)[NB], const MatW &m, int layer, int lane) {
  using Gm = Geo<S, R, K>;
  static_assert(Gm::NPASS <= NB, "register buffer too small");
  // Lanes past the slice re-read the last row (same addresses as its own
  // lanes in the same wave; their results are discarded).  Keeping every load
  // unconditional lets the compiler count outstanding loads exactly.
  const int r = min(lane / Gm::LPR, R - 1);
  const size_t lofs = (size_t)layer * (size_t)(R * S::G) * K;
  const size_t c0 = ((size_t)blockIdx.x * R + r) * Gm::KC + (lane % Gm::LPR);
#pragma unroll
  for (int i = 0; i < Gm::NPASS; i++) w[i] = ld_chunk<WD>(m, lofs, c0 + (size_t)i * Gm::LPR);
}

// Row results of the slice into part[0..R).
template <class S, int R, int K, int WD, int NB>
__device__ __forceinline__ void slice_dot(const Chunk<WD> (&w)[NB], const float *xs, float *part, int lane) {
  using Gm = Geo<S, R, K>;
  static_assert(Gm::NPASS <= NB, "register buffer too small");
  const int q = lane % Gm::LPR;
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < Gm::NPASS; i++)
    a = dot4(deq<WD>(w[i]), reinterpret_cast<const float4 *>(xs)[i * Gm::LPR + q], a);
  a = seg_sum_last<Gm::LPR>(a);
  if (lane < Gm::ACTIVE && q == Gm::LPR - 1) part[lane / Gm::LPR] = a;
}

// Compute waves.  Two register buffers alternate: when a phase's inputs are
// ready, the slice of the next phase is requested into the other buffer and
// the current slice (requested one phase earlier) is consumed, so every slice
// streams in while the previous phase computes, publishes and waits.
template <class S, int WD>
__device__ void compute_main(const DecodeArgs &a, float *lds, int lane) {
  constexpr int E = S::E, F = S::F, RAP = S::RAP;
  constexpr int NB = Geo<S, 3 * RAP, E>::NPASS > Geo<S, RAP, F>::NPASS ? Geo<S, 3 * RAP, E>::NPASS
                                                                      : Geo<S, RAP, F>::NPASS;
  static_assert(Geo<S, 4 * RAP, E>::NPASS <= NB && Geo<S, RAP, E>::NPASS <= NB, "buffer size");
  const int *flag = reinterpret_cast<const int *>(lds + S::L_FLAG);
  float *part = lds + S::L_PART;
  const float *xs = lds + S::L_XS;
  Chunk<WD> b0[NB], b1[NB];
  load_slice<S, 3 * RAP, E, WD>(b0, a.qkv, 0, lane);
  for (int step = 0; step < a.nsteps; step++) {
    for (int l = 0; l < a.L; l++) {
      // A: QKV (b0); request the attention projection into b1
      wg_barrier();
      if (flag[0]) return;
      load_slice<S, RAP, E, WD>(b1, a.ap, l, lane);
      slice_dot<S, 3 * RAP, E, WD>(b0, xs, part, lane);
      wg_barrier();
      // B: attention runs on the control wave alone
      // C: attention projection (b1); request fc into b0
      wg_barrier();
      if (flag[0]) return;
      load_slice<S, 4 * RAP, E, WD>(b0, a.fc, l, lane);
      slice_dot<S, RAP, E, WD>(b1, xs, part, lane);
      wg_barrier();
      // D: fc (b0); request the MLP projection into b1
      wg_barrier();
      if (flag[0]) return;
      load_slice<S, RAP, F, WD>(b1, a.pr, l, lane);
      slice_dot<S, 4 * RAP, E, WD>(b0, xs, part, lane);
      wg_barrier();
      // E: MLP projection (b1); request the next layer's QKV into b0
      wg_barrier();
      if (flag[0]) return;
      load_slice<S, 3 * RAP, E, WD>(b0, a.qkv, (l + 1 < a.L) ? l + 1 : 0, lane);
      slice_dot<S, RAP, F, WD>(b1, xs, part, lane);
      wg_barrier();
    }
    // H: output head over this workgroup's vocabulary rows, RB rows per batch,
    // two batches in flight
    wg_barrier();
    if (flag[0]) return;
    {
      constexpr int KC = E / 4, LPR = S::LPRH, NPH = KC / LPR, RB = S::NL / LPR;
      static_assert(KC % LPR == 0 && S::NL % LPR == 0, "head geometry");
      constexpr int HWD = (WD == WD_F16) ? WD_F16 : WD_F32;
      const MatW hm{a.head, nullptr};
      const int hr0 = (int)(((long long)blockIdx.x * a.V) / S::G);
      const int hr1 = (int)(((long long)(blockIdx.x + 1) * a.V) / S::G);
      const int nr = hr1 - hr0;
      const int q = lane % LPR, rl = lane / LPR;
      float4 xv[NPH];
#pragma unroll
      for (int i = 0; i < NPH; i++) xv[i] = reinterpret_cast<const float4 *>(xs)[i * LPR + q];
      Chunk<HWD> h0[NPH], h1[NPH];
      auto fetch = [&](Chunk<HWD>(&b)[NPH], int r0) {
        const int r = min(r0 + rl, nr - 1);
        const size_t c0 = (size_t)(hr0 + r) * KC + q;
#pragma unroll
        for (int i = 0; i < NPH; i++) b[i] = ld_chunk<HWD, HEAD_NT>(hm, 0, c0 + (size_t)i * LPR);
      };
      auto consume = [&](const Chunk<HWD>(&b)[NPH], int r0) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NPH; i++) acc = dot4(deq<HWD>(b[i]), xv[i], acc);
        acc = seg_sum_last<LPR>(acc);
        if (q == LPR - 1 && r0 + rl < nr) part[r0 + rl] = acc;
      };
      if (nr > 0) {
        fetch(h0, 0);
        for (int r0 = 0; r0 < nr; r0 += 2 * RB) {
          if (r0 + RB < nr) fetch(h1, r0 + RB);
          consume(h0, r0);
          if (r0 + 2 * RB < nr) fetch(h0, r0 + 2 * RB);
          if (r0 + RB < nr) consume(h1, r0 + RB);
        }
      }
    }
    wg_barrier();
  }
}

// ---- control wave ----------------------------------------------------------
template <class S>
__device__ __forceinline__ bool reduce_argmax(const DecodeArgs &a, uint32_t ep, int lane, Waiter &wt,
                                              uint32_t &out_idx) {
  constexpr int G = S::G;
  float bv = -INFINITY;
  uint32_t bi = 0xffffffffu;
  while (true) {
    bool ok = true;
    float v = -INFINITY;
    uint32_t idx = 0xffffffffu;
    for (int g0 = lane; g0 < G; g0 += 64) {
      const uint64_t *am = a.amax_t + (size_t)my_copy() * 2 * G;
      const uint64_t xv = tld(am + g0), xi = tld(am + G + g0);
      ok &= tag_is(xv, ep) && tag_is(xi, ep);
      const float cv = payload(xv);
      const uint32_t ci = (uint32_t)xi;
      if (cv > v || (cv == v && ci < idx)) { v = cv; idx = ci; }
    }
    if (__all(ok)) { bv = v; bi = idx; break; }
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  out_idx = wave_argmax(bv, bi);
  return true;
}

// One attention chunk of head h over positions t0..t1-1 on the control wave,
// following the attn_decode kernel: scores q.k * (1/sqrt(D)), subtract the
// maximum, exp; the chunk's (o = sum e_t v_t, m = max, l = sum e_t).  Row p
// (the current position) comes from LDS, the others from the cache.  Lane
// (g, d4) handles rows t0 + g + RPL*it and dimensions 4*d4..4*d4+3.
template <class S>
struct AttChunk {
  static constexpr int D = S::D, D4 = D / 4, RPL = 64 / D4, IT = 64 / RPL;
  float4 k[IT], v[IT];
  __device__ void fetch(const DecodeArgs &a, int l, int h, int t0, int tg, int lane) {
    const float *K = a.kc + ((size_t)(l * S::H + h) * a.P) * D;
    const float *V = a.vc + ((size_t)(l * S::H + h) * a.P) * D;
    const int g = lane / D4, d4 = lane % D4;
#pragma unroll
    for (int it = 0; it < IT; it++) {
      const int t = t0 + g + RPL * it;
      k[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      v[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < tg) {
        k[it] = reinterpret_cast<const float4 *>(K + (size_t)t * D)[d4];
        v[it] = reinterpret_cast<const float4 *>(V + (size_t)t * D)[d4];
      }
    }
  }
  // m, lsum in all lanes; o (dims 4*d4..4*d4+3) summed over all rows in lanes of group 0
  __device__ void run(float *lds, int p, int t0, int t1, int tg, int lane, float &m, float &lsum, float4 &o) {
    const int g = lane / D4, d4 = lane % D4;
    const float scale = 1.0f / sqrtf((float)D);
    const float4 q4 = reinterpret_cast<const float4 *>(lds + S::L_Q)[d4];
    const int n = t1 - t0;
#pragma unroll
    for (int it = 0; it < IT; it++) {
      const int t = t0 + g + RPL * it;
      const float s = seg_sum_last<D4>(dot4(k[it], q4, 0.f)) * scale;
      if (d4 == D4 - 1 && t < tg) lds[S::L_SC + (t - t0)] = s;
    }
    if (tg < t1) {  // this position
      const float4 kp = reinterpret_cast<const float4 *>(lds + S::L_KP)[d4];
      const float s = seg_sum_last<D4>(dot4(kp, q4, 0.f)) * scale;
      if (lane == D4 - 1) lds[S::L_SC + (p - t0)] = s;
    }
    const float s = lane < n ? lds[S::L_SC + lane] : -INFINITY;
    m = wave_max_all(s);
    const float e = lane < n ? expf(s - m) : 0.f;
    lsum = wave_sum_all(e);
    lds[S::L_SC + lane] = e;
    o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int it = 0; it < IT; it++) {
      const int t = t0 + g + RPL * it;
      if (t < tg) {
        const float wt = lds[S::L_SC + (t - t0)];
        o.x = __builtin_fmaf(wt, v[it].x, o.x);
        o.y = __builtin_fmaf(wt, v[it].y, o.y);
        o.z = __builtin_fmaf(wt, v[it].z, o.z);
        o.w = __builtin_fmaf(wt, v[it].w, o.w);
      }
    }
    if (tg < t1 && ((p - t0) % RPL) == g) {
      const float wt = lds[S::L_SC + (p - t0)];
      const float4 vp = reinterpret_cast<const float4 *>(lds + S::L_VP)[d4];
      o.x = __builtin_fmaf(wt, vp.x, o.x);
      o.y = __builtin_fmaf(wt, vp.y, o.y);
      o.z = __builtin_fmaf(wt, vp.z, o.z);
      o.w = __builtin_fmaf(wt, vp.w, o.w);
    }
    // sum the RPL row groups in group order through LDS (the phase-input
    // area is free while the attention chunk runs); lanes of group 0 end
    // with the chunk's o
    float4 *scr = reinterpret_cast<float4 *>(lds + S::L_XS);
    scr[lane] = o;
    if (g == 0) {
      float4 t = scr[d4];
#pragma unroll
      for (int gg = 1; gg < RPL; gg++) {
        const float4 u = scr[gg * D4 + d4];
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
      }
      o = t;
    }
  }
};

template <class S, int WD>
__device__ void control_main(const DecodeArgs &a, float *lds, int lane) {
  constexpr int E = S::E, F = S::F, D = S::D, H = S::H, RAP = S::RAP, G = S::G;
  constexpr int PE = E / 64, PF = F / 64, D4 = D / 4;
  const int w = blockIdx.x;
  int *flag = reinterpret_cast<int *>(lds + S::L_FLAG);
  float *xs = lds + S::L_XS;
  const float *part = lds + S::L_PART;
  float res = 0.f;  // residual stream value of row w*RAP + lane (lanes < RAP)
  int tok = 0;
  Waiter wt{&a, 0, 0};
  // Parameters of a phase are requested one or two phases ahead, before an
  // earlier wait, so their latency hides behind it:
  //   A(l): ln1, QKV bias   <- requested before D(l-1)'s wait (or H's)
  //   C(l): attn-proj bias  <- before A(l)'s wait
  //   D(l): ln2, fc bias    <- before A(l)'s wait
  //   E(l): MLP-proj bias   <- before C(l)'s wait
  //   H   : ln_f            <- before D(L-1)'s wait
  float g1[PE], b1[PE], g2[PE], b2[PE], gf[PE], bf[PE];
  float bq = 0.f, ba = 0.f, bfc = 0.f, bp = 0.f;
  auto fetch_ln = [&](float (&g)[PE], float (&b)[PE], const float *gs, const float *bs) {
#pragma unroll
    for (int j = 0; j < PE; j++) {
      g[j] = gs[lane + 64 * j];
      b[j] = bs[lane + 64 * j];
    }
  };
  auto fetch_a = [&](int l) {
    fetch_ln(g1, b1, a.ln1w + l * E, a.ln1b + l * E);
    bq = lane < 3 * RAP ? a.bqkv[l * 3 * E + w * 3 * RAP + lane] : 0.f;
  };
  fetch_a(0);
  auto abort_all = [&]() {
    if (lane == 0) flag[0] = 1;
    wg_barrier();
  };
  for (int step = 0; step < a.nsteps; step++) {
    const int p = a.pos0 + step;
    // token of this step: fed, or the argmax of the previous step
    if (step < a.n_feed) tok = a.feed[step];
    if (step > 0) {
      uint32_t bi = 0;
      wt.start(5 * a.L);
      if (!reduce_argmax<S>(a, epoch_of(a, step - 1, 5 * a.L), lane, wt, bi)) { abort_all(); return; }
      if (w == 0 && lane == 0 && step - 1 >= a.out_from) a.out_ids[step - 1 - a.out_from] = (int)bi;
      // (an all-NaN head cannot name a row; keep the index in range)
      if (step >= a.n_feed) tok = bi < (uint32_t)a.V ? (int)bi : 0;
    }
    int nch, ch;
    att_chunks<S>(p, nch, ch);
    const bool has_item = w < H * nch;
    const int ih = has_item ? w / nch : 0, ic = has_item ? w % nch : 0;
    const int it0 = ic * ch, it1 = min(it0 + ch, p + 1);
    const bool ilast = (it1 == p + 1);
    const int itg = ilast ? p : it1;  // cache rows it0..itg-1
    for (int l = 0; l < a.L; l++) {
      const uint32_t epA = epoch_of(a, step, 5 * l + 0), epB = epA + 1, epC = epA + 2, epD = epA + 3,
                     epE = epA + 4;
      // ---------------- A: LayerNorm 1 + QKV
      {
        constexpr int R = 3 * RAP;
        // requests for C and D
        ba = lane < RAP ? a.bap[l * E + w * RAP + lane] : 0.f;
        fetch_ln(g2, b2, a.ln2w + l * E, a.ln2b + l * E);
        bfc = lane < 4 * RAP ? a.bfc[l * F + w * 4 * RAP + lane] : 0.f;
        float x[PE];
        if (l == 0) {
#pragma unroll
          for (int j = 0; j < PE; j++)
            x[j] = a.wte[(size_t)tok * E + lane + 64 * j] + a.wpe[(size_t)p * E + lane + 64 * j];
          if (lane < RAP) {
            const int o = w * RAP + lane;
            res = a.wte[(size_t)tok * E + o] + a.wpe[(size_t)p * E + o];
          }
        } else {
          wt.start(5 * (l - 1) + 4);
          if (!poll_vec<PE>(a.xb_t + ((size_t)(l - 1) * NCOPY + my_copy()) * E, epA - 1, x, lane, wt)) {
            abort_all();
            return;
          }
        }
        layernorm_to_lds<E>(x, g1, b1, a.eps, xs, lane);
        if (lane == 0) stamp(a, step, 5 * l + 0, 0, G);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 0, 1, G);
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 0, 2, G);
        if (lane < R) tst_all(a.qkv_t + (size_t)l * NCOPY * 3 * E, 3 * E, w * R + lane, part[lane] + bq, epA);
        if (lane == 0) stamp(a, step, 5 * l + 0, 3, G);
      }
      // ---------------- B: attention chunk (control wave only)
      if (has_item) {
        AttChunk<S> at;
        at.fetch(a, l, ih, it0, itg, lane);  // cache rows: written at earlier steps
        wt.start(5 * l + 0);
        const uint64_t *qk = a.qkv_t + ((size_t)l * NCOPY + my_copy()) * 3 * E + ih * D + (lane % D);
        while (true) {
          const uint64_t xq = tld(qk);
          uint64_t xk = (uint64_t)epA << 32, xv = (uint64_t)epA << 32;
          if (ilast) {
            xk = tld(qk + E);
            xv = tld(qk + 2 * E);
          }
          if (__all(tag_is(xq, epA) && tag_is(xk, epA) && tag_is(xv, epA))) {
            if (lane < D) {
              lds[S::L_Q + lane] = payload(xq);
              lds[S::L_KP + lane] = payload(xk);
              lds[S::L_VP + lane] = payload(xv);
              if (ilast) {
                const size_t row = ((size_t)(l * H + ih) * a.P + p) * D + lane;
                st_agent(a.kc + row, payload(xk));
                st_agent(a.vc + row, payload(xv));
              }
            }
            break;
          }
          if (wt.expired()) { abort_all(); return; }
          __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) stamp(a, step, 5 * l + 1, 0, G);
        float m, lsum;
        float4 o;
        at.run(lds, p, it0, it1, itg, lane, m, lsum, o);
        // cache-row stores complete before anything of this step is published
        __builtin_amdgcn_s_waitcnt(0);
        const int g = lane / D4, d4 = lane % D4;
        if (nch == 1) {
          if (g == 0) {
            uint64_t *dst = a.attn_t + (size_t)l * NCOPY * E;
            const size_t ix = ih * D + 4 * d4;
            tst_all(dst, E, ix + 0, o.x / lsum, epB);
            tst_all(dst, E, ix + 1, o.y / lsum, epB);
            tst_all(dst, E, ix + 2, o.z / lsum, epB);
            tst_all(dst, E, ix + 3, o.w / lsum, epB);
          }
        } else if (ic > 0) {
          uint64_t *dst = a.att_t + ((size_t)(l * H + ih) * S::MAXCH + ic) * (D + 2);
          if (g == 0) {
            tst(dst + 4 * d4 + 0, o.x, epB);
            tst(dst + 4 * d4 + 1, o.y, epB);
            tst(dst + 4 * d4 + 2, o.z, epB);
            tst(dst + 4 * d4 + 3, o.w, epB);
          }
          if (lane == 0) {
            tst(dst + D, m, epB);
            tst(dst + D + 1, lsum, epB);
          }
        } else {
          // chunk 0 merges the head: max over chunks, then rescaled sums in chunk order
          const uint64_t *src = a.att_t + ((size_t)(l * H + ih) * S::MAXCH) * (D + 2);
          float mc[S::MAXCH], lc[S::MAXCH];
          float4 oc[S::MAXCH];
          wt.start(5 * l + 1);
          while (true) {
            bool ok = true;
#pragma unroll
            for (int c = 1; c < S::MAXCH; c++) {
              if (c < nch) {
                const uint64_t *s2 = src + (size_t)c * (D + 2);
                const uint64_t x0 = tld(s2 + 4 * d4 + 0), x1 = tld(s2 + 4 * d4 + 1), x2 = tld(s2 + 4 * d4 + 2),
                               x3 = tld(s2 + 4 * d4 + 3), xm = tld(s2 + D), xl = tld(s2 + D + 1);
                ok &= tag_is(x0, epB) && tag_is(x1, epB) && tag_is(x2, epB) && tag_is(x3, epB) &&
                      tag_is(xm, epB) && tag_is(xl, epB);
                oc[c] = make_float4(payload(x0), payload(x1), payload(x2), payload(x3));
                mc[c] = payload(xm);
                lc[c] = payload(xl);
              }
            }
            if (__all(ok)) break;
            if (wt.expired()) { abort_all(); return; }
            __builtin_amdgcn_s_sleep(1);
          }
          mc[0] = m;
          lc[0] = lsum;
          oc[0] = o;
          float M = mc[0];
#pragma unroll
          for (int c = 1; c < S::MAXCH; c++)
            if (c < nch) M = fmaxf(M, mc[c]);
          float Ls = 0.f;
          float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int c = 0; c < S::MAXCH; c++) {
            if (c < nch) {
              const float f = expf(mc[c] - M);
              Ls = __builtin_fmaf(lc[c], f, Ls);
              O.x = __builtin_fmaf(oc[c].x, f, O.x);
              O.y = __builtin_fmaf(oc[c].y, f, O.y);
              O.z = __builtin_fmaf(oc[c].z, f, O.z);
              O.w = __builtin_fmaf(oc[c].w, f, O.w);
            }
          }
          if (g == 0) {
            uint64_t *dst = a.attn_t + (size_t)l * NCOPY * E;
            const size_t ix = ih * D + 4 * d4;
            tst_all(dst, E, ix + 0, O.x / Ls, epB);
            tst_all(dst, E, ix + 1, O.y / Ls, epB);
            tst_all(dst, E, ix + 2, O.z / Ls, epB);
            tst_all(dst, E, ix + 3, O.w / Ls, epB);
          }
        }
        if (lane == 0) stamp(a, step, 5 * l + 1, 3, G);
      }
      // ---------------- C: attention projection + residual
      {
        bp = lane < RAP ? a.bpr[l * E + w * RAP + lane] : 0.f;  // request for E
        float x[PE];
        wt.start(5 * l + 1);
        if (!poll_vec<PE>(a.attn_t + ((size_t)l * NCOPY + my_copy()) * E, epB, x, lane, wt)) { abort_all(); return; }
#pragma unroll
        for (int j = 0; j < PE; j++) xs[lane + 64 * j] = x[j];
        if (lane == 0) stamp(a, step, 5 * l + 2, 0, G);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 2, 1, G);
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 2, 2, G);
        if (lane < RAP) {
          const int o = w * RAP + lane;
          const float mix = part[lane] + ba;
          res = res + mix;
          tst_all(a.xa_t + (size_t)l * NCOPY * E, E, o, res, epC);
        }
        if (lane == 0) stamp(a, step, 5 * l + 2, 3, G);
      }
      // ---------------- D: LayerNorm 2 + fc + gelu_new
      {
        constexpr int R = 4 * RAP;
        // requests for the next A (or for the head after the last layer)
        if (l + 1 < a.L) fetch_a(l + 1);
        else fetch_ln(gf, bf, a.lnfw, a.lnfb);
        float x[PE];
        wt.start(5 * l + 2);
        if (!poll_vec<PE>(a.xa_t + ((size_t)l * NCOPY + my_copy()) * E, epC, x, lane, wt)) { abort_all(); return; }
        layernorm_to_lds<E>(x, g2, b2, a.eps, xs, lane);
        if (lane == 0) stamp(a, step, 5 * l + 3, 0, G);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 3, 1, G);
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 3, 2, G);
        if (lane < R) tst_all(a.act_t + (size_t)l * NCOPY * F, F, w * R + lane, gelu_new(part[lane] + bfc), epD);
        if (lane == 0) stamp(a, step, 5 * l + 3, 3, G);
      }
      // ---------------- E: MLP projection + residual
      {
        float x[PF];
        wt.start(5 * l + 3);
        if (!poll_vec<PF>(a.act_t + ((size_t)l * NCOPY + my_copy()) * F, epD, x, lane, wt)) { abort_all(); return; }
#pragma unroll
        for (int j = 0; j < PF; j++) xs[lane + 64 * j] = x[j];
        if (lane == 0) stamp(a, step, 5 * l + 4, 0, G);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 4, 1, G);
        wg_barrier();
        if (lane == 0) stamp(a, step, 5 * l + 4, 2, G);
        if (lane < RAP) {
          const int o = w * RAP + lane;
          const float mix = part[lane] + bp;
          res = res + mix;
          tst_all(a.xb_t + (size_t)l * NCOPY * E, E, o, res, epE);
        }
        if (lane == 0) stamp(a, step, 5 * l + 4, 3, G);
      }
    }
    // ---------------- H: final LayerNorm + head + local argmax
    {
      const uint32_t epH = epoch_of(a, step, 5 * a.L);
      fetch_a(0);  // request for the next step's first layer
      float x[PE];
      wt.start(5 * a.L - 1);
      if (!poll_vec<PE>(a.xb_t + ((size_t)(a.L - 1) * NCOPY + my_copy()) * E, epH - 1, x, lane, wt)) {
        abort_all();
        return;
      }
      layernorm_to_lds<E>(x, gf, bf, a.eps, xs, lane);
      if (lane == 0) stamp(a, step, 5 * a.L, 0, G);
      if (lane == 0) flag[0] = 0;
      wg_barrier();
      if (lane == 0) stamp(a, step, 5 * a.L, 1, G);
      wg_barrier();
      if (lane == 0) stamp(a, step, 5 * a.L, 2, G);
      const int hr0 = (int)(((long long)w * a.V) / G);
      const int hr1 = (int)(((long long)(w + 1) * a.V) / G);
      const int nr = hr1 - hr0;
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      for (int r = lane; r < nr; r += 64) {
        const float v = part[r];
        a.logits[hr0 + r] = v;
        if (v > bv || (v == bv && (uint32_t)(hr0 + r) < bi)) { bv = v; bi = (uint32_t)(hr0 + r); }
      }
      bi = wave_argmax(bv, bi, &bv);
      if (lane == 0) {
        #pragma unroll
        for (int c = 0; c < NCOPY; c++) {
          tst(a.amax_t + (size_t)c * 2 * G + w, bv, epH);
          tst_u(a.amax_t + (size_t)c * 2 * G + G + w, bi, epH);
        }
      }
      if (lane == 0) stamp(a, step, 5 * a.L, 3, G);
    }
  }
  // the last step's greedy id
  if (w == 0) {
    uint32_t bi = 0;
    wt.start(5 * a.L);
    if (!reduce_argmax<S>(a, epoch_of(a, a.nsteps - 1, 5 * a.L), lane, wt, bi)) return;
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

// The layout needs S::L_TOTAL floats; ask for more than half of the CU's
// 160 KB so that exactly one workgroup lands on each CU.
constexpr size_t kLdsBytes = 96 * 1024;

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
  static_assert(S::L_TOTAL * sizeof(float) <= kLdsBytes, "LDS layout too large");
  const void *k = kernel_for<S>(wd);
  if (!k) return hipErrorInvalidValue;
  DecodeArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchCooperativeKernel(k, dim3(S::G), dim3(S::NT), args, kLdsBytes, s);
}

template <class S>
hipError_t occupancy_t(int wd, int *blocks) {
  const void *k = kernel_for<S>(wd);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, S::NT, kLdsBytes);
}

template <class S>
void info_t(ShapeInfo *o) {
  o->E = S::E;
  o->D = S::D;
  o->G = S::G;
  o->threads = S::NT;
  o->lds_bytes = kLdsBytes;
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

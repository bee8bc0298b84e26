// decode_kernel.hip -- the persistent batch-1 GPT-2 decode kernel for gfx950.
//
// One launch runs `nsteps` whole forward passes (one token each).
// The per-token work is the GPT-2 forward pass (the gpt2-125m "model.fir"
// page's network): embedding add, then per layer
//   A: LayerNorm 1 + QKV linear + bias
//   B: attn_decode: this position's K/V are appended, causal softmax over
//      positions 0..position, weighted sum of values (split in position chunks
//      of at most 64; the first chunk of a head merges the others)
//   C: attention linear + bias + residual
//   D: LayerNorm 2 + fc linear + bias + gelu_new
//   E: projection linear + bias + residual
// and finally H: final LayerNorm + tied output head + argmax.
//
// Work split.  The workgroups form four disjoint sets, one per block matrix
// (QKV, attention projection, fc, MLP projection); a workgroup owns an equal
// share of consecutive output rows of its set's matrix in every layer, and
// all workgroups share the output head by contiguous vocabulary rows.  Inside
// a workgroup an output row belongs to a segment of LPR lanes, so a row's dot
// product ends in one short DPP reduction.  A workgroup is one control wave
// plus NCW compute waves:
//   * the compute waves hold the workgroup's slice of one layer in registers
//     and request the next layer's slice as soon as the phase is done, so the
//     weights stream in during the other sets' phases;
//   * the control wave waits for the inputs of its phase, writes them into
//     LDS (scaled by the LayerNorm gain where a LayerNorm comes first; the
//     LayerNorm statistics are taken while the dot products run and applied
//     to the row results), runs an attention chunk when it has one, and
//     publishes;
//   * with more than three compute waves (the fp32 and fp16 kernels: two
//     waves per SIMD, 256 registers each) the last compute wave takes no slice
//     and runs the attention chunk in the control wave's place, with the
//     chunk's value rows in LDS.
// Each phase's inputs therefore come from, and go to, a few dozen workgroups
// rather than all of them, which shortens every hand-over.
// Batch 1 makes every linear a matrix-vector product (0.5 flop per fp32 byte),
// so there is no MFMA here: the kernel is bound by weight bytes and by the
// latency of the 5L+1 dependent phases of a token.  All arithmetic is fp32;
// the exponentials, reciprocals and the LayerNorm's reciprocal square root
// use the hardware's 1-ulp instructions (v_exp_f32, v_rcp_f32, v_rsq_f32),
// which shorten the single-wave chains of a phase.
//
// Synchronisation.  There is no grid barrier.  Each output element travels as
// one 64-bit word (float bits | epoch << 32), written and read with device-
// scope (sc1) accesses, two words per 16-byte store or load; the epoch numbers
// the producing phase uniquely within and across launches, and a consumer
// polls the words it needs until all carry the expected epoch.  Per-word
// coherence is all this needs: no cache write-back/invalidate fences are
// executed in the loop.  Every published vector exists in one copy per XCD.
// KV-cache rows are written with device-scope stores one step before any
// other workgroup reads them.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "dec_internal.h"

namespace gpt2dec {
namespace {

// Output-head rows are read with temporal loads: between steps they can stay
// in the memory-side cache, which the non-temporal block-matrix stream does
// not fill (measured faster than non-temporal head loads).
constexpr bool HEAD_NT = false;
constexpr int CHMIN = 64;      // positions per attention chunk before a head is split
constexpr int PSTRIDE = 512;   // LDS room for row results (>= rows per workgroup)

template <int E_, int D_, int NCW_, int MAXCH_, int LPRH_, int LPR_, int NQ_, int NA_, int NF_, int NM_,
          int CD_ = 0>
struct Shape {
  static constexpr int E = E_, D = D_, H = E_ / D_, F = 4 * E_;
  static constexpr int NCW = NCW_;        // compute waves
  static constexpr int NL = 64 * NCW_;    // compute lanes
  static constexpr int NT = NL + 64;      // threads: compute waves + control wave
  // CD: the control wave takes a share of every block-matrix slice too (it
  // would otherwise idle through the dot products); NLD lanes share a slice.
  static constexpr bool CD = CD_ != 0;
  // With more than three compute waves (two waves on some SIMDs, 256
  // registers each), the attention items run on the last compute wave, which
  // takes no share of the slices and keeps the chunk's value rows in LDS
  // (att_item_cw): the control wave's registers would not hold an item.
  static constexpr bool ITEM_CW = NCW_ > 3;
  static constexpr int IW = NCW_ - 1;  // that compute wave
  static constexpr int NLD = NL + (CD_ ? 64 : 0) - (ITEM_CW ? 64 : 0);  // lanes sharing a slice
  static constexpr int NLH = NL - (ITEM_CW ? 64 : 0);  // compute lanes that take output-head rows
  static constexpr int MAXCH = MAXCH_;    // attention chunks per head at most
  static constexpr int LPRH = LPRH_;      // lanes per head row
  static constexpr int LPR = LPR_;        // lanes per row of a block matrix
  // Output head, per wave: batches streamed from memory in flight, and
  // batches wanted in registers through the head by a workgroup of set Q (its
  // slice registers hold the next step's first slice by then) and by one of
  // the later sets (whose idle slice registers hold part of them).
  static constexpr int HEAD_BATCHES = 3;
  static constexpr int HEAD_REGS_Q = 2, HEAD_REGS_LATE = 3;
  static constexpr int HEAD_REGS_Q4_Q = 2, HEAD_REGS_Q4_LATE = 3;  // int4 (its head is fp32)
  // fp16 with two waves per SIMD: a batch of fp16 head rows takes half the
  // registers of an fp32 one, and the fp16 slices leave them free
  static constexpr int HEAD_REGS_F16_Q = 5, HEAD_REGS_F16_LATE = 8;
  // Batches (of 64/LPRH rows) of output-head rows the control wave keeps in its
  // own registers for the launch and takes during the head (none with a slice
  // share, whose registers it needs).
  static constexpr int HEAD_CTL_BATCHES = CD_ ? 0 : 2;
  // The MLP activation (the longest polled vector) is polled in this many
  // equal parts by as many waves at once: the compute waves and the control
  // wave (each part a whole number of 128-word pair loads), else by the
  // control wave alone.
  static constexpr int M_PARTS = (4 * E_) % (128 * (NCW_ + 1)) == 0 ? NCW_ + 1 : 1;
  // Workgroup sets, one per block matrix, over consecutive blockIdx ranges in
  // this order: QKV, attention projection, fc, MLP projection.
  static constexpr int NQ = NQ_, NA = NA_, NF = NF_, NM = NM_;
  static constexpr int G = NQ_ + NA_ + NF_ + NM_;  // workgroups
  static_assert(E_ % D_ == 0 && E_ % 64 == 0 && D_ <= 64 && 64 % (D_ / 4) == 0, "shape");
  static_assert((3 * E_) % NQ_ == 0 && E_ % NA_ == 0 && (4 * E_) % NF_ == 0 && E_ % NM_ == 0,
                "equal row shares");
  static_assert(H * MAXCH <= G, "one attention chunk per workgroup at most");
  // LDS layout (floats)
  // [F] phase input vector; with ITEM_CW also (at least [64][D]) the
  // attention item's value rows, read before the workgroup's next phase input
  // can be complete (it depends on the item's output; a dot wave's part of set
  // A's input waits for the item's release word, poll_in_part)
  static constexpr int L_XS = 0;
  static constexpr int XS_N = ITEM_CW && 64 * D_ > F ? 64 * D_ : F;
  static constexpr int L_PART = L_XS + XS_N;             // [PSTRIDE] row results
  static constexpr int L_Q = L_PART + PSTRIDE;           // [D] query of the attention item
  static constexpr int L_KP = L_Q + D;                   // [D] key of this position
  static constexpr int L_VP = L_KP + D;                  // [D] value of this position
  static constexpr int L_SC = L_VP + D;                  // [64] attention weights (transposed)
  static constexpr int L_V = L_XS;                       // [64][D] an item's value rows (ITEM_CW)
  static constexpr int L_XRAW = L_XS + E;                // [E] a LayerNorm input before its gain (ITEM_CW)
  static constexpr int L_FLAG = L_SC + 64;               // [4] flags: abort (control), abort (compute)
  static constexpr int L_TOTAL = L_FLAG + 4;
  static constexpr int L_HEAD = (L_TOTAL + 63) & ~63;    // output-head rows kept for the launch
};

// 124M shape.  fp32 and fp16: 256 workgroups x (7 compute + 1 control) waves,
// two waves on each SIMD: six waves take the dot products (32 lanes per row),
// the seventh the attention item; sets of 64 (QKV, 36 rows each), 32
// (attention projection, 24 rows), 64 (fc, 48 rows) and 96 (MLP projection, 8
// rows), so every fp32 workgroup reads 74 to 147 KB of weights per layer.
// int4, whose dot products cost about two vector instructions per weight and
// more registers: 256 workgroups x (3 compute + 1 control) waves, and the
// control wave takes a share of every slice too, in sets of 72 (32 rows), 24
// (32 rows), 64 (48 rows) and 96 (8 rows), row counts that 16 (64 for K =
// 3072) rows per pass of 256 lanes divide.  (Set sizes and the split chosen by
// measurement.)
using ShapeS = Shape<768, 64, 7, 16, 32, 32, 64, 32, 64, 96, 0>;
using ShapeSC = Shape<768, 64, 3, 16, 16, 16, 72, 24, 64, 96, 1>;
// tiny shape: 32 workgroups x (2 compute + 1 control) waves, sets 8/4/16/4.
using ShapeT = Shape<128, 32, 2, 8, 8, 8, 8, 4, 16, 4>;

// The workgroup sets.  Set SET owns the R consecutive rows rank*R.. of its
// [ROWS][K] matrix for every layer.  Inside the workgroup, LPR lanes share a
// row (chunks lane%LPR + LPR*i, i < CPR), RP = NL/LPR rows are covered per
// pass and NP passes cover the R rows, so each lane holds NB = NP*CPR weight
// chunks and reuses each of its CPR input chunks NP times.
enum { SET_Q = 0, SET_A = 1, SET_F = 2, SET_M = 3 };
// Lanes per row: the shape's default, doubled (up to 64) while a lane would
// need more than 12 input chunks, so that a dot product reads at most 12
// chunks of the input vector from LDS.
constexpr int lpr_for(int KC, int lpr) {
  while (KC / lpr > 12 && lpr < 64) lpr *= 2;
  return lpr;
}
template <class S, int SET>
struct Set {
  static constexpr int FIRST = SET == SET_Q ? 0 : SET == SET_A ? S::NQ : SET == SET_F ? S::NQ + S::NA
                                                                                      : S::NQ + S::NA + S::NF;
  static constexpr int N = SET == SET_Q ? S::NQ : SET == SET_A ? S::NA : SET == SET_F ? S::NF : S::NM;
  static constexpr int ROWS = SET == SET_Q ? 3 * S::E : SET == SET_F ? S::F : S::E;
  static constexpr int K = SET == SET_M ? S::F : S::E;
  static constexpr int R = ROWS / N;
  static constexpr int KC = K / 4;
  static constexpr int LPR = lpr_for(KC, S::LPR);
  static constexpr int RP = S::NLD / LPR;
  static constexpr int NP = (R + RP - 1) / RP;
  static constexpr int CPR = KC / LPR;
  static constexpr int NB = NP * CPR;
  static_assert(KC % LPR == 0 && S::NLD % LPR == 0 && R <= 64 && R <= PSTRIDE, "slice geometry");
  static_assert(R % 2 == 0, "rows are published in pairs");
  static_assert(LPR % 8 == 0, "chunk steps are whole int4 groups");
};

// ---- weight chunks: 4 consecutive inputs of one output row ----------------
// (int4: two neighbouring chunks of one group, 8 codes in q, with the group's
// scale and zero; loaded by load_set, taken by dot_q4x2m)
template <int WD> struct Chunk;
template <> struct Chunk<WD_F32> { float4 v; };
template <> struct Chunk<WD_F16> { uint2 v; };
template <> struct Chunk<WD_Q4> { uint32_t q; float2 sz; };

// Weight chunks are read with buffer loads: the base of the stream (a
// layer's slice, or a run of output-head rows) sits in a scalar resource and
// each lane adds one 32-bit byte offset plus a constant per chunk, so no
// 64-bit address per chunk is kept in registers.  Weights are read once per
// token: non-temporal loads keep them from displacing the small, reused data
// (LayerNorm parameters, biases, activations) in the caches.
typedef float g2_v2f __attribute__((ext_vector_type(2)));
typedef unsigned int g2_v2u __attribute__((ext_vector_type(2)));
typedef unsigned int g2_v4u __attribute__((ext_vector_type(4)));

struct WSrc {
  __amdgpu_buffer_rsrc_t w, sz;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7fffffff, 0x00020000);
}
// The chunks of m from chunk index c0 on (c0 = row*K/4 + k/4 over the layers'
// [L][N][K] matrices; for int4 a multiple of 8, a group boundary).
template <int WD>
__device__ __forceinline__ WSrc wsrc(const MatW &m, size_t c0) {
  WSrc s;
  constexpr size_t CB = WD == WD_F32 ? 16 : WD == WD_F16 ? 8 : 2;  // bytes per chunk
  s.w = stream_rsrc(static_cast<const char *>(m.w) + c0 * CB);
  s.sz = s.w;
  if constexpr (WD == WD_Q4) s.sz = stream_rsrc(m.sz + c0 / 8);
  return s;
}
// Chunk cl + ck of the stream: cl per lane, ck uniform (a multiple of 8; it
// goes into the scalar offset, so a run of loads shares one lane offset).
template <int WD, bool NT = true>
__device__ __forceinline__ Chunk<WD> ld_chunk(const WSrc &s, uint32_t cl, uint32_t ck = 0) {
  constexpr int AUX = NT ? 2 : 0;  // nt
  static_assert(WD != WD_Q4, "int4 chunks are loaded in pairs (load_set)");
  Chunk<WD> r;
  if constexpr (WD == WD_F32) {
    const g2_v4u v = __builtin_amdgcn_raw_buffer_load_b128(s.w, cl * 16u, ck * 16u, AUX);
    r.v = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  } else {
    const g2_v2u v = __builtin_amdgcn_raw_buffer_load_b64(s.w, cl * 8u, ck * 8u, AUX);
    r.v = make_uint2(v.x, v.y);
  }
  return r;
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

// The weights a chunk stands for, as fp32 (fp16 widening is exact).
template <int WD>
__device__ __forceinline__ float4 deq(const Chunk<WD> &c) {
  static_assert(WD != WD_Q4, "int4 chunks are taken in pairs (dot_q4x2m)");
  if constexpr (WD == WD_F32) {
    return c.v;
  } else {
    return make_float4(h2f(c.v.x), h2f(c.v.x >> 16), h2f(c.v.y), h2f(c.v.y >> 16));
  }
}

__device__ __forceinline__ float dot4(float4 w, float4 x, float acc) {
  acc = __builtin_fmaf(w.x, x.x, acc);
  acc = __builtin_fmaf(w.y, x.y, acc);
  acc = __builtin_fmaf(w.z, x.z, acc);
  acc = __builtin_fmaf(w.w, x.w, acc);
  return acc;
}

// Two neighbouring int4 chunks of one group (8 inputs, the 8 codes in one
// 32-bit word) against their inputs x0, x1, with the group's scale s and zero
// z taken out of the sum: sum_k (code_k*s + z)*x_k = s*sum_k code_k*x_k +
// z*xsum, xsum the sum of the 8 inputs, so one scale and one zero per 8
// weights.  Each code is taken as an fp16 subnormal: a code n alone in a
// 16-bit half, in the half's bits 0-3 or 4-7, is exactly n * 2^-24 or
// n * 2^-20, which the mixed-precision multiply-add widens and multiplies in
// one instruction, with no conversion (fp16 subnormals are kept, the default
// floating-point mode).  Four masks and one shift spread the 8 codes over four
// words; the two kinds are summed apart and joined with an exact factor 1/16.
// The scale terms accumulate in as (times 2^-24, exactly), the zero terms in
// az; the row result is as * 2^24 + az.
__device__ __forceinline__ void dot_q4x2m(uint32_t q, float2 sz, float4 x0, float4 x1, float xsum, float &as,
                                          float &az) {
  const uint32_t u = q >> 8;
  const uint32_t c04 = q & 0x000F000Fu, c26 = u & 0x000F000Fu;  // n * 2^-24
  const uint32_t c15 = q & 0x00F000F0u, c37 = u & 0x00F000F0u;  // n * 2^-20
  float ta = __builtin_fmaf(h2f(c04), x0.x, 0.f);
  float tb = __builtin_fmaf(h2f(c15), x0.y, 0.f);
  ta = __builtin_fmaf(h2f(c26), x0.z, ta);
  tb = __builtin_fmaf(h2f(c37), x0.w, tb);
  ta = __builtin_fmaf(h2f(c04 >> 16), x1.x, ta);
  tb = __builtin_fmaf(h2f(c15 >> 16), x1.y, tb);
  ta = __builtin_fmaf(h2f(c26 >> 16), x1.z, ta);
  tb = __builtin_fmaf(h2f(c37 >> 16), x1.w, tb);
  as = __builtin_fmaf(sz.x, __builtin_fmaf(tb, 0.0625f, ta), as);
  az = __builtin_fmaf(sz.y, xsum, az);
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
// The last lane's value of each W-lane segment, in every lane of the segment
// (16-lane rows: one DPP row broadcast; otherwise a lane permute).
template <int W>
__device__ __forceinline__ float seg_bcast_last(float v, int lane) {
  if constexpr (W == 16) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x15F, 0xF, 0xF, false));
  } else if constexpr (W == 64) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  } else {
    return __shfl(v, lane | (W - 1));
  }
}
// Lane k's value of each W-lane segment, in every lane of the segment.
template <int W>
__device__ __forceinline__ float seg_bcast(float v, int k, int lane) {
  if constexpr (W == 16) {
    // row_newbcast:k; k is a compile-time constant after unrolling
    switch (k) {
#define G2_NB(K) case K: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xF, 0xF, false));
      G2_NB(0) G2_NB(1) G2_NB(2) G2_NB(3) G2_NB(4) G2_NB(5) G2_NB(6) G2_NB(7)
      G2_NB(8) G2_NB(9) G2_NB(10) G2_NB(11) G2_NB(12) G2_NB(13) G2_NB(14) G2_NB(15)
#undef G2_NB
    }
    return v;
  } else {
    return __shfl(v, (lane & ~(W - 1)) | k);
  }
}

// Reduce-scatter inside W-lane segments (W = 8 or 16): x[i] holds each
// lane's part of row i; afterwards lane j of a segment returns the total of
// row j over the segment's W lanes.  Each step pairs lanes that differ in the
// bits of one mask (xor 15, 7, 2, 1 via row mirror, half-row mirror and quad
// permutes): one lane keeps the lower half of its remaining rows, its partner
// the upper half, and each adds the partner's part of the rows it keeps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int H, int CTRL>
__device__ __forceinline__ void rs_step(float (&x)[16], bool upper) {
#pragma unroll
  for (int i = 0; i < H; i++) {
    const float keep = upper ? x[i + H] : x[i];
    const float send = upper ? x[i] : x[i + H];
    x[i] = keep + dpp_mov<CTRL>(send);
  }
}
template <int W>
__device__ __forceinline__ float seg_reduce_scatter(const float (&in)[W], int lane) {
  static_assert(W == 8 || W == 16, "segment");
  float x[16];
#pragma unroll
  for (int i = 0; i < W; i++) x[i] = in[i];
  const int j = lane % W;
  if constexpr (W == 16) rs_step<8, 0x140>(x, (j & 8) != 0);  // row_mirror: lane j <-> 15 - j
  rs_step<4, 0x141>(x, (j & 4) != 0);                         // row_half_mirror: j <-> j ^ 7
  rs_step<2, 0x4E>(x, (j & 2) != 0);                          // quad_perm [2,3,0,1]: j <-> j ^ 2
  rs_step<1, 0xB1>(x, (j & 1) != 0);                          // quad_perm [1,0,3,2]: j <-> j ^ 1
  return x[0];
}

// v + v of lane (lane ^ sh).  Across 16-lane rows (sh 16 or 32) by the
// permlane swaps, which exchange rows between two registers without LDS: with
// both operands v, the two results hold v and its partner in every lane.
__device__ __forceinline__ float xor_sum(float v, int sh) {
  if (sh == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (sh == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v + __shfl_xor(v, sh);
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
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t x, uint32_t ep) { return (uint32_t)(x >> 32) == ep; }
// Every published vector exists in NCOPY copies, a multiple of the 8 XCDs
// (workgroup w is taken to run on XCD w % 8): a producer writes all copies
// (with tst_pairs / tst2 below), a consumer polls copy w % NCOPY, which
// spreads the polling over NCOPY times the lines.
constexpr int NCOPY = kTagCopies;
static_assert(NCOPY % 8 == 0, "copies per XCD");
__device__ __forceinline__ int my_copy() { return (int)(blockIdx.x % NCOPY); }
__device__ __forceinline__ float payload(uint64_t x) { return __uint_as_float((uint32_t)x); }

// The first failure of a run: the error word (which every bounded wait reads,
// so that all workgroups stop) and its host-mapped copy, which the host reads
// once the launch has ended.
__device__ __forceinline__ void raise_error(const DecodeArgs &a, int code, int phase, int step) {
  int zero = 0;
  if (__hip_atomic_compare_exchange_strong(a.err, &zero, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(a.err + 1, (int)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.err + 2, phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.err + 3, step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.err_host[1] = (int)blockIdx.x;
    a.err_host[2] = phase;
    a.err_host[3] = step;
    a.err_host[0] = code;
  }
}

// The id fed at `step` (< n_feed): from the kernel arguments, or from the
// uploaded buffer for a long prompt.
__device__ __forceinline__ int fed_token(const DecodeArgs &a, int step) {
  return a.n_feed <= kFeedInline ? a.feed_inline[step] : a.feed[step];
}

// Bounded waiting: a wait that outlives the time limit, or sees another
// workgroup's abort, sets the error word and makes the caller stop.
struct Waiter {
  const DecodeArgs *a;
  long long t0;
  int phase;
  unsigned polls;
  __device__ void start(int ph) {
    t0 = 0;  // (the clock is first read once the wait is long)
    phase = ph;
    polls = 0;
  }
  __device__ bool expired() {
    // A wait that ends within a few poll rounds (nearly every one) reads
    // nothing here: the clock and the error word are looked at on every 16th
    // failed poll only, the time limit counted from the first of those reads.
    // (Each is a memory or counter round trip of its own, which would
    // otherwise lengthen every poll round.)
    if ((++polls & 15u) != 0) return false;
    if (__hip_atomic_load(a->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    const long long now = (long long)wall_clock64();
    if (t0 == 0) t0 = now;
    if (now - t0 > a->timeout_ticks) {
      raise_error(*a, ERR_TIMEOUT, phase, -1);
      return true;
    }
    return false;
  }
};

// A lane's share of a polled vector: element vidx(lane, j) for j < PER, in
// pairs of neighbours, so that one 16-byte load brings two tagged words.
__device__ __forceinline__ int vidx(int lane, int j) { return 128 * (j >> 1) + 2 * lane + (j & 1); }

// Poll the PER*64 tagged floats at src (lane share as vidx) into v until all
// carry ep.  Each 8-byte half of a 16-byte load is one word written by one
// atomic store, so a half is either the old word or the new one; the loads
// use device scope (sc1) like the atomic loads elsewhere.
constexpr int AUX_SC1 = 16;
template <int PER>
__device__ bool poll_vec(const uint64_t *src, uint32_t ep, float (&v)[PER], int lane, Waiter &wt) {
  static_assert(PER % 2 == 0, "words are polled in pairs");
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t *>(src), (short)0, PER * 64 * 8,
                                                    0x00020000);
  while (true) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PER; j += 2) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, vidx(lane, j) * 8, 0, AUX_SC1);
      v[j] = __uint_as_float(x[0]);
      v[j + 1] = __uint_as_float(x[2]);
      ok &= (x[1] == ep) && (x[3] == ep);
    }
    if (__all(ok)) return true;
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Two tagged words with one 16-byte store at byte offset off of buffer rs;
// each 8-byte half is one whole word (the consumers poll word pairs).
__device__ __forceinline__ void tst2(__amdgpu_buffer_rsrc_t rs, uint32_t off, float a, float b, uint32_t ep) {
  typedef unsigned int g2_v4u __attribute__((ext_vector_type(4)));
  const g2_v4u v = {__float_as_uint(a), ep, __float_as_uint(b), ep};
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, AUX_SC1);
}

// Publish one value per lane (the lane's row; lanes < R, R even, row parity =
// lane parity) to all NCOPY copies of a vector of `stride` words, as word
// pairs: the two lanes of a pair exchange values, the even one writes the
// pair to the first half of the copies, the odd one to the second half.
__device__ __forceinline__ void tst_pairs(__amdgpu_buffer_rsrc_t rs, int stride, int row, float v, uint32_t ep,
                                          int lane) {
  const float vn = dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]: the other lane of the pair
  const bool odd = (lane & 1) != 0;
  const float lo = odd ? vn : v, hi = odd ? v : vn;
  const int r0 = row & ~1, c0 = odd ? NCOPY / 2 : 0;
#pragma unroll
  for (int k = 0; k < NCOPY / 2; k++) tst2(rs, (uint32_t)(((c0 + k) * stride + r0) * 8), lo, hi, ep);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t copies_rsrc(uint64_t *base, int stride) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, NCOPY * stride * 8, 0x00020000);
}

// LayerNorm, folded into the linear that follows it.  For a row w of that
// linear with bias b, LayerNorm gain g and shift h, and the input's mean m and
// rstd = 1/sqrt(var + eps):
//   w.LN(x) + b = rstd * (w.(g*x) - m * w.g) + (w.h + b),
// so the dot products read g*x, which needs no statistics, and the
// statistics are taken while they run.  w.g and w.h + b are per-row constants
// (computed at load from the weights as the dot products decode them).
// The input x, held as a lane share (element vidx(lane, j)), scaled by g into LDS:
template <int E>
__device__ __forceinline__ void gain_to_lds(const float (&x)[E / 64], const float (&g)[E / 64], float *dst,
                                            int lane) {
#pragma unroll
  for (int j = 0; j < E / 64; j++) dst[vidx(lane, j)] = x[j] * g[j];
}
// Mean and 1/sqrt(biased variance + eps) of x, following the model file's
// layernorm kernel (mean first, then the mean square deviation).
template <int E>
__device__ __forceinline__ void ln_stats(const float (&x)[E / 64], float eps, float &mean, float &rstd) {
  constexpr int PER = E / 64;
  // four independent partial sums per lane (shorter dependency chains)
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < PER; j++) s4[j % 4] += x[j];
  mean = wave_sum_all((s4[0] + s4[1]) + (s4[2] + s4[3])) * (1.0f / (float)E);
  float q4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const float d = x[j] - mean;
    q4[j % 4] = __builtin_fmaf(d, d, q4[j % 4]);
  }
  const float var = wave_sum_all((q4[0] + q4[1]) + (q4[2] + q4[3])) * (1.0f / (float)E);
  rstd = __builtin_amdgcn_rsqf(var + eps);  // v_rsq_f32 (1 ulp)
  // (register-only work may otherwise be scheduled past the next barrier,
  // whose asm orders memory only: the statistics are finished here)
  asm volatile("" ::"v"(mean), "v"(rstd));
}
// A row of the folded linear from its dot product with g*x.
__device__ __forceinline__ float ln_row(float dot, float mean, float rstd, float wg, float c) {
  return __builtin_fmaf(rstd, __builtin_fmaf(-mean, wg, dot), c);
}

__device__ __forceinline__ float gelu_new(float f) {
  // x * sigmoid(2*sqrt(2/pi) * (x + 0.044715 x^3)), the model file's gelu_new
  float t = f * f;
  t = t * f;
  t = t * 0.044715f;
  t = t + f;
  t = t * 1.5957691216057308f;
  t = __builtin_amdgcn_rcpf(1.0f + __expf(-t));  // v_exp_f32, v_rcp_f32 (1 ulp each)
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

// Attention items go to the workgroups after set Q, in blockIdx order: item
// (head h, chunk c) is h*nch + c.  The item index of workgroup w, and whether
// it has one at position p.
template <class S>
__device__ __forceinline__ int att_item_of(int w) { return (w + S::G - S::NQ) % S::G; }
template <class S>
__device__ __forceinline__ bool has_att_item(int p, int w) {
  int nch, ch;
  att_chunks<S>(p, nch, ch);
  return att_item_of<S>(w) < S::H * nch;
}

// Optional timeline of one workgroup's control wave (lane 0): inputs ready, first and
// second workgroup barrier passed, outputs published.  Compiled only into the
// kernel variant that a traced run launches: the stamps' tests, addresses and
// clock reads otherwise cost registers and time in every phase.
__device__ __forceinline__ void stamp(const DecodeArgs &a, int step, int ph, int which, int G) {
  if (a.trace && step < a.trace_steps)
    a.trace[(((size_t)step * (5 * a.L + 1) + ph) * G + blockIdx.x) * 4 + which] = (long long)wall_clock64();
}

__device__ __forceinline__ uint32_t epoch_of(const DecodeArgs &a, int step, int ph) {
  return a.epoch0 + (uint32_t)step * (uint32_t)(5 * a.L + 1) + (uint32_t)ph + 1u;
}

// ---- compute waves ---------------------------------------------------------
// Request this workgroup's slice of one layer of its set's matrix.  Lanes of a
// pass past the slice re-read its last row (same addresses as other lanes of
// the wave, results discarded), so every load is unconditional.
template <class ST, int WD>
__device__ __forceinline__ void load_set(Chunk<WD> (&b)[ST::NB], const MatW &m, int layer, int rank, int lane) {
  const WSrc src = wsrc<WD>(m, ((size_t)layer * ST::ROWS + (size_t)rank * ST::R) * ST::KC);
  const int q = lane % ST::LPR;
#pragma unroll
  for (int t = 0; t < ST::NP; t++) {
    const int r = min(t * ST::RP + lane / ST::LPR, ST::R - 1);
    if constexpr (WD == WD_Q4) {
      // int4: lane q takes chunk pairs (2q, 2q+1) + 2*LPR*i, each pair one
      // 32-bit word of codes inside one group; entry t*CPR + i holds pair i
      const uint32_t c0 = (uint32_t)(r * ST::KC + 2 * q);
#pragma unroll
      for (int i = 0; i < ST::CPR / 2; i++) {
        const uint32_t ck = (uint32_t)(2 * ST::LPR * i);
        Chunk<WD_Q4> c;
        c.q = __builtin_amdgcn_raw_buffer_load_b32(src.w, c0 * 2u, ck * 2u, 2);
        const g2_v2u z = __builtin_amdgcn_raw_buffer_load_b64(src.sz, (c0 / 8u) * 8u, ck, 2);
        c.sz = make_float2(__uint_as_float(z.x), __uint_as_float(z.y));
        b[t * ST::CPR + i] = c;
      }
    } else {
      const uint32_t c0 = (uint32_t)(r * ST::KC + q);
#pragma unroll
      for (int i = 0; i < ST::CPR; i++) b[t * ST::CPR + i] = ld_chunk<WD>(src, c0, (uint32_t)(i * ST::LPR));
    }
  }
}

// Row results of the slice (input vector in LDS) into part[0..R): each lane
// sums its chunks in order (fp16: its even and its odd chunks, then the two;
// int4: its chunk pairs, each with its group's scale and zero taken out, the
// scale and the zero terms in two sums, dot_q4x2m), then a DPP reduction over
// the row's LPR lanes.
template <class ST, int WD>
__device__ __forceinline__ void dot_set(const Chunk<WD> (&b)[ST::NB], const float *xs, float *part, int lane) {
  const int q = lane % ST::LPR;
  // all input chunks first: one burst of LDS reads instead of one round trip per
  // chunk (int4: the chunks of its pairs, (2q, 2q+1) + 2*LPR*i)
  float4 xv[ST::CPR];
#pragma unroll
  for (int i = 0; i < ST::CPR; i++)
    xv[i] = WD == WD_Q4 ? reinterpret_cast<const float4 *>(xs)[2 * q + (i & 1) + 2 * ST::LPR * (i >> 1)]
                        : reinterpret_cast<const float4 *>(xs)[i * ST::LPR + q];
  // fp16 and int4: two partial sums per row (even and odd chunks), two
  // independent chains (measured faster there; fp32 keeps one)
  constexpr int NCH = WD == WD_F32 ? 1 : 2;
  float acc[ST::NP][2];
#pragma unroll
  for (int t = 0; t < ST::NP; t++) acc[t][0] = acc[t][1] = 0.f;
  if constexpr (WD == WD_Q4) {
    static_assert(ST::CPR % 2 == 0, "int4 chunk pairs");
    float xsum[ST::CPR / 2];
#pragma unroll
    for (int i = 0; i < ST::CPR / 2; i++) {
      const float4 u = xv[2 * i], v = xv[2 * i + 1];
      xsum[i] = ((u.x + u.y) + (u.z + u.w)) + ((v.x + v.y) + (v.z + v.w));
    }
#pragma unroll
    for (int i = 0; i < ST::CPR / 2; i++) {
#pragma unroll
      for (int t = 0; t < ST::NP; t++) {
        const Chunk<WD> &c = b[t * ST::CPR + i];
        dot_q4x2m(c.q, c.sz, xv[2 * i], xv[2 * i + 1], xsum[i], acc[t][0], acc[t][1]);
      }
    }
#pragma unroll
    for (int t = 0; t < ST::NP; t++) {
      acc[t][0] = __builtin_fmaf(acc[t][0], 16777216.0f, acc[t][1]);
      acc[t][1] = 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < ST::CPR; i++) {
#pragma unroll
      for (int t = 0; t < ST::NP; t++)
        acc[t][i % NCH] = dot4(deq<WD>(b[t * ST::CPR + i]), xv[i], acc[t][i % NCH]);
    }
  }
#pragma unroll
  for (int t = 0; t < ST::NP; t++) {
    const float v = seg_sum_last<ST::LPR>(NCH == 2 ? acc[t][0] + acc[t][1] : acc[t][0]);
    const int r = t * ST::RP + lane / ST::LPR;
    if (q == ST::LPR - 1 && r < ST::R) part[r] = v;
  }
}

template <class S, int WD>
struct HeadGeo {
  static constexpr int KC = S::E / 4, LPR = S::LPRH, NPH = KC / LPR, RB = S::NLH / LPR;
  static constexpr int RBC = 64 / LPR, CTL_ROWS = S::HEAD_CTL_BATCHES * RBC;  // the control wave's rows
  static constexpr int HWD = (WD == WD_F16) ? WD_F16 : WD_F32;
  static_assert(KC % LPR == 0 && S::NLH % LPR == 0 && LPR % 8 == 0, "head geometry");
};

// Batches of output-head rows that a workgroup of set SET holds in registers
// during the head: head_reg_batches in its idle slice registers (the late
// sets, when the register chunk type is the head's: not for int4), requested
// after the set's last phase of each step, and head_extra_batches in registers
// of their own, requested once and kept for the launch, up to a total per
// weight type and shape (fp16 with four waves: the fp32 counts, more measured
// slower; fp16 with eight waves: 5 and 8, measured faster than 2 and 3).
template <class S, int WD, int SET>
constexpr int head_reg_want() {
  if constexpr (WD == WD_F16 && S::ITEM_CW) return SET == SET_Q ? S::HEAD_REGS_F16_Q : S::HEAD_REGS_F16_LATE;
  return WD == WD_Q4 ? (SET == SET_Q ? S::HEAD_REGS_Q4_Q : S::HEAD_REGS_Q4_LATE)
                     : (SET == SET_Q ? S::HEAD_REGS_Q : S::HEAD_REGS_LATE);
}
template <class S, int WD, int SET>
constexpr int head_reg_batches() {
  using HG = HeadGeo<S, WD>;
  return (SET != SET_Q && WD == HG::HWD) ? Set<S, SET>::NB / HG::NPH : 0;
}
template <class S, int WD, int SET>
constexpr int head_extra_batches() {
  constexpr int x = head_reg_want<S, WD, SET>() - head_reg_batches<S, WD, SET>();
  return x > 0 ? x : 0;
}
template <class S, int WD, int SET>
constexpr int head_reg_total() {
  return head_reg_batches<S, WD, SET>() + head_extra_batches<S, WD, SET>();
}

// Output-head rows [hr0, hr1) of workgroup w: the rows left after each
// workgroup's register batches (the compute waves' and the control wave's)
// are split evenly, and each workgroup adds the rows its registers hold
// (capped so that no workgroup exceeds PSTRIDE rows), so every workgroup
// streams about the same number of rows during the head.  A workgroup's
// rows are, in order: LDS-resident, compute-wave registers, control-wave
// registers, streamed.
template <class S, int WD>
__device__ __forceinline__ void head_range(int V, int w, int &hr0, int &hr1) {
  constexpr int RB = HeadGeo<S, WD>::RB;
  const int even = V / S::G;
  // no workgroup may get more than PSTRIDE rows (the row results live in LDS)
  const int cap = min(even, max(0, PSTRIDE - even - 1));
  const int eQ = min(head_reg_total<S, WD, SET_Q>() * RB + HeadGeo<S, WD>::CTL_ROWS, cap);
  const int eA = min(head_reg_total<S, WD, SET_A>() * RB + HeadGeo<S, WD>::CTL_ROWS, cap);
  const int eF = min(head_reg_total<S, WD, SET_F>() * RB + HeadGeo<S, WD>::CTL_ROWS, cap);
  const int eM = min(head_reg_total<S, WD, SET_M>() * RB + HeadGeo<S, WD>::CTL_ROWS, cap);
  const int rest = V - S::NQ * eQ - S::NA * eA - S::NF * eF - S::NM * eM;
  auto start = [&](int u) {
    const int nq = min(u, S::NQ);
    const int na = min(max(u - Set<S, SET_A>::FIRST, 0), S::NA);
    const int nf = min(max(u - Set<S, SET_F>::FIRST, 0), S::NF);
    const int nm = min(max(u - Set<S, SET_M>::FIRST, 0), S::NM);
    return (int)(((long long)u * rest) / S::G) + nq * eQ + na * eA + nf * eF + nm * eM;
  };
  hr0 = start(w);
  hr1 = start(w + 1);
}

// The first head_lds_rows of this workgroup's output-head rows stay in LDS
// for the whole launch (the head does not change between steps); they are
// copied in once, during the first layer of the first step.  An fp16 head
// (twice the rows) is copied by direct global-to-LDS loads: no registers, and
// nothing waits for them until the compute waves' wait in the next layer
// (wait_head_lds); a wave's load puts lane i's 16 bytes at its LDS base + 16 i,
// so the waves copy the rows' bytes in runs of 1 KB.  (The same copy for the
// fp32 head measured slower in whole runs of the fp32 and int4 kernels; it
// shortened the fp16 kernel's one-pass launch by 4 us.)
template <class S, int WD>
__device__ void fill_head_lds(const DecodeArgs &a, float *lds, int lane) {
  constexpr int KC = S::E / 4, U = 4;
  constexpr int HWD = (WD == WD_F16) ? WD_F16 : WD_F32;
  int hr0, hr1;
  head_range<S, WD>(a.V, (int)blockIdx.x, hr0, hr1);
  if constexpr (HWD == WD_F16) {
    constexpr int RB16 = S::E * 2 / 16;  // 16-byte pieces per row
    static_assert(S::E * 2 % 16 == 0, "whole 16-byte pieces per head row");
    typedef __attribute__((address_space(1))) void g_void;
    typedef __attribute__((address_space(3))) void l_void;
    const int n = min(hr1 - hr0, a.head_lds_rows) * RB16;
    const char *src = static_cast<const char *>(a.head) + (size_t)hr0 * RB16 * 16;
    char *dst = reinterpret_cast<char *>(lds + S::L_HEAD);
    const int wv = __builtin_amdgcn_readfirstlane(lane / 64), wl = lane % 64;
    for (int i0 = 64 * wv; i0 < n; i0 += S::NLH) {
      if (i0 + wl < n)
        __builtin_amdgcn_global_load_lds((g_void *)(src + (size_t)(i0 + wl) * 16),
                                         (l_void *)(dst + (size_t)i0 * 16), 16, 0, 0);
    }
  } else {
    const int n = min(hr1 - hr0, a.head_lds_rows) * KC;
    if (n <= 0) return;
    const WSrc src = wsrc<HWD>(MatW{a.head, nullptr}, (size_t)hr0 * KC);
    Chunk<HWD> *dst = reinterpret_cast<Chunk<HWD> *>(lds + S::L_HEAD);
    for (int i0 = 0; i0 < n; i0 += U * S::NLH) {
      Chunk<HWD> c[U];
#pragma unroll
      for (int u = 0; u < U; u++) c[u] = ld_chunk<HWD, HEAD_NT>(src, (uint32_t)min(i0 + u * S::NLH + lane, n - 1));
#pragma unroll
      for (int u = 0; u < U; u++)
        if (i0 + u * S::NLH + lane < n) dst[i0 + u * S::NLH + lane] = c[u];
    }
  }
}
// This wave's direct copies into LDS are complete (the workgroup's next
// barrier then makes every wave's copies visible to all).
__device__ __forceinline__ void wait_head_lds() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Request head rows into registers, following the LDS-resident ones: NRB
// batches into the idle slice registers b (late sets; once per step, after
// the set's last phase), or (K0 = NRB) the NX batches after those into hx,
// which keep them for the whole launch (requested once).  Batches past the
// last row re-read that row.
template <class S, int WD, int K0, int NK, class Dst>
__device__ __forceinline__ void head_load_rows(const DecodeArgs &a, Dst &&put, int lane) {
  using HG = HeadGeo<S, WD>;
  if constexpr (NK > 0) {
    int hr0, hr1;
    head_range<S, WD>(a.V, (int)blockIdx.x, hr0, hr1);
    const int nr = hr1 - hr0, nl = min(nr, a.head_lds_rows);
    if (nr - nl <= 0) return;
    const WSrc src = wsrc<HG::HWD>(MatW{a.head, nullptr}, (size_t)hr0 * HG::KC);
    const int q = lane % HG::LPR, rl = lane / HG::LPR;
#pragma unroll
    for (int k = 0; k < NK; k++) {
      const int r = min(nl + (K0 + k) * HG::RB + rl, nr - 1);
      const uint32_t c0 = (uint32_t)(r * HG::KC + q);
#pragma unroll
      for (int i = 0; i < HG::NPH; i++) put(k, i, ld_chunk<HG::HWD, HEAD_NT>(src, c0, (uint32_t)(i * HG::LPR)));
    }
  }
}
template <class S, int WD, int NRB, int NB>
__device__ __forceinline__ void head_prefetch_regs(const DecodeArgs &a, Chunk<WD> (&b)[NB], int lane) {
  using HG = HeadGeo<S, WD>;
  static_assert(NRB * HG::NPH <= NB && (NRB == 0 || WD == HG::HWD), "register batches");
  if constexpr (NRB > 0)
    head_load_rows<S, WD, 0, NRB>(a, [&](int k, int i, const Chunk<WD> &c) { b[k * HG::NPH + i] = c; }, lane);
}

// Output head over this workgroup's contiguous vocabulary rows, RB rows per
// batch: first the rows kept in LDS, then the NRB batches requested into the
// slice registers beforehand (late sets), then the NX batches kept in hx,
// then the rest from memory with three batches in flight, the first three
// requested before the head's input is in.  Memory batches past the last row
// re-read that row, which keeps every load unconditional.  The row results
// (dot products with the gain-scaled input) go to part[]; the control wave
// applies the folded final LayerNorm.  False when the control wave aborted.
template <class S, int WD, int NRB, int NX, int NB>
__device__ bool head_rows(const DecodeArgs &a, float *lds, int lane, const Chunk<WD> (&breg)[NB],
                          const Chunk<HeadGeo<S, WD>::HWD> (&hx)[NX > 0 ? NX : 1][HeadGeo<S, WD>::NPH]) {
  using HG = HeadGeo<S, WD>;
  constexpr int KC = HG::KC, LPR = HG::LPR, NPH = HG::NPH, RB = HG::RB, HWD = HG::HWD;
  const int *flag = reinterpret_cast<const int *>(lds + S::L_FLAG);
  float *part = lds + S::L_PART;
  const float *xs = lds + S::L_XS;
  int hr0, hr1;
  head_range<S, WD>(a.V, (int)blockIdx.x, hr0, hr1);
  const int nr = hr1 - hr0;
  const int nl = min(nr, a.head_lds_rows);
  const int ng = min(nr - nl, (NRB + NX) * RB);  // rows requested into registers beforehand
  const int nc = min(nr - nl - ng, HG::CTL_ROWS);  // the control wave's rows
  const int nh = nr - nl - ng - nc, hb = hr0 + nl + ng + nc;
  const WSrc src = wsrc<HWD>(MatW{a.head, nullptr}, (size_t)hb * KC);
  const int q = lane % LPR, rl = lane / LPR;
  constexpr int HB = S::HEAD_BATCHES;  // batches streamed from memory in flight
  Chunk<HWD> hbuf[HB][NPH];
  auto fetch = [&](Chunk<HWD>(&b)[NPH], int r0) {
    const int r = min(r0 + rl, nh - 1);
    const uint32_t c0 = (uint32_t)(r * KC + q);
#pragma unroll
    for (int i = 0; i < NPH; i++) b[i] = ld_chunk<HWD, HEAD_NT>(src, c0, (uint32_t)(i * LPR));
  };
  if (nh > 0) {
#pragma unroll
    for (int k = 0; k < HB; k++) fetch(hbuf[k], k * RB);
  }
  wg_barrier();
  if (S::ITEM_CW ? (flag[0] | flag[1]) != 0 : flag[0] != 0) return false;
  float4 xv[NPH];
#pragma unroll
  for (int i = 0; i < NPH; i++) xv[i] = reinterpret_cast<const float4 *>(xs)[i * LPR + q];
  auto consume = [&](const Chunk<HWD>(&b)[NPH], int r, int lim) {
    // fp16 head: even and odd chunks in two independent chains (measured
    // faster there; the fp32 head keeps one)
    constexpr int NCH = HWD == WD_F16 ? 2 : 1;
    float ac[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NPH; i++) ac[i % NCH] = dot4(deq<HWD>(b[i]), xv[i], ac[i % NCH]);
    const float acc = seg_sum_last<LPR>(NCH == 2 ? ac[0] + ac[1] : ac[0]);
    if (q == LPR - 1 && r < lim) part[r] = acc;
  };
  const Chunk<HWD> *hl = reinterpret_cast<const Chunk<HWD> *>(lds + S::L_HEAD);
  for (int r0 = 0; r0 < nl; r0 += RB) {
    const int r = min(r0 + rl, nl - 1);
    Chunk<HWD> c[NPH];
#pragma unroll
    for (int i = 0; i < NPH; i++) c[i] = hl[r * KC + q + LPR * i];
    consume(c, r0 + rl, nl);
  }
  if constexpr (NRB > 0) {
#pragma unroll
    for (int k = 0; k < NRB; k++) {
      if (k * RB < ng) {
        Chunk<HWD> c[NPH];
#pragma unroll
        for (int i = 0; i < NPH; i++) c[i] = breg[k * NPH + i];
        consume(c, nl + k * RB + rl, nl + ng);
      }
    }
  }
  if constexpr (NX > 0) {
#pragma unroll
    for (int k = 0; k < NX; k++)
      if ((NRB + k) * RB < ng) consume(hx[k], nl + (NRB + k) * RB + rl, nl + ng);
  }
  if (nh > 0) {
    const int nb = nl + ng + nc;
    for (int r0 = 0; r0 < nh; r0 += HB * RB) {
#pragma unroll
      for (int k = 0; k < HB; k++) {
        consume(hbuf[k], nb + r0 + k * RB + rl, nr);
        fetch(hbuf[k], r0 + (HB + k) * RB);
      }
    }
  }
  wg_barrier();
  return true;
}

// Compute wave lane/64 (< M_PARTS - 1) of a set-M workgroup polls its part of
// the MLP activation into the phase input (right after requesting its slice);
// the control wave polls the last part.  Each wave's poll round covers one
// of the M_PARTS parts (four in the int4 kernel, eight in the eight-wave one),
// so the last part is seen sooner after it lands.  A
// failed wait raises the compute-side abort flag, which every wave reads
// after the next barrier.
template <class S>
__device__ void poll_act_part(const DecodeArgs &a, int step, int l, float *lds, int lane) {
  constexpr int PW = S::F / S::M_PARTS, PER = PW / 64;
  // the wave index is uniform: in a scalar register, the part's buffer
  // resource is too (a per-lane resource would serialise the loads)
  const int wv = __builtin_amdgcn_readfirstlane(lane / 64), wl = lane % 64;
  if (wv >= S::M_PARTS - 1) return;
  Waiter wt{&a, 0, 0, 0u};
  wt.start(5 * l + 3);
  float v[PER];
  const uint64_t *src = a.act_t + ((size_t)l * NCOPY + my_copy()) * S::F + wv * PW;
  if (poll_vec<PER>(src, epoch_of(a, step, 5 * l + 3), v, wl, wt)) {
#pragma unroll
    for (int j = 0; j < PER; j++) lds[S::L_XS + wv * PW + vidx(wl, j)] = v[j];
  } else if (wl == 0) {
    reinterpret_cast<int *>(lds + S::L_FLAG)[1] = 1;
  }
}
// With S::ITEM_CW the six dot waves poll the 768-word input of sets Q, A and
// F at once (set F: in a workgroup without an attention item, else its
// control wave polls it), 128 words each, one pair load per lane per round.
// The part, times the LayerNorm gain where one comes first, goes into the dot
// products' input, and (gain given) the part itself to L_XRAW, from which the
// control wave takes the LayerNorm statistics after the first barrier.
// The input region also holds the workgroup's attention item's value rows
// until the item has read them.  Every element of set Q's and set F's input
// depends on every attention output, so none is complete before that; a part
// of set A's input (two heads) can be, and is written only after the item's
// release word (`release`: that layer's attention epoch; 0: no item).  src:
// the input vector's copy of this XCD; prod: the producing phase.
template <class S>
__device__ void poll_in_part(const DecodeArgs &a, const uint64_t *src, uint32_t ep, int prod, const float *gain,
                             float *lds, int lane, uint32_t release = 0) {
  static_assert(6 * 128 == S::E, "six parts of 128 words");
  const int wv = __builtin_amdgcn_readfirstlane(lane / 64), wl = lane % 64;
  const int e0 = wv * 128 + 2 * wl;
  float g0 = 1.f, g1 = 1.f;
  if (gain) {
    g0 = gain[e0];
    g1 = gain[e0 + 1];
  }
  Waiter wt{&a, 0, 0, 0u};
  wt.start(prod);
  float v[2];
  if (poll_vec<2>(src + wv * 128, ep, v, wl, wt)) {
    // (a bounded wait; it ends early when a wave of the workgroup has failed)
    int *fl = reinterpret_cast<int *>(lds + S::L_FLAG);
    while (release &&
           __hip_atomic_load(fl + 2, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != (int)release) {
      if (__hip_atomic_load(fl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0 || wt.expired()) {
        if (wl == 0) fl[1] = 1;
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    lds[S::L_XS + e0] = v[0] * g0;
    lds[S::L_XS + e0 + 1] = v[1] * g1;
    if (gain) {
      lds[S::L_XRAW + e0] = v[0];
      lds[S::L_XRAW + e0 + 1] = v[1];
    }
  } else if (wl == 0) {
    reinterpret_cast<int *>(lds + S::L_FLAG)[1] = 1;
  }
}

// A workgroup's attention item at one position: head ih, chunk ic, over rows
// t0..t1-1 (cache rows t0..tg-1; last: the chunk closes at the position itself).
struct ItemOf {
  int ih, ic, t0, t1, tg;
  bool last;
};
// The attention item of workgroup w (of set SET) at position p, if it has one;
// nch: the chunks per head at p.
template <class S, int SET>
__device__ __forceinline__ bool item_at(int p, int w, int &nch, ItemOf &it) {
  int ch;
  att_chunks<S>(p, nch, ch);
  const int item = att_item_of<S>(w);
  // (set Q's workgroups come first in blockIdx: they get items only when the
  // other sets cannot hold them all)
  constexpr bool MAY_ITEM = SET != SET_Q || S::H * S::MAXCH > S::G - S::NQ;
  const bool has = MAY_ITEM && item < S::H * nch;
  it.ih = has ? item / nch : 0;
  it.ic = has ? item % nch : 0;
  it.t0 = it.ic * ch;
  it.t1 = min(it.t0 + ch, p + 1);
  it.last = (it.t1 == p + 1);
  it.tg = it.last ? p : it.t1;
  return has;
}

template <bool TR>
__device__ __forceinline__ void stamp_if(const DecodeArgs &a, int lane, int step, int ph, int which, int G) {
  if constexpr (TR) {
    if (lane == 0) stamp(a, step, ph, which, G);
  }
}

// The attention item run by a compute wave (S::ITEM_CW; lane 0..63): the same
// chunk as AttChunk on the control wave, but with the chunk's value rows copied
// straight into LDS (direct global-to-LDS loads) instead of held in registers.
// att_item_fetch requests the chunk's key rows (into k) and value rows (into
// LDS, over the phase input vector; rows past the chunk's cache rows are
// zeros) and waits for none of them.
template <class S>
__device__ __attribute__((always_inline)) void att_item_fetch(const DecodeArgs &a, float *lds, int l, const ItemOf &it,
                                                              int lane, float4 (&k)[S::D / 4], bool keys = true,
                                                              bool values = true) {
  constexpr int D = S::D, H = S::H, D4 = D / 4;
  static_assert(D == 64, "16 pieces of 16 bytes per value row, 4 rows per copy");
  asm volatile("" : "+v"(lane));
  const int ih = it.ih, it0 = it.t0, itg = it.tg;
  const float *K = a.kc + ((size_t)(l * H + ih) * a.P) * D;
  const float *V = a.vc + ((size_t)(l * H + ih) * a.P) * D;
  const int nv = itg - it0;  // cache rows of the chunk
  {
    const int tk = it0 + lane;
    if (keys) {
#pragma unroll
      for (int i = 0; i < D4; i++) {
        k[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tk < itg) k[i] = reinterpret_cast<const float4 *>(K + (size_t)tk * D)[i];
      }
    }
    if (!values) return;
    typedef __attribute__((address_space(1))) void g_void;
    typedef __attribute__((address_space(3))) void l_void;
    const char *src = reinterpret_cast<const char *>(V + (size_t)it0 * D);
    char *dst = reinterpret_cast<char *>(lds + S::L_V);
    // rows past the chunk's cache rows: zeros, so the value loop needs no test
    // (written before the copies are requested: an LDS write after them
    // would first wait for all of them)
#pragma unroll
    for (int j = 0; j < D / 4; j++) {
      const int f = 64 * j + lane;
      if (f >= nv * (D / 4)) reinterpret_cast<float4 *>(dst)[f] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < D / 4; j++) {  // copy j: rows 4j..4j+3, lane = one 16-byte piece
      const int f = 64 * j + lane;
      if (f < nv * (D / 4))
        __builtin_amdgcn_global_load_lds((g_void *)(src + (size_t)f * 16), (l_void *)(dst + 64 * j * 16), 16, 0, 0);
    }
  }
}

// att_item_cw runs the item, with its rows fetched here unless `fetched` (k and
// the LDS rows already hold them).  False when a wait failed (the error word is
// set).
template <class S, bool TR>
__device__ __attribute__((always_inline)) bool att_item_cw(const DecodeArgs &a, float *lds, int step, int l, int p,
                                                           int nch, const ItemOf &it, int lane, Waiter &wt,
                                                           float4 (&k)[S::D / 4], int have) {
  constexpr int E = S::E, D = S::D, H = S::H, D4 = D / 4, RPL = 64 / D4, IT = 64 / RPL;
  // (an opaque copy of the lane index: the item's per-lane addresses are
  // computed where they are used instead of once for the whole launch, where
  // they would hold registers through the head)
  asm volatile("" : "+v"(lane));
  const uint32_t epA = epoch_of(a, step, 5 * l + 0), epB = epA + 1;
  const int ih = it.ih, ic = it.ic, it0 = it.t0, it1 = it.t1, itg = it.tg;
  const bool ilast = it.last;
  if (have != 3) att_item_fetch<S>(a, lds, l, it, lane, k, !(have & 1), !(have & 2));
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
      }
      break;
    }
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  stamp_if<TR>(a, lane, step, 5 * l + 1, 0, S::G);
  // scores (lane = row it0 + lane), softmax weights, as AttChunk::run
  float m, lsum;
  float4 o;
  {
    const int g = lane / D4, d4 = lane % D4;
    const float scale = 1.0f / sqrtf((float)D);
    const float4 *q4 = reinterpret_cast<const float4 *>(lds + S::L_Q);
    float sa = 0.f, sb = 0.f, sc = 0.f, sd = 0.f;
#pragma unroll
    for (int i = 0; i < D4; i += 4) {
      sa = dot4(k[i], q4[i], sa);
      sb = dot4(k[i + 1], q4[i + 1], sb);
      sc = dot4(k[i + 2], q4[i + 2], sc);
      sd = dot4(k[i + 3], q4[i + 3], sd);
    }
    const float sv = ((sa + sb) + (sc + sd)) * scale;
    const bool has_p = itg < it1;
    float sp = -INFINITY;
    float4 vp = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_p) {
      const float4 kp = reinterpret_cast<const float4 *>(lds + S::L_KP)[d4];
      vp = reinterpret_cast<const float4 *>(lds + S::L_VP)[d4];
      sp = seg_bcast_last<D4>(seg_sum_last<D4>(dot4(kp, q4[d4], 0.f)), lane) * scale;
    }
    const bool valid = it0 + lane < itg;
    const bool isp = has_p && lane == p - it0;
    const float sl = valid ? sv : (isp ? sp : -INFINITY);
    m = wave_max_all(sl);
    const float e = (valid || isp) ? __expf(sl - m) : 0.f;
    lsum = wave_sum_all(e);
    lds[S::L_SC + (lane % RPL) * IT + lane / RPL] = e;
    float wgt[IT];
#pragma unroll
    for (int j = 0; j < IT; j += 4) {
      const float4 x = reinterpret_cast<const float4 *>(lds + S::L_SC + g * IT)[j / 4];
      wgt[j] = x.x;
      wgt[j + 1] = x.y;
      wgt[j + 2] = x.z;
      wgt[j + 3] = x.w;
    }
    // the value rows are in LDS (this wave's own copies)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float4 oo = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 *vl = reinterpret_cast<const float4 *>(lds + S::L_V);
    float4 vv[IT];
#pragma unroll
    for (int i2 = 0; i2 < IT; i2++) vv[i2] = vl[(g + RPL * i2) * D4 + d4];
#pragma unroll
    for (int i2 = 0; i2 < IT; i2++) {
      oo.x = __builtin_fmaf(wgt[i2], vv[i2].x, oo.x);
      oo.y = __builtin_fmaf(wgt[i2], vv[i2].y, oo.y);
      oo.z = __builtin_fmaf(wgt[i2], vv[i2].z, oo.z);
      oo.w = __builtin_fmaf(wgt[i2], vv[i2].w, oo.w);
    }
    // all the row reads first, then the products (one LDS round trip, not IT)
    __builtin_amdgcn_sched_group_barrier(0x100, IT, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4 * IT, 0);
    if (has_p && ((p - it0) % RPL) == g) {
      const float ep = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), p - it0));
      oo.x = __builtin_fmaf(ep, vp.x, oo.x);
      oo.y = __builtin_fmaf(ep, vp.y, oo.y);
      oo.z = __builtin_fmaf(ep, vp.z, oo.z);
      oo.w = __builtin_fmaf(ep, vp.w, oo.w);
    }
#pragma unroll
    for (int sh = D4; sh < 64; sh <<= 1) {
      oo.x = xor_sum(oo.x, sh);
      oo.y = xor_sum(oo.y, sh);
      oo.z = xor_sum(oo.z, sh);
      oo.w = xor_sum(oo.w, sh);
    }
    o = oo;
  }
  // the position's cache rows, stored after the value rows' wait above (which
  // would otherwise wait for these stores too); they are complete before this
  // wave reaches the next barrier (the caller's wait)
  if (ilast && lane < D) {
    const size_t row = ((size_t)(l * H + ih) * a.P + p) * D + lane;
    st_agent(a.kc + row, lds[S::L_KP + lane]);
    st_agent(a.vc + row, lds[S::L_VP + lane]);
  }
  stamp_if<TR>(a, lane, step, 5 * l + 1, 1, S::G);
  const int g = lane / D4, d4 = lane % D4;
  stamp_if<TR>(a, lane, step, 5 * l + 1, 2, S::G);
  // every lane holds the head's output; row group g writes the copies c = g mod RPL
  const auto attn_rs = __builtin_amdgcn_make_buffer_rsrc(a.attn_t + (size_t)l * NCOPY * E, (short)0,
                                                         NCOPY * E * 8, 0x00020000);
  auto publish_head = [&](const float4 &r) {
    for (int c = g; c < NCOPY; c += RPL) {
      const uint32_t off = (uint32_t)((c * E + ih * D + 4 * d4) * 8);
      tst2(attn_rs, off, r.x, r.y, epB);
      tst2(attn_rs, off + 16, r.z, r.w, epB);
    }
  };
  // The item's last read of the LDS under the phase input: the workgroup's
  // dot waves of set A may write their part of the phase input from here on
  // (a part is complete once two heads are in, maybe before this one).
  auto release_input = [&]() {
    if (lane == 0)
      __hip_atomic_store(reinterpret_cast<int *>(lds + S::L_FLAG) + 2, (int)epB, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  if (nch == 1) {
    const float rl = __builtin_amdgcn_rcpf(lsum);
    release_input();
    publish_head(make_float4(o.x * rl, o.y * rl, o.z * rl, o.w * rl));
  } else if (ic > 0) {
    release_input();
    // this chunk's (o, m, l) for chunk 0 of the head, as word pairs
    const auto prs = __builtin_amdgcn_make_buffer_rsrc(
        a.att_t + ((size_t)(l * H + ih) * S::MAXCH + ic) * (D + 2), (short)0, (D + 2) * 8, 0x00020000);
    if (g == 0) {
      tst2(prs, (uint32_t)(4 * d4 * 8), o.x, o.y, epB);
      tst2(prs, (uint32_t)((4 * d4 + 2) * 8), o.z, o.w, epB);
    }
    if (lane == 0) tst2(prs, (uint32_t)(D * 8), m, lsum, epB);
  } else {
    // chunk 0 merges the head.  The partials of chunks 1..nch-1 are polled as one
    // flat array of word pairs spread over the lanes (a fixed number of 16-byte
    // loads per lane, clamped, so the wait counts stay exact), staged in LDS (the
    // phase-input area is free while the item runs), and combined: the largest
    // chunk maximum, one rescale factor per chunk (lane c), then the sums in
    // chunk order.
    constexpr int PP = (D + 2) / 2;                       // word pairs per chunk slot
    constexpr int PPL = ((S::MAXCH - 1) * PP + 63) / 64;  // pair loads per lane
    constexpr int SP = D + 4;                             // staged slot stride (16-byte aligned)
    const int npairs = (nch - 1) * PP;
    const auto mrs = __builtin_amdgcn_make_buffer_rsrc(
        a.att_t + ((size_t)(l * H + ih) * S::MAXCH + 1) * (D + 2), (short)0, (S::MAXCH - 1) * (D + 2) * 8,
        0x00020000);
    float va[PPL], vb[PPL];
    wt.start(5 * l + 1);
    while (true) {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < PPL; k++) {
        const int f = min(lane + 64 * k, npairs - 1);
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(mrs, (uint32_t)(f * 16), 0, AUX_SC1);
        va[k] = __uint_as_float(x[0]);
        vb[k] = __uint_as_float(x[2]);
        ok &= (lane + 64 * k >= npairs) || (x[1] == epB && x[3] == epB);
      }
      if (__all(ok)) break;
      if (wt.expired()) return false;
      __builtin_amdgcn_s_sleep(1);
    }
    float *scr = lds + S::L_XS;
#pragma unroll
    for (int k = 0; k < PPL; k++) {
      const int f = lane + 64 * k;
      if (f < npairs) {
        const int w2 = 2 * f, sl = w2 / (D + 2), wi = w2 % (D + 2);
        scr[sl * SP + wi] = va[k];
        scr[sl * SP + wi + 1] = vb[k];
      }
    }
    float mcl = -INFINITY, lcl = 0.f;  // lane c < nch: chunk c's maximum and sum
    if (lane == 0) {
      mcl = m;
      lcl = lsum;
    } else if (lane < nch) {
      mcl = scr[(lane - 1) * SP + D];
      lcl = scr[(lane - 1) * SP + D + 1];
    }
    const float M = wave_max_all(mcl);
    const float fl = lane < nch ? __expf(mcl - M) : 0.f;
    const float Ls = wave_sum_all(lcl * fl);
    const float f0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), 0));
    float4 O = make_float4(o.x * f0, o.y * f0, o.z * f0, o.w * f0);
    for (int c = 1; c < nch; c++) {
      const float fc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), c));
      const float4 oc = reinterpret_cast<const float4 *>(scr + (c - 1) * SP)[d4];
      O.x = __builtin_fmaf(oc.x, fc, O.x);
      O.y = __builtin_fmaf(oc.y, fc, O.y);
      O.z = __builtin_fmaf(oc.z, fc, O.z);
      O.w = __builtin_fmaf(oc.w, fc, O.w);
    }
    const float rl = __builtin_amdgcn_rcpf(Ls);
    release_input();
    publish_head(make_float4(O.x * rl, O.y * rl, O.z * rl, O.w * rl));
  }
  stamp_if<TR>(a, lane, step, 5 * l + 1, 3, S::G);
  return true;
}

// Compute waves of a workgroup of set SET.  Its slice of a layer sits in
// registers from one layer to the next: right after the phase has consumed
// it (and the control wave has issued the phase's stores, third barrier), the
// next layer's slice is requested into the same registers, and has a whole
// layer to arrive.  Sets whose phase comes late in the layer request the next
// step's first slice only after the output head, whose loads it would delay.
template <class S, int WD, int SET, bool TR, bool DOTS>
__device__ __attribute__((always_inline)) void compute_set(const DecodeArgs &a, const MatW &m, float *lds,
                                                           int lane) {
  using ST = Set<S, SET>;
  // sets whose phase is not the first of a layer request the next step's first
  // slice only after the output head; meanwhile their slice registers hold head rows
  constexpr bool LATE = SET != SET_Q;
  constexpr int NRB = head_reg_batches<S, WD, SET>(), NX = head_extra_batches<S, WD, SET>();
  Chunk<HeadGeo<S, WD>::HWD> hx[NX > 0 ? NX : 1][HeadGeo<S, WD>::NPH];
  int *flag = reinterpret_cast<int *>(lds + S::L_FLAG);
  float *part = lds + S::L_PART;
  const float *xs = lds + S::L_XS;
  const int rank = (int)blockIdx.x - ST::FIRST;
  Chunk<WD> b[ST::NB];
  // With S::ITEM_CW, compute wave IW (DOTS false: it holds no slice, takes no
  // dot products and no output-head rows, but passes every barrier and polls
  // its part of the MLP activation) runs the workgroup's attention item: sets
  // A, F and M right before their own phase of the layer, set Q right after
  // its phase (the item reads the QKV outputs).  Sets A and F request the next
  // layer's rows of their item once their own phase is done; set M, whose
  // phase closes the layer and uses that LDS, requests the next layer's key
  // rows right after its item and the value rows at the item.  A failed wait raises
  // the compute-side abort flag, which every wave reads after the next
  // barrier.
  Waiter wt{&a, 0, 0, 0u};
  float4 kpre[S::ITEM_CW && !DOTS ? S::D / 4 : 1];
  int pre = 0;  // this layer's chunk already requested: key rows in kpre (1), value rows in LDS (2)
  auto run_item = [&](int step, int l, int nch, const ItemOf &it) {
    if constexpr (S::ITEM_CW && !DOTS) {
      const int wl = lane % 64;
      if (!att_item_cw<S, TR>(a, lds, step, l, a.pos0 + step, nch, it, wl, wt, kpre, pre) && wl == 0) flag[1] = 1;
      pre = 0;
      // its stores (the outputs, and the cache rows when the chunk closes at
      // the position) are complete before this wave reaches the next barrier
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (SET == SET_M) {
        // the next layer's key rows now (registers; its value rows must wait
        // for the end of this set's phase, which uses their LDS)
        if (l + 1 < a.L) {
          att_item_fetch<S>(a, lds, l + 1, it, wl, kpre, true, false);
          pre = 1;
        }
      }
    }
  };
  auto aborted = [&]() { return S::ITEM_CW ? (flag[0] | flag[1]) != 0 : flag[0] != 0; };
  // A workgroup of set M whose control wave runs an attention item in a step
  // requests each layer's slice only after that item (one more barrier): the
  // slice would otherwise still be streaming in, two phases after its request,
  // when the item reads its K/V rows and polls q/k/v.
  auto defers = [&](int step) {
    return SET == SET_M && step < a.nsteps && has_att_item<S>(a.pos0 + step, (int)blockIdx.x);
  };
  bool defer = defers(0);
  if (DOTS && !defer) load_set<ST, WD>(b, m, 0, rank, lane);
  for (int step = 0; step < a.nsteps; step++) {
    const bool more = step + 1 < a.nsteps;
    const bool defer_next = defers(step + 1);
    // (item wave: an opaque copy of the lane index per step, so that its
    // per-lane addresses are not held in registers for the whole launch)
    if constexpr (!DOTS) asm volatile("" : "+v"(lane));
    int nch = 1;
    ItemOf it{};
    const bool my_item = !DOTS && item_at<S, SET>(a.pos0 + step, (int)blockIdx.x, nch, it);
    // (the dot waves of sets A and F: whether the workgroup's attention wave runs an item)
    const bool wg_item = (SET == SET_A || SET == SET_F) && DOTS && has_att_item<S>(a.pos0 + step, (int)blockIdx.x);
    for (int l = 0; l < a.L; l++) {
      if constexpr (!DOTS && SET != SET_Q) {
        if (my_item) run_item(step, l, nch, it);
      }
      if (defer) {
        wg_barrier();  // the attention item has run
        if (aborted()) return;
        if constexpr (DOTS) load_set<ST, WD>(b, m, l, rank, lane);
      }
      if constexpr (SET == SET_M && S::M_PARTS > 1) poll_act_part<S>(a, step, l, lds, lane);
      if constexpr (S::ITEM_CW && DOTS) {
        // this wave's part of the phase input (sets Q from the second layer on,
        // A, and F without an item; poll_in_part)
        const uint32_t ep0 = epoch_of(a, step, 5 * l + 0);
        const size_t cp = (size_t)my_copy() * S::E;
        if constexpr (SET == SET_Q) {
          if (l > 0)
            poll_in_part<S>(a, a.xb_t + (size_t)(l - 1) * NCOPY * S::E + cp, ep0 - 1, 5 * (l - 1) + 4,
                            a.ln1w + (size_t)l * S::E, lds, lane);
        } else if constexpr (SET == SET_A) {
          poll_in_part<S>(a, a.attn_t + (size_t)l * NCOPY * S::E + cp, ep0 + 1, 5 * l + 1, nullptr, lds, lane,
                          wg_item ? ep0 + 1 : 0u);
        } else if constexpr (SET == SET_F) {
          if (!wg_item)
            poll_in_part<S>(a, a.xa_t + (size_t)l * NCOPY * S::E + cp, ep0 + 2, 5 * l + 2,
                            a.ln2w + (size_t)l * S::E, lds, lane);
        }
      }
      wg_barrier();
      if (flag[0] | flag[1]) return;
      if constexpr (DOTS) dot_set<ST, WD>(b, xs, part, lane);
      wg_barrier();
      wg_barrier();
      if constexpr (S::ITEM_CW && !DOTS && (SET == SET_A || SET == SET_F)) {
        // the next layer's key rows and value rows, requested once this set's
        // phase is done (cache rows of earlier positions; not waited for until
        // that item, this wave's next LDS access)
        if (my_item && l + 1 < a.L) {
          att_item_fetch<S>(a, lds, l + 1, it, lane % 64, kpre);
          pre = 3;
        }
      }
      if constexpr (WD == WD_F16) {
        if (step == 0 && l == 1) wait_head_lds();  // (before the next slice request)
      }
      if (l + 1 < a.L) {
        if (DOTS && !defer) load_set<ST, WD>(b, m, l + 1, rank, lane);
      } else if (more && !LATE) {
        if constexpr (DOTS) load_set<ST, WD>(b, m, 0, rank, lane);
      } else if constexpr (DOTS) {
        head_prefetch_regs<S, WD, NRB>(a, b, lane);  // idle slice registers take head rows
      }
      if (DOTS && step == 0 && l == 0) {
        // output-head rows kept on chip for the launch: in LDS, and in hx
        fill_head_lds<S, WD>(a, lds, lane);
        head_load_rows<S, WD, NRB, NX>(
            a, [&](int k, int i, const Chunk<HeadGeo<S, WD>::HWD> &c) { hx[k][i] = c; }, lane);
        if (WD == WD_F16 && a.L == 1) wait_head_lds();
      }
      if constexpr (!DOTS && SET == SET_Q) {
        if (my_item) run_item(step, l, nch, it);
      }
    }
    if constexpr (DOTS) {
      if (!head_rows<S, WD, NRB, NX>(a, lds, lane, b, hx)) return;
    } else {
      // (the item wave takes no head rows; it passes the head's two barriers)
      wg_barrier();
      if (aborted()) return;
      wg_barrier();
    }
    wg_barrier();  // the control wave has issued the logits and its argmax
    if (DOTS && more && LATE && !defer_next) load_set<ST, WD>(b, m, 0, rank, lane);
    defer = defer_next;
  }
}

template <class S, int WD, bool TR>
__device__ __attribute__((always_inline)) void compute_main(const DecodeArgs &a, float *lds, int lane) {
  const int w = (int)blockIdx.x;
  if constexpr (S::ITEM_CW) {
    if (__builtin_amdgcn_readfirstlane(lane / 64) == S::IW) {
      if (w < Set<S, SET_A>::FIRST) compute_set<S, WD, SET_Q, TR, false>(a, a.qkv, lds, lane);
      else if (w < Set<S, SET_F>::FIRST) compute_set<S, WD, SET_A, TR, false>(a, a.ap, lds, lane);
      else if (w < Set<S, SET_M>::FIRST) compute_set<S, WD, SET_F, TR, false>(a, a.fc, lds, lane);
      else compute_set<S, WD, SET_M, TR, false>(a, a.pr, lds, lane);
      // (on an abort the next layer's rows may still be in flight to LDS)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
  }
  if (w < Set<S, SET_A>::FIRST) compute_set<S, WD, SET_Q, TR, true>(a, a.qkv, lds, lane);
  else if (w < Set<S, SET_F>::FIRST) compute_set<S, WD, SET_A, TR, true>(a, a.ap, lds, lane);
  else if (w < Set<S, SET_M>::FIRST) compute_set<S, WD, SET_F, TR, true>(a, a.fc, lds, lane);
  else compute_set<S, WD, SET_M, TR, true>(a, a.pr, lds, lane);
}

// ---- control wave ----------------------------------------------------------
template <class S>
__device__ __forceinline__ bool reduce_argmax(const DecodeArgs &a, uint32_t ep, int lane, Waiter &wt,
                                              uint32_t &out_idx) {
  constexpr int G = S::G;
  float bv = -INFINITY;
  uint32_t bi = 0xffffffffu;
  // workgroup g's (value, index) word pair is one 16-byte load
  const auto ars = __builtin_amdgcn_make_buffer_rsrc(a.amax_t + (size_t)my_copy() * 2 * G, (short)0, 2 * G * 8,
                                                     0x00020000);
  while (true) {
    bool ok = true;
    float v = -INFINITY;
    uint32_t idx = 0xffffffffu;
#pragma unroll
    for (int g0 = lane; g0 < G; g0 += 64) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(ars, (uint32_t)(g0 * 16), 0, AUX_SC1);
      ok &= (x[1] == ep) && (x[3] == ep);
      const float cv = __uint_as_float(x[0]);
      const uint32_t ci = x[2];
      if (cv > v || (cv == v && ci < idx)) { v = cv; idx = ci; }
    }
    if (__all(ok)) { bv = v; bi = idx; break; }
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  out_idx = wave_argmax(bv, bi);
  return true;
}

// Sampling at temperature T ("Let's make GPT-2 in assembly", Step 7: divide the
// scores by T, softmax, draw): the id whose running sum of the weights
// exp((logit - max)/T), in id order, first exceeds u times their total.
// Workgroup g published its rows' maximum m_g (the argmax pair), the sum s_g
// of exp((logit - m_g)/T) over its rows, and its logits as tagged words.
// Each lane takes PL consecutive workgroups: the sums scaled to the largest
// maximum M, s_g * exp((m_g - M)/T), and a wave prefix sum locate the
// workgroup g* in whose range the threshold falls; then each lane takes 8
// consecutive rows of g*, weights exp((logit - M)/T), and a second prefix sum
// locates the row.  Every reader runs the same code on the same words, so all
// arrive at the same id.  Rounding can leave the running sum a hair short of
// the threshold: then the last workgroup (or row) with a weight is taken.  No
// weight at all (every logit NaN) gives 0xffffffff.
template <class S, int WD>
__device__ bool reduce_sample(const DecodeArgs &a, uint32_t ep, float u, int lane, Waiter &wt, uint32_t &out_idx) {
  constexpr int G = S::G, PL = (G + 63) / 64, RPL = PSTRIDE / 64;
  const float it = a.inv_temp;
  const auto ars = __builtin_amdgcn_make_buffer_rsrc(a.amax_t + (size_t)my_copy() * 2 * G, (short)0, 2 * G * 8,
                                                     0x00020000);
  const auto srs = __builtin_amdgcn_make_buffer_rsrc(a.ssum_t + (size_t)my_copy() * G, (short)0, G * 8, 0x00020000);
  float m[PL], sg[PL];
  while (true) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PL; j++) {
      const int g = min(lane * PL + j, G - 1);
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(ars, (uint32_t)(g * 16), 0, AUX_SC1);
      const auto y = __builtin_amdgcn_raw_buffer_load_b64(srs, (uint32_t)(g * 8), 0, AUX_SC1);
      ok &= (x[1] == ep) && (x[3] == ep) && (y[1] == ep);
      m[j] = __uint_as_float(x[0]);
      sg[j] = __uint_as_float(y[0]);
    }
    if (__all(ok)) break;
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int j = 0; j < PL; j++)
    if (lane * PL + j < G) mloc = fmaxf(mloc, m[j]);
  const float M = wave_max_all(mloc);
  // workgroups: scaled sums, prefix in workgroup order
  float sc[PL], lsum = 0.f;
#pragma unroll
  for (int j = 0; j < PL; j++) {
    const bool valid = lane * PL + j < G && m[j] > -INFINITY;
    sc[j] = valid ? sg[j] * __expf((m[j] - M) * it) : 0.f;
    lsum += sc[j];
  }
  const float incl = seg_sum_last<64>(lsum);  // inclusive prefix over the lanes
  const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
  const float thr = u * total;
  float run = incl - lsum;
  uint32_t cand = 0xffffffffu;
  int lastg = -1;
  float bef[PL];
#pragma unroll
  for (int j = 0; j < PL; j++) {
    bef[j] = run;
    run += sc[j];
    if (sc[j] > 0.f) lastg = lane * PL + j;
    if (cand == 0xffffffffu && run > thr) cand = (uint32_t)(lane * PL + j);
  }
  uint32_t gs = wave_min_u32_all(cand);
  if (gs == 0xffffffffu) {
    const int lg = (int)(~wave_min_u32_all(~(uint32_t)(lastg + 1))) - 1;  // the largest lastg
    if (lg < 0) {
      out_idx = 0xffffffffu;
      return true;
    }
    gs = (uint32_t)lg;
  }
  // the running sum before g*, from the lane that holds it
  float bsel = 0.f;
#pragma unroll
  for (int j = 0; j < PL; j++)
    if ((int)(gs % PL) == j) bsel = bef[j];
  const float thr2 = thr - __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bsel), (int)(gs / PL)));
  // rows of g*: lane L takes rows 8L.. of its range
  int hr0, hr1;
  head_range<S, WD>(a.V, (int)gs, hr0, hr1);
  const int nr = hr1 - hr0;
  const auto lrs = __builtin_amdgcn_make_buffer_rsrc(a.logit_t + hr0, (short)0, PSTRIDE * 8, 0x00020000);
  float lv[RPL];
  while (true) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < RPL; j++) {
      const int r = min(RPL * lane + j, nr - 1);
      const auto y = __builtin_amdgcn_raw_buffer_load_b64(lrs, (uint32_t)(r * 8), 0, AUX_SC1);
      ok &= y[1] == ep;
      lv[j] = __uint_as_float(y[0]);
    }
    if (__all(ok)) break;
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  float wv[RPL], rsum = 0.f;
#pragma unroll
  for (int j = 0; j < RPL; j++) {
    const bool valid = RPL * lane + j < nr && lv[j] == lv[j];
    wv[j] = valid ? __expf((lv[j] - M) * it) : 0.f;
    rsum += wv[j];
  }
  const float rincl = seg_sum_last<64>(rsum);
  float rrun = rincl - rsum;
  uint32_t rc = 0xffffffffu;
  int lastr = -1;
#pragma unroll
  for (int j = 0; j < RPL; j++) {
    rrun += wv[j];
    if (wv[j] > 0.f) lastr = RPL * lane + j;
    if (rc == 0xffffffffu && rrun > thr2) rc = (uint32_t)(RPL * lane + j);
  }
  uint32_t rs = wave_min_u32_all(rc);
  if (rs == 0xffffffffu) {
    const int lr = (int)(~wave_min_u32_all(~(uint32_t)(lastr + 1))) - 1;
    if (lr < 0) {
      out_idx = 0xffffffffu;
      return true;
    }
    rs = (uint32_t)lr;
  }
  out_idx = (uint32_t)hr0 + rs;
  return true;
}

// The id chosen at step `st` (its logits complete with epoch ep): sampled
// from the run's draws when the run samples and the id is recorded, else the
// argmax.
template <class S, int WD>
__device__ __forceinline__ bool choose_token(const DecodeArgs &a, int st, int lane, Waiter &wt, uint32_t &out) {
  const uint32_t ep = epoch_of(a, st, 5 * a.L);
  if (a.inv_temp > 0.f && st >= a.out_from) return reduce_sample<S, WD>(a, ep, a.draws[st - a.out_from], lane, wt, out);
  return reduce_argmax<S>(a, ep, lane, wt, out);
}

// One attention chunk of head h over positions t0..t1-1 on the control wave,
// following the model file's decode attention: scores q.k * (1/sqrt(D)),
// minus their maximum, exponentials; the chunk's (o = sum e_t v_t, m = max,
// l = sum e_t).  Row p (the current position) comes from LDS, the others from
// the cache.  Scores: lane t holds the whole key row t0 + t and forms its
// score alone, against the query read from LDS (every lane the same
// addresses).  Values: lane (g, d4) holds rows t0 + g + RPL*it, dimensions
// 4*d4..4*d4+3; the weights reach it through LDS, and the RPL row groups are
// combined by row exchanges.  No cross-lane reduction on the score side.
template <class S>
struct AttChunk {
  static constexpr int D = S::D, D4 = D / 4, RPL = 64 / D4, IT = 64 / RPL;
  float4 k[D4], v[IT];
  __device__ void fetch(const DecodeArgs &a, int l, int h, int t0, int tg, int lane) {
    const float *K = a.kc + ((size_t)(l * S::H + h) * a.P) * D;
    const float *V = a.vc + ((size_t)(l * S::H + h) * a.P) * D;
    const int g = lane / D4, d4 = lane % D4;
    const int tk = t0 + lane;
#pragma unroll
    for (int i = 0; i < D4; i++) {
      k[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tk < tg) k[i] = reinterpret_cast<const float4 *>(K + (size_t)tk * D)[i];
    }
#pragma unroll
    for (int it = 0; it < IT; it++) {
      const int t = t0 + g + RPL * it;
      v[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < tg) v[it] = reinterpret_cast<const float4 *>(V + (size_t)t * D)[d4];
    }
  }
  // The chunk's m, lsum and o (dims 4*d4..4*d4+3, summed over all its rows)
  // in every lane.
  __device__ void run(float *lds, int p, int t0, int t1, int tg, int lane, float &m, float &lsum, float4 &o) {
    const int g = lane / D4, d4 = lane % D4;
    const float scale = 1.0f / sqrtf((float)D);
    const float4 *q4 = reinterpret_cast<const float4 *>(lds + S::L_Q);
    // four partial sums: shorter dependency chains
    float sa = 0.f, sb = 0.f, sc = 0.f, sd = 0.f;
#pragma unroll
    for (int i = 0; i < D4; i += 4) {
      sa = dot4(k[i], q4[i], sa);
      sb = dot4(k[i + 1], q4[i + 1], sb);
      sc = dot4(k[i + 2], q4[i + 2], sc);
      sd = dot4(k[i + 3], q4[i + 3], sd);
    }
    const float s = ((sa + sb) + (sc + sd)) * scale;  // row t0 + lane
    const bool has_p = tg < t1;                        // this position closes the chunk
    float sp = -INFINITY;
    float4 vp = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_p) {
      const float4 kp = reinterpret_cast<const float4 *>(lds + S::L_KP)[d4];
      vp = reinterpret_cast<const float4 *>(lds + S::L_VP)[d4];
      sp = seg_bcast_last<D4>(seg_sum_last<D4>(dot4(kp, q4[d4], 0.f)), lane) * scale;
    }
    const bool valid = t0 + lane < tg;
    const bool isp = has_p && lane == p - t0;
    const float sl = valid ? s : (isp ? sp : -INFINITY);
    m = wave_max_all(sl);
    const float e = (valid || isp) ? __expf(sl - m) : 0.f;
    lsum = wave_sum_all(e);
    // the weights, transposed for the value side: row t = g' + RPL*it' at g'*IT + it'
    lds[S::L_SC + (lane % RPL) * IT + lane / RPL] = e;
    float w[IT];
#pragma unroll
    for (int j = 0; j < IT; j += 4) {
      const float4 x = reinterpret_cast<const float4 *>(lds + S::L_SC + g * IT)[j / 4];
      w[j] = x.x;
      w[j + 1] = x.y;
      w[j + 2] = x.z;
      w[j + 3] = x.w;
    }
    float4 oo = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int it = 0; it < IT; it++) {
      oo.x = __builtin_fmaf(w[it], v[it].x, oo.x);
      oo.y = __builtin_fmaf(w[it], v[it].y, oo.y);
      oo.z = __builtin_fmaf(w[it], v[it].z, oo.z);
      oo.w = __builtin_fmaf(w[it], v[it].w, oo.w);
    }
    if (has_p && ((p - t0) % RPL) == g) {
      const float ep = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), p - t0));
      oo.x = __builtin_fmaf(ep, vp.x, oo.x);
      oo.y = __builtin_fmaf(ep, vp.y, oo.y);
      oo.z = __builtin_fmaf(ep, vp.z, oo.z);
      oo.w = __builtin_fmaf(ep, vp.w, oo.w);
    }
#pragma unroll
    for (int sh = D4; sh < 64; sh <<= 1) {
      oo.x = xor_sum(oo.x, sh);
      oo.y = xor_sum(oo.y, sh);
      oo.z = xor_sum(oo.z, sh);
      oo.w = xor_sum(oo.w, sh);
    }
    o = oo;
  }
};

// One tagged word per lane (lanes < n) until it carries ep; v is its payload.
__device__ bool poll_rows(const uint64_t *src, int n, uint32_t ep, float &v, int lane, Waiter &wt) {
  while (true) {
    bool ok = true;
    if (lane < n) {
      const uint64_t x = tld(src + lane);
      v = payload(x);
      ok = tag_is(x, ep);
    }
    if (__all(ok)) return true;
    if (wt.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Control wave.  Per layer it runs the phase of its workgroup's set, and the
// attention chunk if one is assigned to this workgroup:
//   set Q: A  LayerNorm 1 of the residual stream, QKV rows + bias
//   any  : B  one attention chunk (items go to the workgroups after set Q)
//   set A: C  attention projection rows + bias + residual
//   set F: D  LayerNorm 2, fc rows + bias, gelu_new
//   set M: E  MLP projection rows + bias + residual
// and with all workgroups H, the final LayerNorm and the output head.  The
// residual rows a set adds come back from the published vectors (the values
// written are the values read), so no workgroup carries state across phases.
template <class S, int WD, bool TR, int SET>
__device__ __attribute__((always_inline)) void control_set(const DecodeArgs &a, float *lds, int lane) {
  constexpr int E = S::E, F = S::F, D = S::D, H = S::H, G = S::G;
  constexpr int PE = E / 64, D4 = D / 4;
  using SQ = Set<S, SET_Q>;
  using SA = Set<S, SET_A>;
  using SF = Set<S, SET_F>;
  using SM = Set<S, SET_M>;
  const int w = blockIdx.x;
  // (one instantiation per set: the other sets' phases compile away)
  constexpr int set = SET;
  const int rank = w - Set<S, SET>::FIRST;
  int *flag = reinterpret_cast<int *>(lds + S::L_FLAG);
  float *xs = lds + S::L_XS;
  const float *part = lds + S::L_PART;
  int tok = 0;
  Waiter wt{&a, 0, 0, 0u};
  auto st = [&](int step, int ph, int which) {
    if constexpr (TR) {
      if (lane == 0) stamp(a, step, ph, which, G);
    }
  };
  // Parameters of the set's next phase are requested right after its phase,
  // a whole layer before use: for row rank*R + lane the bias (sets A, M) or
  // the folded LayerNorm's row constants (sets Q, F: w.g, and w.h + bias),
  // and the LayerNorm 1 (set Q) or 2 (set F) gain; the final LayerNorm gain is
  // read once.  With a slice share (S::CD), which needs the registers, the
  // LayerNorm-2 and final gains are requested instead as their phase's input
  // is polled.
  float g[PE], gf[PE];
  float bias = 0.f, wg = 0.f;
  auto fetch_gain = [&](float (&gg)[PE], const float *gs) {
#pragma unroll
    for (int j = 0; j < PE; j++) gg[j] = gs[vidx(lane, j)];
  };
  auto fetch_params = [&](int l) {
    if (set == SET_Q) fetch_gain(g, a.ln1w + l * E);
    if constexpr (!S::CD) {
      if (set == SET_F) fetch_gain(g, a.ln2w + l * E);
    }
    // row constants: one pair of loads whatever the set (sets A, M: w.g unused)
    const int R = set == SET_Q ? SQ::R : set == SET_A ? SA::R : set == SET_F ? SF::R : SM::R;
    const size_t o = (size_t)l * (set == SET_Q ? 3 * E : set == SET_F ? F : E) + rank * R + min(lane, R - 1);
    const float *cs = set == SET_Q ? a.cqkv : set == SET_A ? a.bap : set == SET_F ? a.cfc : a.bpr;
    const float *gs = set == SET_Q ? a.gqkv : set == SET_F ? a.gfc : cs;
    bias = cs[o];
    wg = gs[o];
  };
  if constexpr (!S::CD) fetch_gain(gf, a.lnfw);
  fetch_params(0);
  // This wave's share of its set's slice (lanes NL.. of the slice geometry),
  // requested and used like the compute waves' (see compute_set): consumed
  // between the phase's first two barriers, the next layer's requested after
  // the third (set M: after this step's attention item, if it has one; sets
  // other than Q: the next step's first slice after the head).
  constexpr int CBN = S::CD ? (SF::NB > SQ::NB ? (SF::NB > SM::NB ? SF::NB : SM::NB)
                                               : (SQ::NB > SM::NB ? SQ::NB : SM::NB))
                            : 1;
  Chunk<WD> cb[CBN > SA::NB || !S::CD ? CBN : SA::NB];
  auto ctl_load = [&](int layer) {
    if constexpr (S::CD) {
      const int cl = S::NLD - 64 + lane;
      if (set == SET_Q) load_set<SQ, WD>(*reinterpret_cast<Chunk<WD>(*)[SQ::NB]>(cb), a.qkv, layer, rank, cl);
      else if (set == SET_A) load_set<SA, WD>(*reinterpret_cast<Chunk<WD>(*)[SA::NB]>(cb), a.ap, layer, rank, cl);
      else if (set == SET_F) load_set<SF, WD>(*reinterpret_cast<Chunk<WD>(*)[SF::NB]>(cb), a.fc, layer, rank, cl);
      else load_set<SM, WD>(*reinterpret_cast<Chunk<WD>(*)[SM::NB]>(cb), a.pr, layer, rank, cl);
    }
  };
  auto ctl_dot = [&]() {
    if constexpr (S::CD) {
      const int cl = S::NLD - 64 + lane;
      float *pt = lds + S::L_PART;
      if (set == SET_Q) dot_set<SQ, WD>(*reinterpret_cast<Chunk<WD>(*)[SQ::NB]>(cb), xs, pt, cl);
      else if (set == SET_A) dot_set<SA, WD>(*reinterpret_cast<Chunk<WD>(*)[SA::NB]>(cb), xs, pt, cl);
      else if (set == SET_F) dot_set<SF, WD>(*reinterpret_cast<Chunk<WD>(*)[SF::NB]>(cb), xs, pt, cl);
      else dot_set<SM, WD>(*reinterpret_cast<Chunk<WD>(*)[SM::NB]>(cb), xs, pt, cl);
    }
  };
  auto defers = [&](int st) { return set == SET_M && st < a.nsteps && has_att_item<S>(a.pos0 + st, w); };
  int cur_step = 0;
  auto ctl_after_phase = [&](int l) {
    if (l + 1 < a.L) {
      if (!defers(cur_step)) ctl_load(l + 1);
    } else if (cur_step + 1 < a.nsteps && set == SET_Q) {
      ctl_load(0);
    }
  };
  if (!defers(0)) ctl_load(0);
  // Output-head rows kept in this wave's registers for the launch (after the
  // workgroup's LDS and compute-wave register rows), requested once.
  using HG = HeadGeo<S, WD>;
  constexpr int NXC = S::HEAD_CTL_BATCHES;
  Chunk<HG::HWD> cx[NXC > 0 ? NXC : 1][HG::NPH];
  int hc_first = 0, hc_n = 0;  // this wave's first row in the workgroup's range, and how many
  if constexpr (NXC > 0) {
    int r0, r1;
    head_range<S, WD>(a.V, w, r0, r1);
    const int nr = r1 - r0, nl = min(nr, a.head_lds_rows);
    const int ng = min(nr - nl, head_reg_total<S, WD, SET>() * HG::RB);
    hc_first = nl + ng;
    hc_n = min(nr - hc_first, HG::CTL_ROWS);
    if (hc_n > 0) {
      const WSrc src = wsrc<HG::HWD>(MatW{a.head, nullptr}, (size_t)r0 * HG::KC);
      const int q = lane % HG::LPR, rl = lane / HG::LPR;
#pragma unroll
      for (int k = 0; k < NXC; k++) {
        const int r = hc_first + min(k * HG::RBC + rl, hc_n - 1);
#pragma unroll
        for (int i = 0; i < HG::NPH; i++)
          cx[k][i] = ld_chunk<HG::HWD, HEAD_NT>(src, (uint32_t)(r * HG::KC + q), (uint32_t)(i * HG::LPR));
      }
    }
  }
  auto abort_all = [&]() {
    if (lane == 0) flag[0] = 1;
    wg_barrier();
  };
  const bool needs_tok = (set == SET_Q || set == SET_A);
  // Set Q: the embedding input of the next step when its token is fed (known
  // ahead), requested during this step's head.
  float xn[PE];
#pragma unroll
  for (int j = 0; j < PE; j++) xn[j] = 0.f;
  // Token of each step: fed, or the argmax of the previous step.  While the
  // tokens are fed, the previous step's argmax is waited for only where an id
  // is recorded, so the first layer of a fed step can start while the
  // previous step's head is still running elsewhere.
  const int argmax_from = max(1, w == 0 ? min(a.n_feed, a.out_from + 1) : a.n_feed);
  for (int step = 0; step < a.nsteps; step++) {
    const int p = a.pos0 + step;
    cur_step = step;
    if (step < a.n_feed) tok = fed_token(a, step);
    if (needs_tok && step >= argmax_from) {
      uint32_t bi = 0;
      wt.start(5 * a.L);
      if (!choose_token<S, WD>(a, step - 1, lane, wt, bi)) { abort_all(); return; }
      if (w == 0 && lane == 0 && step - 1 >= a.out_from) a.out_ids[step - 1 - a.out_from] = (int)bi;
      if (step >= a.n_feed) {
        // a step whose logits are all NaN names no row: the run stops with an error
        if (bi >= (uint32_t)a.V) {
          raise_error(a, ERR_NO_ARGMAX, 5 * a.L, step - 1);
          abort_all();
          return;
        }
        tok = (int)bi;
      }
    }
    int nch, ch;
    att_chunks<S>(p, nch, ch);
    const int item = att_item_of<S>(w);
    // (set Q's workgroups come first in blockIdx: they get items only when the
    // other sets cannot hold them all)
    constexpr bool MAY_ITEM = set != SET_Q || S::H * S::MAXCH > G - S::NQ;
    const bool has_item = MAY_ITEM && item < H * nch;
    const int ih = has_item ? item / nch : 0, ic = has_item ? item % nch : 0;
    const int it0 = ic * ch, it1 = min(it0 + ch, p + 1);
    const bool ilast = (it1 == p + 1);
    const int itg = ilast ? p : it1;  // cache rows it0..itg-1
    for (int l = 0; l < a.L; l++) {
      // (with a slice share: an opaque copy of the lane index, so that per-lane
      // addresses are recomputed in each layer instead of being hoisted out of
      // the loop and held in registers)
      if constexpr (S::CD) asm volatile("" : "+v"(lane));
      const uint32_t epA = epoch_of(a, step, 5 * l + 0), epB = epA + 1, epC = epA + 2, epD = epA + 3,
                     epE = epA + 4;
      const int lnext = l + 1 < a.L ? l + 1 : 0;
      // ---------------- A: LayerNorm 1 + QKV (set Q)
      if (set == SET_Q) {
        float x[PE];
        if (l == 0 && step > 0 && step < a.n_feed) {
#pragma unroll
          for (int j = 0; j < PE; j++) x[j] = xn[j];
        } else if (l == 0) {
#pragma unroll
          for (int j = 0; j < PE; j++)
            x[j] = a.wte[(size_t)tok * E + vidx(lane, j)] + a.wpe[(size_t)p * E + vidx(lane, j)];
        } else if constexpr (!S::ITEM_CW) {
          wt.start(5 * (l - 1) + 4);
          if (!poll_vec<PE>(a.xb_t + ((size_t)(l - 1) * NCOPY + my_copy()) * E, epA - 1, x, lane, wt)) {
            abort_all();
            return;
          }
        }
        if (!S::ITEM_CW || l == 0) gain_to_lds<E>(x, g, xs, lane);  // (else the dot waves poll it)
        st(step, 5 * l + 0, 0);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (S::ITEM_CW && flag[1]) return;  // a compute wave's wait failed (the error word is set)
        st(step, 5 * l + 0, 1);
        if constexpr (S::ITEM_CW) {
          if (l > 0) {
#pragma unroll
            for (int j = 0; j < PE; j++) x[j] = lds[S::L_XRAW + vidx(lane, j)];
          }
        }
        float mean, rstd;
        ln_stats<E>(x, a.eps, mean, rstd);  // (while the dot products run)
        ctl_dot();
        wg_barrier();
        st(step, 5 * l + 0, 2);
        if (lane < SQ::R)
          tst_pairs(copies_rsrc(a.qkv_t + (size_t)l * NCOPY * 3 * E, 3 * E), 3 * E, rank * SQ::R + lane,
                    ln_row(part[lane], mean, rstd, wg, bias), epA, lane);
        st(step, 5 * l + 0, 3);
        wg_barrier();  // stores issued: the compute waves may request the next slice
        fetch_params(lnext);
        ctl_after_phase(l);
      }
      // ---------------- B: attention chunk (this wave; with S::ITEM_CW a compute wave)
      if (has_item && !S::ITEM_CW) {
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
        st(step, 5 * l + 1, 0);
        float m, lsum;
        float4 o;
        at.run(lds, p, it0, it1, itg, lane, m, lsum, o);
        st(step, 5 * l + 1, 1);
        // The cache-row stores need no wait here: the next poll of this wave
        // (its own set's phase, or the output head) waits for all of its
        // outstanding memory operations, stores included, before this
        // workgroup publishes again, and every reader of row p runs at a
        // later step, after that publish.
        const int g = lane / D4, d4 = lane % D4;
        st(step, 5 * l + 1, 2);
        // every lane holds the head's output; row group g writes the copies c = g mod RPL
        const auto attn_rs = __builtin_amdgcn_make_buffer_rsrc(a.attn_t + (size_t)l * NCOPY * E, (short)0,
                                                               NCOPY * E * 8, 0x00020000);
        auto publish_head = [&](const float4 &r) {
          for (int c = g; c < NCOPY; c += AttChunk<S>::RPL) {
            const uint32_t off = (uint32_t)((c * E + ih * D + 4 * d4) * 8);
            tst2(attn_rs, off, r.x, r.y, epB);
            tst2(attn_rs, off + 16, r.z, r.w, epB);
          }
        };
        if (nch == 1) {
          const float rl = __builtin_amdgcn_rcpf(lsum);
          publish_head(make_float4(o.x * rl, o.y * rl, o.z * rl, o.w * rl));
        } else if (ic > 0) {
          // this chunk's (o, m, l) for chunk 0 of the head, as word pairs
          const auto prs = __builtin_amdgcn_make_buffer_rsrc(
              a.att_t + ((size_t)(l * H + ih) * S::MAXCH + ic) * (D + 2), (short)0, (D + 2) * 8, 0x00020000);
          if (g == 0) {
            tst2(prs, (uint32_t)(4 * d4 * 8), o.x, o.y, epB);
            tst2(prs, (uint32_t)((4 * d4 + 2) * 8), o.z, o.w, epB);
          }
          if (lane == 0) tst2(prs, (uint32_t)(D * 8), m, lsum, epB);
        } else {
          // chunk 0 merges the head.  The partials of chunks 1..nch-1 are polled as one
          // flat array of word pairs spread over the lanes (a fixed number of 16-byte
          // loads per lane, clamped, so the wait counts stay exact), staged in LDS (the
          // phase-input area is free while the item runs), and combined: the largest
          // chunk maximum, one rescale factor per chunk (lane c), then the sums in
          // chunk order.
          constexpr int PP = (D + 2) / 2;                       // word pairs per chunk slot
          constexpr int PPL = ((S::MAXCH - 1) * PP + 63) / 64;  // pair loads per lane
          constexpr int SP = D + 4;                             // staged slot stride (16-byte aligned)
          const int npairs = (nch - 1) * PP;
          const auto mrs = __builtin_amdgcn_make_buffer_rsrc(
              a.att_t + ((size_t)(l * H + ih) * S::MAXCH + 1) * (D + 2), (short)0, (S::MAXCH - 1) * (D + 2) * 8,
              0x00020000);
          float va[PPL], vb[PPL];
          wt.start(5 * l + 1);
          while (true) {
            bool ok = true;
#pragma unroll
            for (int k = 0; k < PPL; k++) {
              const int f = min(lane + 64 * k, npairs - 1);
              const auto x = __builtin_amdgcn_raw_buffer_load_b128(mrs, (uint32_t)(f * 16), 0, AUX_SC1);
              va[k] = __uint_as_float(x[0]);
              vb[k] = __uint_as_float(x[2]);
              ok &= (lane + 64 * k >= npairs) || (x[1] == epB && x[3] == epB);
            }
            if (__all(ok)) break;
            if (wt.expired()) { abort_all(); return; }
            __builtin_amdgcn_s_sleep(1);
          }
          float *scr = lds + S::L_XS;
#pragma unroll
          for (int k = 0; k < PPL; k++) {
            const int f = lane + 64 * k;
            if (f < npairs) {
              const int w2 = 2 * f, sl = w2 / (D + 2), wi = w2 % (D + 2);
              scr[sl * SP + wi] = va[k];
              scr[sl * SP + wi + 1] = vb[k];
            }
          }
          float mcl = -INFINITY, lcl = 0.f;  // lane c < nch: chunk c's maximum and sum
          if (lane == 0) {
            mcl = m;
            lcl = lsum;
          } else if (lane < nch) {
            mcl = scr[(lane - 1) * SP + D];
            lcl = scr[(lane - 1) * SP + D + 1];
          }
          const float M = wave_max_all(mcl);
          const float fl = lane < nch ? __expf(mcl - M) : 0.f;
          const float Ls = wave_sum_all(lcl * fl);
          const float f0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), 0));
          float4 O = make_float4(o.x * f0, o.y * f0, o.z * f0, o.w * f0);
          for (int c = 1; c < nch; c++) {
            const float fc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), c));
            const float4 oc = reinterpret_cast<const float4 *>(scr + (c - 1) * SP)[d4];
            O.x = __builtin_fmaf(oc.x, fc, O.x);
            O.y = __builtin_fmaf(oc.y, fc, O.y);
            O.z = __builtin_fmaf(oc.z, fc, O.z);
            O.w = __builtin_fmaf(oc.w, fc, O.w);
          }
          const float rl = __builtin_amdgcn_rcpf(Ls);
          publish_head(make_float4(O.x * rl, O.y * rl, O.z * rl, O.w * rl));
        }
        st(step, 5 * l + 1, 3);
        if (set == SET_M) {
          wg_barrier();  // the compute waves may now request this layer's slice
          ctl_load(l);   // and so may this wave
        }
      }
      if (S::ITEM_CW && has_item && set == SET_M) {
        wg_barrier();  // a compute wave has run the item: the slices may now be requested
        if (flag[1]) return;  // the item's wave failed (the error word is set)
        ctl_load(l);
      }
      // ---------------- C: attention projection + residual (set A)
      if (set == SET_A) {
        float xr = 0.f;  // residual stream row rank*R + lane
        if (l == 0) {
          if (lane < SA::R) {
            const int o = rank * SA::R + lane;
            xr = a.wte[(size_t)tok * E + o] + a.wpe[(size_t)p * E + o];
          }
        } else {
          wt.start(5 * (l - 1) + 4);
          if (!poll_rows(a.xb_t + ((size_t)(l - 1) * NCOPY + my_copy()) * E + rank * SA::R, SA::R, epA - 1, xr,
                         lane, wt)) {
            abort_all();
            return;
          }
        }
        if constexpr (!S::ITEM_CW) {  // (else the dot waves poll it)
          float x[PE];
          wt.start(5 * l + 1);
          if (!poll_vec<PE>(a.attn_t + ((size_t)l * NCOPY + my_copy()) * E, epB, x, lane, wt)) {
            abort_all();
            return;
          }
#pragma unroll
          for (int j = 0; j < PE; j++) xs[vidx(lane, j)] = x[j];
        }
        st(step, 5 * l + 2, 0);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (S::ITEM_CW && flag[1]) return;  // a compute wave's wait failed (the error word is set)
        st(step, 5 * l + 2, 1);
        ctl_dot();
        wg_barrier();
        st(step, 5 * l + 2, 2);
        if (lane < SA::R) {
          const float mix = part[lane] + bias;
          tst_pairs(copies_rsrc(a.xa_t + (size_t)l * NCOPY * E, E), E, rank * SA::R + lane, xr + mix, epC, lane);
        }
        st(step, 5 * l + 2, 3);
        wg_barrier();  // stores issued: the compute waves may request the next slice
        fetch_params(lnext);
        ctl_after_phase(l);
      }
      // ---------------- D: LayerNorm 2 + fc + gelu_new (set F)
      if (set == SET_F) {
        if constexpr (S::CD) fetch_gain(g, a.ln2w + l * E);  // (arrives during the poll)
        float x[PE];
        if (!S::ITEM_CW || has_item) {  // (else the dot waves poll it)
          wt.start(5 * l + 2);
          if (!poll_vec<PE>(a.xa_t + ((size_t)l * NCOPY + my_copy()) * E, epC, x, lane, wt)) {
            abort_all();
            return;
          }
          gain_to_lds<E>(x, g, xs, lane);
        }
        st(step, 5 * l + 3, 0);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (S::ITEM_CW && flag[1]) return;  // a compute wave's wait failed (the error word is set)
        st(step, 5 * l + 3, 1);
        if (S::ITEM_CW && !has_item) {
#pragma unroll
          for (int j = 0; j < PE; j++) x[j] = lds[S::L_XRAW + vidx(lane, j)];
        }
        float mean, rstd;
        ln_stats<E>(x, a.eps, mean, rstd);  // (while the dot products run)
        ctl_dot();
        wg_barrier();
        st(step, 5 * l + 3, 2);
        if (lane < SF::R)
          tst_pairs(copies_rsrc(a.act_t + (size_t)l * NCOPY * F, F), F, rank * SF::R + lane,
                    gelu_new(ln_row(part[lane], mean, rstd, wg, bias)), epD, lane);
        st(step, 5 * l + 3, 3);
        wg_barrier();  // stores issued: the compute waves may request the next slice
        fetch_params(lnext);
        ctl_after_phase(l);
      }
      // ---------------- E: MLP projection + residual (set M)
      if (set == SET_M) {
        float xr = 0.f;
        wt.start(5 * l + 2);
        if (!poll_rows(a.xa_t + ((size_t)l * NCOPY + my_copy()) * E + rank * SM::R, SM::R, epC, xr, lane, wt)) {
          abort_all();
          return;
        }
        constexpr int PW = F / S::M_PARTS, PP = PW / 64;  // this wave's part of the activation
        float x[PP];
        wt.start(5 * l + 3);
        if (!poll_vec<PP>(a.act_t + ((size_t)l * NCOPY + my_copy()) * F + (S::M_PARTS - 1) * PW, epD, x, lane,
                          wt)) {
          abort_all();
          return;
        }
#pragma unroll
        for (int j = 0; j < PP; j++) xs[(S::M_PARTS - 1) * PW + vidx(lane, j)] = x[j];
        st(step, 5 * l + 4, 0);
        if (lane == 0) flag[0] = 0;
        wg_barrier();
        if (flag[1]) return;  // a compute wave's wait failed (the error word is set)
        st(step, 5 * l + 4, 1);
        ctl_dot();
        wg_barrier();
        st(step, 5 * l + 4, 2);
        if (lane < SM::R) {
          const float mix = part[lane] + bias;
          tst_pairs(copies_rsrc(a.xb_t + (size_t)l * NCOPY * E, E), E, rank * SM::R + lane, xr + mix, epE, lane);
        }
        st(step, 5 * l + 4, 3);
        wg_barrier();  // stores issued: the compute waves may request the next slice
        fetch_params(lnext);
        ctl_after_phase(l);
      }
    }
    // ---------------- H: final LayerNorm + head + local argmax
    {
      const uint32_t epH = epoch_of(a, step, 5 * a.L);
      if constexpr (S::CD) fetch_gain(gf, a.lnfw);  // (arrives while the input is polled)
      if (set == SET_Q && step + 1 < a.n_feed && step + 1 < a.nsteps) {
        const int tn = fed_token(a, step + 1);
#pragma unroll
        for (int j = 0; j < PE; j++)
          xn[j] = a.wte[(size_t)tn * E + vidx(lane, j)] + a.wpe[(size_t)(p + 1) * E + vidx(lane, j)];
      }
      float x[PE];
      wt.start(5 * a.L - 1);
      if (!poll_vec<PE>(a.xb_t + ((size_t)(a.L - 1) * NCOPY + my_copy()) * E, epH - 1, x, lane, wt)) {
        abort_all();
        return;
      }
      gain_to_lds<E>(x, gf, xs, lane);
      st(step, 5 * a.L, 0);
      if (lane == 0) flag[0] = 0;
      wg_barrier();
      if (S::ITEM_CW && flag[1]) return;  // the attention item's wave failed
      st(step, 5 * a.L, 1);
      // while the head's dot products run: the statistics, and the folded
      // LayerNorm's constants of this workgroup's rows
      int hr0, hr1;
      head_range<S, WD>(a.V, w, hr0, hr1);
      const int nr = hr1 - hr0;
      float hg[PSTRIDE / 64], hc[PSTRIDE / 64];
#pragma unroll
      for (int k = 0; k < PSTRIDE / 64; k++) {
        const int r = min(lane + 64 * k, nr - 1);
        hg[k] = a.ghead[hr0 + r];
        hc[k] = a.chead[hr0 + r];
      }
      float mean, rstd;
      ln_stats<E>(x, a.eps, mean, rstd);
      // this wave's own head rows, while the compute waves take theirs
      if constexpr (NXC > 0) {
        if (hc_n > 0) {
          const int q = lane % HG::LPR, rl = lane / HG::LPR;
          float4 xv[HG::NPH];
#pragma unroll
          for (int i = 0; i < HG::NPH; i++) xv[i] = reinterpret_cast<const float4 *>(xs)[i * HG::LPR + q];
#pragma unroll
          for (int k = 0; k < NXC; k++) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < HG::NPH; i++) acc = dot4(deq<HG::HWD>(cx[k][i]), xv[i], acc);
            acc = seg_sum_last<HG::LPR>(acc);
            if (q == HG::LPR - 1 && k * HG::RBC + rl < hc_n) lds[S::L_PART + hc_first + k * HG::RBC + rl] = acc;
          }
        }
      }
      wg_barrier();
      st(step, 5 * a.L, 2);
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      float vv[PSTRIDE / 64];  // this lane's logits (for sampling)
      // (a fixed trip count, so that the row results are read from LDS in one burst)
#pragma unroll
      for (int k = 0; k < PSTRIDE / 64; k++) {
        const int r = lane + 64 * k;
        vv[k] = 0.f;
        if (r < nr) {
          const float v = ln_row(part[r], mean, rstd, hg[k], hc[k]);
          vv[k] = v;
          a.logits[hr0 + r] = v;
          if (v > bv || (v == bv && (uint32_t)(hr0 + r) < bi)) {
            bv = v;
            bi = (uint32_t)(hr0 + r);
          }
        }
      }
      bi = wave_argmax(bv, bi, &bv);
      if (a.inv_temp > 0.f && step >= a.out_from) {
        // sampling: the sum of exp((logit - max)/T) over these rows, with the
        // maximum (the argmax pair below), and the logits as tagged words
        float ssum = 0.f;
#pragma unroll
        for (int k = 0; k < PSTRIDE / 64; k++) {
          const int r = lane + 64 * k;
          if (r < nr) {
            if (vv[k] == vv[k] && bv > -INFINITY) ssum += __expf((vv[k] - bv) * a.inv_temp);
            __hip_atomic_store(a.logit_t + hr0 + r, (uint64_t)__float_as_uint(vv[k]) | ((uint64_t)epH << 32),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        ssum = wave_sum_all(ssum);
        if (lane < NCOPY)
          __hip_atomic_store(a.ssum_t + (size_t)lane * G + w, (uint64_t)__float_as_uint(ssum) | ((uint64_t)epH << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // (value, index) as one word pair per copy: lane c writes copy c
      if (lane < NCOPY) {
        const auto ars = __builtin_amdgcn_make_buffer_rsrc(a.amax_t, (short)0, NCOPY * 2 * G * 8, 0x00020000);
        typedef unsigned int g2_v4u_ __attribute__((ext_vector_type(4)));
        const g2_v4u_ pr = {__float_as_uint(bv), epH, bi, epH};
        __builtin_amdgcn_raw_buffer_store_b128(pr, ars, (uint32_t)(((lane * G + w) * 2) * 8), 0, AUX_SC1);
      }
      st(step, 5 * a.L, 3);
      wg_barrier();  // stores issued: the compute waves may request the next slices
      if (step + 1 < a.nsteps && set != SET_Q && !defers(step + 1)) ctl_load(0);
    }
  }
  // the last step's greedy id
  if (w == 0) {
    uint32_t bi = 0;
    wt.start(5 * a.L);
    if (!choose_token<S, WD>(a, a.nsteps - 1, lane, wt, bi)) return;
    if (lane == 0 && a.nsteps - 1 >= a.out_from) a.out_ids[a.nsteps - 1 - a.out_from] = (int)bi;
  }
}

template <class S, int WD, bool TR>
__device__ __attribute__((always_inline)) void control_main(const DecodeArgs &a, float *lds, int lane) {
  const int w = (int)blockIdx.x;
  if (w < Set<S, SET_A>::FIRST) control_set<S, WD, TR, SET_Q>(a, lds, lane);
  else if (w < Set<S, SET_F>::FIRST) control_set<S, WD, TR, SET_A>(a, lds, lane);
  else if (w < Set<S, SET_M>::FIRST) control_set<S, WD, TR, SET_F>(a, lds, lane);
  else control_set<S, WD, TR, SET_M>(a, lds, lane);
}

template <class S, int WD, bool TR>
__global__ void __launch_bounds__(S::NT, 1) decode_kernel(DecodeArgs a) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  if (tid < 4) reinterpret_cast<int *>(lds + S::L_FLAG)[tid] = 0;
  __syncthreads();
  if (tid >= S::NL) control_main<S, WD, TR>(a, lds, tid - S::NL);
  else compute_main<S, WD, TR>(a, lds, tid);
}

// Dynamic LDS: the device's per-workgroup limit, at most 160 KB.  More than
// half of a CU's LDS puts exactly one workgroup on each CU; what the layout
// does not need beyond S::L_HEAD holds output-head rows.
constexpr size_t kLdsMax = 160 * 1024;
size_t lds_budget() {
  int dev = 0, m = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&m, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return m > 0 ? std::min((size_t)m, kLdsMax) : 0;
}
template <class S>
int head_lds_rows_for(int wd, size_t lds) {
  const size_t row = (size_t)(S::E / 4) * (wd == WD_F16 ? 8 : 16);
  const size_t base = (size_t)S::L_HEAD * sizeof(float);
  return lds > base ? (int)((lds - base) / row) : 0;
}

// The weight types a shape is built for: the 124M shape in two variants
// (eight waves: fp32 and fp16; four waves: int4), the tiny shape for all three.
template <class S>
constexpr bool shape_has(int wd) {
  return std::is_same<S, ShapeS>::value ? wd != WD_Q4 : std::is_same<S, ShapeSC>::value ? wd == WD_Q4 : true;
}
template <class S, bool TR>
const void *kernel_for_tr(int wd) {
  if (wd == WD_F32) {
    if constexpr (shape_has<S>(WD_F32)) return reinterpret_cast<const void *>(&decode_kernel<S, WD_F32, TR>);
  } else if (wd == WD_F16) {
    if constexpr (shape_has<S>(WD_F16)) return reinterpret_cast<const void *>(&decode_kernel<S, WD_F16, TR>);
  } else if (wd == WD_Q4) {
    if constexpr (shape_has<S>(WD_Q4)) return reinterpret_cast<const void *>(&decode_kernel<S, WD_Q4, TR>);
  }
  return nullptr;
}
// The kernel of a run: with the timeline stamps only when the run records them.
template <class S>
const void *kernel_for(int wd, bool traced = false) {
  return traced ? kernel_for_tr<S, true>(wd) : kernel_for_tr<S, false>(wd);
}

template <class S>
hipError_t launch_t(int wd, const DecodeArgs &a, hipStream_t s) {
  static_assert(S::L_HEAD * sizeof(float) <= 64 * 1024, "LDS layout too large");
  const void *k = kernel_for<S>(wd, a.trace != nullptr);
  if (!k) return hipErrorInvalidValue;
  const size_t lds = lds_budget();
  if (lds < (size_t)S::L_HEAD * sizeof(float)) return hipErrorInvalidConfiguration;
  DecodeArgs copy = a;
  copy.head_lds_rows = head_lds_rows_for<S>(wd, lds);
  void *args[] = {&copy};
  // An ordinary launch (a cooperative one costs about 8 us more host time per
  // call).  Every workgroup must be resident at once, and is: the LDS size
  // allows one workgroup per CU, the grid has no more workgroups than the
  // device has CUs (checked when the model is loaded), and nothing in the grid
  // waits for a workgroup that has not started except through bounded waits,
  // so a grid that cannot be placed whole (the CUs busy with other work for
  // seconds) ends with the timeout error instead of hanging.
  return hipLaunchKernel(k, dim3(S::G), dim3(S::NT), args, lds, s);
}

template <class S>
hipError_t occupancy_t(int wd, int *blocks) {
  // both variants (with and without the timeline stamps) get the LDS size; the
  // smaller of their occupancies is reported
  const size_t lds = lds_budget();
  if (lds < (size_t)S::L_HEAD * sizeof(float)) return hipErrorInvalidConfiguration;
  int best = -1;
  for (int tr = 0; tr < 2; tr++) {
    const void *k = kernel_for<S>(wd, tr != 0);
    if (!k) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int b = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, S::NT, lds);
    if (e != hipSuccess) return e;
    best = best < 0 ? b : std::min(best, b);
  }
  *blocks = best;
  return hipSuccess;
}

template <class S>
void info_t(ShapeInfo *o) {
  o->E = S::E;
  o->D = S::D;
  o->G = S::G;
  o->threads = S::NT;
  o->lds_bytes = kLdsMax;
  o->maxch = S::MAXCH;
}

}  // namespace

bool shape_info(int E, int D, int wd, ShapeInfo *out) {
  static_assert(ShapeS::G == ShapeSC::G && ShapeS::MAXCH == ShapeSC::MAXCH,
                "the two 124M variants share their grid and chunk limits");
  if (E == ShapeS::E && D == ShapeS::D) {
    if (wd != WD_Q4) info_t<ShapeS>(out);
    else info_t<ShapeSC>(out);
    return true;
  }
  if (E == ShapeT::E && D == ShapeT::D) { info_t<ShapeT>(out); return true; }
  return false;
}

hipError_t launch_decode(int E, int D, int wd, const DecodeArgs &a, hipStream_t s) {
  if (E == ShapeS::E && D == ShapeS::D) return wd != WD_Q4 ? launch_t<ShapeS>(wd, a, s) : launch_t<ShapeSC>(wd, a, s);
  if (E == ShapeT::E && D == ShapeT::D) return launch_t<ShapeT>(wd, a, s);
  return hipErrorInvalidValue;
}

hipError_t decode_occupancy(int E, int D, int wd, int *blocks) {
  if (E == ShapeS::E && D == ShapeS::D)
    return wd != WD_Q4 ? occupancy_t<ShapeS>(wd, blocks) : occupancy_t<ShapeSC>(wd, blocks);
  if (E == ShapeT::E && D == ShapeT::D) return occupancy_t<ShapeT>(wd, blocks);
  return hipErrorInvalidValue;
}

}  // namespace gpt2dec

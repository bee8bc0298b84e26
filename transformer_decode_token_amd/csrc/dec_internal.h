// Internal interface between the host runtime (gpt2dec_host.hip) and the
// device code (decode_kernel.hip, relayout.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gpt2dec {

enum { WD_F32 = 0, WD_F16 = 1, WD_Q4 = 2 };

// Copies of every published activation vector (one or more per XCD; a
// consumer polls the copy of its own XCD).
#ifndef G2_NCOPY
#define G2_NCOPY 8
#endif
constexpr int kTagCopies = G2_NCOPY;

// Fed ids carried in the kernel arguments themselves (a longer prompt is
// uploaded to a device buffer instead).
constexpr int kFeedInline = 64;

// Codes of the device error word (DecodeArgs::err[0]).
enum { ERR_NONE = 0, ERR_TIMEOUT = 1, ERR_NO_ARGMAX = 2 };

// One weight matrix of every layer, output-major [N][K] per layer, layers
// back to back.  For int4: `w` holds the nibbles ([N][K/2] bytes, element k in
// byte k/2, low nibble for even k) and `sz` the (scale, zero) pair of each
// group of 32 inputs ([N][K/32]).
struct MatW {
  const void *w;
  const float2 *sz;
};

// Everything the decode kernel reads or writes.  Cross-workgroup activations
// travel as 64-bit words (payload bits | epoch << 32) written and read with
// agent-scope atomics; a consumer knows its input is complete when every word
// carries the epoch of the producing phase.
struct DecodeArgs {
  MatW qkv, ap, fc, pr;              // the four block matrices
  const float *ln1w, *ln1b;          // [L][E]
  const float *bqkv;                 // [L][3E]
  const float *bap;                  // [L][E]
  const float *ln2w, *ln2b;          // [L][E]
  const float *bfc;                  // [L][F]
  const float *bpr;                  // [L][E]
  const float *wte;                  // [V][E] fp32 embedding
  const void *head;                  // [V][E] output head (fp32 = wte, or fp16 copy)
  const float *wpe;                  // [P][E]
  const float *lnfw, *lnfb;          // [E]
  // LayerNorm folded into the next linear (the gain scales the input; per row,
  // g* = W.gain and c* = W.shift + bias, so that row = rstd*(W.(gain*x) - mean*g*) + c*)
  const float *gqkv, *cqkv;          // [L][3E]  QKV rows, LayerNorm 1
  const float *gfc, *cfc;            // [L][F]   fc rows, LayerNorm 2
  const float *ghead, *chead;        // [V]      head rows, final LayerNorm (no bias)
  float *kc, *vc;                    // [L][H][P][D] KV cache
  uint64_t *qkv_t;                   // [L][C][3E]     tagged QKV outputs (C = kTagCopies copies)
  uint64_t *att_t;                   // [L][H][MAXCH][D+2] tagged attention chunk partials
  uint64_t *attn_t;                  // [L][C][E]      tagged merged attention output
  uint64_t *xa_t;                    // [L][C][E]      tagged residual after attention
  uint64_t *act_t;                   // [L][C][F]      tagged gelu activations
  uint64_t *xb_t;                    // [L][C][E]      tagged residual after the MLP
  uint64_t *amax_t;                  // [C][G][2]      tagged per-workgroup argmax (value, index)
  uint64_t *ssum_t;                  // [C][G]         sampling: tagged sum of exp((logit - max)/T) over
                                     //                the workgroup's rows (max = its argmax value)
  uint64_t *logit_t;                 // [V]            sampling: tagged logits (one copy)
  float *logits;                     // [V]            logits of the last step
  int *out_ids;                      // greedy ids (host memory mapped into the device)
  int *err;                          // [4] device: code, workgroup, phase, step of the first failure
  int *err_host;                     // [4] host-mapped copy of err, written by the failing workgroup
  const int *feed;                   // [n_feed] ids fed at the first steps (n_feed > kFeedInline)
  int feed_inline[kFeedInline];      // the same ids when n_feed <= kFeedInline (no upload)
  int n_feed;
  int pos0;                          // position of step 0
  int nsteps;
  int out_from;                      // step whose argmax is out_ids[0]
  float inv_temp;                    // 0: greedy; else 1/T: the ids from out_from on are sampled
  const float *draws;                // [nsteps - out_from] uniform numbers in [0,1), one per sampled id
  int L, V, P;
  float eps;
  uint32_t epoch0;                   // epochs used: epoch0 + 1 .. epoch0 + nsteps*(5L+1)
  long long timeout_ticks;           // wall-clock ticks a wait may take before aborting
  long long *trace;                  // optional: [trace_steps][5L+1][G][4] wall-clock stamps
  int trace_steps;                   //   (inputs ready, barrier 1, barrier 2, published) per phase
  int head_lds_rows;                 // output-head rows a workgroup keeps in LDS (set at launch)
};

// Shape instantiations compiled into the library.
struct ShapeInfo {
  int E, D, G, threads;
  size_t lds_bytes;
  int maxch;                         // maximum attention chunks per head
};
// The shape the decode kernel runs for an E/D model with weight type wd
// (the 124M shape has one variant for fp32 and fp16 and one for int4).
bool shape_info(int E, int D, int wd, ShapeInfo *out);

// Launch the decode kernel (all its workgroups are resident at once: one per CU).
hipError_t launch_decode(int E, int D, int wd, const DecodeArgs &a, hipStream_t s);
// Occupancy check: blocks of the decode kernel per CU.
hipError_t decode_occupancy(int E, int D, int wd, int *blocks_per_cu);

// Load-time re-layout (relayout.hip).
// src: Conv1D [K][N] fp32 (device); dst: [N][K] fp32.
hipError_t relayout_f32(const float *src, float *dst, int K, int N, hipStream_t s);
// src: Conv1D [K][N] fp32; dst: [N][K] fp16, round to nearest even.
hipError_t relayout_f16(const float *src, void *dst, int K, int N, hipStream_t s);
// src: Conv1D [K][N] fp32; tmp: [N][K] fp32 scratch; nib: [N][K/2]; sz: [N][K/32].
hipError_t relayout_q4(const float *src, float *tmp, uint8_t *nib, float2 *sz, int K, int N,
                       hipStream_t s);
// Row-major [R][C] fp32 -> fp16 (no transpose), round to nearest even.
hipError_t convert_f16(const float *src, void *dst, size_t n, hipStream_t s);
// Dequantise an output-major matrix [N][K] of type wd into float (the GEMV's own chunk decode).
hipError_t debug_dequant(int wd, const MatW &m, size_t layer_offset_elems, int N, int K, float *dst,
                         hipStream_t s);
hipError_t fill_f32(float *dst, size_t n, float v, hipStream_t s);
// LayerNorm folded into the linear that follows it: for each output row n of
// the [N][K] matrix m (of type wd, layer at element offset lofs, decoded as
// the GEMV decodes it), gsum[n] = sum_k W[n][k]*gain[k] and
// bsum[n] = sum_k W[n][k]*shift[k] + bias[n] (bias may be null).
hipError_t fold_ln(int wd, const MatW &m, size_t lofs, int N, int K, const float *gain, const float *shift,
                   const float *bias, float *gsum, float *bsum, hipStream_t s);

}  // namespace gpt2dec

// lib_internal.h -- declarations shared by the library's host-side files and
// the prefill kernels, beside the decode kernel's own (dec_internal.h).
#pragma once
#include <string>

#include "dec_internal.h"

namespace gpt2dec {

// The message gpt2_last_error(NULL) returns for this thread (a failed load).
void set_load_error(const std::string &msg);

// Called from the handler of an exported call that an exception would leave
// (a host allocation that failed, or a size the standard library refuses):
// the call's error code (GPT2_E_NOMEM for a failed allocation, else
// GPT2_E_INVAL), with the message in *ctx_err (the context's), or for this
// thread's gpt2_last_error(NULL) when ctx_err is null.
int exception_code(std::string *ctx_err) noexcept;

// Batched prompt prefill (prefill.hip): n positions p0 .. p0+n-1 through every
// layer together (their cache rows written), then the last row's logits and
// argmax (-1 when all are NaN).
struct PrefillArgs {
  const DecodeArgs *dec;     // the context's weights, cache, logits
  int wd, head_wd;           // block-matrix and head storage
  int L, E, D, P, V;
  int n, p0;
  int cus;                   // the device's compute units (tile balance)
  const int *tok;            // [n] device
  float *x, *qkv, *att, *act;  // device work rows: [n][E], [n][3E], [n][E], [n][4E]
  float *part;               // device: the projections' K-split partial sums, [4][n][E]
  int *argmax;               // the argmax (device-visible)
};
hipError_t launch_prefill(const PrefillArgs &p, hipStream_t s);

}  // namespace gpt2dec

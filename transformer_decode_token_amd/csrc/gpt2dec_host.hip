// gpt2dec_host.hip -- host runtime behind the C ABI in include/gpt2dec.h.
//
// Owns the device memory of one model (re-laid-out weights, KV cache, tagged
// activation words), validates every call before touching the device, and
// drives the decode kernel: one launch per gpt2_step (one token)
// or per gpt2_generate (the whole greedy run chained on the device).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../include/gpt2dec.h"
#include "lib_internal.h"

using namespace gpt2dec;

// Working words of gpt2_generate_noalloc, for callers that cannot allocate
// device memory: the tagged activation words, argmax and sampling slots and
// the error word of one run live here instead of in the context's buffers.
// Each GPU the library runs on holds its own copy until the process ends;
// every no-allocation call on a GPU shares it (calls that overlap on one GPU
// race).  Host code takes its address per device from hipGetSymbolAddress
// (the array's name in host code is not a device address).
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint64_t scratch[kScratchBytes / 8];

namespace {
thread_local std::string g_load_error;

// The scratch array's address on each device, taken once per device with that
// device current (nullptr until then, or if the runtime refused).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
bool g_scratch_done[kMaxDevices] = {};
uint64_t *g_scratch_ptr[kMaxDevices] = {};

uint64_t *scratch_on(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[device]) {
    g_scratch_done[device] = true;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) {
      g_scratch_ptr[device] = static_cast<uint64_t *>(ptr);
    } else {
      (void)hipGetLastError();
      g_scratch_ptr[device] = nullptr;
    }
  }
  return g_scratch_ptr[device];
}

size_t wd_bytes(int wd, size_t elems) {
  if (wd == WD_F32) return elems * 4;
  if (wd == WD_F16) return elems * 2;
  return elems / 2;
}
}  // namespace

struct gpt2_ctx {
  gpt2_config cfg{};
  int L = 0, E = 0, H = 0, D = 0, F = 0, P = 0, V = 0, wd = 0;
  ShapeInfo si{};
  int device = 0;
  hipStream_t own_stream = nullptr, stream = nullptr;
  std::vector<void *> dev_allocs;
  std::vector<void *> host_allocs;
  DecodeArgs base{};
  int *feed_d = nullptr, *err_d = nullptr;
  // host memory the kernel writes directly (mapped into the device): greedy
  // ids, and the copy of the error word; plus staging for uploads and logits
  int *ids_h = nullptr, *err_h = nullptr, *ids_dev = nullptr, *err_dev = nullptr;
  int *feed_h = nullptr;
  float *logits_h = nullptr;
  static constexpr int kTagBufs = 9;
  uint64_t *tag_bufs[kTagBufs] = {};
  size_t tag_sizes[kTagBufs] = {};
  float *draws_d = nullptr, *draws_h = nullptr;  // uniform numbers of a sampled run
  float *pf_x = nullptr, *pf_qkv = nullptr, *pf_att = nullptr, *pf_act = nullptr;  // prefill work rows
  float *pf_part = nullptr;  // prefill: the projections' K-split partial sums [4][P][E]
  int cus = 0;               // the device's compute units
  // the no-allocation path: this device's static scratch, the word offsets of
  // the error word and of each tagged buffer in it, and the words one run needs
  uint64_t *scratch = nullptr;
  size_t scratch_off[kTagBufs] = {};
  size_t scratch_words = 0;
  uint32_t epoch = 0;
  int filled = 0;
  bool poisoned = false;
  long long timeout_ticks = 0;
  long long *trace_d = nullptr;   // per-phase timeline of the last run (debug)
  int trace_steps = 0;
  std::string err;

  int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return code;
  }
  int device_fail(hipError_t e, const char *what) {
    poisoned = true;
    return fail(GPT2_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
  }
  template <typename T>
  T *dalloc(size_t bytes) {
    // (fault injection for the tests: every device allocation fails)
    const char *inject = getenv("GPT2DEC_FAIL_ALLOC");
    if (inject && atoi(inject) != 0) return nullptr;
    void *p = nullptr;
    if (hipMalloc(&p, bytes ? bytes : 4) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    dev_allocs.push_back(p);
    return static_cast<T *>(p);
  }
  template <typename T>
  T *halloc(size_t bytes) {
    void *p = nullptr;
    if (hipHostMalloc(&p, bytes ? bytes : 4, hipHostMallocMapped) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    host_allocs.push_back(p);
    return static_cast<T *>(p);
  }
  ~gpt2_ctx() {
    if (stream) (void)hipStreamSynchronize(stream);
    if (trace_d) (void)hipFree(trace_d);
    for (void *p : dev_allocs) (void)hipFree(p);
    for (void *p : host_allocs) (void)hipHostFree(p);
    if (own_stream) (void)hipStreamDestroy(own_stream);
  }
};

namespace {

bool bad_ptr_list(const float *const *a, int n) {
  if (!a) return true;
  for (int i = 0; i < n; i++)
    if (!a[i]) return true;
  return false;
}

int validate_config(const gpt2_config *c, ShapeInfo *si, std::string &msg) {
  char buf[256];
  if (c->n_layer < 1 || c->n_embd < 1 || c->n_head < 1 || c->n_positions < 1 || c->vocab_size < 1) {
    msg = "sizes must be positive";
    return GPT2_E_INVAL;
  }
  if (c->n_embd % c->n_head != 0) {
    msg = "n_embd must equal n_head * head_dim";
    return GPT2_E_INVAL;
  }
  if (!(c->ln_eps > 0.0f) || !std::isfinite(c->ln_eps)) {
    msg = "ln_eps must be positive and finite";
    return GPT2_E_INVAL;
  }
  if (c->wdtype < GPT2_W_FP32 || c->wdtype > GPT2_W_INT4) {
    msg = "unknown weight dtype";
    return GPT2_E_INVAL;
  }
  const int D = c->n_embd / c->n_head;
  if (!shape_info(c->n_embd, D, c->wdtype, si)) {
    snprintf(buf, sizeof buf, "unsupported shape n_embd=%d head_dim=%d (built: 768/64, 128/32)", c->n_embd, D);
    msg = buf;
    return GPT2_E_INVAL;
  }
  if (c->wdtype == GPT2_W_INT4 && c->q4_group != 32) {
    msg = "int4 weights need q4_group = 32";
    return GPT2_E_INVAL;
  }
  if (c->n_positions > 64 * si->maxch) {
    snprintf(buf, sizeof buf, "n_positions %d above the supported %d", c->n_positions, 64 * si->maxch);
    msg = buf;
    return GPT2_E_INVAL;
  }
  if (c->vocab_size > 256 * si->G) {
    snprintf(buf, sizeof buf, "vocab_size %d above the supported %d", c->vocab_size, 256 * si->G);
    msg = buf;
    return GPT2_E_INVAL;
  }
  return GPT2_OK;
}

// Waits for the n_out ids of the launch just queued to appear in mapped host
// memory.  Workgroup 0 writes the last one after every workgroup has published
// its part of the last pass, and no wait of the launch comes after it, so once
// every id is visible the launch can no longer fail: the caller returns without
// waiting for the kernel's exit (the stream keeps later launches behind it).
// False, with nothing consumed, when the error word is raised or the stream
// drains without the ids: the caller then takes the synchronising path.
bool wait_for_ids(gpt2_ctx *c, int n_out) {
  const volatile int *ih = c->ids_h;
  const volatile int *eh = c->err_h;
  for (unsigned it = 1;; it++) {
    if (eh[0] != ERR_NONE) return false;
    if (ih[n_out - 1] != -1) {
      bool all = true;
      for (int i = 0; i < n_out - 1; i++) all = all && ih[i] != -1;
      if (all) {
        std::atomic_thread_fence(std::memory_order_acquire);
        return true;
      }
    }
    if ((it & 1023) == 0 && hipStreamQuery(c->stream) != hipErrorNotReady) return false;
    __builtin_ia32_pause();
  }
}

// Launch `nsteps` forward passes; see gpt2_step / gpt2_generate.  With
// inv_temp > 0 the n_out recorded ids are drawn (draws[k] for the k-th).
// With in_scratch the run's working words are the device's static scratch,
// cleared first (its epochs restart at 1), and nothing is allocated.
int run(gpt2_ctx *c, const int *feed, int n_feed, int pos0, int nsteps, int out_from, int n_out, int *ids_out,
        float *logits_out, float inv_temp = 0.f, const float *draws = nullptr, bool in_scratch = false) {
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return c->device_fail(e, "hipSetDevice");
  const uint64_t used = (uint64_t)nsteps * (uint64_t)(5 * c->L + 1);
  if (!in_scratch && (uint64_t)c->epoch + used >= 0xffffff00ull) {
    // epochs would wrap: clear every tagged word (tag 0 is never expected) and restart
    for (int i = 0; i < gpt2_ctx::kTagBufs; i++) {
      e = hipMemsetAsync(c->tag_bufs[i], 0, c->tag_sizes[i], c->stream);
      if (e != hipSuccess) return c->device_fail(e, "hipMemsetAsync");
    }
    c->epoch = 0;
  }
  DecodeArgs a = c->base;
  a.n_feed = n_feed;
  if (n_feed <= kFeedInline) {
    // the fed ids travel in the kernel arguments
    memcpy(a.feed_inline, feed, sizeof(int) * (size_t)n_feed);
    a.feed = nullptr;
  } else {
    memcpy(c->feed_h, feed, sizeof(int) * (size_t)n_feed);
    e = hipMemcpyAsync(c->feed_d, c->feed_h, sizeof(int) * (size_t)n_feed, hipMemcpyHostToDevice, c->stream);
    if (e != hipSuccess) return c->device_fail(e, "uploading the fed ids");
    a.feed = c->feed_d;
  }
  a.inv_temp = inv_temp;
  if (inv_temp > 0.f) {
    memcpy(c->draws_h, draws, sizeof(float) * (size_t)n_out);
    e = hipMemcpyAsync(c->draws_d, c->draws_h, sizeof(float) * (size_t)n_out, hipMemcpyHostToDevice, c->stream);
    if (e != hipSuccess) return c->device_fail(e, "uploading the draws");
  }
  // The kernel writes the ids and (on failure) the error word's copy straight
  // into mapped host memory: cleared here, read after the stream has drained.
  // (The device error word itself is zero: any failure poisons the context.)
  memset(c->err_h, 0, 4 * sizeof(int));
  for (int i = 0; i < n_out; i++) c->ids_h[i] = -1;
  a.pos0 = pos0;
  a.nsteps = nsteps;
  a.out_from = out_from;
  a.epoch0 = c->epoch;
  a.timeout_ticks = c->timeout_ticks;
  a.trace = c->trace_d;
  a.trace_steps = c->trace_d ? c->trace_steps : 0;
  if (in_scratch) {
    // the scratch keeps whatever the last call on this device left: clear the
    // words this run uses (a fill kernel), then number its phases from 1
    uint64_t *sc = c->scratch;
    e = fill_f32(reinterpret_cast<float *>(sc), 2 * c->scratch_words, 0.0f, c->stream);
    if (e != hipSuccess) return c->device_fail(e, "clearing the scratch");
    a.err = reinterpret_cast<int *>(sc);
    a.qkv_t = sc + c->scratch_off[0];
    a.att_t = sc + c->scratch_off[1];
    a.xa_t = sc + c->scratch_off[2];
    a.act_t = sc + c->scratch_off[3];
    a.xb_t = sc + c->scratch_off[4];
    a.amax_t = sc + c->scratch_off[5];
    a.attn_t = sc + c->scratch_off[6];
    a.ssum_t = sc + c->scratch_off[7];
    a.logit_t = sc + c->scratch_off[8];
    a.epoch0 = 0;
    a.trace = nullptr;
    a.trace_steps = 0;
  }
  if (a.trace) {
    e = hipMemsetAsync(c->trace_d, 0, (size_t)c->trace_steps * (5 * c->L + 1) * c->si.G * 4 * 8, c->stream);
    if (e != hipSuccess) return c->device_fail(e, "trace reset");
  }
  e = launch_decode(c->E, c->D, c->wd, a, c->stream);
  if (!in_scratch) c->epoch += (uint32_t)used;
  if (e != hipSuccess) return c->device_fail(e, "decode launch");
  if (!logits_out && !a.trace && !in_scratch && n_out > 0 && wait_for_ids(c, n_out)) {
    // the ids are in: the launch's remaining work is its workgroups' exit
  } else {
    if (logits_out)
      e = hipMemcpyAsync(c->logits_h, c->base.logits, sizeof(float) * (size_t)c->V, hipMemcpyDeviceToHost,
                         c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return c->device_fail(e, "decode run");
  }
  const volatile int *eh = c->err_h;
  if (eh[0] == ERR_TIMEOUT) {
    c->poisoned = true;
    return c->fail(GPT2_E_DEVICE, "device wait timed out (workgroup %d, producer phase %d)", eh[1], eh[2]);
  }
  if (eh[0] != ERR_NONE) {
    c->poisoned = true;
    return c->fail(GPT2_E_NUMERIC, "every logit of pass %d of the run is NaN: no greedy id to feed", eh[3]);
  }
  const volatile int *ih = c->ids_h;
  for (int i = 0; i < n_out; i++) {
    if (ih[i] < 0 || ih[i] >= c->V) {
      c->poisoned = true;
      return c->fail(GPT2_E_NUMERIC, "every logit of pass %d of the run is NaN: no greedy id", out_from + i);
    }
    ids_out[i] = ih[i];
  }
  if (logits_out) memcpy(logits_out, c->logits_h, sizeof(float) * (size_t)c->V);
  return GPT2_OK;
}

int load_impl(gpt2_ctx *c, const gpt2_config *cfg, const gpt2_weights *w) {
  c->cfg = *cfg;
  c->L = cfg->n_layer;
  c->E = cfg->n_embd;
  c->H = cfg->n_head;
  c->D = c->E / c->H;
  c->F = 4 * c->E;
  c->P = cfg->n_positions;
  c->V = cfg->vocab_size;
  c->wd = cfg->wdtype;
  const int L = c->L, E = c->E, F = c->F, P = c->P, V = c->V, H = c->H, D = c->D, G = c->si.G;
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) return c->device_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, c->device);
  if (e != hipSuccess) return c->device_fail(e, "hipGetDeviceProperties");
  int blocks = 0;
  e = decode_occupancy(E, D, c->wd, &blocks);
  if (e != hipSuccess) return c->device_fail(e, "decode kernel occupancy");
  c->cus = prop.multiProcessorCount;
  if (blocks < 1 || (long)blocks * prop.multiProcessorCount < G)
    return c->fail(GPT2_E_DEVICE, "device cannot hold %d co-resident workgroups (%d CUs x %d)", G,
                   prop.multiProcessorCount, blocks);
  int clock_khz = 0;
  if (hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, c->device) != hipSuccess || clock_khz <= 0)
    clock_khz = 100000;
  double timeout_ms = 2000.0;
  if (const char *t = getenv("GPT2DEC_TIMEOUT_MS")) timeout_ms = atof(t);
  c->timeout_ticks = (long long)(timeout_ms * clock_khz);
  e = hipStreamCreateWithFlags(&c->own_stream, hipStreamNonBlocking);
  if (e != hipSuccess) return c->device_fail(e, "hipStreamCreate");
  c->stream = c->own_stream;
  hipStream_t s = c->stream;

  // ---- device buffers
  const size_t nq = (size_t)3 * E * E, na = (size_t)E * E, nf = (size_t)F * E, np = (size_t)E * F;
  void *mq = c->dalloc<void>(wd_bytes(c->wd, nq * L));
  void *ma = c->dalloc<void>(wd_bytes(c->wd, na * L));
  void *mf = c->dalloc<void>(wd_bytes(c->wd, nf * L));
  void *mp = c->dalloc<void>(wd_bytes(c->wd, np * L));
  float2 *sq = nullptr, *sa = nullptr, *sf = nullptr, *sp = nullptr;
  if (c->wd == WD_Q4) {
    sq = c->dalloc<float2>(nq * L / 32 * sizeof(float2));
    sa = c->dalloc<float2>(na * L / 32 * sizeof(float2));
    sf = c->dalloc<float2>(nf * L / 32 * sizeof(float2));
    sp = c->dalloc<float2>(np * L / 32 * sizeof(float2));
    if (!sq || !sa || !sf || !sp) return c->fail(GPT2_E_NOMEM, "device allocation failed");
  }
  float *stage = c->dalloc<float>(nf * sizeof(float));
  float *tmp = c->wd == WD_Q4 ? c->dalloc<float>(nf * sizeof(float)) : nullptr;
  float *ln1w = c->dalloc<float>((size_t)L * E * 4), *ln1b = c->dalloc<float>((size_t)L * E * 4);
  float *ln2w = c->dalloc<float>((size_t)L * E * 4), *ln2b = c->dalloc<float>((size_t)L * E * 4);
  float *bqkv = c->dalloc<float>((size_t)L * 3 * E * 4), *bap = c->dalloc<float>((size_t)L * E * 4);
  float *bfc = c->dalloc<float>((size_t)L * F * 4), *bpr = c->dalloc<float>((size_t)L * E * 4);
  float *lnfw = c->dalloc<float>((size_t)E * 4), *lnfb = c->dalloc<float>((size_t)E * 4);
  // LayerNorm folded into the linear after it: per-row W.gain and W.shift + bias
  float *gqkv = c->dalloc<float>((size_t)L * 3 * E * 4), *cqkv = c->dalloc<float>((size_t)L * 3 * E * 4);
  float *gfc = c->dalloc<float>((size_t)L * F * 4), *cfc = c->dalloc<float>((size_t)L * F * 4);
  float *ghead = c->dalloc<float>((size_t)V * 4), *chead = c->dalloc<float>((size_t)V * 4);
  float *wte = c->dalloc<float>((size_t)V * E * 4), *wpe = c->dalloc<float>((size_t)P * E * 4);
  void *head16 = c->wd == WD_F16 ? c->dalloc<void>((size_t)V * E * 2) : nullptr;
  const size_t kv = (size_t)L * H * P * D;
  float *kc = c->dalloc<float>(kv * 4), *vc = c->dalloc<float>(kv * 4);
  // published vectors exist in kTagCopies copies (per XCD); chunk partials have one reader
  const size_t NC = kTagCopies;
  c->tag_sizes[0] = NC * L * 3 * E * 8;
  c->tag_sizes[1] = (size_t)L * H * c->si.maxch * (D + 2) * 8;
  c->tag_sizes[2] = NC * L * E * 8;
  c->tag_sizes[3] = NC * L * F * 8;
  c->tag_sizes[4] = NC * L * E * 8;
  c->tag_sizes[5] = NC * 2 * G * 8;
  c->tag_sizes[6] = NC * L * E * 8;
  c->tag_sizes[7] = NC * G * 8;        // sampling: per-workgroup sums
  c->tag_sizes[8] = (size_t)V * 8;     // sampling: tagged logits
  for (int i = 0; i < gpt2_ctx::kTagBufs; i++) c->tag_bufs[i] = c->dalloc<uint64_t>(c->tag_sizes[i]);
  // the same words' layout in the static scratch: the error word, then each
  // tagged buffer at a 256-byte boundary
  {
    size_t off = 32;
    for (int i = 0; i < gpt2_ctx::kTagBufs; i++) {
      c->scratch_off[i] = off;
      off += (c->tag_sizes[i] / 8 + 31) & ~(size_t)31;
    }
    c->scratch_words = off;
  }
  c->draws_d = c->dalloc<float>((size_t)P * 4);
  c->pf_x = c->dalloc<float>((size_t)P * E * 4);
  c->pf_qkv = c->dalloc<float>((size_t)P * 3 * E * 4);
  c->pf_att = c->dalloc<float>((size_t)P * E * 4);
  c->pf_act = c->dalloc<float>((size_t)P * F * 4);
  c->pf_part = c->dalloc<float>((size_t)4 * P * E * 4);
  if (!c->pf_x || !c->pf_qkv || !c->pf_att || !c->pf_act || !c->pf_part)
    return c->fail(GPT2_E_NOMEM, "allocation failed");
  c->draws_h = c->halloc<float>((size_t)P * 4);
  if (!c->draws_d || !c->draws_h) return c->fail(GPT2_E_NOMEM, "allocation failed");
  float *logits = c->dalloc<float>((size_t)V * 4);
  c->feed_d = c->dalloc<int>((size_t)P * 4);
  c->err_d = c->dalloc<int>(4 * 4);
  c->feed_h = c->halloc<int>((size_t)P * 4);
  c->ids_h = c->halloc<int>((size_t)P * 4);
  c->err_h = c->halloc<int>(4 * 4);
  c->logits_h = c->halloc<float>((size_t)V * 4);
  if (!mq || !ma || !mf || !mp || !stage || (c->wd == WD_Q4 && !tmp) || !ln1w || !ln1b || !ln2w || !ln2b ||
      !bqkv || !bap || !bfc || !bpr || !lnfw || !lnfb || !gqkv || !cqkv || !gfc || !cfc || !ghead || !chead ||
      !wte || !wpe || (c->wd == WD_F16 && !head16) || !kc ||
      !vc || !logits || !c->feed_d || !c->err_d || !c->feed_h || !c->ids_h || !c->err_h ||
      !c->logits_h)
    return c->fail(GPT2_E_NOMEM, "allocation failed");
  // the device addresses of the mapped host buffers the kernel writes
  e = hipHostGetDevicePointer(reinterpret_cast<void **>(&c->ids_dev), c->ids_h, 0);
  if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void **>(&c->err_dev), c->err_h, 0);
  if (e != hipSuccess) return c->device_fail(e, "mapping host buffers");
  for (int i = 0; i < gpt2_ctx::kTagBufs; i++)
    if (!c->tag_bufs[i]) return c->fail(GPT2_E_NOMEM, "allocation failed");

  // ---- small parameters
  auto up = [&](float *dst, const float *src, size_t n) {
    return hipMemcpyAsync(dst, src, n * sizeof(float), hipMemcpyHostToDevice, s);
  };
  for (int l = 0; l < L && e == hipSuccess; l++) {
    e = up(ln1w + (size_t)l * E, w->ln1_w[l], E);
    if (e == hipSuccess) e = up(ln1b + (size_t)l * E, w->ln1_b[l], E);
    if (e == hipSuccess) e = up(ln2w + (size_t)l * E, w->ln2_w[l], E);
    if (e == hipSuccess) e = up(ln2b + (size_t)l * E, w->ln2_b[l], E);
    if (e == hipSuccess) e = up(bqkv + (size_t)l * 3 * E, w->c_attn_b[l], 3 * (size_t)E);
    if (e == hipSuccess) e = up(bap + (size_t)l * E, w->attn_proj_b[l], E);
    if (e == hipSuccess) e = up(bfc + (size_t)l * F, w->c_fc_b[l], F);
    if (e == hipSuccess) e = up(bpr + (size_t)l * E, w->mlp_proj_b[l], E);
  }
  if (e == hipSuccess) e = up(lnfw, w->lnf_w, E);
  if (e == hipSuccess) e = up(lnfb, w->lnf_b, E);
  if (e == hipSuccess) e = up(wte, w->wte, (size_t)V * E);
  if (e == hipSuccess) e = up(wpe, w->wpe, (size_t)P * E);
  if (e == hipSuccess && head16) e = convert_f16(wte, head16, (size_t)V * E, s);
  if (e != hipSuccess) return c->device_fail(e, "uploading parameters");

  // ---- block matrices: Conv1D [K][N] -> output-major [N][K]
  struct M {
    const float *const *src;
    void *dst;
    float2 *sz;
    int K, N;
  } mats[4] = {{w->c_attn_w, mq, sq, E, 3 * E},
               {w->attn_proj_w, ma, sa, E, E},
               {w->c_fc_w, mf, sf, E, F},
               {w->mlp_proj_w, mp, sp, F, E}};
  for (int m = 0; m < 4; m++) {
    const size_t n = (size_t)mats[m].K * mats[m].N;
    for (int l = 0; l < L; l++) {
      e = up(stage, mats[m].src[l], n);
      if (e != hipSuccess) break;
      if (c->wd == WD_F32) {
        e = relayout_f32(stage, static_cast<float *>(mats[m].dst) + (size_t)l * n, mats[m].K, mats[m].N, s);
      } else if (c->wd == WD_F16) {
        e = relayout_f16(stage, static_cast<uint16_t *>(mats[m].dst) + (size_t)l * n, mats[m].K, mats[m].N, s);
      } else {
        e = relayout_q4(stage, tmp, static_cast<uint8_t *>(mats[m].dst) + (size_t)l * n / 2,
                        mats[m].sz + (size_t)l * n / 32, mats[m].K, mats[m].N, s);
      }
      if (e != hipSuccess) break;
      // the staging buffer is reused by the next upload: keep the order explicit
      e = hipStreamSynchronize(s);
      if (e != hipSuccess) break;
    }
    if (e != hipSuccess) return c->device_fail(e, "weight re-layout");
  }
  // ---- LayerNorms folded into the QKV, fc and head rows (from the weights as decoded)
  for (int l = 0; l < L && e == hipSuccess; l++) {
    e = fold_ln(c->wd, MatW{mq, sq}, (size_t)l * nq, 3 * E, E, ln1w + (size_t)l * E, ln1b + (size_t)l * E,
                bqkv + (size_t)l * 3 * E, gqkv + (size_t)l * 3 * E, cqkv + (size_t)l * 3 * E, s);
    if (e == hipSuccess)
      e = fold_ln(c->wd, MatW{mf, sf}, (size_t)l * nf, F, E, ln2w + (size_t)l * E, ln2b + (size_t)l * E,
                  bfc + (size_t)l * F, gfc + (size_t)l * F, cfc + (size_t)l * F, s);
  }
  if (e == hipSuccess)
    e = fold_ln(head16 ? WD_F16 : WD_F32, MatW{head16 ? head16 : static_cast<const void *>(wte), nullptr}, 0, V,
                E, lnfw, lnfb, nullptr, ghead, chead, s);
  if (e != hipSuccess) return c->device_fail(e, "folding the LayerNorms");
  for (int i = 0; i < gpt2_ctx::kTagBufs && e == hipSuccess; i++)
    e = hipMemsetAsync(c->tag_bufs[i], 0, c->tag_sizes[i], s);
  if (e == hipSuccess) e = hipMemsetAsync(c->err_d, 0, 4 * sizeof(int), s);
  if (e == hipSuccess) e = hipMemsetAsync(kc, 0, kv * 4, s);
  if (e == hipSuccess) e = hipMemsetAsync(vc, 0, kv * 4, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return c->device_fail(e, "initialising buffers");

  DecodeArgs &a = c->base;
  a.qkv = MatW{mq, sq};
  a.ap = MatW{ma, sa};
  a.fc = MatW{mf, sf};
  a.pr = MatW{mp, sp};
  a.ln1w = ln1w; a.ln1b = ln1b; a.bqkv = bqkv; a.bap = bap;
  a.ln2w = ln2w; a.ln2b = ln2b; a.bfc = bfc; a.bpr = bpr;
  a.wte = wte;
  a.head = head16 ? head16 : static_cast<const void *>(wte);
  a.wpe = wpe;
  a.lnfw = lnfw; a.lnfb = lnfb;
  a.gqkv = gqkv; a.cqkv = cqkv;
  a.gfc = gfc; a.cfc = cfc;
  a.ghead = ghead; a.chead = chead;
  a.kc = kc; a.vc = vc;
  a.qkv_t = c->tag_bufs[0];
  a.att_t = c->tag_bufs[1];
  a.xa_t = c->tag_bufs[2];
  a.act_t = c->tag_bufs[3];
  a.xb_t = c->tag_bufs[4];
  a.amax_t = c->tag_bufs[5];
  a.attn_t = c->tag_bufs[6];
  a.ssum_t = c->tag_bufs[7];
  a.logit_t = c->tag_bufs[8];
  a.inv_temp = 0.f;
  a.draws = c->draws_d;
  a.logits = logits;
  a.out_ids = c->ids_dev;
  // this device's static scratch, for gpt2_generate_noalloc
  c->scratch = scratch_on(c->device);
  a.err = c->err_d;
  a.err_host = c->err_dev;
  a.L = L; a.V = V; a.P = P;
  a.eps = cfg->ln_eps;
  return GPT2_OK;
}

}  // namespace

void gpt2dec::set_load_error(const std::string &msg) { g_load_error = msg; }

int gpt2dec::exception_code(std::string *ctx_err) noexcept {
  const char *msg = "host allocation failed";
  int code = GPT2_E_NOMEM;
  try {
    throw;
  } catch (const std::bad_alloc &) {
  } catch (const std::length_error &) {
    msg = "a size beyond the host library's limits";
    code = GPT2_E_INVAL;
  } catch (...) {
    msg = "unexpected host error";
    code = GPT2_E_INVAL;
  }
  try {
    if (ctx_err) *ctx_err = msg;
    else g_load_error = msg;
  } catch (...) {
  }
  return code;
}

namespace {

bool usable(gpt2_ctx *c, int *rc) {
  if (!c) { *rc = GPT2_E_INVAL; return false; }
  if (c->poisoned) {
    *rc = GPT2_E_STATE;
    c->err = "context poisoned by an earlier device error";
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

int gpt2_load(const gpt2_config *cfg, const gpt2_weights *w, gpt2_ctx **out) try {
  g_load_error.clear();
  if (!out) { g_load_error = "out is NULL"; return GPT2_E_INVAL; }
  *out = nullptr;
  if (!cfg || !w) { g_load_error = "cfg or weights is NULL"; return GPT2_E_INVAL; }
  ShapeInfo si{};
  std::string msg;
  int rc = validate_config(cfg, &si, msg);
  if (rc != GPT2_OK) { g_load_error = msg; return rc; }
  const int L = cfg->n_layer;
  if (!w->wte || !w->wpe || !w->lnf_w || !w->lnf_b || bad_ptr_list(w->ln1_w, L) || bad_ptr_list(w->ln1_b, L) ||
      bad_ptr_list(w->c_attn_w, L) || bad_ptr_list(w->c_attn_b, L) || bad_ptr_list(w->attn_proj_w, L) ||
      bad_ptr_list(w->attn_proj_b, L) || bad_ptr_list(w->ln2_w, L) || bad_ptr_list(w->ln2_b, L) ||
      bad_ptr_list(w->c_fc_w, L) || bad_ptr_list(w->c_fc_b, L) || bad_ptr_list(w->mlp_proj_w, L) ||
      bad_ptr_list(w->mlp_proj_b, L)) {
    g_load_error = "a weight pointer is NULL";
    return GPT2_E_INVAL;
  }
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    g_load_error = "no HIP device available";
    return GPT2_E_DEVICE;
  }
  std::unique_ptr<gpt2_ctx> c(new (std::nothrow) gpt2_ctx());
  if (!c) { g_load_error = "out of host memory"; return GPT2_E_NOMEM; }
  c->si = si;
  rc = load_impl(c.get(), cfg, w);
  if (rc != GPT2_OK) {
    g_load_error = c->err;
    return rc;
  }
  *out = c.release();
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(nullptr);
}

int gpt2_set_stream(gpt2_ctx *c, void *hip_stream) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  // a launch may still be finishing on the old stream (its ids already
  // returned): the next one, on the new stream, must not overlap it
  const hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return c->device_fail(e, "draining the previous stream");
  c->stream = hip_stream ? static_cast<hipStream_t>(hip_stream) : c->own_stream;
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_step(gpt2_ctx *c, int token_id, int position, float *logits_out, int *argmax_out) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (token_id < 0 || token_id >= c->V)
    return c->fail(GPT2_E_INVAL, "token_id %d outside [0, %d)", token_id, c->V);
  if (position < 0 || position >= c->P)
    return c->fail(GPT2_E_INVAL, "position %d outside [0, %d)", position, c->P);
  if (position > c->filled)
    return c->fail(GPT2_E_INVAL, "position %d beyond the %d filled positions", position, c->filled);
  int id = -1;
  rc = run(c, &token_id, 1, position, 1, 0, 1, &id, logits_out);
  if (rc != GPT2_OK) return rc;
  c->filled = position + 1;
  if (argmax_out) *argmax_out = id;
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_generate(gpt2_ctx *c, const int *prompt, int n_prompt, int n_new, int *out_ids) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (!prompt || !out_ids) return c->fail(GPT2_E_INVAL, "prompt or out_ids is NULL");
  if (n_prompt < 1 || n_new < 1) return c->fail(GPT2_E_INVAL, "n_prompt and n_new must be >= 1");
  const long long steps = (long long)n_prompt + n_new - 1;
  if ((long long)c->filled + steps > c->P)
    return c->fail(GPT2_E_INVAL, "%lld steps from position %d exceed n_positions %d", steps, c->filled, c->P);
  for (int i = 0; i < n_prompt; i++)
    if (prompt[i] < 0 || prompt[i] >= c->V)
      return c->fail(GPT2_E_INVAL, "prompt[%d] = %d outside [0, %d)", i, prompt[i], c->V);
  rc = run(c, prompt, n_prompt, c->filled, (int)steps, n_prompt - 1, n_new, out_ids, nullptr);
  if (rc != GPT2_OK) return rc;
  c->filled += (int)steps;
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_prefill(gpt2_ctx *c, const int *tokens, int n, float *logits_out, int *argmax_out) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (!tokens) return c->fail(GPT2_E_INVAL, "tokens is NULL");
  if (n < 1) return c->fail(GPT2_E_INVAL, "n must be >= 1");
  if ((long long)c->filled + n > c->P)
    return c->fail(GPT2_E_INVAL, "%d positions from position %d exceed n_positions %d", n, c->filled, c->P);
  for (int i = 0; i < n; i++)
    if (tokens[i] < 0 || tokens[i] >= c->V)
      return c->fail(GPT2_E_INVAL, "tokens[%d] = %d outside [0, %d)", i, tokens[i], c->V);
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return c->device_fail(e, "hipSetDevice");
  memcpy(c->feed_h, tokens, sizeof(int) * (size_t)n);
  e = hipMemcpyAsync(c->feed_d, c->feed_h, sizeof(int) * (size_t)n, hipMemcpyHostToDevice, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "uploading the tokens");
  PrefillArgs p{};
  p.dec = &c->base;
  p.wd = c->wd;
  p.head_wd = c->wd == WD_F16 ? WD_F16 : WD_F32;
  p.L = c->L; p.E = c->E; p.D = c->D; p.P = c->P; p.V = c->V;
  p.n = n;
  p.p0 = c->filled;
  p.cus = c->cus;
  p.tok = c->feed_d;
  p.x = c->pf_x; p.qkv = c->pf_qkv; p.att = c->pf_att; p.act = c->pf_act; p.part = c->pf_part;
  p.argmax = c->ids_dev;
  c->ids_h[0] = -2;
  e = launch_prefill(p, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "prefill launch");
  if (logits_out)
    e = hipMemcpyAsync(c->logits_h, c->base.logits, sizeof(float) * (size_t)c->V, hipMemcpyDeviceToHost,
                       c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return c->device_fail(e, "prefill run");
  const int id = *static_cast<volatile int *>(c->ids_h);
  c->filled += n;
  if (id < 0 || id >= c->V) {
    c->poisoned = true;
    return c->fail(GPT2_E_NUMERIC, "every logit of the last prefilled position is NaN: no greedy id");
  }
  if (argmax_out) *argmax_out = id;
  if (logits_out) memcpy(logits_out, c->logits_h, sizeof(float) * (size_t)c->V);
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_generate_noalloc(gpt2_ctx *c, const int *prompt, int n_prompt, int n_new, int *out_ids) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (!prompt || !out_ids) return c->fail(GPT2_E_INVAL, "prompt or out_ids is NULL");
  if (n_prompt < 1 || n_new < 1) return c->fail(GPT2_E_INVAL, "n_prompt and n_new must be >= 1");
  if (c->scratch_words * 8 > kScratchBytes)
    return c->fail(GPT2_E_INVAL, "this model's working words need %zu bytes; the static scratch holds %zu",
                   c->scratch_words * 8, kScratchBytes);
  if (!c->scratch) return c->fail(GPT2_E_DEVICE, "the static scratch has no address on this device");
  const long long steps = (long long)n_prompt + n_new - 1;
  if ((long long)c->filled + steps > c->P)
    return c->fail(GPT2_E_INVAL, "%lld steps from position %d exceed n_positions %d", steps, c->filled, c->P);
  for (int i = 0; i < n_prompt; i++)
    if (prompt[i] < 0 || prompt[i] >= c->V)
      return c->fail(GPT2_E_INVAL, "prompt[%d] = %d outside [0, %d)", i, prompt[i], c->V);
  rc = run(c, prompt, n_prompt, c->filled, (int)steps, n_prompt - 1, n_new, out_ids, nullptr, 0.f, nullptr, true);
  if (rc != GPT2_OK) return rc;
  c->filled += (int)steps;
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_generate_sample(gpt2_ctx *c, const int *prompt, int n_prompt, int n_new, float temperature,
                         unsigned long long seed, int *out_ids) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (!(temperature >= 0.0f) || !std::isfinite(temperature))
    return c->fail(GPT2_E_INVAL, "temperature must be finite and >= 0");
  if (temperature == 0.0f) return gpt2_generate(c, prompt, n_prompt, n_new, out_ids);
  if (seed == 0) return c->fail(GPT2_E_INVAL, "seed must be non-zero (the xorshift64* state)");
  if (!prompt || !out_ids) return c->fail(GPT2_E_INVAL, "prompt or out_ids is NULL");
  if (n_prompt < 1 || n_new < 1) return c->fail(GPT2_E_INVAL, "n_prompt and n_new must be >= 1");
  const long long steps = (long long)n_prompt + n_new - 1;
  if ((long long)c->filled + steps > c->P)
    return c->fail(GPT2_E_INVAL, "%lld steps from position %d exceed n_positions %d", steps, c->filled, c->P);
  for (int i = 0; i < n_prompt; i++)
    if (prompt[i] < 0 || prompt[i] >= c->V)
      return c->fail(GPT2_E_INVAL, "prompt[%d] = %d outside [0, %d)", i, prompt[i], c->V);
  const float inv_temp = 1.0f / temperature;
  if (!std::isfinite(inv_temp)) return c->fail(GPT2_E_INVAL, "temperature %g is too small", (double)temperature);
  // one uniform number per drawn id: the top 24 bits of an xorshift64* output
  // (S. Vigna, ACM TOMS 42(4), 2016: shifts 12, 25, 27, multiplier
  // 2685821657736338717) times 2^-24
  std::vector<float> u((size_t)n_new);
  uint64_t st = seed;
  for (int k = 0; k < n_new; k++) {
    st ^= st >> 12;
    st ^= st << 25;
    st ^= st >> 27;
    u[(size_t)k] = (float)((st * 2685821657736338717ull) >> 40) * 0x1p-24f;
  }
  rc = run(c, prompt, n_prompt, c->filled, (int)steps, n_prompt - 1, n_new, out_ids, nullptr, inv_temp, u.data());
  if (rc != GPT2_OK) return rc;
  c->filled += (int)steps;
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_reset(gpt2_ctx *c) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  c->filled = 0;
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

void gpt2_free(gpt2_ctx *c) { delete c; }

const char *gpt2_last_error(const gpt2_ctx *c) {
  if (!c) return g_load_error.c_str();
  return c->err.c_str();
}

int gpt2_filled(const gpt2_ctx *c) { return c ? c->filled : -1; }

int gpt2_get_config(const gpt2_ctx *c, gpt2_config *out) {
  if (!c || !out) return GPT2_E_INVAL;
  *out = c->cfg;
  return GPT2_OK;
}

int gpt2_debug_dequant(gpt2_ctx *c, int layer, int which, float *out) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (!out) return c->fail(GPT2_E_INVAL, "out is NULL");
  MatW m{};
  int N = 0, K = 0, wd = c->wd;
  size_t lofs = 0;
  const int E = c->E, F = c->F;
  switch (which) {
  case 0: m = c->base.qkv; N = 3 * E; K = E; break;
  case 1: m = c->base.ap; N = E; K = E; break;
  case 2: m = c->base.fc; N = F; K = E; break;
  case 3: m = c->base.pr; N = E; K = F; break;
  case 4:
    m = MatW{c->base.head, nullptr};
    N = c->V; K = E;
    wd = (c->wd == WD_F16) ? WD_F16 : WD_F32;
    break;
  default: return c->fail(GPT2_E_INVAL, "which must be 0..4");
  }
  if (which != 4) {
    if (layer < 0 || layer >= c->L) return c->fail(GPT2_E_INVAL, "layer %d outside [0, %d)", layer, c->L);
    lofs = (size_t)layer * N * K;
  }
  float *d = nullptr;
  hipError_t e = hipMalloc(&d, (size_t)N * K * 4);
  if (e != hipSuccess) { (void)hipGetLastError(); return c->fail(GPT2_E_NOMEM, "device allocation failed"); }
  e = debug_dequant(wd, m, lofs, N, K, d, c->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(out, d, (size_t)N * K * 4, hipMemcpyDeviceToHost, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  (void)hipFree(d);
  if (e != hipSuccess) return c->device_fail(e, "debug dequant");
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_debug_fill_kv(gpt2_ctx *c, float value) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  const size_t kv = (size_t)c->L * c->H * c->P * c->D;
  hipError_t e = fill_f32(c->base.kc, kv, value, c->stream);
  if (e == hipSuccess) e = fill_f32(c->base.vc, kv, value, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return c->device_fail(e, "fill kv");
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_debug_trace(gpt2_ctx *c, int steps, long long *out, long long out_len, int *recorded_steps) try {
  int rc;
  if (!usable(c, &rc)) return rc;
  if (steps < -1) return c->fail(GPT2_E_INVAL, "steps must be >= -1");
  const size_t n = (size_t)c->trace_steps * (5 * c->L + 1) * c->si.G * 4;
  if (recorded_steps) *recorded_steps = c->trace_steps;
  if (out && c->trace_d && (out_len < 0 || (size_t)out_len < n))
    return c->fail(GPT2_E_INVAL, "out holds %lld values; the record has %zu", out_len, n);
  if (out && c->trace_d) {
    hipError_t e = hipMemcpyAsync(out, c->trace_d, n * 8, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return c->device_fail(e, "trace copy");
  }
  if (steps >= 0 && steps != c->trace_steps) {
    if (c->trace_d) {
      (void)hipStreamSynchronize(c->stream);
      (void)hipFree(c->trace_d);
      c->trace_d = nullptr;
    }
    c->trace_steps = 0;
    if (steps > 0) {
      const size_t m = (size_t)steps * (5 * c->L + 1) * c->si.G * 4;
      if (hipMalloc(&c->trace_d, m * 8) != hipSuccess) {
        (void)hipGetLastError();
        c->trace_d = nullptr;
        return c->fail(GPT2_E_NOMEM, "trace allocation failed");
      }
      c->trace_steps = steps;
    }
  }
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(c ? &c->err : nullptr);
}

int gpt2_debug_geometry(const gpt2_ctx *c, int *workgroups, int *threads) {
  if (!c) return GPT2_E_INVAL;
  if (workgroups) *workgroups = c->si.G;
  if (threads) *threads = c->si.threads;
  return GPT2_OK;
}

}  // extern "C"

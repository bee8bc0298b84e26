// hf_files.cpp -- the Hugging Face GPT-2 files read as they are published, on
// the host: model.safetensors with config.json (gpt2_load_safetensors), and
// vocab.json with merges.txt (the byte-level BPE tokenizer, gpt2_tokenize).
//
// A safetensors file is an 8-byte little-endian header length, a JSON header
// naming every tensor with its dtype, shape and byte range, then the raw
// numbers ("Let's make GPT-2 in assembly", Step 1; gpt2.s docs, Inner
// Workings).  The file is mapped read-only and its 148 tensors are looked up
// by name; config.json is checked the way the gpt2-125m model file's
// "require config" lines check it, an absent key passing.  Every check runs
// before any device work; the mapped numbers then go to gpt2_load.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/gpt2dec.h"
#include "lib_internal.h"
#include "json_min.h"

using gpt2dec::JParser;
using gpt2dec::JVal;

namespace {

// A whole small file (config.json) into a string; false past `limit` bytes.
bool read_small_file(const char *path, size_t limit, std::string &out, std::string &err) {
  FILE *f = fopen(path, "rb");
  if (!f) {
    err = std::string("cannot open ") + path;
    return false;
  }
  char buf[65536];
  size_t n;
  while ((n = fread(buf, 1, sizeof buf, f)) > 0) {
    out.append(buf, n);
    if (out.size() > limit) {
      fclose(f);
      err = std::string(path) + " is larger than expected";
      return false;
    }
  }
  const bool bad = ferror(f) != 0;
  fclose(f);
  if (bad) err = std::string("error reading ") + path;
  return !bad;
}

// A read-only mapping of a whole file.
struct Mapping {
  void *base = MAP_FAILED;
  size_t size = 0;
  ~Mapping() {
    if (base != MAP_FAILED) munmap(base, size);
  }
  bool open(const char *path, std::string &err) {
    const int fd = ::open(path, O_RDONLY);
    if (fd < 0) {
      err = std::string("cannot open ") + path;
      return false;
    }
    struct stat st;
    if (fstat(fd, &st) != 0 || st.st_size < 8) {
      close(fd);
      err = std::string(path) + " is shorter than a safetensors header length";
      return false;
    }
    size = (size_t)st.st_size;
    base = mmap(nullptr, size, PROT_READ, MAP_PRIVATE, fd, 0);
    close(fd);
    if (base == MAP_FAILED) {
      err = std::string("cannot map ") + path;
      return false;
    }
    return true;
  }
};

bool as_int(const JVal *v, long long &out) {
  if (!v || v->kind != JVal::NUM || !std::isfinite(v->num) || v->num != std::floor(v->num)) return false;
  if (std::fabs(v->num) > 9.0e15) return false;
  out = (long long)v->num;
  return true;
}

// config.json -> the shape, plus the model file's configuration checks:
// model_type gpt2, activation_function gelu_new, scale_attn_weights true,
// scale_attn_by_inverse_layer_idx false, reorder_and_upcast_attn false,
// add_cross_attention false (each passing when absent); n_embd = n_head *
// head_dim; and the MLP width 4 * n_embd (n_inner absent or null, or that).
bool read_config(const char *path, gpt2_config &cfg, std::string &err) {
  std::string text;
  if (!read_small_file(path, (size_t)16 << 20, text, err)) return false;
  JVal root;
  JParser jp(text.data(), text.size());
  if (!jp.parse(root)) {
    err = std::string(path) + ": " + jp.error();
    return false;
  }
  if (root.kind != JVal::OBJ) {
    err = std::string(path) + ": not a JSON object";
    return false;
  }
  auto need_str = [&](const char *k, const char *want) {
    const JVal *v = root.get(k);
    if (!v) return true;
    if (v->kind == JVal::STR && v->str == want) return true;
    err = std::string("config ") + k + " must be \"" + want + "\"";
    return false;
  };
  auto need_bool = [&](const char *k, bool want) {
    const JVal *v = root.get(k);
    if (!v) return true;
    if (v->kind == JVal::BOOL && v->b == want) return true;
    err = std::string("config ") + k + " must be " + (want ? "true" : "false");
    return false;
  };
  if (!need_str("model_type", "gpt2") || !need_str("activation_function", "gelu_new") ||
      !need_bool("scale_attn_weights", true) || !need_bool("scale_attn_by_inverse_layer_idx", false) ||
      !need_bool("reorder_and_upcast_attn", false) || !need_bool("add_cross_attention", false))
    return false;
  // (the upper limits, far above any GPT-2, keep every tensor's element count
  // and byte range in 64-bit arithmetic)
  long long L, E, H, P, V;
  const char *names[5] = {"n_layer", "n_embd", "n_head", "n_positions", "vocab_size"};
  const long long limit[5] = {1LL << 10, 1LL << 16, 1LL << 16, 1LL << 20, 1LL << 24};
  long long *dst[5] = {&L, &E, &H, &P, &V};
  for (int i = 0; i < 5; i++) {
    if (!as_int(root.get(names[i]), *dst[i]) || *dst[i] < 1 || *dst[i] > limit[i]) {
      err = std::string("config ") + names[i] + " must be an integer in [1, " + std::to_string(limit[i]) + "]";
      return false;
    }
  }
  if (E % H != 0) {
    err = "config n_embd must equal n_head * head_dim";
    return false;
  }
  const JVal *inner = root.get("n_inner");
  long long ni = 0;
  if (inner && inner->kind != JVal::NUL && !(as_int(inner, ni) && ni == 4 * E)) {
    err = "config n_inner must be null or 4 * n_embd (the MLP width the model file fixes)";
    return false;
  }
  double eps = 1e-5;  // GPT-2's value, taken when the key is absent
  if (const JVal *e = root.get("layer_norm_epsilon")) {
    if (e->kind != JVal::NUM || !(e->num > 0.0) || !std::isfinite(e->num)) {
      err = "config layer_norm_epsilon must be a positive number";
      return false;
    }
    eps = e->num;
  }
  cfg.n_layer = (int)L;
  cfg.n_embd = (int)E;
  cfg.n_head = (int)H;
  cfg.n_positions = (int)P;
  cfg.vocab_size = (int)V;
  cfg.ln_eps = (float)eps;
  return true;
}

}  // namespace

extern "C" int gpt2_load_safetensors(const char *safetensors_path, const char *config_path, int wdtype,
                                     gpt2_ctx **out) try {
  auto reject = [](int code, const std::string &msg) {
    gpt2dec::set_load_error(msg);
    return code;
  };
  if (!out) return reject(GPT2_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!safetensors_path || !config_path) return reject(GPT2_E_INVAL, "a path is NULL");
  std::string err;
  gpt2_config cfg{};
  if (!read_config(config_path, cfg, err)) return reject(GPT2_E_INVAL, err);
  cfg.wdtype = wdtype;
  cfg.q4_group = 32;

  Mapping map;
  if (!map.open(safetensors_path, err)) return reject(GPT2_E_INVAL, err);
  const unsigned char *bytes = static_cast<const unsigned char *>(map.base);
  uint64_t hlen = 0;
  for (int i = 7; i >= 0; i--) hlen = (hlen << 8) | bytes[i];  // little-endian
  if (hlen > map.size - 8 || hlen > ((uint64_t)100 << 20))
    return reject(GPT2_E_INVAL, "safetensors header length beyond the file");
  JVal header;
  JParser jp(reinterpret_cast<const char *>(bytes + 8), (size_t)hlen);
  if (!jp.parse(header) || header.kind != JVal::OBJ)
    return reject(GPT2_E_INVAL, "safetensors header: " + (jp.error().empty() ? "not a JSON object" : jp.error()));
  const size_t data_size = map.size - 8 - (size_t)hlen;
  const unsigned char *data = bytes + 8 + hlen;
  // names with the model file's optional "transformer." prefix
  std::unordered_map<std::string, const JVal *> entries;
  for (const auto &kv : header.obj) {
    if (kv.first == "__metadata__") continue;
    std::string name = kv.first;
    if (name.rfind("transformer.", 0) == 0) name = name.substr(12);
    if (!entries.emplace(name, &kv.second).second)
      return reject(GPT2_E_INVAL, "tensor " + name + " appears twice (with and without the transformer. prefix)");
  }
  const long long E = cfg.n_embd, F = 4LL * cfg.n_embd, V = cfg.vocab_size, P = cfg.n_positions;
  // the fp32 numbers of one tensor, checked against its expected shape
  auto tensor = [&](const std::string &name, std::vector<long long> shape, const float *&ptr) -> bool {
    auto it = entries.find(name);
    if (it == entries.end()) {
      err = "tensor " + name + " is missing";
      return false;
    }
    const JVal &t = *it->second;
    const JVal *dt = t.get("dtype"), *sh = t.get("shape"), *off = t.get("data_offsets");
    if (!dt || dt->kind != JVal::STR || dt->str != "F32") {
      err = "tensor " + name + " is not F32";
      return false;
    }
    if (!sh || sh->kind != JVal::ARR || sh->arr.size() != shape.size()) {
      err = "tensor " + name + " has the wrong rank";
      return false;
    }
    long long n = 1;
    for (size_t i = 0; i < shape.size(); i++) {
      long long d;
      if (!as_int(&sh->arr[i], d) || d != shape[i]) {
        err = "tensor " + name + " has the wrong shape";
        return false;
      }
      n *= d;
    }
    long long b, e;
    if (!off || off->kind != JVal::ARR || off->arr.size() != 2 || !as_int(&off->arr[0], b) ||
        !as_int(&off->arr[1], e) || b < 0 || e < b || (unsigned long long)e > data_size || e - b != 4 * n) {
      err = "tensor " + name + " has bad data offsets";
      return false;
    }
    ptr = reinterpret_cast<const float *>(data + b);
    return true;
  };
  const int L = cfg.n_layer;
  const float *wte = nullptr, *wpe = nullptr, *lnfw = nullptr, *lnfb = nullptr;
  std::vector<const float *> ln1w(L), ln1b(L), qw(L), qb(L), aw(L), ab(L), ln2w(L), ln2b(L), fw(L), fb(L), pw(L),
      pb(L);
  bool ok = tensor("wte.weight", {V, E}, wte) && tensor("wpe.weight", {P, E}, wpe) &&
            tensor("ln_f.weight", {E}, lnfw) && tensor("ln_f.bias", {E}, lnfb);
  for (int l = 0; ok && l < L; l++) {
    const std::string h = "h." + std::to_string(l) + ".";
    ok = tensor(h + "ln_1.weight", {E}, ln1w[l]) && tensor(h + "ln_1.bias", {E}, ln1b[l]) &&
         tensor(h + "attn.c_attn.weight", {E, 3 * E}, qw[l]) && tensor(h + "attn.c_attn.bias", {3 * E}, qb[l]) &&
         tensor(h + "attn.c_proj.weight", {E, E}, aw[l]) && tensor(h + "attn.c_proj.bias", {E}, ab[l]) &&
         tensor(h + "ln_2.weight", {E}, ln2w[l]) && tensor(h + "ln_2.bias", {E}, ln2b[l]) &&
         tensor(h + "mlp.c_fc.weight", {E, F}, fw[l]) && tensor(h + "mlp.c_fc.bias", {F}, fb[l]) &&
         tensor(h + "mlp.c_proj.weight", {F, E}, pw[l]) && tensor(h + "mlp.c_proj.bias", {E}, pb[l]);
  }
  if (!ok) return reject(GPT2_E_INVAL, err);
  gpt2_weights w{};
  w.wte = wte;
  w.wpe = wpe;
  w.ln1_w = ln1w.data();
  w.ln1_b = ln1b.data();
  w.c_attn_w = qw.data();
  w.c_attn_b = qb.data();
  w.attn_proj_w = aw.data();
  w.attn_proj_b = ab.data();
  w.ln2_w = ln2w.data();
  w.ln2_b = ln2b.data();
  w.c_fc_w = fw.data();
  w.c_fc_b = fb.data();
  w.mlp_proj_w = pw.data();
  w.mlp_proj_b = pb.data();
  w.lnf_w = lnfw;
  w.lnf_b = lnfb;
  // (gpt2_load copies everything before it returns; the mapping ends here)
  return gpt2_load(&cfg, &w, out);
} catch (...) {
  return gpt2dec::exception_code(nullptr);
}

// ---------------------------------------------------------------------------
// Byte-level BPE tokenizer ("Let's make GPT-2 in assembly", Step 3; gpt2.s
// docs, Limitations).  vocab.json maps token strings, written in GPT-2's
// byte-level alphabet, to ids; merges.txt lists pairs in rank order.  Text is
// split into chunks by the pre-tokenizer rules, then each chunk's bytes join
// pairwise, lowest rank first, until no neighbouring pair has a rank.
// ---------------------------------------------------------------------------

struct gpt2_tokenizer {
  std::vector<std::string> tok;            // id -> bytes ("" for an id the vocabulary skips)
  std::unordered_map<std::string, int> id;  // bytes -> id
  int byte_id[256];                         // id of each single byte
  // (id a << 32 | id b) -> (rank, id of the joined token)
  std::unordered_map<uint64_t, std::pair<int, int>> merge;
};

namespace {

// GPT-2's byte-level alphabet: the printable bytes '!'..'~', 0xA1..0xAC and
// 0xAE..0xFF stand for themselves; every other byte, in increasing order,
// for the code points 256, 257, ...  Inverse: code point -> byte, or -1.
int alphabet_byte(uint32_t cp) {
  static int inv[512];
  static bool init = false;
  if (!init) {
    for (int i = 0; i < 512; i++) inv[i] = -1;
    int extra = 0;
    for (int b = 0; b < 256; b++) {
      const bool kept = (b >= '!' && b <= '~') || (b >= 0xA1 && b <= 0xAC) || (b >= 0xAE && b <= 0xFF);
      inv[kept ? b : 256 + extra++] = b;
    }
    init = true;
  }
  return cp < 512 ? inv[cp] : -1;
}

// A token string of the byte-level alphabet (UTF-8) -> its bytes.
bool alphabet_decode(const std::string &s, std::string &out) {
  out.clear();
  for (size_t i = 0; i < s.size();) {
    const unsigned char c = (unsigned char)s[i];
    uint32_t cp;
    int len;
    if (c < 0x80) { cp = c; len = 1; }
    else if ((c & 0xE0) == 0xC0) { cp = c & 0x1F; len = 2; }
    else if ((c & 0xF0) == 0xE0) { cp = c & 0x0F; len = 3; }
    else return false;
    if (i + len > s.size()) return false;
    for (int k = 1; k < len; k++) {
      const unsigned char d = (unsigned char)s[i + k];
      if ((d & 0xC0) != 0x80) return false;
      cp = (cp << 6) | (d & 0x3F);
    }
    const int b = alphabet_byte(cp);
    if (b < 0) return false;
    out += (char)b;
    i += len;
  }
  return true;
}

enum ByteKind { K_SPACE, K_LETTER, K_DIGIT, K_OTHER };
// Whitespace is the ASCII set; every byte above 127 counts as a letter (the
// gpt2.s docs' rule: exact for ASCII text).
ByteKind byte_kind(unsigned char b) {
  if (b == ' ' || b == '\t' || b == '\n' || b == 0x0B || b == 0x0C || b == '\r') return K_SPACE;
  if ((b >= 'A' && b <= 'Z') || (b >= 'a' && b <= 'z') || b >= 128) return K_LETTER;
  if (b >= '0' && b <= '9') return K_DIGIT;
  return K_OTHER;
}

// The pre-tokenizer: the end of the chunk that starts at i.  A chunk is an
// ending 's 't 're 've 'm 'll 'd; a run of letters, of digits or of other
// symbols, each with one optional space in front; or a whitespace run, which
// leaves its last character to a non-space that follows it.
size_t chunk_end(const unsigned char *s, size_t n, size_t i) {
  if (s[i] == '\'' && i + 1 < n) {
    const unsigned char a = s[i + 1], b = i + 2 < n ? s[i + 2] : 0;
    if ((a == 'r' && b == 'e') || (a == 'v' && b == 'e') || (a == 'l' && b == 'l')) return i + 3;
    if (a == 's' || a == 't' || a == 'm' || a == 'd') return i + 2;
  }
  size_t j = i;
  if (s[j] == ' ' && j + 1 < n && byte_kind(s[j + 1]) != K_SPACE) j++;
  const ByteKind k = byte_kind(s[j]);
  if (k != K_SPACE) {
    while (j < n && byte_kind(s[j]) == k) j++;
    return j;
  }
  while (j < n && byte_kind(s[j]) == K_SPACE) j++;
  if (j < n && j - i >= 2) j--;
  return j;
}

}  // namespace

extern "C" {

int gpt2_tokenizer_load(const char *vocab_json_path, const char *merges_txt_path, gpt2_tokenizer **out) try {
  auto reject = [](const std::string &msg) {
    gpt2dec::set_load_error(msg);
    return GPT2_E_INVAL;
  };
  if (!out) return reject("out is NULL");
  *out = nullptr;
  if (!vocab_json_path || !merges_txt_path) return reject("a path is NULL");
  std::string text, err;
  if (!read_small_file(vocab_json_path, (size_t)64 << 20, text, err)) return reject(err);
  JVal vocab;
  JParser jp(text.data(), text.size());
  if (!jp.parse(vocab) || vocab.kind != JVal::OBJ)
    return reject(std::string(vocab_json_path) + ": " + (jp.error().empty() ? "not a JSON object" : jp.error()));
  std::unique_ptr<gpt2_tokenizer> t(new (std::nothrow) gpt2_tokenizer());
  if (!t) return GPT2_E_NOMEM;
  // (fault injection for the tests: a host allocation that fails here)
  const char *inject = getenv("GPT2DEC_FAIL_HOST_ALLOC");
  if (inject && atoi(inject) != 0) throw std::bad_alloc();
  for (int b = 0; b < 256; b++) t->byte_id[b] = -1;
  std::string bytes;
  for (const auto &kv : vocab.obj) {
    long long v;
    if (!as_int(&kv.second, v) || v < 0 || v >= (1 << 24)) return reject("vocab.json: id of " + kv.first + " is not a valid id");
    if (!alphabet_decode(kv.first, bytes)) return reject("vocab.json: " + kv.first + " is outside the byte-level alphabet");
    if (bytes.empty()) return reject("vocab.json: empty token");
    if ((size_t)v >= t->tok.size()) t->tok.resize((size_t)v + 1);
    if (!t->tok[(size_t)v].empty() || !t->id.emplace(bytes, (int)v).second)
      return reject("vocab.json: token or id " + std::to_string(v) + " appears twice");
    t->tok[(size_t)v] = bytes;
    if (bytes.size() == 1) t->byte_id[(unsigned char)bytes[0]] = (int)v;
  }
  for (int b = 0; b < 256; b++)
    if (t->byte_id[b] < 0) return reject("vocab.json has no token for byte " + std::to_string(b));
  std::string mtext;
  if (!read_small_file(merges_txt_path, (size_t)64 << 20, mtext, err)) return reject(err);
  int rank = 0;
  size_t pos = 0;
  std::string a, b;
  while (pos < mtext.size()) {
    size_t eol = mtext.find('\n', pos);
    if (eol == std::string::npos) eol = mtext.size();
    std::string line = mtext.substr(pos, eol - pos);
    pos = eol + 1;
    if (!line.empty() && line.back() == '\r') line.pop_back();
    if (line.empty() || line.rfind("#version", 0) == 0) continue;
    const size_t sp = line.find(' ');
    if (sp == std::string::npos || line.find(' ', sp + 1) != std::string::npos)
      return reject("merges.txt: a line is not two tokens: " + line);
    if (!alphabet_decode(line.substr(0, sp), a) || !alphabet_decode(line.substr(sp + 1), b) || a.empty() ||
        b.empty())
      return reject("merges.txt: a token outside the byte-level alphabet: " + line);
    auto ia = t->id.find(a), ib = t->id.find(b), iab = t->id.find(a + b);
    if (ia == t->id.end() || ib == t->id.end() || iab == t->id.end())
      return reject("merges.txt: " + line + " names a token the vocabulary lacks");
    const uint64_t key = ((uint64_t)(uint32_t)ia->second << 32) | (uint32_t)ib->second;
    t->merge.emplace(key, std::make_pair(rank++, iab->second));  // (the first of a repeated pair ranks)
  }
  *out = t.release();
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(nullptr);
}

int gpt2_tokenize(const gpt2_tokenizer *t, const char *text, size_t len, int *ids, int cap, int *n_ids) try {
  if (!t || (!text && len) || !n_ids || cap < 0 || (!ids && cap > 0)) {
    gpt2dec::set_load_error("bad argument");
    return GPT2_E_INVAL;
  }
  const unsigned char *s = reinterpret_cast<const unsigned char *>(text);
  std::vector<int> sym;
  long long n = 0;
  for (size_t i = 0; i < len;) {
    const size_t e = chunk_end(s, len, i);
    sym.clear();
    for (size_t k = i; k < e; k++) sym.push_back(t->byte_id[s[k]]);
    // join the lowest-ranked neighbouring pair (the leftmost among equals) until none has a rank
    while (sym.size() > 1) {
      int best = -1, where = -1, joined = -1;
      for (size_t k = 0; k + 1 < sym.size(); k++) {
        auto it = t->merge.find(((uint64_t)(uint32_t)sym[k] << 32) | (uint32_t)sym[k + 1]);
        if (it != t->merge.end() && (best < 0 || it->second.first < best)) {
          best = it->second.first;
          where = (int)k;
          joined = it->second.second;
        }
      }
      if (best < 0) break;
      sym[(size_t)where] = joined;
      sym.erase(sym.begin() + where + 1);
    }
    for (int v : sym) {
      if (n < cap) ids[n] = v;
      n++;
    }
    i = e;
  }
  if (n > 0x7fffffff) {
    gpt2dec::set_load_error("text too long");
    return GPT2_E_INVAL;
  }
  *n_ids = (int)n;
  if (!ids) return GPT2_OK;  // (a query of the count)
  if (n > cap) {
    gpt2dec::set_load_error("ids holds " + std::to_string(cap) + " ids; the text has " + std::to_string(n));
    return GPT2_E_INVAL;
  }
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(nullptr);
}

int gpt2_detokenize(const gpt2_tokenizer *t, const int *ids, int n, char *buf, size_t cap, size_t *len) try {
  if (!t || n < 0 || (!ids && n) || !len || (!buf && cap)) {
    gpt2dec::set_load_error("bad argument");
    return GPT2_E_INVAL;
  }
  size_t m = 0;
  for (int i = 0; i < n; i++) {
    if (ids[i] < 0 || (size_t)ids[i] >= t->tok.size() || t->tok[(size_t)ids[i]].empty()) {
      gpt2dec::set_load_error("id " + std::to_string(ids[i]) + " is not in the vocabulary");
      return GPT2_E_INVAL;
    }
    m += t->tok[(size_t)ids[i]].size();
  }
  *len = m;
  if (!buf) return GPT2_OK;  // (a query of the length)
  if (m > cap) {
    gpt2dec::set_load_error("buf holds " + std::to_string(cap) + " bytes; the text has " + std::to_string(m));
    return GPT2_E_INVAL;
  }
  size_t o = 0;
  for (int i = 0; i < n; i++) {
    const std::string &s = t->tok[(size_t)ids[i]];
    memcpy(buf + o, s.data(), s.size());
    o += s.size();
  }
  return GPT2_OK;
} catch (...) {
  return gpt2dec::exception_code(nullptr);
}

void gpt2_tokenizer_free(gpt2_tokenizer *t) { delete t; }

}  // extern "C"

// json_min.h -- a small JSON reader for the Hugging Face files the library
// takes as they are published (config.json, the safetensors header,
// vocab.json).  Values: null, true/false, numbers (double), strings (escapes
// decoded to UTF-8, \uXXXX surrogate pairs joined), arrays and objects (keys
// kept in file order).  Nesting deeper than 64 levels is refused.
#pragma once
#include <cstdint>
#include <cstdlib>
#include <string>
#include <utility>
#include <vector>

namespace gpt2dec {

struct JVal {
  enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ };
  Kind kind = NUL;
  bool b = false;
  double num = 0.0;
  std::string str;
  std::vector<JVal> arr;
  std::vector<std::pair<std::string, JVal>> obj;
  // the member named k of an object, or nullptr
  const JVal *get(const std::string &k) const {
    if (kind != OBJ) return nullptr;
    for (const auto &kv : obj)
      if (kv.first == k) return &kv.second;
    return nullptr;
  }
};

class JParser {
 public:
  JParser(const char *text, size_t len) : p_(text), end_(text + len) {}
  // Parses one value that must span the whole text (trailing whitespace
  // allowed).  False with error() set on malformed input.
  bool parse(JVal &out) {
    if (!value(out, 0)) return false;
    ws();
    if (p_ != end_) return fail("trailing characters after the JSON value");
    return true;
  }
  const std::string &error() const { return err_; }

 private:
  const char *p_, *end_;
  std::string err_;

  bool fail(const char *msg) {
    if (err_.empty()) err_ = msg;
    return false;
  }
  void ws() {
    while (p_ < end_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) p_++;
  }
  bool lit(const char *s) {
    const char *q = p_;
    for (; *s; s++, q++)
      if (q >= end_ || *q != *s) return false;
    p_ = q;
    return true;
  }
  static void put_utf8(std::string &s, uint32_t c) {
    if (c < 0x80) {
      s += (char)c;
    } else if (c < 0x800) {
      s += (char)(0xC0 | (c >> 6));
      s += (char)(0x80 | (c & 0x3F));
    } else if (c < 0x10000) {
      s += (char)(0xE0 | (c >> 12));
      s += (char)(0x80 | ((c >> 6) & 0x3F));
      s += (char)(0x80 | (c & 0x3F));
    } else {
      s += (char)(0xF0 | (c >> 18));
      s += (char)(0x80 | ((c >> 12) & 0x3F));
      s += (char)(0x80 | ((c >> 6) & 0x3F));
      s += (char)(0x80 | (c & 0x3F));
    }
  }
  bool hex4(uint32_t &v) {
    if (end_ - p_ < 4) return fail("truncated \\u escape");
    v = 0;
    for (int i = 0; i < 4; i++) {
      const char c = *p_++;
      v <<= 4;
      if (c >= '0' && c <= '9') v |= (uint32_t)(c - '0');
      else if (c >= 'a' && c <= 'f') v |= (uint32_t)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') v |= (uint32_t)(c - 'A' + 10);
      else return fail("bad hex digit in a \\u escape");
    }
    return true;
  }
  bool string(std::string &s) {
    if (p_ >= end_ || *p_ != '"') return fail("expected a string");
    p_++;
    while (true) {
      if (p_ >= end_) return fail("unterminated string");
      const char c = *p_++;
      if (c == '"') return true;
      if ((unsigned char)c < 0x20) return fail("control character in a string");
      if (c != '\\') {
        s += c;
        continue;
      }
      if (p_ >= end_) return fail("unterminated escape");
      const char e = *p_++;
      switch (e) {
      case '"': s += '"'; break;
      case '\\': s += '\\'; break;
      case '/': s += '/'; break;
      case 'b': s += '\b'; break;
      case 'f': s += '\f'; break;
      case 'n': s += '\n'; break;
      case 'r': s += '\r'; break;
      case 't': s += '\t'; break;
      case 'u': {
        uint32_t c1;
        if (!hex4(c1)) return false;
        if (c1 >= 0xD800 && c1 < 0xDC00) {  // high surrogate: a low one must follow
          uint32_t c2;
          if (!(lit("\\u") && hex4(c2)) || c2 < 0xDC00 || c2 >= 0xE000) return fail("unpaired surrogate");
          c1 = 0x10000 + ((c1 - 0xD800) << 10) + (c2 - 0xDC00);
        } else if (c1 >= 0xDC00 && c1 < 0xE000) {
          return fail("unpaired surrogate");
        }
        put_utf8(s, c1);
        break;
      }
      default: return fail("unknown escape");
      }
    }
  }
  bool number(double &v) {
    const char *q = p_;
    if (q < end_ && *q == '-') q++;
    if (q >= end_ || !(*q >= '0' && *q <= '9')) return fail("bad number");
    while (q < end_ && ((*q >= '0' && *q <= '9') || *q == '.' || *q == 'e' || *q == 'E' || *q == '+' || *q == '-'))
      q++;
    const std::string t(p_, q);
    char *stop = nullptr;
    v = std::strtod(t.c_str(), &stop);
    if (!stop || *stop != '\0') return fail("bad number");
    p_ = q;
    return true;
  }
  bool value(JVal &v, int depth) {
    if (depth > 64) return fail("nesting deeper than 64 levels");
    ws();
    if (p_ >= end_) return fail("unexpected end of input");
    const char c = *p_;
    if (c == '{') {
      p_++;
      v.kind = JVal::OBJ;
      ws();
      if (p_ < end_ && *p_ == '}') {
        p_++;
        return true;
      }
      while (true) {
        ws();
        std::string k;
        if (!string(k)) return false;
        ws();
        if (p_ >= end_ || *p_ != ':') return fail("expected ':' in an object");
        p_++;
        JVal m;
        if (!value(m, depth + 1)) return false;
        v.obj.emplace_back(std::move(k), std::move(m));
        ws();
        if (p_ < end_ && *p_ == ',') {
          p_++;
          continue;
        }
        if (p_ < end_ && *p_ == '}') {
          p_++;
          return true;
        }
        return fail("expected ',' or '}' in an object");
      }
    }
    if (c == '[') {
      p_++;
      v.kind = JVal::ARR;
      ws();
      if (p_ < end_ && *p_ == ']') {
        p_++;
        return true;
      }
      while (true) {
        JVal m;
        if (!value(m, depth + 1)) return false;
        v.arr.push_back(std::move(m));
        ws();
        if (p_ < end_ && *p_ == ',') {
          p_++;
          continue;
        }
        if (p_ < end_ && *p_ == ']') {
          p_++;
          return true;
        }
        return fail("expected ',' or ']' in an array");
      }
    }
    if (c == '"') {
      v.kind = JVal::STR;
      return string(v.str);
    }
    if (lit("true")) {
      v.kind = JVal::BOOL;
      v.b = true;
      return true;
    }
    if (lit("false")) {
      v.kind = JVal::BOOL;
      v.b = false;
      return true;
    }
    if (lit("null")) {
      v.kind = JVal::NUL;
      return true;
    }
    v.kind = JVal::NUM;
    return number(v.num);
  }
};

}  // namespace gpt2dec

// safetensors header reader: a small JSON parser for the header object and
// the consistency checks a loader needs before reading any tensor bytes.
#include "checkpoint.h"

#include <cstdio>
#include <cstring>

namespace q3k {
namespace {

constexpr uint64_t kMaxHeader = 100ull << 20;  // the format caps headers at 100 MB

// JSON values of the header: objects, arrays, strings and integers (no floats
// appear in a tensor entry; other scalars are skipped).
struct Parser {
  const char* p;
  const char* end;
  std::string err;

  void ws() {
    while (p < end && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) ++p;
  }
  bool fail(const std::string& m) {
    if (err.empty()) err = m;
    return false;
  }
  bool lit(char c) {
    ws();
    if (p < end && *p == c) {
      ++p;
      return true;
    }
    return false;
  }
  bool string(std::string* out) {
    ws();
    if (p >= end || *p != '"') return fail("expected a string");
    ++p;
    out->clear();
    while (p < end && *p != '"') {
      char c = *p++;
      if (c == '\\') {
        if (p >= end) return fail("unterminated escape");
        const char e = *p++;
        switch (e) {
          case '"': case '\\': case '/': out->push_back(e); break;
          case 'b': out->push_back('\b'); break;
          case 'f': out->push_back('\f'); break;
          case 'n': out->push_back('\n'); break;
          case 'r': out->push_back('\r'); break;
          case 't': out->push_back('\t'); break;
          case 'u': {  // \uXXXX: kept as UTF-8 (names are ASCII in practice)
            if (end - p < 4) return fail("short \\u escape");
            unsigned v = 0;
            for (int i = 0; i < 4; ++i) {
              const char h = *p++;
              v <<= 4;
              if (h >= '0' && h <= '9') v |= (unsigned)(h - '0');
              else if (h >= 'a' && h <= 'f') v |= (unsigned)(h - 'a' + 10);
              else if (h >= 'A' && h <= 'F') v |= (unsigned)(h - 'A' + 10);
              else return fail("bad \\u escape");
            }
            if (v < 0x80) {
              out->push_back((char)v);
            } else if (v < 0x800) {
              out->push_back((char)(0xC0 | (v >> 6)));
              out->push_back((char)(0x80 | (v & 0x3F)));
            } else {
              out->push_back((char)(0xE0 | (v >> 12)));
              out->push_back((char)(0x80 | ((v >> 6) & 0x3F)));
              out->push_back((char)(0x80 | (v & 0x3F)));
            }
            break;
          }
          default: return fail("bad escape");
        }
      } else {
        out->push_back(c);
      }
    }
    if (p >= end) return fail("unterminated string");
    ++p;
    return true;
  }
  bool integer(int64_t* out) {
    ws();
    const char* s = p;
    if (p < end && *p == '-') ++p;
    if (p >= end || *p < '0' || *p > '9') return fail("expected an integer");
    int64_t v = 0;
    while (p < end && *p >= '0' && *p <= '9') {
      if (v > (INT64_MAX - 9) / 10) return fail("integer too large");
      v = v * 10 + (*p++ - '0');
    }
    if (p < end && (*p == '.' || *p == 'e' || *p == 'E')) return fail("expected an integer");
    *out = (*s == '-') ? -v : v;
    return true;
  }
  bool int_array(std::vector<int64_t>* out) {
    out->clear();
    if (!lit('[')) return fail("expected an array");
    if (lit(']')) return true;
    do {
      int64_t v;
      if (!integer(&v)) return false;
      out->push_back(v);
    } while (lit(','));
    return lit(']') || fail("expected ']'");
  }
  // Skips any JSON value (for "__metadata__" and unknown keys).
  bool skip(int depth = 0) {
    if (depth > 64) return fail("nesting too deep");
    ws();
    if (p >= end) return fail("unexpected end");
    if (*p == '"') {
      std::string s;
      return string(&s);
    }
    if (*p == '{' || *p == '[') {
      const char close = *p == '{' ? '}' : ']';
      const bool obj = *p == '{';
      ++p;
      if (lit(close)) return true;
      do {
        if (obj) {
          std::string k;
          if (!string(&k) || !lit(':')) return fail("bad object");
        }
        if (!skip(depth + 1)) return false;
      } while (lit(','));
      return lit(close) || fail("unterminated container");
    }
    while (p < end && *p != ',' && *p != '}' && *p != ']' && *p != ' ' && *p != '\n' && *p != '\r' &&
           *p != '\t')
      ++p;  // number, true, false, null
    return true;
  }
  bool tensor(StTensor* t) {
    if (!lit('{')) return fail("tensor entry must be an object");
    bool has_dtype = false, has_shape = false, has_off = false;
    if (!lit('}')) {
      do {
        std::string k;
        if (!string(&k) || !lit(':')) return fail("bad tensor entry");
        if (k == "dtype") {
          if (!string(&t->dtype)) return false;
          has_dtype = true;
        } else if (k == "shape") {
          if (!int_array(&t->shape)) return false;
          has_shape = true;
        } else if (k == "data_offsets") {
          std::vector<int64_t> o;
          if (!int_array(&o)) return false;
          if (o.size() != 2 || o[0] < 0 || o[1] < o[0]) return fail("bad data_offsets of " + t->name);
          t->begin = (uint64_t)o[0];
          t->end = (uint64_t)o[1];
          has_off = true;
        } else if (!skip()) {
          return false;
        }
      } while (lit(','));
      if (!lit('}')) return fail("unterminated tensor entry");
    }
    if (!has_dtype || !has_shape || !has_off) return fail("tensor " + t->name + " lacks dtype, shape or offsets");
    return true;
  }
  bool header(std::vector<StTensor>* out) {
    if (!lit('{')) return fail("header must be a JSON object");
    if (lit('}')) return true;
    do {
      std::string k;
      if (!string(&k) || !lit(':')) return fail("bad header object");
      if (k == "__metadata__") {
        if (!skip()) return false;
        continue;
      }
      StTensor t;
      t.name = k;
      if (!tensor(&t)) return false;
      out->push_back(std::move(t));
    } while (lit(','));
    if (!lit('}')) return fail("unterminated header object");
    ws();
    return p == end || fail("trailing bytes after the header object");
  }
};

}  // namespace

int st_dtype_bytes(const std::string& d) {
  if (d == "F64" || d == "I64" || d == "U64") return 8;
  if (d == "F32" || d == "I32" || d == "U32") return 4;
  if (d == "F16" || d == "BF16" || d == "I16" || d == "U16") return 2;
  if (d == "I8" || d == "U8" || d == "BOOL" || d == "F8_E4M3" || d == "F8_E5M2") return 1;
  return 0;
}

bool st_read_header(const std::string& path, StFile* out, std::string* err) {
  out->path = path;
  out->tensors.clear();
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) {
    *err = path + ": cannot open";
    return false;
  }
  bool ok = false;
  do {
    if (std::fseek(f, 0, SEEK_END) != 0) { *err = path + ": cannot seek"; break; }
    const long size_l = std::ftell(f);
    if (size_l < 8) { *err = path + ": shorter than a header"; break; }
    const uint64_t size = (uint64_t)size_l;
    std::fseek(f, 0, SEEK_SET);
    unsigned char lb[8];
    if (std::fread(lb, 1, 8, f) != 8) { *err = path + ": cannot read the header length"; break; }
    uint64_t n = 0;
    for (int i = 7; i >= 0; --i) n = (n << 8) | lb[i];
    if (n == 0 || n > kMaxHeader || n > size - 8) { *err = path + ": bad header length"; break; }
    std::string json(n, '\0');
    if (std::fread(&json[0], 1, n, f) != n) { *err = path + ": cannot read the header"; break; }
    Parser ps{json.data(), json.data() + json.size(), {}};
    if (!ps.header(&out->tensors)) { *err = path + ": " + ps.err; break; }
    out->data_start = 8 + n;
    const uint64_t data_bytes = size - out->data_start;
    bool good = true;
    for (const StTensor& t : out->tensors) {
      const int eb = st_dtype_bytes(t.dtype);
      uint64_t numel = 1;
      bool dims_ok = eb > 0;
      for (int64_t d : t.shape) {
        if (d < 0 || (d > 0 && numel > UINT64_MAX / (uint64_t)d)) dims_ok = false;
        else numel *= (uint64_t)d;
      }
      if (!dims_ok) { *err = path + ": " + t.name + ": unknown dtype or bad shape"; good = false; break; }
      if (t.end > data_bytes) { *err = path + ": " + t.name + ": data past the end of the file"; good = false; break; }
      if (t.end - t.begin != numel * (uint64_t)eb) {
        *err = path + ": " + t.name + ": byte range does not match dtype and shape";
        good = false;
        break;
      }
    }
    ok = good;
  } while (false);
  std::fclose(f);
  return ok;
}

}  // namespace q3k

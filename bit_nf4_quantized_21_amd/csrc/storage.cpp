// Serialization of a quantized weight (codes, q8, s2) as a safetensors file.
//
// The stored format is deterministic (the quantizer is exact), so a saved
// weight reloads bit for bit.  Layout: an 8-byte little-endian header length,
// a JSON header padded with spaces to a multiple of 8 bytes, then the raw
// tensors: "s2" (F32), "codes" (U8), "q8" (U8), back to back.  The header's
// "__metadata__" names the format, the 4-bit type, N, K, the two block sizes
// and the type's 16-entry decode table (fp32 bit patterns), so that a file
// is refused by a library whose table differs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "storage.hpp"

namespace qlora {

namespace {

const char* kTypeNames[3] = {"nf4", "int4", "fp4"};

std::string table_hex(const float table[16]) {
  std::string s;
  char buf[16];
  for (int i = 0; i < 16; ++i) {
    uint32_t u;
    std::memcpy(&u, &table[i], 4);
    std::snprintf(buf, sizeof buf, "%s%08x", i ? "," : "", u);
    s += buf;
  }
  return s;
}

// A minimal reader for the JSON this file writes (objects, arrays, strings
// without escapes, non-negative integers); anything else fails.
struct Json {
  const std::string& t;
  size_t i = 0;
  bool ok = true;
  explicit Json(const std::string& s) : t(s) {}
  void ws() {
    while (i < t.size() && (t[i] == ' ' || t[i] == '\n' || t[i] == '\t' || t[i] == '\r')) ++i;
  }
  bool eat(char c) {
    ws();
    if (i < t.size() && t[i] == c) {
      ++i;
      return true;
    }
    return false;
  }
  std::string str() {
    ws();
    if (i >= t.size() || t[i] != '"') { ok = false; return ""; }
    const size_t j = t.find('"', i + 1);
    if (j == std::string::npos) { ok = false; return ""; }
    std::string s = t.substr(i + 1, j - i - 1);
    if (s.find('\\') != std::string::npos) ok = false;
    i = j + 1;
    return s;
  }
  int64_t num() {
    ws();
    int64_t v = 0;
    size_t n = 0;
    while (i < t.size() && t[i] >= '0' && t[i] <= '9' && n < 18) v = v * 10 + (t[i++] - '0'), ++n;
    if (n == 0) ok = false;
    return v;
  }
};

struct TensorEntry {
  std::string dtype;
  std::vector<int64_t> shape;
  int64_t begin = -1, end = -1;
};

bool parse_header(const std::string& h, std::map<std::string, std::string>* meta,
                  std::map<std::string, TensorEntry>* tensors) {
  Json j(h);
  if (!j.eat('{')) return false;
  if (j.eat('}')) return true;
  do {
    const std::string key = j.str();
    if (!j.ok || !j.eat(':') || !j.eat('{')) return false;
    if (key == "__metadata__") {
      if (!j.eat('}')) {
        do {
          const std::string k = j.str();
          if (!j.eat(':')) return false;
          (*meta)[k] = j.str();
          if (!j.ok) return false;
        } while (j.eat(','));
        if (!j.eat('}')) return false;
      }
    } else {
      TensorEntry e;
      do {
        const std::string k = j.str();
        if (!j.ok || !j.eat(':')) return false;
        if (k == "dtype") {
          e.dtype = j.str();
        } else if (k == "shape" || k == "data_offsets") {
          if (!j.eat('[')) return false;
          std::vector<int64_t> v;
          if (!j.eat(']')) {
            do v.push_back(j.num()); while (j.eat(','));
            if (!j.eat(']')) return false;
          }
          if (k == "shape") e.shape = v;
          else if (v.size() == 2) e.begin = v[0], e.end = v[1];
          else return false;
        } else {
          return false;
        }
        if (!j.ok) return false;
      } while (j.eat(','));
      if (!j.eat('}')) return false;
      (*tensors)[key] = e;
    }
  } while (j.eat(','));
  return j.eat('}') && j.ok;
}

struct Sizes {
  int64_t n2, nb, ng;
};
Sizes sizes(int64_t N, int64_t K) {
  const int64_t n = N * K, nb = (n + 63) / 64;
  return {n / 2, nb, (nb + 255) / 256};
}

}  // namespace

int save_4bit(const char* path, int qtype, const float table[16], int64_t N, int64_t K, const uint8_t* codes,
              const uint8_t* q8, const float* s2, hipStream_t stream, hipError_t* herr) {
  *herr = hipSuccess;
  const Sizes z = sizes(N, K);
  std::vector<char> data((size_t)(4 * z.ng + z.n2 + z.nb));
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(data.data(), s2, (size_t)(4 * z.ng), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(data.data() + 4 * z.ng, codes, (size_t)z.n2, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(data.data() + 4 * z.ng + z.n2, q8, (size_t)z.nb, hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    *herr = e;
    return kStorageHip;
  }
  char buf[512];
  std::string h = "{\"__metadata__\":{\"format\":\"qlora-4bit\",\"qtype\":\"";
  h += kTypeNames[qtype];
  std::snprintf(buf, sizeof buf, "\",\"N\":\"%lld\",\"K\":\"%lld\",\"blocksize\":\"64\",\"blocksize2\":\"256\",\"table\":\"",
                (long long)N, (long long)K);
  h += buf;
  h += table_hex(table);
  std::snprintf(buf, sizeof buf,
                "\"},\"s2\":{\"dtype\":\"F32\",\"shape\":[%lld],\"data_offsets\":[0,%lld]},"
                "\"codes\":{\"dtype\":\"U8\",\"shape\":[%lld],\"data_offsets\":[%lld,%lld]},"
                "\"q8\":{\"dtype\":\"U8\",\"shape\":[%lld],\"data_offsets\":[%lld,%lld]}}",
                (long long)z.ng, (long long)(4 * z.ng), (long long)z.n2, (long long)(4 * z.ng),
                (long long)(4 * z.ng + z.n2), (long long)z.nb, (long long)(4 * z.ng + z.n2),
                (long long)(4 * z.ng + z.n2 + z.nb));
  h += buf;
  while (h.size() % 8) h += ' ';
  FILE* f = std::fopen(path, "wb");
  if (!f) return kStorageIo;
  uint8_t len[8];
  for (int i = 0; i < 8; ++i) len[i] = (uint8_t)((uint64_t)h.size() >> (8 * i));
  bool good = std::fwrite(len, 1, 8, f) == 8 && std::fwrite(h.data(), 1, h.size(), f) == h.size() &&
              std::fwrite(data.data(), 1, data.size(), f) == data.size();
  good = (std::fclose(f) == 0) && good;
  return good ? kStorageOk : kStorageIo;
}

int load_4bit(const char* path, const float* const tables[3], int* qtype, int64_t* N, int64_t* K, uint8_t* codes,
              uint8_t* q8, float* s2, int expect_qtype, int64_t expect_N, int64_t expect_K, hipError_t* herr) {
  *herr = hipSuccess;
  FILE* f = std::fopen(path, "rb");
  if (!f) return kStorageIo;
  uint8_t len[8];
  std::string h;
  std::vector<char> data;
  bool good = std::fread(len, 1, 8, f) == 8;
  uint64_t hl = 0;
  for (int i = 0; i < 8 && good; ++i) hl |= (uint64_t)len[i] << (8 * i);
  good = good && hl > 0 && hl < (1u << 20);
  if (good) {
    h.resize((size_t)hl);
    good = std::fread(&h[0], 1, h.size(), f) == h.size();
  }
  std::map<std::string, std::string> meta;
  std::map<std::string, TensorEntry> ts;
  good = good && parse_header(h, &meta, &ts);
  int q = -1;
  for (int i = 0; i < 3 && good; ++i)
    if (meta["qtype"] == kTypeNames[i]) q = i;
  good = good && meta["format"] == "qlora-4bit" && q >= 0 && meta["blocksize"] == "64" && meta["blocksize2"] == "256";
  int64_t n_ = good ? std::atoll(meta["N"].c_str()) : 0, k_ = good ? std::atoll(meta["K"].c_str()) : 0;
  good = good && n_ > 0 && k_ > 0 && (n_ * k_) % 2 == 0 && n_ <= (int64_t(1) << 28) && k_ <= (int64_t(1) << 28);
  good = good && meta["table"] == table_hex(tables[q]);
  Sizes z{};
  if (good) {
    z = sizes(n_, k_);
    const TensorEntry &a = ts["s2"], &b = ts["codes"], &c = ts["q8"];
    good = ts.size() == 3 && a.dtype == "F32" && b.dtype == "U8" && c.dtype == "U8" &&
           a.shape == std::vector<int64_t>{z.ng} && b.shape == std::vector<int64_t>{z.n2} &&
           c.shape == std::vector<int64_t>{z.nb} && a.begin == 0 && a.end == 4 * z.ng && b.begin == a.end &&
           b.end == b.begin + z.n2 && c.begin == b.end && c.end == c.begin + z.nb;
  }
  if (good) {
    // The tensors must be exactly the rest of the file; checked before any
    // buffer is sized from the header, so a forged shape cannot make the
    // reader allocate more than the file holds.
    const long pos = std::ftell(f);
    good = pos > 0 && std::fseek(f, 0, SEEK_END) == 0;
    const long end = good ? std::ftell(f) : -1;
    good = good && end >= pos && std::fseek(f, pos, SEEK_SET) == 0 &&
           (int64_t)(end - pos) == 4 * z.ng + z.n2 + z.nb;
  }
  if (good) {
    data.resize((size_t)(4 * z.ng + z.n2 + z.nb));
    good = std::fread(data.data(), 1, data.size(), f) == data.size();
  }
  std::fclose(f);
  if (!good) return kStorageIo;
  *qtype = q;
  *N = n_;
  *K = k_;
  if (!codes) return kStorageOk;  // header query only
  if (q != expect_qtype || n_ != expect_N || k_ != expect_K) return kStorageMismatch;
  hipError_t e = hipMemcpy(s2, data.data(), (size_t)(4 * z.ng), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(codes, data.data() + 4 * z.ng, (size_t)z.n2, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(q8, data.data() + 4 * z.ng + z.n2, (size_t)z.nb, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    *herr = e;
    return kStorageHip;
  }
  return kStorageOk;
}

}  // namespace qlora

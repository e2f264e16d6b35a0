/*
 * Host-side checks of libqlora under AddressSanitizer (built with the host
 * part instrumented, no GPU needed): every C entry point with NULL, misaligned
 * and out-of-range arguments, the workspace-size queries across shapes, and
 * the safetensors reader on a valid file, on every truncation of it and on
 * seeded random corruptions of its header.  Nothing here reaches a kernel
 * launch: each call is refused by the host checks, or fails in the HIP
 * runtime for want of a device.  Exit status 0 means every expectation held
 * (AddressSanitizer aborts with its own report on a memory error).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qlora.h"

static int failures = 0;
#define EXPECT(cond, what)                                          \
  do {                                                              \
    if (!(cond)) {                                                  \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__);   \
      ++failures;                                                   \
    }                                                               \
  } while (0)

/* A valid file for an N x K weight of type q, written by hand in the
 * documented layout (8-byte header length, JSON header padded to 8 bytes,
 * then s2, codes, q8). */
static size_t make_file(unsigned char* buf, size_t cap, int q, int64_t N, int64_t K, int with_data) {
  static const char* names[3] = {"nf4", "int4", "fp4"};
  float table[16];
  if (qlora_4bit_table(q, table) != QLORA_OK) return 0;
  char hex[16 * 9 + 1];
  hex[0] = 0;
  for (int i = 0; i < 16; ++i) {
    uint32_t u;
    memcpy(&u, &table[i], 4);
    char b[12];
    snprintf(b, sizeof b, "%s%08x", i ? "," : "", u);
    strcat(hex, b);
  }
  const int64_t n = N * K, n2 = n / 2, nb = (n + 63) / 64, ng = (nb + 255) / 256;
  char h[2048];
  int len = snprintf(h, sizeof h,
                     "{\"__metadata__\":{\"format\":\"qlora-4bit\",\"qtype\":\"%s\",\"N\":\"%lld\",\"K\":\"%lld\","
                     "\"blocksize\":\"64\",\"blocksize2\":\"256\",\"table\":\"%s\"},"
                     "\"s2\":{\"dtype\":\"F32\",\"shape\":[%lld],\"data_offsets\":[0,%lld]},"
                     "\"codes\":{\"dtype\":\"U8\",\"shape\":[%lld],\"data_offsets\":[%lld,%lld]},"
                     "\"q8\":{\"dtype\":\"U8\",\"shape\":[%lld],\"data_offsets\":[%lld,%lld]}}",
                     names[q], (long long)N, (long long)K, hex, (long long)ng, (long long)(4 * ng), (long long)n2,
                     (long long)(4 * ng), (long long)(4 * ng + n2), (long long)nb, (long long)(4 * ng + n2),
                     (long long)(4 * ng + n2 + nb));
  while (len % 8) h[len++] = ' ';
  const size_t total = 8 + (size_t)len + (with_data ? (size_t)(4 * ng + n2 + nb) : 16);
  if (total > cap) return 0;
  for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)((uint64_t)len >> (8 * i));
  memcpy(buf + 8, h, (size_t)len);
  for (size_t i = 8 + (size_t)len; i < total; ++i) buf[i] = (unsigned char)(i * 131u);
  return total;
}

static int write_bytes(const char* path, const unsigned char* b, size_t n) {
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  const int ok = fwrite(b, 1, n, f) == n;
  return fclose(f) == 0 && ok;
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}

static void check_tables(void) {
  float t[16];
  for (int q = 0; q < 3; ++q) EXPECT(qlora_4bit_table(q, t) == QLORA_OK, "table of a known type");
  EXPECT(qlora_4bit_table(3, t) == QLORA_ERR_UNSUPPORTED, "unknown type refused");
  EXPECT(qlora_4bit_table(-1, t) == QLORA_ERR_UNSUPPORTED, "negative type refused");
  EXPECT(qlora_4bit_table(0, NULL) == QLORA_ERR_NULL, "NULL table refused");
  qlora_nf4_codebook(t);
  for (int s = -12; s <= 2; ++s) EXPECT(qlora_status_string(s) != NULL, "status string");
  char buf[8];
  EXPECT(qlora_timing_read(buf, sizeof buf) >= 0 || 1, "timing read into a short buffer");
  EXPECT(qlora_timing_read(NULL, 0) <= 0 || 1, "timing read without a buffer");
}

static void check_refusals(void) {
  /* 16-byte aligned host buffers stand in for device memory: every call
   * below must be refused before anything reads or writes them. */
  static unsigned char mem[1 << 16] __attribute__((aligned(16)));
  const uint16_t* X = (const uint16_t*)mem;
  const uint8_t* c = mem;
  float* f = (float*)mem;
  uint16_t* u = (uint16_t*)mem;
  uint8_t* w = mem;
  EXPECT(qlora_quantize_nf4(NULL, 64, 64, w, f, NULL) == QLORA_ERR_NULL, "quantize NULL W");
  EXPECT(qlora_quantize_nf4(f, 63, 64, w, f, NULL) == QLORA_ERR_SHAPE, "quantize ragged n");
  EXPECT(qlora_quantize_nf4(f, 64, 32, w, f, NULL) == QLORA_ERR_UNSUPPORTED, "quantize blocksize");
  EXPECT(qlora_quantize_nf4(f + 1, 64, 64, w, f, NULL) == QLORA_ERR_ALIGN, "quantize misaligned");
  EXPECT(qlora_quantize_4bit(f, 0, 64, 64, 7, w, f, NULL) == QLORA_ERR_UNSUPPORTED, "quantize unknown type");
  EXPECT(qlora_quantize_dq(NULL, 0, 64, 0, w, w, f, NULL) == QLORA_ERR_NULL, "fused quantize NULL");
  EXPECT(qlora_double_quant(f, -1, 256, w, f, NULL) == QLORA_ERR_SHAPE, "double quant negative count");
  EXPECT(qlora_dequantize_nf4(c, c, f, 64, 0, NULL, NULL) == QLORA_ERR_NULL, "dequantize NULL out");
  /* linear shapes: K % 64, N % 8, the rank, negative T, 31-bit views */
  const size_t ws_ok = qlora_linear_fwd_workspace_bytes(32, 512, 512, 8);
  EXPECT(ws_ok > 0, "fwd workspace of a small problem");
  EXPECT(qlora_linear_fwd(X, 32, 100, 512, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) == QLORA_ERR_SHAPE,
         "fwd K % 64");
  EXPECT(qlora_linear_fwd(X, 32, 512, 510, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) == QLORA_ERR_SHAPE,
         "fwd N % 8");
  EXPECT(qlora_linear_fwd(X, 32, 512, 512, c, c, f, X, X, 4, 16.f, u, f, mem, sizeof mem, NULL) ==
             QLORA_ERR_UNSUPPORTED, "fwd rank below 8");
  EXPECT(qlora_linear_fwd(X, 32, 512, 512, c, c, f, X, X, 136, 16.f, u, f, mem, sizeof mem, NULL) ==
             QLORA_ERR_UNSUPPORTED, "fwd rank above 128");
  EXPECT(qlora_linear_fwd(X, -1, 512, 512, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) == QLORA_ERR_SHAPE,
         "fwd negative T");
  EXPECT(qlora_linear_fwd(X, 4096, (int64_t)1 << 20, 4096, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) ==
             QLORA_ERR_SHAPE, "fwd X view past 31 bits");
  EXPECT(qlora_linear_fwd(NULL, 32, 512, 512, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) == QLORA_ERR_NULL,
         "fwd NULL X");
  EXPECT(qlora_linear_fwd(X + 1, 32, 512, 512, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) ==
             QLORA_ERR_ALIGN, "fwd misaligned X");
  EXPECT(qlora_linear_fwd(X, 32, 512, 512, c, c, f, X, X, 8, 16.f, u, f, mem, ws_ok - 1, NULL) ==
             QLORA_ERR_WORKSPACE, "fwd short workspace");
  EXPECT(qlora_linear_bwd(X, X, f, 32, 512, 512, c, c, f, X, X, 8, 16.f, u, u, u, mem, 0, NULL) ==
             QLORA_ERR_WORKSPACE, "bwd without workspace");
  EXPECT(qlora_linear_bwd(NULL, X, f, 32, 512, 512, c, c, f, X, X, 8, 16.f, u, u, u, mem, sizeof mem, NULL) ==
             QLORA_ERR_NULL, "bwd NULL dY");
  EXPECT(qlora_linear_fwd_4bit(9, X, 32, 512, 512, c, c, f, X, X, 8, 16.f, u, f, mem, sizeof mem, NULL) ==
             QLORA_ERR_UNSUPPORTED, "fwd unknown type");
  /* grouped calls: counts, NULL descriptor arrays, one bad member */
  qlora_linear_desc d[2];
  memset(d, 0, sizeof d);
  d[0].K = d[1].K = 512;
  d[0].N = d[1].N = 512;
  EXPECT(qlora_linear_fwd_grouped(0, 2, NULL, 4, 8, 16.f, mem, sizeof mem, NULL) == QLORA_ERR_NULL,
         "grouped NULL descriptors");
  EXPECT(qlora_linear_fwd_grouped(0, -1, d, 4, 8, 16.f, mem, sizeof mem, NULL) == QLORA_ERR_SHAPE,
         "grouped negative count");
  EXPECT(qlora_linear_fwd_grouped(0, 2, d, 4, 8, 16.f, mem, sizeof mem, NULL) == QLORA_ERR_NULL,
         "grouped member without pointers");
  qlora_linear_bwd_desc e[1];
  memset(e, 0, sizeof e);
  e[0].K = 512;
  e[0].N = 512;
  EXPECT(qlora_linear_bwd_grouped(0, 1, e, 4, 8, 16.f, mem, sizeof mem, NULL) == QLORA_ERR_NULL,
         "grouped backward member without pointers");
  /* optimizer */
  EXPECT(qlora_adamw_step(-1, u, f, f, f, X, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0.f, NULL, mem, sizeof mem, NULL) ==
             QLORA_ERR_SHAPE, "adamw negative count");
  EXPECT(qlora_adamw_step(64, NULL, f, f, f, X, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0.f, NULL, mem, sizeof mem,
                          NULL) == QLORA_ERR_NULL, "adamw NULL param");
  /* no-allocation forward beyond its scratch */
  EXPECT(qlora_linear_fwd_noalloc(X, 1 << 20, 8192, 8192, c, c, f, X, X, 64, 16.f, u, f, NULL) != QLORA_OK,
         "no-allocation forward beyond its scratch");
}

static void check_workspace_queries(void) {
  const int64_t Ts[] = {0, 1, 4, 16, 17, 64, 257, 512, 4096};
  const int64_t KN[][2] = {{64, 8}, {512, 520}, {4096, 4096}, {8192, 22016}, {22016, 8192}};
  const int32_t rs[] = {8, 64, 72, 128};
  for (size_t a = 0; a < sizeof Ts / sizeof *Ts; ++a)
    for (size_t b = 0; b < sizeof KN / sizeof *KN; ++b)
      for (size_t c = 0; c < sizeof rs / sizeof *rs; ++c) {
        const size_t f = qlora_linear_fwd_workspace_bytes(Ts[a], KN[b][0], KN[b][1], rs[c]);
        const size_t g = qlora_linear_bwd_workspace_bytes(Ts[a], KN[b][0], KN[b][1], rs[c]);
        EXPECT(f % 256 == 0 && g % 256 == 0, "workspace sizes in 256-byte units");
        EXPECT(f < ((size_t)1 << 40) && g < ((size_t)1 << 40), "workspace sizes bounded");
      }
  EXPECT(qlora_linear_fwd_workspace_bytes(32, 100, 512, 8) == 0, "no size for an invalid shape");
  EXPECT(qlora_adamw_workspace_bytes(0) == 0, "no optimizer workspace for nothing");
}

static void check_files(const char* dir) {
  static unsigned char good[1 << 16], bad[1 << 16];
  char path[4096];
  snprintf(path, sizeof path, "%s/w.safetensors", dir);
  int32_t q;
  int64_t N, K;
  EXPECT(qlora_load_4bit_info(NULL, &q, &N, &K) == QLORA_ERR_NULL, "info NULL path");
  snprintf(path, sizeof path, "%s/missing.safetensors", dir);
  EXPECT(qlora_load_4bit_info(path, &q, &N, &K) == QLORA_ERR_IO, "info missing file");
  snprintf(path, sizeof path, "%s/w.safetensors", dir);
  for (int t = 0; t < 3; ++t) {
    const size_t n = make_file(good, sizeof good, t, 24, 128, 1);
    EXPECT(n > 0 && write_bytes(path, good, n), "write a valid file");
    EXPECT(qlora_load_4bit_info(path, &q, &N, &K) == QLORA_OK && q == t && N == 24 && K == 128, "valid file read");
    /* every truncation, and one trailing byte too many */
    for (size_t cut = 0; cut < n; cut += (cut < 600 ? 1 : 97)) {
      EXPECT(write_bytes(path, good, cut), "write a truncation");
      EXPECT(qlora_load_4bit_info(path, &q, &N, &K) == QLORA_ERR_IO, "truncated file refused");
    }
    memcpy(bad, good, n);
    bad[n] = 0;
    EXPECT(write_bytes(path, bad, n + 1), "write a long file");
    EXPECT(qlora_load_4bit_info(path, &q, &N, &K) == QLORA_ERR_IO, "trailing bytes refused");
    /* header length fields: zero, past the file, huge */
    const uint64_t lens[] = {0, (uint64_t)n, (uint64_t)1 << 20, ~(uint64_t)0};
    for (size_t i = 0; i < 4; ++i) {
      memcpy(bad, good, n);
      for (int k = 0; k < 8; ++k) bad[k] = (unsigned char)(lens[i] >> (8 * k));
      EXPECT(write_bytes(path, bad, n), "write a bad length");
      EXPECT(qlora_load_4bit_info(path, &q, &N, &K) == QLORA_ERR_IO, "bad header length refused");
    }
    /* seeded corruptions of the header: the reader may accept a mutation
     * that leaves the header meaning the same thing, but must never read
     * outside its buffers or allocate from a forged size */
    const size_t hl = (size_t)good[0] | ((size_t)good[1] << 8);
    for (int it = 0; it < 3000; ++it) {
      memcpy(bad, good, n);
      const int edits = 1 + (int)(next_u32() % 4);
      for (int k = 0; k < edits; ++k) {
        const size_t at = 8 + next_u32() % hl;
        const uint32_t kind = next_u32() % 4;
        if (kind == 0) bad[at] = (unsigned char)next_u32();
        else if (kind == 1) bad[at] = (unsigned char)"{}[]\":,0123456789 \\"[next_u32() % 19];
        else if (kind == 2) bad[at] = '9';
        else bad[at] = '"';
      }
      EXPECT(write_bytes(path, bad, n), "write a corruption");
      const int rc = qlora_load_4bit_info(path, &q, &N, &K);
      EXPECT(rc == QLORA_OK || rc == QLORA_ERR_IO, "corruption read or refused");
      if (rc == QLORA_OK) EXPECT(N * K <= 24 * 128 * 2 && N > 0 && K > 0, "accepted mutation has a consistent shape");
    }
  }
  /* a consistent header whose tensors would be far larger than the file
   * (2^39 bytes of codes): refused from the file size, nothing allocated */
  {
    const size_t n = make_file(good, sizeof good, 0, (int64_t)1 << 20, (int64_t)1 << 20, 0);
    EXPECT(n > 0 && write_bytes(path, good, n), "write a header-only file");
    EXPECT(qlora_load_4bit_info(path, &q, &N, &K) == QLORA_ERR_IO, "oversized tensors refused");
  }
  remove(path);
}

int main(int argc, char** argv) {
  const char* dir = argc > 1 ? argv[1] : ".";
  check_tables();
  check_refusals();
  check_workspace_queries();
  check_files(dir);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_asan: all host checks passed\n");
  return 0;
}

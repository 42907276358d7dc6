// host_checks.cpp -- drives the host side of libenc (header parsing, stream
// info checks, workspace and table sizing, GEMM planning) with valid and
// corrupted inputs, in a build with AddressSanitizer and UndefinedBehavior-
// Sanitizer on the host code only (no device code is compiled, and nothing
// here launches a kernel or touches a GPU).
//
// Usage: host_checks <seed> <stream-file>...
// Each file holds (at least the 256-byte header of) a valid stream. For each
// one: the original header must parse; then many mutated headers (random
// bytes, 64-bit fields set to edge values, short buffers) are parsed, and
// every parse that succeeds is checked against the format's invariants and
// fed to the table sizing and batch preparation checks. Exit 0 when every
// check held; a sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "enc.h"

namespace {

uint64_t g_state = 0;
uint64_t next_u64() {   // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int g_failures = 0;
void expect(bool ok, const char *what, int file, int iter) {
  if (!ok) {
    ++g_failures;
    fprintf(stderr, "FAIL file %d iter %d: %s (%s)\n", file, iter, what, enc_last_error());
  }
}

const uint64_t kEdge[] = {0,           1,           15,          16,          255,
                          256,         257,         1ull << 31,  1ull << 32,  (1ull << 40) + 1,
                          1ull << 63,  ~0ull,       ~0ull - 15,  0x7FFFFFFFFFFFFFFFull};

// Invariants every accepted header satisfies.
void check_accepted(const enc_info &i, uint64_t comp_bytes, int file, int iter) {
  expect(i.version == 1, "version", file, iter);
  expect(i.dtype >= 1 && i.dtype <= 3, "dtype", file, iter);
  expect(i.total_bytes <= comp_bytes, "total within buffer", file, iter);
  if (i.flags == 1) {
    expect(i.raw_off == 256, "raw offset", file, iter);
  } else {
    expect(i.flags == 0 || i.flags == 2, "flags", file, iter);
    expect(i.sm_off == 256 && i.sm_off < i.meta_off && i.meta_off < i.segoff_off &&
               i.segoff_off < i.payload_off && i.payload_off <= i.total_bytes,
           "section order", file, iter);
    expect(i.total_bytes == i.payload_off + i.payload_bytes, "payload end", file, iter);
    expect(i.n_blocks == (i.n_elems + i.block_size - 1) / i.block_size, "block count", file, iter);
    expect(i.n_segments == (i.n_blocks + 63) / 64, "segment count", file, iter);
  }
}

void drive_info(const enc_info &i, int file, int iter) {
  // table sizing reads dtype and n_elems only; preparation validates the
  // item and must stop at the capacity check (table_bytes 0) -- before any
  // copy to the device
  enc_item it;
  memset(&it, 0, sizeof it);
  it.d_comp = reinterpret_cast<const void *>(uintptr_t(0x100000));
  it.d_out = reinterpret_cast<void *>(uintptr_t(0x200000));
  it.info = i;
  const uint64_t tb = enc_batch_table_bytes(&it, 1);
  expect(tb > 0, "table bytes", file, iter);
  enc_batch_plan plan;
  const enc_status st = enc_batch_prepare(&it, 1, reinterpret_cast<void *>(uintptr_t(0x300000)), 0,
                                          nullptr, &plan);
  expect(st == ENC_ERR_CAPACITY, "prepare stops at capacity", file, iter);
}

void mutate(std::vector<uint8_t> &h) {
  const int kind = (int)(next_u64() % 5);
  if (kind == 0) {   // a few random bytes anywhere in the header
    const int n = 1 + (int)(next_u64() % 4);
    for (int k = 0; k < n; ++k) h[next_u64() % 256] = (uint8_t)next_u64();
  } else if (kind == 1) {   // one 64-bit field to an edge value
    const int f = (int)(next_u64() % 10);
    uint64_t v = kEdge[next_u64() % (sizeof kEdge / sizeof kEdge[0])];
    memcpy(&h[24 + 8 * f], &v, 8);
  } else if (kind == 2) {   // one 64-bit field nudged
    const int f = (int)(next_u64() % 10);
    uint64_t v;
    memcpy(&v, &h[24 + 8 * f], 8);
    v += (uint64_t)((int64_t)(next_u64() % 65) - 32);
    memcpy(&h[24 + 8 * f], &v, 8);
  } else if (kind == 3) {   // version / dtype / flags / block size
    const int f = (int)(next_u64() % 4);
    const uint32_t v = (uint32_t)kEdge[next_u64() % (sizeof kEdge / sizeof kEdge[0])] ^
                       (uint32_t)(next_u64() % 8);
    if (f < 2) {
      const uint16_t w = (uint16_t)v;
      memcpy(&h[4 + 2 * f], &w, 2);
    } else {
      memcpy(&h[8 + 4 * (f - 2)], &v, 4);
    }
  } else {   // n_elems to a random value, the rest left as it was
    uint64_t v = next_u64() >> (next_u64() % 64);
    memcpy(&h[24], &v, 8);
  }
}

}  // namespace

int main(int argc, char **argv) {
  if (argc < 3) {
    fprintf(stderr, "usage: %s seed stream-file...\n", argv[0]);
    return 2;
  }
  g_state = strtoull(argv[1], nullptr, 0);
  int accepted = 0, rejected = 0;
  for (int fi = 2; fi < argc; ++fi) {
    FILE *f = fopen(argv[fi], "rb");
    if (!f) {
      fprintf(stderr, "cannot open %s\n", argv[fi]);
      return 2;
    }
    std::vector<uint8_t> orig(256, 0);
    const size_t got = fread(orig.data(), 1, 256, f);
    fseek(f, 0, SEEK_END);
    const uint64_t comp_bytes = (uint64_t)ftell(f);
    fclose(f);
    if (got != 256) {
      fprintf(stderr, "%s: short file\n", argv[fi]);
      return 2;
    }
    enc_info info;
    expect(enc_parse_header(orig.data(), 256, comp_bytes, &info) == ENC_OK, "original parses", fi, -1);
    check_accepted(info, comp_bytes, fi, -1);
    drive_info(info, fi, -1);
    // short and NULL buffers
    expect(enc_parse_header(orig.data(), 255, comp_bytes, &info) == ENC_ERR_INVALID_ARG, "short header", fi, -1);
    expect(enc_parse_header(nullptr, 256, comp_bytes, &info) == ENC_ERR_INVALID_ARG, "NULL header", fi, -1);
    expect(enc_parse_header(orig.data(), 256, comp_bytes - 1, &info) != ENC_OK, "short stream", fi, -1);
    for (int it = 0; it < 20000; ++it) {
      std::vector<uint8_t> h = orig;
      const int rounds = 1 + (int)(next_u64() % 3);
      for (int r = 0; r < rounds; ++r) mutate(h);
      // a heap copy of exactly 256 bytes, so any read past it is reported
      uint8_t *buf = static_cast<uint8_t *>(malloc(256));
      memcpy(buf, h.data(), 256);
      const uint64_t cb = (next_u64() & 1) ? comp_bytes : kEdge[next_u64() % (sizeof kEdge / sizeof kEdge[0])];
      enc_info mi;
      memset(&mi, 0xA5, sizeof mi);
      const enc_status st = enc_parse_header(buf, 256, cb, &mi);
      free(buf);
      if (st == ENC_OK) {
        ++accepted;
        check_accepted(mi, cb, fi, it);
        drive_info(mi, fi, it);
      } else {
        ++rejected;
        expect(st == ENC_ERR_BAD_STREAM || st == ENC_ERR_UNSUPPORTED, "rejection status", fi, it);
        expect(enc_last_error()[0] != 0, "rejection message", fi, it);
      }
    }
  }
  // sizing functions over edge arguments (no launches)
  const uint32_t blocks[] = {0, 1, 64, 127, 128, 512, 4096, 8192, 0xFFFFFFFFu};
  for (uint64_t n : kEdge)
    for (uint32_t b : blocks) {
      (void)enc_compress_bound(n);
      for (uint32_t dt = 0; dt < 5; ++dt) (void)enc_compress_bound_dt(n, dt);
      (void)enc_compress_workspace_bytes(n, b);
      enc_citem ci;
      memset(&ci, 0, sizeof ci);
      ci.n_elems = n;
      (void)enc_compress_batch_workspace_bytes(&ci, 1, b);
    }
  const uint32_t dims[] = {0, 1, 2, 3, 8, 16, 100, 128, 512, 4096, 14336, 65536, 1u << 20, 0xFFFFFFFFu};
  for (uint32_t M : dims)
    for (uint32_t K : dims)
      for (uint32_t N : dims)
        for (uint32_t b : blocks) {
          (void)enc_gemm_workspace_bytes(M, K, N, b);
          (void)enc_gemm_nt_workspace_bytes(M, K, N, b);
        }
  for (int s = -8; s <= 7; ++s) expect(enc_status_string((enc_status)s) != nullptr, "status string", 0, s);
  expect(enc_batch_table_bytes(nullptr, 1) == 0, "NULL items", 0, 0);
  expect(enc_batch_table_bytes(nullptr, -1) == 0, "negative count", 0, 0);
  printf("accepted %d rejected %d failures %d\n", accepted, rejected, g_failures);
  return g_failures ? 1 : 0;
}

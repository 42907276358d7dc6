// noalloc.hip -- enc_decompress_gemm for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).
//
// The fused GEMM's workspace -- per-strip arrival counters, which must be
// zero before a call and which every call leaves at zero, then the split-K
// partial slices -- comes from `scratch`, a file-scope device array of
// fixed size, instead of from the caller. Every device the library runs on
// holds its own copy of the array from module load (zero-filled) until the
// process ends, at its own address. Host code never uses the array's name as
// a device address: the address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device. A
// shape whose workspace would exceed the array is refused before anything
// is launched. Calls on one device share the array, so calls that overlap in
// time on one device race.
#include "enc_common.h"

#include <mutex>

namespace {
constexpr uint64_t kScratchBytes = 64ull << 20;
}

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];

// Device address of `scratch` on the current device.
enc_status current_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return enc::set_error(ENC_ERR_HIP, "current device query: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return enc::set_error(ENC_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table covers",
                          dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return enc::set_error(ENC_ERR_HIP, "scratch address lookup: %s", hipGetErrorString(e));
    if (!p) return enc::set_error(ENC_ERR_HIP, "scratch address lookup returned NULL");
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return ENC_OK;
}

}  // namespace

extern "C" uint64_t enc_gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" enc_status enc_decompress_gemm_noalloc(const uint16_t *d_x, uint32_t M, uint32_t K,
                                                  const void *d_wcomp, const enc_info *h_winfo,
                                                  uint32_t N, float *d_y, void *stream) {
  enc::set_error(ENC_OK, "%s", "");
  if (!h_winfo) return enc::set_error(ENC_ERR_INVALID_ARG, "h_winfo is NULL");
  const uint64_t need = enc_gemm_workspace_bytes(M, K, N, h_winfo->block_size);
  if (need > kScratchBytes)
    return enc::set_error(ENC_ERR_CAPACITY,
                          "M=%u K=%u N=%u needs a %llu-byte workspace, more than the %llu bytes of "
                          "static scratch", M, K, N, (unsigned long long)need,
                          (unsigned long long)kScratchBytes);
  void *ws = nullptr;
  const enc_status st = current_scratch(&ws);
  if (st != ENC_OK) return st;
  return enc_decompress_gemm(d_x, M, K, d_wcomp, h_winfo, N, d_y, ws, kScratchBytes, stream);
}

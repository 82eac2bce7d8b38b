// Streaming bandwidth probes: read-only, write-only and copy kernels, one 16-byte vector per thread, one block per 2-16 KiB chunk.
// They measure what HBM sustains for a given read/write mix; the dispatch
// engine's row-moving kernels are compared against these rates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_hbm_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int TPB>
__global__ __launch_bounds__(TPB) void read_probe(const u32x4* __restrict__ src, int64_t nvec,
                                                  uint32_t* sink) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
  if (i >= nvec) return;
  const u32x4 v = __builtin_nontemporal_load(src + i);
  const uint32_t acc = v.x ^ v.y ^ v.z ^ v.w;
  if (acc == 0x9E3779B9u) *sink = acc;  // keeps the load; practically never taken
}

template <int TPB>
__global__ __launch_bounds__(TPB) void write_probe(u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
  if (i >= nvec) return;
  const u32x4 v = {static_cast<uint32_t>(blockIdx.x), threadIdx.x, 0x5A5A5A5Au, 1u};
  __builtin_nontemporal_store(v, dst + i);
}

template <int TPB>
__global__ __launch_bounds__(TPB) void copy_probe(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
  if (i >= nvec) return;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

template <int TPB>
int launch(int mode, const u32x4* src, u32x4* dst, int64_t nvec, uint32_t* sink, hipStream_t s) {
  const int64_t blocks = (nvec + TPB - 1) / TPB;
  if (blocks > INT32_MAX) return -2;
  const unsigned nb = static_cast<unsigned>(blocks);
  if (mode == 0)
    read_probe<TPB><<<nb, TPB, 0, s>>>(src, nvec, sink);
  else if (mode == 1)
    write_probe<TPB><<<nb, TPB, 0, s>>>(dst, nvec);
  else
    copy_probe<TPB><<<nb, TPB, 0, s>>>(src, dst, nvec);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

extern "C" int moe_probe_stream(int mode, int shape, const void* src, void* dst, int64_t bytes,
                                uint32_t* sink, void* stream) {
  if (mode < 0 || mode > 2 || shape < 0 || shape > 3 || bytes <= 0 || bytes % 16 != 0) return -2;
  if ((mode != 1 && src == nullptr) || (mode != 0 && dst == nullptr) ||
      (mode == 0 && sink == nullptr))
    return -1;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -4;
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  const int64_t nvec = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (shape) {
    case 0: return launch<256>(mode, s, d, nvec, sink, st);
    case 1: return launch<512>(mode, s, d, nvec, sink, st);
    case 2: return launch<1024>(mode, s, d, nvec, sink, st);
    default: return launch<128>(mode, s, d, nvec, sink, st);
  }
}

// Streaming bandwidth probes: read-only, write-only, copy, fan-out and fan-in
// kernels, one 16-byte vector per thread, one block per 2-16 KiB chunk.  They
// measure what HBM sustains for a given read/write mix; the dispatch engine's
// row-moving kernels are compared against these rates.  The fan-out probe is
// the dense ideal of a permute: every vector read once and stored to F
// destination regions, each written front to back.  The fan-in probe is the
// dense ideal of a combine: F source regions read front to back, folded, and
// one region written.
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

// dst holds F regions of nvec vectors, `stride` vectors apart; vector i goes
// to i of every region.
template <int TPB>
__global__ __launch_bounds__(TPB) void fanout_probe(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, int64_t nvec,
                                                    int64_t stride, int fan) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
  if (i >= nvec) return;
  const u32x4 v = __builtin_nontemporal_load(src + i);
  for (int f = 0; f < fan; ++f) __builtin_nontemporal_store(v, dst + f * stride + i);
}

// cap > 0: each block reserves LDS it does not use, so that a CU holds at
// most `cap` of them (160 KiB of LDS per CU on gfx950).
// src holds F regions of nvec vectors, `stride` vectors apart; dst[i] is the
// XOR of vector i of every region (the fold keeps every load).
template <int TPB>
__global__ __launch_bounds__(TPB) void fanin_probe(const u32x4* __restrict__ src, int64_t stride,
                                                   u32x4* __restrict__ dst, int64_t nvec,
                                                   int fan) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
  if (i >= nvec) return;
  u32x4 acc = __builtin_nontemporal_load(src + i);
  for (int f = 1; f < fan; ++f) acc ^= __builtin_nontemporal_load(src + f * stride + i);
  __builtin_nontemporal_store(acc, dst + i);
}

template <int TPB>
int launch_fanin(const u32x4* src, int64_t stride, u32x4* dst, int64_t nvec, int fan, int cap,
                 hipStream_t s) {
  const int64_t blocks = (nvec + TPB - 1) / TPB;
  if (blocks > INT32_MAX) return -2;
  const unsigned lds = cap > 0 ? ((160u * 1024u) / static_cast<unsigned>(cap)) & ~1023u : 0u;
  fanin_probe<TPB><<<static_cast<unsigned>(blocks), TPB, lds, s>>>(src, stride, dst, nvec, fan);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <int TPB>
int launch_fanout(const u32x4* src, u32x4* dst, int64_t nvec, int64_t stride, int fan, int cap,
                  hipStream_t s) {
  const int64_t blocks = (nvec + TPB - 1) / TPB;
  if (blocks > INT32_MAX) return -2;
  const unsigned lds = cap > 0 ? ((160u * 1024u) / static_cast<unsigned>(cap)) & ~1023u : 0u;
  fanout_probe<TPB><<<static_cast<unsigned>(blocks), TPB, lds, s>>>(src, dst, nvec, stride, fan);
  return hipGetLastError() == hipSuccess ? 0 : -6;
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

extern "C" int moe_probe_fanout(int shape, const void* src, void* dst, int64_t bytes,
                                int64_t region_stride, int fan, int cap, void* stream) {
  if (shape < 0 || shape > 3 || bytes <= 0 || bytes % 16 != 0 || region_stride < bytes ||
      region_stride % 16 != 0 || fan < 1 || fan > 64 || cap < 0 || cap == 1 || cap > 32)
    return -2;
  if (src == nullptr || dst == nullptr) return -1;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -4;
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  const int64_t nvec = bytes / 16, stride = region_stride / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (shape) {
    case 0: return launch_fanout<256>(s, d, nvec, stride, fan, cap, st);
    case 1: return launch_fanout<512>(s, d, nvec, stride, fan, cap, st);
    case 2: return launch_fanout<1024>(s, d, nvec, stride, fan, cap, st);
    default: return launch_fanout<128>(s, d, nvec, stride, fan, cap, st);
  }
}

extern "C" int moe_probe_fanin(int shape, const void* src, int64_t region_stride, void* dst,
                               int64_t bytes, int fan, int cap, void* stream) {
  if (shape < 0 || shape > 3 || bytes <= 0 || bytes % 16 != 0 || region_stride < bytes ||
      region_stride % 16 != 0 || fan < 1 || fan > 64 || cap < 0 || cap == 1 || cap > 32)
    return -2;
  if (src == nullptr || dst == nullptr) return -1;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -4;
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  const int64_t nvec = bytes / 16, stride = region_stride / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (shape) {
    case 0: return launch_fanin<256>(s, stride, d, nvec, fan, cap, st);
    case 1: return launch_fanin<512>(s, stride, d, nvec, fan, cap, st);
    case 2: return launch_fanin<1024>(s, stride, d, nvec, fan, cap, st);
    default: return launch_fanin<128>(s, stride, d, nvec, fan, cap, st);
  }
}

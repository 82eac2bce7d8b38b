/*
 * moe_hbm_probe.h -- streaming bandwidth probes for gfx950 (MI355X).
 *
 * A measurement aid beside the dispatch engine, not part of its path: plain
 * streaming kernels whose sustained rates bound what HBM gives a kernel with
 * a given read/write mix, so that each row-moving kernel of the engine can
 * be placed against a measured ceiling as well as the nominal 8 TB/s peak.
 * Built as libmoe_hbm_probe.so; loaded only by the benchmark.
 *
 * moe_probe_stream(mode, shape, src, dst, bytes, sink, stream):
 *   mode 0  read:    every 16-byte vector of src[0, bytes) is loaded
 *                    (nontemporal) and folded into a value that is stored to
 *                    *sink only if it equals a fixed constant, so the loads
 *                    cannot be removed;
 *   mode 1  write:   dst[0, bytes) is filled (nontemporal stores);
 *   mode 2  copy:    dst[0, bytes) = src[0, bytes).
 *   shape   threads per block, each moving one vector: 0 -> 256 (4 KiB per
 *           block), 1 -> 512 (8 KiB), 2 -> 1024 (16 KiB), 3 -> 128 (2 KiB).
 *   bytes   a positive multiple of 16; src, dst 16-byte aligned device
 *           pointers (src unused by mode 1, dst by mode 0); sink an int32
 *           device word (mode 0).
 * Returns 0, -1 (null pointer), -2 (bad mode, shape or size), -4
 * (alignment) or -6 (launch failed).  Enqueued on `stream` (a hipStream_t).
 *
 * moe_probe_fanout(shape, src, dst, bytes, region_stride, fan, cap, stream):
 *   the dense ideal of a permute with `fan` destinations per row: every
 *   16-byte vector i of src[0, bytes) is loaded once (nontemporal) and stored
 *   (nontemporal) to vector i of each of `fan` regions of dst, region f being
 *   dst[f*region_stride, f*region_stride + bytes).  region_stride >= bytes, a
 *   multiple of 16 (a stride that is not a power of two keeps the regions'
 *   same offsets off the same HBM channels, as the permute's irregular
 *   segment offsets do); dst must hold (fan-1)*region_stride + bytes bytes
 *   and must not overlap src.  shape as above; 1 <= fan <= 64.  cap = 0
 *   leaves residency to the hardware; 2 <= cap <= 32 makes each block reserve
 *   160 KiB / cap of LDS it does not use, so that a CU holds at most cap
 *   blocks (how many write streams are open per CU is what sets the rate of
 *   fan-out writes).  Same return codes; enqueued on `stream`.
 *
 * moe_probe_fanin(shape, src, region_stride, dst, bytes, fan, cap, stream):
 *   the dense ideal of a combine over `fan` rows per output row: vector i of
 *   dst[0, bytes) is stored (nontemporal) as the XOR of vector i of each of
 *   `fan` regions of src, region f being src[f*region_stride,
 *   f*region_stride + bytes), each loaded once (nontemporal).  src must hold
 *   (fan-1)*region_stride + bytes bytes and must not overlap dst; the other
 *   arguments and the return codes as for moe_probe_fanout.
 */
#ifndef MOE_HBM_PROBE_H
#define MOE_HBM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int moe_probe_stream(int mode, int shape, const void* src, void* dst, int64_t bytes,
                     uint32_t* sink, void* stream);
int moe_probe_fanout(int shape, const void* src, void* dst, int64_t bytes,
                     int64_t region_stride, int fan, int cap, void* stream);
int moe_probe_fanin(int shape, const void* src, int64_t region_stride, void* dst, int64_t bytes,
                    int fan, int cap, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_HBM_PROBE_H */

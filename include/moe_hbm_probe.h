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
 */
#ifndef MOE_HBM_PROBE_H
#define MOE_HBM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int moe_probe_stream(int mode, int shape, const void* src, void* dst, int64_t bytes,
                     uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_HBM_PROBE_H */

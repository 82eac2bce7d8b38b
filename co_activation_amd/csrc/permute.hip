// Row scatter into rank-contiguous send buffers: the dispatched hidden
// states of "Training Communication-Efficient Mixture-of-Experts Language
// Models with Layer Re-Configuration" (footnote 3), sent once per destination
// rank as in "Expert Coupling in MoE Pretraining ..." (abstract).
//
// Token-major: a group of threads owns one token, reads its row once and
// writes it to each of its (<= 8) destination rows.  The destination list is
// uniform per token and lives in scalar registers; every store instruction of
// a wave writes 64 x 16 contiguous bytes.  HBM-bound: algorithmic bytes per
// token are row_bytes * (1 + destinations) + 4 * width.
//
// Row gather (moe_gather): the destination-ordered form for maps in which
// every output row has exactly one source -- the token shuffle's move into
// the predicted order and the expansion of received rows into expert rows.
// Output rows are written in order (one dense write front), sources are
// gathered; on MI355X this beats the scatter form for such maps.
//
// Shuffle dispatch (moe_shuffle_dispatch): the token shuffle's move and the
// next layer's permute in one pass, in the shuffled order, reading each row
// once ("Expert Coupling in MoE Pretraining ...", abstract: tokens are moved
// toward the rank forecast for their next-layer experts, then dispatched).
#include "common.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPermThreads = 256;

template <bool NT, typename V>
__device__ __forceinline__ V load_row(const V* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// TPT threads own one token (TPT = 64: four tokens per 256-thread block;
// TPT >= 256: one token per block).  Each thread loads U vectors of the row
// (stride TPT), then stores them to every destination of the token.  Loads
// are plain (the row is read once; the caches may keep it for the next
// destination), stores are nontemporal (send rows are not re-read here).
// ONE: exactly one destination per token (a token move such as the shuffle).
template <typename V, int TPT, int U, bool ONE>
__global__ __launch_bounds__(TPT < kPermThreads ? kPermThreads : TPT) void permute_kernel(
    const V* __restrict__ x, int T, int64_t vec_per_row, const int32_t* __restrict__ dest,
    int width, V* __restrict__ out, int64_t out_rows, const int32_t* __restrict__ n_valid,
    int32_t* d_err) {
  constexpr int kBlock = TPT < kPermThreads ? kPermThreads : TPT;
  constexpr int kTokens = kBlock / TPT;
  const int sub = kTokens == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / TPT);
  const int t = blockIdx.x * kTokens + sub;
  if (t >= T || (n_valid != nullptr && t >= *n_valid)) return;
  const int l = kTokens == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x % TPT);

  // Destination rows (uniform per token); -1 marks an absent or rejected one.
  int drow[MOE_MAX_K];
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) drow[q] = -1;
  int nd = 0;
  int errbits = 0;
#pragma unroll
  for (int q = 0; q < (ONE ? 1 : MOE_MAX_K); ++q) {
    drow[q] = -1;
    if (q < width) {
      const int r = __builtin_amdgcn_readfirstlane(dest[static_cast<int64_t>(t) * width + q]);
      if (r >= 0 && r < out_rows) {
        drow[q] = r;
        ++nd;
      } else if (r >= out_rows) {
        errbits = MOE_DERR_ROW_RANGE;
      }
    }
  }
  if (l == 0) report(d_err, errbits);
  if (nd == 0) return;

  const V* src = x + static_cast<int64_t>(t) * vec_per_row;
  for (int64_t c0 = l; c0 < vec_per_row; c0 += TPT * U) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * TPT;
      if (c < vec_per_row) v[u] = load_row<false>(src + c);
    }
#pragma unroll
    for (int q = 0; q < (ONE ? 1 : MOE_MAX_K); ++q) {
      if (q >= width) break;
      if (drow[q] < 0) continue;
      V* dst = out + static_cast<int64_t>(drow[q]) * vec_per_row;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * TPT;
        if (c < vec_per_row) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
}

// Rows narrower than one wave's width of vectors: one thread per
// (token, vector), so every lane moves data.
template <typename V>
__global__ __launch_bounds__(kPermThreads) void permute_flat_kernel(
    const V* __restrict__ x, int T, int vec_per_row, const int32_t* __restrict__ dest, int width,
    V* __restrict__ out, int64_t out_rows, const int32_t* __restrict__ n_valid, int32_t* d_err) {
  const int limit = n_valid != nullptr ? min(T, max(*n_valid, 0)) : T;
  const int64_t n = static_cast<int64_t>(limit) * vec_per_row;
  int errbits = 0;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kPermThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kPermThreads) {
    const int t = static_cast<int>(i / vec_per_row);
    const int c = static_cast<int>(i - static_cast<int64_t>(t) * vec_per_row);
    const V v = __builtin_nontemporal_load(x + i);
    for (int q = 0; q < width; ++q) {
      const int r = dest[static_cast<int64_t>(t) * width + q];
      if (r >= 0 && r < out_rows)
        __builtin_nontemporal_store(v, out + static_cast<int64_t>(r) * vec_per_row + c);
      else if (r >= out_rows)
        errbits = MOE_DERR_ROW_RANGE;
    }
  }
  report(d_err, errbits);
}

// Wide rows: a row is cut into parts of kPartVec vectors (2 KiB of 16-byte
// vectors) and one block of kPartVec threads (two waves, one vector per
// lane) moves one part of one token's row: block b takes token b / parts,
// part b % parts.  The row piece is loaded once and stored to every
// destination with nontemporal 16-byte stores.
//
// How many such blocks a CU holds at once sets how many write streams are
// open, and HBM absorbs the scattered writes best with about 96 of them per
// CU (waves times the places each row goes).  Blocks therefore reserve LDS
// they do not use so that a CU holds about 48 / writes of them (see
// parts_lds_bytes).  Measured on MI355X (stage medians of the benchmark
// step, cold caches): 14 KiB rows to up to 8 ranks 686 -> 646 us against a
// wave per 2 KiB part with no cap; 8 KiB rows to up to 6 ranks 507 -> 499 us
// against 256-thread blocks per token capped at two per CU.  Other part
// sizes (1-16 KiB) and caps were slower.
constexpr int kPartWaves = 2;
constexpr int kPartVec = kPartWaves * kWave;
constexpr unsigned kLdsPerCu = 160 * 1024;

// LDS reserved per block so that a CU holds about 48 / writes part blocks;
// none once that reaches the CU's 16 two-wave blocks.
inline unsigned parts_lds_bytes(int writes) {
  const int blocks = 48 / (writes < 1 ? 1 : writes);
  if (blocks >= 16) return 0;
  return (kLdsPerCu / static_cast<unsigned>(blocks < 2 ? 2 : blocks)) & ~1023u;
}

template <typename V>
__global__ __launch_bounds__(kPartVec) void permute_parts_kernel(
    const V* __restrict__ x, int T, int64_t vec_per_row, int parts,
    const int32_t* __restrict__ dest, int width, V* __restrict__ out, int64_t out_rows,
    const int32_t* __restrict__ n_valid, int32_t* d_err) {
  const int t = static_cast<int>(blockIdx.x / static_cast<unsigned>(parts));
  const int part = static_cast<int>(blockIdx.x - static_cast<unsigned>(t) * parts);
  if (t >= T || (n_valid != nullptr && t >= *n_valid)) return;
  int drow[MOE_MAX_K];
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q)
    drow[q] = q < width ? __builtin_amdgcn_readfirstlane(dest[static_cast<int64_t>(t) * width + q])
                        : -1;
  const int64_t c = static_cast<int64_t>(part) * kPartVec + threadIdx.x;
  if (c >= vec_per_row) return;
  const V v = load_row<false>(x + static_cast<int64_t>(t) * vec_per_row + c);
  int errbits = 0;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    if (q >= width) break;
    if (drow[q] < 0) continue;
    if (drow[q] >= out_rows) {
      errbits = MOE_DERR_ROW_RANGE;
      continue;
    }
    __builtin_nontemporal_store(v, out + static_cast<int64_t>(drow[q]) * vec_per_row + c);
  }
  if (threadIdx.x == 0 && part == 0) report(d_err, errbits);
}

template <typename V>
int launch_parts(const void* x, int T, int64_t vec_per_row, const int32_t* dest, int width,
                 void* out, int64_t out_rows, const int32_t* n_valid, int32_t* d_err,
                 hipStream_t s) {
  const int64_t parts = (vec_per_row + kPartVec - 1) / kPartVec;
  if (parts > INT32_MAX || !grid_ok(static_cast<int64_t>(T) * parts, kPartVec)) return MOE_ERR_SHAPE;
  permute_parts_kernel<V>
      <<<static_cast<unsigned>(static_cast<int64_t>(T) * parts), kPartVec, parts_lds_bytes(width),
         s>>>(static_cast<const V*>(x), T, vec_per_row, static_cast<int>(parts), dest, width,
              static_cast<V*>(out), out_rows, n_valid, d_err);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <typename V, int TPT, int U>
int launch_rows(const void* x, int T, int64_t vec_per_row, const int32_t* dest, int width,
                void* out, int64_t out_rows, const int32_t* n_valid, int32_t* d_err,
                hipStream_t s) {
  constexpr int kBlock = TPT < kPermThreads ? kPermThreads : TPT;
  constexpr int kTokens = kBlock / TPT;
  const int64_t nb = (static_cast<int64_t>(T) + kTokens - 1) / kTokens;
  if (!grid_ok(nb, kBlock)) return MOE_ERR_SHAPE;
  const unsigned blocks = static_cast<unsigned>(nb);
  if (width == 1)
    permute_kernel<V, TPT, U, true><<<blocks, kBlock, 0, s>>>(
        static_cast<const V*>(x), T, vec_per_row, dest, width, static_cast<V*>(out), out_rows,
        n_valid, d_err);
  else
    permute_kernel<V, TPT, U, false><<<blocks, kBlock, 0, s>>>(
        static_cast<const V*>(x), T, vec_per_row, dest, width, static_cast<V*>(out), out_rows,
        n_valid, d_err);
  return MOE_OK;
}

// Launch shape by row size (vectors per row R) and destinations per token
// (width), as measured on MI355X:
//   R < 64                 one thread per (token, vector)
//   64 <= R < 256          one wave per token, 4 vectors per lane per pass
//   384 < R <= 512 and at most 2 destinations
//                          512 threads per token, one vector each
//   R > 384 otherwise      two-wave blocks per 2 KiB part, residency capped
//                          by the destinations (permute_parts_kernel)
//   otherwise              256 threads per token, one vector per pass
template <typename V>
int launch_permute(const void* x, int T, int64_t vec_per_row, const int32_t* dest, int width,
                   void* out, int64_t out_rows, const int32_t* n_valid, int32_t* d_err,
                   hipStream_t s) {
  if (vec_per_row < kWave) {
    const int64_t n = static_cast<int64_t>(T) * vec_per_row;
    int64_t blocks = (n + kPermThreads - 1) / kPermThreads;
    if (blocks > 8192) blocks = 8192;
    permute_flat_kernel<V><<<static_cast<unsigned>(blocks), kPermThreads, 0, s>>>(
        static_cast<const V*>(x), T, static_cast<int>(vec_per_row), dest, width,
        static_cast<V*>(out), out_rows, n_valid, d_err);
  } else if (vec_per_row < 256) {
    const int rc = launch_rows<V, 64, 4>(x, T, vec_per_row, dest, width, out, out_rows, n_valid,
                                         d_err, s);
    if (rc != MOE_OK) return rc;
  } else if (vec_per_row > 384 && vec_per_row <= 512 && width <= 2) {
    const int rc = launch_rows<V, 512, 1>(x, T, vec_per_row, dest, width, out, out_rows, n_valid,
                                          d_err, s);
    if (rc != MOE_OK) return rc;
  } else if (vec_per_row > 384) {
    return launch_parts<V>(x, T, vec_per_row, dest, width, out, out_rows, n_valid, d_err, s);
  } else {
    const int rc = launch_rows<V, 256, 1>(x, T, vec_per_row, dest, width, out, out_rows, n_valid,
                                          d_err, s);
    if (rc != MOE_OK) return rc;
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

// ------------------------------------------------------------ row gather

// TPT threads own one output row: out[i] = x[src[i]].  A negative source
// leaves the row untouched; a source past x_rows is reported and skipped.
template <typename V, int TPT, int U>
__global__ __launch_bounds__(TPT < kPermThreads ? kPermThreads : TPT) void gather_kernel(
    const V* __restrict__ x, int64_t x_rows, int64_t vec_per_row, const int32_t* __restrict__ src,
    int n_rows, V* __restrict__ out, const int32_t* __restrict__ n_valid, int32_t* d_err) {
  constexpr int kBlock = TPT < kPermThreads ? kPermThreads : TPT;
  constexpr int kRows = kBlock / TPT;
  const int sub = kRows == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / TPT);
  const int i = blockIdx.x * kRows + sub;
  if (i >= n_rows || (n_valid != nullptr && i >= *n_valid)) return;
  const int l = kRows == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x % TPT);
  const int s = __builtin_amdgcn_readfirstlane(src[i]);
  if (s < 0) return;
  if (s >= x_rows) {
    if (l == 0) report(d_err, MOE_DERR_ROW_RANGE);
    return;
  }
  const V* a = x + static_cast<int64_t>(s) * vec_per_row;
  V* b = out + static_cast<int64_t>(i) * vec_per_row;
  for (int64_t c0 = l; c0 < vec_per_row; c0 += TPT * U) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * TPT;
      if (c < vec_per_row) v[u] = load_row<false>(a + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * TPT;
      if (c < vec_per_row) __builtin_nontemporal_store(v[u], b + c);
    }
  }
}

// Rows narrower than one wave's width of vectors: one thread per
// (output row, vector).
template <typename V>
__global__ __launch_bounds__(kPermThreads) void gather_flat_kernel(
    const V* __restrict__ x, int64_t x_rows, int vec_per_row, const int32_t* __restrict__ src,
    int n_rows, V* __restrict__ out, const int32_t* __restrict__ n_valid, int32_t* d_err) {
  const int limit = n_valid != nullptr ? min(n_rows, max(*n_valid, 0)) : n_rows;
  const int64_t n = static_cast<int64_t>(limit) * vec_per_row;
  int errbits = 0;
  for (int64_t q = blockIdx.x * static_cast<int64_t>(kPermThreads) + threadIdx.x; q < n;
       q += static_cast<int64_t>(gridDim.x) * kPermThreads) {
    const int i = static_cast<int>(q / vec_per_row);
    const int c = static_cast<int>(q - static_cast<int64_t>(i) * vec_per_row);
    const int s = src[i];
    if (s >= 0 && s < x_rows)
      __builtin_nontemporal_store(x[static_cast<int64_t>(s) * vec_per_row + c], out + q);
    else if (s >= x_rows)
      errbits = MOE_DERR_ROW_RANGE;
  }
  report(d_err, errbits);
}

// Launch shape by row size R (vectors): one thread per (row, vector) below
// 64; a wave per row below 256 (4 vectors per lane per pass); 512 threads
// per row above (measured best for 8 KiB and 14 KiB rows).
template <typename V>
int launch_gather(const void* x, int64_t x_rows, int64_t vec_per_row, const int32_t* src,
                  int n_rows, void* out, const int32_t* n_valid, int32_t* d_err, hipStream_t s) {
  const V* xv = static_cast<const V*>(x);
  V* ov = static_cast<V*>(out);
  if (vec_per_row < kWave) {
    const int64_t n = static_cast<int64_t>(n_rows) * vec_per_row;
    int64_t blocks = (n + kPermThreads - 1) / kPermThreads;
    if (blocks > 8192) blocks = 8192;
    gather_flat_kernel<V><<<static_cast<unsigned>(blocks), kPermThreads, 0, s>>>(
        xv, x_rows, static_cast<int>(vec_per_row), src, n_rows, ov, n_valid, d_err);
  } else if (vec_per_row < 256) {
    constexpr int kRows = kPermThreads / 64;
    const int64_t nb = (static_cast<int64_t>(n_rows) + kRows - 1) / kRows;
    if (!grid_ok(nb, kPermThreads)) return MOE_ERR_SHAPE;
    gather_kernel<V, 64, 4><<<static_cast<unsigned>(nb), kPermThreads, 0, s>>>(
        xv, x_rows, vec_per_row, src, n_rows, ov, n_valid, d_err);
  } else {
    if (!grid_ok(n_rows, 512)) return MOE_ERR_SHAPE;
    gather_kernel<V, 512, 1><<<static_cast<unsigned>(n_rows), 512, 0, s>>>(
        xv, x_rows, vec_per_row, src, n_rows, ov, n_valid, d_err);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

// ------------------------------------------------- shuffle + dispatch

// The token shuffle's move and the next layer's dispatch in one pass, in
// the shuffled order: TPT threads own position p, read the row of token
// t = perm[p] once and write it to x_out[p] and to the send rows
// token_rows[p][*].  Writes stay in few dense streams (x_out in order, the
// send rows of one source rank's positions in G blocks); the reads gather.
template <typename V, int TPT, int U>
__global__ __launch_bounds__(TPT < kPermThreads ? kPermThreads : TPT) void shuffle_dispatch_kernel(
    const V* __restrict__ x, int T, int64_t vec_per_row, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ token_rows, int k, V* __restrict__ x_out, V* __restrict__ send,
    int64_t send_rows, int32_t* d_err) {
  constexpr int kBlock = TPT < kPermThreads ? kPermThreads : TPT;
  constexpr int kTokens = kBlock / TPT;
  const int sub = kTokens == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / TPT);
  const int p = blockIdx.x * kTokens + sub;
  if (p >= T) return;
  const int l = kTokens == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x % TPT);
  const int t = __builtin_amdgcn_readfirstlane(perm[p]);
  if (t < 0 || t >= T) {
    if (l == 0) report(d_err, MOE_DERR_ROW_RANGE);
    return;
  }
  int drow[MOE_MAX_K];
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q)
    drow[q] = q < k ? __builtin_amdgcn_readfirstlane(token_rows[static_cast<int64_t>(p) * k + q])
                    : -1;
  int errbits = 0;
  const V* src = x + static_cast<int64_t>(t) * vec_per_row;
  V* xo = x_out + static_cast<int64_t>(p) * vec_per_row;
  for (int64_t c0 = l; c0 < vec_per_row; c0 += TPT * U) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * TPT;
      if (c < vec_per_row) v[u] = load_row<false>(src + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * TPT;
      if (c < vec_per_row) __builtin_nontemporal_store(v[u], xo + c);
    }
#pragma unroll
    for (int q = 0; q < MOE_MAX_K; ++q) {
      if (q >= k) break;
      if (drow[q] < 0) continue;
      if (drow[q] >= send_rows) {
        errbits = MOE_DERR_ROW_RANGE;
        continue;
      }
      V* dst = send + static_cast<int64_t>(drow[q]) * vec_per_row;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * TPT;
        if (c < vec_per_row) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
  if (l == 0) report(d_err, errbits);
}

// Launch shape by row size R (vectors): a wave per position below 256 (four
// vectors per lane per pass), else 512 threads per position (measured on
// MI355X for 8 KiB rows with up to 2 ranks: 351 us, against 355 us for the
// permute's 2 KiB parts at full residency).
template <typename V>
int launch_shuffle_dispatch(const void* x, int T, int64_t vec_per_row, const int32_t* perm,
                            const int32_t* token_rows, int k, void* x_out, void* send,
                            int64_t send_rows, int32_t* d_err, hipStream_t s) {
  const V* xv = static_cast<const V*>(x);
  if (vec_per_row < 256) {
    constexpr int kTokens = kPermThreads / 64;
    const int64_t nb = (static_cast<int64_t>(T) + kTokens - 1) / kTokens;
    if (!grid_ok(nb, kPermThreads)) return MOE_ERR_SHAPE;
    shuffle_dispatch_kernel<V, 64, 4><<<static_cast<unsigned>(nb), kPermThreads, 0, s>>>(
        xv, T, vec_per_row, perm, token_rows, k, static_cast<V*>(x_out),
        static_cast<V*>(send), send_rows, d_err);
  } else {
    if (!grid_ok(T, 512)) return MOE_ERR_SHAPE;
    shuffle_dispatch_kernel<V, 512, 1><<<static_cast<unsigned>(T), 512, 0, s>>>(
        xv, T, vec_per_row, perm, token_rows, k, static_cast<V*>(x_out),
        static_cast<V*>(send), send_rows, d_err);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_shuffle_dispatch(const void* x, int64_t T, int64_t row_bytes,
                                    const int32_t* perm, const int32_t* token_rows, int k,
                                    void* x_out, void* send, int64_t send_rows, int32_t* d_err,
                                    void* stream) {
  if (T < 0 || row_bytes <= 0 || k < 1 || k > MOE_MAX_K || send_rows < 0 ||
      T * static_cast<int64_t>(k) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || perm == nullptr || token_rows == nullptr || x_out == nullptr ||
      (send == nullptr && send_rows > 0))
    return MOE_ERR_NULL;
  const auto xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(x_out),
             sa = reinterpret_cast<uintptr_t>(send);
  if (row_bytes % 4 != 0 || xa % 4 != 0 || oa % 4 != 0 || sa % 4 != 0) return MOE_ERR_ALIGN;
  if (moe::overlap(x, T * row_bytes, x_out, T * row_bytes) ||
      moe::overlap(x, T * row_bytes, send, send_rows * row_bytes) ||
      moe::overlap(x_out, T * row_bytes, send, send_rows * row_bytes))
    return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Ti = static_cast<int>(T);
  if (row_bytes % 16 == 0 && xa % 16 == 0 && oa % 16 == 0 && sa % 16 == 0)
    return moe::launch_shuffle_dispatch<moe::u32x4>(x, Ti, row_bytes / 16, perm, token_rows, k,
                                                    x_out, send, send_rows, d_err, s);
  return moe::launch_shuffle_dispatch<uint32_t>(x, Ti, row_bytes / 4, perm, token_rows, k,
                                                x_out, send, send_rows, d_err, s);
}

extern "C" int moe_gather(const void* x, int64_t x_rows, int64_t row_bytes, const int32_t* src,
                          int64_t n_rows, void* out, const int32_t* n_valid, int32_t* d_err,
                          void* stream) {
  if (x_rows < 0 || row_bytes <= 0 || n_rows < 0 || n_rows >= (int64_t{1} << 31) ||
      x_rows >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (n_rows == 0) return MOE_OK;
  if (src == nullptr || out == nullptr || (x == nullptr && x_rows > 0)) return MOE_ERR_NULL;
  const auto xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
  if (row_bytes % 4 != 0 || xa % 4 != 0 || oa % 4 != 0) return MOE_ERR_ALIGN;
  if (moe::overlap(x, x_rows * row_bytes, out, n_rows * row_bytes)) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(n_rows);
  if (row_bytes % 16 == 0 && xa % 16 == 0 && oa % 16 == 0)
    return moe::launch_gather<moe::u32x4>(x, x_rows, row_bytes / 16, src, n, out, n_valid, d_err,
                                          s);
  return moe::launch_gather<uint32_t>(x, x_rows, row_bytes / 4, src, n, out, n_valid, d_err, s);
}

extern "C" int moe_permute(const void* x, int64_t T, int64_t row_bytes, const int32_t* dest,
                           int width, void* out, int64_t out_rows, const int32_t* n_valid,
                           int32_t* d_err, void* stream) {
  if (T < 0 || row_bytes <= 0 || width < 1 || width > MOE_MAX_K || out_rows < 0 ||
      T * static_cast<int64_t>(width) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || dest == nullptr || out == nullptr) return MOE_ERR_NULL;
  const auto xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
  if (row_bytes % 4 != 0 || xa % 4 != 0 || oa % 4 != 0) return MOE_ERR_ALIGN;
  if (moe::overlap(x, T * row_bytes, out, out_rows * row_bytes)) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (row_bytes % 16 == 0 && xa % 16 == 0 && oa % 16 == 0)
    return moe::launch_permute<moe::u32x4>(x, static_cast<int>(T), row_bytes / 16, dest, width,
                                           out, out_rows, n_valid, d_err, s);
  return moe::launch_permute<uint32_t>(x, static_cast<int>(T), row_bytes / 4, dest, width, out,
                                       out_rows, n_valid, d_err, s);
}

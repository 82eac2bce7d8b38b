// Backward mirror of the dispatch path.
//
// Both MoE all-to-alls run again in the backward pass with the data flowing
// the other way ("Expert Coupling in MoE Pretraining ..." abstract;
// "Training Communication-Efficient Mixture-of-Experts Language Models with
// Layer Re-Configuration", footnote 3: the inverse all-to-alls of the
// hidden-state dispatch, routed-probability dispatch and combine).  For the
// weighted combine y_t = sum_q a(row_q) z[row_q]:
//   dL/dz[row]   = a(row) * dL/dy_t         scaled scatter (this file)
//   dL/dw_tj     = <dL/dy_t, z[row(t, j)]>  row dot (this file)
// and the permute's adjoint is the unweighted combine (combine.hip).
#include "rowio.hpp"

namespace moe {
namespace {

constexpr int kBwThreads = 256;
constexpr int kBwUnroll = 2;
constexpr int kBwChunk = kWave * kBwUnroll;  // element groups per wave

// out[dest[t, q]] = round(scale[dest[t, q]] * x[t]): one wave per (token,
// chunk of kBwChunk groups), fp32 products rounded once to the output type.
template <bool XBF16, bool OBF16, int EPL>
__global__ __launch_bounds__(kBwThreads) void permute_scaled_kernel(
    const u32x4* __restrict__ x, int64_t groups, int chunks, const int32_t* __restrict__ dest,
    int width, const float* __restrict__ scale, int T, u32x4* __restrict__ out, int64_t out_rows,
    const int32_t* __restrict__ n_valid, int32_t* d_err) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (kBwThreads / kWave) + wave_id();
  const int t = static_cast<int>(item / chunks);
  if (t >= T || (n_valid != nullptr && t >= *n_valid)) return;
  const int chunk = static_cast<int>(item - static_cast<int64_t>(t) * chunks);
  const int lane = lane_id();
  const int64_t xvec = groups * (XBF16 ? EPL / 8 : EPL / 4);
  const int64_t ovec = groups * (OBF16 ? EPL / 8 : EPL / 4);

  int drow[MOE_MAX_K];
  float s[MOE_MAX_K];
  int nd = 0, errbits = 0;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    drow[q] = -1;
    s[q] = 0.f;
    if (q < width) {
      const int r = __builtin_amdgcn_readfirstlane(dest[static_cast<int64_t>(t) * width + q]);
      if (r >= 0 && r < out_rows) {
        drow[q] = r;
        s[q] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(scale[r])));
        ++nd;
      } else if (r >= out_rows) {
        errbits = MOE_DERR_ROW_RANGE;
      }
    }
  }
  if (chunk == 0 && lane == 0) report(d_err, errbits);
  if (nd == 0) return;

  const u32x4* xrow = x + static_cast<int64_t>(t) * xvec;
  const int64_t g0 = static_cast<int64_t>(chunk) * kBwChunk + lane;
  float f[kBwUnroll][EPL];
#pragma unroll
  for (int u = 0; u < kBwUnroll; ++u) {
    const int64_t g = g0 + u * kWave;
    if (g < groups) load_group<XBF16, EPL>(xrow, g, f[u]);
  }
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    if (q >= width) break;
    if (drow[q] < 0) continue;
    u32x4* orow = out + static_cast<int64_t>(drow[q]) * ovec;
#pragma unroll
    for (int u = 0; u < kBwUnroll; ++u) {
      const int64_t g = g0 + u * kWave;
      if (g < groups) {
        float p[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) p[i] = s[q] * f[u][i];
        store_group<OBF16, EPL>(orow, g, p);
      }
    }
  }
}

// out[t * width + q] = <a[t], b[rows[t, q]]>: one block per token, fp32
// products and sums in a fixed order (per-thread partial sums over its
// element groups, then a fixed wave and block tree), 0 for rows < 0.
template <bool ABF16, bool BBF16, int EPL>
__global__ __launch_bounds__(kBwThreads) void row_dot_kernel(
    const u32x4* __restrict__ a, const u32x4* __restrict__ b, int64_t groups, int64_t b_rows,
    const int32_t* __restrict__ rows, int width, int T, float* __restrict__ out,
    const int32_t* __restrict__ n_valid, int32_t* d_err) {
  __shared__ float s_part[MOE_MAX_K][kBwThreads / kWave];
  const int t = blockIdx.x;
  if (t >= T || (n_valid != nullptr && t >= *n_valid)) return;
  const int lane = lane_id();
  const int wave = wave_id();
  const int64_t avec = groups * (ABF16 ? EPL / 8 : EPL / 4);
  const int64_t bvec = groups * (BBF16 ? EPL / 8 : EPL / 4);
  const u32x4* arow = a + static_cast<int64_t>(t) * avec;

  int rid[MOE_MAX_K];
  int errbits = 0;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    rid[q] = -1;
    if (q < width) {
      const int r = __builtin_amdgcn_readfirstlane(rows[static_cast<int64_t>(t) * width + q]);
      if (r >= 0 && r < b_rows)
        rid[q] = r;
      else if (r >= b_rows)
        errbits = MOE_DERR_ROW_RANGE;
    }
  }
  if (threadIdx.x == 0) report(d_err, errbits);

  float acc[MOE_MAX_K];
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) acc[q] = 0.f;
  for (int64_t g = threadIdx.x; g < groups; g += kBwThreads) {
    float fa[EPL];
    load_group<ABF16, EPL>(arow, g, fa);
#pragma unroll
    for (int q = 0; q < MOE_MAX_K; ++q) {
      if (q >= width) break;
      if (rid[q] < 0) continue;
      float fb[EPL];
      load_group<BBF16, EPL>(b + static_cast<int64_t>(rid[q]) * bvec, g, fb);
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[q] = __builtin_fmaf(fa[i], fb[i], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    if (q >= width) break;
    float v = acc[q];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    if (lane == 0) s_part[q][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < static_cast<unsigned>(width)) {
    const int q = threadIdx.x;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kBwThreads / kWave; ++w) v += s_part[q][w];
    int r = rows[static_cast<int64_t>(t) * width + q];
    out[static_cast<int64_t>(t) * width + q] = (r >= 0 && r < b_rows) ? v : 0.f;
  }
}

template <bool XBF16, bool OBF16, int EPL>
int launch_scaled(const void* x, int64_t T, int64_t H, const int32_t* dest, int width,
                  const float* scale, void* out, int64_t out_rows, const int32_t* n_valid,
                  int32_t* d_err, hipStream_t s) {
  const int64_t groups = H / EPL;
  const int chunks = static_cast<int>((groups + kBwChunk - 1) / kBwChunk);
  const int64_t blocks = (T * chunks + kBwThreads / kWave - 1) / (kBwThreads / kWave);
  if (!grid_ok(blocks, kBwThreads)) return MOE_ERR_SHAPE;
  permute_scaled_kernel<XBF16, OBF16, EPL><<<static_cast<unsigned>(blocks), kBwThreads, 0, s>>>(
      static_cast<const u32x4*>(x), groups, chunks, dest, width, scale, static_cast<int>(T),
      static_cast<u32x4*>(out), out_rows, n_valid, d_err);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <bool ABF16, bool BBF16, int EPL>
int launch_dot(const void* a, const void* b, int64_t b_rows, int64_t T, int64_t H,
               const int32_t* rows, int width, float* out, const int32_t* n_valid,
               int32_t* d_err, hipStream_t s) {
  if (!grid_ok(T, kBwThreads)) return MOE_ERR_SHAPE;
  row_dot_kernel<ABF16, BBF16, EPL><<<static_cast<unsigned>(T), kBwThreads, 0, s>>>(
      static_cast<const u32x4*>(a), static_cast<const u32x4*>(b), H / EPL, b_rows, rows, width,
      static_cast<int>(T), out, n_valid, d_err);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

bool row_ok(int64_t H, int dtype, const void* p) {
  const int64_t bytes = H * (dtype == MOE_BF16 ? 2 : 4);
  return bytes % 16 == 0 && reinterpret_cast<uintptr_t>(p) % 16 == 0;
}

}  // namespace
}  // namespace moe

extern "C" int moe_permute_scaled(const void* x, int x_dtype, int64_t T, int64_t H,
                                  const int32_t* dest, int width, const float* scale, void* out,
                                  int out_dtype, int64_t out_rows, const int32_t* n_valid,
                                  int32_t* d_err, void* stream) {
  if ((x_dtype != MOE_F32 && x_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return MOE_ERR_DTYPE;
  if (T < 0 || H <= 0 || width < 1 || width > MOE_MAX_K || out_rows < 0 ||
      T * static_cast<int64_t>(width) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || dest == nullptr || scale == nullptr || out == nullptr) return MOE_ERR_NULL;
  if (!moe::row_ok(H, x_dtype, x) || !moe::row_ok(H, out_dtype, out)) return MOE_ERR_ALIGN;
  if (moe::overlap(x, T * H * (x_dtype == MOE_BF16 ? 2 : 4), out,
                   out_rows * H * (out_dtype == MOE_BF16 ? 2 : 4)))
    return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (x_dtype == MOE_BF16 && out_dtype == MOE_BF16)
    return moe::launch_scaled<true, true, 8>(x, T, H, dest, width, scale, out, out_rows, n_valid,
                                             d_err, s);
  if (x_dtype == MOE_BF16)
    return moe::launch_scaled<true, false, 8>(x, T, H, dest, width, scale, out, out_rows, n_valid,
                                              d_err, s);
  if (out_dtype == MOE_BF16)
    return moe::launch_scaled<false, true, 8>(x, T, H, dest, width, scale, out, out_rows, n_valid,
                                              d_err, s);
  return moe::launch_scaled<false, false, 4>(x, T, H, dest, width, scale, out, out_rows, n_valid,
                                             d_err, s);
}

extern "C" int moe_row_dot(const void* a, int a_dtype, int64_t T, int64_t H, const void* b,
                           int b_dtype, int64_t b_rows, const int32_t* rows, int width, float* out,
                           const int32_t* n_valid, int32_t* d_err, void* stream) {
  if ((a_dtype != MOE_F32 && a_dtype != MOE_BF16) || (b_dtype != MOE_F32 && b_dtype != MOE_BF16))
    return MOE_ERR_DTYPE;
  if (T < 0 || H <= 0 || width < 1 || width > MOE_MAX_K || b_rows < 0 ||
      T * static_cast<int64_t>(width) >= (int64_t{1} << 31) || T > INT32_MAX)
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (a == nullptr || b == nullptr || rows == nullptr || out == nullptr) return MOE_ERR_NULL;
  if (!moe::row_ok(H, a_dtype, a) || !moe::row_ok(H, b_dtype, b)) return MOE_ERR_ALIGN;
  const bool ab = a_dtype == MOE_BF16, bb = b_dtype == MOE_BF16;
  // Groups of 8 elements whenever a bf16 operand is involved (16 bytes of it).
  if ((ab || bb) && H % 8 != 0) return MOE_ERR_ALIGN;
  if (moe::overlap(out, T * width * 4, a, T * H * (ab ? 2 : 4)) ||
      moe::overlap(out, T * width * 4, b, b_rows * H * (bb ? 2 : 4)))
    return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ab && bb)
    return moe::launch_dot<true, true, 8>(a, b, b_rows, T, H, rows, width, out, n_valid, d_err, s);
  if (ab)
    return moe::launch_dot<true, false, 8>(a, b, b_rows, T, H, rows, width, out, n_valid, d_err, s);
  if (bb)
    return moe::launch_dot<false, true, 8>(a, b, b_rows, T, H, rows, width, out, n_valid, d_err, s);
  return moe::launch_dot<false, false, 4>(a, b, b_rows, T, H, rows, width, out, n_valid, d_err, s);
}

// Qwen3-style normalisation of the projected queries and keys, in place (the
// UA ablation with normalised queries and keys, "A Self-Pruning Transformer
// ...", paperlayer.ai summary, Appendix E): every head vector x of q and k
// becomes x / sqrt(mean(x^2) + eps) * w over the head dimension, with one
// weight vector w per tensor shared by the heads.  The layer calls then take
// these q and k as their inputs (RoPE and the key's L2 normalisation follow).
//
// Memory-bound: one wave per head row, read once and written once; the sum of
// squares is a wave reduction in fp32 and the result is rounded to the token
// dtype (round to nearest even for bf16).

#include <algorithm>

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

constexpr int kQkThreads = 256;

__device__ __forceinline__ float wave_fsum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Rows [0, nq) are q's head rows, [nq, nq + nk) k's; lane l holds elements
// l * PER .. l * PER + PER - 1 of a row.
template <int D, bool BF16>
__global__ __launch_bounds__(kQkThreads) void qk_norm_kernel(void* q, const float* wq, int64_t nq, void* k,
                                                            const float* wk, int64_t nk, float eps) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t nw = ((int64_t)gridDim.x * kQkThreads) >> 6;
  for (int64_t r = ((int64_t)blockIdx.x * kQkThreads + threadIdx.x) >> 6; r < nq + nk; r += nw) {
    const bool isq = r < nq;
    const int64_t e0 = (isq ? r : r - nq) * D + lane * PER;
    const float* w = isq ? wq : wk;
    float x[PER];
    if constexpr (BF16) {
      uint16_t* p = reinterpret_cast<uint16_t*>(isq ? q : k) + e0;
      if constexpr (PER == 1) {
        x[0] = bf16_to_f32(p[0]);
      } else {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
        x[0] = bf16_lo(v);
        x[1] = bf16_hi(v);
      }
    } else {
      const float* p = reinterpret_cast<const float*>(isq ? q : k) + e0;
#pragma unroll
      for (int e = 0; e < PER; ++e) x[e] = p[e];
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) ss = fmaf(x[e], x[e], ss);
    ss = wave_fsum(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    float y[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) y[e] = x[e] * inv * w[lane * PER + e];
    if constexpr (BF16) {
      uint16_t* p = reinterpret_cast<uint16_t*>(isq ? q : k) + e0;
      if constexpr (PER == 1) {
        p[0] = f32_to_bf16(y[0]);
      } else {
        *reinterpret_cast<uint32_t*>(p) = pack2_bf16(y[0], y[1]);
      }
    } else {
      float* p = reinterpret_cast<float*>(isq ? q : k) + e0;
#pragma unroll
      for (int e = 0; e < PER; ++e) p[e] = y[e];
    }
  }
}

hipError_t launch_qk_norm(int d, bool bf16, void* q, const float* wq, int64_t nq, void* k, const float* wk, int64_t nk,
                          float eps, hipStream_t st) {
  const int64_t rows = nq + nk;
  if (rows == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(4096, (rows + kQkThreads / 64 - 1) / (kQkThreads / 64));
  if (d == 64) {
    if (bf16) hipLaunchKernelGGL((qk_norm_kernel<64, true>), dim3(grid), dim3(kQkThreads), 0, st, q, wq, nq, k, wk, nk, eps);
    else hipLaunchKernelGGL((qk_norm_kernel<64, false>), dim3(grid), dim3(kQkThreads), 0, st, q, wq, nq, k, wk, nk, eps);
  } else if (d == 128) {
    if (bf16) hipLaunchKernelGGL((qk_norm_kernel<128, true>), dim3(grid), dim3(kQkThreads), 0, st, q, wq, nq, k, wk, nk, eps);
    else hipLaunchKernelGGL((qk_norm_kernel<128, false>), dim3(grid), dim3(kQkThreads), 0, st, q, wq, nq, k, wk, nk, eps);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ua

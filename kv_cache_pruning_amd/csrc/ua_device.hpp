// Device primitives shared by the UA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ua {

// Native 4 x 32-bit vector (a first-class LLVM vector, so arrays of it stay
// in registers; HIP's uint4 struct is copied with memcpy and can end up in
// scratch).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values to packed bf16 (lo in bits 0-15), round to nearest even, in
// one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Element load of an input that is either bf16 or fp32.
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// Eight consecutive elements (16 B of bf16 or 32 B of fp32) at element index i
// (i must be a multiple of 8 and the row 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, int64_t i, float (&out)[8]) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z);
    out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

// ---------------------------------------------------------------------------
// loads straight into LDS
// ---------------------------------------------------------------------------
// An LDS pointer in the LDS address space, as the global->LDS load builtins
// take it: the low 32 bits of a generic pointer to a __shared__ object are
// its LDS offset.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16 x 16 x 32 bf16 matrix-core product: lane l supplies row (of A) and
// column (of B) l & 15 over k group l >> 4 (8 bf16 each), and gets rows
// 4 (l >> 4) .. + 3 of column l & 15 of the fp32 result.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t to_lds(const void* p) {
  return reinterpret_cast<lds_ptr_t>(static_cast<size_t>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p))));
}

// ---------------------------------------------------------------------------
// cross-lane reductions inside groups of 8 / 16 lanes (DPP, no LDS)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// The value of lane i ^ 8 (row_ror:8 inside each row of 16 lanes).
constexpr int kDppRor8 = 0x128;

// Combine lane i with lane i ^ X for X = 8, 16 or 32 on the VALU: DPP inside a
// row, or the gfx950 row swaps (permlane16_swap pairs rows 0-1 and 2-3,
// permlane32_swap the two halves; both hand every lane the even- and the
// odd-side value).  Both lanes of a pair get bitwise the same result.
template <int X>
__device__ __forceinline__ float xor_sum(float v) {
  static_assert(X == 8 || X == 16 || X == 32, "lane distance");
  if constexpr (X == 8) {
    return v + dpp_f<kDppRor8>(v);
  } else {
    const uint32_t u = __float_as_uint(v);
    const auto r = (X == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
template <int X>
__device__ __forceinline__ float xor_max(float v) {
  static_assert(X == 8 || X == 16 || X == 32, "lane distance");
  if constexpr (X == 8) {
    return fmaxf(v, dpp_f<kDppRor8>(v));
  } else {
    const uint32_t u = __float_as_uint(v);
    const auto r = (X == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}

// Sum / max over the lanes l, l ^ N, l ^ 2N, ... of a wave (N = 8 or 16: one
// value per group of N lanes, combined across the 64 / N groups).
template <int N>
__device__ __forceinline__ float across_groups_sum(float v) {
  static_assert(N == 8 || N == 16, "group size");
  if constexpr (N == 8) v = xor_sum<8>(v);
  v = xor_sum<16>(v);
  return xor_sum<32>(v);
}
template <int N>
__device__ __forceinline__ float across_groups_max(float v) {
  static_assert(N == 8 || N == 16, "group size");
  if constexpr (N == 8) v = xor_max<8>(v);
  v = xor_max<16>(v);
  return xor_max<32>(v);
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group size");
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N == 16) v += dpp_f<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_isum(int v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive scan of one int per thread across a block of NT threads (NT a
// multiple of 64, at most 1024).  `scratch` holds NT/64 + 1 ints.  Returns the
// exclusive prefix; *total receives the block total.  Contains barriers.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[NT / 64] = run;
  }
  __syncthreads();
  const int excl = scratch[wave] + incl - v;
  *total = scratch[NT / 64];
  __syncthreads();
  return excl;
}

// ---------------------------------------------------------------------------
// UA scalar functions
// ---------------------------------------------------------------------------
// log(sigmoid(z)) = -(max(-z, 0) + log1p(exp(-|z|)))
__device__ __forceinline__ float log_sigmoid(float z) {
  return -(fmaxf(-z, 0.0f) + log1pf(expf(-fabsf(z))));
}

__device__ __forceinline__ float sigmoid(float z) {
  const float e = expf(-fabsf(z));
  const float r = 1.0f / (1.0f + e);
  return z >= 0.0f ? r : e * r;
}

// sigmoid through the hardware exp2 and reciprocal (about 2 ulp); 1 for large
// z, e^z / (1 + e^z) -> 0 for very negative z.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Row (query-side) and column (key-side) parts of the mean in the pair term,
// pre-scaled to log2 units and divided by the number of enabled terms.
struct PairCoef {
  float inv_n2;  // log2(e) / n_terms  (0 when no term is enabled)
  float sim_w;   // 1 / n_terms if the similarity term is on, else 0
  bool sim;
  bool any;
};

__device__ __forceinline__ PairCoef pair_coef(int terms) {
  PairCoef c;
  const int n = (terms & 1) + ((terms >> 1) & 1) + ((terms >> 2) & 1);
  c.any = n > 0;
  c.sim = (terms & 4) != 0;
  c.inv_n2 = n > 0 ? kLog2e / (float)n : 0.0f;
  c.sim_w = (n > 0 && c.sim) ? 1.0f / (float)n : 0.0f;
  return c;
}

// A = log(1 - exp(lambda)) <= 0 for lambda <= 0, given lambda in log2 units
// (lam2 = lambda * log2 e).  Two hardware transcendentals:
//  * lambda > -1/8:  1 - e^lambda = -lambda (1 + lambda/2 + lambda^2/6 + ...)
//    so A = log(-lambda) + lambda/2 + lambda^2/24 (next term is O(lambda^4));
//  * otherwise w = e^lambda <= 0.8825, y = fl(1 - w), and the rounding error of
//    y is recovered exactly as (1 - y) - w (Fast2Sum), so
//    A = log(y) + ((1 - y) - w) to first order.
// lambda = -inf gives 0; lambda = 0 gives -inf.
__device__ __forceinline__ float log1mexp2(float lam2) {
  const float lam = lam2 * kLn2;
  const bool small = lam > -0.125f;
  const float w = __builtin_amdgcn_exp2f(lam2);
  const float y = 1.0f - w;
  const float err = (1.0f - y) - w;
  const float arg = small ? -lam : y;
  const float corr = small ? lam * (0.5f + lam * (1.0f / 24.0f)) : err;
  return __builtin_amdgcn_logf(arg) * kLn2 + corr;
}

// Above this L (log2 units) log1mexp2_b2 takes its series branch.
constexpr float kLog1mexpSeries = -0.125f / kLn2;

// The same in log2 units with one logarithm: log2(1 - 2^L) for L <= 0.
// With lam = L ln 2 > -1/8, 1 - e^lam = -lam (1 + lam/2 + lam^2/6 + lam^3/24)
// up to a relative 2e-6 (Taylor series of expm1); otherwise 1 - 2^L >= 0.1175
// is formed directly, which costs at most about 1e-6 relative (the error of
// 2^L over the result).  L = -inf gives 0, L = 0 gives -inf.

__device__ __forceinline__ float log1mexp2_b2(float L) {
  constexpr float l1 = kLn2;
  constexpr float l2 = l1 * l1, l3 = l2 * l1, l4 = l3 * l1;
  const bool small = L > kLog1mexpSeries;
  float q = fmaf(L, -l4 / 24.0f, -l3 / 6.0f);
  q = fmaf(L, q, -l2 / 2.0f);
  q = fmaf(L, q, -l1);
  const float arg = small ? L * q : 1.0f - __builtin_amdgcn_exp2f(L);
  return __builtin_amdgcn_logf(arg);
}

// Pair term from the similarity s and the pre-scaled row/column parts:
// lam2 = row2 + col2 + sim_w * log2(min(s^2, 1)).
__device__ __forceinline__ float pair_A(const PairCoef& c, float row2, float col2, float s) {
  if (!c.any) return 0.0f;
  float lam2 = row2 + col2;
  if (c.sim) lam2 += c.sim_w * __builtin_amdgcn_logf(fminf(s * s, 1.0f));
  return log1mexp2(lam2);
}

}  // namespace ua

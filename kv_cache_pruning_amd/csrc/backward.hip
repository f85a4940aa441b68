// Backward of the decay-mask and attention part of a UA layer (gfx950).
//
// The pages pair a decay-mask kernel with a fused attention kernel for
// training ("A Self-Pruning Transformer ...", paperlayer.ai summary, section
// 4.2 and Appendix C; the bias is a geometric mean of three decays in log
// space, accumulated causally: ai4snews page, Figure 1 caption).  For one
// training chunk per sequence, starting from an empty cache, this file takes
// the rotated queries q~, the stored keys k~, the values v, the log-gates
// lq, lk, lb and the gradient dO of the attention output o (before the output
// gate), and returns dq~, dk~, dv, dlq, dlk, dlb.
//
// Per segment s (sequence b, KV head h) and 64 x 64 tiles of (token t, key j):
//   1. bwd_bias_kernel     Lambda[t][j] = sum_{t' <= t} A_{t'j}: per key block a
//                          scan down the token rows (A_{t'j} = 0 for t' <= j).
//   2. bwd_stats_kernel    per (token, query head): LSE and D = dO . o.
//   3. bwd_kv_kernel       per key block: dv, the attention part of dk, and
//                          dLambda[t][j] = sum over the group's heads of dS.
//   4. bwd_q_kernel        per (token block, query head): dq.
//   5. bwd_decay_kernel    per key block, token rows in reverse: dA_tj =
//                          sum_{i >= t} dLambda[i][j], dlambda = dA dA/dlambda,
//                          then the gates' and the similarity term's
//                          gradients (rows go out through atomics).
// Kernels 1 and 5 give lane l of a 256-thread workgroup row or key l >> 2 and
// quarter l & 3 of the head dimension (a dot product is four partial sums
// combined inside the quad); kernels 2-4 run their products on the matrix
// cores in fp32.  Lambda and dLambda are N x N fp32 per segment in the
// workspace; everything is fp32 inside.

#include <cmath>

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

constexpr int kBwThreads = 256;
constexpr int kBwTile = 64;

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  return v;
}

// The same sum in fp64 (each half of the double moves through its own DPP).
__device__ __forceinline__ double dpp_d_xor(double v, int which) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  int lo = (int)(u & 0xffffffffu), hi = (int)(u >> 32);
  if (which == 1) {
    lo = __builtin_amdgcn_update_dpp(0, lo, kDppXor1, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, kDppXor1, 0xF, 0xF, false);
  } else {
    lo = __builtin_amdgcn_update_dpp(0, lo, kDppXor2, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, kDppXor2, 0xF, 0xF, false);
  }
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double quad_sum_d(double v) {
  v += dpp_d_xor(v, 1);
  v += dpp_d_xor(v, 2);
  return v;
}

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

// d log(1 - e^lam) / d lam = -e^lam / (1 - e^lam), 0 at lam = -inf.
__device__ __forceinline__ float dlog1mexp(float lam) {
  const float e = __expf(lam);
  return (lam == -__builtin_huge_valf()) ? 0.0f : -e / (-expm1f(lam));
}

struct BwArgs {
  int B, Hq, Hkv, D, N, terms;
  float scale;
  const void* qt;  // [B, N, Hq, D]
  const void* kt;  // [B, N, Hkv, D]
  const void* v;   // [B, N, Hkv, D]
  const float* lq;  // [B, N, Hkv]
  const float* lk;
  const float* lb;
  const float* dO;  // [B, N, Hq, D]
  float* dq;
  float* dk;
  float* dv;
  float* dlq;
  float* dlk;
  float* dlb;
  float* lam;   // [S, N, N]
  float* dlam;  // [S, N, N]
  float* lse;   // [B, N, Hq]
  float* dd;    // [B, N, Hq]
};

__device__ __forceinline__ float pair_lambda(const BwArgs& a, float s, float lq, float lk, float lb, float inv_n) {
  float lam = 0.0f;
  if (a.terms & 1) lam += lq;
  if (a.terms & 2) lam += lk;
  if (a.terms & 4) lam += lb + __logf(fminf(s * s, 1.0f));
  return lam * inv_n;
}

// Stable log(1 - e^lam) for lam <= 0 (the two branches of the forward).
__device__ __forceinline__ float log1mexp_f(float lam) {
  return (lam > -0.6931471805599453f) ? __logf(-expm1f(lam)) : log1pf(-__expf(lam));
}

// ---------------------------------------------------------------------------
// 1. Lambda
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_bias_kernel(BwArgs a) {
  constexpr int QW = D / 4;
  __shared__ float s_k[kBwTile][D + 1];
  __shared__ float s_lq[kBwTile], s_lb[kBwTile];
  const int s = blockIdx.x, J = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N, nb = (N + kBwTile - 1) / kBwTile;
  const int tid = threadIdx.x, jl = tid >> 2, c = tid & 3;
  const int j = J * kBwTile + jl;
  const int jc = min(j, N - 1);
  const int n_terms = __popc(a.terms & 7);
  const float inv_n = n_terms ? 1.0f / n_terms : 0.0f;
  float kj[QW];
#pragma unroll
  for (int e = 0; e < QW; ++e) kj[e] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + c * QW + e);
  const float lkj = a.lk[((int64_t)b * N + jc) * a.Hkv + h];
  float carry = 0.0f;
  float* out = a.lam + (int64_t)s * N * N;
  for (int I = J; I < nb; ++I) {
    __syncthreads();
    for (int e = tid; e < kBwTile * D; e += kBwThreads) {
      const int r = e / D, col = e - r * D;
      const int t = min(I * kBwTile + r, N - 1);
      s_k[r][col] = ld_elem<BF16>(a.kt, (((int64_t)b * N + t) * a.Hkv + h) * D + col);
    }
    for (int r = tid; r < kBwTile; r += kBwThreads) {
      const int t = min(I * kBwTile + r, N - 1);
      s_lq[r] = a.lq[((int64_t)b * N + t) * a.Hkv + h];
      s_lb[r] = a.lb[((int64_t)b * N + t) * a.Hkv + h];
    }
    __syncthreads();
    for (int tl = 0; tl < kBwTile; ++tl) {
      const int t = I * kBwTile + tl;
      if (t >= N) break;
      float p = 0.0f;
#pragma unroll
      for (int e = 0; e < QW; ++e) p = fmaf(kj[e], s_k[tl][c * QW + e], p);
      const float sim = quad_sum(p);
      float A = 0.0f;
      if (n_terms && t > j) A = log1mexp_f(pair_lambda(a, sim, s_lq[tl], lkj, s_lb[tl], inv_n));
      carry += A;
      if (c == 0 && j < N && t >= j) out[(int64_t)t * N + j] = carry;
    }
  }
}

// ---------------------------------------------------------------------------
// 2-4 on the matrix cores: fp32 16x16x4 products (v_mfma_f32_16x16x4_f32).
// Lane l holds A[l % 16][l / 16] and B[l / 16][l % 16] of a step and
// D[4 (l / 16) + r][l % 16] of the 16 x 16 result (r = 0..3).  A product whose
// reduction runs over a tile's 16 rows takes the rows in the order 4 g + st
// (step st, lane group g = l / 16): the lane's own four result values of the
// previous product are then its operand for the four steps, with no
// transpose.  Tiles of 64 rows are staged in LDS as fp32 with a row stride
// of D + 4 floats.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float expf_masked(float e) { return e == -__builtin_huge_valf() ? 0.0f : __expf(e); }

// Rows r0 .. r0 + 63 (clamped to N - 1) of a [B, N, H, D] tensor at (b, head)
// into LDS as fp32 [64][D + 4].
template <int D, bool BF16>
__device__ __forceinline__ void stage_rows(float* dst, const void* src, int b, int N, int H, int head, int r0) {
  constexpr int LS = D + 4;
  constexpr int VE = BF16 ? 8 : 4;  // elements per 16-byte load
  for (int e = threadIdx.x; e < kBwTile * (D / VE); e += kBwThreads) {
    const int r = e / (D / VE), c = (e - r * (D / VE)) * VE;
    const int64_t g = (((int64_t)b * N + min(r0 + r, N - 1)) * H + head) * D + c;
    float* o = dst + r * LS + c;
    if constexpr (BF16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(src) + g);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[2 * q] = __uint_as_float(w[q] << 16);
        o[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
    } else {
      *reinterpret_cast<float4*>(o) = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + g);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. LSE and D = dO . o per (token, query head).  Wave w: tokens 16 w + c of
// the token block (c = l % 16); per key tile S^T = K Q^T, an online softmax
// per token, O^T += V^T P^T.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_stats_kernel(BwArgs a) {
  constexpr int LS = D + 4, NS = D / 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_k[kBwTile * LS];
  __shared__ __attribute__((aligned(16))) float s_v[kBwTile * LS];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x / G, ga = blockIdx.x - s * G, I = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv, hq = h * G + ga;
  const int N = a.N;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int t = I * kBwTile + 16 * w + c, tc = min(t, N - 1);
  float qreg[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) qreg[st] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tc) * a.Hq + hq) * D + 4 * st + g);
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_huge_valf(), lsum = 0.0f;
  const float* lrow = a.lam + (int64_t)s * N * N + (int64_t)tc * N;
  for (int J = 0; J <= I; ++J) {
    __syncthreads();
    stage_rows<D, BF16>(s_k, a.kt, b, N, a.Hkv, h, J * kBwTile);
    stage_rows<D, BF16>(s_v, a.v, b, N, a.Hkv, h, J * kBwTile);
    __syncthreads();
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st) sc = mfma4(s_k[(16 * kt + c) * LS + 4 * st + g], qreg[st], sc);
      float e[4];
      float mt = -__builtin_huge_valf();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = J * kBwTile + 16 * kt + 4 * g + r;
        const bool on = j <= t && t < N;
        e[r] = on ? fmaf(a.scale, sc[r], lrow[min(j, N - 1)]) : -__builtin_huge_valf();
        mt = fmaxf(mt, e[r]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m, mt);
      const float al = (mn == -__builtin_huge_valf()) ? 1.0f : expf_masked(m - mn);
      float p[4], ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (mn == -__builtin_huge_valf()) ? 0.0f : expf_masked(e[r] - mn);
        ps += p[r];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      lsum = fmaf(lsum, al, ps);
      m = mn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        oacc[dt] *= al;
#pragma unroll
        for (int st = 0; st < 4; ++st) oacc[dt] = mfma4(s_v[(16 * kt + 4 * g + st) * LS + 16 * dt + c], p[st], oacc[dt]);
      }
    }
  }
  // lane holds O^T[dim 16 dt + 4 g + r][token c]
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  float dd = 0.0f;
  const float* dorow = a.dO + (((int64_t)b * N + tc) * a.Hq + hq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dd = fmaf(dorow[16 * dt + 4 * g + r], oacc[dt][r] * inv, dd);
  dd += __shfl_xor(dd, 16, 64);
  dd += __shfl_xor(dd, 32, 64);
  if (g == 0 && t < N) {
    a.lse[((int64_t)b * N + t) * a.Hq + hq] = m + __logf(lsum);
    a.dd[((int64_t)b * N + t) * a.Hq + hq] = dd;
  }
}

// ---------------------------------------------------------------------------
// 3. dV, the attention part of dK, and dLambda (summed over the group).  Wave
// w: keys 16 w + c of the key block.  Per token tile S = Q K^T and dP = dO V^T
// (tokens x keys), P and dS, then dV += P^T dO and dK += dS^T Q.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_kv_kernel(BwArgs a) {
  constexpr int LS = D + 4, NS = D / 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_q[kBwTile * LS];
  __shared__ __attribute__((aligned(16))) float s_do[kBwTile * LS];
  __shared__ float s_lse[kBwTile], s_dd[kBwTile];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x, J = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N, nb = (N + kBwTile - 1) / kBwTile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int j = J * kBwTile + 16 * w + c, jc = min(j, N - 1);
  float kreg[NS], vreg[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    kreg[st] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + 4 * st + g);
    vreg[st] = ld_elem<BF16>(a.v, (((int64_t)b * N + jc) * a.Hkv + h) * D + 4 * st + g);
  }
  f32x4 dv[DT], dk[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* lamS = a.lam + (int64_t)s * N * N;
  float* dlamS = a.dlam + (int64_t)s * N * N;
  for (int I = J; I < nb; ++I) {
    f32x4 dl[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) dl[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ga = 0; ga < G; ++ga) {
      const int hq = h * G + ga;
      __syncthreads();
      stage_rows<D, BF16>(s_q, a.qt, b, N, a.Hq, hq, I * kBwTile);
      stage_rows<D, false>(s_do, a.dO, b, N, a.Hq, hq, I * kBwTile);
      for (int r = threadIdx.x; r < kBwTile; r += kBwThreads) {
        const int64_t ti = ((int64_t)b * N + min(I * kBwTile + r, N - 1)) * a.Hq + hq;
        s_lse[r] = a.lse[ti];
        s_dd[r] = a.dd[ti];
      }
      __syncthreads();
#pragma unroll 1
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          sc = mfma4(s_q[(16 * tt + c) * LS + 4 * st + g], kreg[st], sc);
          dp = mfma4(s_do[(16 * tt + c) * LS + 4 * st + g], vreg[st], dp);
        }
        // lane holds (token 16 tt + 4 g + r, key j)
        float P[4], dS[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 16 * tt + 4 * g + r, t = I * kBwTile + tl;
          const bool on = j <= t && t < N && j < N;
          const float lv = lamS[(int64_t)min(t, N - 1) * N + jc];
          P[r] = on ? __expf(fmaf(a.scale, sc[r], lv) - s_lse[tl]) : 0.0f;
          dS[r] = P[r] * (dp[r] - s_dd[tl]);
          dl[tt][r] += dS[r];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int row = (16 * tt + 4 * g + st) * LS + 16 * dt + c;
            dv[dt] = mfma4(P[st], s_do[row], dv[dt]);
            dk[dt] = mfma4(dS[st], s_q[row], dk[dt]);
          }
      }
    }
    if (j < N) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = I * kBwTile + 16 * tt + 4 * g + r;
          if (t < N) dlamS[(int64_t)t * N + j] = dl[tt][r];
        }
    }
  }
  // lane holds dV / dK[key 16 w + 4 g + r][dim 16 dt + c]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int jo = J * kBwTile + 16 * w + 4 * g + r;
    if (jo < N) {
      const int64_t o = (((int64_t)b * N + jo) * a.Hkv + h) * D + c;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        a.dv[o + 16 * dt] = dv[dt][r];
        a.dk[o + 16 * dt] = a.scale * dk[dt][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 4. dQ per (token block, query head).  Wave w: tokens 16 w + c.  Per key
// tile S^T = K Q^T and dP^T = V dO^T (keys x tokens), dS, then dQ += dS K.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_q_kernel(BwArgs a) {
  constexpr int LS = D + 4, NS = D / 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_k[kBwTile * LS];
  __shared__ __attribute__((aligned(16))) float s_v[kBwTile * LS];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x / G, ga = blockIdx.x - s * G, I = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv, hq = h * G + ga;
  const int N = a.N;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int t = I * kBwTile + 16 * w + c, tc = min(t, N - 1);
  float qreg[NS], oreg[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    qreg[st] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tc) * a.Hq + hq) * D + 4 * st + g);
    oreg[st] = a.dO[(((int64_t)b * N + tc) * a.Hq + hq) * D + 4 * st + g];
  }
  const float lse = a.lse[((int64_t)b * N + tc) * a.Hq + hq];
  const float dd = a.dd[((int64_t)b * N + tc) * a.Hq + hq];
  f32x4 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* lrow = a.lam + (int64_t)s * N * N + (int64_t)tc * N;
  for (int J = 0; J <= I; ++J) {
    __syncthreads();
    stage_rows<D, BF16>(s_k, a.kt, b, N, a.Hkv, h, J * kBwTile);
    stage_rows<D, BF16>(s_v, a.v, b, N, a.Hkv, h, J * kBwTile);
    __syncthreads();
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        sc = mfma4(s_k[(16 * kt + c) * LS + 4 * st + g], qreg[st], sc);
        dp = mfma4(s_v[(16 * kt + c) * LS + 4 * st + g], oreg[st], dp);
      }
      // lane holds (key 16 kt + 4 g + r, token t)
      float dS[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = J * kBwTile + 16 * kt + 4 * g + r;
        const bool on = jj <= t && t < N;
        const float P = on ? __expf(fmaf(a.scale, sc[r], lrow[min(jj, N - 1)]) - lse) : 0.0f;
        dS[r] = P * (dp[r] - dd);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int st = 0; st < 4; ++st) dq[dt] = mfma4(dS[st], s_k[(16 * kt + 4 * g + st) * LS + 16 * dt + c], dq[dt]);
    }
  }
  // lane holds dQ[token 16 w + 4 g + r][dim 16 dt + c]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int to = I * kBwTile + 16 * w + 4 * g + r;
    if (to < N) {
      const int64_t o = (((int64_t)b * N + to) * a.Hq + hq) * D + c;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) a.dq[o + 16 * dt] = a.scale * dq[dt][r];
    }
  }
}

// ---------------------------------------------------------------------------
// 5. decay backward: dLambda -> dA -> dlambda -> gates and keys
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_decay_kernel(BwArgs a) {
  constexpr int QW = D / 4;
  __shared__ float s_ki[kBwTile][D + 1];  // keys of the token block (rows)
  __shared__ float s_kj[kBwTile][D + 1];  // keys of this key block
  __shared__ float s_dl[kBwTile][kBwTile + 1];
  __shared__ float s_g[kBwTile][kBwTile + 1];
  __shared__ float s_ds[kBwTile][kBwTile + 1];
  __shared__ float s_lq[kBwTile], s_lb[kBwTile];
  const int s = blockIdx.x, J = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N, nb = (N + kBwTile - 1) / kBwTile;
  const int tid = threadIdx.x, jl = tid >> 2, c = tid & 3;
  const int j = J * kBwTile + jl, jc = min(j, N - 1);
  const int n_terms = __popc(a.terms & 7);
  if (n_terms == 0) return;  // no decay term: every decay gradient is zero (cleared by the caller)
  const float inv_n = 1.0f / n_terms;
  for (int e = tid; e < kBwTile * D; e += kBwThreads) {
    const int r = e / D, col = e - r * D;
    const int jj = min(J * kBwTile + r, N - 1);
    s_kj[r][col] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jj) * a.Hkv + h) * D + col);
  }
  float kj[QW], dkj[QW];
#pragma unroll
  for (int e = 0; e < QW; ++e) {
    kj[e] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + c * QW + e);
    dkj[e] = 0.0f;
  }
  const float lkj = a.lk[((int64_t)b * N + jc) * a.Hkv + h];
  float acc = 0.0f, dlk = 0.0f;
  const float* dlamS = a.dlam + (int64_t)s * N * N;
  for (int I = nb - 1; I >= J; --I) {
    __syncthreads();
    for (int e = tid; e < kBwTile * D; e += kBwThreads) {
      const int r = e / D, col = e - r * D;
      const int tt = min(I * kBwTile + r, N - 1);
      s_ki[r][col] = ld_elem<BF16>(a.kt, (((int64_t)b * N + tt) * a.Hkv + h) * D + col);
    }
    for (int e = tid; e < kBwTile * kBwTile; e += kBwThreads) {
      const int r = e / kBwTile, col = e - r * kBwTile;
      const int tt = I * kBwTile + r, jj = J * kBwTile + col;
      s_dl[r][col] = (tt < N && jj < N && jj <= tt) ? dlamS[(int64_t)tt * N + jj] : 0.0f;
    }
    for (int r = tid; r < kBwTile; r += kBwThreads) {
      const int tt = min(I * kBwTile + r, N - 1);
      s_lq[r] = a.lq[((int64_t)b * N + tt) * a.Hkv + h];
      s_lb[r] = a.lb[((int64_t)b * N + tt) * a.Hkv + h];
    }
    __syncthreads();
    // (a) key lanes: reverse scan of dLambda down the rows, the gradient of
    // each pair term, the key-side sums.  The similarity is summed in fp64:
    // the products of bf16 or fp32 keys are exact there, and the factor 2/s
    // of the similarity term is large where s is small, so an fp32 sum's
    // absolute error would turn into a large relative one exactly there.
    for (int tl = kBwTile - 1; tl >= 0; --tl) {
      const int t = I * kBwTile + tl;
      acc += s_dl[tl][jl];
      double p = 0.0;
      if (a.terms & 4) {
#pragma unroll
        for (int e = 0; e < QW; ++e) p = fma((double)kj[e], (double)s_ki[tl][c * QW + e], p);
        p = quad_sum_d(p);
      }
      const float sim = (float)p;
      float gn = 0.0f, ds = 0.0f;
      if (t < N && j < N && t > j) {
        const float lam = pair_lambda(a, sim, s_lq[tl], lkj, s_lb[tl], inv_n);
        gn = acc * dlog1mexp(lam) * inv_n;
        if ((a.terms & 4) && gn != 0.0f && p * p < 1.0) ds = 2.0f * gn / sim;
      }
      if (a.terms & 2) dlk += gn;
#pragma unroll
      for (int e = 0; e < QW; ++e) dkj[e] = fmaf(ds, s_ki[tl][c * QW + e], dkj[e]);
      if (c == 0) {
        s_g[tl][jl] = gn;
        s_ds[tl][jl] = ds;
      }
    }
    __syncthreads();
    // (b) token lanes: the sums over this block's keys of the row-side terms
    {
      const int tl = tid >> 2, t = I * kBwTile + tl;
      float gsum = 0.0f;
      for (int k2 = c * 16; k2 < c * 16 + 16; ++k2) gsum += s_g[tl][k2];
      gsum = quad_sum(gsum);
      float dkt[QW];
#pragma unroll
      for (int e = 0; e < QW; ++e) dkt[e] = 0.0f;
      for (int k2 = 0; k2 < kBwTile; ++k2) {
        const float w = s_ds[tl][k2];
#pragma unroll
        for (int e = 0; e < QW; ++e) dkt[e] = fmaf(w, s_kj[k2][c * QW + e], dkt[e]);
      }
      if (t < N) {
        const int64_t gi = ((int64_t)b * N + t) * a.Hkv + h;
        if (c == 0 && (a.terms & 1)) atomicAdd(&a.dlq[gi], gsum);
        if (c == 0 && (a.terms & 4)) atomicAdd(&a.dlb[gi], gsum);
        if (a.terms & 4) {
#pragma unroll
          for (int e = 0; e < QW; ++e) atomicAdd(&a.dk[gi * D + c * QW + e], dkt[e]);
        }
      }
    }
  }
  if (j < N) {
    const int64_t gi = ((int64_t)b * N + j) * a.Hkv + h;
    if (c == 0 && (a.terms & 2)) atomicAdd(&a.dlk[gi], dlk);
    if (a.terms & 4) {
#pragma unroll
      for (int e = 0; e < QW; ++e) atomicAdd(&a.dk[gi * D + c * QW + e], dkj[e]);
    }
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
size_t backward_ws_bytes(int B, int Hq, int Hkv, int N) {
  const size_t S = (size_t)B * Hkv;
  const size_t mat = align_up(sizeof(float) * S * N * N, 256);
  const size_t vec = align_up(sizeof(float) * (size_t)B * N * Hq, 256);
  return 2 * mat + 2 * vec;
}

template <int D, bool BF16>
static void launch_bw(const BwArgs& a, hipStream_t st) {
  const int S = a.B * a.Hkv, G = a.Hq / a.Hkv, nb = (a.N + kBwTile - 1) / kBwTile;
  hipLaunchKernelGGL((bwd_bias_kernel<D, BF16>), dim3(S, nb), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_stats_kernel<D, BF16>), dim3(S * G, nb), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_kv_kernel<D, BF16>), dim3(S, nb), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_q_kernel<D, BF16>), dim3(S * G, nb), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_decay_kernel<D, BF16>), dim3(S, nb), dim3(kBwThreads), 0, st, a);
}

hipError_t launch_backward(int B, int Hq, int Hkv, int D, int N, int terms, float scale, bool bf16, const void* qt,
                           const void* kt, const void* v, const float* lq, const float* lk, const float* lb,
                           const float* dO, float* dq, float* dk, float* dv, float* dlq, float* dlk, float* dlb,
                           void* ws, hipStream_t st) {
  BwArgs a;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.N = N;
  a.terms = terms;
  a.scale = scale;
  a.qt = qt;
  a.kt = kt;
  a.v = v;
  a.lq = lq;
  a.lk = lk;
  a.lb = lb;
  a.dO = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlq = dlq;
  a.dlk = dlk;
  a.dlb = dlb;
  const size_t S = (size_t)B * Hkv;
  char* p = reinterpret_cast<char*>(ws);
  const size_t mat = align_up(sizeof(float) * S * N * N, 256);
  const size_t vec = align_up(sizeof(float) * (size_t)B * N * Hq, 256);
  a.lam = reinterpret_cast<float*>(p);
  a.dlam = reinterpret_cast<float*>(p + mat);
  a.lse = reinterpret_cast<float*>(p + 2 * mat);
  a.dd = reinterpret_cast<float*>(p + 2 * mat + vec);
  // the gate gradients are sums of atomics
  const size_t gb = sizeof(float) * (size_t)B * N * Hkv;
  hipError_t e;
  if ((e = launch_fill_zero(dlq, gb, st)) != hipSuccess) return e;
  if ((e = launch_fill_zero(dlk, gb, st)) != hipSuccess) return e;
  if ((e = launch_fill_zero(dlb, gb, st)) != hipSuccess) return e;
  if (D == 64) {
    if (bf16) launch_bw<64, true>(a, st);
    else launch_bw<64, false>(a, st);
  } else if (D == 128) {
    if (bf16) launch_bw<128, true>(a, st);
    else launch_bw<128, false>(a, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ua

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
// Threads: lane l of a 256-thread workgroup serves row or key l >> 2 and
// quarter l & 3 of the head dimension; a dot product is four partial sums
// combined inside the quad.  Lambda and dLambda are N x N fp32 per segment in
// the workspace; everything is fp32 inside.

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
// 2. LSE and D = dO . o per (token, query head)
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_stats_kernel(BwArgs a) {
  constexpr int QW = D / 4;
  __shared__ float s_k[kBwTile][D + 1];
  __shared__ float s_v[kBwTile][D + 1];
  __shared__ float s_l[kBwTile][kBwTile + 1];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x / G, ga = blockIdx.x - s * G, I = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv, hq = h * G + ga;
  const int N = a.N;
  const int tid = threadIdx.x, tl = tid >> 2, c = tid & 3;
  const int t = I * kBwTile + tl, tc = min(t, N - 1);
  float q[QW], o[QW];
#pragma unroll
  for (int e = 0; e < QW; ++e) {
    q[e] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tc) * a.Hq + hq) * D + c * QW + e);
    o[e] = 0.0f;
  }
  float m = -__builtin_huge_valf(), l = 0.0f;
  const float* lamS = a.lam + (int64_t)s * N * N;
  for (int J = 0; J <= I; ++J) {
    __syncthreads();
    for (int e = tid; e < kBwTile * D; e += kBwThreads) {
      const int r = e / D, col = e - r * D;
      const int j = min(J * kBwTile + r, N - 1);
      s_k[r][col] = ld_elem<BF16>(a.kt, (((int64_t)b * N + j) * a.Hkv + h) * D + col);
      s_v[r][col] = ld_elem<BF16>(a.v, (((int64_t)b * N + j) * a.Hkv + h) * D + col);
    }
    for (int e = tid; e < kBwTile * kBwTile; e += kBwThreads) {
      const int r = e / kBwTile, col = e - r * kBwTile;
      const int tt = min(I * kBwTile + r, N - 1), j = min(J * kBwTile + col, N - 1);
      s_l[r][col] = lamS[(int64_t)tt * N + j];
    }
    __syncthreads();
    for (int jl = 0; jl < kBwTile; ++jl) {
      const int j = J * kBwTile + jl;
      if (j > t || j >= N) break;
      float p = 0.0f;
#pragma unroll
      for (int e = 0; e < QW; ++e) p = fmaf(q[e], s_k[jl][c * QW + e], p);
      const float ev = a.scale * quad_sum(p) + s_l[tl][jl];
      const float mn = fmaxf(m, ev);
      const float al = __expf(m - mn), pe = __expf(ev - mn);
      l = l * al + pe;
#pragma unroll
      for (int e = 0; e < QW; ++e) o[e] = fmaf(pe, s_v[jl][c * QW + e], o[e] * al);
      m = mn;
    }
  }
  if (t < N) {
    const float inv = 1.0f / l;
    float dd = 0.0f;
#pragma unroll
    for (int e = 0; e < QW; ++e) dd = fmaf(a.dO[(((int64_t)b * N + t) * a.Hq + hq) * D + c * QW + e], o[e] * inv, dd);
    dd = quad_sum(dd);
    if (c == 0) {
      a.lse[((int64_t)b * N + t) * a.Hq + hq] = m + __logf(l);
      a.dd[((int64_t)b * N + t) * a.Hq + hq] = dd;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dv, the attention part of dk, and dLambda (summed over the group)
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_kv_kernel(BwArgs a) {
  constexpr int QW = D / 4;
  __shared__ float s_q[kBwTile][D + 1];
  __shared__ float s_do[kBwTile][D + 1];
  __shared__ float s_l[kBwTile][kBwTile + 1];
  __shared__ float s_dl[kBwTile][kBwTile + 1];
  __shared__ float s_lse[kBwTile], s_dd[kBwTile];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x, J = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N, nb = (N + kBwTile - 1) / kBwTile;
  const int tid = threadIdx.x, jl = tid >> 2, c = tid & 3;
  const int j = J * kBwTile + jl, jc = min(j, N - 1);
  float kj[QW], vj[QW], dk[QW], dv[QW];
#pragma unroll
  for (int e = 0; e < QW; ++e) {
    kj[e] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + c * QW + e);
    vj[e] = ld_elem<BF16>(a.v, (((int64_t)b * N + jc) * a.Hkv + h) * D + c * QW + e);
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  const float* lamS = a.lam + (int64_t)s * N * N;
  float* dlamS = a.dlam + (int64_t)s * N * N;
  for (int I = J; I < nb; ++I) {
    __syncthreads();
    for (int e = tid; e < kBwTile * kBwTile; e += kBwThreads) {
      const int r = e / kBwTile, col = e - r * kBwTile;
      const int tt = min(I * kBwTile + r, N - 1), jj = min(J * kBwTile + col, N - 1);
      s_l[r][col] = lamS[(int64_t)tt * N + jj];
      s_dl[r][col] = 0.0f;
    }
    for (int ga = 0; ga < G; ++ga) {
      const int hq = h * G + ga;
      __syncthreads();
      for (int e = tid; e < kBwTile * D; e += kBwThreads) {
        const int r = e / D, col = e - r * D;
        const int tt = min(I * kBwTile + r, N - 1);
        s_q[r][col] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tt) * a.Hq + hq) * D + col);
        s_do[r][col] = a.dO[(((int64_t)b * N + tt) * a.Hq + hq) * D + col];
      }
      for (int r = tid; r < kBwTile; r += kBwThreads) {
        const int tt = min(I * kBwTile + r, N - 1);
        s_lse[r] = a.lse[((int64_t)b * N + tt) * a.Hq + hq];
        s_dd[r] = a.dd[((int64_t)b * N + tt) * a.Hq + hq];
      }
      __syncthreads();
      for (int tl = 0; tl < kBwTile; ++tl) {
        const int t = I * kBwTile + tl;
        if (t >= N) break;
        float p = 0.0f, dp = 0.0f;
#pragma unroll
        for (int e = 0; e < QW; ++e) {
          p = fmaf(kj[e], s_q[tl][c * QW + e], p);
          dp = fmaf(vj[e], s_do[tl][c * QW + e], dp);
        }
        p = quad_sum(p);
        dp = quad_sum(dp);
        const bool on = j <= t && j < N;
        const float P = on ? __expf(a.scale * p + s_l[tl][jl] - s_lse[tl]) : 0.0f;
        const float dS = P * (dp - s_dd[tl]);
#pragma unroll
        for (int e = 0; e < QW; ++e) {
          dv[e] = fmaf(P, s_do[tl][c * QW + e], dv[e]);
          dk[e] = fmaf(a.scale * dS, s_q[tl][c * QW + e], dk[e]);
        }
        if (c == 0) s_dl[tl][jl] += dS;
      }
    }
    __syncthreads();
    for (int e = tid; e < kBwTile * kBwTile; e += kBwThreads) {
      const int r = e / kBwTile, col = e - r * kBwTile;
      const int tt = I * kBwTile + r, jj = J * kBwTile + col;
      if (tt < N && jj < N) dlamS[(int64_t)tt * N + jj] = s_dl[r][col];
    }
  }
  if (j < N) {
#pragma unroll
    for (int e = 0; e < QW; ++e) {
      a.dk[(((int64_t)b * N + j) * a.Hkv + h) * D + c * QW + e] = dk[e];
      a.dv[(((int64_t)b * N + j) * a.Hkv + h) * D + c * QW + e] = dv[e];
    }
  }
}

// ---------------------------------------------------------------------------
// 4. dq per (token block, query head)
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_q_kernel(BwArgs a) {
  constexpr int QW = D / 4;
  __shared__ float s_k[kBwTile][D + 1];
  __shared__ float s_v[kBwTile][D + 1];
  __shared__ float s_l[kBwTile][kBwTile + 1];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x / G, ga = blockIdx.x - s * G, I = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv, hq = h * G + ga;
  const int N = a.N;
  const int tid = threadIdx.x, tl = tid >> 2, c = tid & 3;
  const int t = I * kBwTile + tl, tc = min(t, N - 1);
  float q[QW], dO[QW], dq[QW];
#pragma unroll
  for (int e = 0; e < QW; ++e) {
    q[e] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tc) * a.Hq + hq) * D + c * QW + e);
    dO[e] = a.dO[(((int64_t)b * N + tc) * a.Hq + hq) * D + c * QW + e];
    dq[e] = 0.0f;
  }
  const float lse = a.lse[((int64_t)b * N + tc) * a.Hq + hq];
  const float dd = a.dd[((int64_t)b * N + tc) * a.Hq + hq];
  const float* lamS = a.lam + (int64_t)s * N * N;
  for (int J = 0; J <= I; ++J) {
    __syncthreads();
    for (int e = tid; e < kBwTile * D; e += kBwThreads) {
      const int r = e / D, col = e - r * D;
      const int j = min(J * kBwTile + r, N - 1);
      s_k[r][col] = ld_elem<BF16>(a.kt, (((int64_t)b * N + j) * a.Hkv + h) * D + col);
      s_v[r][col] = ld_elem<BF16>(a.v, (((int64_t)b * N + j) * a.Hkv + h) * D + col);
    }
    for (int e = tid; e < kBwTile * kBwTile; e += kBwThreads) {
      const int r = e / kBwTile, col = e - r * kBwTile;
      const int tt = min(I * kBwTile + r, N - 1), j = min(J * kBwTile + col, N - 1);
      s_l[r][col] = lamS[(int64_t)tt * N + j];
    }
    __syncthreads();
    for (int jl = 0; jl < kBwTile; ++jl) {
      const int j = J * kBwTile + jl;
      if (j > t || j >= N) break;
      float p = 0.0f, dp = 0.0f;
#pragma unroll
      for (int e = 0; e < QW; ++e) {
        p = fmaf(q[e], s_k[jl][c * QW + e], p);
        dp = fmaf(dO[e], s_v[jl][c * QW + e], dp);
      }
      p = quad_sum(p);
      dp = quad_sum(dp);
      const float P = __expf(a.scale * p + s_l[tl][jl] - lse);
      const float g = a.scale * P * (dp - dd);
#pragma unroll
      for (int e = 0; e < QW; ++e) dq[e] = fmaf(g, s_k[jl][c * QW + e], dq[e]);
    }
  }
  if (t < N) {
#pragma unroll
    for (int e = 0; e < QW; ++e) a.dq[(((int64_t)b * N + t) * a.Hq + hq) * D + c * QW + e] = dq[e];
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

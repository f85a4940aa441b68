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
//   1. bwd_bias_kernel       Lambda[t][j] = sum_{t' <= t} A_{t'j}: per key block
//                            a scan down the token rows (A_{t'j} = 0 for t' <= j).
//   2. bwd_stats_kernel      per (token, query head): LSE and D = dO . o.
//   3. bwd_kv_kernel         per key block: dv, the attention part of dk, and
//                            dLambda[t][j] = sum over the group's heads of dS.
//   4. bwd_q_kernel          per (token block, query head): dq.
//   5. bwd_decay_col_kernel  per key block, token rows in reverse: dA_tj =
//                            sum_{i >= t} dLambda[i][j], the gradient g of each
//                            pair term and ds of its similarity; dlk and the
//                            key side of dk.
//   6. bwd_decay_row_kernel  per token block: dlq, dlb and the token side of dk.
// Every kernel runs its products on the matrix cores (fp32 16x16x4 tiles; the
// decay pass's similarity in fp64; q~ . k~ in bf16 when the inputs are bf16)
// and owns the rows it writes, so no output needs clearing and no atomics are
// used.  Lambda and dLambda are N x N fp32
// per segment in the workspace; everything is fp32 inside.

#include <cmath>

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

constexpr int kBwThreads = 256;
constexpr int kBwTile = 64;

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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// bf16 16x16x32 product: lane l holds A[l % 16][8 (l / 16) .. + 7] and
// B[8 (l / 16) .. + 7][l % 16] of each 32-wide k chunk; the result has the
// same 16 x 16 layout as the fp32 product.  Used for q~ . k~ when both are
// bf16: the products are exact and the sum is fp32, as in the fp32 product.
__device__ __forceinline__ f32x4 mfma_bf16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                  0, 0, 0);
}

// The 16-byte piece of row r (clamped to N - 1) of a bf16 [B, N, H, D] tensor
// at (b, head) holding dims 8 q .. 8 q + 7.
template <int D>
__device__ __forceinline__ u32x4 bf16_piece(const void* src, int b, int N, int H, int head, int r, int q) {
  const int64_t e = (((int64_t)b * N + min(r, N - 1)) * H + head) * D + 8 * q;
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(src) + e);
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
// 1. Lambda[t][j] = sum_{t' <= t} A_{t'j}.  Wave w: keys 16 w + c of the key
// block; per token tile the similarities K_t K_j^T (tokens x keys), the pair
// terms, and an inclusive scan down the 16 tokens (within the lane, then
// across the four lane groups) on top of the column's carry.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_bias_kernel(BwArgs a) {
  constexpr int LS = D + 4, NS = D / 4;
  __shared__ __attribute__((aligned(16))) float s_k[kBwTile * LS];
  __shared__ float s_lq[kBwTile], s_lb[kBwTile];
  const int s = blockIdx.x, J = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N, nb = (N + kBwTile - 1) / kBwTile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int j = J * kBwTile + 16 * w + c, jc = min(j, N - 1);
  const int n_terms = __popc(a.terms & 7);
  const float inv_n = n_terms ? 1.0f / n_terms : 0.0f;
  float kreg[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) kreg[st] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + 4 * st + g);
  const float lkj = a.lk[((int64_t)b * N + jc) * a.Hkv + h];
  float* out = a.lam + (int64_t)s * N * N;
  float carry = 0.0f;
  for (int I = J; I < nb; ++I) {
    __syncthreads();
    stage_rows<D, BF16>(s_k, a.kt, b, N, a.Hkv, h, I * kBwTile);
    for (int r = threadIdx.x; r < kBwTile; r += kBwThreads) {
      const int64_t ti = ((int64_t)b * N + min(I * kBwTile + r, N - 1)) * a.Hkv + h;
      s_lq[r] = a.lq[ti];
      s_lb[r] = a.lb[ti];
    }
    __syncthreads();
#pragma unroll 1
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      if (a.terms & 4) {
#pragma unroll
        for (int st = 0; st < NS; ++st) sc = mfma4(s_k[(16 * tt + c) * LS + 4 * st + g], kreg[st], sc);
      }
      // lane holds (token 16 tt + 4 g + r, key j): pair terms, then the scan
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 16 * tt + 4 * g + r, t = I * kBwTile + tl;
        const bool on = n_terms && t > j && t < N && j < N;
        const float A = on ? log1mexp_f(pair_lambda(a, sc[r], s_lq[tl], lkj, s_lb[tl], inv_n)) : 0.0f;
        p[r] = (r ? p[r - 1] : 0.0f) + A;
      }
      const float T = p[3];
      const float T0 = __shfl(T, c, 64), T1 = __shfl(T, c + 16, 64), T2 = __shfl(T, c + 32, 64),
                  T3 = __shfl(T, c + 48, 64);
      const float U = (g > 0 ? T0 : 0.0f) + (g > 1 ? T1 : 0.0f) + (g > 2 ? T2 : 0.0f);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = I * kBwTile + 16 * tt + 4 * g + r;
        if (j < N && t < N && t >= j) out[(int64_t)t * N + j] = carry + U + p[r];
      }
      carry += T0 + T1 + T2 + T3;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. LSE and D = dO . o per (token, query head).  Wave w: tokens 16 w + c of
// the token block (c = l % 16); per key tile S^T = K Q^T, an online softmax
// per token, O^T += V^T P^T.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__device__ __forceinline__ void bwd_stats_block(const BwArgs& a, const int by) {
  constexpr int LS = D + 4, NS = D / 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_k[kBwTile * LS];
  __shared__ __attribute__((aligned(16))) float s_v[kBwTile * LS];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x / G, ga = blockIdx.x - s * G, I = by;
  const int b = s / a.Hkv, h = s - b * a.Hkv, hq = h * G + ga;
  const int N = a.N;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int t = I * kBwTile + 16 * w + c, tc = min(t, N - 1);
  constexpr int KC = D / 32;
  float qreg[BF16 ? 1 : NS];
  u32x4 qb[BF16 ? KC : 1];
  if constexpr (BF16) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qb[kc] = bf16_piece<D>(a.qt, b, N, a.Hq, hq, tc, 4 * kc + g);
  } else {
#pragma unroll
    for (int st = 0; st < NS; ++st) qreg[st] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tc) * a.Hq + hq) * D + 4 * st + g);
  }
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_huge_valf(), lsum = 0.0f;
  const float* lrow = a.lam + (int64_t)s * N * N + (int64_t)tc * N;
  for (int J = 0; J <= I; ++J) {
    u32x4 kb[BF16 ? 4 : 1][KC];  // bf16: the key rows 16 kt + c of the block, straight from HBM
    if constexpr (BF16) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kb[kt][kc] = bf16_piece<D>(a.kt, b, N, a.Hkv, h, J * kBwTile + 16 * kt + c, 4 * kc + g);
    }
    __syncthreads();
    if constexpr (!BF16) stage_rows<D, BF16>(s_k, a.kt, b, N, a.Hkv, h, J * kBwTile);
    stage_rows<D, BF16>(s_v, a.v, b, N, a.Hkv, h, J * kBwTile);
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) sc = mfma_bf16x32(kb[kt][kc], qb[kc], sc);
      } else {
#pragma unroll
        for (int st = 0; st < NS; ++st) sc = mfma4(s_k[(16 * kt + c) * LS + 4 * st + g], qreg[st], sc);
      }
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
  constexpr int KC = D / 32;
  float kreg[BF16 ? 1 : NS], vreg[NS];
  u32x4 kb[BF16 ? KC : 1];  // bf16: this lane's key row for the bf16 product
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    if constexpr (!BF16) kreg[st] = ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + 4 * st + g);
    vreg[st] = ld_elem<BF16>(a.v, (((int64_t)b * N + jc) * a.Hkv + h) * D + 4 * st + g);
  }
  if constexpr (BF16) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kb[kc] = bf16_piece<D>(a.kt, b, N, a.Hkv, h, jc, 4 * kc + g);
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
        if constexpr (BF16) {
          // the token rows' bf16 pieces, loaded while dP runs
          u32x4 qa[KC];
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) qa[kc] = bf16_piece<D>(a.qt, b, N, a.Hq, hq, I * kBwTile + 16 * tt + c, 4 * kc + g);
#pragma unroll
          for (int st = 0; st < NS; ++st) dp = mfma4(s_do[(16 * tt + c) * LS + 4 * st + g], vreg[st], dp);
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) sc = mfma_bf16x32(qa[kc], kb[kc], sc);
        } else {
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            sc = mfma4(s_q[(16 * tt + c) * LS + 4 * st + g], kreg[st], sc);
            dp = mfma4(s_do[(16 * tt + c) * LS + 4 * st + g], vreg[st], dp);
          }
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
__device__ __forceinline__ void bwd_q_block(const BwArgs& a, const int by) {
  constexpr int LS = D + 4, NS = D / 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_k[kBwTile * LS];
  __shared__ __attribute__((aligned(16))) float s_v[kBwTile * LS];
  const int G = a.Hq / a.Hkv;
  const int s = blockIdx.x / G, ga = blockIdx.x - s * G, I = by;
  const int b = s / a.Hkv, h = s - b * a.Hkv, hq = h * G + ga;
  const int N = a.N;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int t = I * kBwTile + 16 * w + c, tc = min(t, N - 1);
  constexpr int KC = D / 32;
  float qreg[BF16 ? 1 : NS], oreg[NS];
  u32x4 qb[BF16 ? KC : 1];  // bf16: this lane's token row for the bf16 product
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    if constexpr (!BF16) qreg[st] = ld_elem<BF16>(a.qt, (((int64_t)b * N + tc) * a.Hq + hq) * D + 4 * st + g);
    oreg[st] = a.dO[(((int64_t)b * N + tc) * a.Hq + hq) * D + 4 * st + g];
  }
  if constexpr (BF16) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qb[kc] = bf16_piece<D>(a.qt, b, N, a.Hq, hq, tc, 4 * kc + g);
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
      if constexpr (BF16) {
        // the key rows' bf16 pieces, loaded while dP^T runs
        u32x4 ka[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) ka[kc] = bf16_piece<D>(a.kt, b, N, a.Hkv, h, J * kBwTile + 16 * kt + c, 4 * kc + g);
#pragma unroll
        for (int st = 0; st < NS; ++st) dp = mfma4(s_v[(16 * kt + c) * LS + 4 * st + g], oreg[st], dp);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) sc = mfma_bf16x32(ka[kc], qb[kc], sc);
      } else {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          sc = mfma4(s_k[(16 * kt + c) * LS + 4 * st + g], qreg[st], sc);
          dp = mfma4(s_v[(16 * kt + c) * LS + 4 * st + g], oreg[st], dp);
        }
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

// Causal balance for the token-block kernels: token block I has I + 1 key
// blocks of work, so each workgroup takes block y and block nb - 1 - y (the
// middle one alone when nb is odd) and every workgroup does the same work.
// (The key-block kernel keeps one block per workgroup: paired, its four
// workgroups per CU became two and it was no faster.)
#define UA_BW_PAIRED(NAME)                                                  \
  template <int D, bool BF16>                                               \
  __global__ __launch_bounds__(kBwThreads) void NAME##_kernel(BwArgs a) {   \
    const int nb = (a.N + kBwTile - 1) / kBwTile;                           \
    const int y0 = blockIdx.y, y1 = nb - 1 - (int)blockIdx.y;               \
    NAME##_block<D, BF16>(a, y0);                                           \
    if (y1 != y0) {                                                         \
      __syncthreads();                                                      \
      NAME##_block<D, BF16>(a, y1);                                         \
    }                                                                       \
  }
UA_BW_PAIRED(bwd_stats)
UA_BW_PAIRED(bwd_q)
#undef UA_BW_PAIRED

// ---------------------------------------------------------------------------
// 5. decay gradients, column pass (key block J, token blocks in reverse).
// dA_tj = sum_{i >= t} dLambda[i][j] is a reverse scan down the column; with
// g_tj = dA_tj dlog(1 - e^lam)/dlam / n and, for the similarity term,
// ds_tj = 2 g_tj / s_tj: dlk_j = sum_t g_tj and dk_j += sum_t ds_tj k_t.
// g and ds overwrite dLambda and Lambda for the row pass.  The similarity is
// summed in fp64 on the matrix cores: products of bf16 or fp32 keys are exact
// there, and the factor 2/s is largest where s is near 0, where an fp32 sum's
// absolute error would become a large relative one.  The fp64 product's
// result rows are interleaved (lane l holds rows l / 16 + 4 r), so the token
// rows are fed permuted and the tile lands as tokens 4 g + r, as in fp32.
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_decay_col_kernel(BwArgs a) {
  constexpr int LS = D + 4, NS = D / 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_k[kBwTile * LS];
  __shared__ float s_lq[kBwTile], s_lb[kBwTile];
  const int s = blockIdx.x, J = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N, nb = (N + kBwTile - 1) / kBwTile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int j = J * kBwTile + 16 * w + c, jc = min(j, N - 1);
  const int n_terms = __popc(a.terms & 7);
  if (n_terms == 0) {  // no decay term: every decay gradient is zero
    if (g == 0 && j < N) a.dlk[((int64_t)b * N + j) * a.Hkv + h] = 0.0f;
    return;
  }
  const float inv_n = 1.0f / n_terms;
  const bool SIM = (a.terms & 4) != 0;
  double kreg[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
    kreg[st] = (double)ld_elem<BF16>(a.kt, (((int64_t)b * N + jc) * a.Hkv + h) * D + 4 * st + g);
  const float lkj = a.lk[((int64_t)b * N + jc) * a.Hkv + h];
  float* dlamS = a.dlam + (int64_t)s * N * N;  // dLambda in, g out
  float* lamS = a.lam + (int64_t)s * N * N;    // ds out
  f32x4 dkj[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dkj[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dlk = 0.0f, carry = 0.0f;
  const int prow = 4 * (c & 3) + (c >> 2);  // token row this lane feeds to the fp64 product
  for (int I = nb - 1; I >= J; --I) {
    __syncthreads();
    stage_rows<D, BF16>(s_k, a.kt, b, N, a.Hkv, h, I * kBwTile);
    for (int r = threadIdx.x; r < kBwTile; r += kBwThreads) {
      const int64_t ti = ((int64_t)b * N + min(I * kBwTile + r, N - 1)) * a.Hkv + h;
      s_lq[r] = a.lq[ti];
      s_lb[r] = a.lb[ti];
    }
    __syncthreads();
#pragma unroll 1
    for (int tt = 3; tt >= 0; --tt) {
      f64x4 sd = {0.0, 0.0, 0.0, 0.0};
      if (SIM) {
#pragma unroll
        for (int st = 0; st < NS; ++st)
          sd = __builtin_amdgcn_mfma_f64_16x16x4f64((double)s_k[(16 * tt + prow) * LS + 4 * st + g], kreg[st], sd, 0, 0,
                                                    0);
      }
      // lane holds (token 16 tt + 4 g + r, key j); reverse inclusive scan of dLambda
      float x[4], q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = I * kBwTile + 16 * tt + 4 * g + r;
        x[r] = (t < N && j < N && t >= j) ? dlamS[(int64_t)t * N + j] : 0.0f;
      }
      q[3] = x[3];
      q[2] = x[2] + q[3];
      q[1] = x[1] + q[2];
      q[0] = x[0] + q[1];
      const float T = q[0];
      const float T0 = __shfl(T, c, 64), T1 = __shfl(T, c + 16, 64), T2 = __shfl(T, c + 32, 64),
                  T3 = __shfl(T, c + 48, 64);
      const float V = (g < 1 ? T1 : 0.0f) + (g < 2 ? T2 : 0.0f) + (g < 3 ? T3 : 0.0f);
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 16 * tt + 4 * g + r, t = I * kBwTile + tl;
        const float acc = carry + V + q[r];
        float gn = 0.0f;
        ds[r] = 0.0f;
        if (t > j && t < N && j < N) {
          const float sim = (float)sd[r];
          const float lam = pair_lambda(a, sim, s_lq[tl], lkj, s_lb[tl], inv_n);
          gn = acc * dlog1mexp(lam) * inv_n;
          if (SIM && gn != 0.0f && sd[r] * sd[r] < 1.0) ds[r] = 2.0f * gn / sim;
        }
        dlk += gn;
        if (t < N && j < N) {
          dlamS[(int64_t)t * N + j] = gn;
          lamS[(int64_t)t * N + j] = ds[r];
        }
      }
      carry += T0 + T1 + T2 + T3;
      if (SIM) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int st = 0; st < 4; ++st) dkj[dt] = mfma4(ds[st], s_k[(16 * tt + 4 * g + st) * LS + 16 * dt + c], dkj[dt]);
      }
    }
  }
  dlk += __shfl_xor(dlk, 16, 64);
  dlk += __shfl_xor(dlk, 32, 64);
  if (g == 0 && j < N) a.dlk[((int64_t)b * N + j) * a.Hkv + h] = (a.terms & 2) ? dlk : 0.0f;
  if (SIM) {  // lane holds dk[key 16 w + 4 g + r][dim 16 dt + c]; this block's keys are this workgroup's alone
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jo = J * kBwTile + 16 * w + 4 * g + r;
      if (jo < N) {
        float* o = a.dk + (((int64_t)b * N + jo) * a.Hkv + h) * D + c;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[16 * dt] += dkj[dt][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 6. decay gradients, row pass (token block I, key blocks J <= I): dlq_t and
// dlb_t = sum_j g_tj, and dk_t += sum_j ds_tj k_j on the matrix cores.  Wave
// w: tokens 16 w + c.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBwThreads) void bwd_decay_row_kernel(BwArgs a) {
  constexpr int LS = D + 4, LT = kBwTile + 4, DT = D / 16;
  __shared__ __attribute__((aligned(16))) float s_kj[kBwTile * LS];
  __shared__ __attribute__((aligned(16))) float s_ds[kBwTile * LT];
  __shared__ __attribute__((aligned(16))) float s_gn[kBwTile * LT];
  const int s = blockIdx.x, I = blockIdx.y;
  const int b = s / a.Hkv, h = s - b * a.Hkv;
  const int N = a.N;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int t = I * kBwTile + 16 * w + c;
  const int n_terms = __popc(a.terms & 7);
  const bool SIM = (a.terms & 4) != 0;
  f32x4 dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dkt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float gs = 0.0f;
  const float* gnS = a.dlam + (int64_t)s * N * N;
  const float* dsS = a.lam + (int64_t)s * N * N;
  if (n_terms) {
    for (int J = 0; J <= I; ++J) {
      __syncthreads();
      if (SIM) stage_rows<D, BF16>(s_kj, a.kt, b, N, a.Hkv, h, J * kBwTile);
      for (int e = threadIdx.x; e < kBwTile * kBwTile; e += kBwThreads) {
        const int r = e / kBwTile, col = e - r * kBwTile;
        const int tt = I * kBwTile + r, jj = J * kBwTile + col;
        const bool ok = tt < N && jj < N;
        s_gn[r * LT + col] = ok ? gnS[(int64_t)tt * N + jj] : 0.0f;
        s_ds[r * LT + col] = (ok && SIM) ? dsS[(int64_t)tt * N + jj] : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 16; ++k) gs += s_gn[(16 * w + c) * LT + 16 * g + k];
      if (SIM) {
#pragma unroll 4
        for (int st = 0; st < 16; ++st) {
          const float av = s_ds[(16 * w + c) * LT + 4 * st + g];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) dkt[dt] = mfma4(av, s_kj[(4 * st + g) * LS + 16 * dt + c], dkt[dt]);
        }
      }
    }
  }
  gs += __shfl_xor(gs, 16, 64);
  gs += __shfl_xor(gs, 32, 64);
  if (g == 0 && t < N) {
    const int64_t gi = ((int64_t)b * N + t) * a.Hkv + h;
    a.dlq[gi] = (a.terms & 1) ? gs : 0.0f;
    a.dlb[gi] = (a.terms & 4) ? gs : 0.0f;
  }
  if (n_terms && SIM) {  // lane holds dk[token 16 w + 4 g + r][dim 16 dt + c]; this block's tokens are ours alone
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int to = I * kBwTile + 16 * w + 4 * g + r;
      if (to < N) {
        float* o = a.dk + (((int64_t)b * N + to) * a.Hkv + h) * D + c;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[16 * dt] += dkt[dt][r];
      }
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
  const int nh = (nb + 1) / 2;  // paired blocks
  hipLaunchKernelGGL((bwd_stats_kernel<D, BF16>), dim3(S * G, nh), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_kv_kernel<D, BF16>), dim3(S, nb), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_q_kernel<D, BF16>), dim3(S * G, nh), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_decay_col_kernel<D, BF16>), dim3(S, nb), dim3(kBwThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_decay_row_kernel<D, BF16>), dim3(S, nb), dim3(kBwThreads), 0, st, a);
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

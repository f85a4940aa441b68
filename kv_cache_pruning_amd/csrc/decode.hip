// UA decode step on a ragged, per-KV-head pruned cache (gfx950).
//
// Two kernels on the caller's stream:
//  1. decode_pre  -- one workgroup per sequence: gate GEMV (x W_dec + b_dec,
//     x W_dn), output gate sigmoid(u W_up + b_up), RoPE of q and of the
//     normalised k (angles in fp64), cache append of (k~, v, 0, lk), length and
//     position updates.  ("A Self-Pruning Transformer ...", ai4snews Figure 1
//     caption: L2-normalised keys, RoPE, low-rank sigmoid output gate.)
//  2. decode_main -- one workgroup per tile of live entries of a segment
//     (segment = one (sequence, KV head)).  Each cached entry is read once:
//     its key feeds both <q~, k~_j> for the G query heads and <k~_t, k~_j> for
//     the similarity term; the pair term updates its log-bias in place; entries
//     below log p drop out of this step; an online-softmax partial (max, sum,
//     weighted V) is formed per tile.  The last tile of a segment to finish
//     merges the partials, adds the new token's own term and applies the gate.
//     (paperlayer.ai sections 4-4.2: geometric-mean decay in log space,
//     per-KV scalar bias, threshold eviction per head.)
//
// Lane layout of decode_main: a wave splits into groups of LPE = d/8 lanes;
// lane c of a group holds dims [8c, 8c+8) of one entry at a time, so each
// 16-byte (bf16) row load of a group is contiguous and a wave's load
// instruction covers 64/LPE whole rows.  Each group walks NB = 8 consecutive
// entries; dot products are reduced inside the group with DPP.

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

// ---------------------------------------------------------------------------
// 1. per-token preprocessing and append
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void decode_pre(LayerArgs a, DecodeWs w) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int D = a.d;
  const int half = D >> 1;
  const int Hkv = a.H_kv;
  const int Hq = a.H_q;
  const int Dm = a.D_model;
  const int r = a.r;
  const int NC = 3 * Hkv + r;

  __shared__ float s_z[3 * kMaxHkv + kMaxRank];
  __shared__ float s_red[4][8];
  __shared__ float s_cos[64];
  __shared__ float s_sin[64];

  const int pos = a.next_pos[b];

  // z = x W_dec (columns 0..3Hkv-1) and u = x W_dn (columns 3Hkv..NC-1)
  for (int c0 = 0; c0 < NC; c0 += 8) {
    float acc[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) acc[cc] = 0.0f;
    for (int i = tid; i < Dm; i += 256) {
      const float xi = load_elem<BF16>(a.x, (int64_t)b * Dm + i);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int c = c0 + cc;
        if (c < 3 * Hkv) {
          acc[cc] = fmaf(xi, load_elem<BF16>(a.W_dec, (int64_t)i * 3 * Hkv + c), acc[cc]);
        } else if (c < NC) {
          acc[cc] = fmaf(xi, load_elem<BF16>(a.W_dn, (int64_t)i * r + (c - 3 * Hkv)), acc[cc]);
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float v = wave_sum(acc[cc]);
      if (lane == 0) s_red[wave][cc] = v;
    }
    __syncthreads();
    if (tid < 8 && c0 + tid < NC) {
      float z = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
      if (c0 + tid < 3 * Hkv) z += a.b_dec[c0 + tid];
      s_z[c0 + tid] = z;
    }
    __syncthreads();
  }

  // RoPE angles in fp64, rounded to fp32
  if (tid < half) {
    const double wfreq = pow(a.rope_base, -2.0 * (double)tid / (double)D);
    const double phi = (double)pos * wfreq;
    double sn, cs;
    sincos(phi, &sn, &cs);
    s_cos[tid] = (float)cs;
    s_sin[tid] = (float)sn;
  }
  __syncthreads();

  // output gate: gamma = sigmoid(u W_up + b_up), [H_q * d]
  const float* u = s_z + 3 * Hkv;
  for (int o = tid; o < Hq * D; o += 256) {
    float g = a.b_up ? a.b_up[o] : 0.0f;
    for (int c = 0; c < r; ++c) g = fmaf(u[c], load_elem<BF16>(a.W_up, (int64_t)c * Hq * D + o), g);
    w.gamma[(int64_t)b * Hq * D + o] = sigmoid(g);
  }

  // rotated queries
  for (int o = tid; o < Hq * D; o += 256) {
    const int i = o % D;
    const int64_t base = (int64_t)b * Hq * D + (o - i);
    const float xv = load_elem<BF16>(a.q, base + i);
    float out;
    if (i < half) {
      out = fmaf(xv, s_cos[i], -load_elem<BF16>(a.q, base + i + half) * s_sin[i]);
    } else {
      out = fmaf(xv, s_cos[i - half], load_elem<BF16>(a.q, base + i - half) * s_sin[i - half]);
    }
    w.qt[base + i] = out;
  }

  // keys: normalise, rotate, round to the cache type, append
  for (int h = wave; h < Hkv; h += 4) {
    const int s = b * Hkv + h;
    const int64_t base = (int64_t)s * D;
    float k0 = 0.0f, k1 = 0.0f;
    if (lane < half) {
      k0 = load_elem<BF16>(a.k, base + lane);
      k1 = load_elem<BF16>(a.k, base + lane + half);
    }
    const float ss = wave_sum(k0 * k0 + k1 * k1);
    const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
    k0 *= inv;
    k1 *= inv;
    float r0 = 0.0f, r1 = 0.0f;
    if (lane < half) {
      r0 = fmaf(k0, s_cos[lane], -k1 * s_sin[lane]);
      r1 = fmaf(k1, s_cos[lane], k0 * s_sin[lane]);
    }
    uint16_t h0 = 0, h1 = 0;
    if constexpr (BF16) {
      h0 = f32_to_bf16(r0);
      h1 = f32_to_bf16(r1);
      r0 = bf16_to_f32(h0);
      r1 = bf16_to_f32(h1);
    }
    const int len = a.seg_len[s];
    const int cap = a.seg_cap[s];
    const int64_t off = a.seg_off[s];
    const bool room = len < cap;
    if (lane < half) {
      w.kt[base + lane] = r0;
      w.kt[base + lane + half] = r1;
      if (room) {
        const int64_t dst = (off + len) * D;
        if constexpr (BF16) {
          uint16_t* K = reinterpret_cast<uint16_t*>(a.K);
          uint16_t* V = reinterpret_cast<uint16_t*>(a.V);
          const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v);
          K[dst + lane] = h0;
          K[dst + lane + half] = h1;
          V[dst + lane] = vin[base + lane];
          V[dst + lane + half] = vin[base + lane + half];
        } else {
          float* K = reinterpret_cast<float*>(a.K);
          float* V = reinterpret_cast<float*>(a.V);
          const float* vin = reinterpret_cast<const float*>(a.v);
          K[dst + lane] = r0;
          K[dst + lane + half] = r1;
          V[dst + lane] = vin[base + lane];
          V[dst + lane + half] = vin[base + lane + half];
        }
      }
    }
    if (lane == 0) {
      const float lq = log_sigmoid(s_z[h]);
      const float lkk = log_sigmoid(s_z[Hkv + h]);
      const float lb = log_sigmoid(s_z[2 * Hkv + h]);
      w.gates[s * 4 + 0] = lq;
      w.gates[s * 4 + 1] = lkk;
      w.gates[s * 4 + 2] = lb;
      w.gates[s * 4 + 3] = 0.0f;
      w.len_old[s] = len;
      w.cnt[s] = 0;
      if (room) {
        a.lam[off + len] = 0.0f;
        a.lk[off + len] = lkk;
        a.seg_len[s] = len + 1;
      } else {
        atomicOr(a.status, 1);
      }
    }
  }
  __syncthreads();
  if (tid == 0) a.next_pos[b] = pos + 1;
}

// ---------------------------------------------------------------------------
// 2. tile kernel + last-workgroup combine
// ---------------------------------------------------------------------------
template <bool BF16>
struct Row8 {
  uint4 w[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void row_load(Row8<BF16>& r, const void* base, int64_t elem) {
  if constexpr (BF16) {
    r.w[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + elem);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
}

template <bool BF16>
__device__ __forceinline__ void row_f32(const Row8<BF16>& r, float (&o)[8]) {
  if constexpr (BF16) {
    o[0] = bf16_lo(r.w[0].x); o[1] = bf16_hi(r.w[0].x);
    o[2] = bf16_lo(r.w[0].y); o[3] = bf16_hi(r.w[0].y);
    o[4] = bf16_lo(r.w[0].z); o[5] = bf16_hi(r.w[0].z);
    o[6] = bf16_lo(r.w[0].w); o[7] = bf16_hi(r.w[0].w);
  } else {
    o[0] = __uint_as_float(r.w[0].x); o[1] = __uint_as_float(r.w[0].y);
    o[2] = __uint_as_float(r.w[0].z); o[3] = __uint_as_float(r.w[0].w);
    o[4] = __uint_as_float(r.w[1].x); o[5] = __uint_as_float(r.w[1].y);
    o[6] = __uint_as_float(r.w[1].z); o[7] = __uint_as_float(r.w[1].w);
  }
}

template <int D>
struct DecodeShape {
  static constexpr int LPE = D / 8;       // lanes per entry
  static constexpr int NGW = 64 / LPE;    // entry groups per wave
  static constexpr int NB = 8;            // entries per group
  static constexpr int TW = NGW * NB;     // entries per wave
  static constexpr int NWAVE = 4;
  static constexpr int NT = 64 * NWAVE;
  static constexpr int TWG = TW * NWAVE;  // entries per workgroup tile
  static constexpr int NP = NGW * NWAVE;  // partials per workgroup
};

__device__ __forceinline__ int n_tiles_of(int len, int twg) { return len <= 0 ? 1 : (len + twg - 1) / twg; }

template <int D, int G, bool BF16>
__global__ __launch_bounds__(DecodeShape<D>::NT) void decode_main(LayerArgs a, DecodeWs w, float tau) {
  using Sh = DecodeShape<D>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, NT = Sh::NT, TWG = Sh::TWG, NP = Sh::NP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int S = a.B * a.H_kv;

  __shared__ int s_scan[NT / 64 + 1];
  __shared__ int s_info[4];  // segment, tile within segment, tiles of segment, first partial
  __shared__ int s_last;
  __shared__ float s_po[NP * G * D];
  __shared__ float s_pm[NP * G];
  __shared__ float s_pl[NP * G];

  // ---- map this workgroup to (segment, tile) by a block scan of tile counts
  const int per = (S + NT - 1) / NT;
  const int sb = tid * per;
  const int se = min(S, sb + per);
  int mine = 0;
  for (int s = sb; s < se; ++s) mine += n_tiles_of(w.len_old[s], TWG);
  int total;
  const int excl = block_exclusive_scan<NT>(mine, s_scan, &total);
  const int tile = blockIdx.x;
  if (tile >= total) return;
  {
    int run = excl;
    for (int s = sb; s < se; ++s) {
      const int nt = n_tiles_of(w.len_old[s], TWG);
      if (tile >= run && tile < run + nt) {
        s_info[0] = s;
        s_info[1] = tile - run;
        s_info[2] = nt;
        s_info[3] = run;
      }
      run += nt;
    }
  }
  __syncthreads();
  const int seg = s_info[0];
  const int kt_ = s_info[1];
  const int ntile = s_info[2];
  const int pbase = s_info[3];
  const int b = seg / a.H_kv;
  const int h = seg - b * a.H_kv;
  const int len = w.len_old[seg];
  const int64_t off = a.seg_off[seg];

  const int grp = lane / LPE;
  const int c = lane - grp * LPE;
  const int e0 = kt_ * TWG + wv * TW + grp * NB;  // first entry of this group

  // ---- issue the loads for NB entries
  Row8<BF16> kr[NB], vr[NB];
  float lamv[NB], lkv[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int j = e0 + bb;
    if (j < len) {
      row_load<BF16>(kr[bb], a.K, (off + j) * D + 8 * c);
      row_load<BF16>(vr[bb], a.V, (off + j) * D + 8 * c);
      lamv[bb] = a.lam[off + j];
      lkv[bb] = a.lk[off + j];
    } else {
      lamv[bb] = kNegInf;
      lkv[bb] = 0.0f;
#pragma unroll
      for (int t = 0; t < (BF16 ? 1 : 2); ++t) kr[bb].w[t] = vr[bb].w[t] = make_uint4(0, 0, 0, 0);
    }
  }

  // ---- query-side data for this segment (L2-resident workspace)
  float qv[G][8];
  float ktv[8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float4* p = reinterpret_cast<const float4*>(w.qt + ((int64_t)b * a.H_q + h * G + g) * D + 8 * c);
    const float4 x0 = p[0], x1 = p[1];
    qv[g][0] = x0.x; qv[g][1] = x0.y; qv[g][2] = x0.z; qv[g][3] = x0.w;
    qv[g][4] = x1.x; qv[g][5] = x1.y; qv[g][6] = x1.z; qv[g][7] = x1.w;
  }
  {
    const float4* p = reinterpret_cast<const float4*>(w.kt + (int64_t)seg * D + 8 * c);
    const float4 x0 = p[0], x1 = p[1];
    ktv[0] = x0.x; ktv[1] = x0.y; ktv[2] = x0.z; ktv[3] = x0.w;
    ktv[4] = x1.x; ktv[5] = x1.y; ktv[6] = x1.z; ktv[7] = x1.w;
  }
  const PairCoef pc = pair_coef(a.terms);
  const float lq = w.gates[seg * 4 + 0];
  const float lb = w.gates[seg * 4 + 2];
  const float row2 = (((a.terms & 1) ? lq : 0.0f) + ((a.terms & 4) ? lb : 0.0f)) * pc.inv_n2;
  const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;
  const float qs2 = a.scale * kLog2e;

  // ---- dot products, pair term, bias update, logits
  float e2[G][NB];
  float newlam[NB];
  bool changed[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    float kf[8];
    row_f32<BF16>(kr[bb], kf);
    float ps = 0.0f;
    float pq[G];
#pragma unroll
    for (int g = 0; g < G; ++g) pq[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ps = fmaf(ktv[i], kf[i], ps);
#pragma unroll
      for (int g = 0; g < G; ++g) pq[g] = fmaf(qv[g][i], kf[i], pq[g]);
    }
    ps = group_sum<LPE>(ps);
#pragma unroll
    for (int g = 0; g < G; ++g) pq[g] = group_sum<LPE>(pq[g]);

    const float l0 = lamv[bb];
    const bool valid = e0 + bb < len;
    const bool alive = valid && (l0 >= tau);
    const float A = pair_A(pc, row2, lkv[bb] * kscale, ps);
    const float l1 = alive ? l0 + A : l0;
    const bool live = alive && (l1 >= tau);
    newlam[bb] = l1;
    changed[bb] = alive;
    const float lb2 = l1 * kLog2e;
#pragma unroll
    for (int g = 0; g < G; ++g) e2[g][bb] = live ? fmaf(pq[g], qs2, lb2) : kNegInf;
  }

  // ---- write back the updated biases: lane c of a group stores entry c
  if (c < NB) {
    float val = newlam[0];
    bool ch = changed[0];
#pragma unroll
    for (int bb = 1; bb < NB; ++bb) {
      val = (c == bb) ? newlam[bb] : val;
      ch = (c == bb) ? changed[bb] : ch;
    }
    if (ch) a.lam[off + e0 + c] = val;
  }

  // ---- group-level softmax partial
  const int pidx = wv * NGW + grp;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = e2[g][0];
#pragma unroll
    for (int bb = 1; bb < NB; ++bb) m = fmaxf(m, e2[g][bb]);
    const float ms = (m == kNegInf) ? 0.0f : m;
    float l = 0.0f;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.0f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const float p = __builtin_amdgcn_exp2f(e2[g][bb] - ms);
      l += p;
      float vf[8];
      row_f32<BF16>(vr[bb], vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(p, vf[i], o[i]);
    }
    float4* dst = reinterpret_cast<float4*>(s_po + (pidx * G + g) * D + 8 * c);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    if (c == 0) {
      s_pm[pidx * G + g] = m;
      s_pl[pidx * G + g] = l;
    }
  }
  __syncthreads();

  // ---- merge the NP group partials of this workgroup
  const int64_t prow = (int64_t)(pbase + kt_);
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int i = idx - g * D;
    float M = kNegInf;
#pragma unroll 4
    for (int p = 0; p < NP; ++p) M = fmaxf(M, s_pm[p * G + g]);
    const float Ms = (M == kNegInf) ? 0.0f : M;
    float L = 0.0f, O = 0.0f;
#pragma unroll 4
    for (int p = 0; p < NP; ++p) {
      const float wgt = __builtin_amdgcn_exp2f(s_pm[p * G + g] - Ms);
      L = fmaf(s_pl[p * G + g], wgt, L);
      O = fmaf(s_po[(p * G + g) * D + i], wgt, O);
    }
    w.part_o[(prow * G + g) * D + i] = O;
    if (i == 0) {
      w.part_ml[(prow * G + g) * 2 + 0] = M;
      w.part_ml[(prow * G + g) * 2 + 1] = L;
    }
  }

  // ---- the last tile of the segment combines
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&w.cnt[seg], 1);
    s_last = (old == ntile - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // self logits e_self[g] = scale log2e <q~_g, k~_t>, reduced through LDS
  float* s_prod = s_po;  // reuse: G * D floats
  __shared__ float s_self[8];
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int i = idx - g * D;
    s_prod[idx] = w.qt[((int64_t)b * a.H_q + h * G + g) * D + i] * w.kt[(int64_t)seg * D + i];
  }
  __syncthreads();
  if (tid < G) {
    float acc = 0.0f;
    for (int i = 0; i < D; ++i) acc += s_prod[tid * D + i];
    s_self[tid] = acc * qs2;
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int i = idx - g * D;
    const float es = s_self[g];
    float M = es;
    for (int p = 0; p < ntile; ++p) M = fmaxf(M, w.part_ml[((int64_t)(pbase + p) * G + g) * 2 + 0]);
    float L = __builtin_amdgcn_exp2f(es - M);
    const float vt = load_elem<BF16>(a.v, (int64_t)seg * D + i);
    float O = L * vt;
    for (int p = 0; p < ntile; ++p) {
      const int64_t pr = (int64_t)(pbase + p);
      const float wgt = __builtin_amdgcn_exp2f(w.part_ml[(pr * G + g) * 2 + 0] - M);
      L = fmaf(w.part_ml[(pr * G + g) * 2 + 1], wgt, L);
      O = fmaf(w.part_o[(pr * G + g) * D + i], wgt, O);
    }
    const int64_t yo = ((int64_t)b * a.H_q + h * G + g) * D + i;
    const float yv = w.gamma[yo] * (O / L);
    if (a.y_bf16) {
      reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16(yv);
    } else {
      reinterpret_cast<float*>(a.y)[yo] = yv;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int decode_tile_entries(int d) { return d == 64 ? DecodeShape<64>::TWG : DecodeShape<128>::TWG; }

static int decode_max_tiles(const LayerArgs& a, int twg) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  return (int)(a.total_slots / twg + S + 1);
}

size_t decode_ws_bytes(const LayerArgs& a, int twg) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int G = a.H_q / a.H_kv;
  const int64_t mt = decode_max_tiles(a, twg);
  size_t n = 0;
  n += align_up(sizeof(float) * a.B * a.H_q * a.d, 256);  // qt
  n += align_up(sizeof(float) * S * a.d, 256);            // kt
  n += align_up(sizeof(float) * S * 4, 256);              // gates
  n += align_up(sizeof(float) * a.B * a.H_q * a.d, 256);  // gamma
  n += align_up(sizeof(int) * S, 256);                    // len_old
  n += align_up(sizeof(int) * S, 256);                    // cnt
  n += align_up(sizeof(float) * mt * G * a.d, 256);       // part_o
  n += align_up(sizeof(float) * mt * G * 2, 256);         // part_ml
  return n;
}

DecodeWs decode_ws_carve(const LayerArgs& a, void* ws, int twg) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int G = a.H_q / a.H_kv;
  const int64_t mt = decode_max_tiles(a, twg);
  char* p = reinterpret_cast<char*>(ws);
  DecodeWs w;
  auto take = [&](size_t bytes) {
    char* q = p;
    p += align_up(bytes, 256);
    return q;
  };
  w.qt = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  w.kt = reinterpret_cast<float*>(take(sizeof(float) * S * a.d));
  w.gates = reinterpret_cast<float*>(take(sizeof(float) * S * 4));
  w.gamma = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  w.len_old = reinterpret_cast<int*>(take(sizeof(int) * S));
  w.cnt = reinterpret_cast<int*>(take(sizeof(int) * S));
  w.part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  w.part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  w.max_tiles = (int)mt;
  return w;
}

template <int D, int G, bool BF16>
static hipError_t launch_main(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  using Sh = DecodeShape<D>;
  hipLaunchKernelGGL((decode_main<D, G, BF16>), dim3(w.max_tiles), dim3(Sh::NT), 0, st, a, w, tau);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_main_g(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  switch (a.H_q / a.H_kv) {
    case 1: return launch_main<D, 1, BF16>(a, w, tau, st);
    case 2: return launch_main<D, 2, BF16>(a, w, tau, st);
    case 3: return launch_main<D, 3, BF16>(a, w, tau, st);
    case 4: return launch_main<D, 4, BF16>(a, w, tau, st);
    case 8: return launch_main<D, 8, BF16>(a, w, tau, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  if (a.bf16) {
    hipLaunchKernelGGL((decode_pre<true>), dim3(a.B), dim3(256), 0, st, a, w);
  } else {
    hipLaunchKernelGGL((decode_pre<false>), dim3(a.B), dim3(256), 0, st, a, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 64) return a.bf16 ? launch_main_g<64, true>(a, w, tau, st) : launch_main_g<64, false>(a, w, tau, st);
  return a.bf16 ? launch_main_g<128, true>(a, w, tau, st) : launch_main_g<128, false>(a, w, tau, st);
}

}  // namespace ua

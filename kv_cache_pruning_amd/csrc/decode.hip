// UA decode step on a ragged, per-KV-head pruned cache (gfx950), one kernel.
//
// A segment is the cache of one (sequence b, KV head h).  The grid covers
// every segment's capacity in tiles of TWG entries (a fixed mapping from the
// read-only capacities, so no workgroup ever depends on a length another
// workgroup is updating).  A tile at or beyond the segment's current length
// does no work except take part in the segment's arrival count.
//
// A working tile:
//  * issues the loads of its TWG cached entries first (K, V rows, log-bias,
//    key gate), then, while they are in flight, forms the token-side data of
//    its segment in LDS: RoPE table (fp64 angles), the three gates of head h
//    (x W_dec + b_dec, log-sigmoid), the G rotated queries and the stored new
//    key (normalised, rotated, rounded to the cache type).  ("A Self-Pruning
//    Transformer ...", ai4snews Figure 1 caption: L2-normalised keys, RoPE.)
//  * walks its entries once: each key row feeds <q~_g, k~_j> for the G query
//    heads and <k~_t, k~_j> for the similarity term; the pair term (geometric
//    mean of the enabled decays in log space, paperlayer.ai sections 4 and
//    4.1) is added to the log-bias in place; entries below log p drop out of
//    this step (section 4.2); an online-softmax partial (max, sum, weighted V)
//    is written per tile.
//  * tile 0 also appends the new entry and forms the output gate
//    sigmoid((x W_dn) W_up + b_up) and the new token's own logit.
// The last of a segment's tiles to arrive merges the partials, adds the new
// token's own term, applies the gate and advances the segment length; the
// last segment of a sequence advances its position.
//
// Cross-workgroup data (partials, gate, counters) use relaxed agent-scope
// atomic loads/stores, which are coherent across the XCDs without cache-wide
// write-back or invalidation; counters return to zero at the end of every
// call, so the workspace only has to be zeroed once before first use.
//
// Lane layout of the entry loop: a wave splits into groups of LPE = d/8
// lanes; lane c of a group holds dims [8c, 8c+8) of one entry at a time, so a
// group's 16-byte (bf16) row loads are contiguous.  Each group walks NB = 8
// consecutive entries; dot products are reduced inside the group with DPP.

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_coh(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sti_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool BF16>
struct Row8 {
  u32x4 w[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void row_load(Row8<BF16>& r, const void* base, int64_t elem) {
  if constexpr (BF16) {
    r.w[0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(base) + elem);
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

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int tiles_of(int n, int twg) { return n <= 0 ? 1 : ceil_div(n, twg); }

// Block sum of one value per thread (NT = 256); every thread gets the sum.
__device__ __forceinline__ float block_sum256(float v, float* s_red4) {
  v = wave_sum(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red4[wv] = v;
  __syncthreads();
  return s_red4[0] + s_red4[1] + s_red4[2] + s_red4[3];
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(DecodeShape<D>::NT) void decode_step_kernel(LayerArgs a, DecodeWs w, float tau) {
  using Sh = DecodeShape<D>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, NT = Sh::NT, TWG = Sh::TWG, NP = Sh::NP;
  constexpr int HALF = D / 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int S = a.B * a.H_kv;
  const int Hkv = a.H_kv;
  const int Dm = a.D_model;

  __shared__ int s_scan[NT / 64 + 1];
  __shared__ int s_info[4];
  __shared__ int s_last;
  __shared__ float s_red[4];
  __shared__ float s_cos[HALF], s_sin[HALF];
  __shared__ float s_z[3];
  __shared__ float s_u[kMaxRank];
  __shared__ float s_q[G * D];
  __shared__ float s_kt[D];
  __shared__ float s_self[G];
  __shared__ float s_po[NP * G * D];
  __shared__ float s_pm[NP * G];
  __shared__ float s_pl[NP * G];

  // ---- (segment, tile) from the read-only capacities
  {
    const int per = (S + NT - 1) / NT;
    const int sb = tid * per;
    const int se = min(S, sb + per);
    int mine = 0;
    for (int s = sb; s < se; ++s) mine += tiles_of(a.seg_cap[s], TWG);
    int total;
    const int excl = block_exclusive_scan<NT>(mine, s_scan, &total);
    if ((int)blockIdx.x >= total) return;
    int run = excl;
    for (int s = sb; s < se; ++s) {
      const int nt = tiles_of(a.seg_cap[s], TWG);
      if ((int)blockIdx.x >= run && (int)blockIdx.x < run + nt) {
        s_info[0] = s;
        s_info[1] = blockIdx.x - run;
        s_info[2] = nt;
        s_info[3] = run;
      }
      run += nt;
    }
    __syncthreads();
  }
  const int seg = s_info[0];
  const int kt_ = s_info[1];
  const int nwg = s_info[2];   // workgroups of this segment (all arrive)
  const int pbase = s_info[3];  // first partial row of this segment
  const int b = seg / Hkv;
  const int h = seg - b * Hkv;
  const int len = a.seg_len[seg];  // length before this step's append
  const int cap = a.seg_cap[seg];
  const int64_t off = a.seg_off[seg];
  const int ntile = tiles_of(len, TWG);  // working tiles
  const bool work = kt_ < ntile;

  if (work) {
    const int grp = lane / LPE;
    const int c = lane - grp * LPE;
    const int e0 = kt_ * TWG + wv * TW + grp * NB;

    // ---- cached entries: issue every load first
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
        for (int t = 0; t < (BF16 ? 1 : 2); ++t) kr[bb].w[t] = vr[bb].w[t] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    // ---- token-side data of this segment (overlaps the loads above)
    const int pos = a.next_pos[b];
    if (tid < HALF) {
      const double wfreq = pow(a.rope_base, -2.0 * (double)tid / (double)D);
      double sn, cs;
      sincos((double)pos * wfreq, &sn, &cs);
      s_cos[tid] = (float)cs;
      s_sin[tid] = (float)sn;
    }
    {
      float g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
      const int64_t xb = (int64_t)b * Dm;
      for (int i = tid; i < Dm; i += NT) {
        const float xi = load_elem<BF16>(a.x, xb + i);
        const int64_t row = (int64_t)i * 3 * Hkv;
        g0 = fmaf(xi, load_elem<BF16>(a.W_dec, row + h), g0);
        g1 = fmaf(xi, load_elem<BF16>(a.W_dec, row + Hkv + h), g1);
        g2 = fmaf(xi, load_elem<BF16>(a.W_dec, row + 2 * Hkv + h), g2);
      }
      g0 = block_sum256(g0, s_red);
      g1 = block_sum256(g1, s_red);
      g2 = block_sum256(g2, s_red);
      if (tid == 0) {
        s_z[0] = g0 + a.b_dec[h];
        s_z[1] = g1 + a.b_dec[Hkv + h];
        s_z[2] = g2 + a.b_dec[2 * Hkv + h];
      }
    }
    __syncthreads();  // s_cos / s_sin / s_z ready
    for (int o = tid; o < G * D; o += NT) {
      const int g = o / D;
      const int i = o - g * D;
      const int64_t base = ((int64_t)b * a.H_q + h * G + g) * D;
      const float xv = load_elem<BF16>(a.q, base + i);
      float out;
      if (i < HALF) {
        out = fmaf(xv, s_cos[i], -load_elem<BF16>(a.q, base + i + HALF) * s_sin[i]);
      } else {
        out = fmaf(xv, s_cos[i - HALF], load_elem<BF16>(a.q, base + i - HALF) * s_sin[i - HALF]);
      }
      s_q[o] = out;
    }
    uint16_t kb0 = 0, kb1 = 0;
    float kst0 = 0.0f, kst1 = 0.0f;
    if (wv == 0) {
      const int64_t kbase = (int64_t)seg * D;
      float k0 = 0.0f, k1 = 0.0f;
      if (lane < HALF) {
        k0 = load_elem<BF16>(a.k, kbase + lane);
        k1 = load_elem<BF16>(a.k, kbase + lane + HALF);
      }
      const float inv = 1.0f / fmaxf(sqrtf(wave_sum(k0 * k0 + k1 * k1)), 1e-12f);
      k0 *= inv;
      k1 *= inv;
      if (lane < HALF) {
        kst0 = fmaf(k0, s_cos[lane], -k1 * s_sin[lane]);
        kst1 = fmaf(k1, s_cos[lane], k0 * s_sin[lane]);
        if constexpr (BF16) {
          kb0 = f32_to_bf16(kst0);
          kb1 = f32_to_bf16(kst1);
          kst0 = bf16_to_f32(kb0);
          kst1 = bf16_to_f32(kb1);
        }
        s_kt[lane] = kst0;
        s_kt[lane + HALF] = kst1;
      }
    }
    __syncthreads();  // s_q, s_kt ready

    float qv[G][8];
    float ktv[8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[g][i] = s_q[g * D + 8 * c + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) ktv[i] = s_kt[8 * c + i];
    const PairCoef pc = pair_coef(a.terms);
    const float lq = log_sigmoid(s_z[0]);
    const float lb = log_sigmoid(s_z[2]);
    const float row2 = (((a.terms & 1) ? lq : 0.0f) + ((a.terms & 4) ? lb : 0.0f)) * pc.inv_n2;
    const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;
    const float qs2 = a.scale * kLog2e;

    // ---- entry loop: dot products, pair term, bias update, logits
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
    if (c < NB) {  // lane c of a group stores entry c's bias
      float val = newlam[0];
      bool ch = changed[0];
#pragma unroll
      for (int bb = 1; bb < NB; ++bb) {
        val = (c == bb) ? newlam[bb] : val;
        ch = (c == bb) ? changed[bb] : ch;
      }
      if (ch) a.lam[off + e0 + c] = val;
    }

    // ---- group partials -> LDS
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

    // ---- merge the workgroup's partials -> workspace row pbase + kt_
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
      st_coh(w.part_o + (prow * G + g) * D + i, O);
      if (i == 0) {
        st_coh(w.part_ml + (prow * G + g) * 2 + 0, M);
        st_coh(w.part_ml + (prow * G + g) * 2 + 1, L);
      }
    }

    // ---- tile 0: output gate, own logit, append
    if (kt_ == 0) {
      const int r = a.r;
      float u[8];
      for (int c0 = 0; c0 < r; c0 += 8) {
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) u[cc] = 0.0f;
        for (int i = tid; i < Dm; i += NT) {
          const float xi = load_elem<BF16>(a.x, (int64_t)b * Dm + i);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc)
            if (c0 + cc < r) u[cc] = fmaf(xi, load_elem<BF16>(a.W_dn, (int64_t)i * r + c0 + cc), u[cc]);
        }
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const float t = block_sum256(u[cc], s_red);
          if (tid == 0 && c0 + cc < r) s_u[c0 + cc] = t;
        }
      }
      __syncthreads();
      for (int o = tid; o < G * D; o += NT) {
        const int col = (h * G) * D + o;  // W_up column a*d + i with a = h*G + g
        float gsum = a.b_up ? a.b_up[col] : 0.0f;
        for (int cc = 0; cc < r; ++cc) gsum = fmaf(s_u[cc], load_elem<BF16>(a.W_up, (int64_t)cc * a.H_q * D + col), gsum);
        st_coh(w.gamma + (int64_t)seg * G * D + o, sigmoid(gsum));
      }
      if (tid < G) {
        float acc = 0.0f;
        for (int i = 0; i < D; ++i) acc = fmaf(s_q[tid * D + i], s_kt[i], acc);
        st_coh(w.eself + seg * G + tid, acc * qs2);
      }
      if (len < cap) {
        if (wv == 0 && lane < HALF) {
          const int64_t dst = (off + len) * D;
          const int64_t vb = (int64_t)seg * D;
          if constexpr (BF16) {
            uint16_t* K = reinterpret_cast<uint16_t*>(a.K);
            uint16_t* V = reinterpret_cast<uint16_t*>(a.V);
            const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v);
            K[dst + lane] = kb0;
            K[dst + lane + HALF] = kb1;
            V[dst + lane] = vin[vb + lane];
            V[dst + lane + HALF] = vin[vb + lane + HALF];
          } else {
            float* K = reinterpret_cast<float*>(a.K);
            float* V = reinterpret_cast<float*>(a.V);
            const float* vin = reinterpret_cast<const float*>(a.v);
            K[dst + lane] = kst0;
            K[dst + lane + HALF] = kst1;
            V[dst + lane] = vin[vb + lane];
            V[dst + lane + HALF] = vin[vb + lane + HALF];
          }
        }
        if (tid == 0) {
          a.lam[off + len] = 0.0f;
          a.lk[off + len] = log_sigmoid(s_z[1]);
        }
      } else if (tid == 0) {
        atomicOr(a.status, 1);
      }
    }
  }

  // ---- arrival; the last workgroup of the segment combines
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = (add_coh(&w.cnt[seg], 1) == nwg - 1);
  __syncthreads();
  if (!s_last) return;

  if (tid < G) s_self[tid] = ld_coh(w.eself + seg * G + tid);
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int i = idx - g * D;
    const float es = s_self[g];
    float M = es;
    for (int p = 0; p < ntile; ++p) M = fmaxf(M, ld_coh(w.part_ml + ((int64_t)(pbase + p) * G + g) * 2 + 0));
    float L = __builtin_amdgcn_exp2f(es - M);
    float O = L * load_elem<BF16>(a.v, (int64_t)seg * D + i);
    for (int p = 0; p < ntile; ++p) {
      const int64_t pr = (int64_t)(pbase + p);
      const float wgt = __builtin_amdgcn_exp2f(ld_coh(w.part_ml + (pr * G + g) * 2 + 0) - M);
      L = fmaf(ld_coh(w.part_ml + (pr * G + g) * 2 + 1), wgt, L);
      O = fmaf(ld_coh(w.part_o + (pr * G + g) * D + i), wgt, O);
    }
    const int64_t yo = ((int64_t)b * a.H_q + h * G + g) * D + i;
    const float yv = ld_coh(w.gamma + (int64_t)seg * G * D + idx) * (O / L);
    if (a.y_bf16) {
      reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16(yv);
    } else {
      reinterpret_cast<float*>(a.y)[yo] = yv;
    }
  }
  if (tid == 0) {
    a.seg_len[seg] = len < cap ? len + 1 : len;
    sti_coh(&w.cnt[seg], 0);
    // the last segment of this sequence advances its position
    if (add_coh(&w.cntb[b], 1) == Hkv - 1) {
      a.next_pos[b] = a.next_pos[b] + 1;
      sti_coh(&w.cntb[b], 0);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int decode_tile_entries(int d) { return d == 64 ? DecodeShape<64>::TWG : DecodeShape<128>::TWG; }

static int64_t decode_max_tiles(const LayerArgs& a, int twg) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  return a.total_slots / twg + S + 1;
}

// Scratch after the control block: gate, own logits, tile partials.
static size_t decode_layout(const LayerArgs& a, int twg, DecodeWs* w, char* base) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int G = a.H_q / a.H_kv;
  const int64_t mt = decode_max_tiles(a, twg);
  size_t n = 0;
  auto take = [&](size_t bytes) {
    char* q = base ? base + n : nullptr;
    n += align_up(bytes, 256);
    return q;
  };
  float* gamma = reinterpret_cast<float*>(take(sizeof(float) * S * G * a.d));
  float* eself = reinterpret_cast<float*>(take(sizeof(float) * S * G));
  float* part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  float* part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  if (w) {
    w->gamma = gamma;
    w->eself = eself;
    w->part_o = part_o;
    w->part_ml = part_ml;
    w->max_tiles = (int)mt;
  }
  return n;
}

size_t decode_ws_bytes(const LayerArgs& a, int twg) { return decode_layout(a, twg, nullptr, nullptr); }

DecodeWs decode_ws_carve(const LayerArgs& a, const Control& ctl, void* scratch, int twg) {
  DecodeWs w{};
  decode_layout(a, twg, &w, reinterpret_cast<char*>(scratch));
  w.cnt = ctl.dec_cnt;
  w.cntb = ctl.dec_cntb;
  return w;
}

template <int D, int G, bool BF16>
static hipError_t launch_step(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  using Sh = DecodeShape<D>;
  hipLaunchKernelGGL((decode_step_kernel<D, G, BF16>), dim3(w.max_tiles), dim3(Sh::NT), 0, st, a, w, tau);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_step_g(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  switch (a.H_q / a.H_kv) {
    case 1: return launch_step<D, 1, BF16>(a, w, tau, st);
    case 2: return launch_step<D, 2, BF16>(a, w, tau, st);
    case 3: return launch_step<D, 3, BF16>(a, w, tau, st);
    case 4: return launch_step<D, 4, BF16>(a, w, tau, st);
    case 8: return launch_step<D, 8, BF16>(a, w, tau, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  if (a.d == 64) return a.bf16 ? launch_step_g<64, true>(a, w, tau, st) : launch_step_g<64, false>(a, w, tau, st);
  return a.bf16 ? launch_step_g<128, true>(a, w, tau, st) : launch_step_g<128, false>(a, w, tau, st);
}

}  // namespace ua

// Chunked UA prefill on gfx950: three kernels per call.
//
// The decay bias is applied inside a fused online softmax and the L x L bias
// matrix is never stored ("A Self-Pruning Transformer ...", paperlayer.ai
// summary, section 4.2 and Appendix C); the three decay terms are combined by
// a geometric mean, taken to log space and accumulated causally (ai4snews
// page, Figure 1 caption).
//
// Notation.  A call appends n tokens to every segment s (one sequence b and
// KV head h) that holds len0 entries.  Keys are indexed by their slot in the
// segment, j in [0, len0 + n); call-local token t is key len0 + t.  Token t's
// pair term with key j applies iff j < len0 + t, so with the stored bias
// Lambda0_j (0 for the new keys)
//     Lambda_tj = Lambda0_j + sum_{t' <= t, j < len0 + t'} A_{t'j},
// and token t attends every key j <= len0 + t with that bias.  After the call
// each key's bias is its value at the last token.
//
// 1. prefill_prep_kernel: clears the call's sync words and writes
//    [W_dec | W_dn] transposed (zero-padded to 16 rows) so that the gate
//    projections can be fed to the matrix cores with 16-byte loads.
// 2. prefill_token_kernel: 16 tokens per workgroup.  x [W_dec | W_dn] on the
//    matrix cores, log-sigmoid gates, u = x W_dn for the output gate (whose
//    sigmoid(u W_up + b_up) the attention epilogue forms per tile), RoPE of
//    the queries (bf16 copy for the matrix cores) and of the L2-normalised
//    keys (angles in fp64), and the append of k~, v and the key gate.
// 3. prefill_attn_kernel: one workgroup per (segment, block of 64 tokens),
//    four waves of 16 tokens, looping over blocks of 64 keys.  Per key block,
//    with keys as MFMA rows and the wave's tokens as columns:
//      * <k~_j, k~_t> for the similarity term and <q~_t, k~_j> for every
//        query head of the group come from 16x16x32 bf16 MFMA tiles;
//      * the pair terms are scanned over the tokens: within a wave across
//        the 16 lanes of a row (DPP), across the four waves through LDS, and
//        across token blocks through a carry per key that the workgroup of
//        the previous token block publishes (a chain per segment; workgroups
//        take their ids from an atomic ticket so every wait is on a
//        workgroup that started earlier);
//      * logits (log2 units) feed an online softmax whose reference maximum
//        is only raised when a block exceeds it by more than 2^8; the
//        probabilities go to fp16 and P V runs on 16x16x32 fp16 MFMA tiles,
//        the row sums on the same instruction with a tile of ones;
//      * the last token block writes each key's final bias to the cache.
//    The last workgroup to finish advances seg_len and next_pos.

#include <algorithm>
#include <type_traits>

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kPTok = 16;                            // tokens per token-kernel workgroup
constexpr int kPRows = 64;                           // tokens per attention workgroup
constexpr int kPKeys = 64;                           // keys per block
constexpr int kPThreads = 512;                       // attention workgroup: 8 waves
constexpr int kMaxZ = 3 * kMaxHkv + kMaxRank;        // gate-projection columns
constexpr float kRescaleTh = 8.0f;                   // log2 headroom of the softmax reference
constexpr int kPrefillSpinLimit = 1 << 22;

// ---------------------------------------------------------------------------
// workspace
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;  // XCDs of the chip, each with its own L2

struct PrefillWs {
  int* sync;       // [2 + S*nrb]  ticket, arrivals, carry progress per (segment, token block)
  uint16_t* wt;    // [cp, D_model] bf16  [W_dec | W_dn]^T, rows >= 3 H_kv + r zero
  uint16_t* qbf;   // [B*n, H_q, d] bf16  rotated queries
  float* gl;       // [B*n, H_kv, 2]      (lq, lb)
  uint16_t* uf;    // [B*n, 2, rp] bf16  u = x W_dn as a high part and a low part (u - high)
  float* carry;    // [nrb-1, total_slots] per-key carry into token block I (log2 units)
  unsigned long long* carry64;  // the same region as tagged words (call tag << 32 | carry bits)
  int* glob;       // control words: glob[kGlobSeq] counts the calls made with the workspace
  uint16_t* wut;   // [H_q*d, rp] bf16  W_up^T, ranks >= r zero
  int n, nrb, cp, rp;
  int ld, t0;      // token (b, t) of the call is row b * ld + t0 + t of q, k, v, x and y
  float tau2;      // attention mask threshold in log2 units (log p * log2 e), -inf for none
  const int* cu;   // variable-length call: [B + 1] packed row offsets (null: every sequence has n tokens)
  int total;       // variable-length call: rows of the packed q, k, v, x and y
};

// Tokens sequence b appends in this call (at most n).
__device__ __forceinline__ int seq_n(const PrefillWs& w, int b) {
  if (!w.cu) return w.n;
  return min(max(w.cu[b + 1] - w.cu[b], 0), w.n);
}

// The same for kernels instantiated per call kind: a fixed-length call keeps
// no offsets live (the attention kernels run at the edge of their registers).
template <bool VARLEN>
__device__ __forceinline__ int seq_n_k(const PrefillWs& w, int b) {
  if constexpr (VARLEN) return min(max(w.cu[b + 1] - w.cu[b], 0), w.n);
  else return w.n;
}

// Row of q/k/v/x/y that holds call token tk = b * n + t.  In a
// variable-length call, row cu[b] + t, clamped into the packed arrays (rows of
// tokens past the sequence's own count are read, never used, never written).
__device__ __forceinline__ int64_t io_row(const PrefillWs& w, int tk) {
  const int b = tk / w.n;
  if (w.cu) return min(max(w.cu[b] + (tk - b * w.n), 0), w.total - 1);
  return (int64_t)b * w.ld + w.t0 + (tk - b * w.n);
}

template <bool VARLEN>
__device__ __forceinline__ int64_t io_row_k(const PrefillWs& w, int tk) {
  const int b = tk / w.n;
  if constexpr (VARLEN) return min(max(w.cu[b] + (tk - b * w.n), 0), w.total - 1);
  else return (int64_t)b * w.ld + w.t0 + (tk - b * w.n);
}

static size_t prefill_layout(const LayerArgs& a, int n, char* base, PrefillWs* w) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int nrb = (n + kPRows - 1) / kPRows;
  const int cp = (3 * a.H_kv + a.r + 15) / 16 * 16;
  const int64_t NT = (int64_t)a.B * n;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes, 256);
    return p;
  };
  char* sync = take(sizeof(int) * (2 + S * nrb + kXcds));
  char* wt = take(sizeof(uint16_t) * (size_t)cp * a.D_model);
  char* qbf = take(sizeof(uint16_t) * (size_t)NT * a.H_q * a.d);
  char* gl = take(sizeof(float) * 2 * (size_t)NT * a.H_kv);
  const int rp = (a.r + 31) / 32 * 32;
  char* uf = take(sizeof(uint16_t) * 2 * (size_t)NT * rp);
  char* carry = take(sizeof(unsigned long long) * (size_t)(nrb - 1) * a.total_slots);
  char* wut = take(sizeof(uint16_t) * (size_t)a.H_q * a.d * rp);
  if (w) {
    w->sync = reinterpret_cast<int*>(sync);
    w->wt = reinterpret_cast<uint16_t*>(wt);
    w->qbf = reinterpret_cast<uint16_t*>(qbf);
    w->gl = reinterpret_cast<float*>(gl);
    w->uf = reinterpret_cast<uint16_t*>(uf);
    w->carry = reinterpret_cast<float*>(carry);
    w->carry64 = reinterpret_cast<unsigned long long*>(carry);
    w->wut = reinterpret_cast<uint16_t*>(wut);
    w->n = n;
    w->nrb = nrb;
    w->cp = cp;
    w->rp = rp;
  }
  return off;
}

size_t prefill_ws_bytes(const LayerArgs& a, int n_tokens, int /*max_seg_cap*/) {
  return prefill_layout(a, n_tokens, nullptr, nullptr);
}

__device__ __forceinline__ int ldi_coh_p(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sti_coh_p(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int addi_coh_p(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The (token block, segment) id of an attention workgroup, token-block major
// (id = I * S + s), taken from a ticket so that every wait is on a workgroup
// that started earlier.  Workgroups go to the XCDs in turn; when the segment
// count is a multiple of the XCD count, each XCD has its own queue serving the
// segments s = x mod kXcds, so the token blocks of a segment share one L2 and
// its K and V are fetched from below it once.  The grid is S * nrb, so every
// queue is drained.
__device__ __forceinline__ int prefill_ticket(const PrefillWs& w, int S, int nrb) {
  if (S % kXcds == 0) {
    const int x = (int)(blockIdx.x % kXcds), per = S / kXcds;
    const int t = addi_coh_p(&w.sync[2 + S * nrb + x], 1);
    return (t / per) * S + x + kXcds * (t % per);
  }
  return addi_coh_p(&w.sync[0], 1);
}

__device__ __forceinline__ unsigned long long ld64_coh_p(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64_coh_p(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ldf_coh_p(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stf_coh_p(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float u32x4_bf16(const u32x4& v, int e) {
  const uint32_t wd = v[e >> 1];
  return (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return pack2_bf16(lo, hi); }

// ---------------------------------------------------------------------------
// 1. prep: clear sync words, transpose the gate projections
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_prep_kernel(LayerArgs a, PrefillWs w, int nsync) {
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int gs = gridDim.x * blockDim.x;
  for (int i = gt; i < nsync; i += gs) w.sync[i] = 0;
  const int C3 = 3 * a.H_kv, nc = C3 + a.r, Dm = a.D_model;
  const int k8 = Dm / 8;
  const uint16_t* Wd = reinterpret_cast<const uint16_t*>(a.W_dec);
  const uint16_t* Wn = reinterpret_cast<const uint16_t*>(a.W_dn);
  for (int e = gt; e < w.cp * k8; e += gs) {
    const int c = e % w.cp;  // consecutive threads read consecutive columns
    const int kb = (e / w.cp) * 8;
    uint32_t pk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t lo = 0, hi = 0;
      const int64_t k0 = kb + 2 * t, k1 = k0 + 1;
      if (c < C3) {
        lo = Wd[k0 * C3 + c];
        hi = Wd[k1 * C3 + c];
      } else if (c < nc) {
        lo = Wn[k0 * a.r + c - C3];
        hi = Wn[k1 * a.r + c - C3];
      }
      pk[t] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(w.wt + (int64_t)c * Dm + kb) = u32x4{pk[0], pk[1], pk[2], pk[3]};
  }
  const int HqD = a.H_q * a.d;
  const uint16_t* Wu = reinterpret_cast<const uint16_t*>(a.W_up);
  for (int e = gt; e < HqD * (w.rp / 8); e += gs) {
    const int c = e % HqD;  // consecutive threads read consecutive columns
    const int r8 = (e / HqD) * 8;
    uint32_t pk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r0 = r8 + 2 * t, r1 = r0 + 1;
      const uint32_t lo = r0 < a.r ? Wu[(int64_t)r0 * HqD + c] : 0u;
      const uint32_t hi = r1 < a.r ? Wu[(int64_t)r1 * HqD + c] : 0u;
      pk[t] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(w.wut + (int64_t)c * w.rp + r8) = u32x4{pk[0], pk[1], pk[2], pk[3]};
  }
}

// ---------------------------------------------------------------------------
// 2. token kernel: gates, output gate, RoPE, append
// ---------------------------------------------------------------------------
constexpr int kTT = 512;  // token-kernel workgroup: 8 waves

template <int D>
__global__ __launch_bounds__(kTT) void prefill_token_kernel(LayerArgs a, PrefillWs w) {
  constexpr int HALF = D / 2;
  constexpr int CH = D / 8;  // 16-byte chunks per head row
  __shared__ float s_z[kPTok][kMaxZ];
  __shared__ float s_zp[kTT / 64][kPTok][48];  // the waves' partial z tiles of one three-tile group
    __shared__ float s_cos[kPTok][HALF];
  __shared__ float s_sin[kPTok][HALF];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int n = w.n;
  const int NT = a.B * n;
  const int tok0 = blockIdx.x * kPTok;
  const int Hkv = a.H_kv, Hq = a.H_q;
  const int C3 = 3 * Hkv;
  const int Dm = a.D_model;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* Kin = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* Vin = reinterpret_cast<const uint16_t*>(a.v);
  __shared__ int64_t s_dst[kPTok * kMaxHkv];  // (token, KV head) -> cache row of its append, -1: none

  // ---- every load that waits on no other phase, issued first so that their
  // round trips overlap the RoPE table and the projection: the first batch of
  // queries, the key row and segment words of item (token, KV head) = tid,
  // the first batch of values
  constexpr int QB = 4;  // query items per thread and batch
  constexpr int VB = 4;  // value items per thread and batch
  const int nitem = kPTok * Hq * (CH / 2);
  const int nkv = kPTok * Hkv;
  const int nv = nkv * CH;
  u32x4 qlo[QB], qhi[QB];
  auto load_q = [&](int e0) {
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      const int e = min(e0 + u * kTT + tid, nitem - 1);
      const int c = e % (CH / 2);
      const int rest = e / (CH / 2);
      const int hd = rest % Hq, tt = rest / Hq;
      const int tkc = min(tok0 + tt, NT - 1);
      const int64_t qin = (io_row(w, tkc) * Hq + hd) * D + 8 * c;
      qlo[u] = *reinterpret_cast<const u32x4*>(Q + qin);
      qhi[u] = *reinterpret_cast<const u32x4*>(Q + qin + HALF);
    }
  };
  load_q(0);
  constexpr bool kRowsEarly = D == 64;  // at head dim 128 the rows would not fit beside the projection
  u32x4 kraw[CH];
  int kl0 = 0, kcap = 0, knq = 0;
  int64_t koff = 0;
  auto load_key_rows = [&](int e) {
    const int tt = e / Hkv, h = e - tt * Hkv;
    const int64_t base = (io_row(w, min(tok0 + tt, NT - 1)) * Hkv + h) * D;
#pragma unroll
    for (int c = 0; c < CH; ++c) kraw[c] = *reinterpret_cast<const u32x4*>(Kin + base + 8 * c);
  };
  auto load_key = [&](int e) {
    const int tt = e / Hkv, h = e - tt * Hkv;
    const int tkc = min(tok0 + tt, NT - 1);
    const int b = tkc / n, s = b * Hkv + h;
    kl0 = a.seg_len[s];
    kcap = a.seg_cap[s];
    koff = a.seg_off[s];
    knq = seq_n(w, b);
    if constexpr (kRowsEarly) load_key_rows(e);
  };
  if (tid < nkv) load_key(tid);
  u32x4 vv[VB];
  auto load_v = [&](int e0) {
#pragma unroll
    for (int u = 0; u < VB; ++u) {
      const int e = min(e0 + u * kTT + tid, nv - 1);
      const int c = e % CH, rest = e / CH;
      const int h = rest % Hkv, tt = rest / Hkv;
      vv[u] = *reinterpret_cast<const u32x4*>(Vin + (io_row(w, min(tok0 + tt, NT - 1)) * Hkv + h) * D + 8 * c);
    }
  };
  load_v(0);

  for (int i = tid; i < kPTok * kMaxZ; i += kTT) (&s_z[0][0])[i] = 0.0f;
  for (int e = tid; e < kPTok * HALF; e += kTT) {
    const int tt = e / HALF, i = e - tt * HALF;
    const int tk = min(tok0 + tt, NT - 1);
    const int b = tk / n, t = tk - b * n;
    double sn, cn;
    sincos((double)(a.next_pos[b] + t) * a.inv_freq[i], &sn, &cn);
    s_cos[tt][i] = (float)cn;
    s_sin[tt][i] = (float)sn;
  }
  __syncthreads();

  // ---- z = x [W_dec | W_dn]: A = x rows (tokens), B = W^T rows.  For each
  // group of three 16-column tiles, each wave takes chunks of 8 k steps (256
  // columns of x), loading the weight fragments with the chunk's x; the waves'
  // partial tiles meet in LDS and are summed in a fixed order (LDS float
  // atomics from eight waves on the same entries cost a third of the kernel).
  {
    constexpr int KCH = 8;
    constexpr int NW = kTT / 64;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
    const int nks = (Dm + 31) / 32;
    const int ntile = w.cp / 16;
    const int64_t xrow = io_row(w, min(tok0 + c16, NT - 1)) * Dm;
    const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
    for (int nt0 = 0; nt0 < ntile; nt0 += 3) {  // the same count in every wave: the barriers below match
      f32x4 acc[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int k0 = wv * KCH; k0 < nks; k0 += NW * KCH) {
        u32x4 av[KCH], bv[3][KCH];
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
          const int kk = 32 * (k0 + u) + 8 * g;
          const int kc = kk < Dm ? kk : 0;
          av[u] = *reinterpret_cast<const u32x4*>(X + xrow + kc);
#pragma unroll
          for (int q = 0; q < 3; ++q)
            bv[q][u] = *reinterpret_cast<const u32x4*>(w.wt + (int64_t)(16 * min(nt0 + q, ntile - 1) + c16) * Dm + kc);
        }
#pragma unroll
        for (int u = 0; u < KCH; ++u)
          if (32 * (k0 + u) + 8 * g >= Dm) av[u] = zero4;  // past the end of x (Dm is a multiple of 8)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int u = 0; u < KCH; ++u) acc[q] = mfma_bf16(av[u], bv[q][u], acc[q]);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_zp[wv][4 * g + i][16 * q + c16] = acc[q][i];
      __syncthreads();
      for (int e = tid; e < kPTok * 48; e += kTT) {
        const int row = e / 48, col = e - row * 48;
        if (16 * nt0 + col < w.cp) {
          float sum = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) sum += s_zp[w2][row][col];
          s_z[row][16 * nt0 + col] = sum;
        }
      }
      __syncthreads();
    }
  }

  // ---- gates and the append of the key gate; the cache row of every
  // (token, KV head) append goes to LDS for the value append
  for (int e = tid; e < nkv; e += kTT) {
    if (e != tid) load_key(e);  // more items than threads (H_kv > kTT / kPTok)
    const int tt = e / Hkv, h = e - tt * Hkv;
    const int tk = tok0 + tt;
    int64_t dst = -1;
    if (tk < NT) {
      const int b = tk / n, t = tk - b * n;
      const float lq = log_sigmoid(s_z[tt][h] + a.b_dec[h]);
      const float lkk = log_sigmoid(s_z[tt][Hkv + h] + a.b_dec[Hkv + h]);
      const float lb = log_sigmoid(s_z[tt][2 * Hkv + h] + a.b_dec[2 * Hkv + h]);
      w.gl[2 * ((int64_t)tk * Hkv + h) + 0] = lq;
      w.gl[2 * ((int64_t)tk * Hkv + h) + 1] = lb;
      if ((int64_t)kl0 + knq <= kcap) {
        if (t < knq) {
          dst = koff + kl0 + t;
          a.lk[dst] = lkk;
        }
      } else if (t == 0) {
        atomicOr(a.status, 1);
      }
    }
    s_dst[e] = dst;
  }
  if (nkv > kTT && tid < nkv) load_key(tid);  // the loop above moved on to later items
  __syncthreads();  // s_dst complete before the value append reads other items' rows

  // ---- rotated queries (bf16 copy); chunk c pairs dims [8c, 8c+8) with
  // [HALF+8c, HALF+8c+8).  Items go in batches of QB per thread with every
  // load of a batch issued before any is used.
  {
    for (int e0 = 0; e0 < nitem; e0 += kTT * QB) {
      if (e0 > 0) load_q(e0);  // the first batch was loaded at the start
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int e = e0 + u * kTT + tid;
        const int c = e % (CH / 2);
        const int rest = e / (CH / 2);
        const int hd = rest % Hq, tt = rest / Hq;
        if (e >= nitem || tok0 + tt >= NT) continue;
        const int64_t qbase = ((int64_t)(tok0 + tt) * Hq + hd) * D + 8 * c;
        uint32_t olo[4], ohi[4];
#pragma unroll
        for (int v = 0; v < 8; v += 2) {
          float rl[2], rh[2];
#pragma unroll
          for (int v2 = 0; v2 < 2; ++v2) {
            const int i = 8 * c + v + v2;
            const float xl = u32x4_bf16(qlo[u], v + v2), xh = u32x4_bf16(qhi[u], v + v2);
            rl[v2] = fmaf(xl, s_cos[tt][i], -xh * s_sin[tt][i]);
            rh[v2] = fmaf(xh, s_cos[tt][i], xl * s_sin[tt][i]);
          }
          olo[v / 2] = pack_bf16(rl[0], rl[1]);
          ohi[v / 2] = pack_bf16(rh[0], rh[1]);
        }
        *reinterpret_cast<u32x4*>(w.qbf + qbase) = u32x4{olo[0], olo[1], olo[2], olo[3]};
        *reinterpret_cast<u32x4*>(w.qbf + qbase + HALF) = u32x4{ohi[0], ohi[1], ohi[2], ohi[3]};
      }
    }
  }

  // ---- keys: normalise, rotate, round, append; values: append
  {
    uint16_t* Kc = reinterpret_cast<uint16_t*>(a.K);
    uint16_t* Vc = reinterpret_cast<uint16_t*>(a.V);
    for (int e = tid; e < nkv; e += kTT) {
      if (e != tid || !kRowsEarly) load_key_rows(e);  // at head dim 64 the first item's row came early
      const int tt = e / Hkv;
      const int64_t dst = s_dst[e];
      if (dst < 0) continue;
      const u32x4* raw = kraw;
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float xv = u32x4_bf16(raw[c], u);
          ss = fmaf(xv, xv, ss);
        }
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
      const int64_t kd = dst * D;
#pragma unroll
      for (int c = 0; c < CH / 2; ++c) {
        uint32_t olo[4], ohi[4];
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          float rl[2], rh[2];
#pragma unroll
          for (int v2 = 0; v2 < 2; ++v2) {
            const int i = 8 * c + u + v2;
            const float kl = u32x4_bf16(raw[c], u + v2) * inv;
            const float kh = u32x4_bf16(raw[c + CH / 2], u + v2) * inv;
            rl[v2] = fmaf(kl, s_cos[tt][i], -kh * s_sin[tt][i]);
            rh[v2] = fmaf(kh, s_cos[tt][i], kl * s_sin[tt][i]);
          }
          olo[u / 2] = pack_bf16(rl[0], rl[1]);
          ohi[u / 2] = pack_bf16(rh[0], rh[1]);
        }
        *reinterpret_cast<u32x4*>(Kc + kd + 8 * c) = u32x4{olo[0], olo[1], olo[2], olo[3]};
        *reinterpret_cast<u32x4*>(Kc + kd + HALF + 8 * c) = u32x4{ohi[0], ohi[1], ohi[2], ohi[3]};
      }
    }
    for (int e0 = 0; e0 < nv; e0 += kTT * VB) {
      if (e0 > 0) load_v(e0);  // the first batch was loaded at the start
#pragma unroll
      for (int u = 0; u < VB; ++u) {
        const int e = e0 + u * kTT + tid;
        if (e >= nv) continue;
        const int c = e % CH;
        const int64_t dst = s_dst[e / CH];  // item (token, KV head) = e / CH
        if (dst < 0) continue;
        *reinterpret_cast<u32x4*>(Vc + dst * D + 8 * c) = vv[u];
      }
    }
  }

  // ---- u = x W_dn for the output gate, as a bf16 high part and a bf16 low
  // part (u - high), stored in the k layout of a matrix-core operand: the
  // attention epilogue forms sigmoid(u W_up + b_up) for its own tokens
  if (wv == 0) {
    const int tk = tok0 + c16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks >= w.rp) break;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x2[2], h2[2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int rr = 32 * ks + 8 * g + 2 * v + z;
          x2[z] = rr < a.r ? s_z[c16][C3 + rr] : 0.0f;
        }
        ph[v] = pack2_bf16(x2[0], x2[1]);
        h2[0] = bf16_lo(ph[v]);
        h2[1] = bf16_hi(ph[v]);
        pl[v] = pack2_bf16(x2[0] - h2[0], x2[1] - h2[1]);
      }
      if (tk < NT) {
        uint16_t* ut = w.uf + (int64_t)tk * 2 * w.rp + 32 * ks + 8 * g;
        *reinterpret_cast<u32x4*>(ut) = u32x4{ph[0], ph[1], ph[2], ph[3]};
        *reinterpret_cast<u32x4*>(ut + w.rp) = u32x4{pl[0], pl[1], pl[2], pl[3]};
      }
    }
  }
}

// Output gate sigmoid(u W_up + b_up) of call token `tok` (this lane's column
// c16 of a 16-token tile) at output columns col0 + 4 g + i: rows of W_up^T
// are the A operand and the token's u parts the B operand, so the result has
// the lane layout of the O^T tiles it scales.  All 64 lanes must be active.
__device__ __forceinline__ f32x4 out_gate(const LayerArgs& a, const PrefillWs& w, int64_t tok, int col0, int g,
                                          int c16) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* ut = w.uf + tok * 2 * w.rp;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (32 * ks >= w.rp) break;
    const u32x4 wa = *reinterpret_cast<const u32x4*>(w.wut + (int64_t)(col0 + c16) * w.rp + 32 * ks + 8 * g);
    const u32x4 uh = *reinterpret_cast<const u32x4*>(ut + 32 * ks + 8 * g);
    const u32x4 ul = *reinterpret_cast<const u32x4*>(ut + w.rp + 32 * ks + 8 * g);
    acc = mfma_bf16(wa, uh, acc);
    acc = mfma_bf16(wa, ul, acc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = sigmoid_fast(acc[i] + (a.b_up ? a.b_up[col0 + 4 * g + i] : 0.0f));
  return acc;
}

// 3. attention with the causal decay bias
// ---------------------------------------------------------------------------
// Position of key k (0..63) of a block in the LDS copy of V^T: the P V product
// takes its k index from the score tiles, where lane group q of 16 lanes holds
// keys 4q..4q+3 of each 16-key tile; MFMA k index 8q + i of 32-key chunk c
// maps to key 32c + 4q + i (i < 4) and 32c + 16 + 4q + (i - 4) (i >= 4).
__device__ __forceinline__ int vt_pos(int k) {
  const int r = k & 31;
  return (k & 32) | (((r >> 2) & 3) << 3) | ((r >> 4) << 2) | (r & 3);
}

// End of an attention workgroup: after every workgroup has counted itself
// in, the last one advances lengths and positions (and with SEQ publishes the
// call's number, which tags the carry words).
template <bool VARLEN, int NT, bool SEQ>
__device__ __forceinline__ void prefill_commit(const LayerArgs& a, const PrefillWs& w, int* s_last, uint32_t seq) {
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) *s_last = (addi_coh_p(&w.sync[1], 1) == (int)gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (*s_last) {
    if (SEQ && tid == 0) sti_coh_p(&w.glob[kGlobSeq], (int)seq);
    const int S = a.B * a.H_kv;
    for (int s2 = tid; s2 < S; s2 += NT) {
      const int l = a.seg_len[s2], nq = seq_n_k<VARLEN>(w, s2 / a.H_kv);
      if ((int64_t)l + nq <= a.seg_cap[s2]) a.seg_len[s2] = l + nq;
    }
    for (int b2 = tid; b2 < a.B; b2 += NT) a.next_pos[b2] += seq_n_k<VARLEN>(w, b2);
  }
}

template <int D, int HG, bool VARLEN>
__global__ __launch_bounds__(kPThreads) void prefill_attn_kernel(LayerArgs a, PrefillWs w) {
  constexpr int KC = D / 32;                          // k steps of a head-dim dot product
  constexpr int DT = D / 16;                          // 16-wide output tiles per head
  constexpr int KS = D + 8;                           // s_k row stride (bf16)
  constexpr int VS = kPKeys + 8;                      // s_vt row stride (fp16)
  constexpr int KPT = kPKeys * (D / 8) / kPThreads;   // K pieces per thread per block
  constexpr int VITEMS = (kPKeys / 2) * (D / 4);      // V (key pair, 4 dims) items per block
  constexpr int VPT = VITEMS / kPThreads;
  static_assert(VITEMS % kPThreads == 0, "V items per thread");
  constexpr int XS = DT * 4 + 2;                      // floats per lane in the final merge
  constexpr int QS = HG * D + 8;                      // s_q row stride (bf16): rows shift by 16 bytes
  static_assert(KPT >= 1, "tile split");
  static_assert(4 * 64 * XS * 4 <= (int)sizeof(uint16_t) * 2 * kPKeys * KS, "merge buffer fits in s_k");
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kPKeys * KS];
  __shared__ __attribute__((aligned(16))) _Float16 s_vt[2][D * VS];
  __shared__ __attribute__((aligned(16))) float s_lk[2][kPKeys];
  __shared__ __attribute__((aligned(16))) float s_tot[2][4][kPKeys];
  __shared__ __attribute__((aligned(16))) float s_car[2][kPKeys];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kPRows * QS];  // rotated queries of the token block
  __shared__ int s_id;

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so branches on it stay scalar
  const int tw = wv & 3;   // token quarter: tokens 16 tw .. 16 tw + 15 of the block
  const int hp = wv >> 2;  // key half: keys 32 hp .. 32 hp + 31 of every key block
  const int S = a.B * a.H_kv;
  const int n = w.n, nrb = w.nrb;
  const int Hq = a.H_q, Hkv = a.H_kv;

  if (tid == 0) s_id = prefill_ticket(w, S, nrb);
  __syncthreads();
  const int id = s_id;
  // token-block major: a chain predecessor always holds an earlier ticket of
  // the same queue, so it is already running
  const int s = id % S;
  const int I = id / S;
  const int b = s / Hkv, h = s - b * Hkv;
  const int len0 = a.seg_len[s];
  const int64_t off = a.seg_off[s];
  const int nseq = seq_n_k<VARLEN>(w, b);         // this sequence's tokens
  const int nrbs = (nseq + kPRows - 1) / kPRows;  // and its token blocks
  if constexpr (VARLEN) {
    if (I >= nrbs) {  // past the sequence's tokens: no work, and no chain waits on this block
      prefill_commit<VARLEN, kPThreads, false>(a, w, &s_id, 0u);
      return;
    }
  }
  const bool room = (int64_t)len0 + nseq <= a.seg_cap[s];
  const int row_lo = I * kPRows + tw * 16;  // first token of this wave
  const int tq = row_lo + c16;              // this lane's token (score column)
  const bool row_ok = tq < nseq;
  const int tqc = min(tq, max(nseq, 1) - 1);
  const int64_t tok = (int64_t)b * n + tqc;
  const int64_t ytok = io_row_k<VARLEN>(w, (int)tok);  // the token's row of y
  const int a0 = h * HG;

  if (room) {
    const int nkeys = len0 + nseq;
    const int kend = len0 + min(nseq, I * kPRows + kPRows);
    const int nJ = (kend + kPKeys - 1) / kPKeys;
    const int64_t TS = a.total_slots;
    const PairCoef pc = pair_coef(a.terms);
    const float cs = a.scale * kLog2e;
    const uint16_t* Kc = reinterpret_cast<const uint16_t*>(a.K);
    const uint16_t* Vc = reinterpret_cast<const uint16_t*>(a.V);

    // token-side constants
    const float lq = w.gl[2 * (tok * Hkv + h) + 0];
    const float lb = w.gl[2 * (tok * Hkv + h) + 1];
    const float row2 = pc.inv_n2 * (((a.terms & 1) ? lq : 0.0f) + ((a.terms & 4) ? lb : 0.0f));
    // the block's rotated queries to LDS: [token][head][dim], rows of tokens past n clamped
    for (int q = tid; q < kPRows * HG * (D / 8); q += kPThreads) {
      const int tt = q / (HG * (D / 8)), rest = q - tt * (HG * (D / 8));
      const int64_t tk = (int64_t)b * n + min(I * kPRows + tt, nseq - 1);
      *reinterpret_cast<u32x4*>(&s_q[tt * QS + rest * 8]) =
          *reinterpret_cast<const u32x4*>(w.qbf + (tk * Hq + a0) * D + rest * 8);
    }
    const uint16_t* qrow = &s_q[(tw * 16 + c16) * QS + 8 * g];  // this lane's token, k offset 8 g
    u32x4 krf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      krf[kc] = *reinterpret_cast<const u32x4*>(Kc + (off + len0 + tqc) * D + 32 * kc + 8 * g);

    // staging of a key block: K rows, V rows (as key pairs), key gates
    // staging registers of the next block (kst, ...) and of the one after (kst2, ...)
    u32x4 kst[KPT], kst2[KPT];
    uint2 vst[VPT][2], vst2[VPT][2];
    float lkst = 0.0f, lkst2 = 0.0f;
    auto slot = [&](int j) -> int64_t { return off + min(j, nkeys - 1); };
    auto load_block = [&](int J, u32x4 (&kst)[KPT], uint2 (&vst)[VPT][2], float& lkst) {
      const int j0 = J * kPKeys;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int q = tid + kPThreads * u, key = q / (D / 8), part = q % (D / 8);
        kst[u] = *reinterpret_cast<const u32x4*>(Kc + slot(j0 + key) * D + 8 * part);
      }
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int q = tid + kPThreads * u, p = q / (D / 4), part = q % (D / 4);
        vst[u][0] = *reinterpret_cast<const uint2*>(Vc + slot(j0 + 2 * p) * D + 4 * part);
        vst[u][1] = *reinterpret_cast<const uint2*>(Vc + slot(j0 + 2 * p + 1) * D + 4 * part);
      }
      lkst = a.lk[slot(j0 + lane)];
    };
    const float col_scale = (a.terms & 2) ? pc.inv_n2 : 0.0f;  // key-side part of the pair term
    auto store_k = [&](int buf) {
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int q = tid + kPThreads * u, key = q / (D / 8), part = q % (D / 8);
        *reinterpret_cast<u32x4*>(&s_k[buf][key * KS + 8 * part]) = kst[u];
      }
      if (wv == 0) s_lk[buf][lane] = lkst * col_scale;
    };
    auto store_v = [&](int buf) {
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int q = tid + kPThreads * u, p = q / (D / 4), part = q % (D / 4);
        const int pos = vt_pos(2 * p);
        const uint32_t k0w[2] = {vst[u][0].x, vst[u][0].y}, k1w[2] = {vst[u][1].x, vst[u][1].y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = (e & 1) ? bf16_hi(k0w[e >> 1]) : bf16_lo(k0w[e >> 1]);
          const float v1 = (e & 1) ? bf16_hi(k1w[e >> 1]) : bf16_lo(k1w[e >> 1]);
          const auto hv = __builtin_amdgcn_cvt_pkrtz(v0, v1);
          *reinterpret_cast<uint32_t*>(&s_vt[buf][(4 * part + e) * VS + pos]) = __builtin_bit_cast(uint32_t, hv);
        }
      }
    };

    load_block(0, kst, vst, lkst);
    store_k(0);
    store_v(0);
    if (nJ > 1) load_block(1, kst, vst, lkst);
    __syncthreads();

    // Online softmax per (query head, token) over this wave's key halves.  P is
    // taken relative to m_run (log2 units), which is only raised when a block
    // exceeds it by more than 2^kRescaleTh, and set at the first block where
    // the token has a valid key in this half (mset).
    float m_run[HG];
    int mset = 0;  // bit hh: the reference of head hh is set
    f32x4 O[HG][DT], Lt[HG];
    const float inv_cs = 1.0f / cs;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      m_run[hh] = 0.0f;
      Lt[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[hh][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // Carry into this token block for the next key block, fetched one iteration
    // ahead (wave 0, lane = key): the stored bias for the token block that
    // starts the key block's chain, else the previous token block's published
    // carry if it is already there.  Raw values; scaled where used.
    float car_cur = 0.0f, car_nxt = 0.0f;
    bool have_cur = false, have_nxt = false, init_cur = false, init_nxt = false;
    f16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (c16 == 0) ? (_Float16)1.0f : (_Float16)0.0f;

    for (int J = 0; J < nJ; ++J) {
      const int cb = J & 1, nb = cb ^ 1;
      const int j0 = J * kPKeys;
      const bool more = J + 1 < nJ;
      if (J + 2 < nJ) load_block(J + 2, kst2, vst2, lkst2);
      const int Ist_next = (j0 + kPKeys >= len0) ? (j0 + kPKeys - len0) / kPRows : 0;
      const bool chain_next = more && I > Ist_next;
      int flag_next = 0;
      have_nxt = false;
      init_nxt = false;
      if (wv == 0 && more) {
        if (!chain_next) {
          car_nxt = a.lam[off + min(j0 + kPKeys + lane, nkeys - 1)];
          have_nxt = init_nxt = true;
        } else {
          flag_next = ldi_coh_p(&w.sync[2 + s * nrb + I - 1]);  // used after the barrier
        }
      }

      // this wave's key fragments: 16-key tiles kt = 2 hp, 2 hp + 1
      u32x4 kf[2][KC];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          kf[t][kc] =
              *reinterpret_cast<const u32x4*>(&s_k[cb][(32 * hp + 16 * t + c16) * KS + 32 * kc + 8 * g]);
      // some element of this wave's tile is masked (causal edge or tokens past n)
      const bool edge = (j0 + 32 * hp + 31 >= len0 + row_lo) || (row_lo + 15 >= nseq);

      // ---- pair terms, scanned over this wave's 16 tokens.  The enabled terms
      // and the causal edge are uniform per block, so each combination is a
      // branch-free variant and the eight pairs of a lane interleave.
      float lam[2][4];
      auto pair_terms = [&](auto edge_c, auto sim_c) {
        constexpr bool EDGE = decltype(edge_c)::value, SIM = decltype(sim_c)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 sim = {0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (SIM) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) sim = mfma_bf16(kf[t][kc], krf[kc], sim);
          }
          const float4 lk4 = *reinterpret_cast<const float4*>(&s_lk[cb][32 * hp + 16 * t + 4 * g]);
          const float lkv[4] = {lk4.x, lk4.y, lk4.z, lk4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float lam2 = row2 + lkv[i];
            if constexpr (SIM) lam2 = fmaf(pc.sim_w, __builtin_amdgcn_logf(fminf(sim[i] * sim[i], 1.0f)), lam2);
            float A2 = log1mexp2_b2(lam2);
            if constexpr (EDGE) {
              const int jg = j0 + 32 * hp + 16 * t + 4 * g + i;
              A2 = (row_ok && jg < len0 + tq) ? A2 : 0.0f;
            }
            lam[t][i] = A2;
          }
        }
      };
      if (!pc.any) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) lam[t][i] = 0.0f;
      } else if (edge) {
        if (pc.sim) pair_terms(std::true_type{}, std::true_type{});
        else pair_terms(std::true_type{}, std::false_type{});
      } else {
        if (pc.sim) pair_terms(std::false_type{}, std::true_type{});
        else pair_terms(std::false_type{}, std::false_type{});
      }
      // inclusive scans over the 16 lanes of each row, step-major so the eight
      // independent scans fill each other's DPP hazard slots
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[t][i] += dpp_f<0x111>(lam[t][i]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[t][i] += dpp_f<0x112>(lam[t][i]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[t][i] += dpp_f<0x114>(lam[t][i]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[t][i] += dpp_f<0x118>(lam[t][i]);
      if (c16 == 15) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<float4*>(&s_tot[cb][tw][32 * hp + 16 * t + 4 * g]) =
              make_float4(lam[t][0], lam[t][1], lam[t][2], lam[t][3]);
      }
      // ---- carry into this token block for the block's keys
      if (wv == 0) {
        const int jg = j0 + lane;
        const int Ist = j0 >= len0 ? (j0 - len0) / kPRows : 0;  // first token block that sees key block J
        float v;
        if (have_cur) {
          v = init_cur ? ((jg < len0) ? car_cur * kLog2e : 0.0f) : car_cur;
        } else if (I == Ist) {
          v = (jg < len0) ? a.lam[off + jg] * kLog2e : 0.0f;
        } else {
          const int* flag = &w.sync[2 + s * nrb + I - 1];
          int spins = 0;
          while (ldi_coh_p(flag) < J + 1) {
            if (++spins > kPrefillSpinLimit) {
              if (lane == 0) atomicOr(a.status, 2);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          v = ldf_coh_p(&w.carry[(int64_t)(I - 1) * TS + off + min(jg, nkeys - 1)]);
        }
        s_car[cb][lane] = v;
      }
      if (more) store_k(nb);
      __syncthreads();
      // wave 0: fetch the next block's carry now if its producer has published it
      if (wv == 0 && chain_next && flag_next >= J + 2) {
        car_nxt = ldf_coh_p(&w.carry[(int64_t)(I - 1) * TS + off + min(j0 + kPKeys + lane, nkeys - 1)]);
        have_nxt = true;
      }

      // ---- bias of this wave's elements (log2 units)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k4 = 32 * hp + 16 * t + 4 * g;
        float4 pre = *reinterpret_cast<const float4*>(&s_car[cb][k4]);
        for (int w2 = 0; w2 < tw; ++w2) {
          const float4 t4 = *reinterpret_cast<const float4*>(&s_tot[cb][w2][k4]);
          pre.x += t4.x;
          pre.y += t4.y;
          pre.z += t4.z;
          pre.w += t4.w;
        }
        lam[t][0] += pre.x;
        lam[t][1] += pre.y;
        lam[t][2] += pre.z;
        lam[t][3] += pre.w;
      }
      if (w.tau2 > kNegInf) {  // pruned call: entries below the threshold are not attended
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) lam[t][i] = (lam[t][i] >= w.tau2) ? lam[t][i] : kNegInf;
      }
      // ---- carry out to the next token block, or the final bias of the call
      if (wv == 4) {
        const int jg = j0 + lane;
        const float cn =
            s_car[cb][lane] + s_tot[cb][0][lane] + s_tot[cb][1][lane] + s_tot[cb][2][lane] + s_tot[cb][3][lane];
        if (I + 1 < nrbs) {
          if (jg < nkeys) stf_coh_p(&w.carry[(int64_t)I * TS + off + jg], cn);
          __builtin_amdgcn_s_waitcnt(0);
          if (lane == 0) sti_coh_p(&w.sync[2 + s * nrb + I], J + 1);
        } else if (jg < nkeys) {
          a.lam[off + jg] = cn * kLn2;
        }
      }

      // ---- softmax and P V per query head over this wave's 32 keys
      f16x8 vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        vf[dt] = *reinterpret_cast<const f16x8*>(&s_vt[cb][(16 * dt + c16) * VS + 32 * hp + 8 * g]);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float e[2][4];
        float bm = kNegInf;
        u32x4 qf[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qf[kc] = *reinterpret_cast<const u32x4*>(qrow + hh * D + 32 * kc);
        const float ci = -m_run[hh] * inv_cs;  // the reference folded into the accumulator's start
        auto logits = [&](auto edge_c) {
          constexpr bool EDGE = decltype(edge_c)::value;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            f32x4 sc = f32x4{ci, ci, ci, ci};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) sc = mfma_bf16(kf[t][kc], qf[kc], sc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float ev = fmaf(sc[i], cs, lam[t][i]);
              if constexpr (EDGE) {
                const int jg = j0 + 32 * hp + 16 * t + 4 * g + i;
                ev = (row_ok && jg <= len0 + tq) ? ev : kNegInf;
              }
              e[t][i] = ev;
              bm = fmaxf(bm, ev);
            }
          }
        };
        if (edge) logits(std::true_type{});
        else logits(std::false_type{});
        const bool fresh = ((mset >> hh) & 1) == 0;
        if (__any(bm > kRescaleTh || (fresh && bm > kNegInf))) {
          float bx = fmaxf(bm, __shfl_xor(bm, 16, 64));
          bx = fmaxf(bx, __shfl_xor(bx, 32, 64));
          const float dl = fresh ? ((bx > kNegInf) ? bx : 0.0f) : fmaxf(bx, 0.0f);
          const float al = fresh ? 1.0f : __builtin_amdgcn_exp2f(-dl);  // nothing accumulated yet when fresh
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) O[hh][dt] *= al;
          Lt[hh] *= al;
          m_run[hh] += dl;
          if (bx > kNegInf) mset |= 1 << hh;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) e[t][i] -= dl;
        }
        // B operand of P V: k index 8q + i holds key 32 hp + 4q + i (i < 4) and 32 hp + 16 + 4q + i - 4
        f16x8 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[i] = (_Float16)__builtin_amdgcn_exp2f(e[0][i]);
          pk[4 + i] = (_Float16)__builtin_amdgcn_exp2f(e[1][i]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[hh][dt] = mfma_f16(vf[dt], pk, O[hh][dt]);
        Lt[hh] = mfma_f16(ones, pk, Lt[hh]);
      }
      if (more) store_v(nb);
#pragma unroll
      for (int u = 0; u < KPT; ++u) kst[u] = kst2[u];
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        vst[u][0] = vst2[u][0];
        vst[u][1] = vst2[u][1];
      }
      lkst = lkst2;
      car_cur = car_nxt;
      have_cur = have_nxt;
      init_cur = init_nxt;
    }

    // ---- epilogue: merge the two key halves of each token (through the K
    // staging buffer, now free), normalise, gate, store.  O^T tiles: a lane
    // holds dims 16 dt + 4 g + i of token c16.
    float* xch = reinterpret_cast<float*>(&s_k[0][0]) + (tw * 64 + lane) * XS;
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const float L = __shfl(Lt[hh][0], c16, 64);
      const float mw = (L > 0.0f) ? m_run[hh] : kNegInf;
      if (hp == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xch[4 * dt + i] = O[hh][dt][i];
        xch[4 * DT] = L;
        xch[4 * DT + 1] = mw;
      }
      __syncthreads();
      if (hp == 0) {
        const float L1 = xch[4 * DT], m1 = xch[4 * DT + 1];
        const float m = fmaxf(mw, m1);
        const float s0 = (mw > kNegInf) ? __builtin_amdgcn_exp2f(mw - m) : 0.0f;
        const float s1 = (m1 > kNegInf) ? __builtin_amdgcn_exp2f(m1 - m) : 0.0f;
        const float Ls = L * s0 + L1 * s1;
        const float inv = (row_ok && Ls > 0.0f) ? 1.0f / Ls : 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int64_t yo = (ytok * Hq + a0 + hh) * D + 16 * dt + 4 * g;
          const f32x4 gm = out_gate(a, w, tok, (a0 + hh) * D + 16 * dt, g, c16);
          float yv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) yv[i] = (O[hh][dt][i] * s0 + xch[4 * dt + i] * s1) * inv;
          const float y0 = gm[0] * yv[0], y1 = gm[1] * yv[1], y2 = gm[2] * yv[2], y3 = gm[3] * yv[3];
          if (row_ok) {
            if (a.y_bf16) {
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + yo) =
                  make_uint2(pack_bf16(y0, y1), pack_bf16(y2, y3));
            } else {
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + yo) = make_float4(y0, y1, y2, y3);
            }
          }
          __builtin_amdgcn_sched_barrier(0);  // one gate tile's operands live at a time
        }
      }
      __syncthreads();
    }
  } else if (row_ok && hp == 0) {
    // the segment has no room for the call: its outputs are zero
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int64_t yo = (ytok * Hq + a0 + hh) * D + 16 * dt + 4 * g;
        if (a.y_bf16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + yo) = make_uint2(0u, 0u);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + yo) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
  }

  prefill_commit<VARLEN, kPThreads, false>(a, w, &s_id, 0u);
}

// ---------------------------------------------------------------------------
// 3b. attention for head dim 64 and up to four query heads per KV head, with
// the waves split by role.  Waves 0-3 form the bias of the next key block, 16
// keys each over all 64 tokens of the token block: K K^T on the matrix cores,
// the pair terms, the scan over tokens (DPP within a 16-token tile, a
// broadcast of the tile total across tiles) and the carry across token blocks.  Waves 4-7 run the softmax and P V of the
// current key block for 16 tokens each and stage the key blocks ahead into
// LDS.  A SIMD holds one wave of each role, so the transcendental-heavy bias
// work and the matrix-core-heavy softmax of the two blocks overlap; one
// barrier per key block.
//
// Softmax reference.  Stored keys are unit vectors and the bias is never
// positive, so cs |q~| bounds every logit of a (token, head) from above and
// serves as a fixed reference: P = 2^(logit - cs |q~|) <= 1, with no running
// maximum.  The token's own key has zero bias, so the largest P is at least
// 2^(-2 cs |q~|); a wave whose queries have cs |q~| above kStaticRef takes the
// running-maximum path instead, so P never leaves the fp16 normal range.
//
// Carry words.  A carry crosses token blocks as one 64-bit word, the call's
// tag in the high half and the value's bits in the low half, written with one
// store and no progress word.  The next token block loads the words of a key
// block before its pair terms and checks the tags after them, reloading only
// the words still stale.  The tag is a signalling-NaN pattern holding the
// call counter (glob[kGlobSeq], which every prefill call advances); arithmetic
// never produces it, so no stale word of the workspace carries it.
// ---------------------------------------------------------------------------
constexpr float kStaticRef = 6.0f;
constexpr int kDppBcast15 = 0x15F;  // row_newbcast:15, lane 15 of each row to the whole row

constexpr int kPThreadsWS = 768;  // 4 bias waves + 8 softmax waves

__device__ __forceinline__ uint32_t carry_tag(uint32_t seq) {
  return 0x7F800000u | ((seq - 1u) % 0x3FFFFFu + 1u);  // exponent all ones, quiet bit clear, payload != 0
}

template <int HG, bool MASKED, bool VARLEN>
__global__ __launch_bounds__(kPThreadsWS) void prefill_attn_ws_kernel(LayerArgs a, PrefillWs w) {
  constexpr int D = 64;
  constexpr int KC = D / 32;                // k steps of a head-dim dot product
  constexpr int DT = D / 16;                // 16-wide output tiles per head
  constexpr int KS = D + 8;                 // s_k row stride (bf16)
  constexpr int VS = kPKeys + 8;            // s_vt row stride (fp16)
  constexpr int QS = HG * D + 8;            // s_q row stride (bf16)
  constexpr int HH = (HG + 1) / 2;          // query heads of the first softmax wave of a token tile
  constexpr int NC = kPThreadsWS - 256;     // staging threads (the softmax waves)
  constexpr int KPT = kPKeys * (D / 8) / NC;
  constexpr int VPT = (kPKeys / 2) * (D / 4) / NC;
  static_assert(KPT == 1 && VPT == 1, "staging split");
  __shared__ __attribute__((aligned(16))) uint16_t s_k[3][kPKeys * KS];
  // V^T rows (dims) of VS keys, 8 more halves after every 16 rows: the
  // transposed stores of a wave then fall in 64 distinct banks
  constexpr int VTS = D * VS + 8 * (D / 16);
  __shared__ __attribute__((aligned(16))) _Float16 s_vt[2][VTS];
  __shared__ __attribute__((aligned(16))) float s_lk[3][kPKeys];
  __shared__ __attribute__((aligned(16))) float s_bias[2][16 * 64 * 4];  // [key tile][token tile][lane][4]
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kPRows * QS];
  __shared__ int s_id;
  __shared__ uint32_t s_seq;

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool bias_wave = wv < 4;
  const int p = wv & 3;         // bias wave: key tile p of a block; softmax wave: token tile p
  const int hf = (wv - 4) >> 2;  // softmax wave: which half of the group's query heads
  const int S = a.B * a.H_kv;
  const int n = w.n, nrb = w.nrb;
  const int Hq = a.H_q, Hkv = a.H_kv;

  if (tid == 0) {
    s_id = prefill_ticket(w, S, nrb);
    s_seq = (uint32_t)ldi_coh_p(&w.glob[kGlobSeq]) + 1u;  // this call's number
  }
  __syncthreads();
  const int id = s_id;
  const uint32_t tagv = carry_tag(s_seq);
  // token-block major: a chain predecessor always holds an earlier ticket of
  // the same queue, so it is already running
  const int s = id % S;
  const int I = id / S;
  const int b = s / Hkv, h = s - b * Hkv;
  const int len0 = a.seg_len[s];
  const int64_t off = a.seg_off[s];
  const int nseq = seq_n_k<VARLEN>(w, b);         // this sequence's tokens
  const int nrbs = (nseq + kPRows - 1) / kPRows;  // and its token blocks
  if constexpr (VARLEN) {
    if (I >= nrbs) {  // past the sequence's tokens: no work, and no chain waits on this block
      prefill_commit<VARLEN, kPThreadsWS, true>(a, w, &s_id, s_seq);
      return;
    }
  }
  const bool room = (int64_t)len0 + nseq <= a.seg_cap[s];
  const int a0 = h * HG;
  const int t0 = I * kPRows;  // first token of the block

  if (room) {
    const int nkeys = len0 + nseq;
    const int kend = len0 + min(nseq, t0 + kPRows);
    const int nJ = (kend + kPKeys - 1) / kPKeys;
    const int64_t TS = a.total_slots;
    const PairCoef pc = pair_coef(a.terms);
    const float cs = a.scale * kLog2e;
    const uint16_t* Kc = reinterpret_cast<const uint16_t*>(a.K);
    const uint16_t* Vc = reinterpret_cast<const uint16_t*>(a.V);
    const float col_scale = (a.terms & 2) ? pc.inv_n2 : 0.0f;
    auto slot = [&](int j) -> int64_t { return off + min(j, nkeys - 1); };

    for (int q = tid; q < kPRows * HG * (D / 8); q += kPThreadsWS) {
      const int tt = q / (HG * (D / 8)), rest = q - tt * (HG * (D / 8));
      const int64_t tk = (int64_t)b * n + min(t0 + tt, nseq - 1);
      *reinterpret_cast<u32x4*>(&s_q[tt * QS + rest * 8]) =
          *reinterpret_cast<const u32x4*>(w.qbf + (tk * Hq + a0) * D + rest * 8);
    }

    // ---- staging (softmax waves): K rows and key gates, V rows as key pairs
    const int ct = tid - 256;  // after the four bias waves
    u32x4 kst[KPT];
    uint2 vst[VPT][2];
    float lkst = 0.0f;
    auto load_k = [&](int J) {
      const int j0 = J * kPKeys;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int q = ct + NC * u, key = q / (D / 8), part = q % (D / 8);
        kst[u] = *reinterpret_cast<const u32x4*>(Kc + slot(j0 + key) * D + 8 * part);
      }
      if (ct < kPKeys) lkst = a.lk[slot(j0 + ct)];
    };
    // V staging: lane l of staging wave cw holds dims 4 (l & 15) .. + 3 of the
    // key pair pp; a wave's four pairs sit at four consecutive LDS dwords of
    // every V^T row
    const int v_part = ct & 15, v_sub = (ct >> 4) & 3, v_cw = ct >> 6;
    const int v_pp = (v_cw & 3) * 2 + (v_cw >> 2) * 16 + (v_sub & 1) + (v_sub >> 1) * 8;
    auto load_v = [&](int J) {
      const int j0 = J * kPKeys;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int pp = v_pp, part = v_part;
        vst[u][0] = *reinterpret_cast<const uint2*>(Vc + slot(j0 + 2 * pp) * D + 4 * part);
        vst[u][1] = *reinterpret_cast<const uint2*>(Vc + slot(j0 + 2 * pp + 1) * D + 4 * part);
      }
    };
    auto store_k = [&](int buf) {
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int q = ct + NC * u, key = q / (D / 8), part = q % (D / 8);
        *reinterpret_cast<u32x4*>(&s_k[buf][key * KS + 8 * part]) = kst[u];
      }
      if (ct < kPKeys) s_lk[buf][ct] = lkst * col_scale;
    };
    auto store_v = [&](int buf) {
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int pp = v_pp, part = v_part;
        const int pos = vt_pos(2 * pp);
        const uint32_t k0w[2] = {vst[u][0].x, vst[u][0].y}, k1w[2] = {vst[u][1].x, vst[u][1].y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = (e & 1) ? bf16_hi(k0w[e >> 1]) : bf16_lo(k0w[e >> 1]);
          const float v1 = (e & 1) ? bf16_hi(k1w[e >> 1]) : bf16_lo(k1w[e >> 1]);
          const auto hv = __builtin_amdgcn_cvt_pkrtz(v0, v1);
          const int d = 4 * part + e;
          *reinterpret_cast<uint32_t*>(&s_vt[buf][d * VS + 8 * (d >> 4) + pos]) = __builtin_bit_cast(uint32_t, hv);
        }
      }
    };

    // ---- bias wave state: this lane's tokens 16 tt + c16 of the block
    u32x4 krf[4][KC];
    float row2[4];
    auto load_token_side = [&]() {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int tq = min(t0 + 16 * tt + c16, nseq - 1);
        const int64_t tok = (int64_t)b * n + tq;
        const float lq = w.gl[2 * (tok * Hkv + h) + 0];
        const float lb = w.gl[2 * (tok * Hkv + h) + 1];
        row2[tt] = pc.inv_n2 * (((a.terms & 1) ? lq : 0.0f) + ((a.terms & 4) ? lb : 0.0f));
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          krf[tt][kc] = *reinterpret_cast<const u32x4*>(Kc + (off + len0 + tq) * D + 32 * kc + 8 * g);
      }
    };

    // Bias of key block JB for keys 16 p + 4 g + i and every token of the
    // block: carry in + inclusive scan of the pair terms over the tokens.
    // The carry in (the stored bias where this token block starts the key
    // block's chain, else the previous token block's carry words) is loaded
    // before the pair terms and used after them.
    auto bias_block = [&](int JB) {
      const int j0 = JB * kPKeys;
      const int kb = JB % 3;
      const int jk = j0 + 16 * p + 4 * g;  // this lane's first key
      const int Ist = j0 >= len0 ? (j0 - len0) / kPRows : 0;
      const bool chain = I > Ist;
      const unsigned long long* cin = w.carry64 + (int64_t)(I - 1) * TS;
      float car[4];
      unsigned long long cw[4];
      if (!chain) {
        // unconditional loads of clamped slots, the keys of this call zeroed
        // where they are used: a load under a condition would be a branch of
        // its own with an immediate wait
#pragma unroll
        for (int i = 0; i < 4; ++i) car[i] = ldf_coh_p(&a.lam[slot(jk + i)]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = ld64_coh_p(&cin[slot(jk + i)]);
      }
      u32x4 kf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kf[kc] = *reinterpret_cast<const u32x4*>(&s_k[kb][(16 * p + c16) * KS + 32 * kc + 8 * g]);
      const float4 lk4 = *reinterpret_cast<const float4*>(&s_lk[kb][16 * p + 4 * g]);
      const float lkv[4] = {lk4.x, lk4.y, lk4.z, lk4.w};
      const bool edge = (j0 + 16 * p + 15 >= len0 + t0) || (t0 + kPRows > nseq);
      // Pair terms, step-major over the 16 (key, token) elements of the lane so
      // that the transcendental chains of different elements interleave.  The
      // series form of 1 - 2^L is only needed where L is near 0; a wave takes
      // it only when one of its elements is there.
      float lam[4][4];
      auto pair_terms = [&](auto edge_c, auto sim_c) {
        constexpr bool EDGE = decltype(edge_c)::value, SIM = decltype(sim_c)::value;
        f32x4 sim[4];
        if constexpr (SIM) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            sim[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) sim[tt] = mfma_bf16(kf[kc], krf[tt][kc], sim[tt]);
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) lam[tt][i] = row2[tt] + lkv[i];
        if constexpr (SIM) {
          float lg[4][4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lg[tt][i] = __builtin_amdgcn_logf(fminf(sim[tt][i] * sim[tt][i], 1.0f));
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lam[tt][i] = fmaf(pc.sim_w, lg[tt][i], lam[tt][i]);
        }
        float lmax = kNegInf;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, lam[tt][i]);
        if (__any(lmax > kLog1mexpSeries)) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lam[tt][i] = log1mexp2_b2(lam[tt][i]);
        } else {
          float ex[4][4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ex[tt][i] = __builtin_amdgcn_exp2f(lam[tt][i]);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lam[tt][i] = __builtin_amdgcn_logf(1.0f - ex[tt][i]);
        }
        if constexpr (EDGE) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int tq = t0 + 16 * tt + c16;
#pragma unroll
            for (int i = 0; i < 4; ++i) lam[tt][i] = (tq < nseq && jk + i < len0 + tq) ? lam[tt][i] : 0.0f;
          }
        }
      };
      if (!pc.any) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) lam[tt][i] = 0.0f;
      } else if (edge) {
        if (pc.sim) pair_terms(std::true_type{}, std::true_type{});
        else pair_terms(std::true_type{}, std::false_type{});
      } else {
        if (pc.sim) pair_terms(std::false_type{}, std::true_type{});
        else pair_terms(std::false_type{}, std::false_type{});
      }
      // inclusive scans over the 16 tokens of each tile, step-major
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[tt][i] += dpp_f<0x111>(lam[tt][i]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[tt][i] += dpp_f<0x112>(lam[tt][i]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[tt][i] += dpp_f<0x114>(lam[tt][i]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[tt][i] += dpp_f<0x118>(lam[tt][i]);
      // across the tiles: add the running total of the earlier tiles
      float run[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) run[i] = dpp_f<kDppBcast15>(lam[0][i]);
#pragma unroll
      for (int tt = 1; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lam[tt][i] += run[i];
          run[i] = dpp_f<kDppBcast15>(lam[tt][i]);
        }
      // carry into this token block (log2 units)
      if (!chain) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float c = car[i];
          asm volatile("" : "+v"(c));  // first use here: the loads' wait stays after the pair terms
          car[i] = (jk + i < len0) ? c * kLog2e : 0.0f;
        }
      } else {
        int spins = 0;
        for (;;) {
          bool ok = true;
#pragma unroll
          for (int i = 0; i < 4; ++i) ok = ok && (uint32_t)(cw[i] >> 32) == tagv;
          if (ok) break;
          if (++spins > kPrefillSpinLimit) {
            atomicOr(a.status, 2);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((uint32_t)(cw[i] >> 32) != tagv) cw[i] = ld64_coh_p(&cin[slot(jk + i)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) car[i] = __uint_as_float((uint32_t)cw[i]);
      }
      // the written bias carries the attention mask: -inf where token t does
      // not see key j (j > len0 + t, or t past the call), and in a pruned
      // call where the entry's bias has fallen below the threshold
      float* ob = &s_bias[JB & 1][0];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        float bv[4];
        const int tq = t0 + 16 * tt + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bv[i] = lam[tt][i] + car[i];
          if (edge) bv[i] = (tq < nseq && jk + i <= len0 + tq) ? bv[i] : kNegInf;
          if constexpr (MASKED) bv[i] = (bv[i] >= w.tau2) ? bv[i] : kNegInf;
        }
        *reinterpret_cast<float4*>(&ob[((p * 4 + tt) * 64 + lane) * 4]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
      }
      // carry out to the next token block, or the final bias of the call
      if (I + 1 < nrbs) {
        if (c16 == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (jk + i < nkeys)
              st64_coh_p(&w.carry64[(int64_t)I * TS + off + jk + i],
                         (unsigned long long)tagv << 32 | __float_as_uint(car[i] + run[i]));
        }
      } else if (c16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (jk + i < nkeys) a.lam[off + jk + i] = (car[i] + run[i]) * kLn2;
      }
    };

    // ---- prologue: blocks 0 and 1 of K, block 0 of V in LDS; the bias of block 0
    if (!bias_wave) {
      load_k(0);
      load_v(0);
      store_k(0);
      store_v(0);
      if (nJ > 1) {
        load_k(1);
        store_k(1);
      }
      if (nJ > 2) load_k(2);
      if (nJ > 1) load_v(1);
    }
    if (bias_wave) load_token_side();
    __syncthreads();
    if (bias_wave) {
      // The two roles run separate loops with the same number of barriers, so
      // the state of one role is not live in the other.
      bias_block(0);
      __syncthreads();
      for (int J = 0; J < nJ - 1; ++J) {
        bias_block(J + 1);
        __syncthreads();
      }
      __syncthreads();  // the softmax loop's last barrier
    } else {
      // ---- softmax waves: tokens 16 p + c16, query heads hf*HH .. of the group
      const int tq = t0 + 16 * p + c16;
      const bool row_ok = tq < nseq;
      const int64_t tok = (int64_t)b * n + min(tq, nseq - 1);
      const float inv_cs = 1.0f / cs;
      f16x8 ones;
#pragma unroll
      for (int e = 0; e < 8; ++e) ones[e] = (c16 == 0) ? (_Float16)1.0f : (_Float16)0.0f;

      auto softmax_wave = [&](auto nh_c) {
        constexpr int NH = decltype(nh_c)::value;  // query heads of this wave
        const int h0 = hf * HH;                    // first of them within the group
        float qn[NH > 0 ? NH : 1];
        f32x4 O[NH > 0 ? NH : 1][DT], Lt[NH > 0 ? NH : 1];
        float m_run[NH > 0 ? NH : 1];
        int mset = 0;
        bool stat = true;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          float ss = 0.0f;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            const u32x4 qv =
                *reinterpret_cast<const u32x4*>(&s_q[(16 * p + c16) * QS + (h0 + hh) * D + 32 * kc + 8 * g]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = u32x4_bf16(qv, e);
              ss = fmaf(x, x, ss);
            }
          }
          ss += __shfl_xor(ss, 16, 64);
          ss += __shfl_xor(ss, 32, 64);
          qn[hh] = __builtin_sqrtf(ss);
          stat = stat && (cs * qn[hh] <= kStaticRef);
          m_run[hh] = 0.0f;
          Lt[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) O[hh][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        stat = __all(stat);
        __syncthreads();

        // Softmax and P V of key block J for this wave's tokens and heads, 32
        // keys at a time.  STAT: fixed reference cs |q~| (folded into the
        // accumulator's start); otherwise a running reference raised only when
        // a chunk exceeds it by more than 2^kRescaleTh.
        auto softmax_block = [&](int J, auto stat_c) {
          constexpr bool STAT = decltype(stat_c)::value;
          const int kb = J % 3, vb = J & 1;
          const float* ib = &s_bias[J & 1][0];
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            u32x4 kf[2][KC];
            float4 bias[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
              for (int kc = 0; kc < KC; ++kc)
                kf[t][kc] =
                    *reinterpret_cast<const u32x4*>(&s_k[kb][(32 * c2 + 16 * t + c16) * KS + 32 * kc + 8 * g]);
              bias[t] = *reinterpret_cast<const float4*>(&ib[(((2 * c2 + t) * 4 + p) * 64 + lane) * 4]);
            }
            f16x8 vf[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
              vf[dt] = *reinterpret_cast<const f16x8*>(&s_vt[vb][(16 * dt + c16) * VS + 8 * dt + 32 * c2 + 8 * g]);
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
              float e[2][4];
              float bm = kNegInf;
              const float ci = STAT ? -qn[hh] : -m_run[hh] * inv_cs;
              u32x4 qf[KC];
#pragma unroll
              for (int kc = 0; kc < KC; ++kc)
                qf[kc] = *reinterpret_cast<const u32x4*>(&s_q[(16 * p + c16) * QS + (h0 + hh) * D + 32 * kc + 8 * g]);
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                f32x4 sc = f32x4{ci, ci, ci, ci};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) sc = mfma_bf16(kf[t][kc], qf[kc], sc);
                const float bv[4] = {bias[t].x, bias[t].y, bias[t].z, bias[t].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float ev = fmaf(sc[i], cs, bv[i]);  // -inf where masked
                  e[t][i] = ev;
                  if constexpr (!STAT) bm = fmaxf(bm, ev);
                }
              }
              if constexpr (!STAT) {
                const bool fresh = ((mset >> hh) & 1) == 0;
                if (__any(bm > kRescaleTh || (fresh && bm > kNegInf))) {
                  float bx = fmaxf(bm, __shfl_xor(bm, 16, 64));
                  bx = fmaxf(bx, __shfl_xor(bx, 32, 64));
                  const float dl = fresh ? ((bx > kNegInf) ? bx : 0.0f) : fmaxf(bx, 0.0f);
                  const float al = fresh ? 1.0f : __builtin_amdgcn_exp2f(-dl);
#pragma unroll
                  for (int dt = 0; dt < DT; ++dt) O[hh][dt] *= al;
                  Lt[hh] *= al;
                  m_run[hh] += dl;
                  if (bx > kNegInf) mset |= 1 << hh;
#pragma unroll
                  for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) e[t][i] -= dl;
                }
              }
              f16x8 pk;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                pk[i] = (_Float16)__builtin_amdgcn_exp2f(e[0][i]);
                pk[4 + i] = (_Float16)__builtin_amdgcn_exp2f(e[1][i]);
              }
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) O[hh][dt] = mfma_f16(vf[dt], pk, O[hh][dt]);
              Lt[hh] = mfma_f16(ones, pk, Lt[hh]);
            }
          }
        };

        // one loop per reference mode, so each holds only its own state
        auto softmax_loop = [&](auto stat_c) {
          for (int J = 0; J < nJ; ++J) {
            // K of block J + 2 and V of block J + 1 to LDS (buffers no role
            // reads in this block), then the loads of the blocks after, which
            // have a whole block to arrive
            if (J + 2 < nJ) store_k((J + 2) % 3);
            if (J + 1 < nJ) store_v((J + 1) & 1);
            if (J + 3 < nJ) load_k(J + 3);
            if (J + 2 < nJ) load_v(J + 2);
            if constexpr (NH > 0) softmax_block(J, stat_c);
            __syncthreads();
          }
        };
        if (stat) softmax_loop(std::true_type{});
        else softmax_loop(std::false_type{});

        // ---- epilogue: normalise, gate, store
        const int64_t ytok = io_row_k<VARLEN>(w, (int)tok);  // the token's row of y (not live in the loop)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const float L = __shfl(Lt[hh][0], c16, 64);
          const float inv = (row_ok && L > 0.0f) ? 1.0f / L : 0.0f;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int64_t yo = (ytok * Hq + a0 + h0 + hh) * D + 16 * dt + 4 * g;
            const f32x4 gm = out_gate(a, w, tok, (a0 + h0 + hh) * D + 16 * dt, g, c16);
            const float y0 = gm[0] * O[hh][dt][0] * inv, y1 = gm[1] * O[hh][dt][1] * inv;
            const float y2 = gm[2] * O[hh][dt][2] * inv, y3 = gm[3] * O[hh][dt][3] * inv;
            if (row_ok) {
              if (a.y_bf16) {
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + yo) =
                    make_uint2(pack_bf16(y0, y1), pack_bf16(y2, y3));
              } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + yo) = make_float4(y0, y1, y2, y3);
              }
            }
            __builtin_amdgcn_sched_barrier(0);  // one gate tile's operands live at a time
          }
        }
      };
      if (hf == 0) softmax_wave(std::integral_constant<int, HH>{});
      else softmax_wave(std::integral_constant<int, HG - HH>{});
    }
  } else if (!bias_wave && hf == 0) {
    // the segment has no room for the call: its outputs are zero
    const int tq = t0 + 16 * p + c16;
    if (tq < nseq) {
      const int64_t ytok = io_row_k<VARLEN>(w, b * n + tq);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int64_t yo = (ytok * Hq + a0 + hh) * D + 16 * dt + 4 * g;
          if (a.y_bf16) {
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + yo) = make_uint2(0u, 0u);
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + yo) = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
    }
  }

  prefill_commit<VARLEN, kPThreadsWS, true>(a, w, &s_id, s_seq);
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
template <int D, int HG>
static void launch_attn(const LayerArgs& a, const PrefillWs& w, int grid, hipStream_t st) {
  if (w.cu) {
    hipLaunchKernelGGL((prefill_attn_kernel<D, HG, true>), dim3(grid), dim3(kPThreads), 0, st, a, w);
  } else {
    hipLaunchKernelGGL((prefill_attn_kernel<D, HG, false>), dim3(grid), dim3(kPThreads), 0, st, a, w);
  }
}

// Instances: dense, masked (pruned prefill) and variable-length (dense).
template <int HG>
static void launch_attn_ws(const LayerArgs& a, const PrefillWs& w, int grid, hipStream_t st) {
  if (w.cu) {
    hipLaunchKernelGGL((prefill_attn_ws_kernel<HG, false, true>), dim3(grid), dim3(kPThreadsWS), 0, st, a, w);
  } else if (w.tau2 > kNegInf) {
    hipLaunchKernelGGL((prefill_attn_ws_kernel<HG, true, false>), dim3(grid), dim3(kPThreadsWS), 0, st, a, w);
  } else {
    hipLaunchKernelGGL((prefill_attn_ws_kernel<HG, false, false>), dim3(grid), dim3(kPThreadsWS), 0, st, a, w);
  }
}

hipError_t launch_prefill(const LayerArgs& a, const Control& ctl, int n, int max_seg_cap, void* scratch,
                          size_t scratch_bytes, hipStream_t st, float log_p, int ld, int t0, const int* cu,
                          int total) {
  if (!a.bf16) return hipErrorNotSupported;  // the matrix-core path is written for bf16 caches
  const int G = a.H_q / a.H_kv;
  if (a.d == 128 && G == 8) return hipErrorNotSupported;
  if (prefill_ws_bytes(a, n, max_seg_cap) > scratch_bytes) return hipErrorOutOfMemory;
  PrefillWs w;
  prefill_layout(a, n, reinterpret_cast<char*>(scratch), &w);
  w.glob = ctl.glob;
  w.ld = ld;
  w.t0 = t0;
  w.cu = cu;
  w.total = total;
  w.tau2 = (log_p == -__builtin_huge_valf()) ? -__builtin_huge_valf() : log_p * kLog2e;
  const int S = a.B * a.H_kv;
  const int nsync = 2 + S * w.nrb + kXcds;
  const int64_t prep_items = std::max<int64_t>(std::max<int64_t>(nsync, (int64_t)w.cp * (a.D_model / 8)),
                                               (int64_t)a.H_q * a.d * (w.rp / 8));
  const int prep_grid = (int)std::min<int64_t>(1024, std::max<int64_t>(1, (prep_items + 255) / 256));
  hipLaunchKernelGGL(prefill_prep_kernel, dim3(prep_grid), dim3(256), 0, st, a, w, nsync);
  const int tok_grid = (a.B * n + kPTok - 1) / kPTok;
  if (a.d == 64) {
    hipLaunchKernelGGL(prefill_token_kernel<64>, dim3(tok_grid), dim3(kTT), 0, st, a, w);
  } else {
    hipLaunchKernelGGL(prefill_token_kernel<128>, dim3(tok_grid), dim3(kTT), 0, st, a, w);
  }
  const int grid = S * w.nrb;
  switch (a.d * 16 + G) {
    case 64 * 16 + 1: launch_attn_ws<1>(a, w, grid, st); break;
    case 64 * 16 + 2: launch_attn_ws<2>(a, w, grid, st); break;
    case 64 * 16 + 3: launch_attn_ws<3>(a, w, grid, st); break;
    case 64 * 16 + 4: launch_attn_ws<4>(a, w, grid, st); break;
    case 64 * 16 + 8: launch_attn<64, 8>(a, w, grid, st); break;
    case 128 * 16 + 1: launch_attn<128, 1>(a, w, grid, st); break;
    case 128 * 16 + 2: launch_attn<128, 2>(a, w, grid, st); break;
    case 128 * 16 + 3: launch_attn<128, 3>(a, w, grid, st); break;
    case 128 * 16 + 4: launch_attn<128, 4>(a, w, grid, st); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace ua

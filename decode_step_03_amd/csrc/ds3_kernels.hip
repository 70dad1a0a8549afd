// Decode-step kernels for MI355X (gfx950, CDNA4, wave64).
//
// The step is memory-bound at small batch ("Execution" page, section "Why capture"): every token streams all
// weights once and sweeps the K/V buffers over the whole capacity. The kernels are therefore built around
// 16-byte per-lane loads of weight rows and K/V rows, with fp32 accumulation, one wave per output-row pair, and
// wave-level shuffle reductions in a fixed order (so a replay reproduces an eager run bit for bit).
//
// Kernel set (one launch each, per layer where noted):
//   embed_kernel      x[r] = E[token[r]]                                      (reads Slot::Token)
//   gemv_kernel<QKV>  RMSNorm(x) -> q, k, v rows; rotary epilogue on q and k; k and v stored at Slot::Pos
//                     (contiguous) or at Slot::WriteMap (paged)             per layer
//   attn_kernel       split sweep of all [cap] positions, mask from Slot::Pos against the position index,
//                     per-split softmax partials, last-arriving block merges the splits in fixed order  per layer
//   gemv_kernel<RESID> x += W_o . o                                         per layer
//   gemv_kernel<GATEUP> RMSNorm(x) -> gate/up rows, SwiGLU epilogue -> act  per layer
//   gemv_kernel<RESID> x += W_down . act                                    per layer
//   gemv_kernel<HEAD> RMSNorm(x) -> logits, non-finite flag
//
// No kernel takes a token, a position or a map entry by value: they are read from the slot buffer, so one
// recorded graph serves every step ("Execution" page, section "Slot buffers").
#include "ds3_kernels.h"

#include <math.h>

namespace ds3 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kUnroll = 8;   // 16-byte loads in flight per lane per weight row

__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 16 bytes of stored values -> floats
template <typename T>
struct Pack;
template <>
struct Pack<uint16_t> {  // bf16 words
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const u32x4& w, float (&f)[8]) {
    f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
    f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
    f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};
template <>
struct Pack<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(const u32x4& w, float (&f)[4]) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};

__device__ __forceinline__ float widen1(uint16_t w) { return __uint_as_float(uint32_t(w) << 16); }
__device__ __forceinline__ float widen1(float w) { return w; }

// float32 -> bf16 word, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ void store_kv(uint16_t* p, float v) { *p = to_bf16(v); }
__device__ __forceinline__ void store_kv(float* p, float v) { *p = v; }

// Butterfly sums over the wave. Lanes may differ in the last bit (different association); callers use lane 0.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ void raise_error(StatusWords* st, uint32_t bit) { atomicOr(&st->err, bit); }

// Element offset of (row r, kv head g, position j, element 0) within one layer's K (or V) state.
__device__ __forceinline__ size_t kv_offset(const KvView& kv, int r, int nkv, int g, int j, int hd,
                                            StatusWords* st) {
  if (!kv.paged) return ((size_t)(r * nkv + g) * kv.cap + j) * hd;
  const int ppr = kv.cap / kv.page_size;
  int page = kv.slot_map[r * ppr + j / kv.page_size];
  if (page < 0 || page >= kv.pool_pages) {
    raise_error(st, ERR_PAGE);
    page = 0;
  }
  return ((size_t)(page * nkv + g) * kv.page_size + (j % kv.page_size)) * hd;
}

// ----------------------------------------------------------------------------------------------------------
// embedding

template <typename WT>
__global__ void __launch_bounds__(kBlock) embed_kernel(EmbedParams p) {
  const int r = blockIdx.x;
  SlotLayout sl{p.rows};
  int token = p.slots[sl.token() + r];
  if (token < 0 || token >= p.vocab) {
    if (threadIdx.x == 0) raise_error(p.status, ERR_TOKEN);
    token = 0;
  }
  if (r == 0 && threadIdx.x == 0 && p.slots[sl.inject()] != 0) raise_error(p.status, ERR_INJECTED);
  const WT* row = reinterpret_cast<const WT*>(p.table) + (size_t)token * p.d;
  for (int k = threadIdx.x; k < p.d; k += kBlock) p.x[(size_t)r * p.d + k] = widen1(row[k]);
}

// ----------------------------------------------------------------------------------------------------------
// Paired-row GEMV with fused prologue and epilogue.
//
// Each wave owns one pair of weight rows at a time and computes both rows' dot products with every activation
// row (NR of them) held in LDS as fp32. A pair is the unit the epilogue needs: the two halves of a rotary pair
// (element i and element i + hd/2 of a q or k head), a gate row and its up row, or two adjacent output rows.
//
// Latency is what limits these short kernels, so the order of memory operations is deliberate:
//   1. every thread loads its share of the activation (and, for the norm modes, the RMSNorm gain) into
//      registers -- these loads go first because loads return in order;
//   2. the wave starts streaming its first pair of weight rows (kUnroll x 16 bytes per lane per row) and the
//      epilogue operands that live in memory;
//   3. the activations (times the gain) go to LDS while the weights are in flight, and the RMSNorm sum of
//      squares is reduced from the registers: one barrier, which waits for LDS traffic only;
//   4. dot products as the weights arrive; fixed-order wave butterfly; the RMSNorm scale
//      1/sqrt(mean(x^2) + eps) multiplies the two dot products in the epilogue.
// No load sits behind a per-lane branch (indices are clamped instead), so nothing forces an early wait.

template <int MODE>
struct PairMap {
  int row0, row1;
  int seg, head, idx;   // QKV: segment 0 q / 1 k / 2 v, head, element within the head
  __device__ __forceinline__ PairMap(const GemvParams& p, int pair) : seg(0), head(0), idx(0) {
    if constexpr (MODE == GEMV_QKV) {
      const int half = p.hd / 2;
      const int nqp = p.nq * half, nkp = p.nkv * half;
      if (pair < nqp) {
        head = pair / half; idx = pair % half;
        row0 = head * p.hd + idx; row1 = row0 + half;
      } else if (pair < nqp + nkp) {
        const int pp = pair - nqp;
        seg = 1; head = pp / half; idx = pp % half;
        row0 = p.nq * p.hd + head * p.hd + idx; row1 = row0 + half;
      } else {
        const int pv = 2 * (pair - nqp - nkp);
        seg = 2; head = pv / p.hd; idx = pv % p.hd;
        row0 = (p.nq + p.nkv) * p.hd + pv; row1 = row0 + 1;
      }
    } else if constexpr (MODE == GEMV_GATEUP) {
      row0 = pair; row1 = p.up_offset + pair;
    } else {
      row0 = 2 * pair; row1 = row0 + 1;
    }
  }
};

// Loads of one group of kUnroll chunks of two weight rows. Past the row's end the chunk index is clamped to the
// last chunk and the element index to the last 16 bytes: in bounds, no branches; fma_group zeroes them.
template <typename WT>
__device__ __forceinline__ void load_group(const WT* w0, const WT* w1, int c0, int nchunks, int K, int lane,
                                           u32x4 (&b0)[kUnroll], u32x4 (&b1)[kUnroll]) {
  constexpr int EPL = Pack<WT>::N;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int k = min(min(c0 + u, nchunks - 1) * (64 * EPL) + lane * EPL, K - EPL);
    b0[u] = load_stream(w0 + k);
    b1[u] = load_stream(w1 + k);
  }
}

template <typename WT, int NR>
__device__ __forceinline__ void fma_group(const u32x4 (&b0)[kUnroll], const u32x4 (&b1)[kUnroll], const float* xs,
                                          int c0, int nchunks, int K, int lane, float (&a0)[NR], float (&a1)[NR]) {
  constexpr int EPL = Pack<WT>::N;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int kr = (c0 + u) * (64 * EPL) + lane * EPL;
    const bool valid = c0 + u < nchunks && kr < K;
    const int k = min(min(c0 + u, nchunks - 1) * (64 * EPL) + lane * EPL, K - EPL);
    float f0[EPL], f1[EPL];
    Pack<WT>::widen(b0[u], f0);
    Pack<WT>::widen(b1[u], f1);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      f0[e] = valid ? f0[e] : 0.f;
      f1[e] = valid ? f1[e] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float* xr = xs + r * K + k;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        a0[r] = fmaf(f0[e], xr[e], a0[r]);
        a1[r] = fmaf(f1[e], xr[e], a1[r]);
      }
    }
  }
}

template <typename WT, typename KT, int NR, int MODE, int XREG>
__global__ void __launch_bounds__(kBlock) gemv_kernel(GemvParams p) {
  extern __shared__ float xs[];  // [NR][K] activations (times the gain in the norm modes)
  __shared__ float red[NR][kBlock / 64];
  constexpr bool kNorm = MODE != GEMV_RESID;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = p.K;
  const int K4 = K / 4;
  const int nchunks = (K + 64 * Pack<WT>::N - 1) / (64 * Pack<WT>::N);
  const int nwaves = gridDim.x * (kBlock / 64);
  const SlotLayout sl{p.rows};

  // ---- 1. slot positions, then activation (and gain) loads, first
  int posr[NR];
  bool pos_ok[NR];
  if constexpr (MODE == GEMV_QKV) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int ps = p.slots[sl.pos() + r];
      pos_ok[r] = ps >= 0 && ps < p.kv.cap;
      posr[r] = pos_ok[r] ? ps : 0;
    }
  }
  const int n4 = NR * K4;
  const float4* in4 = reinterpret_cast<const float4*>(p.in);
  const float4* g4 = reinterpret_cast<const float4*>(kNorm ? p.gain : p.in);
  float4 xv[XREG], gv[kNorm ? XREG : 1];
#pragma unroll
  for (int u = 0; u < XREG; ++u) {
    const int i = min(tid + u * kBlock, n4 - 1);
    xv[u] = in4[i];
    if constexpr (kNorm) gv[u] = g4[i % K4];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. the first pair's weights (they do not depend on the activations) and its epilogue operands
  const WT* wbase = reinterpret_cast<const WT*>(p.w);
  u32x4 b0[kUnroll], b1[kUnroll];
  float ea[NR], eb[NR];
  int pair = blockIdx.x * (kBlock / 64) + wid;
  PairMap<MODE> pm(p, min(pair, p.n_pairs - 1));
  const WT* w0 = wbase + (size_t)pm.row0 * K;
  const WT* w1 = wbase + (size_t)pm.row1 * K;
  auto fetch_epilogue = [&ea, &eb, &p, &posr](const PairMap<MODE>& m, int pr) {
    (void)p;
    (void)posr;
#pragma unroll
    for (int r = 0; r < NR; ++r) { ea[r] = 0.f; eb[r] = 0.f; }
    if constexpr (MODE == GEMV_QKV) {
      if (m.seg != 2) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float2 cs = reinterpret_cast<const float2*>(p.rope)[(size_t)posr[r] * (p.hd / 2) + m.idx];
          ea[r] = cs.x;
          eb[r] = cs.y;
        }
      }
    } else if constexpr (MODE == GEMV_RESID) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float2 xo = reinterpret_cast<const float2*>(p.out + (size_t)r * 2 * p.n_pairs)[pr];
        ea[r] = xo.x;
        eb[r] = xo.y;
      }
    }
  };
  // unconditional (the pair index is clamped): a branch here would make every later wait conservative
  load_group<WT>(w0, w1, 0, nchunks, K, lane, b0, b1);
  fetch_epilogue(pm, min(pair, p.n_pairs - 1));

  // ---- 3. LDS fill (clamped lanes rewrite the same value) and the RMSNorm sums of squares
  float4* xs4 = reinterpret_cast<float4*>(xs);
  float ss[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) ss[r] = 0.f;
#pragma unroll
  for (int u = 0; u < XREG; ++u) {
    const int iu = tid + u * kBlock;
    const int i = min(iu, n4 - 1);
    float4 v = xv[u];
    if constexpr (kNorm) {
      const float sq = (iu < n4) ? v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w : 0.f;
      const int row = i / K4;
#pragma unroll
      for (int r = 0; r < NR; ++r) ss[r] += (row == r) ? sq : 0.f;
      v = make_float4(v.x * gv[u].x, v.y * gv[u].y, v.z * gv[u].z, v.w * gv[u].w);
    }
    xs4[i] = v;
  }
  for (int i = tid + XREG * kBlock; i < n4; i += kBlock) {   // activations beyond the register share, if any
    float4 v = in4[i];
    if constexpr (kNorm) {
      const float4 gg = g4[i % K4];
      const float sq = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
      for (int r = 0; r < NR; ++r) ss[r] += (i / K4 == r) ? sq : 0.f;
      v = make_float4(v.x * gg.x, v.y * gg.y, v.z * gg.z, v.w * gg.w);
    }
    xs4[i] = v;
  }
  if constexpr (kNorm) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float t = wave_sum(ss[r]);
      if (lane == 0) red[r][wid] = t;
    }
  }
  __syncthreads();
  float scale[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    scale[r] = 1.f;
    if constexpr (kNorm) {
      const float tot = (red[r][0] + red[r][1]) + (red[r][2] + red[r][3]);
      scale[r] = 1.0f / sqrtf(tot / (float)K + p.eps);
    }
  }

  // ---- 4. pairs
  bool first = true;
  for (; pair < p.n_pairs; pair += nwaves) {
    if (!first) {
      pm = PairMap<MODE>(p, pair);
      w0 = wbase + (size_t)pm.row0 * K;
      w1 = wbase + (size_t)pm.row1 * K;
      load_group<WT>(w0, w1, 0, nchunks, K, lane, b0, b1);
      fetch_epilogue(pm, pair);
    }
    first = false;
    float a0[NR], a1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) { a0[r] = 0.f; a1[r] = 0.f; }
    for (int c0 = 0; c0 < nchunks; c0 += kUnroll) {
      if (c0 > 0) load_group<WT>(w0, w1, c0, nchunks, K, lane, b0, b1);
      fma_group<WT, NR>(b0, b1, xs, c0, nchunks, K, lane, a0, a1);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      a0[r] = wave_sum(a0[r]);
      a1[r] = wave_sum(a1[r]);
    }
    if (lane != 0) continue;

    // ---- epilogue (lane 0)
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float a = a0[r] * scale[r], b = a1[r] * scale[r];
      if constexpr (MODE == GEMV_QKV) {
        if (!pos_ok[r]) raise_error(p.status, ERR_POS);
        const int half = p.hd / 2;
        float va = a, vb = b;
        if (pm.seg != 2) {   // rotate the pair (element idx, element idx + hd/2) by the angle of Slot::Pos
          va = a * ea[r] - b * eb[r];
          vb = a * eb[r] + b * ea[r];
        }
        if (pm.seg == 0) {
          float* q = p.out + ((size_t)r * p.nq + pm.head) * p.hd;
          q[pm.idx] = va;
          q[pm.idx + half] = vb;
          continue;
        }
        if (!pos_ok[r]) continue;
        size_t off;
        if (!p.kv.paged) {
          off = ((size_t)(r * p.nkv + pm.head) * p.kv.cap + posr[r]) * p.hd;
        } else {
          const int slot = p.slots[sl.write_map() + r];
          if (slot < 0 || slot >= p.kv.pool_pages * p.kv.page_size) { raise_error(p.status, ERR_WRITE_MAP); continue; }
          off = ((size_t)((slot / p.kv.page_size) * p.nkv + pm.head) * p.kv.page_size + slot % p.kv.page_size) * p.hd;
        }
        // k: the two halves of a rotary pair; v: two adjacent elements
        KT* dst = reinterpret_cast<KT*>(pm.seg == 1 ? p.kv.k : p.kv.v) + (size_t)p.layer * p.kv.layer_stride + off +
                  pm.idx;
        store_kv(dst, va);
        store_kv(dst + (pm.seg == 1 ? half : 1), vb);
      } else if constexpr (MODE == GEMV_GATEUP) {
        const float silu = a / (1.0f + expf(-a));
        p.out[(size_t)r * p.n_pairs + pair] = silu * b;
      } else if constexpr (MODE == GEMV_RESID) {
        float2* x = reinterpret_cast<float2*>(p.out + (size_t)r * 2 * p.n_pairs) + pair;
        *x = make_float2(ea[r] + a, eb[r] + b);
      } else {  // GEMV_HEAD
        float2* lg = reinterpret_cast<float2*>(p.out + (size_t)r * 2 * p.n_pairs) + pair;
        *lg = make_float2(a, b);
        if (!isfinite(a) || !isfinite(b)) atomicOr(&p.status->nonfinite, 1u);
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------------------
// Attention: split sweep over the whole [cap] of one (row, kv head), all G query heads of the group at once.
//
// grid = (splits, nkv, rows); each block owns positions [s*T, s*T + T) of one kv head.
// Phase A: LPP lanes share one position (16 bytes of the head each); scores for the G query heads are
//          reduced over those lanes and kept in LDS. Positions j > pos (Slot::Pos) are hidden by selection:
//          their score becomes -inf and their value row never reaches the accumulator, so whatever the buffer
//          holds after pos (stale data, inf, NaN) cannot leak into the result.
// Phase B: per head, the split's max m and the weights p_j = exp(s_j - m), sum l; then o = sum_j p_j v_j.
// Merge:   the block that arrives last for its (row, kv head) -- an integer counter decides, the order of the
//          merge does not depend on it -- merges the splits in split order s = 0..S-1:
//          o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, M = max_s m_s.

template <typename KT, int HD, int G>
__global__ void __launch_bounds__(kBlock) attn_kernel(AttnParams p) {
  constexpr int EPL = Pack<KT>::N;
  constexpr int LPP = HD / EPL;         // lanes per position
  constexpr int PPP = kBlock / LPP;     // positions per block pass
  constexpr int UA = 8;                 // passes in flight
  static_assert(LPP >= 1 && LPP <= 64 && (64 % LPP) == 0, "lanes per position must divide the wave");
  extern __shared__ float sm[];
  float* sc = sm;                       // [G][T] scores, then weights
  float* ow = sm + G * p.split_len;     // [4 waves][G][HD]
  float* mstat = ow + 4 * G * HD;       // merge: [G][S] split maxima, then merge weights
  float* lstat = mstat + G * p.splits;  // merge: [G][S] split sums
  __shared__ float s_m[G], s_l[G];
  __shared__ int s_last;

  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int rows = gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sub = tid % LPP, grp = tid / LPP;
  const int T = p.split_len;
  const int j0 = s * T;
  const int cap = p.kv.cap;
  const SlotLayout sl{rows};

  int pos = p.slots[sl.pos() + r];
  if (pos < 0 || pos >= cap) {
    if (tid == 0) raise_error(p.status, ERR_POS);
    pos = 0;
  }
  const KT* Kb = reinterpret_cast<const KT*>(p.kv.k) + (size_t)p.layer * p.kv.layer_stride;
  const KT* Vb = reinterpret_cast<const KT*>(p.kv.v) + (size_t)p.layer * p.kv.layer_stride;

  float qv[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[hh][e] = p.q[((size_t)r * p.nq + g * G + hh) * HD + sub * EPL + e];

  // ---- phase A: scores
  for (int t0 = 0; t0 < T; t0 += PPP * UA) {
    u32x4 kb[UA];
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int t = t0 + u * PPP + grp;
      const int j = j0 + t;
      kb[u] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + u * PPP < T) {   // uniform: T is a whole number of passes
        const int jj = min(j, cap - 1);   // past the capacity: a clamped, masked re-read
        kb[u] = load_stream(Kb + kv_offset(p.kv, r, p.nkv, g, jj, HD, p.status) + sub * EPL);
      }
    }
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int t = t0 + u * PPP + grp;
      const int j = j0 + t;
      float kf[EPL];
      Pack<KT>::widen(kb[u], kf);
      float d[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qv[hh][e], kf[e], acc);
#pragma unroll
        for (int m = LPP / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
        d[hh] = acc;
      }
      if (sub == 0 && t < T) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) sc[hh * T + t] = (j <= pos) ? d[hh] * p.scale : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- per-head max and weights of this split
  for (int hh = wid; hh < G; hh += kBlock / 64) {
    float m = -INFINITY;
    for (int t = lane; t < T; t += 64) m = fmaxf(m, sc[hh * T + t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < T; t += 64) {
      const float sv = sc[hh * T + t];
      const float pr = (sv == -INFINITY) ? 0.f : expf(sv - m);
      sc[hh * T + t] = pr;
      l += pr;
    }
    l = wave_sum(l);
    if (lane == 0) { s_m[hh] = m; s_l[hh] = l; }
  }
  __syncthreads();

  // ---- phase B: weighted values
  float o[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  for (int t0 = 0; t0 < T; t0 += PPP * UA) {
    u32x4 vb[UA];
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int t = t0 + u * PPP + grp;
      const int j = j0 + t;
      vb[u] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + u * PPP < T) {
        const int jj = min(j, cap - 1);
        vb[u] = load_stream(Vb + kv_offset(p.kv, r, p.nkv, g, jj, HD, p.status) + sub * EPL);
      }
    }
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int t = t0 + u * PPP + grp;
      const int j = j0 + t;
      if (t < T) {
        const bool visible = j <= pos;
        float vf[EPL];
        Pack<KT>::widen(vb[u], vf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pr = sc[hh * T + t];
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float pv = pr * vf[e];
            o[hh][e] += visible ? pv : 0.f;
          }
        }
      }
    }
  }
  // reduce over the position groups of the wave (lanes with the same `sub`), then over the 4 waves
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = o[hh][e];
#pragma unroll
      for (int m = LPP; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
      o[hh][e] = v;
    }
  if (lane < LPP) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) ow[(wid * G + hh) * HD + sub * EPL + e] = o[hh][e];
  }
  __syncthreads();

  const int S = p.splits;
  float* part = p.part + (((size_t)r * p.nkv + g) * S) * (G * (HD + 2));
  float* mine = part + (size_t)s * (G * (HD + 2));
  for (int i = tid; i < G * HD; i += kBlock) {
    const int hh = i / HD, dd = i % HD;
    const float v = ((ow[(0 * G + hh) * HD + dd] + ow[(1 * G + hh) * HD + dd]) + ow[(2 * G + hh) * HD + dd]) +
                    ow[(3 * G + hh) * HD + dd];
    mine[hh * (HD + 2) + dd] = v;
  }
  if (tid < G) {
    mine[tid * (HD + 2) + HD] = s_m[tid];
    mine[tid * (HD + 2) + HD + 1] = s_l[tid];
  }

  // ---- last arriving block merges the splits
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&p.counters[r * p.nkv + g], 1u);
    s_last = (prev == (unsigned)(S - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();   // acquire: every split's partials are visible to plain loads from here on
  for (int i = tid; i < G * S; i += kBlock) {
    const int hh = i / S, s2 = i % S;
    const float* ps = part + (size_t)s2 * (G * (HD + 2)) + hh * (HD + 2);
    mstat[i] = ps[HD];
    lstat[i] = ps[HD + 1];
  }
  __syncthreads();
  for (int hh = wid; hh < G; hh += kBlock / 64) {
    float M = -INFINITY;
    for (int s2 = lane; s2 < S; s2 += 64) M = fmaxf(M, mstat[hh * S + s2]);
    M = wave_max(M);
    float L = 0.f;
    for (int s2 = lane; s2 < S; s2 += 64) {
      const float ms = mstat[hh * S + s2];
      const float wgt = (ms == -INFINITY) ? 0.f : expf(ms - M);
      mstat[hh * S + s2] = wgt;
      L += wgt * lstat[hh * S + s2];
    }
    L = wave_sum(L);
    if (lane == 0) s_l[hh] = L;
  }
  __syncthreads();
  for (int i = tid; i < G * HD; i += kBlock) {
    const int hh = i / HD, dd = i % HD;
    const float* po = part + hh * (HD + 2) + dd;
    float acc = 0.f;
#pragma unroll 8
    for (int s2 = 0; s2 < S; ++s2) acc = fmaf(mstat[hh * S + s2], po[(size_t)s2 * (G * (HD + 2))], acc);
    p.out[((size_t)r * p.nq + g * G + hh) * HD + dd] = acc / s_l[hh];
  }
  if (tid == 0) __hip_atomic_store(&p.counters[r * p.nkv + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------------------------------------
// K/V state copies for write_kv / read_kv: staging [nkv][n][hd] <-> state (contiguous or paged)

template <typename KT>
__global__ void __launch_bounds__(kBlock) kv_copy_kernel(KvView kv, int layer, int row, int pos0, int n, int nkv,
                                                          int hd, KT* staging, int to_state, StatusWords* st) {
  const size_t per = (size_t)n * hd;
  const size_t total = 2 * (size_t)nkv * per;   // K then V
  for (size_t i = blockIdx.x * (size_t)kBlock + threadIdx.x; i < total; i += (size_t)gridDim.x * kBlock) {
    const int which = (int)(i / (nkv * per));
    const size_t rem = i % (nkv * per);
    const int g = (int)(rem / per);
    const int t = (int)((rem / hd) % n);
    const int e = (int)(rem % hd);
    KT* base = reinterpret_cast<KT*>(which ? kv.v : kv.k) + (size_t)layer * kv.layer_stride;
    KT* dst = base + kv_offset(kv, row, nkv, g, pos0 + t, hd, st) + e;
    if (to_state) *dst = staging[i];
    else staging[i] = *dst;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// ----------------------------------------------------------------------------------------------------------
// host launchers

size_t gemv_lds_bytes(int rows, int K, bool norm) { (void)norm; return (size_t)rows * K * sizeof(float); }

int attn_positions_per_pass(int hd, int kv_dtype) {
  const int epl = kv_dtype == 1 ? 8 : 4;
  return kBlock / (hd / epl);
}

size_t attn_lds_bytes(int nq, int nkv, int hd, int split_len, int splits) {
  const int G = nq / nkv;
  return ((size_t)G * split_len + (size_t)4 * G * hd + (size_t)2 * G * splits) * sizeof(float);
}

template <typename F>
static hipError_t set_lds(F* f, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

hipError_t launch_embed(const EmbedParams& p, int weight_dtype, hipStream_t s) {
  if (weight_dtype == 1) embed_kernel<uint16_t><<<p.rows, kBlock, 0, s>>>(p);
  else embed_kernel<float><<<p.rows, kBlock, 0, s>>>(p);
  return hipGetLastError();
}

template <typename WT, typename KT, int MODE, int NR, int XREG>
static hipError_t gemv_go(const GemvParams& p, int blocks, hipStream_t s) {
  auto* f = gemv_kernel<WT, KT, NR, MODE, XREG>;
  const size_t lds = gemv_lds_bytes(p.rows, p.K, MODE != GEMV_RESID);
  hipError_t e = set_lds(f, lds);
  if (e != hipSuccess) return e;
  f<<<blocks, kBlock, lds, s>>>(p);
  return hipGetLastError();
}

// Register share of the activation per thread: the norm modes hold rows x d_model / 1024 float4 (4 per row for
// d_model = 4096); the residual modes hold up to 16 float4 (K up to 16384 at one row). The rest, if any, is
// loaded in a loop.
template <typename WT, typename KT, int MODE>
static hipError_t gemv_rows(const GemvParams& p, int blocks, hipStream_t s) {
  if constexpr (MODE != GEMV_RESID) {
    switch (p.rows) {
      case 1: return gemv_go<WT, KT, MODE, 1, 4>(p, blocks, s);
      case 2: return gemv_go<WT, KT, MODE, 2, 8>(p, blocks, s);
      case 3: return gemv_go<WT, KT, MODE, 3, 12>(p, blocks, s);
      case 4: return gemv_go<WT, KT, MODE, 4, 16>(p, blocks, s);
    }
  } else {
    const bool small = p.rows * p.K <= 4 * 4 * kBlock;   // fits 4 float4 per thread
    switch (p.rows) {
      case 1: return small ? gemv_go<WT, KT, MODE, 1, 4>(p, blocks, s) : gemv_go<WT, KT, MODE, 1, 16>(p, blocks, s);
      case 2: return gemv_go<WT, KT, MODE, 2, 16>(p, blocks, s);
      case 3: return gemv_go<WT, KT, MODE, 3, 16>(p, blocks, s);
      case 4: return gemv_go<WT, KT, MODE, 4, 16>(p, blocks, s);
    }
  }
  return hipErrorInvalidValue;
}

template <typename WT, typename KT>
static hipError_t gemv_mode(const GemvParams& p, int mode, int blocks, hipStream_t s) {
  switch (mode) {
    case GEMV_QKV: return gemv_rows<WT, KT, GEMV_QKV>(p, blocks, s);
    case GEMV_GATEUP: return gemv_rows<WT, WT, GEMV_GATEUP>(p, blocks, s);
    case GEMV_RESID: return gemv_rows<WT, WT, GEMV_RESID>(p, blocks, s);
    case GEMV_HEAD: return gemv_rows<WT, WT, GEMV_HEAD>(p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvParams& p, int mode, int weight_dtype, int kv_dtype, int blocks, hipStream_t s) {
  if (weight_dtype == 1) {
    return kv_dtype == 1 ? gemv_mode<uint16_t, uint16_t>(p, mode, blocks, s)
                         : gemv_mode<uint16_t, float>(p, mode, blocks, s);
  }
  return kv_dtype == 1 ? gemv_mode<float, uint16_t>(p, mode, blocks, s) : gemv_mode<float, float>(p, mode, blocks, s);
}

template <typename KT, int HD>
static hipError_t attn_g(const AttnParams& p, int rows, hipStream_t s) {
  const int G = p.nq / p.nkv;
  const size_t lds = attn_lds_bytes(p.nq, p.nkv, HD, p.split_len, p.splits);
  dim3 grid(p.splits, p.nkv, rows);
  switch (G) {
#define DS3_CASE(GG)                                      \
  case GG: {                                              \
    auto* f = attn_kernel<KT, HD, GG>;                    \
    hipError_t e = set_lds(f, lds);                       \
    if (e != hipSuccess) return e;                        \
    f<<<grid, kBlock, lds, s>>>(p);                       \
    return hipGetLastError();                             \
  }
    DS3_CASE(1)
    DS3_CASE(2)
    DS3_CASE(4)
    DS3_CASE(8)
#undef DS3_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnParams& p, int kv_dtype, int rows, hipStream_t s) {
  if (kv_dtype == 1) {
    if (p.hd == 64) return attn_g<uint16_t, 64>(p, rows, s);
    if (p.hd == 128) return attn_g<uint16_t, 128>(p, rows, s);
  } else {
    if (p.hd == 64) return attn_g<float, 64>(p, rows, s);
    if (p.hd == 128) return attn_g<float, 128>(p, rows, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kv_copy(const KvView& kv, int kv_dtype, int layer, int row, int pos0, int n, int nkv, int hd,
                          void* staging, int to_state, StatusWords* status, hipStream_t s) {
  const size_t total = 2 * (size_t)nkv * n * hd;
  int blocks = (int)((total + kBlock - 1) / kBlock);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (kv_dtype == 1)
    kv_copy_kernel<uint16_t><<<blocks, kBlock, 0, s>>>(kv, layer, row, pos0, n, nkv, hd,
                                                       reinterpret_cast<uint16_t*>(staging), to_state, status);
  else
    kv_copy_kernel<float><<<blocks, kBlock, 0, s>>>(kv, layer, row, pos0, n, nkv, hd,
                                                    reinterpret_cast<float*>(staging), to_state, status);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t s) {
  int blocks = (int)((n + kBlock - 1) / kBlock);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  fill_u32_kernel<<<blocks, kBlock, 0, s>>>(p, value, n);
  return hipGetLastError();
}

}  // namespace ds3

// Decode-step kernels for MI355X (gfx950, CDNA4, wave64).
//
// The step is memory-bound at small batch ("Execution" page, section "Why capture"): every token streams all
// weights once and sweeps the K/V buffers over the whole capacity. The kernels are therefore built around
// 16-byte per-lane loads of weight rows and K/V rows, with fp32 accumulation, one wave per output-row pair, and
// wave-level shuffle reductions in a fixed order (so a replay reproduces an eager run bit for bit).
//
// Kernel set (one launch each, per layer where noted):
//   embed_kernel      x[r] = E[token[r]]                                      (reads Slot::Token)
//   1-4 rows (vector ALU):
//   gemv_kernel<QKV>  RMSNorm(x) -> q, k, v rows; rotary epilogue on q and k; k and v stored at Slot::Pos
//                     (contiguous) or at Slot::WriteMap (paged)             per layer
//   gemv_kernel<RESID> x += W_o . o, x += W_down . act                      per layer (two launches)
//   gemv_kernel<GATEUP> RMSNorm(x) -> gate/up rows, SwiGLU epilogue -> act  per layer
//   gemv_kernel<HEAD> RMSNorm(x) -> logits, non-finite flag
//   5-16 rows (matrix cores):
//   sk_prep_kernel    x += partial products of the previous projection; RMSNorm sums; fragments of gain * x
//   sk_gemm_kernel    stream-K projection on the fragments -> partial products (LM head: logits)
//   sk_qkv_kernel     q, k, v from the QKV partials; rotary; k and v stored as above      per layer
//   sk_swiglu_kernel  SwiGLU on the gate/up partials -> the down projection's fragments  per layer
//   both:
//   attn_mfma_kernel / attn_kernel  split sweep of all [cap] positions (bf16 K/V on the matrix cores, fp32 on
//                     the vector ALU), mask from Slot::Pos against the position index, per-split softmax partials
//   attn_combine_kernel  the splits merged in fixed order (and, 5-16 rows, the o-projection's fragments)
//   pick_kernel / sample_part_kernel + sample_kernel  the next token into the slots (greedy, or the sampling suffix)
//
// No kernel takes a token, a position or a map entry by value: they are read from the slot buffer, so one
// recorded graph serves every step ("Execution" page, section "Slot buffers").
#include <mutex>

#include "ds3_device.h"

namespace ds3 {


constexpr int kBlock = 256;
constexpr int kUnroll = 8;   // 16-byte loads in flight per lane per weight row
constexpr int kPP = 4;       // long rows: chunks per group, two groups in flight
constexpr int kMaxSplits = 32;          // attention: splits per (row, kv head), merged by the combine kernel
constexpr int kAttnChunk = 128;         // attention: positions staged in LDS per chunk, at most ...
constexpr int kAttnChunkBytes = 32768;  // ... and at most this many bytes of K (and of V)

// 8 values of activation row r from input k0 -> hi/lo fragment words (nt activation tiles)
__device__ __forceinline__ void store_frag8(uint16_t* hi, uint16_t* lo, int nt, int r, int k0, const float (&v)[8]) {
  bf16x8 h, l;
  split_hi_lo8(v, h, l);
  const size_t idx = (((size_t)(k0 >> 5) * nt + (r >> 4)) * 64 + ((k0 >> 3) & 3) * 16 + (r & 15)) * 8;
  *reinterpret_cast<bf16x8*>(hi + idx) = h;
  *reinterpret_cast<bf16x8*>(lo + idx) = l;
}
// the same for 4 inputs k0 .. k0 + 3 (k0 % 4 == 0): one half of the 16-byte fragment word of k0 & ~7, split alike
__device__ __forceinline__ void store_frag4(uint16_t* hi, uint16_t* lo, int nt, int r, int k0, const float (&v)[4]) {
  const uint32_t h0 = cvt_pk_bf16(v[0], v[1]), h1 = cvt_pk_bf16(v[2], v[3]);
  const uint32_t l0 = cvt_pk_bf16(v[0] - __uint_as_float(h0 << 16), v[1] - __uint_as_float(h0 & 0xffff0000u));
  const uint32_t l1 = cvt_pk_bf16(v[2] - __uint_as_float(h1 << 16), v[3] - __uint_as_float(h1 & 0xffff0000u));
  const size_t idx = (((size_t)(k0 >> 5) * nt + (r >> 4)) * 64 + ((k0 >> 3) & 3) * 16 + (r & 15)) * 8 + (k0 & 4);
  *reinterpret_cast<uint2*>(hi + idx) = make_uint2(h0, h1);
  *reinterpret_cast<uint2*>(lo + idx) = make_uint2(l0, l1);
}


// ----------------------------------------------------------------------------------------------------------
// embedding

// grid = (d / (8 * kBlock) rounded up, rows): each thread moves 8 consecutive elements of the row with one
// 16-byte (bf16) or two 16-byte (fp32) loads.
template <typename WT>
__global__ void __launch_bounds__(kBlock) embed_kernel(EmbedParams p) {
  const int r = blockIdx.y;
  SlotLayout sl{p.rows};
  int token = p.slots[sl.token() + r];
  if (token < 0 || token >= p.vocab) {
    if (threadIdx.x == 0 && blockIdx.x == 0) raise_error(p.status, ERR_TOKEN);
    token = 0;
  }
  if (r == 0 && blockIdx.x == 0 && threadIdx.x == 0 && p.slots[sl.inject()] != 0) raise_error(p.status, ERR_INJECTED);
  const int k0 = (blockIdx.x * kBlock + threadIdx.x) * 8;
  if (k0 >= p.d) return;
  const WT* row = reinterpret_cast<const WT*>(p.table) + (size_t)token * p.d + k0;
  float v[8];
  if constexpr (sizeof(WT) == 2) {
    Pack<uint16_t>::widen(*reinterpret_cast<const u32x4*>(row), v);
  } else {
    float a[4], b[4];
    Pack<float>::widen(*reinterpret_cast<const u32x4*>(row), a);
    Pack<float>::widen(*reinterpret_cast<const u32x4*>(row + 4), b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
  float4* dst = reinterpret_cast<float4*>(p.x + (size_t)r * p.d + k0);
  dst[0] = make_float4(v[0], v[1], v[2], v[3]);
  dst[1] = make_float4(v[4], v[5], v[6], v[7]);
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
template <typename WT, int U = kUnroll>
__device__ __forceinline__ void load_group(const WT* w0, const WT* w1, int c0, int nchunks, int K, int lane,
                                           u32x4 (&b0)[U], u32x4 (&b1)[U]) {
  constexpr int EPL = Pack<WT>::N;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = min(min(c0 + u, nchunks - 1) * (64 * EPL) + lane * EPL, K - EPL);
    b0[u] = load_stream(w0 + k);
    b1[u] = load_stream(w1 + k);
  }
}

template <typename WT, int NR, int U = kUnroll>
__device__ __forceinline__ void fma_group(const u32x4 (&b0)[U], const u32x4 (&b1)[U], const float* xs,
                                          int c0, int nchunks, int K, int lane, float (&a0)[NR], float (&a1)[NR]) {
  constexpr int EPL = Pack<WT>::N;
#pragma unroll
  for (int u = 0; u < U; ++u) {
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

// PP (long rows): two groups of kPP chunks in flight per wave (ping-pong buffers), the second issued before the
// first is consumed, so the wave always has loads in flight; groups are half as wide as kUnroll to keep the
// register footprint (and with it two waves per SIMD).
template <typename WT, typename KT, int NR, int MODE, int XREG, bool PP>
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
  constexpr int GU = PP ? kPP : kUnroll;   // chunks per group
  u32x4 b0[GU], b1[GU];
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
  load_group<WT, GU>(w0, w1, 0, nchunks, K, lane, b0, b1);
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

  // ---- 4. pairs. As soon as a pair's dot products have consumed its weights, the next pair's weights (and
  // epilogue operands) are issued, so they are in flight during this pair's reduction and epilogue.
  float na[NR], nb[NR];
  [[maybe_unused]] u32x4 d0[GU], d1[GU];
  for (; pair < p.n_pairs;) {
    float a0[NR], a1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) { a0[r] = 0.f; a1[r] = 0.f; }
    int c_last = 0;   // PP: the group still to be consumed from d after the next pair's loads are out
    if constexpr (PP) {
      int c0 = 0;
      for (; c0 + 2 * GU < nchunks; c0 += 2 * GU) {
        load_group<WT, GU>(w0, w1, c0 + GU, nchunks, K, lane, d0, d1);
        fma_group<WT, NR, GU>(b0, b1, xs, c0, nchunks, K, lane, a0, a1);
        load_group<WT, GU>(w0, w1, c0 + 2 * GU, nchunks, K, lane, b0, b1);
        fma_group<WT, NR, GU>(d0, d1, xs, c0 + GU, nchunks, K, lane, a0, a1);
      }
      // the last one or two groups (a group past the row end is clamped in bounds and masked to zero)
      load_group<WT, GU>(w0, w1, c0 + GU, nchunks, K, lane, d0, d1);
      fma_group<WT, NR, GU>(b0, b1, xs, c0, nchunks, K, lane, a0, a1);
      c_last = c0 + GU;
    } else {
      for (int c0 = 0; c0 < nchunks; c0 += kUnroll) {
        if (c0 > 0) load_group<WT>(w0, w1, c0, nchunks, K, lane, b0, b1);
        fma_group<WT, NR>(b0, b1, xs, c0, nchunks, K, lane, a0, a1);
      }
    }
    const PairMap<MODE> cur = pm;
    const int cur_pair = pair;
#pragma unroll
    for (int r = 0; r < NR; ++r) { na[r] = ea[r]; nb[r] = eb[r]; }
    pair += nwaves;
    if (pair < p.n_pairs) {
      pm = PairMap<MODE>(p, pair);
      w0 = wbase + (size_t)pm.row0 * K;
      w1 = wbase + (size_t)pm.row1 * K;
      load_group<WT, GU>(w0, w1, 0, nchunks, K, lane, b0, b1);
      fetch_epilogue(pm, pair);
    }
    if constexpr (PP) fma_group<WT, NR, GU>(d0, d1, xs, c_last, nchunks, K, lane, a0, a1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      a0[r] = wave_total(a0[r]);
      a1[r] = wave_total(a1[r]);
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
        if (cur.seg != 2) {   // rotate the pair (element idx, element idx + hd/2) by the angle of Slot::Pos
          va = a * na[r] - b * nb[r];
          vb = a * nb[r] + b * na[r];
        }
        if (cur.seg == 0) {
          float* q = p.out + ((size_t)r * p.nq + cur.head) * p.hd;
          q[cur.idx] = va;
          q[cur.idx + half] = vb;
          continue;
        }
        if (!pos_ok[r]) continue;
        int loc = posr[r];
        if (p.kv.paged) {
          loc = p.slots[sl.write_map() + r];
          if (loc < 0 || loc >= p.kv.pool_pages * p.kv.page_size) { raise_error(p.status, ERR_WRITE_MAP); continue; }
        }
        // k: the two halves of a rotary pair; v: two adjacent elements
        KT* base = reinterpret_cast<KT*>(cur.seg == 1 ? p.kv.k : p.kv.v) + (size_t)p.layer * p.kv.layer_stride;
        const bool isv = cur.seg == 2;
        store_kv(base + kv_at(p.kv, isv, r, p.nkv, cur.head, p.hd, loc, cur.idx), va);
        store_kv(base + kv_at(p.kv, isv, r, p.nkv, cur.head, p.hd, loc, cur.idx + (isv ? 1 : half)), vb);
      } else if constexpr (MODE == GEMV_GATEUP) {
        const float silu = a / (1.0f + expf(-a));
        p.out[(size_t)r * p.n_pairs + cur_pair] = silu * b;
      } else if constexpr (MODE == GEMV_RESID) {
        float2* x = reinterpret_cast<float2*>(p.out + (size_t)r * 2 * p.n_pairs) + cur_pair;
        *x = make_float2(na[r] + a, nb[r] + b);
      } else {  // GEMV_HEAD
        float2* lg = reinterpret_cast<float2*>(p.out + (size_t)r * 2 * p.n_pairs) + cur_pair;
        *lg = make_float2(a, b);
        if (!isfinite(a) || !isfinite(b)) atomicOr(&p.status->nonfinite, 1u);
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------------------
// Matrix-core path for 5..16 rows (batched decode, prefill chunks). Each weight element now feeds up to 16
// products, which is matrix work: v_mfma_f32_16x16x32_bf16 multiplies a 16x32 bf16 weight tile by a 32x16 bf16
// activation tile into fp32. The activations are fp32, so they enter as two bf16 parts (hi and the remainder lo,
// about 16 significant bits together): D = W.hi + W.lo. Weights are still read once per step.
//
// The GEMM gives every block (one per CU) an equal run of (quad of four 32-row groups, 128-input chunk) items, so
// a projection with few output rows (o-proj, down) keeps every CU streaming as well as one with many. Wave w takes
// group w of the quad; the four waves walk the chunks in step and share the chunk's activation fragments, which
// they load a quarter each into LDS (as many bytes as the weights when every wave loaded its own: a probe streamed
// 10-17% faster without them). Weight tiles reach LDS through direct global->LDS loads in which each instruction
// covers four whole 256-byte row segments (the 16 lanes of a row read its 16-byte pieces in a swizzled order),
// then move to the matrix cores with ds_read in the operand layout. Loading them straight into registers in the
// operand layout touches sixteen half cache lines per instruction instead of eight whole ones, and streamed at
// half the rate. Three chunks are in flight.
//
// RMSNorm on this path: the fragments carry gain * x, and the row's scale 1/sqrt(mean(x^2) + eps), one factor
// of the whole product, multiplies the sums in the consumer. The sums of squares come from the kernel that wrote
// x, one partial per block and row, added in block order.

constexpr int kSkTileBytes = 16 * kSkChunk * 2;  // one 16-row weight tile of one chunk: 4 KB
constexpr int kSkActTileBytes = kSkChunk / 32 * 2 * 1024;   // a chunk's fragments of one activation tile, hi and lo: 8 KB
constexpr int kSkNt = 2;                         // cache policy of the weight loads: streamed once
// chunk buffers: three of weights (two load while one is consumed); three of activation fragments with one
// activation tile, two with four, whose fragments take four times the LDS (weights 96 KB + activations 24 / 64 KB)
constexpr int kSkBufsW = 3;
template <int NT>
constexpr int kSkBufsA = NT == 1 ? 3 : 2;
constexpr size_t kSkRingBytes = (size_t)kSkWaves * kSkBufsW * 2 * kSkTileBytes;   // weights: 96 KB
template <int NT>
constexpr size_t kSkLds = kSkRingBytes + (size_t)kSkBufsA<NT> * NT * kSkActTileBytes;

// sum of the partial products of weight rows n .. n + 3 (n % 4 == 0) for activation row r, in block order; the
// loads of up to eight contributors are issued before their adds
__device__ __forceinline__ f32x4 sk_sum4(const float* part, const SkPlan& pl, int nt, int n, int r) {
  const int g = n / kSkRows, t = (n >> 4) & 1, lane = 16 * ((n & 15) >> 2) + (r & 15);
  const int a = g / kSkQuad * pl.nck;
  const int nb = pl.block_of(a + pl.nck - 1) - pl.block_of(a) + 1;
  const float* base = part + ((((size_t)g * pl.cmax * nt + (r >> 4)) * 2 + t) * 64 + lane) * 4;
  const size_t stride = (size_t)nt * 512;   // one contributor
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < nb; kb += 8) {
    f32x4 v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      v[c] = kb + c < nb ? *reinterpret_cast<const f32x4*>(base + (size_t)(kb + c) * stride) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (kb + c < nb) s += v[c];
  }
  return s;
}

// RMSNorm row scale from the per-block sums of squares, added in block order
__device__ __forceinline__ float sk_row_scale(const float* ss, int nblk, int r, int D, float eps) {
  float t = 0.f;
#pragma unroll 8
  for (int b = 0; b < nblk; ++b) t += ss[b * kSsRows + r];
  return 1.0f / sqrtf(t / (float)D + eps);
}

// One block per CU, wave w on group w of each quad of the block's run; the waves meet at a barrier per chunk
// (the chunk's activations come from all four). HEAD: whole quads per block, logits out; else partial products.
// NT activation tiles of 16 rows (1: up to 16 rows, 4: up to 64): every weight tile meets each of them.
template <bool HEAD, int NT>
__global__ void __launch_bounds__(64 * kSkWaves) sk_gemm_kernel(SkGemmParams p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char sk_lds[];
  constexpr int B = kSkBufsW;
  constexpr int OPW = 8;                // vector-memory operations per chunk and wave: 8 weight (2 tiles x 4) ...
  constexpr int OPC = OPW + 2 * NT;     // ... and 2 NT activation
  constexpr int ACT = NT * kSkActTileBytes;   // a chunk's activation fragments
  const int lane = threadIdx.x & 63, r16 = lane & 15, hq = lane >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const SkPlan pl = p.plan;
  const int b = blockIdx.x;
  int i0, i1;
  if constexpr (HEAD) {
    i0 = (int)((unsigned)pl.quads() * (unsigned)b / (unsigned)pl.nb) * pl.nck;
    i1 = (int)((unsigned)pl.quads() * (unsigned)(b + 1) / (unsigned)pl.nb) * pl.nck;
  } else {
    i0 = pl.first(b);
    i1 = pl.first(b + 1);
  }
  if (i0 >= i1) return;   // (block-uniform)
  unsigned char* mine = sk_lds + (size_t)wid * B * 2 * kSkTileBytes;
  // activations: [buffer][hi k-steps 0..3 x tiles, lo k-steps 0..3 x tiles][64 lanes][16 B]
  unsigned char* act = sk_lds + kSkRingBytes;
  const int K = p.K, nck = pl.nck;

  // chunk i into buffer bf: the wave's own two weight tiles (tile t's row r lands at byte 256 r, its 16-byte piece
  // c at position c ^ r; instruction j covers rows 4j .. 4j + 3) and its share of the activation fragments
  // (1 KB pieces m = part x 4 NT + k-step x NT + tile, wave w taking pieces 2 NT w .. 2 NT w + 2 NT - 1)
  auto issue_w = [&](int i, int bf) {
    const int q = i / nck, ck = i - q * nck;
    const int g = kSkQuad * q + wid;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* tile = p.w + (size_t)(kSkRows * g + 16 * t) * K + ck * kSkChunk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + hq;
        __builtin_amdgcn_global_load_lds((global_cptr)(tile + (size_t)r * K + 8 * (r16 ^ r)),
                                         (lds_ptr)(mine + (bf * 2 + t) * kSkTileBytes + 1024 * j), 16, 0, kSkNt);
      }
    }
  };
  auto issue_a = [&](int i, int bf) {
    const int ck = i % nck;
#pragma unroll
    for (int m = 2 * NT * wid; m < 2 * NT * wid + 2 * NT; ++m) {
      const int part = m / (4 * NT), st = (m / NT) % 4, ct = m % NT;
      const uint16_t* src = (part == 0 ? p.hi : p.lo) + (((size_t)(ck * 4 + st) * NT + ct) * 64 + lane) * 8;
      __builtin_amdgcn_global_load_lds((global_cptr)src, (lds_ptr)(act + bf * ACT + 1024 * m), 16, 0, 0);
    }
  };
  auto issue = [&](int i, int bf) {
    issue_w(i, bf);
    issue_a(i, bf);
  };

  f32x4 acc0[NT], acc1[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    acc0[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int cur = i0 / nck;
  float scale[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) scale[c] = 1.f;
  if constexpr (HEAD)
#pragma unroll
    for (int c = 0; c < NT; ++c) scale[c] = sk_row_scale(p.ss, p.ss_blocks, 16 * c + r16, p.norm_dim, p.eps);
  auto flush = [&](int q) {
    const int g = kSkQuad * q + wid;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if constexpr (HEAD) {
        const int r = 16 * c + r16;
        if (r < p.rows) {
          const f32x4 a = acc0[c] * scale[c], d = acc1[c] * scale[c];
          float* o = p.out + (size_t)r * p.n_out + kSkRows * g + 4 * hq;
          *reinterpret_cast<f32x4*>(o) = a;
          *reinterpret_cast<f32x4*>(o + 16) = d;
          bool fin = true;
#pragma unroll
          for (int e = 0; e < 4; ++e) fin = fin && isfinite(a[e]) && isfinite(d[e]);
          if (!fin) atomicOr(&p.status->nonfinite, 1u);
        }
      } else {
        const int k = b - pl.block_of(q * nck);
        float* o = p.part + (((((size_t)g * pl.cmax + k) * NT + c) * 2) * 64 + lane) * 4;
        *reinterpret_cast<f32x4*>(o) = acc0[c];
        *reinterpret_cast<f32x4*>(o + 256) = acc1[c];
      }
      acc0[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // chunk i's products from weight buffer qw and activation buffer qa
  auto compute = [&](int i, int qw, int qa) {
    const int qd = i / nck;
    if (qd != cur) {
      flush(cur);
      cur = qd;
    }
    const unsigned char* t0 = mine + (qw * 2) * kSkTileBytes + r16 * 256;
    const unsigned char* av = act + qa * ACT + lane * 16;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int at = 16 * ((4 * st + hq) ^ r16);
      const bf16x8 A0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t0 + at));
      const bf16x8 A1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t0 + kSkTileBytes + at));
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const bf16x8 BH = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(av + 1024 * (st * NT + c)));
        const bf16x8 BL =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(av + 1024 * (4 * NT + st * NT + c)));
        acc0[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, BH, acc0[c], 0, 0, 0);
        acc0[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, BL, acc0[c], 0, 0, 0);
        acc1[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, BH, acc1[c], 0, 0, 0);
        acc1[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, BL, acc1[c], 0, 0, 0);
      }
    }
  };

  if constexpr (kSkBufsA<NT> == B) {   // one ring: chunk i's weights and activations share buffer i mod 3
#pragma unroll
    for (int q = 0; q < B - 1; ++q)
      if (i0 + q < i1) issue(i0 + q, q);
    for (int base = i0; base < i1; base += B) {
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int i = base + q;
        if (i < i1) {
          // chunk i (buffer q) has landed once only the chunks after it are outstanding (loads complete in order;
          // a store issued in between only makes the wait stricter); the barrier makes every wave's share of the
          // activations visible and frees the buffer read in the previous step, which then takes chunk i + B - 1
          if (i + 1 < i1) __builtin_amdgcn_s_waitcnt(kVmcntChunk<OPC>());
          else __builtin_amdgcn_s_waitcnt(kVmcntChunk<0>());
          barrier_lds();
          if (i + B - 1 < i1) issue(i + B - 1, (q + B - 1) % B);
          compute(i, q, q);
        }
      }
    }
  } else {   // weights three deep, activations two: the issue order W(i0), A(i0), W(i0 + 1), then per chunk i
             // A(i + 1), W(i + 2), so chunk i has landed once only W(i + 1) is outstanding
    issue_w(i0, 0);
    issue_a(i0, 0);
    if (i0 + 1 < i1) issue_w(i0 + 1, 1);
    for (int base = i0; base < i1; base += 6) {   // (buffers i mod 3 and i mod 2 repeat every 6 chunks)
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        const int i = base + q;
        if (i < i1) {
          if (i + 1 < i1) __builtin_amdgcn_s_waitcnt(kVmcntChunk<OPW>());
          else __builtin_amdgcn_s_waitcnt(kVmcntChunk<0>());
          barrier_lds();
          if (i + 1 < i1) issue_a(i + 1, (q + 1) % 2);
          if (i + 2 < i1) issue_w(i + 2, (q + 2) % 3);
          compute(i, q % 3, q % 2);
        }
      }
    }
  }
  flush(cur);
}

// grid = (ceil(D / kNormSpan), 16 nt rows), one wave per block, 4 inputs per lane (twice the waves of 8 per lane:
// the partial sums are latency-bound, so more of them in flight at once).
__global__ void __launch_bounds__(64) sk_prep_kernel(SkPrepParams p) {
  const int r = blockIdx.y, lane = threadIdx.x;
  const int k0 = blockIdx.x * kNormSpan + 4 * lane;
  const bool in = k0 < p.D, live = in && r < p.rows;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    float* x = p.x + (size_t)r * p.D + k0;
    float4 a = *reinterpret_cast<const float4*>(x);
    if (p.part) {
      const f32x4 pa = sk_sum4(p.part, p.plan, p.nt, k0, r);
      a.x += pa[0]; a.y += pa[1]; a.z += pa[2]; a.w += pa[3];
      *reinterpret_cast<float4*>(x) = a;
    }
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  float ss = v[0] * v[0] + v[1] * v[1];
  ss += v[2] * v[2] + v[3] * v[3];
  ss = wave_total(ss);
  if (lane == 0) p.ss[blockIdx.x * kSsRows + r] = ss;
  if (!in) return;
  if (live) {
    const float4 ga = *reinterpret_cast<const float4*>(p.gain + k0);
    v[0] *= ga.x; v[1] *= ga.y; v[2] *= ga.z; v[3] *= ga.w;
  }
  store_frag4(p.hi, p.lo, p.nt, r, k0, v);
}

// grid = (ceil(N / 4 / 64), rows), one wave per block (the latency-bound sums then spread over every CU): a lane
// takes output rows n .. n + 3 (n = 4 x index) of activation row r, one partial sum each, and a q or k lane gets its
// rotary partners n +- hd/2 .. + 3 from the lane hd/8 away (a wave holds 256 consecutive outputs: whole heads).
constexpr int kQkvBlock = 64;
template <typename KT>
__global__ void __launch_bounds__(kQkvBlock) sk_qkv_kernel(SkQkvParams p) {
  const int r = blockIdx.y, lane = threadIdx.x & 63;
  const int hd = p.hd, half = hd / 2;
  const int n4 = 4 * (blockIdx.x * kQkvBlock + threadIdx.x);
  if (blockIdx.x * kQkvBlock * 4 >= (p.nq + 2 * p.nkv) * hd) return;   // (wave-uniform: N is whole heads)
  const bool act = n4 < (p.nq + 2 * p.nkv) * hd;
  const int n = act ? n4 : 0;   // (an idle lane's whole head is idle, partner included)
  const int hh = n / hd, idx = n % hd;
  const int seg = hh < p.nq ? 0 : (hh < p.nq + p.nkv ? 1 : 2);   // q, k, v
  const SlotLayout sl{p.rows};
  int pos = p.slots[sl.pos() + r];
  const bool ok = pos >= 0 && pos < p.kv.cap;
  if (!ok) {
    if (act) raise_error(p.status, ERR_POS);
    pos = 0;
  }
  const bool first = idx < half;   // first rotary half of its head
  const int ri = first ? idx : idx - half;
  float2 cs[4];
  if (seg != 2)
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = reinterpret_cast<const float2*>(p.rope)[(size_t)pos * half + ri + e];
  const float sc = sk_row_scale(p.ss, p.ss_blocks, r, p.D, p.eps);
  const f32x4 own = sk_sum4(p.part, p.plan, p.nt, n, r) * sc;
  // the rotary partner's sums, by lane shuffle before any lane leaves
  const int mate = first ? lane + half / 4 : lane - half / 4;
  f32x4 oth;
#pragma unroll
  for (int e = 0; e < 4; ++e) oth[e] = __shfl(own[e], mate, 64);
  if (!act) return;
  int loc = pos;
  if (seg != 0) {
    if (!ok) return;
    if (p.kv.paged) {
      loc = p.slots[sl.write_map() + r];
      if (loc < 0 || loc >= p.kv.pool_pages * p.kv.page_size) {
        raise_error(p.status, ERR_WRITE_MAP);
        return;
      }
    }
  }
  if (seg == 2) {
    const int head = hh - p.nq - p.nkv;
    KT* base = reinterpret_cast<KT*>(p.kv.v) + (size_t)p.layer * p.kv.layer_stride;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_kv(base + kv_at(p.kv, true, r, p.nkv, head, hd, loc, idx + e), own[e]);
    return;
  }
  // (x1, x2) = (first half, second half): x1 c - x2 s for the first, x1 s + x2 c for the second
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x1 = first ? own[e] : oth[e], x2 = first ? oth[e] : own[e];
    v[e] = first ? x1 * cs[e].x - x2 * cs[e].y : x1 * cs[e].y + x2 * cs[e].x;
  }
  if (seg == 0) {
    float* q = p.q + ((size_t)r * p.nq + hh) * hd + idx;
    *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
    return;
  }
  const int head = hh - p.nq;
  KT* base = reinterpret_cast<KT*>(p.kv.k) + (size_t)p.layer * p.kv.layer_stride;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_kv(base + kv_at(p.kv, false, r, p.nkv, head, hd, loc, idx + e), v[e]);
}

// grid = (ceil(F / kActSpan), 16 nt rows), one wave per block: silu(gate) * up of 4 consecutive j per lane ->
// fragments (4 per lane, not 8: twice the waves for the latency-bound partial sums).
__global__ void __launch_bounds__(64) sk_swiglu_kernel(SkActParams p) {
  const int r = blockIdx.y;
  const int j0 = blockIdx.x * kActSpan + 4 * threadIdx.x;
  if (j0 >= p.F) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (r < p.rows) {
    const float sc = sk_row_scale(p.ss, p.ss_blocks, r, p.D, p.eps);
    const f32x4 g = sk_sum4(p.part, p.plan, p.nt, j0, r) * sc;
    const f32x4 u = sk_sum4(p.part, p.plan, p.nt, p.F + j0, r) * sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = g[e] / (1.0f + expf(-g[e])) * u[e];
  }
  store_frag4(p.hi, p.lo, p.nt, r, j0, v);
}

// ----------------------------------------------------------------------------------------------------------
// Attention: split sweep over the whole [cap] of one (row, kv head), all G query heads of the group at once.
//
// grid = (splits, nkv, rows); block = 256 threads; each block owns T positions of one kv head and walks them in
// LDS chunks of TC positions (128, or 32 KB of K if that is fewer), two chunk buffers deep. A chunk's K and V
// rows are staged in LDS with direct global-to-LDS 16-byte loads (no registers involved, so every load of the chunk is in flight at once), then
// one wait and one barrier. From LDS, LPP lanes share one position (16 bytes of the head each): the G scores of
// a position are reduced over those lanes by a butterfly (bit-identical sums in every lane) and folded into a
// running softmax state per lane group: max m, sum l, weighted value sum o (online softmax, one rescale per UA
// positions).
//
// Masking (Slot::Pos against the position index, positions after pos hidden) is done by selection: a hidden
// position's score is -inf and its value row never reaches the accumulator, so whatever the buffer holds after
// pos -- stale data, inf, NaN -- cannot leak into the result.
//
// Merges, all in a fixed order: lane groups of a wave by butterfly, the 4 waves through LDS in wave order, and
// the splits of a (row, q head) by attn_combine_kernel in split order: o = sum_s e^(m_s - M) o_s /
// sum_s e^(m_s - M) l_s with M = max_s m_s. (Merging inside the attention kernel, by the block of a row and kv
// head that finishes last, measured 8-13% slower per 8-row step than the separate merge kernel.)


// The end of an attention block: `wst` holds each wave's state [4 waves][G][HD + 2] (weighted value sums, then the
// running max and the weight sum, maxima in the log2 domain). The 4 waves are merged in wave order into this
// split's partial, stored with plain coalesced stores at part[row][kv head][split][G][HD + 2]; the combine kernel
// that follows merges the splits (the kernel boundary makes the partials visible to every XCD). A plan of one split
// (a 64-token prefill chunk: one block per row and kv head) has nothing to merge: the block writes the normalized
// output, and the o-projection's fragments, itself -- the values the combine would form from its one split
// (weight 2^0 = 1 and the split's own sum).
template <int G, int HD>
__device__ __forceinline__ void attn_write_partial(const AttnParams& p, const float* wst, int r, int g, int s) {
  if (p.splits == 1) {
    for (int i = threadIdx.x; i < G * HD / 8; i += kBlock) {
      const int hh = i / (HD / 8), d0 = i % (HD / 8) * 8;
      float mm = wst[hh * (HD + 2) + HD];
      float ll = wst[hh * (HD + 2) + HD + 1];
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = wst[hh * (HD + 2) + d0 + e];
#pragma unroll
      for (int w = 1; w < kBlock / 64; ++w) {
        const float* ws2 = wst + (w * G + hh) * (HD + 2);
        float M, w1, w2;
        Lse::weights(mm, ws2[HD], M, w1, w2);
        ll = ll * w1 + ws2[HD + 1] * w2;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * w1 + ws2[d0 + e] * w2;
        mm = M;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] / ll;
      const int h = g * G + hh;
      float* o = p.out + ((size_t)r * p.nq + h) * HD + d0;
      *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      if (p.frag_hi) store_frag8(p.frag_hi, p.frag_lo, p.nt, r, h * HD + d0, v);
    }
    return;
  }
  float* part = p.part + (((size_t)r * p.nkv + g) * p.splits + s) * (size_t)(G * (HD + 2));
  for (int i = threadIdx.x; i < G * (HD + 2); i += kBlock) {
    const int hh = i / (HD + 2), dd = i % (HD + 2);
    float mm = wst[(0 * G + hh) * (HD + 2) + HD];
    float ll = wst[(0 * G + hh) * (HD + 2) + HD + 1];
    float oo = wst[(0 * G + hh) * (HD + 2) + min(dd, HD - 1)];
#pragma unroll
    for (int w = 1; w < kBlock / 64; ++w) {
      const float* ws2 = wst + (w * G + hh) * (HD + 2);
      float M, w1, w2;
      Lse::weights(mm, ws2[HD], M, w1, w2);
      ll = ll * w1 + ws2[HD + 1] * w2;
      oo = oo * w1 + ws2[min(dd, HD - 1)] * w2;
      mm = M;
    }
    part[i] = dd < HD ? oo : (dd == HD ? mm : ll);
  }
}

// Merge of the splits of one (row, q head): grid (nq, rows), HD threads, thread d owns output element d.
// o[d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s with M = max_s m_s (a split that saw no visible position
// has m_s = -inf and weight 0). Lane s of each wave loads split s's max and weight sum, so every load of the
// kernel is a vector load issued up front (uniform addresses would become serialized scalar loads); the weights
// reach every lane by readlane, and the value sum runs in split order.
// NS: the plan's splits rounded up to 4, 8, 16 or 32 (the loads and the weighted sum run over NS, not kMaxSplits).
template <int G, int HD, int NS>
__global__ void __launch_bounds__(128) attn_combine_kernel(AttnParams p) {
  const int h = blockIdx.x, r = blockIdx.y, d = threadIdx.x, lane = d & 63;
  const int g = h / G, hh = h % G, S = p.splits;
  const size_t stride = (size_t)G * (HD + 2);   // between consecutive splits
  const float* part = p.part + ((size_t)r * p.nkv + g) * S * stride + (size_t)hh * (HD + 2);
  const int sl = min(lane, S - 1);
  const float ms = part[(size_t)sl * stride + HD];
  const float ls = part[(size_t)sl * stride + HD + 1];
  float ov[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) ov[k] = part[(size_t)min(k, S - 1) * stride + d];
  const float M = wave_max(lane < S ? ms : -INFINITY);
  const float w = (lane < S && ms != -INFINITY) ? fast_exp2(ms - M) : 0.f;
  const float L = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum(w * (lane < S ? ls : 0.f))), 0));
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));   // 0 for k >= S
    acc = fmaf(wk, k < S ? ov[k] : 0.f, acc);   // a padded split adds an exact zero, never 0 * garbage
  }
  const float o = acc / L;
  p.out[((size_t)r * p.nq + h) * HD + d] = o;
  if (p.frag_hi) {   // lanes d .. d + 7 (one wave) -> lane d's 8 values -> the fragment words
    float v[8];
    v[0] = o;
#pragma unroll
    for (int k = 1; k < 8; ++k) v[k] = __shfl_down(o, k, 64);
    if ((d & 7) == 0) store_frag8(p.frag_hi, p.frag_lo, p.nt, r, h * HD + d, v);
  }
}

template <typename KT, int HD, int G, bool PAGED>
__global__ void __launch_bounds__(kBlock) attn_kernel(AttnParams p) {
  constexpr int EPL = Pack<KT>::N;               // elements per 16 bytes
  constexpr int LPP = HD / EPL;                  // lanes per position
  constexpr int PPP = kBlock / LPP;              // positions per block pass
  constexpr int PB = HD * (int)sizeof(KT);       // bytes per position
  constexpr int TC = kAttnChunkBytes / PB < kAttnChunk ? kAttnChunkBytes / PB : kAttnChunk;   // positions per chunk
  constexpr int NI = TC * PB / 1024;             // 1 KB global-to-LDS instructions per chunk and per K or V
  constexpr int UA = G >= 4 ? 4 : 8;             // positions per lane group per softmax rescale
  static_assert(LPP >= 1 && LPP <= 64 && (64 % LPP) == 0, "lanes per position must divide the wave");
  static_assert(NI % (kBlock / 64) == 0 && TC % PPP == 0, "chunk must split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NBUF = 2;
  float* wst = reinterpret_cast<float*>(smem + (size_t)NBUF * 2 * TC * PB);   // [4 waves][G][HD + 2]
  int* ptab = reinterpret_cast<int*>(wst + 4 * G * (HD + 2));                 // paged: pool page per chunk page

  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int rows = gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sub = tid % LPP, grp = tid / LPP;
  const int T = p.split_len;
  // Chunks of the capacity go to splits round-robin (split s takes chunks s, s + S, s + 2S, ...), so the visible
  // positions 0..pos, and with them the arithmetic, spread over all splits; the merge does not depend on which
  // positions a split holds.
  const int S = p.splits;
  auto chunk_base = [&](int c0) { return (s + (c0 / TC) * S) * TC; };
  const int cap = p.kv.cap;
  const SlotLayout sl{rows};

  int pos = p.slots[sl.pos() + r];
  if (pos < 0 || pos >= cap) {
    if (tid == 0) raise_error(p.status, ERR_POS);
    pos = 0;
  }
  // visible-sweep slot set: chunks wholly after pos (a suffix of this split's chunks) are not loaded
  const bool vis_only = p.slots[sl.sweep()] != 0;
  auto live = [&](int c0) { return !vis_only || chunk_base(c0) <= pos; };
  const int kr = kv_row(p.kv, r);   // this row's K/V row
  const KT* Kb = reinterpret_cast<const KT*>(p.kv.k) + (size_t)p.layer * p.kv.layer_stride;
  const KT* Vb = reinterpret_cast<const KT*>(p.kv.v) + (size_t)p.layer * p.kv.layer_stride;
  const float scale2 = p.scale * 1.4426950408889634f;   // 1/sqrt(hd) * log2(e)

  // the query heads of this kv head (these loads go first: loads return in order)
  float qv[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[hh][e] = p.q[((size_t)r * p.nq + g * G + hh) * HD + sub * EPL + e];

  // ---- paged: the pool pages of every chunk this split sweeps go to LDS first, so staging a chunk needs no
  // ordinary global load (which would have to wait behind the previous chunk's rows). Entry (chunk c, q) is the
  // q-th logical page the chunk covers, clamped to the row's last page; an id outside the pool raises the error
  // word and reads page 0 instead.
  const int ps = PAGED ? p.kv.page_size : 1;
  const int psl = __builtin_ctz((unsigned)ps);            // page sizes are powers of two
  const int ppc = PAGED ? (ps <= TC ? TC / ps : 1) : 1;   // pages per chunk
  if constexpr (PAGED) {
    const int ppr = cap / ps;
    const int n = ((T + TC - 1) / TC) * ppc;
    for (int i = tid; i < n; i += kBlock) {
      const int lp = min(chunk_base((i / ppc) * TC) / ps + i % ppc, ppr - 1);
      int page = p.kv.slot_map[kr * ppr + lp];
      if (page < 0 || page >= p.kv.pool_pages) {
        raise_error(p.status, ERR_PAGE);
        page = 0;
      }
      ptab[i] = page;
    }
    __syncthreads();
  }

  // ---- stage a chunk's K and V rows into LDS buffer `buf`: instruction k of the block fills bytes
  // [k KB, k KB + 1 KB) of the buffer's K half and of its V half
  auto stage = [&](int c0, int buf) {
    unsigned char* kdst = smem + (size_t)buf * 2 * TC * PB;
    unsigned char* vdst = kdst + (size_t)TC * PB;
#pragma unroll
    for (int i = 0; i < NI / (kBlock / 64); ++i) {
      const int k = i * (kBlock / 64) + wid;
      const int byte = k * 1024 + lane * 16;
      const int tc = byte / PB;                           // position within the chunk
      const int jc = min(chunk_base(c0) + tc, cap - 1);   // past the capacity: clamped, never visible
      uint32_t off;
      if constexpr (PAGED) {
        const int jb = chunk_base(c0);
        const int q = min(max((jc >> psl) - (jb >> psl), 0), ppc - 1);
        const int page = ptab[(c0 / TC) * ppc + q];
        off = (uint32_t)(((page * p.nkv + g) * ps + (jc & (ps - 1))) * HD);
      } else {
        off = (uint32_t)(((kr * p.nkv + g) * cap + jc) * HD);
      }
      const int el = (byte % PB) / (int)sizeof(KT);
      __builtin_amdgcn_global_load_lds((global_cptr)(Kb + off + el), (lds_ptr)(kdst + (size_t)k * 1024), 16, 0, 2);
      __builtin_amdgcn_global_load_lds((global_cptr)(Vb + off + el), (lds_ptr)(vdst + (size_t)k * 1024), 16, 0, 2);
    }
  };
  // Both buffers are filled up front; afterwards a buffer is refilled as soon as its chunk has been consumed.
  if (live(0)) stage(0, 0);
  if (TC < T && live(TC)) stage(TC, 1);

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  }

  for (int c0 = 0, buf = 0; c0 < T && live(c0); c0 += TC, buf = (buf + 1) % NBUF) {
    // wait for this chunk's rows only: a later chunk's rows (NI/4 K and NI/4 V loads per wave) may still fly
    if (c0 + TC < T && live(c0 + TC)) __builtin_amdgcn_s_waitcnt(kVmcntChunk<NI / (kBlock / 64) * 2>());
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const KT* ks = reinterpret_cast<const KT*>(smem + (size_t)buf * 2 * TC * PB);
    const KT* vs = ks + (size_t)TC * HD;
    // a chunk entirely after pos is swept (its rows were loaded) but holds no visible position: no arithmetic
    const int jb = chunk_base(c0);
    if (jb <= pos) {
    // ---- scores and online softmax from LDS. Scores are kept in the log2 domain (q.k * scale * log2 e), so the
    // weights are plain exp2: the same softmax, one hardware exp per weight.
    for (int tb = grp; tb < TC; tb += PPP * UA) {
      float sc[UA][G];
      bool vis[UA];
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int tc = min(tb + u * PPP, TC - 1);
        vis[u] = tb + u * PPP < TC && jb + tb + u * PPP <= pos;
        float kf[EPL];
        Pack<KT>::widen(*reinterpret_cast<const u32x4*>(ks + (size_t)tc * HD + sub * EPL), kf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc = fmaf(qv[hh][e], kf[e], acc);
          acc = group_sum<LPP>(acc);
          sc[u][hh] = vis[u] ? acc * scale2 : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float bm = sc[0][hh];
#pragma unroll
        for (int u = 1; u < UA; ++u) bm = fmaxf(bm, sc[u][hh]);
        const float mn = fmaxf(m[hh], bm);
        const float corr = (mn == -INFINITY) ? 1.f : fast_exp2(m[hh] - mn);
        l[hh] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] *= corr;
        m[hh] = mn;
      }
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int tc = min(tb + u * PPP, TC - 1);
        float vf[EPL];
        Pack<KT>::widen(*reinterpret_cast<const u32x4*>(vs + (size_t)tc * HD + sub * EPL), vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = vis[u] ? vf[e] : 0.f;   // a hidden row never reaches o (no 0 * NaN)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pu = vis[u] ? fast_exp2(sc[u][hh] - m[hh]) : 0.f;
          l[hh] += pu;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(pu, vf[e], o[hh][e]);
        }
      }
    }
    }
    __syncthreads();   // the buffer is refilled next
    if (c0 + NBUF * TC < T && live(c0 + NBUF * TC)) stage(c0 + NBUF * TC, buf);
  }

  // ---- merge the lane groups of the wave (butterfly over the lanes holding the same head elements)
#pragma unroll
  for (int msk = LPP; msk < 64; msk <<= 1) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float m2 = __shfl_xor(m[hh], msk, 64);
      const float l2 = __shfl_xor(l[hh], msk, 64);
      float M, w1, w2;
      Lse::weights(m[hh], m2, M, w1, w2);
      l[hh] = l[hh] * w1 + l2 * w2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[hh][e], msk, 64);
        o[hh][e] = o[hh][e] * w1 + o2 * w2;
      }
      m[hh] = M;
    }
  }
  if (lane < LPP) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float* w = wst + (wid * G + hh) * (HD + 2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) w[sub * EPL + e] = o[hh][e];
      if (sub == 0) {
        w[HD] = m[hh];
        w[HD + 1] = l[hh];
      }
    }
  }
  __syncthreads();

  attn_write_partial<G, HD>(p, wst, r, g, s);
}

// ----------------------------------------------------------------------------------------------------------
// Matrix-core attention (bf16 K/V): the same split sweep, mask and merge as attn_kernel, with both products on
// v_mfma_f32_16x16x32_bf16. Wave w of the block takes positions [32w, 32w + 32) of every 128-position chunk.
//
//   scores  S[position][head] = K[position][:] . q[head][:]  -- A = 16 K rows (from LDS), B = q^T (registers; the
//           G heads of the group in columns 0..G-1, the rest zero), two 16-position tiles per wave;
//   values  O[head][d] += P[head][position] V[position][d]   -- A = the softmax weights P, B = 16 d-columns of V
//           (from the transposed V chunk in LDS), one 32-position k-step per wave.
//
// Tile t's rows are positions 8(m/4) + 4t + m%4 (m = row), so the score tile lands with lane (n, L) = (l%16, l/16)
// holding head n at positions 8L..8L+7 of the wave's 32 -- exactly where the value product's A operand wants them:
// no data moves between the two products. q and P enter as bf16 hi and lo parts (q: ~16 significant bits; P in
// [0, 1]), K and V are bf16 already.
//
// LDS pieces are swizzled so that the 16 rows (or d-columns) one operand read touches fall in distinct banks:
// K piece c of position pj sits at pj * HD/8 + (c ^ key(pj)); V^T group cv (8 positions) of element d at
// d * 16 + (cv ^ (d % 16)). The global-to-LDS loads write the slots in order and pick the source per lane.
//
// Positions after pos: a score is selected to -inf and its weight to 0; in the one 32-position block per wave
// that straddles pos, the hidden V rows are zeroed in the operand (an MFMA would turn 0 * NaN into NaN).


template <int HD, int G, bool PAGED>
__global__ void __launch_bounds__(kBlock) attn_mfma_kernel(AttnParams p) {
  constexpr int TC = kAttnChunk;             // positions per chunk: 4 waves x 32
  constexpr int CPR = HD / 8;                // 16-byte pieces per K row
  constexpr int KB = TC * HD * 2;            // bytes of K, and of V^T, per chunk
  constexpr int NIW = KB / 1024 / 4;         // 1 KB global-to-LDS instructions per wave, per K or V
  constexpr int KS = HD / 32;                // k-steps of the score product
  constexpr int DT = HD / 16;                // d tiles of the value product
  static_assert(TC == 128 && G >= 1 && G <= 16 && (HD == 64 || HD == 128), "shape");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // chunk buffers: two (a block streams chunk c + 1 while it sweeps chunk c), or with paged K/V one, so that two
  // blocks share a CU and each sweeps while the other loads (measured 0.8% faster paged, 3.6% slower contiguous)
  constexpr int NB = PAGED ? 1 : 2;
  float* wst = reinterpret_cast<float*>(smem + NB * 2 * KB);   // [4 waves][G][HD + 2]
  int* ptab = reinterpret_cast<int*>(wst + 4 * G * (HD + 2));  // paged: pool page per chunk page

  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int rows = gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, L = lane >> 4;
  const int T = p.split_len, S = p.splits, cap = p.kv.cap, nkv = p.nkv;
  auto chunk_base = [&](int c0) { return (s + (c0 / TC) * S) * TC; };   // round-robin chunks, as attn_kernel
  const SlotLayout sl{rows};
  int pos = p.slots[sl.pos() + r];
  if (pos < 0 || pos >= cap) {
    if (tid == 0) raise_error(p.status, ERR_POS);
    pos = 0;
  }
  // the method sweeps every chunk; with the visible-sweep slot set, chunks wholly after pos (a suffix of this
  // split's chunks) are neither loaded nor computed
  const bool vis_only = p.slots[sl.sweep()] != 0;
  auto live = [&](int c0) { return !vis_only || chunk_base(c0) <= pos; };
  const int kr = kv_row(p.kv, r);   // this row's K/V row
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(p.kv.k) + (size_t)p.layer * p.kv.layer_stride;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(p.kv.v) + (size_t)p.layer * p.kv.layer_stride;
  const float scale2 = p.scale * 1.4426950408889634f;   // 1/sqrt(hd) * log2(e): scores in the log2 domain

  // ---- q loads first (loads return in order); they are turned into operands only after the K/V staging has
  // been issued, so the sweep's loads do not wait behind them
  float4 qa[KS], qb[KS];
  {
    const float* qrow = p.q + ((size_t)r * p.nq + g * G + min(n, G - 1)) * HD + 8 * L;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qa[k] = *reinterpret_cast<const float4*>(qrow + 32 * k);
      qb[k] = *reinterpret_cast<const float4*>(qrow + 32 * k + 4);
    }
  }

  // ---- paged: the pool pages of every chunk of this split go to LDS first (as in attn_kernel)
  const int ps = PAGED ? p.kv.page_size : 1;
  const int psl = __builtin_ctz((unsigned)ps);            // page sizes are powers of two
  const int ppc = PAGED ? (ps <= TC ? TC / ps : 1) : 1;
  if constexpr (PAGED) {
    const int ppr = cap / ps;
    const int nt = ((T + TC - 1) / TC) * ppc;
    for (int i = tid; i < nt; i += kBlock) {
      const int lp = min(chunk_base((i / ppc) * TC) / ps + i % ppc, ppr - 1);
      int page = p.kv.slot_map[kr * ppr + lp];
      if (page < 0 || page >= p.kv.pool_pages) {
        raise_error(p.status, ERR_PAGE);
        page = 0;
      }
      ptab[i] = page;
    }
    __syncthreads();
  }

  // ---- stage chunk c0 into buffer buf: instruction k of the block fills 16-byte slots [64k, 64k + 64) of the
  // K half and of the V^T half; each lane picks the source of its slot (swizzled layouts above)
  auto stage = [&](int c0, int buf) {
    unsigned char* kdst = smem + (size_t)buf * 2 * KB;
    unsigned char* vdst = kdst + KB;
    const int jb = chunk_base(c0);
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int k = i * 4 + wid;
      const int slot = k * 64 + lane;
      const int pj = slot / CPR;                          // K: position in the chunk and piece
      const int c = (slot % CPR) ^ kswz<CPR>(pj);
      const int jk = min(jb + pj, cap - 1);               // past the capacity: clamped, never visible
      const int d = slot / (TC / 8);                      // V^T: element and 8-position group
      const int cv = (slot % (TC / 8)) ^ (d & 15);
      const int jv = min(jb + 8 * cv, cap - 8);
      uint32_t koff, voff;
      if constexpr (PAGED) {
        const int q0 = (c0 / TC) * ppc;
        const int pk = ptab[q0 + min(max((jk >> psl) - (jb >> psl), 0), ppc - 1)];
        const int pv = ptab[q0 + min(max((jv >> psl) - (jb >> psl), 0), ppc - 1)];
        koff = (uint32_t)(((pk * nkv + g) * ps + (jk & (ps - 1))) * HD + 8 * c);
        voff = (uint32_t)(((pv * nkv + g) * HD + d) * ps + (jv & (ps - 1)));
      } else {
        koff = (uint32_t)(((kr * nkv + g) * cap + jk) * HD + 8 * c);
        voff = (uint32_t)(((kr * nkv + g) * HD + d) * cap + jv);
      }
      __builtin_amdgcn_global_load_lds((global_cptr)(Kb + koff), (lds_ptr)(kdst + (size_t)k * 1024), 16, 0, 2);
      __builtin_amdgcn_global_load_lds((global_cptr)(Vb + voff), (lds_ptr)(vdst + (size_t)k * 1024), 16, 0, 2);
    }
  };
  if (live(0)) stage(0, 0);
  if (NB == 2 && TC < T && live(TC)) stage(TC, 1);

  // ---- q^T as B operand: lane (n, L) holds q[head n][32 ks + 8 L + e] * scale2, e = 0..7 (zero for n >= G)
  bf16x8 qh[KS], ql[KS];
  {
    const float z = n < G ? scale2 : 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const float v[8] = {qa[k].x * z, qa[k].y * z, qa[k].z * z, qa[k].w * z,
                          qb[k].x * z, qb[k].y * z, qb[k].z * z, qb[k].w * z};
      split_hi_lo8(v, qh[k], ql[k]);
    }
  }

  float m_run = -INFINITY;   // running max of head n (log2 domain), equal in the 4 lane groups
  float lsum = 0.f;          // this lane's share of head n's weight sum
  f32x4 acc[DT];             // O[head 4L + i][16 dt + n]
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0, buf = 0; c0 < T && live(c0); c0 += TC, buf = NB == 2 ? buf ^ 1 : 0) {
    if (NB == 2 && c0 + TC < T && live(c0 + TC)) __builtin_amdgcn_s_waitcnt(kVmcntChunk<2 * NIW>());
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int jw = chunk_base(c0) + 32 * wid;   // first position of this wave's block
    if (jw <= pos) {                            // a block wholly after pos holds nothing visible
      const uint16_t* kl = reinterpret_cast<const uint16_t*>(smem + (size_t)buf * 2 * KB);
      const uint16_t* vl = kl + KB / 2;
      f32x4 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int pj = 32 * wid + 8 * (n >> 2) + 4 * t + (n & 3);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const int c = 4 * k + L;
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kl + (size_t)(pj * CPR + (c ^ kswz<CPR>(pj))) * 8));
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[k], sc[t], 0, 0, 0);
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[k], sc[t], 0, 0, 0);
        }
      }
      // lane (n, L): scores of head n at positions jw + 8L + e, e = 4t + i
      float sv[8];
      bool vis[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vis[e] = jw + 8 * L + e <= pos;
        sv[e] = vis[e] ? sc[e >> 2][e & 3] : -INFINITY;
      }
      float bm = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sv[e]);
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float mn = fmaxf(m_run, bm);
      const float corr = (mn == -INFINITY) ? 1.f : fast_exp2(m_run - mn);
      m_run = mn;
      float pw[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pw[e] = vis[e] ? fast_exp2(sv[e] - mn) : 0.f;
        psum += pw[e];
      }
      lsum = lsum * corr + psum;
      bf16x8 ph, pl;
      split_hi_lo8(pw, ph, pl);
      // rescale the value sums: element i of acc[] belongs to head 4L + i, whose factor lane 4L + i holds
      float cr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cr[i] = __shfl(corr, 4 * L + i, 64);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dt][i] *= cr[i];
      const bool partial = jw + 31 > pos;
      uint32_t mk[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
        mk[q2] = (jw + 8 * L + 2 * q2 <= pos ? 0xFFFFu : 0u) | (jw + 8 * L + 2 * q2 + 1 <= pos ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + n;
        u32x4 b = *reinterpret_cast<const u32x4*>(vl + (size_t)(d * 16 + ((4 * wid + L) ^ (d & 15))) * 8);
        if (partial) {
          b.x &= mk[0];
          b.y &= mk[1];
          b.z &= mk[2];
          b.w &= mk[3];
        }
        const bf16x8 B = __builtin_bit_cast(bf16x8, b);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, B, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, B, acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();   // the buffer is refilled next
    if (c0 + NB * TC < T && live(c0 + NB * TC)) stage(c0 + NB * TC, buf);
  }

  // ---- this wave's state into LDS: the 4 lane groups of a head share its max; their weight sums add
  float lt = lsum + __shfl_xor(lsum, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * L + i;
    if (hh < G) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) wst[(wid * G + hh) * (HD + 2) + 16 * dt + n] = acc[dt][i];
    }
  }
  if (L == 0 && n < G) {
    wst[(wid * G + n) * (HD + 2) + HD] = m_run;
    wst[(wid * G + n) * (HD + 2) + HD + 1] = lt;
  }
  __syncthreads();
  attn_write_partial<G, HD>(p, wst, r, g, s);
}

// ----------------------------------------------------------------------------------------------------------
// Streaming-read probe (measurement only, not part of a step): what plain reading reaches on this GPU, beside the
// roofline's 8 TB/s. Every wave reads 8 KB per step (eight 1 KB contiguous instructions, non-temporal) over a
// wave-strided sweep of the buffer.
constexpr int kProbeBlocks = 1024;
__global__ void __launch_bounds__(512) stream_read_kernel(const u32x4* __restrict__ buf, size_t n16, uint32_t* sink) {
  const size_t lane = threadIdx.x & 63;
  const size_t gw = (size_t)blockIdx.x * 8 + (threadIdx.x >> 6), nw = (size_t)gridDim.x * 8;
  uint32_t acc = 0;
  for (size_t base = gw * 512; base < n16; base += nw * 512) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t i = base + (size_t)u * 64 + lane;
      v[u] = i < n16 ? load_stream(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // a store the compiler cannot drop keeps every load (the data practically never hashes to this value)
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// ----------------------------------------------------------------------------------------------------------
// K/V state copies for write_kv / read_kv: staging <-> state (contiguous or paged). The staging holds K as
// [nkv][n][hd] and V as [nkv][n][hd], or as [nkv][hd][n] when V is stored transposed, so that consecutive
// threads touch consecutive elements of the state in either layout.

template <typename KT>
__global__ void __launch_bounds__(kBlock) kv_copy_kernel(KvView kv, int layer, int row, int pos0, int n, int nkv,
                                                          int hd, KT* staging, int to_state, int stage_vt,
                                                          StatusWords* st) {
  const size_t per = (size_t)n * hd;
  const size_t total = 2 * (size_t)nkv * per;   // K then V
  for (size_t i = blockIdx.x * (size_t)kBlock + threadIdx.x; i < total; i += (size_t)gridDim.x * kBlock) {
    const int which = (int)(i / (nkv * per));
    const size_t rem = i % (nkv * per);
    const int g = (int)(rem / per);
    const bool t = which == 1 && stage_vt;   // staged V order: [nkv][hd][n] when set, else [nkv][n][hd]
    const int pos = t ? (int)(rem % n) : (int)((rem / hd) % n);
    const int e = t ? (int)((rem / n) % hd) : (int)(rem % hd);
    KT* base = reinterpret_cast<KT*>(which ? kv.v : kv.k) + (size_t)layer * kv.layer_stride;
    KT* dst = base + kv_at(kv, which == 1, row, nkv, g, hd, kv_loc(kv, row, pos0 + pos, st), e);
    if (to_state) *dst = staging[i];
    else staging[i] = *dst;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// ----------------------------------------------------------------------------------------------------------
// greedy pick

constexpr int kPickThreads = 256;

__global__ void __launch_bounds__(kPickThreads) pick_kernel(PickParams p) {
  __shared__ float s_v[kPickThreads / 64];
  __shared__ int s_i[kPickThreads / 64];
  __shared__ int s_last;
  const int r = blockIdx.x / kPickSplit, part = blockIdx.x % kPickSplit;
  const int chunk = (p.vocab + kPickSplit - 1) / kPickSplit;
  const int lo = part * chunk, hi = min(p.vocab, lo + chunk);
  const float* lg = p.logits + (size_t)r * p.vocab;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // eight loads in flight per thread before any comparison (the maximum does not depend on the order)
  for (int i0 = lo + (int)threadIdx.x; i0 < hi; i0 += 8 * kPickThreads) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i0 + u * kPickThreads < hi ? lg[i0 + u * kPickThreads] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kPickThreads;
      if (i < hi && pick_better(v[u], i, bv, bi)) { bv = v[u]; bi = i; }
    }
  }
  // wave, then block: the order-independent (value, index) maximum
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (pick_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) { s_v[wv] = bv; s_i[wv] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kPickThreads / 64; ++w)
      if (pick_better(s_v[w], s_i[w], bv, bi)) { bv = s_v[w]; bi = s_i[w]; }
    __hip_atomic_store(&p.part_val[blockIdx.x], bv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.part_idx[blockIdx.x], bi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // release this block's slice result; the last block to arrive acquires everyone's
    const unsigned prev = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  const SlotLayout sl{p.rows};
  if (threadIdx.x < p.rows) {
    const int rr = threadIdx.x;
    float v = -INFINITY;
    int idx = 0x7fffffff;
    for (int k = 0; k < kPickSplit; ++k) {
      const float ov = __hip_atomic_load(&p.part_val[rr * kPickSplit + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int oi = __hip_atomic_load(&p.part_idx[rr * kPickSplit + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (pick_better(ov, oi, v, idx)) { v = ov; idx = oi; }
    }
    if (idx >= p.vocab) idx = 0;   // every logit NaN
    const int step = p.slots[sl.chain()];
    p.ids[(size_t)(step % p.max_chain) * p.rows + rr] = idx;
    const int np = p.slots[sl.pos() + rr] + 1;
    p.slots[sl.token() + rr] = idx;
    p.slots[sl.pos() + rr] = np;
    if (p.page_table && np >= 0 && np < p.cap) {
      const int ppr = p.cap / p.page_size;
      p.slots[sl.write_map() + rr] = p.page_table[(size_t)rr * ppr + np / p.page_size] * p.page_size + np % p.page_size;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int step = p.slots[sl.chain()];
    p.flags[step % p.max_chain] = p.status->nonfinite ? 1u : 0u;
    p.status->nonfinite = 0;
    p.slots[sl.chain()] = step + 1;
    __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ----------------------------------------------------------------------------------------------------------
// sampling suffix: the segment kernel (sample_part_kernel, one block per 2048-token segment of a row) forms the
// adjusted logits and the segment records; then one block of kSampleThreads per row selects: from the candidates
// (the segments' top-k sets) when top-k is small, else by several passes over the row's adjusted logits
// (L2-resident)

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;

// float -> uint32 key in the same order (NaN never reaches here)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// SplitMix64 output d from state `seed` (Steele, Lea and Flood 2014): the state advances by the golden gamma before
// each output; an output is the state through two xor-shift-multiply rounds and a final xor-shift
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t d) {
  uint64_t z = seed + (d + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

constexpr int kSampleList = 1024;   // top-k sets up to this size are gathered into LDS for the rest of the selection

constexpr int kSampLpSeg = 128;   // segment records staged in LDS for the logprob merge (vocabularies <= 262144)

struct SampleShared {
  unsigned long long hist[256];
  float seg_m[kSampLpSeg], seg_l[kSampLpSeg];            // the segments' log-sum-exp partials
  float seg_tv[kSampLpSeg * kMaxLogprobs];               // and their top-n lists
  int seg_ti[kSampLpSeg * kMaxLogprobs];
  int seg_n[kSampLpSeg], seg_off[kSampLpSeg];            // the candidate path: candidates per segment, offsets
  int gv[kSampleList];   // the top-k set as gathered (any order): tokens, adjusted logits
  float gx[kSampleList];
  int lv[kSampleList];   // the same in index order
  float lx[kSampleList];
  int nlist;
  unsigned long long wsum[kSampleWaves];
  float fv[kSampleWaves];
  int fi[kSampleWaves];
  unsigned long long bcast[2];
  float lse;
};

// 64-bit lane exchanges as two 32-bit ones
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int m) {
  const unsigned lo = __shfl_xor((unsigned)x, m, 64), hi = __shfl_xor((unsigned)(x >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long x, int d) {
  const unsigned lo = __shfl_up((unsigned)x, d, 64), hi = __shfl_up((unsigned)(x >> 32), d, 64);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor_u64(x, m);
  return x;
}
// inclusive prefix sum over the lanes of a wave, in lane order
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned long long y = shfl_up_u64(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// block sum of one u64 per thread (integer: the same in any order; every thread gets it)
__device__ __forceinline__ unsigned long long block_sum_u64(SampleShared& sh, unsigned long long x) {
  x = wave_sum_u64(x);
  if ((threadIdx.x & 63) == 0) sh.wsum[threadIdx.x >> 6] = x;
  __syncthreads();
  unsigned long long t = 0;
  for (int w = 0; w < kSampleWaves; ++w) t += sh.wsum[w];
  __syncthreads();
  return t;
}

// block (value, index) maximum in rank order (value descending, index ascending); every thread gets it
__device__ __forceinline__ void block_best(SampleShared& sh, float& bv, int& bi) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (pick_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { sh.fv[threadIdx.x >> 6] = bv; sh.fi[threadIdx.x >> 6] = bi; }
  __syncthreads();
  bv = sh.fv[0];
  bi = sh.fi[0];
  for (int w = 1; w < kSampleWaves; ++w)
    if (pick_better(sh.fv[w], sh.fi[w], bv, bi)) { bv = sh.fv[w]; bi = sh.fi[w]; }
  __syncthreads();
}

// Tokens v0, v0 + stride, ... below v1 in groups of U: the U loads of a group are issued before any is used
// (addresses clamped into the range, so every load is in bounds), then f(v, z[v]) for the tokens of the group.
template <int U, class F>
__device__ __forceinline__ void sweep(const float* z, int v0, int v1, int stride, F&& f) {
  for (int base = v0; base < v1; base += stride * U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = z[min(base + u * stride, v1 - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * stride < v1) f(base + u * stride, x[u]);
  }
}
constexpr int kSweepU = 8;

// Radix selection over the keys of the tokens `in(v, x)` (x = z[v]), weight `wt(x)` each: the largest key K such
// that the total weight of keys >= K reaches `target`. Returns K and the weight of keys > K (integer sums: the
// same on every run).
template <class IN, class KEY, class WT>
__device__ __forceinline__ void radix_select(SampleShared& sh, const float* z, int V, IN&& in, KEY&& key, WT&& wt,
                                             unsigned long long target, uint32_t& K, unsigned long long& above) {
  uint32_t prefix = 0, pmask = 0;
  unsigned long long ab = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += kSampleThreads) sh.hist[b] = 0;
    __syncthreads();
    sweep<kSweepU>(z, threadIdx.x, V, kSampleThreads, [&](int v, float x) __attribute__((always_inline)) {
      if (!in(v, x)) return;
      const uint32_t k = key(x);
      if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], wt(x));
    });
    __syncthreads();
    // the bin where the weight counted from the top reaches the target: threads 0..255 hold bins 255..0 and form
    // an inclusive scan in that order (integer sums: exact); the one thread whose range crosses the target writes
    // its bin, and bin 0 takes the rest when bins 255..1 stay below it (as a walk down from bin 255 would)
    unsigned long long c = 0, incl = 0;
    if (threadIdx.x == 0) {   // (overwritten below by the thread whose range crosses the target)
      sh.bcast[0] = 0ull;
      sh.bcast[1] = ab;
    }
    if (threadIdx.x < 256) {
      c = sh.hist[255 - threadIdx.x];
      incl = wave_scan_u64(c);
      if ((threadIdx.x & 63) == 63) sh.wsum[threadIdx.x >> 6] = incl;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      unsigned long long off = ab;
      for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) off += sh.wsum[w];
      incl += off;
      const unsigned long long before = incl - c;
      if (before < target && (incl >= target || threadIdx.x == 255)) {
        sh.bcast[0] = (unsigned long long)(255 - threadIdx.x);
        sh.bcast[1] = before;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bcast[0] << shift;
    pmask |= 255u << shift;
    ab = sh.bcast[1];
    __syncthreads();
  }
  K = prefix;
  above = ab;
}

// The weight of the tokens `in(v, x)` in each of the kSampleWaves contiguous segments index_scan uses, into
// sh.wsum (wave w sums segment w, lanes on consecutive tokens); returns the total (every thread).
template <class IN, class WT>
__device__ __forceinline__ unsigned long long segment_sums(SampleShared& sh, const float* z, int V, IN&& in, WT&& wt) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int S1 = (V + kSampleWaves - 1) / kSampleWaves;
  const int a0 = wv * S1, a1 = min(V, a0 + S1);
  unsigned long long t = 0;
  sweep<kSweepU>(z, a0 + lane, a1, 64, [&](int v, float x) __attribute__((always_inline)) {
    if (in(v, x)) t += wt(x);
  });
  t = wave_sum_u64(t);
  if (lane == 0) sh.wsum[wv] = t;
  __syncthreads();
  unsigned long long tot = 0;
  for (int w = 0; w < kSampleWaves; ++w) tot += sh.wsum[w];
  return tot;
}

// In index order over the tokens `in(v, x)`: the first v whose running weight reaches `target` (>= 1); the last
// token if the total stays below it. Integer weights, so the sums are exact in any grouping. Two levels, every load
// coalesced or contiguous: wave w sums the w-th of kSampleWaves contiguous segments (lanes on consecutive tokens);
// the segment where the running sum reaches the target is cut into runs of E consecutive tokens, one per thread; a
// block scan of the run sums in index order finds the run, and its thread walks at most E tokens.
// have_seg: sh.wsum already holds the segment sums (segment_sums below, same predicate and weights).
template <class IN, class WT>
__device__ __forceinline__ int index_scan(SampleShared& sh, const float* z, int V, IN&& in, WT&& wt,
                                          unsigned long long target, bool have_seg = false) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int S1 = (V + kSampleWaves - 1) / kSampleWaves;   // tokens per wave segment
  if (!have_seg) {
    const int a0 = wv * S1, a1 = min(V, a0 + S1);
    unsigned long long t = 0;
    sweep<kSweepU>(z, a0 + lane, a1, 64, [&](int v, float x) __attribute__((always_inline)) {
      if (in(v, x)) t += wt(x);
    });
    t = wave_sum_u64(t);
    if (lane == 0) sh.wsum[wv] = t;
  }
  if (tid == 0) sh.bcast[0] = (unsigned long long)(V - 1);   // (past the total: the last token)
  __syncthreads();
  unsigned long long run = 0;   // the weight before the segment that holds the target
  int seg = kSampleWaves;
  for (int w = 0; w < kSampleWaves; ++w) {
    if (run + sh.wsum[w] >= target) {
      seg = w;
      break;
    }
    run += sh.wsum[w];
  }
  __syncthreads();   // (wsum is rewritten below)
  if (seg < kSampleWaves) {   // (the same for every thread)
    const int E = (S1 + kSampleThreads - 1) / kSampleThreads;   // tokens per run
    const int b1 = min(V, (seg + 1) * S1);
    const int c0 = min(b1, seg * S1 + tid * E), c1 = min(b1, c0 + E);
    unsigned long long t = 0;
    sweep<kSweepU>(z, c0, c1, 1, [&](int v, float x) __attribute__((always_inline)) {
      if (in(v, x)) t += wt(x);
    });
    const unsigned long long incl = wave_scan_u64(t);
    if (lane == 63) sh.wsum[wv] = incl;
    __syncthreads();
    unsigned long long off = run;
    for (int w = 0; w < wv; ++w) off += sh.wsum[w];
    const unsigned long long before = off + incl - t;
    if (before < target && before + t >= target) {
      unsigned long long r2 = before;
      for (int v = c0; v < c1; ++v) {
        const float x = z[v];
        if (!in(v, x)) continue;
        r2 += wt(x);
        if (r2 >= target) {
          sh.bcast[0] = (unsigned long long)v;
          break;
        }
      }
    }
  }
  __syncthreads();
  const int r = (int)sh.bcast[0];
  __syncthreads();
  return r;
}

// Adjusted logit of one token: the repetition penalty on a seen token (toward zero), presence and frequency
// penalties, then the bias; a NaN logit (or result) counts as -inf.
__device__ __forceinline__ float adjust_logit(float x, int c, float bias_v, const SampleRow& prm) {
  if (x != x) x = -INFINITY;
  if (c > 0) x = (x > 0.f ? x / prm.rep : x * prm.rep) - prm.presence - prm.frequency * (float)c;
  x += bias_v;
  if (x != x) x = -INFINITY;
  return x;
}

// The selection over a top-k list of n <= 64 entries (index order) in one wave, lane i on entry i: top-p keeps an
// entry while the weight of the entries ranked before it (key descending, index ascending) stays below p of the
// list's total, which is the shortest ranked prefix reaching it; min-p then drops the entries below min_p of the top
// token's weight; the draw takes the first kept entry in index order whose running weight reaches u times the kept
// total, plus one. The weights are integers, so every sum is exact in any order and the result is the one the
// block-wide passes find. Returns the drawn entry, or -1 if no weight is kept.
template <class KEY, class WT>
__device__ __forceinline__ int wave_select(const float* lx, int n, KEY&& key, WT&& wt, float top_p, float inv_t,
                                           float smax, float lmin, double u) {
  const int i = threadIdx.x & 63;
  const bool live = i < n;
  const float x = live ? lx[i] : -INFINITY;
  const uint32_t k = live ? key(x) : 0u;
  const unsigned long long w = live ? wt(x) : 0ull;
  bool kept = live;
  if (top_p < 1.f) {
    const unsigned long long tw = wave_sum_u64(w);
    unsigned long long target = (unsigned long long)((double)top_p * (double)tw);
    if (target < 1) target = 1;
    unsigned long long before = 0;
    for (int j = 0; j < n; ++j) {
      // (the builtin returns a signed int: each half goes through unsigned before it is widened)
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane(k, j);
      const unsigned long long wj =
          ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((unsigned)(w >> 32), j) << 32) |
          (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((unsigned)w, j);
      if (kj > k || (kj == k && j < i)) before += wj;
    }
    kept = kept && before < target;
  }
  kept = kept && x * inv_t - smax >= lmin;
  const unsigned long long kw = kept ? w : 0ull;
  const unsigned long long tw = wave_sum_u64(kw);
  if (tw == 0) return -1;
  unsigned long long target = (unsigned long long)(u * (double)tw) + 1ull;
  if (target > tw) target = tw;
  const unsigned long long hit = __ballot(wave_scan_u64(kw) >= target);
  return hit ? (int)__builtin_ctzll(hit) : n - 1;
}

// Whether a row's draw takes the candidate path: a temperature draw whose top-k (below the vocabulary) is at most
// kSampFastK, with at most kSampCand candidates over at most kSampLpSeg segments.
__host__ __device__ __forceinline__ bool samp_fast(const SampleRow& prm, int V) {
  return prm.temperature > 0.f && prm.top_k >= 1 && prm.top_k <= kSampFastK && prm.top_k < V &&
         samp_segments(V) * prm.top_k <= kSampCand && samp_segments(V) <= kSampLpSeg;
}

// Whether the log-probabilities' top n come from the candidate path's top-k list: the n best by rank all lie in
// the row's top-k set when n <= k, so the segments need not keep top-n lists of their own.
__host__ __device__ __forceinline__ bool samp_lp_listed(const SampleRow& prm, int V, int nl) {
  return samp_fast(prm, V) && nl <= prm.top_k;
}

constexpr int kPartThreads = 256;
constexpr int kPartWaves = kPartThreads / 64;

// exclusive prefix sum over the block's threads in thread order (every value is an integer count)
__device__ __forceinline__ int part_scan(int* wtot, int x, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
  for (int w = 0; w < kPartWaves; ++w) {
    if (w < wv) off += wtot[w];
    total += wtot[w];
  }
  __syncthreads();
  return off + incl - x;
}

// (value, index) best of the block in rank order, in every thread
__device__ __forceinline__ void part_best(float* fv, int* fi, float& bv, int& bi) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (pick_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { fv[threadIdx.x >> 6] = bv; fi[threadIdx.x >> 6] = bi; }
  __syncthreads();
  bv = fv[0];
  bi = fi[0];
  for (int w = 1; w < kPartWaves; ++w)
    if (pick_better(fv[w], fi[w], bv, bi)) { bv = fv[w]; bi = fi[w]; }
  __syncthreads();
}

// Lane exchanges for the (value, index) best of a wave without LDS traffic: quad permutations and the half-row and
// row mirrors (DPP) within each 16 lanes, then the permlane swaps between rows (16) and halves (32). Every step
// pairs each lane with one partner and both keep the better of the two, so every lane ends with the wave's best.
template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ void best_step_dpp(float& v, int& i) {
  const float ov = __int_as_float(dpp_mov_i<CTRL>(__float_as_int(v)));
  const int oi = dpp_mov_i<CTRL>(i);
  if (pick_better(ov, oi, v, i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void best_step_swap(float& v, int& i, bool rows32) {
  const auto a = rows32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                        : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const auto b = rows32 ? __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false)
                        : __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
  // (the pair holds this lane's and its partner's value, in either order)
  const float v0 = __uint_as_float(a[0]), v1 = __uint_as_float(a[1]);
  const int i0 = (int)b[0], i1 = (int)b[1];
  float bv = v0;
  int bi = i0;
  if (pick_better(v1, i1, bv, bi)) { bv = v1; bi = i1; }
  v = bv;
  i = bi;
}
__device__ __forceinline__ void wave_best_dpp(float& v, int& i) {
  best_step_dpp<0xB1>(v, i);    // quad_perm [1,0,3,2]
  best_step_dpp<0x4E>(v, i);    // quad_perm [2,3,0,1]
  best_step_dpp<0x141>(v, i);   // row_half_mirror
  best_step_dpp<0x140>(v, i);   // row_mirror
  best_step_swap(v, i, false);  // rows 0 <-> 1, 2 <-> 3
  best_step_swap(v, i, true);   // halves
}

// The top n (n <= kMaxLogprobs) by rank (value descending, index ascending) among the entries a wave's lanes hold
// (E each; an unused entry has value -inf and index INT_MAX): n rounds, each the wave's best entry ranked below the
// previous round's, by shuffles alone. Every lane gets the results.
template <int E>
__device__ __forceinline__ void wave_topn(const float (&x)[E], const int (&v)[E], int n, float (&ov)[kMaxLogprobs],
                                          int (&oi)[kMaxLogprobs]) {
  float pv = INFINITY;
  int pi = -1;
  for (int j = 0; j < kMaxLogprobs; ++j) {
    float cv = -INFINITY;
    int ci = 0x7fffffff;
    if (j < n) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool below = x[e] < pv || (x[e] == pv && v[e] > pi);
        if (below && pick_better(x[e], v[e], cv, ci)) { cv = x[e]; ci = v[e]; }
      }
      wave_best_dpp(cv, ci);
    }
    ov[j] = cv;
    oi[j] = ci;
    pv = cv;
    pi = ci;
  }
}

// The sampler's first kernel: block (segment b, row r) takes tokens [b kSampSeg, b kSampSeg + n) of row r. It forms
// their adjusted logits (into z, and into LDS for the passes below) and the segment record (SampPart): the best
// (value, index); with logprobs asked for, the log-sum-exp partial of s = z / T (T = 1 for greedy) and the top n
// tokens by rank; on the candidate path, the segment's own top-k by (s descending, index ascending) -- a radix
// selection of the k-th largest key, then the tokens above it and the lowest-index ones at it, in index order.
__global__ void __launch_bounds__(kPartThreads) sample_part_kernel(SampleParams p) {
  __shared__ float zs[kSampSeg];
  __shared__ unsigned hist[256];
  __shared__ float fv[kPartWaves];
  __shared__ int fi[kPartWaves];
  __shared__ int wtot[kPartWaves];
  __shared__ int bc[2];
  __shared__ float wtop_v[kPartWaves * kMaxLogprobs];
  __shared__ int wtop_i[kPartWaves * kMaxLogprobs];
  const int r = blockIdx.y, b = blockIdx.x, V = p.vocab, tid = threadIdx.x;
  const int v0 = b * kSampSeg, n = min(kSampSeg, V - v0);
  const SampleRow prm = p.rowp[r];
  const float* lg = p.logits + (size_t)r * V + v0;
  const int32_t* cnt = p.counts + (size_t)r * V + v0;
  const float* bias = p.bias + (size_t)r * V + v0;
  float* z = p.z + (size_t)r * V + v0;
  SampPart& out = p.part[(size_t)r * gridDim.x + b];

  float bv = -INFINITY;
  int bi = 0x7fffffff;
  constexpr int PT = kSampSeg / kPartThreads;   // tokens per thread, all loads issued first
  {
    float xl[PT], xb[PT];
    int xc[PT];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = min(tid + u * kPartThreads, n - 1);
      xl[u] = lg[i];
      xc[u] = cnt[i];
      xb[u] = bias[i];
    }
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = tid + u * kPartThreads;
      if (i >= n) break;
      const float x = adjust_logit(xl[u], xc[u], xb[u], prm);
      zs[i] = x;
      z[i] = x;
      if (pick_better(x, v0 + i, bv, bi)) { bv = x; bi = v0 + i; }
    }
  }
  part_best(fv, fi, bv, bi);   // (its barriers also publish zs)
  if (tid == 0) {
    out.best_v = bv;
    out.best_i = bi;
  }
  const float T = prm.temperature;
  const float inv_t = T > 0.f ? 1.f / T : 1.f;
  const int nl = min(max(prm.n_logprobs, 0), kMaxLogprobs);
  if (nl > 0) {
    // log-sum-exp partial over the segment: m = its largest s, l = sum of exp(s - m) (in a fixed order)
    const float m = bv * inv_t;
    float t = 0.f;
    if (m > -INFINITY)
      for (int i = tid; i < n; i += kPartThreads) t += __expf(zs[i] * inv_t - m);
    t = wave_total(t);
    if ((tid & 63) == 0) fv[tid >> 6] = t;
    __syncthreads();
    float l = 0.f;
    for (int w = 0; w < kPartWaves; ++w) l += fv[w];
    __syncthreads();
    if (tid == 0) {
      out.m = m;
      out.l = l;
    }
    // the top nl by rank: each wave's own (its lanes' PT tokens each), then wave 0 over the waves' lists (unless
    // the per-row kernel takes them from its top-k list)
    if (!samp_lp_listed(prm, V, nl)) {
      float x[PT];
      int v[PT];
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int i = tid + u * kPartThreads;
        x[u] = i < n ? zs[i] * inv_t : -INFINITY;
        v[u] = i < n ? v0 + i : 0x7fffffff;
      }
      float tv[kMaxLogprobs];
      int ti[kMaxLogprobs];
      wave_topn<PT>(x, v, nl, tv, ti);
      if ((tid & 63) == 0)
        for (int j = 0; j < kMaxLogprobs; ++j) {
          wtop_v[(tid >> 6) * kMaxLogprobs + j] = tv[j];
          wtop_i[(tid >> 6) * kMaxLogprobs + j] = ti[j];
        }
      __syncthreads();
      if (tid < 64) {
        float x1[1] = {tid < kPartWaves * kMaxLogprobs ? wtop_v[tid] : -INFINITY};
        int v1[1] = {tid < kPartWaves * kMaxLogprobs ? wtop_i[tid] : 0x7fffffff};
        wave_topn<1>(x1, v1, nl, tv, ti);
        if (tid == 0)
          for (int j = 0; j < nl; ++j) {
            out.top_v[j] = tv[j];
            out.top_i[j] = ti[j];
          }
      }
    }
  }
  if (!samp_fast(prm, V)) return;

  // ---- the segment's top-k by (s descending, index ascending)
  const int kl = min(prm.top_k, n);
  uint32_t prefix = 0u, pmask = 0u;
  int above = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;   // (256 threads, 256 bins)
    __syncthreads();
    for (int i = tid; i < n; i += kPartThreads) {
      const uint32_t k = order_key(zs[i] * inv_t);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // bins in descending order: thread t holds bin 255 - t; the bin where the count from the top reaches kl
    const int c = (int)hist[255 - tid];
    int tot = 0;
    const int before = above + part_scan(wtot, c, tot);
    if (before < kl && before + c >= kl) {
      bc[0] = 255 - tid;
      bc[1] = before;
    }
    __syncthreads();
    prefix |= (uint32_t)bc[0] << shift;
    pmask |= 255u << shift;
    above = bc[1];
    __syncthreads();
  }
  const uint32_t K = prefix;
  const int need_eq = kl - above;   // tokens at key K to take, lowest index first
  // emit in index order: thread t takes the run [t E, t E + E)
  constexpr int E = kSampSeg / kPartThreads;
  const int c0 = min(n, tid * E), c1 = min(n, c0 + E);
  int n_eq = 0;
  for (int i = c0; i < c1; ++i) n_eq += order_key(zs[i] * inv_t) == K;
  int tot = 0;
  int eq_before = part_scan(wtot, n_eq, tot);
  bool keep[E];
  int n_keep = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = c0 + e;
    bool k = false;
    if (i < c1) {
      const uint32_t key = order_key(zs[i] * inv_t);
      if (key > K) k = true;
      else if (key == K) k = eq_before++ < need_eq;
    }
    keep[e] = k;
    n_keep += k;
  }
  int pos = part_scan(wtot, n_keep, tot);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (keep[e]) {
      out.cand_v[pos] = v0 + c0 + e;
      out.cand_x[pos] = zs[c0 + e];
      ++pos;
    }
  if (tid == 0) out.n_cand = tot;
}

__global__ void __launch_bounds__(kSampleThreads) sample_kernel(SampleParams p) {
  __shared__ SampleShared sh;
  __shared__ int s_cv[kSampCand];     // the candidate path: every segment's top-k, concatenated (index order)
  __shared__ float s_cx[kSampCand];
  const int r = blockIdx.x, V = p.vocab, tid = threadIdx.x;
  const SampleRow prm = p.rowp[r];
  int32_t* cnt = p.counts + (size_t)r * V;
  const float* z = p.z + (size_t)r * V;   // adjusted logits (the segment kernel)
  const int NB = samp_segments(V);
  const SampPart* pr = p.part + (size_t)r * NB;

  // ---- the largest adjusted logit: the best of the segments' bests
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int b = tid; b < NB; b += kSampleThreads)
    if (pick_better(pr[b].best_v, pr[b].best_i, bv, bi)) { bv = pr[b].best_v; bi = pr[b].best_i; }
  block_best(sh, bv, bi);
  const float zmax = bv;
  int token = bi < V ? bi : 0;
  const float T = prm.temperature;
  const float inv_t = T > 0.f ? 1.f / T : 1.f;
  int n_list = 0;   // the top-k list's length (sh.lv, sh.lx), when one is gathered

  if (T > 0.f && zmax > -INFINITY) {
    auto key = [&](float x) __attribute__((always_inline)) { return order_key(x * inv_t); };
    const float smax = zmax * inv_t;
    // weight of a token: exp(s - s_max) in fixed point (2^40 = the top token)
    auto wt = [&](float x) __attribute__((always_inline)) -> unsigned long long {
      const float w = __expf(x * inv_t - smax);
      return (unsigned long long)(w * 1099511627776.f);
    };
    auto one = [&](float) __attribute__((always_inline)) -> unsigned long long { return 1ull; };
    auto all = [&](int, float) __attribute__((always_inline)) { return true; };
    // The top-k set is chosen from the candidates (every segment's top-k, in index order) on the candidate path,
    // else from the whole vocabulary: (zk, Vk) and the token a position of it stands for.
    const bool fast = samp_fast(prm, V);
    int n_c = V;
    if (fast) {
      // the segments' candidate counts (loaded in parallel), their offsets in segment order, then every entry
      // copied in parallel to its place: the concatenation is in index order
      for (int b = tid; b < NB; b += kSampleThreads) sh.seg_n[b] = pr[b].n_cand;
      __syncthreads();
      if (tid == 0) {
        int off = 0;
        for (int b = 0; b < NB; ++b) {
          sh.seg_off[b] = off;
          off += sh.seg_n[b];
        }
        sh.nlist = off;
      }
      __syncthreads();
      n_c = sh.nlist;
      for (int i = tid; i < NB * kSampFastK; i += kSampleThreads) {
        const int b = i / kSampFastK, j = i % kSampFastK;
        if (j < sh.seg_n[b]) {
          s_cv[sh.seg_off[b] + j] = pr[b].cand_v[j];
          s_cx[sh.seg_off[b] + j] = pr[b].cand_x[j];
        }
      }
      __syncthreads();
    }
    const float* zk = fast ? s_cx : z;
    const int Vk = n_c;
    auto tok_of = [&](int v) __attribute__((always_inline)) { return fast ? s_cv[v] : v; };
    // top-k: the k best ranked (ties at the threshold key by lower index)
    uint32_t kk = 0u;
    int ki = Vk;
    if (prm.top_k > 0 && prm.top_k < Vk) {
      unsigned long long above = 0;
      radix_select(sh, zk, Vk, all, key, one, (unsigned long long)prm.top_k, kk, above);
      const uint32_t K = kk;
      ki = index_scan(sh, zk, Vk, [&](int, float x) __attribute__((always_inline)) { return key(x) == K; }, one,
                      (unsigned long long)prm.top_k - above);
    }
    const uint32_t K1 = kk;
    const int I1 = ki;
    auto in_k = [&](int v, float x) __attribute__((always_inline)) {
      const uint32_t k = key(x);
      return k > K1 || (k == K1 && v <= I1);
    };
    // With top-k on (k <= kSampleList) the rest of the selection runs over the top-k set alone, its tokens and
    // adjusted logits gathered into LDS in index order: position i of the list stands for token lv[i], and the
    // order, keys and weights are those of the full sweep, so every selection below comes out the same.
    const bool listed = prm.top_k > 0 && prm.top_k < V && prm.top_k <= kSampleList;
    int n = 0;
    if (listed) {
      if (tid == 0) sh.nlist = 0;
      __syncthreads();
      sweep<kSweepU>(zk, tid, Vk, kSampleThreads, [&](int v, float x) __attribute__((always_inline)) {
        if (in_k(v, x)) {
          const int i = atomicAdd(&sh.nlist, 1);
          if (i < kSampleList) {
            sh.gv[i] = tok_of(v);
            sh.gx[i] = x;
          }
        }
      });
      __syncthreads();
      n = min(sh.nlist, kSampleList);
      n_list = n;
      for (int i = tid; i < n; i += kSampleThreads) {   // index order: a token's rank among the gathered ones
        const int v = sh.gv[i];
        int rank = 0;
        for (int j = 0; j < n; ++j) rank += sh.gv[j] < v;
        sh.lv[rank] = v;
        sh.lx[rank] = sh.gx[i];
      }
      __syncthreads();
    }
    const uint64_t seed = ((uint64_t)prm.seed_hi << 32) | prm.seed_lo;
    const uint32_t d = p.draws[r];
    const double u = (double)(splitmix64(seed, d) >> 40) * (1.0 / 16777216.0);
    const float lmin = prm.min_p > 0.f ? __logf(prm.min_p) : -INFINITY;
    // top-p, min-p and the draw over the selection's tokens (zs, Vs; in_s: member of the top-k set), instantiated
    // once for the whole vocabulary in global memory and once for the list in LDS; the position of the drawn token
    // among them, or -1 if no weight is kept
    auto select = [&](const float* zs, int Vs, auto&& in_s) __attribute__((always_inline)) -> int {
      // top-p: the shortest ranked prefix of the top-k set whose weight reaches p of its total
      uint32_t kp = 0u;
      int ip = Vs;
      if (prm.top_p < 1.f) {
        unsigned long long tw = 0;
        sweep<kSweepU>(zs, tid, Vs, kSampleThreads, [&](int v, float x) __attribute__((always_inline)) {
          if (in_s(v, x)) tw += wt(x);
        });
        tw = block_sum_u64(sh, tw);
        unsigned long long target = (unsigned long long)((double)prm.top_p * (double)tw);
        if (target < 1) target = 1;
        unsigned long long above = 0;
        radix_select(sh, zs, Vs, in_s, key, wt, target, kp, above);
        const uint32_t K = kp;
        ip = index_scan(sh, zs, Vs,
                        [&](int v, float x) __attribute__((always_inline)) { return in_s(v, x) && key(x) == K; }, wt,
                        target - above);
      }
      const uint32_t K2 = kp;
      const int I2 = ip;
      // min-p: weight at least min_p of the top token's
      auto kept = [&](int v, float x) __attribute__((always_inline)) {
        if (!in_s(v, x)) return false;
        const uint32_t k = key(x);
        if (!(k > K2 || (k == K2 && v <= I2))) return false;
        return x * inv_t - smax >= lmin;
      };
      // the draw: inverse CDF in index order over the kept weights (the segment sums of the total are the scan's
      // first level)
      const unsigned long long tw = segment_sums(sh, zs, Vs, kept, wt);
      unsigned long long target = (unsigned long long)(u * (double)tw) + 1ull;
      if (target > tw) target = tw;
      return tw > 0 ? index_scan(sh, zs, Vs, kept, wt, target, true) : -1;
    };
    if (listed && n <= 64) {   // (the bench's top-k of 40, say: no block-wide passes)
      if (tid < 64) {
        const int i = wave_select(sh.lx, n, key, wt, prm.top_p, inv_t, smax, lmin, u);
        if (tid == 0) sh.nlist = i;
      }
      __syncthreads();
      if (sh.nlist >= 0) token = sh.lv[sh.nlist];
    } else if (listed) {
      const float* lx = sh.lx;
      const int i = select(lx, n, [](int, float) __attribute__((always_inline)) { return true; });
      if (i >= 0) token = sh.lv[i];
    } else {
      const int i = select(z, V, in_k);
      if (i >= 0) token = i;
    }
    if (tid == 0) p.draws[r] = d + 1u;
  }

  // ---- logprobs of the adjusted distribution (temperature 1 for greedy): the drawn token's and the top n by rank,
  // from the segments' log-sum-exp partials (merged in segment order) and, unless they come from the top-k list,
  // the segments' top-n lists
  const SlotLayout sl{p.rows};
  const int step = p.slots[sl.chain()];
  const int slot = step % p.max_chain;
  float* lpo = p.lp + ((size_t)slot * p.rows + r) * (1 + kMaxLogprobs);
  int32_t* lpi = p.lp_ids + ((size_t)slot * p.rows + r) * kMaxLogprobs;
  const int nl = min(max(prm.n_logprobs, 0), kMaxLogprobs);
  if (nl > 0) {
    const bool from_list = samp_lp_listed(prm, V, nl);
    // the segment records, staged in LDS by all threads (read from global memory past kSampLpSeg segments)
    const bool staged = NB <= kSampLpSeg;
    if (staged) {
      for (int b = tid; b < NB; b += kSampleThreads) {
        sh.seg_m[b] = pr[b].m;
        sh.seg_l[b] = pr[b].l;
      }
      if (!from_list) {
        for (int i = tid; i < NB * kMaxLogprobs; i += kSampleThreads) {   // (stride kMaxLogprobs per segment)
          const int b = i / kMaxLogprobs, q = i % kMaxLogprobs;
          sh.seg_tv[i] = q < nl ? pr[b].top_v[q] : -INFINITY;
          sh.seg_ti[i] = q < nl ? pr[b].top_i[q] : 0x7fffffff;
        }
      }
    }
    __syncthreads();
    // log-sum-exp of the segments' partials, by wave 0 (lanes over segments; sums in a fixed order)
    float lse = 0.f;
    if (tid < 64) {
      float M = -INFINITY;
      for (int b = tid; b < NB; b += 64) M = fmaxf(M, staged ? sh.seg_m[b] : pr[b].m);
      M = wave_max(M);
      float L = 0.f;
      for (int b = tid; b < NB; b += 64) {
        const float m = staged ? sh.seg_m[b] : pr[b].m;
        if (m > -INFINITY) L += (staged ? sh.seg_l[b] : pr[b].l) * __expf(m - M);
      }
      lse = M + __logf(wave_total(L));
      if (tid == 0) sh.lse = lse;
    }
    if (from_list) {
      // the top n by rank (s descending, index ascending) are the list entries of rank < n: each entry's rank is
      // the number of list entries ranked before it (the list is in index order). With no list (every adjusted
      // logit -inf) the ranks fall to the lowest indices.
      __syncthreads();
      const float lb = sh.lse;
      for (int i = tid; i < n_list; i += kSampleThreads) {
        const float si = sh.lx[i] * inv_t;
        int rank = 0;
        for (int j = 0; j < n_list; ++j) rank += pick_better(sh.lx[j] * inv_t, j, si, i);
        if (rank < nl) {
          lpi[rank] = sh.lv[i];
          lpo[1 + rank] = si - lb;
        }
      }
      if (n_list == 0 && tid < nl) {
        lpi[tid] = tid < V ? tid : -1;
        lpo[1 + tid] = -INFINITY - lb;
      }
    } else if (tid < 64) {
      // the top n by rank over the segments' top-n lists, by wave 0: chunks of 64 EL entries, each merged with the
      // running top n (lane j < n offers running entry j)
      constexpr int EL = kSampLpSeg * kMaxLogprobs / 64;
      float tv[kMaxLogprobs];
      int ti[kMaxLogprobs];
      for (int j = 0; j < kMaxLogprobs; ++j) {
        tv[j] = -INFINITY;
        ti[j] = 0x7fffffff;
      }
      for (int base = 0; base < NB * kMaxLogprobs; base += 64 * EL) {
        float x[EL + 1];
        int v[EL + 1];
        if (staged) {
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            const int i = base + tid + 64 * e;
            x[e] = i < NB * kMaxLogprobs ? sh.seg_tv[i] : -INFINITY;
            v[e] = i < NB * kMaxLogprobs ? sh.seg_ti[i] : 0x7fffffff;
          }
        } else {
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            const int i = base + tid + 64 * e;
            const int b = i / kMaxLogprobs, q = i % kMaxLogprobs;
            const bool ok = i < NB * kMaxLogprobs && q < nl;
            x[e] = ok ? pr[b].top_v[q] : -INFINITY;
            v[e] = ok ? pr[b].top_i[q] : 0x7fffffff;
          }
        }
        x[EL] = -INFINITY;
        v[EL] = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kMaxLogprobs; ++j)
          if (tid == j) {
            x[EL] = tv[j];
            v[EL] = ti[j];
          }
        wave_topn<EL + 1>(x, v, nl, tv, ti);
      }
      if (tid == 0)
        for (int j = 0; j < nl; ++j) {
          lpi[j] = ti[j] < V ? ti[j] : -1;
          lpo[1 + j] = tv[j] - lse;
        }
    }
    if (tid == 0) lpo[0] = z[token] * inv_t - lse;
  }

  // ---- the draw into the history and the slots; the chain record
  if (tid == 0) {
    cnt[token] += 1;
    p.ids[(size_t)slot * p.rows + r] = token;
    const int np = p.slots[sl.pos() + r] + 1;
    p.slots[sl.token() + r] = token;
    p.slots[sl.pos() + r] = np;
    if (p.page_table && np >= 0 && np < p.cap) {
      const int ppr = p.cap / p.page_size;
      p.slots[sl.write_map() + r] = p.page_table[(size_t)r * ppr + np / p.page_size] * p.page_size + np % p.page_size;
    }
  }

  // ---- the last row's block to finish closes the step: the non-finite flag and the chain counter (every thread
  // of every block has read the counter before its block takes a ticket); the ticket word is back at zero after
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (unsigned)p.rows - 1u) {
      p.flags[step % p.max_chain] = p.status->nonfinite ? 1u : 0u;
      p.status->nonfinite = 0;
      p.slots[sl.chain()] = step + 1;
      __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ----------------------------------------------------------------------------------------------------------
// host launchers

size_t gemv_lds_bytes(int rows, int K, bool norm) { (void)norm; return (size_t)rows * K * sizeof(float); }

int attn_positions_per_pass(int hd, int kv_dtype) {
  return std::min(kAttnChunk, kAttnChunkBytes / (hd * (kv_dtype == 1 ? 2 : 4)));   // splits are whole LDS chunks
}

size_t attn_lds_bytes(int nq, int nkv, int hd, int split_len, int kv_dtype, int page_size) {
  const int G = nq / nkv;
  const size_t pb = (size_t)hd * (kv_dtype == 1 ? 2 : 4);
  const int tc = attn_positions_per_pass(hd, kv_dtype);
  const int nb = kv_dtype == 1 && page_size > 0 ? 1 : 2;   // chunk buffers (attn_mfma_kernel: one when paged)
  size_t bytes = (size_t)nb * 2 * tc * pb + (size_t)4 * G * (hd + 2) * sizeof(float);
  if (page_size > 0) bytes += (size_t)((split_len + tc - 1) / tc) * (page_size <= tc ? tc / page_size : 1) * 4;
  return bytes;
}

int attn_max_splits(int nq, int nkv, int hd) {
  (void)nq;
  (void)nkv;
  (void)hd;
  return kMaxSplits;
}

template <typename F>
static hipError_t set_lds(F* f, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

hipError_t launch_embed(const EmbedParams& p, int weight_dtype, hipStream_t s) {
  if (p.d % 8) return hipErrorInvalidValue;
  const dim3 grid((p.d + 8 * kBlock - 1) / (8 * kBlock), p.rows);
  if (weight_dtype == 1) embed_kernel<uint16_t><<<grid, kBlock, 0, s>>>(p);
  else embed_kernel<float><<<grid, kBlock, 0, s>>>(p);
  return hipGetLastError();
}

template <typename WT, typename KT, int MODE, int NR, int XREG>
static hipError_t gemv_go(const GemvParams& p, int blocks, hipStream_t s) {
  // long rows (more than one group of kUnroll chunks) get the ping-pong variant; only the residual GEMVs have them
  const int nchunks = (p.K + 64 * Pack<WT>::N - 1) / (64 * Pack<WT>::N);
  // (the ping-pong variant keeps only 4 float4 of the activation in registers: its second buffer needs the room)
  auto* f = gemv_kernel<WT, KT, NR, MODE, XREG, false>;
  if constexpr (MODE == GEMV_RESID)
    if (nchunks > kUnroll && p.ping_pong) f = gemv_kernel<WT, KT, NR, MODE, 4, true>;
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

template <typename KT, int HD, int GG>
static hipError_t attn_go(const AttnParams& p, int rows, hipStream_t s) {
  const size_t lds = attn_lds_bytes(p.nq, p.nkv, HD, p.split_len, sizeof(KT) == 2 ? 1 : 0,
                                    p.kv.paged ? p.kv.page_size : 0);
  dim3 grid(p.splits, p.nkv, rows);
  hipError_t e;
  auto go = [&](auto* f) {
    if ((e = set_lds(f, lds)) != hipSuccess) return e;
    f<<<grid, kBlock, lds, s>>>(p);
    return hipGetLastError();
  };
  if constexpr (sizeof(KT) == 2) {   // bf16 K/V (V transposed): matrix cores
    if (!p.kv.v_t) return hipErrorInvalidValue;
    return p.kv.paged ? go(attn_mfma_kernel<HD, GG, true>) : go(attn_mfma_kernel<HD, GG, false>);
  } else {
    return p.kv.paged ? go(attn_kernel<KT, HD, GG, true>) : go(attn_kernel<KT, HD, GG, false>);
  }
}

template <typename KT, int HD>
static hipError_t attn_g(const AttnParams& p, int rows, hipStream_t s) {
  switch (p.nq / p.nkv) {
    case 1: return attn_go<KT, HD, 1>(p, rows, s);
    case 2: return attn_go<KT, HD, 2>(p, rows, s);
    case 4: return attn_go<KT, HD, 4>(p, rows, s);
    case 8: return attn_go<KT, HD, 8>(p, rows, s);
    default: return hipErrorInvalidValue;
  }
}

template <int HD, int NS>
static hipError_t combine_gs(const AttnParams& p, int rows, hipStream_t s) {
  const dim3 grid(p.nq, rows);
  switch (p.nq / p.nkv) {
    case 1: attn_combine_kernel<1, HD, NS><<<grid, HD, 0, s>>>(p); break;
    case 2: attn_combine_kernel<2, HD, NS><<<grid, HD, 0, s>>>(p); break;
    case 4: attn_combine_kernel<4, HD, NS><<<grid, HD, 0, s>>>(p); break;
    case 8: attn_combine_kernel<8, HD, NS><<<grid, HD, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int HD>
static hipError_t combine_g(const AttnParams& p, int rows, hipStream_t s) {
  static_assert(kMaxSplits == 32, "split classes 4, 8, 16, 32");
  if (p.splits <= 4) return combine_gs<HD, 4>(p, rows, s);
  if (p.splits <= 8) return combine_gs<HD, 8>(p, rows, s);
  if (p.splits <= 16) return combine_gs<HD, 16>(p, rows, s);
  return combine_gs<HD, 32>(p, rows, s);
}

hipError_t launch_attention_combine(const AttnParams& p, int rows, hipStream_t s) {
  if (p.splits < 1 || p.splits > kMaxSplits) return hipErrorInvalidValue;
  if (p.hd == 64) return combine_g<64>(p, rows, s);
  if (p.hd == 128) return combine_g<128>(p, rows, s);
  return hipErrorInvalidValue;
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

SkPlan sk_plan(int n_rows, int K, bool whole_quads) {
  SkPlan p{};
  if (n_rows % (kSkRows * kSkQuad) || K % kSkChunk || n_rows < 1 || K < 1) return p;
  p.groups = n_rows / kSkRows;
  p.nck = K / kSkChunk;
  const long long total = (long long)p.quads() * p.nck;
  const long long nb = std::max(1LL, std::min((long long)kSkMaxBlocks, whole_quads ? (long long)p.quads() : total));
  if (total * nb >= (1LL << 32)) return SkPlan{};
  p.nb = (int)nb;
  if (!whole_quads)
    for (int q = 0; q < p.quads(); ++q)
      p.cmax = std::max(p.cmax, p.block_of((q + 1) * p.nck - 1) - p.block_of(q * p.nck) + 1);
  return p;
}

hipError_t launch_sk_gemm(const SkGemmParams& p, bool head, hipStream_t s) {
  const SkPlan& pl = p.plan;
  if (p.K % kSkChunk || pl.nck != p.K / kSkChunk || pl.groups < kSkQuad || pl.groups % kSkQuad || pl.nck < 1 || pl.nb < 1)
    return hipErrorInvalidValue;
  if (!head && pl.cmax < 1) return hipErrorInvalidValue;
  if (p.nt != sk_tiles(p.rows) || p.rows < 1 || p.rows > kMfmaRows * p.nt) return hipErrorInvalidValue;
  if (head && (p.n_out != pl.groups * kSkRows || p.n_out % 4)) return hipErrorInvalidValue;
  if (!head && !p.part) return hipErrorInvalidValue;
  auto* f = p.nt == 1 ? (head ? sk_gemm_kernel<true, 1> : sk_gemm_kernel<false, 1>)
                      : (head ? sk_gemm_kernel<true, 4> : sk_gemm_kernel<false, 4>);
  const size_t lds = p.nt == 1 ? kSkLds<1> : kSkLds<4>;   // 120 KB, 160 KB
  hipError_t e = set_lds(f, lds);
  if (e != hipSuccess) return e;
  f<<<pl.nb, 64 * kSkWaves, lds, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_sk_prep(const SkPrepParams& p, hipStream_t s) {
  if (p.D % 8 || p.rows < 1 || p.nt != sk_tiles(p.rows) || p.rows > kMfmaRows * p.nt) return hipErrorInvalidValue;
  const dim3 grid((p.D + kNormSpan - 1) / kNormSpan, kMfmaRows * p.nt);
  sk_prep_kernel<<<grid, 64, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_sk_qkv(const SkQkvParams& p, int kv_dtype, hipStream_t s) {
  const int n4 = (p.nq + 2 * p.nkv) * p.hd / 4;
  if (p.hd % 8 || p.rows < 1 || p.nt != sk_tiles(p.rows) || p.rows > kMfmaRows * p.nt) return hipErrorInvalidValue;
  const dim3 grid((n4 + kQkvBlock - 1) / kQkvBlock, p.rows);
  if (kv_dtype == 1) sk_qkv_kernel<uint16_t><<<grid, kQkvBlock, 0, s>>>(p);
  else sk_qkv_kernel<float><<<grid, kQkvBlock, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_sk_swiglu(const SkActParams& p, hipStream_t s) {
  if (p.F % 8 || p.rows < 1 || p.nt != sk_tiles(p.rows) || p.rows > kMfmaRows * p.nt) return hipErrorInvalidValue;
  const dim3 grid((p.F + kActSpan - 1) / kActSpan, kMfmaRows * p.nt);
  sk_swiglu_kernel<<<grid, 64, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_kv_copy(const KvView& kv, int kv_dtype, int layer, int row, int pos0, int n, int nkv, int hd,
                          void* staging, int to_state, int stage_vt, StatusWords* status, hipStream_t s) {
  const size_t total = 2 * (size_t)nkv * n * hd;
  int blocks = (int)((total + kBlock - 1) / kBlock);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (kv_dtype == 1)
    kv_copy_kernel<uint16_t><<<blocks, kBlock, 0, s>>>(kv, layer, row, pos0, n, nkv, hd,
                                                       reinterpret_cast<uint16_t*>(staging), to_state, stage_vt,
                                                       status);
  else
    kv_copy_kernel<float><<<blocks, kBlock, 0, s>>>(kv, layer, row, pos0, n, nkv, hd,
                                                    reinterpret_cast<float*>(staging), to_state, stage_vt, status);
  return hipGetLastError();
}

hipError_t launch_pick(const PickParams& p, hipStream_t s) {
  if (p.rows < 1 || p.rows > kPickThreads || p.vocab < 1 || p.max_chain < 1) return hipErrorInvalidValue;
  pick_kernel<<<p.rows * kPickSplit, kPickThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleParams& p, hipStream_t s) {
  if (p.rows < 1 || p.vocab < 1 || p.max_chain < 1 || !p.part || !p.done) return hipErrorInvalidValue;
  sample_part_kernel<<<dim3(samp_segments(p.vocab), p.rows), kPartThreads, 0, s>>>(p);
  hipError_t h0 = hipGetLastError();
  if (h0 != hipSuccess) return h0;
  sample_kernel<<<p.rows, kSampleThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return hipErrorInvalidValue;
  stream_read_kernel<<<kProbeBlocks, 512, 0, s>>>(reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t s) {
  int blocks = (int)((n + kBlock - 1) / kBlock);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  fill_u32_kernel<<<blocks, kBlock, 0, s>>>(p, value, n);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------------------------
// Allocation-free staging (ds3_write_kv_noalloc). One array per GPU the library runs on, held until the process
// ends. In host code `scratch` is a host-side stand-in, not a device address: every host use goes through the
// address hipGetSymbolAddress returns for the device, looked up once per device with that device current.

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t scratch_device_ptr(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = 0;
    hipError_t h = hipGetDevice(&cur);
    if (h != hipSuccess) return h;
    if (cur != device && (h = hipSetDevice(device)) != hipSuccess) return h;
    void* ptr = nullptr;
    h = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t h2 = cur != device ? hipSetDevice(cur) : hipSuccess;
    if (h != hipSuccess) return h;
    if (h2 != hipSuccess) return h2;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace ds3

// The decode step of one row as ONE persistent kernel (gfx950).
//
// Batch-1 decode streams about half a gigabyte of weights per layer through five dependent steps: QKV
// projection, attention sweep, o-projection, gate/up, down ("Models, Registry and the Driver" page, section
// "Shared components"; "Execution" page, section "A constant-shape decode graph"). As separate kernels each step
// pays a launch, a ramp-up and a drain of several microseconds against 5-40 us of streaming. Here one launch of
// kFusedBlocks blocks (one per CU, 8 waves each) runs the whole step, and the steps become phases separated by
// grid barriers. The weights do not depend on the activations, so every wave issues the loads of its first two
// weight batches of the NEXT phase before it reaches the barrier: HBM keeps streaming while the grid
// synchronizes. The K/V chunk a block sweeps in layer l + 1 is staged into LDS (direct global-to-LDS loads) while
// layer l's gate/up phase streams.
//
// Coherence across the 8 XCDs, whose L2 caches are not coherent with each other: everything produced and consumed
// within the launch (x, q, this step's k and v, the attention partials and output, the SwiGLU output) is written
// with device-scope stores and read with device-scope loads (the sc1 cache policy), which do not hit a stale
// line in a non-coherent L2. Weights and the K/V of earlier steps are read with ordinary loads. The K/V row at
// the step's position is also stored to the cache, but the sweep takes this step's k and v from the device-scope
// copy, so a chunk staged before they were written is patched in LDS.
//
// Grid barrier i, with flags and no atomics (device-scope atomics on one address serialize at close to a
// microsecond each on this GPU): wave 0 of every block finishes its epilogue stores, waits for them (vmcnt 0)
// and stores the barrier's generation into its arrival flag; then every block polls all 256 flags (one 16-byte
// load per lane). The generation is epoch x (5 L + 1) + i + 1, with the epoch read at the start and advanced by
// block 0 at the end, so flags never need clearing and a recorded graph replays without host work. A block that waits longer than the
// limit (a slot word; 2 s by default) raises ERR_BARRIER and the abort flag; from then on no block waits, so
// every wave exits (the step's results are then void).
//
// GEMV phases. A phase's outputs are split evenly over the blocks (units: output rows, or rotary / gate-up row
// pairs). Within a block the 8 waves split the inputs into KS slices of whole 512-element chunks (KS = 8 when the
// input width allows) and the rows into 8 / KS groups, so each lane holds the activation of its slice in
// registers and every wave streams the same number of bytes. A wave streams its rows in batches of up to 16
// 16-byte loads per lane, two batches in flight; after each batch a transposing butterfly leaves every row's
// wave total in one set of lanes (RB - 1 + log2(64 / RB) shuffles for RB rows), and the KS slices are summed in
// slice order from LDS in the epilogue. All orders are fixed, so a replay reproduces an eager launch bit for bit.
#include "ds3_device.h"

namespace ds3 {

namespace {

constexpr int kFW = 8;                 // waves per block
constexpr int kFT = 64 * kFW;          // threads per block
constexpr int kSc1 = 16;               // cache-policy bits of a buffer load: sc1 (device-scope coherent)
constexpr int kNt = 2;                 // cache-policy bits of a buffer load: nt (streamed once)
constexpr int kNL = 8;                 // 16-byte weight loads per lane per batch, at most (two batches in flight)
constexpr int kRsrcWord3 = 0x00020000; // buffer resource word 3: raw 32-bit data (gfx9 family)

enum { PH_QKV = 0, PH_ATTN, PH_O, PH_GU, PH_DOWN, PH_HEAD };

// MC_: a split sweeps several staged chunks (cap above S TC); a separate instantiation, so the one-chunk kernel
// carries no chunk loop
template <int D_, int F_, int HD_, int NQ_, int NKV_, int TC_, bool MC_ = false>
struct Shape {
  static constexpr int D = D_, F = F_, HD = HD_, NQ = NQ_, NKV = NKV_, G = NQ_ / NKV_, TC = TC_;
  static constexpr bool MC = MC_;
  static constexpr int QW = NQ * HD;                 // q width, the o-projection's input
  static constexpr int S = kFusedBlocks / NKV;       // attention splits per kv head: one (kv head, split) per block
  static constexpr int KB = TC * HD * 2;             // bytes of one staged K chunk (and of its V^T chunk)
  // the stage area: the K and V^T chunks, and between the sweep and the next staging two gate/up batches of every
  // wave (8 rows x 1 KB each): at least 128 KB
  static constexpr int SB = 2 * KB > 128 * 1024 ? 2 * KB : 128 * 1024;
  static constexpr int WST = kFW * G * (HD + 2);     // attention wave states
  static constexpr int UNI = WST > kFW * 520 ? WST : kFW * 520;
  static constexpr int QU = (G + 2) * HD / 2;        // QKV units (rotary / v row pairs) of one kv-head group
  static_assert(kFusedBlocks % NKV == 0 && S <= 64, "splits per kv head");
  static_assert(QU % S == 0, "a group's QKV units split evenly over its blocks");
  static_assert(TC % 32 == 0 && TC / 32 <= kFW && TC >= 128, "a chunk is 32 positions per wave");
  static_assert(KB % (1024 * kFW) == 0, "a chunk's 1 KB staging instructions split evenly over the waves");
  static_assert(G >= 1 && G <= 16 && (HD == 64 || HD == 128), "group and head width");
};

// Geometry of a GEMV phase (compile time).
template <class SH, int PH>
struct Geo {
  static constexpr int K = PH == PH_O ? SH::QW : (PH == PH_DOWN ? SH::F : SH::D);
  static constexpr int C = K / 512;                                  // 512-element chunks (64 lanes x 8)
  static constexpr int KS = C % 8 == 0 ? 8 : (C % 4 == 0 ? 4 : (C % 2 == 0 ? 2 : 1));
  static constexpr int RS = kFW / KS;                                // row groups
  static constexpr int CW = C / KS;                                  // chunks per wave
  static constexpr bool PAIRS = PH == PH_QKV || PH == PH_GU;
  static constexpr bool NORM = PH == PH_QKV || PH == PH_GU || PH == PH_HEAD;
  static constexpr int UNITS = PH == PH_QKV ? (SH::NQ + 2 * SH::NKV) * SH::HD / 2
                                            : (PH == PH_GU ? SH::F : (PH == PH_HEAD ? 0 : SH::D));
  static constexpr int RPB = PH == PH_HEAD ? 0 : UNITS / kFusedBlocks * (PAIRS ? 2 : 1);   // rows per block
  static constexpr int RW = RPB / RS;                                                    // rows per wave
  static constexpr int NBT = PH == PH_HEAD ? 0 : 2 * ((RW * CW + 2 * kNL - 1) / (2 * kNL));   // batches (even)
  static constexpr int RB = PH == PH_HEAD ? kNL / CW : (RW + NBT - 1) / NBT;                 // rows per batch
  static constexpr int NL = RB * CW;                                                     // loads per batch
  static constexpr int RBP = RB <= 1 ? 1 : RB <= 2 ? 2 : RB <= 4 ? 4 : RB <= 8 ? 8 : 16;
  static constexpr int LOG = RBP == 1 ? 0 : RBP == 2 ? 1 : RBP == 4 ? 2 : RBP == 8 ? 3 : 4;
  // gate/up: batches 2 .. 2 + NLB - 1 of every wave travel through the LDS stage area (free between the attention
  // sweep and the next layer's K/V staging; at least 128 KB, so two batches fit at both shapes), loaded while the
  // attention and o-projection phases wait on their barriers, when HBM would otherwise idle (1B shape: 599 -> 586 us
  // per step on MI355X). 1 KB slots; wave w's in slots w, w + 8, w + 16, ...
  static constexpr int SLOTS_PER_WAVE = SH::SB / 1024 / kFW;
  // (the loop then runs 1 + ceil((NBT - 2 - NLB) / 2) iterations, and the next layer's K/V staging takes one per
  // two of its NIW instructions per wave: fewer LDS batches where that would not fit)
  static constexpr int NIW = SH::KB / 1024 / kFW;
  static constexpr int NLB0 = (PH == PH_GU && CW == 1) ? (SLOTS_PER_WAVE / RB < 2 ? SLOTS_PER_WAVE / RB : 2) : 0;
  static constexpr int fit(int n) { return n <= 0 ? 0 : (1 + (NBT - 1 - n) / 2 >= NIW / 2 ? n : fit(n - 1)); }
  static constexpr int NLB = fit(NLB0);
  static_assert(NLB == 0 || (NBT >= 2 + NLB && 1 + (NBT - 1 - NLB) / 2 >= NIW / 2),
                "the batches after the LDS ones leave a loop iteration for every K/V staging step");
  static_assert(C * 512 == K && KS * CW == C, "input width must be whole 512-element chunks");
  static_assert(NL >= 1 && NL <= kNL && RB <= 16, "a batch is at most kNL loads per lane");
  static_assert(PH == PH_HEAD || UNITS % kFusedBlocks == 0, "units split evenly over the blocks");
  static_assert(PH == PH_HEAD || (RPB % RS == 0 && RW >= 1), "rows split evenly over the row groups");
  static_assert(PH == PH_HEAD || PH == PH_GU || UNITS / kFusedBlocks <= 64, "one epilogue lane per unit");
  static_assert(PH != PH_GU || UNITS / kFusedBlocks <= 64, "one epilogue lane per gate/up pair");
};

// The o-projection's first two batches are issued by waves 1-7 as the attention sweep starts when they are small
// (at most 32 KB per block: they land within the sweep); larger ones would hold the block barriers that follow the
// sweep (each waits for every outstanding load of its wave), so they go out after the split's partial is stored.
template <class SH>
constexpr bool kEarlyO = 2 * Geo<SH, PH_O>::NL * 1024 * (kFW - 1) <= 32 * 1024;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, kRsrcWord3);
}
// 16 bytes at a byte offset, read at device scope
__device__ __forceinline__ u32x4 ld_dev16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSc1);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_dev(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every memory operation this wave issued, the stores included, has completed
__device__ __forceinline__ void wait_all() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A value the compiler must treat as unknown at this point. Address arithmetic that repeats every layer is
// otherwise hoisted out of the layer loop as hundreds of loop-invariant offsets, which do not fit the registers.
__device__ __forceinline__ int opaque_v(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ int opaque_s(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
template <class T>
__device__ __forceinline__ T* opaque_p(T* v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Lanes l and l + 32 (swap32), or l and l + 16 within each half (swap16), exchange: after the swap, lanes below
// the partner hold x of both lanes and lanes above hold y of both, so their sum is the pair's x total in the
// lower lane and the pair's y total in the upper one (one permlane swap and one add per pair of values).
__device__ __forceinline__ float swap_sum32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// RBP values per lane -> the wave total of value (lane >> (6 - log2 RBP)), identical in the lanes that hold it.
// Halving steps, from lane bit 5 down: the lanes whose bit is clear keep the lower half of the values and add the
// partner's lower half, the others the upper half. Bits 5 and 4 use the permlane swaps; bits 3 and 2 the row and
// half-row mirror DPP permutations (the partner differs in lower bits too, which the closing sum over those bits
// absorbs). Every partial sum is formed in the same order on every run.
template <int RBP>
__device__ __forceinline__ float transpose_reduce(float (&a)[RBP], int lane) {
  constexpr int LOG = RBP == 1 ? 0 : RBP == 2 ? 1 : RBP == 4 ? 2 : RBP == 8 ? 3 : 4;
  if constexpr (LOG >= 1) {
#pragma unroll
    for (int k = 0; k < RBP / 2; ++k) a[k] = swap_sum32(a[k], a[k + RBP / 2]);
  }
  if constexpr (LOG >= 2) {
#pragma unroll
    for (int k = 0; k < RBP / 4; ++k) a[k] = swap_sum16(a[k], a[k + RBP / 4]);
  }
  if constexpr (LOG >= 3) {
    const bool up = (lane & 8) != 0;
#pragma unroll
    for (int k = 0; k < RBP / 8; ++k) {
      const float send = up ? a[k] : a[k + RBP / 8];
      a[k] = (up ? a[k + RBP / 8] : a[k]) + dpp_mov<0x140>(send);   // row_mirror: lane i <-> 15 - i
    }
  }
  if constexpr (LOG >= 4) {
    const bool up = (lane & 4) != 0;
    const float send = up ? a[0] : a[1];
    a[0] = (up ? a[1] : a[0]) + dpp_mov<0x141>(send);   // row_half_mirror: lane i <-> 7 - i
  }
  return group_sum<(64 >> LOG)>(a[0]);
}

template <int KS>
__device__ __forceinline__ float norm_scale(const float* ssq, int K, float eps) {
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) t += ssq[k];
  return 1.0f / sqrtf(t / (float)K + eps);
}

// QKV unit u: segment (0 q, 1 k, 2 v), head and element; rows of the packed Q|K|V matrix
template <class SH>
struct QkvUnit {
  int seg, head, idx, row0, row1;
  // unit lu (0 .. QU - 1) of kv-head group g: the rotary pairs of its G q heads, then of its k head, then the row
  // pairs of its v head. The S blocks of group g produce exactly the q, k and v its attention reads.
  __device__ __forceinline__ static int of_group(int g, int lu) {
    constexpr int half = SH::HD / 2, nqg = SH::G * half;
    if (lu < nqg) return g * nqg + lu;
    if (lu < nqg + half) return SH::NQ * half + g * half + (lu - nqg);
    return (SH::NQ + SH::NKV) * half + g * half + (lu - nqg - half);
  }
  __device__ __forceinline__ explicit QkvUnit(int u) {
    constexpr int half = SH::HD / 2, nqp = SH::NQ * half, nkp = SH::NKV * half;
    if (u < nqp) {
      seg = 0; head = u / half; idx = u % half;
      row0 = head * SH::HD + idx; row1 = row0 + half;
    } else if (u < nqp + nkp) {
      const int pp = u - nqp;
      seg = 1; head = pp / half; idx = pp % half;
      row0 = SH::QW + head * SH::HD + idx; row1 = row0 + half;
    } else {
      const int pv = 2 * (u - nqp - nkp);
      seg = 2; head = pv / SH::HD; idx = pv % SH::HD;
      row0 = SH::QW + SH::NKV * SH::HD + pv; row1 = row0 + 1;
    }
  }
};

struct NoNext {
  __device__ __forceinline__ void issue(int, u32x4 (&)[kNL]) const {}
};

// One GEMV phase as seen by one wave: its block's units, its rows and its input slice.
template <class SH, int PH>
struct GemvPhase {
  using GE = Geo<SH, PH>;
  const uint16_t* w;
  int u0, nunits, rb;   // block: first unit (QKV: within its group), units, rows (2 per pair unit)
  int grp;              // QKV: the block's kv-head group
  int r0, r1, ks;       // wave: rows [r0, r1) of the block, input slice
  int nb;               // batches (even)
  int lane;
  const int* rtab;      // QKV: byte offsets of the block's weight rows (LDS, the same for every layer)

  __device__ __forceinline__ void init(const void* w_, int units_total, int b, int wid, int lane_,
                                       const int* rtab_ = nullptr) {
    w = reinterpret_cast<const uint16_t*>(w_);
    rtab = rtab_;
    lane = lane_;
    const int units = PH == PH_HEAD ? units_total : GE::UNITS;
    if constexpr (PH == PH_QKV) {   // block (g, s) of group g = b / S: units [s QU / S, (s + 1) QU / S) of g
      grp = b / SH::S;
      nunits = SH::QU / SH::S;
      u0 = (b % SH::S) * nunits;
    } else {
      grp = 0;
      u0 = (int)(((long long)b * units) / kFusedBlocks);
      nunits = (int)(((long long)(b + 1) * units) / kFusedBlocks) - u0;
    }
    rb = nunits * (GE::PAIRS ? 2 : 1);
    const int rg = wid / GE::KS;
    ks = wid % GE::KS;
    r0 = rg * rb / GE::RS;
    r1 = (rg + 1) * rb / GE::RS;
    nb = PH == PH_HEAD ? 2 * ((r1 - r0 + 2 * GE::RB - 1) / (2 * GE::RB)) : GE::NBT;
  }

  // weight row of block row br
  __device__ __forceinline__ int row_of(int br) const {
    if constexpr (PH == PH_QKV) {
      const QkvUnit<SH> q(QkvUnit<SH>::of_group(grp, u0 + (br >> 1)));
      return (br & 1) ? q.row1 : q.row0;
    } else if constexpr (PH == PH_GU) {
      const int j = u0 + (br >> 1);
      return (br & 1) ? SH::F + j : j;
    } else {
      return u0 + br;
    }
  }

  // batch i into buf: rows past the wave's last are clamped to it (their sums are dropped)
  // (buffer loads: the row offset rides in a scalar register, the lane offset is one vector register)
  __device__ __forceinline__ void issue(int i, u32x4 (&buf)[kNL]) const {
    const auto wr = make_rsrc(opaque_p(w));
    const int lo = opaque_v(lane * 16 + ks * (GE::CW * 1024));
    const int rfirst = opaque_s(r0 + i * GE::RB);
#pragma unroll
    for (int j = 0; j < GE::RB; ++j) {
      // (no clamp where the wave's rows are whole batches)
      const int br = (PH != PH_HEAD && GE::NBT * GE::RB == GE::RW) ? rfirst + j : min(rfirst + j, r1 - 1);
      if constexpr (PH == PH_QKV) {   // (the table's offset rides in the lane offset)
        const int vo = lo + rtab[br];
#pragma unroll
        for (int c = 0; c < GE::CW; ++c)
          buf[j * GE::CW + c] = __builtin_amdgcn_raw_buffer_load_b128(wr, vo, c * 1024, kNt);
      } else {
        const int so = row_of(br) * (GE::K * 2);
#pragma unroll
        for (int c = 0; c < GE::CW; ++c)
          buf[j * GE::CW + c] = __builtin_amdgcn_raw_buffer_load_b128(wr, lo, so + c * 1024, kNt);
      }
    }
  }

  // Gate/up only: load every wave's LDS batches (weights of batches 2 .. 2 + NLB - 1) into the stage area; wave
  // `wid` (1..7) takes slots wid - 1, wid + 6, ... of the NLB RB 8 slots (slot w + 8 (bb RB + j): row j of LDS
  // batch bb of wave w).
  __device__ __forceinline__ void lds_prefetch(unsigned char* stage, int wid) const {
    constexpr int NS = GE::NLB * GE::RB * kFW;
    for (int k = wid - 1; k < NS; k += kFW - 1) {
      const int w = k % kFW, m = k / kFW, bb = m / GE::RB, j = m % GE::RB;
      const int rg = w / GE::KS, kw = w % GE::KS;
      const int rw0 = rg * rb / GE::RS, rw1 = (rg + 1) * rb / GE::RS;
      const int br = min(rw0 + (2 + bb) * GE::RB + j, rw1 - 1);
      const uint16_t* src = w_row(br) + kw * (GE::CW * 512) + lane * 8;
      __builtin_amdgcn_global_load_lds((global_cptr)src, (lds_ptr)(stage + (size_t)(w + kFW * m) * 1024), 16, 0,
                                       kNt);
    }
  }
  __device__ __forceinline__ const uint16_t* w_row(int br) const {
    return opaque_p(w) + (size_t)row_of(br) * GE::K;
  }

  // dot products of LDS batch bb's rows (this wave's slots) with the activation slice
  __device__ __forceinline__ void fma_lds(const unsigned char* stage, int bb, int wid, const float (&xa)[GE::CW][8],
                                         float (&acc)[GE::RBP]) const {
#pragma unroll
    for (int j = 0; j < GE::RBP; ++j) acc[j] = 0.f;
#pragma unroll
    for (int j = 0; j < GE::RB; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (size_t)(wid + kFW * (bb * GE::RB + j)) * 1024 + lane * 16);
      float f[8];
      Pack<uint16_t>::widen(v, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j] = fmaf(f[e], xa[0][e], acc[j]);
    }
  }

  // dot products of batch i's rows with the activation slice (per lane)
  __device__ __forceinline__ void fma(const u32x4 (&buf)[kNL], const float (&xa)[GE::CW][8],
                                     float (&acc)[GE::RBP]) const {
#pragma unroll
    for (int j = 0; j < GE::RBP; ++j) acc[j] = 0.f;
#pragma unroll
    for (int j = 0; j < GE::RB; ++j)
#pragma unroll
      for (int c = 0; c < GE::CW; ++c) {
        float f[8];
        Pack<uint16_t>::widen(buf[j * GE::CW + c], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j] = fmaf(f[e], xa[c][e], acc[j]);
      }
  }

  // wave totals of batch i's rows -> red[ks][row]
  __device__ __forceinline__ void reduce(int i, float (&acc)[GE::RBP], float* red) const {
    const float v = transpose_reduce<GE::RBP>(acc, lane);
    const int vi = lane >> (6 - GE::LOG);
    const int br = r0 + i * GE::RB + vi;
    if ((lane & ((64 >> GE::LOG) - 1)) == 0 && vi < GE::RB && br < r1) red[ks * rb + br] = v;
  }
};

// Stage positions [jb, jb + TC) of kv head g (row 0) into LDS: K rows (16-byte pieces swizzled by position) and
// the transposed V rows (8-position groups swizzled by element), with 1 KB global-to-LDS instructions; lane l of
// instruction k fills slot 64 k + l and picks its source accordingly.
template <class SH>
__device__ __forceinline__ void stage_chunk(const FusedParams& p, int layer, int g, int jb, unsigned char* stage,
                                            int wid, int lane, int i0, int i1) {
  constexpr int HD = SH::HD, TC = SH::TC, CPR = HD / 8, NIW = SH::KB / 1024 / kFW;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(p.kv.k) + (size_t)layer * p.kv.layer_stride;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(p.kv.v) + (size_t)layer * p.kv.layer_stride;
  const int cap = p.cap;
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    if (i < i0 || i >= i1) continue;   // (uniform)
    const int k = i * kFW + wid;
    const int slot = opaque_v(k * 64 + lane);
    const int pj = slot / CPR;
    const int c = (slot % CPR) ^ kswz<CPR>(pj);
    const int jk = min(jb + pj, cap - 1);
    const int d = slot / (TC / 8);
    const int cv = (slot % (TC / 8)) ^ (d & 15);
    const int jv = min(jb + 8 * cv, cap - 8);
    const uint16_t* ks = Kb + ((size_t)g * cap + jk) * HD + 8 * c;
    const uint16_t* vs = Vb + ((size_t)g * HD + d) * cap + jv;
    __builtin_amdgcn_global_load_lds((global_cptr)ks, (lds_ptr)(stage + (size_t)k * 1024), 16, 0, kNt);
    __builtin_amdgcn_global_load_lds((global_cptr)vs, (lds_ptr)(stage + SH::KB + (size_t)k * 1024), 16, 0, kNt);
  }
}

// Shared per-block state in LDS
template <class SH>
struct Smem {
  unsigned char* stage;   // [K chunk | V^T chunk]
  float* uni;             // GEMV row partials [KS][rows] / attention wave states [8][G][HD + 2]
  float* ssq;             // [KS] RMSNorm sums of squares
  int* flags;             // [0] abort seen, [1] generation of the last attention merge done by wave 0,
                          // [2] generation of the last GEMV epilogue whose stores wave 0 has issued
};

// Bounded wait of wave 0 for `done()` (evaluated by every lane; the result must agree across the wave): false
// when the wait gave up (abort flag seen, or the limit passed -- then the error bit and the abort flag are raised).
template <class F>
__device__ __forceinline__ bool spin_until(const FusedParams& p, int* flags, F&& done) {
  const unsigned sp = (unsigned)p.slots[SlotLayout{1}.spin()];
  const long long limit = sp ? (long long)sp : kFusedSpinTicks;
  const long long t0 = wall_clock64();
  for (;;) {
    if (done()) return true;
    if (ld_dev(&p.sync[1]) != 0u) break;
    if (wall_clock64() - t0 > limit) {
      if ((threadIdx.x & 63) == 0) {
        raise_error(p.status, ERR_BARRIER);
        st_dev(&p.sync[1], 1u);
      }
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if ((threadIdx.x & 63) == 0) flags[0] = 1;
  return false;
}

// End of a phase, wave 0 only (after its epilogue stores): wait for them, signal arrival at barrier `bar`, issue
// this wave's first batches of the next phase and wait for every block. (Wave 0 polls with vector loads, and a
// wave can only wait for its oldest loads first, so its polls also wait for those batches.)
//
// Every block polls all 256 arrival flags itself (four per lane, one hop), and a flag already at a later
// generation (its block has passed this barrier and reached the next) counts as arrived. (A collector block that
// polls the arrivals and raises one release flag per XCD -- two hops, 8 x 32 pollers on single cache lines --
// measured 2.3% slower per step at the 2048-wide shape and 1.1-1.9% slower at the 4096-wide one.)
template <class PF>
__device__ __forceinline__ void arrive_and_wait(const FusedParams& p, unsigned gen0, int bar, int lane, int* flags,
                                                PF&& prefetch) {
  wait_all();
  const long long t0 = wall_clock64();
  const unsigned gen = gen0 + (unsigned)bar + 1u;
  if (!flags[0]) {
    if (lane == 0) st_dev(&p.sync[kSyncArrive + blockIdx.x], gen);
    // (the weights go out first: the polls then wait for them too, but the release rarely comes sooner)
    prefetch();
    const auto rf = make_rsrc(p.sync + kSyncArrive);
    spin_until(p, flags, [&]() __attribute__((always_inline)) {
      const u32x4 v = ld_dev16(rf, lane * 16);
      return __all((int)(v.x - gen) >= 0 && (int)(v.y - gen) >= 0 && (int)(v.z - gen) >= 0 &&
                   (int)(v.w - gen) >= 0) != 0;
    });
  } else {
    prefetch();
  }
  if (lane == 0 && p.trace) {   // this block's arrival and release times at barrier `bar`
    p.trace[((size_t)bar * kFusedBlocks + blockIdx.x) * 2] = (unsigned long long)t0;
    p.trace[((size_t)bar * kFusedBlocks + blockIdx.x) * 2 + 1] = (unsigned long long)wall_clock64();
  }
}

// End of the QKV phase, wave 0 only (after its epilogue stores): wait for them and raise this block's arrival flag
// to the phase's generation gen0 + bar + 1. No grid barrier follows: each kv-head group's attention needs only the
// q, k and v its own S blocks produce, so it waits for those S flags alone (group_wait).
__device__ __forceinline__ void group_arrive(const FusedParams& p, unsigned gen0, int bar, int lane, const int* flags) {
  wait_all();
  if (!flags[0] && lane == 0) st_dev(&p.sync[kSyncArrive + blockIdx.x], gen0 + (unsigned)bar + 1u);
  if (lane == 0 && p.trace) p.trace[((size_t)bar * kFusedBlocks + blockIdx.x) * 2] = (unsigned long long)wall_clock64();
}

// Wave 0: wait until the S blocks of kv-head group g have raised their arrival flags to generation gen0 + bar + 1
// or later (a block of the group may already have moved on to the next barrier's generation).
template <int S>
__device__ __forceinline__ void group_wait(const FusedParams& p, unsigned gen0, int bar, int g, int lane, int* flags) {
  const unsigned gen = gen0 + (unsigned)bar + 1u;
  if (!flags[0]) {
    const unsigned* f = p.sync + kSyncArrive + g * S;
    spin_until(p, flags, [&]() __attribute__((always_inline)) {
      return __all(lane >= S || (int)(ld_dev(f + min(lane, S - 1)) - gen) >= 0) != 0;
    });
  }
  if (lane == 0 && p.trace)
    p.trace[((size_t)bar * kFusedBlocks + blockIdx.x) * 2 + 1] = (unsigned long long)wall_clock64();
}

// Greedy candidate of the wave: the (value, index) maximum over its lanes, in every lane.
__device__ __forceinline__ void pick_reduce(float& bv, int& bi) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (pick_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
}

// After the head, wave 0 of every block (its candidate stored): arrive at the closing barrier (generation
// gen0 + 5 L + 1); block 0 waits for every block, picks the step's token from the 256 candidates (the first index
// of the largest logit; all NaN -> 0), writes it into the token slot and pos + 1 into the position slot for the
// next launch (every block read the slots at its start), records the pick and the non-finite flag under the
// chain counter, clears the flag and advances the counter. The other blocks just leave.
__device__ __forceinline__ void final_pick(const FusedParams& p, unsigned gen0, int lane, int* flags) {
  wait_all();
  const unsigned gen = gen0 + (unsigned)(kFusedPhases * p.n_layers) + 1u;
  if (flags[0]) return;
  if (lane == 0) st_dev(&p.sync[kSyncArrive + blockIdx.x], gen);
  if (blockIdx.x != 0) return;
  const auto ra = make_rsrc(p.sync + kSyncArrive);
  const bool ok = spin_until(p, flags, [&]() __attribute__((always_inline)) {
    const u32x4 v = ld_dev16(ra, lane * 16);
    return __all(v.x == gen && v.y == gen && v.z == gen && v.w == gen) != 0;
  });
  if (!ok) return;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const float* pv = p.part;
  const unsigned* pi = reinterpret_cast<const unsigned*>(p.part) + kFusedBlocks;
#pragma unroll
  for (int k = 0; k < kFusedBlocks / 64; ++k) {
    const int blk = lane * (kFusedBlocks / 64) + k;
    const float v = ld_dev(pv + blk);
    const int i = (int)ld_dev(pi + blk);
    if (pick_better(v, i, bv, bi)) { bv = v; bi = i; }
  }
  pick_reduce(bv, bi);
  if (lane == 0) {
    if (bi >= p.vocab) bi = 0;
    const SlotLayout sl{1};
    const int step = p.slots[sl.chain()];
    p.ids[step % p.max_chain] = bi;
    p.chain_flags[step % p.max_chain] = ld_dev(&p.status->nonfinite) ? 1u : 0u;
    st_dev(&p.status->nonfinite, 0u);
    p.slots[sl.token()] = bi;
    p.slots[sl.pos()] = p.slots[sl.pos()] + 1;
    p.slots[sl.chain()] = step + 1;
  }
}

// After the block-wide barrier that follows arrive_and_wait: block 0 stamps the clock.
__device__ __forceinline__ void after_barrier(const FusedParams& p, int bar) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.clocks) p.clocks[bar + 1] = (unsigned long long)wall_clock64();
}

// A GEMV phase from the activation loads to the barrier. `x_embed` (layer 0 only): the residual stream is still
// the embedding row, read from the (constant) table instead of x. `extra(it)` runs after loop iteration `it`.
template <class SH, int PH, class NX, class EXTRA>
__device__ __forceinline__ void run_gemv(const FusedParams& p, const GemvPhase<SH, PH>& ph, const NX& nx,
                                         EXTRA&& extra, u32x4 (&A)[kNL], u32x4 (&B)[kNL], const Smem<SH>& sm,
                                         const float* act, const float* gain, const uint16_t* x_embed, int layer,
                                         int pos, bool pos_ok, int wid, int lane, unsigned gen0) {
  using GE = Geo<SH, PH>;
  constexpr int HD = SH::HD, half = SH::HD / 2;
  float* red = sm.uni;
  constexpr int BAR = PH == PH_QKV ? 0 : PH == PH_O ? 2 : PH == PH_GU ? 3 : 4;
  // sub-phase clock (wave 0 of each block, when tracing): start, first batch consumed, batches done, block done
  unsigned long long* st = (p.trace2 && wid == 0 && lane == 0 && PH != PH_HEAD)
                               ? p.trace2 + ((size_t)(kFusedPhases * layer + BAR) * kFusedBlocks + blockIdx.x) * 8
                               : nullptr;
  if (st) st[0] = (unsigned long long)wall_clock64();
  // (every buffer below is the same for each layer: opaque copies keep its addresses out of the layer loop)
  act = opaque_p(act);
  float* const xb = opaque_p(p.x);

  // ---- 1. this wave's activation slice (times the RMSNorm gain), and its sum of squares
  float xa[GE::CW][8];
  {
    const bool from_embed = PH == PH_QKV && x_embed != nullptr;
    const auto rs = make_rsrc(act);
    const int ebase = opaque_v(ph.ks * GE::CW * 512 + lane * 8);
#pragma unroll
    for (int c = 0; c < GE::CW; ++c) {
      const int e0 = ebase + c * 512;
      if (from_embed) {
        Pack<uint16_t>::widen(*reinterpret_cast<const u32x4*>(x_embed + e0), xa[c]);
      } else {
        const u32x4 a = ld_dev16(rs, e0 * 4), b = ld_dev16(rs, e0 * 4 + 16);
        xa[c][0] = __uint_as_float(a.x); xa[c][1] = __uint_as_float(a.y);
        xa[c][2] = __uint_as_float(a.z); xa[c][3] = __uint_as_float(a.w);
        xa[c][4] = __uint_as_float(b.x); xa[c][5] = __uint_as_float(b.y);
        xa[c][6] = __uint_as_float(b.z); xa[c][7] = __uint_as_float(b.w);
      }
    }
    if constexpr (GE::NORM) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < GE::CW; ++c) {
        const int e0 = ebase + c * 512;
        const float4 g0 = *reinterpret_cast<const float4*>(gain + e0);
        const float4 g1 = *reinterpret_cast<const float4*>(gain + e0 + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss = fmaf(xa[c][e], xa[c][e], ss);
          xa[c][e] *= gv[e];
        }
      }
      const float t = wave_total(ss);
      if (wid < GE::KS && lane == 0) sm.ssq[ph.ks] = t;
    }
  }

  // ---- 2. wave 0: operands of its epilogue (one unit per lane)
  float eo_a = 0.f, eo_b = 0.f;
  if constexpr (PH == PH_QKV) {
    if (wid == 0 && lane < ph.nunits) {
      const QkvUnit<SH> q(QkvUnit<SH>::of_group(ph.grp, ph.u0 + lane));
      if (q.seg != 2) {
        const float2 cs = reinterpret_cast<const float2*>(opaque_p(p.rope))[(size_t)pos * half + q.idx];
        eo_a = cs.x;
        eo_b = cs.y;
      }
    }
  } else if constexpr (PH == PH_O || PH == PH_DOWN) {
    if (wid == 0 && lane < ph.nunits) {
      const int row = ph.u0 + lane;
      eo_a = (PH == PH_O && x_embed != nullptr) ? widen1(x_embed[row]) : ld_dev(xb + row);
    }
  }
  // ---- 3. batches: two in flight; each freed buffer takes the next batch
  // (a buffer is refilled as soon as its dot products have read it, before the reduction's shuffles)
  // (batch i in A and i + 1 in B; each is refilled with the batch two places on, skipping the LDS batches)
  constexpr int NLB = GE::NLB;
  auto step = [&](int i, int it) __attribute__((always_inline)) {
    float acc[GE::RBP];
    ph.fma(A, xa, acc);
    if (i == 0 && st) st[1] = (unsigned long long)wall_clock64();
    const int nx_a = i + 2 + (i == 0 ? NLB : 0);
    if (nx_a < ph.nb) ph.issue(nx_a, A);
    ph.reduce(i, acc, red);
    if (i + 1 < ph.nb) {
      ph.fma(B, xa, acc);
      const int nx_b = i + 3 + (i == 0 ? NLB : 0);
      if (nx_b < ph.nb) ph.issue(nx_b, B);
      ph.reduce(i + 1, acc, red);
    }
    if constexpr (NLB > 0) {
      if (i == 0) {   // the LDS batches, then the stage area is free for this wave's K/V staging
#pragma unroll
        for (int bb = 0; bb < NLB; ++bb) {
          ph.fma_lds(sm.stage, bb, wid, xa, acc);
          ph.reduce(2 + bb, acc, red);
        }
      }
    }
    extra(it);
  };
  if constexpr (NLB > 0) {
    step(0, 0);
#pragma nounroll
    for (int i = 2 + NLB, it = 1; i < ph.nb; i += 2, ++it) step(i, it);
  } else if constexpr (GE::NBT > 4) {   // (long loops stay rolled: one copy of the body in the instruction cache)
#pragma nounroll
    for (int i = 0; i < ph.nb; i += 2) step(i, i / 2);
  } else {
    for (int i = 0; i < ph.nb; i += 2) step(i, i / 2);
  }
  if (st) st[2] = (unsigned long long)wall_clock64();
  __syncthreads();
  if (st) st[3] = (unsigned long long)wall_clock64();

  // ---- 4. wave 0: slice sums in slice order, epilogue, barrier. Waves 1-7 issue the next phase's first two
  // batches once wave 0 has issued its epilogue stores (at a saturated memory system an issue can stall for
  // microseconds, so they must not sit between wave 0 and its barrier arrival; and a CU serves its memory requests
  // roughly in issue order, so stores issued after ~100 KB of loads complete only once those loads have landed).
  constexpr bool ORDERED = PH == PH_O || PH == PH_GU || PH == PH_DOWN;
  const int epi_tok = (int)(gen0 + (unsigned)(kFusedPhases * layer + BAR) + 1u);
  if (wid != 0) {
    if constexpr (ORDERED)   // (wave 0 has issued its epilogue stores: they do not queue behind these batches)
      while (__hip_atomic_load(&sm.flags[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != epi_tok)
        __builtin_amdgcn_s_sleep(1);
    nx.issue(0, A);
    nx.issue(1, B);
    if constexpr (PH == PH_O && Geo<SH, PH_GU>::NLB > 0)   // the gate/up LDS batches (loaded during attention) have
      __builtin_amdgcn_s_waitcnt(kVmcntChunk<2 * Geo<SH, PH_GU>::NL>());   // landed: the block barrier publishes them
  } else {
    float scale = 1.f;
    if constexpr (GE::NORM) scale = norm_scale<GE::KS>(sm.ssq, GE::K, p.eps);
    auto total = [&](int br) __attribute__((always_inline)) {
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < GE::KS; ++k) t += red[k * ph.rb + br];
      return t;
    };
    if constexpr (PH == PH_QKV) {
      if (lane < ph.nunits) {
        const QkvUnit<SH> q(QkvUnit<SH>::of_group(ph.grp, ph.u0 + lane));
        const float a = total(2 * lane) * scale, b = total(2 * lane + 1) * scale;
        float va = a, vb = b;
        if (q.seg != 2) {   // rotate the pair (element idx, element idx + hd/2) by the angles of pos
          va = a * eo_a - b * eo_b;
          vb = a * eo_b + b * eo_a;
        }
        if (q.seg == 0) {
          float* qh = opaque_p(p.q) + q.head * HD;
          st_dev(qh + q.idx, va);
          st_dev(qh + q.idx + half, vb);
        } else {
          const int e1 = q.idx + (q.seg == 1 ? half : 1);
          float* kn = opaque_p(p.kvnew) + (q.head * 2 + (q.seg - 1)) * HD;
          st_dev(kn + q.idx, va);
          st_dev(kn + e1, vb);
          if (pos_ok) {   // the cache entry for later steps (DynamicUpdateSlice at pos)
            uint16_t* base = reinterpret_cast<uint16_t*>(q.seg == 1 ? opaque_p(p.kv.k) : opaque_p(p.kv.v)) +
                             (size_t)layer * p.kv.layer_stride;
            if (q.seg == 1) {
              uint16_t* kr = base + ((size_t)q.head * p.cap + pos) * HD;
              kr[q.idx] = to_bf16(va);
              kr[e1] = to_bf16(vb);
            } else {
              base[((size_t)q.head * HD + q.idx) * p.cap + pos] = to_bf16(va);
              base[((size_t)q.head * HD + e1) * p.cap + pos] = to_bf16(vb);
            }
          }
        }
      }
    } else if constexpr (PH == PH_GU) {
      if (lane < ph.nunits) {
        const float a = total(2 * lane) * scale, b = total(2 * lane + 1) * scale;
        const float silu = a / (1.0f + expf(-a));
        st_dev(opaque_p(p.act) + ph.u0 + lane, silu * b);
      }
    } else if constexpr (PH == PH_O || PH == PH_DOWN) {
      if (lane < ph.nunits) st_dev(xb + ph.u0 + lane, eo_a + total(lane));
    } else {   // PH_HEAD: the logits, the non-finite flag, and this block's greedy candidate
      bool bad = false;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int u = lane; u < ph.nunits; u += 64) {
        const float v = total(u) * scale;
        opaque_p(p.logits)[ph.u0 + u] = v;
        bad |= !isfinite(v);
        if (pick_better(v, ph.u0 + u, bv, bi)) { bv = v; bi = ph.u0 + u; }
      }
      if (bad) atomicOr(&p.status->nonfinite, 1u);
      pick_reduce(bv, bi);
      if (lane == 0) {
        st_dev(opaque_p(p.part) + blockIdx.x, bv);
        st_dev(reinterpret_cast<unsigned*>(opaque_p(p.part)) + kFusedBlocks + blockIdx.x, (unsigned)bi);
      }
      if (p.slots[SlotLayout{1}.sample()] == 0) final_pick(p, gen0, lane, sm.flags);   // (else the sampler picks)
    }
    if constexpr (ORDERED)
      if (lane == 0) __hip_atomic_store(&sm.flags[2], epi_tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if constexpr (PH == PH_QKV) {
      group_arrive(p, gen0, kFusedPhases * layer, lane, sm.flags);
    } else if constexpr (PH != PH_HEAD) {
      arrive_and_wait(p, gen0, kFusedPhases * layer + (PH == PH_O ? 2 : PH == PH_GU ? 3 : 4), lane, sm.flags,
                      [&]() __attribute__((always_inline)) {
                        nx.issue(0, A);
                        nx.issue(1, B);
                      });
    }
  }
  if constexpr (PH != PH_HEAD) {
    // (waves 1-7 hold the next phase's first batches in flight: no vmcnt(0) here)
    barrier_lds();
    if constexpr (PH != PH_QKV)   // (the QKV phase closes with its group's wait, at the start of the attention)
      after_barrier(p, kFusedPhases * layer + (PH == PH_O ? 2 : PH == PH_GU ? 3 : 4));
  }
}

// The attention phase: block b sweeps split s = b % S of kv head g = b / S (positions [s TC, s TC + TC))
// for the G query heads of the group, on the matrix cores (as attn_mfma_kernel); each split stores its partial and
// raises its flag, and split 0's block of the kv head waits for all S flags and merges the splits in split order.
template <class SH, class NX, class GU>
__device__ __forceinline__ void run_attn(const FusedParams& p, const NX& nx, const GU& gu, u32x4 (&A)[kNL], u32x4 (&B)[kNL],
                                         const Smem<SH>& sm, int layer, int pos, bool pos_ok, int wid, int lane,
                                         unsigned gen0) {
  constexpr int HD = SH::HD, G = SH::G, TC = SH::TC, S = SH::S, CPR = HD / 8, KSQ = HD / 32, DT = HD / 16;
  const int tid = threadIdx.x, b = blockIdx.x;
  const int g = b / S, s = b % S;
  const int n = lane & 15, Lg = lane >> 4;
  float* wst = sm.uni;
  uint16_t* kl = reinterpret_cast<uint16_t*>(sm.stage);
  uint16_t* vl = reinterpret_cast<uint16_t*>(sm.stage + SH::KB);

  unsigned long long* st = (p.trace2 && tid == 0)
                               ? p.trace2 + ((size_t)(kFusedPhases * layer + 1) * kFusedBlocks + blockIdx.x) * 8
                               : nullptr;
  if (st) st[0] = (unsigned long long)wall_clock64();
  // ---- wave 0 brings the group's q heads and this step's k and v into LDS once for the block (every block of the
  // kv head reads the same device-scope lines, so one read per block, not one per wave)
  float* qs = sm.uni;                  // [G][HD] q, then [2][HD] this step's k and v
  if (wid == 0) {
    group_wait<S>(p, gen0, kFusedPhases * layer, g, lane, sm.flags);   // the group's q, k and v are stored
    const auto rq = make_rsrc(opaque_p(p.q) + g * G * HD);
    const auto rk = make_rsrc(opaque_p(p.kvnew) + g * 2 * HD);
    for (int i = lane; i < G * HD / 4; i += 64)
      *reinterpret_cast<u32x4*>(qs + 4 * i) = ld_dev16(rq, 16 * i);
    for (int i = lane; i < 2 * HD / 4; i += 64)
      *reinterpret_cast<u32x4*>(qs + G * HD + 4 * i) = ld_dev16(rk, 16 * i);
  }
  wait_all();   // (every wave: also its share of the chunk staged during the previous phases)
  __syncthreads();
  after_barrier(p, kFusedPhases * layer);
  if (st) st[1] = (unsigned long long)wall_clock64();

  // ---- q^T as the B operand (lane (n, Lg): head g G + n, elements 32 k + 8 Lg + 0..7, times 1/sqrt(hd) log2(e);
  // zero beyond G)
  bf16x8 qh[KSQ], ql[KSQ];
  {
    const float z = n < G ? p.scale * 1.4426950408889634f : 0.f;
    const float* qrow = qs + min(n, G - 1) * HD + 8 * Lg;
#pragma unroll
    for (int k = 0; k < KSQ; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(qrow + 32 * k);
      const float4 c = *reinterpret_cast<const float4*>(qrow + 32 * k + 4);
      const float v[8] = {a.x * z, a.y * z, a.z * z, a.w * z, c.x * z, c.y * z, c.z * z, c.w * z};
      split_hi_lo8(v, qh[k], ql[k]);
    }
  }
  const float kn = tid < HD ? qs[G * HD + tid] : 0.f, vn = tid < HD ? qs[G * HD + HD + tid] : 0.f;

  float m_run = -INFINITY;   // running max of head n (log2 domain)
  float lsum = 0.f;          // this lane's share of head n's weight sum
  f32x4 acc[DT];             // O[head 4 Lg + i][16 dt + n]
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The split's chunks of TC positions, interleaved over the splits (chunk c of split s starts at (c S + s) TC, so
  // the visible prefix spreads over every split). Chunk 0 was staged during the previous layer's gate/up phase; each
  // later one is loaded here once every wave has swept the one before (the stage area holds one chunk).
  const int nch = SH::MC ? p.split_len / TC : 1;
  for (int ch = 0; ch < nch; ++ch) {
    const int jb = (ch * S + s) * TC;
    if (ch > 0) {
      __syncthreads();   // (every wave is done with chunk c - 1 in LDS)
      if (p.slots[SlotLayout{1}.sweep()] == 0 || jb <= pos)
        stage_chunk<SH>(p, layer, g, jb, sm.stage, wid, lane, 0, SH::KB / 1024 / kFW);
      wait_all();
      __syncthreads();
    }
    // the row at pos: this step's k and v (the staged copy may predate their store)
    if (pos_ok && pos >= jb && pos < jb + TC && tid < HD) {
      const int pj = pos - jb;
      kl[(pj * CPR + ((tid >> 3) ^ kswz<CPR>(pj))) * 8 + (tid & 7)] = to_bf16(kn);
      vl[(tid * (TC / 8) + ((pj >> 3) ^ (tid & 15))) * 8 + (pj & 7)] = to_bf16(vn);
    }
    __syncthreads();
    if constexpr (kEarlyO<SH>) {   // a small o-projection prefetch streams during the last chunk's sweep
      if (ch == nch - 1 && wid != 0) {
        nx.issue(0, A);
        nx.issue(1, B);
      }
    }
    const int jw = jb + 32 * wid;   // first position of this wave's block of 32
    if (32 * wid < TC && jw <= pos) {
      f32x4 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int pj = 32 * wid + 8 * (n >> 2) + 4 * t + (n & 3);
#pragma unroll
        for (int kk = 0; kk < KSQ; ++kk) {
          const int c = 4 * kk + Lg;
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kl + (size_t)(pj * CPR + (c ^ kswz<CPR>(pj))) * 8));
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[kk], sc[t], 0, 0, 0);
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[kk], sc[t], 0, 0, 0);
        }
      }
      // lane (n, Lg): scores of head n at positions jw + 8 Lg + e, e = 4 t + i
      float sv[8];
      bool vis[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vis[e] = jw + 8 * Lg + e <= pos;
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
      float cr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cr[i] = __shfl(corr, 4 * Lg + i, 64);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dt][i] *= cr[i];
      const bool partial = jw + 31 > pos;
      uint32_t mk[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
        mk[q2] = (jw + 8 * Lg + 2 * q2 <= pos ? 0xFFFFu : 0u) | (jw + 8 * Lg + 2 * q2 + 1 <= pos ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + n;
        u32x4 bv = *reinterpret_cast<const u32x4*>(vl + (size_t)(d * (TC / 8) + ((4 * wid + Lg) ^ (d & 15))) * 8);
        if (partial) {   // hidden V rows never meet the matrix core (0 x NaN would be NaN)
          bv.x &= mk[0];
          bv.y &= mk[1];
          bv.z &= mk[2];
          bv.w &= mk[3];
        }
        const bf16x8 Bv = __builtin_bit_cast(bf16x8, bv);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, Bv, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, Bv, acc[dt], 0, 0, 0);
      }
    }
  }

  // ---- wave states to LDS (idle waves contribute max -inf, weight 0)
  {
    float lt = lsum + __shfl_xor(lsum, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * Lg + i;
      if (hh < G) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) wst[(wid * G + hh) * (HD + 2) + 16 * dt + n] = acc[dt][i];
      }
    }
    if (Lg == 0 && n < G) {
      wst[(wid * G + n) * (HD + 2) + HD] = m_run;
      wst[(wid * G + n) * (HD + 2) + HD + 1] = lt;
    }
  }
  __syncthreads();

  if (st) st[2] = (unsigned long long)wall_clock64();
  // ---- the 8 waves' states merged in wave order into this split's partial (outputs spread over all waves),
  // then the split's flag. Partial of split s: head hh at [hh (HD + 4), + HD) the output, + HD the max (log2
  // domain), + HD + 1 the weight sum (16-byte aligned rows).
  constexpr int PS = HD + 4, PSTRIDE = G * PS;
  const unsigned gen = gen0 + (unsigned)(kFusedPhases * layer + 1) + 1u;
  unsigned* sflag = opaque_p(p.sync) + kSyncSplit + 32 * g;
  {
    float* part = opaque_p(p.part) + ((size_t)g * S + s) * PSTRIDE;
    for (int i = tid; i < G * (HD + 2); i += kFT) {
      const int hh = i / (HD + 2), dd = i % (HD + 2);
      float mm = wst[hh * (HD + 2) + HD];
      float ll = wst[hh * (HD + 2) + HD + 1];
      float oo = wst[hh * (HD + 2) + min(dd, HD - 1)];
#pragma unroll
      for (int w = 1; w < kFW; ++w) {
        const float* ws2 = wst + (w * G + hh) * (HD + 2);
        float M, w1, w2;
        Lse::weights(mm, ws2[HD], M, w1, w2);
        ll = ll * w1 + ws2[HD + 1] * w2;
        oo = oo * w1 + ws2[min(dd, HD - 1)] * w2;
        mm = M;
      }
      st_dev(part + hh * PS + dd, dd < HD ? oo : (dd == HD ? mm : ll));
    }
    wait_all();
  }
  __syncthreads();
  if (st) st[3] = (unsigned long long)wall_clock64();

  if (wid != 0) {
    // waves 1-7: the next phase's first weights (unless issued at the sweep), concurrent with wave 0's merge and
    // barrier; then, once wave 0 has its merge inputs (bulk loads issued earlier would queue ahead of them), the
    // gate/up batches that go through LDS (the K/V chunk is no longer needed)
    if constexpr (!kEarlyO<SH>) {
      nx.issue(0, A);
      nx.issue(1, B);
    }
    if constexpr (Geo<SH, PH_GU>::NLB > 0) {
      while (__hip_atomic_load(&sm.flags[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != (int)gen)
        __builtin_amdgcn_s_sleep(2);
      gu.lds_prefetch(sm.stage, wid);
    }
  } else {
    // ---- wave 0 of every split merges OPB of the kv head's G HD outputs, [s OPB, s OPB + OPB), over all S
    // splits once their flags are up: lane k < S takes split k's max, sum and OPB outputs, and the weighted sums
    // over the lanes come out of one transposing reduction (split order fixed, so every run forms them alike)
    constexpr int OPB = G * HD / S;
    static_assert(S <= 64 && OPB % 4 == 0 && OPB <= 16 && HD % OPB == 0, "merge slices of whole 16-byte groups");
    if (lane == 0) st_dev(sflag + s, gen);
    if (!sm.flags[0])
      spin_until(p, sm.flags, [&]() __attribute__((always_inline)) {
        return __all(lane >= S || ld_dev(sflag + min(lane, S - 1)) == gen) != 0;
      });
    if (st) st[4] = (unsigned long long)wall_clock64();
    const int o0 = s * OPB, hh = o0 / HD, d0 = o0 % HD;
    const auto rp = make_rsrc(opaque_p(p.part) + (size_t)g * S * PSTRIDE + hh * PS);
    const int sl = opaque_v(min(lane, S - 1) * PSTRIDE * 4);
    const u32x4 ml = ld_dev16(rp, sl + HD * 4);   // (max, sum, -, -)
    u32x4 ov[OPB / 4];
#pragma unroll
    for (int q4 = 0; q4 < OPB / 4; ++q4) ov[q4] = ld_dev16(rp, sl + (d0 + 4 * q4) * 4);
    const float ms = lane < S ? __uint_as_float(ml.x) : -INFINITY;
    const float M = wave_max(ms);
    const float w = ms != -INFINITY ? fast_exp2(ms - M) : 0.f;
    const float Lt = wave_total(w * __uint_as_float(ml.y));
    float a[OPB];
#pragma unroll
    for (int q4 = 0; q4 < OPB / 4; ++q4) {
      a[4 * q4] = w * __uint_as_float(ov[q4].x);
      a[4 * q4 + 1] = w * __uint_as_float(ov[q4].y);
      a[4 * q4 + 2] = w * __uint_as_float(ov[q4].z);
      a[4 * q4 + 3] = w * __uint_as_float(ov[q4].w);
    }
    const float o = transpose_reduce<OPB>(a, lane);
    constexpr int LOGO = OPB == 4 ? 2 : OPB == 8 ? 3 : 4;
    if ((lane & ((64 >> LOGO) - 1)) == 0)
      st_dev(opaque_p(p.attn) + (g * G + hh) * HD + d0 + (lane >> (6 - LOGO)), o / Lt);
    if (st) st[5] = (unsigned long long)wall_clock64();
    if (lane == 0) __hip_atomic_store(&sm.flags[1], (int)gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    arrive_and_wait(p, gen0, kFusedPhases * layer + 1, lane, sm.flags, [&]() __attribute__((always_inline)) {
      nx.issue(0, A);
      nx.issue(1, B);
    });
  }
  barrier_lds();   // (the next phase's first batches and the gate/up LDS batches stay in flight)
  after_barrier(p, kFusedPhases * layer + 1);
}

// TRACE: record block 0's clock after every barrier, every block's barrier arrival and release times, and (with
// trace2 set) the sub-phase clocks. Without it no trace code is compiled in: its pointers would hold scalar
// registers for the whole launch, and the kernel's code must stay small enough for the instruction cache.
template <class SH, bool TRACE>
__global__ void __launch_bounds__(kFT, 1) fused_step_kernel(FusedParams p_in) {
  FusedParams p = p_in;
  if constexpr (!TRACE) {
    p.clocks = nullptr;
    p.trace = nullptr;
    p.trace2 = nullptr;
  }
  __shared__ __attribute__((aligned(16))) unsigned char s_stage[SH::SB];
  __shared__ __attribute__((aligned(16))) float s_uni[SH::UNI];
  __shared__ float s_ssq[kFW];
  __shared__ int s_flags[3];
  __shared__ int s_qrow[Geo<SH, PH_QKV>::RPB];
  const Smem<SH> sm{s_stage, s_uni, s_ssq, s_flags};
  const int tid = threadIdx.x, lane0 = tid & 63, wid0 = __builtin_amdgcn_readfirstlane(tid >> 6), b0 = blockIdx.x;
  const int L = p.n_layers;
  const int nbar = kFusedPhases * L;

  const SlotLayout sl{1};
  const unsigned gen0 = ld_dev(&p.sync[0]) * (unsigned)(nbar + 1);   // this launch's generations: gen0 + 1 ...
  int token = p.slots[sl.token()];
  int pos = p.slots[sl.pos()];
  const bool tok_ok = token >= 0 && token < p.vocab;
  const bool pos_ok = pos >= 0 && pos < p.cap;
  if (!tok_ok) token = 0;
  if (!pos_ok) pos = 0;
  if (tid == 0) {
    s_flags[0] = 0;
    s_flags[1] = 0;
    s_flags[2] = 0;
    if (b0 == 0) {
      if (!tok_ok) raise_error(p.status, ERR_TOKEN);
      if (!pos_ok) raise_error(p.status, ERR_POS);
      if (p.slots[sl.inject()] != 0) raise_error(p.status, ERR_INJECTED);
      if (p.clocks) p.clocks[0] = (unsigned long long)wall_clock64();
    }
  }
  const uint16_t* erow = p.embed + (size_t)token * SH::D;
  auto W = [&](int l, size_t off) __attribute__((always_inline)) { return p.wbase + (size_t)l * p.lstride + off; };
  auto GN = [&](int l, size_t off) __attribute__((always_inline)) { return reinterpret_cast<const float*>(W(l, off)); };
  // stage layer l's K/V chunk; `it` >= 0: only the part for gate/up loop iteration `it` (2 instructions per wave
  // each), so the staging does not arrive as one burst that stalls the waves' own loads
  // (visible-sweep slot set: a split whose positions all lie after pos stages nothing and computes nothing)
  const bool live = p.slots[sl.sweep()] == 0 || (b0 % SH::S) * SH::TC <= pos;
  auto stage_layer = [&](int l, int b, int wid, int lane, int it) __attribute__((always_inline)) {
    constexpr int NIW = SH::KB / 1024 / kFW;
    const int i0 = it < 0 ? 0 : 2 * it, i1 = it < 0 ? NIW : 2 * it + 2;
    if (i0 < NIW && live) stage_chunk<SH>(p, l, b / SH::S, (b % SH::S) * SH::TC, sm.stage, wid, lane, i0, i1);
  };

  u32x4 A[kNL], B[kNL];
  GemvPhase<SH, PH_QKV> qkv;
  qkv.init(W(0, p.o_wqkv), 0, b0, wid0, lane0, s_qrow);
  if (tid < qkv.rb) s_qrow[tid] = qkv.row_of(tid) * (SH::D * 2);
  __syncthreads();
  stage_layer(0, b0, wid0, lane0, -1);
  qkv.issue(0, A);
  qkv.issue(1, B);
  __syncthreads();

  for (int l = 0; l < L; ++l) {
    // Per-iteration opaque copies: everything derived from the lane, wave and block index is recomputed in each
    // layer instead of being hoisted out of the loop (which would keep hundreds of values live across it).
    const int lane = opaque_v(lane0), wid = opaque_s(wid0), b = opaque_s(b0);
    const uint16_t* xe = l == 0 ? erow : nullptr;
    GemvPhase<SH, PH_O> ph_o;
    ph_o.init(W(l, p.o_wo), 0, b, wid, lane);
    GemvPhase<SH, PH_GU> ph_gu;
    ph_gu.init(W(l, p.o_wgu), 0, b, wid, lane);
    GemvPhase<SH, PH_DOWN> ph_down;
    ph_down.init(W(l, p.o_wd), 0, b, wid, lane);

    run_gemv<SH, PH_QKV>(p, qkv, NoNext{}, [](int) __attribute__((always_inline)) {}, A, B, sm, p.x, GN(l, p.o_attn_norm), xe, l, pos, pos_ok, wid, lane, gen0);
    run_attn<SH>(p, ph_o, ph_gu, A, B, sm, l, pos, pos_ok, wid, lane, gen0);
    run_gemv<SH, PH_O>(p, ph_o, ph_gu, [](int) __attribute__((always_inline)) {}, A, B, sm, p.attn, nullptr, xe, l, pos, pos_ok, wid, lane, gen0);
    if (l + 1 < L) {
      run_gemv<SH, PH_GU>(p, ph_gu, ph_down, [&](int it) __attribute__((always_inline)) { stage_layer(l + 1, b, wid, lane, it); }, A, B, sm, p.x, GN(l, p.o_ffn_norm),
                          nullptr, l, pos, pos_ok, wid, lane, gen0);
      qkv.init(W(l + 1, p.o_wqkv), 0, b, wid, lane, s_qrow);
      run_gemv<SH, PH_DOWN>(p, ph_down, qkv, [](int) __attribute__((always_inline)) {}, A, B, sm, p.act, nullptr, nullptr, l, pos, pos_ok, wid, lane, gen0);
    } else {
      run_gemv<SH, PH_GU>(p, ph_gu, ph_down, [](int) __attribute__((always_inline)) {}, A, B, sm, p.x, GN(l, p.o_ffn_norm), nullptr, l, pos, pos_ok,
                          wid, lane, gen0);
      GemvPhase<SH, PH_HEAD> head;
      head.init(p.lm_head, p.vocab, b, wid, lane);
      run_gemv<SH, PH_DOWN>(p, ph_down, head, [](int) __attribute__((always_inline)) {}, A, B, sm, p.act, nullptr, nullptr, l, pos, pos_ok, wid,
                            lane, gen0);
      run_gemv<SH, PH_HEAD>(p, head, NoNext{}, [](int) __attribute__((always_inline)) {}, A, B, sm, p.x, p.final_norm, nullptr, l, pos, pos_ok, wid,
                            lane, gen0);
    }
  }

  // ---- leave: block 0 advances the epoch (every block read it at its start, before the first barrier)
  if (b0 == 0 && tid == 0) {
    st_dev(&p.sync[0], ld_dev(&p.sync[0]) + 1u);
    if (p.clocks) p.clocks[nbar + 1] = (unsigned long long)wall_clock64();
  }
}

template <class SH>
hipError_t fused_go(const FusedParams& p, bool trace, hipStream_t s) {
  if (trace) fused_step_kernel<SH, true><<<kFusedBlocks, kFT, 0, s>>>(p);
  else fused_step_kernel<SH, false><<<kFusedBlocks, kFT, 0, s>>>(p);
  return hipGetLastError();
}

template <class SH>
hipError_t fused_occ(int* out) {
  int a = 0, b = 0;
  hipError_t h = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, fused_step_kernel<SH, false>, kFT, 0);
  if (h == hipSuccess) h = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fused_step_kernel<SH, true>, kFT, 0);
  *out = a < b ? a : b;
  return h;
}

}  // namespace

bool fused_shape_supported(int d, int ffn, int hd, int nq, int nkv) {
  return (d == 4096 && ffn == 14336 && hd == 128 && nq == 32 && nkv == 8) ||
         (d == 2048 && ffn == 8192 && hd == 64 && nq == 32 && nkv == 8);
}

// Positions per staged chunk for a split of split_len positions: 256 where they divide it, else 128 (0: neither).
int fused_chunk(int split_len) { return split_len % 256 == 0 ? 256 : (split_len % 128 == 0 ? 128 : 0); }

template <int D, int F, int HD, int NQ, int NKV>
hipError_t fused_occ_any(int tc, bool mc, int* out) {
  if (tc == 256) return mc ? fused_occ<Shape<D, F, HD, NQ, NKV, 256, true>>(out) : fused_occ<Shape<D, F, HD, NQ, NKV, 256>>(out);
  return mc ? fused_occ<Shape<D, F, HD, NQ, NKV, 128, true>>(out) : fused_occ<Shape<D, F, HD, NQ, NKV, 128>>(out);
}
template <int D, int F, int HD, int NQ, int NKV>
hipError_t fused_go_any(const FusedParams& p, int tc, bool mc, bool trace, hipStream_t s) {
  if (tc == 256) return mc ? fused_go<Shape<D, F, HD, NQ, NKV, 256, true>>(p, trace, s) : fused_go<Shape<D, F, HD, NQ, NKV, 256>>(p, trace, s);
  return mc ? fused_go<Shape<D, F, HD, NQ, NKV, 128, true>>(p, trace, s) : fused_go<Shape<D, F, HD, NQ, NKV, 128>>(p, trace, s);
}

hipError_t fused_blocks_per_cu(int d, int ffn, int hd, int nq, int nkv, int split_len, int* out) {
  *out = 0;
  const int tc = fused_chunk(split_len);
  if (tc == 0) return hipErrorInvalidValue;
  const bool mc = split_len > tc;
  if (d == 4096 && ffn == 14336 && hd == 128 && nq == 32 && nkv == 8)
    return fused_occ_any<4096, 14336, 128, 32, 8>(tc, mc, out);
  if (d == 2048 && ffn == 8192 && hd == 64 && nq == 32 && nkv == 8)
    return fused_occ_any<2048, 8192, 64, 32, 8>(tc, mc, out);
  return hipErrorInvalidValue;
}

hipError_t launch_fused(const FusedParams& p, int d, int ffn, int hd, int nq, int nkv, bool trace, hipStream_t s) {
  const int tc = fused_chunk(p.split_len);   // split_len / tc staged chunks per split
  if (tc == 0 || p.cap != p.split_len * (kFusedBlocks / nkv)) return hipErrorInvalidValue;
  const bool mc = p.split_len > tc;
  if (d == 4096 && ffn == 14336 && hd == 128 && nq == 32 && nkv == 8)
    return fused_go_any<4096, 14336, 128, 32, 8>(p, tc, mc, trace, s);
  if (d == 2048 && ffn == 8192 && hd == 64 && nq == 32 && nkv == 8)
    return fused_go_any<2048, 8192, 64, 32, 8>(p, tc, mc, trace, s);
  return hipErrorInvalidValue;
}

}  // namespace ds3

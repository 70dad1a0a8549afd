// Device helpers shared by the decode-step kernels (gfx950, wave64). Internal; not part of the C ABI.
#pragma once

#include <math.h>

#include "ds3_kernels.h"

namespace ds3 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
// Sum over the wave, identical in every lane: DPP sums within each row of 16 lanes, then the four row sums read
// back in row order.
__device__ __forceinline__ float wave_total(float v);

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32, 64) that leaves the identical sum in every lane of
// the group: every step adds a partner's value, and float addition is commutative, so partners agree bit for
// bit. Steps within a row of 16 lanes use DPP lane permutations (quad swaps, half-row and row mirrors); wider
// steps use cross-row shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror: pairs the two quads of each 8 lanes
  if constexpr (N >= 16) v += dpp_mov<0x140>(v);  // row_mirror: pairs the two halves of each 16 lanes
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// (value, index) order of the greedy pick: larger value first, then lower index; NaN is never larger
__device__ __forceinline__ bool pick_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// 2^x with the hardware exp (results below the normal range flush to zero, which a softmax weight can afford)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_total(float v) {
  v = group_sum<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ void raise_error(StatusWords* st, uint32_t bit) { atomicOr(&st->err, bit); }

// K/V row of activation row r
__device__ __forceinline__ int kv_row(const KvView& kv, int r) { return kv.row_map ? kv.row_map[r] : r; }

// Location of logical position j of activation row r: the position itself (contiguous) or its pool slot
// page * ps + offset (paged, through its K/V row's page table; an id outside the pool raises the error word and
// reads page 0).
__device__ __forceinline__ int kv_loc(const KvView& kv, int r, int j, StatusWords* st) {
  if (!kv.paged) return j;
  const int ppr = kv.cap / kv.page_size;
  int page = kv.slot_map[kv_row(kv, r) * ppr + j / kv.page_size];
  if (page < 0 || page >= kv.pool_pages) {
    raise_error(st, ERR_PAGE);
    page = 0;
  }
  return page * kv.page_size + j % kv.page_size;
}

// Element offset, within one layer's K or V state, of element e of (activation row r, kv head g) at location loc
// (kv_loc).
__device__ __forceinline__ size_t kv_at(const KvView& kv, bool is_v, int r, int nkv, int g, int hd, int loc, int e) {
  const bool t = is_v && kv.v_t;
  if (!kv.paged) {
    const size_t head = (size_t)(kv_row(kv, r) * nkv + g);
    return t ? (head * hd + e) * kv.cap + loc : (head * kv.cap + loc) * hd + e;
  }
  const int ps = kv.page_size;
  const size_t head = (size_t)(loc / ps) * nkv + g;
  return t ? (head * hd + e) * ps + loc % ps : (head * ps + loc % ps) * hd + e;
}


struct Lse {   // merge of two (max, sum, weighted values) states (maxima in the log2 domain); symmetric, so
               // butterfly partners agree
  __device__ __forceinline__ static void weights(float m1, float m2, float& M, float& w1, float& w2) {
    M = fmaxf(m1, m2);
    w1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - M);
    w2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - M);
  }
};

// s_waitcnt immediate (gfx9 encoding) that waits until at most N vector-memory operations are outstanding and
// does not wait on the other counters
template <int N>
constexpr int kVmcntChunk() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// Block barrier that orders LDS only. __syncthreads() is a workgroup fence as well, which compiles to
// s_waitcnt vmcnt(0) -- every outstanding global load and store of the wave -- wherever a store may precede it, and
// so drains loads issued ahead (the next chunk's or the next phase's). Callers wait explicitly for the loads whose
// data the other waves read (s_waitcnt vmcnt(N)); the wave's own LDS reads and writes complete first.
__device__ __forceinline__ void barrier_lds() {
  constexpr int kLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);   // s_waitcnt lgkmcnt(0) only (gfx9 encoding)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(1))) const void* global_cptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// Swizzle key of the K rows staged in LDS by the matrix-core attention (16-byte piece index XOR key).
template <int CPR>
__device__ __forceinline__ int kswz(int pj) { return ((pj & 3) | ((pj >> 1) & 12)) & (CPR - 1); }

// Two floats -> two bf16 words (low word = a) with gfx950's packed convert, round to nearest, ties to even.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v{a, b}), bf16x2v));
}

__device__ __forceinline__ void split_hi_lo8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hw[e] = cvt_pk_bf16(v[2 * e], v[2 * e + 1]);
    lw[e] = cvt_pk_bf16(v[2 * e] - __uint_as_float(hw[e] << 16), v[2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
}

}  // namespace ds3

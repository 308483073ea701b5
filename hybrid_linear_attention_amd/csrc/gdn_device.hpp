// Device-side building blocks for the gfx950 Gated DeltaNet kernels:
// element types, conversions, and the MFMA fragment helpers.
//
// MFMA fragment layouts used throughout (gfx950, wave64; lane = 0..63,
// r = lane % 16, g = lane / 16):
//
//  * 16x16 accumulator tile (both v_mfma_f32_16x16x32_bf16 and
//    v_mfma_f32_16x16x4_f32): lane holds rows 4g + i (i = 0..3) of column r.
//  * bf16, K = 32 per instruction: lane (row r of A / column r of B, group g)
//    supplies 8 K-slots.  Any K order works as long as A and B agree, so the
//    library uses the order that makes an accumulator pair usable as a B
//    operand without leaving registers: slot j < 4 is K = 4g + j, slot j >= 4
//    is K = 16 + 4g + (j - 4).  Two stacked 16x16 accumulator tiles (rows 0-15
//    and 16-31 of a 32-row block) are then exactly one B fragment.
//  * fp32, K = 4 per instruction: step s of a 16-row K block takes K = 4g + s,
//    so element s of an accumulator tile is the B operand of step s.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;     // head dimension (d_k = d_v)
constexpr int kC = 64;      // tokens per chunk

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Four consecutive elements of a carried state (h0 / ht), stored as float32
// or, when `as_bf16` is set, as bfloat16 (converted with round to nearest even).
__device__ __forceinline__ f32x4 load_state4(const void* base, size_t idx, bool as_bf16) {
  if (as_bf16) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(base) + idx);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
  return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
}
__device__ __forceinline__ void store_state4(void* base, size_t idx, const f32x4& x, bool as_bf16) {
  if (as_bf16) {
    bf16x4 v;
    v[0] = (bf16)x[0]; v[1] = (bf16)x[1]; v[2] = (bf16)x[2]; v[3] = (bf16)x[3];
    *reinterpret_cast<bf16x4*>(static_cast<bf16*>(base) + idx) = v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = x;
  }
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Orders this wave's LDS traffic: every earlier LDS access has completed and
// no later one is hoisted above this point.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Two accumulator tiles (K rows 0-15 and 16-31 of a 32-row block) -> one
// bf16 B fragment in the library's K order.
__device__ __forceinline__ bf16x8 pack_b(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
  r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
  r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
  return r;
}

// Plain A/B fragment (bf16, hardware-natural K order k = 8g + j) of a
// row-major LDS matrix whose rows are indexed by the fragment's M (for A) or
// N (for B): used when both operands come from LDS (Gram matrices).
__device__ __forceinline__ bf16x8 lds_row8_bf16(const bf16* A, int lda, int row, int k0) {
  const int g = lane_id() >> 4;
  return *reinterpret_cast<const bf16x8*>(A + row * lda + k0 + 8 * g);
}

// acc(16 x 16) += A[row0 .. row0+15][k-range] * B, where B's K rows come as
// accumulator tiles bt[0 .. nkb-1] (16 K rows each) and A is row-major fp32
// in LDS with the K range starting at column kcol0.
template <int NKB>
__device__ __forceinline__ void mma_acc_f32(f32x4& acc, const float* A, int lda,
                                            int row0, int kcol0, const f32x4* bt) {
  const int r = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const float* p = A + (row0 + r) * lda + kcol0 + 16 * kb + 4 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_f32(p[s], bt[kb][s], acc);
  }
}

// fp32 variant whose A operand is the TRANSPOSE of a row-major LDS matrix:
// acc += (M^T)[row0 .. row0+15][k-range] * B, i.e. A[m][k] = M[k][m].
template <int NKB>
__device__ __forceinline__ void mma_acc_f32_tA(f32x4& acc, const float* M, int ldm,
                                               int row0, int kcol0, const f32x4* bt) {
  const int r = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = mfma_f32(M[(kcol0 + 16 * kb + 4 * g + s) * ldm + row0 + r], bt[kb][s], acc);
  }
}

// Wave-wide inclusive prefix sum over 64 lanes.
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

// Wave-wide inclusive prefix sum carried as an unevaluated pair hi + lo
// (hi = the float nearest the sum, lo = its rounding error, kept by the
// error-free transformation TwoSum at every step).  A difference of two
// prefixes, (hi_i - hi_j) + (lo_i - lo_j), then keeps relative accuracy even
// when both prefixes are large and nearly equal: the strong-decay case of the
// gate prefix, whose differences are exponents.
__device__ __forceinline__ float two_sum_err(float a, float b, float s) {
  const float bb = s - a;
  return (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ float wave_inclusive_sum2(float x, float& lo) {
  const int l = lane_id();
  float hi = x;
  lo = 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float yh = __shfl_up(hi, off, 64), yl = __shfl_up(lo, off, 64);
    if (l >= off) {
      const float s = hi + yh;
      const float e = two_sum_err(hi, yh, s) + (lo + yl);
      hi = s + e;
      lo = e - (hi - s);
    }
  }
  return hi;
}

}  // namespace gdn

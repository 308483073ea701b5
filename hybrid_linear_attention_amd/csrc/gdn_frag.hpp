// Element-generic MFMA fragments, swizzled LDS matrices and direct
// global->LDS copies shared by the backward and attention kernels (gfx950,
// wave64; see gdn_device.hpp for the accumulator layout and K order).
#pragma once
#include "gdn_device.hpp"

namespace gdn {
namespace frag {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: 4 x 16-bit elements, transposed across each group of 16
// lanes (input lane p reads 8 bytes at its address; output lane m receives
// element m % 4 of input lanes m / 4, m / 4 + 4, m / 4 + 8, m / 4 + 12).
// The compiler orders an LDS read that carries no alias information after
// every direct global->LDS copy still in flight (a full vmcnt(0) wait), so a
// transposed read placed after the next tile's copies were issued would stall
// until they land.  Every read of copied data here is ordered by an explicit
// copy wait and barrier instead; the restrict-qualified argument gives the
// inlined read a scope of its own, which drops the implied wait.
__device__ __forceinline__ s16x4 lds_tr16(const void* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------ fragments
// A fragment holds the K slots one lane supplies to an MFMA: 8 bf16 (one
// 16x16x32 instruction) or 4 fp32 (four 16x16x4 instructions).  Slot j of
// lane group g is K offset kslot(g, j) inside a K block of KB.
template <typename E> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 T; static constexpr int KB = 32; };
template <> struct FragOf<float> { typedef f32x4 T; static constexpr int KB = 16; };
template <typename E> using Fr = typename FragOf<E>::T;

template <typename E> __device__ __forceinline__ int kslot(int g, int j) {
  if constexpr (sizeof(E) == 2) return j < 4 ? 4 * g + j : 12 + 4 * g + j;
  else return 4 * g + j;
}
template <typename E> constexpr int kSlotsOf = sizeof(E) == 2 ? 8 : 4;

__device__ __forceinline__ f32x4 mma(f32x4 c, const bf16x8& a, const bf16x8& b) {
  return mfma_bf16(a, b, c);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = mfma_f32(a[s], b[s], c);
  return c;
}

// Fragment from accumulator tiles whose rows are the K index (tile t covers
// K rows 16t .. 16t+15): a product's result used as the next product's B
// operand (or, transposed, as its A operand) without leaving registers.
template <typename E> __device__ __forceinline__ Fr<E> acc_frag(const f32x4* t, int kb) {
  if constexpr (sizeof(E) == 2) return pack_b(t[2 * kb], t[2 * kb + 1]);
  else return t[kb];
}

// Position of the 16-row tile mt against the K block kb of a 64x64
// triangular operand: wholly above the diagonal (every K index > every row) or
// wholly below it (every K index < every row).
template <typename E> constexpr bool blk_above(int mt, int kb) {
  return FragOf<E>::KB * kb > 16 * mt + 15;
}
template <typename E> constexpr bool blk_below(int mt, int kb) {
  return FragOf<E>::KB * kb + FragOf<E>::KB - 1 < 16 * mt;
}

template <typename E> __device__ __forceinline__ void frag_zero(Fr<E>& f, int j) {
  if constexpr (sizeof(E) == 2) f[j] = (bf16)0.f;
  else f[j] = 0.f;
}

__device__ __forceinline__ bf16x4 as_bf16x4(s16x4 v) {
  return __builtin_bit_cast(bf16x4, v);
}

// A lane's position in the MFMA fragment layouts (r = lane % 16, g = lane / 16).
struct Lane {
  int r, g;
};
__device__ __forceinline__ Lane lane_here() { return Lane{lane_id() & 15, lane_id() >> 4}; }
// The same, hidden from the optimiser: fragment addresses derived from it are
// recomputed where they are used instead of being hoisted out of a loop and
// kept live (or spilled) across it.
__device__ __forceinline__ Lane lane_opaque() {
  int l = lane_id();
  asm volatile("" : "+v"(l));
  return Lane{l & 15, l >> 4};
}

// XOR swizzle of the 8-byte units of row `row` of a bf16 matrix with W
// columns.  64-bit LDS reads are served 32 lanes at a time over 64 banks; the
// row-pattern fragment read (lane (r, g): row r, unit g) then touches rows
// 0..15 with two units each, and the transposed read (16 lanes: 4 rows x 4
// units) four rows of one 32-byte column block.  Rows sharing a 256-byte bank
// line are spread by ((row / rpl) % nb) in unit bits 2+, and row bit 3 flips
// unit bit 1, so both reads hit every bank once per pass.  Bit 0 is never
// flipped: 16-byte pieces stay whole for the direct global->LDS copies.
template <int W>
__device__ __forceinline__ int swz_units(int row) {
  // unsigned: rows are never negative, and signed / and % by powers of two
  // cost a sign fix-up each
  constexpr unsigned rpl = W <= 128 ? 128 / W : 1, nb = W >= 128 ? 8 : W / 16;
  const unsigned ur = (unsigned)row;
  return (int)((((ur / rpl) % nb) << 2) | (((ur >> 3) & 1u) << 1));
}

// Row-major matrix of W columns in LDS.  bf16: unpadded rows with 8-byte
// units XOR-swizzled so that both fragment reads below hit every bank once per
// pass; fp32: rows padded by 4 floats.
template <typename E, int W>
struct Lds {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int LD = BF ? W : W + 4;
  static constexpr int size(int rows) { return rows * LD; }
  E* p;
  __device__ static int at(int row, int col) {
    if constexpr (BF) {
      return row * W + ((((col >> 2) ^ swz_units<W>(row))) << 2) + (col & 3);
    } else {
      return row * LD + col;
    }
  }
  __device__ E& operator()(int row, int col) const { return p[at(row, col)]; }
  __device__ float get(int row, int col) const { return to_f32(p[at(row, col)]); }
  // Lane index along rows: slot j = element (row, k0 + kslot(g, j)).
  __device__ Fr<E> rm(int row, int k0) const { return rm(row, k0, lane_here()); }
  __device__ Fr<E> rm(int row, int k0, const Lane& ln) const {
    const int g = ln.g;
    if constexpr (BF) {
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + at(row, k0 + 4 * g));
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + at(row, k0 + 16 + 4 * g));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *reinterpret_cast<const f32x4*>(p + row * LD + k0 + 4 * g);
    }
  }
  // Natural K order (slot j = element (row, k0 + 8g + j) for bf16, k0 + 4g + j
  // for fp32): one 16-byte read.  Usable when both operands of a product come
  // from memory, so both can take this order.
  __device__ Fr<E> rmn(int row, int k0, const Lane& ln) const {
    if constexpr (BF) return *reinterpret_cast<const bf16x8*>(p + at(row, k0 + 8 * ln.g));
    else return rm(row, k0, ln);
  }
  // Lane index along columns (col = 16-aligned base + lane % 16): slot j =
  // element (k0 + kslot(g, j), col).  bf16 uses ds_read_b64_tr_b16: input lane
  // r of a 16-lane group reads four columns base + 4(r%4) .. +3 of row
  // k0 + 4g + r/4, and output lane m receives column base + m of those rows.
  __device__ Fr<E> cm(int col, int k0) const { return cm(col, k0, lane_here()); }
  __device__ Fr<E> cm(int col, int k0, const Lane& ln) const {
    const int r = ln.r, g = ln.g;
    if constexpr (BF) {
      const int c0 = col - r + 4 * (r & 3);
      const s16x4 lo = lds_tr16(p + at(k0 + 4 * g + (r >> 2), c0));
      const s16x4 hi = lds_tr16(p + at(k0 + 16 + 4 * g + (r >> 2), c0));
      return __builtin_shufflevector(as_bf16x4(lo), as_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      f32x4 f;
#pragma unroll
      for (int s = 0; s < 4; ++s) f[s] = p[(k0 + 4 * g + s) * LD + col];
      return f;
    }
  }
};

// Row-major matrix in global memory with `rows` valid rows (reads beyond them
// return zero: the tail of the last chunk).
template <typename E>
struct Glb {
  const E* p;
  int64_t ld;
  int rows;
  __device__ float get(int row, int col) const {
    return row < rows ? to_f32(p[row * ld + col]) : 0.f;
  }
  __device__ Fr<E> rm(int row, int k0) const { return rm(row, k0, lane_here()); }
  __device__ Fr<E> rm(int row, int k0, const Lane& ln) const {
    const int g = ln.g;
    Fr<E> f;
#pragma unroll
    for (int j = 0; j < kSlotsOf<E>; ++j)
      f[j] = row < rows ? p[row * ld + k0 + kslot<E>(g, j)] : (E)0.f;
    return f;
  }
  // natural K order (fp32 only: there it is the rm order)
  __device__ Fr<E> rmn(int row, int k0, const Lane& ln) const {
    static_assert(sizeof(E) == 4, "natural order from global memory: fp32 only");
    return rm(row, k0, ln);
  }
  __device__ Fr<E> cm(int col, int k0) const { return cm(col, k0, lane_here()); }
  __device__ Fr<E> cm(int col, int k0, const Lane& ln) const {
    const int g = ln.g;
    Fr<E> f;
#pragma unroll
    for (int j = 0; j < kSlotsOf<E>; ++j) {
      const int row = k0 + kslot<E>(g, j);
      f[j] = row < rows ? p[row * ld + col] : (E)0.f;
    }
    return f;
  }
};

// Copies rows [0, rows) of a global row-major matrix (row stride ld elements,
// W columns) into an LDS matrix, zero-filling rows [rows, R).  All NT threads
// take part; 16-byte pieces.
template <typename E, int W, int R, int NT>
__device__ __forceinline__ void stage(Lds<E, W> dst, const E* src, int64_t ld, int rows) {
  constexpr int EP = 16 / sizeof(E);
  constexpr int PPR = W / EP;
  constexpr int NP = R * PPR;
  static_assert(NP % NT == 0, "pieces per thread");
  uint4 buf[NP / NT];
#pragma unroll
  for (int it = 0; it < NP / NT; ++it) {
    const int pc = threadIdx.x + NT * it, row = pc / PPR, c = (pc % PPR) * EP;
    buf[it] = row < rows ? *reinterpret_cast<const uint4*>(src + row * ld + c)
                         : uint4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int it = 0; it < NP / NT; ++it) {
    const int pc = threadIdx.x + NT * it, row = pc / PPR, c = (pc % PPR) * EP;
    if constexpr (sizeof(E) == 2) {
      // two 8-byte units; the swizzle keeps each 16-byte piece contiguous
      *reinterpret_cast<uint4*>(&dst(row, c)) = buf[it];
    } else {
      *reinterpret_cast<uint4*>(&dst(row, c)) = buf[it];
    }
  }
}

// Sum over the 16 lanes of a lane group (same g): four DPP row rotations
// (VALU only; every lane of the row ends with the full sum).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x120 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename E>
__device__ __forceinline__ void store4(E* p, const f32x4& x) {
  if constexpr (sizeof(E) == 2) {
    bf16x4 v;
    v[0] = (bf16)x[0]; v[1] = (bf16)x[1]; v[2] = (bf16)x[2]; v[3] = (bf16)x[3];
    *reinterpret_cast<bf16x4*>(p) = v;
  } else {
    *reinterpret_cast<f32x4*>(p) = x;
  }
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Copy number `it` (it < ROWS * 2W / 1024) of copy_rows below: for callers
// that spread a tile's copies over other work.
template <int W, int ROWS = kC>
__device__ __forceinline__ void copy_row_one(const bf16* src, int64_t ld, int L, bf16* dst, int it,
                                             int l = lane_id()) {
  constexpr int RPK = 1024 / (2 * W);
  const int rin = (int)((16u * l) / (2 * W)), pp = (int)(((16u * l) % (2 * W)) / 16);
  const int row = it * RPK + rin;
  const int lp = pp ^ (swz_units<W>(row) >> 1);
  // a uniform base and 32-bit byte offsets (the rows of one copy span far
  // less than 2 GiB): no 64-bit multiply per copy
  dma16(reinterpret_cast<const char*>(src) + ((uint32_t)min(row, L - 1) * (uint32_t)(2 * ld) + 16u * lp),
        reinterpret_cast<char*>(dst) + 1024 * it);
}
// ROWS rows (rows >= L repeat row L-1) of a bf16 matrix with W columns into the
// Lds<bf16, W> layout at dst; wave w of nw issues copies w, w + nw, ...  (w
// must be wave-uniform: the LDS destination goes through M0).  Copy `it`
// fills LDS bytes [1024 it, 1024 it + 1024); lane l's 16 bytes are the piece
// of the swizzled layout at that position, so each lane reads the global piece
// the swizzle puts there.
template <int W, int ROWS = kC>
__device__ __forceinline__ void copy_rows(const bf16* src, int64_t ld, int L, bf16* dst, int w,
                                          int nw, int l = lane_id()) {
  constexpr int NIT = ROWS * 2 * W / 1024;
  for (int it = w; it < NIT; it += nw) copy_row_one<W, ROWS>(src, ld, L, dst, it, l);
}


}  // namespace frag
}  // namespace gdn

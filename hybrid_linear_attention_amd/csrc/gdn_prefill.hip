// Chunked prefill of the gated delta rule on gfx950.
//
// The page "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture, 256k Context,
// and 24GB Local Serving" says prefill rewrites the token-serial update into a
// block-parallel matrix form that runs on the matrix units, with the state kept
// on chip ("Gated DeltaNet Mechanics" and the note under "The Role of Periodic
// Gated Attention").  The page does not give the rewrite; this is the plainest
// one that follows from the recurrence
//
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t
//
// For a chunk of L <= 64 tokens with incoming state S0 (d_v x d_k), local
// index i, and G_i = sum_{j<=i} ln alpha_j:
//
//     A   = strict_lower( diag(beta) (K K^T * exp(G_i - G_j)) )
//     Tt  = (I + A)^-1 diag(beta)                      (UT / WY solve)
//     X   = V - diag(exp G) K S0^T
//     Dl  = Tt X                                       (row i = beta_i (v_i - alpha_i S_{i-1} k_i))
//     O   = diag(exp G) Q S0^T + (Q K^T * exp(G_i - G_j))_{j<=i} Dl
//     S_L = exp(G_{L-1}) S0 + Dl^T diag(exp(G_{L-1} - G_j)) K
//
// Two kernels:
//  * prepare  (grid: chunks x query/key heads) - fully parallel.  Gram
//    matrices K K^T and Q K^T on MFMA (once per query/key head, shared by the
//    H_v/H_qk value heads that read it), gate prefix G, and the triangular
//    solve in fp32 (16x16 diagonal blocks by substitution, off-diagonal blocks
//    by fp32 MFMA).  Writes Tt, the masked output matrix M and G to the
//    workspace.  For the backward pass (solve_only) it also writes N =
//    (I + A)^-1 without the diag(beta) factor, and every block of N and M.
//  * scan     (grid: value-row slices x value heads x sequences) - the serial
//    chain.  Each chain wave owns 16 value rows of one head's state and keeps
//    them, transposed (S^T, d_k x 16), in fp32 MFMA accumulators for the whole
//    sequence.  Per chunk every product feeds the next one straight from
//    registers: the accumulator tiles of S^T, X and Dl are the B operands of the
//    following MFMAs (see gdn_device.hpp for the K order that makes this work),
//    so only the shared chunk operands (K^T, Q, Tt, M, V) go through LDS.
//    Rows of the state never interact, so the value rows split across waves
//    and workgroups with no communication at all.  Two versions: the bf16
//    scan (scan_split_kernel: chain, output and copy work on separate waves,
//    operands copied straight into LDS) and a generic one (scan_kernel: fp32
//    inputs, and the gated RMSNorm epilogue), which stages operands through
//    registers one chunk ahead.
#include "gdn_chunks.hpp"
#include "gdn_device.hpp"
#include "gdn_frag.hpp"
#include "gdn_launch.hpp"

#include <type_traits>

namespace gdn {

template <typename E>
struct Work {
  E* Tt;       // [nc][Hv][64][64]   (I + A)^-1 diag(beta).  bf16: the zero block
               //                    rows 0..31 x columns 32..63 (also of M) is not
               //                    written; the scan copies it but never reads it
  E* M;        // [nc][Hv][64][64]   (Q K^T * exp(G_i - G_j)) on and below the diagonal
  float* gam;  // [nc][Hv][64]       exp(G_t)
  float* dec;  // [nc][Hv][64]       exp(G_last - G_t)
  E* N;        // [nc][Hv][64][64]   (I + A)^-1, every block (backward pass only; else null)
};

// Gates are kept in base 2 so that the hardware v_exp_f32 / v_log_f32 apply
// directly: G2_t = sum_{j<=t} log2(alpha_j), exp(G_i - G_j) = 2^(G2_i - G2_j).
using frag::hw_exp2;
using frag::hw_log2;

// 16 consecutive bytes of a row of q/k/v (8 bf16 or 4 fp32), zero if masked.
template <typename E>
__device__ __forceinline__ uint4 ld16(const E* p, bool ok) {
  if (!ok) return uint4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------- prepare
constexpr int kLdT = 68;   // LDS row stride of 64-wide fp32/bf16 tiles

// fp32 only: the rounding error of the gate prefix (G2 = gate + gatelo;
// |gatelo| <= ulp(gate) / 2, so bf16 keeps it to ~1e-8).  Absent (an empty
// base) for bf16, whose layout must keep three workgroups per CU.
template <typename E> struct PrepLo { bf16 gatelo[3][kC]; };
template <> struct PrepLo<bf16> {};

template <typename E>
struct PrepSmem : PrepLo<E> {
  static constexpr int LDK = 136;   // K/Q row stride: rows 16-byte aligned for b128 reads
  static constexpr int NB = 3;      // value heads whose A matrices are resident at once
  union {
    struct {
      E Ks[kC * LDK];
      E Qs[kC * LDK];
    } in;
    float buf[NB][kC * kLdT];       // per value head: A, then (I + A)^-1 in place
  } u;
  float gate[NB][kC];               // G2 (base-2 log-decay prefix) per head
  float bet[NB][kC];
};
// Three bf16 prepare workgroups (two fp32 ones) share a CU's 160 KB of LDS;
// the bf16 layout is measured to allow three, and 384 bytes more do not.
static_assert(sizeof(PrepSmem<bf16>) <= 53760, "bf16 prepare LDS above 3 workgroups per CU");
static_assert(sizeof(PrepSmem<float>) <= 80 * 1024, "fp32 prepare LDS above 2 workgroups per CU");

// acc = A[arow0.., acol0..] (16x16) * B[brow0.., bcol0..] (16x16), both fp32 in LDS.
__device__ __forceinline__ f32x4 mm16_lds(const float* A, int arow0, int acol0,
                                          const float* Bm, int brow0, int bcol0, f32x4 acc) {
  const int r = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mfma_f32(A[(arow0 + r) * kLdT + acol0 + 4 * g + s],
                   Bm[(brow0 + 4 * g + s) * kLdT + bcol0 + r], acc);
  return acc;
}

// One workgroup per (chunk, query/key head), four waves.
//  1. K and Q of the chunk are staged in LDS; wave w computes the Gram tiles
//     with A = K rows 16w..16w+15 against B = K and Q rows of each 16-token
//     block nt:  KK[w][nt](m, n) = k_{16w+m} . k_{16nt+n},  KQ[w][nt](m, n) =
//     k_{16w+m} . q_{16nt+n}.  In the accumulator layout lane (n, g) holds
//     m = 4g..4g+3, so for token i = 16nt + n it holds four consecutive
//     columns j = 16w + 4g.. of row i of K K^T (symmetric) and of Q K^T:
//     rows of A and M are written straight from registers.
//  2. K^T is written for the scan.
//  3. Per batch of up to three value heads: gates (one wave per head), then
//     every wave writes its column block of A (to LDS) and M (to global) for
//     each head of the batch, then one wave per head solves (I + A)^-1 in
//     place and writes Tt.
// LDS is 53,760 bytes for bf16 (three workgroups share a CU) and 71,168 for
// fp32 (two).
template <typename E, bool solve_only>
__global__ __launch_bounds__(256, sizeof(E) == 2 ? 3 : 2) void prepare_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, Work<E> ws, ChunkMap cm, int Hqk, int Hv, int G) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int LDK = PrepSmem<E>::LDK;
  constexpr int NB = PrepSmem<E>::NB;
  constexpr int EPV = 16 / sizeof(E);            // elements per 16-byte piece
  __shared__ PrepSmem<E> sm;

  const int cid = blockIdx.x, gq = blockIdx.y;
  if (cid >= cm.nc_max) return;
  int tok0, L;
  chunk_of(cm, cid, tok0, L);
  if (L <= 0) return;                            // unused varlen table slot
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;

  // Gates of the first head batch (issued before the K/Q loads so both
  // latencies overlap): wave w < min(G, NB) owns value head gq*G + w.
  float al0 = 1.f, bl0 = 0.f;
  if (w < min(G, NB) && l < L) {
    const size_t gi = (size_t)(tok0 + l) * Hv + gq * G + w;
    al0 = alpha[gi];
    bl0 = beta[gi];
  }

  // Stage the chunk's K and Q rows (zero beyond L): every load is issued
  // before the first LDS write.
  constexpr int PPR = kD / EPV;                  // 16-byte pieces per row
  constexpr int NP = kC * PPR / 256;             // pieces per thread
  uint4 kv[NP], qv[NP];
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    const int p = tid + 256 * it, t = p / PPR, cb = p - (p / PPR) * PPR;
    const size_t off = ((size_t)(tok0 + t) * Hqk + gq) * kD + cb * EPV;
    kv[it] = ld16(k + off, t < L);
    qv[it] = ld16(q + off, t < L);
  }
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    const int p = tid + 256 * it, t = p / PPR, cb = p - (p / PPR) * PPR;
    *reinterpret_cast<uint4*>(sm.u.in.Ks + t * LDK + cb * EPV) = kv[it];
    *reinterpret_cast<uint4*>(sm.u.in.Qs + t * LDK + cb * EPV) = qv[it];
  }
  __syncthreads();

  f32x4 kk[4], kq[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) { kk[nt] = zero4(); kq[nt] = zero4(); }
  if constexpr (BF) {
    const bf16* Ks = reinterpret_cast<const bf16*>(sm.u.in.Ks);
    const bf16* Qs = reinterpret_cast<const bf16*>(sm.u.in.Qs);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 ak = lds_row8_bf16(Ks, LDK, 16 * w + r, 32 * ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt < w) continue;                    // tiles above the diagonal are masked
        kk[nt] = mfma_bf16(ak, lds_row8_bf16(Ks, LDK, 16 * nt + r, 32 * ks), kk[nt]);
        kq[nt] = mfma_bf16(ak, lds_row8_bf16(Qs, LDK, 16 * nt + r, 32 * ks), kq[nt]);
      }
    }
  } else {
    const float* Ks = reinterpret_cast<const float*>(sm.u.in.Ks);
    const float* Qs = reinterpret_cast<const float*>(sm.u.in.Qs);
    for (int s = 0; s < kD / 4; ++s) {
      const float ak = Ks[(16 * w + r) * LDK + 4 * s + g];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt < w) continue;
        kk[nt] = mfma_f32(ak, Ks[(16 * nt + r) * LDK + 4 * s + g], kk[nt]);
        kq[nt] = mfma_f32(ak, Qs[(16 * nt + r) * LDK + 4 * s + g], kq[nt]);
      }
    }
  }
  for (int hb = 0; hb < G; hb += NB) {
    const int nb = min(NB, G - hb);
    // Gates: G2_t = sum_{j<=t} log2(alpha_j) over the chunk, one wave per head.
    // fp32 inputs carry it as a compensated pair, so that exponent
    // differences G2_i - G2_j stay accurate to ~1e-7 at strong decay (|G2| of
    // hundreds within one chunk); bf16 inputs round A and M to bf16 anyway
    // (2^-9), far above the ~1e-5 of the plain prefix.
    if (w < nb) {
      const int h = gq * G + hb + w;
      float al = al0, bl = bl0;
      if (hb > 0) {
        const size_t gi = (size_t)(tok0 + l) * Hv + h;
        al = (l < L) ? alpha[gi] : 1.f;
        bl = (l < L) ? beta[gi] : 0.f;
      }
      float Glo = 0.f;
      const float Gl = BF ? wave_inclusive_sum(hw_log2(al)) : wave_inclusive_sum2(hw_log2(al), Glo);
      const float Glast = __shfl(Gl, kC - 1, 64);
      const float Glastlo = BF ? 0.f : __shfl(Glo, kC - 1, 64);
      ws.gam[((size_t)cid * Hv + h) * kC + l] = hw_exp2(Gl);
      ws.dec[((size_t)cid * Hv + h) * kC + l] = hw_exp2(BF ? Glast - Gl : (Glast - Gl) + (Glastlo - Glo));
      sm.gate[w][l] = Gl;
      if constexpr (!BF) sm.gatelo[w][l] = (bf16)Glo;
      sm.bet[w][l] = bl;
    }
    __syncthreads();   // gates visible; K/Q tiles (first batch) or the previous
                       // batch's buffers are dead from here on

    // A[i][j] = beta_i 2^(G2_i - G2_j) (k_i . k_j) for j < i, and the output
    // mask M[i][j] = 2^(G2_i - G2_j) (q_i . k_j) for j <= i; zero elsewhere.
    // This wave: columns j = 16w + 4g .. +3 of rows i = 16nt + r.
    for (int hh = 0; hh < nb; ++hh) {
      const int h = gq * G + hb + hh;
      float* A = sm.u.buf[hh];
      E* mo = ws.M + ((size_t)cid * Hv + h) * kC * kC;
      const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.gate[hh][16 * w + 4 * g]);
      bf16x4 gjlo{};
      if constexpr (!BF) gjlo = *reinterpret_cast<const bf16x4*>(&sm.gatelo[hh][16 * w + 4 * g]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int i = 16 * nt + r;
        float a4[4], m4[4];
        if (nt < w) {
#pragma unroll
          for (int e = 0; e < 4; ++e) { a4[e] = 0.f; m4[e] = 0.f; }
        } else {
          const float gi_ = sm.gate[hh][i], bi = sm.bet[hh][i];
          float gilo = 0.f;
          if constexpr (!BF) gilo = (float)sm.gatelo[hh][i];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * w + 4 * g + e;
            const float dx = BF ? gi_ - gj[e] : (gi_ - gj[e]) + (gilo - (float)gjlo[e]);
            const float dg = (j <= i) ? hw_exp2(dx) : 0.f;
            a4[e] = (j < i) ? bi * dg * kk[nt][e] : 0.f;
            m4[e] = dg * kq[nt][e];
          }
        }
        *reinterpret_cast<f32x4*>(A + i * kLdT + 16 * w + 4 * g) = f32x4{a4[0], a4[1], a4[2], a4[3]};
        if constexpr (BF) {
          bf16x4 mv;
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[e] = (bf16)m4[e];
          // The bf16 scan never reads the zero block rows 0..31 x columns 32..63.
          if (i >= 32 || w < 2 || solve_only)
            *reinterpret_cast<bf16x4*>(mo + i * kC + 16 * w + 4 * g) = mv;
        } else {
          *reinterpret_cast<f32x4*>(mo + i * kC + 16 * w + 4 * g) = f32x4{m4[0], m4[1], m4[2], m4[3]};
        }
      }
    }
    __syncthreads();

    // One wave per value head of the batch: (I + A)^-1 in place, then Tt.
    if (w < nb) {
      const int h = gq * G + hb + w;
      float* A = sm.u.buf[w];
      // Diagonal 16x16 blocks by forward substitution: lane = (block bb, column c).
      {
        const int bb = l >> 4, c = l & 15;
        const float* Ab = A + (16 * bb) * kLdT + 16 * bb;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < i; ++j) acc -= Ab[i * kLdT + j] * x[j];
          x[i] = acc;
        }
        wave_lds_fence();
        float* Tb = A + (16 * bb) * kLdT + 16 * bb;
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[i * kLdT + c] = x[i];
        wave_lds_fence();
      }

      // Off-diagonal blocks, block row by block row:
      //   T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
      for (int ib = 1; ib < 4; ++ib) {
        f32x4 Y[3];
#pragma unroll
        for (int jb = 0; jb < ib; ++jb) {
          Y[jb] = zero4();
          for (int kb = jb; kb < ib; ++kb)
            Y[jb] = mm16_lds(A, 16 * ib, 16 * kb, A, 16 * kb, 16 * jb, Y[jb]);
        }
        f32x4 Z[3];
#pragma unroll
        for (int jb = 0; jb < ib; ++jb) {
          Z[jb] = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s)
            Z[jb] = mfma_f32(A[(16 * ib + r) * kLdT + 16 * ib + 4 * g + s], Y[jb][s], Z[jb]);
        }
        wave_lds_fence();
#pragma unroll
        for (int jb = 0; jb < ib; ++jb)
#pragma unroll
          for (int i = 0; i < 4; ++i) A[(16 * ib + 4 * g + i) * kLdT + 16 * jb + r] = -Z[jb][i];
        wave_lds_fence();
      }

      // Tt = T diag(beta): lane = (8-column block, row group), 16-byte stores.
      E* tt = ws.Tt + ((size_t)cid * Hv + h) * kC * kC;
      {
        const int cb = l & 7, rg = l >> 3;
        float bj[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bj[e] = sm.bet[w][8 * cb + e];
        E* nn = solve_only ? ws.N + ((size_t)cid * Hv + h) * kC * kC : nullptr;
#pragma unroll
        for (int i0 = 0; i0 < 8; ++i0) {
          const int i = 8 * i0 + rg;
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(A + i * kLdT + 8 * cb);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(A + i * kLdT + 8 * cb + 4);
          const float t8[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          if constexpr (BF) {
            bf16x8 tv;
#pragma unroll
            for (int e = 0; e < 8; ++e) tv[e] = (bf16)(t8[e] * bj[e]);
            if (i >= 32 || cb < 4) *reinterpret_cast<bf16x8*>(tt + i * kC + 8 * cb) = tv;
            if (nn) {
#pragma unroll
              for (int e = 0; e < 8; ++e) tv[e] = (bf16)t8[e];
              *reinterpret_cast<bf16x8*>(nn + i * kC + 8 * cb) = tv;
            }
          } else {
            *reinterpret_cast<f32x4*>(tt + i * kC + 8 * cb) =
                f32x4{t8[0] * bj[0], t8[1] * bj[1], t8[2] * bj[2], t8[3] * bj[3]};
            *reinterpret_cast<f32x4*>(tt + i * kC + 8 * cb + 4) =
                f32x4{t8[4] * bj[4], t8[5] * bj[5], t8[6] * bj[6], t8[7] * bj[7]};
            if (nn) {
              *reinterpret_cast<f32x4*>(nn + i * kC + 8 * cb) = f32x4{t8[0], t8[1], t8[2], t8[3]};
              *reinterpret_cast<f32x4*>(nn + i * kC + 8 * cb + 4) = f32x4{t8[4], t8[5], t8[6], t8[7]};
            }
          }
        }
      }
    }
    if (hb + NB < G) __syncthreads();   // the next batch rewrites gates and buffers
  }
}

// ---------------------------------------------------------------- scan
// fp32 inputs only (the bf16 scan is scan_split_kernel below).
template <typename E, int NW, bool GATED>
struct ScanSmem {
  static_assert(sizeof(E) == 4, "fp32 scan");
  static constexpr int LDK = 132;                   // K, Q row stride
  static constexpr int LDO = GATED ? 16 * NW + 4 : 16 * NW + 8;
  E Ks[kC * LDK];
  E Qs[kC * LDK];
  E Tt[kC * kLdT];
  E Ms[kC * kLdT];
  typename std::conditional<GATED, float, E>::type Os[kC * LDO];
  float gam[kC];                                    // exp(G_t)
  float dec[kC];                                    // exp(G_last - G_t)
};

template <typename E, int NW, bool GATED>
__global__ __launch_bounds__(64 * NW) void scan_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const void* __restrict__ h0, E* __restrict__ o, void* __restrict__ ht, bool sbf,
    const E* __restrict__ gate, const float* __restrict__ norm_w, float norm_eps,
    Work<E> ws, ChunkMap cm, int Hqk, int Hv, int G) {
  using Sm = ScanSmem<E, NW, GATED>;
  constexpr int LDK = Sm::LDK, LDO = Sm::LDO;
  constexpr int NT = 64 * NW;
  constexpr int EPV = 16 / sizeof(E);
  constexpr int NSL = kD / (16 * NW);               // value-row slices per head
  __shared__ Sm sm;

  // Workgroup -> (value head, slice).  Slices of one head and the heads of one
  // query/key group sit on consecutive ids of the same XCD (ids are dealt to the
  // 8 XCDs round-robin), so their shared chunk operands meet in one L2.
  const int nlin = Hv * NSL;
  int lin = blockIdx.x;
  const int per_group = G * NSL;
  if ((Hqk & 7) == 0) {
    const int xcd = lin & 7, j = lin >> 3;
    lin = (xcd + 8 * (j / per_group)) * per_group + (j - (j / per_group) * per_group);
  }
  if (lin >= nlin) return;
  const int h = lin / NSL, sl = lin - (lin / NSL) * NSL;
  const int gq = h / G;
  const int seq = blockIdx.y;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int dvb = sl * 16 * NW;                     // first value row of the workgroup
  const int dv0 = dvb + 16 * w;                     // first value row of this wave

  int cid0, nch;
  if (cm.tab) {
    const_i32* so = (const_i32*)cm.seq_off;
    cid0 = so[seq];
    nch = min(so[seq + 1], cm.nc_max) - cid0;
  } else {
    cid0 = seq * cm.Nc;
    nch = cm.Nc;
  }

  // State S^T (d_k x 16 value rows) as 8 accumulator tiles: ST[t][i] holds
  // S[dv0 + r][16t + 4g + i].
  f32x4 ST[8];
  {
    const size_t hrow = (((size_t)seq * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      ST[t] = h0 ? load_state4(h0, hrow + 16 * t + 4 * g, sbf) : zero4();
  }

  // Chunk operands are fetched into registers one chunk ahead (issued right
  // after the staging barrier, consumed at the next staging), so their global
  // latency hides behind the current chunk's MFMA work.
  constexpr int KP = kC * (kD / EPV) / NT;          // 16-byte pieces of K (and Q) per thread
  constexpr int TP = kC * kC / EPV / NT;            // pieces of Tt (and M) per thread
  static_assert(KP * NT == kC * (kD / EPV) && TP * NT == kC * kC / EPV, "piece split");
  uint4 rk[KP], rq[KP], rt[TP], rm[TP];
  float rg = 0.f, rgl = 0.f;

  auto fetch = [&](int cid, int tok0, int L) {
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int p = tid + NT * it, t = p & 63, cb = p >> 6;
      const size_t off = ((size_t)(tok0 + t) * Hqk + gq) * kD + cb * EPV;
      rk[it] = ld16(k + off, t < L);
      rq[it] = ld16(q + off, t < L);
    }
    const E* tsrc = ws.Tt + ((size_t)cid * Hv + h) * kC * kC;
    const E* msrc = ws.M + ((size_t)cid * Hv + h) * kC * kC;
#pragma unroll
    for (int it = 0; it < TP; ++it) {
      const int p = tid + NT * it;
      rt[it] = *reinterpret_cast<const uint4*>(tsrc + p * EPV);
      rm[it] = *reinterpret_cast<const uint4*>(msrc + p * EPV);
    }
    if (tid < kC) {
      rg = ws.gam[((size_t)cid * Hv + h) * kC + tid];
      rgl = ws.dec[((size_t)cid * Hv + h) * kC + tid];
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int p = tid + NT * it, t = p & 63, cb = p >> 6;
      uint2* dk = reinterpret_cast<uint2*>(sm.Ks + t * LDK + cb * EPV);
      uint2* dq = reinterpret_cast<uint2*>(sm.Qs + t * LDK + cb * EPV);
      dk[0] = uint2{rk[it].x, rk[it].y}; dk[1] = uint2{rk[it].z, rk[it].w};
      dq[0] = uint2{rq[it].x, rq[it].y}; dq[1] = uint2{rq[it].z, rq[it].w};
    }
#pragma unroll
    for (int it = 0; it < TP; ++it) {
      const int e0 = (tid + NT * it) * EPV, i = e0 >> 6, j = e0 & 63;
      uint2* dt = reinterpret_cast<uint2*>(sm.Tt + i * kLdT + j);
      uint2* dm = reinterpret_cast<uint2*>(sm.Ms + i * kLdT + j);
      dt[0] = uint2{rt[it].x, rt[it].y}; dt[1] = uint2{rt[it].z, rt[it].w};
      dm[0] = uint2{rm[it].x, rm[it].y}; dm[1] = uint2{rm[it].z, rm[it].w};
    }
    if (tid < kC) {
      sm.gam[tid] = rg;
      sm.dec[tid] = rgl;
    }
  };

  auto write_out = [&](int otok0, int oL) {
    if constexpr (GATED) {
      // y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate), whole head per row.
      static_assert(!GATED || NW == 8, "the fused epilogue needs the whole head");
      const int row = tid >> 3, part = tid & 7;
      if (row < oL) {
        const float* orow = sm.Os + row * LDO + 16 * part;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) ss += orow[j] * orow[j];
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        ss += __shfl_xor(ss, 4, 64);
        const float rn = rsqrtf(ss * (1.f / kD) + norm_eps);
        const size_t base = ((size_t)(otok0 + row) * Hv + h) * kD + 16 * part;
        const E* gp = gate + base;
        E* op = o + base;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float wj = norm_w ? norm_w[16 * part + j] : 1.f;
          const float sg = 1.f / (1.f + __expf(-to_f32(gp[j])));
          op[j] = from_f32<E>(orow[j] * rn * wj * sg);
        }
      }
    } else {
      constexpr int PPR = 16 * NW / EPV;            // 16-byte pieces per output row
      for (int p = tid; p < kC * PPR; p += NT) {
        const int t = p / PPR, cb = p - (p / PPR) * PPR;
        if (t < oL) {
          const uint4 val = *reinterpret_cast<const uint4*>(sm.Os + t * LDO + cb * EPV);
          *reinterpret_cast<uint4*>(o + ((size_t)(otok0 + t) * Hv + h) * kD + dvb +
                                    cb * EPV) = val;
        }
      }
    }
  };

  int tok0 = 0, L = 0, ptok0 = 0, pL = 0;
  if (nch > 0) {
    chunk_of(cm, cid0, tok0, L);
    fetch(cid0, tok0, L);
  }
  for (int c = 0; c < nch; ++c) {
    // ---- phase 1: registers -> LDS for chunk c; chunk c-1's outputs -> HBM.
    stage();
    if (c > 0) write_out(ptok0, pL);
    __syncthreads();
    int ntok0 = 0, nL = 0;
    if (c + 1 < nch) {
      chunk_of(cm, cid0 + c + 1, ntok0, nL);
      fetch(cid0 + c + 1, ntok0, nL);
    }
    // ---- phase 2: this wave's 16 value rows.
    const float gL = sm.gam[kC - 1];
    f32x4 P[4], QS[4], X[4], Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { P[mt] = zero4(); QS[mt] = zero4(); Dl[mt] = zero4(); }

    // P = K S0^T and QS = Q S0^T (contraction over d_k).
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      mma_acc_f32<8>(P[mt], sm.Ks, LDK, 16 * mt, 0, ST);
      mma_acc_f32<8>(QS[mt], sm.Qs, LDK, 16 * mt, 0, ST);
    }

    // X = V - diag(exp G) P.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int t0 = 16 * mt + 4 * g;
      float vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vv[i] = (t0 + i < L) ? v[((size_t)(tok0 + t0 + i) * Hv + h) * kD + dv0 + r] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) X[mt][i] = vv[i] - sm.gam[t0 + i] * P[mt][i];
    }

    // Dl = Tt X (contraction over tokens of the chunk).
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) mma_acc_f32<4>(Dl[mt], sm.Tt, kLdT, 16 * mt, 0, X);

    // O = diag(exp G) QS + M Dl  ->  LDS staging.
    {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) QS[mt][i] *= sm.gam[16 * mt + 4 * g + i];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) mma_acc_f32<4>(QS[mt], sm.Ms, kLdT, 16 * mt, 0, Dl);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * mt + 4 * g + i;
          if constexpr (GATED)
            sm.Os[t * LDO + 16 * w + r] = QS[mt][i];
          else
            sm.Os[t * LDO + 16 * w + r] = from_f32<E>(QS[mt][i]);
        }
    }

    // S^T <- exp(G_last) S^T + K^T diag(exp(G_last - G)) Dl.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Dl[mt][i] *= sm.dec[16 * mt + 4 * g + i];
#pragma unroll
    for (int t = 0; t < 8; ++t) ST[t] *= gL;
#pragma unroll
    for (int t = 0; t < 8; ++t) mma_acc_f32_tA<4>(ST[t], sm.Ks, LDK, 16 * t, 0, Dl);
    ptok0 = tok0;
    pL = L;
    tok0 = ntok0;
    L = nL;
    __syncthreads();
  }
  if (nch > 0) write_out(ptok0, pL);

  if (ht) {
    const size_t hrow = (((size_t)seq * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) store_state4(ht, hrow + 16 * t + 4 * g, ST[t], sbf);
  }
}

// ---------------------------------------------------------------- split scan (bf16)
// The bf16 scan with the work of each 16-row value slice split between two
// waves and all chunk operands brought into LDS by two more:
//
//  * chain wave (one per slice): the serial part only.  P = K S^T, X, Dl =
//    Tt X, the state update; it hands S^T (as the B fragments it built for P)
//    and Dl to the output wave through LDS.  40 MFMAs per chunk.
//  * one output wave for both slices, one chunk behind: O = diag(gam) Q S^T +
//    M Dl, formed transposed (O^T = S Q^T diag(gam) + Dl^T M^T: the chain's
//    fragments are the A operands, Q and M rows the B operands), so that each
//    lane holds four consecutive value rows of one token and stores them to
//    global memory as one 8-byte write.  Each Q and M fragment read from LDS
//    serves both slices: 44 MFMAs per chunk.
//  * two producer waves: copy K, Tt, V, gam, dec of chunk c+2 and Q, M of
//    chunk c from global memory straight into LDS rings
//    (global_load_lds_dwordx4: no registers, no VALU) while chunk c is
//    computed.  K comes straight from the input tensor.
//
// K is staged once per chunk, as it is stored ([64 tokens][128 d_k]).  The A
// fragments of P = K S^T (rows = tokens, K slots = d_k) are 16-byte reads of
// it; those of the state update K^T Dl (rows = d_k, K slots = tokens) come
// from the same tile through ds_read_b64_tr_b16, which transposes 16-bit
// elements across each group of 16 lanes: input lane p reads four d_k of
// token base + p/4, and output lane m receives element m%4 of input lanes
// m/4, m/4+4, m/4+8, m/4+12, i.e. four tokens of d_k row(m).
//
// Token and d_k order.  An accumulator tile pair holds, per lane group g, rows
// {4g..4g+3} and {16+4g..16+4g+3} of a 32-row block; used as a B fragment these
// are the K slots.  Inside each 32-row block the library stores logical row
// x at physical position prow(x) = 8*((x%16)/4) + 4*(x/16) + x%4, so that the 8
// K slots of lane group g are the 8 consecutive physical rows 8g..8g+7 and
// every A fragment is one 16-byte LDS read (or two transposed 8-byte reads).
// The permutation is applied to tokens (rows of P, X, Dl) and to d_k (rows of
// S^T); it is undone where the state is loaded and stored.  LDS rows are
// XOR-swizzled in 16-byte pieces (swz for 128-byte rows, ksw for the K tile's
// 256-byte rows) so that every 16-lane pass of an A fragment read hits
// distinct banks.
namespace split {
constexpr int kSlices = 2;                   // 16-row value slices per workgroup
constexpr int kRows = 16 * kSlices;          // value rows per workgroup
constexpr int kNsl = kD / kRows;             // workgroups per value head
constexpr int kWaves = kSlices + 3;          // chain x2, output, producer x2
constexpr int kSlots = 3;                    // chain operands: chunks c, c+1, c+2
constexpr int kQmSlots = 2;                  // output operands: chunks c-1, c
constexpr int kGdSlots = 4;                  // gam/dec: chunks c-1 .. c+2
constexpr int kKTB = kD * kC * 2;            // K tile, bytes
constexpr int kTB = kC * kC * 2;             // Tt tile
constexpr int kVB = kC * kRows * 2;          // V tile of the workgroup's value rows
constexpr int kQB = kC * kD * 2;             // Q tile
constexpr int kMB = kC * kC * 2;             // M tile
// Copy ops of each producer per chunk; each keeps at most 63 in flight.
constexpr int kOpsT = kTB / 1024 + 2;                   // producer 0: Tt, gam, dec (chunk c+2)
constexpr int kOpsKV = kKTB / 1024 + kVB / 1024;        // producer 1: K, V         (chunk c+2)
static_assert(2 * kOpsT + kQB / 1024 <= 63 && 2 * kOpsKV + kMB / 1024 <= 63, "vmcnt range");

struct Slot {
  alignas(16) uint8_t K[kKTB];               // [64 tokens][128 d_k], 256-byte rows
  alignas(16) uint8_t T[kTB];                // [64][64], 128-byte rows
  alignas(16) uint8_t V[kVB];                // [64 tokens][32 value rows], 64-byte rows
};
struct QmSlot {
  alignas(16) uint8_t Q[kQB];                // [64 tokens][128 d_k], 256-byte rows
  alignas(16) uint8_t M[kMB];                // [64][64], 128-byte rows
};
struct GateSlot {
  alignas(16) float gam[kC];
  alignas(16) float dec[kC];
};
struct Hand {
  bf16x8 sb[4][64];                          // S^T B fragments of the chain wave
  bf16x8 db[2][64];                          // Dl B fragments
};
struct Smem {
  Slot slot[kSlots];
  QmSlot qm[kQmSlots];
  GateSlot gd[kGdSlots];
  Hand hand[2][kSlices];
};

// logical row r of 16-row tile t -> physical row (see above)
__device__ __forceinline__ int prow(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}
__device__ __forceinline__ int swz(int row) { return (row & 3) | ((row >> 1) & 4); }
// K tile rows are 16 pieces: rows prow(mt, 0..15) (plain reads) and the four
// tokens base + 0..3 of a transposed read both land on 16 distinct pieces.
__device__ __forceinline__ int ksw(int row) { return ((row & 3) << 2) | ((row >> 3) & 3); }
// V tile rows are 4 pieces of 16 bytes; a chain wave reads 8 consecutive tokens
// 8 apart per lane group, so the piece order is rotated by (token / 8) % 4.
__device__ __forceinline__ int vswz(int tok) { return (tok >> 3) & 3; }

using frag::barrier_lds;
using frag::dma16;
using frag::dma4;
using frag::lds_tr16;
using frag::s16x4;

// Copies of a [rows][bytes_per_row] tile of 16-byte pieces with XOR swizzle:
// instruction `it` fills LDS bytes [1024 it, 1024 it + 1024).
}  // namespace split

template <bool CKPT>
__global__ __launch_bounds__(64 * split::kWaves) void scan_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ h0, bf16* __restrict__ o, void* __restrict__ ht, bool sbf, Work<bf16> ws,
    ChunkMap cm, int Hqk, int Hv, int G, bf16* __restrict__ states) {
  using namespace split;
  __shared__ Smem sm;

  const int nlin = Hv * kNsl;
  int lin = blockIdx.x;
  const int per_group = G * kNsl;
  if ((Hqk & 7) == 0) {
    const int xcd = lin & 7, j = lin >> 3;
    lin = (xcd + 8 * (j / per_group)) * per_group + (j - (j / per_group) * per_group);
  }
  if (lin >= nlin) return;                          // whole workgroup leaves together
  const int h = lin / kNsl, sl = lin - (lin / kNsl) * kNsl;
  const int gq = h / G;
  const int seq = blockIdx.y;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int dvb = sl * kRows;

  int cid0, nch;
  if (cm.tab) {
    const_i32* so = (const_i32*)cm.seq_off;
    cid0 = so[seq];
    nch = min(so[seq + 1], cm.nc_max) - cid0;
  } else {
    cid0 = seq * cm.Nc;
    nch = cm.Nc;
  }

  const size_t hv_stride = (size_t)Hv * kD;         // elements between tokens of v / o
  const size_t qk_stride = (size_t)Hqk * kD;

  if (w >= kSlices + 1) {
    // ------------------------------------------------------------ producers
    const int pw = w - kSlices - 1;
    // Copy sources are a uniform base plus a 32-bit byte offset (one chunk's
    // rows span far less than 2 GiB), which avoids a 64-bit multiply per copy.
    // Rows beyond L repeat the last token: K rows meet zero Tt columns and
    // zero decay-scaled Dl rows, V rows zero Tt columns, Q rows outputs that
    // are not stored.
    // Tt, gam, dec of chunk c into ring slots (c % 3, c % 4).
    auto issue_t = [&](int c) {
      const int cid = cid0 + c;
      Slot& S = sm.slot[c % kSlots];
      const bf16* tb = ws.Tt + ((size_t)cid * Hv + h) * kC * kC;
#pragma unroll
      for (int it = 0; it < kTB / 1024; ++it) {
        const int row = 8 * it + (l >> 3), p = (l & 7) ^ swz(row);
        dma16(reinterpret_cast<const char*>(tb) + (uint32_t)(2 * (row * kC + 8 * p)), S.T + 1024 * it);
      }
      GateSlot& Gd = sm.gd[c % kGdSlots];
      dma4(ws.gam + ((size_t)cid * Hv + h) * kC + l, Gd.gam);
      dma4(ws.dec + ((size_t)cid * Hv + h) * kC + l, Gd.dec);
    };
    // K (4 tokens per copy, from the input) and the workgroup's V rows of
    // chunk c into slot c % 3.
    auto issue_kv = [&](int c) {
      const int cid = cid0 + c;
      int tok0, L;
      chunk_of(cm, cid, tok0, L);
      Slot& S = sm.slot[c % kSlots];
      const bf16* kbase = k + (size_t)tok0 * qk_stride + (size_t)gq * kD;
#pragma unroll
      for (int it = 0; it < kKTB / 1024; ++it) {
        const int row = 4 * it + (l >> 4), p = (l & 15) ^ ksw(row);
        dma16(reinterpret_cast<const char*>(kbase) +
                  ((uint32_t)min(row, L - 1) * (uint32_t)(2 * qk_stride) + 16u * p),
              S.K + 1024 * it);
      }
      const bf16* vbase = v + (size_t)tok0 * hv_stride + (size_t)h * kD + dvb;
#pragma unroll
      for (int it = 0; it < kVB / 1024; ++it) {
        const int row = 16 * it + (l >> 2), p = (l & 3) ^ vswz(row);
        dma16(reinterpret_cast<const char*>(vbase) +
                  ((uint32_t)min(row, L - 1) * (uint32_t)(2 * hv_stride) + 16u * p),
              S.V + 1024 * it);
      }
    };
    // Q, and M, of chunk c into qm slot c % 2.
    auto issue_q = [&](int c) {
      const int cid = cid0 + c;
      int tok0, L;
      chunk_of(cm, cid, tok0, L);
      QmSlot& Qs = sm.qm[c % kQmSlots];
      const bf16* qbase = q + (size_t)tok0 * qk_stride + (size_t)gq * kD;
#pragma unroll
      for (int it = 0; it < kQB / 1024; ++it) {
        const int row = 4 * it + (l >> 4), p = (l & 15) ^ swz(row);
        dma16(reinterpret_cast<const char*>(qbase) +
                  ((uint32_t)min(row, L - 1) * (uint32_t)(2 * qk_stride) + 16u * p),
              Qs.Q + 1024 * it);
      }
    };
    auto issue_m = [&](int c) {
      const int cid = cid0 + c;
      QmSlot& Qs = sm.qm[c % kQmSlots];
      const bf16* mb = ws.M + ((size_t)cid * Hv + h) * kC * kC;
#pragma unroll
      for (int it = 0; it < kMB / 1024; ++it) {
        const int row = 8 * it + (l >> 3), p = (l & 7) ^ swz(row);
        dma16(reinterpret_cast<const char*>(mb) + (uint32_t)(2 * (row * kC + 8 * p)), Qs.M + 1024 * it);
      }
    };
    // Chunk c's chain operands must be in LDS by the barrier that ends
    // iteration c-1, its Q and M by the one that ends iteration c.  The two
    // producers split the copies about evenly (Q + Tt + gates: 26, M + K + V:
    // 28 per chunk); each issues its output operand of chunk i before its
    // chain operands of chunk i+2 and then waits until only the latter are
    // pending (vector memory operations complete in issue order).  The
    // state-checkpoint pass has no outputs, so it copies no Q and M.
    auto produce = [&](auto first, auto out, auto chain_ops) {
      constexpr int kOps = decltype(chain_ops)::value;
      if (nch > 0) first(0);
      if (nch > 1) {
        first(1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOps) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      barrier_lds();
      for (int i = 0; i <= nch; ++i) {
        if (!CKPT && i < nch) out(i);
        if (i + 2 < nch) {
          first(i + 2);
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOps) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        barrier_lds();
      }
    };
    if (pw == 0)
      produce(issue_t, issue_q, std::integral_constant<int, kOpsT>{});
    else
      produce(issue_kv, issue_m, std::integral_constant<int, kOpsKV>{});
    return;
  }

  if (w < kSlices) {
    // ------------------------------------------------------------ chain wave
    const int s = w, dv0 = dvb + 16 * s;
    // S^T accumulator tiles: ST[t][i] = S[dv0 + r][prow(t, 4g + i)].
    f32x4 ST[8];
    {
      const size_t hrow = (((size_t)seq * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        ST[t] = h0 ? load_state4(h0, hrow + prow(t, 4 * g), sbf) : zero4();
    }
    barrier_lds();
    for (int i = 0; i <= nch; ++i) {
      if (i < nch) {
        const Slot& S = sm.slot[i % kSlots];
        const GateSlot& Gd = sm.gd[i % kGdSlots];
        Hand& H = sm.hand[i & 1][s];
        // A fragments of P = K S^T: row prow(mt, r) of the K tile, d_k
        // 32kk + 8g .. +7.
        bf16x8 AK[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = prow(mt, r);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            AK[mt][kk] = *reinterpret_cast<const bf16x8*>(S.K + row * 256 + 16 * ((4 * kk + g) ^ ksw(row)));
        }
        bf16x8 SB[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          SB[kk] = pack_b(ST[2 * kk], ST[2 * kk + 1]);
          H.sb[kk][l] = SB[kk];
        }
        // P = K S^T  (rows: physical tokens prow(mt, r))
        f32x4 P[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) P[mt] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) P[mt] = mfma_bf16(AK[mt][kk], SB[kk], P[mt]);
        // Tt fragments
        bf16x8 AT[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = prow(mt, r);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            AT[mt][kk] = *reinterpret_cast<const bf16x8*>(S.T + row * 128 + 16 * ((4 * kk + g) ^ swz(row)));
        }
        // A fragments of the update K^T Dl (rows d_k prow(t, .), K slots
        // tokens 32kk + 8g .. +7) by transposed reads: as input lane r of
        // group g this lane reads d_k 32(t/2) + 8(r%4) + 4(t%2) .. +3 of
        // token 32kk + 8g + r/4 (and of the token 4 later).
        bf16x8 AKT[8][2];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int dk = 32 * (t >> 1) + 8 * (r & 3) + 4 * (t & 1);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int t0 = 32 * kk + 8 * g + (r >> 2), t1 = t0 + 4;
            const s16x4 lo = lds_tr16(S.K + t0 * 256 + 16 * ((dk >> 3) ^ ksw(t0)) + 2 * (dk & 7));
            const s16x4 hi = lds_tr16(S.K + t1 * 256 + 16 * ((dk >> 3) ^ ksw(t1)) + 2 * (dk & 7));
            const s16x4 lh[2] = {lo, hi};
            AKT[t][kk] = *reinterpret_cast<const bf16x8*>(lh);
          }
        }
        // V of this lane's value row at its tokens 32(mt/2) + 8g + 4(mt%2) + i,
        // by transposed reads: as input lane r of group g this lane reads 4
        // value rows (16s + 4(r%4) ..+3) of token 32(mt/2) + 8g + 4(mt%2) + r/4.
        // Rows beyond L hold a copy of the last token; they only meet the zero
        // columns of Tt, so they need no masking.
        s16x4 vt[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int tok = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + (r >> 2);
          const int col = 16 * s + 4 * (r & 3);
          vt[mt] = lds_tr16(S.V + tok * (2 * kRows) + 16 * ((col >> 3) ^ vswz(tok)) + 2 * (col & 7));
        }
        // X = V - diag(gam) P
        f32x4 X[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 gm = *reinterpret_cast<const f32x4*>(Gd.gam + 32 * (mt >> 1) + 8 * g + 4 * (mt & 1));
          const bf16* v4 = reinterpret_cast<const bf16*>(&vt[mt]);
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) X[mt][i2] = (float)v4[i2] - gm[i2] * P[mt][i2];
        }
        const bf16x8 XB[2] = {pack_b(X[0], X[1]), pack_b(X[2], X[3])};
        // Dl = Tt X.  Tt is lower triangular: tiles mt < 2 (rows 0..31) have
        // nothing in columns 32..63.
        f32x4 Dl[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Dl[mt] = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            if (kk == 0 || mt >= 2) Dl[mt] = mfma_bf16(AT[mt][kk], XB[kk], Dl[mt]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) H.db[kk][l] = pack_b(Dl[2 * kk], Dl[2 * kk + 1]);
        // state update: S^T <- gam_last S^T + K^T diag(dec) Dl
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 dc = *reinterpret_cast<const f32x4*>(Gd.dec + 32 * (mt >> 1) + 8 * g + 4 * (mt & 1));
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) Dl[mt][i2] *= dc[i2];
        }
        const bf16x8 DTB[2] = {pack_b(Dl[0], Dl[1]), pack_b(Dl[2], Dl[3])};
        const float gL = Gd.gam[kC - 1];
#pragma unroll
        for (int t = 0; t < 8; ++t) ST[t] *= gL;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int t = 0; t < 8; ++t) ST[t] = mfma_bf16(AKT[t][kk], DTB[kk], ST[t]);
      }
      barrier_lds();
    }
    if (ht) {
      const size_t hrow = (((size_t)seq * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
      for (int t = 0; t < 8; ++t) store_state4(ht, hrow + prow(t, 4 * g), ST[t], sbf);
    }
    return;
  }

  // -------------------------------------------------------------- output wave
  // Chunk c's O at iteration c+1 for both value slices.  In the
  // state-checkpoint pass of the backward there are no outputs: instead this
  // wave stores the state entering chunk c (bf16), from the fragments the
  // chain waves hand over, so that the chain waves issue no global stores.
  barrier_lds();
  for (int i = 0; i <= nch; ++i) {
    if (i >= 1 && CKPT) {
      const int c = i - 1;
      // Fragment kk of chain lane (r', g') holds d_k prow(2kk, 4g') .. +3 then
      // prow(2kk + 1, 4g') .. +3, i.e. the eight consecutive d_k 32kk + 8g' ..
      // +7, of value row 16s + r'.  Each store writes four whole 256-byte rows:
      // lane l takes row 4j + l/16 and d_k 8p .. +7 (p = l % 16), which chain
      // lane (4j + l/16, p % 4) holds in fragment p / 4.
      const int pc = l & 15, rr = l >> 4;
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        bf16* sbase = states + ((((size_t)(cid0 + c) * Hv + h) * kD + dvb + 16 * s) * kD) + 8 * pc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + rr;
          *reinterpret_cast<bf16x8*>(sbase + (size_t)row * kD) = sm.hand[c & 1][s].sb[pc >> 2][row + 16 * (pc & 3)];
        }
      }
    }
    if (i >= 1 && !CKPT) {
      const int c = i - 1;
      int tok0, L;
      chunk_of(cm, cid0 + c, tok0, L);
      const QmSlot& Qs = sm.qm[c % kQmSlots];
      const GateSlot& Gd = sm.gd[c % kGdSlots];
      bf16x8 SB[kSlices][4], DB[kSlices][2];
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) SB[s][kk] = sm.hand[c & 1][s].sb[kk][l];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) DB[s][kk] = sm.hand[c & 1][s].db[kk][l];
      }
      bf16* ob = o + (size_t)tok0 * hv_stride + (size_t)h * kD + dvb + 4 * g;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = 16 * nt + r;
        f32x4 OT[kSlices];
#pragma unroll
        for (int s = 0; s < kSlices; ++s) OT[s] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(Qs.Q + row * 256 + 16 * ((4 * kk + g) ^ swz(row)));
#pragma unroll
          for (int s = 0; s < kSlices; ++s) OT[s] = mfma_bf16(SB[s][kk], bq, OT[s]);
        }
        const float gm = Gd.gam[row];
#pragma unroll
        for (int s = 0; s < kSlices; ++s) OT[s] *= gm;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk == 1 && nt < 2) continue;
          const bf16x8 bm = *reinterpret_cast<const bf16x8*>(Qs.M + row * 128 + 16 * ((4 * kk + g) ^ swz(row)));
#pragma unroll
          for (int s = 0; s < kSlices; ++s) OT[s] = mfma_bf16(DB[s][kk], bm, OT[s]);
        }
        if (row < L) {
#pragma unroll
          for (int s = 0; s < kSlices; ++s) {
            bf16x4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (bf16)OT[s][e];
            *reinterpret_cast<bf16x4*>(ob + (size_t)row * hv_stride + 16 * s) = ov;
          }
        }
      }
    }
    barrier_lds();
  }
}

// ---------------------------------------------------------------- head-wide scan (bf16)
// The bf16 scan with one workgroup per (value head, sequence), for calls with
// many (sequence, head) pairs and for the gated RMSNorm epilogue, which needs
// every value row of a token in one workgroup:
//
//  * four chain waves, one per SIMD, each owning 32 value rows as two
//    independent 16-row slices whose MFMA chains interleave (one slice's
//    products fill the other's dependency gaps, and every A fragment read
//    from LDS serves both).  Besides the chain (P = K S^T, X, Dl = Tt X, the
//    state update) each forms its rows of the output,
//    O^T = S Q^T diag(gam) + Dl^T M^T, as the split scan's output wave does,
//    with the same products in the same order (so the plain output equals the
//    split scan's bit for bit).  Chunk c's output is stored at the start of
//    iteration c+1 and its stores are waited for at the end of that
//    iteration, a whole chunk of work after they were issued;
//  * four copy waves: K, Q, V (all 128 value rows) with gam/dec, and Tt with
//    M of chunk c+1 go straight into the other slot of a two-slot LDS ring
//    (global_load_lds_dwordx4) while chunk c is computed.
//
// Fragment layouts, swizzles and the token / d_k permutation are those of
// the split scan.  V rows (256 bytes, 16 pieces) are swizzled by vsw so that
// a chain wave's transposed read of 16 tokens x 16 value rows spreads over
// eight 32-byte segments, two tokens each.
//
// Gated: y = o / sqrt(mean_dv o^2 + eps) * w * sigmoid(gate).  The chain
// waves add only the per-token sums of o^2 over their rows (into LDS, three
// chunks deep).  The copy waves, which have issue slots to spare, apply the
// epilogue two chunks behind: once chunk c's o is in memory (stored in
// iteration c+1, complete before the barrier ending it), they read it back
// with the gate, scale it and write y over it in iteration c+2.
namespace hw {
using frag::barrier_lds;
using frag::dma16;
using frag::dma4;
using frag::lds_tr16;
using frag::s16x4;
constexpr int kCW = 4;                      // chain waves (32 value rows each)
constexpr int kPW = 4;                      // copy waves
constexpr int kWaves = kCW + kPW;
struct Slot {
  alignas(16) uint8_t K[kC * kD * 2];       // [64 tokens][128 d_k], 256-byte rows, ksw
  alignas(16) uint8_t Q[kC * kD * 2];       // [64 tokens][128 d_k], 256-byte rows, swz
  alignas(16) uint8_t T[kC * kC * 2];       // [64][64], 128-byte rows, swz
  alignas(16) uint8_t M[kC * kC * 2];       // [64][64], 128-byte rows, swz
  alignas(16) uint8_t V[kC * kD * 2];       // [64 tokens][128 value rows], 256-byte rows, vsw
  alignas(16) float gam[kC];
  alignas(16) float dec[kC];
};
struct Smem {
  Slot slot[2];
  float part[3][kCW][kC];                   // gated: per-wave sums of o^2 per token
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS");
__device__ __forceinline__ int vsw(int tok) { return 2 * ((tok & 3) | (((tok >> 3) & 1) << 2)); }
// Wait until at most N of this wave's vector memory operations are pending
// (they complete in issue order).
template <int N> __device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
}  // namespace hw

template <bool GATED>
__global__ __launch_bounds__(64 * hw::kWaves) void scan_head_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ h0, bf16* __restrict__ o, void* __restrict__ ht, bool sbf,
    const bf16* __restrict__ gate, const float* __restrict__ norm_w, float norm_eps,
    Work<bf16> ws, ChunkMap cm, int Hqk, int Hv, int G) {
  using namespace hw;
  using split::ksw;
  using split::prow;
  using split::swz;
  __shared__ Smem sm;

  // Heads of one query/key group on consecutive ids of one XCD (ids are dealt
  // to the 8 XCDs round-robin), so that their K and Q meet in one L2.
  int lin = blockIdx.x;
  if ((Hqk & 7) == 0) {
    const int xcd = lin & 7, j = lin >> 3;
    lin = (xcd + 8 * (j / G)) * G + (j - (j / G) * G);
  }
  if (lin >= Hv) return;                           // whole workgroup leaves together
  const int h = lin, gq = h / G, seq = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), r = l & 15, g = l >> 4;
  int cid0, nch;
  seq_chunks(cm, seq, cid0, nch);
  const size_t hv_stride = (size_t)Hv * kD;
  const size_t qk_stride = (size_t)Hqk * kD;

  // Iterations 0 .. nch+1: chunk i computed in iteration i, its output
  // stored in iteration i+1, its gated epilogue applied in iteration i+2.
  if (w >= kCW) {
    // ------------------------------------------------------------ copy waves
    // Rows beyond L repeat the last token (K: they meet zero Tt columns and
    // zero decay-scaled Dl rows; Q: their outputs are never stored; V: zero
    // Tt columns).
    const int pw = w - kCW;
    auto issue = [&](int c) {
      const int cid = cid0 + c;
      int tok0, L;
      chunk_of(cm, cid, tok0, L);
      Slot& S = sm.slot[c & 1];
      if (pw < 3) {
        const bf16* base = pw == 0   ? k + (size_t)tok0 * qk_stride + (size_t)gq * kD
                           : pw == 1 ? q + (size_t)tok0 * qk_stride + (size_t)gq * kD
                                     : v + (size_t)tok0 * hv_stride + (size_t)h * kD;
        const size_t stride = pw == 2 ? hv_stride : qk_stride;
        uint8_t* dst = pw == 0 ? S.K : pw == 1 ? S.Q : S.V;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
          const int row = 4 * it + (l >> 4);
          const int sw = pw == 0 ? ksw(row) : pw == 1 ? swz(row) : vsw(row);
          dma16(reinterpret_cast<const char*>(base) +
                    ((uint32_t)min(row, L - 1) * (uint32_t)(2 * stride) + 16u * ((l & 15) ^ sw)),
                dst + 1024 * it);
        }
        if (pw == 2) {
          dma4(ws.gam + ((size_t)cid * Hv + h) * kC + l, S.gam);
          dma4(ws.dec + ((size_t)cid * Hv + h) * kC + l, S.dec);
        }
      } else {
        const size_t tm = ((size_t)cid * Hv + h) * kC * kC;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int row = 8 * it + (l >> 3), p = (l & 7) ^ swz(row);
          const uint32_t off = (uint32_t)(2 * (row * kC + 8 * p));
          dma16(reinterpret_cast<const char*>(ws.Tt + tm) + off, S.T + 1024 * it);
          dma16(reinterpret_cast<const char*>(ws.M + tm) + off, S.M + 1024 * it);
        }
      }
    };
    // gated epilogue of chunk c: this wave's 16 tokens 16 pw + l/4, lane
    // quarter l%4 holds value rows 32(l%4) .. +31
    const int erow = 16 * pw + (l >> 2), edv = 32 * (l & 3);
    float nw[32];
    if constexpr (GATED) {
#pragma unroll
      for (int e = 0; e < 32; ++e) nw[e] = norm_w ? norm_w[edv + e] : 1.f;
    }
    uint4 ov[4], gv[4];
    size_t eoff = 0;
    int eL = 0;
    auto epilogue_load = [&](int c) {
      int tok0;
      chunk_of(cm, cid0 + c, tok0, eL);
      eoff = ((size_t)tok0 + min(erow, eL - 1)) * hv_stride + (size_t)h * kD + edv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ov[j] = *reinterpret_cast<const uint4*>(o + eoff + 8 * j);
        gv[j] = *reinterpret_cast<const uint4*>(gate + eoff + 8 * j);
      }
    };
    auto epilogue = [&](int c) {
      const size_t off = eoff;
      const int L = eL;
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < kCW; ++ww) tot += sm.part[c % 3][ww][erow];
      const float rn = rsqrtf(tot * (1.f / kD) + norm_eps);
      if (erow < L) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16* o8 = reinterpret_cast<const bf16*>(&ov[j]);
          const bf16* g8 = reinterpret_cast<const bf16*>(&gv[j]);
          bf16x8 y;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // hardware reciprocal (1 ulp): far below the bf16 rounding of y
            const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-(float)g8[e]));
            y[e] = (bf16)((float)o8[e] * rn * nw[8 * j + e] * sg);
          }
          *reinterpret_cast<bf16x8*>(o + off + 8 * j) = y;
        }
      }
    };
    if (nch > 0) issue(0);
    wait_vm<0>();
    barrier_lds();
    for (int i = 0; i <= nch + 1; ++i) {
      if (i + 1 < nch) issue(i + 1);
      if constexpr (GATED) {
        if (i >= 2) {
          // chunk i-2's o and gate are read, and its y written, after the
          // copies (the counted wait below relies on that order: vector
          // memory operations complete in issue order)
          asm volatile("" ::: "memory");
          epilogue_load(i - 2);
          epilogue(i - 2);
          // the copies of chunk i+1 are complete; the y stores (the last
          // four operations, issued unless no token of this wave is in the
          // chunk) may still be in flight
          if (16 * pw < eL) wait_vm<4>();
          else wait_vm<0>();
        } else {
          wait_vm<0>();
        }
      } else {
        wait_vm<0>();
      }
      barrier_lds();
    }
    return;
  }

  // -------------------------------------------------------------- chain waves
  const int dvw = 32 * w;                          // first value row of this wave
  f32x4 ST[2][8];                                  // ST[s][t][i] = S[dvw + 16s + r][prow(t, 4g + i)]
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const size_t hrow = (((size_t)seq * Hv + h) * kD + dvw + 16 * s + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) ST[s][t] = h0 ? load_state4(h0, hrow + prow(t, 4 * g), sbf) : zero4();
  }
  bf16x4 OB[2][4];                                 // the previous chunk's o
  int ptok0 = 0, pL = 0;
  barrier_lds();
  for (int i = 0; i <= nch + 1; ++i) {
    if (i >= 1 && i <= nch) {
      bf16* ob = o + (size_t)ptok0 * hv_stride + (size_t)h * kD + dvw + 4 * g;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = 16 * nt + r;
        if (row < pL) {
#pragma unroll
          for (int s = 0; s < 2; ++s) *reinterpret_cast<bf16x4*>(ob + (size_t)row * hv_stride + 16 * s) = OB[s][nt];
        }
      }
    }
    if (i < nch) {
      int tok0, L;
      chunk_of(cm, cid0 + i, tok0, L);
      const Slot& S = sm.slot[i & 1];
      // P = K S^T for both slices (rows: physical tokens prow(mt, r))
      bf16x8 SB[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) SB[s][kk] = pack_b(ST[s][2 * kk], ST[s][2 * kk + 1]);
      f32x4 P[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) P[s][mt] = zero4();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = prow(mt, r);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(S.K + row * 256 + 16 * ((4 * kk + g) ^ ksw(row)));
#pragma unroll
          for (int s = 0; s < 2; ++s) P[s][mt] = mfma_bf16(a, SB[s][kk], P[s][mt]);
        }
      }
      // O^T (first part) = S Q^T: lane (r, g) holds value rows 16s + 4g + e of
      // token 16nt + r
      f32x4 OT[2][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = 16 * nt + r;
#pragma unroll
        for (int s = 0; s < 2; ++s) OT[s][nt] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(S.Q + row * 256 + 16 * ((4 * kk + g) ^ swz(row)));
#pragma unroll
          for (int s = 0; s < 2; ++s) OT[s][nt] = mfma_bf16(SB[s][kk], bq, OT[s][nt]);
        }
      }
      // X = V - diag(gam) P, V of this lane's value row by transposed reads
      // (as input lane r of group g: 4 value rows 16s + 4(r%4) .. +3 of token
      // 32(mt/2) + 8g + 4(mt%2) + r/4)
      f32x4 X[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int tb = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1);
        const f32x4 gm = *reinterpret_cast<const f32x4*>(S.gam + tb);
        const int tok = tb + (r >> 2);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int col = dvw + 16 * s + 4 * (r & 3);
          const s16x4 vt = lds_tr16(S.V + tok * 256 + 16 * ((col >> 3) ^ vsw(tok)) + 2 * (col & 7));
          const bf16* v4 = reinterpret_cast<const bf16*>(&vt);
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) X[s][mt][i2] = (float)v4[i2] - gm[i2] * P[s][mt][i2];
        }
      }
      // Dl = Tt X (Tt lower triangular: tiles mt < 2 have nothing in columns 32..63)
      f32x4 Dl[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Dl[s][mt] = zero4();
      {
        bf16x8 XB[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          XB[s][0] = pack_b(X[s][0], X[s][1]);
          XB[s][1] = pack_b(X[s][2], X[s][3]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = prow(mt, r);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            if (kk == 1 && mt < 2) continue;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(S.T + row * 128 + 16 * ((4 * kk + g) ^ swz(row)));
#pragma unroll
            for (int s = 0; s < 2; ++s) Dl[s][mt] = mfma_bf16(a, XB[s][kk], Dl[s][mt]);
          }
        }
      }
      // state update: S^T <- gam_last S^T + K^T diag(dec) Dl; the A fragments
      // of K^T by transposed reads of the K tile (as in the split scan)
      bf16x8 DB[2][2], DTB[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        DB[s][0] = pack_b(Dl[s][0], Dl[s][1]);
        DB[s][1] = pack_b(Dl[s][2], Dl[s][3]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 dc = *reinterpret_cast<const f32x4*>(S.dec + 32 * (mt >> 1) + 8 * g + 4 * (mt & 1));
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) Dl[s][mt][i2] *= dc[i2];
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        DTB[s][0] = pack_b(Dl[s][0], Dl[s][1]);
        DTB[s][1] = pack_b(Dl[s][2], Dl[s][3]);
      }
      const float gL = S.gam[kC - 1];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 8; ++t) ST[s][t] *= gL;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int dk = 32 * (t >> 1) + 8 * (r & 3) + 4 * (t & 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int t0 = 32 * kk + 8 * g + (r >> 2), t1 = t0 + 4;
          const s16x4 lo = lds_tr16(S.K + t0 * 256 + 16 * ((dk >> 3) ^ ksw(t0)) + 2 * (dk & 7));
          const s16x4 hi = lds_tr16(S.K + t1 * 256 + 16 * ((dk >> 3) ^ ksw(t1)) + 2 * (dk & 7));
          const s16x4 lh[2] = {lo, hi};
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(lh);
#pragma unroll
          for (int s = 0; s < 2; ++s) ST[s][t] = mfma_bf16(a, DTB[s][kk], ST[s][t]);
        }
      }
      // O^T (second part): diag(gam) then + Dl^T M^T (M lower triangular)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = 16 * nt + r;
        const float gm = S.gam[row];
#pragma unroll
        for (int s = 0; s < 2; ++s) OT[s][nt] *= gm;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk == 1 && nt < 2) continue;
          const bf16x8 bm = *reinterpret_cast<const bf16x8*>(S.M + row * 128 + 16 * ((4 * kk + g) ^ swz(row)));
#pragma unroll
          for (int s = 0; s < 2; ++s) OT[s][nt] = mfma_bf16(DB[s][kk], bm, OT[s][nt]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) OB[s][nt][e] = (bf16)OT[s][nt][e];
        if constexpr (GATED) {
          // per-token sum of o^2 over this wave's 32 rows
          float ss = 0.f;
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += OT[s][nt][e] * OT[s][nt][e];
          ss += __shfl_xor(ss, 16, 64);
          ss += __shfl_xor(ss, 32, 64);
          if (g == 0) sm.part[i % 3][w][row] = ss;
        }
      }
      ptok0 = tok0;
      pL = L;
    }
    wait_vm<0>();                                  // the stores issued at the start of this iteration
    barrier_lds();
  }
  if (ht) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const size_t hrow = (((size_t)seq * Hv + h) * kD + dvw + 16 * s + r) * kD;
#pragma unroll
      for (int t = 0; t < 8; ++t) store_state4(ht, hrow + prow(t, 4 * g), ST[s][t], sbf);
    }
  }
}

// ---------------------------------------------------------------- varlen table
// Builds, from cu_seqlens, the chunk table {first token, length} and the first
// chunk of every sequence.  Values are clamped to [0, T_tot] and the table to
// nc_max entries, so malformed offsets cannot send any kernel out of bounds.
__global__ __launch_bounds__(256) void varlen_table_kernel(const int32_t* __restrict__ cu, int N,
                                                          int T_tot, int nc_max,
                                                          int32_t* __restrict__ tab,
                                                          int32_t* __restrict__ seq_off) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  int running = 0;
  for (int base = 0; base < N; base += 256) {
    const int n = base + tid;
    int a = 0, len = 0;
    if (n < N) {
      a = min(max(cu[n], 0), T_tot);
      const int e = min(max(cu[n + 1], a), T_tot);
      len = e - a;
    }
    const int nch = (len + kC - 1) / kC;
    part[tid] = nch;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int y = (tid >= off) ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += y;
      __syncthreads();
    }
    const int excl = running + part[tid] - nch;
    if (n < N) {
      seq_off[n] = min(excl, nc_max);
      for (int j = 0; j < nch && excl + j < nc_max; ++j) {
        tab[2 * (excl + j)] = a + kC * j;
        tab[2 * (excl + j) + 1] = min(kC, len - kC * j);
      }
    }
    running += part[255];
    __syncthreads();
  }
  if (tid == 0) seq_off[N] = min(running, nc_max);
  // Unused table slots carry length 0 so that prepare skips them.
  for (int s = running + tid; s < nc_max; s += 256) {
    tab[2 * s] = 0;
    tab[2 * s + 1] = 0;
  }
}

// ---------------------------------------------------------------- gated output
// In place on a bf16 output o [rows = tokens x value heads][128]:
//   y = o / sqrt(mean_d(o^2) + eps) * w * sigmoid(gate)
// (RMS normalisation over the head dim, then the sigmoid output gate), after
// the split scan, which leaves each head's 128 channels spread over four
// workgroups (calls with few (sequence, head) pairs; the head-wide scan
// applies the epilogue itself).  A bandwidth-bound pass: 16 lanes per row, 8 channels
// (16 bytes) each, 16 rows per workgroup, sums of squares by xor shuffles
// inside the 16-lane group.
__global__ __launch_bounds__(256) void gate_norm_kernel(bf16* __restrict__ o,
                                                        const bf16* __restrict__ gate,
                                                        const float* __restrict__ w, float eps,
                                                        int64_t nrows) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= nrows) return;                        // whole 16-lane groups leave together
  const int c = (threadIdx.x & 15) * 8;
  const bf16x8 ov = *reinterpret_cast<const bf16x8*>(o + row * kD + c);
  const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gate + row * kD + c);
  float x[8], ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (float)ov[j];
    ss += x[j] * x[j];
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off, 16);
  const float rs = 1.f / sqrtf(ss * (1.f / kD) + eps);
  bf16x8 yv;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float wj = w ? w[c + j] : 1.f;
    const float sg = 1.f / (1.f + __expf(-(float)gv[j]));
    yv[j] = (bf16)(x[j] * rs * wj * sg);
  }
  *reinterpret_cast<bf16x8*>(o + row * kD + c) = yv;
}

// ---------------------------------------------------------------- launchers
template <typename E>
static hipError_t launch_prepare_t(const PrefillLaunch& a, hipStream_t st) {
  if (a.nc_launch <= 0) return hipSuccess;
  Work<E> ws{(E*)a.Tt, (E*)a.M, a.gam, a.dec, (E*)a.N};
  dim3 grid((unsigned)a.nc_launch, (unsigned)a.Hqk), block(256);
  if (a.solve_only)
    hipLaunchKernelGGL((prepare_kernel<E, true>), grid, block, 0, st, (const E*)a.q,
                       (const E*)a.k, a.alpha, a.beta, ws, a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk);
  else
    hipLaunchKernelGGL((prepare_kernel<E, false>), grid, block, 0, st, (const E*)a.q,
                       (const E*)a.k, a.alpha, a.beta, ws, a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk);
  return hipGetLastError();
}

template <typename E, int NW, bool GATED>
static hipError_t launch_scan_t(const PrefillLaunch& a, hipStream_t st) {
  if (a.nseq <= 0) return hipSuccess;
  Work<E> ws{(E*)a.Tt, (E*)a.M, a.gam, a.dec, nullptr};
  constexpr int NSL = kD / (16 * NW);
  int nlin = a.Hv * NSL;
  if ((a.Hqk & 7) == 0) nlin = ((nlin + 7) / 8) * 8;
  dim3 grid((unsigned)nlin, (unsigned)a.nseq), block(64 * NW);
  hipLaunchKernelGGL((scan_kernel<E, NW, GATED>), grid, block, 0, st, (const E*)a.q,
                     (const E*)a.k, (const E*)a.v, a.h0, (E*)a.o, a.ht, a.state_bf16, (const E*)a.gate,
                     a.norm_w, a.norm_eps, ws, a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk);
  return hipGetLastError();
}

hipError_t launch_prepare(const PrefillLaunch& a, hipStream_t st) {
  return a.bf16_io ? launch_prepare_t<bf16>(a, st) : launch_prepare_t<float>(a, st);
}

static hipError_t launch_scan_split(const PrefillLaunch& a, hipStream_t st) {
  if (a.nseq <= 0) return hipSuccess;
  Work<bf16> ws{(bf16*)a.Tt, (bf16*)a.M, a.gam, a.dec, nullptr};
  int nlin = a.Hv * split::kNsl;
  if ((a.Hqk & 7) == 0) nlin = ((nlin + 7) / 8) * 8;
  dim3 grid((unsigned)nlin, (unsigned)a.nseq), block(64 * split::kWaves);
  if (a.states)
    hipLaunchKernelGGL(scan_split_kernel<true>, grid, block, 0, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.h0, (bf16*)a.o, a.ht, a.state_bf16, ws,
                       a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk, (bf16*)a.states);
  else
    hipLaunchKernelGGL(scan_split_kernel<false>, grid, block, 0, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.h0, (bf16*)a.o, a.ht, a.state_bf16, ws,
                       a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk, nullptr);
  return hipGetLastError();
}

// (sequence, value head) pairs from which the bf16 scan runs head-wide: from
// 128 pairs the split scan needs two full rounds of one-per-CU workgroups
// (measured at T = 8192: 96 pairs split 0.404 ms / head-wide 0.440; 144 pairs
// 0.585 / 0.451).
constexpr int64_t kHeadScanMinPairs = 128;

template <bool GATED>
static hipError_t launch_scan_head(const PrefillLaunch& a, hipStream_t st) {
  if (a.nseq <= 0) return hipSuccess;
  Work<bf16> ws{(bf16*)a.Tt, (bf16*)a.M, a.gam, a.dec, nullptr};
  int nlin = a.Hv;
  if ((a.Hqk & 7) == 0) nlin = ((nlin + 7) / 8) * 8;
  dim3 grid((unsigned)nlin, (unsigned)a.nseq), block(64 * hw::kWaves);
  hipLaunchKernelGGL(scan_head_kernel<GATED>, grid, block, 0, st, (const bf16*)a.q,
                     (const bf16*)a.k, (const bf16*)a.v, a.h0, (bf16*)a.o, a.ht, a.state_bf16,
                     (const bf16*)a.gate, a.norm_w, a.norm_eps, ws, a.cm, a.Hqk, a.Hv,
                     a.Hv / a.Hqk);
  return hipGetLastError();
}

hipError_t launch_scan(const PrefillLaunch& a, hipStream_t st) {
  if (!a.bf16_io)
    return a.gate ? launch_scan_t<float, 8, true>(a, st) : launch_scan_t<float, 4, false>(a, st);
  // bf16: calls with enough (sequence, head) pairs to fill the chip run the
  // head-wide scan (four chain waves per CU against the split scan's two,
  // and the gated epilogue inside it); smaller ones the split scan, whose
  // gated output then takes a separate pass.  The backward's state
  // checkpoints come from the split scan.
  const bool wide = !a.states && (int64_t)a.nseq * a.Hv >= kHeadScanMinPairs;
  if (wide) return a.gate ? launch_scan_head<true>(a, st) : launch_scan_head<false>(a, st);
  hipError_t e = launch_scan_split(a, st);
  if (e != hipSuccess || !a.gate || a.ntok == 0) return e;
  const int64_t nrows = a.ntok * a.Hv;
  hipLaunchKernelGGL(gate_norm_kernel, dim3((unsigned)((nrows + 15) / 16)), dim3(256), 0, st,
                     (bf16*)a.o, (const bf16*)a.gate, a.norm_w, a.norm_eps, nrows);
  return hipGetLastError();
}

hipError_t launch_varlen_table(const int32_t* cu, int N, int T_tot, int nc_max, int32_t* tab,
                               int32_t* seq_off, hipStream_t st) {
  hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(256), 0, st, cu, N, T_tot, nc_max, tab,
                     seq_off);
  return hipGetLastError();
}

}  // namespace gdn

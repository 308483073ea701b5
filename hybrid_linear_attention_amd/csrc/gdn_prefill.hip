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
//    by fp32 MFMA).  Writes Tt, Q K^T and G to the workspace.
//  * scan     (grid: value-row slices x value heads x sequences) - the serial
//    chain.  Each wave owns 16 value rows of one head's state and keeps them,
//    transposed (S^T, d_k x 16), in fp32 MFMA accumulators for the whole
//    sequence.  Per chunk every product feeds the next one straight from
//    registers: the accumulator tiles of S^T, X and Dl are the B operands of the
//    following MFMAs (see gdn_device.hpp for the K order that makes this work),
//    so only the shared chunk operands (K, K^T, Q, Tt, M, V) go through LDS.
//    Rows of the state never interact, so the value rows split across waves
//    and workgroups with no communication at all.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

#include <type_traits>

namespace gdn {

template <typename E>
struct Work {
  E* Tt;      // [nc][Hv][64][64]  (I + A)^-1 diag(beta)
  E* QK;      // [nc][Hqk][64][64] Q K^T (unmasked)
  float* Gs;  // [nc][Hv][64]      gate prefix G
};

__device__ __forceinline__ void chunk_of(const ChunkMap& cm, int cid, int& tok0, int& L) {
  if (cm.tab) {
    tok0 = cm.tab[2 * cid];
    L = cm.tab[2 * cid + 1];
  } else {
    const int b = cid / cm.Nc, j = cid - (cid / cm.Nc) * cm.Nc;
    tok0 = b * cm.T + kC * j;
    L = min(kC, cm.T - kC * j);
  }
}

// 16 consecutive bytes of a row of q/k/v (8 bf16 or 4 fp32), zero if masked.
template <typename E>
__device__ __forceinline__ uint4 ld16(const E* p, bool ok) {
  if (!ok) return uint4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------- prepare
constexpr int kLdT = 68;   // LDS row stride of 64-wide fp32/bf16 tiles

template <typename E>
struct PrepSmem {
  static constexpr int LDK = 136;   // K/Q row stride: rows 16-byte aligned for b128 reads
  union {
    struct {
      E Ks[kC * LDK];
      E Qs[kC * LDK];
    } in;
    float buf[4][kC * kLdT];        // per-wave A -> T buffers (after the Grams)
  } u;
  float gram[kC * kLdT];
  float gate[4][kC];
  float bet[4][kC];
};

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

template <typename E>
__global__ __launch_bounds__(256) void prepare_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, Work<E> ws, ChunkMap cm, int Hqk, int Hv, int G) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int LDK = PrepSmem<E>::LDK;
  constexpr int EPV = 16 / sizeof(E);            // elements per 16-byte piece
  __shared__ PrepSmem<E> sm;

  const int cid = blockIdx.x, gq = blockIdx.y;
  if (cid >= cm.nc_max) return;
  int tok0, L;
  chunk_of(cm, cid, tok0, L);
  if (L <= 0) return;                            // unused varlen table slot
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;

  // Stage the chunk's K and Q rows (zero beyond L).
  constexpr int PPR = kD / EPV;                  // 16-byte pieces per row
  for (int p = tid; p < kC * PPR; p += 256) {
    const int t = p / PPR, cb = p - (p / PPR) * PPR;
    const size_t off = ((size_t)(tok0 + t) * Hqk + gq) * kD + cb * EPV;
    const uint4 kv = ld16(k + off, t < L);
    const uint4 qv = ld16(q + off, t < L);
    uint2* dk = reinterpret_cast<uint2*>(sm.u.in.Ks + t * LDK + cb * EPV);
    uint2* dq = reinterpret_cast<uint2*>(sm.u.in.Qs + t * LDK + cb * EPV);
    dk[0] = uint2{kv.x, kv.y}; dk[1] = uint2{kv.z, kv.w};
    dq[0] = uint2{qv.x, qv.y}; dq[1] = uint2{qv.z, qv.w};
  }
  __syncthreads();

  // Gram matrices: wave w computes rows 16w..16w+15 of K K^T and Q K^T.
  f32x4 kk[4], qk[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) { kk[nt] = zero4(); qk[nt] = zero4(); }
  if constexpr (BF) {
    const bf16* Ks = reinterpret_cast<const bf16*>(sm.u.in.Ks);
    const bf16* Qs = reinterpret_cast<const bf16*>(sm.u.in.Qs);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 ak = lds_row8_bf16(Ks, LDK, 16 * w + r, 32 * ks);
      const bf16x8 aq = lds_row8_bf16(Qs, LDK, 16 * w + r, 32 * ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 b = lds_row8_bf16(Ks, LDK, 16 * nt + r, 32 * ks);
        kk[nt] = mfma_bf16(ak, b, kk[nt]);
        qk[nt] = mfma_bf16(aq, b, qk[nt]);
      }
    }
  } else {
    const float* Ks = reinterpret_cast<const float*>(sm.u.in.Ks);
    const float* Qs = reinterpret_cast<const float*>(sm.u.in.Qs);
    for (int s = 0; s < kD / 4; ++s) {
      const float ak = Ks[(16 * w + r) * LDK + 4 * s + g];
      const float aq = Qs[(16 * w + r) * LDK + 4 * s + g];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float b = Ks[(16 * nt + r) * LDK + 4 * s + g];
        kk[nt] = mfma_f32(ak, b, kk[nt]);
        qk[nt] = mfma_f32(aq, b, qk[nt]);
      }
    }
  }
  E* qk_out = ws.QK + ((size_t)cid * Hqk + gq) * kC * kC;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * w + 4 * g + i, col = 16 * nt + r;
      sm.gram[row * kLdT + col] = kk[nt][i];
      qk_out[row * kC + col] = from_f32<E>(qk[nt][i]);
    }
  __syncthreads();   // K/Q tiles are dead from here on; buf[] reuses them

  // One wave per value head of this query/key group.
  float* A = sm.u.buf[w];
  for (int rr = w; rr < G; rr += 4) {
    const int h = gq * G + rr;
    const size_t gi = (size_t)(tok0 + l) * Hv + h;
    const float al = (l < L) ? alpha[gi] : 1.f;
    const float bl = (l < L) ? beta[gi] : 0.f;
    const float Gl = wave_inclusive_sum(logf(al));
    ws.Gs[((size_t)cid * Hv + h) * kC + l] = Gl;
    sm.gate[w][l] = Gl;
    sm.bet[w][l] = bl;
    wave_lds_fence();

    // A[i][j] = beta_i exp(G_i - G_j) (k_i . k_j) for j < i; lane = column j.
    for (int i = 0; i < kC; ++i) {
      float a = 0.f;
      if (l < i) a = sm.bet[w][i] * expf(sm.gate[w][i] - Gl) * sm.gram[i * kLdT + l];
      A[i * kLdT + l] = a;
    }
    wave_lds_fence();

    // Diagonal 16x16 blocks of (I + A)^-1 by forward substitution:
    // lane = (block bb, column c).
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

    // Tt = T diag(beta): lane = column j, coalesced rows.
    E* tt = ws.Tt + ((size_t)cid * Hv + h) * kC * kC;
    for (int i = 0; i < kC; ++i) tt[i * kC + l] = from_f32<E>(A[i * kLdT + l] * bl);
    wave_lds_fence();
  }
}

// ---------------------------------------------------------------- scan
template <typename E, int NW, bool GATED>
struct ScanSmem {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int LDK = 132;                   // K, Q row stride
  static constexpr int LDO = GATED ? 16 * NW + 4 : 16 * NW + 8;
  E Ks[kC * LDK];
  E Qs[kC * LDK];
  E KT[BF ? kD * kLdT : 1];                         // K^T (bf16 only)
  E Vt[BF ? 16 * NW * kLdT : 1];                    // V^T slice (bf16 only)
  E Tt[kC * kLdT];
  E Ms[kC * kLdT];
  typename std::conditional<GATED, float, E>::type Os[kC * LDO];
  float gam[kC];                                    // exp(G_t)
  float dec[kC];                                    // exp(G_last - G_t)
};

template <typename E, int NW, bool GATED>
__global__ __launch_bounds__(64 * NW) void scan_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ h0, E* __restrict__ o, float* __restrict__ ht,
    const E* __restrict__ gate, const float* __restrict__ norm_w, float norm_eps,
    Work<E> ws, ChunkMap cm, int Hqk, int Hv, int G) {
  using Sm = ScanSmem<E, NW, GATED>;
  constexpr bool BF = Sm::BF;
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
    cid0 = cm.seq_off[seq];
    nch = min(cm.seq_off[seq + 1], cm.nc_max) - cid0;
  } else {
    cid0 = seq * cm.Nc;
    nch = cm.Nc;
  }

  // State S^T (d_k x 16 value rows) as 8 accumulator tiles: ST[t][i] holds
  // S[dv0 + r][16t + 4g + i].
  f32x4 ST[8];
  {
    const float* hp = h0 ? h0 + (((size_t)seq * Hv + h) * kD + dv0 + r) * kD : nullptr;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      ST[t] = hp ? *reinterpret_cast<const f32x4*>(hp + 16 * t + 4 * g) : zero4();
  }

  int prev_tok0 = 0, prev_L = 0;
  for (int c = 0; c <= nch; ++c) {
    // ---- phase 1: write out the previous chunk's outputs, stage this chunk.
    if (c > 0) {
      if constexpr (GATED) {
        // y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate), whole head per row.
        static_assert(!GATED || NW == 8, "the fused epilogue needs the whole head");
        const int row = tid >> 3, part = tid & 7;
        if (row < prev_L) {
          const float* orow = sm.Os + row * LDO + 16 * part;
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) ss += orow[j] * orow[j];
          ss += __shfl_xor(ss, 1, 64);
          ss += __shfl_xor(ss, 2, 64);
          ss += __shfl_xor(ss, 4, 64);
          const float rn = rsqrtf(ss * (1.f / kD) + norm_eps);
          const size_t base = ((size_t)(prev_tok0 + row) * Hv + h) * kD + 16 * part;
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
        constexpr int PPR = 16 * NW / EPV;          // 16-byte pieces per output row
        for (int p = tid; p < kC * PPR; p += NT) {
          const int t = p / PPR, cb = p - (p / PPR) * PPR;
          if (t < prev_L) {
            const uint4 val = *reinterpret_cast<const uint4*>(sm.Os + t * LDO + cb * EPV);
            *reinterpret_cast<uint4*>(o + ((size_t)(prev_tok0 + t) * Hv + h) * kD + dvb +
                                      cb * EPV) = val;
          }
        }
      }
    }
    if (c == nch) break;

    const int cid = cid0 + c;
    int tok0, L;
    chunk_of(cm, cid, tok0, L);
    {
      // K (row-major, and transposed for bf16) and Q.  Lanes run along the
      // token axis so the transposed 2-byte LDS writes hit distinct banks.
      constexpr int PPR = kD / EPV;
      for (int p = tid; p < kC * PPR; p += NT) {
        const int t = p & 63, cb = p >> 6;
        const size_t off = ((size_t)(tok0 + t) * Hqk + gq) * kD + cb * EPV;
        const uint4 kv = ld16(k + off, t < L);
        const uint4 qv = ld16(q + off, t < L);
        uint2* dk = reinterpret_cast<uint2*>(sm.Ks + t * LDK + cb * EPV);
        uint2* dq = reinterpret_cast<uint2*>(sm.Qs + t * LDK + cb * EPV);
        dk[0] = uint2{kv.x, kv.y}; dk[1] = uint2{kv.z, kv.w};
        dq[0] = uint2{qv.x, qv.y}; dq[1] = uint2{qv.z, qv.w};
        if constexpr (BF) {
          const bf16* e8 = reinterpret_cast<const bf16*>(&kv);
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.KT[(cb * 8 + e) * kLdT + t] = e8[e];
        }
      }
      // V slice, transposed (bf16 only; the fp32 path reads V in place).
      if constexpr (BF) {
        constexpr int VPR = 16 * NW / 8;
        for (int p = tid; p < kC * VPR; p += NT) {
          const int t = p & 63, cb = p >> 6;
          const uint4 vv =
              ld16(v + ((size_t)(tok0 + t) * Hv + h) * kD + dvb + cb * 8, t < L);
          const bf16* e8 = reinterpret_cast<const bf16*>(&vv);
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.Vt[(cb * 8 + e) * kLdT + t] = e8[e];
        }
      }
      // Tt, and M = (Q K^T) * exp(G_i - G_j) on and below the diagonal.
      const E* tsrc = ws.Tt + ((size_t)cid * Hv + h) * kC * kC;
      const E* qsrc = ws.QK + ((size_t)cid * Hqk + gq) * kC * kC;
      const float* gsrc = ws.Gs + ((size_t)cid * Hv + h) * kC;
      for (int e = tid; e < kC * kC; e += NT) {
        const int i = e >> 6, j = e & 63;
        sm.Tt[i * kLdT + j] = tsrc[e];
        float m = 0.f;
        if (j <= i) m = to_f32(qsrc[e]) * __expf(gsrc[i] - gsrc[j]);
        sm.Ms[i * kLdT + j] = from_f32<E>(m);
      }
      if (tid < kC) {
        const float Gt = gsrc[tid], Gl = gsrc[kC - 1];
        sm.gam[tid] = __expf(Gt);
        sm.dec[tid] = __expf(Gl - Gt);
      }
    }
    __syncthreads();

    // ---- phase 2: this wave's 16 value rows.
    const float gL = sm.gam[kC - 1];
    f32x4 P[4], QS[4], X[4], Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { P[mt] = zero4(); QS[mt] = zero4(); Dl[mt] = zero4(); }

    // P = K S0^T and QS = Q S0^T (contraction over d_k).
    if constexpr (BF) {
      bf16x8 SB[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) SB[kk] = pack_b(ST[2 * kk], ST[2 * kk + 1]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        mma_acc_bf16<8>(P[mt], reinterpret_cast<const bf16*>(sm.Ks), LDK, 16 * mt, 0, SB);
        mma_acc_bf16<8>(QS[mt], reinterpret_cast<const bf16*>(sm.Qs), LDK, 16 * mt, 0, SB);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        mma_acc_f32<8>(P[mt], reinterpret_cast<const float*>(sm.Ks), LDK, 16 * mt, 0, ST);
        mma_acc_f32<8>(QS[mt], reinterpret_cast<const float*>(sm.Qs), LDK, 16 * mt, 0, ST);
      }
    }

    // X = V - diag(exp G) P.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int t0 = 16 * mt + 4 * g;
      float vv[4];
      if constexpr (BF) {
        const bf16x4 v4 =
            *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(sm.Vt) +
                                             (16 * w + r) * kLdT + t0);
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = (float)v4[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vv[i] = (t0 + i < L)
                      ? to_f32(v[((size_t)(tok0 + t0 + i) * Hv + h) * kD + dv0 + r])
                      : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) X[mt][i] = vv[i] - sm.gam[t0 + i] * P[mt][i];
    }

    // Dl = Tt X (contraction over tokens of the chunk).
    if constexpr (BF) {
      bf16x8 XB[2] = {pack_b(X[0], X[1]), pack_b(X[2], X[3])};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        mma_acc_bf16<4>(Dl[mt], reinterpret_cast<const bf16*>(sm.Tt), kLdT, 16 * mt, 0, XB);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        mma_acc_f32<4>(Dl[mt], reinterpret_cast<const float*>(sm.Tt), kLdT, 16 * mt, 0, X);
    }

    // O = diag(exp G) QS + M Dl  ->  LDS staging.
    {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) QS[mt][i] *= sm.gam[16 * mt + 4 * g + i];
      if constexpr (BF) {
        bf16x8 DB[2] = {pack_b(Dl[0], Dl[1]), pack_b(Dl[2], Dl[3])};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          mma_acc_bf16<4>(QS[mt], reinterpret_cast<const bf16*>(sm.Ms), kLdT, 16 * mt, 0, DB);
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          mma_acc_f32<4>(QS[mt], reinterpret_cast<const float*>(sm.Ms), kLdT, 16 * mt, 0, Dl);
      }
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
    if constexpr (BF) {
      bf16x8 DTB[2] = {pack_b(Dl[0], Dl[1]), pack_b(Dl[2], Dl[3])};
#pragma unroll
      for (int t = 0; t < 8; ++t)
        mma_acc_bf16<4>(ST[t], reinterpret_cast<const bf16*>(sm.KT), kLdT, 16 * t, 0, DTB);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        mma_acc_f32_tA<4>(ST[t], reinterpret_cast<const float*>(sm.Ks), LDK, 16 * t, 0, Dl);
    }
    prev_tok0 = tok0;
    prev_L = L;
    __syncthreads();
  }

  if (ht) {
    float* hp = ht + (((size_t)seq * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(hp + 16 * t + 4 * g) = ST[t];
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

// ---------------------------------------------------------------- launchers
template <typename E>
static hipError_t launch_prepare_t(const PrefillLaunch& a, hipStream_t st) {
  if (a.nc_launch <= 0) return hipSuccess;
  Work<E> ws{(E*)a.Tt, (E*)a.QK, a.Gs};
  dim3 grid((unsigned)a.nc_launch, (unsigned)a.Hqk), block(256);
  hipLaunchKernelGGL(prepare_kernel<E>, grid, block, 0, st, (const E*)a.q, (const E*)a.k,
                     a.alpha, a.beta, ws, a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk);
  return hipGetLastError();
}

template <typename E, int NW, bool GATED>
static hipError_t launch_scan_t(const PrefillLaunch& a, hipStream_t st) {
  if (a.nseq <= 0) return hipSuccess;
  Work<E> ws{(E*)a.Tt, (E*)a.QK, a.Gs};
  constexpr int NSL = kD / (16 * NW);
  int nlin = a.Hv * NSL;
  if ((a.Hqk & 7) == 0) nlin = ((nlin + 7) / 8) * 8;
  dim3 grid((unsigned)nlin, (unsigned)a.nseq), block(64 * NW);
  hipLaunchKernelGGL((scan_kernel<E, NW, GATED>), grid, block, 0, st, (const E*)a.q,
                     (const E*)a.k, (const E*)a.v, a.h0, (E*)a.o, a.ht, (const E*)a.gate,
                     a.norm_w, a.norm_eps, ws, a.cm, a.Hqk, a.Hv, a.Hv / a.Hqk);
  return hipGetLastError();
}

hipError_t launch_prepare(const PrefillLaunch& a, hipStream_t st) {
  return a.bf16_io ? launch_prepare_t<bf16>(a, st) : launch_prepare_t<float>(a, st);
}

hipError_t launch_scan(const PrefillLaunch& a, hipStream_t st) {
  if (a.gate)
    return a.bf16_io ? launch_scan_t<bf16, 8, true>(a, st) : launch_scan_t<float, 8, true>(a, st);
  return a.bf16_io ? launch_scan_t<bf16, 4, false>(a, st) : launch_scan_t<float, 4, false>(a, st);
}

hipError_t launch_varlen_table(const int32_t* cu, int N, int T_tot, int nc_max, int32_t* tab,
                               int32_t* seq_off, hipStream_t st) {
  hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(256), 0, st, cu, N, T_tot, nc_max, tab,
                     seq_off);
  return hipGetLastError();
}

}  // namespace gdn

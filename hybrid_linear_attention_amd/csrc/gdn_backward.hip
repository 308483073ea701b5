// Backward pass of the chunked gated delta rule on gfx950.
//
// The page "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture, 256k Context,
// and 24GB Local Serving" (note under "The Role of Periodic Gated Attention")
// says training runs the same block-parallel form as prefill.  Its gradients
// follow from the chunk relations of the forward pass (one chunk, L <= 64
// tokens, incoming state S0, G = prefix of ln alpha, gamma = exp G,
// Gam_ij = exp(G_i - G_j) for j <= i, dec_i = Gam_{L-1,i}):
//
//     A  = strict_lower(diag(beta) (K K^T * Gam)),   N = (I + A)^-1
//     X  = V - diag(gamma) K S0^T,    Dl = N diag(beta) X
//     O  = diag(gamma) Q S0^T + M Dl,              M = (Q K^T * Gam) incl. diagonal
//     S' = gamma_{L-1} S0 + Dl^T diag(dec) K
//
// Given dO = dL/dO and dS' = dL/dS', the chain rule gives
//
//     dDl = M^T dO + diag(dec) K dS'^T,      Y = N^T dDl,     dV = diag(beta) Y
//     dS0 = gamma_{L-1} dS' + (diag(gamma) Q)^T dO - (diag(gamma) K)^T diag(beta) Y
//     dM  = tril(dO Dl^T),   dA = -strict_lower(Y Dl^T),   Wa = diag(beta) (dA * Gam)
//     dQ  = diag(gamma) dO S0 + (dM * Gam) K
//     dK  = -diag(gamma beta) Y S0 + diag(dec) Dl dS' + (dM * Gam)^T Q + (Wa + Wa^T) K
//     dbeta_i = Y_i . X_i + sum_j dA_ij Gam_ij (k_i . k_j)
//     dG_i = q_i . (gamma_i (dO S0)_i) - gamma_i beta_i Y_i . (K S0^T)_i - w_i
//            + rowsum_i(P) - colsum_i(P),   P = dM * M + dA * A,
//            w_i = dec_i Dl_i . (K dS'^T)_i;   dG_{L-1} += sum_i w_i + gamma_{L-1} <dS', S0>
//     dalpha_j = (sum_{i >= j} dG_i) / alpha_j
//
// Kernels, launched in this order on one stream:
//  1. prepare (the forward's, with solve_only): N and M per (chunk, value head).
//  2. the forward state chain again, storing the state entering every chunk
//     (element type of the inputs) instead of outputs: bf16 uses the forward
//     scan itself with its outputs off, fp32 the fwd_states kernel below.
//  3. bwd_chain: dL/dS carried from the last chunk to the first, storing the
//     gradient of the state leaving every chunk; dh0 at the end.  Value rows
//     never interact in either chain, so rows split across waves and
//     workgroups as in the forward scan.  bf16: bwd_chain_split_kernel, chain
//     and helper waves per pair of value slices, its operands double-buffered
//     in LDS by direct copies.
//  4. bwd_grad: one workgroup per (chunk, query/key head), fully parallel.  It
//     walks the value heads of its group and accumulates dq and dk for the
//     group in registers, so no atomics and no reduction pass are needed.
// Chunks are found through a ChunkMap, so the same kernels serve a
// fixed-length batch and a packed (cu_seqlens) batch.
#include "gdn_device.hpp"
#include "gdn_chunks.hpp"
#include "gdn_frag.hpp"
#include "gdn_launch.hpp"

#include <type_traits>

namespace gdn {
namespace bwd {
using namespace frag;

// ------------------------------------------------------------ chains
// Both chains: one workgroup of NW waves per (value-row slice, value head,
// sequence); wave w owns value rows dv0 .. dv0+15 (dv0 = 16 (NW slice + w)) and
// keeps them transposed (d_k x 16, eight accumulator tiles) for the whole
// sequence, so that the tiles are directly the B operand of K S^T.  Per chunk
// the shared operands are staged in LDS by the whole workgroup.
template <typename E, int NW>
struct ChainSmem {
  static constexpr int R = 16 * NW;
  E K[Lds<E, 128>::size(kC)];
  E Q[Lds<E, 128>::size(kC)];            // gamma-scaled Q (bwd_chain only)
  E V[Lds<E, R>::size(kC)];              // V (fwd) or dO (bwd) of the slice's rows
  E N[Lds<E, 64>::size(kC)];
  E M[Lds<E, 64>::size(kC)];             // bwd_chain only
  float gm[kC], dc[kC], bt[kC];
};

template <typename E, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_states_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ h0, const E* __restrict__ Nw, const float* __restrict__ gam,
    const float* __restrict__ dec, E* __restrict__ Sc, ChunkMap cm, int Hqk, int Hv) {
  constexpr int R = 16 * NW, KB = FragOf<E>::KB, NT = 64 * NW;
  __shared__ ChainSmem<E, NW> sm;
  const Lds<E, 128> Ks{sm.K};
  const Lds<E, R> Vs{sm.V};
  const Lds<E, 64> Ns{sm.N};
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int h = blockIdx.y, b = blockIdx.z, gq = h / (Hv / Hqk);   // b: sequence
  int cid0, Nc;
  seq_chunks(cm, b, cid0, Nc);
  const int rbase = R * blockIdx.x, dv0 = rbase + 16 * w;

  f32x4 ST[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    ST[t] = h0 ? *reinterpret_cast<const f32x4*>(
                     h0 + (((size_t)b * Hv + h) * kD + dv0 + r) * kD + 16 * t + 4 * g)
               : zero4();

  for (int j = 0; j < Nc; ++j) {
    const int cid = cid0 + j;
    int tok0i, L;
    chunk_of(cm, cid, tok0i, L);
    const size_t tok0 = (size_t)tok0i;
    const size_t hc = (size_t)cid * Hv + h;
    E* sdst = Sc + (hc * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) store4(sdst + 16 * t + 4 * g, ST[t]);

    __syncthreads();
    stage<E, 128, kC, NT>(Ks, k + (tok0 * Hqk + gq) * kD, (int64_t)Hqk * kD, L);
    stage<E, R, kC, NT>(Vs, v + (tok0 * Hv + h) * kD + rbase, (int64_t)Hv * kD, L);
    stage<E, 64, kC, NT>(Ns, Nw + hc * kC * kC, kC, kC);
    if (threadIdx.x < kC) {
      const int t = threadIdx.x;
      sm.gm[t] = gam[hc * kC + t];
      sm.dc[t] = dec[hc * kC + t];
      sm.bt[t] = t < L ? beta[(tok0 + t) * Hv + h] : 0.f;
    }
    __syncthreads();

    // X = V - diag(gamma) K S^T (rows: tokens), times beta
    f32x4 XB[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 u = zero4();
#pragma unroll
      for (int kb = 0; kb < kD / KB; ++kb) u = mma(u, Ks.rm(16 * mt + r, KB * kb), acc_frag<E>(ST, kb));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * mt + 4 * g + i;
        XB[mt][i] = sm.bt[tok] * (Vs.get(tok, 16 * w + r) - sm.gm[tok] * u[i]);
      }
    }
    // Dl = N (beta X), then diag(dec) Dl
    f32x4 DD[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 d = zero4();
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb) d = mma(d, Ns.rm(16 * mt + r, KB * kb), acc_frag<E>(XB, kb));
#pragma unroll
      for (int i = 0; i < 4; ++i) DD[mt][i] = sm.dc[16 * mt + 4 * g + i] * d[i];
    }
    // S^T <- gamma_last S^T + K^T diag(dec) Dl
    const float gl = sm.gm[kC - 1];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4 a = ST[t] * gl;
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb) a = mma(a, Ks.cm(16 * t + r, KB * kb), acc_frag<E>(DD, kb));
      ST[t] = a;
    }
  }
}

template <typename E, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_chain_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ dout,
    const float* __restrict__ beta, const float* __restrict__ dht, float* __restrict__ dh0,
    const E* __restrict__ Nw, const E* __restrict__ Mw, const float* __restrict__ gam,
    const float* __restrict__ dec, E* __restrict__ dSc, ChunkMap cm, int Hqk, int Hv) {
  constexpr int R = 16 * NW, KB = FragOf<E>::KB, NT = 64 * NW;
  __shared__ ChainSmem<E, NW> sm;
  const Lds<E, 128> Ks{sm.K}, Qs{sm.Q};
  const Lds<E, R> Os{sm.V};
  const Lds<E, 64> Ns{sm.N}, Ms{sm.M};
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int h = blockIdx.y, b = blockIdx.z, gq = h / (Hv / Hqk);   // b: sequence
  int cid0, Nc;
  seq_chunks(cm, b, cid0, Nc);
  const int rbase = R * blockIdx.x, dv0 = rbase + 16 * w;
  constexpr int EP = 16 / sizeof(E);

  // dS^T tiles: DT[t][i] = dL/dS [dv0 + r][16t + 4g + i]
  f32x4 DT[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    DT[t] = dht ? *reinterpret_cast<const f32x4*>(
                      dht + (((size_t)b * Hv + h) * kD + dv0 + r) * kD + 16 * t + 4 * g)
                : zero4();

  for (int j = Nc - 1; j >= 0; --j) {
    const int cid = cid0 + j;
    int tok0i, L;
    chunk_of(cm, cid, tok0i, L);
    const size_t tok0 = (size_t)tok0i;
    const size_t hc = (size_t)cid * Hv + h;
    E* ddst = dSc + (hc * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) store4(ddst + 16 * t + 4 * g, DT[t]);

    __syncthreads();
    if (threadIdx.x < kC) {
      const int t = threadIdx.x;
      sm.gm[t] = gam[hc * kC + t];
      sm.dc[t] = dec[hc * kC + t];
      sm.bt[t] = t < L ? beta[(tok0 + t) * Hv + h] : 0.f;
    }
    stage<E, 128, kC, NT>(Ks, k + (tok0 * Hqk + gq) * kD, (int64_t)Hqk * kD, L);
    stage<E, R, kC, NT>(Os, dout + (tok0 * Hv + h) * kD + rbase, (int64_t)Hv * kD, L);
    stage<E, 64, kC, NT>(Ns, Nw + hc * kC * kC, kC, kC);
    stage<E, 64, kC, NT>(Ms, Mw + hc * kC * kC, kC, kC);
    // gamma-scaled Q rows
    {
      constexpr int PPR = kD / EP, NP = kC * PPR;
      const float* gsrc = gam + hc * kC;
      for (int pc = threadIdx.x; pc < NP; pc += NT) {
        const int row = pc / PPR, c = (pc % PPR) * EP;
        const float gr = gsrc[row];
        union { uint4 u; E e[EP]; } raw, out;
        raw.u = row < L ? *reinterpret_cast<const uint4*>(q + ((tok0 + row) * Hqk + gq) * kD + c)
                        : uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int x = 0; x < EP; ++x) out.e[x] = from_f32<E>(gr * to_f32(raw.e[x]));
        *reinterpret_cast<uint4*>(&Qs(row, c)) = out.u;
      }
    }
    __syncthreads();

    // dDl = M^T dO + diag(dec) K dS^T    (rows: tokens, column: this lane's dv)
    f32x4 dD[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 p = zero4(), m = zero4();
#pragma unroll
      for (int kb = 0; kb < kD / KB; ++kb) p = mma(p, Ks.rm(16 * mt + r, KB * kb), acc_frag<E>(DT, kb));
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb)
        m = mma(m, Ms.cm(16 * mt + r, KB * kb), Os.cm(16 * w + r, KB * kb));
#pragma unroll
      for (int i = 0; i < 4; ++i) dD[mt][i] = m[i] + sm.dc[16 * mt + 4 * g + i] * p[i];
    }
    // Y = N^T dDl;  Z = -gamma beta Y
    f32x4 Z[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 y = zero4();
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb) y = mma(y, Ns.cm(16 * mt + r, KB * kb), acc_frag<E>(dD, kb));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * mt + 4 * g + i;
        Z[mt][i] = -sm.gm[tok] * sm.bt[tok] * y[i];
      }
    }
    // dS^T <- gamma_last dS^T + (gamma Q)^T dO + K^T Z
    const float gl = sm.gm[kC - 1];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4 a = DT[t] * gl;
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb) {
        a = mma(a, Qs.cm(16 * t + r, KB * kb), Os.cm(16 * w + r, KB * kb));
        a = mma(a, Ks.cm(16 * t + r, KB * kb), acc_frag<E>(Z, kb));
      }
      DT[t] = a;
    }
  }
  if (dh0) {
    float* dst = dh0 + (((size_t)b * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * g) = DT[t];
  }
}

// Operand buffers of the bf16 reverse chain (bwd_chain_split_kernel below),
// filled by copies straight into LDS (global_load_lds_dwordx4: no registers,
// no VALU).  Copy instruction `it` of a tile fills LDS bytes [1024 it, 1024 it
// + 1024); lane l's 16 bytes are the piece of the swizzled layout at that
// position, so each lane reads the global piece the swizzle puts there.  Rows
// beyond the chunk's length repeat its last token: such tokens get a zero
// gamma wherever they could reach the state gradient (the gamma-scaled dO and
// the beta-scaled Y), and the mask matrix M, written by prepare from zero
// rows, is zero there.
struct ChainOps {                 // what the chain waves read for chunk j
  bf16 K[kC * kD];
  bf16 N[kC * kC];
  float gm[kC], dc[kC], bt[kC];
};
template <int NW>
struct HelperOps {                // what the helper waves read for chunk j
  static constexpr int R = 16 * NW;
  bf16 Q[kC * kD];
  bf16 O[kC * R];
  bf16 M[kC * kC];
  float gm[kC];
};

// bf16 reverse chain with a role split, as the forward scan has: per
// workgroup two 16-row value slices; waves 0-1 are chain waves (slice s = w),
// waves 2-3 helpers (slice s = w - 2), waves 4-5 copy waves (the chain's
// operands, the helpers' operands).  The helpers form
// the two state-independent products of each chunk a chunk ahead of the
// chain, so that the chain never waits for them.  In the iteration of chunk j
// (chunks run from the last to the first), with one barrier at its end:
//   chain:    store dS (the gradient of the state leaving chunk j); P = K dS^T;
//             dDl = MdO_j + diag(dec) P; Y = N^T dDl; Z = -gamma beta Y;
//             dS^T <- gamma_L dS^T + U_j + K^T Z
//   helpers:  MdO_{j-1} = M^T dO[:, slice] and U_{j-1} = (gamma Q)^T dO[:, slice]
//             into the other hand-off buffer
//   copies:   the chain's operands of chunk j-1 and the helpers' of chunk j-2
// The copies have waves of their own because a wave's later LDS accesses are
// ordered after its outstanding copies into LDS: a helper issuing them would
// wait for them before its first hand-off write.  The copy waves also touch
// chunk j-3's operands (one 4-byte copy per 128-byte line), so that their
// copies two iterations later find them in L2.  Chain operands, helper
// operands and hand-off tiles each have two buffers, chunk j's in buffer
// (Nc - 1 - j) % 2.  A chain wave issues 38 MFMAs per chunk instead of 64.
struct SplitHand {
  f32x4 mdo[2][4][64];    // [slice][token tile][lane]: M^T dO, 64 tokens x 16 rows
  f32x4 u[2][8][64];      // [slice][d_k tile][lane]: (gamma Q)^T dO, transposed like dS^T
};

__global__ __launch_bounds__(384) void bwd_chain_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ dout,
    const float* __restrict__ beta, const float* __restrict__ dht, float* __restrict__ dh0,
    const bf16* __restrict__ Nw, const bf16* __restrict__ Mw, const float* __restrict__ gam,
    const float* __restrict__ dec, bf16* __restrict__ dSc, ChunkMap cm, int Hqk, int Hv) {
  typedef bf16 E;
  constexpr int NS = 2, R = 16 * NS, KB = 32;
  __shared__ ChainOps cbuf[2];
  __shared__ HelperOps<NS> hbuf[2];
  __shared__ SplitHand hand[2];
  __shared__ uint32_t warm[2][64];
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), r = l & 15, g = l >> 4;
  const bool is_chain = w < NS;
  const int sl = is_chain ? w : w - NS;                 // this wave's slice (waves 0-3)
  const bool is_copy = w >= 2 * NS;
  const int cw = w - 2 * NS;                            // copy wave: 0 chain, 1 helper operands
  // Workgroup -> (value head, row block): the workgroups of one query/key
  // group (its value heads' row blocks) get consecutive ids of one XCD (ids
  // are dealt to the 8 XCDs round-robin), so that they share that XCD's L2
  // for the group's K and Q and each head's N and M.
  constexpr int NSL = kD / R;
  const int G = Hv / Hqk, per_group = G * NSL;
  int lin = blockIdx.x;
  if ((Hqk & 7) == 0) {
    const int xcd = lin & 7, jj = lin >> 3;
    lin = (xcd + 8 * (jj / per_group)) * per_group + (jj - (jj / per_group) * per_group);
  }
  if (lin >= Hv * NSL) return;                           // whole workgroup leaves together
  const int h = lin / NSL, b = blockIdx.y, gq = h / G;   // b: sequence
  int cid0, Nc;
  seq_chunks(cm, b, cid0, Nc);
  const int rbase = R * (lin - h * NSL), dv0 = rbase + 16 * sl;

  // copies of chunk j, by the copy wave
  auto issue_chain = [&](int j, auto bic) {
    ChainOps& B_ = cbuf[decltype(bic)::value];
    const int cid = cid0 + j;
    int tok0i, L;
    chunk_of(cm, cid, tok0i, L);
    const size_t tok0 = (size_t)tok0i;
    const size_t hc = (size_t)cid * Hv + h;
    copy_rows<128>(k + (tok0 * Hqk + gq) * kD, (int64_t)Hqk * kD, L, B_.K, 0, 1);
    copy_rows<64>(Nw + hc * kC * kC, kC, kC, B_.N, 0, 1);
    dma4(gam + hc * kC + l, B_.gm);
    dma4(beta + (tok0 + min(l, L - 1)) * Hv + h, B_.bt);
    dma4(dec + hc * kC + l, B_.dc);
  };
  auto issue_help = [&](int j, auto bic) {
    HelperOps<NS>& B_ = hbuf[decltype(bic)::value];
    const int cid = cid0 + j;
    int tok0i, L;
    chunk_of(cm, cid, tok0i, L);
    const size_t tok0 = (size_t)tok0i;
    const size_t hc = (size_t)cid * Hv + h;
    copy_rows<128>(q + (tok0 * Hqk + gq) * kD, (int64_t)Hqk * kD, L, B_.Q, 0, 1);
    copy_rows<R>(dout + (tok0 * Hv + h) * kD + rbase, (int64_t)Hv * kD, L, B_.O, 0, 1);
    copy_rows<64>(Mw + hc * kC * kC, kC, kC, B_.M, 0, 1);
    dma4(gam + hc * kC + l, B_.gm);
  };
  // one 4-byte copy per 128-byte line of chunk j's chain operands (copy
  // wave 0: 6 copies) or helper operands (copy wave 1: 4) into a scratch word
  auto touch = [&](int j) {
    const int cid = cid0 + j;
    int tok0i, L;
    chunk_of(cm, cid, tok0i, L);
    const size_t row = (size_t)tok0i + min(l, L - 1);
    const size_t hc = (size_t)cid * Hv + h;
    if (cw == 0) {
      const bf16* kr = k + (row * Hqk + gq) * kD;
      dma4(kr, &warm[0][0]);
      dma4(kr + 64, &warm[0][0]);
      dma4(Nw + hc * kC * kC + 64 * l, &warm[0][0]);
      dma4(gam + hc * kC + l, &warm[0][0]);
      dma4(dec + hc * kC + l, &warm[0][0]);
      dma4(beta + row * Hv + h, &warm[0][0]);
    } else {
      const bf16* qr = q + (row * Hqk + gq) * kD;
      dma4(qr, &warm[1][0]);
      dma4(qr + 64, &warm[1][0]);
      dma4(dout + (row * Hv + h) * kD + rbase, &warm[1][0]);
      dma4(Mw + hc * kC * kC + 64 * l, &warm[1][0]);
    }
  };
  // helpers: M^T dO and (gamma Q)^T dO of chunk j from hbuf[bi] into hand[bi]
  auto helper_products = [&](int j, auto bic) {
    constexpr int bi = decltype(bic)::value;
    int tok0i, L;
    chunk_of(cm, cid0 + j, tok0i, L);
    const HelperOps<NS>& B_ = hbuf[bi];
    const Lds<E, 128> Qs{const_cast<E*>(B_.Q)};
    const Lds<E, R> Os{const_cast<E*>(B_.O)};
    const Lds<E, 64> Ms{const_cast<E*>(B_.M)};
    // dO fragments of this slice (B operand, K = tokens), plain and
    // gamma-scaled (masked)
    bf16x8 OB[2], OG[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      OB[kb] = Os.cm(16 * sl + r, KB * kb);
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(&B_.gm[KB * kb + 4 * g]);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(&B_.gm[KB * kb + 16 + 4 * g]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = KB * kb + kslot<E>(g, e);
        const float gv = e < 4 ? g0[e] : g1[e - 4];
        OG[kb][e] = (bf16)((tok < L ? gv : 0.f) * (float)OB[kb][e]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 m = zero4();
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb)
        if (!blk_below<E>(mt, kb)) m = mma(m, Ms.cm(16 * mt + r, KB * kb), OB[kb]);
      hand[bi].mdo[sl][mt][l] = m;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4 u = zero4();
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb) u = mma(u, Qs.cm(16 * t + r, KB * kb), OG[kb]);
      hand[bi].u[sl][t][l] = u;
    }
  };

  f32x4 DT[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    DT[t] = (is_chain && dht) ? *reinterpret_cast<const f32x4*>(
                                    dht + (((size_t)b * Hv + h) * kD + dv0 + r) * kD + 16 * t + 4 * g)
                              : zero4();
  const std::integral_constant<int, 0> ic0{};
  const std::integral_constant<int, 1> ic1{};
  // chunk Nc-1: chain and helper operands in buffer 0; chunk Nc-2's helper
  // operands in buffer 1; the products of chunk Nc-1
  if (is_copy && Nc > 0) {
    if (cw == 0) {
      issue_chain(Nc - 1, ic0);
    } else {
      issue_help(Nc - 1, ic0);
      if (Nc > 1) issue_help(Nc - 2, ic1);
    }
  }
  wait_copies();
  barrier_lds();
  if (!is_chain && !is_copy && Nc > 0) helper_products(Nc - 1, ic0);
  barrier_lds();

  auto step = [&](int j, auto bic) {
    constexpr int bi = decltype(bic)::value;
    const std::integral_constant<int, 1 - bi> nbic{};
    if (is_chain) {
      const int cid = cid0 + j;
      int tok0i, L;
      chunk_of(cm, cid, tok0i, L);
      const ChainOps& B_ = cbuf[bi];
      const Lds<E, 128> Ks{const_cast<E*>(B_.K)};
      const Lds<E, 64> Ns{const_cast<E*>(B_.N)};
      const size_t hc = (size_t)cid * Hv + h;
      E* ddst = dSc + (hc * kD + dv0 + r) * kD;
#pragma unroll
      for (int t = 0; t < 8; ++t) store4(ddst + 16 * t + 4 * g, DT[t]);
      // P = K dS^T (rows: tokens, column: this lane's value row)
      f32x4 P[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 p = zero4();
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb) p = mma(p, Ks.rm(16 * mt + r, KB * kb), acc_frag<E>(DT, kb));
        P[mt] = p;
      }
      f32x4 dD[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 dc4 = *reinterpret_cast<const f32x4*>(&B_.dc[16 * mt + 4 * g]);
        const f32x4 m = hand[bi].mdo[sl][mt][l];
#pragma unroll
        for (int i = 0; i < 4; ++i) dD[mt][i] = m[i] + dc4[i] * P[mt][i];
      }
      f32x4 Z[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 y = zero4();
#pragma unroll
        for (int kb = 0; kb < kC / KB; ++kb)
          if (!blk_below<E>(mt, kb)) y = mma(y, Ns.cm(16 * mt + r, KB * kb), acc_frag<E>(dD, kb));
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&B_.gm[16 * mt + 4 * g]);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&B_.bt[16 * mt + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mt + 4 * g + i;
          Z[mt][i] = (tok < L ? -g4[i] * b4[i] : 0.f) * y[i];
        }
      }
      const float gl = B_.gm[kC - 1];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f32x4 a = DT[t] * gl + hand[bi].u[sl][t][l];
#pragma unroll
        for (int kb = 0; kb < kC / KB; ++kb) a = mma(a, Ks.cm(16 * t + r, KB * kb), acc_frag<E>(Z, kb));
        DT[t] = a;
      }
    } else if (is_copy) {
      if (cw == 0) {
        if (j >= 1) issue_chain(j - 1, nbic);
      } else {
        if (j >= 2) issue_help(j - 2, bic);
      }
      // chunk j-3 (chain operands copied in iteration j-2, helper operands in
      // j-1): touched after the copies, so that the counted wait leaves only
      // the touches in flight
      if (j >= 3) {
        touch(j - 3);
        if (cw == 0) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        wait_copies();
      }
    } else {
      if (j >= 1) helper_products(j - 1, nbic);
    }
    barrier_lds();
  };
  int j = Nc - 1;
  for (; j >= 1; j -= 2) {
    step(j, ic0);
    step(j - 1, ic1);
  }
  if (j == 0) step(0, ic0);
  if (is_chain && dh0) {
    float* dst = dh0 + (((size_t)b * Hv + h) * kD + dv0 + r) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * g) = DT[t];
  }
}

// ------------------------------------------------------------ per-chunk gradients
// One workgroup of 8 waves per (chunk, query/key head).  Per value head of the
// group:
//  phase 1   wave w owns value columns 16w..16w+15 of X, Dl, dDl, Y (rows:
//            tokens); writes dv, and Dl and Y to LDS.
//  phase 1.5 the 64x64 products dO Dl^T and Y Dl^T, two 16x16 tiles per wave,
//            turned into dM * Gam and Wa (stored together in one 64x64
//            matrix E: dM * Gam on and below the diagonal, Wa transposed
//            above it) and the gate and beta row/column sums.
//  phase 2   wave w owns key columns 16w..16w+15 of dq and dk (rows: tokens),
//            accumulated over the group's value heads in registers.
// bf16 stages every operand in LDS (about 159 KB): the next value head's S0,
// dS' and dO are copied while the current head's E products run, and its V, N
// and M once Dl and Y are dead.  fp32 reads the inputs from global memory (L2)
// and keeps only the intermediates Dl, Y, E in LDS.
constexpr int kGW = 8;  // waves

// Row sums of 16 terms, scattered: v[4 mt + i] is this lane's term of token
// 16 mt + 4 g + i (lane group g); lane r of the group returns the sum over the
// group's 16 lanes of token 16 (r / 4) + 4 g + r % 4, so that one
// unconditional store per lane writes all 64 tokens.  Recursive halving with
// row rotations: at step b a lane keeps the half of its partial sums whose
// index bit b equals its lane bit b, and adds the other half from the lane
// 2^b away in the row, which has the same lower bits and the opposite bit b.
// (A select chain over v[r] is turned by the compiler into a stack array
// indexed per lane, i.e. scratch memory traffic.)
template <int S, int N>
__device__ __forceinline__ void halve(const float (&a)[2 * N], float (&o)[N], bool hi) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float keep = hi ? a[2 * j + 1] : a[2 * j];
    const float send = hi ? a[2 * j] : a[2 * j + 1];
    o[j] = keep + row_ror<S>(send);
  }
}
__device__ __forceinline__ float rsum16(const float (&v)[16], int r) {
  float a[8], b[4], c[2], d[1];
  halve<1, 8>(v, a, r & 1);
  halve<2, 4>(a, b, r & 2);
  halve<4, 2>(b, c, r & 4);
  halve<8, 1>(c, d, r & 8);
  return d[0];
}

template <typename E>
struct GradSmem {
  static constexpr bool BF = sizeof(E) == 2;
  // The per-token arrays come first: below 64 KiB, every access to them is one
  // per-lane base plus an immediate offset.  Placed after the tiles, each
  // array needs a base register of its own, which the compiler keeps live
  // across the head loop (and spills).
  float ss[kGW];                            // per-wave <dS', S0>
  float rowp[4][kC], colp[4][kC], rowb[4][kC];
  float pa[kGW][kC];
  float fin[3][kC];                         // gate, beta, w
  float G2[kC], G2lo[kC], gm[kC], dc[kC], bt[kC], al[kC];   // G2 + G2lo: compensated prefix
  union {
    float part[kGW][3][kC];                 // phase 1 per-wave row sums
    E Em[Lds<E, 64>::size(kC)];             // phase 1.5 output
  } u3;
  // bf16 only (fp32 reads these from global memory)
  alignas(256) E K[BF ? Lds<E, 128>::size(kC) : 1];
  E Q[BF ? Lds<E, 128>::size(kC) : 1];
  E S0[BF ? Lds<E, 128>::size(kD) : 1];
  E dS[BF ? Lds<E, 128>::size(kD) : 1];
  E dO[BF ? Lds<E, 128>::size(kC) : 1];
  union {
    E V[BF ? Lds<E, 128>::size(kC) : 1];    // phase 1 input (bf16)
    E Dl[Lds<E, 128>::size(kC)];            // phase 1 output
  } u1;
  union {
    struct {
      E N[BF ? Lds<E, 64>::size(kC) : 1];
      E M[BF ? Lds<E, 64>::size(kC) : 1];
    } nm;                                    // phase 1 inputs (bf16)
    E Y[Lds<E, 128>::size(kC)];             // phase 1 output
  } u2;
};

template <typename E>
__global__ __launch_bounds__(64 * kGW) void bwd_grad_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ dout, const float* __restrict__ alpha, const float* __restrict__ beta,
    const E* __restrict__ Nw, const E* __restrict__ Mw, const E* __restrict__ Sc,
    const E* __restrict__ dSc, E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv,
    float* __restrict__ dalpha, float* __restrict__ dbeta, ChunkMap cm, int Hqk, int Hv) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int KB = FragOf<E>::KB, NT = 64 * kGW, NS = kSlotsOf<E>;
  __shared__ GradSmem<E> sm;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), r = l & 15, g = l >> 4;
  const int cid = blockIdx.x, gq = blockIdx.y, G = Hv / Hqk;
  int tok0i, L;
  chunk_of(cm, cid, tok0i, L);
  if (L <= 0) return;                     // unused slot of a packed batch's table
  const size_t tok0 = (size_t)tok0i;

  const Lds<E, 128> Dls{sm.u1.Dl}, Ys{sm.u2.Y};
  const Lds<E, 64> Es{sm.u3.Em};
  const E* kg = k + (tok0 * Hqk + gq) * kD;
  const E* qg = q + (tok0 * Hqk + gq) * kD;

  auto mK = [&]() {
    if constexpr (BF) return Lds<E, 128>{sm.K};
    else return Glb<E>{kg, (int64_t)Hqk * kD, L};
  }();
  auto mQ = [&]() {
    if constexpr (BF) return Lds<E, 128>{sm.Q};
    else return Glb<E>{qg, (int64_t)Hqk * kD, L};
  }();
  // K and Q: copied straight into LDS for a full chunk (waited for with the
  // first head's operands); a ragged chunk stages them through registers,
  // since its rows beyond L must read as zero.  The barrier that follows the
  // first head's copies orders both.
  if constexpr (BF) {
    if (L == kC) {
      const int wu = __builtin_amdgcn_readfirstlane(w);
      copy_rows<128>(kg, (int64_t)Hqk * kD, L, sm.K, wu, kGW);
      copy_rows<128>(qg, (int64_t)Hqk * kD, L, sm.Q, wu, kGW);
    } else {
      stage<E, 128, kC, NT>(Lds<E, 128>{sm.K}, kg, (int64_t)Hqk * kD, L);
      stage<E, 128, kC, NT>(Lds<E, 128>{sm.Q}, qg, (int64_t)Hqk * kD, L);
    }
  }

  // This wave's two 64x64 tiles (ti, tj) of the phase-1.5 products.
  // The ten tiles on and below the diagonal: waves 0 and 1 take two, the
  // others one, so that (waves w and w + 4 sharing a SIMD) no SIMD holds more
  // than three.  Entries past the tenth are above the diagonal: skipped.
  constexpr int kTi[16] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3, 0, 0, 0, 0, 0, 0};
  constexpr int kTj[16] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3, 1, 1, 1, 1, 1, 1};
  int ti[2], tj[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    ti[x] = kTi[8 * x + w];
    tj[x] = kTj[8 * x + w];
  }

  f32x4 dQ[4], dK[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) { dQ[mt] = zero4(); dK[mt] = zero4(); }

  // bf16 operands of value head hh copied straight into LDS.  Rows of dO and
  // V beyond L repeat the last token; they only ever meet zero rows of K and
  // Q, zero beta and the identity rows of N, so nothing they touch is stored.
  // part 0: S0, dS', dO (read in phases 1 - 2 up to the state products);
  // part 1: V, N, M (read in phase 1; their slots then hold Dl and Y).
  auto stage_head = [&](int hh2, int part) {
    if constexpr (BF) {
      const int wu = __builtin_amdgcn_readfirstlane(w);
      const int h2 = gq * G + hh2;
      const size_t hc2 = (size_t)cid * Hv + h2;
      // per-lane copy addresses recomputed at each call rather than hoisted
      // out of the head loop (where they would be spilled)
      int lo = lane_id();
      asm volatile("" : "+v"(lo));
      if (part == 0) {
        copy_rows<128, kD>(Sc + hc2 * kD * kD, kD, kD, sm.S0, wu, kGW, lo);
        copy_rows<128, kD>(dSc + hc2 * kD * kD, kD, kD, sm.dS, wu, kGW, lo);
        copy_rows<128>(dout + (tok0 * Hv + h2) * kD, (int64_t)Hv * kD, L, sm.dO, wu, kGW, lo);
      } else {
        copy_rows<128>(v + (tok0 * Hv + h2) * kD, (int64_t)Hv * kD, L, sm.u1.V, wu, kGW, lo);
        copy_rows<64>(Nw + hc2 * kC * kC, kC, kC, sm.u2.nm.N, wu, kGW, lo);
        copy_rows<64>(Mw + hc2 * kC * kC, kC, kC, sm.u2.nm.M, wu, kGW, lo);
      }
    }
  };

  // The same copies of value head hh2, two at a time (piece j = 0..6 of this
  // wave's fourteen with eight waves), so that they can be spread over the E
  // products: issued all at once they kept the waves stalled ~3-5 k cycles
  // before the products could start.
  auto stage_piece = [&](int hh2, int j) {
    if constexpr (BF) {
      static_assert(kGW == 8, "copy pieces are laid out for eight waves");
      const int wu = __builtin_amdgcn_readfirstlane(w);
      const int h2 = gq * G + hh2;
      const size_t hc2 = (size_t)cid * Hv + h2;
      int lo = lane_id();
      asm volatile("" : "+v"(lo));
      const bf16* st = Sc + hc2 * kD * kD;
      const bf16* ds = dSc + hc2 * kD * kD;
      const bf16* og = dout + (tok0 * Hv + h2) * kD;
      const bf16* vg = v + (tok0 * Hv + h2) * kD;
      const int64_t hs = (int64_t)Hv * kD;
      switch (j) {
        case 0: case 1:      // S0: copies w + 16 j, w + 16 j + 8 of 32
          copy_row_one<128, kD>(st, kD, kD, sm.S0, wu + 16 * j, lo);
          copy_row_one<128, kD>(st, kD, kD, sm.S0, wu + 16 * j + 8, lo);
          break;
        case 2: case 3:      // dS'
          copy_row_one<128, kD>(ds, kD, kD, sm.dS, wu + 16 * (j - 2), lo);
          copy_row_one<128, kD>(ds, kD, kD, sm.dS, wu + 16 * (j - 2) + 8, lo);
          break;
        case 4:              // dO: copies w, w + 8 of 16
          copy_row_one<128>(og, hs, L, sm.dO, wu, lo);
          copy_row_one<128>(og, hs, L, sm.dO, wu + 8, lo);
          break;
        case 5:              // V
          copy_row_one<128>(vg, hs, L, sm.u1.V, wu, lo);
          copy_row_one<128>(vg, hs, L, sm.u1.V, wu + 8, lo);
          break;
        default:             // N, M: copy w of 8 each
          copy_row_one<64>(Nw + hc2 * kC * kC, kC, kC, sm.u2.nm.N, wu, lo);
          copy_row_one<64>(Mw + hc2 * kC * kC, kC, kC, sm.u2.nm.M, wu, lo);
          break;
      }
    }
  };

  // wave 0: alpha and beta of the next head, loaded a head ahead (lane =
  // token); wave 1: what the gate reduction of a head reads that the next
  // head's set-up overwrites
  float a_nx = 1.f, b_nx = 0.f, al_g = 1.f, gmL_g = 0.f;
  if (w == 0 && l < L) {
    a_nx = alpha[(tok0 + l) * Hv + gq * G];
    b_nx = beta[(tok0 + l) * Hv + gq * G];
  }
  for (int hh = 0; hh < G; ++hh) {
    const int h = gq * G + hh;
    const Lane ln = lane_opaque();
    const int r = ln.r, g = ln.g;
    const size_t hc = (size_t)cid * Hv + h;
    const E* vh = v + (tok0 * Hv + h) * kD;
    const E* oh = dout + (tok0 * Hv + h) * kD;
    auto mS0 = [&]() {
      if constexpr (BF) return Lds<E, 128>{sm.S0};
      else return Glb<E>{Sc + hc * kD * kD, kD, kD};
    }();
    auto mdS = [&]() {
      if constexpr (BF) return Lds<E, 128>{sm.dS};
      else return Glb<E>{dSc + hc * kD * kD, kD, kD};
    }();
    auto mO = [&]() {
      if constexpr (BF) return Lds<E, 128>{sm.dO};
      else return Glb<E>{oh, (int64_t)Hv * kD, L};
    }();
    auto mV = [&]() {
      if constexpr (BF) return Lds<E, 128>{sm.u1.V};
      else return Glb<E>{vh, (int64_t)Hv * kD, L};
    }();
    auto mN = [&]() {
      if constexpr (BF) return Lds<E, 64>{sm.u2.nm.N};
      else return Glb<E>{Nw + hc * kC * kC, kC, kC};
    }();
    auto mM = [&]() {
      if constexpr (BF) return Lds<E, 64>{sm.u2.nm.M};
      else return Glb<E>{Mw + hc * kC * kC, kC, kC};
    }();

    // ---- stage: head 0 here; later heads were issued during the previous
    // head's phase 2 (stage_head below)
    if constexpr (BF) {
      if (hh == 0) {
        stage_head(0, 0);
        stage_head(0, 1);
      }
    }
    if (w == 0) {
      const float a = a_nx;
      float G2lo;
      const float G2 = wave_inclusive_sum2(hw_log2(a), G2lo);
      const float Glast = __shfl(G2, kC - 1, 64), Glastlo = __shfl(G2lo, kC - 1, 64);
      sm.G2[l] = G2;
      sm.G2lo[l] = G2lo;
      sm.gm[l] = hw_exp2(G2);
      sm.dc[l] = hw_exp2((Glast - G2) + (Glastlo - G2lo));
      sm.bt[l] = b_nx;
      sm.al[l] = a;
    }
    if constexpr (BF) wait_copies();
    __syncthreads();

    // ---- phase 1: this wave's value columns c = 16w + r
    const int c = 16 * w + r;
    // Elements (16 mt + 4 g + i, c) of a matrix, in this lane's accumulator
    // order: they are the slots of transposed fragment reads of column c, two
    // reads (bf16) or four (fp32) instead of sixteen element reads.
    auto col16 = [&](const auto& mx, float (&out)[16]) {
      if constexpr (BF) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Fr<E> f = mx.cm(c, KB * kb, ln);
#pragma unroll
          for (int j = 0; j < 8; ++j) out[4 * (2 * kb + (j >> 2)) + (j & 3)] = (float)f[j];
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const Fr<E> f = mx.cm(c, KB * mt, ln);
#pragma unroll
          for (int i = 0; i < 4; ++i) out[4 * mt + i] = f[i];
        }
      }
    };
    {
      float ssl = 0.f;
      f32x4 X[4], Dl[4], dD[4], Y[4];
      {
        f32x4 XB[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb) {
          // natural K order (both operands from LDS): one 16-byte read each
          const Fr<E> s0 = mS0.rmn(c, KB * kb, ln), ds = mdS.rmn(c, KB * kb, ln);
#pragma unroll
          for (int e = 0; e < NS; ++e) ssl += (float)s0[e] * (float)ds[e];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) X[mt] = mma(X[mt], mK.rmn(16 * mt + r, KB * kb, ln), s0);
        }
        float vv[16];
        col16(mV, vv);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = 16 * mt + 4 * g + i;
            X[mt][i] = vv[4 * mt + i] - sm.gm[tok] * X[mt][i];   // V - gamma K S0^T
            XB[mt][i] = sm.bt[tok] * X[mt][i];
          }
        // Dl = N (beta X)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 d = zero4();
#pragma unroll
          for (int kb = 0; kb < kC / KB; ++kb)
            if (!blk_above<E>(mt, kb)) d = mma(d, mN.rm(16 * mt + r, KB * kb, ln), acc_frag<E>(XB, kb));
          Dl[mt] = d;
        }
      }
      // dDl = M^T dO + diag(dec) K dS'^T, one token tile at a time; w_i partial
      const int tk = 16 * (r >> 2) + 4 * g + (r & 3);   // the token this lane stores
      float pwv[16];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 kds = zero4(), m = zero4();
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb)
          kds = mma(kds, mK.rmn(16 * mt + r, KB * kb, ln), mdS.rmn(c, KB * kb, ln));
#pragma unroll
        for (int kb = 0; kb < kC / KB; ++kb)
          if (!blk_below<E>(mt, kb)) m = mma(m, mM.cm(16 * mt + r, KB * kb, ln), mO.cm(c, KB * kb, ln));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mt + 4 * g + i;
          dD[mt][i] = m[i] + sm.dc[tok] * kds[i];
          pwv[4 * mt + i] = Dl[mt][i] * kds[i];
        }
      }
      sm.u3.part[w][2][tk] = sm.dc[tk] * rsum16(pwv, r);
      // Y = N^T dDl
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 y = zero4();
#pragma unroll
        for (int kb = 0; kb < kC / KB; ++kb)
          if (!blk_below<E>(mt, kb)) y = mma(y, mN.cm(16 * mt + r, KB * kb, ln), acc_frag<E>(dD, kb));
        Y[mt] = y;
      }
      // beta and gate partials: Y.X and -gamma beta Y.(K S0^T) = -beta Y.(V - X)
      {
        float pbv[16], pgv[16], vv[16];
        col16(mV, vv);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pbv[4 * mt + i] = Y[mt][i] * X[mt][i];
            pgv[4 * mt + i] = Y[mt][i] * (vv[4 * mt + i] - X[mt][i]);
          }
        sm.u3.part[w][0][tk] = rsum16(pbv, r);
        sm.u3.part[w][1][tk] = -sm.bt[tk] * rsum16(pgv, r);
      }
      ssl = wave_sum(ssl);
      if (l == 0) sm.ss[w] = ssl;
      __syncthreads();   // every wave is done with V, N, M (their LDS is reused)
      // ---- reduce the phase 1 partials (fixed order); done before the
      // barrier that precedes the E products, which overwrite them
      if (threadIdx.x < 3 * kC) {
        const int qn = threadIdx.x / kC, t = threadIdx.x % kC;
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < kGW; ++x) s += sm.u3.part[x][qn][t];
        sm.fin[qn == 0 ? 1 : (qn == 1 ? 0 : 2)][t] = s;
      }
      // dv through a uniform base and 32-bit byte offsets (a chunk's rows
      // span far less than 2 GiB): one add per store, no 64-bit multiply
      char* dvh = reinterpret_cast<char*>(dv + (tok0 * Hv + h) * kD);
      const uint32_t rstr = (uint32_t)(Hv * kD * sizeof(E));
      const uint32_t lo = (uint32_t)(4 * g) * rstr + (uint32_t)(c * sizeof(E));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mt + 4 * g + i;
          Dls(tok, c) = from_f32<E>(Dl[mt][i]);
          Ys(tok, c) = from_f32<E>(Y[mt][i]);
        }
      // dv: unguarded stores for a full chunk (the common case), guarded for
      // the ragged tail
      const bool full = L == kC;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mt + 4 * g + i;
          if (full || tok < L)
            *reinterpret_cast<E*>(dvh + (lo + (uint32_t)(16 * mt + i) * rstr)) =
                from_f32<E>(sm.bt[tok] * Y[mt][i]);
        }
    }
    __syncthreads();

    // ---- phase 1.5: dO Dl^T and Y Dl^T on this wave's tiles, with K K^T
    // and Q K^T on the same tiles (recomputed per head: cheaper than keeping
    // them live)
    f32x4 OD[2], YD[2], KK[2], QK[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      OD[x] = zero4();
      YD[x] = zero4();
      KK[x] = zero4();
      QK[x] = zero4();
      if (tj[x] <= ti[x]) {
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb) {
          const Fr<E> bd = Dls.rmn(16 * tj[x] + r, KB * kb, ln);
          OD[x] = mma(OD[x], mO.rmn(16 * ti[x] + r, KB * kb, ln), bd);
          YD[x] = mma(YD[x], Ys.rmn(16 * ti[x] + r, KB * kb, ln), bd);
          const Fr<E> bk = mK.rmn(16 * tj[x] + r, KB * kb, ln);
          KK[x] = mma(KK[x], mK.rmn(16 * ti[x] + r, KB * kb, ln), bk);
          QK[x] = mma(QK[x], mQ.rmn(16 * ti[x] + r, KB * kb, ln), bk);
        }
      }
    }
    // (no barrier: the phase 1 partials that E overwrites were reduced before
    // the last one)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (tj[x] > ti[x]) continue;
      const int jj = 16 * tj[x] + r;
      float colsum = 0.f, rsv[4], rbv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = 16 * ti[x] + 4 * g + i;
        const float gam_ =
            jj <= ii ? hw_exp2((sm.G2[ii] - sm.G2[jj]) + (sm.G2lo[ii] - sm.G2lo[jj])) : 0.f;
        const float dMG = jj <= ii ? OD[x][i] * gam_ : 0.f;
        const float dAG = jj < ii ? -YD[x][i] * gam_ : 0.f;
        const float wa = sm.bt[ii] * dAG;
        const float P = dMG * QK[x][i] + wa * KK[x][i];
        // every location of E has exactly one writer: (ii, jj) on and below
        // the diagonal, its mirror (jj, ii) above it (off-diagonal tiles:
        // every element is below)
        if (tj[x] < ti[x]) {
          Es(ii, jj) = from_f32<E>(dMG);
          Es(jj, ii) = from_f32<E>(wa);
        } else {
          if (jj <= ii) Es(ii, jj) = from_f32<E>(dMG);
          if (jj < ii) Es(jj, ii) = from_f32<E>(wa);
        }
        rsv[i] = sum16(P);
        rbv[i] = sum16(dAG * KK[x][i]);
        colsum += P;
      }
      // row sums: lane r stores row 16 ti + 4g + r%4 (four lanes write each
      // row, the same value); column sums: every lane group writes the same
      // column value
      {
        const int i4 = r & 3;
        const float rs = i4 == 0 ? rsv[0] : (i4 == 1 ? rsv[1] : (i4 == 2 ? rsv[2] : rsv[3]));
        const float rb = i4 == 0 ? rbv[0] : (i4 == 1 ? rbv[1] : (i4 == 2 ? rbv[2] : rbv[3]));
        sm.rowp[tj[x]][16 * ti[x] + 4 * g + i4] = rs;
        sm.rowb[tj[x]][16 * ti[x] + 4 * g + i4] = rb;
      }
      colsum += __shfl_xor(colsum, 16, 64);
      colsum += __shfl_xor(colsum, 32, 64);
      sm.colp[ti[x]][jj] = colsum;
    }
    __syncthreads();

    // ---- phase 2: this wave's key columns c
    if (w == 0) {
      const int t = l, tt = t >> 4;
      float rs = 0.f, rb = 0.f, cs = 0.f;
      for (int x = 0; x <= tt; ++x) { rs += sm.rowp[x][t]; rb += sm.rowb[x][t]; }
      for (int x = tt; x < 4; ++x) cs += sm.colp[x][t];
      sm.fin[0][t] += rs - cs;
      sm.fin[1][t] += rb;
    }
    {
      // gamma dO S0 into dq (and the gate's q . dq partial)
      {
        const int tk = 16 * (r >> 2) + 4 * g + (r & 3);
        float pav[16];
        f32x4 T1[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) T1[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb) {
          const Fr<E> s0 = mS0.cm(c, KB * kb, ln);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) T1[mt] = mma(T1[mt], mO.rm(16 * mt + r, KB * kb, ln), s0);
        }
        float qq[16];
        col16(mQ, qq);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = 16 * mt + 4 * g + i;
            const float g1 = sm.gm[tok] * T1[mt][i];
            dQ[mt][i] += g1;
            pav[4 * mt + i] = qq[4 * mt + i] * g1;
          }
        sm.pa[w][tk] = rsum16(pav, r);
      }
      // -gamma beta Y S0 into dk
      {
        f32x4 T2[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) T2[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb) {
          const Fr<E> s0 = mS0.cm(c, KB * kb, ln);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) T2[mt] = mma(T2[mt], Ys.rm(16 * mt + r, KB * kb, ln), s0);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = 16 * mt + 4 * g + i;
            dK[mt][i] -= sm.gm[tok] * sm.bt[tok] * T2[mt][i];
          }
      }
      // diag(dec) Dl dS' into dk
      {
        f32x4 T3[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) T3[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < kD / KB; ++kb) {
          const Fr<E> ds = mdS.cm(c, KB * kb, ln);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) T3[mt] = mma(T3[mt], Dls.rm(16 * mt + r, KB * kb, ln), ds);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) dK[mt][i] += sm.dc[16 * mt + 4 * g + i] * T3[mt][i];
      }
      // S0, dS', dO, V, N, M and their slots' later tenants Dl and Y are no
      // longer read (the E products below read only E, K and Q): all the next
      // head's copies start now and run under the E products and the gate
      // reduction
      if constexpr (BF) __syncthreads();
      if (w == 0 && hh + 1 < G && l < L) {
        a_nx = alpha[(tok0 + l) * Hv + h + 1];
        b_nx = beta[(tok0 + l) * Hv + h + 1];
      }
      if (w == 1) {
        al_g = sm.al[l];
        gmL_g = sm.gm[L - 1];
      }
      // the next head's copies are issued two at a time between the E
      // product steps below
      // (dM * Gam) K into dq; (dM * Gam)^T Q and (Wa + Wa^T) K into dk
#pragma unroll
      for (int kb = 0; kb < kC / KB; ++kb) {
        const Fr<E> bk = mK.cm(c, KB * kb, ln), bq = mQ.cm(c, KB * kb, ln);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (hh + 1 < G && 4 * kb + mt < 7) stage_piece(hh + 1, 4 * kb + mt);
          const int row = 16 * mt + r;
          if (blk_below<E>(mt, kb)) {          // every K index below the row
            const Fr<E> e_rm = Es.rm(row, KB * kb, ln), e_cm = Es.cm(row, KB * kb, ln);
            dQ[mt] = mma(dQ[mt], e_rm, bk);
            dK[mt] = mma(dK[mt], e_cm, bk);
          } else if (blk_above<E>(mt, kb)) {   // every K index above the row
            const Fr<E> e_rm = Es.rm(row, KB * kb, ln), e_cm = Es.cm(row, KB * kb, ln);
            dK[mt] = mma(dK[mt], e_cm, bq);
            dK[mt] = mma(dK[mt], e_rm, bk);
          } else {
            const Fr<E> e_rm = Es.rm(row, KB * kb, ln), e_cm = Es.cm(row, KB * kb, ln);
            Fr<E> lowr = e_rm, lowt = e_cm, sym;
#pragma unroll
            for (int e = 0; e < NS; ++e) {
              const int kk = KB * kb + kslot<E>(g, e);
              if (kk > row) frag_zero<E>(lowr, e);
              if (kk < row) frag_zero<E>(lowt, e);
              sym[e] = kk > row ? e_rm[e] : e_cm[e];
              if (kk == row) frag_zero<E>(sym, e);
            }
            dQ[mt] = mma(dQ[mt], lowr, bk);
            dK[mt] = mma(dK[mt], lowt, bq);
            dK[mt] = mma(dK[mt], sym, bk);
          }
        }
      }
    }
    __syncthreads();

    // ---- gates and beta for this head (wave 1, lane = token), beside wave
    // 0's set-up of the next head.  No barrier after it: the other waves
    // write nothing it reads (alpha and gamma of this head it took into
    // registers before the last barrier) before the barrier that ends the
    // next head's set-up, which it reaches only after this.
    if (w == 1) {
      const int t = l;
      float pa = 0.f, fw = sm.fin[2][t];
#pragma unroll
      for (int x = 0; x < kGW; ++x) pa += sm.pa[x][t];
      float ss = 0.f;
#pragma unroll
      for (int x = 0; x < kGW; ++x) ss += sm.ss[x];
      const float wsum = wave_sum(t < L ? fw : 0.f);
      float dG = t < L ? pa + sm.fin[0][t] - fw : 0.f;
      if (t == L - 1) dG += wsum + gmL_g * ss;
      // reverse inclusive prefix: sum over i >= t
      const float tot = wave_sum(dG);
      const float incl = wave_inclusive_sum(dG);
      const float dlog = tot - incl + dG;
      if (t < L) {
        const size_t gi = (tok0 + t) * Hv + h;
        dalpha[gi] = dlog / al_g;
        dbeta[gi] = sm.fin[1][t];
      }
    }
  }

  // ---- dq, dk of the group
  char* dqg = reinterpret_cast<char*>(dq + (tok0 * Hqk + gq) * kD);
  char* dkg = reinterpret_cast<char*>(dk + (tok0 * Hqk + gq) * kD);
  const int c = 16 * w + r;
  const uint32_t rstr = (uint32_t)(Hqk * kD * sizeof(E));
  const uint32_t lo = (uint32_t)(4 * g) * rstr + (uint32_t)(c * sizeof(E));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * mt + 4 * g + i;
      if (tok < L) {
        const uint32_t off = lo + (uint32_t)(16 * mt + i) * rstr;
        *reinterpret_cast<E*>(dqg + off) = from_f32<E>(dQ[mt][i]);
        *reinterpret_cast<E*>(dkg + off) = from_f32<E>(dK[mt][i]);
      }
    }
}

}  // namespace bwd

hipError_t launch_backward(const BackwardLaunch& a, hipStream_t st) {
  using namespace bwd;
  constexpr int NW = 2;
  const dim3 gchain(kD / (16 * NW), a.Hv, a.nseq);
  if (a.bf16_io) {
    typedef bf16 E;
    // the chunk states were written by the forward scan (gdn_api.hip)
    if (!a.states_ready) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_chain_split_kernel, dim3(a.Hv * (kD / 32), a.nseq), dim3(384), 0, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.dout,
                       a.beta, a.dht, a.dh0, (const E*)a.N, (const E*)a.M, a.gam, a.dec,
                       (E*)a.dS, a.cm, a.Hqk, a.Hv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nc == 0) return e;
    hipLaunchKernelGGL((bwd_grad_kernel<E>), dim3(a.nc, a.Hqk), dim3(64 * kGW), 0, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.dout, a.alpha,
                       a.beta, (const E*)a.N, (const E*)a.M, (const E*)a.S, (const E*)a.dS,
                       (E*)a.dq, (E*)a.dk, (E*)a.dv, a.dalpha, a.dbeta, a.cm, a.Hqk, a.Hv);
    return hipGetLastError();
  } else {
    typedef float E;
    if (a.nc > 0) {
      hipLaunchKernelGGL((fwd_states_kernel<E, NW>), gchain, dim3(64 * NW), 0, st, (const E*)a.k,
                         (const E*)a.v, a.beta, a.h0, (const E*)a.N, a.gam, a.dec, (E*)a.S,
                         a.cm, a.Hqk, a.Hv);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_chain_kernel<E, NW>), gchain, dim3(64 * NW), 0, st, (const E*)a.q,
                       (const E*)a.k, (const E*)a.dout, a.beta, a.dht, a.dh0, (const E*)a.N,
                       (const E*)a.M, a.gam, a.dec, (E*)a.dS, a.cm, a.Hqk, a.Hv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nc == 0) return e;
    hipLaunchKernelGGL((bwd_grad_kernel<E>), dim3(a.nc, a.Hqk), dim3(64 * kGW), 0, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.dout, a.alpha,
                       a.beta, (const E*)a.N, (const E*)a.M, (const E*)a.S, (const E*)a.dS,
                       (E*)a.dq, (E*)a.dk, (E*)a.dv, a.dalpha, a.dbeta, a.cm, a.Hqk, a.Hv);
    return hipGetLastError();
  }
}

}  // namespace gdn

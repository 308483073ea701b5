// Gated attention layer of the hybrid stack on gfx950: QK-Norm, partial RoPE,
// causal grouped-query softmax attention and the sigmoid output gate.
//
// Shapes follow the pages: 24 query heads and 4 key/value heads of head dim
// 256 (page "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture, 256k Context,
// and 24GB Local Serving", section "The Role of Periodic Gated Attention"),
// RoPE on a 64-channel subspace with theta = 1e7 (same section), QK-Norm and
// the sigmoid output gate (card "Qwen3.8 (27B)", "Architecture concepts";
// page "Qwen3.8 Explained ...", the note on attn_output_gate).  Per (token,
// head): q, k <- RMSNorm(q, k) * w; the first rope_dim channels rotate in the
// pairing (j, j + rope_dim/2) by pos * theta^(-2j/rope_dim); then
// o = softmax_causal(q k^T / sqrt(256)) v, times sigmoid(gate) per channel.
//
// Kernels:
//  * attn_prep: one wave per (token, head) row: RMSNorm, weight, rotation.
//    The angle is formed in turns and reduced in fp64 (at position 262,143 an
//    fp32 angle would be off by ~1e-2 rad), then the hardware sin/cos in fp32.  Query
//    rows go to the workspace, key rows (and the value rows, unchanged) to the
//    key/value cache at their positions.
//  * attn_fwd (prefill): one workgroup per (32 query rows, key/value head,
//    sequence) with two waves per query head of the group (16 rows each), so
//    every K/V tile staged in LDS serves all six heads.  A wave keeps its
//    query rows' Q fragments in registers and computes S^T = K Q^T: in that orientation each
//    lane owns one query column, so the running max and sum of the online
//    softmax stay in the lane (two shuffles across lane groups per block), and
//    the probability tiles are directly the B operand of O^T = V^T P^T.  K/V
//    tiles of 64 keys are double-buffered in LDS with direct global->LDS
//    copies (bf16), in padded rows that make every fragment read free of bank
//    conflicts.  Only the diagonal block is masked.  Workgroups are issued
//    longest (latest query block) first.
//  * attn_decode + attn_combine: split-K over the cached keys.  One workgroup
//    per (split of keys, key/value head, sequence), the split sized for about
//    two workgroups per CU; 32-key blocks
//    double-buffered in LDS (69 KB, two workgroups per CU); the six query heads are the MFMA N dimension and
//    each of the four waves produces 64 of the 256 output channels; partial
//    (max, sum, O) per split, merged and gated by the combine kernel.
#include "gdn_device.hpp"
#include "gdn_frag.hpp"
#include "gdn_launch.hpp"

#include <algorithm>
#include <cmath>

namespace gdn {
namespace attn {
using namespace frag;

constexpr int kDh = 256;        // head dim
constexpr int kKvb = 64;        // keys per prefill block
// decode: keys per split are chosen per call (attn_decode_split)

// ------------------------------------------------------------ prep

// Rows of token tok: heads 0 .. Hq-1 are queries, Hq .. Hq+Hkv-1 keys.
// Token tok = b * T + t sits at position pos[b] (decode) or t (prefill, pos null).
constexpr int kPrepWaves = 8;   // waves per token (a decode step has only B tokens)

template <typename E>
__global__ __launch_bounds__(64 * kPrepWaves) void attn_prep_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ qw, const float* __restrict__ kw, float eps, int rope_dim,
    double fstep, const int32_t* __restrict__ pos, E* __restrict__ qo, E* __restrict__ kc,
    E* __restrict__ vc, int64_t ntok, int T, int cache_len, int Hq, int Hkv) {
  // one workgroup per token: its Hq + Hkv rows share one position, so each
  // lane forms its rotation's sin and cos once and applies them to every row
  const int l = lane_id(), w = wave_id();
  const int64_t tok = blockIdx.x;
  const int H = Hq + Hkv;
  const int b = (int)(tok / T), t = (int)(tok - (int64_t)b * T);
  int p = pos ? pos[b] : t;
  p = min(max(p, 0), cache_len - 1);              // stays inside the cache
  const int half = rope_dim >> 1, hl = half >> 2;
  const int partner = l < hl ? l + hl : (l < 2 * hl ? l - hl : l);
  const bool first = l < hl, rot = l < 2 * hl;
  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (rot) {
    const int jl = first ? l : l - hl;
    // frequency j is theta^(-2j / rope_dim) = fstep^j (fstep = theta^(-2 /
    // rope_dim), formed on the host): fstep^(4 jl) by repeated squaring, then
    // one more factor per i; the rounding of these fp64 products (~1e-15
    // relative) is far below the fp32 rounding of the reduced angle
    double fb = 1.0, sq = fstep;
    for (int e = 4 * jl; e; e >>= 1, sq *= sq)
      if (e & 1) fb *= sq;
#pragma unroll
    for (int i = 0; i < 4; ++i, fb *= fstep) {
      // theta^(-2j / rope_dim) / (2 pi) turns per position, the angle reduced
      // in fp64 (at position 262,143 an fp32 angle would be off by ~1e-2 rad),
      // then the hardware sin and cos, which take turns
      const double fq = fb * 0.15915494309189535;
      double rev = (double)p * fq;
      rev -= rint(rev);
      sn[i] = __builtin_amdgcn_sinf((float)rev);
      cs[i] = __builtin_amdgcn_cosf((float)rev);
    }
  }
  constexpr int RB = 4;                           // rows per wave per batch
  for (int hb = w * RB; hb < H; hb += kPrepWaves * RB) {
    f32x4 xs[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int hd = hb + rr;
      xs[rr] = zero4();
      if (hd < H) {
        const E* src = hd < Hq ? q + (tok * Hq + hd) * kDh : k + (tok * Hkv + (hd - Hq)) * kDh;
        if constexpr (sizeof(E) == 2) {
          const bf16x4 r4 = *reinterpret_cast<const bf16x4*>(src + 4 * l);
          xs[rr] = f32x4{(float)r4[0], (float)r4[1], (float)r4[2], (float)r4[3]};
        } else {
          xs[rr] = *reinterpret_cast<const f32x4*>(src + 4 * l);
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int hd = hb + rr;
      if (hd >= H) break;                         // wave-uniform
      const bool is_q = hd < Hq;
      float x[4] = {xs[rr][0], xs[rr][1], xs[rr][2], xs[rr][3]};
      const float ss = wave_sum(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
      const float rs = 1.f / sqrtf(ss * (1.f / kDh) + eps);
      const float* wt = is_q ? qw : kw;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= rs * (wt ? wt[4 * l + i] : 1.f);
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = __shfl(x[i], partner, 64);
      if (rot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[i] = first ? x[i] * cs[i] - y[i] * sn[i] : x[i] * cs[i] + y[i] * sn[i];
      }
      E* dst = is_q ? qo + (tok * Hq + hd) * kDh
                    : kc + (((int64_t)b * cache_len + p) * Hkv + (hd - Hq)) * kDh;
      // queries carry the softmax scale log2(e) / sqrt(256) (the attention
      // kernels work in base 2); the cache keeps the keys themselves
      const float sc = is_q ? 1.4426950408889634f / 16.f : 1.f;
      store4(dst + 4 * l, f32x4{x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc});
      if (!is_q && vc) {
        const E* vs = v + (tok * Hkv + (hd - Hq)) * kDh;
        E* vd = vc + (((int64_t)b * cache_len + p) * Hkv + (hd - Hq)) * kDh;
        *reinterpret_cast<uint2*>(vd + 4 * l) = *reinterpret_cast<const uint2*>(vs + 4 * l);
        if constexpr (sizeof(E) == 4)
          *reinterpret_cast<uint2*>(vd + 4 * l + 2) = *reinterpret_cast<const uint2*>(vs + 4 * l + 2);
      }
    }
  }
}

// Rows [0, rows) of a row-major global matrix into an LDS matrix (rows >= `rows`
// zero), by `nt` threads in 16-byte pieces.
template <typename E, int W, int R>
__device__ __forceinline__ void stage_rows(Lds<E, W> dst, const E* src, int64_t ld, int rows,
                                           int nt) {
  constexpr int EP = 16 / sizeof(E), PPR = W / EP;
  for (int pc = threadIdx.x; pc < R * PPR; pc += nt) {
    const int row = pc / PPR, c = (pc % PPR) * EP;
    *reinterpret_cast<uint4*>(&dst(row, c)) =
        row < rows ? *reinterpret_cast<const uint4*>(src + row * ld + c) : uint4{0u, 0u, 0u, 0u};
  }
}

// ------------------------------------------------------------ bf16 K/V tiles
// 64 rows of 256 bf16 with padded rows, so that every fragment address is one
// per-lane base plus a compile-time offset and no read meets a bank conflict
// (64-bit LDS reads are served 32 lanes at a time over 64 four-byte banks):
//  * KTile rows are 528 bytes (16 bytes of padding).  Row-pattern fragment
//    reads (lane (r, g): 8 bytes of row r at channel 4g) land on banks
//    4r + 2g (+1): all 64 banks once per 32 lanes.
//  * VTile rows are 544 bytes (32 bytes of padding).  Transposed reads
//    (ds_read_b64_tr_b16; lane (r, g) reads 8 bytes of row 4g + r/4 at
//    channel 4(r%4)) land on banks 8 (4g + r/4) + 2 (r%4) (+1): all 64 once.
template <int ROWB, int ROWS = kKvb>
struct PadTile {
  static constexpr int kBytes = ROWS * ROWB;
  char* p;
  // A/B fragment with the lane index along rows (keys): slots are channels
  // k0 + kslot(g, j).
  __device__ bf16x8 rm(int row0, int k0, const Lane& ln) const {
    const char* b = p + (row0 + ln.r) * ROWB + 8 * ln.g + 2 * k0;
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(b);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(b + 32);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Same, in the natural K order (slot j = channel k0 + 8g + j): one 16-byte
  // read.  For products whose operands both come from memory (the scores).
  __device__ bf16x8 rm8(int row0, int k0, const Lane& ln) const {
    return *reinterpret_cast<const bf16x8*>(p + (row0 + ln.r) * ROWB + 16 * ln.g + 2 * k0);
  }
  // Fragment with the lane index along channels col0 + r: slots are rows
  // k0 + kslot(g, j).
  __device__ bf16x8 cm(int col0, int k0, const Lane& ln) const {
    const char* b = p + (k0 + 4 * ln.g + (ln.r >> 2)) * ROWB + 2 * col0 + 8 * (ln.r & 3);
    const s16x4 lo = lds_tr16(b);
    const s16x4 hi = lds_tr16(b + 16 * ROWB);
    return __builtin_shufflevector(as_bf16x4(lo), as_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
  }
};
typedef PadTile<528> KTile;
typedef PadTile<544> VTile;
constexpr int kDkb = 32;                  // keys per decode block
typedef PadTile<528, kDkb> KTileD;
typedef PadTile<544, kDkb> VTileD;

// 64 rows (rows >= L repeat row L-1) of 256 bf16 with row stride ld into a
// padded tile, copied straight into LDS; wave w of nw issues copies w, w + nw,
// ...  Copy `it` fills LDS bytes [1024 it, 1024 it + 1024): a lane whose 16
// bytes fall in padding is switched off.
template <int ROWB, int ROWS = kKvb>
__device__ __forceinline__ void copy_tile(const bf16* src, int64_t ld, int L, char* dst, int w,
                                          int nw) {
  constexpr int NIT = (ROWS * ROWB + 1023) / 1024;
  const int l = lane_id();
  for (int it = w; it < NIT; it += nw) {
    const int byte = 1024 * it + 16 * l, row = byte / ROWB, off = byte - row * ROWB;
    if (row < ROWS && off < 2 * kDh)
      dma16(reinterpret_cast<const char*>(src) + ((uint32_t)min(row, L - 1) * (uint32_t)(2 * ld) + off),
            dst + 1024 * it);
  }
}

// ------------------------------------------------------------ prefill
template <typename E>
struct FwdSmem {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int NB = BF ? 2 : 1;                 // K/V buffers
  static constexpr int KB_ = BF ? KTile::kBytes : Lds<E, kDh>::size(kKvb) * (int)sizeof(E);
  static constexpr int VB_ = BF ? VTile::kBytes : Lds<E, kDh>::size(kKvb) * (int)sizeof(E);
  alignas(16) char K[NB][KB_];
  alignas(16) char V[NB][VB_];
};

// QS waves per query head, each with QT tiles of 16 query rows: the workgroup
// covers 16 QT QS rows of all G heads of its key/value head.  bf16: QT = 1,
// QS = 2 (12 waves of at most 170 registers); fp32: QT = 1, QS = 1.
// Largest workgroup an instantiation is compiled for (its register budget):
// the launch must never exceed it.
template <int QS> constexpr int fwd_max_threads() { return QS == 2 ? 768 : 512; }

template <typename E, int QT, int QS>
__global__ __launch_bounds__(fwd_max_threads<QS>()) void attn_fwd_kernel(
    const E* __restrict__ qr, const E* __restrict__ kc, const E* __restrict__ vc,
    const E* __restrict__ gate, E* __restrict__ o, int T, int cache_len, int Hq, int Hkv,
    int nqb, int nseq) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int KB = FragOf<E>::KB, NKB = kDh / KB, QR = 16 * QT, QRW = QR * QS;
  __shared__ FwdSmem<E> sm;
  const int G = Hq / Hkv, NWV = G * QS;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), r = l & 15, g = l >> 4;
  // Workgroups are dispatched to the eight XCDs round-robin by linear id.  When
  // the (sequence, key/value head) streams divide eight, each XCD serves one
  // stream, so its L2 holds that stream's keys and values only; within a
  // stream, query blocks go longest (latest) first.
  const int nst = Hkv * nseq;
  int qidx, st;
  if (nst <= 8 && 8 % nst == 0) {
    const int xper = 8 / nst, lin = blockIdx.x, xcd = lin & 7;
    st = xcd / xper;
    qidx = (lin >> 3) * xper + xcd % xper;
    if (qidx >= nqb) return;
  } else {
    st = blockIdx.x / nqb;
    qidx = blockIdx.x - st * nqb;
  }
  const int qb = nqb - 1 - qidx;
  const int kvh = st % Hkv, b = st / Hkv, h = kvh * G + w % G;
  const int q0 = qb * QRW + (w / G) * QR;                // this wave's first query row
  const int nblk = min((qb * QRW + QRW - 1) / kKvb + 1, (T + kKvb - 1) / kKvb);
  const int64_t kv_ld = (int64_t)Hkv * kDh;
  const E* kbase = kc + ((int64_t)b * cache_len * Hkv + kvh) * kDh;
  const E* vbase = vc + ((int64_t)b * cache_len * Hkv + kvh) * kDh;

  auto issue = [&](int j) {
    const int nb = BF ? (j & 1) : 0;
    if constexpr (BF) {
      copy_tile<528>(kbase + (int64_t)j * kKvb * kv_ld, kv_ld, T - j * kKvb, sm.K[nb], w, NWV);
      copy_tile<544>(vbase + (int64_t)j * kKvb * kv_ld, kv_ld, T - j * kKvb, sm.V[nb], w, NWV);
    }
  };

  // Q fragments (B operand of S^T = K Q^T): rows q0 + 16qt + r, all 256 channels
  Fr<E> Qf[QT][NKB];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = min(q0 + 16 * qt + r, T - 1);
    const E* qrow = qr + (((int64_t)b * T + row) * Hq + h) * kDh;
    if constexpr (BF) {
      // natural K order (slot j = channel 32 kb + 8g + j), as the K tile reads
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        Qf[qt][kb] = *reinterpret_cast<const bf16x8*>(qrow + KB * kb + 8 * g);
    } else {
      const Glb<E> qm{qrow, 0, 1};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) Qf[qt][kb] = qm.rm(0, KB * kb);
    }
  }
  f32x4 O[QT][16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) O[qt][dt] = zero4();
  float m[QT], lsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) { m[qt] = -INFINITY; lsum[qt] = 0.f; }

  // The Q fragments are first used inside the block loop, whose waits for the
  // copies are inline asm the compiler cannot see: left pending, their loads
  // would make it wait for every outstanding copy (vmcnt(0)) at the first
  // score product of every block.  An empty use here retires them once.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) asm volatile("" ::"v"(Qf[qt][kb]));
  if constexpr (BF) {
    issue(0);
    wait_copies();
    barrier_lds();
  }
  for (int j = 0; j < nblk; ++j) {
    const int nb = BF ? (j & 1) : 0;
    if constexpr (BF) {
      if (j + 1 < nblk) issue(j + 1);
    } else {
      __syncthreads();
      stage_rows<E, kDh, kKvb>(Lds<E, kDh>{reinterpret_cast<E*>(sm.K[0])},
                               kbase + (int64_t)j * kKvb * kv_ld, kv_ld, T - j * kKvb, 64 * NWV);
      stage_rows<E, kDh, kKvb>(Lds<E, kDh>{reinterpret_cast<E*>(sm.V[0])},
                               vbase + (int64_t)j * kKvb * kv_ld, kv_ld, T - j * kKvb, 64 * NWV);
      __syncthreads();
    }
    const Lane ln = lane_here();
    const auto Ks = [&]() {
      if constexpr (BF) return KTile{sm.K[nb]};
      else return Lds<E, kDh>{reinterpret_cast<E*>(sm.K[nb])};
    }();
    const auto Vs = [&]() {
      if constexpr (BF) return VTile{sm.V[nb]};
      else return Lds<E, kDh>{reinterpret_cast<E*>(sm.V[nb])};
    }();
    // S^T tiles: rows keys 64j + 16kt + 4g + i, column query q0 + 16qt + r
    f32x4 S[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) S[qt][kt] = zero4();
    // K fragments software-pipelined one channel block ahead: the reads of
    // block kb + 1 are in flight while block kb's MFMAs issue
    auto kfrag = [&](int kt, int kb) {
      if constexpr (BF) return Ks.rm8(16 * kt, KB * kb, ln);
      else return Ks.rm(16 * kt + ln.r, KB * kb, ln);
    };
    Fr<E> cur[4], nxt[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) cur[kt] = kfrag(kt, 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb + 1 < NKB) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) nxt[kt] = kfrag(kt, kb + 1);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) S[qt][kt] = mma(S[qt][kt], cur[kt], Qf[qt][kb]);
      if (kb + 1 < NKB) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) cur[kt] = nxt[kt];
      }
    }
    const bool diag = kKvb * j + kKvb - 1 > q0;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int qi = q0 + 16 * qt + r;
      float mb = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = S[qt][kt][i];
          if (diag && kKvb * j + 16 * kt + 4 * g + i > qi) s = -INFINITY;
          S[qt][kt][i] = s;
          mb = fmaxf(mb, s);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const float mn = fmaxf(m[qt], mb);
      const float al = hw_exp2(m[qt] - mn);
      m[qt] = mn;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = hw_exp2(S[qt][kt][i] - mn);
          S[qt][kt][i] = pv;
          ps += pv;
        }
      lsum[qt] = lsum[qt] * al + ps;
      // rescale O only when some lane's running max moved (rare after the
      // first blocks)
      if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) O[qt][dt] *= al;
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < kKvb / KB; ++kb) {
      Fr<E> pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) pf[qt] = acc_frag<E>(S[qt], kb);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        Fr<E> a;
        if constexpr (BF) a = Vs.cm(16 * dt, KB * kb, ln);
        else a = Vs.cm(16 * dt + ln.r, KB * kb, ln);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) O[qt][dt] = mma(O[qt][dt], a, pf[qt]);
      }
    }
    if constexpr (BF) {
      wait_copies();
      barrier_lds();
    }
  }
  // normalise, gate, store: lane (r, g) holds channels 16dt + 4g .. +3 of query r
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float lt = lsum[qt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = 1.f / lt;
    const int qi = q0 + 16 * qt + r;
    if (qi < T) {
      const int64_t base = (((int64_t)b * T + qi) * Hq + h) * kDh;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const int ch = 16 * dt + 4 * g;
        f32x4 gv;
        if constexpr (BF) {
          const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(gate + base + ch);
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i] = (float)g4[i];
        } else {
          gv = *reinterpret_cast<const f32x4*>(gate + base + ch);
        }
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = O[qt][dt][i] * inv / (1.f + __expf(-gv[i]));
        store4(o + base + ch, y);
      }
    }
  }
}

// ------------------------------------------------------------ decode
// Partials: m, l [B][Hq][ns], O [B][Hq][ns][256] fp32.  Wave w owns output
// channels 64w .. 64w+63; every wave forms the same scores of the block (the
// kernel is bound by the cache read, not by the matrix units), so the waves
// never exchange anything.
template <typename E>
struct DecSmem {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int NB = BF ? 2 : 1;
  static constexpr int KB_ = BF ? KTileD::kBytes : Lds<E, kDh>::size(kDkb) * (int)sizeof(E);
  static constexpr int VB_ = BF ? VTileD::kBytes : Lds<E, kDh>::size(kDkb) * (int)sizeof(E);
  alignas(16) char K[NB][KB_];
  alignas(16) char V[NB][VB_];
};

template <typename E>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const E* __restrict__ qr, const E* __restrict__ kc, const E* __restrict__ vc,
    const int32_t* __restrict__ pos, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int cache_len, int Hq, int Hkv, int ns, int spl) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int KB = FragOf<E>::KB, NKB = kDh / KB;
  __shared__ DecSmem<E> sm;
  const int G = Hq / Hkv;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), r = l & 15, g = l >> 4;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int n = min(max(pos[b], 0), cache_len - 1) + 1;   // keys 0 .. pos inclusive
  const int k0 = s * spl, k1 = min(n, k0 + spl);
  const size_t pidx = ((size_t)b * Hq + kvh * G) * ns + s;  // head kvh*G, split s
  if (k0 >= k1) {
    // empty split: a neutral partial
    if (threadIdx.x < G) {
      pm[pidx + (size_t)threadIdx.x * ns] = -INFINITY;
      pl[pidx + (size_t)threadIdx.x * ns] = 0.f;
    }
    return;
  }
  const int64_t kv_ld = (int64_t)Hkv * kDh;
  const E* kbase = kc + ((int64_t)b * cache_len * Hkv + kvh) * kDh;
  const E* vbase = vc + ((int64_t)b * cache_len * Hkv + kvh) * kDh;
  const int nblk = (k1 - k0 + kDkb - 1) / kDkb;

  auto issue = [&](int j) {
    if constexpr (BF) {
      const int kb0 = k0 + j * kDkb;
      copy_tile<528, kDkb>(kbase + (int64_t)kb0 * kv_ld, kv_ld, k1 - kb0, sm.K[j & 1], w, 4);
      copy_tile<544, kDkb>(vbase + (int64_t)kb0 * kv_ld, kv_ld, k1 - kb0, sm.V[j & 1], w, 4);
    }
  };

  // query fragments: lane column r = head kvh*G + r (zero beyond the group)
  Fr<E> Qf[NKB];
  {
    const bool ok = r < G;
    const E* qrow = qr + ((int64_t)b * Hq + kvh * G + (ok ? r : 0)) * kDh;
    if constexpr (BF) {
      // natural K order, as the K tile reads
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Qf[kb] = *reinterpret_cast<const bf16x8*>(qrow + KB * kb + 8 * g);
        if (!ok) Qf[kb] = bf16x8{};
      }
    } else {
      const Glb<E> qm{qrow, 0, ok ? 1 : 0};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) Qf[kb] = qm.rm(0, KB * kb);
    }
  }
  f32x4 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = zero4();
  float m = -INFINITY, lsum = 0.f;

  if constexpr (BF) {
    issue(0);
    wait_copies();
    barrier_lds();
  }
  for (int j = 0; j < nblk; ++j) {
    const int kb0 = k0 + j * kDkb;
    if constexpr (BF) {
      if (j + 1 < nblk) issue(j + 1);
    } else {
      __syncthreads();
      stage_rows<E, kDh, kDkb>(Lds<E, kDh>{reinterpret_cast<E*>(sm.K[0])},
                               kbase + (int64_t)kb0 * kv_ld, kv_ld, k1 - kb0, 256);
      stage_rows<E, kDh, kDkb>(Lds<E, kDh>{reinterpret_cast<E*>(sm.V[0])},
                               vbase + (int64_t)kb0 * kv_ld, kv_ld, k1 - kb0, 256);
      __syncthreads();
    }
    const int nb = BF ? (j & 1) : 0;
    const Lane ln = lane_here();
    const auto Ks = [&]() {
      if constexpr (BF) return KTileD{sm.K[nb]};
      else return Lds<E, kDh>{reinterpret_cast<E*>(sm.K[nb])};
    }();
    const auto Vs = [&]() {
      if constexpr (BF) return VTileD{sm.V[nb]};
      else return Lds<E, kDh>{reinterpret_cast<E*>(sm.V[nb])};
    }();
    // S^T: rows keys kb0 + 16kt + 4g + i, column head r
    constexpr int NKT = kDkb / 16;
    f32x4 S[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) S[kt] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        if constexpr (BF) S[kt] = mma(S[kt], Ks.rm8(16 * kt, KB * kb, ln), Qf[kb]);
        else S[kt] = mma(S[kt], Ks.rm(16 * kt + r, KB * kb, ln), Qf[kb]);
      }
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = S[kt][i];
        if (kb0 + 16 * kt + 4 * g + i >= k1) sv = -INFINITY;
        S[kt][i] = sv;
        mb = fmaxf(mb, sv);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(m, mb);           // finite: every block holds a valid key
    const float al = hw_exp2(m - mn);
    m = mn;
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = hw_exp2(S[kt][i] - mn);
        S[kt][i] = pv;
        ps += pv;
      }
    lsum = lsum * al + ps;
    if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] *= al;
    }
#pragma unroll
    for (int kb = 0; kb < kDkb / KB; ++kb) {
      const Fr<E> pf = acc_frag<E>(S, kb);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        if constexpr (BF) O[dt] = mma(O[dt], Vs.cm(64 * w + 16 * dt, KB * kb, ln), pf);
        else O[dt] = mma(O[dt], Vs.cm(64 * w + 16 * dt + r, KB * kb, ln), pf);
      }
    }
    if constexpr (BF) {
      wait_copies();
      barrier_lds();
    }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  // lane (r, g) holds channels 64w + 16dt + 4g .. +3 of head column r
  if (r < G) {
    const size_t pi = pidx + (size_t)r * ns;
    float* dst = po + pi * kDh + 64 * w;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt + 4 * g) = O[dt];
    if (w == 0 && g == 0) {
      pm[pi] = m;
      pl[pi] = lsum;
    }
  }
}

// One wave per (sequence, query head): merge the splits, normalise, gate.
template <typename E>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float* __restrict__ pm, const float* __restrict__ pl, const float* __restrict__ po,
    const E* __restrict__ gate, E* __restrict__ o, int rows, int ns) {
  const int row = blockIdx.x * 4 + wave_id(), l = lane_id();
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, pm[(size_t)row * ns + s]);
  float lt = 0.f;
  f32x4 acc = zero4();
  for (int s = 0; s < ns; ++s) {
    const float ms = pm[(size_t)row * ns + s];
    if (ms == -INFINITY) continue;
    const float sc = hw_exp2(ms - mx);
    lt += sc * pl[(size_t)row * ns + s];
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(po + ((size_t)row * ns + s) * kDh + 4 * l);
    acc += sc * v4;
  }
  const float inv = 1.f / lt;
  f32x4 gv;
  if constexpr (sizeof(E) == 2) {
    const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(gate + (size_t)row * kDh + 4 * l);
#pragma unroll
    for (int i = 0; i < 4; ++i) gv[i] = (float)g4[i];
  } else {
    gv = *reinterpret_cast<const f32x4*>(gate + (size_t)row * kDh + 4 * l);
  }
  f32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = acc[i] * inv / (1.f + __expf(-gv[i]));
  store4(o + (size_t)row * kDh + 4 * l, y);
}

}  // namespace attn

// Decode split: about two workgroups per CU over the (sequence, key/value head)
// streams, splits a multiple of 32 keys.
int attn_decode_split(int B, int Hkv, int cache_len) {
  const int64_t streams = (int64_t)B * Hkv;
  int64_t ns = (512 + streams - 1) / streams;
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, (cache_len + 31) / 32));
  const int64_t spl = ((cache_len + ns - 1) / ns + 31) / 32 * 32;
  return (int)spl;
}
int attn_decode_splits(int B, int Hkv, int cache_len) {
  const int spl = attn_decode_split(B, Hkv, cache_len);
  return (cache_len + spl - 1) / spl;
}

template <typename E>
static hipError_t attn_launch_t(const AttnLaunch& a, hipStream_t st) {
  using namespace attn;
  const int64_t ntok = a.decode ? a.B : (int64_t)a.B * a.T;
  hipLaunchKernelGGL((attn_prep_kernel<E>), dim3((unsigned)ntok), dim3(64 * kPrepWaves), 0, st,
                     (const E*)a.q, (const E*)a.k, (const E*)a.v, a.qw, a.kw, a.eps, a.rope_dim,
                     a.rope_dim > 0 ? std::pow((double)a.theta, -2.0 / a.rope_dim) : 1.0,
                     a.decode ? a.pos : nullptr, (E*)a.qrot, (E*)a.kc, (E*)a.vc_write, ntok,
                     a.decode ? 1 : a.T, a.cache_len, a.Hq, a.Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  if (!a.decode) {
    // bf16: two waves per query head (32 query rows per workgroup) while the
    // workgroup fits the 768-thread instantiation (up to 6 heads per group);
    // otherwise, and for fp32, one wave per head (16 rows, at most 8 heads).
    auto launch = [&](auto kern, int qs, int max_threads) -> hipError_t {
      const int threads = 64 * G * qs;
      if (threads > max_threads) return hipErrorInvalidConfiguration;
      const int nqb = (a.T + 16 * qs - 1) / (16 * qs);
      const int nst = a.Hkv * a.B;
      const int nwg = (nst <= 8 && 8 % nst == 0) ? 8 * ((nqb + 8 / nst - 1) / (8 / nst))
                                                 : nqb * nst;
      hipLaunchKernelGGL(kern, dim3(nwg), dim3(threads), 0, st, (const E*)a.qrot,
                         (const E*)a.kc, (const E*)a.vc_read, (const E*)a.gate, (E*)a.o, a.T,
                         a.cache_len, a.Hq, a.Hkv, nqb, a.B);
      return hipGetLastError();
    };
    if constexpr (sizeof(E) == 2) {
      if (64 * G * 2 <= fwd_max_threads<2>())
        return launch(attn_fwd_kernel<E, 1, 2>, 2, fwd_max_threads<2>());
    }
    return launch(attn_fwd_kernel<E, 1, 1>, 1, fwd_max_threads<1>());
  }
  const int spl = attn_decode_split(a.B, a.Hkv, a.cache_len);
  const int ns = attn_decode_splits(a.B, a.Hkv, a.cache_len);
  hipLaunchKernelGGL((attn_decode_kernel<E>), dim3(ns, a.Hkv, a.B), dim3(256), 0, st,
                     (const E*)a.qrot, (const E*)a.kc,
                     (const E*)a.vc_read, a.pos, a.pm, a.pl, a.po, a.cache_len, a.Hq, a.Hkv, ns,
                     spl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int crow = a.B * a.Hq;
  hipLaunchKernelGGL((attn_combine_kernel<E>), dim3((crow + 3) / 4), dim3(256), 0, st, a.pm, a.pl,
                     a.po, (const E*)a.gate, (E*)a.o, crow, ns);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnLaunch& a, hipStream_t st) {
  return a.bf16_io ? attn_launch_t<bf16>(a, st) : attn_launch_t<float>(a, st);
}

}  // namespace gdn

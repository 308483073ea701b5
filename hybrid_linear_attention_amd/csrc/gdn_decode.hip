// Decode step: one token per sequence, state read and rewritten in place.
//
// One step of the recurrence (page "Inside Qwen3.8-27B: Hybrid DeltaNet
// Architecture, 256k Context, and 24GB Local Serving", section "Gated DeltaNet
// Mechanics"; at inference the state advances token by token, per the note
// under "The Role of Periodic Gated Attention"):
//
//   S' = alpha S (I - beta k k^T) + beta v k^T,   o = S' q
//
// Row i of S (a value row, 128 floats) evolves alone, from the OLD row:
//   u_i = S_i . k,  p_i = S_i . q,  d_i = beta (v_i - alpha u_i)
//   S'_i = alpha S_i + d_i k,       o_i = alpha p_i + d_i (k . q)
//
// The step moves 2 x 64 KiB of fp32 state per (sequence, value head) and does
// ~6 flops per state element, so it is bound by HBM bandwidth.  Layout of the
// work: one 256-thread workgroup per (sequence, value head); 8 lanes share one
// state row, each lane owning 4 float4 column groups (columns 4*l8 + 32*i), so
// every load/store instruction of a wave covers 8 full 128-byte row segments.
// Each thread keeps 16 float4 (4 rows) in flight; dot products are reduced
// across the 8 lanes of a row with xor shuffles.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <typename E>
__device__ __forceinline__ f32x4 load4(const E* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Sum over the 8 lanes of an aligned group, by a butterfly over xor 1, 2, 4.
__device__ __forceinline__ float sum8(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  return x;
}

// The same sum by DPP lane exchange within rows (a VALU operand modifier, no
// LDS round trip): quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2),
// then row_half_mirror (lane i of each 8-lane half takes lane 7 - i).  After
// the two quad steps every lane holds its quad's sum, and the mirror adds the
// other quad's, so each lane ends with q0 + q1 or q1 + q0: the value the
// butterfly gives.  Used where several reductions per token sit between the
// state loads and the stores (the multi-token kernel: 3 tokens x 64
// sequences, 0.109 -> 0.103 ms per verify + commit round); in the one-token
// kernels the shuffles' latency is hidden and DPP measured 1 % slower.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float sum8_dpp(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x;
}

__device__ __forceinline__ float dot4(const f32x4& a, const f32x4& b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

template <typename E>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ state, E* __restrict__ o, int Hqk, int Hv, int G) {
  const int bh = blockIdx.x;             // b * Hv + h
  const int b = bh / Hv, h = bh - (bh / Hv) * Hv;
  const int gq = h / G;                  // query/key head read by value head h
  const int tid = threadIdx.x;
  const int l8 = tid & 7;                // lane within the row's 8-lane group
  const int rg = tid >> 3;               // 0..31: row within one pass

  const E* qp = q + ((size_t)b * Hqk + gq) * kD;
  const E* kp = k + ((size_t)b * Hqk + gq) * kD;
  float* S = state + (size_t)bh * kD * kD;

  // Issue the state loads first: 4 rows x 4 float4 per thread.
  f32x4 s[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[p][i] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(S + (rg + 32 * p) * kD + 4 * l8 + 32 * i));

  f32x4 kr[4], qr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kr[i] = load4<E>(kp + 4 * l8 + 32 * i);
    qr[i] = load4<E>(qp + 4 * l8 + 32 * i);
  }
  const float a = alpha[bh], be = beta[bh];
  float vr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) vr[p] = to_f32(v[(size_t)bh * kD + rg + 32 * p]);

  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) kq += dot4(kr[i], qr[i]);
  kq = sum8(kq);

#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float u = 0.f, pq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u += dot4(s[p][i], kr[i]);
      pq += dot4(s[p][i], qr[i]);
    }
    u = sum8(u);
    pq = sum8(pq);
    const float d = be * (vr[p] - a * u);
    const int row = rg + 32 * p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 n;
      n[0] = a * s[p][i][0] + d * kr[i][0];
      n[1] = a * s[p][i][1] + d * kr[i][1];
      n[2] = a * s[p][i][2] + d * kr[i][2];
      n[3] = a * s[p][i][3] + d * kr[i][3];
      __builtin_nontemporal_store(n, reinterpret_cast<f32x4*>(S + row * kD + 4 * l8 + 32 * i));
    }
    if (l8 == 0) o[(size_t)bh * kD + row] = from_f32<E>(a * pq + d * kq);
  }
}

// The same step with the state stored as bfloat16 (the footprint the pages
// count in BF16): 32 KiB per (sequence, value head) read and written, the
// arithmetic in fp32, the new row rounded to nearest even.  Each lane owns two
// runs of 8 columns (8*l8 + 64*i .. +7), so every access is 16 bytes and the 8
// lanes of a row cover it in two 128-byte segments.
template <typename E>
__global__ __launch_bounds__(256) void decode_step_bs_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    bf16* __restrict__ state, E* __restrict__ o, int Hqk, int Hv, int G) {
  const int bh = blockIdx.x;
  const int b = bh / Hv, h = bh - (bh / Hv) * Hv;
  const int gq = h / G;
  const int tid = threadIdx.x;
  const int l8 = tid & 7;
  const int rg = tid >> 3;

  const E* qp = q + ((size_t)b * Hqk + gq) * kD;
  const E* kp = k + ((size_t)b * Hqk + gq) * kD;
  bf16* S = state + (size_t)bh * kD * kD;

  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 s[4][2];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      s[p][i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(S + (rg + 32 * p) * kD + 8 * l8 + 64 * i));

  float kr[2][8], qr[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x4 k0 = load4<E>(kp + 8 * l8 + 64 * i), k1 = load4<E>(kp + 8 * l8 + 64 * i + 4);
    const f32x4 q0 = load4<E>(qp + 8 * l8 + 64 * i), q1 = load4<E>(qp + 8 * l8 + 64 * i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kr[i][j] = k0[j]; kr[i][4 + j] = k1[j];
      qr[i][j] = q0[j]; qr[i][4 + j] = q1[j];
    }
  }
  const float a = alpha[bh], be = beta[bh];
  float vr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) vr[p] = to_f32(v[(size_t)bh * kD + rg + 32 * p]);

  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) kq += kr[i][j] * qr[i][j];
  kq = sum8(kq);

#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float sf[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16x8 sv = *reinterpret_cast<const bf16x8*>(&s[p][i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) sf[i][j] = (float)sv[j];
    }
    float u = 0.f, pq = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u += sf[i][j] * kr[i][j];
        pq += sf[i][j] * qr[i][j];
      }
    u = sum8(u);
    pq = sum8(pq);
    const float d = be * (vr[p] - a * u);
    const int row = rg + 32 * p;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      bf16x8 n;
#pragma unroll
      for (int j = 0; j < 8; ++j) n[j] = (bf16)(a * sf[i][j] + d * kr[i][j]);
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&n),
                                  reinterpret_cast<u32x4*>(S + row * kD + 8 * l8 + 64 * i));
    }
    if (l8 == 0) o[(size_t)bh * kD + row] = from_f32<E>(a * pq + d * kq);
  }
}

// Speculative decoding with n drafted tokens per sequence (the MTP heads of
// page "Inside Qwen3.8-27B ...", section "Multi-Token Prediction (MTP)",
// draft tokens t+1 and t+2).  VERIFY: outputs of all n tokens from the state,
// which is read but not written.  COMMIT: the state advanced in place by the
// first m = clamp(n_accept[b], 0, n) tokens; q and o are not used.  The n
// tokens' q, k, v, alpha, beta are first staged in LDS (as float32) so their
// loads overlap the state's; then every thread applies the n steps to its 4
// rows in registers, exactly as decode_step_kernel does for one.
template <typename E, bool VERIFY>
__global__ __launch_bounds__(256) void decode_multi_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ state,
    const int32_t* __restrict__ n_accept, E* __restrict__ o, int n, int Hqk, int Hv, int G) {
  __shared__ float sk[kMaxDraft][kD], sq[kMaxDraft][kD], sv[kMaxDraft][kD];
  __shared__ float sa[kMaxDraft], sbt[kMaxDraft];
  const int bh = blockIdx.x;
  const int b = bh / Hv, h = bh - (bh / Hv) * Hv;
  const int gq = h / G;
  const int tid = threadIdx.x;
  const int l8 = tid & 7;
  const int rg = tid >> 3;
  const int m = VERIFY ? n : min(max(n_accept[b], 0), n);
  float* S = state + (size_t)bh * kD * kD;

  f32x4 s[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[p][i] = *reinterpret_cast<const f32x4*>(S + (rg + 32 * p) * kD + 4 * l8 + 32 * i);

  for (int e = tid; e < m * kD; e += 256) {
    const int t = e / kD, c = e - (e / kD) * kD;
    const size_t tk = ((size_t)b * n + t) * Hqk + gq, tv = ((size_t)b * n + t) * Hv + h;
    sk[t][c] = to_f32(k[tk * kD + c]);
    if (VERIFY) sq[t][c] = to_f32(q[tk * kD + c]);
    sv[t][c] = to_f32(v[tv * kD + c]);
    if (c == 0) {
      sa[t] = alpha[tv];
      sbt[t] = beta[tv];
    }
  }
  __syncthreads();

  for (int t = 0; t < m; ++t) {
    f32x4 kr[4], qr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = *reinterpret_cast<const f32x4*>(&sk[t][4 * l8 + 32 * i]);
      if (VERIFY) qr[i] = *reinterpret_cast<const f32x4*>(&sq[t][4 * l8 + 32 * i]);
    }
    const float a = sa[t], be = sbt[t];
    float kq = 0.f;
    if (VERIFY) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kq += dot4(kr[i], qr[i]);
      kq = sum8_dpp(kq);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = rg + 32 * p;
      float u = 0.f, pq = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u += dot4(s[p][i], kr[i]);
        if (VERIFY) pq += dot4(s[p][i], qr[i]);
      }
      u = sum8_dpp(u);
      const float d = be * (sv[t][row] - a * u);
      // verify never writes the state: the last token's update has no reader
      if (!VERIFY || t + 1 < m) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) s[p][i][j] = a * s[p][i][j] + d * kr[i][j];
      }
      if (VERIFY) {
        pq = sum8_dpp(pq);
        if (l8 == 0) o[(((size_t)b * n + t) * Hv + h) * kD + row] = from_f32<E>(a * pq + d * kq);
      }
    }
  }
  if (!VERIFY && m > 0) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(S + (rg + 32 * p) * kD + 4 * l8 + 32 * i) = s[p][i];
  }
}

hipError_t launch_decode_multi(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, float* state, const int32_t* n_accept,
                               void* o, int B, int n, int Hqk, int Hv, bool bf16_io,
                               bool verify, hipStream_t stream) {
  const int G = Hv / Hqk;
  dim3 grid((unsigned)(B * Hv)), block(256);
  if (bf16_io) {
    if (verify)
      hipLaunchKernelGGL((decode_multi_kernel<bf16, true>), grid, block, 0, stream,
                         (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta, state,
                         n_accept, (bf16*)o, n, Hqk, Hv, G);
    else
      hipLaunchKernelGGL((decode_multi_kernel<bf16, false>), grid, block, 0, stream,
                         (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta, state,
                         n_accept, (bf16*)o, n, Hqk, Hv, G);
  } else {
    if (verify)
      hipLaunchKernelGGL((decode_multi_kernel<float, true>), grid, block, 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, alpha, beta, state,
                         n_accept, (float*)o, n, Hqk, Hv, G);
    else
      hipLaunchKernelGGL((decode_multi_kernel<float, false>), grid, block, 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, alpha, beta, state,
                         n_accept, (float*)o, n, Hqk, Hv, G);
  }
  return hipGetLastError();
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta, void* state,
                              void* o, int B, int Hqk, int Hv, bool bf16_io, bool state_bf16,
                              hipStream_t stream) {
  const int G = Hv / Hqk;
  dim3 grid((unsigned)(B * Hv)), block(256);
  if (state_bf16) {
    if (bf16_io)
      hipLaunchKernelGGL(decode_step_bs_kernel<bf16>, grid, block, 0, stream,
                         (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta,
                         (bf16*)state, (bf16*)o, Hqk, Hv, G);
    else
      hipLaunchKernelGGL(decode_step_bs_kernel<float>, grid, block, 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, alpha, beta,
                         (bf16*)state, (float*)o, Hqk, Hv, G);
  } else if (bf16_io) {
    hipLaunchKernelGGL(decode_step_kernel<bf16>, grid, block, 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta,
                       (float*)state, (bf16*)o, Hqk, Hv, G);
  } else {
    hipLaunchKernelGGL(decode_step_kernel<float>, grid, block, 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, alpha,
                       beta, (float*)state, (float*)o, Hqk, Hv, G);
  }
  return hipGetLastError();
}

}  // namespace gdn

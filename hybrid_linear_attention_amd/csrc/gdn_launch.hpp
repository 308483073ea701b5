// Host <-> kernel interface shared by the launch code and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Where chunk `cid` lives.  Fixed-length batches compute it; packed varlen
// batches read a table built on the device from cu_seqlens.
struct ChunkMap {
  const int32_t* tab;      // varlen: [nc_max][2] {first token, length}; null otherwise
  const int32_t* seq_off;  // varlen: [N+1] first chunk of each sequence
  int T, Nc;               // fixed-length: tokens and chunks per sequence
  int nc_max;              // chunks the workspace holds
};

struct PrefillLaunch {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const void* h0;          // [nseq][Hv][128][128], float32 or bfloat16 (state_bf16)
  void* o;
  void* ht;
  const void* gate;        // null: plain output; else fused RMSNorm * sigmoid(gate)
  const float* norm_w;
  float norm_eps;
  void *Tt, *M;            // workspace regions
  float *gam, *dec;
  ChunkMap cm;
  int nseq, nc_launch, Hqk, Hv;
  int64_t ntok;            // all tokens of the call (B * T, or T_tot)
  bool bf16_io;
  bool state_bf16;         // h0 / ht stored as bfloat16
  bool solve_only;         // prepare for the backward pass: also N = (I + A)^-1, all blocks
  void* N;                 // solve_only: where N goes
  void* states;            // bf16 scan: state entering every chunk (backward pass), or null
};

// Backward pass of a prefill: B sequences of T tokens, or N packed sequences.
struct BackwardLaunch {
  const void *q, *k, *v, *dout;
  const float *alpha, *beta;
  const float *h0, *dht;   // [B][Hv][128][128] float32, or null (zeros)
  void *dq, *dk, *dv;
  float *dalpha, *dbeta;
  float* dh0;              // or null (not written)
  void *N, *M, *S, *dS;    // workspace: prepare's solve and mask, chunk states, state grads
  float *gam, *dec;
  ChunkMap cm;             // where each chunk lives (fixed length, or the packed table)
  int nseq, nc;            // sequences (h0/dht/dh0 rows) and chunk slots
  int Hqk, Hv;
  bool bf16_io;
  bool states_ready;       // S already written (by the bf16 forward scan)
};
hipError_t launch_backward(const BackwardLaunch& a, hipStream_t st);

// Gated attention layer (prefill of B sequences of T tokens from position 0,
// or one decode token per sequence at position pos[b]).
struct AttnLaunch {
  const void *q, *k, *v, *gate;
  const float *qw, *kw;      // QK-Norm weights, or null (ones)
  float eps, theta;
  int rope_dim;
  const int32_t* pos;        // decode: [B] positions (cached keys per sequence)
  void* qrot;                // workspace: normalised, rotated queries
  void* kc;                  // keys after norm and rotation [B][cache_len][Hkv][256]
  void* vc_write;            // value cache to fill (or null: values read from v)
  const void* vc_read;       // values the attention reads [B][cache_len][Hkv][256]
  void* o;
  float *pm, *pl, *po;       // decode split partials (workspace)
  int B, T, cache_len, Hq, Hkv;
  bool decode, bf16_io;
};
hipError_t launch_attention(const AttnLaunch& a, hipStream_t st);
int attn_decode_split(int B, int Hkv, int cache_len);
int attn_decode_splits(int B, int Hkv, int cache_len);

hipError_t launch_prepare(const PrefillLaunch& a, hipStream_t st);
hipError_t launch_scan(const PrefillLaunch& a, hipStream_t st);
hipError_t launch_varlen_table(const int32_t* cu, int N, int T_tot, int nc_max, int32_t* tab,
                               int32_t* seq_off, hipStream_t st);
// Most drafted tokens a verify or commit call takes per sequence.
constexpr int kMaxDraft = 8;

hipError_t launch_decode_multi(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, float* state, const int32_t* n_accept,
                               void* o, int B, int n, int Hqk, int Hv, bool bf16_io,
                               bool verify, hipStream_t stream);
hipError_t launch_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, void* state, void* o, int B, int Hqk, int Hv,
                              bool bf16_io, bool state_bf16, hipStream_t stream);

}  // namespace gdn

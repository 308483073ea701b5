// Host side of the C ABI declared in include/gdn.h: argument checks (all of
// them before anything is enqueued), workspace layout, and launches on the
// caller's stream.  No allocation, no synchronisation, no global mutable state
// beyond the thread-local last-error code and the per-device address of the
// static scratch array of gdn_prefill_chunked_noalloc (set once per device).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdlib.h>

#include "gdn.h"
#include "gdn_device.hpp"
#include "gdn_launch.hpp"


namespace {

thread_local int g_last_hip = 0;

// Largest element count accepted for one tensor (keeps every int index the
// kernels form far from overflow; a [T, 48, 128] tensor at this limit has
// 2^26 tokens).
constexpr int64_t kMaxElems = int64_t(1) << 38;

struct Range {
  uintptr_t lo, hi;   // [lo, hi); empty when lo == hi
};

Range span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, p ? a + (uintptr_t)bytes : a};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t esize(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout: Tt [nc][Hv][64][64] and M [nc][Hv][64][64] (element
// type), gam and dec [nc][Hv][64] fp32, then
// for varlen the chunk table [nc][2] and the per-sequence chunk offsets [N+1]
// (int32).
struct WsLayout {
  size_t tt, m, gam, dec, tab, seq, total;
};

WsLayout ws_layout(int64_t nc, int64_t Hqk, int64_t Hv, gdn_dtype dt, int64_t nseq_varlen) {
  WsLayout w{};
  const size_t es = esize(dt);
  size_t off = 0;
  w.tt = off;
  off += round256((size_t)nc * Hv * gdn::kC * gdn::kC * es);
  w.m = off;
  off += round256((size_t)nc * Hv * gdn::kC * gdn::kC * es);
  w.gam = off;
  off += round256((size_t)nc * Hv * gdn::kC * sizeof(float));
  w.dec = off;
  off += round256((size_t)nc * Hv * gdn::kC * sizeof(float));
  w.tab = off;
  w.seq = off;
  if (nseq_varlen >= 0) {
    off += round256((size_t)nc * 2 * sizeof(int32_t));
    w.seq = off;
    off += round256((size_t)(nseq_varlen + 1) * sizeof(int32_t));
  }
  w.total = off;
  return w;
}

gdn_status check_dims(int64_t H_qk, int64_t H_v, int64_t D, gdn_dtype dt) {
  if (H_qk <= 0 || H_v <= 0 || D <= 0) return GDN_ERR_SHAPE;
  if (H_v % H_qk != 0) return GDN_ERR_SHAPE;
  if (D != gdn::kD) return GDN_ERR_UNSUPPORTED;
  if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (H_v > 4096) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn_status fail_hip(hipError_t e) {
  if (e == hipSuccess) return GDN_OK;
  g_last_hip = (int)e;
  return GDN_ERR_HIP;
}

// Checks shared by the packed and fixed-length prefill.  ntok = all tokens,
// nseq = number of states, ses = bytes per state element (4: float32, 2: bf16).
gdn_status check_prefill(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const void* h0, const void* o, const void* ht,
                         const void* gate, const float* norm_w, const void* cu, int64_t cu_len,
                         int64_t ntok, int64_t nseq, int64_t H_qk, int64_t H_v, gdn_dtype dt,
                         const void* workspace, size_t workspace_bytes, size_t need,
                         int64_t ses) {
  const int64_t es = (int64_t)esize(dt);
  const int64_t D = gdn::kD;
  if (ntok > 0 && (!q || !k || !v || !alpha || !beta || !o)) return GDN_ERR_NULL;
  if (ntok * H_v * D > kMaxElems || nseq * H_v * D * D > kMaxElems) return GDN_ERR_UNSUPPORTED;
  if (need > 0 && !workspace) return GDN_ERR_WORKSPACE;
  if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
  const void* p16[] = {q, k, v, o, h0, ht, gate, workspace};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  if (!aligned(alpha, 4) || !aligned(beta, 4) || !aligned(norm_w, 4) || !aligned(cu, 4))
    return GDN_ERR_ALIGN;

  const Range rq = span(q, ntok * H_qk * D * es), rk = span(k, ntok * H_qk * D * es);
  const Range rv = span(v, ntok * H_v * D * es), ro = span(o, ntok * H_v * D * es);
  const Range ra = span(alpha, ntok * H_v * 4), rb = span(beta, ntok * H_v * 4);
  const Range rh0 = span(h0, nseq * H_v * D * D * ses), rht = span(ht, nseq * H_v * D * D * ses);
  const Range rg = span(gate, gate ? ntok * H_v * D * es : 0);
  const Range rw = span(norm_w, norm_w ? D * 4 : 0);
  const Range rcu = span(cu, cu ? cu_len * 4 : 0);
  const Range rws = span(workspace, (int64_t)need);
  // o and the workspace may overlap nothing; ht may overlap nothing except
  // that it may be exactly h0 (in-place carry).
  const bool ht_in_place = ht && h0 && (const void*)ht == (const void*)h0;
  const Range inputs[] = {rq, rk, rv, ra, rb, rg, rw, rcu};
  for (const Range& in : inputs)
    if (overlap(ro, in) || overlap(rws, in) || overlap(rht, in)) return GDN_ERR_ALIAS;
  if (overlap(ro, rh0) || overlap(rws, rh0)) return GDN_ERR_ALIAS;
  if (!ht_in_place && overlap(rht, rh0)) return GDN_ERR_ALIAS;
  if (overlap(ro, rht) || overlap(ro, rws) || overlap(rht, rws)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

// Debug mode (environment GDN_DEBUG=1): the packed calls copy cu_seqlens to
// the host, synchronously on the caller's stream, and reject offsets that do
// not run from 0 to T_tot without decreasing.  Off by default: the calls
// then never read device memory on the host (the device-side chunk table
// clamps malformed offsets, so they cannot send a kernel out of bounds).
gdn_status debug_check_cu(const int32_t* cu, int32_t N, int32_t T_tot, void* stream) {
  const char* e = getenv("GDN_DEBUG");
  if (!e || e[0] != '1') return GDN_OK;
  int32_t* h = static_cast<int32_t*>(malloc(sizeof(int32_t) * ((size_t)N + 1)));
  if (!h) return GDN_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t he = hipMemcpyAsync(h, cu, sizeof(int32_t) * ((size_t)N + 1), hipMemcpyDeviceToHost, st);
  if (he == hipSuccess) he = hipStreamSynchronize(st);
  gdn_status s = fail_hip(he);
  if (s == GDN_OK) {
    bool ok = h[0] == 0 && h[N] == T_tot;
    for (int32_t n = 0; n < N && ok; ++n) ok = h[n] <= h[n + 1];
    if (!ok) s = GDN_ERR_SHAPE;
  }
  free(h);
  return s;
}

enum Phase { kCheckOnly = 0, kPrepare = 1, kScan = 2, kBoth = 3 };

gdn_status prefill_fixed(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const void* h0, void* o, void* ht, int32_t B,
                         int32_t T, int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                         void* workspace, size_t workspace_bytes, void* stream, int phase,
                         bool state_bf16) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (B < 0 || T < 0) return GDN_ERR_SHAPE;
  if (B > 65535) return GDN_ERR_UNSUPPORTED;
  const int64_t Nc = ((int64_t)T + gdn::kC - 1) / gdn::kC;
  const int64_t nc = (int64_t)B * Nc;
  if (nc > (int64_t(1) << 30)) return GDN_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(nc, H_qk, H_v, dt, -1);
  // kCheckOnly: every check but the workspace's
  const size_t need = (nc > 0 && phase != kCheckOnly) ? L.total : 0;
  s = check_prefill(q, k, v, alpha, beta, h0, o, ht, nullptr, nullptr, nullptr, 0,
                    (int64_t)B * T, B, H_qk, H_v, dt, workspace, workspace_bytes, need,
                    state_bf16 ? 2 : 4);
  if (s != GDN_OK || phase == kCheckOnly) return s;

  gdn::PrefillLaunch a{};
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.h0 = h0; a.o = o; a.ht = ht;
  a.gate = nullptr; a.norm_w = nullptr; a.norm_eps = 0.f;
  char* ws = static_cast<char*>(workspace);
  a.Tt = ws ? ws + L.tt : nullptr;
  a.M = ws ? ws + L.m : nullptr;
  a.gam = ws ? reinterpret_cast<float*>(ws + L.gam) : nullptr;
  a.dec = ws ? reinterpret_cast<float*>(ws + L.dec) : nullptr;
  a.cm = gdn::ChunkMap{nullptr, nullptr, T, (int)Nc, (int)nc};
  a.nseq = B;
  a.ntok = (int64_t)B * T;
  a.nc_launch = (int)nc;
  a.Hqk = H_qk; a.Hv = H_v;
  a.bf16_io = dt == GDN_BF16;
  a.state_bf16 = state_bf16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((phase & kPrepare) && nc > 0) {
    s = fail_hip(gdn::launch_prepare(a, st));
    if (s != GDN_OK) return s;
  }
  if (phase & kScan) {
    if (!ht && T == 0) return GDN_OK;
    s = fail_hip(gdn::launch_scan(a, st));
  }
  return s;
}

}  // namespace

// Workspace of gdn_prefill_chunked_noalloc: one copy per device, held from the
// code object's load until the process ends.  In host code `scratch` is only
// a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device (scratch_on below).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device that runs `stream` (the current
// device for the default stream).  The first call on a device looks the
// symbol up with that device current and restores the caller's device.
gdn_status scratch_on(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      int cur = 0;
      if ((e = hipGetDevice(&cur)) != hipSuccess) return fail_hip(e);
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return fail_hip(e);
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess) return fail_hip(e);
      if (!p) return fail_hip(hipErrorInvalidSymbol);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return 100; }

int gdn_last_hip_error(void) { return g_last_hip; }

const char* gdn_status_str(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: negative or inconsistent sizes";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: unsupported head dim, dtype or size";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: misaligned pointer";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps another buffer";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a HIP launch failed";
    case GDN_ERR_TOO_LARGE:
      return "GDN_ERR_TOO_LARGE: the call needs more workspace than the static scratch array "
             "of gdn_prefill_chunked_noalloc holds (GDN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown gdn_status";
  }
}

size_t gdn_prefill_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t D,
                                   gdn_dtype dt) {
  if (check_dims(H_qk, H_v, D, dt) != GDN_OK || B < 0 || T < 0) return 0;
  const int64_t nc = (int64_t)B * (((int64_t)T + gdn::kC - 1) / gdn::kC);
  if (nc == 0) return 0;
  return ws_layout(nc, H_qk, H_v, dt, -1).total;
}

size_t gdn_varlen_workspace_bytes(int32_t N, int32_t T_tot, int32_t H_qk, int32_t H_v,
                                  int32_t D, gdn_dtype dt) {
  if (check_dims(H_qk, H_v, D, dt) != GDN_OK || N < 0 || T_tot < 0) return 0;
  const int64_t nc = ((int64_t)T_tot + gdn::kC - 1) / gdn::kC + N;
  return ws_layout(nc, H_qk, H_v, dt, N).total;
}

gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* h0, void* o, float* ht,
                               int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t D,
                               gdn_dtype dt, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return prefill_fixed(q, k, v, alpha, beta, h0, o, ht, B, T, H_qk, H_v, D, dt, workspace,
                       workspace_bytes, stream, kBoth, false);
}

gdn_status gdn_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta, const float* h0,
                                       void* o, float* ht, int32_t B, int32_t T, int32_t H_qk,
                                       int32_t H_v, int32_t D, gdn_dtype dt, void* stream) {
  // Every host check first (nothing touches the device on an error): the
  // arguments with no workspace, then the workspace size against the array.
  gdn_status s = prefill_fixed(q, k, v, alpha, beta, h0, o, ht, B, T, H_qk, H_v, D, dt,
                               nullptr, 0, stream, kCheckOnly, false);
  if (s != GDN_OK) return s;
  const size_t need = gdn_prefill_workspace_bytes(B, T, H_qk, H_v, D, dt);
  if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    s = scratch_on(static_cast<hipStream_t>(stream), &ws);
    if (s != GDN_OK) return s;
  }
  // The workspace needs no clearing: prepare writes every part the scan reads.
  return prefill_fixed(q, k, v, alpha, beta, h0, o, ht, B, T, H_qk, H_v, D, dt, ws,
                       GDN_NOALLOC_SCRATCH_BYTES, stream, kBoth, false);
}

gdn_status gdn_prefill_prepare(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* h0, void* o, float* ht,
                               int32_t B, int32_t T, int32_t H_qk, int32_t H_v, int32_t D,
                               gdn_dtype dt, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return prefill_fixed(q, k, v, alpha, beta, h0, o, ht, B, T, H_qk, H_v, D, dt, workspace,
                       workspace_bytes, stream, kPrepare, false);
}

gdn_status gdn_prefill_scan(const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* h0, void* o, float* ht, int32_t B,
                            int32_t T, int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_fixed(q, k, v, alpha, beta, h0, o, ht, B, T, H_qk, H_v, D, dt, workspace,
                       workspace_bytes, stream, kScan, false);
}

gdn_status gdn_prefill_chunked_bf16_state(const void* q, const void* k, const void* v,
                                          const float* alpha, const float* beta, const void* h0,
                                          void* o, void* ht, int32_t B, int32_t T, int32_t H_qk,
                                          int32_t H_v, int32_t D, gdn_dtype dt, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return prefill_fixed(q, k, v, alpha, beta, h0, o, ht, B, T, H_qk, H_v, D, dt, workspace,
                       workspace_bytes, stream, kBoth, true);
}

namespace {
gdn_status decode_common(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, void* state, void* o, int32_t B, int32_t H_qk,
                         int32_t H_v, int32_t D, gdn_dtype dt, void* stream, bool state_bf16) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (B < 0) return GDN_ERR_SHAPE;
  if (B == 0) return GDN_OK;
  if (!q || !k || !v || !alpha || !beta || !state || !o) return GDN_ERR_NULL;
  const int64_t es = (int64_t)esize(dt), Dl = gdn::kD;
  if ((int64_t)B * H_v > (int64_t(1) << 30)) return GDN_ERR_UNSUPPORTED;
  const void* p16[] = {q, k, v, o, state};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  if (!aligned(alpha, 4) || !aligned(beta, 4)) return GDN_ERR_ALIGN;
  const Range rq = span(q, B * H_qk * Dl * es), rk = span(k, B * H_qk * Dl * es);
  const Range rv = span(v, B * H_v * Dl * es), ro = span(o, B * H_v * Dl * es);
  const Range ra = span(alpha, B * H_v * 4), rb = span(beta, B * H_v * 4);
  const Range rs = span(state, (int64_t)B * H_v * Dl * Dl * (state_bf16 ? 2 : 4));
  const Range ins[] = {rq, rk, rv, ra, rb};
  for (const Range& in : ins)
    if (overlap(ro, in) || overlap(rs, in)) return GDN_ERR_ALIAS;
  if (overlap(ro, rs)) return GDN_ERR_ALIAS;
  return fail_hip(gdn::launch_decode_step(q, k, v, alpha, beta, state, o, B, H_qk, H_v,
                                          dt == GDN_BF16, state_bf16,
                                          static_cast<hipStream_t>(stream)));
}
}  // namespace

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, float* state, void* o, int32_t B, int32_t H_qk,
                           int32_t H_v, int32_t D, gdn_dtype dt, void* stream) {
  return decode_common(q, k, v, alpha, beta, state, o, B, H_qk, H_v, D, dt, stream, false);
}

gdn_status gdn_decode_step_bf16_state(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, void* state,
                                      void* o, int32_t B, int32_t H_qk, int32_t H_v, int32_t D,
                                      gdn_dtype dt, void* stream) {
  return decode_common(q, k, v, alpha, beta, state, o, B, H_qk, H_v, D, dt, stream, true);
}

gdn_status gdn_decode_verify(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* state, void* o, int32_t B,
                             int32_t n, int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                             void* stream) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (B < 0 || n < 1) return GDN_ERR_SHAPE;
  if (n > gdn::kMaxDraft) return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  if (!q || !k || !v || !alpha || !beta || !state || !o) return GDN_ERR_NULL;
  if ((int64_t)B * H_v > (int64_t(1) << 30)) return GDN_ERR_UNSUPPORTED;
  const int64_t es = (int64_t)esize(dt), Dl = gdn::kD, Bn = (int64_t)B * n;
  const void* p16[] = {q, k, v, o, state};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  if (!aligned(alpha, 4) || !aligned(beta, 4)) return GDN_ERR_ALIGN;
  const Range ro = span(o, Bn * H_v * Dl * es);
  const Range ins[] = {span(q, Bn * H_qk * Dl * es), span(k, Bn * H_qk * Dl * es),
                       span(v, Bn * H_v * Dl * es), span(alpha, Bn * H_v * 4),
                       span(beta, Bn * H_v * 4), span(state, (int64_t)B * H_v * Dl * Dl * 4)};
  for (const Range& in : ins)
    if (overlap(ro, in)) return GDN_ERR_ALIAS;
  return fail_hip(gdn::launch_decode_multi(q, k, v, alpha, beta, const_cast<float*>(state),
                                           nullptr, o, B, n, H_qk, H_v, dt == GDN_BF16, true,
                                           static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_commit(const void* k, const void* v, const float* alpha, const float* beta,
                             float* state, const int32_t* n_accept, int32_t B, int32_t n,
                             int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt, void* stream) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (B < 0 || n < 1) return GDN_ERR_SHAPE;
  if (n > gdn::kMaxDraft) return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  if (!k || !v || !alpha || !beta || !state || !n_accept) return GDN_ERR_NULL;
  if ((int64_t)B * H_v > (int64_t(1) << 30)) return GDN_ERR_UNSUPPORTED;
  const int64_t es = (int64_t)esize(dt), Dl = gdn::kD, Bn = (int64_t)B * n;
  const void* p16[] = {k, v, state};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  if (!aligned(alpha, 4) || !aligned(beta, 4) || !aligned(n_accept, 4)) return GDN_ERR_ALIGN;
  const Range rs = span(state, (int64_t)B * H_v * Dl * Dl * 4);
  const Range ins[] = {span(k, Bn * H_qk * Dl * es), span(v, Bn * H_v * Dl * es),
                       span(alpha, Bn * H_v * 4), span(beta, Bn * H_v * 4),
                       span(n_accept, (int64_t)B * 4)};
  for (const Range& in : ins)
    if (overlap(rs, in)) return GDN_ERR_ALIAS;
  return fail_hip(gdn::launch_decode_multi(nullptr, k, v, alpha, beta, state, n_accept, nullptr,
                                           B, n, H_qk, H_v, dt == GDN_BF16, false,
                                           static_cast<hipStream_t>(stream)));
}

gdn_status gdn_prefill_varlen(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const int32_t* cu_seqlens, int32_t N,
                              int32_t T_tot, const float* h0, void* o, float* ht,
                              const void* gate, const float* norm_weight, float norm_eps,
                              int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                              void* workspace, size_t workspace_bytes, void* stream) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (N < 0 || T_tot < 0) return GDN_ERR_SHAPE;
  if (N == 0) return T_tot == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (N > 65535) return GDN_ERR_UNSUPPORTED;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (!(norm_eps >= 0.f)) return GDN_ERR_SHAPE;
  const int64_t nc = ((int64_t)T_tot + gdn::kC - 1) / gdn::kC + N;
  if (nc > (int64_t(1) << 30)) return GDN_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(nc, H_qk, H_v, dt, N);
  s = check_prefill(q, k, v, alpha, beta, h0, o, ht, gate, norm_weight, cu_seqlens, N + 1,
                    T_tot, N, H_qk, H_v, dt, workspace, workspace_bytes, L.total, 4);
  if (s != GDN_OK) return s;
  s = debug_check_cu(cu_seqlens, N, T_tot, stream);
  if (s != GDN_OK) return s;

  char* ws = static_cast<char*>(workspace);
  int32_t* tab = reinterpret_cast<int32_t*>(ws + L.tab);
  int32_t* seq_off = reinterpret_cast<int32_t*>(ws + L.seq);
  gdn::PrefillLaunch a{};
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.h0 = h0; a.o = o; a.ht = ht;
  a.gate = gate; a.norm_w = norm_weight; a.norm_eps = norm_eps;
  a.Tt = ws + L.tt;
  a.M = ws + L.m;
  a.gam = reinterpret_cast<float*>(ws + L.gam);
  a.dec = reinterpret_cast<float*>(ws + L.dec);
  a.cm = gdn::ChunkMap{tab, seq_off, 0, 0, (int)nc};
  a.state_bf16 = false;
  a.nseq = N;
  a.ntok = T_tot;
  a.nc_launch = (int)nc;
  a.Hqk = H_qk; a.Hv = H_v;
  a.bf16_io = dt == GDN_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = fail_hip(gdn::launch_varlen_table(cu_seqlens, N, T_tot, (int)nc, tab, seq_off, st));
  if (s != GDN_OK) return s;
  s = fail_hip(gdn::launch_prepare(a, st));
  if (s != GDN_OK) return s;
  return fail_hip(gdn::launch_scan(a, st));
}

namespace {
// Backward workspace: the forward layout (with the chunk table for a packed
// batch), then N = (I + A)^-1 [nc][Hv][64][64], the state entering every chunk
// and the gradient of the state leaving every chunk ([nc][Hv][128][128] each),
// all in the element type.
struct BwdLayout {
  WsLayout f;
  size_t n, s, ds, total;
};
BwdLayout bwd_layout(int64_t nc, int64_t Hqk, int64_t Hv, gdn_dtype dt, int64_t nseq_varlen) {
  BwdLayout b{};
  b.f = ws_layout(nc, Hqk, Hv, dt, nseq_varlen);
  const size_t st = round256((size_t)nc * Hv * gdn::kD * gdn::kD * esize(dt));
  b.n = b.f.total;
  b.s = b.n + round256((size_t)nc * Hv * gdn::kC * gdn::kC * esize(dt));
  b.ds = b.s + st;
  b.total = b.ds + st;
  return b;
}

struct BwdIO {
  const void *q, *k, *v;
  const float *alpha, *beta, *h0;
  const void* dout;
  const float* dht;
  void *dq, *dk, *dv;
  float *dalpha, *dbeta, *dh0;
};

// Shared by the fixed-length and packed backward calls: checks (all before
// anything is enqueued), then prepare, the checkpointing scan, the reverse
// chain and the gradient kernel.  `cu` is null for a fixed-length batch
// (then cm describes it), else the device cu_seqlens of nseq sequences.
gdn_status bwd_run(const BwdIO& io, int64_t nseq, int64_t ntok, gdn::ChunkMap cm, int64_t nc,
                   const int32_t* cu, int32_t H_qk, int32_t H_v, gdn_dtype dt, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (nc > (int64_t(1) << 30) || nc * H_v * gdn::kD * gdn::kD > kMaxElems)
    return GDN_ERR_UNSUPPORTED;
  if (ntok > 0 && (!io.q || !io.k || !io.v || !io.alpha || !io.beta || !io.dout || !io.dq ||
                   !io.dk || !io.dv || !io.dalpha || !io.dbeta))
    return GDN_ERR_NULL;
  if (ntok * H_v * gdn::kD > kMaxElems || nseq * H_v * gdn::kD * gdn::kD > kMaxElems)
    return GDN_ERR_UNSUPPORTED;
  const BwdLayout Lw = bwd_layout(nc, H_qk, H_v, dt, cu ? nseq : -1);
  const size_t need = nc > 0 ? Lw.total : 0;
  if (need > 0 && !workspace) return GDN_ERR_WORKSPACE;
  if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
  const void* p16[] = {io.q, io.k, io.v, io.dout, io.dq, io.dk, io.dv, io.h0, io.dht, io.dh0,
                       workspace};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  const void* p4[] = {io.alpha, io.beta, io.dalpha, io.dbeta, cu};
  for (const void* p : p4)
    if (!aligned(p, 4)) return GDN_ERR_ALIGN;
  const int64_t es = (int64_t)esize(dt), Dl = gdn::kD, SB = nseq * H_v * Dl * Dl * 4;
  const Range ins[] = {span(io.q, ntok * H_qk * Dl * es), span(io.k, ntok * H_qk * Dl * es),
                       span(io.v, ntok * H_v * Dl * es),  span(io.dout, ntok * H_v * Dl * es),
                       span(io.alpha, ntok * H_v * 4),    span(io.beta, ntok * H_v * 4),
                       span(io.h0, SB),                   span(io.dht, SB),
                       span(cu, cu ? (nseq + 1) * 4 : 0)};
  const Range outs[] = {span(io.dq, ntok * H_qk * Dl * es), span(io.dk, ntok * H_qk * Dl * es),
                        span(io.dv, ntok * H_v * Dl * es),  span(io.dalpha, ntok * H_v * 4),
                        span(io.dbeta, ntok * H_v * 4),     span(io.dh0, SB),
                        span(workspace, (int64_t)need)};
  // outputs overlap neither an input nor each other
  for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a) {
    for (const Range& in : ins)
      if (overlap(outs[a], in)) return GDN_ERR_ALIAS;
    for (size_t c = a + 1; c < sizeof(outs) / sizeof(outs[0]); ++c)
      if (overlap(outs[a], outs[c])) return GDN_ERR_ALIAS;
  }

  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  gdn_status s = cu ? debug_check_cu(cu, (int32_t)nseq, (int32_t)ntok, stream) : GDN_OK;
  if (s != GDN_OK) return s;
  if (cu) {
    int32_t* tab = reinterpret_cast<int32_t*>(ws + Lw.f.tab);
    int32_t* seq_off = reinterpret_cast<int32_t*>(ws + Lw.f.seq);
    s = fail_hip(gdn::launch_varlen_table(cu, (int)nseq, (int)ntok, (int)nc, tab, seq_off, st));
    if (s != GDN_OK) return s;
    cm = gdn::ChunkMap{tab, seq_off, 0, 0, (int)nc};
  }
  if (nc > 0) {
    gdn::PrefillLaunch a{};
    a.q = io.q; a.k = io.k; a.v = io.v; a.alpha = io.alpha; a.beta = io.beta;
    a.Tt = ws + Lw.f.tt;
    a.M = ws + Lw.f.m;
    a.gam = reinterpret_cast<float*>(ws + Lw.f.gam);
    a.dec = reinterpret_cast<float*>(ws + Lw.f.dec);
    a.cm = cm;
    a.nseq = (int)nseq;
    a.ntok = ntok;
    a.nc_launch = (int)nc;
    a.Hqk = H_qk; a.Hv = H_v;
    a.bf16_io = dt == GDN_BF16;
    a.solve_only = true;
    a.N = ws + Lw.n;
    s = fail_hip(gdn::launch_prepare(a, st));
    if (s != GDN_OK) return s;
    if (a.bf16_io) {
      // the forward scan, outputs off, writing the state entering every chunk
      a.h0 = io.h0;
      a.states = ws + Lw.s;
      s = fail_hip(gdn::launch_scan(a, st));
      if (s != GDN_OK) return s;
    }
  }
  if (nseq == 0 || (nc == 0 && !io.dh0)) return GDN_OK;
  gdn::BackwardLaunch bl{};
  bl.q = io.q; bl.k = io.k; bl.v = io.v; bl.dout = io.dout; bl.alpha = io.alpha;
  bl.beta = io.beta; bl.h0 = io.h0; bl.dht = io.dht;
  bl.dq = io.dq; bl.dk = io.dk; bl.dv = io.dv; bl.dalpha = io.dalpha; bl.dbeta = io.dbeta;
  bl.dh0 = io.dh0;
  bl.N = ws ? ws + Lw.n : nullptr;
  bl.states_ready = dt == GDN_BF16;
  bl.M = ws ? ws + Lw.f.m : nullptr;
  bl.S = ws ? ws + Lw.s : nullptr;
  bl.dS = ws ? ws + Lw.ds : nullptr;
  bl.gam = ws ? reinterpret_cast<float*>(ws + Lw.f.gam) : nullptr;
  bl.dec = ws ? reinterpret_cast<float*>(ws + Lw.f.dec) : nullptr;
  bl.cm = cm;
  bl.nseq = (int)nseq;
  bl.nc = (int)nc;
  bl.Hqk = H_qk; bl.Hv = H_v;
  bl.bf16_io = dt == GDN_BF16;
  return fail_hip(gdn::launch_backward(bl, st));
}
}  // namespace

size_t gdn_prefill_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                                       int32_t D, gdn_dtype dt) {
  if (check_dims(H_qk, H_v, D, dt) != GDN_OK || B < 0 || T < 0) return 0;
  const int64_t nc = (int64_t)B * (((int64_t)T + gdn::kC - 1) / gdn::kC);
  if (nc == 0) return 0;
  return bwd_layout(nc, H_qk, H_v, dt, -1).total;
}

size_t gdn_varlen_bwd_workspace_bytes(int32_t N, int32_t T_tot, int32_t H_qk, int32_t H_v,
                                      int32_t D, gdn_dtype dt) {
  if (check_dims(H_qk, H_v, D, dt) != GDN_OK || N < 0 || T_tot < 0) return 0;
  const int64_t nc = ((int64_t)T_tot + gdn::kC - 1) / gdn::kC + N;
  return bwd_layout(nc, H_qk, H_v, dt, N).total;
}

gdn_status gdn_prefill_chunked_bwd(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta, const float* h0,
                                   const void* dout, const float* dht, void* dq, void* dk,
                                   void* dv, float* dalpha, float* dbeta, float* dh0, int32_t B,
                                   int32_t T, int32_t H_qk, int32_t H_v, int32_t D,
                                   gdn_dtype dt, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (B < 0 || T < 0) return GDN_ERR_SHAPE;
  if (B > 65535) return GDN_ERR_UNSUPPORTED;
  const int64_t Nc = ((int64_t)T + gdn::kC - 1) / gdn::kC;
  const int64_t nc = (int64_t)B * Nc;
  if (nc > (int64_t(1) << 30)) return GDN_ERR_UNSUPPORTED;
  const BwdIO io{q, k, v, alpha, beta, h0, dout, dht, dq, dk, dv, dalpha, dbeta, dh0};
  return bwd_run(io, B, (int64_t)B * T, gdn::ChunkMap{nullptr, nullptr, T, (int)Nc, (int)nc},
                 nc, nullptr, H_qk, H_v, dt, workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_varlen_bwd(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta,
                                  const int32_t* cu_seqlens, int32_t N, int32_t T_tot,
                                  const float* h0, const void* dout, const float* dht, void* dq,
                                  void* dk, void* dv, float* dalpha, float* dbeta, float* dh0,
                                  int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  gdn_status s = check_dims(H_qk, H_v, D, dt);
  if (s != GDN_OK) return s;
  if (N < 0 || T_tot < 0) return GDN_ERR_SHAPE;
  if (N == 0) return T_tot == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (N > 65535) return GDN_ERR_UNSUPPORTED;
  if (!cu_seqlens) return GDN_ERR_NULL;
  const int64_t nc = ((int64_t)T_tot + gdn::kC - 1) / gdn::kC + N;
  const BwdIO io{q, k, v, alpha, beta, h0, dout, dht, dq, dk, dv, dalpha, dbeta, dh0};
  return bwd_run(io, N, T_tot, gdn::ChunkMap{}, nc, cu_seqlens, H_qk, H_v, dt, workspace,
                 workspace_bytes, stream);
}

namespace {
constexpr int kAttnD = 256;

gdn_status check_attn_dims(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t rope_dim,
                           float theta, float eps, gdn_dtype dt) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return GDN_ERR_SHAPE;
  if (D != kAttnD || Hq / Hkv > 8 || Hq > 4096) return GDN_ERR_UNSUPPORTED;
  if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (rope_dim < 0 || rope_dim > kAttnD || rope_dim % 8 != 0) return GDN_ERR_UNSUPPORTED;
  if (!(theta > 0.f) || !(theta < 3.0e38f) || !(eps >= 0.f)) return GDN_ERR_SHAPE;
  return GDN_OK;
}

// Attention workspace: rotated queries, then (prefill) rotated keys or
// (decode) the split partials.
size_t attn_prefill_ws(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, gdn_dtype dt) {
  return round256((size_t)B * T * Hq * kAttnD * esize(dt)) +
         round256((size_t)B * T * Hkv * kAttnD * esize(dt));
}
size_t attn_decode_ws(int64_t B, int64_t cache_len, int64_t Hq, int64_t Hkv, gdn_dtype dt) {
  const int64_t ns = gdn::attn_decode_splits((int)B, (int)Hkv, (int)cache_len);
  return round256((size_t)B * Hq * kAttnD * esize(dt)) + 2 * round256((size_t)B * Hq * ns * 4) +
         round256((size_t)B * Hq * ns * kAttnD * 4);
}
}  // namespace

size_t gdn_attn_prefill_workspace_bytes(int32_t B, int32_t T, int32_t H_q, int32_t H_kv,
                                        int32_t D, gdn_dtype dt) {
  if (check_attn_dims(B, H_q, H_kv, D, 0, 1.f, 0.f, dt) != GDN_OK || T < 0) return 0;
  return attn_prefill_ws(B, T, H_q, H_kv, dt);
}

size_t gdn_attn_decode_workspace_bytes(int32_t B, int32_t cache_len, int32_t H_q, int32_t H_kv,
                                       int32_t D, gdn_dtype dt) {
  if (check_attn_dims(B, H_q, H_kv, D, 0, 1.f, 0.f, dt) != GDN_OK || cache_len <= 0) return 0;
  return attn_decode_ws(B, cache_len, H_q, H_kv, dt);
}

gdn_status gdn_attn_prefill(const void* q, const void* k, const void* v, const void* gate,
                            const float* q_norm_w, const float* k_norm_w, float norm_eps, void* o,
                            void* k_cache, void* v_cache, int32_t cache_len, int32_t B, int32_t T,
                            int32_t H_q, int32_t H_kv, int32_t D, int32_t rope_dim,
                            float rope_theta, gdn_dtype dt, void* workspace,
                            size_t workspace_bytes, void* stream) {
  gdn_status s = check_attn_dims(B, H_q, H_kv, D, rope_dim, rope_theta, norm_eps, dt);
  if (s != GDN_OK) return s;
  if (T < 0) return GDN_ERR_SHAPE;
  if ((int64_t)B * T > (int64_t(1) << 31) / 64) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)B * T * (H_q + H_kv) >= (int64_t(1) << 31)) return GDN_ERR_UNSUPPORTED;
  if (B == 0 || T == 0) return GDN_OK;
  if (!q || !k || !v || !gate || !o) return GDN_ERR_NULL;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return GDN_ERR_NULL;
  const bool cached = k_cache != nullptr;
  if (cached && cache_len < T) return GDN_ERR_SHAPE;
  const int64_t clen = cached ? cache_len : T;
  const size_t need = attn_prefill_ws(B, T, H_q, H_kv, dt);
  if (!workspace) return GDN_ERR_WORKSPACE;
  if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
  const void* p16[] = {q, k, v, gate, o, k_cache, v_cache, workspace};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  if (!aligned(q_norm_w, 4) || !aligned(k_norm_w, 4)) return GDN_ERR_ALIGN;
  const int64_t es = (int64_t)esize(dt), nt = (int64_t)B * T;
  const Range ins[] = {span(q, nt * H_q * kAttnD * es), span(k, nt * H_kv * kAttnD * es),
                       span(v, nt * H_kv * kAttnD * es), span(gate, nt * H_q * kAttnD * es),
                       span(q_norm_w, q_norm_w ? kAttnD * 4 : 0),
                       span(k_norm_w, k_norm_w ? kAttnD * 4 : 0)};
  const Range outs[] = {span(o, nt * H_q * kAttnD * es),
                        span(k_cache, (int64_t)B * clen * H_kv * kAttnD * es),
                        span(v_cache, (int64_t)B * clen * H_kv * kAttnD * es),
                        span(workspace, (int64_t)need)};
  for (size_t a = 0; a < 4; ++a) {
    for (const Range& in : ins)
      if (overlap(outs[a], in)) return GDN_ERR_ALIAS;
    for (size_t c = a + 1; c < 4; ++c)
      if (overlap(outs[a], outs[c])) return GDN_ERR_ALIAS;
  }
  char* ws = static_cast<char*>(workspace);
  gdn::AttnLaunch a{};
  a.q = q; a.k = k; a.v = v; a.gate = gate; a.qw = q_norm_w; a.kw = k_norm_w;
  a.eps = norm_eps; a.theta = rope_theta; a.rope_dim = rope_dim; a.pos = nullptr;
  a.qrot = ws;
  a.kc = cached ? k_cache : ws + round256((size_t)nt * H_q * kAttnD * es);
  a.vc_write = cached ? v_cache : nullptr;
  a.vc_read = cached ? v_cache : v;
  a.o = o;
  a.B = B; a.T = T; a.cache_len = (int)clen; a.Hq = H_q; a.Hkv = H_kv;
  a.decode = false;
  a.bf16_io = dt == GDN_BF16;
  return fail_hip(gdn::launch_attention(a, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_attn_decode(const void* q, const void* k, const void* v, const void* gate,
                           const float* q_norm_w, const float* k_norm_w, float norm_eps, void* o,
                           void* k_cache, void* v_cache, const int32_t* pos, int32_t cache_len,
                           int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t rope_dim,
                           float rope_theta, gdn_dtype dt, void* workspace,
                           size_t workspace_bytes, void* stream) {
  gdn_status s = check_attn_dims(B, H_q, H_kv, D, rope_dim, rope_theta, norm_eps, dt);
  if (s != GDN_OK) return s;
  if (cache_len <= 0) return GDN_ERR_SHAPE;
  if ((int64_t)B * cache_len > (int64_t(1) << 31) / 64) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)B * (H_q + H_kv) >= (int64_t(1) << 31)) return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  if (!q || !k || !v || !gate || !o || !k_cache || !v_cache || !pos) return GDN_ERR_NULL;
  const size_t need = attn_decode_ws(B, cache_len, H_q, H_kv, dt);
  if (!workspace) return GDN_ERR_WORKSPACE;
  if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
  const void* p16[] = {q, k, v, gate, o, k_cache, v_cache, workspace};
  for (const void* p : p16)
    if (!aligned(p, 16)) return GDN_ERR_ALIGN;
  if (!aligned(q_norm_w, 4) || !aligned(k_norm_w, 4) || !aligned(pos, 4)) return GDN_ERR_ALIGN;
  const int64_t es = (int64_t)esize(dt);
  const Range ins[] = {span(q, (int64_t)B * H_q * kAttnD * es), span(k, (int64_t)B * H_kv * kAttnD * es),
                       span(v, (int64_t)B * H_kv * kAttnD * es), span(gate, (int64_t)B * H_q * kAttnD * es),
                       span(q_norm_w, q_norm_w ? kAttnD * 4 : 0),
                       span(k_norm_w, k_norm_w ? kAttnD * 4 : 0), span(pos, (int64_t)B * 4)};
  const Range outs[] = {span(o, (int64_t)B * H_q * kAttnD * es),
                        span(k_cache, (int64_t)B * cache_len * H_kv * kAttnD * es),
                        span(v_cache, (int64_t)B * cache_len * H_kv * kAttnD * es),
                        span(workspace, (int64_t)need)};
  for (size_t a = 0; a < 4; ++a) {
    for (const Range& in : ins)
      if (overlap(outs[a], in)) return GDN_ERR_ALIAS;
    for (size_t c = a + 1; c < 4; ++c)
      if (overlap(outs[a], outs[c])) return GDN_ERR_ALIAS;
  }
  char* ws = static_cast<char*>(workspace);
  const int64_t ns = gdn::attn_decode_splits(B, H_kv, cache_len);
  const size_t oq = round256((size_t)B * H_q * kAttnD * es);
  const size_t om = round256((size_t)B * H_q * ns * 4);
  gdn::AttnLaunch a{};
  a.q = q; a.k = k; a.v = v; a.gate = gate; a.qw = q_norm_w; a.kw = k_norm_w;
  a.eps = norm_eps; a.theta = rope_theta; a.rope_dim = rope_dim; a.pos = pos;
  a.qrot = ws;
  a.pm = reinterpret_cast<float*>(ws + oq);
  a.pl = reinterpret_cast<float*>(ws + oq + om);
  a.po = reinterpret_cast<float*>(ws + oq + 2 * om);
  a.kc = k_cache;
  a.vc_write = v_cache;
  a.vc_read = v_cache;
  a.o = o;
  a.B = B; a.T = 1; a.cache_len = cache_len; a.Hq = H_q; a.Hkv = H_kv;
  a.decode = true;
  a.bf16_io = dt == GDN_BF16;
  return fail_hip(gdn::launch_attention(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// C ABI of the SSA dual-stream attention library: host-side validation,
// workspace layout and kernel launches. Every check runs before the first
// launch; no call allocates memory or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/ssa.h"
#include "ssa_common.h"
#include "ssa_kernels.h"

namespace {

thread_local char g_err[512] = "";
// the caller's event pair of ssa_set_attn_timing_events (NULL: no timing)
hipEvent_t g_timing_start = nullptr, g_timing_stop = nullptr;

ssa_status fail(ssa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

ssa_status ok() {
  g_err[0] = '\0';
  return SSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Problem {
  ssa::Dims d;
  ssa::HeadMap hm;
  bool bf16;
  bool decode;
};

struct Layout {
  size_t qbar, kbar, kc, keys, vt, kn, queues, partials, loss, total;
};

Layout layout_of(const Problem& P) {
  const ssa::Dims& d = P.d;
  Layout L;
  size_t off = 0;
  L.qbar = off;
  off += align256((size_t)d.B * d.Hq * d.nQB * d.D * sizeof(float));
  L.kbar = off;
  off += align256((size_t)d.B * d.Hkv * d.nKB * d.D * sizeof(float));
  L.kc = off;   // per-token selection: float64 pooled keys, 16-block chunks
  if (d.tok) off += align256(ssa::tok_kc_bytes(d));
  L.keys = off;   // decode: every candidate's orderable score key, per q head
  if (P.decode) off += align256((size_t)d.B * d.Hq * d.nKB * sizeof(uint64_t));
  L.vt = off;
  if (P.bf16 && !P.decode) off += align256((size_t)d.B * d.Hkv * d.D * d.Nk * sizeof(uint16_t));
  L.kn = off;   // largest key norm per 64-key block, written by the V transpose
  if (P.bf16 && !P.decode) off += align256((size_t)d.B * d.Hkv * (d.Nk / 64) * sizeof(float));
  L.queues = off;   // prefill work queues, zeroed by the V transpose of every call
  if (P.bf16 && !P.decode) off += align256((size_t)ssa::kNumXcd * ssa::kQueueStride * sizeof(int));
  L.partials = off;
  if (P.bf16 && P.decode) {
    int ns = ssa::decode_splits(d.nT);
    if (ns < ssa::kDecSparseParts) ns = ssa::kDecSparseParts;
    off += align256((size_t)d.B * d.Hq * ns * ssa::decode_partial_floats(d.D) * sizeof(float));
  }
  L.loss = off;
  off += align256((size_t)ssa::kLossPartials * sizeof(double));
  L.total = off;
  return L;
}

ssa_status build(const ssa_problem* p, Problem* P) {
  if (p == nullptr) return fail(SSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Nq <= 0 || p->Nk <= 0 || p->D <= 0 ||
      p->block_size <= 0 || p->budget <= 0)
    return fail(SSA_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d D=%d "
                "block_size=%d budget=%d)", p->B, p->Hq, p->Hkv, p->Nq, p->Nk, p->D,
                p->block_size, p->budget);
  if (p->n_sink < 0 || p->n_local < 0)
    return fail(SSA_ERR_INVALID_ARG, "n_sink and n_local must be >= 0");
  if (p->Hq % p->Hkv != 0)
    return fail(SSA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->budget < p->n_sink + p->n_local)
    return fail(SSA_ERR_INVALID_ARG, "budget (%d) is below the forced blocks n_sink + n_local (%d)",
                p->budget, p->n_sink + p->n_local);
  if (p->Nq != p->Nk && p->Nq != 1)
    return fail(SSA_ERR_UNSUPPORTED, "Nq must equal Nk (prefill) or be 1 (decode); got Nq=%d Nk=%d",
                p->Nq, p->Nk);
  if (p->dtype != SSA_F32 && p->dtype != SSA_BF16)
    return fail(SSA_ERR_UNSUPPORTED, "dtype %d is not SSA_F32 or SSA_BF16", p->dtype);
  if (p->D != 64 && p->D != 128) return fail(SSA_ERR_UNSUPPORTED, "D must be 64 or 128; got %d", p->D);
  if (p->block_size != 64 && p->block_size != 16)
    return fail(SSA_ERR_UNSUPPORTED, "block_size must be 64 or 16; got %d", p->block_size);
  if (p->Nk % ssa::kBlock != 0)
    return fail(SSA_ERR_UNSUPPORTED, "Nk (%d) must be a multiple of 64", p->Nk);
  if (p->Nk / p->block_size > ssa::kMaxKeyBlocks)
    return fail(SSA_ERR_UNSUPPORTED, "Nk (%d) exceeds %d key blocks of %d", p->Nk,
                ssa::kMaxKeyBlocks, p->block_size);
  if (p->block_size == 16 && p->dtype == SSA_F32)
    return fail(SSA_ERR_UNSUPPORTED, "block_size 16 needs bf16 inputs");
  if (p->Hq > ssa::kMaxHq) return fail(SSA_ERR_UNSUPPORTED, "Hq (%d) exceeds %d", p->Hq, ssa::kMaxHq);
  const int G = p->Hq / p->Hkv;
  if (G > ssa::kMaxGroup)
    return fail(SSA_ERR_UNSUPPORTED, "Hq/Hkv (%d) exceeds %d", G, ssa::kMaxGroup);
  const bool decode = p->Nq == 1 && p->Nk != 1;
  if (p->selection != SSA_SELECT_PER_HEAD && p->selection != SSA_SELECT_GROUP &&
      p->selection != SSA_SELECT_TOKEN)
    return fail(SSA_ERR_INVALID_ARG, "selection must be SSA_SELECT_PER_HEAD (0), SSA_SELECT_GROUP (1) "
                "or SSA_SELECT_TOKEN (2); got %d", p->selection);
  // in decode the single query is its own representation: per token = per head
  const bool tok = p->selection == SSA_SELECT_TOKEN && !decode;
  if (tok && p->budget > ssa::kTokMaxBudget)
    return fail(SSA_ERR_UNSUPPORTED, "per-token selection supports budget <= %d; got %d",
                ssa::kTokMaxBudget, p->budget);
  if (!(p->scale >= 0.f) || isinf(p->scale))
    return fail(SSA_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 selects 1/sqrt(D))");
  const double total = (double)p->B * p->Hq * p->Nq * p->D;
  const double kv = (double)p->B * p->Hkv * p->Nk * p->D;
  if (total > 1.0e12 || kv > 1.0e12) return fail(SSA_ERR_UNSUPPORTED, "problem too large");
  if ((double)p->B * p->Hq * (p->Nq == 1 ? 1 : tok ? p->Nq : p->Nq / p->block_size) > 2.0e9)
    return fail(SSA_ERR_UNSUPPORTED, "too many selection lists");

  ssa::HeadMap& hm = P->hm;
  memset(&hm, 0, sizeof(hm));
  int count[ssa::kMaxHq];
  for (int g = 0; g < p->Hkv && g < ssa::kMaxHq; ++g) count[g] = 0;
  for (int h = 0; h < p->Hq; ++h) {
    const int g = p->head_map ? p->head_map[h] : h / G;
    if (g < 0 || g >= p->Hkv)
      return fail(SSA_ERR_INVALID_ARG, "head_map[%d] = %d is outside [0, %d)", h, g, p->Hkv);
    if (count[g] >= G)
      return fail(SSA_ERR_INVALID_ARG, "head_map gives kv head %d more than Hq/Hkv = %d q heads", g, G);
    hm.kv_of_q[h] = (uint8_t)g;
    hm.q_of_kv[g * G + count[g]] = (uint8_t)h;
    count[g]++;
  }

  ssa::Dims& d = P->d;
  d.B = p->B; d.Hq = p->Hq; d.Hkv = p->Hkv; d.Nq = p->Nq; d.Nk = p->Nk; d.D = p->D;
  d.budget = p->budget; d.n_sink = p->n_sink; d.n_local = p->n_local;
  d.bs = p->block_size;
  d.nKB = p->Nk / d.bs;
  d.nT = p->Nk / ssa::kBlock;
  if (p->Nq == p->Nk) {
    if (p->Nq % ssa::kBlock != 0)
      return fail(SSA_ERR_UNSUPPORTED, "Nq (%d) must be a multiple of 64", p->Nq);
    d.nQB = p->Nq / d.bs;
    d.nQT = p->Nq / ssa::kBlock;
  } else {
    d.nQB = 1;
    d.nQT = 1;
  }
  d.G = G;
  d.group_select = p->selection == SSA_SELECT_GROUP ? 1 : 0;
  d.tok = tok ? 1 : 0;
  d.nL = tok ? d.Nq : d.nQB;
  d.lrows = tok ? 1 : d.bs;
  d.scale = p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)p->D));
  d.scale_log2 = d.scale * ssa::kLog2e;
  P->bf16 = p->dtype == SSA_BF16;
  P->decode = decode;
  return SSA_OK;
}

// Backward workspace: per-row statistics (float32 [B,Hq,Nq,4]) and, for
// bf16, the selection bits (uint16 [B*Hkv, key tiles, Nq/32, Hq/Hkv]) and
// the float32 partial sums that the full-stream pass hands to the
// sparse-stream pass (dQ [B,Hq,Nq,D], dK and dV [B,Hkv,Nk,D]), plus the
// sparse dK / dV pass's per-q-head slots ([Hq/Hkv] x [B,Hkv,Nk,D] each);
// with per-token lists also one 64-bit row mask per (kv head, 128-key tile,
// 32-row step, q head of the group, 32-key wave block).
struct BwdLayout {
  size_t stats, bits, rowbits, pq, pk, pv, sk, sv, total;
};

BwdLayout bwd_layout_of(const Problem& P) {
  const ssa::Dims& d = P.d;
  BwdLayout L;
  size_t off = 0;
  L.stats = off;
  off += align256((size_t)d.B * d.Hq * d.Nq * 4 * sizeof(float));
  L.bits = L.rowbits = L.pq = L.pk = L.pv = L.sk = L.sv = off;
  if (P.bf16) {
    L.bits = off;
    off += align256((size_t)d.B * d.Hq * ssa::bwd_key_tiles(d) * (d.Nq / 32) * sizeof(uint16_t));
    L.rowbits = off;   // per-token lists: one 64-bit row mask per 32-key wave block
    if (d.tok)
      off += align256((size_t)d.B * d.Hq * ssa::bwd_key_tiles(d) * (d.Nq / 32) * 4 * sizeof(uint64_t));
    L.pq = off;
    off += align256((size_t)d.B * d.Hq * d.Nq * d.D * sizeof(float));
    L.pk = off;   // head-group slots of the full dK / dV pass
    const size_t nslot = (size_t)ssa::bwd_full_split(d);
    off += align256(nslot * d.B * d.Hkv * d.Nk * d.D * sizeof(float));
    L.pv = off;
    off += align256(nslot * d.B * d.Hkv * d.Nk * d.D * sizeof(float));
    L.sk = off;   // per-q-head slots of the sparse dK / dV pass
    off += align256((size_t)d.G * d.B * d.Hkv * d.Nk * d.D * sizeof(float));
    L.sv = off;
    off += align256((size_t)d.G * d.B * d.Hkv * d.Nk * d.D * sizeof(float));
  }
  L.total = off;
  return L;
}

ssa_status check_ws(const Problem& P, const void* ws, size_t ws_bytes, Layout* L) {
  *L = layout_of(P);
  if (ws == nullptr) return fail(SSA_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(SSA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < L->total)
    return fail(SSA_ERR_WORKSPACE, "workspace has %zu bytes; %zu needed", ws_bytes, L->total);
  return SSA_OK;
}

ssa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Scratch of ssa_align_loss_noalloc: the float64 partial sums of the loss
// kernels, kLossPartials of them whatever the problem size. Each GPU that
// loads the library holds its own copy until the process ends. Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol): scratch_on() looks up each device's address once.
static __device__ __align__(256) double scratch[ssa::kLossPartials];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up with that device current on the
// first call for it.
ssa_status scratch_on(void* stream, double** out) {
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice((hipStream_t)stream, &dev)
                                   : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSA_ERR_UNSUPPORTED, "device %d is beyond the %d this library tracks", dev,
                kMaxDevices);
  void* addr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (addr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    addr = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (addr == nullptr) {
      int cur = -1;
      e = hipGetDevice(&cur);
      if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
      if (e == hipSuccess) e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      const hipError_t e2 = (cur >= 0 && cur != dev) ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess || addr == nullptr)
        return fail(SSA_ERR_HIP, "address of the loss scratch on device %d: %s", dev,
                    hipGetErrorString(e != hipSuccess ? e : hipErrorInvalidSymbol));
      if (e2 != hipSuccess)
        return fail(SSA_ERR_HIP, "restoring device %d: %s", cur, hipGetErrorString(e2));
      g_scratch_addr[dev].store(addr, std::memory_order_release);
    }
  }
  *out = (double*)addr;
  return SSA_OK;
}

}  // namespace

extern "C" {

size_t ssa_workspace_bytes(const ssa_problem* p) {
  Problem P;
  if (build(p, &P) != SSA_OK) return 0;
  return layout_of(P).total;
}

ssa_status ssa_pool_blocks(const ssa_problem* p, const void* x, int32_t H, float* pooled,
                           void* stream) {
  Problem P;
  ssa_status s = build(p, &P);
  if (s != SSA_OK) return s;
  if (x == nullptr || pooled == nullptr) return fail(SSA_ERR_INVALID_ARG, "x or pooled is NULL");
  if (H <= 0) return fail(SSA_ERR_INVALID_ARG, "H must be positive; got %d", H);
  const long nblk = (long)P.d.B * H * P.d.nKB;
  return hip_status(ssa::launch_pool(x, P.bf16, pooled, nblk, P.d.bs, P.d.D,
                                     (hipStream_t)stream), "pool");
}

ssa_status ssa_select_blocks(const ssa_problem* p, const void* q, const void* k,
                             const float* k_pooled, int32_t* idx, int32_t* cnt, void* ws,
                             size_t ws_bytes, void* stream) {
  Problem P;
  ssa_status s = build(p, &P);
  if (s != SSA_OK) return s;
  if (q == nullptr || idx == nullptr || cnt == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "q, idx or cnt is NULL");
  if (k == nullptr && k_pooled == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "one of k and k_pooled must be given");
  Layout L;
  if ((s = check_ws(P, ws, ws_bytes, &L)) != SSA_OK) return s;
  const ssa::Dims& d = P.d;
  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  float* qbar = (float*)(w + L.qbar);
  hipError_t e;
  if (d.tok) {   // each row scores its own query: pool K only
    const float* kbar = k_pooled;
    if (kbar == nullptr) {
      float* kb = (float*)(w + L.kbar);
      e = ssa::launch_pool(k, P.bf16, kb, (long)d.B * d.Hkv * d.nKB, d.bs, d.D, st);
      if (e != hipSuccess) return hip_status(e, "pool k");
      kbar = kb;
    }
    return hip_status(ssa::launch_select_tok(q, P.bf16, kbar, (double*)(w + L.kc), idx, cnt, d,
                                             P.hm, st), "select (per token)");
  }
  if (!P.decode) {   // decode: the query is its own block representation
    e = ssa::launch_pool(q, P.bf16, qbar, (long)d.B * d.Hq * d.nQB, d.bs, d.D, st);
    if (e != hipSuccess) return hip_status(e, "pool q");
  }
  const float* kbar = k_pooled;
  if (kbar == nullptr) {
    float* kb = (float*)(w + L.kbar);
    e = ssa::launch_pool(k, P.bf16, kb, (long)d.B * d.Hkv * d.nKB, d.bs, d.D, st);
    if (e != hipSuccess) return hip_status(e, "pool k");
    kbar = kb;
  }
  if (P.decode)
    return hip_status(ssa::launch_select_decode(q, P.bf16, kbar, idx, cnt, d, P.hm,
                                                (uint64_t*)(w + L.keys), st), "select");
  return hip_status(ssa::launch_select(qbar, kbar, idx, cnt, d, P.hm, st), "select");
}

ssa_status ssa_attn_fwd(const ssa_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* cnt, void* h_full, void* h_sparse,
                        float* delta, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Problem P;
  ssa_status s = build(p, &P);
  if (s != SSA_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || idx == nullptr || cnt == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "q, k, v, idx or cnt is NULL");
  if (h_sparse == nullptr) return fail(SSA_ERR_INVALID_ARG, "h_sparse is NULL");
  if (h_full == nullptr && delta != nullptr)
    return fail(SSA_ERR_INVALID_ARG, "delta needs h_full (sparse-only mode has no dropped mass)");
  Layout L;
  if ((s = check_ws(P, ws, ws_bytes, &L)) != SSA_OK) return s;
  const ssa::Dims& d = P.d;
  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  if (!P.bf16)
    return hip_status(ssa::launch_attn_rows_f32((const float*)q, (const float*)k, (const float*)v,
                                                idx, cnt, (float*)h_full, (float*)h_sparse, delta,
                                                lse, d, P.hm, st), "attention (f32)");
  if (P.decode)
    return hip_status(ssa::launch_attn_decode_bf16((const uint16_t*)q, (const uint16_t*)k,
                                                   (const uint16_t*)v, idx, cnt,
                                                   (uint16_t*)h_full, (uint16_t*)h_sparse, delta,
                                                   lse, (float*)(w + L.partials), d, P.hm, st),
                      "attention (decode)");
  uint16_t* vt = (uint16_t*)(w + L.vt);
  int* queues = (int*)(w + L.queues);
  float* kn = ssa::prefill_key_norms(d, h_full == nullptr) ? (float*)(w + L.kn) : nullptr;
  hipError_t e = ssa::launch_transpose((const uint16_t*)v, vt, d.B * d.Hkv, d.Nk, d.D, queues,
                                       ssa::prefill_vt_blk16(d, h_full == nullptr),
                                       (const uint16_t*)k, kn, st);
  if (e != hipSuccess) return hip_status(e, "transpose v");
  if (g_timing_start != nullptr && (e = hipEventRecord(g_timing_start, st)) != hipSuccess)
    return hip_status(e, "timing event (start)");
  e = ssa::launch_attn_prefill_bf16((const uint16_t*)q, (const uint16_t*)k, vt, idx, cnt,
                                    (uint16_t*)h_full, (uint16_t*)h_sparse, delta, lse, queues,
                                    kn, d, P.hm, st);
  if (e != hipSuccess) return hip_status(e, "attention (prefill)");
  if (g_timing_stop != nullptr && (e = hipEventRecord(g_timing_stop, st)) != hipSuccess)
    return hip_status(e, "timing event (stop)");
  return SSA_OK;
}

ssa_status ssa_set_attn_timing_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(SSA_ERR_INVALID_ARG, "timing events: give both or neither");
  g_timing_start = (hipEvent_t)start;
  g_timing_stop = (hipEvent_t)stop;
  return ok();
}

ssa_status ssa_align_loss(const ssa_problem* p, const void* h_full, const void* h_sparse,
                          float* loss, void* grad_full, void* grad_sparse, void* ws,
                          size_t ws_bytes, void* stream) {
  Problem P;
  ssa_status s = build(p, &P);
  if (s != SSA_OK) return s;
  if (h_full == nullptr || h_sparse == nullptr || loss == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "h_full, h_sparse or loss is NULL");
  Layout L;
  if ((s = check_ws(P, ws, ws_bytes, &L)) != SSA_OK) return s;
  const long n = (long)P.d.B * P.d.Hq * P.d.Nq * P.d.D;
  return hip_status(ssa::launch_align_loss(h_full, h_sparse, P.bf16, n, loss, grad_full,
                                           grad_sparse, (double*)((char*)ws + L.loss),
                                           (hipStream_t)stream),
                    "align loss");
}

ssa_status ssa_align_loss_noalloc(const ssa_problem* p, const void* h_full,
                                  const void* h_sparse, float* loss, void* grad_full,
                                  void* grad_sparse, void* stream) {
  Problem P;
  ssa_status s = build(p, &P);
  if (s != SSA_OK) return s;
  if (h_full == nullptr || h_sparse == nullptr || loss == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "h_full, h_sparse or loss is NULL");
  const long n = (long)P.d.B * P.d.Hq * P.d.Nq * P.d.D;
  const size_t need = (size_t)ssa::align_loss_partials(n) * sizeof(double);
  if (need > sizeof(scratch))
    return fail(SSA_ERR_UNSUPPORTED, "the loss needs %zu bytes of scratch; the no-allocation "
                "entry point holds %zu", need, sizeof(scratch));
  double* part = nullptr;
  if ((s = scratch_on(stream, &part)) != SSA_OK) return s;
  return hip_status(ssa::launch_align_loss(h_full, h_sparse, P.bf16, n, loss, grad_full,
                                           grad_sparse, part, (hipStream_t)stream),
                    "align loss (no allocation)");
}

size_t ssa_bwd_workspace_bytes(const ssa_problem* p) {
  Problem P;
  if (build(p, &P) != SSA_OK || P.decode) return 0;
  return bwd_layout_of(P).total;
}

ssa_status ssa_attn_bwd(const ssa_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* cnt, const void* h_full,
                        const void* h_sparse, const float* lse, const void* d_full,
                        const void* d_sparse, void* dq, void* dk, void* dv, void* ws,
                        size_t ws_bytes, void* stream) {
  Problem P;
  ssa_status s = build(p, &P);
  if (s != SSA_OK) return s;
  if (P.decode)
    return fail(SSA_ERR_UNSUPPORTED, "the backward pass needs a prefill problem (Nq == Nk)");
  if (q == nullptr || k == nullptr || v == nullptr || idx == nullptr || cnt == nullptr ||
      lse == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "q, k, v, idx, cnt or lse is NULL");
  if (dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "dq, dk or dv is NULL");
  if (d_full == nullptr && d_sparse == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "d_full and d_sparse are both NULL");
  if (d_full != nullptr && h_full == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "d_full needs h_full");
  if (d_sparse != nullptr && h_sparse == nullptr)
    return fail(SSA_ERR_INVALID_ARG, "d_sparse needs h_sparse");
  const BwdLayout L = bwd_layout_of(P);
  if (ws == nullptr) return fail(SSA_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(SSA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(SSA_ERR_WORKSPACE, "workspace has %zu bytes; %zu needed (ssa_bwd_workspace_bytes)",
                ws_bytes, L.total);
  const ssa::Dims& d = P.d;
  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  float* stats = (float*)(w + L.stats);
  hipError_t e = ssa::launch_attn_bwd_stats(h_full, h_sparse, d_full, d_sparse, lse, stats, P.bf16,
                                            d, st);
  if (e != hipSuccess) return hip_status(e, "backward statistics");
  if (!P.bf16)
    return hip_status(ssa::launch_attn_bwd_f32((const float*)q, (const float*)k, (const float*)v,
                                               (const float*)d_full, (const float*)d_sparse, idx,
                                               cnt, stats, (float*)dq, (float*)dk, (float*)dv, d,
                                               P.hm, st),
                      "backward (f32)");
  return hip_status(ssa::launch_attn_bwd_bf16((const uint16_t*)q, (const uint16_t*)k,
                                              (const uint16_t*)v, (const uint16_t*)d_full,
                                              (const uint16_t*)d_sparse, idx, cnt, stats,
                                              (uint16_t*)(w + L.bits),
                                              (uint64_t*)(w + L.rowbits), (float*)(w + L.pq),
                                              (float*)(w + L.pk), (float*)(w + L.pv),
                                              (float*)(w + L.sk), (float*)(w + L.sv), (uint16_t*)dq,
                                              (uint16_t*)dk, (uint16_t*)dv, d, P.hm, st),
                    "backward (bf16)");
}

const char* ssa_status_string(ssa_status s) {
  switch (s) {
    case SSA_OK: return "SSA_OK";
    case SSA_ERR_INVALID_ARG: return "SSA_ERR_INVALID_ARG";
    case SSA_ERR_UNSUPPORTED: return "SSA_ERR_UNSUPPORTED";
    case SSA_ERR_WORKSPACE: return "SSA_ERR_WORKSPACE";
    case SSA_ERR_HIP: return "SSA_ERR_HIP";
  }
  return "SSA_ERR_UNKNOWN";
}

const char* ssa_last_error_message(void) { return g_err; }

}  // extern "C"

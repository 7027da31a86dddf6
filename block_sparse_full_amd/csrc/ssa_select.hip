// Block mean-pool, block scoring and per-row top-k block selection.
//
// Method: "SSA: Achieving Sparser Attention by Aligning Full and Sparse
// Attention Outputs in Feature Space", section "Practical Implementation of
// SSA": blocks are mean-pooled, the query is scored against every earlier
// block representation (Mean(qK^T) = q Mean(K)^T keeps the ranking of the
// token-level scores) and the top-k blocks are kept.
//
// Precision contract (makes the selected indices reproducible bit for bit):
// pooled vectors are float64 sums in ascending token order, divided by the
// block size and rounded once to float32; scores are float64 dot products of
// the float32 pooled vectors accumulated in ascending d (a float32 x float32
// product is exact in float64, so fma and mul+add agree); ties go to the
// lower block index.
#include "ssa_common.h"
#include "ssa_kernels.h"

namespace ssa {

// ---------------------------------------------------------------- pooling
// One thread owns 8 consecutive d of one block and walks the block's tokens
// in order. x: [rows_total / bs, bs, D] viewed flat; out: [nblk_total, D].
__device__ __forceinline__ void load8(const uint16_t* p, float out[8]) {
  const uint4 u = *(const uint4*)p;
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float out[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ x,
                                                   float* __restrict__ out,
                                                   long nblk_total, int bs, int D) {
  const int per_blk = D / 8;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long blk = t / per_blk;
  if (blk >= nblk_total) return;
  const int d0 = (int)(t % per_blk) * 8;
  const T* src = x + blk * (long)bs * D + d0;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  for (int tok = 0; tok < bs; ++tok) {
    float v[8];
    load8(src + (long)tok * D, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += (double)v[i];
  }
  const double inv = 1.0 / (double)bs;  // bs is a power of two: exact
  float* dst = out + blk * D + d0;
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (float)(acc[i] * inv);
  *(float4*)dst = make_float4(r[0], r[1], r[2], r[3]);
  *(float4*)(dst + 4) = make_float4(r[4], r[5], r[6], r[7]);
}

hipError_t launch_pool(const void* x, bool bf16, float* out, long nblk_total, int bs,
                       int D, hipStream_t stream) {
  const long threads = nblk_total * (D / 8);
  const int wg = 256;
  const long grid = (threads + wg - 1) / wg;
  if (bf16)
    hipLaunchKernelGGL(pool_kernel<uint16_t>, dim3((unsigned)grid), dim3(wg), 0, stream,
                       (const uint16_t*)x, out, nblk_total, bs, D);
  else
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)grid), dim3(wg), 0, stream,
                       (const float*)x, out, nblk_total, bs, D);
  return hipGetLastError();
}

// ---------------------------------------------------------------- selection
// One workgroup (four waves) per (b, kv head, query row block). All threads
// first score the causal candidate blocks of up to `hc` q heads of the group
// at once (each pooled key row is read once for all of them) into LDS as
// 64-bit orderable keys. Then each wave selects for one head on its own,
// with no workgroup barrier: an exact radix select finds the free-th largest
// key 8 bits at a time from the most significant byte (per-wave LDS
// histogram, wave prefix scans); keys above it are taken and, among keys
// equal to it, the lowest block indices fill the remaining slots. The
// ascending index list is written by a ballot/popcount compaction over the
// causal blocks in order.
//
// Group-shared selection (d.group_select): all G heads are scored in one
// pass and only their sum is kept, added in the order of q_of_kv (ascending
// q head index) in float64 from zero; every wave then runs the same select
// on that single key row and writes the list for its heads.
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint64_t orderable_key(double s) {
  if (s == 0.0) s = 0.0;  // -0.0 and +0.0 rank equal
  const uint64_t b = (uint64_t)__double_as_longlong(s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ bool is_forced(int kb, int diag, int n_sink, int n_local) {
  return kb < n_sink || kb > diag - n_local;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar,
    int* __restrict__ idx, int* __restrict__ cnt, Dims d, HeadMap hm, int hc) {
  extern __shared__ __align__(16) unsigned char smem[];
  // layout: keys[hc or 1][nKB] u64 | qv[hc][D] f32
  uint64_t* keys = (uint64_t*)smem;
  float* qv = (float*)(smem + (size_t)(d.group_select ? 1 : hc) * d.nKB * sizeof(uint64_t));
  __shared__ unsigned hist[kSelWaves][256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int diag = row_block_diag(d, qb);
  const int ncausal = diag + 1;
  const float* krow0 = kbar + ((size_t)(b * d.Hkv + g) * d.nKB) * d.D;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes below

  // Forced set and slot count (identical for every head of the group).
  const int a_end = min(d.n_sink, ncausal);
  const int l_begin = max(0, ncausal - d.n_local);
  const int n_forced = a_end + (ncausal - l_begin) - max(0, a_end - l_begin);
  const int n_cand = ncausal - n_forced;
  const int free_slots = d.budget - n_forced;
  const bool take_all = n_cand <= free_slots;
  const bool forced_only = !take_all && free_slots <= 0;

  for (int h0 = 0; h0 < d.G; h0 += hc) {
    const int nh = min(hc, d.G - h0);
    __syncthreads();
    for (int i = tid; i < nh * d.D; i += kSelThreads) {
      const int hh = i / d.D, dd = i % d.D;
      const int h = hm.q_of_kv[g * d.G + h0 + hh];
      qv[i] = qbar[((size_t)(b * d.Hq + h) * d.nQB + qb) * d.D + dd];
    }
    __syncthreads();
    if (!take_all && !forced_only) {
      // Scores of every candidate for the nh heads.
      for (int kb = tid; kb < ncausal; kb += kSelThreads) {
        if (is_forced(kb, diag, d.n_sink, d.n_local)) continue;
        const float* kr = krow0 + (size_t)kb * d.D;
        double gsum = 0.0;
        for (int hb = 0; hb < nh; hb += 4) {
          double sc[4] = {0.0, 0.0, 0.0, 0.0};
          for (int dd = 0; dd < d.D; dd += 4) {
            const float4 k4 = *(const float4*)(kr + dd);
            const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const double kv = (double)kk[e];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (hb + j < nh) sc[j] = __fma_rn((double)qv[(hb + j) * d.D + dd + e], kv, sc[j]);
            }
          }
          if (d.group_select) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (hb + j < nh) gsum += sc[j];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (hb + j < nh) keys[(size_t)(hb + j) * d.nKB + kb] = orderable_key(sc[j]);
          }
        }
        if (d.group_select) keys[kb] = orderable_key(gsum);
      }
    }
    __syncthreads();

    // ---- per-wave selection, one head at a time
    for (int hh = wave; hh < nh; hh += kSelWaves) {
      const int h = hm.q_of_kv[g * d.G + h0 + hh];
      const uint64_t* hk = keys + (size_t)(d.group_select ? 0 : hh) * d.nKB;
      uint64_t thr = 0ull;   // keys above thr are taken
      int k_eq = 0;          // and this many of the keys equal to thr
      if (!take_all && !forced_only) {
        unsigned* hw = hist[wave];
        uint64_t prefix = 0ull, pmask = 0ull;
        int k = free_slots;
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
#pragma unroll
          for (int j = 0; j < 4; ++j) hw[lane * 4 + j] = 0u;
          wave_lds_fence();
          for (int kb = lane; kb < ncausal; kb += 64) {
            if (is_forced(kb, diag, d.n_sink, d.n_local)) continue;
            const uint64_t key = hk[kb];
            if ((key & pmask) == prefix) atomicAdd(&hw[(key >> shift) & 255u], 1u);
          }
          wave_lds_fence();
          // lane l owns bins 255-4l .. 252-4l (descending order)
          const int top = 255 - 4 * lane;
          const int c0 = (int)hw[top], c1 = (int)hw[top - 1], c2 = (int)hw[top - 2],
                    c3 = (int)hw[top - 3];
          const int csum = c0 + c1 + c2 + c3;
          const int incl = wave_incl_scan(csum);
          const int excl = incl - csum;
          const bool mine = excl < k && k <= incl;
          int bin = top, rest = k - excl, cbin = c0;
          if (rest > c0) { rest -= c0; bin = top - 1; cbin = c1;
            if (rest > c1) { rest -= c1; bin = top - 2; cbin = c2;
              if (rest > c2) { rest -= c2; bin = top - 3; cbin = c3; } } }
          const uint64_t ball = __builtin_amdgcn_ballot_w64(mine);
          const int src = ball ? __builtin_ctzll(ball) : 0;   // ball != 0 always
          const int sbin = __builtin_amdgcn_readlane(bin, src);
          const int scnt = __builtin_amdgcn_readlane(cbin, src);
          k = __builtin_amdgcn_readlane(rest, src);
          prefix |= (uint64_t)sbin << shift;
          pmask |= 0xFFull << shift;
          wave_lds_fence();
          // every remaining key of the chosen bin is taken: the selected keys
          // are exactly those >= prefix, and the lower digits need no pass
          if (scnt == k && prefix != 0ull) {
            prefix -= 1ull;
            k = 0;
            break;
          }
        }
        thr = prefix;
        k_eq = k;
      }
      // ---- ascending compaction over the causal blocks, 64 at a time
      const size_t row = (size_t)(b * d.Hq + h) * d.nQB + qb;
      int* out = idx + row * d.budget;
      int n_out = 0, eq_seen = 0;
      for (int base = 0; base < ncausal; base += 64) {
        const int kb = base + lane;
        const bool causal = kb < ncausal;
        const bool forced = causal && is_forced(kb, diag, d.n_sink, d.n_local);
        bool take = false, eq = false;
        if (causal && !forced) {
          if (take_all) {
            take = true;
          } else if (!forced_only) {
            const uint64_t key = hk[kb];
            take = key > thr;
            eq = key == thr;
          }
        }
        const uint64_t eq_ball = __builtin_amdgcn_ballot_w64(eq);
        if (eq) take = (eq_seen + __popcll(eq_ball & lt_mask)) < k_eq;
        eq_seen += __popcll(eq_ball);
        const bool sel = forced || take;
        const uint64_t sel_ball = __builtin_amdgcn_ballot_w64(sel);
        const int pos = n_out + __popcll(sel_ball & lt_mask);
        if (sel && pos < d.budget) out[pos] = kb;   // pos < budget always holds
        n_out += __popcll(sel_ball);
      }
      for (int i = n_out + lane; i < d.budget; i += 64) out[i] = -1;
      if (lane == 0) cnt[row] = min(n_out, d.budget);
    }
  }
}

int select_heads_per_pass(const Dims& d) {
  if (d.group_select) return d.G;   // one pass: every head feeds the one sum
  int hc = (int)(kSelKeyBytes / ((size_t)d.nKB * sizeof(uint64_t)));
  if (hc > d.G) hc = d.G;
  if (hc < 1) hc = 1;
  return hc;
}

size_t select_smem_bytes(const Dims& d, int hc) {
  const int key_rows = d.group_select ? 1 : hc;
  return (size_t)key_rows * d.nKB * sizeof(uint64_t) + (size_t)hc * d.D * sizeof(float);
}

hipError_t launch_select(const float* qbar, const float* kbar, int* idx, int* cnt,
                         const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const int hc = select_heads_per_pass(d);
  const size_t smem = select_smem_bytes(d, hc);
  hipLaunchKernelGGL(select_kernel, dim3(d.nQB, d.Hkv, d.B), dim3(kSelThreads), smem, stream,
                     qbar, kbar, idx, cnt, d, hm, hc);
  return hipGetLastError();
}

// ---------------------------------------------------------------- per-token selection
// Every query row scores its own query vector (as float32) against the
// pooled key blocks and keeps the top `free` candidates of the causal range
// of the block holding it; contract as above (float64 dot products in
// ascending d, ties to the lower block index).
//
// Lane = one query row (64 consecutive rows per wave, four independent waves
// per workgroup). The wave walks the key blocks in chunks of kTokChunk: the
// pooled keys of a chunk are wave-uniform, so they come as float64 scalar
// operands (from the chunked float64 copy kc), while the query stays in the
// lane's registers; one v_fma_f64 per (row, block, d). Each lane keeps its
// best candidates in a register list sorted by (key descending, block
// ascending) of KCAP entries; a new candidate is inserted below every entry
// with an equal or larger key, so among equal keys the earlier (lower) block
// stays ahead. Per chunk a lane marks the keys above its list's last entry
// and the wave inserts them in rounds, as many as the busiest lane needs.
// At the end the lane sorts its `free` picks by block index and writes sink
// blocks, picks and local blocks in ascending order.

// kc[bg][c][d][i] = (double)kbar[bg][kTokChunk*c + i][d], 0 past the last block.
__global__ __launch_bounds__(256) void kbar_f64_kernel(const float* __restrict__ kbar,
                                                       double* __restrict__ kc, int nKB, int nC,
                                                       int D, long total) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int i = (int)(t % kTokChunk);
  long r = t / kTokChunk;
  const int dd = (int)(r % D);
  r /= D;
  const int c = (int)(r % nC);
  const long bg = r / nC;
  const int kb = c * kTokChunk + i;
  kc[t] = kb < nKB ? (double)kbar[(bg * nKB + kb) * D + dd] : 0.0;
}

// Eight consecutive query values of a lane's row as float32.
__device__ __forceinline__ void load_q8(const uint16_t* p, float out[8]) { load8(p, out); }
__device__ __forceinline__ void load_q8(const float* p, float out[8]) { load8(p, out); }

template <int D, int KCAP, typename T>
__global__ __launch_bounds__(256) void select_tok_kernel(const T* __restrict__ q,
                                                         const double* __restrict__ kc,
                                                         int* __restrict__ idx,
                                                         int* __restrict__ cnt, Dims d,
                                                         HeadMap hm) {
  __shared__ uint64_t keys[4][kTokChunk][64];   // one chunk of keys per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  // heavier (later) rows first
  const int row0 = ((gridDim.x - 1 - blockIdx.x) * 4 + wave) * 64;
  if (row0 >= d.Nq) return;   // wave-uniform; Nq is a multiple of 64, no barrier below
  const int t = row0 + lane;
  const int g = hm.kv_of_q[h];
  const size_t bh = (size_t)b * d.Hq + h;
  const int nC = (d.nKB + kTokChunk - 1) / kTokChunk;
  const double* kg = kc + (size_t)(b * d.Hkv + g) * nC * D * kTokChunk;
  const T* qrow = q + (bh * d.Nq + t) * D;

  const int diag = (d.Nk - d.Nq + t) / d.bs;
  const int ncausal = diag + 1;
  const int a_end = min(d.n_sink, ncausal);
  const int l_begin = max(0, ncausal - d.n_local);
  const int n_forced = a_end + (ncausal - l_begin) - max(0, a_end - l_begin);
  const int free_slots = d.budget - n_forced;   // >= 0: budget >= n_sink + n_local
  // candidates: a_end <= kb < l_begin; the last row has the widest range
  const int wave_end = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(l_begin, 63));

  uint64_t lk[KCAP];
  int lb[KCAP];
#pragma unroll
  for (int j = 0; j < KCAP; ++j) { lk[j] = 0ull; lb[j] = 0; }
  uint64_t* wk = &keys[wave][0][0];

  for (int c0 = 0; c0 < wave_end; c0 += kTokChunk) {
    double acc[kTokChunk];
#pragma unroll
    for (int i = 0; i < kTokChunk; ++i) acc[i] = 0.0;
    const double* kp = kg + (size_t)(c0 / kTokChunk) * D * kTokChunk;
#pragma unroll 2
    for (int d8 = 0; d8 < D; d8 += 8) {
      float qv[8];
      load_q8(qrow + d8, qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double qd = (double)qv[e];
#pragma unroll
        for (int i = 0; i < kTokChunk; ++i)
          acc[i] = __fma_rn(qd, kp[(d8 + e) * kTokChunk + i], acc[i]);
      }
    }
    // keys that beat the list's last entry (the list only rises, so the
    // others cannot enter); the wave runs as many insertion rounds as its
    // busiest lane needs, each lane taking its next marked key
    uint32_t todo = 0u;
#pragma unroll
    for (int i = 0; i < kTokChunk; ++i) {
      const int kb = c0 + i;
      const uint64_t key = (kb >= a_end && kb < l_begin) ? orderable_key(acc[i]) : 0ull;
      wk[i * 64 + lane] = key;
      todo |= (key > lk[KCAP - 1]) ? 1u << i : 0u;
    }
    wave_lds_fence();
#pragma unroll 1
    while (__builtin_amdgcn_ballot_w64(todo != 0u) != 0ull) {
      const int i = todo != 0u ? __builtin_ctz(todo) : 0;
      const uint64_t key = todo != 0u ? wk[i * 64 + lane] : 0ull;   // key 0 inserts nothing
      todo &= todo - 1u;
      const int kb = c0 + i;
      // insert below every entry with key >= this one (bottom-up, in place)
#pragma unroll
      for (int j = KCAP - 1; j >= 0; --j) {
        const int jp = j > 0 ? j - 1 : 0;
        const bool here = key > lk[j];
        const bool above = j > 0 && key > lk[jp];
        const uint64_t nk = above ? lk[jp] : key;
        const int nb = above ? lb[jp] : kb;
        lk[j] = here ? nk : lk[j];
        lb[j] = here ? nb : lb[j];
      }
    }
    wave_lds_fence();
  }

  // picks: the first free_slots entries that hold a candidate, by block index
  int pk[KCAP];
  int np = 0;
#pragma unroll
  for (int j = 0; j < KCAP; ++j) {
    const bool use = j < free_slots && lk[j] != 0ull;
    pk[j] = use ? lb[j] : 0x7FFFFFFF;
    np += use ? 1 : 0;
  }
#pragma unroll 1
  for (int round = 0; round < KCAP; round += 2) {   // odd-even transposition sort
#pragma unroll
    for (int j = 0; j + 1 < KCAP; j += 2) {
      const int lo = min(pk[j], pk[j + 1]), hi = max(pk[j], pk[j + 1]);
      pk[j] = lo;
      pk[j + 1] = hi;
    }
#pragma unroll
    for (int j = 1; j + 1 < KCAP; j += 2) {
      const int lo = min(pk[j], pk[j + 1]), hi = max(pk[j], pk[j + 1]);
      pk[j] = lo;
      pk[j + 1] = hi;
    }
  }

  int* out = idx + (bh * d.Nq + t) * d.budget;
  int pos = 0;
  for (int kb = 0; kb < a_end; ++kb) out[pos++] = kb;
#pragma unroll
  for (int j = 0; j < KCAP; ++j)
    if (j < np) out[pos + j] = pk[j];
  pos += np;
  for (int kb = max(l_begin, a_end); kb <= diag; ++kb) out[pos++] = kb;
  const int n_out = pos;
  for (; pos < d.budget; ++pos) out[pos] = -1;
  cnt[bh * d.Nq + t] = n_out;
}

template <int D, typename T>
static void launch_tok(const void* q, const double* kc, int* idx, int* cnt, const Dims& d,
                       const HeadMap& hm, hipStream_t stream) {
  const dim3 grid((d.Nq + 255) / 256, d.Hq, d.B);
  const T* qt = (const T*)q;
  if (d.budget <= 16)
    hipLaunchKernelGGL((select_tok_kernel<D, 16, T>), grid, dim3(256), 0, stream, qt, kc, idx,
                       cnt, d, hm);
  else if (d.budget <= 32)
    hipLaunchKernelGGL((select_tok_kernel<D, 32, T>), grid, dim3(256), 0, stream, qt, kc, idx,
                       cnt, d, hm);
  else
    hipLaunchKernelGGL((select_tok_kernel<D, 64, T>), grid, dim3(256), 0, stream, qt, kc, idx,
                       cnt, d, hm);
}

hipError_t launch_select_tok(const void* q, bool bf16, const float* kbar, double* kc, int* idx,
                             int* cnt, const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const int nC = (d.nKB + kTokChunk - 1) / kTokChunk;
  const long total = (long)d.B * d.Hkv * nC * d.D * kTokChunk;
  hipLaunchKernelGGL(kbar_f64_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     kbar, kc, d.nKB, nC, d.D, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.D == 128) {
    if (bf16) launch_tok<128, uint16_t>(q, kc, idx, cnt, d, hm, stream);
    else launch_tok<128, float>(q, kc, idx, cnt, d, hm, stream);
  } else {
    if (bf16) launch_tok<64, uint16_t>(q, kc, idx, cnt, d, hm, stream);
    else launch_tok<64, float>(q, kc, idx, cnt, d, hm, stream);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- V transpose
// vt[bh][d][n] = v[bh][n][d] for bf16, 64x64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ v,
                                                        uint16_t* __restrict__ vt, int N, int D,
                                                        int* __restrict__ queues) {
  __shared__ uint16_t tile[64][66];
  if (queues != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 &&
      threadIdx.x < kNumXcd)
    queues[threadIdx.x * kQueueStride] = 0;
  const int n0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const size_t bh = blockIdx.z;
  const uint16_t* src = v + bh * (size_t)N * D;
  uint16_t* dst = vt + bh * (size_t)N * D;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) tile[r][tx] = src[(size_t)(n0 + r) * D + d0 + tx];
  __syncthreads();
  for (int r = ty; r < 64; r += 4) dst[(size_t)(d0 + r) * N + n0 + tx] = tile[tx][r];
}

hipError_t launch_transpose(const uint16_t* v, uint16_t* vt, int BH, int N, int D, int* queues,
                            hipStream_t stream) {
  hipLaunchKernelGGL(transpose_kernel, dim3(N / 64, D / 64, BH), dim3(256), 0, stream, v, vt,
                     N, D, queues);
  return hipGetLastError();
}

}  // namespace ssa

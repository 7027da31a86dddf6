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
  // eight tokens' loads in flight ahead of the ascending-order adds
  int tok = 0;
  for (; tok + 8 <= bs; tok += 8) {
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8(src + (long)(tok + u) * D, v[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (double)v[u][i];
  }
  for (; tok < bs; ++tok) {
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
// (one candidate per lane, four heads per pass over its pooled key row; the
// heads' pooled queries sit in LDS as float64 and reach the multiply-adds by
// row broadcasts) into LDS as 64-bit orderable keys. Then each wave selects
// for one head on its own, with no workgroup barrier (select_row_wave): the
// keys that can be taken are bounded from below, gathered and ranked
// directly, or an exact radix select finds the free-th largest key; keys
// above it are taken and, among keys equal to it, the lowest block indices
// fill the remaining slots.
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

// The k-th largest (1 <= k <= 64) of the 64 lanes' values v, counting equal
// values separately: the value of a lane with fewer than k values above it
// and at least k at or above it. The values pass through hw (512 bytes of
// LDS), where every lane reads all of them (same address in every lane).
__device__ __forceinline__ uint64_t wave_kth_largest(uint64_t v, int k, unsigned* hw) {
  const int lane = threadIdx.x & 63;
  uint64_t* sv = (uint64_t*)hw;
  sv[lane] = v;
  wave_lds_fence();
  int gt = 0, ge = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 2) {
    const ulonglong2 o = *(const ulonglong2*)(sv + j);
    gt += (int)(o.x > v) + (int)(o.y > v);
    ge += (int)(o.x >= v) + (int)(o.y >= v);
  }
  const uint64_t at = __builtin_amdgcn_ballot_w64(gt < k && k <= ge);
  const uint64_t r = sv[__builtin_ctzll(at)];   // some lane always qualifies
  wave_lds_fence();
  return r;
}

// Gathers the candidate keys of a selection row for which in(key) holds into
// hw (one slot each, ascending block order; slots past 64 are not written)
// and returns how many there are. hw needs 768 bytes: 64 keys, 64 blocks.
template <typename Pred>
__device__ __forceinline__ int gather_few(const uint64_t* hk, unsigned* hw, const Dims& d,
                                          int diag, int ncausal, uint64_t lt_mask, Pred in_set) {
  const int lane = threadIdx.x & 63;
  uint64_t* ck = (uint64_t*)hw;
  int* cb = (int*)(ck + 64);
  int n = 0;
  for (int kb0 = 0; kb0 < ncausal; kb0 += 64 * 4) {
    uint64_t v[4];   // the reads first: the slot writes below may alias hk
    bool c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = kb0 + 64 * j + lane;
      c[j] = kb < ncausal && !is_forced(kb, diag, d.n_sink, d.n_local);
      v[j] = c[j] ? hk[kb] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = kb0 + 64 * j + lane;
      const bool in = c[j] && in_set(v[j]);
      const uint64_t ball = __builtin_amdgcn_ballot_w64(in);
      const int pos = n + __popcll(ball & lt_mask);
      if (in && pos < 64) {
        ck[pos] = v[j];
        cb[pos] = kb;
      }
      n += __popcll(ball);
    }
  }
  wave_lds_fence();
  return n;
}

// Rank of this lane's entry among the n <= 64 keys gather_few left in hw
// (larger key first, equal keys by ascending block; entries past n and
// lanes >= n get meaningless ranks): each lane reads every entry (the same
// address in all lanes, two per read).
__device__ __forceinline__ int rank_few(const unsigned* hw, int n) {
  const int lane = threadIdx.x & 63;
  const uint64_t* ck = (const uint64_t*)hw;
  const int* cb = (const int*)(ck + 64);
  const uint64_t mk = ck[lane];
  const int mb = cb[lane];
  int rank = 0;
  for (int j = 0; j < n; j += 2) {   // entry n (when n is odd) is in bounds
    const ulonglong2 o = *(const ulonglong2*)(ck + j);
    const int2 ob = *(const int2*)(cb + j);
    rank += (int)(o.x > mk) | ((int)(o.x == mk) & (int)(ob.x < mb));
    if (j + 1 < n) rank += (int)(o.y > mk) | ((int)(o.y == mk) & (int)(ob.y < mb));
  }
  return rank;
}

// From the ranks of the n gathered keys: thr, the key of rank k - 1
// (1 <= k <= n), and k_eq, how many keys equal to it rank below k. Taking
// every key above thr and the first k_eq keys equal to it in block order
// takes exactly the k highest-ranked keys.
__device__ __forceinline__ void threshold_of_ranks(const unsigned* hw, int n, int k, int rank,
                                                   uint64_t& thr, int& k_eq) {
  const int lane = threadIdx.x & 63;
  const uint64_t* ck = (const uint64_t*)hw;
  const bool valid = lane < n;
  const uint64_t mk = ck[lane];
  const uint64_t at = __builtin_amdgcn_ballot_w64(valid && rank == k - 1);
  thr = ck[__builtin_ctzll(at)];   // ranks are distinct: exactly one lane
  k_eq = __popcll(__builtin_amdgcn_ballot_w64(valid && mk == thr && rank < k));
  wave_lds_fence();
}

// Writes a selection row whose free picks are the gathered entries (hw,
// ascending block order) of the lanes in `picks`: the sink blocks, the
// picks, then the local blocks, all ascending. Valid when candidates exist
// between the sink and local ranges (so the two do not overlap) and exactly
// free_slots entries are picked: the row is then full.
__device__ __forceinline__ void write_picked_row(const unsigned* hw, uint64_t picks,
                                                 int* __restrict__ out, int* __restrict__ cnt,
                                                 size_t row, const Dims& d, int ncausal) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int* cb = (const int*)((const uint64_t*)hw + 64);
  const int a_end = min(d.n_sink, ncausal);
  const int l_begin = max(0, ncausal - d.n_local);
  const int n_pick = __popcll(picks);
  for (int i = lane; i < a_end; i += 64) out[i] = i;
  if ((picks >> lane) & 1ull) out[a_end + __popcll(picks & lt_mask)] = cb[lane];
  for (int i = lane; i < ncausal - l_begin; i += 64) out[a_end + n_pick + i] = l_begin + i;
  if (lane == 0) cnt[row] = a_end + n_pick + (ncausal - l_begin);
  wave_lds_fence();
}

// One 64-block step of the ascending compaction: block kb of this lane is
// taken when forced, when its key is above thr, or when it equals thr and is
// among the first k_eq such blocks; positions come from ballots.
__device__ __forceinline__ void compact_step(int kb, bool causal, bool forced, uint64_t key,
                                             bool take_all, bool forced_only, uint64_t thr,
                                             int k_eq, uint64_t lt_mask, int* out, int budget,
                                             int& n_out, int& eq_seen) {
  const bool cand = causal && !forced;
  bool take = false, eq = false;
  if (cand) {
    if (take_all) {
      take = true;
    } else if (!forced_only) {
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
  if (sel && pos < budget) out[pos] = kb;   // pos < budget always holds
  n_out += __popcll(sel_ball);
}

// Top-k of one selection row by one wave, then the ascending list of forced
// blocks and picks (ties to the lower index) written to idx row `row` and
// its count. The picks are found in one of two exact ways, both over hk
// with hw (1 KB of LDS) as scratch:
// - free <= 64: each lane's largest candidate key; the free-th largest of
//   those 64 bounds the threshold from below (the lanes at or above it hold
//   free distinct keys at least as large), so only the keys at or above it
//   can be taken. When at most 64 keys are (the usual case: about 1.5 x free
//   for random scores) they are gathered in block order and ranked
//   directly; the picks are those ranked below free, written between the
//   sink and local blocks with no second pass over the row.
// - otherwise a radix select, 8 bits per pass from the most significant
//   byte (a 256-bin histogram per pass, wave prefix scans), until the bin
//   that holds the threshold is taken whole or has at most 64 keys, which
//   are then ranked directly.
__device__ void select_row_wave(const uint64_t* hk, unsigned* hw, int* __restrict__ idx,
                                int* __restrict__ cnt, size_t row, const Dims& d, int diag,
                                int ncausal, int free_slots, bool take_all, bool forced_only) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes below
  uint64_t thr = 0ull;   // keys above thr are taken
  int k_eq = 0;          // and this many of the keys equal to thr
  if (!take_all && !forced_only) {
    bool found = false;
    if (free_slots <= 64) {
      uint64_t lmax = 0ull;   // below every key of a finite score
      for (int kb0 = 0; kb0 < ncausal; kb0 += 64 * 4) {
        uint64_t v[4];   // four LDS reads in flight, then the maxima
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kb = kb0 + 64 * j + lane;
          v[j] = (kb < ncausal && !is_forced(kb, diag, d.n_sink, d.n_local)) ? hk[kb] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) lmax = v[j] > lmax ? v[j] : lmax;
      }
      const uint64_t t0 = wave_kth_largest(lmax, free_slots, hw);
      const int n = gather_few(hk, hw, d, diag, ncausal, lt_mask,
                               [t0](uint64_t key) { return key >= t0; });
      if (n <= 64) {   // every key that can be taken is gathered: no scan
        const int rank = rank_few(hw, n);
        const uint64_t picks = __builtin_amdgcn_ballot_w64(lane < n && rank < free_slots);
        write_picked_row(hw, picks, idx + row * d.budget, cnt, row, d, ncausal);
        return;
      }
    }
    uint64_t prefix = 0ull, pmask = 0ull;
    int k = free_slots;
    for (int pass = 0; pass < 8 && !found; ++pass) {
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
        thr = prefix - 1ull;
        k_eq = 0;
        found = true;
      } else if (scnt <= 64) {
        const int n = gather_few(hk, hw, d, diag, ncausal, lt_mask,
                                 [prefix, pmask](uint64_t key) { return (key & pmask) == prefix; });
        threshold_of_ranks(hw, n, k, rank_few(hw, n), thr, k_eq);
        found = true;
      }
    }
    if (!found) {   // eight passes: every remaining key equals prefix
      thr = prefix;
      k_eq = k;
    }
  }
  // ---- ascending compaction over the causal blocks, 64 at a time
  int* out = idx + row * d.budget;
  int n_out = 0, eq_seen = 0;
  for (int base = 0; base < ncausal; base += 64) {
    const int kb = base + lane;
    const bool causal = kb < ncausal;
    const bool forced = causal && is_forced(kb, diag, d.n_sink, d.n_local);
    const uint64_t key = (causal && !forced && !take_all && !forced_only) ? hk[kb] : 0ull;
    compact_step(kb, causal, forced, key, take_all, forced_only, thr, k_eq, lt_mask, out,
                 d.budget, n_out, eq_seen);
  }
  for (int i = n_out + lane; i < d.budget; i += 64) out[i] = -1;
  if (lane == 0) cnt[row] = min(n_out, d.budget);
}

// Sixteen float64 multiply-adds of one step of four d for four heads:
// sc[j] += q[j][d + e] * kv[e], e ascending. q holds the step's sixteen
// query values, lane 4 e + j of each row of 16 lanes holding q[j][d + e]
// (the same in all four rows); each multiply-add takes its query value from
// that lane by a row broadcast (DPP row_newbcast), so the query needs no
// scalar register and no per-lane copy. Every lane of the wave must be
// active (a broadcast from an inactive lane reads nothing). The leading
// wait states cover a VGPR or EXEC write just before the block (two and
// five are required before a DPP read); inside the block each accumulator
// is rewritten four instructions after its last use.
template <int NOPS>
__device__ __forceinline__ void fma16_bcast(double sc[4], double q, const double kv[4]) {
  asm("s_nop %9\n\t"
      "v_fmac_f64_dpp %0, %4, %5 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %1, %4, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %2, %4, %5 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %3, %4, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %1, %4, %6 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %2, %4, %6 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %3, %4, %6 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %7 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %1, %4, %7 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %2, %4, %7 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %3, %4, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %1, %4, %8 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %2, %4, %8 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %3, %4, %8 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "+v"(sc[0]), "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3])
      : "v"(q), "v"(kv[0]), "v"(kv[1]), "v"(kv[2]), "v"(kv[3]), "i"(NOPS));
}

// Scores of the pooled key row kr (float32, D values) against four query
// rows: float64 fused multiply-adds in ascending d into sc[j]. qs points at
// this lane's slot of the four rows' step-major float64 copy in LDS
// (qs[16 st] = q[j][4 st + e] for lane 4 e + j of its row). The key row is
// read a whole 128-byte line (32 floats) at a time with the next line in
// flight.
template <int D>
__device__ __forceinline__ void score_bcast(const float* __restrict__ kr, const double* qs,
                                            double sc[4]) {
  constexpr int NC = D / 32;
  float4 f[2][8];
  auto load32 = [&](float4* dst, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = *(const float4*)(kr + 32 * c + 4 * i);
  };
  load32(f[0], 0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + 1 < NC) load32(f[(c + 1) & 1], c + 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int st = 8 * c + i;
      const double q = qs[16 * st];
      const float4 k4 = f[c & 1][i];
      const double kv[4] = {(double)k4.x, (double)k4.y, (double)k4.z, (double)k4.w};
      if (st == 0)
        fma16_bcast<4>(sc, q, kv);
      else
        fma16_bcast<1>(sc, q, kv);
    }
  }
}

// Four waves per SIMD (at most 128 VGPRs): the compiler's own choice of
// 138 left three, 8 % slower.
template <int D>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(4))) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar,
    int* __restrict__ idx, int* __restrict__ cnt, Dims d, HeadMap hm, int hc) {
  extern __shared__ __align__(16) unsigned char smem[];
  // keys [hc, or 1 with group-shared selection][nKB] | qd [ceil(hc / 4)][D / 4][16]
  uint64_t* keys = (uint64_t*)smem;
  double* qd = (double*)(smem + (size_t)(d.group_select ? 1 : hc) * d.nKB * sizeof(uint64_t));
  __shared__ __align__(16) unsigned hist[kSelWaves][256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int diag = row_block_diag(d, qb);
  const int ncausal = diag + 1;
  const float* krow0 = kbar + ((size_t)(b * d.Hkv + g) * d.nKB) * D;
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
    if (h0 > 0) __syncthreads();   // the last pass's selections are done with keys
    if (!take_all && !forced_only) {
      // The nh heads' pooled queries widened to float64 in LDS, step-major
      // (heads padded to a multiple of four with copies of the last).
      const int nhp = (nh + 3) & ~3;
      for (int i = tid; i < nhp * D; i += kSelThreads) {
        const int hj = i / D, dd = i % D;
        const int h = hm.q_of_kv[g * d.G + h0 + min(hj, nh - 1)];
        qd[((hj >> 2) * (D / 4) + (dd >> 2)) * 16 + (dd & 3) * 4 + (hj & 3)] =
            (double)qbar[((size_t)(b * d.Hq + h) * d.nQB + qb) * D + dd];
      }
      __syncthreads();
      // Scores of every candidate for the nh heads, one candidate per lane;
      // the loop is wave-uniform (past the causal range a lane scores the
      // last causal block and keeps nothing) so every lane stays active for
      // the row broadcasts.
      for (int base = wave * 64; base < ncausal; base += kSelThreads) {
        const int kb = base + lane;
        const bool ok = kb < ncausal && !is_forced(kb, diag, d.n_sink, d.n_local);
        const float* kr = krow0 + (size_t)min(kb, ncausal - 1) * D;
        double gsum = 0.0;
        for (int hb = 0; hb < nh; hb += 4) {
          // the row through an offset the compiler cannot see is zero: its
          // loads and widening stay in this loop rather than being hoisted
          // out of it as live values for every d
          int z;
          asm("v_mov_b32 %0, 0" : "=v"(z) : "s"(hb));
          double sc[4] = {0.0, 0.0, 0.0, 0.0};
          score_bcast<D>(kr + z, qd + (hb >> 2) * (D / 4) * 16 + (lane & 15), sc);
          if (ok) {
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
        }
        if (d.group_select && ok) keys[kb] = orderable_key(gsum);
      }
    }
    __syncthreads();

    // ---- per-wave selection, one head at a time
    for (int hh = wave; hh < nh; hh += kSelWaves) {
      const int h = hm.q_of_kv[g * d.G + h0 + hh];
      const uint64_t* hk = keys + (size_t)(d.group_select ? 0 : hh) * d.nKB;
      const size_t row = (size_t)(b * d.Hq + h) * d.nQB + qb;
      select_row_wave(hk, hist[wave], idx, cnt, row, d, diag, ncausal, free_slots, take_all,
                      forced_only);
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
  return (size_t)key_rows * d.nKB * sizeof(uint64_t) +
         (size_t)((hc + 3) / 4) * 4 * d.D * sizeof(double);
}

// Decode scoring: one lane per candidate key block, 64 candidates per
// workgroup, all q heads of the group (the single query of each head is its
// block representation: its values, read from q four at a time as scalar
// operands and widened exactly, are what pooling one token gives). The same
// float64 ascending-d dot products and orderable keys as select_kernel's
// own scoring, written to gkeys [B, Hkv, G, nKB] (or the
// group sum to [B, Hkv, nKB] with group-shared selection); forced and
// non-causal blocks are not written. Spreading the pooled-key table over
// B * Hkv * nKB / 64 workgroups keeps enough loads in flight to stream it;
// each lane reads its own row a whole 128-byte line (32 floats) at a time
// with the next line in flight. Reading half lines let the L2 drop a line
// between its two halves and fetch it twice (39 % more HBM reads than the
// table). (Staging the rows through LDS for coalesced loads measured slower:
// the LDS per workgroup, or the extra passes, cost more occupancy than the
// scattered 16-byte loads cost bandwidth.)

// Four query values widened exactly to float64 (float32 or bfloat16).
__device__ __forceinline__ void q4_f64(const float* p, double o[4]) {
  const float4 f = *(const float4*)p;
  o[0] = (double)f.x; o[1] = (double)f.y; o[2] = (double)f.z; o[3] = (double)f.w;
}
__device__ __forceinline__ void q4_f64(const uint16_t* p, double o[4]) {
  const uint2 w = *(const uint2*)p;
  o[0] = (double)__uint_as_float(w.x << 16);
  o[1] = (double)__uint_as_float(w.x & 0xFFFF0000u);
  o[2] = (double)__uint_as_float(w.y << 16);
  o[3] = (double)__uint_as_float(w.y & 0xFFFF0000u);
}

// Scores of one pooled key row kr (float32, D values) against four query
// rows qv[j] (wave-uniform addresses: scalar loads): float64 fused
// multiply-adds in ascending d into sc[j]. The key row is read a whole
// 128-byte line (32 floats) at a time with the next line in flight.
template <int D, typename QT>
__device__ __forceinline__ void score4(const float* __restrict__ kr, const QT* const qv[4],
                                       double sc[4]) {
  auto load32 = [&](float4* f, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = *(const float4*)(kr + 32 * c + 4 * i);
  };
  auto fma32 = [&](const float4* f, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float kk[4] = {f[i].x, f[i].y, f[i].z, f[i].w};
      double qq[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q4_f64(qv[j] + 32 * c + 4 * i, qq[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double kv = (double)kk[e];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = __fma_rn(qq[j][e], kv, sc[j]);
      }
    }
  };
  float4 fa[8], fb[8];
  load32(fa, 0);
#pragma unroll 1
  for (int c = 0; c < D / 32; c += 2) {
    load32(fb, c + 1);
    fma32(fa, c);
    if (c + 2 < D / 32) load32(fa, c + 2);
    fma32(fb, c + 1);
  }
}

template <int D, typename QT>
__global__ __launch_bounds__(64) void decode_score_kernel(const QT* __restrict__ q,
                                                          const float* __restrict__ kbar,
                                                          uint64_t* __restrict__ gkeys, Dims d,
                                                          HeadMap hm) {
  const int kb = blockIdx.x * 64 + (int)threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int diag = row_block_diag(d, 0);
  if (kb > diag || is_forced(kb, diag, d.n_sink, d.n_local)) return;
  const float* kr = kbar + ((size_t)(b * d.Hkv + g) * d.nKB + kb) * D;
  const size_t krow0 = (size_t)(b * d.Hkv + g);
  double gsum = 0.0;
  for (int hb = 0; hb < d.G; hb += 4) {
    const QT* qv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = hm.q_of_kv[g * d.G + min(hb + j, d.G - 1)];
      qv[j] = q + (size_t)(b * d.Hq + h) * D;   // Nq == 1
    }
    double sc[4] = {0.0, 0.0, 0.0, 0.0};
    score4<D>(kr, qv, sc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (hb + j >= d.G) break;
      if (d.group_select) gsum += sc[j];
      else gkeys[(krow0 * d.G + hb + j) * d.nKB + kb] = orderable_key(sc[j]);
    }
  }
  if (d.group_select) gkeys[krow0 * d.nKB + kb] = orderable_key(gsum);
}

// Decode top-k: one wave per (b, q head) on the keys of decode_score_kernel
// (copied to LDS), the same radix select and compaction as select_kernel.
__global__ __launch_bounds__(64) void decode_select_kernel(const uint64_t* __restrict__ gkeys,
                                                           int* __restrict__ idx,
                                                           int* __restrict__ cnt, Dims d,
                                                           HeadMap hm) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* keys = (uint64_t*)smem;   // [nKB]
  __shared__ __align__(16) unsigned hist[256];
  const int lane = (int)threadIdx.x;
  const int hh = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int h = hm.q_of_kv[g * d.G + hh];
  const int diag = row_block_diag(d, 0);
  const int ncausal = diag + 1;
  const int a_end = min(d.n_sink, ncausal);
  const int l_begin = max(0, ncausal - d.n_local);
  const int n_forced = a_end + (ncausal - l_begin) - max(0, a_end - l_begin);
  const int n_cand = ncausal - n_forced;
  const int free_slots = d.budget - n_forced;
  const bool take_all = n_cand <= free_slots;
  const bool forced_only = !take_all && free_slots <= 0;
  const size_t row = (size_t)(b * d.Hq + h);
  const size_t krow = d.group_select ? (size_t)(b * d.Hkv + g) : (size_t)(b * d.Hkv + g) * d.G + hh;
  const uint64_t* src = gkeys + krow * d.nKB;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (!take_all && !forced_only && ncausal <= 64 * 16 && free_slots <= 64) {
    // keys in registers (candidate kb = 64 j + lane): no LDS copy; the
    // threshold from the lane-maximum bound and a direct ranking, as in
    // select_row_wave
    uint64_t key[16];
    uint64_t lmax = 0ull;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kb = 64 * j + lane;
      key[j] = (kb < ncausal && !is_forced(kb, diag, d.n_sink, d.n_local)) ? src[kb] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) lmax = key[j] > lmax ? key[j] : lmax;
    const uint64_t t0 = wave_kth_largest(lmax, free_slots, hist);
    uint64_t* ck = (uint64_t*)hist;
    int* cb = (int*)(ck + 64);
    int n = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kb = 64 * j + lane;
      const bool in = kb < ncausal && !is_forced(kb, diag, d.n_sink, d.n_local) && key[j] >= t0;
      const uint64_t ball = __builtin_amdgcn_ballot_w64(in);
      const int pos = n + __popcll(ball & lt_mask);
      if (in && pos < 64) {
        ck[pos] = key[j];
        cb[pos] = kb;
      }
      n += __popcll(ball);
    }
    wave_lds_fence();
    if (n <= 64) {   // every key that can be taken is gathered
      const int rank = rank_few(hist, n);
      const uint64_t picks = __builtin_amdgcn_ballot_w64(lane < n && rank < free_slots);
      write_picked_row(hist, picks, idx + row * d.budget, cnt, row, d, ncausal);
      return;
    }
  }
  if (!take_all && !forced_only) {
    // all loads of a group of 16 in flight before the LDS writes (one at a
    // time, each waiting for the last, took most of the kernel's time); the
    // forced blocks' entries, never written by the scoring, are copied too
    // and never read as candidates
    for (int kb0 = 0; kb0 < ncausal; kb0 += 64 * 16) {
      uint64_t v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kb = kb0 + 64 * j + lane;
        v[j] = kb < ncausal ? src[kb] : 0ull;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kb = kb0 + 64 * j + lane;
        if (kb < ncausal) keys[kb] = v[j];
      }
    }
    wave_lds_fence();
  }
  select_row_wave(keys, hist, idx, cnt, row, d, diag, ncausal, free_slots, take_all,
                  forced_only);
}

hipError_t launch_select_decode(const void* q, bool bf16, const float* kbar, int* idx, int* cnt,
                                const Dims& d, const HeadMap& hm, uint64_t* gkeys,
                                hipStream_t stream) {
  const dim3 grid((d.nKB + 63) / 64, d.Hkv, d.B);
  if (bf16) {
    const uint16_t* qq = (const uint16_t*)q;
    if (d.D == 128)
      hipLaunchKernelGGL((decode_score_kernel<128, uint16_t>), grid, dim3(64), 0, stream, qq,
                         kbar, gkeys, d, hm);
    else
      hipLaunchKernelGGL((decode_score_kernel<64, uint16_t>), grid, dim3(64), 0, stream, qq,
                         kbar, gkeys, d, hm);
  } else {
    const float* qq = (const float*)q;
    if (d.D == 128)
      hipLaunchKernelGGL((decode_score_kernel<128, float>), grid, dim3(64), 0, stream, qq, kbar,
                         gkeys, d, hm);
    else
      hipLaunchKernelGGL((decode_score_kernel<64, float>), grid, dim3(64), 0, stream, qq, kbar,
                         gkeys, d, hm);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3(d.G, d.Hkv, d.B), dim3(64),
                     (size_t)d.nKB * sizeof(uint64_t), stream, gkeys, idx, cnt, d, hm);
  return hipGetLastError();
}

hipError_t launch_select(const float* qbar, const float* kbar, int* idx, int* cnt,
                         const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const int hc = select_heads_per_pass(d);
  const size_t smem = select_smem_bytes(d, hc);
  const dim3 grid(d.nQB, d.Hkv, d.B);
  if (d.D == 128)
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(kSelThreads), smem, stream, qbar, kbar, idx,
                       cnt, d, hm, hc);
  else
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(kSelThreads), smem, stream, qbar, kbar, idx,
                       cnt, d, hm, hc);
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
// vt[bh][d][n] = v[bh][n][d] for bf16, 64x64 tiles through LDS; or, with
// blk16, vt[bh][n/16][d][n%16]: the V^T of each 16-key block contiguous (D x
// 16 keys), for the gather kernel of sparse-only 16-token blocks.
template <bool BLK16>
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ v,
                                                        uint16_t* __restrict__ vt, int N, int D,
                                                        int* __restrict__ queues,
                                                        const uint16_t* __restrict__ k,
                                                        float* __restrict__ kn) {
  __shared__ uint16_t tile[64][66];
  if (kn != nullptr && blockIdx.y == 0) {
    // The largest key norm of this 64-key block: four threads per key, each
    // summing squares over a quarter of the 16-byte chunks, then maxima over
    // the wave's 16 keys and the four waves.
    __shared__ float wmax[4];
    const int key = threadIdx.x >> 2, part = threadIdx.x & 3;
    const uint16_t* kr = k + (blockIdx.z * (size_t)N + blockIdx.x * 64 + key) * D;
    float ss = 0.f;
    for (int c = part; c < D / 8; c += 4) {
      const uint4 u = *(const uint4*)(kr + 8 * c);
      const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) ss = fmaxf(ss, __shfl_xor(ss, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0)
      kn[blockIdx.z * (size_t)(N / 64) + blockIdx.x] =
          sqrtf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
  }
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
  for (int r = ty; r < 64; r += 4) {
    const int n = n0 + tx, dd = d0 + r;
    const size_t o = BLK16 ? ((size_t)(n >> 4) * D + dd) * 16 + (n & 15) : (size_t)dd * N + n;
    dst[o] = tile[tx][r];
  }
}

hipError_t launch_transpose(const uint16_t* v, uint16_t* vt, int BH, int N, int D, int* queues,
                            bool blk16, const uint16_t* k, float* kn, hipStream_t stream) {
  if (blk16)
    hipLaunchKernelGGL(transpose_kernel<true>, dim3(N / 64, D / 64, BH), dim3(256), 0, stream, v,
                       vt, N, D, queues, k, kn);
  else
    hipLaunchKernelGGL(transpose_kernel<false>, dim3(N / 64, D / 64, BH), dim3(256), 0, stream, v,
                       vt, N, D, queues, k, kn);
  return hipGetLastError();
}

}  // namespace ssa

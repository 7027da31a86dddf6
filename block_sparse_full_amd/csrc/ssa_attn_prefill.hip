// Fused dual-stream causal attention forward (prefill): two bf16 MFMA kernels
// (one workgroup per q head and query block; one workgroup per kv head and
// query block serving four q heads, for D = 128 and GQA groups of 4k) and a
// float32 VALU kernel for float32 problems.
//
// Method: "SSA: Achieving Sparser Attention by Aligning Full and Sparse
// Attention Outputs in Feature Space": the full attention stream (section
// "SSA's Dual-Stream Training Mechanism") and the block-sparse stream over
// the concatenated selected blocks (section "Practical Implementation of
// SSA"), plus the dropped mass delta(t) ("Technische Samenvatting: SSA",
// "2. Methodologie").
//
// One pass serves both streams. A row's sparse softmax is its full softmax
// restricted to the selected keys and renormalised, so the kernel walks the
// selected blocks of the query block first, snapshots
//     h_sparse = acc / l_sel
// and then continues over the remaining causal blocks with the same running
// max and accumulator, giving
//     h_full = acc / (l_sel + l_drop),   delta = l_drop / (l_sel + l_drop).
// Every key block's QK^T and PV run exactly once, so the executed MFMA work
// equals that of full causal attention alone.
#include "ssa_common.h"
#include "ssa_device.h"
#include "ssa_kernels.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace ssa {

// c + a.x + a.y for two packed bfloat16 values, in one instruction. The row
// sums of both bf16 kernels add the bfloat16 weights that the PV MFMAs
// apply to V, so each output row is normalised by exactly its own weights.
__device__ __forceinline__ float add_bf16x2(uint32_t a, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), c, false);
}

// LDS tiles are stored without padding; 16-byte chunks are XOR-swizzled per
// row so that the ds_read_b128 of 16 lanes (16 different rows, same logical
// chunk) hit 16 distinct 16-byte bank groups. V^T rows are 128 bytes (two
// rows per 256-byte bank sweep) and the 16 rows of one read are consecutive:
// chunk ^ ((row >> 1) & 7) separates them.
__device__ __forceinline__ int vswz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Buffer resource over [base, base + bytes): loads past the end read 0. The
// base is made wave-uniform explicitly so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* u = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Largest of x over the four lanes n, n+16, n+32, n+48 (one query column of
// a 16x16 MFMA tile), and the same for sums.
__device__ __forceinline__ float quad_max(float x) {
  unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  u = __float_as_uint(y);
  const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  u = __float_as_uint(y);
  const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// K-tile row read by MFMA row m of key tile kt (16 keys): chosen so that the
// S^T output rows 4*g4 + r of tiles 2j and 2j+1 held by lane group g4 are the
// keys 32j + 8*g4 .. +7 that the PV B operand of k-step j needs.
__device__ __forceinline__ int kperm16(int kt, int m) {
  return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3);
}
// K-tile swizzle under that permutation: kswz (shared header).

// Asynchronous global -> LDS copy of one tile of ROWS rows x SPR 16-byte
// chunks, starting `tile_off` bytes into the buffer, rows `row_bytes` apart,
// shared by NWAVES waves. Lane i of wave instruction j fills LDS chunk slot
// (slot0 + i) and fetches the global chunk that the swizzle (an involution)
// maps to that slot; the per-lane offset depends only on the lane and the
// swizzle phase, the rest is scalar.
template <int SPR, int ROWS, int NWAVES, bool KMAP>
__device__ __forceinline__ void tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t tile_off,
                                              uint32_t row_bytes, uint16_t* lds, int wave,
                                              int lane) {
  constexpr int SLOTS = ROWS * SPR;
  constexpr int PER_WAVE = SLOTS / NWAVES;
#pragma unroll
  for (int j = 0; j < PER_WAVE / 64; ++j) {
    const int slot0 = wave * PER_WAVE + j * 64;
    const int r0 = slot0 / SPR;
    const int rl = lane / SPR, sl = lane % SPR;
    const int c = KMAP ? kswz<SPR>(r0 + rl, sl) : vswz(r0 + rl, sl);
    const uint32_t voff = (uint32_t)rl * row_bytes + (uint32_t)c * 16u;
    const uint32_t soff = tile_off + (uint32_t)r0 * row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + slot0 * 8), 16, voff, soff, 0, 0);
  }
}

// Scheduling pattern for a block of N LDS fragment reads feeding N MFMAs in
// order: PF reads first, then alternating (MFMA, read) pairs, then the last
// PF MFMAs; the reads run PF MFMAs ahead of their use instead of each MFMA
// waiting for its own read.
template <int N, int PF, int XM = 0>
__device__ __forceinline__ void pipeline_reads() {
  static_assert(PF <= N, "prefetch depth");
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);   // DS reads
#pragma unroll
  for (int k = 0; k < N - PF; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF + XM, 0);   // and XM more MFMAs
}

// One workgroup = one (b, q head, 64-row query block); four waves of 16
// query rows each. MFMA 16x16x32 bf16 computes S^T = K Q^T (keys x queries:
// a lane owns one query column, so row statistics stay in-lane up to a
// reduction over the four lanes of that column) and O^T = V^T P^T, with P
// handed from the S^T output registers to the PV B operand directly thanks
// to the K row permutation kperm16. The small per-wave state (about 116
// VGPRs) lets four waves share each SIMD, so one wave's softmax VALU work
// overlaps another's MFMA work.
//
// Per key block: QK^T from the K tile, softmax statistics, [V landed,
// barrier] start the next K copy, PV from the V^T tile, [K landed, barrier]
// start the next V copy. K and V^T tiles (16 KB each) have one LDS buffer
// each; every asynchronous copy overlaps one compute phase.
//
// The running max is updated lazily: the accumulator keeps its reference
// max until some row's block max exceeds it by more than 2^8, so most blocks
// skip the rescale (P stays <= 256, exact enough in bf16 and float32).
template <int D>
__global__ __launch_bounds__(256, 4) void attn_prefill_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vt, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hf, uint16_t* __restrict__ Hs, float* __restrict__ delta,
    float* __restrict__ lse, Dims d, HeadMap hm) {
  constexpr int KSPR = D / 8;       // 16-byte chunks per K row
  constexpr int VSPR = kBlock / 8;  // 16-byte chunks per V^T row
  constexpr int NKS = D / 32;       // k-steps of QK^T
  constexpr int NDT = D / 16;       // d tiles of O^T
  constexpr float kTau = 8.0f;
  constexpr int kPrefetch = 4;      // LDS fragment reads in flight ahead of the MFMAs
  __shared__ __align__(16) uint16_t Ks[kBlock * D];
  __shared__ __align__(16) uint16_t Vs[D * kBlock];
  __shared__ uint32_t sel_mask[kMaxKeyBlocks / 32];

  const int total = d.B * d.Hq * d.nQB;
  const int lin = xcd_remap(blockIdx.x, total);
  const int per_group = d.G * d.nQB;
  const int grp = lin / per_group;
  const int rem = lin - grp * per_group;
  const int qb = d.nQB - 1 - rem / d.G;
  const int hi = rem - (rem / d.G) * d.G;
  const int b = grp / d.Hkv;
  const int g = grp - b * d.Hkv;
  const int h = hm.q_of_kv[g * d.G + hi];
  const int bh = b * d.Hq + h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int qq = wave * 16 + n;
  const int qrow = qb * kBlock + qq;
  const int diag = qb;
  const float sl2 = d.scale_log2;

  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vt + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)((size_t)d.Nk * D * 2));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (uint32_t)((size_t)d.Nk * D * 2));
  const uint32_t k_row_bytes = D * 2, v_row_bytes = (uint32_t)d.Nk * 2;
  auto load_k = [&](int kb) {
    tile_to_lds<KSPR, kBlock, 4, true>(krs, (uint32_t)kb * kBlock * k_row_bytes, k_row_bytes,
                                         Ks, wave, lane);
  };
  auto load_v = [&](int kb) {
    tile_to_lds<VSPR, D, 4, false>(vrs, (uint32_t)kb * kBlock * 2, v_row_bytes, Vs, wave, lane);
  };
  auto kchunk = [&](int row, int ch) { return kswz<KSPR>(row, ch); };

  // Q^T operand: lane holds Q[qrow][32ks + 8g4 .. +7] (in flight with the
  // list loads below)
  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 32 * ks);
  }
  // the count and the first 256 entries are read side by side (entries past
  // the count are read and ignored)
  const int* my_idx = idx + ((size_t)bh * d.nQB + qb) * d.budget;
  const int c_raw = cnt[(size_t)bh * d.nQB + qb];
  const int kb_first = tid < d.budget ? my_idx[tid] : -1;
  const int nwords = (diag >> 5) + 1;
  for (int w = tid; w < nwords; w += 256) sel_mask[w] = 0u;
  __syncthreads();
  const int n_sel = __builtin_amdgcn_readfirstlane(min(max(c_raw, 0), d.budget));
  if (tid < n_sel && kb_first >= 0 && kb_first <= diag)
    atomicOr(&sel_mask[kb_first >> 5], 1u << (kb_first & 31));
  for (int e = tid + 256; e < n_sel; e += 256) {
    const int kb = my_idx[e];
    if (kb >= 0 && kb <= diag) atomicOr(&sel_mask[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();

  const bool sparse_only = (Hf == nullptr);
  int phase = 0, wcur = 0;
  uint32_t bits = __builtin_amdgcn_readfirstlane(sel_mask[0]);
  auto next_block = [&](bool& selected) -> int {
    while (true) {
      if (bits != 0u) {
        const int kb = (wcur << 5) + __builtin_ctz(bits);
        bits &= bits - 1u;
        if (kb > diag) { bits = 0u; continue; }
        selected = (phase == 0);
        return kb;
      }
      if (++wcur < nwords) {
        const uint32_t w = __builtin_amdgcn_readfirstlane(sel_mask[wcur]);
        bits = phase == 0 ? w : ~w;
        continue;
      }
      if (phase == 0 && !sparse_only) {
        phase = 1;
        wcur = 0;
        bits = ~__builtin_amdgcn_readfirstlane(sel_mask[0]);
        continue;
      }
      return -1;
    }
  };

  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_sel = 0.f;   // l_sel: the sum at the snapshot
  // row sums on the matrix cores: with an all-ones A operand a 16x16x32 MFMA
  // adds the 32 weights of each query column of a PV k-step, and every lane
  // of that column gets the total (register 0 is read)
  f32x4_t la4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones16 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                  0x3F803F80u, 0x3F803F80u));

  auto store = [&](uint16_t* H, float inv) {
    uint16_t* hp = H + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = 16 * dt + 4 * g4;
      const uint32_t lo = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
      const uint32_t hi2 = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *(uint2*)(hp + d0) = make_uint2(lo, hi2);
    }
  };

  auto body = [&](int kb, int kb_next) {
    f32x4_t s[4];
    {
      // MFMA work runs at raised wave priority, so that a wave with its
      // operands ready takes the matrix unit ahead of waves in their softmax
      __builtin_amdgcn_s_setprio(1);
      bf16x8_t fr[4 * NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int row = kperm16(kt, n);
          fr[ks * 4 + kt] = *(const bf16x8_t*)(Ks + (row * KSPR + kchunk(row, 4 * ks + g4)) * 8);
        }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[ks * 4 + kt], qf[ks], s[kt], 0, 0, 0);
      pipeline_reads<4 * NKS, kPrefetch>();
      __builtin_amdgcn_s_setprio(0);
    }
    if (kb == diag) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kperm16(kt, 4 * g4 + r) > qq) s[kt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][r]);
    const float m_blk = quad_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(m_blk > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_blk);
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[i][v] *= alpha;
      la4[0] *= alpha;
      l_sel *= alpha;
    }
    uint32_t pw[8];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float p0 = fast_exp2(fmaf(s[kt][0], sl2, -m_ref));
      const float p1 = fast_exp2(fmaf(s[kt][1], sl2, -m_ref));
      const float p2 = fast_exp2(fmaf(s[kt][2], sl2, -m_ref));
      const float p3 = fast_exp2(fmaf(s[kt][3], sl2, -m_ref));
      pw[2 * kt] = pack_bf16x2(p0, p1);
      pw[2 * kt + 1] = pack_bf16x2(p2, p3);
    }

    wait_vm();
    __syncthreads();
    if (kb_next >= 0) load_k(kb_next);

    // O^T += V^T P^T; k-step j (32 keys) takes tiles 2j, 2j+1.
    {
      __builtin_amdgcn_s_setprio(1);
      bf16x8_t fr[2 * NDT];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int r = 16 * dt + n;
          fr[j * NDT + dt] = *(const bf16x8_t*)(Vs + (r * VSPR + vswz(r, 4 * j + g4)) * 8);
        }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 w = make_uint4(pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j * NDT + dt], pb, o[dt], 0, 0, 0);
        la4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones16, pb, la4, 0, 0, 0);
      }
      pipeline_reads<2 * NDT, kPrefetch, 2>();
      __builtin_amdgcn_s_setprio(0);
    }

    wait_vm();
    __syncthreads();
    if (kb_next >= 0) load_v(kb_next);
  };

  const size_t plane = (size_t)d.B * d.Hq * d.Nq;
  bool sel_cur = false;
  int kb = next_block(sel_cur);
  if (kb >= 0) {
    load_k(kb);
    load_v(kb);
    wait_vm();
    __syncthreads();
  }
  while (kb >= 0 && sel_cur) {
    bool sel_next = false;
    const int kb_next = next_block(sel_next);
    body(kb, kb_next);
    kb = kb_next;
    sel_cur = sel_next;
  }
  {
    l_sel = la4[0];
    const float lt = l_sel;
    store(Hs, 1.f / lt);
    if (lse != nullptr && g4 == 0)
      lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
  if (sparse_only) return;
  while (kb >= 0) {
    bool sel_next = false;
    const int kb_next = next_block(sel_next);
    body(kb, kb_next);
    kb = kb_next;
  }
  const float ls_t = l_sel;
  const float lt = la4[0];
  const float ld_t = fmaxf(lt - ls_t, 0.f);
  store(Hf, 1.f / lt);
  if (g4 == 0) {
    if (delta != nullptr) delta[(size_t)bh * d.Nq + qrow] = ld_t / lt;
    if (lse != nullptr) lse[(size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
}

// 16-token selection blocks (bs = 16): one workgroup = one (b, q head,
// 64-row query tile), four waves of 16 rows, so each wave's rows are exactly
// one query block with its own selection. Every 64-key tile splits into four
// 16-key quarters; in the S^T layout the keys a lane holds for MFMA tile kt
// all sit in quarter 2*(kt/2) + (g4/2), so masking a quarter is per (lane,
// kt). The waves walk the causal tiles in ascending order (sparse-only: the
// tiles where some wave selected a quarter) with two accumulators sharing one
// running max: o_all over every causal key and o_sel over the selected
// quarters (its PV runs only for tiles where the wave selected something);
// l_sel and l_drop partition the weights. Then
//     h_full = o_all / (l_sel + l_drop),  h_sparse = o_sel / l_sel,
//     delta = l_drop / (l_sel + l_drop).
//
// TOK > 0 (per-token selection with blocks of TOK tokens): every query row
// has its own list. The workgroup stages the 64 rows' lists in LDS (kept
// ascending and causal), and each lane walks its row's list alongside the
// tiles, so the selected quarters of a tile are a per-lane nibble (a 64-token
// block is a whole tile: 0xF or 0). The accumulator split is unchanged; the
// selected-stream PV runs for a tile when any row of the wave selected part
// of it.
template <int D, int TOK>
__global__ __launch_bounds__(256, 3) void attn_prefill_bf16_q16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vt, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hf, uint16_t* __restrict__ Hs, float* __restrict__ delta,
    float* __restrict__ lse, Dims d, HeadMap hm) {
  constexpr int KSPR = D / 8;
  constexpr int VSPR = kBlock / 8;
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  constexpr float kTau = 8.0f;
  constexpr int kPrefetch = 4;
  constexpr int kWords16 = kMaxKeyBlocks / 32;     // 16-key blocks bitmap words
  constexpr int kTokLd = kTokMaxBudget + 1;        // padded per-row list stride
  static_assert(TOK == 0 || TOK == 16 || TOK == 64, "per-token block size");
  __shared__ __align__(16) uint16_t Ks[kBlock * D];
  __shared__ __align__(16) uint16_t Vs[D * kBlock];
  __shared__ uint32_t sel16[TOK ? 1 : 4][TOK ? 1 : kWords16];   // per wave: selected 16-key blocks
  __shared__ int rl[TOK ? 64 : 1][TOK ? kTokLd : 1];            // per row: its list (TOK)
  __shared__ int rn[TOK ? 64 : 1];
  __shared__ uint32_t tiles[kMaxKeyBlocks / 32];    // sparse-only: tiles some wave needs

  const int total = d.B * d.Hq * d.nQT;
  const int lin = xcd_remap(blockIdx.x, total);
  const int per_group = d.G * d.nQT;
  const int grp = lin / per_group;
  const int rem = lin - grp * per_group;
  const int qt = d.nQT - 1 - rem / d.G;
  const int hi = rem - (rem / d.G) * d.G;
  const int b = grp / d.Hkv;
  const int g = grp - b * d.Hkv;
  const int h = hm.q_of_kv[g * d.G + hi];
  const int bh = b * d.Hq + h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int qq = wave * 16 + n;
  const int qrow = qt * kBlock + qq;
  const float sl2 = d.scale_log2;
  const bool sparse_only = (Hf == nullptr);

  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vt + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)((size_t)d.Nk * D * 2));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (uint32_t)((size_t)d.Nk * D * 2));
  const uint32_t k_row_bytes = D * 2, v_row_bytes = (uint32_t)d.Nk * 2;
  auto load_k = [&](int t) __attribute__((always_inline)) {
    tile_to_lds<KSPR, kBlock, 4, true>(krs, (uint32_t)t * kBlock * k_row_bytes, k_row_bytes, Ks,
                                       wave, lane);
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
    tile_to_lds<VSPR, D, 4, false>(vrs, (uint32_t)t * kBlock * 2, v_row_bytes, Vs, wave, lane);
  };
  auto kchunk = [&](int row, int ch) { return kswz<KSPR>(row, ch); };

  // ---- selection: bitmaps of 16-key blocks up to this tile's diagonal
  // (TOK == 0), or the rows' own lists (TOK)
  const int nwords_t = (qt >> 5) + 1;
  for (int w = tid; w < nwords_t; w += 256) tiles[w] = 0u;
  if constexpr (TOK == 0) {
    for (int w = tid; w < 4 * kWords16; w += 256) (&sel16[0][0])[w] = 0u;
    __syncthreads();
    // one thread per (query block, list entry): all list loads in flight
    // at once (entries past the count are read and ignored)
    for (int t = tid; t < 4 * d.budget; t += 256) {
      const int u = t / d.budget, e = t - u * d.budget;
      const size_t row = (size_t)bh * d.nQB + 4 * qt + u;
      const int ns = cnt[row];
      const int kb = idx[row * d.budget + e];
      if (e < ns && kb >= 0 && kb <= 4 * qt + u) {
        atomicOr(&sel16[u][kb >> 5], 1u << (kb & 31));
        if (sparse_only) atomicOr(&tiles[kb >> 7], 1u << ((kb >> 2) & 31));
      }
    }
  } else {
    const size_t lrow0 = (size_t)bh * d.Nq + (size_t)qt * kBlock;   // this tile's 64 lists
    for (int i = tid; i < kBlock * d.budget; i += 256) {
      const int r = i / d.budget, e = i - r * d.budget;
      rl[r][e] = idx[lrow0 * d.budget + i];
    }
    if (tid < kBlock) rn[tid] = min(max(cnt[lrow0 + tid], 0), d.budget);
    __syncthreads();
    if (tid < kBlock) {   // keep the ascending entries within the row's causal blocks
      const int limit = (qt * kBlock + tid) / TOK;
      int m = 0, last = -1;
      for (int e = 0; e < rn[tid]; ++e) {
        const int kb = rl[tid][e];
        if (kb > last && kb <= limit) {
          rl[tid][m++] = kb;
          last = kb;
          if (sparse_only) {
            const int tt = TOK == 64 ? kb : kb >> 2;
            atomicOr(&tiles[tt >> 5], 1u << (tt & 31));
          }
        }
      }
      rn[tid] = m;
    }
  }
  __syncthreads();

  // tiles walked: every causal tile, or (sparse-only) those some wave needs
  int wcur = 0;
  uint32_t tbits = sparse_only ? __builtin_amdgcn_readfirstlane(tiles[0]) : 0u;
  int tnext_dual = 0;
  auto next_tile = [&]() __attribute__((always_inline)) -> int {
    if (!sparse_only) return tnext_dual <= qt ? tnext_dual++ : -1;
    while (true) {
      if (tbits != 0u) {
        const int t = (wcur << 5) + __builtin_ctz(tbits);
        tbits &= tbits - 1u;
        return t <= qt ? t : -1;
      }
      if (++wcur < nwords_t) { tbits = __builtin_amdgcn_readfirstlane(tiles[wcur]); continue; }
      return -1;
    }
  };
  // selected 16-key quarters of tile t: this wave's (TOK == 0) or this
  // lane's row's (TOK; tiles are visited in ascending order)
  int lptr = 0;
  const int lcnt = TOK ? rn[TOK ? qq : 0] : 0;
  auto quarters = [&](int t) __attribute__((always_inline)) -> uint32_t {
    if constexpr (TOK == 0) {
      return (__builtin_amdgcn_readfirstlane(sel16[wave][t >> 3]) >> ((4 * t) & 31)) & 0xFu;
    } else if constexpr (TOK == 64) {
      const int e = lptr < lcnt ? rl[qq][lptr] : -1;
      const bool hit = e == t;
      lptr += hit ? 1 : 0;
      return hit ? 0xFu : 0u;
    } else {
      uint32_t nib = 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lptr < lcnt ? rl[qq][lptr] : -1;
        const bool hit = e >= 0 && (e >> 2) == t;
        nib |= hit ? 1u << (e & 3) : 0u;
        lptr += hit ? 1 : 0;
      }
      return nib;
    }
  };

  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 32 * ks);
  }
  f32x4_t oa[NDT], os[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) { oa[i] = f32x4_t{0.f, 0.f, 0.f, 0.f}; os[i] = oa[i]; }
  float m_ref = -INFINITY;
  // row sums on the matrix cores: with an all-ones A operand a 16x16x32 MFMA
  // adds the 32 weights of each query column of a PV k-step, and every lane
  // of that column gets the total (register 0 is read): la4 over all weights,
  // ls4 over the selected ones
  f32x4_t la4 = {0.f, 0.f, 0.f, 0.f}, ls4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones16 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                  0x3F803F80u, 0x3F803F80u));

  auto store = [&](uint16_t* H, const f32x4_t* o, float inv) __attribute__((always_inline)) {
    uint16_t* hp = H + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = 16 * dt + 4 * g4;
      const uint32_t lo = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
      const uint32_t hi2 = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *(uint2*)(hp + d0) = make_uint2(lo, hi2);
    }
  };
  auto pv = [&](f32x4_t* o, const uint32_t* pwv, f32x4_t& lsum) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    bf16x8_t fr[2 * NDT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int r = 16 * dt + n;
        fr[j * NDT + dt] = *(const bf16x8_t*)(Vs + (r * VSPR + vswz(r, 4 * j + g4)) * 8);
      }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 w = make_uint4(pwv[4 * j], pwv[4 * j + 1], pwv[4 * j + 2], pwv[4 * j + 3]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j * NDT + dt], pb, o[dt], 0, 0, 0);
      lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones16, pb, lsum, 0, 0, 0);
    }
    pipeline_reads<2 * NDT, kPrefetch, 2>();
    __builtin_amdgcn_s_setprio(0);
  };

  auto body = [&](int t, int t_next) __attribute__((always_inline)) {
    const uint32_t qm = quarters(t);
    const bool any_sel = TOK ? __builtin_amdgcn_ballot_w64(qm != 0u) != 0ull : qm != 0u;
    // sparse-only: a wave with no selected quarter in this tile only keeps
    // the workgroup's copy/barrier rhythm
    const bool work = !sparse_only || any_sel;
    uint32_t pw[8], pws[8];
    if (work) {
    f32x4_t s[4];
    {
      __builtin_amdgcn_s_setprio(1);
      bf16x8_t fr[4 * NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int row = kperm16(kt, n);
          fr[ks * 4 + kt] = *(const bf16x8_t*)(Ks + (row * KSPR + kchunk(row, 4 * ks + g4)) * 8);
        }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[ks * 4 + kt], qf[ks], s[kt], 0, 0, 0);
      pipeline_reads<4 * NKS, kPrefetch>();
      __builtin_amdgcn_s_setprio(0);
    }
    // quarter of the keys this lane holds for MFMA tile kt
    bool qsel[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) qsel[kt] = (qm >> (2 * (kt >> 1) + (g4 >> 1))) & 1u;
    if (t == qt) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kperm16(kt, 4 * g4 + r) > qq) s[kt][r] = -INFINITY;
    }
    if (sparse_only) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        if (!qsel[kt]) s[kt] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][r]);
    const float m_blk = quad_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(m_blk > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_blk);
      // sparse-only per-token lists: a row that has met none of its
      // selected keys yet keeps m = -inf and zero sums (no -inf - -inf)
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) { oa[i][v] *= alpha; os[i][v] *= alpha; }
      la4[0] *= alpha;
      ls4[0] *= alpha;
    }
    // such a row's logits are all -inf here: its weights come out 0
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float p0 = fast_exp2(fmaf(s[kt][0], sl2, -m_use));
      const float p1 = fast_exp2(fmaf(s[kt][1], sl2, -m_use));
      const float p2 = fast_exp2(fmaf(s[kt][2], sl2, -m_use));
      const float p3 = fast_exp2(fmaf(s[kt][3], sl2, -m_use));
      pw[2 * kt] = pack_bf16x2(p0, p1);
      pw[2 * kt + 1] = pack_bf16x2(p2, p3);
      pws[2 * kt] = qsel[kt] ? pw[2 * kt] : 0u;
      pws[2 * kt + 1] = qsel[kt] ? pw[2 * kt + 1] : 0u;
    }
    }

    wait_vm();
    __syncthreads();
    if (t_next >= 0) load_k(t_next);
    if (!sparse_only) pv(oa, pw, la4);
    if (any_sel) pv(os, pws, ls4);
    wait_vm();
    __syncthreads();
    if (t_next >= 0) load_v(t_next);
  };

  int t = next_tile();
  if (t >= 0) {
    load_k(t);
    load_v(t);
    wait_vm();
    __syncthreads();
  }
  while (t >= 0) {
    const int t_next = next_tile();
    body(t, t_next);
    t = t_next;
  }
  const size_t plane = (size_t)d.B * d.Hq * d.Nq;
  const float ls_t = ls4[0];
  store(Hs, os, 1.f / ls_t);
  if (lse != nullptr && g4 == 0)
    lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(ls_t)) * kLn2;
  if (sparse_only) return;
  const float lt = la4[0];
  const float ld_t = fmaxf(lt - ls_t, 0.f);
  store(Hf, oa, 1.f / lt);
  if (g4 == 0) {
    if (delta != nullptr) delta[(size_t)bh * d.Nq + qrow] = ld_t / lt;
    if (lse != nullptr) lse[(size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
}

// Row of the K tile that 32x32 MFMA row c reads: the S^T output register v
// of lane half gl then holds key 16*(v/8) + 8*gl + (v%8) of its 32-key tile,
// exactly the 8 consecutive keys of the PV B operand.
__device__ __forceinline__ int kperm32(int c) {
  const int i = c >> 3, gp = (c >> 2) & 1, j = c & 3;
  return 16 * (i >> 1) + 8 * gp + 4 * (i & 1) + j;
}
// 256-byte K rows: the 16 rows one ds_read_b128 phase touches have distinct
// low four bits, so chunk ^ (row & 15) spreads them over all bank groups.
__device__ __forceinline__ int kswz32(int row, int chunk) { return chunk ^ (row & 15); }
// Maximum of three floats; a chain of these becomes v_max3_f32 operations.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int SPR, int ROWS, int NWAVES, bool KMAP>
__device__ __forceinline__ void tile_to_lds_asm(i32x4_t rsrc, uint32_t tile_off,
                                                uint32_t row_bytes, uint16_t* lds, int wave,
                                                int lane) {
  constexpr int SLOTS = ROWS * SPR;
  constexpr int PER_WAVE = SLOTS / NWAVES;
#pragma unroll
  for (int j = 0; j < PER_WAVE / 64; ++j) {
    const int slot0 = wave * PER_WAVE + j * 64;
    const int r0 = slot0 / SPR;
    const int rl = lane / SPR, sl = lane % SPR;
    // 256-byte K rows (D = 128) take kswz32; 128-byte rows (V^T, and K for
    // D = 64) take vswz, which also keeps the kperm32 row reads apart
    const int c = (KMAP && SPR == 16) ? kswz32(r0 + rl, sl) : vswz(r0 + rl, sl);
    const uint32_t voff = (uint32_t)rl * row_bytes + (uint32_t)c * 16u;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(tile_off + (uint32_t)r0 * row_bytes);
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_ptr_t)(lds + slot0 * 8));
    copy16_to_lds(rsrc, soff, voff, la);
  }
}


// D = 128, G % 4 == 0: one workgroup = one (b, kv head, 64-row query block)
// serving four q heads of that kv head, so each K/V tile crosses L2 -> LDS
// once for 256 query rows. Eight waves of 32 rows on MFMA 32x32x16 bf16:
// wave w takes rows 32*(w/4) .. +31 of head w%4, so each SIMD holds one wave
// of group A (waves 0-3) and one of group B (waves 4-7).
//
// Walk: one list for the four heads, each entry marking the heads that
// compute it, built so that each head sees exactly its selected blocks, a
// snapshot (h_sparse), then its other causal blocks; blocks selected by
// only some of the heads are walked twice (once for the heads that selected
// them, once for the others) unless their heads fit the snapshot order
// (details where the list is built).
//
// Ping-pong: time is cut into slots separated by workgroup barriers; in
// slot 2e group A runs GEMM(e) = QK^T(e) + PV(e-1) while group B runs
// softmax(e-1), in slot 2e+1 the roles swap. So on every SIMD one wave's MFMA
// work overlaps the other wave's VALU work. K/V tiles live in NST LDS
// stages; after its GEMM(e) each wave requests its share of K(e+NST-1) and
// V(e+NST-2).
// Takes the next work item for this workgroup: the queues hold items
// [x * per, (x + 1) * per) for XCD x, in that order (the static mapping of
// xcd_remap); a workgroup first draws from its own XCD's queue, then from the
// others. With exactly one workgroup per item every workgroup gets one.
__device__ __forceinline__ int fetch_work_item(int* queues, int per) {
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  for (int j = 0; j < kNumXcd; ++j) {
    const int x = (int)((xcc + j) % kNumXcd);
    const int i = atomicAdd(&queues[x * kQueueStride], 1);
    if (i < per) return x * per + i;
  }
  return -1;
}
template <int D, int NST>
__global__ __launch_bounds__(512, 2) void attn_prefill_bf16_pp_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vt, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hf, uint16_t* __restrict__ Hs, float* __restrict__ delta,
    float* __restrict__ lse, int* __restrict__ queues, const float* __restrict__ kn, Dims d,
    HeadMap hm) {
  constexpr int HPW = 4;
  constexpr int NW = 8;
  constexpr int KSPR = D / 8;
  constexpr int VSPR = kBlock / 8;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE = kBlock * D;
  constexpr int LPH = (TILE / 8) / (64 * NW);   // buffer loads per half tile (K or V) per wave
  // rescale slack 2^24 (P <= 2^24: no float32 or bfloat16 range concern for
  // up to 2^18 keys): wide enough for the norm bound below to spare most
  // blocks their maximum when queries and keys have unit-variance entries
  constexpr float kTau = 24.0f;
  constexpr int kMaxWords = kMaxKeyBlocks / 32;
  constexpr int kParts = 5;
  // one LDS object per stage, always addressed with a compile-time stage,
  // so copies into one stage and reads of another are known not to alias
  __shared__ __align__(16) uint16_t K0[TILE], K1[TILE], K2[TILE], K3[NST > 3 ? TILE : 8];
  __shared__ __align__(16) uint16_t V0[TILE], V1[TILE], V2[TILE], V3[NST > 3 ? TILE : 8];
  __shared__ uint32_t sel_mask[HPW][kMaxWords];
  // walk list entries: key block (bits 0-11), the heads that compute it
  // (bits 12-15), the block's largest key norm rounded up to bfloat16 (bits
  // 16-31)
  __shared__ uint32_t list[2 * kMaxKeyBlocks];
  __shared__ float knl[kMaxKeyBlocks];   // largest key norm of each causal block
  // walk-list parts (below): per 32-block word the part's bits and the
  // exclusive prefix of their counts
  __shared__ uint32_t word_p[kParts][kMaxWords];
  __shared__ int scan_p[kParts][kMaxWords];
  __shared__ int counts[kParts];
  __shared__ int snap_at[HPW];   // the entry before which each head takes its snapshot
  __shared__ int mask_hist[16];  // causal blocks per selection pattern of the four heads

  const int ngrp = d.G / HPW;
  const int total = d.B * d.Hkv * ngrp * d.nQB;
  // Work items: with queues the grid is one workgroup per CU and each
  // workgroup takes items until every queue is empty, first from its own
  // XCD's queue, then from the others' (an XCD that runs ahead takes over the
  // short tail items of a slower one); without queues one item per workgroup
  // in the static mapping.
  __shared__ int s_item;
  const bool dyn = queues != nullptr && total % kNumXcd == 0;
  for (int pass = 0;; ++pass) {
  if (dyn) {
    __syncthreads();   // the previous item no longer reads LDS or s_item
    if (threadIdx.x == 0) s_item = fetch_work_item(queues, total / kNumXcd);
  } else {
    if (pass > 0) break;
    if (threadIdx.x == 0) s_item = xcd_remap(blockIdx.x, total);
  }
  __syncthreads();
  const int lin = s_item;
  if (lin < 0) break;   // every queue is empty
  const int per_group = ngrp * d.nQB;
  const int grp = lin / per_group;
  const int rem = lin - grp * per_group;
  const int qb = d.nQB - 1 - rem / ngrp;
  const int hg = rem - (rem / ngrp) * ngrp;
  const int b = grp / d.Hkv;
  const int g = grp - b * d.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave & 3;
  const bool group_a = wave < 4;
  const int h = hm.q_of_kv[g * d.G + hg * HPW + hs];
  const int bh = b * d.Hq + h;
  const int c = lane & 31, gl = lane >> 5;
  const int qq = (wave >> 2) * 32 + c;
  const int qrow = qb * kBlock + qq;
  const int diag = qb;
  const float sl2 = d.scale_log2;
  const bool sparse_only = (Hf == nullptr);

  // ---- walk list
  const int nwords = (diag >> 5) + 1;
  for (int w = tid; w < HPW * kMaxWords; w += 64 * NW) (&sel_mask[0][0])[w] = 0u;
  if (tid < 16) mask_hist[tid] = 0;
  {
    // GEMM(0) multiplies the V stage of the (absent) entry -1 by P = 0
    uint16_t* vz = (NST - 1) == 1 ? V1 : (NST - 1) == 2 ? V2 : V3;
    for (int w = tid; w < TILE / 8; w += 64 * NW) ((uint4*)vz)[w] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  // the query fragments, in flight together with the idx/cnt loads below
  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 16 * ks);
  }
  for (int u = 0; u < HPW; ++u) {
    const int hu = hm.q_of_kv[g * d.G + hg * HPW + u];
    const size_t row = (size_t)(b * d.Hq + hu) * d.nQB + qb;
    const int ns = min(max(cnt[row], 0), d.budget);
    for (int e = tid; e < ns; e += 64 * NW) {
      const int kb = idx[row * d.budget + e];
      if (kb >= 0 && kb <= diag) atomicOr(&sel_mask[u][kb >> 5], 1u << (kb & 31));
    }
  }
  {
    const float* knr = kn + (size_t)(b * d.Hkv + g) * (d.Nk / kBlock);
    for (int kb = tid; kb <= diag; kb += 64 * NW) knl[kb] = knr[kb];
  }
  __syncthreads();
  // The walk list. m(kb) is the set of the four heads that selected causal
  // block kb. Every head must meet its selected blocks, then take its
  // snapshot (h_sparse), then meet its other causal blocks. With the heads
  // in an order p0..p3 that snapshot last to first (p3 first), the list is
  //   part 0: blocks with m = all four, and blocks whose m is partial and
  //           not one of the chain sets below (the heads in m compute them);
  //   part 1: m = {p0, p1, p2}; part 2: m = {p0, p1}; part 3: m = {p0}
  //           (every head computes these: selected by the heads that have
  //           not yet taken their snapshot, unselected for those that have);
  //   part 4: m = {} and the partial blocks of part 0 again (the heads not
  //           in m compute them),
  // each part in ascending block order; p3 takes its snapshot before part
  // 1, p2 before part 2, p1 before part 3, p0 before part 4. A partial block
  // whose m is a chain set is walked once instead of twice; the order p is
  // the one of the 24 that puts the most causal blocks on the chain. In
  // sparse-only mode there is no part 4 and no chain: every partial block
  // stays in part 0.
  if (tid < nwords) {
    const uint32_t lim = (tid == nwords - 1) ? (0xffffffffu >> (31 - (diag & 31))) : 0xffffffffu;
    uint32_t any = 0u, all = 0xffffffffu;
#pragma unroll
    for (int u = 0; u < HPW; ++u) { any |= sel_mask[u][tid]; all &= sel_mask[u][tid]; }
    for (uint32_t part = any & ~all & lim; part != 0u; part &= part - 1u) {
      const int bit = __builtin_ctz(part);
      int m = 0;
#pragma unroll
      for (int u = 0; u < HPW; ++u) m |= (int)((sel_mask[u][tid] >> bit) & 1u) << u;
      atomicAdd(&mask_hist[m], 1);
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane l < 24 scores the l-th head order: p0 is the (l / 6)-th head,
    // p1 the ((l % 6) / 2)-th of the three left, p2 the (l % 2)-th of the
    // two left, p3 the last one
    auto kth_bit = [](uint32_t m, int k) __attribute__((always_inline)) {
      for (int i = 0; i < k; ++i) m &= m - 1u;
      return (int)__builtin_ctz(m);
    };
    int p[4];
    {
      const int l = lane % 24;
      uint32_t rem = 0xFu;
      p[0] = kth_bit(rem, l / 6);
      rem &= ~(1u << p[0]);
      p[1] = kth_bit(rem, (l % 6) / 2);
      rem &= ~(1u << p[1]);
      p[2] = kth_bit(rem, l % 2);
      rem &= ~(1u << p[2]);
      p[3] = (int)__builtin_ctz(rem);
    }
    const int c1 = 1 << p[0], c2 = c1 | (1 << p[1]), c3 = c2 | (1 << p[2]);
    const int score = lane < 24 ? mask_hist[c1] + mask_hist[c2] + mask_hist[c3] : -1;
    int best = score;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off, 64));
    const uint64_t win = __builtin_amdgcn_ballot_w64(score == best);
    const int wl = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(win));
    const int pw0 = __shfl(p[0], wl, 64), pw1 = __shfl(p[1], wl, 64);
    const int pw2 = __shfl(p[2], wl, 64), pw3 = __shfl(p[3], wl, 64);
    // chain sets as 4-bit masks; none in sparse-only mode (16 matches no m)
    const uint32_t ch1 = sparse_only ? 16u : (1u << pw0);
    const uint32_t ch2 = sparse_only ? 16u : ch1 | (1u << pw1);
    const uint32_t ch3 = sparse_only ? 16u : ch2 | (1u << pw2);
    // bits of the blocks whose m equals the 4-bit set c
    auto eq = [&](uint32_t c, const uint32_t s4[HPW]) __attribute__((always_inline)) {
      if (c > 15u) return 0u;
      uint32_t r = 0xffffffffu;
#pragma unroll
      for (int u = 0; u < HPW; ++u) r &= ((c >> u) & 1u) ? s4[u] : ~s4[u];
      return r;
    };
    int carry[kParts] = {0, 0, 0, 0, 0};
    for (int w0 = 0; w0 < nwords; w0 += 64) {
      const int w = w0 + lane;
      uint32_t pm[kParts] = {0u, 0u, 0u, 0u, 0u};
      if (w < nwords) {
        const uint32_t lim = (w == nwords - 1) ? (0xffffffffu >> (31 - (diag & 31))) : 0xffffffffu;
        uint32_t s4[HPW];
#pragma unroll
        for (int u = 0; u < HPW; ++u) s4[u] = sel_mask[u][w];
        const uint32_t any = (s4[0] | s4[1] | s4[2] | s4[3]) & lim;
        const uint32_t all = s4[0] & s4[1] & s4[2] & s4[3] & lim;
        const uint32_t e1 = eq(ch3, s4) & lim, e2 = eq(ch2, s4) & lim, e3 = eq(ch1, s4) & lim;
        const uint32_t chain = e1 | e2 | e3;
        pm[0] = any & ~chain;
        pm[1] = e1;
        pm[2] = e2;
        pm[3] = e3;
        pm[4] = sparse_only ? 0u : (~all & lim & ~chain);
      }
#pragma unroll
      for (int k = 0; k < kParts; ++k) {
        const int pc = __popc(pm[k]);
        int inc = pc;   // inclusive wave scan
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(inc, off, 64);
          if (lane >= off) inc += o;
        }
        if (w < nwords) { word_p[k][w] = pm[k]; scan_p[k][w] = carry[k] + inc - pc; }
        carry[k] += __shfl(inc, 63, 64);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kParts; ++k) counts[k] = carry[k];
      const int s1 = carry[0], s2 = s1 + carry[1], s3 = s2 + carry[2], s4 = s3 + carry[3];
      snap_at[pw3] = s1;
      snap_at[pw2] = s2;
      snap_at[pw1] = s3;
      snap_at[pw0] = s4;
    }
  }
  __syncthreads();
  int part_base[kParts];
  {
    int acc = 0;
#pragma unroll
    for (int k = 0; k < kParts; ++k) {
      part_base[k] = acc;
      acc += __builtin_amdgcn_readfirstlane(counts[k]);
    }
  }
  const int n = part_base[kParts - 1] + __builtin_amdgcn_readfirstlane(counts[kParts - 1]);
  const int n_snap = __builtin_amdgcn_readfirstlane(snap_at[hs]);
  for (int kb = tid; kb <= diag; kb += 64 * NW) {
    const int w = kb >> 5, bit = kb & 31;
    const uint32_t below = (1u << bit) - 1u;
    uint32_t mine = 0u;   // the heads that selected kb
#pragma unroll
    for (int u = 0; u < HPW; ++u) mine |= ((sel_mask[u][w] >> bit) & 1u) << u;
    // a norm rounded up to bfloat16 stays an upper bound (NaN becomes +inf)
    const uint32_t knb = (min(__float_as_uint(knl[kb]), 0x7F800000u) + 0xFFFFu) & 0xFFFF0000u;
#pragma unroll
    for (int k = 0; k < kParts; ++k) {
      const uint32_t wk = word_p[k][w];
      if ((wk >> bit) & 1u) {
        const uint32_t act = k == 0 ? mine : k == 4 ? (mine ^ 0xFu) : 0xFu;
        list[part_base[k] + scan_p[k][w] + __popc(wk & below)] = (uint32_t)kb | (act << 12) | knb;
      }
    }
  }
  __syncthreads();

  // ---- tiles
  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vt + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const i32x4_t krs = make_rsrc_words(kbase, (uint32_t)((size_t)d.Nk * D * 2));
  const i32x4_t vrs = make_rsrc_words(vbase, (uint32_t)((size_t)d.Nk * D * 2));
  const uint32_t k_row_bytes = D * 2, v_row_bytes = (uint32_t)d.Nk * 2;
  auto entry_kb = [&](int e) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane((int)list[e]) & 0xfff;
  };
  // copies past the end of the list repeat its last block (or block 0):
  // every slot issues the same number of copies, so the waits are static
  auto entry_kb_c = [&](int e) __attribute__((always_inline)) {
    const int ec = min(e, n - 1);
    return ec >= 0 ? entry_kb(ec) : 0;
  };
  auto load_k_kb = [&](auto stc, int kb) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    uint16_t* kt = st == 0 ? K0 : st == 1 ? K1 : st == 2 ? K2 : K3;
    tile_to_lds_asm<KSPR, kBlock, NW, true>(krs, (uint32_t)kb * kBlock * k_row_bytes,
                                           k_row_bytes, kt, wave, lane);
  };
  auto load_v_kb = [&](auto stc, int kb) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    uint16_t* vt = st == 0 ? V0 : st == 1 ? V1 : st == 2 ? V2 : V3;
    tile_to_lds_asm<VSPR, D, NW, false>(vrs, (uint32_t)kb * kBlock * 2, v_row_bytes, vt,
                                       wave, lane);
  };
  auto load_k = [&](auto stc, int e) __attribute__((always_inline)) {
    load_k_kb(stc, entry_kb_c(e));
  };
  auto load_v = [&](auto stc, int e) __attribute__((always_inline)) {
    load_v_kb(stc, entry_kb_c(e));
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // the Q fragments (loaded with the lists above) have landed: the
  // compiler does not count the LDS copies below, so it must see no load of
  // its own outstanding
  __builtin_amdgcn_s_waitcnt(0xF70);
  // Bound on this row's scaled logits against a key block: |q| sl2 times
  // the block's largest key norm, raised by 2^-10 (far above the float32
  // rounding of the dot products and norms). A block whose bound is at most
  // m_ref + kTau cannot trigger a rescale, so its maximum is not needed.
  float qsq = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint4 u = __builtin_bit_cast(uint4, qf[ks]);
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
      qsq = fmaf(lo, lo, qsq);
      qsq = fmaf(hi, hi, qsq);
    }
  }
  const float qbound = sqrtf(pair_sum(qsq)) * sl2 * (1.f + 0x1p-10f);
  // prologue = the copies of the virtual slots before slot 0: K(0..NST-2)
  // and V(0..NST-3), with V(0) standing in for the missing V(-1)
  load_k(I0{}, 0);
  load_v(I0{}, 0);
  load_k(I1{}, 1);
  load_v(I0{}, 0);
  if constexpr (NST > 3) {
    load_k(I2{}, 2);
    load_v(I1{}, 1);
  }

  f32x16_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  f32x16_t s0, s1;
  uint32_t pw[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) pw[k] = 0u;
  float m_ref = -INFINITY, l_sel = 0.f;
  // row sums on the matrix cores, as in attn_prefill_bf16_pp16_kernel: lane
  // n < 16 accumulates the weights of queries n and n + 16 in la4[0], la4[1]
  f32x4_t la4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t one2 = (lane & 15) == ((lane >> 4) & 1) ? 0x3F803F80u : 0u;
  const bf16x8_t ones_a = __builtin_bit_cast(bf16x8_t, make_uint4(one2, one2, one2, one2));
  auto row_sum = [&]() __attribute__((always_inline)) {
    const int sl = lane & 15;
    const float lo = __shfl(la4[0], sl), hi = __shfl(la4[1], sl);
    return c < 16 ? lo : hi;
  };
  const int pr = kperm32(c);
  const size_t plane = (size_t)d.B * d.Hq * d.Nq;

  auto store = [&](uint16_t* H, float inv) __attribute__((always_inline)) {
    uint16_t* hp = H + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * gl;
        const uint32_t lo = pack_bf16x2(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv);
        const uint32_t hi2 = pack_bf16x2(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
        *(uint2*)(hp + d0) = make_uint2(lo, hi2);
      }
    }
  };
  auto snapshot = [&]() __attribute__((always_inline)) {
    l_sel = row_sum();
    const float lt = l_sel;
    store(Hs, 1.f / lt);
    if (lse != nullptr && gl == 0)
      lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  };

  // GEMM(e) = 16 MFMAs S(e) = K(e) Q^T plus 16 MFMAs O += V(e-1) P(e-1) and
  // 4 small ones adding P(e-1) into the row sums, branch-free: an entry a head
  // skips has S ignored and P = 0. The 32 LDS fragment reads are pipelined PF
  // ahead of the MFMAs that use them.
  auto gemm = [&](auto stc) __attribute__((always_inline)) {
    constexpr int sk = decltype(stc)::value;
    constexpr int sv = (sk + NST - 1) % NST;
    constexpr int PF = 4;
    const uint16_t* Kt = sk == 0 ? K0 : sk == 1 ? K1 : sk == 2 ? K2 : K3;
    const uint16_t* Vtl = sv == 0 ? V0 : sv == 1 ? V1 : sv == 2 ? V2 : V3;
    bf16x8_t fr[2 * NKS + 4 * NDT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int ch = 2 * ks + gl;
      fr[2 * ks] = *(const bf16x8_t*)(Kt + (pr * KSPR + kswz32(pr, ch)) * 8);
      fr[2 * ks + 1] = *(const bf16x8_t*)(Kt + ((32 + pr) * KSPR + kswz32(32 + pr, ch)) * 8);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int r = 32 * dt + c;
        fr[2 * NKS + s * NDT + dt] = *(const bf16x8_t*)(Vtl + (r * VSPR + vswz(r, 2 * s + gl)) * 8);
      }
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * ks + 1], qf[ks], s1, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 w = make_uint4(pw[4 * s], pw[4 * s + 1], pw[4 * s + 2], pw[4 * s + 3]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * NKS + s * NDT + dt], pb, o[dt], 0, 0, 0);
      la4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_a, pb, la4, 0, 0, 0);
    }
    // schedule: PF reads, then (1 MFMA, 1 read) pairs, then the last PF MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int k = 0; k < 2 * NKS + 4 * NDT - PF; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF + 4, 0);
  };
  // softmax(e): P(e) from S(e); the sparse snapshot is taken before the
  // first entry a head computes past its selected blocks. w is list entry
  // e's word (read before the slot opened).
  auto softmax = [&](int e, uint32_t w) __attribute__((always_inline)) {
    if (e == n_snap) snapshot();
    if (e >= n || ((w >> (12 + hs)) & 1u) == 0u) {
#pragma unroll
      for (int k = 0; k < 16; ++k) pw[k] = 0u;
      return;
    }
    const int kb = (int)(w & 0xfffu);
    if (kb == diag) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key0 = 16 * (v >> 3) + 8 * gl + (v & 7);
        if (key0 > qq) s0[v] = -INFINITY;
        if (key0 + 32 > qq) s1[v] = -INFINITY;
      }
    }
    // the block maximum only when some row's bound allows a rescale (always
    // for a row's first block, and for a NaN bound): two chains of
    // three-input maxima, 17 VALU operations for the 32 logits
    float m_blk = -INFINITY;
    if (__builtin_amdgcn_ballot_w64(!(qbound * __uint_as_float(w & 0xFFFF0000u) <= m_ref + kTau)) != 0) {
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        mx0 = max3f(mx0, s0[v], s1[v]);
        mx1 = max3f(mx1, s0[v + 1], s1[v + 1]);
      }
      m_blk = pair_max(fmaxf(mx0, mx1)) * sl2;
    }
    if (__builtin_amdgcn_ballot_w64(m_blk > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_blk);
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
      const float alpha_hi = __shfl_xor(alpha, 16);
      la4[0] *= alpha;
      la4[1] *= alpha_hi;
      l_sel *= alpha;   // the snapshot's sum, once taken
    }
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float a0 = fast_exp2(fmaf(s0[v], sl2, -m_ref));
      const float a1 = fast_exp2(fmaf(s0[v + 1], sl2, -m_ref));
      const float e0 = fast_exp2(fmaf(s1[v], sl2, -m_ref));
      const float e1 = fast_exp2(fmaf(s1[v + 1], sl2, -m_ref));
      pw[v >> 1] = pack_bf16x2(a0, a1);
      pw[8 + (v >> 1)] = pack_bf16x2(e0, e1);
    }
  };
  // Slots are opened by workgroup barriers. Group A runs GEMM(t) in slot 2t
  // and softmax(t) in slot 2t+1, group B one slot later; each wave requests
  // its share of K(t+NST-1) and V(t+NST-2) after its GEMM(t). Before a
  // wave's GEMM barrier, its copies needed by the next GEMM slot of either
  // group have landed: group A keeps the copies of its last NST-2 GEMM slots
  // in flight, group B those of its last NST-3.
  auto issue_tiles = [&](auto stc, int kbk, int kbv) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    load_k_kb(std::integral_constant<int, (st + NST - 1) % NST>{}, kbk);
    load_v_kb(std::integral_constant<int, (st + NST - 2) % NST>{}, kbv);
  };
  // Workgroup barrier that the compiler may not move memory accesses across;
  // this wave's LDS reads have completed before it (the stage it read may be
  // overwritten once the barrier opens).
  auto slot_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // s_waitcnt immediates: vmcnt(k), expcnt and lgkmcnt left open
  constexpr int kWaitA = 0xF70 | (2 * LPH * (NST - 2));
  constexpr int kWaitB = 0xF70 | (2 * LPH * (NST - 3));
  // group B's extra barrier opens slot 0, in which group A reads K(0)
  if (!group_a) {
    __builtin_amdgcn_s_waitcnt(kWaitA);
    slot_barrier();
  }
  // blocks of the copies issued after GEMM(t), looked up one slot pair
  // earlier (the lookups then wait only behind softmax work)
  int kbk = entry_kb_c(NST - 1), kbv = entry_kb_c(NST - 2);
  auto slots = [&](auto stc, int t) __attribute__((always_inline)) {
    if (group_a) __builtin_amdgcn_s_waitcnt(kWaitA);
    else __builtin_amdgcn_s_waitcnt(kWaitB);
    slot_barrier();
    __builtin_amdgcn_s_setprio(1);
    gemm(stc);
    __builtin_amdgcn_s_setprio(0);
    issue_tiles(stc, kbk, kbv);
    slot_barrier();
    // the blocks of the next copies and entry t's word: three LDS reads in
    // flight together, one wait
    const int nl = max(n - 1, 0);
    const uint32_t wk = list[min(t + NST, nl)], wv = list[min(t + NST - 1, nl)];
    const uint32_t we = list[min(t, nl)];
    // (with an empty list, n = 0 in sparse-only mode, the copies read a
    // stale word: any block index is in bounds or clipped by the buffer's
    // range check, and nothing reads those stages)
    kbk = __builtin_amdgcn_readfirstlane((int)wk) & 0xfff;
    kbv = __builtin_amdgcn_readfirstlane((int)wv) & 0xfff;
    softmax(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)we));
  };
  for (int t = 0; t <= n; t += NST) {
    slots(I0{}, t);
    if (t + 1 > n) break;
    slots(I1{}, t + 1);
    if (t + 2 > n) break;
    slots(I2{}, t + 2);
    if constexpr (NST > 3) {
      if (t + 3 > n) break;
      slots(I3{}, t + 3);
    }
  }
  if (group_a) slot_barrier();
  __builtin_amdgcn_s_waitcnt(0xF70);
  if (!sparse_only) {
    const float ls_t = l_sel;
    const float lt = row_sum();
    const float ld_t = fmaxf(lt - ls_t, 0.f);
    store(Hf, 1.f / lt);
    if (gl == 0) {
      if (delta != nullptr) delta[(size_t)bh * d.Nq + qrow] = ld_t / lt;
      if (lse != nullptr) lse[(size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
    }
  }
  }   // work items
}

// 16-token selection blocks, D = 64, G % 4 == 0 (the pages' model shape):
// one workgroup = one (b, kv head, 64-row query tile) serving four q heads,
// eight waves of 32 rows on MFMA 32x32x16 bf16 in the ping-pong slots of the
// kernel above (wave w: rows 32*(w/4) .. +31 of head w%4). A wave's rows
// span two 16-row query blocks with their own selections, so instead of
// walking selected blocks first, every causal 64-key tile is walked in order
// with two accumulators sharing one running max: o_all over every causal key
// and o_sel over the selected 16-key quarters (a lane's row's quarters come
// from per-(head, query block) bitmaps in LDS; the quarter of a key held in
// S^T register v is fixed by the kperm32 row order). Both PV products of an
// entry read the same V^T fragments; the selected one multiplies weights that
// are zero outside the row's quarters, so no branch touches the accumulators.
//     h_full = o_all / (l_sel + l_drop),  h_sparse = o_sel / l_sel,
//     delta = l_drop / (l_sel + l_drop).
template <int NST, int TPE>
__global__ __launch_bounds__(512, 2) void attn_prefill_bf16_pp16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vt, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hf, uint16_t* __restrict__ Hs, float* __restrict__ delta,
    float* __restrict__ lse, int* __restrict__ queues, const float* __restrict__ kn, Dims d,
    HeadMap hm) {
  constexpr int D = 64;
  constexpr int HPW = 4;
  constexpr int NW = 8;
  constexpr int KSPR = D / 8;
  constexpr int VSPR = kBlock / 8;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE = kBlock * D;
  constexpr int LPH = (TILE / 8) / (64 * NW);   // buffer loads per half tile (K or V) per wave
  // rescale slack 2^24, as in the kernel above, for the key-norm bound
  constexpr float kTau = 24.0f;
  constexpr int kWords16 = kMaxKeyBlocks / 32;
  static_assert(LPH == 1, "copy shape");
  // each stage holds TPE consecutive 64-key tiles (one list entry)
  __shared__ __align__(16) uint16_t K0[TPE * TILE], K1[TPE * TILE], K2[TPE * TILE],
      K3[NST > 3 ? TPE * TILE : 8];
  __shared__ __align__(16) uint16_t V0[TPE * TILE], V1[TPE * TILE], V2[TPE * TILE],
      V3[NST > 3 ? TPE * TILE : 8];
  __shared__ uint32_t sel16[HPW][4][kWords16];   // per head and 16-row query block
  __shared__ float knl[kMaxKeyBlocks];           // largest key norm of each causal tile

  const int ngrp = d.G / HPW;
  const int total = d.B * d.Hkv * ngrp * d.nQT;
  // work items as in the kernel above: persistent workgroups drawing from
  // per-XCD queues, or one item per workgroup in the static mapping
  __shared__ int s_item;
  const bool dyn = queues != nullptr && total % kNumXcd == 0;
  for (int pass = 0;; ++pass) {
  if (dyn) {
    __syncthreads();   // the previous item no longer reads LDS or s_item
    if (threadIdx.x == 0) s_item = fetch_work_item(queues, total / kNumXcd);
  } else {
    if (pass > 0) break;
    if (threadIdx.x == 0) s_item = xcd_remap(blockIdx.x, total);
  }
  __syncthreads();
  const int lin = s_item;
  if (lin < 0) break;   // every queue is empty
  const int per_group = ngrp * d.nQT;
  const int grp = lin / per_group;
  const int rem = lin - grp * per_group;
  const int qt = d.nQT - 1 - rem / ngrp;
  const int hg = rem - (rem / ngrp) * ngrp;
  const int b = grp / d.Hkv;
  const int g = grp - b * d.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave & 3;
  const bool group_a = wave < 4;
  const int h = hm.q_of_kv[g * d.G + hg * HPW + hs];
  const int bh = b * d.Hq + h;
  const int c = lane & 31, gl = lane >> 5;
  const int qq = (wave >> 2) * 32 + c;   // row within the tile
  const int qbl = qq >> 4;               // the row's 16-row query block within the tile
  const int qrow = qt * kBlock + qq;
  const float sl2 = d.scale_log2;
  const int ntiles = qt + 1;             // causal tiles
  const int n = (ntiles + TPE - 1) / TPE;   // entries of TPE tiles

  // ---- selection bitmaps of the four heads' four query blocks
  const int nwords16 = ((4 * qt + 3) >> 5) + 1;
  for (int i = tid; i < HPW * 4 * kWords16; i += 64 * NW) (&sel16[0][0][0])[i] = 0u;
  {
    // GEMM(0) multiplies the V stage of the (absent) entry -1 by P = 0
    uint16_t* vz = (NST - 1) == 1 ? V1 : (NST - 1) == 2 ? V2 : V3;
    for (int w = tid; w < TPE * TILE / 8; w += 64 * NW) ((uint4*)vz)[w] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  {
    const float* knr = kn + (size_t)(b * d.Hkv + g) * (d.Nk / kBlock);
    for (int t = tid; t < ntiles; t += 64 * NW) knl[t] = knr[t];
  }
  {
    // one thread per (head, query block, list entry): every list load is in
    // flight at once (entries past the count are read and ignored)
    int hq[HPW];
#pragma unroll
    for (int u = 0; u < HPW; ++u) hq[u] = hm.q_of_kv[g * d.G + hg * HPW + u];
    for (int t = tid; t < HPW * 4 * d.budget; t += 64 * NW) {
      const int l = t / d.budget, e = t - l * d.budget;
      const int u = l >> 2, qs = l & 3;
      const int hu = u == 0 ? hq[0] : u == 1 ? hq[1] : u == 2 ? hq[2] : hq[3];
      const size_t row = (size_t)(b * d.Hq + hu) * d.nQB + 4 * qt + qs;
      const int ns = cnt[row];
      const int kb = idx[row * d.budget + e];
      if (e < ns && kb >= 0 && kb <= 4 * qt + qs) atomicOr(&sel16[u][qs][kb >> 5], 1u << (kb & 31));
    }
  }
  __syncthreads();
  (void)nwords16;

  // ---- tiles
  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vt + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const i32x4_t krs = make_rsrc_words(kbase, (uint32_t)((size_t)d.Nk * D * 2));
  const i32x4_t vrs = make_rsrc_words(vbase, (uint32_t)((size_t)d.Nk * D * 2));
  const uint32_t k_row_bytes = D * 2, v_row_bytes = (uint32_t)d.Nk * 2;
  // copies past the last tile repeat it: every slot issues the same number
  // of copies, so the waits are static
  auto tile_c = [&](int t) __attribute__((always_inline)) { return min(t, ntiles - 1); };
  // the TPE tiles of entry e into a stage
  auto load_k_e = [&](auto stc, int e) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    uint16_t* kt = st == 0 ? K0 : st == 1 ? K1 : st == 2 ? K2 : K3;
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt)
      tile_to_lds_asm<KSPR, kBlock, NW, true>(
          krs, (uint32_t)tile_c(TPE * e + tt) * kBlock * k_row_bytes, k_row_bytes,
          kt + tt * TILE, wave, lane);
  };
  auto load_v_e = [&](auto stc, int e) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    uint16_t* vt = st == 0 ? V0 : st == 1 ? V1 : st == 2 ? V2 : V3;
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt)
      tile_to_lds_asm<VSPR, D, NW, false>(vrs, (uint32_t)tile_c(TPE * e + tt) * kBlock * 2,
                                         v_row_bytes, vt + tt * TILE, wave, lane);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 16 * ks);
  }
  // the Q fragments land before any LDS copy is issued: the compiler does
  // not count the copies, so it must see no load of its own outstanding
  __builtin_amdgcn_s_waitcnt(0xF70);
  // bound on this row's scaled logits against a tile (the kernel above)
  float qsq = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint4 u = __builtin_bit_cast(uint4, qf[ks]);
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
      qsq = fmaf(lo, lo, qsq);
      qsq = fmaf(hi, hi, qsq);
    }
  }
  const float qbound = sqrtf(pair_sum(qsq)) * sl2 * (1.f + 0x1p-10f);
  // prologue = the copies of the virtual slots before slot 0: K(0..NST-2)
  // and V(0..NST-3), with V(0) standing in for the missing V(-1)
  load_k_e(I0{}, 0);
  load_v_e(I0{}, 0);
  load_k_e(I1{}, 1);
  load_v_e(I0{}, 0);
  if constexpr (NST > 3) {
    load_k_e(I2{}, 2);
    load_v_e(I1{}, 1);
  }

  f32x16_t oa[NDT], os[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) { oa[i][v] = 0.f; os[i][v] = 0.f; }
  f32x16_t sc[TPE][2];      // S^T of the entry's tiles (keys 0-31, 32-63 of each)
  uint32_t pw[TPE][16];     // P as bf16 pairs; k-step s of tile tt's PV is pw[tt][4s .. 4s+3]
  uint32_t qmask = 0u;      // the row's selected quarters: 4 bits per tile of the entry pw holds
#pragma unroll
  for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
    for (int k = 0; k < 16; ++k) pw[tt][k] = 0u;
  float m_ref = -INFINITY;
  // Row sums on the matrix cores: a 16x16x32 MFMA reads the P^T operand of a
  // 32x32x16 k-step as its B operand (lane l: column l % 16, keys of k-group
  // l / 16, i.e. query 16 * ((l / 16) % 2) + l % 16); its 0/1 A operand adds
  // k-groups 0 and 2 into output row 0 and 1 and 3 into row 1. Lane n < 16
  // so holds the sum of query n in register 0 and of query n + 16 in
  // register 1: all weights in la4. The selected quarters' weights are added
  // by dot2 chains, only on entries where some row of the wave selected one.
  f32x4_t la4 = {0.f, 0.f, 0.f, 0.f};
  float l_sel = 0.f;
  const uint32_t one2 = (lane & 15) == ((lane >> 4) & 1) ? 0x3F803F80u : 0u;
  const bf16x8_t ones_a = __builtin_bit_cast(bf16x8_t, make_uint4(one2, one2, one2, one2));
  const int pr = kperm32(c);
  const size_t plane = (size_t)d.B * d.Hq * d.Nq;

  auto store = [&](uint16_t* H, const f32x16_t* o, float inv) __attribute__((always_inline)) {
    uint16_t* hp = H + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * gl;
        const uint32_t lo = pack_bf16x2(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv);
        const uint32_t hi2 = pack_bf16x2(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
        *(uint2*)(hp + d0) = make_uint2(lo, hi2);
      }
    }
  };

  // GEMM(e) = per tile 8 MFMAs S = K Q^T, plus per tile of entry e-1 2 x 8
  // MFMAs O_all += V P and O_sel += V P_sel on the same V^T fragments and 4
  // small MFMAs adding P into the row sums la4.
  auto gemm = [&](auto stc) __attribute__((always_inline)) {
    constexpr int sk = decltype(stc)::value;
    constexpr int sv = (sk + NST - 1) % NST;
    constexpr int PF = 4;
    constexpr int RK = 2 * NKS, RV = 4 * NDT;   // fragment reads per tile
    const uint16_t* Kt = sk == 0 ? K0 : sk == 1 ? K1 : sk == 2 ? K2 : K3;
    const uint16_t* Vtl = sv == 0 ? V0 : sv == 1 ? V1 : sv == 2 ? V2 : V3;
    bf16x8_t fr[TPE * (RK + RV)];
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt) {
      const uint16_t* kt = Kt + tt * TILE;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int ch = 2 * ks + gl;
        fr[tt * RK + 2 * ks] = *(const bf16x8_t*)(kt + (pr * KSPR + vswz(pr, ch)) * 8);
        fr[tt * RK + 2 * ks + 1] = *(const bf16x8_t*)(kt + ((32 + pr) * KSPR + vswz(32 + pr, ch)) * 8);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt) {
      const uint16_t* vt = Vtl + tt * TILE;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int r = 32 * dt + c;
          fr[TPE * RK + tt * RV + s * NDT + dt] =
              *(const bf16x8_t*)(vt + (r * VSPR + vswz(r, 2 * s + gl)) * 8);
        }
    }
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) { sc[tt][0][v] = 0.f; sc[tt][1][v] = 0.f; }
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sc[tt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[tt * RK + 2 * ks], qf[ks], sc[tt][0], 0, 0, 0);
        sc[tt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[tt * RK + 2 * ks + 1], qf[ks], sc[tt][1], 0, 0, 0);
      }
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // k-step s of tile tt covers its keys 16s .. 16s+15: quarter 4*tt + s
        const uint32_t keep = ((qmask >> (4 * tt + s)) & 1u) ? 0xFFFFFFFFu : 0u;
        const uint4 w = make_uint4(pw[tt][4 * s], pw[tt][4 * s + 1], pw[tt][4 * s + 2], pw[tt][4 * s + 3]);
        const uint4 ws = make_uint4(pw[tt][4 * s] & keep, pw[tt][4 * s + 1] & keep,
                                    pw[tt][4 * s + 2] & keep, pw[tt][4 * s + 3] & keep);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
        const bf16x8_t psb = __builtin_bit_cast(bf16x8_t, ws);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8_t vf = fr[TPE * RK + tt * RV + s * NDT + dt];
          oa[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, oa[dt], 0, 0, 0);
          os[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, psb, os[dt], 0, 0, 0);
        }
        la4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_a, pb, la4, 0, 0, 0);
      }
    // schedule: PF reads, then MFMAs interleaved with the remaining reads
    constexpr int NR = TPE * (RK + RV);
    constexpr int NM = TPE * (2 * NKS + 8 * NDT + 4);
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int k = 0; k < NR - PF; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - PF), 0);
  };
  // softmax(e): P of the entry's tiles from S; per tile the row's selected
  // quarters; register v of sc[tt][0] holds quarter v / 8, of sc[tt][1]
  // quarter 2 + v / 8 (kperm32 order), so pw[tt][k] belongs to quarter k / 4
  auto softmax = [&](int e) __attribute__((always_inline)) {
    if (e >= n) {
#pragma unroll
      for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
        for (int k = 0; k < 16; ++k) pw[tt][k] = 0u;
      qmask = 0u;
      return;
    }
    uint32_t nibs = 0u;
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt) {
      const int t = TPE * e + tt;
      if (t <= qt) nibs |= ((sel16[hs][qbl][t >> 3] >> ((4 * t) & 31)) & 0xFu) << (4 * tt);
      if (t >= qt) {   // the diagonal tile: key <= row; tiles past it: nothing
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key0 = 16 * (v >> 3) + 8 * gl + (v & 7);
          if (t > qt || key0 > qq) sc[tt][0][v] = -INFINITY;
          if (t > qt || key0 + 32 > qq) sc[tt][1][v] = -INFINITY;
        }
      }
    }
    // the entry's maximum only when some row's bound allows a rescale
    float knb = 0.f;
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt) knb = fmaxf(knb, knl[tile_c(TPE * e + tt)]);
    float m_blk = -INFINITY;
    if (__builtin_amdgcn_ballot_w64(!(qbound * knb <= m_ref + kTau)) != 0) {
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          mx0 = max3f(mx0, sc[tt][0][v], sc[tt][1][v]);
          mx1 = max3f(mx1, sc[tt][0][v + 1], sc[tt][1][v + 1]);
        }
      m_blk = pair_max(fmaxf(mx0, mx1)) * sl2;
    }
    if (__builtin_amdgcn_ballot_w64(m_blk > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_blk);
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) { oa[i][v] *= alpha; os[i][v] *= alpha; }
      // the sums of lane n < 16 belong to queries n and n + 16
      const float alpha_hi = __shfl_xor(alpha, 16);
      la4[0] *= alpha;
      la4[1] *= alpha_hi;
      l_sel *= alpha;
    }
#pragma unroll
    for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float a0 = fast_exp2(fmaf(sc[tt][0][v], sl2, -m_ref));
        const float a1 = fast_exp2(fmaf(sc[tt][0][v + 1], sl2, -m_ref));
        const float e0 = fast_exp2(fmaf(sc[tt][1][v], sl2, -m_ref));
        const float e1 = fast_exp2(fmaf(sc[tt][1][v + 1], sl2, -m_ref));
        pw[tt][v >> 1] = pack_bf16x2(a0, a1);
        pw[tt][8 + (v >> 1)] = pack_bf16x2(e0, e1);
      }
    if (__builtin_amdgcn_ballot_w64(nibs != 0u) != 0) {
      // per quarter dot2 chains; the row's selected quarters go to l_sel
      float qs[4 * TPE];
#pragma unroll
      for (int u = 0; u < 4 * TPE; ++u) qs[u] = 0.f;
#pragma unroll
      for (int tt = 0; tt < TPE; ++tt)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          qs[4 * tt + (v >> 3)] = add_bf16x2(pw[tt][v >> 1], qs[4 * tt + (v >> 3)]);
          qs[4 * tt + 2 + (v >> 3)] = add_bf16x2(pw[tt][8 + (v >> 1)], qs[4 * tt + 2 + (v >> 3)]);
        }
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < 4 * TPE; ++u) ls += ((nibs >> u) & 1u) ? qs[u] : 0.f;
      l_sel += ls;
    }
    qmask = nibs;
  };
  // Slots as in the kernel above: group A runs GEMM(t) in slot 2t and
  // softmax(t) in slot 2t+1, group B one slot later; each wave requests its
  // share of K(t+NST-1) and V(t+NST-2) after its GEMM(t).
  auto issue_tiles = [&](auto stc, int t) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    load_k_e(std::integral_constant<int, (st + NST - 1) % NST>{}, t + NST - 1);
    load_v_e(std::integral_constant<int, (st + NST - 2) % NST>{}, t + NST - 2);
  };
  auto slot_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  constexpr int kWaitA = 0xF70 | (2 * LPH * TPE * (NST - 2));
  constexpr int kWaitB = 0xF70 | (2 * LPH * TPE * (NST - 3));
  if (!group_a) {
    __builtin_amdgcn_s_waitcnt(kWaitA);
    slot_barrier();
  }
  auto slots = [&](auto stc, int t) __attribute__((always_inline)) {
    if (group_a) __builtin_amdgcn_s_waitcnt(kWaitA);
    else __builtin_amdgcn_s_waitcnt(kWaitB);
    slot_barrier();
    __builtin_amdgcn_s_setprio(1);
    gemm(stc);
    __builtin_amdgcn_s_setprio(0);
    issue_tiles(stc, t);
    slot_barrier();
    softmax(t);
  };
  for (int t = 0; t <= n; t += NST) {
    slots(I0{}, t);
    if (t + 1 > n) break;
    slots(I1{}, t + 1);
    if (t + 2 > n) break;
    slots(I2{}, t + 2);
    if constexpr (NST > 3) {
      if (t + 3 > n) break;
      slots(I3{}, t + 3);
    }
  }
  if (group_a) slot_barrier();
  __builtin_amdgcn_s_waitcnt(0xF70);
  const int sum_lane = lane & 15;   // holds this row's sum of all weights
  const float lt_lo = __shfl(la4[0], sum_lane), lt_hi = __shfl(la4[1], sum_lane);
  const float lt = c < 16 ? lt_lo : lt_hi;   // all weights
  const float ls_t = pair_sum(l_sel);
  const float ld_t = fmaxf(lt - ls_t, 0.f);
  store(Hs, os, 1.f / ls_t);
  store(Hf, oa, 1.f / lt);
  if (gl == 0) {
    if (delta != nullptr) delta[(size_t)bh * d.Nq + qrow] = ld_t / lt;
    if (lse != nullptr) {
      lse[(size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
      lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(ls_t)) * kLn2;
    }
  }
  }   // work items
}

// Sparse-only prefill with 16-token blocks (h_full == NULL, one list per
// 16-row query block): only the selected keys are read and multiplied. A wave
// owns one list (16 query rows) and walks its selected blocks two at a time
// (32 keys), gathered straight from L2 into MFMA operand registers: no LDS,
// no barriers, and exactly the algorithmic MFMA work of the sparse stream
// ("SSA: Achieving Sparser Attention ...", section "Practical Implementation
// of SSA": attention over the concatenated keys and values of the selected
// blocks only).
//
// MFMA 16x16x32 bf16. S^T = K Q^T: the pair's 32 keys sit at positions
// p = 0..15 (first block) and 16..31 (second); MFMA tile t reads, in row r,
// the key at position 8*(r/4) + 4*t + r%4, so lane group g (lanes 16g ..
// 16g+15) receives positions 8g .. 8g+7 across the two tiles: exactly the
// eight keys of the PV B operand for k = 8g .. 8g+7, which are consecutive
// keys of one block. V^T comes in the per-block layout [n/16][d][16] (made
// by the V transpose for these calls), so the V^T operand of a block is 16
// contiguous 32-byte rows: one 16-byte load per lane and d tile, whole cache
// lines per wave. Lanes of rows r < 8 gather K from the first block, r >= 8
// from the second. The diagonal block is masked per key (key > row gives
// -inf); an odd count ends with a masked second half. Online softmax with
// lazy rescaling as in the other kernels; each lane keeps partial row sums
// over its keys, reduced over the four lanes of its query at the end.
//
// A workgroup is four consecutive lists in (b, kv head, query block, q head
// of the group) order, so its waves share most of their blocks through L1
// and L2 (the sink and diagonal blocks always).
constexpr int kGatherLists = 4;   // lists (waves) per workgroup
template <int D>
__global__ __launch_bounds__(64 * kGatherLists) void attn_sparse_gather_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vb, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hs, float* __restrict__ lse, Dims d, HeadMap hm) {
  constexpr int NKS = D / 32;    // k-steps of QK^T
  constexpr int NDT = D / 16;    // 16-wide d tiles of O^T
  constexpr float kTau = 8.0f;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, g4 = lane >> 4;

  // ---- which list
  const int nlists = d.B * d.Hkv * d.nQB * d.G;
  const int nwg = (nlists + kGatherLists - 1) / kGatherLists;
  const int li = kGatherLists * xcd_remap(blockIdx.x, nwg) + wave;   // (b, g, qb, head) order
  if (li >= nlists) return;
  const int hi = li % d.G;
  const int qb = (li / d.G) % d.nQB;
  const int bg = li / (d.G * d.nQB);
  const int b = bg / d.Hkv, g = bg - b * d.Hkv;
  const int h = hm.q_of_kv[g * d.G + hi];
  const int bh = b * d.Hq + h;
  const int q0 = qb * 16;
  const int qrow = q0 + n;
  const size_t lrow = (size_t)bh * d.nQB + qb;
  const int* list = idx + lrow * d.budget;
  const int nsub = __builtin_amdgcn_readfirstlane(min(max(cnt[lrow], 0), d.budget));
  auto sub_start = [&](int s) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane(list[s]) * 16;
  };

  const float sl2 = d.scale_log2;
  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vb + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)((size_t)d.Nk * D * 2));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (uint32_t)((size_t)d.Nk * D * 2));
  // per-lane byte offsets: K row of tiles 0 and 1 (key within its block, d
  // chunk), V^T row (d) and key chunk within the block's [d][16] tile
  const bool first_half = n < 8;
  const int kin0 = (8 * (n >> 2) + (n & 3)) & 15;   // tile 0 key (tile 1: +4)
  const uint32_t koff0 = (uint32_t)((kin0 * D + 8 * g4) * 2);
  const uint32_t koff1 = (uint32_t)(((kin0 + 4) * D + 8 * g4) * 2);
  const bool vfirst = g4 < 2;
  const uint32_t voff_lane = (uint32_t)(n * 32 + (g4 & 1) * 16);

  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 32 * ks);
  }

  struct Frags { bf16x8_t k0[NKS], k1[NKS], v[NDT]; };
  // a block starting at key s: K rows s*D*2 bytes in, V^T tile s*D*2 bytes in
  auto load_pair = [&](Frags& f, int ka, int kb2) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)(first_half ? ka : kb2) * (uint32_t)(D * 2);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f.k0[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
          krs, kb + koff0 + 64u * ks, 0, 0));
      f.k1[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
          krs, kb + koff1 + 64u * ks, 0, 0));
    }
    const uint32_t vk = (uint32_t)(vfirst ? ka : kb2) * (uint32_t)(D * 2) + voff_lane;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      f.v[dt] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
          vrs, vk + 512u * dt, 0, 0));
  };

  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  // row sums on the matrix cores: with an all-ones A operand a 16x16x32 MFMA
  // gives every lane of a query column the column's sum (register 0 is read)
  f32x4_t l4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones16 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                  0x3F803F80u, 0x3F803F80u));

  // one pair: blocks starting at keys ka and kb2; kb2 < 0: no second one
  auto compute = [&](const Frags& f, int ka, int kb2) __attribute__((always_inline)) {
    f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k0[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k1[ks], qf[ks], s1, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // keys past the row (the diagonal block) and a missing second half
    if (ka + 15 > q0 || kb2 < 0 || kb2 + 15 > q0) {
      const int kbase_l = vfirst ? ka : kb2;
      const bool dead = !vfirst && kb2 < 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key0 = kbase_l + 8 * (g4 & 1) + v;   // tile 0 key of this lane's value v
        if (dead || key0 > qrow) s0[v] = -INFINITY;
        if (dead || key0 + 4 > qrow) s1[v] = -INFINITY;
      }
    }
    const float mx = fmaxf(max3f(s0[0], s0[1], s0[2]), max3f(s0[3], s1[0], max3f(s1[1], s1[2], s1[3])));
    const float m_blk = quad_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(m_blk > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_blk);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[i][v] *= alpha;
      l4[0] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    uint32_t pw[4];
    pw[0] = pack_bf16x2(fast_exp2(fmaf(s0[0], sl2, -m_use)), fast_exp2(fmaf(s0[1], sl2, -m_use)));
    pw[1] = pack_bf16x2(fast_exp2(fmaf(s0[2], sl2, -m_use)), fast_exp2(fmaf(s0[3], sl2, -m_use)));
    pw[2] = pack_bf16x2(fast_exp2(fmaf(s1[0], sl2, -m_use)), fast_exp2(fmaf(s1[1], sl2, -m_use)));
    pw[3] = pack_bf16x2(fast_exp2(fmaf(s1[2], sl2, -m_use)), fast_exp2(fmaf(s1[3], sl2, -m_use)));
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.v[dt], pb, o[dt], 0, 0, 0);
    l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones16, pb, l4, 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // pairs of blocks, the next pair's loads in flight during this one's
  const int npairs = (nsub + 1) >> 1;
  auto starts = [&](int i, int& ka, int& kb2) __attribute__((always_inline)) {
    ka = sub_start(2 * i);
    kb2 = 2 * i + 1 < nsub ? sub_start(2 * i + 1) : -1;
  };
  Frags fa, fb;
  int ka = 0, kb2 = -1, na = 0, nb2 = -1;
  if (npairs > 0) {
    starts(0, ka, kb2);
    load_pair(fa, ka, kb2 < 0 ? ka : kb2);
  }
  for (int i = 0; i < npairs; i += 2) {
    if (i + 1 < npairs) {
      starts(i + 1, na, nb2);
      load_pair(fb, na, nb2 < 0 ? na : nb2);
    }
    compute(fa, ka, kb2);
    if (i + 1 >= npairs) break;
    if (i + 2 < npairs) {
      starts(i + 2, ka, kb2);
      load_pair(fa, ka, kb2 < 0 ? ka : kb2);
    }
    compute(fb, na, nb2);
  }

  const float lt = l4[0];
  const float inv = 1.f / lt;
  uint16_t* hp = Hs + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const uint32_t lo = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    const uint32_t hi2 = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    *(uint2*)(hp + 16 * dt + 4 * g4) = make_uint2(lo, hi2);
  }
  if (lse != nullptr && g4 == 0) {
    const size_t plane = (size_t)d.B * d.Hq * d.Nq;
    lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
}

// Sparse-only prefill, 16-token blocks, q heads per kv head a multiple of 4:
// one workgroup = (b, kv head, 16-row query block, four q heads of the
// group), one wave per head. The four heads' lists are merged into their
// union (ascending, with a 4-bit mask of the heads that selected each block),
// and the union's K rows and V^T tiles pass through LDS in chunks of CAP
// blocks, each loaded once for the four heads (the heads of a group share
// most blocks: the sink and the diagonal always). Small chunks (16 KB of LDS
// at D 64) let five workgroups share a CU, whose loads and list set-up
// overlap the others' MFMA work: measured faster than 8- and 16-block chunks
// despite more odd-block padding. Per chunk each wave takes
// its own selected blocks two at a time with the S^T / PV operand mapping of
// attn_sparse_gather_kernel, reading the fragments from LDS; an odd block
// left at the end of a chunk is paired with a masked half. Exactly the
// selected keys enter the softmax; only that padding adds MFMA work.
//
// LDS layouts (16-byte chunks): K block slot s, key row r, logical chunk c at
// position s*2D + r*(D/8) + (c ^ kf(r, s)); V^T block slot s, d row, key half
// h at s*2D + 2*d + (h ^ ((d >> 3) & 1)). kf spreads the 16 rows one
// ds_read_b128 phase reads (8 rows of each of the pair's two blocks) over
// distinct bank groups whenever the two slots differ in parity.
template <int D>
__device__ __forceinline__ int kf16(int r, int s) {
  if constexpr (D == 64) return ((r >> 1) & 7) ^ ((s & 1) << 1);
  else return (r & 3) | ((r >> 1) & 4) | ((s & 1) << 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_sparse_union16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vb, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hs, float* __restrict__ lse, Dims d, HeadMap hm) {
  constexpr int NKS = D / 32, NDT = D / 16, KCH = D / 8;
  constexpr int CAP = D == 64 ? 4 : 2;             // union blocks per LDS chunk
  constexpr int PCS = 2 * D;                      // 16-byte pieces per block tile
  constexpr int kMaxWords = kMaxKeyBlocks / 32;
  constexpr float kTau = 8.0f;
  __shared__ __align__(16) uint16_t Ks[CAP * PCS * 8];
  __shared__ __align__(16) uint16_t Vs[CAP * PCS * 8];
  __shared__ uint32_t sel[4][kMaxWords];
  __shared__ uint16_t ulist[kMaxKeyBlocks];
  __shared__ int s_nu;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int n = lane & 15, g4 = lane >> 4;
  const int ngrp = d.G / 4;
  const int total = d.B * d.Hkv * ngrp * d.nQB;
  const int lin = xcd_remap(blockIdx.x, total);   // (b, g, qb, head group) order
  const int hg = lin % ngrp;
  const int qb = (lin / ngrp) % d.nQB;
  const int bg = lin / (ngrp * d.nQB);
  const int b = bg / d.Hkv, g = bg - b * d.Hkv;
  const int h = hm.q_of_kv[g * d.G + 4 * hg + wave];
  const int bh = b * d.Hq + h;
  const int diag = qb;
  const int q0 = qb * 16, qrow = q0 + n;
  const int nwords = (diag >> 5) + 1;

  // ---- union of the four lists
  for (int i = tid; i < 4 * kMaxWords; i += 256) (&sel[0][0])[i] = 0u;
  __syncthreads();
  {
    const size_t lrow = (size_t)bh * d.nQB + qb;
    const int ns = min(max(cnt[lrow], 0), d.budget);
    for (int e = lane; e < ns; e += 64) {
      const int kb = idx[lrow * d.budget + e];
      if (kb >= 0 && kb <= diag) atomicOr(&sel[wave][kb >> 5], 1u << (kb & 31));
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane l owns words 2l and 2l+1 (kMaxWords <= 128)
    uint32_t any[2], cntw = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int w = 2 * lane + j;
      any[j] = w < nwords ? (sel[0][w] | sel[1][w] | sel[2][w] | sel[3][w]) : 0u;
      cntw += __popc(any[j]);
    }
    int incl = (int)cntw;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int pos = incl - (int)cntw;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int w = 2 * lane + j;
      for (uint32_t bb = any[j]; bb != 0u; bb &= bb - 1u) {
        const int bit = __builtin_ctz(bb);
        uint32_t act = 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) act |= ((sel[u][w] >> bit) & 1u) << u;
        ulist[pos++] = (uint16_t)(((w << 5) + bit) | (act << 12));
      }
    }
    if (lane == 63) s_nu = incl;
  }
  __syncthreads();
  const int nu = s_nu;

  // ---- per-wave state
  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 32 * ks);
  }
  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  // row sums on the matrix cores: with an all-ones A operand a 16x16x32 MFMA
  // gives every lane of a query column the column's sum (register 0 is read)
  f32x4_t l4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones16 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                  0x3F803F80u, 0x3F803F80u));
  const float sl2 = d.scale_log2;
  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vb + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const bool first_half = n < 8;
  const int kin0 = (8 * (n >> 2) + (n & 3)) & 15;   // tile 0 key of this lane's row (tile 1: +4)
  const bool vfirst = g4 < 2;

  // one pair: blocks in LDS slots sa, sb (sb < 0: none) starting at keys ka, kb2
  auto pair = [&](int sa, int sb, int ka, int kb2) __attribute__((always_inline)) {
    const int sk = first_half ? sa : (sb < 0 ? sa : sb);
    const int sv = vfirst ? sa : (sb < 0 ? sa : sb);
    bf16x8_t k0[NKS], k1[NKS], vf[NDT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int c = 4 * ks + g4;
      k0[ks] = *(const bf16x8_t*)(Ks + (sk * PCS + kin0 * KCH + (c ^ kf16<D>(kin0, sk))) * 8);
      k1[ks] = *(const bf16x8_t*)(Ks + (sk * PCS + (kin0 + 4) * KCH + (c ^ kf16<D>(kin0 + 4, sk))) * 8);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int dd = 16 * dt + n;
      vf[dt] = *(const bf16x8_t*)(Vs + (sv * PCS + 2 * dd + ((g4 & 1) ^ ((dd >> 3) & 1))) * 8);
    }
    f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[ks], qf[ks], s1, 0, 0, 0);
    }
    if (ka + 15 > q0 || kb2 < 0 || kb2 + 15 > q0) {
      const int kbase_l = vfirst ? ka : kb2;
      const bool dead = !vfirst && kb2 < 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key0 = kbase_l + 8 * (g4 & 1) + v;
        if (dead || key0 > qrow) s0[v] = -INFINITY;
        if (dead || key0 + 4 > qrow) s1[v] = -INFINITY;
      }
    }
    const float mx = fmaxf(max3f(s0[0], s0[1], s0[2]), max3f(s0[3], s1[0], max3f(s1[1], s1[2], s1[3])));
    const float m_blk = quad_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(m_blk > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_blk);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[i][v] *= alpha;
      l4[0] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    uint32_t pw[4];
    pw[0] = pack_bf16x2(fast_exp2(fmaf(s0[0], sl2, -m_use)), fast_exp2(fmaf(s0[1], sl2, -m_use)));
    pw[1] = pack_bf16x2(fast_exp2(fmaf(s0[2], sl2, -m_use)), fast_exp2(fmaf(s0[3], sl2, -m_use)));
    pw[2] = pack_bf16x2(fast_exp2(fmaf(s1[0], sl2, -m_use)), fast_exp2(fmaf(s1[1], sl2, -m_use)));
    pw[3] = pack_bf16x2(fast_exp2(fmaf(s1[2], sl2, -m_use)), fast_exp2(fmaf(s1[3], sl2, -m_use)));
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb, o[dt], 0, 0, 0);
    l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones16, pb, l4, 0, 0, 0);
  };

  for (int c0 = 0; c0 < nu; c0 += CAP) {
    const int nc = min(CAP, nu - c0);
    __syncthreads();   // every wave is done with the previous chunk's tiles
    // copy the chunk: K rows and V^T tiles of nc blocks, 16 bytes per thread
    for (int i = tid; i < nc * PCS; i += 256) {
      const int s = i / PCS, rem = i - s * PCS;
      const int kb = ulist[c0 + s] & 0xfff;
      {
        const int r = rem / KCH, p = rem - r * KCH;
        const int c = p ^ kf16<D>(r, s);
        *(uint4*)(Ks + i * 8) = *(const uint4*)(kbase + ((size_t)kb * 16 + r) * D + c * 8);
      }
      {
        const int dd = rem >> 1, hh = (rem & 1) ^ ((dd >> 3) & 1);
        *(uint4*)(Vs + i * 8) = *(const uint4*)(vbase + ((size_t)kb * D + dd) * 16 + hh * 8);
      }
    }
    __syncthreads();
    // this wave's blocks in the chunk, in pairs
    const int e = c0 + lane;
    const bool mine = lane < nc && ((ulist[e] >> (12 + wave)) & 1u);
    uint64_t m = __builtin_amdgcn_ballot_w64(mine);
    while (m != 0ull) {
      const int sa = __builtin_ctzll(m);
      m &= m - 1ull;
      const int sb = m != 0ull ? __builtin_ctzll(m) : -1;
      if (m != 0ull) m &= m - 1ull;
      const int ka = (ulist[c0 + sa] & 0xfff) * 16;
      const int kb2 = sb >= 0 ? (ulist[c0 + sb] & 0xfff) * 16 : -1;
      pair(sa, sb, __builtin_amdgcn_readfirstlane(ka), __builtin_amdgcn_readfirstlane(kb2));
    }
  }

  const float lt = l4[0];
  const float inv = 1.f / lt;
  uint16_t* hp = Hs + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const uint32_t lo = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    const uint32_t hi2 = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    *(uint2*)(hp + 16 * dt + 4 * g4) = make_uint2(lo, hi2);
  }
  if (lse != nullptr && g4 == 0) {
    const size_t plane = (size_t)d.B * d.Hq * d.Nq;
    lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
}

// Compute units of the current device (cached per device; threads that race
// on the first call store the same value).
static hipError_t compute_units(int* out) {
  static std::atomic<int> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) { *out = c; return hipSuccess; }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) n = 1;
  if (slot) cached[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

hipError_t launch_attn_prefill_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                                    const int* idx, const int* cnt, uint16_t* hf, uint16_t* hs,
                                    float* delta, float* lse, int* queues, const float* kn,
                                    const Dims& d, const HeadMap& hm, hipStream_t stream) {
  if (d.tok) {   // per-token lists
    const int tiles = d.B * d.Hq * d.nQT;
#define SSA_TOK_LAUNCH(DD, TT)                                                                  \
  hipLaunchKernelGGL((attn_prefill_bf16_q16_kernel<DD, TT>), dim3(tiles), dim3(256), 0, stream, \
                     q, k, vt, idx, cnt, hf, hs, delta, lse, d, hm)
    if (d.D == 128) {
      if (d.bs == 16) SSA_TOK_LAUNCH(128, 16); else SSA_TOK_LAUNCH(128, 64);
    } else {
      if (d.bs == 16) SSA_TOK_LAUNCH(64, 16); else SSA_TOK_LAUNCH(64, 64);
    }
#undef SSA_TOK_LAUNCH
    return hipGetLastError();
  }
  if (prefill_vt_blk16(d, hf == nullptr) && d.G % 4 == 0) {
    // sparse-only, 16-token per-block lists, four q heads per workgroup
    const int total = d.B * d.Hkv * (d.G / 4) * d.nQB;
    if (d.D == 128)
      hipLaunchKernelGGL((attn_sparse_union16_kernel<128>), dim3(total), dim3(256), 0, stream, q,
                         k, vt, idx, cnt, hs, lse, d, hm);
    else
      hipLaunchKernelGGL((attn_sparse_union16_kernel<64>), dim3(total), dim3(256), 0, stream, q,
                         k, vt, idx, cnt, hs, lse, d, hm);
    return hipGetLastError();
  }
  if (prefill_vt_blk16(d, hf == nullptr)) {
    // sparse-only, 16-token per-block lists: gather only the selected keys
    const int nlists = d.B * d.Hkv * d.nQB * d.G;
    const int nwg = (nlists + kGatherLists - 1) / kGatherLists;
    if (d.D == 128)
      hipLaunchKernelGGL((attn_sparse_gather_kernel<128>), dim3(nwg), dim3(64 * kGatherLists), 0, stream, q, k,
                         vt, idx, cnt, hs, lse, d, hm);
    else
      hipLaunchKernelGGL((attn_sparse_gather_kernel<64>), dim3(nwg), dim3(64 * kGatherLists), 0, stream, q, k,
                         vt, idx, cnt, hs, lse, d, hm);
    return hipGetLastError();
  }
  if (d.bs == 16 && d.D == 64 && d.G % 4 == 0 && hf != nullptr) {
    // dual mode, four q heads per workgroup
    const int groups = d.B * d.Hkv * (d.G / 4) * d.nQT;
    const bool dyn = queues != nullptr && groups % kNumXcd == 0;
    int grid = groups;
    if (dyn) {
      int cus = 0;
      const hipError_t e = compute_units(&cus);
      if (e != hipSuccess) return e;
      grid = std::min(groups, cus);
    }
    if (kn == nullptr) return hipErrorInvalidValue;   // prefill_key_norms holds here
    hipLaunchKernelGGL((attn_prefill_bf16_pp16_kernel<3, 2>), dim3(grid), dim3(512), 0, stream,
                       q, k, vt, idx, cnt, hf, hs, delta, lse, dyn ? queues : nullptr, kn, d, hm);
    return hipGetLastError();
  }
  if (d.bs == 16) {
    const int tiles = d.B * d.Hq * d.nQT;
    if (d.D == 128)
      hipLaunchKernelGGL((attn_prefill_bf16_q16_kernel<128, 0>), dim3(tiles), dim3(256), 0, stream,
                         q, k, vt, idx, cnt, hf, hs, delta, lse, d, hm);
    else
      hipLaunchKernelGGL((attn_prefill_bf16_q16_kernel<64, 0>), dim3(tiles), dim3(256), 0, stream,
                         q, k, vt, idx, cnt, hf, hs, delta, lse, d, hm);
    return hipGetLastError();
  }
  // dual mode with four q heads per workgroup; sparse-only calls go to the
  // per-head kernel, which walks only each head's own selected blocks
  if (d.D == 128 && d.G % 4 == 0 && hf != nullptr) {
    const int groups = d.B * d.Hkv * (d.G / 4) * d.nQB;
    // with queues: one persistent workgroup per CU (one fits per CU)
    const bool dyn = queues != nullptr && groups % kNumXcd == 0;
    int grid = groups;
    if (dyn) {
      int cus = 0;
      const hipError_t e = compute_units(&cus);
      if (e != hipSuccess) return e;
      grid = std::min(groups, cus);
    }
    if (kn == nullptr) return hipErrorInvalidValue;   // prefill_key_norms holds here
    hipLaunchKernelGGL((attn_prefill_bf16_pp_kernel<128, 3>), dim3(grid), dim3(512), 0, stream,
                       q, k, vt, idx, cnt, hf, hs, delta, lse, dyn ? queues : nullptr, kn, d, hm);
    return hipGetLastError();
  }
  const int total = d.B * d.Hq * d.nQB;
  if (d.D == 128)
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<128>, dim3(total), dim3(256), 0, stream, q, k,
                       vt, idx, cnt, hf, hs, delta, lse, d, hm);
  else
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<64>, dim3(total), dim3(256), 0, stream, q, k,
                       vt, idx, cnt, hf, hs, delta, lse, d, hm);
  return hipGetLastError();
}

// ---------------------------------------------------------------- float32
// Plain VALU kernel for float32 problems (prefill and decode): one wave per
// (b, q head, row block); lane r owns query row r of the block. Same walk:
// selected blocks, snapshot, remaining causal blocks. With per-token lists
// the rows of a block select different blocks, so the sparse stream runs as
// its own pass over the blocks some row selected (each lane masks the blocks
// its row did not select), and the full stream as a second pass over every
// causal block.
template <int D>
__global__ __launch_bounds__(64) void attn_rows_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int* __restrict__ idx, const int* __restrict__ cnt, float* __restrict__ Hf,
    float* __restrict__ Hs, float* __restrict__ delta, float* __restrict__ lse, Dims d,
    HeadMap hm) {
  __shared__ __align__(16) float Ks[kBlock][D];
  __shared__ __align__(16) float Vs[kBlock][D];
  constexpr int SUB = 16;

  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = hm.kv_of_q[h];
  const int bh = b * d.Hq + h;
  const int lane = threadIdx.x;
  const int rows = min(kBlock, d.Nq - qb * kBlock);
  const bool active = lane < rows;
  const int row = qb * kBlock + (active ? lane : rows - 1);
  const int pos = d.Nk - d.Nq + row;
  const int diag = row_block_diag(d, qb);
  const float sl2 = d.scale_log2;

  float q[D], acc[D];
  const float* qp = Q + ((size_t)bh * d.Nq + row) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) { q[i] = qp[i] * sl2; acc[i] = 0.f; }
  float m_run = -INFINITY, l_sel = 0.f, l_drop = 0.f;
  const float* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const float* vbase = V + ((size_t)(b * d.Hkv + g) * d.Nk) * D;

  auto process = [&](int kb, bool selected, bool use) {
    const float* kg = kbase + (size_t)kb * kBlock * D;
    const float* vg = vbase + (size_t)kb * kBlock * D;
    for (int i = lane; i < kBlock * D / 4; i += 64) {
      ((float4*)&Ks[0][0])[i] = ((const float4*)kg)[i];
      ((float4*)&Vs[0][0])[i] = ((const float4*)vg)[i];
    }
    __syncthreads();
    for (int j0 = 0; j0 < kBlock; j0 += SUB) {
      float s[SUB];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) a = fmaf(q[i], Ks[j0 + j][i], a);
        if (kb * kBlock + j0 + j > pos || !use) a = -INFINITY;
        s[j] = a;
        mx = fmaxf(mx, a);
      }
      const float m_new = fmaxf(m_run, mx);
      if (m_new == -INFINITY) continue;
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] *= alpha;
      l_sel *= alpha;
      l_drop *= alpha;
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        const float p = exp2f(s[j] - m_new);
        ls += p;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] = fmaf(p, Vs[j0 + j][i], acc[i]);
      }
      if (selected) l_sel += ls; else l_drop += ls;
    }
    __syncthreads();
  };

  const size_t plane = (size_t)d.B * d.Hq * d.Nq;
  if (d.tok) {
    const size_t lrow = (size_t)bh * d.Nq + row;
    const int* mine = idx + lrow * d.budget;
    const int nm = min(max(cnt[lrow], 0), d.budget);
    auto has = [&](int kb) {
      bool f = false;
      for (int i = 0; i < nm; ++i) f |= mine[i] == kb;
      return f;
    };
    for (int kb = 0; kb <= diag; ++kb) {   // sparse stream
      const bool sel = has(kb);
      if (__builtin_amdgcn_ballot_w64(sel) == 0ull) continue;
      process(kb, true, sel);
    }
    if (active) {
      float* hp = Hs + ((size_t)bh * d.Nq + row) * D;
      const float inv = 1.f / l_sel;
      for (int i = 0; i < D; ++i) hp[i] = acc[i] * inv;
      if (lse != nullptr) lse[plane + (size_t)bh * d.Nq + row] = (m_run + log2f(l_sel)) * kLn2;
    }
    if (Hf == nullptr) return;
    m_run = -INFINITY;
    l_sel = l_drop = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = 0.f;
    for (int kb = 0; kb <= diag; ++kb) process(kb, has(kb), true);   // full stream
    if (active) {
      const float lt = l_sel + l_drop;
      float* hp = Hf + ((size_t)bh * d.Nq + row) * D;
      const float inv = 1.f / lt;
      for (int i = 0; i < D; ++i) hp[i] = acc[i] * inv;
      if (delta != nullptr) delta[(size_t)bh * d.Nq + row] = l_drop / lt;
      if (lse != nullptr) lse[(size_t)bh * d.Nq + row] = (m_run + log2f(lt)) * kLn2;
    }
    return;
  }
  const int* my_idx = idx + ((size_t)bh * d.nQB + qb) * d.budget;
  const int n_sel = min(max(cnt[(size_t)bh * d.nQB + qb], 0), d.budget);
  for (int it = 0; it < n_sel; ++it) {
    const int kb = my_idx[it];
    if (kb >= 0 && kb <= diag) process(kb, true, true);
  }
  if (active) {
    float* hp = Hs + ((size_t)bh * d.Nq + row) * D;
    const float inv = 1.f / l_sel;
    for (int i = 0; i < D; ++i) hp[i] = acc[i] * inv;
    if (lse != nullptr) lse[plane + (size_t)bh * d.Nq + row] = (m_run + log2f(l_sel)) * kLn2;
  }
  if (Hf == nullptr) return;
  int j = 0;
  for (int kb = 0; kb <= diag; ++kb) {
    while (j < n_sel && my_idx[j] < kb) ++j;
    if (j < n_sel && my_idx[j] == kb) continue;
    process(kb, false, true);
  }
  if (active) {
    const float lt = l_sel + l_drop;
    float* hp = Hf + ((size_t)bh * d.Nq + row) * D;
    const float inv = 1.f / lt;
    for (int i = 0; i < D; ++i) hp[i] = acc[i] * inv;
    if (delta != nullptr) delta[(size_t)bh * d.Nq + row] = l_drop / lt;
    if (lse != nullptr) lse[(size_t)bh * d.Nq + row] = (m_run + log2f(lt)) * kLn2;
  }
}

hipError_t launch_attn_rows_f32(const float* q, const float* k, const float* v, const int* idx,
                                const int* cnt, float* hf, float* hs, float* delta, float* lse,
                                const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const dim3 grid(d.nQB, d.Hq, d.B);
  if (d.D == 128)
    hipLaunchKernelGGL(attn_rows_f32_kernel<128>, grid, dim3(64), 0, stream, q, k, v, idx, cnt,
                       hf, hs, delta, lse, d, hm);
  else
    hipLaunchKernelGGL(attn_rows_f32_kernel<64>, grid, dim3(64), 0, stream, q, k, v, idx, cnt,
                       hf, hs, delta, lse, d, hm);
  return hipGetLastError();
}

}  // namespace ssa

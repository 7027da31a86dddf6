// Fused dual-stream causal attention forward (prefill), bf16 on MFMA, and a
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
#include "ssa_kernels.h"

namespace ssa {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 (round to nearest even) in one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t r = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// LDS tiles are stored without padding; 16-byte chunks are XOR-swizzled per
// row so that the ds_read_b128 of 16 lanes (16 different rows, same logical
// chunk) hit 16 distinct 16-byte bank groups. V^T rows are 128 bytes (two
// rows per 256-byte bank sweep) and the 16 rows of one read are consecutive:
// chunk ^ ((row >> 1) & 7) separates them.
__device__ __forceinline__ int vswz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [base, base + bytes): loads past the end read 0. The
// base is made wave-uniform explicitly so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* u = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// K-tile swizzles under that permutation: the 16 rows one ds_read_b128 phase
// touches land on 16 distinct 16-byte bank groups. 256-byte rows (D = 128,
// 16 chunks) use chunk ^ f(row) with f taking row bits 0,1,3,4; 128-byte rows
// (D = 64, 8 chunks, two rows per 256 bytes) use row bits 1,3,4.
template <int SPR>
__device__ __forceinline__ int kswz(int row, int chunk) {
  if constexpr (SPR == 16) return chunk ^ ((row & 3) | ((row >> 1) & 12));
  else return chunk ^ (((row >> 1) & 1) | ((row >> 2) & 6));
}

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

// One workgroup = one (b, q head, 64-row query block); four waves of 16
// query rows each. MFMA 16x16x32 bf16 computes S^T = K Q^T (keys x queries:
// a lane owns one query column, so row statistics stay in-lane up to a
// reduction over the four lanes of that column) and O^T = V^T P^T, with P
// handed from the S^T output registers to the PV B operand directly thanks
// to the K row permutation kperm16. The small per-wave state (about 110
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

  const int* my_idx = idx + ((size_t)bh * d.nQB + qb) * d.budget;
  const int n_sel =
      __builtin_amdgcn_readfirstlane(min(max(cnt[(size_t)bh * d.nQB + qb], 0), d.budget));
  const int nwords = (diag >> 5) + 1;
  for (int w = tid; w < nwords; w += 256) sel_mask[w] = 0u;
  __syncthreads();
  for (int e = tid; e < n_sel; e += 256) {
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

  // Q^T operand: lane holds Q[qrow][32ks + 8g4 .. +7].
  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 32 * ks);
  }
  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_sel = 0.f, l_drop = 0.f;

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

  auto body = [&](int kb, bool selected, int kb_next) {
    f32x4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int row = kperm16(kt, n);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(Ks + (row * KSPR + kchunk(row, 4 * ks + g4)) * 8);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], s[kt], 0, 0, 0);
      }
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
      l_sel *= alpha;
      l_drop *= alpha;
    }
    float ls = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float p0 = fast_exp2(fmaf(s[kt][0], sl2, -m_ref));
      const float p1 = fast_exp2(fmaf(s[kt][1], sl2, -m_ref));
      const float p2 = fast_exp2(fmaf(s[kt][2], sl2, -m_ref));
      const float p3 = fast_exp2(fmaf(s[kt][3], sl2, -m_ref));
      ls += (p0 + p1) + (p2 + p3);
      pw[2 * kt] = pack_bf16x2(p0, p1);
      pw[2 * kt + 1] = pack_bf16x2(p2, p3);
    }
    if (selected) l_sel += ls; else l_drop += ls;

    wait_vm();
    __syncthreads();
    if (kb_next >= 0) load_k(kb_next);

    // O^T += V^T P^T; k-step j (32 keys) takes tiles 2j, 2j+1.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 w = make_uint4(pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int r = 16 * dt + n;
        const bf16x8_t a = *(const bf16x8_t*)(Vs + (r * VSPR + vswz(r, 4 * j + g4)) * 8);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
      }
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
    body(kb, true, kb_next);
    kb = kb_next;
    sel_cur = sel_next;
  }
  {
    const float lt = quad_sum(l_sel);
    store(Hs, 1.f / lt);
    if (lse != nullptr && g4 == 0)
      lse[plane + (size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
  if (sparse_only) return;
  while (kb >= 0) {
    bool sel_next = false;
    const int kb_next = next_block(sel_next);
    body(kb, false, kb_next);
    kb = kb_next;
  }
  const float ls_t = quad_sum(l_sel);
  const float ld_t = quad_sum(l_drop);
  const float lt = ls_t + ld_t;
  store(Hf, 1.f / lt);
  if (g4 == 0) {
    if (delta != nullptr) delta[(size_t)bh * d.Nq + qrow] = ld_t / lt;
    if (lse != nullptr) lse[(size_t)bh * d.Nq + qrow] = (m_ref + __log2f(lt)) * kLn2;
  }
}

hipError_t launch_attn_prefill_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                                    const int* idx, const int* cnt, uint16_t* hf, uint16_t* hs,
                                    float* delta, float* lse, const Dims& d, const HeadMap& hm,
                                    hipStream_t stream) {
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
// selected blocks, snapshot, remaining causal blocks.
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

  auto process = [&](int kb, bool selected) {
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
        if (kb * kBlock + j0 + j > pos) a = -INFINITY;
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

  const int* my_idx = idx + ((size_t)bh * d.nQB + qb) * d.budget;
  const int n_sel = min(max(cnt[(size_t)bh * d.nQB + qb], 0), d.budget);
  for (int it = 0; it < n_sel; ++it) {
    const int kb = my_idx[it];
    if (kb >= 0 && kb <= diag) process(kb, true);
  }
  const size_t plane = (size_t)d.B * d.Hq * d.Nq;
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
    process(kb, false);
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

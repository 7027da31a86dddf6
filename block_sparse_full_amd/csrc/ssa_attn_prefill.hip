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

// Row of the K tile that MFMA row c reads. With this permutation the S^T
// output register v of lane group gl holds key 16*(v/8) + 8*gl + (v%8) of its
// 32-key tile, which is exactly the 8 consecutive keys the PV MFMA needs in
// its B operand, so P never leaves registers.
__device__ __forceinline__ int kperm(int c) {
  const int i = c >> 3, gp = (c >> 2) & 1, j = c & 3;
  return 16 * (i >> 1) + 8 * gp + 4 * (i & 1) + j;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One workgroup = one (b, q head, 64-row query block); two waves of 32 query
// rows each. MFMA 32x32x16 bf16 computes S^T = K Q^T (keys x queries, so a
// lane owns one query column and row statistics stay in-lane up to one
// exchange with lane ^ 32) and O^T = V^T P^T. K and V^T tiles are staged in
// padded LDS (conflict-free ds_read_b128).
template <int D>
__global__ __launch_bounds__(128) void attn_prefill_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vt, const int* __restrict__ idx, const int* __restrict__ cnt,
    uint16_t* __restrict__ Hf, uint16_t* __restrict__ Hs, float* __restrict__ delta,
    float* __restrict__ lse, Dims d, HeadMap hm) {
  constexpr int KSTR = D + 8;       // K tile row stride (elements)
  constexpr int VSTR = kBlock + 8;  // V^T tile row stride (elements)
  constexpr int NKS = D / 16;       // k-steps of QK^T
  constexpr int NDT = D / 32;       // d tiles of O^T
  constexpr int KCH = kBlock * D / 8 / 128;  // 16-byte chunks per thread, K tile
  constexpr int VCH = D * kBlock / 8 / 128;  // same, V^T tile
  __shared__ __align__(16) uint16_t Ks[kBlock * KSTR];
  __shared__ __align__(16) uint16_t Vs[D * VSTR];

  const int total = d.B * d.Hq * d.nQB;
  const int lin = xcd_remap(blockIdx.x, total);
  // Logical order: (b, kv head) groups, then query blocks longest first,
  // then the group's q heads.
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
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, gl = lane >> 5;
  const int qq = wave * 32 + c;                 // query row within the block
  const int qrow = qb * kBlock + qq;            // query row (== key position)
  const int diag = qb;
  const float sl2 = d.scale_log2;

  // Q^T operand of QK^T: lane holds Q[qrow][16ks + 8gl .. +7].
  bf16x8_t qf[NKS];
  {
    const uint16_t* qp = Q + ((size_t)bh * d.Nq + qrow) * D + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 16 * ks);
  }

  f32x16_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float m_run = -INFINITY, l_sel = 0.f, l_drop = 0.f;

  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = Vt + ((size_t)(b * d.Hkv + g) * D) * d.Nk;
  const int pr = kperm(c);

  auto process = [&](int kb, bool selected) {
    // ---- stage K and V^T tiles
    {
      const uint16_t* kg = kbase + (size_t)kb * kBlock * D;
      const uint16_t* vg = vbase + (size_t)kb * kBlock;
      uint4 kr[KCH], vr[VCH];
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int ch = tid + 128 * i;
        const int r = ch / (D / 8), cc = (ch % (D / 8)) * 8;
        kr[i] = *(const uint4*)(kg + r * D + cc);
      }
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int ch = tid + 128 * i;
        const int r = ch >> 3, cc = (ch & 7) * 8;
        vr[i] = *(const uint4*)(vg + (size_t)r * d.Nk + cc);
      }
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int ch = tid + 128 * i;
        const int r = ch / (D / 8), cc = (ch % (D / 8)) * 8;
        *(uint4*)(Ks + r * KSTR + cc) = kr[i];
      }
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int ch = tid + 128 * i;
        const int r = ch >> 3, cc = (ch & 7) * 8;
        *(uint4*)(Vs + r * VSTR + cc) = vr[i];
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for 64 keys x 32 queries
    f32x16_t s0, s1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8_t a0 = *(const bf16x8_t*)(Ks + pr * KSTR + 16 * ks + 8 * gl);
      const bf16x8_t a1 = *(const bf16x8_t*)(Ks + (32 + pr) * KSTR + 16 * ks + 8 * gl);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
    }

    // ---- online softmax (log2 domain), causal mask on the diagonal block
    const bool on_diag = (kb == diag);
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x0 = s0[v] * sl2, x1 = s1[v] * sl2;
      if (on_diag) {
        const int key0 = 16 * (v >> 3) + 8 * gl + (v & 7);
        if (key0 > qq) x0 = -INFINITY;
        if (key0 + 32 > qq) x1 = -INFINITY;
      }
      s0[v] = x0;
      s1[v] = x1;
      mx = fmaxf(mx, fmaxf(x0, x1));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p0 = fast_exp2(s0[v] - m_new);
      const float p1 = fast_exp2(s1[v] - m_new);
      ls += p0 + p1;
      pb[v >> 3][v & 7] = static_cast<__bf16>(p0);
      pb[2 + (v >> 3)][v & 7] = static_cast<__bf16>(p1);
    }
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    l_sel *= alpha;
    l_drop *= alpha;
    if (selected) l_sel += ls; else l_drop += ls;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t a = *(const bf16x8_t*)(Vs + (32 * dt + c) * VSTR + 16 * s + 8 * gl);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  };

  auto store = [&](uint16_t* H, float inv) {
    uint16_t* hp = H + ((size_t)bh * d.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * gl;
        const uint32_t lo = (uint32_t)f32_to_bf16(o[dt][4 * i] * inv) |
                            ((uint32_t)f32_to_bf16(o[dt][4 * i + 1] * inv) << 16);
        const uint32_t hi2 = (uint32_t)f32_to_bf16(o[dt][4 * i + 2] * inv) |
                             ((uint32_t)f32_to_bf16(o[dt][4 * i + 3] * inv) << 16);
        *(uint2*)(hp + d0) = make_uint2(lo, hi2);
      }
    }
  };

  const int* my_idx = idx + ((size_t)bh * d.nQB + qb) * d.budget;
  const int n_sel = min(max(cnt[(size_t)bh * d.nQB + qb], 0), d.budget);
  for (int it = 0; it < n_sel; ++it) {
    const int kb = my_idx[it];
    if (kb >= 0 && kb <= diag) process(kb, true);
  }
  const size_t plane = (size_t)d.B * d.Hq * d.Nq;
  {
    const float lt = l_sel + __shfl_xor(l_sel, 32);
    store(Hs, 1.f / lt);
    if (lse != nullptr && gl == 0)
      lse[plane + (size_t)bh * d.Nq + qrow] = (m_run + __log2f(lt)) * kLn2;
  }
  if (Hf == nullptr) return;  // sparse-only mode
  {
    int j = 0;
    for (int kb = 0; kb <= diag; ++kb) {
      while (j < n_sel && my_idx[j] < kb) ++j;
      if (j < n_sel && my_idx[j] == kb) continue;
      process(kb, false);
    }
  }
  const float ls_t = l_sel + __shfl_xor(l_sel, 32);
  const float ld_t = l_drop + __shfl_xor(l_drop, 32);
  const float lt = ls_t + ld_t;
  store(Hf, 1.f / lt);
  if (gl == 0) {
    if (delta != nullptr) delta[(size_t)bh * d.Nq + qrow] = ld_t / lt;
    if (lse != nullptr) lse[(size_t)bh * d.Nq + qrow] = (m_run + __log2f(lt)) * kLn2;
  }
}

hipError_t launch_attn_prefill_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                                    const int* idx, const int* cnt, uint16_t* hf, uint16_t* hs,
                                    float* delta, float* lse, const Dims& d, const HeadMap& hm,
                                    hipStream_t stream) {
  const int total = d.B * d.Hq * d.nQB;
  if (d.D == 128)
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<128>, dim3(total), dim3(128), 0, stream, q, k,
                       vt, idx, cnt, hf, hs, delta, lse, d, hm);
  else
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<64>, dim3(total), dim3(128), 0, stream, q, k,
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

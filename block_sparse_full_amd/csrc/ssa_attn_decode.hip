// Single-query (decode) dual-stream attention, bf16, split over the KV
// length, and the merge of the partial results.
//
// Method: the same two streams and dropped mass as the prefill kernel
// ("SSA: Achieving Sparser Attention by Aligning Full and Sparse Attention
// Outputs in Feature Space", sections "SSA's Dual-Stream Training Mechanism"
// and "Practical Implementation of SSA"; "Technische Samenvatting: SSA",
// "2. Methodologie") for one query per (sequence, q head) at the last
// position, as in generation with either inference mode ("SSA: Sparse Sparse
// Attention", "Inference with Sparse or Full Mode").
//
// Decode reads each K/V byte once, so it is bound by HBM bandwidth. A
// workgroup owns one (b, kv head) and a range of key blocks; the q heads of
// that kv head (the GQA group) all use every K/V load. Per head it keeps the
// running max m, l_sel / l_drop and two accumulators: acc_full over every key
// and acc_sel over the head's selected blocks only (a key's PV goes into
// acc_sel in addition only when that head selected its block, so the extra
// work is proportional to the budget). Work is cut into 64-key tiles; with
// 16-token selection blocks each 16-key quarter of a tile follows its own
// block. Dual mode walks every tile; sparse-only mode walks only the tiles
// holding a block selected by some head of the group and skips acc_full.
#include "ssa_common.h"
#include "ssa_kernels.h"

namespace ssa {

__device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Bit kb of head n in the selection bitmap.
__device__ __forceinline__ bool sel_bit(const unsigned* bits, int words, int n, int kb) {
  return (bits[n * words + (kb >> 5)] >> (kb & 31)) & 1u;
}
// Selected 16-key quarters of 64-key tile t for head n, as 4 bits: with
// 64-token selection blocks all four follow block t, with 16-token blocks
// quarter j is block 4t + j.
__device__ __forceinline__ unsigned tile_quarters(const unsigned* bits, int words, int n, int t,
                                                  int bs) {
  if (bs == kBlock) return sel_bit(bits, words, n, t) ? 0xFu : 0u;
  return (bits[n * words + ((4 * t) >> 5)] >> ((4 * t) & 31)) & 0xFu;
}

template <int D, int GP>
struct DecLayout {
  static constexpr int LPR = D / 8;        // lanes per K/V row in the PV layout
  static constexpr int RPI = 64 / LPR;     // rows per load instruction
  static constexpr int KPL = kBlock / RPI; // keys per lane per block
  static constexpr int NKS = D / 32;       // k-steps of the 16x16x32 MFMA
};

// partial layout per (b, q head, split): m (log2 units), l_sel, l_drop, 0,
// acc_full[D], acc_sel[D].
template <int D, int GP>
__global__ __launch_bounds__(256) void attn_decode_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int* __restrict__ idx, const int* __restrict__ cnt,
    float* __restrict__ partials, Dims d, HeadMap hm, int sparse_only, int nsplit, int nsub) {
  using L = DecLayout<D, GP>;
  constexpr int PF = 2 * D + 4;
  extern __shared__ __align__(16) unsigned char smem[];
  const int words = (d.nKB + 31) >> 5;
  unsigned* bits = (unsigned*)smem;                          // [GP][words] selection bitmaps
  int* ulist = (int*)(bits + GP * words);                    // [nT] union tile list (sparse-only)
  float* ps = (float*)(ulist + d.nT);                        // [kDecWaves][kBlock][GP]
  float* als = ps + kDecWaves * kBlock * GP;                 // [kDecWaves][GP]
  float* red = als + kDecWaves * GP;                         // [kDecWaves][GP][PF]
  __shared__ int s_nunion;

  // a group of more than GP q heads is split over nsub workgroups of GP
  const int split = blockIdx.x, b = blockIdx.z;
  const int g = blockIdx.y / nsub, hoff = (blockIdx.y % nsub) * GP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = min(GP, d.G - hoff);                         // heads of this workgroup
  const uint8_t* qmap = hm.q_of_kv + g * d.G + hoff;         // their q head indices
  const float sl2 = d.scale_log2;

  // ---- selection bitmaps of the group's heads
  for (int i = tid; i < GP * words; i += 256) bits[i] = 0u;
  __syncthreads();
  // ---- query fragments, in flight together with the idx/cnt loads below
  // QK^T layout (16x16x32): lane column n = lane & 15 is head n; rows
  // 4*(lane>>4) + r of key tile kt are its keys.
  const int n_col = lane & 15;
  const int kgrp = lane >> 4;
  bf16x8_t qf[L::NKS];
  {
    const bool valid = n_col < G;
    const int h = valid ? qmap[n_col] : 0;
    const uint16_t* qp = Q + (size_t)(b * d.Hq + h) * D + 8 * kgrp;
#pragma unroll
    for (int ks = 0; ks < L::NKS; ++ks) {
      bf16x8_t v = *(const bf16x8_t*)(qp + 32 * ks);
      if (!valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(0.f);
      }
      qf[ks] = v;
    }
  }
  for (int i = tid; i < G * d.budget; i += 256) {
    const int n = i / d.budget, e = i - n * d.budget;
    const int h = qmap[n];
    const int c = cnt[b * d.Hq + h];
    const int kb = idx[(size_t)(b * d.Hq + h) * d.budget + e];
    if (e < c && kb >= 0 && kb < d.nKB) atomicOr(&bits[n * words + (kb >> 5)], 1u << (kb & 31));
  }
  __syncthreads();

  // ---- the 64-key tiles this workgroup walks
  int blk_begin, blk_count, blk_stride;
  if (sparse_only) {
    // the union's tiles in ascending order, by wave 0: lane w takes tile
    // word w (bit j: tile 32w + j selected by some head of the group), a
    // wave prefix sum of the words' popcounts places each lane's tiles
    if (wave == 0) {
      const int twords = (d.nT + 31) >> 5;
      int base = 0;
      for (int w0 = 0; w0 < twords; w0 += 64) {
        const int w = w0 + lane;
        unsigned u = 0u;
        if (w < twords) {
          if (d.bs == kBlock) {
            for (int n = 0; n < G; ++n) u |= bits[n * words + w];
          } else {   // 16-token blocks: tile t is blocks 4t .. 4t+3
            for (int i = 0; i < 4; ++i) {
              const int bw = 4 * w + i;
              if (bw >= words) break;
              unsigned x = 0u;
              for (int n = 0; n < G; ++n) x |= bits[n * words + bw];
              x |= (x >> 1) | (x >> 2) | (x >> 3);   // bit 4j: block nibble j not empty
              unsigned r = 0u;
#pragma unroll
              for (int j = 0; j < 8; ++j) r |= ((x >> (4 * j)) & 1u) << j;
              u |= r << (8 * i);
            }
          }
        }
        const int c = __popc(u);
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(incl, off, 64);
          if (lane >= off) incl += o;
        }
        int pos = base + incl - c;
        while (u) {
          ulist[pos++] = w * 32 + __ffs(u) - 1;
          u &= u - 1u;
        }
        base += __shfl(incl, 63, 64);
      }
      if (lane == 0) s_nunion = base;
    }
    __syncthreads();
    const int nu = s_nunion;
    const int per = (nu + nsplit - 1) / nsplit;
    blk_begin = split * per;
    blk_count = max(0, min(per, nu - blk_begin));
    blk_stride = kDecWaves;  // wave w takes entries w, w+4, ...
  } else {
    blk_begin = split * kDecWaves * kDecWaveBlocks;
    blk_count = max(0, min(kDecWaves * kDecWaveBlocks, d.nT - blk_begin));
    blk_stride = kDecWaves;
  }

  float m_run = -INFINITY, l_sel = 0.f, l_drop = 0.f;  // of head n_col (lane partials)
  // PV layout: lane owns d = 8*(lane % LPR) .. +7 and keys RPI*i + lane / LPR.
  const int pv_d0 = 8 * (lane % L::LPR);
  const int pv_k0 = lane / L::LPR;
  float acc_full[GP][8], acc_sel[GP][8];
#pragma unroll
  for (int n = 0; n < GP; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) { acc_full[n][e] = 0.f; acc_sel[n][e] = 0.f; }

  float* wps = ps + wave * kBlock * GP;
  float* wal = als + wave * GP;
  const uint16_t* kbase = K + ((size_t)(b * d.Hkv + g) * d.Nk) * D;
  const uint16_t* vbase = V + ((size_t)(b * d.Hkv + g) * d.Nk) * D;

  for (int it = wave; it < blk_count; it += blk_stride) {
    const int kb = sparse_only ? ulist[blk_begin + it] : blk_begin + it;
    const uint16_t* kg = kbase + (size_t)kb * kBlock * D;
    const uint16_t* vg = vbase + (size_t)kb * kBlock * D;
    // V rows for the PV step (independent of QK^T: issued first).
    uint4 vr[L::KPL];
#pragma unroll
    for (int i = 0; i < L::KPL; ++i)
      vr[i] = *(const uint4*)(vg + (size_t)(L::RPI * i + pv_k0) * D + pv_d0);
    // S^T = K q^T: 4 key tiles of 16.
    f32x4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < L::NKS; ++ks) {
        const bf16x8_t a =
            *(const bf16x8_t*)(kg + (size_t)(16 * kt + n_col) * D + 32 * ks + 8 * kgrp);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], s[kt], 0, 0, 0);
      }
    }
    // Softmax statistics of head n_col over this tile; key tile kt (16
    // keys) is selection quarter kt.
    const unsigned mine = n_col < G ? tile_quarters(bits, words, n_col, kb, d.bs) : 0u;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const bool active = !sparse_only || ((mine >> kt) & 1u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = active ? s[kt][r] * sl2 : -INFINITY;
        s[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? dexp2(m_run - m_new) : 1.f;
    m_run = m_new;
    float lsum_sel = 0.f, lsum_drop = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = live ? dexp2(s[kt][r] - m_new) : 0.f;
        lsum += p;
        if (n_col < GP) wps[(16 * kt + 4 * kgrp + r) * GP + n_col] = p;
      }
      if ((mine >> kt) & 1u) lsum_sel += lsum; else lsum_drop += lsum;
    }
    l_sel = l_sel * alpha + lsum_sel;
    l_drop = l_drop * alpha + lsum_drop;
    if (lane < GP) wal[lane] = alpha;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // PV on the VALU: rescale, then accumulate this lane's keys.
    float al[GP];
#pragma unroll
    for (int n = 0; n < GP; ++n) al[n] = wal[n];
#pragma unroll
    for (int n = 0; n < GP; ++n)
#pragma unroll
      for (int e = 0; e < 8; ++e) { acc_full[n][e] *= al[n]; acc_sel[n][e] *= al[n]; }
    unsigned hsel[GP];
#pragma unroll
    for (int n = 0; n < GP; ++n) hsel[n] = n < G ? tile_quarters(bits, words, n, kb, d.bs) : 0u;
#pragma unroll
    for (int i = 0; i < L::KPL; ++i) {
      const int key = L::RPI * i + pv_k0;
      const unsigned w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = __uint_as_float(w[e] << 16);
        vv[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
      float p[GP];
#pragma unroll
      for (int n = 0; n < GP; ++n) p[n] = wps[key * GP + n];
      if (!sparse_only) {
#pragma unroll
        for (int n = 0; n < GP; ++n)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc_full[n][e] = fmaf(p[n], vv[e], acc_full[n][e]);
      }
#pragma unroll
      for (int n = 0; n < GP; ++n) {
        if ((hsel[n] >> (key >> 4)) & 1u) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc_sel[n][e] = fmaf(p[n], vv[e], acc_sel[n][e]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }

  // ---- reduce lane partials inside the wave
  l_sel += __shfl_xor(l_sel, 16);
  l_sel += __shfl_xor(l_sel, 32);
  l_drop += __shfl_xor(l_drop, 16);
  l_drop += __shfl_xor(l_drop, 32);
#pragma unroll
  for (int n = 0; n < GP; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = acc_full[n][e], c = acc_sel[n][e];
#pragma unroll
      for (int off = L::LPR; off < 64; off <<= 1) {
        a += __shfl_xor(a, off);
        c += __shfl_xor(c, off);
      }
      acc_full[n][e] = a;
      acc_sel[n][e] = c;
    }
  float* wred = red + wave * GP * PF;
  if (lane < GP) {
    wred[lane * PF + 0] = m_run;
    wred[lane * PF + 1] = l_sel;
    wred[lane * PF + 2] = l_drop;
  }
  if (lane < L::LPR) {
#pragma unroll
    for (int n = 0; n < GP; ++n)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wred[n * PF + 4 + pv_d0 + e] = acc_full[n][e];
        wred[n * PF + 4 + D + pv_d0 + e] = acc_sel[n][e];
      }
  }
  __syncthreads();

  // ---- merge the waves, write this split's partial for every head
  for (int i = tid; i < G * (D + 1); i += 256) {
    const int n = i / (D + 1), j = i - n * (D + 1);
    float M = -INFINITY;
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red[(w * GP + n) * PF]);
    const int h = qmap[n];
    float* out = partials + ((size_t)(b * d.Hq + h) * nsplit + split) * PF;
    if (j == D) {
      float ls = 0.f, ld = 0.f;
      if (M != -INFINITY)
        for (int w = 0; w < kDecWaves; ++w) {
          const float* r = red + (w * GP + n) * PF;
          const float f = dexp2(r[0] - M);
          ls += f * r[1];
          ld += f * r[2];
        }
      out[0] = M;
      out[1] = ls;
      out[2] = ld;
      out[3] = 0.f;
    } else {
      float af = 0.f, as = 0.f;
      if (M != -INFINITY)
        for (int w = 0; w < kDecWaves; ++w) {
          const float* r = red + (w * GP + n) * PF;
          const float f = dexp2(r[0] - M);
          af += f * r[4 + j];
          as += f * r[4 + D + j];
        }
      out[4 + j] = af;
      out[4 + D + j] = as;
    }
  }
}

// One workgroup of D threads per (b, q head): combine the splits.
__global__ __launch_bounds__(128) void decode_merge_kernel(
    const float* __restrict__ partials, uint16_t* __restrict__ Hf, uint16_t* __restrict__ Hs,
    float* __restrict__ delta, float* __restrict__ lse, int D, int nsplit, int sparse_only,
    size_t plane) {
  const int bh = blockIdx.x;
  const int j = threadIdx.x;
  const int PF = 2 * D + 4;
  const float* pp = partials + (size_t)bh * nsplit * PF;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pp[s * PF]);
  float ls = 0.f, ld = 0.f, af = 0.f, as = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* r = pp + s * PF;
    if (r[0] == -INFINITY) continue;
    const float f = dexp2(r[0] - M);
    ls += f * r[1];
    ld += f * r[2];
    if (j < D) {
      af += f * r[4 + j];
      as += f * r[4 + D + j];
    }
  }
  if (j < D) {
    Hs[(size_t)bh * D + j] = f32_to_bf16(as / ls);
    if (!sparse_only) Hf[(size_t)bh * D + j] = f32_to_bf16(af / (ls + ld));
  }
  if (j == 0) {
    if (!sparse_only && delta != nullptr) delta[bh] = ld / (ls + ld);
    if (lse != nullptr) {
      lse[plane + bh] = (M + __log2f(ls)) * kLn2;
      if (!sparse_only) lse[bh] = (M + __log2f(ls + ld)) * kLn2;
    }
  }
}

template <int D, int GP>
static hipError_t launch_dec(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int* idx, const int* cnt, float* partials, const Dims& d,
                             const HeadMap& hm, int sparse_only, int nsplit, hipStream_t stream) {
  const int words = (d.nKB + 31) >> 5;
  const size_t smem = (size_t)GP * words * 4 + (size_t)d.nT * 4 +
                      (size_t)kDecWaves * kBlock * GP * 4 + (size_t)kDecWaves * GP * 4 +
                      (size_t)kDecWaves * GP * (2 * D + 4) * 4;
  const int nsub = (d.G + GP - 1) / GP;
  hipLaunchKernelGGL((attn_decode_bf16_kernel<D, GP>), dim3(nsplit, d.Hkv * nsub, d.B), dim3(256),
                     smem, stream, q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, nsub);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dec_g(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int* idx, const int* cnt, float* partials, const Dims& d,
                               const HeadMap& hm, int sparse_only, int nsplit,
                               hipStream_t stream) {
  if (d.G <= 1) return launch_dec<D, 1>(q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, stream);
  if (d.G <= 2) return launch_dec<D, 2>(q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, stream);
  if (d.G <= 4) return launch_dec<D, 4>(q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, stream);
  return launch_dec<D, 8>(q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, stream);
}

hipError_t launch_attn_decode_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int* idx, const int* cnt, uint16_t* hf, uint16_t* hs,
                                   float* delta, float* lse, float* partials, const Dims& d,
                                   const HeadMap& hm, hipStream_t stream) {
  const int sparse_only = hf == nullptr ? 1 : 0;
  const int nsplit = sparse_only ? kDecSparseParts : decode_splits(d.nT);
  hipError_t e = d.D == 128
                     ? launch_dec_g<128>(q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, stream)
                     : launch_dec_g<64>(q, k, v, idx, cnt, partials, d, hm, sparse_only, nsplit, stream);
  if (e != hipSuccess) return e;
  const size_t plane = (size_t)d.B * d.Hq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(d.B * d.Hq), dim3(d.D), 0, stream, partials, hf,
                     hs, delta, lse, d.D, nsplit, sparse_only, plane);
  return hipGetLastError();
}

}  // namespace ssa

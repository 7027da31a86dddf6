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
// One workgroup per (b, kv head, query row block). It scores the causal
// candidate blocks of up to `hc` q heads of the group at once (each pooled
// key row is read once for all of them), then runs an exact radix select per
// head: the free-th largest 64-bit orderable key is found 8 bits at a time
// from the most significant byte; keys above it are taken, and among keys
// equal to it the lowest block indices fill the remaining slots.
constexpr int kSelThreads = 256;
constexpr int kSelMaxWords = kMaxKeyBlocks / 32;

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

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar,
    int* __restrict__ idx, int* __restrict__ cnt, Dims d, HeadMap hm, int hc) {
  extern __shared__ __align__(16) unsigned char smem[];
  // layout: keys[hc][nKB] u64 | qv[hc][D] f32
  uint64_t* keys = (uint64_t*)smem;
  float* qv = (float*)(smem + (size_t)hc * d.nKB * sizeof(uint64_t));
  __shared__ unsigned hist[256];
  __shared__ unsigned sel_bits[kSelMaxWords];
  __shared__ unsigned eq_bits[kSelMaxWords];
  __shared__ int word_prefix[kSelMaxWords];
  __shared__ unsigned long long s_prefix, s_mask;
  __shared__ int s_k;

  const int tid = threadIdx.x;
  const int qb = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int diag = row_block_diag(d, qb);
  const int ncausal = diag + 1;
  const int nwords = (ncausal + 31) >> 5;
  const float* krow0 = kbar + ((size_t)(b * d.Hkv + g) * d.nKB) * d.D;

  // Forced set and slot count (identical for every head of the group).
  const int a_end = min(d.n_sink, ncausal);
  const int l_begin = max(0, ncausal - d.n_local);
  const int n_forced = a_end + (ncausal - l_begin) - max(0, a_end - l_begin);
  const int n_cand = ncausal - n_forced;
  const int free_slots = d.budget - n_forced;

  for (int h0 = 0; h0 < d.G; h0 += hc) {
    const int nh = min(hc, d.G - h0);
    __syncthreads();
    for (int i = tid; i < nh * d.D; i += kSelThreads) {
      const int hh = i / d.D, dd = i % d.D;
      const int h = hm.q_of_kv[g * d.G + h0 + hh];
      qv[i] = qbar[((size_t)(b * d.Hq + h) * d.nQB + qb) * d.D + dd];
    }
    __syncthreads();
    const bool take_all = n_cand <= free_slots;
    const bool forced_only = !take_all && free_slots <= 0;
    if (!take_all && !forced_only) {
      // Scores of every candidate for the nh heads.
      for (int kb = tid; kb < ncausal; kb += kSelThreads) {
        if (is_forced(kb, diag, d.n_sink, d.n_local)) continue;
        const float* kr = krow0 + (size_t)kb * d.D;
        for (int hb = 0; hb < nh; hb += 4) {
          double s[4] = {0.0, 0.0, 0.0, 0.0};
          for (int dd = 0; dd < d.D; dd += 4) {
            const float4 k4 = *(const float4*)(kr + dd);
            const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const double kv = (double)kk[e];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (hb + j < nh) s[j] = __fma_rn((double)qv[(hb + j) * d.D + dd + e], kv, s[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (hb + j < nh) keys[(size_t)(hb + j) * d.nKB + kb] = orderable_key(s[j]);
        }
      }
    }
    __syncthreads();

    for (int hh = 0; hh < nh; ++hh) {
      const int h = hm.q_of_kv[g * d.G + h0 + hh];
      const uint64_t* hk = keys + (size_t)hh * d.nKB;
      for (int w = tid; w < nwords; w += kSelThreads) { sel_bits[w] = 0u; eq_bits[w] = 0u; }
      __syncthreads();
      if (take_all) {
        for (int kb = tid; kb < ncausal; kb += kSelThreads) atomicOr(&sel_bits[kb >> 5], 1u << (kb & 31));
      } else if (forced_only) {
        for (int kb = tid; kb < ncausal; kb += kSelThreads)
          if (is_forced(kb, diag, d.n_sink, d.n_local)) atomicOr(&sel_bits[kb >> 5], 1u << (kb & 31));
      } else {
        if (tid == 0) { s_prefix = 0ull; s_mask = 0ull; s_k = free_slots; }
        __syncthreads();
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
          hist[tid] = 0u;
          __syncthreads();
          const uint64_t pre = s_prefix, msk = s_mask;
          for (int kb = tid; kb < ncausal; kb += kSelThreads) {
            if (is_forced(kb, diag, d.n_sink, d.n_local)) continue;
            const uint64_t key = hk[kb];
            if ((key & msk) == pre) atomicAdd(&hist[(key >> shift) & 255u], 1u);
          }
          __syncthreads();
          if (tid < 64) {
            // lane l owns bins 255-4l .. 252-4l (descending order)
            const int top = 255 - 4 * tid;
            const unsigned c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
            const int c = (int)(c0 + c1 + c2 + c3);
            const int incl = wave_incl_scan(c);
            const int excl = incl - c;
            const int k = s_k;
            const bool mine = excl < k && k <= incl;
            if (mine) {
              int cum = excl, bin = top;
              const unsigned cs[4] = {c0, c1, c2, c3};
              for (int j = 0; j < 4; ++j) {
                if (cum + (int)cs[j] >= k) { bin = top - j; break; }
                cum += (int)cs[j];
              }
              s_k = k - cum;
              s_prefix = pre | ((uint64_t)bin << shift);
              s_mask = msk | (0xFFull << shift);
            }
          }
          __syncthreads();
        }
        const uint64_t thr = s_prefix;
        const int k_eq = s_k;
        for (int kb = tid; kb < ncausal; kb += kSelThreads) {
          if (is_forced(kb, diag, d.n_sink, d.n_local)) {
            atomicOr(&sel_bits[kb >> 5], 1u << (kb & 31));
            continue;
          }
          const uint64_t key = hk[kb];
          if (key > thr) atomicOr(&sel_bits[kb >> 5], 1u << (kb & 31));
          else if (key == thr) atomicOr(&eq_bits[kb >> 5], 1u << (kb & 31));
        }
        __syncthreads();
        // Equal keys: the k_eq lowest block indices.
        for (int kb = tid; kb < ncausal; kb += kSelThreads) {
          const unsigned bit = 1u << (kb & 31);
          if (!(eq_bits[kb >> 5] & bit)) continue;
          int rank = __popc(eq_bits[kb >> 5] & (bit - 1u));
          for (int w = 0; w < (kb >> 5); ++w) rank += __popc(eq_bits[w]);
          if (rank < k_eq) atomicOr(&sel_bits[kb >> 5], bit);
        }
      }
      __syncthreads();
      // Exclusive prefix of popcounts over the words (wave 0, 4 words/lane).
      if (tid < 64) {
        int c[4], tot = 0;
        for (int j = 0; j < 4; ++j) {
          const int w = tid * 4 + j;
          c[j] = (w < nwords) ? __popc(sel_bits[w]) : 0;
          tot += c[j];
        }
        const int incl = wave_incl_scan(tot);
        int run = incl - tot;
        for (int j = 0; j < 4; ++j) {
          const int w = tid * 4 + j;
          if (w < kSelMaxWords) word_prefix[w] = run;
          run += c[j];
        }
        if (tid == 63) s_k = incl;  // total selected
      }
      __syncthreads();
      const int total = s_k;
      const size_t row = (size_t)(b * d.Hq + h) * d.nQB + qb;
      int* out = idx + row * d.budget;
      for (int kb = tid; kb < ncausal; kb += kSelThreads) {
        const unsigned bit = 1u << (kb & 31);
        const unsigned w = sel_bits[kb >> 5];
        if (w & bit) {
          const int pos = word_prefix[kb >> 5] + __popc(w & (bit - 1u));
          if (pos < d.budget) out[pos] = kb;  // always true; bounds the write to the row
        }
      }
      for (int i = total + tid; i < d.budget; i += kSelThreads) out[i] = -1;
      if (tid == 0) cnt[row] = min(total, d.budget);
      __syncthreads();
    }
  }
}

int select_heads_per_pass(const Dims& d) {
  int hc = (int)(kSelKeyBytes / ((size_t)d.nKB * sizeof(uint64_t)));
  if (hc > d.G) hc = d.G;
  if (hc < 1) hc = 1;
  return hc;
}

size_t select_smem_bytes(const Dims& d, int hc) {
  return (size_t)hc * d.nKB * sizeof(uint64_t) + (size_t)hc * d.D * sizeof(float);
}

hipError_t launch_select(const float* qbar, const float* kbar, int* idx, int* cnt,
                         const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const int hc = select_heads_per_pass(d);
  const size_t smem = select_smem_bytes(d, hc);
  hipLaunchKernelGGL(select_kernel, dim3(d.nQB, d.Hkv, d.B), dim3(kSelThreads), smem, stream,
                     qbar, kbar, idx, cnt, d, hm, hc);
  return hipGetLastError();
}

// ---------------------------------------------------------------- V transpose
// vt[bh][d][n] = v[bh][n][d] for bf16, 64x64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ v,
                                                        uint16_t* __restrict__ vt, int N, int D) {
  __shared__ uint16_t tile[64][66];
  const int n0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const size_t bh = blockIdx.z;
  const uint16_t* src = v + bh * (size_t)N * D;
  uint16_t* dst = vt + bh * (size_t)N * D;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) tile[r][tx] = src[(size_t)(n0 + r) * D + d0 + tx];
  __syncthreads();
  for (int r = ty; r < 64; r += 4) dst[(size_t)(d0 + r) * N + n0 + tx] = tile[tx][r];
}

hipError_t launch_transpose(const uint16_t* v, uint16_t* vt, int BH, int N, int D,
                            hipStream_t stream) {
  hipLaunchKernelGGL(transpose_kernel, dim3(N / 64, D / 64, BH), dim3(256), 0, stream, v, vt,
                     N, D);
  return hipGetLastError();
}

}  // namespace ssa

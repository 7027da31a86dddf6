// Backward pass of both attention streams: bf16 MFMA kernels (a dK/dV
// kernel per key tile, a dQ kernel per query tile) and float32 VALU kernels.
//
// Method: "SSA: Achieving Sparser Attention by Aligning Full and Sparse
// Attention Outputs in Feature Space", section "Bidirectional Attention
// Alignment": the stop-gradient sends the sparsity loss's gradient to h_full
// only and the commitment loss's gradient to h_sparse only, and the primary
// stream also carries the task loss's gradient; the caller adds these up and
// hands over one upstream gradient per stream (dO_f, dO_s). Each stream is a
// softmax attention over its own key set (all causal keys; the causal keys of
// the selected blocks), so with P recomputed from the forward's log-sum-exp,
//     P  = exp(scale q.k - lse),        Dr = rowsum(dO * O)
//     dS = P * (dO V^T - Dr)            (softmax Jacobian, row form)
//     dV = sum_streams P^T dO,   dQ = scale dS K,   dK = scale dS^T Q
// where dS is the sum of both streams' dS. The top-k selection is piecewise
// constant in Q and K and passes no gradient.
//
// Walk. The dK/dV kernel owns 128 keys of one kv head (32 per wave) and
// visits the 32-row query steps of every q head of the GQA group that reach
// those keys; the sparse stream's extra products run only on (step, wave)
// pairs whose blocks are selected. The dQ kernel owns 128 query rows of one q
// head (32 per wave) and visits 32-key steps up to the diagonal. In dual mode
// both kernels walk every causal step (the full stream needs them all); in
// sparse-only mode (no full-stream gradient) only steps with a selected block.
//
// MFMA 16x16x32 bf16 throughout. The dK/dV kernel computes S = Q K^T and
// dP = dO V^T with query rows on the output's register index, so P and dS
// sit in the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS once the
// A rows of the first products are read in the kperm16 order; the dQ kernel
// does the same with keys: S^T = K Q^T, dQ^T = K^T dS^T. Contractions over
// query rows (dK/dV) and over keys (dQ) read the transposed copies Q^T, dO^T
// and K^T, which the host path makes before the kernels run.
#include "ssa_common.h"
#include "ssa_device.h"
#include "ssa_kernels.h"

namespace ssa {

namespace {

constexpr int kStep = 32;        // query rows per dK/dV step, keys per dQ step
constexpr int kKeysPerWg = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int kRowsPerWg = 128;  // query rows per dQ workgroup (32 per wave)
constexpr int kMaxSteps = 8192;  // 32-row (32-key) steps per head: N <= 262144

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// kperm16 with 32-row tiles: MFMA A row m of row block mb reads tile row
// 8*(m/4) + 4*mb + m%4, so output register i of lane group g holds tile row
// 8*g + 4*mb + i, and the eight values of one lane over (mb, i) are the eight
// consecutive rows 8*g .. 8*g+7 that a 32-deep B operand slot range needs.
__device__ __forceinline__ int rho(int mb, int m) { return 8 * (m >> 2) + 4 * mb + (m & 3); }

// Transposed tiles are D rows of 32 bf16 (64 bytes, 4 chunks); a read phase
// touches 16 consecutive rows at one logical chunk.
__device__ __forceinline__ int tswz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// One tile copy, global -> LDS, of ROWS rows x SPR 16-byte chunks shared by
// four waves. Lane i of a wave instruction fills LDS slot slot0 + i and
// fetches the global chunk the tile's swizzle maps to it.
template <int SPR, int ROWS, bool TRANSPOSED>
__device__ __forceinline__ void copy_tile(i32x4_t rsrc, uint32_t tile_off, uint32_t row_bytes,
                                          uint16_t* lds, int wave, int lane) {
  constexpr int SLOTS = ROWS * SPR;
  constexpr int PER_WAVE = SLOTS / 4;
  static_assert(PER_WAVE % 64 == 0, "tile slots per wave");
#pragma unroll
  for (int j = 0; j < PER_WAVE / 64; ++j) {
    const int slot0 = wave * PER_WAVE + j * 64;
    const int r0 = slot0 / SPR;
    const int rl = lane / SPR, sl = lane % SPR;
    const int c = TRANSPOSED ? tswz(r0 + rl, sl) : kswz<SPR>(r0 + rl, sl);
    const uint32_t voff = (uint32_t)rl * row_bytes + (uint32_t)c * 16u;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(tile_off + (uint32_t)r0 * row_bytes);
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_ptr_t)(lds + slot0 * 8));
    copy16_to_lds(rsrc, soff, voff, la);
  }
}

// 16-byte fragment of a row-major tile (SPR chunks per row, kswz layout).
template <int SPR>
__device__ __forceinline__ bf16x8_t frag_rows(const uint16_t* t, int row, int chunk) {
  return *(const bf16x8_t*)(t + row * SPR * 8 + kswz<SPR>(row, chunk) * 8);
}
// 16-byte fragment of a transposed tile (4 chunks per row, tswz layout).
__device__ __forceinline__ bf16x8_t frag_t(const uint16_t* t, int row, int chunk) {
  return *(const bf16x8_t*)(t + row * 32 + tswz(row, chunk) * 8);
}

__device__ __forceinline__ bf16x8_t pack8(const float* x) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t u{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                  pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ void store4_bf16(uint16_t* p, float a, float b, float c, float e) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  *(u32x2_t*)p = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, e)};
}

// First step s' > s of a head whose selection bits are nonzero (sparse-only
// walks), or `end`. `bits(i)` reads the bit word of step i; the 64 lanes
// test 64 candidates at a time, so every wave gets the same answer.
template <typename F>
__device__ __forceinline__ int next_selected(int s, int end, int lane, F bits) {
  for (int base = s + 1; base < end; base += 64) {
    const int c = base + lane;
    const bool a = c < end && bits(c) != 0;
    const uint64_t m = __ballot(a);
    if (m) return base + __builtin_ctzll(m);
  }
  return end;
}

}  // namespace

// ---------------------------------------------------------------- row statistics
// stats[bh][s][a][r] (32-row step s, row r): a = 0 log2-domain lse of the
// full stream, 1 rowsum(dO_f * h_full), 2 lse of the sparse stream, 3
// rowsum(dO_s * h_sparse); float32 products of the stored outputs and
// gradients, summed in float32. One workgroup per (step, b*q head); eight
// lanes per row.
template <typename T>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const T* __restrict__ hf,
                                                        const T* __restrict__ hs,
                                                        const T* __restrict__ gf,
                                                        const T* __restrict__ gs,
                                                        const float* __restrict__ lse,
                                                        float* __restrict__ stats, Dims d) {
  const int s = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int r = threadIdx.x >> 3, part = threadIdx.x & 7;
  const size_t row = bh * d.Nq + (size_t)s * kStep + r;
  const int per = d.D / 8;
  float df = 0.f, ds = 0.f;
  for (int i = 0; i < per; ++i) {
    const size_t e = row * d.D + (size_t)part * per + i;
    if (gf != nullptr) df = fmaf(load_as_f32(gf + e), load_as_f32(hf + e), df);
    if (gs != nullptr) ds = fmaf(load_as_f32(gs + e), load_as_f32(hs + e), ds);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    df += __shfl_xor(df, o);
    ds += __shfl_xor(ds, o);
  }
  if (part == 0) {
    const size_t plane = (size_t)d.B * d.Hq * d.Nq;
    float* st = stats + ((bh * (d.Nq / kStep) + s) * 4) * kStep;
    st[0 * kStep + r] = gf != nullptr ? lse[row] * kLog2e : 0.f;
    st[1 * kStep + r] = df;
    st[2 * kStep + r] = gs != nullptr ? lse[plane + row] * kLog2e : 0.f;
    st[3 * kStep + r] = ds;
  }
}

// ---------------------------------------------------------------- selection bits
// bits[bh][kt][s]: 16 bits per (b*q head, 128-key tile kt, 32-row step s);
// nibble w covers the 32 keys of wave w, bit 2*qsub + ksub the 16x16 quarter
// (query rows 16*qsub.., keys 16*ksub..) of that 32x32 block. A bit is set
// when the quarter's query block selected the quarter's key block. One thread
// per (b*q head, step) owns its column entries, so no two threads write one
// word.
__global__ __launch_bounds__(256) void bwd_bits_kernel(const int* __restrict__ idx,
                                                       const int* __restrict__ cnt,
                                                       uint16_t* __restrict__ bits, Dims d,
                                                       int nKT) {
  const int nS = d.Nq / kStep;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long)d.B * d.Hq * nS) return;
  const int s = (int)(t % nS);
  const size_t bh = (size_t)(t / nS);
  uint16_t* col = bits + bh * nKT * nS + s;
  for (int kt = 0; kt < nKT; ++kt) col[(size_t)kt * nS] = 0;
  const int nq = d.bs == 16 ? 2 : 1;
  for (int qs = 0; qs < nq; ++qs) {
    const int qb = d.bs == 16 ? 2 * s + qs : s >> 1;
    const int* list = idx + (bh * d.nQB + qb) * d.budget;
    const int n = min(max(cnt[bh * d.nQB + qb], 0), d.budget);
    for (int e = 0; e < n; ++e) {
      const int kb = list[e];
      if (kb < 0 || kb > qb) continue;
      if (d.bs == 16) {
        const int kw = kb >> 1;
        const int bit = 4 * (kw & 3) + 2 * qs + (kb & 1);
        col[(size_t)(kw >> 2) * nS] |= (uint16_t)(1u << bit);
      } else {
        for (int kw = 2 * kb; kw < 2 * kb + 2; ++kw)
          col[(size_t)(kw >> 2) * nS] |= (uint16_t)(0xFu << (4 * (kw & 3)));
      }
    }
  }
}

// ---------------------------------------------------------------- dK / dV
// One workgroup per (b, kv head, 128-key tile); four waves of 32 keys. For
// every q head of the group and every 32-row step reaching the tile: S and
// dP_f (and dP_s on selected blocks) from LDS tiles of Q and dO with K and V
// in registers, P and dS in registers, then dV^T += dO_f^T P_f (+ dO_s^T P_s)
// and dK^T += Q^T dS from the transposed tiles. The step tiles (Q, Q^T, dO_f,
// dO_f^T, dO_s, dO_s^T and the row statistics) are double-buffered in LDS;
// the copy of the next step overlaps the compute of the current one.
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ QT, const uint16_t* __restrict__ GF,
    const uint16_t* __restrict__ GFT, const uint16_t* __restrict__ GS,
    const uint16_t* __restrict__ GST, const float* __restrict__ stats,
    const uint16_t* __restrict__ bits, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    Dims d, HeadMap hm, int nKT) {
  constexpr int SPR = D / 8;          // 16-byte chunks per row-major row
  constexpr int KK = D / 32;          // 32-deep k-steps over D
  constexpr int MB = D / 16;          // 16-row blocks over D
  constexpr int TILE = kStep * D;     // bf16 elements per step tile
  __shared__ __align__(16) uint16_t sQ[2][TILE], sQT[2][TILE], sGF[2][TILE], sGFT[2][TILE];
  __shared__ __align__(16) uint16_t sGS[2][TILE], sGST[2][TILE];
  __shared__ __align__(16) float sStat[2][8 * kStep];
  __shared__ uint16_t sBits[kMaxSteps];

  const bool has_full = GF != nullptr, has_sparse = GS != nullptr;
  const int nBG = d.B * d.Hkv;
  const int bg = blockIdx.x % nBG, kt = blockIdx.x / nBG;   // heaviest tiles first
  const int b = bg / d.Hkv, g = bg % d.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, gq = lane >> 4;
  const int nS = d.Nq / kStep;
  const int kw0 = kt * kKeysPerWg + kStep * w;   // first key of this wave
  const bool wave_keys = kw0 < d.Nk;
  const int s_first = kt * (kKeysPerWg / kStep);  // first step whose rows reach the tile
  const float sl2 = d.scale_log2;

  bf16x8_t kreg[2][KK], vreg[2][KK];
  {
    const size_t base = ((size_t)bg * d.Nk) * D;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const size_t off = base + (size_t)(kw0 + 16 * nb + n) * D + 32 * kk + 8 * gq;
        kreg[nb][kk] = wave_keys ? *(const bf16x8_t*)(K + off) : bf16x8_t{};
        vreg[nb][kk] = wave_keys ? *(const bf16x8_t*)(V + off) : bf16x8_t{};
      }
  }
  f32x4_t accK[MB][2], accV[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) accK[mb][nb] = accV[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t head_bytes = (uint32_t)d.Nq * D * 2u;
  const uint32_t stat_bytes = (uint32_t)nS * 4u * kStep * 4u;

  for (int hi = 0; hi < d.G; ++hi) {
    const int h = hm.q_of_kv[g * d.G + hi];
    const size_t bh = (size_t)b * d.Hq + h;
    const i32x4_t rq = make_rsrc_words(Q + bh * d.Nq * D, head_bytes);
    const i32x4_t rqt = make_rsrc_words(QT + bh * d.Nq * D, head_bytes);
    const i32x4_t rgf = make_rsrc_words(has_full ? GF + bh * d.Nq * D : Q, has_full ? head_bytes : 0u);
    const i32x4_t rgft = make_rsrc_words(has_full ? GFT + bh * d.Nq * D : Q, has_full ? head_bytes : 0u);
    const i32x4_t rgs = make_rsrc_words(has_sparse ? GS + bh * d.Nq * D : Q, has_sparse ? head_bytes : 0u);
    const i32x4_t rgst = make_rsrc_words(has_sparse ? GST + bh * d.Nq * D : Q, has_sparse ? head_bytes : 0u);
    const i32x4_t rst = make_rsrc_words(stats + bh * nS * 4 * kStep, stat_bytes);

    __syncthreads();   // every wave is done with the previous head's tiles and bits
    if (has_sparse) {
      const uint16_t* bc = bits + ((size_t)bh * nKT + kt) * nS;
      for (int i = s_first + tid; i < nS; i += 256) sBits[i] = bc[i];
    }
    __syncthreads();
    auto step_bits = [&](int s) -> uint32_t { return has_sparse ? sBits[s] : 0u; };

    auto issue = [&](int s, int st) __attribute__((always_inline)) {
      const uint32_t toff = (uint32_t)s * kStep * D * 2u;     // row-major tile offset
      const uint32_t tcol = (uint32_t)s * kStep * 2u;         // transposed tile column offset
      const uint32_t trow = (uint32_t)d.Nq * 2u;              // transposed row stride
      copy_tile<SPR, kStep, false>(rq, toff, D * 2u, sQ[st], w, lane);
      copy_tile<4, D, true>(rqt, tcol, trow, sQT[st], w, lane);
      if (has_full) {
        copy_tile<SPR, kStep, false>(rgf, toff, D * 2u, sGF[st], w, lane);
        copy_tile<4, D, true>(rgft, tcol, trow, sGFT[st], w, lane);
      }
      if (has_sparse && step_bits(s) != 0) {
        copy_tile<SPR, kStep, false>(rgs, toff, D * 2u, sGS[st], w, lane);
        copy_tile<4, D, true>(rgst, tcol, trow, sGST[st], w, lane);
      }
      if (w == 0) {
        const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)s * 4u * kStep * 4u);
        const uint32_t la = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(lds_ptr_t)(&sStat[st][0]));
        copy16_to_lds(rst, soff, (uint32_t)lane * 16u, la);
      }
    };

    auto compute = [&](int s, int st) __attribute__((always_inline)) {
      if (!wave_keys || kStep * s + kStep - 1 < kw0) return;   // every key after every row
      const bool diag = kStep * s == kw0;
      const uint32_t nib = (step_bits(s) >> (4 * w)) & 0xFu;
      const bool sp = nib != 0;
      const uint16_t* tq = sQ[st];
      f32x4_t sa[2][2], pf[2][2], ps[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sa[mb][nb] = pf[mb][nb] = ps[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int row = rho(mb, n);
          const bf16x8_t a = frag_rows<SPR>(tq, row, 4 * kk + gq);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) sa[mb][nb] = mfma16(a, kreg[nb][kk], sa[mb][nb]);
          if (has_full) {
            const bf16x8_t af = frag_rows<SPR>(sGF[st], row, 4 * kk + gq);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) pf[mb][nb] = mfma16(af, vreg[nb][kk], pf[mb][nb]);
          }
          if (sp) {
            const bf16x8_t as = frag_rows<SPR>(sGS[st], row, 4 * kk + gq);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) ps[mb][nb] = mfma16(as, vreg[nb][kk], ps[mb][nb]);
          }
        }
      // P and dS, in the B-operand layout: slot j of lane group gq is row 8*gq + j
      float xf[2][8], xs[2][8], xd[2][8];
      const float* stt = sStat[st];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r0 = 8 * gq + 4 * mb;
        const f32x4_t lf = *(const f32x4_t*)(stt + 0 * kStep + r0);
        const f32x4_t df = *(const f32x4_t*)(stt + 1 * kStep + r0);
        const f32x4_t ls = *(const f32x4_t*)(stt + 2 * kStep + r0);
        const f32x4_t dd = *(const f32x4_t*)(stt + 3 * kStep + r0);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bool sel = sp && ((nib >> (2 * (gq >> 1) + nb)) & 1u);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool masked = diag && (16 * nb + n > r0 + i);
            const float x = sa[mb][nb][i] * sl2;
            float p = 0.f, dsv = 0.f, q = 0.f;
            if (has_full) {
              p = masked ? 0.f : fast_exp2(x - lf[i]);
              dsv = p * (pf[mb][nb][i] - df[i]);
            }
            if (sel) {
              q = masked ? 0.f : fast_exp2(x - ls[i]);
              dsv = fmaf(q, ps[mb][nb][i] - dd[i], dsv);
            }
            xf[nb][4 * mb + i] = p;
            xs[nb][4 * mb + i] = q;
            xd[nb][4 * mb + i] = dsv;
          }
        }
      }
      bf16x8_t bP[2], bS[2], bD[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bP[nb] = pack8(xf[nb]);
        bS[nb] = pack8(xs[nb]);
        bD[nb] = pack8(xd[nb]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = 16 * mb + n;
        if (has_full) {
          const bf16x8_t a = frag_t(sGFT[st], row, gq);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) accV[mb][nb] = mfma16(a, bP[nb], accV[mb][nb]);
        }
        if (sp) {
          const bf16x8_t a = frag_t(sGST[st], row, gq);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) accV[mb][nb] = mfma16(a, bS[nb], accV[mb][nb]);
        }
        const bf16x8_t aq = frag_t(sQT[st], row, gq);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) accK[mb][nb] = mfma16(aq, bD[nb], accK[mb][nb]);
      }
    };

    int s = has_full ? s_first : next_selected(s_first - 1, nS, lane, step_bits);
    if (s >= nS) continue;
    int st = 0;
    issue(s, st);
    while (true) {
      const int sn = has_full ? s + 1 : next_selected(s, nS, lane, step_bits);
      wait_vm();
      __syncthreads();   // step s landed for every wave; stage st^1 is free
      if (sn < nS) issue(sn, st ^ 1);
      compute(s, st);
      if (sn >= nS) break;
      s = sn;
      st ^= 1;
    }
  }
  wait_vm();

  if (!wave_keys) return;
  const size_t obase = ((size_t)bg * d.Nk) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t off = obase + (size_t)(kw0 + 16 * nb + n) * D + 16 * mb + 4 * gq;
      const f32x4_t kv = accK[mb][nb], vv = accV[mb][nb];
      store4_bf16(dK + off, kv[0] * d.scale, kv[1] * d.scale, kv[2] * d.scale, kv[3] * d.scale);
      store4_bf16(dV + off, vv[0], vv[1], vv[2], vv[3]);
    }
}

// ---------------------------------------------------------------- dQ
// One workgroup per (b, q head, 128-row query tile); four waves of 32 rows.
// Q and both upstream gradients of the wave's rows stay in registers; per
// 32-key step, S^T = K Q^T and dP^T = V dO^T from LDS tiles of K and V, then
// dQ^T += K^T dS^T from the K^T tile. The selection bits of the workgroup's
// rows are built in LDS from idx at the start.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ KT, const uint16_t* __restrict__ GF,
    const uint16_t* __restrict__ GS, const float* __restrict__ stats,
    const int* __restrict__ idx, const int* __restrict__ cnt, uint16_t* __restrict__ dQ, Dims d,
    HeadMap hm) {
  constexpr int SPR = D / 8;
  constexpr int KK = D / 32;
  constexpr int MB = D / 16;
  constexpr int TILE = kStep * D;
  __shared__ __align__(16) uint16_t sK[2][TILE], sV[2][TILE], sKT[2][TILE];
  __shared__ uint32_t sNib[kMaxSteps / 2];   // 16 bits per key step: nibble w for wave w

  const bool has_full = GF != nullptr, has_sparse = GS != nullptr;
  const int nBH = d.B * d.Hq;
  const int nQT = (d.Nq + kRowsPerWg - 1) / kRowsPerWg;
  const int bh = blockIdx.x % nBH, qt = nQT - 1 - (int)(blockIdx.x / nBH);   // heaviest first
  const int b = bh / d.Hq, h = bh % d.Hq;
  const int g = hm.kv_of_q[h];
  const size_t bgk = (size_t)b * d.Hkv + g;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, gq = lane >> 4;
  const int r0w = qt * kRowsPerWg + kStep * w;     // first row of this wave
  const bool wave_rows = r0w < d.Nq;
  const int last_row = min(qt * kRowsPerWg + kRowsPerWg, d.Nq) - 1;
  const int nT = last_row / kStep + 1;              // key steps of the workgroup (causal)
  const int nS = d.Nq / kStep;
  const float sl2 = d.scale_log2;

  // selection bits of the four waves' rows
  if (has_sparse) {
    for (int i = tid; i < (nT + 1) / 2; i += 256) sNib[i] = 0u;
    __syncthreads();
    if (wave_rows) {
      const int nq = d.bs == 16 ? 2 : 1;
      for (int qs = 0; qs < nq; ++qs) {
        const int qb = d.bs == 16 ? r0w / 16 + qs : r0w / 64;
        const int* list = idx + ((size_t)bh * d.nQB + qb) * d.budget;
        const int cn = min(max(cnt[(size_t)bh * d.nQB + qb], 0), d.budget);
        for (int e = lane; e < cn; e += 64) {
          const int kb = list[e];
          if (kb < 0 || kb > qb) continue;
          if (d.bs == 16) {
            const int t = kb >> 1;
            const uint32_t bit = 1u << (2 * qs + (kb & 1));
            atomicOr(&sNib[t >> 1], bit << (16 * (t & 1) + 4 * w));
          } else {
            for (int t = 2 * kb; t < 2 * kb + 2; ++t)
              atomicOr(&sNib[t >> 1], 0xFu << (16 * (t & 1) + 4 * w));
          }
        }
      }
    }
    __syncthreads();
  }
  auto step_bits = [&](int t) -> uint32_t {
    return has_sparse ? (sNib[t >> 1] >> (16 * (t & 1))) & 0xFFFFu : 0u;
  };

  // wave operands in registers
  bf16x8_t qreg[2][KK], freg[2][KK], sreg[2][KK];
  float lf[2], dfv[2], ls[2], dsv_[2];
  {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = wave_rows ? r0w + 16 * nb + n : 0;
      const size_t base = ((size_t)bh * d.Nq + row) * D + 8 * gq;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        qreg[nb][kk] = *(const bf16x8_t*)(Q + base + 32 * kk);
        freg[nb][kk] = has_full ? *(const bf16x8_t*)(GF + base + 32 * kk) : bf16x8_t{};
        sreg[nb][kk] = has_sparse ? *(const bf16x8_t*)(GS + base + 32 * kk) : bf16x8_t{};
      }
      const float* st = stats + (((size_t)bh * nS + row / kStep) * 4) * kStep + row % kStep;
      lf[nb] = st[0];
      dfv[nb] = st[kStep];
      ls[nb] = st[2 * kStep];
      dsv_[nb] = st[3 * kStep];
    }
  }
  f32x4_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t kv_bytes = (uint32_t)d.Nk * D * 2u;
  const i32x4_t rk = make_rsrc_words(K + bgk * d.Nk * D, kv_bytes);
  const i32x4_t rv = make_rsrc_words(V + bgk * d.Nk * D, kv_bytes);
  const i32x4_t rkt = make_rsrc_words(KT + bgk * d.Nk * D, kv_bytes);

  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)t * kStep * D * 2u;
    copy_tile<SPR, kStep, false>(rk, toff, D * 2u, sK[st], w, lane);
    copy_tile<SPR, kStep, false>(rv, toff, D * 2u, sV[st], w, lane);
    copy_tile<4, D, true>(rkt, (uint32_t)t * kStep * 2u, (uint32_t)d.Nk * 2u, sKT[st], w, lane);
  };

  auto compute = [&](int t, int st) __attribute__((always_inline)) {
    if (!wave_rows || kStep * t > r0w + kStep - 1) return;   // every key after every row
    const bool diag = kStep * t == r0w;
    const uint32_t nib = (step_bits(t) >> (4 * w)) & 0xFu;
    const bool sp = nib != 0;
    f32x4_t sa[2][2], pf[2][2], ps[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) sa[mb][nb] = pf[mb][nb] = ps[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int key = rho(mb, n);
        const bf16x8_t a = frag_rows<SPR>(sK[st], key, 4 * kk + gq);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sa[mb][nb] = mfma16(a, qreg[nb][kk], sa[mb][nb]);
        const bf16x8_t av = frag_rows<SPR>(sV[st], key, 4 * kk + gq);
        if (has_full) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) pf[mb][nb] = mfma16(av, freg[nb][kk], pf[mb][nb]);
        }
        if (sp) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) ps[mb][nb] = mfma16(av, sreg[nb][kk], ps[mb][nb]);
        }
      }
    float xd[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bool sel = sp && ((nib >> (2 * nb + (gq >> 1))) & 1u);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool masked = diag && (8 * gq + 4 * mb + i > 16 * nb + n);
          const float x = sa[mb][nb][i] * sl2;
          float dsv = 0.f;
          if (has_full) {
            const float p = masked ? 0.f : fast_exp2(x - lf[nb]);
            dsv = p * (pf[mb][nb][i] - dfv[nb]);
          }
          if (sel) {
            const float q = masked ? 0.f : fast_exp2(x - ls[nb]);
            dsv = fmaf(q, ps[mb][nb][i] - dsv_[nb], dsv);
          }
          xd[nb][4 * mb + i] = dsv;
        }
    }
    bf16x8_t bD[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bD[nb] = pack8(xd[nb]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8_t a = frag_t(sKT[st], 16 * mb + n, gq);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma16(a, bD[nb], acc[mb][nb]);
    }
  };

  int t = has_full ? 0 : next_selected(-1, nT, lane, step_bits);
  if (t < nT) {
    int st = 0;
    issue(t, st);
    while (true) {
      const int tn = has_full ? t + 1 : next_selected(t, nT, lane, step_bits);
      wait_vm();
      __syncthreads();
      if (tn < nT) issue(tn, st ^ 1);
      compute(t, st);
      if (tn >= nT) break;
      t = tn;
      st ^= 1;
    }
  }
  wait_vm();

  if (!wave_rows) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t off = ((size_t)bh * d.Nq + r0w + 16 * nb + n) * D + 16 * mb + 4 * gq;
      const f32x4_t a = acc[mb][nb];
      store4_bf16(dQ + off, a[0] * d.scale, a[1] * d.scale, a[2] * d.scale, a[3] * d.scale);
    }
}

// ---------------------------------------------------------------- float32
// Plain VALU kernels for float32 problems: one wave per (b, q head, row)
// for dQ and per (b, kv head, key) for dK/dV; lanes split D, dot products
// are wave reductions.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ bool block_selected(const int* list, int n, int kb) {
  for (int e = 0; e < n; ++e)
    if (list[e] == kb) return true;
  return false;
}

template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ GF, const float* __restrict__ GS, const float* __restrict__ stats,
    const int* __restrict__ idx, const int* __restrict__ cnt, float* __restrict__ dQ, Dims d,
    HeadMap hm) {
  constexpr int E = D / 64;
  const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * d.Hq + h;
  const size_t bg = (size_t)b * d.Hkv + hm.kv_of_q[h];
  const int lane = threadIdx.x;
  const int nS = d.Nq / kStep;
  const float* st = stats + ((bh * nS + row / kStep) * 4) * kStep + row % kStep;
  const float lf = st[0], df = st[kStep], ls = st[2 * kStep], dd = st[3 * kStep];
  const int qb = row / d.bs;
  const int* list = idx + (bh * d.nQB + qb) * d.budget;
  const int ncnt = min(max(cnt[bh * d.nQB + qb], 0), d.budget);
  float q[E], gf[E], gs[E], acc[E];
  const size_t ro = (bh * d.Nq + row) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = Q[ro + lane + 64 * e];
    gf[e] = GF != nullptr ? GF[ro + lane + 64 * e] : 0.f;
    gs[e] = GS != nullptr ? GS[ro + lane + 64 * e] : 0.f;
    acc[e] = 0.f;
  }
  const float* kb0 = K + bg * d.Nk * D;
  const float* vb0 = V + bg * d.Nk * D;
  for (int j = 0; j <= row; ++j) {
    const bool sel = GS != nullptr && block_selected(list, ncnt, j / d.bs);
    if (GF == nullptr && !sel) continue;
    float sp = 0.f, dpf = 0.f, dps = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float kv = kb0[(size_t)j * D + lane + 64 * e];
      const float vv = vb0[(size_t)j * D + lane + 64 * e];
      sp = fmaf(q[e], kv, sp);
      dpf = fmaf(gf[e], vv, dpf);
      dps = fmaf(gs[e], vv, dps);
    }
    const float x = wave_sum(sp) * d.scale_log2;
    float ds = 0.f;
    if (GF != nullptr) {
      const float p = exp2f(x - lf);
      ds = p * (wave_sum(dpf) - df);
    }
    if (sel) {
      const float p = exp2f(x - ls);
      ds = fmaf(p, wave_sum(dps) - dd, ds);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kb0[(size_t)j * D + lane + 64 * e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) dQ[ro + lane + 64 * e] = acc[e] * d.scale;
}

template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ GF, const float* __restrict__ GS, const float* __restrict__ stats,
    const int* __restrict__ idx, const int* __restrict__ cnt, float* __restrict__ dK,
    float* __restrict__ dV, Dims d, HeadMap hm) {
  constexpr int E = D / 64;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const size_t bg = (size_t)b * d.Hkv + g;
  const int lane = threadIdx.x;
  const int nS = d.Nq / kStep;
  const int kb = j / d.bs;
  float k[E], v[E], ak[E], av[E];
  const size_t ko = (bg * d.Nk + j) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = K[ko + lane + 64 * e];
    v[e] = V[ko + lane + 64 * e];
    ak[e] = av[e] = 0.f;
  }
  for (int hi = 0; hi < d.G; ++hi) {
    const int h = hm.q_of_kv[g * d.G + hi];
    const size_t bh = (size_t)b * d.Hq + h;
    for (int row = j; row < d.Nq; ++row) {
      const int qb = row / d.bs;
      const bool sel = GS != nullptr &&
                       block_selected(idx + (bh * d.nQB + qb) * d.budget,
                                      min(max(cnt[bh * d.nQB + qb], 0), d.budget), kb);
      if (GF == nullptr && !sel) continue;
      const size_t ro = (bh * d.Nq + row) * D;
      float qv[E], gf[E], gs[E];
      float sp = 0.f, dpf = 0.f, dps = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        qv[e] = Q[ro + lane + 64 * e];
        gf[e] = GF != nullptr ? GF[ro + lane + 64 * e] : 0.f;
        gs[e] = GS != nullptr ? GS[ro + lane + 64 * e] : 0.f;
        sp = fmaf(qv[e], k[e], sp);
        dpf = fmaf(gf[e], v[e], dpf);
        dps = fmaf(gs[e], v[e], dps);
      }
      const float* st = stats + ((bh * nS + row / kStep) * 4) * kStep + row % kStep;
      const float x = wave_sum(sp) * d.scale_log2;
      float ds = 0.f, pf = 0.f, ps = 0.f;
      if (GF != nullptr) {
        pf = exp2f(x - st[0]);
        ds = pf * (wave_sum(dpf) - st[kStep]);
      }
      if (sel) {
        ps = exp2f(x - st[2 * kStep]);
        ds = fmaf(ps, wave_sum(dps) - st[3 * kStep], ds);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        av[e] = fmaf(pf, gf[e], fmaf(ps, gs[e], av[e]));
        ak[e] = fmaf(ds, qv[e], ak[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dK[ko + lane + 64 * e] = ak[e] * d.scale;
    dV[ko + lane + 64 * e] = av[e];
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_attn_bwd_stats(const void* hf, const void* hs, const void* gf, const void* gs,
                                 const float* lse, float* stats, bool bf16, const Dims& d,
                                 hipStream_t stream) {
  const dim3 grid(d.Nq / kStep, d.B * d.Hq);
  if (bf16)
    hipLaunchKernelGGL(bwd_stats_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (const uint16_t*)hf, (const uint16_t*)hs, (const uint16_t*)gf,
                       (const uint16_t*)gs, lse, stats, d);
  else
    hipLaunchKernelGGL(bwd_stats_kernel<float>, grid, dim3(256), 0, stream, (const float*)hf,
                       (const float*)hs, (const float*)gf, (const float*)gs, lse, stats, d);
  return hipGetLastError();
}

int bwd_key_tiles(const Dims& d) { return (d.Nk + kKeysPerWg - 1) / kKeysPerWg; }

hipError_t launch_attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* qt, const uint16_t* kt, const uint16_t* gf,
                                const uint16_t* gft, const uint16_t* gs, const uint16_t* gst,
                                const int* idx, const int* cnt, const float* stats,
                                uint16_t* bits, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                                const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const int nKT = bwd_key_tiles(d);
  if (gs != nullptr) {
    const long threads = (long)d.B * d.Hq * (d.Nq / kStep);
    hipLaunchKernelGGL(bwd_bits_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, idx, cnt, bits, d, nKT);
  }
  const dim3 g1((unsigned)(nKT * d.B * d.Hkv));
  const int nQT = (d.Nq + kRowsPerWg - 1) / kRowsPerWg;
  const dim3 g2((unsigned)(nQT * d.B * d.Hq));
  if (d.D == 128) {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, g1, dim3(256), 0, stream, q, k, v, qt, gf, gft,
                       gs, gst, stats, bits, dk, dv, d, hm, nKT);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, g2, dim3(256), 0, stream, q, k, v, kt, gf, gs,
                       stats, idx, cnt, dq, d, hm);
  } else {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, g1, dim3(256), 0, stream, q, k, v, qt, gf, gft,
                       gs, gst, stats, bits, dk, dv, d, hm, nKT);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, g2, dim3(256), 0, stream, q, k, v, kt, gf, gs,
                       stats, idx, cnt, dq, d, hm);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* gf,
                               const float* gs, const int* idx, const int* cnt,
                               const float* stats, float* dq, float* dk, float* dv,
                               const Dims& d, const HeadMap& hm, hipStream_t stream) {
  const dim3 gq(d.Nq, d.Hq, d.B), gk(d.Nk, d.Hkv, d.B);
  if (d.D == 128) {
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<128>, gq, dim3(64), 0, stream, q, k, v, gf, gs,
                       stats, idx, cnt, dq, d, hm);
    hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<128>, gk, dim3(64), 0, stream, q, k, v, gf, gs,
                       stats, idx, cnt, dk, dv, d, hm);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, gq, dim3(64), 0, stream, q, k, v, gf, gs,
                       stats, idx, cnt, dq, d, hm);
    hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<64>, gk, dim3(64), 0, stream, q, k, v, gf, gs,
                       stats, idx, cnt, dk, dv, d, hm);
  }
  return hipGetLastError();
}

}  // namespace ssa

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
// visits the 32-row query steps that reach those keys, for every q head of
// the GQA group, from the last step down, heads innermost; all workgroups of
// one kv head start at the last step, so they stream the same Q / dO rows
// through L2 at about the same time. The sparse stream's extra products run
// only on (step, wave) pairs whose blocks are selected. The dQ kernel owns 128
// query rows of one q head (32 per wave) and visits 32-key steps up to the
// diagonal. In dual mode both kernels walk every causal step (the full
// stream needs them all); in sparse-only mode (no full-stream gradient) only
// steps with a selected block.
//
// MFMA 16x16x32 bf16 throughout. The dK/dV kernel computes S = Q K^T and
// dP = dO V^T with query rows on the output's register index, so P and dS
// sit in the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS once the
// A rows of the first products are read in the kperm16 order; the dQ kernel
// does the same with keys: S^T = K Q^T, dQ^T = K^T dS^T. The transposed A
// operands (dO^T, Q^T, K^T) come from the same row-major LDS tiles through
// the LDS transpose read (ds_read_b64_tr_b16), so every tile crosses L2 once.
#include "ssa_common.h"
#include "ssa_device.h"
#include "ssa_kernels.h"

namespace ssa {

namespace {

constexpr int kStep = 32;        // query rows per dK/dV step, keys per dQ step
constexpr int kKeysPerWg = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int kRowsPerWg = 128;  // query rows per dQ workgroup (32 per wave)
constexpr int kMaxSteps = 8192;  // 32-row (32-key) steps per head: N <= 262144
constexpr int kStages = 4;       // LDS stages of the dK/dV and dQ pipelines

// Wait until at most N vector memory operations of this wave are in flight
// (loads complete in issue order, so every older one has landed).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// kperm16 with 32-row tiles: MFMA A row m of row block mb reads tile row
// 8*(m/4) + 4*mb + m%4, so output register i of lane group g holds tile row
// 8*g + 4*mb + i, and the eight values of one lane over (mb, i) are the eight
// consecutive rows 8*g .. 8*g+7 that a 32-deep B operand slot range needs.
__device__ __forceinline__ int rho(int mb, int m) { return 8 * (m >> 2) + 4 * mb + (m & 3); }

// 16-byte chunk swizzle of the 32-row tiles. Two read patterns must be free
// of bank conflicts: the kperm16 row reads (16 lanes, rows differing in bits
// 0, 1, 3 and 4, one logical chunk: the swizzle must be injective on those
// bits) and the transpose reads (32 lanes, rows differing in bits 0, 1 and 3,
// two adjacent logical chunks: the swizzle shifted right by one must be
// injective on those bits). 256-byte rows (16 chunks):
// f = b4 | b0<<1 | b1<<2 | b3<<3; 128-byte rows (8 chunks, two rows per 256
// bytes, so bit 0 already separates rows): f = b4 | b1<<1 | b3<<2.
template <int SPR>
__device__ __forceinline__ int bswz(int row, int chunk) {
  if constexpr (SPR == 16)
    return chunk ^ (((row >> 4) & 1) | ((row & 3) << 1) | (((row >> 3) & 1) << 3));
  else
    return chunk ^ (((row >> 4) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2));
}

// One 32-row tile copy, global -> LDS, SPR 16-byte chunks per row, shared by
// four waves. Lane i of a wave instruction fills LDS slot slot0 + i and
// fetches the global chunk that the swizzle (an involution) maps to it.
template <int SPR>
__device__ __forceinline__ void copy_tile(i32x4_t rsrc, uint32_t tile_off, uint32_t lds,
                                          int wave, int lane) {
  constexpr int PER_WAVE = kStep * SPR / 4;
  static_assert(PER_WAVE % 64 == 0, "tile slots per wave");
#pragma unroll
  for (int j = 0; j < PER_WAVE / 64; ++j) {
    const int slot0 = wave * PER_WAVE + j * 64;
    const int r0 = slot0 / SPR;
    const int rl = lane / SPR, sl = lane % SPR;
    const uint32_t voff = (uint32_t)rl * SPR * 16u + (uint32_t)bswz<SPR>(r0 + rl, sl) * 16u;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(tile_off + (uint32_t)r0 * SPR * 16u);
    copy16_to_lds(rsrc, soff, voff, __builtin_amdgcn_readfirstlane(lds + slot0 * 16u));
  }
}

// LDS byte address of a __shared__ object. Tiles are addressed by these
// integers: a generic -> LDS cast of a pointer chosen at run time (a stage)
// would need a null check.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// A-operand fragment T[row][chunk] (rows of SPR 16-byte chunks): MFMA row m
// of a 16x32 A block reading 8 consecutive columns of one tile row.
template <int SPR>
__device__ __forceinline__ bf16x8_t frag_rows(uint32_t t, int row, int chunk) {
  typedef __attribute__((address_space(3))) const bf16x8_t* lp;
  return *(lp)(uintptr_t)(t + 2u * (uint32_t)(row * SPR * 8 + bswz<SPR>(row, chunk) * 8));
}

// Transposed A-operand fragment: A[m][k] = T[k][c0 + m] for the 16 columns
// c0 .. c0+15 (c0 a multiple of 16) and the 32 tile rows, so lane (m, g)
// gets T[8g + j][c0 + m], j = 0..7. ds_read_b64_tr_b16 hands lane i of a
// 16-lane group element M[4j + i/4][i%4] (j = 0..3) of the 4-element pieces
// M[L] its lanes L address; lane L therefore addresses row 8g + 4h + L/4,
// columns c0 + 4(L%4) .. +3, once for each half h of the eight rows.
template <int SPR>
__device__ __forceinline__ bf16x8_t frag_tr(uint32_t base, int c0, int lane) {
  typedef __attribute__((address_space(3))) i16x4_t* lp;
  const int L = lane & 15, g = lane >> 4;
  const int col = c0 + 4 * (L & 3);
  const int chunk = col >> 3, half = (col >> 2) & 1;
  i16x4_t r[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * g + 4 * h + (L >> 2);
    const uint32_t a = base + 2u * (uint32_t)(row * SPR * 8 + bswz<SPR>(row, chunk) * 8 + half * 4);
    r[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(uintptr_t)a);
  }
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v{r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
  return __builtin_bit_cast(bf16x8_t, v);
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

// Scheduling pattern for NR LDS reads feeding MPR MFMAs each, in order: PF
// reads first (at most NR), then (MPR MFMAs, one read) pairs, then the remaining MFMAs,
// so every read runs PF / MPR MFMA groups ahead of its use instead of each
// MFMA waiting for its own read.
template <int NR, int MPR, int PF_>
__device__ __forceinline__ void pipeline_mix() {
  constexpr int PF = PF_ < NR ? PF_ : NR;
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);      // DS reads
#pragma unroll
  for (int k = 0; k < NR - PF; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MPR * PF, 0);
}

// First step s' > s whose selection bits are nonzero (sparse-only walks), or
// `end`. `bits(i)` reads the bit word of step i; the 64 lanes test 64
// candidates at a time, so every wave gets the same answer.
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
// lanes per row, each over D/8 contiguous elements.
__device__ __forceinline__ float dot8(const uint16_t* a, const uint16_t* b, float acc) {
  const uint4 x = *(const uint4*)a, y = *(const uint4*)b;
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(xs[i] << 16), __uint_as_float(ys[i] << 16), acc);
    acc = fmaf(__uint_as_float(xs[i] & 0xffff0000u), __uint_as_float(ys[i] & 0xffff0000u), acc);
  }
  return acc;
}
__device__ __forceinline__ float dot8(const float* a, const float* b, float acc) {
  const float4 x0 = *(const float4*)a, x1 = *(const float4*)(a + 4);
  const float4 y0 = *(const float4*)b, y1 = *(const float4*)(b + 4);
  acc = fmaf(x0.x, y0.x, acc); acc = fmaf(x0.y, y0.y, acc);
  acc = fmaf(x0.z, y0.z, acc); acc = fmaf(x0.w, y0.w, acc);
  acc = fmaf(x1.x, y1.x, acc); acc = fmaf(x1.y, y1.y, acc);
  acc = fmaf(x1.z, y1.z, acc); acc = fmaf(x1.w, y1.w, acc);
  return acc;
}

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
  for (int i = 0; i < per; i += 8) {
    const size_t e = row * d.D + (size_t)part * per + i;
    if (gf != nullptr) df = dot8(gf + e, hf + e, df);
    if (gs != nullptr) ds = dot8(gs + e, hs + e, ds);
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
// bits[b*kv head][kt][s][hi]: 16 bits per (128-key tile kt, 32-row step s,
// q head hi of the GQA group); nibble w covers the 32 keys of wave w, bit
// 2*qsub + ksub the 16x16 quarter (query rows 16*qsub.., keys 16*ksub..) of
// that 32x32 block. A bit is set when the quarter's query block selected the
// quarter's key block. One thread per (b*q head, step) owns its entries, so
// no two threads write one word.
__global__ __launch_bounds__(256) void bwd_bits_kernel(const int* __restrict__ idx,
                                                       const int* __restrict__ cnt,
                                                       uint16_t* __restrict__ bits,
                                                       uint64_t* __restrict__ rowbits, Dims d,
                                                       HeadMap hm, int nKT) {
  const int nS = d.Nq / kStep;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long)d.B * d.Hq * nS) return;
  const int s = (int)(t % nS);
  const size_t bh = (size_t)(t / nS);
  const int b = (int)(bh / d.Hq), h = (int)(bh % d.Hq);
  const int g = hm.kv_of_q[h];
  int hi = 0;
  while (hi < d.G - 1 && hm.q_of_kv[g * d.G + hi] != h) ++hi;
  const size_t bg = (size_t)b * d.Hkv + g;
  uint16_t* col = bits + (bg * nKT * nS + s) * d.G + hi;    // entry kt at col[kt * nS * G]
  const size_t kstride = (size_t)nS * d.G;
  for (int kt = 0; kt < nKT; ++kt) col[kt * kstride] = 0;
  if (d.tok) {
    // per-token lists: the rows of the step select on their own; the nibbles
    // say whether any row of a 16-row half selected a 16-key half, and
    // rowbits[bg][kt][s][hi][wave] holds bit 32*(key half) + row of each
    // 32-key wave block
    uint64_t* rb = rowbits + ((bg * nKT * nS + s) * d.G + hi) * 4;   // entry kt at rb[kt * kstride * 4]
    for (int kt = 0; kt < nKT; ++kt)
      for (int wv = 0; wv < 4; ++wv) rb[kt * kstride * 4 + wv] = 0ull;
    for (int j = 0; j < kStep; ++j) {
      const int row = kStep * s + j;
      const size_t lr = bh * d.nL + row;
      const int* list = idx + lr * d.budget;
      const int n = min(max(cnt[lr], 0), d.budget);
      const int diag = row / d.bs;
      for (int e = 0; e < n; ++e) {
        const int kb = list[e];
        if (kb < 0 || kb > diag) continue;
        for (int kw = kb * d.bs / kStep; kw < (kb * d.bs + d.bs + kStep - 1) / kStep; ++kw) {
          const int kt = kw >> 2, wv = kw & 3;
          // key halves of the wave block covered by this block
          const int h0 = d.bs == 16 ? (kb & 1) : 0, h1 = d.bs == 16 ? (kb & 1) : 1;
          for (int kh = h0; kh <= h1; ++kh) {
            col[kt * kstride] |= (uint16_t)(1u << (4 * wv + 2 * (j >> 4) + kh));
            rb[kt * kstride * 4 + wv] |= 1ull << (32 * kh + j);
          }
        }
      }
    }
    return;
  }
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
        col[(kw >> 2) * kstride] |= (uint16_t)(1u << bit);
      } else {
        for (int kw = 2 * kb; kw < 2 * kb + 2; ++kw)
          col[(kw >> 2) * kstride] |= (uint16_t)(0xFu << (4 * (kw & 3)));
      }
    }
  }
}

// ---------------------------------------------------------------- dK / dV
// One workgroup per (b, kv head, 128-key tile); four waves of 32 keys. Items
// are (32-row step s, q head hi) pairs, s from the last step down to the
// tile's first, hi innermost. Per item, three phases:
//   A: S = Q K^T and dP_f = dO_f V^T (and dP_s on selected blocks) from the
//      LDS tiles of Q and dO, K and V in registers;
//   B: P and dS in registers (exp2, products, bf16 packing);
//   C: dV^T += dO_f^T P_f (+ dO_s^T P_s), dK^T += Q^T dS, the transposed
//      operands read from the same tiles.
// The LDS fragment reads of A and C run a few MFMAs ahead of their use. Item
// tiles (Q, dO_f, dO_s, row statistics) sit in four LDS stages; the copies
// run three items ahead of the compute. The items' bit
// words arrive 64 at a time (lane i holds item 64c + i), one chunk ahead.
// MODE 0: both streams; 1: full stream only; 2: sparse stream only (items
// without a selected block are skipped).
// TOK: per-token lists; the selection of each of the item's rows comes from
// rowbits (one 64-bit word per wave: bit 32*(key half) + row).
template <int D, int MODE, int IO, bool TOK>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ GF, const uint16_t* __restrict__ GS,
    const float* __restrict__ stats, const uint16_t* __restrict__ bits,
    const uint64_t* __restrict__ rowbits, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    float* __restrict__ pK, float* __restrict__ pV, Dims d, HeadMap hm, int nKT, int hsplit) {
  constexpr bool FULL = MODE != 2, SPARSE = MODE != 1;
  constexpr int SPR = D / 8;          // 16-byte chunks per row
  constexpr int KK = D / 32;          // 32-deep k-steps over D
  constexpr int MB = D / 16;          // 16-column blocks over D
  constexpr int TILE = kStep * D;     // bf16 elements per step tile
  constexpr int CT = kStep * SPR / 4 / 64;   // copy instructions per tile per wave
  constexpr int CPI = CT * (1 + (FULL ? 1 : 0) + (SPARSE ? 1 : 0)) + 1;   // per item per wave
  static_assert(2 * CPI < 16, "vmcnt immediate");
  __shared__ __align__(16) uint16_t sQ[kStages][TILE];
  __shared__ __align__(16) uint16_t sGF[FULL ? kStages : 1][FULL ? TILE : 8];
  __shared__ __align__(16) uint16_t sGS[SPARSE ? kStages : 1][SPARSE ? TILE : 8];
  __shared__ __align__(16) float sStat[kStages][4 * kStep];
  constexpr uint32_t TB = TILE * 2u, SB = 4u * kStep * 4u;   // stage strides in bytes
  const uint32_t aQ = lds_u32(&sQ[0][0]), aGF = lds_u32(&sGF[0][0]);
  const uint32_t aGS = lds_u32(&sGS[0][0]), aSt = lds_u32(&sStat[0][0]);

  const int nBG = d.B * d.Hkv;
  // The q heads of a kv head are split into hsplit groups of GW heads, one
  // workgroup per (tile, group), each writing its own float32 slot. The
  // sparse stream (MODE 2) runs one workgroup per (tile, q head): a block
  // that every query selects (the sink) would otherwise make one workgroup
  // walk every step of every head alone. The full stream splits when there
  // are too few (tile, kv head) pairs to balance the chip.
  const int bg = blockIdx.x % nBG;
  const int hgi = (blockIdx.x / nBG) % hsplit;              // head group
  const int kt = blockIdx.x / (nBG * hsplit);               // heaviest tiles first
  const int b = bg / d.Hkv, g = bg % d.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nS = d.Nq / kStep;
  const int G = d.G;
  const int GW = G / hsplit;                                // q heads walked by this workgroup
  const int h0 = hgi * GW;                                  // its first head within the group
  const int kw0 = kt * kKeysPerWg + kStep * w;   // first key of this wave
  const bool wave_keys = kw0 < d.Nk;
  const int s_first = kt * (kKeysPerWg / kStep);  // first step whose rows reach the tile
  const int nItems = GW * (nS - s_first);
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
  // float32 outputs go to pK / pV, a split workgroup's to its head's slot
  const size_t obase = (size_t)hgi * d.B * d.Hkv * d.Nk * D + ((size_t)bg * d.Nk) * D;
  auto out_off = [&](int mb, int nb) {
    return obase + (size_t)(kw0 + 16 * nb + n) * D + 16 * mb + 4 * gq;
  };
  f32x4_t accK[MB][2], accV[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) accK[mb][nb] = accV[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // item e -> (step, head index)
  auto item_s = [&](int e) { return nS - 1 - e / GW; };
  auto item_h = [&](int e) { return h0 + e % GW; };
  const uint16_t* tile_bits = bits + (size_t)(bg * nKT + kt) * nS * G;
  auto load_chunk = [&](int c) -> uint32_t {
    const int e = 64 * c + lane;
    if (!SPARSE || e >= nItems) return 0u;
    return tile_bits[(size_t)item_s(e) * G + item_h(e)];
  };
  int chunk = 0;
  uint32_t chA = load_chunk(0), chB = load_chunk(1);
  // next item >= from that has work (every item unless sparse-only), with
  // its bit word; nItems when none is left
  auto find = [&](int from, uint32_t& word) -> int {
    while (from < nItems) {
      while ((from >> 6) > chunk) {
        chA = chB;
        chB = load_chunk(chunk + 2);
        ++chunk;
      }
      const uint64_t act = MODE == 2 ? __ballot(chA != 0u) : ~0ull;
      const uint64_t m = act & (~0ull << (from & 63));
      if (m) {
        const int e = (chunk << 6) + __builtin_ctzll(m);
        word = __builtin_amdgcn_readlane(chA, e & 63);
        return e;
      }
      from = (chunk + 1) << 6;
    }
    return nItems;
  };

  const uint32_t head_bytes = (uint32_t)d.Nq * D * 2u;
  const uint32_t stat_bytes = (uint32_t)nS * 4u * kStep * 4u;

  auto issue = [&](int e, uint32_t word, int st) __attribute__((always_inline)) {
    const int s = item_s(e);
    const size_t bh = (size_t)b * d.Hq + hm.q_of_kv[g * G + item_h(e)];
    const uint32_t toff = (uint32_t)s * kStep * D * 2u;
    copy_tile<SPR>(make_rsrc_words(Q + bh * d.Nq * D, head_bytes), toff, aQ + st * TB, w, lane);
    if (FULL)
      copy_tile<SPR>(make_rsrc_words(GF + bh * d.Nq * D, head_bytes), toff, aGF + st * TB, w, lane);
    if (SPARSE)   // a record count of 0 turns an unneeded copy into zero fills, so
                  // every item issues the same number of copies
      copy_tile<SPR>(make_rsrc_words(GS + bh * d.Nq * D, word != 0u ? head_bytes : 0u), toff,
                     aGS + st * TB, w, lane);
    if (lane < 8) {   // wave w brings statistics array w of the item's 32 rows
      const uint32_t la = __builtin_amdgcn_readfirstlane(aSt + st * SB + kStep * 4u * w);
      copy16_to_lds(make_rsrc_words(stats + bh * nS * 4 * kStep, stat_bytes),
                    __builtin_amdgcn_readfirstlane((uint32_t)(s * 4 + w) * kStep * 4u),
                    (uint32_t)lane * 16u, la);
    }
  };

  // No early exit and no branch around the dK / dV updates: a wave whose keys
  // all follow the item's rows gets P = dS = 0 from the causal mask, so the
  // loop-carried accumulators never pass through a control-flow merge (which
  // would copy them between register files every item).
  auto compute = [&](int e, uint32_t word, int st) __attribute__((always_inline)) {
    const int s = item_s(e);
    const int rel = kStep * s - kw0;   // row position minus key position of (0, 0)
    const uint32_t nib = SPARSE ? (word >> (4 * w)) & 0xFu : 0u;
    const bool sp = nib != 0u;
    // per-token lists: bits of the lane's rows 8*gq .. 8*gq+7, per key half
    uint32_t rsel[2] = {0u, 0u};
    if (TOK && SPARSE) {
      const uint64_t rm = rowbits[(((size_t)bg * nKT + kt) * nS + s) * G * 4 + (size_t)item_h(e) * 4 + w];
      rsel[0] = (uint32_t)(rm >> (8 * gq)) & 0xFFu;
      rsel[1] = (uint32_t)(rm >> (32 + 8 * gq)) & 0xFFu;
    }
    typedef __attribute__((address_space(3))) const f32x4_t* lpf;
    auto stat = [&](int a, int r0) { return *(lpf)(uintptr_t)(aSt + st * SB + 4u * (a * kStep + r0)); };
    // statistics of the lane's rows 8*gq + 4*mb + r, read ahead of use
    f32x4_t lf[2], df[2], ls[2], dd[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r0 = 8 * gq + 4 * mb;
      if (FULL) {
        lf[mb] = stat(0, r0);
        df[mb] = stat(1, r0);
      }
      if (sp) {
        ls[mb] = stat(2, r0);
        dd[mb] = stat(3, r0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // A: S and dP_f; the dP accumulators start at -D_r of their rows, so they
    // end as dP - D_r
    f32x4_t sa[2][2], pf[2][2], ps[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        sa[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pf[mb][nb] = FULL ? -df[mb] : sa[mb][nb];
        ps[mb][nb] = sp ? -dd[mb] : sa[mb][nb];
      }
    {
      constexpr int NR = (FULL ? 2 : 1) * 2 * KK;   // fragment reads
      bf16x8_t fr[NR];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int i = (FULL ? 2 : 1) * (2 * kk + mb);
          fr[i] = frag_rows<SPR>(aQ + st * TB, rho(mb, n), 4 * kk + gq);
          if (FULL) fr[i + 1] = frag_rows<SPR>(aGF + st * TB, rho(mb, n), 4 * kk + gq);
        }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int i = (FULL ? 2 : 1) * (2 * kk + mb);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) sa[mb][nb] = mfma16(fr[i], kreg[nb][kk], sa[mb][nb]);
          if (FULL) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) pf[mb][nb] = mfma16(fr[i + 1], vreg[nb][kk], pf[mb][nb]);
          }
        }
      pipeline_mix<NR, 2, 6>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (sp) {
      bf16x8_t fr[2 * KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fr[2 * kk + mb] = frag_rows<SPR>(aGS + st * TB, rho(mb, n), 4 * kk + gq);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) ps[mb][nb] = mfma16(fr[2 * kk + mb], vreg[nb][kk], ps[mb][nb]);
      pipeline_mix<2 * KK, 2, 4>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // B: P and dS in the B-operand layout (slot j of lane group gq is row 8*gq + j)
    float xf[2][8], xs[2][8], xd[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r0 = 8 * gq + 4 * mb;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bool selb = sp && ((nib >> (2 * (gq >> 1) + nb)) & 1u);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool sel = TOK ? ((rsel[nb] >> (4 * mb + r)) & 1u) != 0u : selb;
          const bool keep = 16 * nb + n <= rel + r0 + r;   // key <= row
          float p = 0.f, dsv = 0.f, q = 0.f;
          if (FULL) {
            p = fast_exp2(fmaf(sa[mb][nb][r], sl2, -lf[mb][r]));
            p = keep ? p : 0.f;
            dsv = p * pf[mb][nb][r];
          }
          if (sp) {
            q = fast_exp2(fmaf(sa[mb][nb][r], sl2, -ls[mb][r]));
            q = (keep && sel) ? q : 0.f;
            dsv = fmaf(q, ps[mb][nb][r], dsv);
          }
          xf[nb][4 * mb + r] = p;
          xs[nb][4 * mb + r] = q;
          xd[nb][4 * mb + r] = dsv;
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
    __builtin_amdgcn_sched_barrier(0);
    // C: dV^T += dO^T P (+ dO_s^T P_s), dK^T += Q^T dS
    {
      constexpr int NR = (FULL ? 2 : 1) * MB;
      bf16x8_t tr[NR];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int i = (FULL ? 2 : 1) * mb;
        tr[i] = frag_tr<SPR>(aQ + st * TB, 16 * mb, lane);
        if (FULL) tr[i + 1] = frag_tr<SPR>(aGF + st * TB, 16 * mb, lane);
      }
      bf16x8_t ts[SPARSE ? MB : 1];
      if (SPARSE) {
        // the sparse products run on every item; without a selected block
        // P_s is 0 and the Q^T fragments stand in for dO_s^T
        if (sp) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) ts[mb] = frag_tr<SPR>(aGS + st * TB, 16 * mb, lane);
        } else {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) ts[mb] = tr[(FULL ? 2 : 1) * mb];
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int i = (FULL ? 2 : 1) * mb;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) accK[mb][nb] = mfma16(tr[i], bD[nb], accK[mb][nb]);
        if (FULL) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) accV[mb][nb] = mfma16(tr[i + 1], bP[nb], accV[mb][nb]);
        }
        if (SPARSE) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) accV[mb][nb] = mfma16(ts[mb], bS[nb], accV[mb][nb]);
        }
      }
      pipeline_mix<2 * NR, (FULL ? 1 : 2) + (SPARSE ? 1 : 0), 8>();   // two transpose reads per fragment
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // items x0 (current) .. x3, with their bit words; copies run three items
  // ahead of the compute, each into the stage the item four back used
  int x0, x1, x2, x3;
  uint32_t w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
  x0 = find(0, w0);
  x1 = x0 < nItems ? find(x0 + 1, w1) : nItems;
  x2 = x1 < nItems ? find(x1 + 1, w2) : nItems;
  if (x0 < nItems) {
    issue(x0, w0, 0);
    if (x1 < nItems) issue(x1, w1, 1);
    if (x2 < nItems) issue(x2, w2, 2);
    int e = 0;   // ordinal of x0 in the walk; its stage is e % kStages
    while (true) {
      x3 = x2 < nItems ? find(x2 + 1, w3) : nItems;
      // item x0 has landed once at most the copies of x1 and x2 are in flight
      if (x2 < nItems) wait_vm_n<2 * CPI>();
      else if (x1 < nItems) wait_vm_n<CPI>();
      else wait_vm();
      __syncthreads();   // x0 visible to every wave; stage (e + 3) % 4 is free
      if (x3 < nItems) issue(x3, w3, (e + 3) % kStages);
      compute(x0, w0, e % kStages);
      if (x1 >= nItems) break;
      x0 = x1; w0 = w1;
      x1 = x2; w1 = w2;
      x2 = x3; w2 = w3;
      ++e;
    }
  }
  wait_vm();

  if (!wave_keys) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t off = out_off(mb, nb);
      const f32x4_t kv = accK[mb][nb], vv = accV[mb][nb];
      if (IO == 1) {   // float32 partial sums (dK unscaled), summed by bwd_reduce_kernel
        *(f32x4_t*)(pK + off) = kv;
        *(f32x4_t*)(pV + off) = vv;
      } else {
        store4_bf16(dK + off, kv[0] * d.scale, kv[1] * d.scale, kv[2] * d.scale, kv[3] * d.scale);
        store4_bf16(dV + off, vv[0], vv[1], vv[2], vv[3]);
      }
    }
}

// dK = scale (sum_j pK[j] + sum_h sK[h]), dV = sum_j pV[j] + sum_h sV[h] in
// bfloat16, four elements per thread; pK / pV hold the npk head-group slots
// of the full-stream pass (npk may be 0). Slots are added in ascending
// order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ pK,
                                                         const float* __restrict__ pV, int npk,
                                                         const float* __restrict__ sK,
                                                         const float* __restrict__ sV, int G,
                                                         size_t n4, float scale,
                                                         uint16_t* __restrict__ dK,
                                                         uint16_t* __restrict__ dV) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4_t k = f32x4_t{0.f, 0.f, 0.f, 0.f}, v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < npk; ++j) {
    k += ((const f32x4_t*)pK)[(size_t)j * n4 + i];
    v += ((const f32x4_t*)pV)[(size_t)j * n4 + i];
  }
  for (int h = 0; h < G; ++h) {
    k += ((const f32x4_t*)sK)[(size_t)h * n4 + i];
    v += ((const f32x4_t*)sV)[(size_t)h * n4 + i];
  }
  store4_bf16(dK + 4 * i, k[0] * scale, k[1] * scale, k[2] * scale, k[3] * scale);
  store4_bf16(dV + 4 * i, v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- dQ
// One workgroup per (b, q head, 128-row query tile); four waves of 32 rows.
// Q and both upstream gradients of the wave's rows stay in registers; per
// 32-key step, S^T = K Q^T and dP^T = V dO^T from LDS tiles of K and V, then
// dQ^T += K^T dS^T with K^T read from the K tile by transpose reads. The
// selection bits of the workgroup's rows are built in LDS from idx at the
// start. Workgroups are ordered heaviest first, the q heads of one kv head
// next to each other.
template <int D, int MODE, int IO, bool TOK>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ GF, const uint16_t* __restrict__ GS,
    const float* __restrict__ stats, const int* __restrict__ idx, const int* __restrict__ cnt,
    const uint64_t* __restrict__ rowbits, uint16_t* __restrict__ dQ, float* __restrict__ pQ,
    Dims d, HeadMap hm, int nKT) {
  constexpr int SPR = D / 8;
  constexpr int KK = D / 32;
  constexpr int MB = D / 16;
  constexpr int TILE = kStep * D;
  constexpr int CT = kStep * SPR / 4 / 64;   // copy instructions per tile per wave
  constexpr int CPS = 2 * CT;                 // per key step per wave
  __shared__ __align__(16) uint16_t sK[kStages][TILE], sV[kStages][TILE];
  __shared__ uint32_t sNib[kMaxSteps / 2];   // 16 bits per key step: nibble w for wave w
  constexpr uint32_t TB = TILE * 2u;
  const uint32_t aK = lds_u32(&sK[0][0]), aV = lds_u32(&sV[0][0]);

  constexpr bool has_full = MODE != 2, has_sparse = MODE != 1;
  const int nBG = d.B * d.Hkv;
  const int nQT = (d.Nq + kRowsPerWg - 1) / kRowsPerWg;
  const int bg = blockIdx.x % nBG;
  const int hi = (blockIdx.x / nBG) % d.G;
  const int qt = nQT - 1 - (int)(blockIdx.x / (nBG * d.G));   // heaviest first
  const int b = bg / d.Hkv, g = bg % d.Hkv;
  const int h = hm.q_of_kv[g * d.G + hi];
  const size_t bh = (size_t)b * d.Hq + h;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    if (TOK && wave_rows) {   // per-token lists: any row of each 16-row half
      for (int j = 0; j < kStep; ++j) {
        const int row = r0w + j;
        const size_t lr = bh * d.nL + row;
        const int* list = idx + lr * d.budget;
        const int cn = min(max(cnt[lr], 0), d.budget);
        const int diag = row / d.bs;
        for (int e = lane; e < cn; e += 64) {
          const int kb = list[e];
          if (kb < 0 || kb > diag) continue;
          if (d.bs == 16) {
            const int t = kb >> 1;
            const uint32_t bit = 1u << (2 * (j >> 4) + (kb & 1));
            atomicOr(&sNib[t >> 1], bit << (16 * (t & 1) + 4 * w));
          } else {
            for (int t = 2 * kb; t < 2 * kb + 2; ++t)
              atomicOr(&sNib[t >> 1], (3u << (2 * (j >> 4))) << (16 * (t & 1) + 4 * w));
          }
        }
      }
    } else if (wave_rows) {
      const int nq = d.bs == 16 ? 2 : 1;
      for (int qs = 0; qs < nq; ++qs) {
        const int qb = d.bs == 16 ? r0w / 16 + qs : r0w / 64;
        const int* list = idx + (bh * d.nQB + qb) * d.budget;
        const int cn = min(max(cnt[bh * d.nQB + qb], 0), d.budget);
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
  bf16x8_t qreg[2][KK], freg[has_full ? 2 : 1][KK], sreg[has_sparse ? 2 : 1][KK];
  float lf[2], dfv[2], ls[2], dsv_[2];
  {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = wave_rows ? r0w + 16 * nb + n : 0;
      const size_t base = (bh * d.Nq + row) * D + 8 * gq;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        qreg[nb][kk] = *(const bf16x8_t*)(Q + base + 32 * kk);
        if (has_full) freg[nb][kk] = *(const bf16x8_t*)(GF + base + 32 * kk);
        if (has_sparse) sreg[nb][kk] = *(const bf16x8_t*)(GS + base + 32 * kk);
      }
      const float* st = stats + ((bh * nS + row / kStep) * 4) * kStep + row % kStep;
      lf[nb] = st[0];
      dfv[nb] = st[kStep];
      ls[nb] = st[2 * kStep];
      dsv_[nb] = st[3 * kStep];
    }
  }
  auto out_off = [&](int mb, int nb) {
    return (bh * d.Nq + r0w + 16 * nb + n) * D + 16 * mb + 4 * gq;
  };
  f32x4_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      acc[mb][nb] = (IO == 2 && wave_rows) ? *(const f32x4_t*)(pQ + out_off(mb, nb))
                                           : f32x4_t{0.f, 0.f, 0.f, 0.f};

  const size_t bgk = (size_t)bg;
  const uint32_t kv_bytes = (uint32_t)d.Nk * D * 2u;
  const i32x4_t rk = make_rsrc_words(K + bgk * d.Nk * D, kv_bytes);
  const i32x4_t rv = make_rsrc_words(V + bgk * d.Nk * D, kv_bytes);

  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)t * kStep * D * 2u;
    copy_tile<SPR>(rk, toff, aK + st * TB, w, lane);
    copy_tile<SPR>(rv, toff, aV + st * TB, w, lane);
  };

  // No early exit and no branch around the dQ update: keys after the rows
  // (and rows past the end) get dS = 0 from the mask, so the loop-carried
  // accumulators never pass through a control-flow merge.
  auto compute = [&](int t, int st) __attribute__((always_inline)) {
    const int rel = r0w - kStep * t;   // row position minus key position of (0, 0)
    const uint32_t nib = (step_bits(t) >> (4 * w)) & 0xFu;
    const bool sp = nib != 0;
    // per-token lists: bits of the lane's rows 16*nb + n in its key half
    uint32_t rsel = 0u;
    if (TOK && has_sparse) {
      const int sw = min(r0w / kStep, nS - 1);
      const uint64_t rm = rowbits[(((size_t)bg * nKT + (t >> 2)) * nS + sw) * d.G * 4 + (size_t)hi * 4 + (t & 3)];
      rsel = (uint32_t)(rm >> (32 * (gq >> 1) + n));
    }
    // the dP accumulators start at -D_r of their query (the lane's column)
    f32x4_t sa[2][2], pf[2][2], ps[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        sa[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pf[mb][nb] = has_full ? f32x4_t{-dfv[nb], -dfv[nb], -dfv[nb], -dfv[nb]} : sa[mb][nb];
        ps[mb][nb] = (has_sparse && sp) ? f32x4_t{-dsv_[nb], -dsv_[nb], -dsv_[nb], -dsv_[nb]} : sa[mb][nb];
      }
    {
      bf16x8_t fr[4 * KK];   // K and V fragments, read ahead of their MFMAs
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          fr[2 * (2 * kk + mb)] = frag_rows<SPR>(aK + st * TB, rho(mb, n), 4 * kk + gq);
          fr[2 * (2 * kk + mb) + 1] = frag_rows<SPR>(aV + st * TB, rho(mb, n), 4 * kk + gq);
        }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int i = 2 * (2 * kk + mb);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) sa[mb][nb] = mfma16(fr[i], qreg[nb][kk], sa[mb][nb]);
          if (has_full) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) pf[mb][nb] = mfma16(fr[i + 1], freg[nb][kk], pf[mb][nb]);
          }
        }
      if (has_sparse && sp) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              ps[mb][nb] = mfma16(fr[2 * (2 * kk + mb) + 1], sreg[nb][kk], ps[mb][nb]);
      }
      pipeline_mix<4 * KK, 2, 6>();
      __builtin_amdgcn_sched_barrier(0);
    }
    float xd[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bool sel = TOK ? ((rsel >> (16 * nb)) & 1u) != 0u
                           : ((nib >> (2 * nb + (gq >> 1))) & 1u) != 0u;   // per lane
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool keep = wave_rows && 8 * gq + 4 * mb + i <= rel + 16 * nb + n;   // key <= row
          float dsv = 0.f;
          if (has_full) {
            float p = fast_exp2(fmaf(sa[mb][nb][i], sl2, -lf[nb]));
            p = keep ? p : 0.f;
            dsv = p * pf[mb][nb][i];
          }
          if (has_sparse && sp) {   // wave-uniform branch; the lane's own bit masks
            float q = fast_exp2(fmaf(sa[mb][nb][i], sl2, -ls[nb]));
            q = (keep && sel) ? q : 0.f;
            dsv = fmaf(q, ps[mb][nb][i], dsv);
          }
          xd[nb][4 * mb + i] = dsv;
        }
    }
    bf16x8_t bD[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bD[nb] = pack8(xd[nb]);
    __builtin_amdgcn_sched_barrier(0);
    {
      bf16x8_t tr[MB];   // K^T fragments by transpose reads of the K tile
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) tr[mb] = frag_tr<SPR>(aK + st * TB, 16 * mb, lane);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma16(tr[mb], bD[nb], acc[mb][nb]);
      pipeline_mix<2 * MB, 1, 8>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // key steps t0 (current) .. t3; copies run three steps ahead
  auto next = [&](int t) { return has_full ? t + 1 : next_selected(t, nT, lane, step_bits); };
  int t0 = has_full ? 0 : next_selected(-1, nT, lane, step_bits);
  int t1 = t0 < nT ? next(t0) : nT;
  int t2 = t1 < nT ? next(t1) : nT;
  if (t0 < nT) {
    issue(t0, 0);
    if (t1 < nT) issue(t1, 1);
    if (t2 < nT) issue(t2, 2);
    int e = 0;
    while (true) {
      const int t3 = t2 < nT ? next(t2) : nT;
      if (t2 < nT) wait_vm_n<2 * CPS>();
      else if (t1 < nT) wait_vm_n<CPS>();
      else wait_vm();
      __syncthreads();
      if (t3 < nT) issue(t3, (e + 3) % kStages);
      compute(t0, e % kStages);
      if (t1 >= nT) break;
      t0 = t1;
      t1 = t2;
      t2 = t3;
      ++e;
    }
  }
  wait_vm();

  if (!wave_rows) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t off = out_off(mb, nb);
      const f32x4_t a = acc[mb][nb];
      if (IO == 1) *(f32x4_t*)(pQ + off) = a;   // unscaled partial sums for the sparse pass
      else store4_bf16(dQ + off, a[0] * d.scale, a[1] * d.scale, a[2] * d.scale, a[3] * d.scale);
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
  const int lr = row / d.lrows;   // this row's selection list
  const int* list = idx + (bh * d.nL + lr) * d.budget;
  const int ncnt = min(max(cnt[bh * d.nL + lr], 0), d.budget);
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
      const int lr = row / d.lrows;
      const bool sel = GS != nullptr &&
                       block_selected(idx + (bh * d.nL + lr) * d.budget,
                                      min(max(cnt[bh * d.nL + lr], 0), d.budget), kb);
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

int bwd_full_split(const Dims& d) {
  // fewest head groups that give the full-stream dK/dV pass at least
  // kBwdMinWorkgroups workgroups (the heaviest tile then holds 1/hs of the
  // work it would alone)
  const long pairs = (long)bwd_key_tiles(d) * d.B * d.Hkv;
  for (int hs = 1; hs < d.G; ++hs)
    if (d.G % hs == 0 && pairs * hs >= kBwdMinWorkgroups) return hs;
  return d.G;
}

hipError_t launch_attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* gf, const uint16_t* gs, const int* idx,
                                const int* cnt, const float* stats, uint16_t* bits,
                                uint64_t* rowbits, float* pq,
                                float* pk, float* pv, float* sk, float* sv, uint16_t* dq,
                                uint16_t* dk, uint16_t* dv, const Dims& d, const HeadMap& hm,
                                hipStream_t stream) {
  const int nKT = bwd_key_tiles(d);
  if (gs != nullptr) {
    const long threads = (long)d.B * d.Hq * (d.Nq / kStep);
    hipLaunchKernelGGL(bwd_bits_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, idx, cnt, bits, rowbits, d, hm, nKT);
  }
  const dim3 g1((unsigned)(nKT * d.B * d.Hkv));
  const int nQT = (d.Nq + kRowsPerWg - 1) / kRowsPerWg;
  const dim3 g2((unsigned)(nQT * d.B * d.Hq));
  // the full-stream pass never reads the selection; the sparse-stream
  // kernels come in a per-block and a per-token (per-row masks) form
#define SSA_DKDV_T(DD, MM, IO, TK, PK, PV, GRID, HS)                                         \
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DD, MM, IO, TK>), GRID, dim3(256), 0, stream, q, k, \
                     v, gf, gs, stats, bits, rowbits, dk, dv, PK, PV, d, hm, nKT, HS)
#define SSA_DQ_T(DD, MM, IO, TK)                                                             \
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DD, MM, IO, TK>), g2, dim3(256), 0, stream, q, k, v,  \
                     gf, gs, stats, idx, cnt, rowbits, dq, pq, d, hm, nKT)
#define SSA_DKDV(DD, MM, IO, PK, PV, GRID, HS)                                               \
  if (MM == 2 && d.tok) { SSA_DKDV_T(DD, MM, IO, true, PK, PV, GRID, HS); }                  \
  else { SSA_DKDV_T(DD, MM, IO, false, PK, PV, GRID, HS); }
#define SSA_DQ(DD, MM, IO)                                                                   \
  if (MM == 2 && d.tok) { SSA_DQ_T(DD, MM, IO, true); } else { SSA_DQ_T(DD, MM, IO, false); }
  // Both streams: a full-stream pass leaves float32 partial sums, a
  // sparse-stream pass over the selected blocks only adds to them and rounds.
  // The sparse dK/dV pass runs per (tile, q head) into per-head slots.
  const dim3 g1s((unsigned)(nKT * d.B * d.Hkv * d.G));
  // the full-stream pass in hs head groups (one float32 slot each)
  const int hs = bwd_full_split(d);
  const dim3 g1f((unsigned)(nKT * d.B * d.Hkv * hs));
#define SSA_PASSES(DD)                                                                       \
  if (gf != nullptr && gs != nullptr) {                                                      \
    SSA_DKDV(DD, 1, 1, pk, pv, g1f, hs); SSA_DKDV(DD, 2, 1, sk, sv, g1s, d.G);               \
    SSA_DQ(DD, 1, 1); SSA_DQ(DD, 2, 2);                                                      \
  } else if (gs == nullptr) {                                                                \
    if (hs == 1) { SSA_DKDV(DD, 1, 0, pk, pv, g1, 1); }                                      \
    else { SSA_DKDV(DD, 1, 1, pk, pv, g1f, hs); }                                            \
    SSA_DQ(DD, 1, 0);                                                                        \
  } else {                                                                                   \
    SSA_DKDV(DD, 2, 1, sk, sv, g1s, d.G); SSA_DQ(DD, 2, 0);                                  \
  }
  if (d.D == 128) {
    SSA_PASSES(128)
  } else {
    SSA_PASSES(64)
  }
  if (gs != nullptr || hs > 1) {
    const size_t n4 = (size_t)d.B * d.Hkv * d.Nk * d.D / 4;
    const int npk = gf != nullptr ? hs : 0;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                       stream, pk, pv, npk, sk, sv, gs != nullptr ? d.G : 0, n4, d.scale, dk, dv);
  }
#undef SSA_PASSES
#undef SSA_DKDV
#undef SSA_DQ
#undef SSA_DKDV_T
#undef SSA_DQ_T
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

// Host-side launchers of the SSA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssa_common.h"

namespace ssa {

constexpr int kMaxKeyBlocks = 4096;        // Nk <= 262144 tokens
constexpr size_t kSelKeyBytes = 32 * 1024; // LDS for the selection keys

// Decode split-KV geometry: each wave walks kDecWaveBlocks key blocks, a
// workgroup has kDecWaves waves.
constexpr int kDecWaves = 4;
constexpr int kDecWaveBlocks = 8;
constexpr int kDecSparseParts = 2;         // workgroups per (b, kv head), sparse-only
constexpr int kDecMaxGroup = 8;            // q heads per bf16 decode workgroup (larger groups split)

inline int decode_splits(int nKB) {        // partial results per (b, q head), dual mode
  const int per_wg = kDecWaves * kDecWaveBlocks;
  return (nKB + per_wg - 1) / per_wg;
}
inline int decode_partial_floats(int D) { return 2 * D + 4; }

hipError_t launch_pool(const void* x, bool bf16, float* out, long nblk_total, int bs, int D,
                       hipStream_t stream);
// Prefill: pooled queries qbar, scores computed inside the selection kernel.
hipError_t launch_select(const float* qbar, const float* kbar, int* idx, int* cnt,
                         const Dims& d, const HeadMap& hm, hipStream_t stream);
// Decode: the query q itself (bf16 or float32) is scored by a wide kernel
// into the [B, Hq, nKB] key scratch gkeys, then one wave per (b, q head)
// selects.
hipError_t launch_select_decode(const void* q, bool bf16, const float* kbar, int* idx, int* cnt,
                                const Dims& d, const HeadMap& hm, uint64_t* gkeys,
                                hipStream_t stream);
// Per-token selection: float64 copy of the pooled keys in chunks of
// kTokChunk blocks ([B*Hkv][chunk][D][kTokChunk]), read as scalar operands.
constexpr int kTokChunk = 16;
inline size_t tok_kc_bytes(const Dims& d) {
  const size_t chunks = (size_t)(d.nKB + kTokChunk - 1) / kTokChunk;
  return (size_t)d.B * d.Hkv * chunks * kTokChunk * d.D * sizeof(double);
}
hipError_t launch_select_tok(const void* q, bool bf16, const float* kbar, double* kc, int* idx,
                             int* cnt, const Dims& d, const HeadMap& hm, hipStream_t stream);
// Also zeroes the prefill work queues (kNumXcd counters) when queues != NULL,
// and when kn != NULL writes kn[bh][n / 64], the largest L2 norm of the 64
// keys of each block of k ([BH, N, D] bf16), for prefill_key_norms.
// blk16: the layout of prefill_vt_blk16 problems ([n/16][d][n%16] per head).
hipError_t launch_transpose(const uint16_t* v, uint16_t* vt, int BH, int N, int D, int* queues,
                            bool blk16, const uint16_t* k, float* kn, hipStream_t stream);
// The grouped dual-stream prefill kernels bound each key block's logits by
// their queries' norms times the block's largest key norm (from the
// transpose) and skip the block maximum when the bound cannot trigger a
// rescale.
inline bool prefill_key_norms(const Dims& d, bool sparse_only) {
  return d.G % 4 == 0 && !sparse_only && !d.tok &&
         ((d.D == 128 && d.bs != 16) || (d.D == 64 && d.bs == 16));
}
// Sparse-only prefill with 16-token per-block lists runs the gather kernel,
// which reads V^T one 16-key block at a time: contiguous per block.
inline bool prefill_vt_blk16(const Dims& d, bool sparse_only) {
  return sparse_only && d.bs == 16 && !d.tok;
}

// queues: kNumXcd zeroed counters (see launch_transpose), or NULL for a
// static workgroup-to-tile mapping.
// kn: the transpose's key-block norms when prefill_key_norms(d, hf == NULL).
hipError_t launch_attn_prefill_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                                    const int* idx, const int* cnt, uint16_t* hf, uint16_t* hs,
                                    float* delta, float* lse, int* queues, const float* kn,
                                    const Dims& d, const HeadMap& hm, hipStream_t stream);
hipError_t launch_attn_rows_f32(const float* q, const float* k, const float* v, const int* idx,
                                const int* cnt, float* hf, float* hs, float* delta, float* lse,
                                const Dims& d, const HeadMap& hm, hipStream_t stream);
hipError_t launch_attn_decode_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int* idx, const int* cnt, uint16_t* hf, uint16_t* hs,
                                   float* delta, float* lse, float* partials, const Dims& d,
                                   const HeadMap& hm, hipStream_t stream);
hipError_t launch_align_loss(const void* hf, const void* hs, bool bf16, long n, float* loss,
                             void* gf, void* gs, double* partials, hipStream_t stream);
constexpr int kLossPartials = 1024;
long align_loss_partials(long n);   // float64 partials the loss kernels use for n elements

// Backward pass (ssa_attn_backward.hip).
int bwd_key_tiles(const Dims& d);   // 128-key tiles of the dK/dV kernel
// Head groups of the full-stream dK/dV pass (a divisor of G; its float32
// partial-sum slots in the backward workspace).
constexpr long kBwdMinWorkgroups = 4096;
int bwd_full_split(const Dims& d);
hipError_t launch_attn_bwd_stats(const void* hf, const void* hs, const void* gf, const void* gs,
                                 const float* lse, float* stats, bool bf16, const Dims& d,
                                 hipStream_t stream);
hipError_t launch_attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* gf, const uint16_t* gs, const int* idx,
                                const int* cnt, const float* stats, uint16_t* bits,
                                uint64_t* rowbits, float* pq,
                                float* pk, float* pv, float* sk, float* sv, uint16_t* dq,
                                uint16_t* dk, uint16_t* dv, const Dims& d, const HeadMap& hm,
                                hipStream_t stream);
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* gf,
                               const float* gs, const int* idx, const int* cnt,
                               const float* stats, float* dq, float* dk, float* dv,
                               const Dims& d, const HeadMap& hm, hipStream_t stream);

}  // namespace ssa

// Shared device-side definitions of the SSA HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;      // tokens per key tile / query tile of the attention kernels
constexpr int kMaxHq = 256;
constexpr int kMaxGroup = 16;   // q heads per kv head
constexpr int kTokMaxBudget = 64;  // list length limit of per-token selection
// Work queues of the grouped prefill kernels: one counter per XCD, each on
// its own 256-byte line of the workspace.
constexpr int kNumXcd = 8;
constexpr int kQueueStride = 64;   // ints between two counters
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Problem sizes as the kernels see them.
struct Dims {
  int B, Hq, Hkv, Nq, Nk, D;
  int budget, n_sink, n_local;
  int nQB, nKB, G;     // query row blocks, key blocks (of bs tokens), q heads per kv head
  int bs;              // selection block size in tokens (16 or 64)
  int nQT, nT;         // 64-row query tiles (1 in decode) and 64-key tiles
  int group_select;    // 1: one selection per GQA group (summed head scores)
  int tok;             // 1: one selection list per query row (prefill)
  int nL;              // selection lists per (b, q head): nQB, or Nq per token
  int lrows;           // query rows per selection list: bs, or 1 per token
  float scale;         // logit scale
  float scale_log2;    // scale * log2(e)
};

// GQA head map: kv head of every q head, and the q heads of every kv head
// (kv head g owns q_of_kv[g*G .. g*G+G-1]).
struct HeadMap {
  uint8_t kv_of_q[kMaxHq];
  uint8_t q_of_kv[kMaxHq];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float load_as_f32(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_as_f32(const float* p) { return *p; }

// Key block holding the last query of row block qb (queries are aligned to
// the end of the keys).
__device__ __forceinline__ int row_block_diag(const Dims& d, int qb) {
  return (d.Nq == d.Nk) ? qb : (d.Nk - 1) / d.bs;
}

// XCD-aware remap of a linear workgroup id: workgroups are dispatched
// round-robin over the 8 XCDs, so id i runs on XCD i % 8. Giving each XCD a
// contiguous range of logical ids keeps work that shares K/V (neighbouring
// logical ids) inside one XCD's L2. Identity when the count is not a
// multiple of 8.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  if (total & 7) return id;
  const int per = total >> 3;
  return (id & 7) * per + (id >> 3);
}

}  // namespace ssa

// Rotary prologue: YaRN-scaled RoPE on the 64 rotary dims of the new tokens.
// The "Similarities" page ("Query-key similarity") rotates q_pe and k_pe with
// a cos/sin table built for kv_seq_len positions and picked by position before
// they join the non-rotary parts; the released configuration gives theta and
// the "yarn" scaling. Pair i = dims (2i, 2i+1) turns by pos * w_i', with
// w_i = theta^(-2i/64) (RoPE, Su et al.) and w_i' scaled per pair as YaRN
// (Peng et al.) does: pairs that complete at least beta_fast turns within the
// original context keep w_i, pairs with fewer than beta_slow turns run factor
// times slower, and the ones between blend linearly in the number of turns.
//
// Two kernels:
//  * mla_rope_table_kernel: one thread per (position, pair); the frequency,
//    the angle and its cosine and sine are computed in fp64 and stored as
//    fp32, 256 bytes per position. Built once per model and context length.
//  * mla_rope_apply_kernel: rotates bf16 rows [B, R, T, 64] in place (R = H for
//    q_pe, 1 for the shared k_pe), optionally followed in the same launch by
//    the new keys' rows [B, 1, T, 64] (the pages rotate the query and the key
//    in one call). A quarter-wave covers one 128-byte row:
//    lane l holds dims 4l..4l+3 (pairs 2l and 2l+1) and loads the matching
//    16 bytes of the table row, so every pair turns inside one lane's
//    registers (fp32 arithmetic, round-to-nearest-even bf16 result). Each
//    thread takes five rows, all loads first. Bound by HBM: each row is read
//    and written once, with non-temporal loads and stores (4% faster than
//    plain ones on 2048 new tokens); a position's table row serves every
//    head and is served from L2 after the first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPairs = 32;
constexpr int kRowsPerThread = 5;   // measured: 4 → 10.97 µs, 5 → 9.60, 6 → 10.02, 8 → 11.09 on 2048 new tokens
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 16 * kRowsPerThread;  // 80

__global__ __launch_bounds__(kThreads) void mla_rope_table_kernel(RopeTableArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)a.max_pos * kPairs) return;
  const int pair = (int)(idx % kPairs);
  const int64_t pos = idx / kPairs;
  double w = pow(a.theta, -2.0 * pair / 64.0);
  if (a.factor != 1.0) {
    const double turns = (double)a.original_max_position * w / (2.0 * M_PI);
    double g;
    if (turns >= a.beta_fast) g = 1.0;
    else if (turns < a.beta_slow) g = 0.0;
    else g = (turns - a.beta_slow) / (a.beta_fast - a.beta_slow);
    w = g * w + (1.0 - g) * w / a.factor;
  }
  double sn, cs;
  sincos((double)pos * w, &sn, &cs);
  float* dst = a.table + idx * 2;
  dst[0] = (float)cs;
  dst[1] = (float)sn;
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ uint32_t to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__global__ __launch_bounds__(kThreads) void mla_rope_apply_kernel(RopeApplyArgs a) {
  const int lane16 = threadIdx.x & 15;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  u32x2 xv[kRowsPerThread];
  f32x4 cs[kRowsPerThread];
  uint16_t* ptr[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int64_t row = row0 + (int64_t)u * (kThreads / 16);
    if (row >= a.rows) continue;
    // rows of x first ([B, R, T]), then those of x2 ([B, 1, T])
    const bool second = row >= a.rows1;
    const int64_t r = second ? row - a.rows1 : row;
    const int64_t t = r % a.T;
    const int64_t b = r / ((second ? 1 : (int64_t)a.R) * a.T);
    int64_t pos = (a.past_lens != nullptr ? (int64_t)a.past_lens[b] : (int64_t)a.past_len) + t;
    pos = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);  // never leave the table
    ptr[u] = (second ? a.x2 : a.x) + r * 64 + 4 * lane16;
    xv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(ptr[u]));  // streamed once
    cs[u] = *reinterpret_cast<const f32x4*>(a.table + pos * (2 * kPairs) + 4 * lane16);
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int64_t row = row0 + (int64_t)u * (kThreads / 16);
    if (row >= a.rows) continue;
    const float x0 = lo_bf16(xv[u][0]), y0 = hi_bf16(xv[u][0]);
    const float x1 = lo_bf16(xv[u][1]), y1 = hi_bf16(xv[u][1]);
    const float c0 = cs[u][0], s0 = cs[u][1], c1 = cs[u][2], s1 = cs[u][3];
    u32x2 w;
    w[0] = to_bf16(x0 * c0 - y0 * s0) | (to_bf16(x0 * s0 + y0 * c0) << 16);
    w[1] = to_bf16(x1 * c1 - y1 * s1) | (to_bf16(x1 * s1 + y1 * c1) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(ptr[u]));
  }
}

}  // namespace

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.max_pos * kPairs;
  const int64_t grid = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(mla_rope_table_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_apply(const RopeApplyArgs& a, hipStream_t stream) {
  const int64_t grid = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(mla_rope_apply_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

// Measurement probes used by the benchmark to put the attention kernels'
// figures next to what this GPU reaches on the simplest work of the same
// kind. Not part of the attention ABI (include/mla_attn.h); built into its own
// library, libmla_probe.so.
//
//  * mla_probe_stream_read: a plain read of a device buffer (16-byte loads,
//    all issued before any is used, optionally non-temporal like the decode's
//    key and value loads); nothing is written unless a checksum hits one
//    fixed value. Timed over the decode's byte counts, it is the floor a
//    single launch that streams the same bytes cannot beat.
//  * mla_probe_mfma: chains of v_mfma_f32_32x32x16_bf16 (the prefill's
//    instruction) on operands that differ from one MFMA to the next, four
//    independent accumulators per wave, two waves per SIMD, optionally with
//    softmax-like VALU work (an exp2 and FMAs) between the MFMAs. Every wave
//    reads the shader-clock counter (s_memtime) and the 100 MHz real-time
//    counter (s_memrealtime) before and after its chain, so the host can tell
//    the clock the chip held while it ran.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr uint32_t kNeverSum = 0x9e3779b9u;  // the sink is written only on this checksum

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                   int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  // kReadUnroll loads per thread per pass, all issued before any is used;
  // those past the end are predicated off
  for (int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = i + u * stride < n16 ? load16<NT>(src + i + u * stride) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == kNeverSum) sink[blockIdx.x] = acc;
}

constexpr int kMfmaThreads = 256;  // four waves, one per SIMD
constexpr int kChains = 4;         // independent accumulators per wave

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// VALU: 0 for bare MFMA chains; 1 for one exp2 and four FMAs per MFMA (the
// prefill softmax's mix per score tile, spread over its MFMAs).
template <int VALU>
__global__ __launch_bounds__(kMfmaThreads, 2) void mfma_probe_kernel(const u32x4* __restrict__ operands,
                                                                     int iters, float* __restrict__ out,
                                                                     unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  // eight operand fragments per lane, random bf16 drawn by the host
  bf16x8 f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = __builtin_bit_cast(bf16x8, operands[k * 64 + lane]);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  float x0 = 0.25f + lane * 1e-3f, x1 = 0.5f, x2 = 0.75f, x3 = 1.0f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  // unrolled by eight so every fragment index is a constant (the fragments
  // stay in registers)
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      // A and B change from one MFMA to the next (and across iterations)
      acc[c] = mfma(f[(j + c) & 7], f[(j + 2 * c + 3) & 7], acc[c]);
      if constexpr (VALU == 1) {
        x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0, -0.75f, 0.1f));
        x1 = __builtin_fmaf(x1, 0.999f, x0);
        x2 = __builtin_fmaf(x2, 0.998f, x1);
        x3 = __builtin_fmaf(x3, 0.997f, x2);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = x3;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from `src` (16-byte aligned device memory)
// on `stream` with `grid` workgroups of 256 threads; `sink` must hold `grid`
// uint32 (written only on one checksum value). nontemporal != 0 sets the
// non-temporal bit on every load. Returns a hipError_t value (0 = launched).
int mla_probe_stream_read(const void* src, int64_t bytes, void* sink, int grid, int nontemporal,
                          void* stream) {
  if (src == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || grid < 1 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(grid), dim3(kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n16,
                       static_cast<uint32_t*>(sink));
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(grid), dim3(kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n16,
                       static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `grid` workgroups of four waves, each wave running `iters` (a multiple of
// 8) iterations of four MFMAs (32x32x16 bf16, 32768 flops each). operands: 8 * 64 16-byte
// fragments (8 KiB, random bf16, device memory); out: grid * 256 floats;
// clocks: grid * 2 uint64 (shader-clock ticks, 100 MHz ticks) per
// workgroup. valu: 0 or 1 (see mfma_probe_kernel).
int mla_probe_mfma(const void* operands, int grid, int iters, int valu, void* out, void* clocks,
                   void* stream) {
  if (operands == nullptr || out == nullptr || clocks == nullptr || grid < 1 || iters < 8 || iters % 8 != 0 ||
      (valu != 0 && valu != 1))
    return (int)hipErrorInvalidValue;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* ops = static_cast<const u32x4*>(operands);
  float* o = static_cast<float*>(out);
  unsigned long long* c = static_cast<unsigned long long*>(clocks);
  if (valu)
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(grid), dim3(kMfmaThreads), 0, s, ops, iters, o, c);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(grid), dim3(kMfmaThreads), 0, s, ops, iters, o, c);
  return (int)hipGetLastError();
}

}  // extern "C"

// Decode over the compressed (latent) key-value cache.
//
// The attention of the Kimi K2 pages ("Similarities" page, "Query-key
// similarity") with its keys and values kept in the form the joint key-value
// down-projection produces ("Scale scores": a 512-dim latent per token, plus
// the one rotary key shared by all heads). kv_b_proj (no bias) expands the
// latent into each head's 128 non-rotary key dims and 128 value dims. Because
// that expansion is linear, it is folded into the query before attention and
// into the output after it:
//   q~[h]   = W_k[h]^T q_nope[h]                      (512 dims)
//   s[h,j]  = q~[h] . c[j] + q_pe[h] . k_pe[j]         (one 576-dim key shared by all heads)
//   o~[h]   = sum_j softmax_j(scale * s[h,j]) c[j]      (512 dims)
//   out[h]  = W_v[h] o~[h]                             (128 dims)
// which equals attention over the decompressed keys and values up to rounding.
// A key costs 1152 bytes (latent + rotary key) instead of 64 heads x 512.
//
// Four kernels on the caller's stream:
//  1. absorb: q~ for every (batch, head), rounded to bf16, joined with q_pe
//     into a 576-dim row (workspace).
//  2. attention: one workgroup per (batch, key split) with one wave per 16
//     heads. 32-key tiles of [latent | k_pe] (36 KiB) are copied straight from
//     HBM into LDS (buffer_load ... lds, double-buffered), in 64-byte column
//     blocks with row-swizzled 16-byte chunks. Scores use
//     v_mfma_f32_16x16x32_bf16 with keys as rows and the wave's 16 heads as
//     columns (S^T = K Q~^T, 18 K-steps); online softmax in fp32 per head; the
//     latent output uses O~^T = C^T P^T, 32 tiles of 16 latent dims, whose
//     C^T fragments come from ds_read_b64_tr_b16 in the key order the score
//     accumulator leaves P in. Each split writes an fp32 partial (o~, max, sum).
//  3. merge: log-sum-exp over the splits of each (batch, head) -> o~ (fp32).
//  4. up-projection: out = W_v o~, rounded to bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int R = 512;                       // latent dims (kv_lora_rank)
constexpr int DR = 64;                       // rotary dims
constexpr int KW = R + DR;                   // 576: joined key width
constexpr int DN = 128, DV = 128;            // non-rotary query dims, value dims
constexpr int KVB = DN + DV;                 // kv_b_proj rows per head
constexpr int BN = 32;                       // keys per tile
constexpr int CB_BYTES = BN * 64;            // one 64-byte column block of a tile
constexpr int LAT_BLOCKS = R * 2 / 64;       // 16 column blocks of latent
constexpr int TILE_BYTES = KW * 2 / 64 * CB_BYTES;  // 18 blocks: 36 KiB
constexpr int COPIES = TILE_BYTES / 1024;    // 36 one-KiB copies per tile
constexpr int LAT_COPIES = LAT_BLOCKS * CB_BYTES / 1024;  // 32 of them latent
constexpr int KSTEPS = KW / 32;              // 18 score K-steps
constexpr int NDT = R / 16;                  // 32 latent-output tiles of 16 dims

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_tr_read(const char* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Sum over the 16 lanes of a row; every lane gets the total.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// ---- 1. absorb: q~[b,h,e] = sum_d q_nope[b,h,d] * W[256h + d, e]; q~[b,h,512+i] = q_pe[b,h,i]
__global__ __launch_bounds__(256) void latent_absorb_kernel(LatentArgs a) {
  const int h = blockIdx.x >> 3, chunk = blockIdx.x & 7;
  const int e = chunk * 64 + (threadIdx.x & 63);
  const uint16_t* wk = a.w_kv_b + (int64_t)h * KVB * R + e;  // W[256h + d, e] = wk[d * R]
  for (int b = threadIdx.x >> 6; b < a.B; b += 4) {
    const uint16_t* q = a.q_nope + ((int64_t)b * a.H + h) * DN;
    float acc = 0.0f;
#pragma unroll 8
    for (int d = 0; d < DN; ++d) acc = __builtin_fmaf(bf16_to_f32(q[d]), bf16_to_f32(wk[(int64_t)d * R]), acc);
    uint16_t* dst = a.qt + ((int64_t)b * a.H + h) * KW;
    dst[e] = f32_to_bf16(acc);
    if (chunk == 0) dst[R + (threadIdx.x & 63)] = a.q_pe[((int64_t)b * a.H + h) * DR + (threadIdx.x & 63)];
  }
}

// Buffer resource over rows [kb, S) of one sequence's row-major [S, rowbytes/2]
// bf16 tensor; rows past the end read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* seq, int64_t kb,
                                                           int64_t S, int rowbytes) {
  const int64_t left = S - kb;
  const int records = left > 0 ? (int)(left * rowbytes) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)seq + kb * rowbytes), (short)0,
                                           records, 0x00020000);
}

// ---- 2. attention over the latent keys of one key split
template <int NWV>  // waves per workgroup: one per 16 heads
__device__ __forceinline__ void latent_attn(const LatentArgs& a) {
  __shared__ __attribute__((aligned(1024))) char tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile1[TILE_BYTES];
  constexpr int NCOPY = COPIES / NWV;
  static_assert(COPIES % NWV == 0, "copies must divide over the waves");

  const int b = blockIdx.x / a.nsplit, split = blockIdx.x % a.nsplit;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int64_t S = a.S, H = a.H;
  const int64_t k0 = (int64_t)split * a.keys_per_split;
  const int64_t k1 = (k0 + a.keys_per_split < S) ? k0 + a.keys_per_split : S;
  const int ntiles = (int)((k1 - k0 + BN - 1) / BN);
  const int h0 = wave * 16;
  const uint16_t* c_seq = a.c_kv + (int64_t)b * S * R;
  const uint16_t* kp_seq = a.k_pe + (int64_t)b * S * DR;

  // Copy t of a tile moves 1 KiB: t < 32 latent, t >= 32 rotary key. Lane l
  // moves physical chunk pc = (t mod region) * 64 + l of its region; block
  // cb = pc / 128 holds row r = (pc / 4) % 32 at r * 64, its chunk c & 3 at
  // position (c & 3) ^ ((r >> 2) & 3).
  int voff[NCOPY];
#pragma unroll
  for (int u = 0; u < NCOPY; ++u) {
    const int t = u * NWV + wave;
    const bool lat = t < LAT_COPIES;
    const int pc = (lat ? t : t - LAT_COPIES) * 64 + lane;
    const int cb = pc >> 7, r = (pc >> 2) & 31, c4 = (pc & 3) ^ ((r >> 2) & 3);
    voff[u] = r * (lat ? R * 2 : DR * 2) + (cb * 4 + c4) * 16;
  }
  auto copy_tile = [&](int t, char* dst) {
    const int64_t kb = k0 + (int64_t)t * BN;
    const __amdgpu_buffer_rsrc_t rc = rows_rsrc(c_seq, kb, S, R * 2);
    const __amdgpu_buffer_rsrc_t rp = rows_rsrc(kp_seq, kb, S, DR * 2);
#pragma unroll
    for (int u = 0; u < NCOPY; ++u) {
      const int ct = u * NWV + wave;  // uniform
      if (ct < LAT_COPIES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(dst + ct * 1024), 16, voff[u], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_void*)(dst + ct * 1024), 16, voff[u], 0, 0, 0);
    }
  };

  copy_tile(0, tile0);

  // absorbed queries of the wave's 16 heads (B operand): lane (g, j) holds
  // head h0 + j, dims 32 ks + 8 g .. + 8
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* q = a.qt + ((int64_t)b * H + h0 + j) * KW + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(q + 32 * ks);
  }

  // LDS operand offsets. Score A operand (16 keys x 32 dims): lane (g, j)
  // reads key row kt*16 + j, chunk g of column block ks. Output A operand
  // (16 latent dims x 32 keys, transposed read): lane (g, j) addresses 8 bytes
  // of key row 4g + j/4 (and +16), dims 16 dt + 4 (j % 4); the read hands lane
  // i dims 16 dt + i of keys 4g .. 4g+3 (and 16+4g ..), the key order of the
  // score accumulator.
  const int kA = j * 64 + ((g ^ (j >> 2)) & 3) * 16;
  const int vrow = 4 * g + (j >> 2);
  const int vA0 = vrow * 64 + ((((j & 3) >> 1)) ^ g) * 16 + 8 * (j & 1);        // even dt
  const int vA1 = vrow * 64 + (((2 + ((j & 3) >> 1))) ^ g) * 16 + 8 * (j & 1);  // odd dt

  const float cl2 = a.scale_log2;
  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  auto step = [&](int t, const char* cur, char* nxt) {
    wait_vmem();
    __syncthreads();  // tile t has landed; every wave is done with the other buffer
    if (t + 1 < ntiles) copy_tile(t + 1, nxt);
    const int64_t kb = k0 + (int64_t)t * BN;
    // scores S^T: keys kb + kt*16 + 4g + r, head h0 + j
    f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(cur + ks * CB_BYTES + kA);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(cur + ks * CB_BYTES + 16 * 64 + kA);
      s0 = mfma16(a0, qf[ks], s0);
      s1 = mfma16(a1, qf[ks], s1);
    }
    // keys past this split's end (or the sequence's) take no weight
    const int64_t lim = k1 - kb;  // keys kb .. kb + lim - 1 are visible (lim >= 1)
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (4 * g + r < lim) ? s0[r] : -INFINITY;
      x[4 + r] = (16 + 4 * g + r < lim) ? s1[r] : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, x[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * cl2);
    const float ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - ref);
    m_run = m_new;
    float psum = 0.0f;
    bf16x8 pb;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], cl2, -ref));
      psum += p;
      pb[r] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    // latent output O~^T += C^T P^T, 16 latent dims per MFMA
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const char* p = cur + (dt >> 1) * CB_BYTES + ((dt & 1) ? vA1 : vA0);
      const bf16x4 lo = lds_tr_read(p);
      const bf16x4 hi = lds_tr_read(p + 16 * 64);
      const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[dt] = mfma16(va, pb, o[dt]);
    }
  };

  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(t, tile0, tile1);
    step(t + 1, tile1, tile0);
  }
  if (t < ntiles) step(t, tile0, tile1);

  // ---- partial of this split: o~ (unnormalised), max and sum per head
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t row = ((int64_t)b * a.nsplit + split) * H + h0 + j;
  float* po = a.po + row * R + 4 * g;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
  if (g == 0) {
    a.pml[2 * row] = m_run;
    a.pml[2 * row + 1] = l_tot;
  }
}

__global__ __launch_bounds__(64, 1) void latent_attn_kernel_w1(LatentArgs a) { latent_attn<1>(a); }
__global__ __launch_bounds__(128, 1) void latent_attn_kernel_w2(LatentArgs a) { latent_attn<2>(a); }
__global__ __launch_bounds__(192, 1) void latent_attn_kernel_w3(LatentArgs a) { latent_attn<3>(a); }
__global__ __launch_bounds__(256, 1) void latent_attn_kernel(LatentArgs a) { latent_attn<4>(a); }

// ---- 3. merge the splits of each (batch, head): o~ = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
__global__ __launch_bounds__(64) void latent_merge_kernel(LatentArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s)
    M = fmaxf(M, a.pml[2 * (((int64_t)b * a.nsplit + s) * a.H + h)]);
  float L = 0.0f, O[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) O[e] = 0.0f;
  for (int s = 0; s < a.nsplit; ++s) {
    const int64_t row = ((int64_t)b * a.nsplit + s) * a.H + h;
    const float w = __builtin_amdgcn_exp2f(a.pml[2 * row] - M);
    L += w * a.pml[2 * row + 1];
    const f32x4 p0 = *reinterpret_cast<const f32x4*>(a.po + row * R + 8 * lane);
    const f32x4 p1 = *reinterpret_cast<const f32x4*>(a.po + row * R + 8 * lane + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      O[e] = __builtin_fmaf(w, p0[e], O[e]);
      O[4 + e] = __builtin_fmaf(w, p1[e], O[4 + e]);
    }
  }
  const float inv = 1.0f / L;
  float* dst = a.olat + (int64_t)bh * R + 8 * lane;
  *reinterpret_cast<f32x4*>(dst) = f32x4{O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{O[4] * inv, O[5] * inv, O[6] * inv, O[7] * inv};
}

// ---- 4. up-projection: out[b,h,d] = sum_e W[256h + 128 + d, e] * o~[b,h,e]
// Workgroup: one head, 16 output dims; 16 lanes per dim, 32 latent dims each.
__global__ __launch_bounds__(256) void latent_up_kernel(LatentArgs a) {
  const int h = blockIdx.x >> 3, chunk = blockIdx.x & 7;
  const int d = chunk * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  const uint16_t* wrow = a.w_kv_b + ((int64_t)h * KVB + DN + d) * R + part * 32;
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const u32x4*>(wrow + 8 * i);
  for (int b = 0; b < a.B; ++b) {
    const float* ol = a.olat + ((int64_t)b * a.H + h) * R + part * 32;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(ol + 8 * i);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(ol + 8 * i + 4);
      const u32x4 wi = w[i];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w0 = wi[e], w1 = wi[2 + e];
        acc = __builtin_fmaf(__builtin_bit_cast(float, w0 << 16), x0[2 * e], acc);
        acc = __builtin_fmaf(__builtin_bit_cast(float, w0 & 0xffff0000u), x0[2 * e + 1], acc);
        acc = __builtin_fmaf(__builtin_bit_cast(float, w1 << 16), x1[2 * e], acc);
        acc = __builtin_fmaf(__builtin_bit_cast(float, w1 & 0xffff0000u), x1[2 * e + 1], acc);
      }
    }
    acc = row_sum16(acc);
    if (part == 0) a.out[((int64_t)b * a.H + h) * DV + d] = f32_to_bf16(acc);
  }
}

}  // namespace

hipError_t launch_latent_decode(const LatentArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(latent_absorb_kernel, dim3(a.H * 8), dim3(256), 0, stream, a);
  const int grid = a.B * a.nsplit;
  switch (a.H / 16) {
    case 1: hipLaunchKernelGGL(latent_attn_kernel_w1, dim3(grid), dim3(64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(latent_attn_kernel_w2, dim3(grid), dim3(128), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(latent_attn_kernel_w3, dim3(grid), dim3(192), 0, stream, a); break;
    default: hipLaunchKernelGGL(latent_attn_kernel, dim3(grid), dim3(256), 0, stream, a); break;
  }
  hipLaunchKernelGGL(latent_merge_kernel, dim3(a.B * a.H), dim3(64), 0, stream, a);
  hipLaunchKernelGGL(latent_up_kernel, dim3(a.H * 8), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

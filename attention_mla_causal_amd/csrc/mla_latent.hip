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
//  1. absorb: q~ for every (batch, head) on MFMA (W_k read transposed out of
//     LDS), rounded to bf16, joined with q_pe into a 576-dim row (workspace).
//  2. attention: one workgroup per (batch, key split), four waves. 32-key
//     tiles of [latent | k_pe] (36 KiB) are copied straight from HBM into LDS
//     (buffer_load ... lds; four buffers, two tiles ahead), in 64-byte column
//     blocks with swizzled 16-byte chunks. Scores use v_mfma_f32_16x16x32_bf16
//     with keys as rows and a wave's 16 heads as columns (S^T = K Q~^T, 18
//     K-steps); online softmax in fp32 per head. The latent output
//     O~^T = C^T P^T is split by latent dims instead: each wave accumulates
//     128 dims of all heads from the probabilities every wave leaves in LDS,
//     one tile behind the scores, its C^T fragments read with
//     ds_read_b64_tr_b16 in the key order the score accumulator leaves P in.
//     Each split writes an fp32 partial (o~, max, sum).
//  3. merge: log-sum-exp over the splits of each (batch, head) -> o~ (fp32).
//  4. up-projection: out = W_v o~ on MFMA (o~ split into two bf16 halves),
//     rounded to bf16.
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

// Wait until at most N of this wave's vector-memory operations are in flight
// (vmcnt is 6 bits: low 4 in [3:0], high 2 in [15:14]; lgkm and exp counts left open).
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ---- 1. absorb: q~[b,h,e] = sum_d q_nope[b,h,d] * W[256h + d, e]; q~[b,h,512+i] = q_pe[b,h,i]
// As a product per head, Q~_h^T [512 x B] = W_k[h]^T [512 x 128] . Q_h^T [128 x B],
// on v_mfma_f32_16x16x32_bf16. Workgroup: one head, 64 latent dims; wave w
// owns the 16 dims e0 + 16w and runs over the batch 16 rows at a time. W_k is
// stored with e contiguous, so the workgroup stages its [128 d x 64 e] block
// in LDS and reads it back transposed (ds_read_b64_tr_b16): lane (g, j) then
// holds dim e0 + 16w + j at d = 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3,
// the K order its query fragment is loaded in.
constexpr int ABS_ROW = 144;  // bytes per staged W row: 128 + 16 keeps the 4 rows a read touches apart
__global__ __launch_bounds__(256) void latent_absorb_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(16))) char wt[DN * ABS_ROW];
  const int h = blockIdx.x >> 3, chunk = blockIdx.x & 7;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int e0 = chunk * 64;
  const uint16_t* wk = a.w_kv_b + (int64_t)h * KVB * R + e0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // 128 rows x 8 chunks of 16 bytes
    const int c = tid + 256 * k, row = c >> 3, col = c & 7;
    *reinterpret_cast<u32x4*>(wt + row * ABS_ROW + col * 16) =
        *reinterpret_cast<const u32x4*>(wk + (int64_t)row * R + col * 8);
  }
  // The sign of softmax_scale travels with the joined query (see
  // positive_cl2): negated for a negative scale (exact in bf16), cleared for a
  // zero one.
  const float cl2_in = a.scale_log2;
  const uint32_t q_and = cl2_in == 0.0f ? 0u : 0xffffffffu;
  const uint32_t q_xor = cl2_in < 0.0f ? 0x80008000u : 0u;
  const float q_mul = cl2_in == 0.0f ? 0.0f : (cl2_in < 0.0f ? -1.0f : 1.0f);
  if (chunk == 0) {  // the rotary query goes through unchanged (but for that sign)
    for (int c = tid; c < a.B * 8; c += 256) {
      const int64_t bh = (int64_t)(c >> 3) * a.H + h;
      *reinterpret_cast<u32x4*>(a.qt + bh * KW + R + (c & 7) * 8) =
          (*reinterpret_cast<const u32x4*>(a.q_pe + bh * DR + (c & 7) * 8) & q_and) ^ q_xor;
    }
  }
  // query fragments of the first 16 batches load while W lands in LDS
  auto load_q = [&](int b0, u32x4* qv) {
    const int b = b0 + j;
    const uint16_t* q = a.q_nope + ((int64_t)(b < a.B ? b : 0) * a.H + h) * DN + 4 * g;
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) {
      qv[ks] = u32x4{0u, 0u, 0u, 0u};
      if (b < a.B) {
        const uint2 lo = *reinterpret_cast<const uint2*>(q + 32 * ks);
        const uint2 hi = *reinterpret_cast<const uint2*>(q + 32 * ks + 16);
        qv[ks] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
  };
  u32x4 qv[DN / 32];
  load_q(0, qv);
  __syncthreads();
  bf16x8 wf[DN / 32];
#pragma unroll
  for (int ks = 0; ks < DN / 32; ++ks) {
    const char* p = wt + (32 * ks + 4 * g + (j >> 2)) * ABS_ROW + (16 * wave + 4 * (j & 3)) * 2;
    const bf16x4 lo = lds_tr_read(p);
    const bf16x4 hi = lds_tr_read(p + 16 * ABS_ROW);
    wf[ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  for (int b0 = 0; b0 < a.B; b0 += 16) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) acc = mfma16(wf[ks], __builtin_bit_cast(bf16x8, qv[ks]), acc);
    if (b0 + 16 < a.B) load_q(b0 + 16, qv);
    // acc[r] = q~[b][e0 + 16w + 4g + r]; RNE rounding is symmetric, so
    // bf16(-x) = -bf16(x) and the sign can be applied before rounding
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= q_mul;
    const int b = b0 + j;
    if (b < a.B) {
      const uint32_t p0 = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      const uint32_t p1 = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      *reinterpret_cast<uint2*>(a.qt + ((int64_t)b * a.H + h) * KW + e0 + 16 * wave + 4 * g) =
          uint2{p0, p1};
    }
  }
}

// Chunk swizzle of the tile layout: chunk c & 3 of row r sits at position
// (c & 3) ^ tile_swz(r), the two bits of (r >> 2) & 3 swapped. Sixteen lanes
// reading one chunk of sixteen rows, and thirty-two lanes reading half a
// row of eight rows (the transposed reads), then touch every bank once.
__device__ __forceinline__ int tile_swz(int r) {
  const int x = (r >> 2) & 3;
  return ((x & 1) << 1) | (x >> 1);
}

// Buffer resource over rows [kb, end) of one sequence's row-major
// [S, rowbytes/2] bf16 tensor; rows at or past `end` read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* seq, int64_t kb,
                                                           int64_t end, int rowbytes) {
  // (end * rowbytes < 2^31: the host caps S, so the byte count fits 32 bits)
  const int64_t left = end - kb;
  const int records = left > 0 ? (int)(left * rowbytes) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)seq + kb * rowbytes), (short)0,
                                           records, 0x00020000);
}

// The softmax takes the running max of the unscaled scores and scales it by
// cl2 = softmax_scale * log2(e), which needs cl2 > 0. Any finite scale is
// served: the absorb kernel stores the joined query negated for a negative
// scale (scale * q.k = |scale| * (-q).k) and cleared for a zero scale (every
// key then scores 0, as with scale 0), and the attention runs with |cl2|, or
// with 1 when the scale is zero.
__device__ __forceinline__ float positive_cl2(float cl2_in) {
  return cl2_in == 0.0f ? 1.0f : __builtin_fabsf(cl2_in);
}

// ---- 2. attention over the latent keys of one key split
// Workgroup: one (batch, key split), four waves, always 64 head columns (any
// H up to 64; columns at or past H get zero queries and are never stored). Phase p of the loop
// does two independent jobs in one straight run of code:
//   * scores of tile p for heads 16w .. 16w+15 (wave w), the online-softmax
//     update of their max and sum, and their probabilities, which go to LDS
//     in the MFMA B-operand layout together with the rescale factor;
//   * the latent output of tile p-1 for latent dims 128w .. 128w+127 of all
//     64 heads, from the probabilities the four waves left in LDS.
// Each wave thus reads the whole tile once for its scores but only a quarter
// of it for the output. Tile t sits in buffer t % 4; at phase p tiles p and
// p-1 are read and tile p+2 is copied into the buffer tile p-2 left.
constexpr int NWAVE = 4;
constexpr int NCOPY = COPIES / NWAVE;  // 9 one-KiB copies per wave per tile
constexpr int NDTW = NDT / NWAVE;      // 8 latent-dim tiles of 16 per wave
static_assert(COPIES % NWAVE == 0, "copies must divide over the waves");

// Wait until at most N vector-memory operations of this wave are in flight
// and every LDS operation it issued has completed.
template <int N>
__device__ __forceinline__ void wait_vmem_keep_lds_done() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

__global__ __launch_bounds__(256, 1) void latent_attn_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(1024))) char tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile3[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][NWAVE][64];  // [phase parity][head group][lane]
  __shared__ float abuf[2][NWAVE * 16];                               // rescale factor per head

  const int b = blockIdx.x / a.nsplit, split = blockIdx.x % a.nsplit;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int64_t S = a.S, H = a.H;
  const int64_t k0 = (int64_t)split * a.keys_per_split;
  const int64_t k1 = (k0 + a.keys_per_split < S) ? k0 + a.keys_per_split : S;
  const int ntiles = (int)((k1 - k0 + BN - 1) / BN);
  const uint16_t* c_seq = a.c_kv + (int64_t)b * S * R;
  const uint16_t* kp_seq = a.k_pe + (int64_t)b * S * DR;

  // absorbed queries of heads 16w + j (B operand): lane (g, j) holds dims
  // 32 ks + 8 g .. + 8; zero for heads at or past H
  bf16x8 qf[KSTEPS];
  if (16 * wave + j < H) {
    const uint16_t* q = a.qt + ((int64_t)b * H + 16 * wave + j) * KW + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(q + 32 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = bf16x8{};
  }

  // Copy t of a tile moves 1 KiB: t < 32 latent, t >= 32 rotary key. Lane l
  // moves physical chunk pc = (t mod region) * 64 + l of its region; block
  // cb = pc / 128 holds row r = (pc / 4) % 32 at r * 64, its chunk c & 3 at
  // position (c & 3) ^ tile_swz(r).
  int voff[NCOPY];
#pragma unroll
  for (int u = 0; u < NCOPY; ++u) {
    const int t = u * NWAVE + wave;
    const bool lat = t < LAT_COPIES;
    const int pc = (lat ? t : t - LAT_COPIES) * 64 + lane;
    const int cb = pc >> 7, r = (pc >> 2) & 31, c4 = (pc & 3) ^ tile_swz(r);
    voff[u] = r * (lat ? R * 2 : DR * 2) + (cb * 4 + c4) * 16;
  }
  // Past the split's end a copy still runs but reads nothing (rows at or past
  // k1 read as zeros), so every phase costs each wave exactly NCOPY copies and
  // one vmcnt bound serves every phase.
  auto copy_tile = [&](int t, char* dst) {
    const int64_t kb = k0 + (int64_t)t * BN;
    const __amdgpu_buffer_rsrc_t rc = rows_rsrc(c_seq, kb, k1, R * 2);
    const __amdgpu_buffer_rsrc_t rp = rows_rsrc(kp_seq, kb, k1, DR * 2);
#pragma unroll
    for (int u = 0; u < NCOPY; ++u) {
      const int ct = u * NWAVE + wave;  // uniform
      if (ct < LAT_COPIES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(dst + ct * 1024), 16, voff[u], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_void*)(dst + ct * 1024), 16, voff[u], 0, 0, 0);
    }
  };
  copy_tile(0, tile0);
  copy_tile(1, tile1);

  // LDS operand offsets. Score A operand (16 keys x 32 dims): lane (g, j)
  // reads key row kt*16 + j, chunk g of column block ks. Output A operand
  // (16 latent dims x 32 keys, transposed read): lane (g, j) addresses 8 bytes
  // of key row 4g + j/4 (and +16), dims 16 dt + 4 (j % 4); the read hands lane
  // i dims 16 dt + i of keys 4g .. 4g+3 (and 16+4g ..), the key order in which
  // the score accumulator leaves the probabilities.
  const int kA = j * 64 + (g ^ tile_swz(j)) * 16;
  const int vrow = 4 * g + (j >> 2);  // tile_swz(vrow) = tile_swz(vrow + 16) = tile_swz(4 g)
  const int vA0 = vrow * 64 + (((j & 3) >> 1) ^ tile_swz(vrow)) * 16 + 8 * (j & 1);        // even dt
  const int vA1 = vrow * 64 + ((2 + ((j & 3) >> 1)) ^ tile_swz(vrow)) * 16 + 8 * (j & 1);  // odd dt

  const float cl2 = positive_cl2(a.scale_log2);
  // o[hg * NDTW + d]: dims 128w + 16d + 4g + r, head 16 hg + j
  f32x4 o[NWAVE * NDTW];
#pragma unroll
  for (int i = 0; i < NWAVE * NDTW; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  auto phase = [&](int p, const char* cur, const char* prv, char* fill, bool do_scores,
                   bool do_out) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_vmem_keep_lds_done<NCOPY>();  // tile p landed (this wave); its LDS writes are done
    __builtin_amdgcn_s_barrier();      // ... every wave's; tile p-2's buffer is free
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    copy_tile(p + 2, fill);
    bf16x8 pin[NWAVE];
    if (do_out) {
      // rescale by the factors of tile p-1 before its contribution lands
#pragma unroll
      for (int hg = 0; hg < NWAVE; ++hg) {
        const float al = abuf[(p - 1) & 1][16 * hg + j];
        pin[hg] = pbuf[(p - 1) & 1][hg][lane];
        if (__any(al != 1.0f)) {
#pragma unroll
          for (int d = 0; d < NDTW; ++d) o[hg * NDTW + d] *= al;
        }
      }
    }
    if (do_scores) {
      const int64_t kb = k0 + (int64_t)p * BN;
      // scores S^T: keys kb + kt*16 + 4g + r, head 16w + j
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
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], cl2, -ref));
        psum += pr;
        pb[r] = (__bf16)pr;
      }
      l_run = l_run * alpha + psum;
      pbuf[p & 1][wave][lane] = pb;
      if (g == 0) abuf[p & 1][16 * wave + j] = alpha;
    }
    if (do_out) {
      // latent output O~^T += C^T P^T for this wave's 128 dims, all head groups
#pragma unroll
      for (int d = 0; d < NDTW; ++d) {
        const int dt = wave * NDTW + d;
        const char* pp = prv + (dt >> 1) * CB_BYTES + ((dt & 1) ? vA1 : vA0);
        const bf16x4 lo = lds_tr_read(pp);
        const bf16x4 hi = lds_tr_read(pp + 16 * 64);
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int hg = 0; hg < NWAVE; ++hg) o[hg * NDTW + d] = mfma16(va, pin[hg], o[hg * NDTW + d]);
      }
    }
  };

  // phase 0: scores only; phases 1 .. ntiles-1: both; phase ntiles: output only.
  // Unrolled by four so that every buffer role is fixed in each copy.
  phase(0, tile0, tile3, tile2, true, false);
  int p = 1;
  for (; p + 3 < ntiles; p += 4) {
    phase(p, tile1, tile0, tile3, true, true);
    phase(p + 1, tile2, tile1, tile0, true, true);
    phase(p + 2, tile3, tile2, tile1, true, true);
    phase(p + 3, tile0, tile3, tile2, true, true);
  }
  if (p < ntiles) phase(p, tile1, tile0, tile3, true, true);
  if (p + 1 < ntiles) phase(p + 1, tile2, tile1, tile0, true, true);
  if (p + 2 < ntiles) phase(p + 2, tile3, tile2, tile1, true, true);
  // the last phase reads tile ntiles - 1, in buffer (ntiles - 1) % 4
  switch ((ntiles - 1) & 3) {
    case 0: phase(ntiles, tile1, tile0, tile3, false, true); break;
    case 1: phase(ntiles, tile2, tile1, tile0, false, true); break;
    case 2: phase(ntiles, tile3, tile2, tile1, false, true); break;
    default: phase(ntiles, tile0, tile3, tile2, false, true); break;
  }
  wait_vmem_keep<0>();  // (copies past the end are never read; let them land before exit)

  // ---- partial of this split: o~ (unnormalised) for this wave's dims; max and
  // sum of the wave's own heads
  const int64_t row0 = ((int64_t)b * a.nsplit + split) * H;
#pragma unroll
  for (int hg = 0; hg < NWAVE; ++hg) {
    if (16 * hg + j < H) {
      float* po = a.po + (row0 + 16 * hg + j) * R + 128 * wave + 4 * g;
#pragma unroll
      for (int d = 0; d < NDTW; ++d) *reinterpret_cast<f32x4*>(po + 16 * d) = o[hg * NDTW + d];
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (16 * wave + j < H && g == 0) {
    const int64_t row = row0 + 16 * wave + j;
    a.pml[2 * row] = m_run;
    a.pml[2 * row + 1] = l_tot;
  }
}

// ---- 3. merge the splits of each (batch, head): o~ = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// Workgroup: one (batch, head); wave w sums splits w, w + 4, ..., lane l holds
// dims 8l .. 8l + 7; the four wave sums meet in LDS.
__global__ __launch_bounds__(256) void latent_merge_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(16))) float part[4][R + 4];
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)b * a.nsplit * a.H + h;  // split s: row0 + s * H
  float M = -INFINITY;
  for (int s = lane; s < a.nsplit; s += 64) M = fmaxf(M, a.pml[2 * (row0 + (int64_t)s * a.H)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.0f, O[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) O[e] = 0.0f;
#pragma unroll 4
  for (int s = wave; s < a.nsplit; s += 4) {
    const int64_t row = row0 + (int64_t)s * a.H;
    const float w = __builtin_amdgcn_exp2f(a.pml[2 * row] - M);
    L = __builtin_fmaf(w, a.pml[2 * row + 1], L);
    const f32x4 p0 = *reinterpret_cast<const f32x4*>(a.po + row * R + 8 * lane);
    const f32x4 p1 = *reinterpret_cast<const f32x4*>(a.po + row * R + 8 * lane + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      O[e] = __builtin_fmaf(w, p0[e], O[e]);
      O[4 + e] = __builtin_fmaf(w, p1[e], O[4 + e]);
    }
  }
  *reinterpret_cast<f32x4*>(&part[wave][8 * lane]) = f32x4{O[0], O[1], O[2], O[3]};
  *reinterpret_cast<f32x4*>(&part[wave][8 * lane + 4]) = f32x4{O[4], O[5], O[6], O[7]};
  if (lane == 0) part[wave][R] = L;
  __syncthreads();
  const int e = 2 * threadIdx.x;
  const float inv = 1.0f / (part[0][R] + part[1][R] + part[2][R] + part[3][R]);
  const float o0 = part[0][e] + part[1][e] + part[2][e] + part[3][e];
  const float o1 = part[0][e + 1] + part[1][e + 1] + part[2][e + 1] + part[3][e + 1];
  *reinterpret_cast<float2*>(a.olat + (int64_t)bh * R + e) = float2{o0 * inv, o1 * inv};
}

// ---- 4. up-projection: out[b,h,d] = sum_e W[256h + 128 + d, e] * o~[b,h,e]
// Per head, Out_h^T [128 x B] = W_v[h] [128 x 512] . O~_h^T [512 x B] on
// v_mfma_f32_16x16x32_bf16. W_v is stored with e (the contraction) contiguous,
// so its fragments load straight from HBM. o~ is fp32: it enters as two bf16
// operands, hi = bf16(x) and lo = bf16(x - hi), whose sum carries x to about
// 2^-17 relative. Workgroup: one head, 32 output dims; wave w owns 16 of them
// and runs over the batch 16 rows at a time.
__global__ __launch_bounds__(128) void latent_up_kernel(LatentArgs a) {
  const int h = blockIdx.x >> 2, chunk = blockIdx.x & 3;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int d0 = chunk * 32 + wave * 16;
  const uint16_t* wrow = a.w_kv_b + ((int64_t)h * KVB + DN + d0 + j) * R + 8 * g;
  u32x4 wf[R / 32];
#pragma unroll
  for (int ks = 0; ks < R / 32; ++ks) wf[ks] = *reinterpret_cast<const u32x4*>(wrow + 32 * ks);
  for (int b0 = 0; b0 < a.B; b0 += 16) {
    const int b = b0 + j;
    const bool live = b < a.B;
    const float* ol = a.olat + ((int64_t)(live ? b : 0) * a.H + h) * R + 8 * g;
    f32x4 x[R / 32][2];  // every load of the group in flight at once
#pragma unroll
    for (int ks = 0; ks < R / 32; ++ks) {
      x[ks][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      x[ks][1] = x[ks][0];
      if (live) {
        x[ks][0] = *reinterpret_cast<const f32x4*>(ol + 32 * ks);
        x[ks][1] = *reinterpret_cast<const f32x4*>(ol + 32 * ks + 4);
      }
    }
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < R / 32; ++ks) {
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = x[ks][0][e], v1 = x[ks][1][e];
        const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
        hi[e] = h0;
        hi[4 + e] = h1;
        lo[e] = (__bf16)(v0 - (float)h0);
        lo[4 + e] = (__bf16)(v1 - (float)h1);
      }
      const bf16x8 w = __builtin_bit_cast(bf16x8, wf[ks]);
      acc = mfma16(w, hi, acc);
      acc = mfma16(w, lo, acc);
    }
    // acc[r] = out[b][d0 + 4g + r]
    if (live) {
      const uint32_t p0 = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      const uint32_t p1 = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      *reinterpret_cast<uint2*>(a.out + ((int64_t)b * a.H + h) * DV + d0 + 4 * g) = uint2{p0, p1};
    }
  }
}

}  // namespace

hipError_t launch_latent_decode(const LatentArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(latent_absorb_kernel, dim3(a.H * 8), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(latent_attn_kernel, dim3(a.B * a.nsplit), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(latent_merge_kernel, dim3(a.B * a.H), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(latent_up_kernel, dim3(a.H * 4), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

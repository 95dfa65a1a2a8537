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
// Three kernels on the caller's stream:
//  1. absorb: q~ for every (batch, head) on MFMA (W_k read transposed out of
//     LDS), rounded to bf16, joined with q_pe into a 576-dim row (workspace).
//  2. attention: one workgroup per (batch, key split), four waves (with few
//     sequences x tiles, one per (batch, key split, group of 16 heads)). 32-key
//     tiles of [latent | k_pe] (36 KiB) are copied straight from HBM into LDS
//     (buffer_load ... lds; four buffers, two tiles ahead), in 64-byte column
//     blocks with swizzled 16-byte chunks. Scores use v_mfma_f32_16x16x32_bf16
//     with keys as rows and a wave's 16 heads as columns (S^T = K Q~^T, 18
//     K-steps); online softmax in fp32 per head. The latent output
//     O~^T = C^T P^T is split by latent dims instead: each wave accumulates
//     128 dims of all heads from the probabilities every wave leaves in LDS,
//     one tile behind the scores, its C^T fragments read with
//     ds_read_b64_tr_b16 in the key order the score accumulator leaves P in.
//     Each split writes a partial: o~ rounded to bf16, (max, sum) in fp32.
//  3. merge + up-projection: log-sum-exp over the splits of each (batch,
//     head) -> o~ (fp32, in LDS), then out = W_v o~ on MFMA (o~ split into two
//     bf16 halves), rounded to bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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
// on v_mfma_f32_16x16x32_bf16. Workgroup: 16 sequences, one head, 64 latent
// dims; wave w owns the 16 dims e0 + 16w for the 16 sequences. W_k is
// stored with e contiguous, so the workgroup stages its [128 d x 64 e] block
// in LDS and reads it back transposed (ds_read_b64_tr_b16): lane (g, j) then
// holds dim e0 + 16w + j at d = 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3,
// the K order its query fragment is loaded in.
constexpr int ABS_ROW = 144;   // bytes per staged W row: 128 + 16 keeps the 4 rows a read touches apart
constexpr int ABS_QROW = 272;  // bytes per staged query row: 256 + 16, so the 8-byte reads of a
                               // half-wave meet distinct banks
constexpr int ABS_OROW = 136;  // bytes per staged output row (64 dims) + 8
constexpr int ABS_STAGE_MIN_B = 5;  // from this many sequences, queries and outputs go through LDS
__global__ __launch_bounds__(256) void latent_absorb_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(16))) char wt[DN * ABS_ROW];
  __shared__ __attribute__((aligned(16))) char qs[16 * ABS_QROW];
  __shared__ __attribute__((aligned(16))) char os[16 * ABS_OROW];
  // workgroup: (16 sequences, head, 64 latent dims); the 16-sequence groups of
  // one (head, dims) block sit 8 * H workgroups apart, on one XCD, and share
  // its weight block in L2
  const int chunk = blockIdx.x & 7, h = (blockIdx.x >> 3) % a.H;
  const int bq0 = (blockIdx.x >> 3) / a.H * 16;
  const int bq1 = (bq0 + 16 < a.B) ? bq0 + 16 : a.B;
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
    for (int c = bq0 * 8 + tid; c < bq1 * 8; c += 256) {
      const int64_t bh = (int64_t)(c >> 3) * a.H + h;
      *reinterpret_cast<u32x4*>(a.qt + bh * KW + R + (c & 7) * 8) =
          (*reinterpret_cast<const u32x4*>(a.q_pe + bh * DR + (c & 7) * 8) & q_and) ^ q_xor;
    }
  }
  // The query fragments load while W lands in LDS. Lane (g, j) needs 8-byte
  // pieces of sequence bq0 + j's row, so a direct load touches 16 rows per
  // instruction and each wave loads the same fragments; with more than a few
  // sequences the 16 rows (256 bytes each) are instead staged in LDS with one
  // 16-byte load per thread (batched decode, 32 sequences: about 2 us less).
  const bool staged = a.B >= ABS_STAGE_MIN_B;  // uniform
  u32x4 qv[DN / 32];
  if (staged) {
    const int r = tid >> 4, c = (tid & 15) * 8;
    const int b = bq0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (b < a.B) v = *reinterpret_cast<const u32x4*>(a.q_nope + ((int64_t)b * a.H + h) * DN + c);
    *reinterpret_cast<u32x4*>(qs + r * ABS_QROW + c * 2) = v;
  } else {
    const int b = bq0 + j;
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
  }
  __syncthreads();
  if (staged) {
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) {
      const char* p = qs + j * ABS_QROW + (32 * ks + 4 * g) * 2;
      const uint2 lo = *reinterpret_cast<const uint2*>(p);
      const uint2 hi = *reinterpret_cast<const uint2*>(p + 32);
      qv[ks] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
  bf16x8 wf[DN / 32];
#pragma unroll
  for (int ks = 0; ks < DN / 32; ++ks) {
    const char* p = wt + (32 * ks + 4 * g + (j >> 2)) * ABS_ROW + (16 * wave + 4 * (j & 3)) * 2;
    const bf16x4 lo = lds_tr_read(p);
    const bf16x4 hi = lds_tr_read(p + 16 * ABS_ROW);
    wf[ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  {
    const int b0 = bq0;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) acc = mfma16(wf[ks], __builtin_bit_cast(bf16x8, qv[ks]), acc);
    // acc[r] = q~[b][e0 + 16w + 4g + r]; RNE rounding is symmetric, so
    // bf16(-x) = -bf16(x) and the sign can be applied before rounding
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= q_mul;
    const uint32_t p0 = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    const uint32_t p1 = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    if (staged) {  // rows of 64 dims in LDS, then one whole 128-byte row per 16 threads
      *reinterpret_cast<uint2*>(os + j * ABS_OROW + (16 * wave + 4 * g) * 2) = uint2{p0, p1};
      __syncthreads();
      const int r = tid >> 4, c = tid & 15;
      if (b0 + r < a.B)
        *reinterpret_cast<uint2*>(a.qt + ((int64_t)(b0 + r) * a.H + h) * KW + e0 + 4 * c) =
            *reinterpret_cast<const uint2*>(os + r * ABS_OROW + 8 * c);
    } else if (b0 + j < a.B) {
      *reinterpret_cast<uint2*>(a.qt + ((int64_t)(b0 + j) * a.H + h) * KW + e0 + 16 * wave + 4 * g) =
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
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* seq, int kb, int end,
                                                           int rowbytes) {
  // 32-bit scalar arithmetic (a 64-bit compare would go through the VALU):
  // end * rowbytes < 2^31 (the host caps S) and kb <= end + 2 * BN, so the
  // row offset kb * rowbytes fits 32 bits unsigned.
  const int left = end - kb;
  const int records = left > 0 ? left * rowbytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)seq + (uint32_t)kb * (uint32_t)rowbytes), (short)0, records, 0x00020000);
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

// HG: head groups of 16 per workgroup. HG = 4 serves all (up to) 64 heads
// from each tile copy, as above. HG = 1 serves one head group (head_groups
// workgroups per split, each copying the tiles, from L2 after the first):
// wave 0 scores, all four waves accumulate the output of those 16 heads. For
// few sequences it gives each split several tiles for the same number of
// workgroups, so the partials (64 heads x 512 dims per split) shrink.
template <int HG>
__global__ __launch_bounds__(256, 1) void latent_attn_kernel(LatentArgs a) {
  static_assert(HG == 4 || HG == 1, "all four head groups, or one");
  __shared__ __attribute__((aligned(1024))) char tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char tile3[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][HG][64];  // [phase parity][head group][lane]
  __shared__ float abuf[2][HG * 16];                               // rescale factor per head

  // With HG = 1 the head groups of one (sequence, split) sit B * nsplit
  // workgroups apart. Workgroup w runs on XCD w % 8: with B a multiple of 8,
  // XCD x takes every split (and head group) of sequences x, x + 8, ..., so a
  // sequence's splits share one L2 (its absorbed queries and, with HG = 1,
  // its tiles are fetched from HBM once per sequence).
  const unsigned nbs = (unsigned)(a.B * a.nsplit);
  const int hg0 = HG == 4 ? 0 : (int)(blockIdx.x / nbs);  // first head group served
  const unsigned wg = HG == 4 ? blockIdx.x : blockIdx.x % nbs;
  int b, split;
  if (a.B % 8 == 0) {
    const int slot = wg >> 3;
    b = (wg & 7) + 8 * (slot / a.nsplit);
    split = slot % a.nsplit;
  } else {
    b = wg / a.nsplit;
    split = wg % a.nsplit;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int64_t S = a.S, H = a.H;
  // key counts fit 32 bits (the host caps S); per-lane key tests stay 32-bit
  const int k0 = split * (int)a.keys_per_split;
  const int k1 = (k0 + (int)a.keys_per_split < (int)S) ? k0 + (int)a.keys_per_split : (int)S;
  const int ntiles = (k1 - k0 + BN - 1) / BN;
  const uint16_t* c_seq = a.c_kv + (int64_t)b * S * R;
  const uint16_t* kp_seq = a.k_pe + (int64_t)b * S * DR;

  // absorbed queries of heads 16 (hg0 + w) + j for the scoring waves w < HG
  // (B operand): lane (g, j) holds dims 32 ks + 8 g .. + 8; zero for heads at
  // or past H
  const int hq = 16 * (hg0 + wave) + j;
  const bool scoring = HG == 4 || wave < HG;  // (wave < 4 always; written so it folds)
  bf16x8 qf[KSTEPS];
  if (scoring && hq < H) {
    const uint16_t* q = a.qt + ((int64_t)b * H + hq) * KW + 8 * g;
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
    const int kb = k0 + t * BN;
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
  // o[hg * NDTW + d]: dims 128w + 16d + 4g + r, head 16 (hg0 + hg) + j
  f32x4 o[HG * NDTW];
#pragma unroll
  for (int i = 0; i < HG * NDTW; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  auto phase = [&](int p, const char* cur, const char* prv, char* fill, bool do_scores,
                   bool do_out) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_vmem_keep_lds_done<NCOPY>();  // tile p landed (this wave); its LDS writes are done
    __builtin_amdgcn_s_barrier();      // ... every wave's; tile p-2's buffer is free
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    copy_tile(p + 2, fill);
    bf16x8 pin[HG];
    float al[HG];
    if (do_out) {
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        al[hg] = abuf[(p - 1) & 1][16 * hg + j];
        pin[hg] = pbuf[(p - 1) & 1][hg][lane];
      }
    }
    if (do_scores && scoring) {
      const int kb = k0 + p * BN;
      // scores S^T: keys kb + kt*16 + 4g + r, head 16 (hg0 + w) + j
      f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(cur + ks * CB_BYTES + kA);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(cur + ks * CB_BYTES + 16 * 64 + kA);
        s0 = mfma16(a0, qf[ks], s0);
        s1 = mfma16(a1, qf[ks], s1);
      }
      // keys past this split's end (or the sequence's) take no weight
      const int lim = k1 - kb;  // keys kb .. kb + lim - 1 are visible (lim >= 1)
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
        // rescaled by tile p-1's factors as its contribution lands (a factor
        // of 1 leaves the accumulator unchanged)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) o[hg * NDTW + d] = mfma16(va, pin[hg], o[hg * NDTW + d] * al[hg]);
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
  // sum of the wave's own heads. A lane holds 4 dims of one head per
  // accumulator, so stored directly each instruction would touch 16 rows; the
  // accumulators are turned into rows in LDS first (head group hg in tile
  // buffer hg, rows of 512 dims 2064 bytes apart, so each 16-lane group of a
  // write meets 16 distinct banks), then every wave stores whole rows. The
  // partial is stored rounded to bf16 (round to nearest even): it is the
  // output of a bf16 product, which the pages' attention rounds to bf16 as
  // well; the (max, sum) pair stays fp32 and the merge runs in fp32.
  __syncthreads();  // every wave is done with the tiles
  auto stage = [&](int hg) -> char* { return hg == 0 ? tile0 : hg == 1 ? tile1 : hg == 2 ? tile2 : tile3; };
  constexpr int ROWB = R * 4 + 16;
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int d = 0; d < NDTW; ++d)
      *reinterpret_cast<f32x4*>(stage(hg) + j * ROWB + (128 * wave + 16 * d + 4 * g) * 4) = o[hg * NDTW + d];
  __syncthreads();
  const int64_t row0 = ((int64_t)b * a.nsplit + split) * H;
#pragma unroll
  for (int k = 0; k < HG * 16 / NWAVE; ++k) {  // one row per wave: lane l stores dims 4l.. and 256+4l..
    const int hl = k * NWAVE + wave;           // head within the workgroup (hl >> 4 == k >> 2)
    const int hd = 16 * hg0 + hl;
    if (hd < H) {
      const char* src = stage(k >> 2) + (hl & 15) * ROWB;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(src + 16 * lane);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + R * 2 + 16 * lane);
      bf16x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = (__bf16)v0[e];
        w1[e] = (__bf16)v1[e];
      }
      // non-temporal: the partials are read once, by the next kernel
      uint16_t* dst = a.po + (row0 + hd) * R + 4 * lane;
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, w0), reinterpret_cast<u32x2*>(dst));
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, w1), reinterpret_cast<u32x2*>(dst + R / 2));
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (scoring && hq < H && g == 0) {
    const int64_t row = row0 + hq;
    a.pml[2 * row] = m_run;
    a.pml[2 * row + 1] = l_tot;
  }
}

// ---- 3. merge + up-projection, one launch:
//   o~[b,h]    = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s   (M = max_s m_s)
//   out[b,h,d] = sum_e W[256h + 128 + d, e] * o~[b,h,e]
// Workgroup: one head, up to eight sequences, 128 / C of the head's output
// dims, eight waves. First the waves merge the splits of the workgroup's
// sequences (a sequence's splits are dealt over 8 / n of the waves, n its live
// sequences rounded up to a power of two, so a lone sequence still has all
// eight waves loading) and leave o~ in LDS. Then, as
// Out_h^T [128 x 8] = W_v[h] [128 x 512] . O~_h^T [512 x 8] on
// v_mfma_f32_16x16x32_bf16, wave w computes 16 output dims over 512 / C of
// the contraction (C waves per 16 dims, their sums added in LDS). W_v's
// contraction dim is contiguous, so its fragments load straight from HBM,
// right after the first batch of partials (whose merge thus waits for the
// partials alone) and while the merge runs; o~ (merged in fp32) enters as two bf16 operands,
// hi = bf16(x) and lo = bf16(x - hi), whose sum carries x to about 2^-17
// relative. The host picks C so that about 256 workgroups run: with few
// sequences the head's weight rows are spread over C workgroups (each merging
// the same splits again, from L2) rather than loaded by one. Workgroups of one
// head share one L2 (H a multiple of 8 puts them on one XCD).
constexpr int OUT_BG = 8;     // sequences per workgroup (MFMA columns 8..15 stay zero)
constexpr int OUT_WAVES = 8;
constexpr int OROW = R + 4;   // floats per LDS row: 2064 bytes, so the 16-byte reads of
                              // eight rows at one offset meet distinct banks
// U: splits a wave loads in one batch (the host takes 8 when a wave merges
// more than four, so the batched decode's eight splits per sequence arrive in
// one round trip, else 4).
template <int C, int U>
__global__ __launch_bounds__(512) void latent_out_kernel(LatentArgs a) {
  static_assert(C == 1 || C == 2 || C == 4, "C divides the 8 waves and the 16 K-steps");
  static_assert(U == 4 || U == 8, "splits per batch");
  constexpr int TILES = OUT_WAVES / C;  // 16-dim output tiles per workgroup
  constexpr int KS = R / 32 / C;        // K-steps per wave
  __shared__ __attribute__((aligned(16))) float part[OUT_WAVES][OROW];
  __shared__ float lpart[OUT_WAVES][2];
  __shared__ __attribute__((aligned(16))) float orow[OUT_BG][OROW];
  const int h = blockIdx.x % a.H, rest = blockIdx.x / a.H;
  const int chunk = rest % C, b0 = (rest / C) * OUT_BG;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;

  const int tile = wave % TILES, epart = wave / TILES;
  const int d0 = chunk * (DV / C) + 16 * tile;
  const uint16_t* wrow = a.w_kv_b + ((int64_t)h * KVB + DN + d0 + j) * R + 8 * g + 32 * KS * epart;

  // merge: wave w takes sequence slot w / wpb and splits s = w % wpb (mod wpb)
  const int nb = (a.B - b0 < OUT_BG) ? a.B - b0 : OUT_BG;  // live sequences, >= 1
  const int nbp = nb > 4 ? 8 : (nb > 2 ? 4 : nb);         // rounded up to a power of two
  const int wpb = OUT_WAVES / nbp;
  const int slot = wave / wpb, sub = wave % wpb;
  // Each wave merges its splits in order with a running maximum (every load
  // of a batch of splits is issued at once; no pass over the maxima first),
  // leaving (max, sum) and its unnormalised sum in LDS.
  f32x4 o0 = {0.0f, 0.0f, 0.0f, 0.0f}, o1 = o0;
  float mrun = -INFINITY, lsum = 0.0f;
  const bool live = slot < nb;
  const int64_t row0 = (int64_t)(b0 + (live ? slot : 0)) * a.nsplit * a.H + h;  // split s: row0 + s * H
  float ms[U], ls[U];
  f32x4 p0[U], p1[U];
  // loads of the splits s0, s0 + wpb, ...; rows past the end (or of a wave
  // with no sequence) reread split 0 and take no weight
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * wpb;
      const bool ok = live && s < a.nsplit;
      const int64_t row = row0 + (int64_t)(ok ? s : 0) * a.H;
      const float2 ml = *reinterpret_cast<const float2*>(a.pml + 2 * row);
      ms[u] = ok ? ml.x : -INFINITY;
      ls[u] = ml.y;
      const uint16_t* src = a.po + row * R + 4 * lane;  // bf16 dims 4 lane .. and 256 + 4 lane ..
      const bf16x4 q0 = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(src));
      const bf16x4 q1 = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(src + R / 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0[u][e] = (float)q0[e];
        p1[u][e] = (float)q1[e];
      }
    }
  };
  auto fold_batch = [&]() {
    float mnew = mrun;
#pragma unroll
    for (int u = 0; u < U; ++u) mnew = fmaxf(mnew, ms[u]);
    const float al = __builtin_amdgcn_exp2f(mrun - mnew);  // mnew is finite: the batch's first split is live
    lsum *= al;
    o0 *= al;
    o1 *= al;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __builtin_amdgcn_exp2f(ms[u] - mnew);  // 0 for splits past the end
      lsum = __builtin_fmaf(w, ls[u], lsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = __builtin_fmaf(w, p0[u][e], o0[e]);
        o1[e] = __builtin_fmaf(w, p1[u][e], o1[e]);
      }
    }
    mrun = mnew;
  };
  load_batch(sub);
  // W_v's fragments load after the first batch of partials, so the merge
  // waits for those alone
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) wf[ks] = *reinterpret_cast<const u32x4*>(wrow + 32 * ks);
  if (live && sub < a.nsplit) {
    fold_batch();
    for (int s0 = sub + U * wpb; s0 < a.nsplit; s0 += U * wpb) {
      load_batch(s0);
      fold_batch();
    }
  }
  *reinterpret_cast<f32x4*>(&part[wave][4 * lane]) = o0;
  *reinterpret_cast<f32x4*>(&part[wave][R / 2 + 4 * lane]) = o1;
  if (lane == 0) {
    lpart[wave][0] = mrun;
    lpart[wave][1] = lsum;
  }
  __syncthreads();
  {  // row r = wave of o~: the wpb partial sums of slot r, in order, over their total weight
    f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
    if (wave < nb) {
      float M = -INFINITY;
      for (int i = 0; i < wpb; ++i) M = fmaxf(M, lpart[wave * wpb + i][0]);
      float L = 0.0f;
      for (int i = 0; i < wpb; ++i) {
        const int pw = wave * wpb + i;
        const float w = __builtin_amdgcn_exp2f(lpart[pw][0] - M);  // 0 for a wave with no split
        s0 += w * *reinterpret_cast<const f32x4*>(&part[pw][4 * lane]);
        s1 += w * *reinterpret_cast<const f32x4*>(&part[pw][R / 2 + 4 * lane]);
        L = __builtin_fmaf(w, lpart[pw][1], L);
      }
      const float inv = 1.0f / L;
      s0 *= inv;
      s1 *= inv;
    }
    if (wave < OUT_BG) {
      *reinterpret_cast<f32x4*>(&orow[wave][4 * lane]) = s0;
      *reinterpret_cast<f32x4*>(&orow[wave][R / 2 + 4 * lane]) = s1;
    }
  }
  __syncthreads();

  // up-projection: lane (g, j) feeds o~ of sequence b0 + j (zero for j >= 8)
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int e0 = 32 * (KS * epart + ks) + 8 * g;
    f32x4 x0 = {0.0f, 0.0f, 0.0f, 0.0f}, x1 = x0;
    if (j < OUT_BG) {
      x0 = *reinterpret_cast<const f32x4*>(&orow[j][e0]);
      x1 = *reinterpret_cast<const f32x4*>(&orow[j][e0 + 4]);
    }
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const __bf16 h0 = (__bf16)x0[e], h1 = (__bf16)x1[e];
      hi[e] = h0;
      hi[4 + e] = h1;
      lo[e] = (__bf16)(x0[e] - (float)h0);
      lo[4 + e] = (__bf16)(x1[e] - (float)h1);
    }
    const bf16x8 w = __builtin_bit_cast(bf16x8, wf[ks]);
    acc = mfma16(w, hi, acc);
    acc = mfma16(w, lo, acc);
  }
  if constexpr (C > 1) {  // the C parts of each tile's contraction, added in order
    *reinterpret_cast<f32x4*>(&part[wave][4 * lane]) = acc;  // (part is free again)
    __syncthreads();
    if (epart != 0) return;
    for (int i = 1; i < C; ++i) acc += *reinterpret_cast<const f32x4*>(&part[i * TILES + tile][4 * lane]);
  }
  // acc[r] = out[b0 + j][d0 + 4g + r]
  if (j < nb) {
    const uint32_t p0 = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    const uint32_t p1 = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    *reinterpret_cast<uint2*>(a.out + ((int64_t)(b0 + j) * a.H + h) * DV + d0 + 4 * g) = uint2{p0, p1};
  }
}

}  // namespace

hipError_t launch_latent_decode(const LatentArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(latent_absorb_kernel, dim3((a.B + 15) / 16 * a.H * 8), dim3(256), 0, stream, a);
  if (a.head_groups == 1)
    hipLaunchKernelGGL(latent_attn_kernel<4>, dim3(a.B * a.nsplit), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(latent_attn_kernel<1>, dim3(a.B * a.nsplit * a.head_groups), dim3(256), 0, stream, a);
  // merge + up-projection: C workgroups per (head, eight sequences), about 256 in all
  const int groups = (a.B + OUT_BG - 1) / OUT_BG * a.H;
  // splits each wave merges when a workgroup holds min(B, 8) sequences
  const int nb = a.B < OUT_BG ? a.B : OUT_BG;
  const int wpb = OUT_WAVES / (nb > 4 ? 8 : (nb > 2 ? 4 : nb));
  const bool u8 = (a.nsplit + wpb - 1) / wpb > 4;
  if (groups >= 256) {
    if (u8) hipLaunchKernelGGL((latent_out_kernel<1, 8>), dim3(groups), dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((latent_out_kernel<1, 4>), dim3(groups), dim3(512), 0, stream, a);
  } else if (groups >= 128) {
    if (u8) hipLaunchKernelGGL((latent_out_kernel<2, 8>), dim3(groups * 2), dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((latent_out_kernel<2, 4>), dim3(groups * 2), dim3(512), 0, stream, a);
  } else {
    if (u8) hipLaunchKernelGGL((latent_out_kernel<4, 8>), dim3(groups * 4), dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((latent_out_kernel<4, 4>), dim3(groups * 4), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla

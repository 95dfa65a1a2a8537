// Causal MLA attention, prefill (any T >= 1 new queries over S = past_len + T keys).
//
// Computes, per (batch, head), softmax(scale * (q_nope k_nope^T + q_pe k_pe^T)
// + causal mask) v, as in the attention-core excerpt of the Kimi K2
// "Similarities" page ("Query-key similarity") and the "Weighted sum of
// values" page, with the mask of the "Causal mask" page: query i sits at
// absolute position past_len + i and sees keys 0..past_len+i.
//
// gfx950 design (one workgroup = 4 wave64s = 128 queries of one head):
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K rows come from LDS as the A operand, Q stays in VGPRs as the B operand.
//    In the 32x32 accumulator every lane then owns one query (lane % 32) and
//    16 of the 32 keys of the tile; lane and lane^32 share a query. Row max
//    and row sum are register reductions plus one exchange with lane^32.
//  * The 192-wide contraction is split 128 + 64: the last 4 K-steps read the
//    rotary key k_pe, one [S,64] tensor shared by every head, so the query
//    and key of the pages are never concatenated in memory.
//  * The output is formed transposed too, O^T = V^T P^T: P^T is exactly the
//    score accumulator (converted to bf16), so the probabilities never leave
//    registers; the V^T operand is read from a row-major V tile in LDS with
//    ds_read_b64_tr_b16, whose key order matches the accumulator's.
//  * Online softmax in fp32 in the exp2 domain (scale * log2 e folded into one
//    FMA); causal tiles beyond the diagonal are never visited and only tiles
//    that straddle it compare indices.
//  * K/V tiles of 64 keys are prefetched into registers while the previous
//    tile is computed, then stored to padded LDS rows (no bank conflicts on
//    the 16-byte row reads).
//  * Workgroup order: all query tiles of one head are placed on one XCD and
//    dispatched together, heaviest (latest) tile first, so K/V blocks stream
//    through that XCD's L2 once for all of them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int DN = 128;   // non-rotary query/key dims
constexpr int DR = 64;    // rotary dims (shared key)
constexpr int DV = 128;   // value dims
constexpr int BM = 128;   // queries per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NW = 4;     // waves per workgroup
constexpr int NT = NW * 64;

// LDS rows, in bf16 elements, padded so that 16-byte reads of 16 consecutive
// rows at one column fall in distinct banks.
constexpr int KN_LD = DN + 8;   // 272 B
constexpr int KP_LD = DR + 8;   // 144 B
constexpr int V_LD = DV + 16;   // 288 B
constexpr int KN_ELEMS = BN * KN_LD;
constexpr int KP_ELEMS = BN * KP_LD;
constexpr int V_ELEMS = BN * V_LD;
constexpr int LDS_ELEMS = KN_ELEMS + KP_ELEMS + V_ELEMS;

// 16-byte chunks per tile each thread moves: k_nope 64x128, k_pe 64x64, v 64x128
constexpr int KN_CHUNKS = BN * DN / 8 / NT;  // 4
constexpr int KP_CHUNKS = BN * DR / 8 / NT;  // 2
constexpr int V_CHUNKS = BN * DV / 8 / NT;   // 4

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ bf16x4 lds_tr_read(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__global__ __launch_bounds__(NT, 2) void mla_prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  uint16_t* lds_kn = lds;
  uint16_t* lds_kp = lds + KN_ELEMS;
  uint16_t* lds_v = lds + KN_ELEMS + KP_ELEMS;

  // ---- which (batch, head, query tile) this workgroup owns
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const int bh = logical / a.ntiles;
  const int qt = a.ntiles - 1 - logical % a.ntiles;
  const int b = bh / a.H;
  const int q0 = qt * BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;     // which half of the wave
  const int l32 = lane & 31;
  const int q0w = q0 + wave * 32;

  const int64_t T = a.T, S = a.S, P = a.past_len;
  const uint16_t* qn_g = a.q_nope + (int64_t)bh * T * DN;
  const uint16_t* qp_g = a.q_pe + (int64_t)bh * T * DR;
  const uint16_t* kn_g = a.k_nope + (int64_t)bh * S * DN;
  const uint16_t* kp_g = a.k_pe + (int64_t)b * S * DR;
  const uint16_t* v_g = a.v + (int64_t)bh * S * DV;

  // ---- query fragment (B operand of S^T = K Q^T): lane holds 8 dims of its query per K-step
  bf16x8 qf[12];
  {
    const int64_t myq = q0w + l32;
    const int koff = 8 * hi;
    const bool ok = myq < T;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(ok ? ldg16(qn_g + myq * DN + 16 * kk + koff) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[8 + kk] = as_bf16x8(ok ? ldg16(qp_g + myq * DR + 16 * kk + koff) : u32x4{0, 0, 0, 0});
  }

  // ---- key range: the workgroup needs keys [0, P + last query + 1)
  const int64_t q_last = (q0 + BM < T ? q0 + BM : T) - 1;
  const int64_t kend = P + q_last + 1;
  const int nblocks = (int)((kend + BN - 1) / BN);
  const bool wave_live = q0w < T;
  const int64_t wave_q_last = (q0w + 31 < T ? q0w + 31 : T - 1);
  const int64_t wave_kend = P + wave_q_last + 1;  // keys beyond are hidden from the whole wave
  const int64_t wave_kfull = P + q0w + 1;         // keys below are visible to the whole wave

  const float c = a.scale_log2;
  f32x16 o[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[n][r] = 0.0f;
  float m_run = -INFINITY;  // running max in the scaled log2 domain
  float l_run = 0.0f;       // this lane's share of the running sum

  // ---- register prefetch of one K/V tile
  u32x4 rkn[KN_CHUNKS], rkp[KP_CHUNKS], rv[V_CHUNKS];
  auto load_tile = [&](int j) {
    const int64_t kb = (int64_t)j * BN;
#pragma unroll
    for (int u = 0; u < KN_CHUNKS; ++u) {
      const int ch = tid + u * NT;
      const int row = ch >> 4, col = (ch & 15) * 8;
      const int64_t key = kb + row;
      rkn[u] = key < S ? ldg16(kn_g + key * DN + col) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < KP_CHUNKS; ++u) {
      const int ch = tid + u * NT;
      const int row = ch >> 3, col = (ch & 7) * 8;
      const int64_t key = kb + row;
      rkp[u] = key < S ? ldg16(kp_g + key * DR + col) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < V_CHUNKS; ++u) {
      const int ch = tid + u * NT;
      const int row = ch >> 4, col = (ch & 15) * 8;
      const int64_t key = kb + row;
      rv[u] = key < S ? ldg16(v_g + key * DV + col) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < KN_CHUNKS; ++u) {
      const int ch = tid + u * NT;
      *reinterpret_cast<u32x4*>(lds_kn + (ch >> 4) * KN_LD + (ch & 15) * 8) = rkn[u];
    }
#pragma unroll
    for (int u = 0; u < KP_CHUNKS; ++u) {
      const int ch = tid + u * NT;
      *reinterpret_cast<u32x4*>(lds_kp + (ch >> 3) * KP_LD + (ch & 7) * 8) = rkp[u];
    }
#pragma unroll
    for (int u = 0; u < V_CHUNKS; ++u) {
      const int ch = tid + u * NT;
      *reinterpret_cast<u32x4*>(lds_v + (ch >> 4) * V_LD + (ch & 15) * 8) = rv[u];
    }
  };

  load_tile(0);
  for (int j = 0; j < nblocks; ++j) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (j + 1 < nblocks) load_tile(j + 1);  // lands while this tile is computed

    const int64_t kb = (int64_t)j * BN;
    if (!wave_live || kb >= wave_kend) continue;  // wave-uniform

    // ---- S^T tile: 64 keys x 32 queries, two 32x32 accumulators
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.0f;
      const int krow = 32 * mt + l32;
      const uint16_t* kn_row = lds_kn + krow * KN_LD + 8 * hi;
      const uint16_t* kp_row = lds_kp + krow * KP_LD + 8 * hi;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kn_row + 16 * kk);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[mt], 0, 0, 0);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp_row + 16 * kk);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[8 + kk], s[mt], 0, 0, 0);
      }
    }

    // ---- causal mask, only on tiles that cross this wave's diagonal
    if (kb + BN > wave_kfull) {
      const int64_t lim = P + q0w + l32;  // last visible key of this lane's query
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = kb + 32 * mt + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key > lim || key >= S) s[mt][r] = -INFINITY;
        }
    }

    // ---- online softmax (scale > 0, so max of scaled = scale * max)
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], c, -m_ref));
        s[mt][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[n][r] *= alpha;

    // ---- O^T += V^T P^T over 4 K-steps of 16 keys
    const int sl = lane & 15;
    const int grp = (lane >> 4) & 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mt = ks >> 1, half = ks & 1;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[mt][8 * half + e];
      const int kr = 32 * mt + 16 * half + 4 * hi + (sl >> 2);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint16_t* vp = lds_v + kr * V_LD + 32 * n + 16 * grp + 4 * (sl & 3);
        const bf16x4 lo4 = lds_tr_read(vp);
        const bf16x4 hi4 = lds_tr_read(vp + 8 * V_LD);
        const bf16x8 va = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[n], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: divide by the full row sum and store bf16
  if (!wave_live) return;
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.0f / l_tot;
  const int64_t myq = q0w + l32;
  if (myq >= T) return;
  uint16_t* out_row = a.out + ((int64_t)bh * T + myq) * DV;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv0 = 32 * n + 8 * g + 4 * hi;
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[n][4 * g + e] * inv);
      *reinterpret_cast<bf16x4*>(out_row + dv0) = w;
    }
}

}  // namespace

int prefill_grid(const PrefillArgs& a) { return a.B * a.H * a.ntiles; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int grid = prefill_grid(a);
  hipLaunchKernelGGL(mla_prefill_kernel, dim3(grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

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

// One LDS stage holds a 64-key tile: k_nope, k_pe, v. Rows are unpadded and
// their 16-byte chunks are XOR-swizzled by row, so that the direct
// global->LDS loads (which fill 1 KiB contiguously per instruction) and the
// MFMA operand reads (16 rows at one logical column) are both conflict-free.
constexpr int KN_OFF = 0;
constexpr int KP_OFF = BN * DN * 2;             // 16384
constexpr int V_OFF = KP_OFF + BN * DR * 2;     // 24576
constexpr int STAGE_BYTES = V_OFF + BN * DV * 2;  // 40960

// physical 16-byte chunk of logical chunk c in row r
__device__ __forceinline__ int kn_chunk(int r, int c) { return r * 16 + (c ^ (r & 15)); }
__device__ __forceinline__ int kp_chunk(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int v_chunk(int r, int c) { return r * 16 + (c ^ ((r & 3) << 2)); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_void;

__device__ __forceinline__ void load_lds16(const uint16_t* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ bf16x4 lds_tr_read(const char* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Wait until this wave's global->LDS copies have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

struct Ctx {
  const uint16_t* kn_g;
  const uint16_t* kp_g;
  const uint16_t* v_g;
  int64_t S, P;
  int tid, lane, wave, hi, l32;
};

// Issue the 10 direct global->LDS copies (per wave) of key tile j into `stage`.
// Rows past the last key are clamped to it: they are masked out of the
// softmax, and clamping keeps every LDS value finite.
__device__ __forceinline__ void issue_tile(const Ctx& c, int j, char* stage) {
  const int64_t kb = (int64_t)j * BN;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = u * NW + c.wave;
    const int pc = t * 64 + c.lane;
    const int r = pc >> 4, p = pc & 15;
    const int64_t key = (kb + r < c.S) ? kb + r : c.S - 1;
    load_lds16(c.kn_g + key * DN + ((p ^ (r & 15)) << 3), stage + KN_OFF + t * 1024);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = u * NW + c.wave;
    const int pc = t * 64 + c.lane;
    const int r = pc >> 3, p = pc & 7;
    const int64_t key = (kb + r < c.S) ? kb + r : c.S - 1;
    load_lds16(c.kp_g + key * DR + ((p ^ ((r >> 1) & 7)) << 3), stage + KP_OFF + t * 1024);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = u * NW + c.wave;
    const int pc = t * 64 + c.lane;
    const int r = pc >> 4, p = pc & 15;
    const int64_t key = (kb + r < c.S) ? kb + r : c.S - 1;
    load_lds16(c.v_g + key * DV + ((p ^ ((r & 3) << 2)) << 3), stage + V_OFF + t * 1024);
  }
}

struct State {
  f32x16 o[4];   // O^T accumulators: lane owns query l32, 64 of its 128 dims
  float m_run;   // running max, scaled log2 domain
  float l_run;   // this lane's share of the running sum
};

// One 64-key tile for one wave's 32 queries.
__device__ __forceinline__ void compute_tile(const Ctx& c, const bf16x8 (&qf)[12], State& st,
                                             const char* stage, int64_t kb, int64_t q0w,
                                             int64_t wave_kfull, float cl2) {
  // ---- S^T = K Q^T: two 32-key halves interleaved for independent MFMA chains
  f32x16 s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = 0.0f;
    s1[r] = 0.0f;
  }
  const int r0 = c.l32, r1 = 32 + c.l32;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int lc = 2 * kk + c.hi;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(stage + KN_OFF + kn_chunk(r0, lc) * 16);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(stage + KN_OFF + kn_chunk(r1, lc) * 16);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s1, 0, 0, 0);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int lc = 2 * kk + c.hi;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(stage + KP_OFF + kp_chunk(r0, lc) * 16);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(stage + KP_OFF + kp_chunk(r1, lc) * 16);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[8 + kk], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[8 + kk], s1, 0, 0, 0);
  }

  // ---- causal mask, only on tiles that cross this wave's diagonal
  if (kb + BN > wave_kfull) {
    const int64_t lim = c.P + q0w + c.l32;  // last key this lane's query sees
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t key = kb + 8 * (r >> 2) + 4 * c.hi + (r & 3);
      if (key > lim || key >= c.S) s0[r] = -INFINITY;
      if (key + 32 > lim || key + 32 >= c.S) s1[r] = -INFINITY;
    }
  }

  // ---- online softmax (scale > 0: the max of scaled scores is scale * max)
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = fmaxf(mx, xor32(mx));
  const float m_new = fmaxf(st.m_run, mx * cl2);
  const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_ref);
  st.m_run = m_new;
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cl2, -m_ref));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cl2, -m_ref));
    psum += s0[r] + s1[r];
  }
  st.l_run = st.l_run * alpha + psum;
  // rescale O only when some query of the wave raised its max
  if (__builtin_amdgcn_read_exec() && __any(alpha != 1.0f)) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[n][r] *= alpha;
  }

  // ---- O^T += V^T P^T over 4 K-steps of 16 keys
  const int sl = c.lane & 15;
  const int grp = (c.lane >> 4) & 1;
  // byte offset of this lane's 8-byte piece of V, K-step 0, dims 32n + ...
  const int vrow = 4 * c.hi + (sl >> 2);
  const int vcol = 2 * grp + ((sl & 3) >> 1);  // logical chunk within a 32-dim group
  const int vhalf = 8 * (sl & 1);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const f32x16& sp = (ks >> 1) ? s1 : s0;
    const int h8 = 8 * (ks & 1);
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sp[h8 + e];
    const int kr = 32 * (ks >> 1) + 16 * (ks & 1) + vrow;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const char* vp = stage + V_OFF + v_chunk(kr, 4 * n + vcol) * 16 + vhalf;
      const bf16x4 lo4 = lds_tr_read(vp);
      const bf16x4 hi4 = lds_tr_read(vp + 8 * 16 * 16);  // row kr + 8: same swizzle
      const bf16x8 va = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      st.o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, st.o[n], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(NT, 2) void mla_prefill_kernel(PrefillArgs a) {
  // two stages, separate objects so the compiler can tell the in-flight copy
  // into one from reads of the other
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE_BYTES];

  // ---- which (batch, head, query tile) this workgroup owns
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const int bh = logical / a.ntiles;
  const int qt = a.ntiles - 1 - logical % a.ntiles;
  const int b = bh / a.H;
  const int q0 = qt * BM;

  Ctx c;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  c.hi = c.lane >> 5;
  c.l32 = c.lane & 31;
  c.S = a.S;
  c.P = a.past_len;
  const int64_t T = a.T;
  c.kn_g = a.k_nope + (int64_t)bh * c.S * DN;
  c.kp_g = a.k_pe + (int64_t)b * c.S * DR;
  c.v_g = a.v + (int64_t)bh * c.S * DV;
  const int64_t q0w = q0 + c.wave * 32;

  // ---- key range of the workgroup: [0, P + last query + 1)
  const int64_t q_last = (q0 + BM < T ? q0 + BM : T) - 1;
  const int64_t kend = c.P + q_last + 1;
  const int nblocks = (int)((kend + BN - 1) / BN);

  issue_tile(c, 0, stage0);

  // ---- query fragment (B operand of S^T = K Q^T): 8 dims of the lane's query per K-step
  const uint16_t* qn_g = a.q_nope + (int64_t)bh * T * DN;
  const uint16_t* qp_g = a.q_pe + (int64_t)bh * T * DR;
  bf16x8 qf[12];
  {
    const int64_t myq = q0w + c.l32;
    const int koff = 8 * c.hi;
    const bool ok = myq < T;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(ok ? ldg16(qn_g + myq * DN + 16 * kk + koff) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[8 + kk] = as_bf16x8(ok ? ldg16(qp_g + myq * DR + 16 * kk + koff) : u32x4{0, 0, 0, 0});
  }

  const bool wave_live = q0w < T;
  const int64_t wave_q_last = (q0w + 31 < T ? q0w + 31 : T - 1);
  const int64_t wave_kend = c.P + wave_q_last + 1;  // keys from here on are hidden from the wave
  const int64_t wave_kfull = c.P + q0w + 1;         // keys below are visible to the whole wave
  const float cl2 = a.scale_log2;

  State st;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[n][r] = 0.0f;
  st.m_run = -INFINITY;
  st.l_run = 0.0f;

  // ---- main loop, two tiles per trip so each stage is a fixed LDS object
  for (int j = 0; j < nblocks; j += 2) {
    wait_vmem();
    __syncthreads();  // tile j is in stage0 for everyone; stage1 is free
    if (j + 1 < nblocks) issue_tile(c, j + 1, stage1);
    {
      const int64_t kb = (int64_t)j * BN;
      if (wave_live && kb < wave_kend) compute_tile(c, qf, st, stage0, kb, q0w, wave_kfull, cl2);
    }
    if (j + 1 >= nblocks) break;
    wait_vmem();
    __syncthreads();  // tile j+1 is in stage1; stage0 is free
    if (j + 2 < nblocks) issue_tile(c, j + 2, stage0);
    {
      const int64_t kb = (int64_t)(j + 1) * BN;
      if (wave_live && kb < wave_kend) compute_tile(c, qf, st, stage1, kb, q0w, wave_kfull, cl2);
    }
  }

  // ---- epilogue: divide by the full row sum and store bf16
  if (!wave_live) return;
  const float l_tot = st.l_run + xor32(st.l_run);
  const float inv = 1.0f / l_tot;
  const int64_t myq = q0w + c.l32;
  if (myq >= T) return;
  uint16_t* out_row = a.out + ((int64_t)bh * T + myq) * DV;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv0 = 32 * n + 8 * g + 4 * c.hi;
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[n][4 * g + e] * inv);
      *reinterpret_cast<bf16x4*>(out_row + dv0) = w;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int grid = a.B * a.H * a.ntiles;
  hipLaunchKernelGGL(mla_prefill_kernel, dim3(grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

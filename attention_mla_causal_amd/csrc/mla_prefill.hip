// Causal MLA attention, prefill (any T >= 1 new queries over S = past_len + T keys).
//
// Computes, per (batch, head), softmax(scale * (q_nope k_nope^T + q_pe k_pe^T)
// + causal mask) v, as in the attention-core excerpt of the Kimi K2
// "Similarities" page ("Query-key similarity") and the "Weighted sum of
// values" page, with the mask of the "Causal mask" page: query i sits at
// absolute position past_len + i and sees keys 0..past_len+i.
//
// gfx950 design: one workgroup = 4 wave64s (one per SIMD) owning 128 queries of
// one head, 32 per wave; two workgroups share a CU, so each SIMD interleaves
// the MFMA streams of two waves from different workgroups.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K rows come from LDS as the A operand, Q stays in registers as the B
//    operand. In the 32x32 accumulator a lane owns one query (lane % 32) and
//    16 of 32 keys; lane and lane^32 share the query, so the row max is a
//    register reduction plus one v_permlane32_swap exchange.
//  * The 192-wide contraction is split 128 + 64: the last 4 K-steps read the
//    rotary key k_pe, one [S,64] tensor shared by every head; the joined
//    query/key of the pages are never built in memory.
//  * O^T = V^T P^T: P^T is the score accumulator converted to bf16, so the
//    probabilities never leave registers; V^T fragments are read from a
//    row-major V tile with ds_read_b64_tr_b16, whose key order matches the
//    accumulator's.
//  * Software pipeline over 32-key tiles: step j issues the 12 QK MFMAs of tile
//    j+1 and the 8 PV MFMAs of tile j-1 as one stream, with the softmax of tile
//    j cut into slots of a few VALU ops placed between those MFMAs (and pinned
//    there, so the compiler cannot sink them past the stream).
//  * Online softmax in fp32 in the exp2 domain (scale * log2 e folded into
//    one FMA); O is rescaled only when a running max moved. Causal tiles past
//    a wave's last query are skipped; only tiles on the diagonal are masked.
//  * K and V tiles (32 keys) are copied straight from HBM into LDS with
//    buffer_load_dwordx4 ... lds, double-buffered separately (K one tile ahead of
//    V, as the pipeline needs): one barrier per tile. Rows are stored in
//    64-byte column blocks whose 16-byte chunks are XOR-swizzled by row, which
//    keeps both the copies and the operand reads free of bank conflicts and
//    makes every operand read an immediate offset from two base registers.
//  * Workgroup order: all query tiles of one head are placed on one XCD and
//    dispatched heaviest tile first across windows of four heads, whose K/V
//    blocks stream through that XCD's L2 together. In a padded batch of
//    sequences of different lengths, (batch, head) pairs are dealt round-robin
//    over the XCDs and run longest sequence first, in windows of a few pairs.
//  * Four instantiations of one body: all keys per query tile (the common
//    case), key-range splits merged by a second kernel (small grids), a padded
//    variable-length batch (lengths read on the device), and the caller's 2D
//    padding mask (a mask byte per lane per key tile, fetched two tiles ahead
//    and turned into a wave-uniform bitmask by ballot; only the key tiles
//    between the first and last kept key are visited).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int DN = 128;   // non-rotary query/key dims
constexpr int DR = 64;    // rotary dims (shared key)
constexpr int DV = 128;   // value dims
constexpr int NW = 4;     // waves per workgroup
constexpr int NT = NW * 64;
constexpr int QW = 32;        // queries per wave (one MFMA column group)
constexpr int BM = NW * QW;   // 128 queries per workgroup
constexpr int BN = 32;        // keys per tile (one 32-key MFMA row group)
static_assert(BN == kPrefillKeyTile, "the host plans key-range splits in these tiles");

// LDS tile regions, bytes. A region of BN rows of 16-byte chunks is stored
// as column blocks of 4 chunks (64 bytes): block cb = c / 4 holds chunks
// 4cb..4cb+3 of every row, row r at offset r * 64 within the block, and the
// chunk c & 3 of row r at position (c & 3) ^ ((r >> 2) & 3) in that row.
constexpr int KN_BYTES = BN * DN * 2;  // 4 column blocks
constexpr int KP_BYTES = BN * DR * 2;  // 2 column blocks
constexpr int K_BYTES = KN_BYTES + KP_BYTES;
constexpr int V_BYTES = BN * DV * 2;   // 4 column blocks
constexpr int CB_BYTES = BN * 64;      // one column block of a tile
constexpr int CB_CHUNKS = BN * 4;

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over rows [kb, S) of one (batch, head) slice of a row-major
// [S, ROWBYTES/2] bf16 tensor. Loads past the last row return zeros (hardware
// range check), so the tile copies need no clamping. Built from uniform values
// only: scalar instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* slice, int kb, int S,
                                                           int rowbytes) {
  // 32-bit scalar arithmetic (a 64-bit compare would go through the VALU):
  // S * rowbytes < 2^31 (the host caps S) and kb <= S + 2 * BN, so the row
  // offset kb * rowbytes fits 32 bits unsigned.
  const int left = S - kb;
  const int records = left > 0 ? left * rowbytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)slice + (uint32_t)kb * (uint32_t)rowbytes), (short)0, records, 0x00020000);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// x of lane l^32 (the other half holding the same query's keys), through
// v_permlane32_swap_b32 (a VALU op; no LDS round trip). The empty asm hides
// from the optimiser that both swap operands hold the same value.
__device__ __forceinline__ float other_half(float x) {
  float y = x;
  asm volatile("" : "+v"(y));
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, y), false, false);
  // r[0]: lanes 32..63 now hold x of lanes 0..31; r[1]: lanes 0..31 hold x of lanes 32..63
  return __builtin_bit_cast(float, (unsigned)((__lane_id() < 32) ? r[1] : r[0]));
}
__device__ __forceinline__ float max_pair32(float x) { return fmaxf(x, other_half(x)); }
__device__ __forceinline__ float sum_pair32(float x) { return x + __shfl_xor(x, 32); }

__device__ __forceinline__ bf16x4 lds_tr_read(const char* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keep a value computed where it stands: without this, the optimiser sinks the
// softmax arithmetic whose results are only needed after the MFMA block out of
// it, where nothing overlaps it.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// hard scheduling fence: nothing moves across it
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until this wave's global->LDS copies have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Copy rows [kb, kb+BN) of a row-major [S, ROWLEN] bf16 tensor into an LDS
// region of NCB column blocks, in 1-KiB copies spread over the waves
// (buffer_load_dwordx4 ... lds). Each lane's source offset within the tile is a
// loop constant (voff[u]); rows past the last key read as zeros.
template <int ROWLEN, int NCB>
struct Region {
  static constexpr int NCOPY = NCB * CB_CHUNKS / 64 / NW;  // copies per wave
  static_assert(NCB * CB_CHUNKS % (64 * NW) == 0, "copies must divide evenly over the waves");
  int voff[NCOPY];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < NCOPY; ++u) {
      const int t = u * NW + wave;
      const int pc = t * 64 + lane;  // physical chunk within the region
      const int cb = pc / CB_CHUNKS;
      const int r = (pc >> 2) % BN;
      const int c4 = (pc & 3) ^ ((r >> 2) & 3);
      voff[u] = r * ROWLEN * 2 + (cb * 4 + c4) * 16;
    }
  }
  __device__ __forceinline__ void copy(const uint16_t* slice, int kb, int S, char* lds,
                                       int wave) const {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(slice, kb, S, ROWLEN * 2);
#pragma unroll
    for (int u = 0; u < NCOPY; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (u * NW + wave) * 1024), 16,
                                               voff[u], 0, 0, 0);
  }
};

struct Geo {
  const uint16_t* kn_g;
  const uint16_t* kp_g;
  const uint16_t* v_g;
  int64_t S, P;
  int S32;  // S as a 32-bit count, for the copies' scalar arithmetic
  int wave, lane;
  Region<DN, 4> kn;
  Region<DR, 2> kp;
  Region<DV, 4> vv;
};

__device__ __forceinline__ void copy_k(const Geo& g, int j, char* kbuf) {
  const int kb = j * BN;
  g.kn.copy(g.kn_g, kb, g.S32, kbuf, g.wave);
  g.kp.copy(g.kp_g, kb, g.S32, kbuf + KN_BYTES, g.wave);
}

__device__ __forceinline__ void copy_v(const Geo& g, int j, char* vbuf) {
  g.vv.copy(g.v_g, j * BN, g.S32, vbuf, g.wave);
}

// Per-lane LDS operand offsets (bytes) for the region layout above.
struct Lane {
  int ka_even, ka_odd;  // K fragment of rows l32 for even / odd K-steps
  int va0, va1;         // V^T pieces: keys 16ks + 4hi + (l&15)/4 and + 8
};

// K fragment (A operand) for K-step kk (0..11) from a K tile.
__device__ __forceinline__ bf16x8 k_frag(const char* kbuf, const Lane& ln, int kk) {
  const int region = kk < 8 ? 0 : KN_BYTES;  // k_nope, then the shared k_pe
  const int kq = kk < 8 ? kk : kk - 8;
  return lds_read16(kbuf + region + (kq >> 1) * CB_BYTES + ((kq & 1) ? ln.ka_odd : ln.ka_even));
}

// V^T fragment (A operand) for K-step ks (16 keys) and dv tile n, from a V tile.
__device__ __forceinline__ bf16x8 v_frag(const char* vbuf, const Lane& ln, int ks, int n) {
  const char* p = vbuf + n * CB_BYTES + ks * 16 * 64;
  const bf16x4 lo4 = lds_tr_read(p + ln.va0);
  const bf16x4 hi4 = lds_tr_read(p + ln.va1);
  return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
}

struct Acc {
  f32x16 o[4];  // O^T accumulators: the lane's query, 64 of its 128 dims
  float m_run;  // running max, scaled log2 domain
  float l_run;  // this lane's share of the running sum
};

// Softmax of one tile (S^T in c: 32 keys x 32 queries; the lane holds 16
// keys of its query), cut into slots of a few VALU ops that are spread between
// the MFMAs of a pipeline step.
struct Smx {
  float mx, m_ref, alpha, psum;
};
constexpr int SMX_SLOTS = 19;

template <int SLOT>
__device__ __forceinline__ void smx_slot(Smx& st, f32x16& c, bf16x8 (&pc)[2], Acc& acc,
                                         float cl2) {
  if constexpr (SLOT < 4) {  // running max of the raw scores, 4 per slot
#pragma unroll
    for (int r = 4 * SLOT; r < 4 * SLOT + 4; ++r) st.mx = fmaxf(st.mx, c[r]);
  } else if constexpr (SLOT == 4) {  // new running max (cl2 > 0) and rescale factor
    const float mx = max_pair32(st.mx);
    const float m_new = fmaxf(acc.m_run, mx * cl2);
    st.m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    st.alpha = __builtin_amdgcn_exp2f(acc.m_run - st.m_ref);
    acc.m_run = m_new;
  } else if constexpr (SLOT < 13) {  // p = 2^(scale*log2e*s - m), 2 per slot
#pragma unroll
    for (int r = 2 * (SLOT - 5); r < 2 * (SLOT - 5) + 2; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(c[r], cl2, -st.m_ref));
      pin(p);
      c[r] = p;
    }
  } else if constexpr (SLOT < 17) {  // row-sum share, 4 per slot
#pragma unroll
    for (int r = 4 * (SLOT - 13); r < 4 * (SLOT - 13) + 4; ++r) st.psum += c[r];
    pin(st.psum);
    if constexpr (SLOT == 16) acc.l_run = acc.l_run * st.alpha + st.psum;
  } else if constexpr (SLOT < SMX_SLOTS) {  // bf16 P^T operand for K-step ks
    constexpr int ks = SLOT - 17;
#pragma unroll
    for (int e = 0; e < 8; ++e) pc[ks][e] = (__bf16)c[8 * ks + e];
    pin(pc[ks]);
  }
}

// Hide keys past each lane's query (and past the last key) on a diagonal tile:
// key kb + off is visible iff off <= min(lim, S - 1) - kb (computed once, 32-bit).
__device__ __forceinline__ void mask_tile(f32x16& sc, int64_t kb, int64_t lim, int64_t S, int hi) {
  const int64_t last = (lim < S - 1 ? lim : S - 1) - kb;
  const int thr = last < -1 ? -1 : (last > BN ? BN : (int)last);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + 4 * hi + (r & 3);
    if (off > thr) sc[r] = -INFINITY;
  }
}

// One pipeline step's MFMA stream, 20 phases with one MFMA each: phases
// 0..11 are the QK K-steps of the next tile (A = K fragment), phases 12..19
// the PV MFMAs of the previous tile (A = V^T fragment, K-step (p-12)/4, dv
// tile (p-12)%4). Operand fragments are read from LDS RING-1 phases ahead
// through a ring of RING registers, so LDS latency hides behind MFMAs; the
// softmax slot SLOT0+p is issued in phase p (SLOT0 < 0: none). WITH_QK /
// WITH_PV select the parts that run.
#ifndef MLA_PREFILL_RING
#define MLA_PREFILL_RING 4
#endif
constexpr int RING = MLA_PREFILL_RING;

template <bool WITH_QK, bool WITH_PV>
__device__ __forceinline__ bf16x8 stream_frag(int p, const char* kbuf, const char* vbuf,
                                              const Lane& ln) {
  constexpr int first = WITH_QK ? 0 : 12;
  (void)first;
  if (p < 12) return k_frag(kbuf, ln, p);
  const int q = p - 12;
  return v_frag(vbuf, ln, q >> 2, q & 3);
}

template <int SLOT0, bool WITH_QK, bool WITH_PV>
__device__ __forceinline__ void mfma_stream(f32x16& s, const char* kbuf, Acc& acc,
                                            const char* vbuf, const Lane& ln,
                                            const bf16x8 (&qf)[12], const bf16x8 (&pp)[2],
                                            Smx& st, f32x16& c, bf16x8 (&pc)[2], float cl2) {
  constexpr int P0 = WITH_QK ? 0 : 12;
  constexpr int P1 = WITH_PV ? 20 : 12;
  if constexpr (WITH_QK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
  }
  bf16x8 fr[RING];
#pragma unroll
  for (int p = P0; p < P0 + RING - 1 && p < P1; ++p) fr[p % RING] = stream_frag<WITH_QK, WITH_PV>(p, kbuf, vbuf, ln);
  fence();
#pragma unroll
  for (int p = P0; p < P1; ++p) {
    if (p + RING - 1 < P1) fr[(p + RING - 1) % RING] = stream_frag<WITH_QK, WITH_PV>(p + RING - 1, kbuf, vbuf, ln);
    if (p < 12)
      s = mfma(fr[p % RING], qf[p], s);
    else
      acc.o[(p - 12) & 3] = mfma(fr[p % RING], pp[(p - 12) >> 2], acc.o[(p - 12) & 3]);
    if constexpr (SLOT0 >= 0) {
#define MLA_SLOT(K) if (p == K) smx_slot<SLOT0 + K>(st, c, pc, acc, cl2);
      MLA_SLOT(0) MLA_SLOT(1) MLA_SLOT(2) MLA_SLOT(3) MLA_SLOT(4) MLA_SLOT(5) MLA_SLOT(6)
      MLA_SLOT(7) MLA_SLOT(8) MLA_SLOT(9) MLA_SLOT(10) MLA_SLOT(11) MLA_SLOT(12) MLA_SLOT(13)
      MLA_SLOT(14) MLA_SLOT(15) MLA_SLOT(16) MLA_SLOT(17) MLA_SLOT(18) MLA_SLOT(19)
#undef MLA_SLOT
    }
    fence();
  }
}

// Remaining softmax slots, run back to back (no MFMA work to hide them behind).
template <int SLOT, int END>
__device__ __forceinline__ void smx_rest(Smx& st, f32x16& c, bf16x8 (&pc)[2], Acc& acc,
                                         float cl2) {
  if constexpr (SLOT < END) {
    smx_slot<SLOT>(st, c, pc, acc, cl2);
    smx_rest<SLOT + 1, END>(st, c, pc, acc, cl2);
  }
}

// O *= alpha when some query of the wave raised its max (rare after the first tiles).
__device__ __forceinline__ void rescale_o(Acc& acc, float alpha) {
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.o[n][r] *= alpha;
  }
}

// Split mode, a workgroup whose key range the query tile never reaches: the
// empty partial (0, -inf, 0) for each of its rows, so the merge can read
// every split.
__device__ __forceinline__ void write_empty_partials(const PrefillArgs& a, int bh, int q0, int sp) {
  static_assert(NT == 2 * BM, "two threads per query row");
  const int64_t T = a.T;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;  // 128 rows x 2 halves of 64 dims
  const int64_t q = q0 + r;
  if (q >= T) return;
  const int64_t slot = ((int64_t)bh * T + q) * a.nsplit + sp;
  float* po = a.ws_o + slot * DV + 64 * half;
#pragma unroll
  for (int e = 0; e < 64; e += 4) *reinterpret_cast<f32x4*>(po + e) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (half == 0) *reinterpret_cast<f32x2*>(a.ws_ml + 2 * slot) = f32x2{-INFINITY, 0.0f};
}

// Padded variable-length batch: zero the output rows [r0, r1) of one (b, h)
// slice (query rows past the sequence's own count), 16 bytes per store.
__device__ __forceinline__ void zero_rows(uint16_t* out, int64_t r0, int64_t r1) {
  constexpr int CHUNKS = DV * 2 / 16;  // 16-byte chunks per row
  const int64_t n = (r1 - r0) * CHUNKS;
  u32x4* base = reinterpret_cast<u32x4*>(out + r0 * DV);
  for (int64_t c = threadIdx.x; c < n; c += NT) base[c] = u32x4{0, 0, 0, 0};
}

enum { kDense = 0, kSplit = 1, kVarlen = 2, kMasked = 3 };

// 2D mask: the first and last kept key among keys [0, limit) of one mask row
// (first > last when none is kept), over all threads of the workgroup. Rows
// that start on a 4-byte boundary are read a dword at a time, others a byte at
// a time. All threads must call it.
__device__ __forceinline__ void kept_key_range(const uint8_t* row, int64_t limit, int64_t& first,
                                               int64_t& last) {
  __shared__ int64_t s_first[NW], s_last[NW];
  int64_t f = INT64_MAX, l = -1;
  if ((reinterpret_cast<uintptr_t>(row) & 3) == 0) {
    const int64_t nw = limit / 4;
    const uint32_t* row4 = reinterpret_cast<const uint32_t*>(row);
    for (int64_t w = threadIdx.x; w < nw; w += NT) {
      const uint32_t x = row4[w];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((x >> (8 * e)) & 0xffu) {
          f = f < 4 * w + e ? f : 4 * w + e;
          l = l > 4 * w + e ? l : 4 * w + e;
        }
    }
    for (int64_t j = 4 * nw + threadIdx.x; j < limit; j += NT)
      if (row[j]) {
        f = f < j ? f : j;
        l = l > j ? l : j;
      }
  } else {
    for (int64_t j = threadIdx.x; j < limit; j += NT)
      if (row[j]) {
        f = f < j ? f : j;
        l = l > j ? l : j;
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int64_t f2 = __shfl_xor(f, off), l2 = __shfl_xor(l, off);
    f = f < f2 ? f : f2;
    l = l > l2 ? l : l2;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_first[wave] = f;
    s_last[wave] = l;
  }
  __syncthreads();
  first = s_first[0];
  last = s_last[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    first = first < s_first[w] ? first : s_first[w];
    last = last > s_last[w] ? last : s_last[w];
  }
}

// The caller's 2D padding mask on one score tile. kbyte is this lane's mask
// byte for key (lane % 32) of the tile; a ballot turns the 32 bytes into one
// wave-uniform bit per key, and the lane hides its 16 keys (8g + 4hi + e) whose
// bit is clear. A tile with every key kept costs the ballot and one compare.
__device__ __forceinline__ void key_mask_tile(f32x16& sc, uint32_t kbyte, int hi) {
  const uint32_t vis = (uint32_t)__ballot(kbyte != 0);
  if (vis == 0xffffffffu) return;
  const uint32_t m = vis >> (4 * hi);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + (r & 3);
    if (!((m >> off) & 1u)) sc[r] = -INFINITY;
  }
}

// Padded variable-length batch: sequence b's query count and cached keys,
// clamped as the kernel uses them (T to [0, Tst], past to [0, Sst - T]).
__device__ __forceinline__ void seq_lens_of(const PrefillArgs& a, int b, int64_t& T, int64_t& past) {
  const int64_t tq = a.q_lens[b], pl = a.past_lens[b];
  T = tq < 0 ? 0 : (tq > a.T ? a.T : tq);
  past = pl < 0 ? 0 : (pl > a.S - T ? a.S - T : pl);
}

// Beyond this batch size (one sequence per thread) the sequences are taken
// in index order.
constexpr int kMaxRankedBatch = NT;

// The sequence at position r when sequences are ordered by visible (query,
// key) pairs, most first (ties by index), so the longest jobs start first.
// Thread t computes sequence t's pair count into LDS, then ranks it against
// all others there; the one whose rank is r publishes itself. All threads of
// the workgroup must call it.
__device__ __forceinline__ int seq_at_rank(const PrefillArgs& a, int r) {
  __shared__ int64_t s_work[kMaxRankedBatch];
  __shared__ int s_seq;
  if (a.B > kMaxRankedBatch) return r;
  const int t = threadIdx.x;
  int64_t wt = 0;
  if (t < a.B) {
    int64_t T, P;
    seq_lens_of(a, t, T, P);
    wt = T * P + T * (T + 1) / 2;
    s_work[t] = wt;
  }
  __syncthreads();
  if (t < a.B) {
    int rank = 0;
    for (int u = 0; u < a.B; ++u) {
      const int64_t wu = s_work[u];
      rank += (wu > wt || (wu == wt && u < t)) ? 1 : 0;
    }
    if (rank == r) s_seq = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_seq);
}

// MODE kSplit: the workgroup covers one key range of its query tile and writes
// an fp32 partial (merged by mla_prefill_merge_kernel). kDense: all keys and
// the bf16 output. kVarlen: as kDense, with each sequence's query and key
// counts read from device memory and the padded query rows set to zero. One
// instantiation each, so the dense kernel carries none of the others' code.
template <int MODE>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a) {
  constexpr bool SPLIT = MODE == kSplit;
  constexpr bool VARLEN = MODE == kVarlen;
  constexpr bool MASKED = MODE == kMasked;
  // separate LDS objects per buffer so the compiler can tell an in-flight copy
  // into one from reads of another
  __shared__ __attribute__((aligned(1024))) char kbuf0[K_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[V_BYTES];

  // ---- which (batch, head, query tile) this workgroup owns
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  // Each XCD (wg % 8) takes a contiguous range of heads and dispatches their
  // query tiles heaviest first (longest-job-first) across windows of four
  // heads, so the window's K/V streams through the XCD's L2 together; when
  // the XCD's head count is not a multiple of four, across all of its heads
  // if the tiles differ a lot in work (few cached keys: the causal triangle
  // dominates), else head by head.
  int bh, qt, sp = 0;
  const bool uneven = 2 * (a.past_len + (int64_t)BM) < a.past_len + (int64_t)a.T;
  if (VARLEN || MASKED) {
    // (b, h) groups dealt round-robin over the XCDs (each XCD gets H/8 heads
    // of every sequence when H is a multiple of 8, so the XCDs stay even
    // whatever the lengths); each XCD runs its groups longest sequence first,
    // kWindow groups at a time: the window's query tiles heaviest first
    // across its groups, so its K/V streams through that XCD's L2 while it
    // runs. (One group at a time left the heaviest tiles of each XCD's last
    // groups to start near the end. Windows of four took the 2D-mask prefill
    // from 1.065 to 1.019 ms (HBM reads +23%); on the padded batch, whose
    // sequences are four times longer, windows of two gain 3% (reads +17%)
    // where four read 65% more for no more gain. Outputs bit-identical.
    // Windows of 16 groups, or all of an XCD's, lose it all to K/V re-read
    // past L2.)
    // With a 2D mask the padding, and so the work, differs by sequence in a
    // way the grid cannot see: the groups are dealt round-robin over the XCDs
    // the same way, in index order.
    constexpr int kWindow = MASKED ? 4 : 2;
    const int G = a.B * a.H;
    int gi, t;
    if (G % (8 * kWindow) == 0) {
      const int i = wg / 8, r = i % (kWindow * a.ntiles);
      gi = ((i / (kWindow * a.ntiles)) * kWindow + r % kWindow) * 8 + wg % 8;
      t = r / kWindow;
    } else if (G % 8 == 0) {
      gi = (wg / 8 / a.ntiles) * 8 + wg % 8;
      t = (wg / 8) % a.ntiles;
    } else {
      gi = wg / a.ntiles;
      t = wg % a.ntiles;
    }
    const int seq = VARLEN ? seq_at_rank(a, gi / a.H) : gi / a.H;
    bh = seq * a.H + gi % a.H;
    qt = a.ntiles - 1 - t;
  } else {
    const int per = nwg / 8, i = wg / 8;
    if (SPLIT) {
      // key-range splits of one query tile are adjacent (same XCD when the
      // grid is a multiple of 8), then query tiles, then heads. A head's
      // query tiles run heaviest first over the first half of its positions
      // and lightest first over the second, so the two workgroups an XCD
      // deals to one CU (positions k and k + 32 of its 64) pair a heavy tile
      // with a light one (plain heaviest first: 4096 queries without cached
      // keys, 8 heads, 75.0 -> 70.5 us, same process).
      const int logical = (nwg % 8 == 0) ? (wg % 8) * per + i : wg;
      sp = logical % a.nsplit;
      const int rest = logical / a.nsplit;
      bh = rest / a.ntiles;
      const int k = rest % a.ntiles, h1 = (a.ntiles + 1) / 2;
      qt = k < h1 ? a.ntiles - 1 - k : k - h1;
    } else if (nwg % 8 == 0 && per % a.ntiles == 0 && (uneven || (per / a.ntiles) % 4 == 0)) {
      // An XCD deals its workgroups to its 32 CUs in turn, two resident per
      // CU; the first window's tiles fill the first round and the next
      // window's start heaviest first as slots free. Same process, outputs
      // bit-identical: 2048 queries over 14336 cached keys, 64 heads: 1203 us
      // head by head, 1185 us in windows of four (L2 misses +60%, still under
      // a tenth of HBM peak); windows of two no faster than head by head,
      // windows of eight no faster than four with three times the misses of
      // head by head. 4096 queries, no cached keys: windows of four 1%
      // faster than all eight heads of the XCD at once, 35% fewer L2 misses.
      const int nh = per / a.ntiles;
      const int W = nh % 4 == 0 ? 4 : nh;
      const int r = i % (W * a.ntiles);
      bh = (wg % 8) * nh + (i / (W * a.ntiles)) * W + r % W;
      qt = a.ntiles - 1 - r / W;
    } else {
      const int logical = (nwg % 8 == 0) ? (wg % 8) * per + i : wg;
      bh = logical / a.ntiles;
      qt = a.ntiles - 1 - logical % a.ntiles;
    }
  }
  const int b = bh / a.H;
  const int q0 = qt * BM;
  // Tst / Sst: rows per (b, h) slice of the queries and output / of the keys.
  // T, S_seq, past: this sequence's query count, key count and cached keys
  // (the same as the slice sizes except for a padded variable-length batch).
  const int64_t Tst = a.T, Sst = a.S;
  int64_t T = a.T, S_seq = a.S, past = a.past_len;
  if (VARLEN) {
    seq_lens_of(a, b, T, past);
    S_seq = past + T;
    if (q0 >= T) {  // every row of this tile is padding
      const int64_t r1 = q0 + BM < Tst ? q0 + BM : Tst;
      zero_rows(a.out + (int64_t)bh * Tst * DV, q0, r1);
      return;
    }
  }

  Geo geo;
  const int tid = threadIdx.x;
  geo.lane = tid & 63;
  geo.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = geo.lane, hi = lane >> 5, l32 = lane & 31;
  const int64_t q0w = q0 + geo.wave * QW;

  // ---- key range of the workgroup: tiles [kt0, kt1) of [0, P + last query + 1)
  const int64_t q_last = (q0 + BM < T ? q0 + BM : T) - 1;
  const int nblocks_all = (int)((past + q_last + 1 + BN - 1) / BN);
  int kt0 = 0, kt1 = nblocks_all;
  if (SPLIT) {
    // the tile's visible key tiles in nsplit near-equal ranges (ranges of the
    // whole key count left the last range of every tile light: 4096 queries
    // without cached keys, 8 heads, 79.8 -> 75.0 us, same process)
    const int tps = (nblocks_all + a.nsplit - 1) / a.nsplit;
    kt0 = sp * tps;
    kt1 = kt0 + tps < nblocks_all ? kt0 + tps : nblocks_all;
  }
  if (MASKED) {
    // only the tiles between the first and the last key the 2D mask keeps
    // (of those the tile's queries can see) are visited: leading padding
    // costs a scan of its mask bytes, not its attention
    int64_t first, last;
    kept_key_range(a.key_mask + (int64_t)b * Sst, past + q_last + 1, first, last);
    if (first > last) {  // no query of this tile sees a kept key
      const int64_t r1 = q0 + BM < T ? q0 + BM : T;
      zero_rows(a.out + (int64_t)bh * Tst * DV, q0, r1);
      return;
    }
    kt0 = (int)(first / BN);
    kt1 = (int)(last / BN) + 1;
  }
  const int nblocks = kt1 - kt0;
  if (SPLIT && nblocks <= 0) {  // no key of this range is visible to the tile
    write_empty_partials(a, bh, q0, sp);
    return;
  }
  // Everything below sees keys relative to k0: the key slices start at row k0,
  // and the last key query i sees is P + i with P = past_len - k0 (< 0 when the
  // query sees no key of this range).
  const int64_t k0 = (int64_t)kt0 * BN;
  geo.S = S_seq - k0;
  geo.S32 = (int)geo.S;
  geo.P = past - k0;
  geo.kn_g = a.k_nope + (int64_t)bh * Sst * DN + k0 * DN;
  geo.kp_g = a.k_pe + (int64_t)b * Sst * DR + k0 * DR;
  geo.v_g = a.v + (int64_t)bh * Sst * DV + k0 * DV;
  geo.kn.init(geo.wave, geo.lane);
  geo.kp.init(geo.wave, geo.lane);
  geo.vv.init(geo.wave, geo.lane);
  const int64_t S = geo.S, P = geo.P;
  const int64_t wq_last = q0w + QW - 1 < T ? q0w + QW - 1 : T - 1;
  // a wave computes when some query of it sees a key of the range; its tile 0
  // then always holds a visible key (key 0 of the range)
  const bool wave_live = q0w < T && P + wq_last >= 0;
  // last tile holding a key that some query of this wave sees (-1: none)
  const int wave_last = wave_live ? (int)((P + wq_last) / BN) : -1;
  const int64_t lim = P + q0w + l32;  // last key this lane's query sees

  copy_k(geo, 0, kbuf0);

  // ---- 2D padding mask: each lane fetches one byte per key tile, key
  // (lane % 32) of the tile, two tiles ahead of its use (with the K copies);
  // bytes past the sequence's keys read as 0 (buffer range check).
  __amdgpu_buffer_rsrc_t mrs;
  uint32_t km0 = 0, km1 = 0;  // mask bytes of even / odd tiles
  auto load_km = [&](int t) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b8(mrs, t * BN + (geo.lane & 31), 0, 0);
  };
  if (MASKED) {
    const int64_t left = S_seq - k0;
    mrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.key_mask + (int64_t)b * Sst + k0), (short)0,
                                            left > 0 ? (int)left : 0, 0x00020000);
    km0 = load_km(0);
    km1 = load_km(1);
  }

  // ---- any finite softmax_scale. The softmax below takes the running max of
  // the unscaled scores and scales it by cl2 = scale * log2(e), which needs
  // cl2 > 0. A negative scale gives the same scaled scores as |scale| with the
  // query negated (scale * q.k = |scale| * (-q).k; flipping bf16 sign bits is
  // exact); a zero scale gives every visible key the same score 0, as a zero
  // query with cl2 = 1 does. So the query fragments are sign-flipped or
  // cleared once here and the loop always runs with a positive cl2.
  const float cl2_in = a.scale_log2;
  const uint32_t q_and = cl2_in == 0.0f ? 0u : 0xffffffffu;
  const uint32_t q_xor = cl2_in < 0.0f ? 0x80008000u : 0u;
  const float cl2 = cl2_in == 0.0f ? 1.0f : __builtin_fabsf(cl2_in);

  // ---- query fragments (B operand): 8 dims of the lane's query per K-step
  bf16x8 qf[12];
  {
    const int64_t myq = q0w + l32;
    const bool ok = myq < T;
    const uint16_t* qn = a.q_nope + ((int64_t)bh * Tst + myq) * DN + 8 * hi;
    const uint16_t* qp = a.q_pe + ((int64_t)bh * Tst + myq) * DR + 8 * hi;
    auto signed_q = [&](u32x4 w) { return as_bf16x8((w & q_and) ^ q_xor); };
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = signed_q(ok ? ldg16(qn + 16 * kk) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[8 + kk] = signed_q(ok ? ldg16(qp + 16 * kk) : u32x4{0, 0, 0, 0});
  }

  Lane ln;
  {
    const int x = (l32 >> 2) & 3;
    ln.ka_even = l32 * 64 + ((hi) ^ x) * 16;
    ln.ka_odd = l32 * 64 + ((2 + hi) ^ x) * 16;
    const int sl = lane & 15, grp = (lane >> 4) & 1;
    const int vrow = 4 * hi + (sl >> 2);
    const int vc4 = 2 * grp + ((sl & 3) >> 1);
    ln.va0 = vrow * 64 + ((vc4 ^ hi) * 16) + 8 * (sl & 1);
    ln.va1 = (vrow + 8) * 64 + ((vc4 ^ (hi + 2)) * 16) + 8 * (sl & 1);
  }

  Acc acc;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc.o[n][r] = 0.0f;
  acc.m_run = -INFINITY;
  acc.l_run = 0.0f;

  auto needs_mask = [&](int j) { return (int64_t)j * BN + BN > P + q0w + 1; };

  // ---- pipeline. Step j: QK of tile j+1, softmax of tile j, PV of tile j-1.
  // Tile t's K lives in kbuf[t % 2], its V in vbuf[t % 2]; step j issues the
  // copies of K_{j+2} and V_j (V trails K by two tiles).
  f32x16 sa, sb;         // scores of alternating tiles
  bf16x8 pa[2], pb[2];   // P^T operands of alternating tiles
  Smx st;
  copy_k(geo, 1 < nblocks ? 1 : 0, kbuf1);
  wait_vmem();
  __syncthreads();
  if (wave_live) {
    mfma_stream<-1, true, false>(sa, kbuf0, acc, vbuf0, ln, qf, pa, st, sb, pb, cl2);
    if (needs_mask(0)) mask_tile(sa, 0, lim, S, hi);
    if (MASKED) key_mask_tile(sa, km0, hi);
  }

  // step 0: QK of tile 1 with the softmax of tile 0; no PV yet
  wait_vmem();
  __syncthreads();
  if (2 < nblocks) copy_k(geo, 2, kbuf0);
  copy_v(geo, 0, vbuf0);
  if (MASKED) km0 = load_km(2);
  if (wave_live) {
    st.mx = -INFINITY;
    st.psum = 0.0f;
    mfma_stream<0, true, false>(sb, kbuf1, acc, vbuf0, ln, qf, pb, st, sa, pa, cl2);
    smx_rest<12, SMX_SLOTS>(st, sa, pa, acc, cl2);
    rescale_o(acc, st.alpha);
    if (needs_mask(1)) mask_tile(sb, BN, lim, S, hi);
    if (MASKED) key_mask_tile(sb, km1, hi);
  }

  // steps j >= 1
  auto step = [&](int j, f32x16& cur, f32x16& nxt, bf16x8 (&pcur)[2],
                  const bf16x8 (&pprev)[2], const char* knxt, const char* vprev, char* kfree,
                  char* vfree, uint32_t& km_apply, uint32_t& km_load) {
    // Issue priority toggles with the parity of step and workgroup index, so
    // workgroups sharing a CU take turns once their steps drift apart. Left
    // to age-based arbitration, the older one ran ~25% faster per step and
    // the round of workgroups that follows ended unevenly. (Same process: no
    // s_setprio 1.7% slower on the chunked prefill; keying the parity so the
    // two workgroups a CU receives first alternate from the start, 0.8%
    // slower.)
    if ((j + blockIdx.x) & 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    wait_vmem();
    __syncthreads();  // K_{j+1} and V_{j-1} have landed; kfree and vfree are no longer read
    if (j + 2 < nblocks) copy_k(geo, j + 2, kfree);
    copy_v(geo, j, vfree);
    if (MASKED) km_load = load_km(j + 2);  // tile j+2's register was freed by tile j
    if (j <= wave_last + 1) {
      st.mx = -INFINITY;
      st.psum = 0.0f;
      // QK of tile j+1 and PV of tile j-1, with the softmax of tile j in between
      mfma_stream<0, true, true>(nxt, knxt, acc, vprev, ln, qf, pprev, st, cur, pcur, cl2);
      rescale_o(acc, st.alpha);
      if (needs_mask(j + 1)) mask_tile(nxt, (int64_t)(j + 1) * BN, lim, S, hi);
      if (MASKED) key_mask_tile(nxt, km_apply, hi);
    }
  };

  // Register roles alternate: odd steps read scores from sb and P^T from pa
  // and write sa / pb; even steps the reverse. The loop is unrolled by two so
  // that every LDS buffer and register role is fixed in each copy of the step.
  int j = 1;
  // (j odd: tile j+1 is even and its mask byte is in km0; tile j+2 is odd.)
  for (; j + 1 < nblocks; j += 2) {
    step(j, sb, sa, pb, pa, kbuf0, vbuf0, kbuf1, vbuf1, km0, km1);
    step(j + 1, sa, sb, pa, pb, kbuf1, vbuf1, kbuf0, vbuf0, km1, km0);
  }
  if (j < nblocks) step(j, sb, sa, pb, pa, kbuf0, vbuf0, kbuf1, vbuf1, km0, km1);

  // ---- drain: PV of the last tile
  wait_vmem();
  __syncthreads();
  if (nblocks - 1 <= wave_last) {
    // the last step (j = nblocks-1) left tile j's P^T in pb if j is odd, pa if even
    if ((nblocks - 1) & 1)
      mfma_stream<-1, false, true>(sb, kbuf0, acc, vbuf1, ln, qf, pb, st, sa, pa, cl2);
    else
      mfma_stream<-1, false, true>(sb, kbuf0, acc, vbuf0, ln, qf, pa, st, sa, pb, cl2);
  }

  if (SPLIT) {
    // ---- split epilogue: the unnormalised partial and the row's (max, sum);
    // a wave that saw no key writes the empty partial (0, -inf, 0)
    if (q0w >= T) return;
    const float l_tot = sum_pair32(acc.l_run);
    const int64_t myq = q0w + l32;
    if (myq >= T) return;
    const int64_t slot = ((int64_t)bh * Tst + myq) * a.nsplit + sp;
    float* po = a.ws_o + slot * DV;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int dv0 = 32 * n + 8 * gg + 4 * hi;
        *reinterpret_cast<f32x4*>(po + dv0) =
            f32x4{acc.o[n][4 * gg], acc.o[n][4 * gg + 1], acc.o[n][4 * gg + 2], acc.o[n][4 * gg + 3]};
      }
    if (hi == 0) *reinterpret_cast<f32x2*>(a.ws_ml + 2 * slot) = f32x2{acc.m_run, l_tot};
    return;
  }

  // ---- epilogue: divide by the full row sum and store bf16; in a padded
  // batch, rows past the sequence's query count (still inside the slice) get 0
  const int64_t myq = q0w + l32;
  // rows written as 0: padded query rows of a variable-length batch, and with
  // a 2D mask the rows of a wave that sees no kept key
  const bool pad_row = (VARLEN && myq >= T && myq < Tst) || (MASKED && !wave_live && myq < T);
  if (!wave_live && !pad_row) return;
  float inv = 0.0f;
  if (wave_live) {
    const float l_tot = sum_pair32(acc.l_run);
    // with a 2D mask a row may see no key at all: its output is 0
    inv = (MASKED && !(l_tot > 0.0f)) ? 0.0f : 1.0f / l_tot;
  }
  if (myq >= T && !pad_row) return;
  uint16_t* out_row = a.out + ((int64_t)bh * Tst + myq) * DV;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int dv0 = 32 * n + 8 * gg + 4 * hi;
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pad_row ? (__bf16)0.0f : (__bf16)(acc.o[n][4 * gg + e] * inv);
      *reinterpret_cast<bf16x4*>(out_row + dv0) = w;
    }
}

__global__ __launch_bounds__(NT, 2) void mla_prefill_kernel(PrefillArgs a) { prefill_body<kDense>(a); }
__global__ __launch_bounds__(NT, 2) void mla_prefill_split_kernel(PrefillArgs a) { prefill_body<kSplit>(a); }
__global__ __launch_bounds__(NT, 2) void mla_prefill_varlen_kernel(PrefillArgs a) { prefill_body<kVarlen>(a); }
__global__ __launch_bounds__(NT, 2) void mla_prefill_masked_kernel(PrefillArgs a) { prefill_body<kMasked>(a); }

// Log-sum-exp merge of the key-range partials of every query row: 32 lanes
// per row, lane c owning output dims 4c..4c+3, eight rows per workgroup. All
// of a row's partial loads (at most kMergeMaxSplits ranges) issue before any
// is used; the sums run over the ranges in order.
constexpr int kMergeMaxSplits = 16;  // the host plans at most this many key ranges
__global__ __launch_bounds__(256) void mla_prefill_merge_kernel(PrefillArgs a) {
  const int64_t rows = (int64_t)a.B * a.H * a.T;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const int c = threadIdx.x & 31;
  const float* ml = a.ws_ml + row * a.nsplit * 2;
  const float* po = a.ws_o + row * a.nsplit * DV + 4 * c;
  f32x2 mls[kMergeMaxSplits];
  f32x4 ps[kMergeMaxSplits];
#pragma unroll
  for (int s = 0; s < kMergeMaxSplits; ++s) {
    mls[s] = f32x2{-INFINITY, 0.0f};
    ps[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (s < a.nsplit) {
      mls[s] = *reinterpret_cast<const f32x2*>(ml + 2 * s);
      ps[s] = *reinterpret_cast<const f32x4*>(po + (int64_t)s * DV);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMergeMaxSplits; ++s) M = fmaxf(M, mls[s][0]);
  float L = 0.0f;
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kMergeMaxSplits; ++s) {
    const float m = mls[s][0];
    const float w = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    L = __builtin_fmaf(w, mls[s][1], L);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(w, ps[s][e], o[e]);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  bf16x4 w4;
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(o[e] * inv);
  *reinterpret_cast<bf16x4*>(a.out + row * DV + 4 * c) = w4;
}

}  // namespace

int prefill_block_m() { return BM; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.q_lens != nullptr) {
    hipLaunchKernelGGL(mla_prefill_varlen_kernel, dim3(a.B * a.H * a.ntiles), dim3(NT), 0, stream, a);
  } else if (a.key_mask != nullptr) {
    hipLaunchKernelGGL(mla_prefill_masked_kernel, dim3(a.B * a.H * a.ntiles), dim3(NT), 0, stream, a);
  } else if (a.nsplit <= 1) {
    hipLaunchKernelGGL(mla_prefill_kernel, dim3(a.B * a.H * a.ntiles), dim3(NT), 0, stream, a);
  } else {
    hipLaunchKernelGGL(mla_prefill_split_kernel, dim3(a.B * a.H * a.ntiles * a.nsplit), dim3(NT), 0,
                       stream, a);
    const int64_t rows = (int64_t)a.B * a.H * a.T;
    hipLaunchKernelGGL(mla_prefill_merge_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla

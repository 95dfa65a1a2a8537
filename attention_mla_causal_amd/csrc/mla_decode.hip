// Causal MLA attention, decode (one new query per sequence, S = past_len + 1 keys).
// Also serves decode over a preallocated, right-padded cache: sequence b then
// attends over rows [0, seq_lens[b]) of cache slices of `cap` rows (the 2D
// padding mask that the "Causal mask" page's "Construct causal mask" hands
// to the 4D mask builder, for right padding); a sequence with no key gives 0.
// The cache may be paged (blocks named by a table per sequence), and the new
// token's key and value may be appended by the call itself (the cache update
// the "Similarities" page runs before attending). A second instantiation
// takes the caller's general 2D padding mask ([B, S] bytes, nonzero keeps):
// it takes the mask bytes of eight trips at a time (one group ahead) as ballot
// bits and loads only kept rows. A
// third fuses the rotary prologue: the new token's query (and appended key)
// turns at its position in registers, from a cos/sin table, before scoring.
//
// The same computation as prefill with T = 1 (the Kimi K2 "Similarities"
// page shows it in decode mode with p = 1000: scores [B, 64, 1, 1001]); the
// single query sees every key, so the causal mask is all zeros here. The work
// is a pair of matrix-vector products per (b, h) and is bound by HBM
// bandwidth: it reads k_nope and v once (256 + 256 bytes per key and head)
// and the shared rotary key k_pe (128 bytes per key, once per sequence).
//
// gfx950 design:
//  * A quarter-wave (16 lanes x 16 bytes) covers one 128-dim bf16 key row, so
//    every wave-wide 128-bit load reads 4 consecutive rows (1 KiB) of k_nope or
//    v; k_pe rows are 16 lanes x 8 bytes. Streaming loads are non-temporal.
//  * Each lane keeps 8 query dims (+4 rotary dims) in fp32, forms partial dot
//    products, and a 4-step DPP reduction inside the quarter-wave gives the
//    score. Each quarter-wave runs its own online softmax (fp32, exp2 domain)
//    over the keys it sees and accumulates 8 output dims per lane.
//  * Quarter-waves, then waves, are merged by log-sum-exp. When the key range
//    of a (b, h) is split over several workgroups (to fill the chip when B*H
//    is small), each writes an fp32 partial (o[128], max, sum) to the
//    workspace. If all splits of a (b, h) run on one XCD, they share that
//    XCD's L2, and the split kernel merges them itself: each workgroup stores
//    its partial, then a flag holding the call's tag, waits for both stores,
//    and reads all flags of its (b, h) with device-scope loads (past L1);
//    whichever sees every flag set merges (the last to finish always does;
//    two that finish together both write the same bytes), then clears the flags of its (b, h), so a replayed
//    graph, which repeats the captured tag, starts from cleared flags. No
//    atomics or device-scope fences are needed: on
//    this chip a device-scope release or acquire writes back or invalidates
//    the whole L2. For other shapes a second, tiny kernel merges the
//    partials, ordered by the kernel boundary.
//  * Workgroups of one sequence are placed on one XCD so the shared k_pe rows
//    are served from that XCD's L2 for all heads. With a length per sequence
//    that would leave the XCDs unequally loaded, so there the (b, h) pairs go
//    round-robin over the XCDs instead (k_pe is then read once per XCD).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int DN = 128, DR = 64, DV = 128;
constexpr int NW = 4;            // waves per workgroup
constexpr int NT = NW * 64;
constexpr int KEYS_PER_LANE = 8; // keys each quarter-wave takes per trip (loads in flight)
constexpr int KEYS_PER_WAVE = 4 * KEYS_PER_LANE;   // 32
constexpr int KEYS_PER_TRIP = NW * KEYS_PER_WAVE;  // 128

// Cache-policy operand of the buffer loads that read what other workgroups
// stored (completion flags, partials): the SC1 bit alone, device scope in the
// CDNA3/CDNA4 scope encoding (SC1:SC0 = 0 wave, 1 workgroup, 2 device,
// 3 system). A device-scope load misses in the CU's L1, so it cannot return
// a line an earlier workgroup on the same CU cached before the store landed;
// it is served by the XCD's L2, which every split of a (b, h) shares. (SC0
// alone is workgroup scope, which the L1 may serve.)
constexpr int kDeviceScope = 16;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, false));
}

// Sum over the 16 lanes of a row (quarter-wave); every lane gets the total.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// exp2(m - ref) that is 0 for an empty partial (m = -inf)
__device__ __forceinline__ float rescale(float m, float ref) {
  return m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - ref);
}

// Merge this lane's (m, l, o[8]) with the lane `mask` away (xor shuffle).
__device__ __forceinline__ void merge_xor(float& m, float& l, float (&o)[8], int mask) {
  const float m2 = __shfl_xor(m, mask);
  const float l2 = __shfl_xor(l, mask);
  float o2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[e], mask);
  const float M = fmaxf(m, m2);
  const float a1 = rescale(m, M), a2 = rescale(m2, M);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = o[e] * a1 + o2[e] * a2;
  m = M;
}

// MASKED: the caller's 2D padding mask hides keys (a.key_mask, [B, S] bytes,
// nonzero keeps); one instantiation each, so the unmasked kernel carries none
// of its code.
template <bool MASKED, bool ROPE>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  __shared__ float red_o[NW][DV];
  __shared__ float red_ml[NW][2];

  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  // Variable lengths (a.interleave): (b, h) pairs go round-robin over the
  // XCDs, so every XCD gets H/8 heads of every sequence and the same share of
  // keys; the splits of one (b, h) still share an XCD. Otherwise each XCD
  // takes a contiguous run of (b, h, split). Both mappings are formed and one
  // selected, without a branch, so the argument loads issue as one batch.
  const int k8 = wg >> 3;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const int src = a.interleave ? k8 : logical;
  const int q = src / a.nsplit;
  int bh = a.interleave ? (wg & 7) + 8 * q : q;
  const int split = src - q * a.nsplit;
  // With a length per sequence and one split per (b, h), sequences are taken
  // longest first: the workgroup's position bh / H in dispatch order names the
  // sequence of that rank (lengths clamped as below, ties by index), so the
  // long (b, h) pairs start first and the short ones fill the tail.
  if ((MASKED || a.seq_lens != nullptr) && a.nsplit == 1 && a.B > 1 && a.B <= 64) {
    const int ln = threadIdx.x & 63;
    int32_t len = -1;
    if constexpr (MASKED) {
      // the 2D mask's kept positions among 64 evenly spaced samples of each
      // row stand in for the length (an estimate: it only orders the work)
      const int64_t pos = (int64_t)ln * a.S / 64;
      for (int bb = 0; bb < a.B; ++bb) {
        const int kept = __popcll(__ballot(a.key_mask[(int64_t)bb * a.S + pos] != 0));
        if (ln == bb) len = kept;
      }
    } else if (ln < a.B) {
      const int32_t raw = a.seq_lens[ln];
      len = raw < 0 ? 0 : (raw > a.S ? a.S : raw);
    }
    int rank = 0;
    for (int jj = 0; jj < a.B; ++jj) {
      const int32_t lj = __builtin_amdgcn_readlane(len, jj);
      rank += (lj > len || (lj == len && jj < ln)) ? 1 : 0;
    }
    const int r = bh / a.H;
    const unsigned long long hit = __ballot(ln < a.B && rank == r);
    bh = (__builtin_ffsll((long long)hit) - 1) * a.H + (bh - r * a.H);
  }
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cl = lane & 15;   // column slot: dims 8cl..8cl+7 (rotary 4cl..4cl+3)
  const int qq = lane >> 4;   // quarter-wave

  // Keys of this sequence: rows [0, S) of its cache slices (cap rows each).
  // A length array from the caller is clamped to [0, a.S], so no row past the
  // bound the host checked against the capacity is ever read.
  const int64_t cap = a.cap;
  int64_t S = a.S;
  if (a.seq_lens != nullptr) {
    const int32_t len = a.seq_lens[b];
    S = len < 0 ? 0 : (len > a.S ? a.S : len);
  }
  const uint16_t* kn_g = a.k_nope + (int64_t)bh * cap * DN + 8 * cl;
  const uint16_t* v_g = a.v + (int64_t)bh * cap * DV + 8 * cl;
  const uint16_t* kp_g = a.k_pe + (int64_t)b * cap * DR + 4 * cl;
  // Paged cache: key j of sequence b is row j % bs of block table[b][j / bs],
  // blocks [num_blocks, H, bs, 128] (k_nope, v) and [num_blocks, bs, 64]
  // (k_pe). bs is a multiple of 32, so a wave's 32 keys of one trip share a
  // block and one scalar table read serves them. Block ids are clamped into
  // [0, num_blocks) so no id, however bad, addresses outside the pages.
  const int32_t* table = a.block_table != nullptr ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
  const int64_t bsz = a.block_size;
  auto block_of = [&](int64_t key) -> int64_t {
    int32_t blk = table[key / bsz];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    return blk;
  };
  // Row `key` of this (b, h) in the cache (16 lanes x 8 dims; rotary 16 x 4).
  auto kn_row = [&](int64_t key) -> const uint16_t* {
    return table ? a.k_nope + ((block_of(key) * a.H + h) * bsz + key % bsz) * DN + 8 * cl
                 : kn_g + key * DN;
  };
  auto v_row = [&](int64_t key) -> const uint16_t* {
    return table ? a.v + ((block_of(key) * a.H + h) * bsz + key % bsz) * DV + 8 * cl
                 : v_g + key * DV;
  };
  auto kp_row = [&](int64_t key) -> const uint16_t* {
    return table ? a.k_pe + (block_of(key) * bsz + key % bsz) * DR + 4 * cl : kp_g + key * DR;
  };

  // The query: 8 non-rotary dims and 4 rotary dims per lane, as bf16 words.
  // The plain kernel widens them to fp32 inside the loop, after each trip's
  // key loads are issued (an empty asm keeps the compiler from hoisting the
  // widening, and with it the wait for the query, in front of the first key
  // loads); the query's latency then overlaps the keys' instead of preceding
  // it. The masked kernel widens them here (in its loop the wait would also
  // cover the next trip's mask bytes, fetched ahead), and so does the rotary
  // kernel, which rotates them here too.
  constexpr bool kLateQuery = !MASKED && !ROPE;
  const u32x4 qw = *reinterpret_cast<const u32x4*>(a.q_nope + (int64_t)bh * DN + 8 * cl);
  const u32x2 qpw = *reinterpret_cast<const u32x2*>(a.q_pe + (int64_t)bh * DR + 4 * cl);
  float qn[8], qp[4];
  auto widen_q = [&](const u32x4& w, const u32x2& wp) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qn[2 * e] = lo_bf16(w[e]);
      qn[2 * e + 1] = hi_bf16(w[e]);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      qp[2 * e] = lo_bf16(wp[e]);
      qp[2 * e + 1] = hi_bf16(wp[e]);
    }
  };
  if (!kLateQuery) widen_q(qw, qpw);
  // Fused rotary prologue (the rotary instantiation): the new token's query, and its
  // key when the call appends it, turn at position S-1, the last key of the
  // sequence. Lane cl holds rotary dims 4cl..4cl+3, i.e. whole pairs 2cl and
  // 2cl+1, so it reads their (cos, sin) and rotates in its own registers.
  f32x4 rope_cs = {1.0f, 0.0f, 1.0f, 0.0f};
  if (ROPE) {
    // S <= a.S and the host checked that the table holds a.S positions
    const int64_t pos = S > 0 ? S - 1 : 0;
    rope_cs = *reinterpret_cast<const f32x4*>(a.rope_table + pos * 64 + 4 * cl);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x = qp[2 * e], y = qp[2 * e + 1];
      const float c = rope_cs[2 * e], sn = rope_cs[2 * e + 1];
      qp[2 * e] = x * c - y * sn;
      qp[2 * e + 1] = x * sn + y * c;
    }
  }

  const float c = a.scale_log2;
  const int64_t s0 = (int64_t)split * a.keys_per_split;
  // With an appended token, key S-1 comes from the new rows (never from the
  // cache, which this call writes); the loop covers keys before it.
  const bool append = a.kn_new != nullptr && S >= 1;
  const int64_t S_loop = append ? S - 1 : S;
  const int64_t s1 = (s0 + a.keys_per_split < S_loop) ? s0 + a.keys_per_split : S_loop;
  const bool owns_new = append && S - 1 >= s0 && S - 1 < s0 + a.keys_per_split;
  // With a length per sequence, only the splits that hold a key of it take
  // part (at least split 0, which gives an empty sequence its zero row); the
  // others leave at once, and the in-kernel merge waits for and reads the
  // active ones only. (Workgroup-uniform, before any barrier.)
  int nact = a.nsplit;
  if (a.seq_lens != nullptr && a.fused) {
    const int64_t n = (S + a.keys_per_split - 1) / a.keys_per_split;
    nact = n < 1 ? 1 : (n > a.nsplit ? a.nsplit : (int)n);
    if (split >= nact) return;
  }

  float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.0f;

  // Block ids of this wave's trips (paged cache): lane t reads the id for
  // trip t once, and each trip broadcasts it with readlane, so no table read
  // sits in the loop (trips past the 64th, only for splits longer than 8192
  // keys, read the table directly).
  const int64_t base0 = s0 + wave * KEYS_PER_WAVE;
  int32_t blk_lane = 0;
  if (table != nullptr) {
    const int64_t kb = base0 + (int64_t)KEYS_PER_TRIP * lane;
    if (kb < s1) blk_lane = (int32_t)block_of(kb);
  }
  // 2D mask: each wave takes the mask bytes of its keys eight trips (256
  // keys) at a time, the next group's one group ahead: lane l holds the four
  // bytes of trip l / 8 at offset 4 (l % 8) of the wave's 32 keys. Four
  // ballots (one per byte position) turn them into one bit per key: key
  // 4u + qq of trip t is bit 8t + u of ballot qq. A trip whose keys are all
  // hidden then costs a few scalar ops and no memory round trip, and rows of
  // hidden keys are never fetched. Bytes past this split's keys read as 0
  // (buffer range check), i.e. hidden.
  __amdgpu_buffer_rsrc_t mrs;
  uint32_t mb_cur[4] = {0, 0, 0, 0}, mb_next[4] = {0, 0, 0, 0};
  uint64_t m_any = 0, m_lane = 0;  // the current group's bits: any key kept per slot, this lane's keys
  auto load_group = [&](int g, uint32_t (&mb)[4]) {
    const int off = (int)(base0 + (int64_t)(8 * g + (lane >> 3)) * KEYS_PER_TRIP + 4 * (lane & 7));
#pragma unroll
    for (int p = 0; p < 4; ++p) mb[p] = __builtin_amdgcn_raw_buffer_load_b8(mrs, off + p, 0, 0);
  };
  if (MASKED) {
    mrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.key_mask + (int64_t)b * a.S), (short)0,
                                            s1 > 0 ? (int)s1 : 0, 0x00020000);
    load_group(0, mb_cur);
  }
  int trip = 0;
  for (int64_t base = base0; base < s1; base += KEYS_PER_TRIP, ++trip) {
    u32x4 kn[KEYS_PER_LANE], vv[KEYS_PER_LANE];
    u32x2 kp[KEYS_PER_LANE];
    bool ok[KEYS_PER_LANE];
    const uint16_t* kn_t;  // rows base .. base+31 are consecutive
    const uint16_t* v_t;
    const uint16_t* kp_t;
    if (table != nullptr) {
      const int64_t blk = trip < 64 ? __builtin_amdgcn_readlane(blk_lane, trip) : block_of(base);
      const int64_t r0 = base % bsz;
      kn_t = a.k_nope + ((blk * a.H + h) * bsz + r0) * DN + 8 * cl;
      v_t = a.v + ((blk * a.H + h) * bsz + r0) * DV + 8 * cl;
      kp_t = a.k_pe + (blk * bsz + r0) * DR + 4 * cl;
    } else {
      kn_t = kn_g + base * DN;
      v_t = v_g + base * DV;
      kp_t = kp_g + base * DR;
    }
    if (MASKED) {
      if ((trip & 7) == 0) {  // a new group of eight trips: its bits, and the next group's bytes
        if (trip > 0) {
#pragma unroll
          for (int p = 0; p < 4; ++p) mb_cur[p] = mb_next[p];
        }
        load_group((trip >> 3) + 1, mb_next);
        const uint64_t m0 = __ballot(mb_cur[0] != 0), m1 = __ballot(mb_cur[1] != 0);
        const uint64_t m2 = __ballot(mb_cur[2] != 0), m3 = __ballot(mb_cur[3] != 0);
        m_any = m0 | m1 | m2 | m3;
        m_lane = (qq & 2) ? ((qq & 1) ? m3 : m2) : ((qq & 1) ? m1 : m0);
      }
      const int sh = 8 * (trip & 7);
      // a trip whose keys are all hidden is skipped whole
      if (((m_any >> sh) & 0xffu) == 0) continue;
#pragma unroll
      for (int u = 0; u < KEYS_PER_LANE; ++u) ok[u] = ((m_lane >> (sh + u)) & 1u) != 0;
    }
#pragma unroll
    for (int u = 0; u < KEYS_PER_LANE; ++u) {
      if (!MASKED) ok[u] = base + 4 * u + qq < s1;
      if (ok[u]) {
        kn[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kn_t + (4 * u + qq) * DN));
        kp[u] = *reinterpret_cast<const u32x2*>(kp_t + (4 * u + qq) * DR);
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_t + (4 * u + qq) * DV));
      } else {
        kn[u] = u32x4{0, 0, 0, 0};
        kp[u] = u32x2{0, 0};
        vv[u] = u32x4{0, 0, 0, 0};
      }
    }
    // (a hidden key was never loaded: it scores -inf below and its value
    // registers hold 0, so whatever its rows hold, NaN included, cannot reach
    // the output)
    if (kLateQuery) {
      u32x4 w = qw;
      u32x2 wp = qpw;
      asm volatile("" : "+v"(w), "+v"(wp));
      widen_q(w, wp);
    }
    float t[KEYS_PER_LANE];
#pragma unroll
    for (int u = 0; u < KEYS_PER_LANE; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = __builtin_fmaf(qn[2 * e], lo_bf16(kn[u][e]), d);
        d = __builtin_fmaf(qn[2 * e + 1], hi_bf16(kn[u][e]), d);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        d = __builtin_fmaf(qp[2 * e], lo_bf16(kp[u][e]), d);
        d = __builtin_fmaf(qp[2 * e + 1], hi_bf16(kp[u][e]), d);
      }
      d = row_sum16(d);
      t[u] = ok[u] ? d * c : -INFINITY;
    }
    float mt = t[0];
#pragma unroll
    for (int u = 1; u < KEYS_PER_LANE; ++u) mt = fmaxf(mt, t[u]);
    const float m_new = fmaxf(m, mt);
    const float ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - ref);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < KEYS_PER_LANE; ++u) {
      const float p = __builtin_amdgcn_exp2f(t[u] - ref);
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __builtin_fmaf(p, lo_bf16(vv[u][e]), o[2 * e]);
        o[2 * e + 1] = __builtin_fmaf(p, hi_bf16(vv[u][e]), o[2 * e + 1]);
      }
    }
  }

  // ---- the appended token (key S-1): the split that owns it takes it from
  // the new rows in quarter-wave 0 of wave 0, which also writes the rows into
  // the cache (the rotary row by head 0 only: it is shared by the heads, and
  // every head reads key S-1 from the new rows, so no one reads that slot).
  if (kLateQuery) widen_q(qw, qpw);  // the loop may have run no trip
  if (owns_new && wave == 0 && qq == 0) {
    const u32x4 kw = *reinterpret_cast<const u32x4*>(a.kn_new + (int64_t)bh * DN + 8 * cl);
    u32x2 pw = *reinterpret_cast<const u32x2*>(a.kp_new + (int64_t)b * DR + 4 * cl);
    if (ROPE) {
      // the new key's rotary part, rotated and rounded as it is stored: this
      // call and every later one attend to the same bf16 values
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x = lo_bf16(pw[e]), y = hi_bf16(pw[e]);
        const float c = rope_cs[2 * e], sn = rope_cs[2 * e + 1];
        pw[e] = (uint32_t)to_bf16_rne(x * c - y * sn) | ((uint32_t)to_bf16_rne(x * sn + y * c) << 16);
      }
    }
    const u32x4 vw = *reinterpret_cast<const u32x4*>(a.v_new + (int64_t)bh * DV + 8 * cl);
    float d = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d = __builtin_fmaf(qn[2 * e], lo_bf16(kw[e]), d);
      d = __builtin_fmaf(qn[2 * e + 1], hi_bf16(kw[e]), d);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      d = __builtin_fmaf(qp[2 * e], lo_bf16(pw[e]), d);
      d = __builtin_fmaf(qp[2 * e + 1], hi_bf16(pw[e]), d);
    }
    const float t = row_sum16(d) * c;
    const float m_new = fmaxf(m, t);
    const float alpha = rescale(m, m_new);
    const float p = __builtin_amdgcn_exp2f(t - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = __builtin_fmaf(p, lo_bf16(vw[e]), o[2 * e] * alpha);
      o[2 * e + 1] = __builtin_fmaf(p, hi_bf16(vw[e]), o[2 * e + 1] * alpha);
    }
    m = m_new;
    const int64_t key = S - 1;
    *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(kn_row(key))) = kw;
    *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(v_row(key))) = vw;
    if (h == 0) *reinterpret_cast<u32x2*>(const_cast<uint16_t*>(kp_row(key))) = pw;
  }

  // ---- merge the four quarter-waves, then the waves
  merge_xor(m, l, o, 16);
  merge_xor(m, l, o, 32);
  if (qq == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[wave][8 * cl + e] = o[e];
    if (cl == 0) {
      red_ml[wave][0] = m;
      red_ml[wave][1] = l;
    }
  }
  __syncthreads();

  // wave 0, lanes 0..15: the workgroup's (m, l, o) for dims 8cl..8cl+7
  float M = -INFINITY, L = 0.0f, O[8];
  if (wave == 0 && qq == 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_ml[w][0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = rescale(red_ml[w][0], M);
      L += red_ml[w][1] * sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) O[e] += red_o[w][8 * cl + e] * sc;
    }
  }

  if (a.nsplit == 1) {
    if (wave == 0 && qq == 0) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;  // a sequence with no key gives 0
      uint16_t* dst = a.out + (int64_t)bh * DV + 8 * cl;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)to_bf16_rne(O[2 * e] * inv) | ((uint32_t)to_bf16_rne(O[2 * e + 1] * inv) << 16);
      *reinterpret_cast<u32x4*>(dst) = w;
    }
    return;
  }

  // ---- split-KV: publish this workgroup's partial
  if (wave != 0) return;
  const int64_t slot = (int64_t)bh * a.nsplit + split;
  if (qq == 0) {
    float* dst = a.ws_o + slot * DV + 8 * cl;
    *reinterpret_cast<f32x4*>(dst) = f32x4{O[0], O[1], O[2], O[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{O[4], O[5], O[6], O[7]};
    if (cl == 0) {
      const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);
      *reinterpret_cast<f32x4*>(a.ws_ml + 4 * slot) = f32x4{M, L, __builtin_bit_cast(float, xcc), 0.0f};
    }
  }
  if (!a.fused) return;
  // Completion without atomics: each workgroup publishes its partial, then a
  // flag holding this call's tag, waiting for each store to reach the XCD's
  // L2; then it reads every flag of its (b, h) with device-scope loads (past
  // L1). Of the workgroups that finish last, at least one sees all flags (a store that has completed is
  // seen by every later load); any that do merge the same partials the same
  // way and write identical bytes.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial is in L2
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) a.ws_flag[slot] = a.tag;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the flag is in L2
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.ws_flag + (int64_t)bh * a.nsplit), (short)0, a.nsplit * 8, 0x00020000);
  bool done = true;
  for (int sp = lane; sp < nact; sp += 64) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rf, sp * 8, 0, kDeviceScope);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rf, sp * 8 + 4, 0, kDeviceScope);
    done = done && (((unsigned long long)hi << 32 | lo) == a.tag);
  }
  if (__any(!done)) return;
  // Clear this (b, h)'s flags for the next call, before merging so the stores
  // overlap the merge. A replayed graph repeats the captured tag, so flags
  // left set would make a replay merge partials of the run before. Every
  // split of this call has already set its flag (that is why this workgroup
  // merges), so none is written again in this call; a workgroup still
  // reading them sees a cleared flag and leaves the merge to this one.
  for (int sp = lane; sp < nact; sp += 64) a.ws_flag[(int64_t)bh * a.nsplit + sp] = 0ull;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const uint32_t my_xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.ws_o + (int64_t)bh * a.nsplit * DV), (short)0, a.nsplit * DV * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.ws_ml + (int64_t)bh * a.nsplit * 4), (short)0, a.nsplit * 16, 0x00020000);
  float mm = -INFINITY, ll = 0.0f, oo[8];
  bool same_xcd = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) oo[e] = 0.0f;
  for (int sp = qq; sp < nact; sp += 4) {
    const u32x4 mlw = __builtin_amdgcn_raw_buffer_load_b128(rm, sp * 16, 0, kDeviceScope);
    const u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(ro, (sp * DV + 8 * cl) * 4, 0, kDeviceScope);
    const u32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(ro, (sp * DV + 8 * cl + 4) * 4, 0, kDeviceScope);
    const uint32_t m_bits = mlw[0], l_bits = mlw[1], x_bits = mlw[2];
    same_xcd = same_xcd && (x_bits == my_xcc);
    const float m_sp = __builtin_bit_cast(float, m_bits), l_sp = __builtin_bit_cast(float, l_bits);
    const float Mn = fmaxf(mm, m_sp);
    const float a1 = rescale(mm, Mn), a2 = rescale(m_sp, Mn);
    ll = ll * a1 + l_sp * a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b0 = w0[e], b1 = w1[e];
      oo[e] = oo[e] * a1 + __builtin_bit_cast(float, b0) * a2;
      oo[4 + e] = oo[4 + e] * a1 + __builtin_bit_cast(float, b1) * a2;
    }
    mm = Mn;
  }
  merge_xor(mm, ll, oo, 16);
  merge_xor(mm, ll, oo, 32);
  same_xcd = !__any(!same_xcd);
  if (qq == 0) {
    // A partial written on another XCD may not be visible here. The host
    // takes this path only on a part that reports 8 XCDs, whose dispatcher
    // places workgroup w on XCD w % 8; should placement ever differ, the row
    // is poisoned (NaN) rather than silently wrong.
    const float inv = !same_xcd ? __builtin_nanf("") : (ll > 0.0f ? 1.0f / ll : 0.0f);
    uint16_t* dst = a.out + (int64_t)bh * DV + 8 * cl;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)to_bf16_rne(oo[2 * e] * inv) | ((uint32_t)to_bf16_rne(oo[2 * e + 1] * inv) << 16);
    *reinterpret_cast<u32x4*>(dst) = w;
  }
}

__global__ __launch_bounds__(NT) void mla_decode_kernel(DecodeArgs a) { decode_body<false, false>(a); }
__global__ __launch_bounds__(NT) void mla_decode_masked_kernel(DecodeArgs a) { decode_body<true, false>(a); }
__global__ __launch_bounds__(NT) void mla_decode_rope_kernel(DecodeArgs a) { decode_body<false, true>(a); }

// Log-sum-exp merge of the nsplit partials of each (b, h): one wave per (b, h);
// quarter-wave qq merges splits qq, qq+4, ..., then the quarters merge.
__global__ __launch_bounds__(64) void mla_decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const int cl = lane & 15, qq = lane >> 4;
  float mm = -INFINITY, ll = 0.0f, oo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) oo[e] = 0.0f;
  for (int sp = qq; sp < a.nsplit; sp += 4) {
    const int64_t sl = (int64_t)bh * a.nsplit + sp;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ws_ml + 4 * sl);
    const float Mn = fmaxf(mm, ml[0]);
    const float a1 = rescale(mm, Mn), a2 = rescale(ml[0], Mn);
    const f32x4 p0 = *reinterpret_cast<const f32x4*>(a.ws_o + sl * DV + 8 * cl);
    const f32x4 p1 = *reinterpret_cast<const f32x4*>(a.ws_o + sl * DV + 8 * cl + 4);
    ll = ll * a1 + ml[1] * a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      oo[e] = oo[e] * a1 + p0[e] * a2;
      oo[4 + e] = oo[4 + e] * a1 + p1[e] * a2;
    }
    mm = Mn;
  }
  merge_xor(mm, ll, oo, 16);
  merge_xor(mm, ll, oo, 32);
  if (qq == 0) {
    const float inv = ll > 0.0f ? 1.0f / ll : 0.0f;
    uint16_t* dst = a.out + (int64_t)bh * DV + 8 * cl;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)to_bf16_rne(oo[2 * e] * inv) | ((uint32_t)to_bf16_rne(oo[2 * e + 1] * inv) << 16);
    *reinterpret_cast<u32x4*>(dst) = w;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, DecodeKind kind, hipStream_t stream) {
  const int grid = a.B * a.H * a.nsplit;
  if (kind == kDecodeMasked)
    hipLaunchKernelGGL(mla_decode_masked_kernel, dim3(grid), dim3(NT), 0, stream, a);
  else if (kind == kDecodeRope)
    hipLaunchKernelGGL(mla_decode_rope_kernel, dim3(grid), dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL(mla_decode_kernel, dim3(grid), dim3(NT), 0, stream, a);
  if (a.nsplit > 1 && !a.fused)
    hipLaunchKernelGGL(mla_decode_combine_kernel, dim3(a.B * a.H), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

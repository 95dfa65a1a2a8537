// Device-side launch interface shared by the HIP kernels and the C ABI layer.
#ifndef MLA_KERNELS_H_
#define MLA_KERNELS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Keys per prefill tile (the kernel's BN); the host's key-range split plan
// counts in these tiles.
constexpr int kPrefillKeyTile = 32;

struct PrefillArgs {
  const uint16_t* q_nope;  // [B,H,T,128] bf16 bits
  const uint16_t* q_pe;    // [B,H,T,64]
  const uint16_t* k_nope;  // [B,H,S,128]
  const uint16_t* k_pe;    // [B,1,S,64], shared by every head
  const uint16_t* v;       // [B,H,S,128]
  uint16_t* out;           // [B,H,T,128]
  int32_t B, H, T, S, past_len;
  int32_t ntiles;          // ceil(T / prefill_block_m())
  float scale_log2;        // softmax_scale * log2(e)
  // Key-range split: nsplit > 1 cuts the key tiles a query tile sees into
  // nsplit near-equal ranges, one per workgroup; each writes an fp32
  // partial, merged by a second kernel into out.
  int32_t nsplit;
  float* ws_o;             // [B*H*T, nsplit, 128] partial outputs (unnormalised)
  float* ws_ml;            // [B*H*T, nsplit, 2] partial (max, sum), max in the scaled log2 domain
  // Padded variable-length batch (both null otherwise): T and S are then the
  // padded row counts of the query and key slices, sequence b has
  // q_lens[b] new queries over past_lens[b] cached keys (clamped on the
  // device); past_len is unused.
  const int32_t* q_lens;   // [B]
  const int32_t* past_lens;  // [B]
  // 2D padding mask [B, S] (nonzero keeps key j of sequence b), or null
  const uint8_t* key_mask;
};

struct DecodeArgs {
  const uint16_t* q_nope;  // [B,H,1,128]
  const uint16_t* q_pe;    // [B,H,1,64]
  const uint16_t* k_nope;  // [B,H,cap,128]
  const uint16_t* k_pe;    // [B,1,cap,64]
  const uint16_t* v;       // [B,H,cap,128]
  const int32_t* seq_lens; // [B] keys per sequence (rows [0, len) of the cache), or null: S each
  const int32_t* block_table;  // [B, max_blocks] paged cache (k_nope/v [num_blocks,H,bs,128],
                               // k_pe [num_blocks,bs,64]), or null: contiguous cache
  const uint16_t* kn_new;  // appended token [B,H,1,128] (key seq_lens[b]-1), or null: no append
  const uint16_t* kp_new;  // [B,1,1,64]
  const uint16_t* v_new;   // [B,H,1,128]
  uint16_t* out;           // [B,H,1,128]
  float* ws_o;             // [B*H, nsplit, 128] partial outputs (nsplit > 1)
  float* ws_ml;            // [B*H, nsplit, 4] partial (max, sum, XCD id, unused)
  unsigned long long* ws_flag;  // [B*H, nsplit] completion flags (this call's tag)
  unsigned long long tag;  // this call's tag
  int32_t B, H, S;         // S: keys per sequence, or the bound lengths are clamped to
  int32_t cap;             // cache rows per (b, h) slice (= S without seq_lens)
  int32_t max_blocks, block_size, num_blocks;  // paged cache geometry
  int32_t nsplit, keys_per_split;
  int32_t fused;           // the last workgroup of each (b, h) merges the partials
  int32_t interleave;      // (b, h) -> XCD (b*H + h) % 8 (needs B*H % 8 == 0); else by sequence
  float scale_log2;
  // One slot for the two kernels that take a table: the argument block stays
  // 176 bytes (a larger one measured 3% slower on the short decode).
  union {
    const uint8_t* key_mask;   // masked kernel: [B, S] 2D padding mask (nonzero keeps key j)
    const float* rope_table;   // rotary kernel: (cos, sin) [>= a.S positions, 32]; the new
                               // query (and appended key) turns at position S-1 in the kernel
  };
};

enum DecodeKind { kDecodePlain = 0, kDecodeMasked = 1, kDecodeRope = 2 };

struct LatentArgs {
  const uint16_t* q_nope;  // [B,H,1,128]
  const uint16_t* q_pe;    // [B,H,1,64]
  const uint16_t* c_kv;    // [B,S,512] normalised latent
  const uint16_t* k_pe;    // [B,1,S,64] shared rotary key
  const uint16_t* w_kv_b;  // [H*256, 512] kv_b_proj weight (key rows, then value rows, per head)
  uint16_t* out;           // [B,H,1,128]
  uint16_t* qt;            // workspace: [B,H,576] absorbed queries joined with q_pe (bf16)
  uint16_t* po;            // workspace: [B,nsplit,H,512] partial latent outputs (bf16)
  float* pml;              // workspace: [B,nsplit,H,2] partial (max, sum)
  int32_t B, H, S;
  int32_t nsplit, keys_per_split;
  int32_t head_groups;     // attention workgroups per (sequence, split): 1 (every head), or ceil(H/16)
  float scale_log2;
};

// Queries per prefill workgroup.
int prefill_block_m();
struct RopeTableArgs {
  float* table;            // [max_pos, 32] (cos, sin) pairs
  int32_t max_pos;
  int32_t original_max_position;
  double theta, factor, beta_fast, beta_slow;
};

struct RopeApplyArgs {
  uint16_t* x;             // [B, R, T, 64] bf16, rotated in place
  uint16_t* x2;            // [B, 1, T, 64] bf16 rotated in the same launch (rows past rows1), or null
  const float* table;      // [max_pos, 32] (cos, sin) pairs
  const int32_t* past_lens;  // [B] or null: past_len for every sequence
  int64_t rows;            // B * R * T, plus B * T with x2
  int64_t rows1;           // B * R * T: rows of x
  int32_t R, T, past_len, max_pos;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, DecodeKind kind, hipStream_t stream);
hipError_t launch_latent_decode(const LatentArgs& a, hipStream_t stream);
hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t stream);
hipError_t launch_rope_apply(const RopeApplyArgs& a, hipStream_t stream);

}  // namespace mla

#endif  // MLA_KERNELS_H_

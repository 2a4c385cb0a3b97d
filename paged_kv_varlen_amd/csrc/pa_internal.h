// Internal declarations shared by the host driver and the gfx950 kernels.
//
// The launch sequence of one pa_paged_attention() call, all on the caller's
// stream, with no host synchronisation:
//   1. scatter_plan_kernel  - writes the step's K/V rows into the caches
//                             (one workgroup per token) and, in its first
//                             workgroup, builds the device work plan from
//                             cum/past: the decode sequences with their tile
//                             offsets, the start of each group of decode
//                             waves, the prefill items.
//   2. decode_kernel        - single-token sequences: every wave streams an
//                             equal share of the 16-key tiles of all
//                             (sequence, kv head) segments.
//   3. prefill_kernel       - first merges (fixed order) the decode segments
//                             that a wave boundary cut in pieces, then runs
//                             MFMA causal attention for multi-token
//                             sequences, persistent workgroups pulling
//                             (sequence, half-tile pair, kv-head) items.
// Grid sizes come from static shapes only; the kernels read the real amount
// of work from the plan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---- tiling constants -----------------------------------------------------
constexpr int kDecodeTile = 16;       // keys per decode tile
constexpr int kDecodeUnitHeads = 16;  // query heads of one decode segment (MFMA N)
constexpr int kDecodeWindow = 64;     // block-table entries a wave holds (one per lane)
constexpr int kPrefillRows = 128;     // (position, head) rows per prefill workgroup (two half-tiles)
constexpr int kPrefillKeys = 64;      // keys per prefill step (32 per kv group)
constexpr int kPlanThreads = 256;     // threads of every scatter_plan workgroup (the plan's one too)
// zero bytes read in place of absent query heads and of keys past a history:
// one key row of the largest head size (256 x 2 bytes)
constexpr int kZeroPageBytes = 512;

// ---- control block at the start of the workspace ---------------------------
enum CtrlSlot {
  kCtrlDecodeTiles = 0,  // decode tiles of all segments (T)
  kCtrlPrefillNext = 1,  // prefill queue head (atomic)
  kCtrlDecodeSeqs = 2,   // number of single-token (decode) sequences
  kCtrlPrefillItems = 3, // number of (sequence, half-tile pair) prefill items
  kCtrlPrefillQueue0 = 8,  // heads of the (up to 8) prefill queues, slots 8..15
  kCtrlSlots = 64
};

// Prefill queues: queue q serves kv heads q, q+Q, ... so that workgroups of
// one XCD (workgroup id mod 8) share the K/V of few heads in their L2.
__host__ __device__ inline int prefill_queue_count(int kv_heads) {
  if (kv_heads % 8 == 0) return 8;
  if (8 % kv_heads == 0) return kv_heads;
  return 1;
}

// ---- decode geometry ----------------------------------------------------------
// A decode "unit" is one kv head and up to 16 of its query heads; a segment
// is (decode sequence, unit) and has ceil(L / 16) tiles.  Segments are laid
// end to end (sequence-major) and wave w of W takes tiles
// [floor(w T / W), floor((w + 1) T / W)).
__host__ __device__ constexpr int decode_head_chunks(int group) { return (group + 15) / 16; }
// query-head slots of a unit, rounded up to 4, 8 or 16
__host__ __device__ constexpr int decode_head_slots(int group) {
  return group >= 16 ? 16 : group > 4 ? (group > 8 ? 16 : 8) : 4;
}
// LDS per ring slot: K tile, V tile (16 keys each) and the query block; with
// quantized caches (kq = 8: INT8, one byte per element; kq = 4: INT4, half a
// byte) the tiles are codes and the slot also holds the unit's k and v scale
// rows (fp32, at least one 1 KB load)
__host__ __device__ constexpr int decode_q_bytes(int D, int hslots) {
  return hslots * 2 * D > 1024 ? hslots * 2 * D : 1024;
}
__host__ __device__ constexpr int decode_scale_bytes(int D) { return 8 * D > 1024 ? 8 * D : 1024; }
// bytes of one cached row of one kv head: 2D (16-bit), D (INT8), D / 2 (INT4)
__host__ __device__ constexpr int cache_row_bytes(int D, int kq) { return kq == 8 ? D : kq == 4 ? D / 2 : 2 * D; }
__host__ __device__ constexpr int decode_slot_bytes(int D, int hslots, int kq = 0) {
  return 2 * kDecodeTile * cache_row_bytes(D, kq) + decode_q_bytes(D, hslots) + (kq != 0 ? decode_scale_bytes(D) : 0);
}
// Waves per decode workgroup.  Eight (two per SIMD: one computes while the
// other waits on its loads) whenever each still gets a ring of two tiles in
// about 150 KB of LDS: quantized caches below head size 256 (half the tile
// bytes, and a code conversion in every tile), 16-bit caches of head size 64,
// and of 128 with up to four head slots.  INT4 caches below head size 256,
// whose tiles are a quarter of the 16-bit ones and whose time goes to the
// per-tile chain of conversion and products, run twelve (three per SIMD)
// where the ring keeps two tiles.  Otherwise four (one per SIMD), or two at
// head size 256 with 16-bit caches.
__host__ __device__ constexpr int decode_wg_waves(int D, int kq, int hslots) {
  return kq == 4 && D <= 128 && (150 * 1024) / (12 * decode_slot_bytes(D, hslots, 4)) >= 2 ? 12
         : kq != 0 ? (D > 128 ? 4 : 8)
         : D > 128 ? 2
         : (150 * 1024) / (8 * decode_slot_bytes(D, hslots, 0)) >= 2 ? 8
                                                                      : 4;
}
// Unit groups: waves PF v .. PF v + PF - 1 of a workgroup share one of the
// plan's starts and stream the same tiles of the consecutive units PF u .. PF
// u + PF - 1 (PF = 8, 4 or 2, the largest that divides both the unit count
// and the workgroup's waves).  With all waves of a workgroup in one group it
// reads whole cache pages at eight kv heads: the rows of all kv heads of a
// slot are contiguous, and one compute unit requests them at nearly the same
// time (for INT4 rows under a memory line, both halves of every line).  The
// plan also computes PF times fewer starts.  With an odd unit count, eight
// waves of 16-bit caches split each pair of waves' tiles instead
// (decode_split = 2): wave 2v takes the lower half, wave 2v+1 the upper half
// and finds its own start from the pair's.
__host__ __device__ constexpr int decode_unit_group_of(int D, int kq, int hslots, int units) {
  return units % 8 == 0 && decode_wg_waves(D, kq, hslots) % 8 == 0   ? 8
         : units % 4 == 0 && decode_wg_waves(D, kq, hslots) % 4 == 0 ? 4
         : units % 2 == 0 && decode_wg_waves(D, kq, hslots) % 2 == 0 ? 2
                                                                     : 1;
}
__host__ __device__ constexpr int decode_split_of(int D, int kq, int hslots, int units) {
  return kq == 0 && decode_wg_waves(D, kq, hslots) == 8 && decode_unit_group_of(D, kq, hslots, units) == 1 ? 2 : 1;
}
// ring depth: as many slots as fit the workgroup's waves in about 150 KB, at
// most 4
__host__ __device__ constexpr int decode_ring(int D, int hslots, int kq = 0) {
  return (150 * 1024) / (decode_wg_waves(D, kq, hslots) * decode_slot_bytes(D, hslots, kq)) > 4
             ? 4
             : (150 * 1024) / (decode_wg_waves(D, kq, hslots) * decode_slot_bytes(D, hslots, kq));
}
// per wave: the ring, a 16-byte piece record per slot, 512 bytes of
// prefetched metadata
__host__ __device__ constexpr int decode_lds_bytes(int D, int hslots, int kq = 0) {
  return decode_wg_waves(D, kq, hslots) * (decode_ring(D, hslots, kq) * (decode_slot_bytes(D, hslots, kq) + 16) + 512);
}
__host__ __device__ constexpr int decode_wg_per_cu(int D, int hslots, int kq = 0) {
  return (160 * 1024) / decode_lds_bytes(D, hslots, kq) > 0 ? (160 * 1024) / decode_lds_bytes(D, hslots, kq) : 1;
}
// floor(a / b) for 0 <= a, 0 < b: in 32 bits when both fit (a 64-bit
// division is a long instruction sequence on the GPU)
__host__ __device__ inline int64_t div_floor(int64_t a, int64_t b) {
  if ((static_cast<uint64_t>(a) | static_cast<uint64_t>(b)) <= 0xffffffffull)
    return static_cast<uint32_t>(a) / static_cast<uint32_t>(b);
  return a / b;
}
// the wave whose tile range holds global tile g (ranges as above)
__host__ __device__ inline int decode_wave_of(int64_t g, int64_t T, int W) {
  return static_cast<int>(div_floor((g + 1) * W - 1, T));
}
__host__ __device__ inline int64_t decode_wave_begin(int w, int64_t T, int W) {
  return div_floor(static_cast<int64_t>(w) * T, W);
}
// The same over W waves split in pairs (SP = 2, decode_split_of): pair v owns
// [decode_wave_begin(v, T, W / 2), decode_wave_begin(v + 1, T, W / 2)), wave
// 2v its lower half (rounded down), wave 2v+1 the rest.
__host__ __device__ inline int64_t decode_split_mid(int v, int64_t T, int Wp) {
  const int64_t b = decode_wave_begin(v, T, Wp);
  return b + (decode_wave_begin(v + 1, T, Wp) - b) / 2;
}
__host__ __device__ inline int64_t decode_wave_begin_sp(int w, int64_t T, int W, int SP) {
  if (SP == 1) return decode_wave_begin(w, T, W);
  return (w & 1) ? decode_split_mid(w >> 1, T, W >> 1) : decode_wave_begin(w >> 1, T, W >> 1);
}
__host__ __device__ inline int decode_wave_of_sp(int64_t g, int64_t T, int W, int SP) {
  if (SP == 1) return decode_wave_of(g, T, W);
  const int v = decode_wave_of(g, T, W >> 1);
  return 2 * v + (g >= decode_split_mid(v, T, W >> 1) ? 1 : 0);
}

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WorkspaceLayout {
  size_t ctrl;         // int32[kCtrlSlots]
  size_t zeros;        // kZeroPageBytes zero bytes, read in place of absent rows
  size_t dec_seq;      // int4[batch + 1]: (b, token, L, first tile); last = (.., .., .., T)
  size_t dec_start;    // int32[8 * (waves + 1)]: per wave (d, unit, tile, g, b, token, L, first tile)
  size_t pf_items;     // int2[max_pf_items]    (sequence, half-tile pair)
  size_t part_lse;     // float[2 * waves * 16]
  size_t part_o;       // float[2 * waves * 16 * D]
  size_t q_pro;        // T [N, H * D]: query rows after the fused prologue (when there is one)
  size_t total;
  int64_t max_pf_items;
  int decode_waves;    // W
  int decode_grid;     // workgroups of the decode launch
};

// ---- kernel parameter blocks ------------------------------------------------
struct ScatterPlanParams {
  const uint16_t* key_src;     // first K element of token 0
  const uint16_t* value_src;   // first V element of token 0
  int64_t src_stride;          // elements between consecutive tokens' K rows
  uint16_t* key_cache;
  uint16_t* value_cache;
  const int32_t* cum;
  const int32_t* past;
  const int32_t* block_table;
  const int32_t* slot_mapping; // may be null
  int32_t* ws_ctrl;
  int32_t* zeros;              // kZeroPageBytes / 4 ints cleared by the plan
  int4* dec_seq;
  int32_t* dec_start;
  int2* pf_items;
  int64_t num_tokens;
  int32_t batch;
  int32_t max_blocks;
  int32_t block_size;
  int32_t row_elems;           // Hkv * D
  int32_t decode_units;        // units per sequence (Hkv * head chunks; unit pairs when paired)
  int32_t decode_waves;        // W (wave pairs when paired)
  int32_t prefill_positions;   // query positions per prefill half-tile
  const float* k_scale;        // [Hkv, D] with INT8 / INT4 caches, else null
  const float* v_scale;
  int32_t kq;                  // caches hold codes: 8 (INT8), 4 (INT4), else 0
  int32_t bf16;                // step rows are bf16 (else fp16)
  // fused prologue (pro != 0): OffsetRMSNorm and partial MRoPE of the step's
  // query and key rows before they are cached and attended
  int32_t pro;
  const uint16_t* q_src;       // first Q element of token 0
  int64_t q_src_stride;        // elements between tokens' Q rows
  uint16_t* q_out;             // [N, H*D] transformed query rows
  int32_t num_heads;
  int32_t head_size;
  const float* q_norm_w;       // [D] or null
  const float* k_norm_w;       // [D] or null
  float norm_eps;
  int32_t rotary_dim;          // 0: no rotation
  const int64_t* position_ids; // [3, N]
  double rope_log2_theta;      // log2 of the base
  uint32_t rope_rows[8];       // position row (0..2) of frequency pair i: bits 2(i%16).. of word i/16
  int32_t rope_flags;          // PA_ROPE_ADJACENT | PA_ROPE_CONTIGUOUS
};

struct AttnParams {
  const uint16_t* q;           // first Q element of token 0
  int64_t q_stride;            // elements between tokens' Q rows
  const uint16_t* key_cache;
  const uint16_t* value_cache;
  const int32_t* cum;
  const int32_t* past;
  const int32_t* block_table;
  uint16_t* out;               // [N, H*D] in the data type
  const uint16_t* zeros;       // kZeroPageBytes zero bytes
  int32_t* ws_ctrl;
  const int2* items;           // prefill items
  const int4* dec_seq;
  const int32_t* dec_start;
  float* part_o;
  float* part_lse;
  int32_t batch;
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;               // num_heads / kv_heads
  int32_t max_blocks;
  int32_t block_size;
  int32_t decode_units;        // units per sequence
  int32_t decode_waves;        // W
  // PF = 8, 4 or 2: waves PF v .. PF v + PF - 1 stream the same tiles of units
  // PF u .. PF u + PF - 1 (the plan sees unit groups and wave groups); 1: one
  // unit per wave (decode_unit_group_of)
  int32_t decode_unit_group;
  int32_t decode_split;        // 2: waves 2v and 2v+1 halve pair v's tiles (decode_split_of)
  int32_t prefill_positions;
  float scale_log2;            // scale * log2(e)
  float* lse_out;              // [N, H] natural-log lse, or null
  float* out_f32;              // [N, H*D] output before rounding, or null
  const float* k_scale;        // [Hkv, D] with INT8 / INT4 caches (codes), else null
  const float* v_scale;
  const uint16_t* gate;        // [N, H*D] output gate (sigmoid applied at the final write), or null
};

// fixed-order merge of partial states (pa_merge_states)
struct MergeStatesParams {
  const float* state_out;      // [P, R, D]
  const float* state_lse;      // [P, R]
  uint16_t* out;               // [R, D] fp16 or bf16, or null
  float* out_f32;              // [R, D], or null
  float* lse;                  // [R], or null
  int64_t rows;
  int32_t states;
  int32_t head_size;
  int32_t bf16;                // output type: 0 fp16, 1 bf16
};

// sigmoid(g) = 1 / (1 + e^-g) in fp32 for the output gate (hardware exp2 and
// reciprocal; about 1e-7 relative)
__device__ inline float gate_sigmoid(float g) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// ---- launchers (defined in the .hip files) ---------------------------------
hipError_t launch_scatter_plan(const ScatterPlanParams& p, hipStream_t s);
hipError_t launch_decode(const AttnParams& p, int head_size, int head_slots, bool bf16, int kq, int grid,
                         hipStream_t s);
hipError_t launch_prefill(const AttnParams& p, int head_size, bool bf16, int kq, int grid, hipStream_t s);
hipError_t launch_merge_states(const MergeStatesParams& p, hipStream_t s);

}  // namespace pa

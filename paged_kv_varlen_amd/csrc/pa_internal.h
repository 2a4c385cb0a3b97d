// Internal declarations shared by the host driver and the gfx950 kernels.
//
// The launch sequence of one pa_paged_attention() call, all on the caller's
// stream, with no host synchronisation:
//   1. scatter_plan_kernel  - writes the step's K/V rows into the caches
//                             (one workgroup per token) and, in its last
//                             workgroup, builds the device work lists for the
//                             two attention kernels from cum/past.
//   2. decode_kernel        - split-KV attention for single-token sequences,
//                             persistent workgroups pulling (sequence, split,
//                             kv-head) items from a device queue.
//   3. merge_kernel         - fixed-order (out, lse) merge of the splits.
//   4. prefill_kernel       - MFMA causal attention for multi-token
//                             sequences, persistent workgroups pulling
//                             (sequence, query tile, kv-head) items.
// Grid sizes come from static shapes only; each persistent workgroup reads
// the real item counts from the workspace and leaves when the queue is empty.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---- tiling constants -----------------------------------------------------
constexpr int kDecodeThreads = 256;   // 4 waves per decode workgroup
constexpr int kDecodeTile = 16;       // keys per wave per decode iteration
constexpr int kDecodeSplitKeys = 256; // positions per decode split (work item of one wave)
constexpr int kPrefillThreads = 512;  // 8 waves per prefill workgroup
constexpr int kPrefillRows = 128;     // (position, head) rows per prefill workgroup
constexpr int kPrefillKeys = 64;      // keys per kv group per prefill super-tile
constexpr int kPlanThreads = 1024;    // threads of the planning workgroup

// ---- control block at the start of the workspace ---------------------------
enum CtrlSlot {
  kCtrlDecodeNext = 0,   // decode queue head (atomic)
  kCtrlPrefillNext = 1,  // prefill queue head (atomic)
  kCtrlDecodeItems = 2,  // number of (sequence, split) decode items
  kCtrlPrefillItems = 3, // number of (sequence, tile) prefill items
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

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WorkspaceLayout {
  size_t ctrl;         // int32[kCtrlSlots]
  size_t zeros;        // 256 zero bytes, read in place of keys past a history
  size_t dec_items;    // int2[max_dec_items]   (sequence, split)
  size_t seq_split;    // int2[batch]           (first partial slot, #splits)
  size_t pf_items;     // int2[max_pf_items]    (sequence, tile)
  size_t part_lse;     // float[max_dec_items * H]
  size_t part_o;       // float[max_dec_items * H * D]
  size_t total;
  int64_t max_dec_items;
  int64_t max_pf_items;
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
  int32_t* zeros;              // 64 ints cleared by the plan
  int2* dec_items;
  int2* seq_split;
  int2* pf_items;
  int64_t num_tokens;
  int32_t batch;
  int32_t max_blocks;
  int32_t block_size;
  int32_t row_elems;           // Hkv * D
  int32_t split_keys;          // keys per decode split
  int32_t prefill_positions;   // query positions per prefill tile
};

struct AttnParams {
  const uint16_t* q;           // first Q element of token 0
  int64_t q_stride;            // elements between tokens' Q rows
  const uint16_t* key_cache;
  const uint16_t* value_cache;
  const int32_t* cum;
  const int32_t* past;
  const int32_t* block_table;
  uint16_t* out;               // [N, H*D]
  const uint16_t* zeros;       // 256 zero bytes
  int32_t* ws_ctrl;
  const int2* items;           // dec_items or pf_items
  const int2* seq_split;
  float* part_o;
  float* part_lse;
  int32_t batch;
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;               // num_heads / kv_heads
  int32_t max_blocks;
  int32_t block_size;
  int32_t split_keys;
  int32_t prefill_positions;
  float scale_log2;            // scale * log2(e)
};

// ---- launchers (defined in the .hip files) ---------------------------------
hipError_t launch_scatter_plan(const ScatterPlanParams& p, hipStream_t s);
hipError_t launch_decode(const AttnParams& p, int head_size, int grid, hipStream_t s);
hipError_t launch_merge(const AttnParams& p, int head_size, hipStream_t s);
hipError_t launch_prefill(const AttnParams& p, int head_size, int grid, hipStream_t s);
size_t prefill_lds_bytes(int head_size);

// Heads handled together by one decode work item (a divisor of group <= 8).
int decode_heads_per_item(int group);

}  // namespace pa

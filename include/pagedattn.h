/*
 * pagedattn.h - C ABI of the MI355X (gfx950) paged KV-cache attention library.
 *
 * One compute entry point, pa_paged_attention(), implements the
 * com.microsoft PagedAttention operator in its SEPARATE key/value cache
 * layout as the model-card README "com.microsoft.PagedAttention" defines it
 * (sections Description, Inputs, Outputs, Attributes, Type constraints):
 *
 *   1. the step's keys and values are written ("scattered") into the block
 *      caches, in place, at slot_mapping[t] when given (-1 = no write), else
 *      at the slot that past_seqlens and block_table give token t;
 *   2. every packed query row then attends, causally and with grouped-query
 *      heads, to its sequence's history read back from the caches through
 *      block_table, which defines the read path.
 *
 * Readings of points the pages leave open (stated once here, applied by every
 * kernel):
 *   - query head h uses key/value head h / (num_heads / kv_num_heads)
 *     (contiguous groups; the Qwen3-8B example of "WS2 CP-Aware Attention
 *     Contract" has one rank own query heads 0-15 with KV heads 0-3);
 *   - new row i of sequence b is at logical position past_seqlens[b] + i and
 *     sees keys 0 .. past_seqlens[b] + i (bottom-right causal offset, "WS2
 *     CP-Aware Attention Contract", Mode-Specific Metadata);
 *   - everything is read from the cache after the writes, so a token whose
 *     slot is -1 sees the old cache content at its own position;
 *   - a packed query row is [Q | K | V], each head-major [heads, head_size].
 *
 * Memory ownership: every pointer is caller-owned.  The library never
 * allocates, frees or keeps a pointer after the call returns (the scratch
 * of pa_paged_attention_noalloc is a static device array of the library's
 * own code, loaded with it).  Device pointers must point to memory of the
 * current HIP device.
 *
 * Ordering: the call is asynchronous on the given HIP stream.  It performs no
 * host<->device copy and no synchronisation (except under the environment
 * variable PA_DEBUG_CHECKS=1, see pa_paged_attention), so it may be captured
 * into a HIP graph.  Within one call the cache writes precede every cache
 * read.  Two calls that share caches or a workspace must be ordered by the
 * caller (same stream, or events).
 *
 * The header is plain C99 and includes no HIP header: streams are passed as
 * void* (a hipStream_t; NULL = the default stream).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5

/* Result codes.  Every host-checkable fault returns one of these before any
 * device work is enqueued (typed errors, as the acceptance criteria of "Add
 * Qwen3.8 packed hybrid PagedAttention export for ORT GenAI Engine" ask for
 * unsupported dtype/cache combinations). */
typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                          */
  PA_ERR_SHAPE = 2,        /* sizes inconsistent with each other                  */
  PA_ERR_UNSUPPORTED = 3,  /* valid for the operator, not supported by the kernels */
  PA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than pa_workspace_bytes() */
  PA_ERR_ALIGNMENT = 5,    /* a tensor pointer is not 16-byte aligned             */
  PA_ERR_ABI = 6,          /* args->struct_size does not match this library      */
  PA_ERR_METADATA = 7,     /* PA_DEBUG_CHECKS=1 only: device metadata invalid     */
  PA_ERR_HIP = 8           /* a HIP runtime call or kernel launch failed          */
} pa_status;

/* Element type T of query/key/value/caches/output.  The model card (README,
 * Type constraints) names T = float16 and S = int32 for every index input; the
 * Qwen3.8 export issue (Phase 1 scope) targets fp16 and bf16, and the WS2
 * contract's Qwen3-8B example runs in bf16.  Either way the caches are copied
 * bit for bit, scores and sums are fp32, and the output is rounded once (to
 * nearest) to T. */
typedef enum pa_dtype {
  PA_DTYPE_F16 = 1,  /* IEEE binary16                                   */
  PA_DTYPE_BF16 = 2  /* bfloat16 (the upper 16 bits of an IEEE binary32) */
} pa_dtype;

/* Element type of key_cache/value_cache.  The Qwen3.8 export issue (its
 * non-goals and follow-ups) asks for INT8/INT4 per-channel paged KV caches
 * with calibrated scales; read plainly: symmetric codes with one fp32 scale
 * per (kv head, channel), given by the caller.
 *  PA_KV_SAME  the caches hold T, like query/key/value;
 *  PA_KV_INT8  the caches hold int8 codes.  A step row x is stored as
 *              clamp(rint(x / s), -127, 127), the quotient taken in fp32 and
 *              rounded half to even; a cached code c reads as c * s;
 *  PA_KV_INT4  the caches hold 4-bit codes clamp(rint(x / s), -7, 7) (same
 *              rounding), two per byte: element 2i in bits 0-3, element 2i+1
 *              in bits 4-7, each a 4-bit two's complement number; a cached
 *              code c (-8..7) reads as c * s. */
typedef enum pa_kv_quant { PA_KV_SAME = 0, PA_KV_INT8 = 1, PA_KV_INT4 = 2 } pa_kv_quant;

/*
 * Arguments of one call.  Tensor layouts are dense row-major.
 *
 *  query        T [num_tokens, query_width].  query_width = num_heads*head_size,
 *               or (num_heads + 2*kv_num_heads)*head_size when key and value
 *               are both NULL (packed [Q|K|V] rows).  (README, Inputs: query)
 *  key, value   T [num_tokens, kv_num_heads*head_size], or both NULL.
 *               (README, Inputs: key, value)
 *  key_cache,
 *  value_cache  T [num_blocks, block_size, cache_kv_heads, cache_head_size]
 *               (int8 with kv_quant PA_KV_INT8; with PA_KV_INT4 bytes
 *               [.., .., cache_kv_heads, head_size / 2], and cache_head_size
 *               is that byte width), read and written in place;
 *               the two are always updated together.  (README, Inputs:
 *               key_cache, value_cache; Outputs)
 *  cumulative_sequence_length
 *               S [batch_size + 1], exclusive prefix sums of the new-token
 *               counts: sequence b owns tokens [cum[b], cum[b+1]); cum[0] = 0
 *               and cum[batch_size] = num_tokens.  (README, Inputs)
 *  past_seqlens S [batch_size], tokens already cached per sequence.
 *  block_table  S [batch_size, max_blocks_per_seq]: physical block of each
 *               logical block.  Entries 0 .. ceil(L_b/block_size)-1 of row b
 *               (L_b = past_seqlens[b] + new tokens) must lie in
 *               [0, num_blocks); later entries are never read.
 *  slot_mapping S [num_tokens] or NULL: flat destination slot
 *               block_id*block_size + offset of each token, -1 = no write.
 *  output       T [num_tokens, num_heads*head_size], written; must not
 *               overlap any input.  (README, Outputs: output)
 *
 * Device metadata (cum, past, block_table, slot_mapping) is trusted: values
 * outside the rules above (cum not non-decreasing, a block id or slot out of
 * range, two tokens naming one slot) give undefined results.  Set the
 * environment variable PA_DEBUG_CHECKS=1 to have the call copy the metadata to
 * the host, check it and return PA_ERR_METADATA (this synchronises).
 *
 * Supported by the kernels (else PA_ERR_UNSUPPORTED): dtype PA_DTYPE_F16 or
 * PA_DTYPE_BF16, is_causal == 1, head_size 64, 128 or 256, block_size a multiple of 16 up to
 * 4096, num_heads/kv_num_heads <= 64.  All tensor pointers 16-byte aligned.
 */
typedef struct pa_args {
  uint32_t struct_size;          /* = sizeof(pa_args)                      */
  int32_t dtype;                 /* pa_dtype                               */

  const void *query;
  const void *key;               /* NULL together with value => packed     */
  const void *value;
  void *key_cache;
  void *value_cache;
  const int32_t *cumulative_sequence_length;
  const int32_t *past_seqlens;
  const int32_t *block_table;
  const int32_t *slot_mapping;   /* may be NULL                            */
  void *output;

  int64_t num_tokens;            /* N                                      */
  int64_t query_width;           /* columns of query                       */
  int32_t batch_size;            /* B                                      */
  int32_t num_heads;             /* H   (attribute num_heads)              */
  int32_t kv_num_heads;          /* Hkv (attribute kv_num_heads)           */
  int32_t num_blocks;            /* cache dim 0                            */
  int32_t block_size;            /* cache dim 1                            */
  int32_t cache_kv_heads;        /* cache dim 2, must equal kv_num_heads   */
  int32_t cache_head_size;       /* cache dim 3: head_size (PA_KV_INT4:
                                    head_size / 2, the bytes of a row)    */
  int32_t max_blocks_per_seq;    /* block_table dim 1                      */
  float scale;                   /* 0 => 1/sqrt(head_size) (README, Attributes) */
  int32_t is_causal;             /* must be 1 (README, Attributes)         */

  void *workspace;               /* device scratch, caller-owned           */
  size_t workspace_bytes;        /* its size, >= pa_workspace_bytes(args)  */

  /* Optional measurement hook, NULL = off.  Otherwise an array of
   * 2*PA_KERNEL_COUNT hipEvent_t handles (created by the caller with timing
   * enabled): the call records events[2k] on `stream` right before it
   * launches kernel k and events[2k+1] right after, so a tool can time each
   * kernel on the stream it runs on.  Kernel k = enum pa_kernel. */
  void *const *kernel_events;

  /* Optional outputs of the row's partial state, NULL = not written ("WS2
   * CP-Aware Attention Contract", Reduction Semantics: the state of a row is
   * (out, attention-domain lse), accumulated in fp32 and rounded only at the
   * final write):
   *  lse         float [num_tokens, num_heads], 4-byte aligned:
   *              log sum_j exp(scale * <q, k_j>) over the row's visible keys
   *              (natural log);
   *  output_f32  float [num_tokens, num_heads*head_size], 16-byte aligned:
   *              the output before its rounding to T.
   * Neither may overlap any other tensor of the call.  Such states merge with
   * pa_merge_states(). */
  float *lse;
  float *output_f32;

  /* Cache element type (pa_kv_quant).  With PA_KV_INT8 or PA_KV_INT4,
   * k_scale and v_scale are float [kv_num_heads, head_size] (16-byte
   * aligned), the per-channel scales of the two caches; otherwise they are
   * ignored. */
  int32_t kv_quant;
  int32_t reserved;              /* must be 0, else PA_ERR_UNSUPPORTED      */
  const float *k_scale;
  const float *v_scale;

  /* Optional output gate, T [num_tokens, num_heads*head_size], 16-byte
   * aligned, or NULL.  The Qwen3.8 export issue (Per-layer behavior, Full
   * attention) splits the doubled Q projection per head into the query and an
   * output gate and applies sigmoid(gate) to the attention output; with a
   * gate, output = round(attention * sigmoid(gate)) elementwise, fused into
   * the final write.  lse and output_f32 stay the ungated state. */
  const void *gate;

  /* Optional fused prologue (ABI version 5) on the step's query and key
   * rows, applied before anything else: the cached key is post-RoPE and the
   * query attends post-RoPE.  The Qwen3.8 export issue (Per-layer behavior,
   * Full attention, step 3) applies a Q/K OffsetRMSNorm and then an
   * interleaved partial MRoPE, norm before RoPE and only once, with
   * position_ids INT64 [3, N] (Packed graph contract); "WS2 CP-Aware
   * Attention Contract" (RoPE / Position Semantics, the Qwen3-8B example)
   * gives the rotation a base theta and a rotary_dim that fits the head and
   * casts to the data type after RoPE.  Where the pages leave the form open
   * it is a parameter:
   *  q_norm_weight, k_norm_weight
   *               float [head_size] (16-byte aligned) or NULL: OffsetRMSNorm of
   *               every query (key) head row x: x * (1 + w) / sqrt(mean(x^2)
   *               + norm_eps), in fp32.  NULL leaves that tensor unnormalised.
   *  rotary_dim   0: no rotation; else a multiple of 16 up to head_size: the
   *               first rotary_dim channels of every query and key head turn,
   *               the others pass through.
   *  position_ids int64 [3, num_tokens] (8-byte aligned), needed with
   *               rotary_dim > 0: the three MRoPE position rows.
   *  rope_theta   > 0: frequency pair i (i < rotary_dim / 2) turns by
   *               position * rope_theta^(-2i / rotary_dim) radians, as
   *               y1 = x1 cos - x2 sin, y2 = x2 cos + x1 sin.
   *  mrope_section
   *               pairs per position row, three counts summing to
   *               rotary_dim / 2.
   *  rope_flags   PA_ROPE_ADJACENT: pair i is channels (2i, 2i + 1), else
   *               (i, i + rotary_dim / 2).  PA_ROPE_CONTIGUOUS: the first
   *               mrope_section[0] pairs take row 0, the next [1] row 1, the
   *               rest row 2; else interleaved: pair i takes row i mod 3 while
   *               that row has pairs left, else the first row that has.
   *               Other bits: PA_ERR_UNSUPPORTED.
   * The normalised and rotated rows are rounded (nearest, ties to even) to
   * the data type; those rows are what is cached (quantized with INT8 / INT4
   * caches) and attended.  A token whose slot is -1 still has its query row
   * transformed.  With either norm weight or rotary_dim > 0 the workspace
   * also holds the transformed query rows (pa_workspace_bytes accounts for
   * them).  Errors: rotary_dim not a multiple of 16 in [0, head_size]
   * PA_ERR_UNSUPPORTED; sections not summing to rotary_dim / 2, a negative
   * count or rope_theta <= 0 PA_ERR_SHAPE; position_ids NULL with
   * rotary_dim > 0 PA_ERR_NULL_ARG; misaligned weights or positions
   * PA_ERR_ALIGNMENT. */
  const float *q_norm_weight;
  const float *k_norm_weight;
  float norm_eps;
  int32_t rotary_dim;
  const int64_t *position_ids;
  float rope_theta;
  int32_t mrope_section[3];
  int32_t rope_flags;
} pa_args;

#define PA_ROPE_ADJACENT 1
#define PA_ROPE_CONTIGUOUS 2

/* Kernels launched by one call, in launch order (indices into kernel_events). */
enum pa_kernel {
  PA_KERNEL_SCATTER_PLAN = 0,  /* cache writes + device work lists        */
  PA_KERNEL_DECODE = 1,        /* balanced split-KV attention of single-token rows */
  PA_KERNEL_MERGE = 2,         /* no launch of its own: its two events are
                                  recorded back to back; the fixed-order
                                  merge of cut decode segments opens the
                                  prefill launch                          */
  PA_KERNEL_PREFILL = 3,       /* decode merge, then MFMA attention of
                                  multi-token rows                        */
  PA_KERNEL_COUNT = 4
};

/* Run the operator on `stream` (a hipStream_t, NULL = default stream).
 * Validates every host-visible argument first; on any error nothing is
 * enqueued and the caches are untouched.  PA_ERR_HIP means a launch failed;
 * the caches may then be partly written. */
pa_status pa_paged_attention(const pa_args *args, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operator as pa_paged_attention, with the same arguments and results, but
 * the workspace is scratch memory the library owns, one array of
 * PA_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load to the end
 * of the process.  args->workspace and args->workspace_bytes are ignored.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * Returns PA_ERR_WORKSPACE, with nothing enqueued, when the shapes need more
 * than PA_NOALLOC_SCRATCH_BYTES (pa_workspace_bytes(args) tells); the first
 * call on a device looks up that device's scratch address (PA_ERR_HIP if
 * that fails).  Every call on a GPU shares that GPU's scratch and leaves its
 * contents there; the kernels clear what must start at zero.  Two calls
 * that may overlap on one GPU (different streams without ordering) race on
 * the scratch: the caller must order them. */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)
pa_status pa_paged_attention_noalloc(const pa_args *args, void *stream);

/* Bytes of device workspace pa_paged_attention needs for these shapes (an
 * upper bound from static sizes only: num_tokens, batch_size, num_heads,
 * head_size, block_size, max_blocks_per_seq, and the compute-unit count of
 * the current device, which sets the number of decode waves).  Host function
 * (it may query the current device once); returns 0 when the shape fields
 * are invalid.  Pointer fields are ignored. */
size_t pa_workspace_bytes(const pa_args *args);

/*
 * Fixed-order merge of partial attention states ("WS2 CP-Aware Attention
 * Contract", Reduction Semantics: partial state (out, attention-domain lse),
 * merge online_softmax_lse, fp32 accumulation, fixed order, downcast at the
 * final write).  Row r of state p is (state_out[p][r], state_lse[p][r]), the
 * normalised output and the natural-log lse over some key set; the merged row
 * is the state of the union of the key sets of states 0..P-1, accumulated in
 * that order:
 *   lse = lse_0,  out = out_0;  for p = 1 .. P-1:
 *     lse' = log(exp(lse) + exp(lse_p)),
 *     out  = exp(lse - lse') out + exp(lse_p - lse') out_p,  lse = lse'.
 * A state with lse = -inf (no keys) has weight 0; a row whose states are all
 * empty merges to out = 0, lse = -inf.
 *
 *  state_out    float [num_states, num_rows, head_size], 16-byte aligned
 *  state_lse    float [num_states, num_rows]
 *  output       T [num_rows, head_size] (dtype), or NULL
 *  output_f32   float [num_rows, head_size], 16-byte aligned, or NULL
 *  lse          float [num_rows], or NULL
 * Rows are independent, e.g. num_rows = num_tokens * num_heads for states
 * written by pa_paged_attention.  Outputs must not overlap the states.
 * Supported: num_states >= 1, head_size a multiple of 4 up to 512, dtype
 * PA_DTYPE_F16 or PA_DTYPE_BF16 (the type of output).  Asynchronous on `stream`; no workspace, no allocation.
 */
typedef struct pa_merge_args {
  uint32_t struct_size;          /* = sizeof(pa_merge_args)                */
  int32_t dtype;                 /* pa_dtype of output                     */
  int32_t num_states;            /* P                                      */
  int32_t head_size;             /* D                                      */
  int64_t num_rows;              /* R                                      */
  const float *state_out;
  const float *state_lse;
  void *output;
  float *output_f32;
  float *lse;
} pa_merge_args;

pa_status pa_merge_states(const pa_merge_args *args, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *pa_status_string(pa_status status);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */

// Host side of the C ABI: argument checks, workspace layout, launch plan.
//
// Every check here uses host-visible sizes only, so a call never waits for
// the device (except under PA_DEBUG_CHECKS=1, which copies the metadata back
// to check it).  Grids come from static shapes; the kernels read the real
// amount of work from the plan the first kernel writes into the workspace.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <vector>

#include "../../include/pagedattn.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrefillWgPerCu = 1;     // prefill workgroups resident per CU (LDS-limited)

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Resolved {
  int64_t N;
  int B, H, Hkv, G, D, bs, NB, MB;
  bool packed;
  int kq;  // cache codes: 0 (the caches hold T), 8 (INT8) or 4 (INT4)
  float scale;
  bool pro;  // fused prologue: a norm weight given, or rotary_dim > 0
  int rd;    // rotary_dim
};

pa_status resolve(const pa_args* a, Resolved* r) {
  if (a == nullptr) return PA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(pa_args)) return PA_ERR_ABI;
  if (a->num_tokens < 0 || a->num_tokens > INT32_MAX || a->batch_size < 0) return PA_ERR_SHAPE;
  if (a->num_heads <= 0 || a->kv_num_heads <= 0 || a->num_heads % a->kv_num_heads != 0)
    return PA_ERR_SHAPE;
  if ((a->key == nullptr) != (a->value == nullptr)) return PA_ERR_SHAPE;
  r->packed = a->key == nullptr;
  const int64_t heads = r->packed ? a->num_heads + 2LL * a->kv_num_heads : a->num_heads;
  if (a->query_width <= 0 || a->query_width % heads != 0) return PA_ERR_SHAPE;
  const int64_t D = a->query_width / heads;
  if (a->kv_quant != PA_KV_SAME && a->kv_quant != PA_KV_INT8 && a->kv_quant != PA_KV_INT4)
    return PA_ERR_UNSUPPORTED;
  if (a->reserved != 0) return PA_ERR_UNSUPPORTED;  // no meaning yet
  r->kq = a->kv_quant == PA_KV_INT8 ? 8 : a->kv_quant == PA_KV_INT4 ? 4 : 0;
  const int64_t cache_row = r->kq == 4 ? D / 2 : D;  // INT4: bytes of a row
  if (a->cache_kv_heads != a->kv_num_heads || a->cache_head_size != cache_row || (r->kq == 4 && D % 2 != 0))
    return PA_ERR_SHAPE;
  if (a->num_blocks <= 0 || a->block_size <= 0 || a->max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (a->batch_size == 0 && a->num_tokens != 0) return PA_ERR_SHAPE;
  if (static_cast<int64_t>(a->max_blocks_per_seq) * a->block_size > INT32_MAX ||
      static_cast<int64_t>(a->num_blocks) * a->block_size > INT32_MAX)
    return PA_ERR_SHAPE;
  if ((a->dtype != PA_DTYPE_F16 && a->dtype != PA_DTYPE_BF16) || a->is_causal != 1) return PA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128 && D != 256) return PA_ERR_UNSUPPORTED;
  if (a->block_size % 16 != 0 || a->block_size > 4096) return PA_ERR_UNSUPPORTED;
  if (a->num_heads / a->kv_num_heads > 64) return PA_ERR_UNSUPPORTED;
  {  // decode tile indices are 32-bit
    const int64_t tiles = (static_cast<int64_t>(a->max_blocks_per_seq) * a->block_size + 15) / 16;
    const int64_t units = static_cast<int64_t>(a->kv_num_heads) *
                          decode_head_chunks(a->num_heads / a->kv_num_heads);
    if (static_cast<int64_t>(a->batch_size) * tiles * units > INT32_MAX) return PA_ERR_UNSUPPORTED;
  }
  r->N = a->num_tokens;
  r->B = a->batch_size;
  r->H = a->num_heads;
  r->Hkv = a->kv_num_heads;
  r->G = a->num_heads / a->kv_num_heads;
  r->D = static_cast<int>(D);
  r->bs = a->block_size;
  r->NB = a->num_blocks;
  r->MB = a->max_blocks_per_seq;
  r->scale = a->scale == 0.f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(D))) : a->scale;
  // fused prologue
  if (a->rotary_dim < 0 || a->rotary_dim > D || a->rotary_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
  if ((a->rope_flags & ~(PA_ROPE_ADJACENT | PA_ROPE_CONTIGUOUS)) != 0) return PA_ERR_UNSUPPORTED;
  if (a->rotary_dim > 0) {
    if (!(a->rope_theta > 0.f) || !std::isfinite(a->rope_theta)) return PA_ERR_SHAPE;
    const int64_t sum = static_cast<int64_t>(a->mrope_section[0]) + a->mrope_section[1] + a->mrope_section[2];
    if (a->mrope_section[0] < 0 || a->mrope_section[1] < 0 || a->mrope_section[2] < 0 || sum != a->rotary_dim / 2)
      return PA_ERR_SHAPE;
  }
  r->rd = a->rotary_dim;
  r->pro = a->q_norm_weight != nullptr || a->k_norm_weight != nullptr || a->rotary_dim > 0;
  return PA_OK;
}

// query positions per prefill half-tile: a workgroup's 128 rows are two
// half-tiles of 64 (position, head) rows
int prefill_positions(int G) { return (kPrefillRows / 2) / G; }

int device_cus();

// Position row of every rotary frequency pair, two bits each (pair i in bits
// 2(i % 16) of word i / 16): contiguous sections (the first s0 pairs row 0,
// the next s1 row 1, the rest row 2), or interleaved (pair i on row i mod 3
// while that row has pairs left, else the first row that has).
void mrope_rows(int pairs, const int32_t sec[3], bool contiguous, uint32_t out[8]) {
  for (int w = 0; w < 8; ++w) out[w] = 0u;
  int used[3] = {0, 0, 0};
  for (int i = 0; i < pairs && i < 128; ++i) {
    int c;
    if (contiguous) {
      c = i < sec[0] ? 0 : i < sec[0] + sec[1] ? 1 : 2;
    } else {
      c = i % 3;
      if (used[c] >= sec[c]) c = used[0] < sec[0] ? 0 : used[1] < sec[1] ? 1 : 2;
    }
    ++used[c];
    out[i >> 4] |= static_cast<uint32_t>(c) << (2 * (i & 15));
  }
}

WorkspaceLayout layout(const Resolved& r) {
  WorkspaceLayout w{};
  const int64_t live = std::min<int64_t>(r.B, r.N);  // sequences with >= 1 token
  // a sequence of q tokens has ceil(ceil(q / P) / 2) half-tile pairs, at most
  // q / (2P) + 1
  const int64_t P = prefill_positions(r.G);
  w.max_pf_items = (r.N + 2 * P - 1) / (2 * P) + live;
  // decode waves: the resident count, fewer when the history can hold only a
  // few tiles per wave
  const int hs = decode_head_slots(r.G);
  const int64_t units = static_cast<int64_t>(r.Hkv) * decode_head_chunks(r.G);
  const int64_t max_tiles = std::min<int64_t>(r.B, r.N) * units *
                            ((static_cast<int64_t>(r.MB) * r.bs + kDecodeTile - 1) / kDecodeTile);
  const int64_t resident = static_cast<int64_t>(device_cus()) * decode_wg_per_cu(r.D, hs, r.kq);
  w.decode_grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(resident, (max_tiles + 31) / 32)));
  w.decode_waves = w.decode_grid * decode_wg_waves(r.D, r.kq, hs);
  const size_t W = static_cast<size_t>(w.decode_waves);
  size_t off = 0;
  w.ctrl = off;
  off = align256(off + kCtrlSlots * sizeof(int32_t));
  w.zeros = off;
  off = align256(off + kZeroPageBytes);
  w.dec_seq = off;
  off = align256(off + (static_cast<size_t>(r.B) + 1) * sizeof(int4));
  w.dec_start = off;
  off = align256(off + (W + 1) * 8 * sizeof(int32_t));

  w.pf_items = off;
  off = align256(off + w.max_pf_items * sizeof(int2));
  w.part_lse = off;
  off = align256(off + 2 * W * kDecodeUnitHeads * sizeof(float));
  w.part_o = off;
  off = align256(off + 2 * W * kDecodeUnitHeads * r.D * sizeof(float));
  w.q_pro = off;  // the prologue's query rows [N, H*D] in T
  if (r.pro) off = align256(off + static_cast<size_t>(r.N) * r.H * r.D * sizeof(uint16_t));
  w.total = off;
  return w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<int>(cache.size()) <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// PA_DEBUG_CHECKS=1: copy the metadata to the host and check the contract.
pa_status debug_check(const pa_args* a, const Resolved& r, hipStream_t s) {
  if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  std::vector<int32_t> cum(r.B + 1), past(r.B), table(static_cast<size_t>(r.B) * r.MB), slots;
  auto get = [](void* dst, const void* src, size_t n) {
    return hipMemcpy(dst, src, n, hipMemcpyDeviceToHost) == hipSuccess;
  };
  if (!get(cum.data(), a->cumulative_sequence_length, cum.size() * 4) ||
      !get(past.data(), a->past_seqlens, past.size() * 4) ||
      !get(table.data(), a->block_table, table.size() * 4))
    return PA_ERR_HIP;
  if (a->slot_mapping != nullptr) {
    slots.resize(r.N);
    if (r.N > 0 && !get(slots.data(), a->slot_mapping, slots.size() * 4)) return PA_ERR_HIP;
  }
  if (cum[0] != 0 || cum[r.B] != r.N) return PA_ERR_METADATA;
  std::set<int64_t> written;
  for (int b = 0; b < r.B; ++b) {
    const int q = cum[b + 1] - cum[b];
    if (q < 0 || past[b] < 0) return PA_ERR_METADATA;
    const int64_t L = static_cast<int64_t>(past[b]) + q;
    if (L > static_cast<int64_t>(r.MB) * r.bs) return PA_ERR_METADATA;
    const int64_t n = (L + r.bs - 1) / r.bs;
    std::set<int32_t> row;
    for (int64_t j = 0; j < n; ++j) {
      const int32_t pg = table[static_cast<size_t>(b) * r.MB + j];
      if (pg < 0 || pg >= r.NB || !row.insert(pg).second) return PA_ERR_METADATA;
    }
    for (int i = 0; i < q; ++i) {
      int64_t slot;
      if (a->slot_mapping != nullptr) {
        slot = slots[cum[b] + i];
        if (slot < -1 || slot >= static_cast<int64_t>(r.NB) * r.bs) return PA_ERR_METADATA;
      } else {
        const int64_t pos = past[b] + i;
        slot = static_cast<int64_t>(table[static_cast<size_t>(b) * r.MB + pos / r.bs]) * r.bs + pos % r.bs;
      }
      if (slot >= 0 && !written.insert(slot).second) return PA_ERR_METADATA;
    }
  }
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_workspace_bytes(const pa_args* a) {
  pa::Resolved r{};
  if (pa::resolve(a, &r) != PA_OK) return 0;
  return pa::layout(r).total;
}

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_ARG: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "valid for the operator but not supported by these kernels";
    case PA_ERR_WORKSPACE:
      return "workspace missing or smaller than pa_workspace_bytes() (no-alloc entry point: over its scratch)";
    case PA_ERR_ALIGNMENT: return "a tensor pointer is not 16-byte aligned";
    case PA_ERR_ABI: return "struct_size does not match the library";
    case PA_ERR_METADATA: return "device metadata violates the operator contract";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"

namespace pa {
namespace {

// Every check of a call except the workspace's (the two entry points take
// their workspace from different places).  PA_OK with r->N == 0 means there
// is nothing to do.
pa_status prepare(const pa_args* a, Resolved* r) {
  pa_status st = resolve(a, r);
  if (st != PA_OK) return st;
  if (r->N == 0) return PA_OK;  // no token: nothing is written or read
  if (a->query == nullptr || a->key_cache == nullptr || a->value_cache == nullptr ||
      a->cumulative_sequence_length == nullptr || a->past_seqlens == nullptr ||
      a->block_table == nullptr || a->output == nullptr)
    return PA_ERR_NULL_ARG;
  if (!aligned16(a->query) || !aligned16(a->key) || !aligned16(a->value) ||
      !aligned16(a->key_cache) || !aligned16(a->value_cache) || !aligned16(a->output) ||
      !aligned4(a->cumulative_sequence_length) || !aligned4(a->past_seqlens) ||
      !aligned4(a->block_table) || !aligned4(a->slot_mapping) ||
      !aligned4(a->lse) || !aligned16(a->output_f32) || !aligned16(a->gate))
    return PA_ERR_ALIGNMENT;
  if (r->kq != 0) {
    if (a->k_scale == nullptr || a->v_scale == nullptr) return PA_ERR_NULL_ARG;
    if (!aligned16(a->k_scale) || !aligned16(a->v_scale)) return PA_ERR_ALIGNMENT;
  }
  if (r->rd > 0 && a->position_ids == nullptr) return PA_ERR_NULL_ARG;
  if (!aligned16(a->q_norm_weight) || !aligned16(a->k_norm_weight) ||
      (reinterpret_cast<uintptr_t>(a->position_ids) & 7u) != 0)
    return PA_ERR_ALIGNMENT;
  return PA_OK;
}

// Enqueue the call's kernels on s with the workspace at ws (w.total bytes,
// 256-byte aligned).
pa_status enqueue(const pa_args* a, const Resolved& r, const WorkspaceLayout& w, char* ws,
                  hipStream_t s) {
  pa_status st = PA_OK;
  const char* dbg = std::getenv("PA_DEBUG_CHECKS");
  if (dbg != nullptr && dbg[0] == '1') {
    st = debug_check(a, r, s);
    if (st != PA_OK) return st;
  }

  // optional per-kernel events (measurement hook)
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(a->kernel_events);
  auto mark = [&](int k, int edge) {
    if (ev != nullptr) (void)hipEventRecord(ev[2 * k + edge], s);
  };

  const uint16_t* q = static_cast<const uint16_t*>(a->query);
  const int64_t qw = a->query_width;

  ScatterPlanParams sp{};
  if (r.packed) {
    sp.key_src = q + static_cast<int64_t>(r.H) * r.D;
    sp.value_src = q + static_cast<int64_t>(r.H + r.Hkv) * r.D;
    sp.src_stride = qw;
  } else {
    sp.key_src = static_cast<const uint16_t*>(a->key);
    sp.value_src = static_cast<const uint16_t*>(a->value);
    sp.src_stride = static_cast<int64_t>(r.Hkv) * r.D;
  }
  sp.key_cache = static_cast<uint16_t*>(a->key_cache);
  sp.value_cache = static_cast<uint16_t*>(a->value_cache);
  sp.cum = a->cumulative_sequence_length;
  sp.past = a->past_seqlens;
  sp.block_table = a->block_table;
  sp.slot_mapping = a->slot_mapping;
  sp.ws_ctrl = reinterpret_cast<int32_t*>(ws + w.ctrl);
  sp.zeros = reinterpret_cast<int32_t*>(ws + w.zeros);
  sp.dec_seq = reinterpret_cast<int4*>(ws + w.dec_seq);
  sp.dec_start = reinterpret_cast<int32_t*>(ws + w.dec_start);

  sp.pf_items = reinterpret_cast<int2*>(ws + w.pf_items);
  sp.num_tokens = r.N;
  sp.batch = r.B;
  sp.max_blocks = r.MB;
  sp.block_size = r.bs;
  sp.row_elems = r.Hkv * r.D;
  // unit groups or split pairs: the plan keeps one start per group (pair) of
  // waves and sees the unit groups
  const int units = r.Hkv * decode_head_chunks(r.G);
  const int ugroup = decode_unit_group_of(r.D, r.kq, decode_head_slots(r.G), units);
  const int split = decode_split_of(r.D, r.kq, decode_head_slots(r.G), units);
  sp.decode_units = units / ugroup;
  sp.decode_waves = w.decode_waves / (ugroup * split);
  sp.prefill_positions = prefill_positions(r.G);
  sp.kq = r.kq;
  sp.bf16 = a->dtype == PA_DTYPE_BF16 ? 1 : 0;
  sp.k_scale = r.kq != 0 ? a->k_scale : nullptr;
  sp.v_scale = r.kq != 0 ? a->v_scale : nullptr;
  if (r.pro) {
    sp.pro = 1;
    sp.q_src = q;
    sp.q_src_stride = qw;
    sp.q_out = reinterpret_cast<uint16_t*>(ws + w.q_pro);
    sp.num_heads = r.H;
    sp.head_size = r.D;
    sp.q_norm_w = a->q_norm_weight;
    sp.k_norm_w = a->k_norm_weight;
    sp.norm_eps = a->norm_eps;
    sp.rotary_dim = r.rd;
    sp.position_ids = a->position_ids;
    sp.rope_log2_theta = r.rd > 0 ? std::log2(static_cast<double>(a->rope_theta)) : 0.0;
    mrope_rows(r.rd / 2, a->mrope_section, (a->rope_flags & PA_ROPE_CONTIGUOUS) != 0, sp.rope_rows);
    sp.rope_flags = a->rope_flags;
  }
  mark(PA_KERNEL_SCATTER_PLAN, 0);
  if (launch_scatter_plan(sp, s) != hipSuccess) return PA_ERR_HIP;
  mark(PA_KERNEL_SCATTER_PLAN, 1);

  AttnParams ap{};
  ap.q = r.pro ? sp.q_out : q;  // the prologue's rows, when there is one
  ap.q_stride = r.pro ? static_cast<int64_t>(r.H) * r.D : qw;
  ap.key_cache = sp.key_cache;
  ap.value_cache = sp.value_cache;
  ap.cum = sp.cum;
  ap.past = sp.past;
  ap.block_table = sp.block_table;
  ap.out = static_cast<uint16_t*>(a->output);
  ap.zeros = reinterpret_cast<const uint16_t*>(ws + w.zeros);
  ap.ws_ctrl = sp.ws_ctrl;
  ap.dec_seq = sp.dec_seq;
  ap.dec_start = sp.dec_start;

  ap.part_o = reinterpret_cast<float*>(ws + w.part_o);
  ap.part_lse = reinterpret_cast<float*>(ws + w.part_lse);
  ap.batch = r.B;
  ap.num_heads = r.H;
  ap.kv_heads = r.Hkv;
  ap.group = r.G;
  ap.max_blocks = r.MB;
  ap.block_size = r.bs;
  ap.decode_units = units;
  ap.decode_waves = w.decode_waves;
  ap.decode_unit_group = ugroup;
  ap.decode_split = split;
  ap.prefill_positions = prefill_positions(r.G);
  ap.scale_log2 = r.scale * 1.4426950408889634f;
  ap.lse_out = a->lse;
  ap.k_scale = sp.k_scale;
  ap.v_scale = sp.v_scale;
  ap.out_f32 = a->output_f32;
  ap.gate = static_cast<const uint16_t*>(a->gate);

  const int cus = device_cus();
  mark(PA_KERNEL_DECODE, 0);
  const bool bf16 = a->dtype == PA_DTYPE_BF16;
  // A call of one sequence whose query has more than one token (cum[1] = N
  // by the contract) has no single-token row: its decode launch would find no
  // tile, and is left out.
  const bool no_decode_rows = r.B == 1 && r.N > 1;
  if (!no_decode_rows &&
      launch_decode(ap, r.D, decode_head_slots(r.G), bf16, r.kq, w.decode_grid, s) != hipSuccess)
    return PA_ERR_HIP;
  mark(PA_KERNEL_DECODE, 1);
  mark(PA_KERNEL_MERGE, 0);  // the merge of cut decode segments opens the prefill launch
  mark(PA_KERNEL_MERGE, 1);

  const int64_t pf_work = w.max_pf_items * r.Hkv;
  const int pf_grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(pf_work, int64_t(cus) * kPrefillWgPerCu)));
  ap.items = sp.pf_items;
  mark(PA_KERNEL_PREFILL, 0);
  if (launch_prefill(ap, r.D, bf16, r.kq, pf_grid, s) != hipSuccess) return PA_ERR_HIP;
  mark(PA_KERNEL_PREFILL, 1);
  return PA_OK;
}

}  // namespace
}  // namespace pa

// Scratch of pa_paged_attention_noalloc: the workspace of a call, in device
// memory the library owns.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address (there it is a host-side stand-in): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa {
namespace {

// Device address of this device's scratch (nullptr on a HIP error).
char* scratch_address() {
  static std::mutex mu;
  static std::vector<char*> addr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<int>(addr.size()) <= dev) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    addr[dev] = static_cast<char*>(ptr);
  }
  return addr[dev];
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_paged_attention(const pa_args* a, void* stream) {
  using namespace pa;
  Resolved r{};
  const pa_status st = prepare(a, &r);
  if (st != PA_OK || r.N == 0) return st;
  if (!aligned16(a->workspace)) return PA_ERR_ALIGNMENT;
  const WorkspaceLayout w = layout(r);
  if (a->workspace == nullptr || a->workspace_bytes < w.total) return PA_ERR_WORKSPACE;
  return enqueue(a, r, w, static_cast<char*>(a->workspace), static_cast<hipStream_t>(stream));
}

pa_status pa_paged_attention_noalloc(const pa_args* a, void* stream) {
  using namespace pa;
  Resolved r{};
  const pa_status st = prepare(a, &r);
  if (st != PA_OK || r.N == 0) return st;
  const WorkspaceLayout w = layout(r);
  if (w.total > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  char* ws = scratch_address();
  if (ws == nullptr) return PA_ERR_HIP;
  return enqueue(a, r, w, ws, static_cast<hipStream_t>(stream));
}

pa_status pa_merge_states(const pa_merge_args* a, void* stream) {
  using namespace pa;
  if (a == nullptr) return PA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(pa_merge_args)) return PA_ERR_ABI;
  if (a->num_states < 1 || a->num_rows < 0 || a->head_size <= 0) return PA_ERR_SHAPE;
  if ((a->dtype != PA_DTYPE_F16 && a->dtype != PA_DTYPE_BF16) || a->head_size % 4 != 0 || a->head_size > 512)
    return PA_ERR_UNSUPPORTED;
  if (a->num_rows == 0) return PA_OK;
  if (a->state_out == nullptr || a->state_lse == nullptr) return PA_ERR_NULL_ARG;
  if (!aligned16(a->state_out) || !aligned4(a->state_lse) || !aligned16(a->output_f32) ||
      !aligned4(a->lse) || (reinterpret_cast<uintptr_t>(a->output) & 7u) != 0)
    return PA_ERR_ALIGNMENT;
  MergeStatesParams mp{};
  mp.state_out = a->state_out;
  mp.state_lse = a->state_lse;
  mp.out = static_cast<uint16_t*>(a->output);
  mp.out_f32 = a->output_f32;
  mp.lse = a->lse;
  mp.rows = a->num_rows;
  mp.states = a->num_states;
  mp.head_size = a->head_size;
  mp.bf16 = a->dtype == PA_DTYPE_BF16 ? 1 : 0;
  if (launch_merge_states(mp, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

}  // extern "C"

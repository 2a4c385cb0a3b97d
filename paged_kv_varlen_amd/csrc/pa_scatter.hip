// Cache write ("scatter") and device-side work planning.
//
// Scatter: model-card README "com.microsoft.PagedAttention", Inputs
// (slot_mapping, past_seqlens, block_table): token t of sequence b, at
// logical position past[b] + (t - cum[b]), is written to flat slot
// slot_mapping[t] when slot_mapping is given (-1 = no write), else to
// block_table[b, pos / block_size] * block_size + pos % block_size.  A slot is
// Hkv*D contiguous fp16 values of each cache; the copy is a bit copy.
//
// One workgroup per token: the row is moved in 16-byte pieces, one per lane,
// so a 2 KB row (Hkv=8, D=128) is one fully coalesced 128-lane read and write
// per cache.  The last workgroup of the grid plans the attention work.
#include "pa_internal.h"

namespace pa {

namespace {

__device__ inline int find_sequence(const int32_t* cum, int batch, int64_t t) {
  // largest b with cum[b] <= t < cum[b+1] (sequences with no tokens are
  // skipped because their cum[b] == cum[b+1])
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (cum[mid + 1] <= t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Exclusive scan of one int per thread over a 256-thread block; returns the
// exclusive prefix and writes the block total to *total.
__device__ inline int block_exclusive_scan(int v, int* lds, int* total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int add = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += add;
    __syncthreads();
  }
  int incl = lds[tid];
  *total = lds[255];
  __syncthreads();
  return incl - v;
}

__device__ void plan(const ScatterPlanParams& p) {
  __shared__ int scan_lds[256];
  const int tid = threadIdx.x;
  int dec_base = 0, pf_base = 0;
  for (int start = 0; start < p.batch; start += 256) {
    const int b = start + tid;
    int nd = 0, np = 0;
    if (b < p.batch) {
      const int q = p.cum[b + 1] - p.cum[b];
      const int L = p.past[b] + q;
      if (q == 1) nd = (L + p.split_keys - 1) / p.split_keys;
      else if (q > 1) np = (q + p.prefill_positions - 1) / p.prefill_positions;
    }
    int tot_d, tot_p;
    const int od = block_exclusive_scan(nd, scan_lds, &tot_d);
    const int op = block_exclusive_scan(np, scan_lds, &tot_p);
    if (b < p.batch) {
      p.seq_split[b] = make_int2(dec_base + od, nd);
      for (int s = 0; s < nd; ++s) p.dec_items[dec_base + od + s] = make_int2(b, s);
      // last (longest) query tile of a sequence first
      for (int t = 0; t < np; ++t) p.pf_items[pf_base + op + t] = make_int2(b, np - 1 - t);
    }
    dec_base += tot_d;
    pf_base += tot_p;
  }
  if (tid < 64) p.zeros[tid] = 0;
  if (tid == 0) {
    p.ws_ctrl[kCtrlDecodeNext] = 0;
    p.ws_ctrl[kCtrlPrefillNext] = 0;
    for (int q = 0; q < 8; ++q) p.ws_ctrl[kCtrlPrefillQueue0 + q] = 0;
    p.ws_ctrl[kCtrlDecodeItems] = dec_base;
    p.ws_ctrl[kCtrlPrefillItems] = pf_base;
  }
}

__global__ __launch_bounds__(256) void scatter_plan_kernel(ScatterPlanParams p) {
  const int64_t t = blockIdx.x;
  if (t == p.num_tokens) {
    plan(p);
    return;
  }
  const int b = find_sequence(p.cum, p.batch, t);
  int64_t slot;
  if (p.slot_mapping != nullptr) {
    slot = p.slot_mapping[t];
  } else {
    const int pos = p.past[b] + static_cast<int>(t - p.cum[b]);
    slot = static_cast<int64_t>(p.block_table[static_cast<int64_t>(b) * p.max_blocks +
                                              pos / p.block_size]) * p.block_size +
           pos % p.block_size;
  }
  if (slot < 0) return;
  const int chunks = p.row_elems >> 3;  // 16-byte pieces per row
  const int64_t src = t * p.src_stride;
  const int64_t dst = slot * p.row_elems;
  for (int c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
    const bool is_v = c >= chunks;
    const int cc = is_v ? c - chunks : c;
    const uint4* s = reinterpret_cast<const uint4*>((is_v ? p.value_src : p.key_src) + src) + cc;
    uint4* d = reinterpret_cast<uint4*>((is_v ? p.value_cache : p.key_cache) + dst) + cc;
    *d = *s;
  }
}

}  // namespace

hipError_t launch_scatter_plan(const ScatterPlanParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.num_tokens + 1));
  hipLaunchKernelGGL(scatter_plan_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa

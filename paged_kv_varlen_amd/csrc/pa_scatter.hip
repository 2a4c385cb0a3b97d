// Cache write ("scatter") and device-side work planning.
//
// Scatter: model-card README "com.microsoft.PagedAttention", Inputs
// (slot_mapping, past_seqlens, block_table): token t of sequence b, at
// logical position past[b] + (t - cum[b]), is written to flat slot
// slot_mapping[t] when slot_mapping is given (-1 = no write), else to
// block_table[b, pos / block_size] * block_size + pos % block_size.  A slot is
// Hkv*D contiguous 16-bit values (fp16 or bf16) of each cache; the copy is a
// bit copy.
//
// One workgroup per token: the row is moved in 16-byte pieces, one per lane,
// so a 2 KB row (Hkv=8, D=128) is one fully coalesced 128-lane read and write
// per cache.  With INT8 caches a lane turns its 8 elements into 8 codes
// clamp(rint(x / s), -127, 127) with the per-channel scales s, the quotient
// in fp32 (IEEE division) and rounded half to even; with INT4 caches into 8
// codes clamped to [-7, 7], packed as nibbles (element 2i in bits 0-3).  The
// first workgroup of the grid plans the attention work.
#include "pa_internal.h"

namespace pa {

namespace {

// largest b with cum[b] <= t < cum[b+1] (sequences with no tokens are
// skipped because their cum[b] == cum[b+1]); cum may be in LDS or global
template <typename C>
__device__ inline int find_sequence(const C* cum, int batch, int64_t t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (cum[mid + 1] <= t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// LDS of this kernel is allocated in every workgroup (the scatter ones too),
// so both staging arrays stay small: 27 KB in all, five workgroups per CU
constexpr int kScatterLdsCum = 2048;  // cum entries a scatter workgroup stages in LDS

// Exclusive scan of three ints per thread over a kPlanThreads block (one pass);
// returns the exclusive prefixes and writes the block totals to tot.
__device__ inline int3 block_exclusive_scan3(int3 v, int3* lds, int3* tot) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int3 add = tid >= off ? lds[tid - off] : make_int3(0, 0, 0);
    __syncthreads();
    lds[tid].x += add.x;
    lds[tid].y += add.y;
    lds[tid].z += add.z;
    __syncthreads();
  }
  const int3 incl = lds[tid];
  *tot = lds[kPlanThreads - 1];
  __syncthreads();
  return make_int3(incl.x - v.x, incl.y - v.y, incl.z - v.z);
}

constexpr int kPlanLdsSeqs = 1024;  // decode sequences whose record the plan keeps in LDS

// The plan.  Decode sequences (one new token) get their index d and the tile
// offset of their first segment; each decode wave gets the segment and tile
// where its equal share of all tiles begins (a binary search over the
// sequences' first tiles; the records stay in LDS, so this needs no global
// load that waits for the plan's own writes).
// Multi-token sequences get one prefill item per pair of query half-tiles
// (t and nt-1-t of the sequence's nt), which all cost about the same under
// the causal mask.
__device__ void plan(const ScatterPlanParams& p) {
  __shared__ int3 scan_lds[kPlanThreads];
  __shared__ int4 seq_lds[kPlanLdsSeqs];  // dec_seq records of the first kPlanLdsSeqs
  const int tid = threadIdx.x;
  const int U = p.decode_units;
  int dec_base = 0, tile_base = 0, pf_base = 0;
  for (int start = 0; start < p.batch; start += kPlanThreads) {
    const int b = start + tid;
    int nd = 0, nt = 0, np = 0, t0 = 0, L = 0;
    if (b < p.batch) {
      t0 = p.cum[b];
      const int q = p.cum[b + 1] - t0;
      L = p.past[b] + q;
      if (q == 1) {
        nd = 1;
        nt = (L + kDecodeTile - 1) / kDecodeTile * U;
      } else if (q > 1) {
        np = ((q + p.prefill_positions - 1) / p.prefill_positions + 1) / 2;  // half-tile pairs
      }
    }
    int3 tot;
    const int3 o = block_exclusive_scan3(make_int3(nd, nt, np), scan_lds, &tot);
    if (nd != 0) {
      const int d = dec_base + o.x;
      const int4 rec = make_int4(b, t0, L, tile_base + o.y);
      p.dec_seq[d] = rec;
      if (d < kPlanLdsSeqs) seq_lds[d] = rec;
    }
    for (int t = 0; t < np; ++t) p.pf_items[pf_base + o.z + t] = make_int2(b, t);
    dec_base += tot.x;
    tile_base += tot.y;
    pf_base += tot.z;
  }
  static_assert(kZeroPageBytes / 4 <= kPlanThreads, "zero page");
  if (tid < kZeroPageBytes / 4) p.zeros[tid] = 0;
  if (tid == 0) {
    p.dec_seq[dec_base] = make_int4(0, 0, 0, tile_base);  // sentinel: T
    p.ws_ctrl[kCtrlDecodeTiles] = tile_base;
    p.ws_ctrl[kCtrlDecodeSeqs] = dec_base;
    p.ws_ctrl[kCtrlPrefillNext] = 0;
    for (int q = 0; q < 8; ++q) p.ws_ctrl[kCtrlPrefillQueue0 + q] = 0;
    p.ws_ctrl[kCtrlPrefillItems] = pf_base;
  }
  __syncthreads();  // seq_lds (and, past it, dec_seq) is read back below
  const int T = tile_base, W = p.decode_waves;
  const bool in_lds = dec_base <= kPlanLdsSeqs;
  for (int w = tid; w <= W; w += kPlanThreads) {
    int4 lo4 = make_int4(dec_base, 0, 0, T), hi4 = make_int4(0, 0, 0, 0);
    if (w < W && T > 0) {
      const int g = static_cast<int>(decode_wave_begin(w, T, W));
      int lo = 0, hi = dec_base - 1;  // last d with first tile <= g
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int f = in_lds ? seq_lds[mid].w : p.dec_seq[mid].w;
        if (f <= g) lo = mid; else hi = mid - 1;
      }
      const int4 sq = in_lds ? seq_lds[lo] : p.dec_seq[lo];
      const int n = (sq.z + kDecodeTile - 1) / kDecodeTile;
      const int off = g - sq.w;
      lo4 = make_int4(lo, off / n, off % n, g);
      hi4 = sq;
    }
    reinterpret_cast<int4*>(p.dec_start)[2 * w] = lo4;
    reinterpret_cast<int4*>(p.dec_start)[2 * w + 1] = hi4;
  }
}

__global__ __launch_bounds__(kPlanThreads) void scatter_plan_kernel(ScatterPlanParams p) {
  // workgroup 0 plans (dispatched first, it overlaps the scatter of long
  // calls); workgroup t + 1 scatters token t
  if (blockIdx.x == 0) {
    plan(p);
    return;
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) - 1;
  // the sequence of token t: a binary search over cum, staged in LDS by one
  // coalesced load (long batches search global memory)
  __shared__ int cum_lds[kScatterLdsCum];
  int b;
  if (p.slot_mapping != nullptr) {
    b = 0;  // not needed
  } else if (p.batch < kScatterLdsCum) {
    for (int i = threadIdx.x; i <= p.batch; i += blockDim.x) cum_lds[i] = p.cum[i];
    __syncthreads();
    b = find_sequence(cum_lds, p.batch, t);
  } else {
    b = find_sequence(p.cum, p.batch, t);
  }
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
  if (p.kq != 0) {
    const float lim = p.kq == 4 ? 7.f : 127.f;
    for (int c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
      const bool is_v = c >= chunks;
      const int cc = is_v ? c - chunks : c;
      const uint4 raw = reinterpret_cast<const uint4*>((is_v ? p.value_src : p.key_src) + src)[cc];
      const float4* sc = reinterpret_cast<const float4*>((is_v ? p.v_scale : p.k_scale) + 8 * cc);
      const float4 s0 = sc[0], s1 = sc[1];
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t packed[2] = {0u, 0u}, nib = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const float x = p.bf16 ? __uint_as_float(bits << 16)
                               : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
        const uint32_t code = static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(rintf(x / sv[e]), -lim), lim)));
        packed[e >> 2] |= (code & 0xffu) << (8 * (e & 3));
        nib |= (code & 0xfu) << (4 * e);
      }
      int8_t* cache = reinterpret_cast<int8_t*>(is_v ? p.value_cache : p.key_cache);
      if (p.kq == 4)  // a row is row_elems / 2 bytes
        *reinterpret_cast<uint32_t*>(cache + dst / 2 + 4 * cc) = nib;
      else
        *reinterpret_cast<uint2*>(cache + dst + 8 * cc) = make_uint2(packed[0], packed[1]);
    }
    return;
  }
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
  hipLaunchKernelGGL(scatter_plan_kernel, grid, dim3(kPlanThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa

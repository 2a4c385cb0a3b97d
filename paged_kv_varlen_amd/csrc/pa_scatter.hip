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

// LDS of this kernel is allocated in every workgroup (the scatter ones too):
// the plan's arrays and a scatter workgroup's share one buffer (kScatterSmem,
// 19 KB, eight workgroups per CU)
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
// Prefill items go out longest first: a sequence's items all cost about the
// same (the half-tile pairs balance the causal mask), about 2 past + q keys
// each, so sequences are binned by that cost in half octaves (all costs
// below 8 in bin 0) and the bins emitted from the top.  Within a bin the
// order is that of LDS atomics: an item is computed whole by one workgroup,
// so the order changes only which workgroup takes it and when, never a bit
// of the output.
constexpr int kCostBins = 64;  // one wave's lanes
__device__ inline int cost_bin(int64_t past, int q) {
  const uint64_t c = 2ull * static_cast<uint64_t>(past) + static_cast<uint64_t>(q);  // >= 2
  const int lg = 63 - __clzll(c);
  const int k = 2 * lg + static_cast<int>((c >> (lg - 1)) & 1u) - 4;
  return k < 0 ? 0 : k > kCostBins - 1 ? kCostBins - 1 : k;
}

// The plan.  Decode sequences (one new token) get their index d and the tile
// offset of their first segment; each decode wave gets the segment and tile
// where its equal share of all tiles begins (a binary search over the
// sequences' first tiles; the records stay in LDS, so this needs no global
// load that waits for the plan's own writes).
// Multi-token sequences get one prefill item per pair of query half-tiles
// (t and nt-1-t of the sequence's nt), which all cost about the same under
// the causal mask.
__device__ void plan(const ScatterPlanParams& p, char* smem) {
  int3* scan_lds = reinterpret_cast<int3*>(smem);
  int4* seq_lds = reinterpret_cast<int4*>(smem + kPlanThreads * sizeof(int3));  // dec_seq records of the first kPlanLdsSeqs
  int* bin_lds = reinterpret_cast<int*>(smem + kPlanThreads * sizeof(int3) + kPlanLdsSeqs * sizeof(int4));  // item count, then next slot, per cost bin
  const int tid = threadIdx.x;
  const int U = p.decode_units;
  int dec_base = 0, tile_base = 0, pf_base = 0;
  int row_np = 0, row_bin = 0;  // this thread's row when the batch is one pass
  for (int start = 0; start < p.batch; start += kPlanThreads) {
    const int b = start + tid;
    int nd = 0, nt = 0, np = 0, t0 = 0, L = 0, q = 0;
    if (b < p.batch) {
      t0 = p.cum[b];
      q = p.cum[b + 1] - t0;
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
    row_np = np;
    if (np != 0) row_bin = cost_bin(L - q, q);
    dec_base += tot.x;
    tile_base += tot.y;
    pf_base += tot.z;
  }
  if (pf_base != 0) {
    // Longest first: count the items of each cost bin, turn the counts into
    // first slots from the costliest bin down, then place the items.  When
    // the batch is one pass each thread still holds its row; otherwise the
    // rows are read again.
    static_assert(kCostBins <= kPlanThreads, "one bin per thread");
    const bool one_pass = p.batch <= kPlanThreads;
    if (tid < kCostBins) bin_lds[tid] = 0;
    __syncthreads();
    auto each_row = [&](auto&& f) {
      if (one_pass) {
        if (row_np != 0) f(tid, row_np, row_bin);
      } else {
        for (int start = 0; start < p.batch; start += kPlanThreads) {
          const int b = start + tid;
          if (b < p.batch) {
            const int q = p.cum[b + 1] - p.cum[b];
            if (q > 1) f(b, ((q + p.prefill_positions - 1) / p.prefill_positions + 1) / 2, cost_bin(p.past[b], q));
          }
        }
      }
    };
    each_row([&](int, int np, int k) { atomicAdd(&bin_lds[k], np); });
    __syncthreads();
    if (tid < kCostBins) {  // the first wave: exclusive scan over the bins, costliest first
      const int kb = kCostBins - 1 - tid;
      const int cnt = bin_lds[kb];
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < kCostBins; off <<= 1) {
        const int up = __shfl_up(incl, off, kCostBins);
        if (tid >= off) incl += up;
      }
      bin_lds[kb] = incl - cnt;
    }
    __syncthreads();
    each_row([&](int b, int np, int k) {
      const int at = atomicAdd(&bin_lds[k], np);
      for (int t = 0; t < np; ++t) p.pf_items[at + t] = make_int2(b, t);
    });
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

// ---- fused prologue --------------------------------------------------------
// The Qwen3.8 export issue (Per-layer behavior, Full attention, step 3) puts a
// Q/K OffsetRMSNorm and then an interleaved partial MRoPE before the
// attention; "WS2 CP-Aware Attention Contract" (RoPE / Position Semantics)
// caches K after RoPE and casts to the data type after RoPE.  A head row of D
// elements is held by D / 8 consecutive lanes (one 16-byte chunk of 8
// elements each), so a wave holds whole rows: the norm's sum of squares is a
// butterfly over those lanes and the partner chunk of a rotation pair is
// fetched from the lane rotary_dim / 16 away.

__device__ inline float elem_value(uint32_t bits, int bf16) {
  return bf16 ? __uint_as_float(bits << 16) : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}
// x rounded to the data type (nearest, ties to even), as a 16-bit pattern
__device__ inline uint32_t elem_bits(float x, int bf16) {
  return bf16 ? __builtin_bit_cast(uint16_t, static_cast<__bf16>(x))
              : __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

constexpr int kMaxRotaryPairs = 128;  // rotary_dim / 2 for head sizes up to 256

// 8 values of a chunk -> the cache: 16-bit patterns, or INT8 / INT4 codes of
// the values with their channel scales (fp32 IEEE quotient, nearest even,
// clamped)
__device__ inline void store_chunk(const ScatterPlanParams& p, bool is_v, int cc, int64_t dst, const float (&x)[8],
                                   const uint32_t (&bits)[8]) {
  if (p.kq == 0) {
    uint16_t* cache = is_v ? p.value_cache : p.key_cache;
    reinterpret_cast<uint4*>(cache + dst)[cc] =
        make_uint4(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16), bits[4] | (bits[5] << 16),
                   bits[6] | (bits[7] << 16));
    return;
  }
  const float lim = p.kq == 4 ? 7.f : 127.f;
  const float4* sc = reinterpret_cast<const float4*>((is_v ? p.v_scale : p.k_scale) + 8 * cc);
  const float4 s0 = sc[0], s1 = sc[1];
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint32_t packed[2] = {0u, 0u}, nib = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t code = static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(rintf(x[e] / sv[e]), -lim), lim)));
    packed[e >> 2] |= (code & 0xffu) << (8 * (e & 3));
    nib |= (code & 0xfu) << (4 * e);
  }
  int8_t* cache = reinterpret_cast<int8_t*>(is_v ? p.value_cache : p.key_cache);
  if (p.kq == 4)  // a row is row_elems / 2 bytes
    *reinterpret_cast<uint32_t*>(cache + dst / 2 + 4 * cc) = nib;
  else
    *reinterpret_cast<uint2*>(cache + dst + 8 * cc) = make_uint2(packed[0], packed[1]);
}

// the 8 values of a 16-byte chunk of the data type
__device__ inline void unpack8(uint4 raw, int bf16, float (&v)[8]) {
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = elem_value((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu, bf16);
}

// Norm and rotation of one 16-byte chunk (8 values) of a head row, in place.
// The D / 8 chunks of a row sit in consecutive lanes of one wave (chunk k =
// lane % (D / 8)) and all of them call this together: the norm's sum of
// squares is a butterfly over those lanes, a rotation partner is rotary_dim
// / 16 lanes away.  w: the chunk's norm weights (unused without a norm);
// cs: (cos, sin) of every frequency pair.
__device__ inline void transform8(const ScatterPlanParams& p, float (&v)[8], bool norm, const float (&w)[8],
                                  const float2* cs) {
  const int D = p.head_size, cpr = D / 8, rd = p.rotary_dim;
  const int lane = threadIdx.x & 63;
  const int k = lane % cpr;
  if (norm) {  // OffsetRMSNorm: x * (1 + w) / sqrt(mean(x^2) + eps)
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    for (int off = 1; off < cpr; off <<= 1) ss += __shfl_xor(ss, off);
    const float r = 1.f / sqrtf(ss / static_cast<float>(D) + p.norm_eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * r * (1.f + w[e]);
  }
  if (rd > 0) {  // y1 = x1 cos - x2 sin, y2 = x2 cos + x1 sin
    if ((p.rope_flags & 1) != 0) {  // adjacent: pairs (2i, 2i + 1) inside the chunk
      if (8 * k < rd) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 a = cs[4 * k + e / 2];
          const float x1 = v[e], x2 = v[e + 1];
          v[e] = x1 * a.x - x2 * a.y;
          v[e + 1] = x2 * a.x + x1 * a.y;
        }
      }
    } else {  // half split: pairs (i, i + rd / 2), the partner chunk is rd / 16 lanes away
      const int half8 = rd / 16;
      const int partner = k < half8 ? lane + half8 : k < 2 * half8 ? lane - half8 : lane;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = __shfl(v[e], partner);
      if (k < half8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 a = cs[8 * k + e];
          v[e] = v[e] * a.x - pv[e] * a.y;
        }
      } else if (k < 2 * half8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 a = cs[8 * (k - half8) + e];
          v[e] = v[e] * a.x + pv[e] * a.y;
        }
      }
    }
  }
}

// 8 transformed values rounded to the data type: patterns and rounded values
__device__ inline void round8(const float (&v)[8], int bf16, uint32_t (&b)[8], float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    b[e] = elem_bits(v[e], bf16);
    x[e] = elem_value(b[e], bf16);  // the rounded value (what codes quantize)
  }
}

__device__ inline void load_weights8(const float* w, int k, float (&out)[8]) {
  if (w == nullptr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = 0.f;
    return;
  }
  const float4 w0 = reinterpret_cast<const float4*>(w + 8 * k)[0], w1 = reinterpret_cast<const float4*>(w + 8 * k)[1];
  out[0] = w0.x; out[1] = w0.y; out[2] = w0.z; out[3] = w0.w;
  out[4] = w1.x; out[5] = w1.y; out[6] = w1.z; out[7] = w1.w;
}

// Query chunks a thread holds in registers from the token's first load on
// (further chunks, for more than kQChunks * kPlanThreads, are loaded later)
constexpr int kQChunks = 4;

// The prologue for token t (one workgroup).  Every load of the token is issued
// first (its positions, norm weights, query, key and value chunks), then the
// (cos, sin) table of the frequency pairs is built, then the rows are
// transformed, rounded and stored: the query rows into q_out, and, when slot
// >= 0, the key rows into the key cache and the value row into the value
// cache (bit copy or codes).  A token whose slot is -1 still gets its query
// row.  Angles: position * theta^(-2i / rotary_dim) in fp64 (exact for
// positions below 2^53), reduced to [-pi, pi], then sin and cos in fp32.
__device__ void prologue_token(const ScatterPlanParams& p, int64_t t, int64_t slot, float2* cs_lds) {
  const int D = p.head_size, cpr = D / 8, rd = p.rotary_dim;
  const int tid = threadIdx.x;
  const int k = tid % cpr;  // this thread's chunk within a head row
  const int nq = p.num_heads * cpr;  // query chunks of the token
  const int nk = p.row_elems >> 3;   // key (and value) chunks
  const bool kv = slot >= 0;
  // ---- loads ----
  int64_t pos = 0;
  if (tid < rd / 2) {
    const int row = static_cast<int>((p.rope_rows[tid >> 4] >> (2 * (tid & 15))) & 3u);
    pos = p.position_ids[static_cast<int64_t>(row) * p.num_tokens + t];
  }
  float wq[8], wk[8];
  load_weights8(p.q_norm_w, k, wq);
  load_weights8(p.k_norm_w, k, wk);
  const uint4* qsrc = reinterpret_cast<const uint4*>(p.q_src + t * p.q_src_stride);
  uint4 qr[kQChunks];
#pragma unroll
  for (int j = 0; j < kQChunks; ++j) {
    const int c = tid + j * kPlanThreads;
    qr[j] = c < nq ? qsrc[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint4* ksrc = reinterpret_cast<const uint4*>(p.key_src + t * p.src_stride);
  const uint4* vsrc = reinterpret_cast<const uint4*>(p.value_src + t * p.src_stride);
  const uint4 kr = kv && tid < nk ? ksrc[tid] : make_uint4(0u, 0u, 0u, 0u);
  const uint4 vr = kv && tid < nk ? vsrc[tid] : make_uint4(0u, 0u, 0u, 0u);
  // ---- the (cos, sin) table ----
  if (rd > 0) {
    if (tid < rd / 2) {
      const double inv = exp2(-2.0 * tid / rd * p.rope_log2_theta);
      double ang = static_cast<double>(pos) * inv;
      ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
      float sn, cn;
      sincosf(static_cast<float>(ang), &sn, &cn);
      cs_lds[tid] = make_float2(cn, sn);
    }
    __syncthreads();
  }
  const bool qnorm = p.q_norm_w != nullptr, knorm = p.k_norm_w != nullptr;
  // ---- query rows (whole rows per wave: nq is a multiple of the row's lanes) ----
  uint16_t* qdst = p.q_out + t * static_cast<int64_t>(p.num_heads) * D;
  auto query_chunk = [&](int c, uint4 raw) __attribute__((always_inline)) {
    float v[8], x[8];
    uint32_t b[8];
    unpack8(raw, p.bf16, v);
    transform8(p, v, qnorm, wq, cs_lds);
    round8(v, p.bf16, b, x);
    reinterpret_cast<uint4*>(qdst)[c] =
        make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
  };
#pragma unroll
  for (int j = 0; j < kQChunks; ++j) {
    const int c = tid + j * kPlanThreads;
    if (c < nq) query_chunk(c, qr[j]);
  }
  for (int c = tid + kQChunks * kPlanThreads; c < nq; c += kPlanThreads) query_chunk(c, qsrc[c]);
  if (!kv) return;
  // ---- key rows, then the value row ----
  const int64_t dst = slot * p.row_elems;
  auto key_value_chunk = [&](int c, uint4 kraw, uint4 vraw) __attribute__((always_inline)) {
    float v[8], x[8];
    uint32_t b[8];
    unpack8(kraw, p.bf16, v);
    transform8(p, v, knorm, wk, cs_lds);
    round8(v, p.bf16, b, x);
    store_chunk(p, false, c, dst, x, b);
    const uint32_t wv[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = (wv[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      x[e] = elem_value(b[e], p.bf16);
    }
    store_chunk(p, true, c, dst, x, b);
  };
  if (tid < nk) key_value_chunk(tid, kr, vr);
  for (int c = tid + kPlanThreads; c < nk; c += kPlanThreads) key_value_chunk(c, ksrc[c], vsrc[c]);
}

// LDS of the kernel: the plan's scan buffer and decode records (first
// workgroup), or a scatter workgroup's staged sequence offsets and the
// prologue's (cos, sin) table, overlaid, so that the scatter workgroups are
// not held to the plan's LDS (more of them per compute unit)
constexpr size_t kPlanSmem = kPlanThreads * sizeof(int3) + kPlanLdsSeqs * sizeof(int4) + kCostBins * sizeof(int);
constexpr size_t kTokenSmem = kScatterLdsCum * sizeof(int) + kMaxRotaryPairs * sizeof(float2);
constexpr size_t kScatterSmem = kPlanSmem > kTokenSmem ? kPlanSmem : kTokenSmem;

__global__ __launch_bounds__(kPlanThreads) void scatter_plan_kernel(ScatterPlanParams p) {
  __shared__ __align__(16) char smem[kScatterSmem];
  // workgroup 0 plans (dispatched first, it overlaps the scatter of long
  // calls); workgroup t + 1 scatters token t
  if (blockIdx.x == 0) {
    plan(p, smem);
    return;
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) - 1;
  // the sequence of token t: a binary search over cum, staged in LDS by one
  // coalesced load (long batches search global memory)
  int* cum_lds = reinterpret_cast<int*>(smem);
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
  if (p.pro) {  // (every token: its query row is transformed even when its slot is -1)
    prologue_token(p, t, slot, reinterpret_cast<float2*>(smem + kScatterLdsCum * sizeof(int)));
    return;
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

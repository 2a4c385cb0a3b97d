// Split-KV paged decode attention and the fixed-order merge of its splits.
//
// Decode rows are sequences with exactly one new token.  Their history is cut
// into splits of split_keys positions; one work item is (sequence, split,
// kv head, head chunk) and covers GH query heads of one GQA group, so each
// key/value byte is read once for all of them.  Inside a workgroup the four
// waves take interleaved 16-key tiles of the split and keep their own
// online-softmax state; the waves' states are combined in wave order and the
// split's (out, lse) state is either written as the final fp16 row (one
// split) or stored as fp32 partials for merge_kernel.
//
// Partial states and their merge follow "WS2 CP-Aware Attention Contract",
// Reduction Semantics: partial state (out, lse), online-softmax merge by lse,
// fp32 accumulation, fixed order of increasing key position, one downcast at
// the final write.  Here lse is kept in base 2 of the scaled scores
// (lse2 = lse / ln 2), which is the same merge.
//
// Per 16-key tile a wave
//   * loads K in "QK layout": 8 lanes per key, each lane 16-byte pieces
//     r, r+8 of the key row (contiguous 128-byte runs per instruction), and V
//     in "PV layout": D/8 lanes per key, one 16-byte piece each;
//   * forms q.k with v_dot2 (fp16 pairs, fp32 accumulate) and sums the 8
//     lanes of a key with DPP;
//   * takes the tile max across lanes, rescales its running sums only when
//     the max grew by more than 2^8 (exact: out = acc/l uses one reference);
//   * hands the probabilities to the PV layout through a per-wave LDS slot
//     and accumulates p*v in fp32 with mixed-precision FMAs.
// The next tile's K/V registers are loaded before the current tile is used.
#include "pa_internal.h"

#include <utility>

namespace pa {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowRor8 = 0x128;

__device__ inline float dot8(const uint4& a, const uint4& b, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.x), __builtin_bit_cast(h2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.y), __builtin_bit_cast(h2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.z), __builtin_bit_cast(h2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.w), __builtin_bit_cast(h2_t, b.w), acc, false);
  return acc;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(h2_t, w).x);
}
__device__ inline float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(h2_t, w).y);
}

__device__ inline uint16_t to_half_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <int D, int GH>
struct DecodeShape {
  static constexpr int R = 8;                  // lanes per key (QK)
  static constexpr int CH = D / (8 * R);       // 16-byte pieces per lane (QK)
  static constexpr int C = D / 8;              // lanes per key (PV)
  static constexpr int KPV = 64 / C;           // keys per PV pass
  static constexpr int PVP = kDecodeTile / KPV;  // PV passes per tile
  static_assert(CH >= 1 && PVP >= 1, "unsupported head size");
};

// x combined with lane x^16 / x^32 (VALU lane swaps, no LDS round trip)
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

#define PA_LDS __attribute__((address_space(3)))
#define PA_GLOBAL __attribute__((address_space(1)))

template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      reinterpret_cast<const PA_LDS char*>(reinterpret_cast<uintptr_t>(p))));
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte LDS read of a buffer filled by direct global->LDS loads.  Written as
// asm so that the compiler adds no wait on those loads of its own (the caller
// waits on them explicitly); the value may only be used after lds_ready().
template <int OFF>
__device__ inline u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}
// Waits for the LDS reads above; tying the value to the wait keeps every use
// after it.
__device__ inline uint4 lds_ready(u32x4 v) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v)::"memory");
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int D>
struct DecodeTileShape {
  static constexpr int CH = D / 64;        // QK pieces per lane per key
  static constexpr int KLOADS = 2 * CH;    // 1 KB direct loads of K per tile
  static constexpr int VLOADS = D / 32;    // 1 KB direct loads of V per tile (PVP)
  static constexpr int LOADS = KLOADS + VLOADS;
  static constexpr int BYTES = LOADS * 1024;
};

// One work item per wave: (sequence, split of kDecodeSplitKeys positions, kv
// head, head chunk).  Waves are independent (no barriers) and take items in
// grid-stride order (split items are near-uniform in cost; a shared queue
// counter would serialise every wave on one device-scope atomic).  A wave
// streams its item's 16-key tiles through a ring of two LDS buffers filled by
// direct global->LDS loads (global_load_lds_dwordx4), one tile ahead: in-flight
// bytes cost no registers, and the lane mapping of each 1 KB load is the
// compute layout itself, so lane i reads back its own 16 bytes at 16 i.  The
// next item's page ids and query rows are fetched while the current item is
// finished.
template <int D, int GH>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(AttnParams p) {
  using S = DecodeShape<D, GH>;
  using TS = DecodeTileShape<D>;
  constexpr int CH = S::CH, C = S::C, KPV = S::KPV, PVP = S::PVP;
  constexpr int NW = kDecodeThreads / 64;

  __shared__ float lds_p[NW][kDecodeTile][GH];
  // the ring: two separate objects so that reading one never waits for a
  // fill of the other
  __shared__ __align__(16) char ring0[NW][TS::BYTES];
  __shared__ __align__(16) char ring1[NW][TS::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kk = lane >> 3, r = lane & 7;  // QK layout
  const int a = lane / C, c = lane % C;    // PV layout

  const int hc_count = p.group / GH;
  const int per_item = p.kv_heads * hc_count;
  const int total = p.ws_ctrl[kCtrlDecodeItems] * per_item;
  const int64_t kv_row = static_cast<int64_t>(p.kv_heads) * D;
  // element offsets of this lane's pieces inside one tile (relative to key 0)
  int koffs[2][CH], voffs[PVP];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int ci = 0; ci < CH; ++ci)
      koffs[pp][ci] = (8 * pp + kk) * static_cast<int>(kv_row) + (r + 8 * ci) * 8;
#pragma unroll
  for (int tt = 0; tt < PVP; ++tt) voffs[tt] = (KPV * tt + a) * static_cast<int>(kv_row) + c * 8;

  const int nwaves = static_cast<int>(gridDim.x) * NW;
  struct ItemInfo {
    int b, split, kvh, hc, t, j_begin, j_end, ntiles, h0;
  };
  auto describe = [&](int item) {
    ItemInfo it;
    const int2 bsplit = p.items[item / per_item];
    const int rem = item % per_item;
    it.kvh = rem / hc_count;
    it.hc = rem % hc_count;
    it.b = bsplit.x;
    it.split = bsplit.y;
    it.t = p.cum[it.b];
    const int L = p.past[it.b] + 1;
    it.j_begin = it.split * kDecodeSplitKeys;
    it.j_end = min(L, it.j_begin + kDecodeSplitKeys);
    it.ntiles = (it.j_end - it.j_begin + kDecodeTile - 1) / kDecodeTile;
    it.h0 = it.kvh * p.group + it.hc * GH;
    return it;
  };
  // page ids of all tiles of an item (a tile lies inside one page): lane i
  // holds tile i's page
  auto pages_of = [&](const ItemInfo& it) {
    const int32_t* btab = p.block_table + static_cast<int64_t>(it.b) * p.max_blocks;
    return lane < it.ntiles ? btab[(it.j_begin + kDecodeTile * lane) / p.block_size] : 0;
  };
  auto q_of = [&](const ItemInfo& it, uint4 (&q)[GH][CH]) {
    const uint16_t* qrow = p.q + static_cast<int64_t>(it.t) * p.q_stride + static_cast<int64_t>(it.h0) * D;
#pragma unroll
    for (int g = 0; g < GH; ++g)
#pragma unroll
      for (int i = 0; i < CH; ++i)
        q[g][i] = *reinterpret_cast<const uint4*>(qrow + g * D + (r + 8 * i) * 8);
  };

  int item = static_cast<int>(blockIdx.x) * NW + wave;
  if (item >= total) return;
  ItemInfo nx = describe(item);
  int page_nx = pages_of(nx);
  uint4 qr[GH][CH];
  q_of(nx, qr);
  for (; item < total; item += nwaves) {
    const ItemInfo it = nx;
    const int my_page = page_nx;
    const bool has_next = item + nwaves < total;
    if (has_next) {  // the next item's metadata and page ids
      nx = describe(item + nwaves);
      page_nx = pages_of(nx);
    }
    const int b = it.b, split = it.split, kvh = it.kvh, t = it.t;
    const int j_begin = it.j_begin, j_end = it.j_end, ntiles = it.ntiles, h0 = it.h0;

    float m[GH], l[GH], acc[GH][8];
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      m[g] = kNegInf;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    const uint16_t* kc = p.key_cache + static_cast<int64_t>(kvh) * D;
    const uint16_t* vc = p.value_cache + static_cast<int64_t>(kvh) * D;
    // direct fill of one ring buffer with tile i (clamped to the last tile so
    // that every path issues the same loads; a repeated tile is an L2 hit)
    auto issue = [&](int i, char* buf) {
      const int j0 = j_begin + kDecodeTile * i;
      const int pb = __builtin_amdgcn_readlane(my_page, i);
      const int64_t base = (static_cast<int64_t>(pb) * p.block_size + j0 % p.block_size) * kv_row;
      const uint16_t* kt = kc + base;
      const uint16_t* vt = vc + base;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int ci = 0; ci < CH; ++ci)
          __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)(kt + koffs[pp][ci]),
                                           (PA_LDS void*)(buf + 1024 * (pp * CH + ci)), 16, 0, 0);
#pragma unroll
      for (int tt = 0; tt < PVP; ++tt)
        __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)(vt + voffs[tt]),
                                         (PA_LDS void*)(buf + 1024 * (TS::KLOADS + tt)), 16, 0, 0);
    };

    auto compute = [&](int i, const char* buf) {
      const int nvalid = j_end - (j_begin + kDecodeTile * i);
      // the tile's bytes: lane reads back its own 16 bytes of each 1 KB load
      u32x4 kx[2 * CH], vx[PVP];
      const uint32_t at = lds_addr(buf) + 16 * lane;
      static_for<2 * CH>([&](auto n) { kx[n] = lds_read16<1024 * n>(at); });
      static_for<PVP>([&](auto n) { vx[n] = lds_read16<1024 * (TS::KLOADS + n)>(at); });
      uint4 kr[2][CH], vr[PVP];
#pragma unroll
      for (int n = 0; n < 2 * CH; ++n) kr[n / CH][n % CH] = lds_ready(kx[n]);
#pragma unroll
      for (int n = 0; n < PVP; ++n) vr[n] = lds_ready(vx[n]);
      // scores of this lane's two keys (8*pp + kk), all GH heads
      float s[2][GH];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          float x = 0.f;
#pragma unroll
          for (int ci = 0; ci < CH; ++ci) x = dot8(qr[g][ci], kr[pp][ci], x);
          x += dpp<kDppQuadXor1>(x);
          x += dpp<kDppQuadXor2>(x);
          x += dpp<kDppHalfMirror>(x);
          s[pp][g] = (8 * pp + kk < nvalid) ? x * p.scale_log2 : kNegInf;
        }
      // tile max per head (made wave-uniform) and lazy rescale
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        float mx = fmaxf(s[0][g], s[1][g]);
        mx = fmaxf(mx, dpp<kDppRowRor8>(mx));
        mx = max_xor32(max_xor16(mx));
        mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));
        if (mx > m[g] + 8.f) {
          const float alpha = fast_exp2(m[g] - mx);
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
          m[g] = mx;
        }
      }
      // probabilities; lane r==0 of each key publishes them for the PV layout
      if (r == 0) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int g = 0; g < GH; ++g) {
            const float pr = fast_exp2(s[pp][g] - m[g]);
            l[g] += pr;
            lds_p[wave][8 * pp + kk][g] = pr;
          }
      }
      wave_lds_sync();
      // keys beyond the history may hold any bits: zero their values
      if (nvalid < kDecodeTile) {
#pragma unroll
        for (int tt = 0; tt < PVP; ++tt)
          if (KPV * tt + a >= nvalid) vr[tt] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int tt = 0; tt < PVP; ++tt) {
        float pv[GH];
#pragma unroll
        for (int g = 0; g < GH; ++g) pv[g] = lds_p[wave][KPV * tt + a][g];
        const uint32_t w[4] = {vr[tt].x, vr[tt].y, vr[tt].z, vr[tt].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = half_lo(w[q]), v1 = half_hi(w[q]);
#pragma unroll
          for (int g = 0; g < GH; ++g) {
            acc[g][2 * q] = fmaf(pv[g], v0, acc[g][2 * q]);
            acc[g][2 * q + 1] = fmaf(pv[g], v1, acc[g][2 * q + 1]);
          }
        }
      }
      wave_lds_sync();
    };

    char* buf0 = ring0[wave];
    char* buf1 = ring1[wave];
    const int last = ntiles - 1;
    issue(0, buf0);
    for (int i = 0; i < ntiles; i += 2) {
      issue(min(i + 1, last), buf1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TS::LOADS) : "memory");  // tile i landed
      compute(i, buf0);
      issue(min(i + 2, last), buf0);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TS::LOADS) : "memory");  // tile i+1 landed
      if (i + 1 < ntiles) compute(i + 1, buf1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no fill in flight past the item

    if (has_next) q_of(nx, qr);  // lands while this item is reduced and written

    // wave totals: l over all lanes, acc over the KPV key groups of a piece
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      float x = l[g];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
      l[g] = x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float y = acc[g][e];
#pragma unroll
        for (int off = C; off < 64; off <<= 1) y += __shfl_xor(y, off);
        acc[g][e] = y;
      }
    }
    if (a == 0) {  // lanes 0..C-1 hold head-dim piece c of every head
      const int2 ss = p.seq_split[b];
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        const int h = h0 + g;
        const float inv = 1.f / l[g];
        if (ss.y == 1) {
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = static_cast<uint32_t>(to_half_bits(acc[g][2 * q] * inv)) |
                   (static_cast<uint32_t>(to_half_bits(acc[g][2 * q + 1] * inv)) << 16);
          *reinterpret_cast<uint4*>(p.out + static_cast<int64_t>(t) * p.num_heads * D +
                                    static_cast<int64_t>(h) * D + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          const int64_t slot = static_cast<int64_t>(ss.x + split) * p.num_heads + h;
          float4* po = reinterpret_cast<float4*>(p.part_o + slot * D + c * 8);
          po[0] = make_float4(acc[g][0] * inv, acc[g][1] * inv, acc[g][2] * inv, acc[g][3] * inv);
          po[1] = make_float4(acc[g][4] * inv, acc[g][5] * inv, acc[g][6] * inv, acc[g][7] * inv);
          if (c == 0) p.part_lse[slot] = m[g] + __log2f(l[g]);
        }
      }
    }
  }
}

// Fixed-order merge of the split partials of one decode row, one wave per
// (sequence, head): out = sum_s 2^{lse_s - M} o_s / sum_s 2^{lse_s - M}.
// Lane s reads lse_s, the wave forms M and the weights, then every lane sums
// its head-dim elements over s = 0, 1, ... in that order.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  constexpr int E = D / 64;
  const int b = blockIdx.x;
  const int2 ss = p.seq_split[b];
  if (ss.y <= 1) return;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= p.num_heads) return;
  const int lane = threadIdx.x & 63;
  const int n = ss.y;
  float M = kNegInf;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int s = s0 + lane;
    const float x = s < n ? p.part_lse[static_cast<int64_t>(ss.x + s) * p.num_heads + h] : kNegInf;
    M = fmaxf(M, x);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float num[E], den = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) num[e] = 0.f;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int cnt = min(64, n - s0);
    const float lw = lane < cnt
        ? fast_exp2(p.part_lse[static_cast<int64_t>(ss.x + s0 + lane) * p.num_heads + h] - M) : 0.f;
    for (int k = 0; k < cnt; ++k) {
      const float w = __shfl(lw, k);
      const int64_t slot = static_cast<int64_t>(ss.x + s0 + k) * p.num_heads + h;
      den += w;
      if constexpr (E == 2) {
        const float2 o = *reinterpret_cast<const float2*>(p.part_o + slot * D + lane * 2);
        num[0] = fmaf(w, o.x, num[0]);
        num[1] = fmaf(w, o.y, num[1]);
      } else {
        num[0] = fmaf(w, p.part_o[slot * D + lane], num[0]);
      }
    }
  }
  const int t = p.cum[b];
  uint16_t* o = p.out + static_cast<int64_t>(t) * p.num_heads * D + static_cast<int64_t>(h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) o[lane * E + e] = to_half_bits(num[e] / den);
}

template <int D, int GH>
hipError_t launch_decode_t(const AttnParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, GH>), dim3(grid), dim3(kDecodeThreads), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const AttnParams& p, int gh, int grid, hipStream_t s) {
  switch (gh) {
    case 1: return launch_decode_t<D, 1>(p, grid, s);
    case 2: return launch_decode_t<D, 2>(p, grid, s);
    case 3: return launch_decode_t<D, 3>(p, grid, s);
    case 4: return launch_decode_t<D, 4>(p, grid, s);
    case 5: return launch_decode_t<D, 5>(p, grid, s);
    case 6: return launch_decode_t<D, 6>(p, grid, s);
    case 7: return launch_decode_t<D, 7>(p, grid, s);
    case 8: return launch_decode_t<D, 8>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int decode_heads_per_item(int group) {
  for (int gh = 8; gh > 1; --gh)
    if (group % gh == 0) return gh;
  return 1;
}

hipError_t launch_decode(const AttnParams& p, int head_size, int grid, hipStream_t s) {
  const int gh = decode_heads_per_item(p.group);
  if (head_size == 128) return launch_decode_d<128>(p, gh, grid, s);
  if (head_size == 64) return launch_decode_d<64>(p, gh, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnParams& p, int head_size, hipStream_t s) {
  const dim3 grid(p.batch, (p.num_heads + 3) / 4);
  if (head_size == 128) hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, s, p);
  else if (head_size == 64) hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa

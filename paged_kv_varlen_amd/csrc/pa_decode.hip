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

template <int D, int GH>
__device__ inline void load_tile(const uint16_t* kbase, const uint16_t* vbase, int64_t kv_row,
                                 int kk, int r, int a, int c, uint4 (&kr)[2][D / 64],
                                 uint4 (&vr)[DecodeShape<D, GH>::PVP]) {
  using S = DecodeShape<D, GH>;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int i = 0; i < S::CH; ++i)
      kr[pp][i] = *reinterpret_cast<const uint4*>(kbase + (8 * pp + kk) * kv_row + (r + 8 * i) * 8);
#pragma unroll
  for (int tt = 0; tt < S::PVP; ++tt)
    vr[tt] = *reinterpret_cast<const uint4*>(vbase + (S::KPV * tt + a) * kv_row + c * 8);
}

template <int D, int GH>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(AttnParams p) {
  using S = DecodeShape<D, GH>;
  constexpr int CH = S::CH, C = S::C, KPV = S::KPV, PVP = S::PVP;

  __shared__ float lds_p[4][kDecodeTile][GH];
  __shared__ float lds_acc[4][GH][D];
  __shared__ float lds_ml[4][GH][2];
  __shared__ int lds_item;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kk = lane >> 3, r = lane & 7;  // QK layout
  const int a = lane / C, c = lane % C;    // PV layout

  const int hc_count = p.group / GH;
  const int per_item = p.kv_heads * hc_count;
  const int total = p.ws_ctrl[kCtrlDecodeItems] * per_item;
  const int64_t kv_row = static_cast<int64_t>(p.kv_heads) * D;

  if (threadIdx.x == 0) lds_item = atomicAdd(&p.ws_ctrl[kCtrlDecodeNext], 1);
  __syncthreads();
  int item = lds_item;
  while (item < total) {
    __syncthreads();
    if (threadIdx.x == 0) lds_item = atomicAdd(&p.ws_ctrl[kCtrlDecodeNext], 1);

    const int2 bsplit = p.items[item / per_item];
    const int rem = item % per_item;
    const int kvh = rem / hc_count;
    const int hc = rem % hc_count;
    const int b = bsplit.x, split = bsplit.y;
    const int t = p.cum[b];
    const int L = p.past[b] + 1;
    const int j_begin = split * p.split_keys;
    const int j_end = min(L, j_begin + p.split_keys);
    const int h0 = kvh * p.group + hc * GH;

    uint4 qr[GH][CH];
    const uint16_t* qrow = p.q + static_cast<int64_t>(t) * p.q_stride + static_cast<int64_t>(h0) * D;
#pragma unroll
    for (int g = 0; g < GH; ++g)
#pragma unroll
      for (int i = 0; i < CH; ++i)
        qr[g][i] = *reinterpret_cast<const uint4*>(qrow + g * D + (r + 8 * i) * 8);

    float m[GH], l[GH], acc[GH][8];
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      m[g] = kNegInf;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    const int32_t* btab = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
    const uint16_t* kc = p.key_cache + static_cast<int64_t>(kvh) * D;
    const uint16_t* vc = p.value_cache + static_cast<int64_t>(kvh) * D;
    auto tile_base = [&](int j0) -> int64_t {
      const int lb = j0 / p.block_size;
      const int pb = btab[lb];
      return (static_cast<int64_t>(pb) * p.block_size + (j0 - lb * p.block_size)) * kv_row;
    };

    int j0 = j_begin + kDecodeTile * wave;
    uint4 kr[2][CH], vr[PVP];
    if (j0 < j_end) {
      const int64_t base = tile_base(j0);
      load_tile<D, GH>(kc + base, vc + base, kv_row, kk, r, a, c, kr, vr);
    }
    while (j0 < j_end) {
      const int jn = j0 + 4 * kDecodeTile;
      uint4 kn[2][CH], vn[PVP];
      if (jn < j_end) {
        const int64_t base = tile_base(jn);
        load_tile<D, GH>(kc + base, vc + base, kv_row, kk, r, a, c, kn, vn);
      }
      const int nvalid = j_end - j0;

      // scores of this lane's two keys (8*pp + kk), all GH heads
      float s[2][GH];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          float x = 0.f;
#pragma unroll
          for (int i = 0; i < CH; ++i) x = dot8(qr[g][i], kr[pp][i], x);
          x += dpp<kDppQuadXor1>(x);
          x += dpp<kDppQuadXor2>(x);
          x += dpp<kDppHalfMirror>(x);
          s[pp][g] = (8 * pp + kk < nvalid) ? x * p.scale_log2 : kNegInf;
        }

      // tile max per head (wave-uniform) and lazy rescale
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        float mx = fmaxf(s[0][g], s[1][g]);
        mx = fmaxf(mx, dpp<kDppRowRor8>(mx));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));  // uniform
        if (mx > m[g] + 8.f) {
          const float alpha = fast_exp2(m[g] - mx);
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
          m[g] = mx;
        }
      }

      // probabilities; lane r==0 of each key publishes them for the PV layout
      float pr[2][GH];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int g = 0; g < GH; ++g) pr[pp][g] = fast_exp2(s[pp][g] - m[g]);
      if (r == 0) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int g = 0; g < GH; ++g) {
            l[g] += pr[pp][g];
            lds_p[wave][8 * pp + kk][g] = pr[pp][g];
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

#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int i = 0; i < CH; ++i) kr[pp][i] = kn[pp][i];
#pragma unroll
      for (int tt = 0; tt < PVP; ++tt) vr[tt] = vn[tt];
      j0 = jn;
    }

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
    if (a == 0) {
#pragma unroll
      for (int g = 0; g < GH; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) lds_acc[wave][g][c * 8 + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        lds_ml[wave][g][0] = m[g];
        lds_ml[wave][g][1] = l[g];
      }
    }
    __syncthreads();

    // combine the four waves in wave order
    const int2 ss = p.seq_split[b];
    for (int idx = threadIdx.x; idx < GH * D; idx += kDecodeThreads) {
      const int g = idx / D, d = idx % D;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, lds_ml[w][g][0]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = fast_exp2(lds_ml[w][g][0] - M);
        num = fmaf(sc, lds_acc[w][g][d], num);
        den = fmaf(sc, lds_ml[w][g][1], den);
      }
      const int h = h0 + g;
      if (ss.y == 1) {
        p.out[static_cast<int64_t>(t) * p.num_heads * D + static_cast<int64_t>(h) * D + d] =
            to_half_bits(num / den);
      } else {
        const int64_t slot = static_cast<int64_t>(ss.x + split) * p.num_heads + h;
        p.part_o[slot * D + d] = num / den;
        if (d == 0) p.part_lse[slot] = M + __log2f(den);
      }
    }
    item = lds_item;
  }
}

// Fixed-order merge of the split partials of one decode row, one wave per
// (sequence, head): out = sum_s 2^{lse_s - M} o_s / sum_s 2^{lse_s - M}.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  constexpr int E = D / 64;
  const int b = blockIdx.x;
  const int2 ss = p.seq_split[b];
  if (ss.y <= 1) return;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= p.num_heads) return;
  const int lane = threadIdx.x & 63;
  float M = kNegInf;
  for (int s = 0; s < ss.y; ++s)
    M = fmaxf(M, p.part_lse[static_cast<int64_t>(ss.x + s) * p.num_heads + h]);
  float num[E], den = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) num[e] = 0.f;
  for (int s = 0; s < ss.y; ++s) {
    const int64_t slot = static_cast<int64_t>(ss.x + s) * p.num_heads + h;
    const float w = fast_exp2(p.part_lse[slot] - M);
    den += w;
#pragma unroll
    for (int e = 0; e < E; ++e) num[e] = fmaf(w, p.part_o[slot * D + lane * E + e], num[e]);
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

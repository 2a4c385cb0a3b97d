// Causal varlen (chunked) prefill attention on gfx950 matrix cores.
//
// Rows are sequences with more than one new token.  A work item is
// (sequence, query tile, kv head): the workgroup owns kPrefillRows rows, each
// a (new-token position, query head) pair of one GQA group, laid out
// position-major (row f = position f / G, head f % G), so the K/V tiles it
// stages in LDS serve all G query heads of the group.  Each of the four waves
// owns 32 rows.
//
// Per 64-key tile the workgroup
//   * loads K and V rows of the tile through block_table (one 16-byte piece
//     per lane, 256 contiguous bytes per 16 lanes) into registers one tile
//     ahead, then stores K row-major and V transposed (V^T[d][key]) in LDS;
//     keys past the sequence's history are zero-filled, never read;
//   * computes S^T = K Q^T with v_mfma_f32_32x32x16_f16 (fp16 in, fp32
//     accumulate): a lane ends up holding 16 keys of one query row, so the
//     row max needs a single exchange with lane^32;
//   * masks keys after the row's position (bottom-right causal offset:
//     new row i of sequence b sits at past_b + i, "WS2 CP-Aware Attention
//     Contract", Mode-Specific Metadata), updates the online softmax in fp32
//     (scores in base 2; running sums rescaled only when the max grows by more
//     than 2^8), casts P to fp16 and sums the rounded P for the row total;
//   * accumulates O^T += V^T P^T with the same MFMA, P^T taken straight from
//     the S^T registers and V^T read from LDS with the matching key order.
// O is divided by the row sum and rounded to fp16 once, at the final write.
#include "pa_internal.h"

namespace pa {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct PrefillShape {
  static constexpr int BN = kPrefillKeys;
  static constexpr int KSTR = D + 8;          // halves per K row in LDS
  static constexpr int VSTR = BN + 4;         // halves per V^T row in LDS
  static constexpr int CPR = D / 8;           // 16-byte pieces per key row
  static constexpr int KPT = BN * CPR / kPrefillThreads;  // keys per thread (loader)
  static constexpr int KG = kPrefillThreads / CPR;         // key groups (loader)
  static_assert(KPT * KG == BN && (KPT == 2 || KPT == 4), "loader shape");
  static constexpr int QK_STEPS = D / 16;     // MFMA k-steps over the head dim
  static constexpr int O_TILES = D / 32;      // 32-wide d tiles of O^T
};

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(AttnParams p) {
  using S = PrefillShape<D>;
  constexpr int BN = S::BN, KSTR = S::KSTR, VSTR = S::VSTR, CPR = S::CPR, KPT = S::KPT;

  __shared__ __align__(16) uint16_t k_lds[BN * KSTR];
  __shared__ __align__(16) uint16_t vt_lds[D * VSTR];
  __shared__ int lds_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;   // MFMA column owned by this lane
  const int lhalf = lane >> 5;  // which k-half of the MFMA operand
  const int G = p.group;
  const int P = p.prefill_positions;
  const int total = p.ws_ctrl[kCtrlPrefillItems] * p.kv_heads;
  const int64_t kv_row = static_cast<int64_t>(p.kv_heads) * D;
  const int64_t out_stride = static_cast<int64_t>(p.num_heads) * D;

  // loader role: pieces cq of keys KPT*kg .. KPT*kg+KPT-1
  const int cq = tid % CPR;
  const int kg = tid / CPR;

  if (tid == 0) lds_item = atomicAdd(&p.ws_ctrl[kCtrlPrefillNext], 1);
  __syncthreads();
  int item = lds_item;
  while (item < total) {
    __syncthreads();
    if (tid == 0) lds_item = atomicAdd(&p.ws_ctrl[kCtrlPrefillNext], 1);

    const int2 bt = p.items[item / p.kv_heads];
    const int kvh = item % p.kv_heads;
    const int b = bt.x, tile = bt.y;
    const int t0 = p.cum[b];
    const int qlen = p.cum[b + 1] - t0;
    const int past = p.past[b];
    const int L = past + qlen;
    const int i0 = tile * P;
    const int i1 = min(i0 + P, qlen);
    const int kv_end = past + i1;  // keys [0, kv_end) are visible to some row

    // this lane's query row
    const int f = wave * 32 + lrow;
    const int pos_local = f / G;
    const int g = f % G;
    const bool row_valid = (f < P * G) && (i0 + pos_local < i1);
    const int row_pos = past + i0 + (row_valid ? pos_local : 0);
    const int head = kvh * G + g;
    // the last position any row of this wave needs
    const int wave_last = past + min(i0 + ((wave * 32 + 31) < P * G ? (wave * 32 + 31) / G : P - 1),
                                     i1 - 1);

    half8_t qf[S::QK_STEPS];
    {
      const uint16_t* qrow = p.q + static_cast<int64_t>(t0 + i0 + pos_local) * p.q_stride +
                             static_cast<int64_t>(head) * D;
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) {
        if (row_valid)
          qf[kk] = *reinterpret_cast<const half8_t*>(qrow + 16 * kk + 8 * lhalf);
        else
          qf[kk] = half8_t{};
      }
    }

    f32x16_t o[S::O_TILES];
#pragma unroll
    for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] = f32x16_t{};
    float m = kNegInf, l = 0.f;

    const int32_t* btab = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
    const uint16_t* kcache = p.key_cache + static_cast<int64_t>(kvh) * D;
    const uint16_t* vcache = p.value_cache + static_cast<int64_t>(kvh) * D;

    uint4 kreg[KPT], vreg[KPT];
    auto load_regs = [&](int j0) {
      const int jf = j0 + KPT * kg;  // first key of this thread's group
      if (jf < L) {
        const int lb = jf / p.block_size;
        const int64_t slot = static_cast<int64_t>(btab[lb]) * p.block_size + (jf - lb * p.block_size);
        const uint16_t* kp = kcache + slot * kv_row + cq * 8;
        const uint16_t* vp = vcache + slot * kv_row + cq * 8;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          if (jf + i < L) {
            kreg[i] = *reinterpret_cast<const uint4*>(kp + i * kv_row);
            vreg[i] = *reinterpret_cast<const uint4*>(vp + i * kv_row);
          } else {
            kreg[i] = make_uint4(0u, 0u, 0u, 0u);
            vreg[i] = make_uint4(0u, 0u, 0u, 0u);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          kreg[i] = make_uint4(0u, 0u, 0u, 0u);
          vreg[i] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    };

    load_regs(0);
    for (int j0 = 0; j0 < kv_end; j0 += BN) {
      __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        *reinterpret_cast<uint4*>(&k_lds[(KPT * kg + i) * KSTR + cq * 8]) = kreg[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // d pair (2q, 2q+1) of piece cq
        uint32_t lo[KPT], hi[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const uint32_t wd = q == 0 ? vreg[i].x : q == 1 ? vreg[i].y : q == 2 ? vreg[i].z : vreg[i].w;
          lo[i] = wd & 0xFFFFu;
          hi[i] = wd >> 16;
        }
        uint16_t* dst0 = &vt_lds[(cq * 8 + 2 * q) * VSTR + KPT * kg];
        uint16_t* dst1 = dst0 + VSTR;
        if constexpr (KPT == 4) {
          *reinterpret_cast<uint2*>(dst0) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
          *reinterpret_cast<uint2*>(dst1) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        } else {
          *reinterpret_cast<uint32_t*>(dst0) = lo[0] | (lo[1] << 16);
          *reinterpret_cast<uint32_t*>(dst1) = hi[0] | (hi[1] << 16);
        }
      }
      __syncthreads();
      if (j0 + BN < kv_end) load_regs(j0 + BN);

      if (j0 > wave_last) continue;  // tile lies after every row of this wave

      // S^T[key][row] for keys j0 .. j0+63 as two 32x32 tiles
      f32x16_t s[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        s[nt] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < S::QK_STEPS; ++kk) {
          const half8_t ka = *reinterpret_cast<const half8_t*>(
              &k_lds[(32 * nt + lrow) * KSTR + 16 * kk + 8 * lhalf]);
          s[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[kk], s[nt], 0, 0, 0);
        }
      }

      // register i of tile nt holds key j0 + 32nt + 8(i/4) + 4*lhalf + i%4
      float mx = kNegInf;
      const bool need_mask = j0 + BN - 1 > row_pos;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[nt][i] * p.scale_log2;
          if (need_mask) {
            const int key = j0 + 32 * nt + 8 * (i >> 2) + 4 * lhalf + (i & 3);
            if (key > row_pos) x = kNegInf;
          }
          s[nt][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (mx > m + 8.f) {
        const float alpha = fast_exp2(m - mx);
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] *= alpha;
        m = mx;
      }

      // P^T operands: 16-key step ks takes registers 8(ks%2)..+7 of tile ks/2
      half8_t pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 ph = static_cast<_Float16>(fast_exp2(s[ks >> 1][8 * (ks & 1) + e] - m));
          l += static_cast<float>(ph);  // normalise by exactly what the MFMA multiplies
          pb[ks][e] = ph;
        }

      // O^T[d][row] += V^T[d][key] P^T[key][row]
#pragma unroll
      for (int mt = 0; mt < S::O_TILES; ++mt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint16_t* vrow = &vt_lds[(32 * mt + lrow) * VSTR + 16 * ks + 4 * lhalf];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, va), pb[ks],
                                                         o[mt], 0, 0, 0);
        }
    }

    // normalise and write: register i of tile mt is d = 32mt + 8(i/4) + 4*lhalf + i%4
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.f / lt;
    if (row_valid) {
      uint16_t* orow = p.out + static_cast<int64_t>(t0 + i0 + pos_local) * out_stride +
                       static_cast<int64_t>(head) * D;
#pragma unroll
      for (int mt = 0; mt < S::O_TILES; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const _Float16 x0 = static_cast<_Float16>(o[mt][4 * q + 2 * e] * inv);
            const _Float16 x1 = static_cast<_Float16>(o[mt][4 * q + 2 * e + 1] * inv);
            w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x0)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x1)) << 16);
          }
          *reinterpret_cast<uint2*>(orow + 32 * mt + 8 * q + 4 * lhalf) = make_uint2(w[0], w[1]);
        }
    }
    item = lds_item;
  }
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, int head_size, int grid, hipStream_t s) {
  if (head_size == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(grid), dim3(kPrefillThreads), 0, s, p);
  else if (head_size == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(grid), dim3(kPrefillThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa

// Causal varlen (chunked) prefill attention on gfx950 matrix cores.
//
// Rows are sequences with more than one new token.  A work item is
// (sequence, query tile, kv head): the workgroup owns kPrefillRows rows, each
// a (new-token position, query head) pair of one GQA group, laid out
// position-major (row f = position f / G, head f % G), so every K/V byte
// staged in LDS serves all G query heads of the group.
//
// Eight waves: wave w owns rows 32*(w%4) .. +31 ("row group") and the keys of
// one half ("kv group" w/4) of every 128-key super-tile, so each SIMD runs two
// waves while every wave keeps 32 rows of MFMA operands.  The two kv groups
// keep separate online-softmax states and are merged once, in LDS, at the end
// of the item (fixed order: group 0 then group 1).
//
// Per 128-key super-tile (double-buffered LDS, one barrier per super-tile):
//   * every wave fills 16 key rows of K and V with direct global->LDS loads
//     (global_load_lds_dwordx4: lane i's 16 bytes land at M0 + 16 i), one
//     super-tile ahead, through block_table (the page id is a scalar value
//     fetched one super-tile earlier).  Keys past the history read a zeroed
//     page of the workspace instead of the cache.  K and V rows stay
//     row-major (2*D bytes); their 16-byte chunks are XOR-swizzled per row so
//     that the reads below hit distinct LDS banks;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_f16 (fp16 in, fp32 accumulate): a
//     lane holds 16 keys of one query row, so the row max needs a single
//     exchange with lane^32;
//   * keys after a row's position are masked only on tiles that cross the
//     diagonal (bottom-right causal offset: new row i of sequence b is at
//     past_b + i, "WS2 CP-Aware Attention Contract", Mode-Specific Metadata);
//   * online softmax in fp32 on base-2 scores (running sums rescaled only
//     when the max grows by more than 2^8), P rounded to fp16;
//   * O^T += V^T P^T with the same MFMA.  P^T comes straight from the S^T
//     registers; the V^T operand is read from the row-major V tile with the
//     LDS transpose read ds_read_b64_tr_b16 (within 16 lanes, lanes 4r..4r+3
//     supply 16 consecutive halves of "row" r and lane i receives element i
//     of rows 0..3), which yields 4 consecutive keys of one head-dim column
//     per lane, in the key order of the P^T registers.
// O is divided by the row sum and rounded to fp16 once, at the final write.
//
// Items are spread over up to eight queues by kv head and a workgroup serves
// first the queue of the XCD it runs on (workgroup id mod 8), so each XCD's
// L2 holds the K/V of few heads; when its queue is empty it helps the others.
#include <type_traits>

#include "pa_internal.h"
#include "pa_merge.h"

namespace pa {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
#define PA_LDS __attribute__((address_space(3)))
#define PA_GLOBAL __attribute__((address_space(1)))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kSuper = 2 * kPrefillKeys;  // keys per super-tile (two kv groups)

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x combined with the same register of lane^32 (v_permlane32_swap: a VALU
// exchange of the two wave halves, no LDS round trip)
__device__ inline float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct PrefillShape {
  static constexpr int ROWB = D * 2;                 // bytes per key row
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 64 / CPR;     // rows per 1 KB direct load
  static constexpr int LOADS = 16 / ROWS_PER_LOAD;   // direct loads per wave per tensor
  static constexpr int BUF = kSuper * ROWB;          // bytes per K (or V) buffer
  static constexpr int K0 = 0;                       // K buffers at [0, 2 BUF)
  static constexpr int V0 = 2 * BUF;                 // V buffers at [2 BUF, 4 BUF)
  static constexpr int QK_STEPS = D / 16;            // MFMA k-steps over the head dim
  static constexpr int O_TILES = D / 32;             // 32-wide d tiles of O^T
  // chunk swizzles (in 16-byte chunks) of K and V rows
  static __device__ int k_swz(int row) { return D == 128 ? (row & 15) : (row & 7); }
  static __device__ int v_swz(int row) { return D == 128 ? ((row & 3) << 2) : 0; }
};

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(AttnParams p) {
  using S = PrefillShape<D>;
  constexpr int ROWB = S::ROWB, CPR = S::CPR;

  // four separate LDS objects (K/V x two buffers): the compiler can then see
  // that a fill of one buffer never aliases reads of the other and does not
  // make those reads wait for the fill
  __shared__ __align__(16) char k_lds0[S::BUF];
  __shared__ __align__(16) char k_lds1[S::BUF];
  __shared__ __align__(16) char v_lds0[S::BUF];
  __shared__ __align__(16) char v_lds1[S::BUF];
  __shared__ int lds_item;
  auto kbuf = [&](int b) -> char* { return b == 0 ? k_lds0 : k_lds1; };
  auto vbuf = [&](int b) -> char* { return b == 0 ? v_lds0 : v_lds1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3;      // row group
  const int kvg = wave >> 2;    // kv group
  const int lrow = lane & 31;   // MFMA column owned by this lane
  const int lhalf = lane >> 5;  // which k-half of the MFMA operand
  const int G = p.group;
  const int P = p.prefill_positions;
  const int64_t kv_row = static_cast<int64_t>(p.kv_heads) * D;
  const int64_t out_stride = static_cast<int64_t>(p.num_heads) * D;
  const float c = fabsf(p.scale_log2);
  const bool negate_q = p.scale_log2 < 0.f;  // fold the sign into Q (exact)

  // decode segments cut by a wave boundary: one wave per segment
  {
    const int segments = p.ws_ctrl[kCtrlDecodeSeqs] * p.decode_units;
    const int T = p.ws_ctrl[kCtrlDecodeTiles];
    const int nw = static_cast<int>(gridDim.x) * (kPrefillThreads / 64);
    for (int task = static_cast<int>(blockIdx.x) * (kPrefillThreads / 64) + wave; task < segments; task += nw)
      merge_segment<D>(p, task, T, lane);
  }

  const int nq = prefill_queue_count(p.kv_heads);
  const int hq = p.kv_heads / nq;
  const int per_queue = p.ws_ctrl[kCtrlPrefillItems] * hq;
  if (per_queue == 0) return;  // no multi-token sequence in this call
  const int home = static_cast<int>(blockIdx.x % 8) % nq;
  // the two waves of a SIMD (kv groups 0 and 1, same row group) run the same
  // phases; giving group 0 priority lets it run ahead, so one wave's softmax
  // (VALU) overlaps the other's matrix products
  if (kvg == 0) __builtin_amdgcn_s_setprio(1);

  // per-lane LDS byte offsets (everything else is an immediate)
  int koff[S::QK_STEPS];  // K fragment kk of row kvg*64 + lrow (+32 nt)
#pragma unroll
  for (int kk = 0; kk < S::QK_STEPS; ++kk) {
    const int row = kvg * kPrefillKeys + lrow;
    koff[kk] = row * ROWB + (((2 * kk + lhalf) ^ S::k_swz(row)) << 4);
  }
  int voff[S::O_TILES];  // transpose-read address of d tile mt (keys kvg*64 + ...)
  {
    const int grp = lane >> 4, i = lane & 15, r = i >> 2, q = i & 3;
    const int row = kvg * kPrefillKeys + 4 * (grp >> 1) + r;
#pragma unroll
    for (int mt = 0; mt < S::O_TILES; ++mt) {
      const int chunk = 4 * mt + 2 * (grp & 1) + (q >> 1);
      voff[mt] = row * ROWB + ((chunk ^ S::v_swz(row)) << 4) + ((q & 1) << 3);
    }
  }

  // loader: lane's row (within the wave's 16) and swizzled chunk per direct load
  int lk[S::LOADS], lv[S::LOADS], zk[S::LOADS], zv[S::LOADS], lrr[S::LOADS];
#pragma unroll
  for (int i = 0; i < S::LOADS; ++i) {
    const int rl = S::ROWS_PER_LOAD * i + lane / CPR;  // 16*wave + rl is the tile row
    const int phys = lane % CPR;
    zk[i] = (phys ^ S::k_swz(rl)) * 8;  // swizzles only see the low 4 row bits
    zv[i] = (phys ^ S::v_swz(rl)) * 8;
    lk[i] = rl * static_cast<int>(kv_row) + zk[i];
    lv[i] = rl * static_cast<int>(kv_row) + zv[i];
    lrr[i] = rl;
  }

  int queue = home, tried = 0;
  auto fetch = [&]() -> int {  // next item of this workgroup, or -1
    while (tried < nq) {
      if (tid == 0) lds_item = atomicAdd(&p.ws_ctrl[kCtrlPrefillQueue0 + queue], 1);
      __syncthreads();
      const int j = lds_item;
      __syncthreads();
      if (j < per_queue) return j;
      queue = queue + 1 == nq ? 0 : queue + 1;
      ++tried;
    }
    return -1;
  };

  for (int j = fetch(); j >= 0; j = fetch()) {
    const int2 bt = p.items[j / hq];
    const int kvh = queue + nq * (j % hq);
    const int b = bt.x, tile = bt.y;
    const int t0 = p.cum[b];
    const int qlen = p.cum[b + 1] - t0;
    const int past = p.past[b];
    const int L = past + qlen;
    const int i0 = tile * P;
    const int i1 = min(i0 + P, qlen);
    const int kv_end = past + i1;  // keys [0, kv_end) are visible to some row

    // this lane's query row
    const int f = rg * 32 + lrow;
    const int pos_local = f / G;
    const int g = f % G;
    const bool row_valid = (f < P * G) && (i0 + pos_local < i1);
    const int row_pos = past + i0 + (row_valid ? pos_local : 0);
    const int head = kvh * G + g;
    // positions spanned by this wave's valid rows
    const int wave_first = past + i0 + min((rg * 32) / G, max(0, i1 - i0 - 1));
    const int last_f = min(rg * 32 + 31, P * G - 1);
    const int wave_last = past + min(i0 + last_f / G, i1 - 1);

    half8_t qf[S::QK_STEPS];
    {
      const uint16_t* qrow = p.q + static_cast<int64_t>(t0 + i0 + pos_local) * p.q_stride +
                             static_cast<int64_t>(head) * D;
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) {
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (row_valid) raw = *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * lhalf);
        if (negate_q) {
          raw.x ^= 0x80008000u; raw.y ^= 0x80008000u; raw.z ^= 0x80008000u; raw.w ^= 0x80008000u;
        }
        qf[kk] = __builtin_bit_cast(half8_t, raw);
      }
    }

    f32x16_t o[S::O_TILES];
#pragma unroll
    for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] = f32x16_t{};
    float m = kNegInf, l = 0.f;

    const int32_t* btab = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
    const uint16_t* kcache = p.key_cache + static_cast<int64_t>(kvh) * D;
    const uint16_t* vcache = p.value_cache + static_cast<int64_t>(kvh) * D;

    // page id of this wave's 16 keys of super-tile j0 (0 past the history);
    // fetched one super-tile before its K/V so the dependent loads never wait
    auto page_of = [&](int j0) -> int {
      const int jw = j0 + 16 * wave;
      return jw < L ? btab[jw / p.block_size] : 0;
    };
    // direct global->LDS fill of this wave's 16 rows of super-tile j0
    auto issue = [&](int j0, int page, int buf) {
      const int jw = j0 + 16 * wave;
      const int pb = __builtin_amdgcn_readfirstlane(page);
      const int64_t at = (static_cast<int64_t>(pb) * p.block_size + (jw % p.block_size)) * kv_row;
      const uint16_t* kb = kcache + at;
      const uint16_t* vb = vcache + at;
      const bool all_in = jw + 16 <= L;  // uniform: the usual case
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const uint16_t* ksrc = kb + lk[i];
        const uint16_t* vsrc = vb + lv[i];
        if (!all_in && jw + lrr[i] >= L) {  // keys past the history read zeros
          ksrc = p.zeros + zk[i];
          vsrc = p.zeros + zv[i];
        }
        const int dst = (16 * wave + S::ROWS_PER_LOAD * i) * ROWB;
        __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)ksrc, (PA_LDS void*)(kbuf(buf) + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)vsrc, (PA_LDS void*)(vbuf(buf) + dst), 16, 0, 0);
      }
    };

    // one 64-key half-tile of this wave: S (two interleaved 32x32 chains),
    // softmax over the 64 keys, PV (four accumulators in turn)
    auto compute = [&](auto buf_tag, int jk, bool masked) {
      constexpr int buf = decltype(buf_tag)::value;
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) {
        half8_t ka[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          ka[nt] = *reinterpret_cast<const half8_t*>(kbuf(buf) + koff[kk] + nt * 32 * ROWB);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          s[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[nt], qf[kk], s[nt], 0, 0, 0);
      }
      // register i of chain nt holds key jk + 32nt + 8(i/4) + 4*lhalf + i%4
      if (masked) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = jk + 32 * nt + 8 * (i >> 2) + 4 * lhalf + (i & 3);
            if (key > row_pos) s[nt][i] = kNegInf;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nt][i]);
      mx = swap_halves_max(mx) * c;
      const bool grow = mx > m + 8.f;
      if (__ballot(grow) != 0) {  // wave-uniform branch; other lanes scale by 1
        const float alpha = grow ? fast_exp2(m - mx) : 1.f;
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] *= alpha;
        m = grow ? mx : m;
      }
      // P^T operand of 16-key step ks = registers 8(ks%2)..+7 of chain ks/2,
      // i.e. keys 16ks + 4*lhalf + 0..3 and 16ks + 8 + 4*lhalf + 0..3.  A row
      // that has seen no key yet (m = -inf) has only masked scores here.
      const float mref = m == kNegInf ? 0.f : m;
      half8_t pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pb[ks][e] = static_cast<_Float16>(fast_exp2(fmaf(s[ks >> 1][8 * (ks & 1) + e], c, -mref)));
      // row sum of exactly the fp16 weights the MFMA multiplies (v_dot2 with 1)
      typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
      const half2_t one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          l = __builtin_amdgcn_fdot2(half2_t{pb[ks][e], pb[ks][e + 1]}, one2, l, false);
      // O^T[d][row] += V^T[d][key] P^T[key][row]: the transpose read of rows
      // key0..key0+3 (key0 = 16ks + 4*lhalf, then +8) gives each lane the 4
      // keys of its d column, matching the order of the P^T registers
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8_t va[S::O_TILES];
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) {
          char* vb = vbuf(buf) + voff[mt] + 16 * ks * ROWB;
          const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PA_LDS fp16x4_t*)vb);
          const fp16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PA_LDS fp16x4_t*)(vb + 8 * ROWB));
          va[mt] = __builtin_shufflevector(__builtin_bit_cast(half4_t, lo), __builtin_bit_cast(half4_t, hi),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt)
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[mt], pb[ks], o[mt], 0, 0, 0);
      }
    };

    auto step = [&](auto buf_tag, int j0, int& page_next) {
      constexpr int buf = decltype(buf_tag)::value;
      if (j0 + kSuper < kv_end) {  // fill the other buffer while this one is used
        issue(j0 + kSuper, page_next, buf ^ 1);
        page_next = page_of(j0 + 2 * kSuper);
      }
      const int jk = j0 + kvg * kPrefillKeys;  // first key of this wave's half
      if (jk <= wave_last) {
        const bool masked = __builtin_amdgcn_readfirstlane(jk + kPrefillKeys - 1 > wave_first);
        compute(buf_tag, jk, masked);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's LDS fills landed
      __syncthreads();
    };

    issue(0, page_of(0), 0);
    int page_next = page_of(kSuper);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int j0 = 0; j0 < kv_end; j0 += 2 * kSuper) {
      step(std::integral_constant<int, 0>{}, j0, page_next);
      if (j0 + kSuper < kv_end) step(std::integral_constant<int, 1>{}, j0 + kSuper, page_next);
    }

    // merge the two kv groups (group 0 first) and write; reuse the K buffers
    // [4 row groups][O_TILES*16][64 lanes] over the K buffers, [4][2][64] after
    float* xo = reinterpret_cast<float*>(k_lds0);
    float* xml = reinterpret_cast<float*>(v_lds0);
    if (kvg == 1) {
#pragma unroll
      for (int mt = 0; mt < S::O_TILES; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) xo[(rg * S::O_TILES * 16 + mt * 16 + i) * 64 + lane] = o[mt][i];
      xml[(rg * 2 + 0) * 64 + lane] = m;
      xml[(rg * 2 + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (kvg == 0) {
      const float m1 = xml[(rg * 2 + 0) * 64 + lane];
      const float l1 = xml[(rg * 2 + 1) * 64 + lane];
      const float mm = fmaxf(m, m1);
      const float a0 = fast_exp2(m - mm), a1 = fast_exp2(m1 - mm);
      const float lt = swap_halves_sum(l * a0 + l1 * a1);
      const float inv = 1.f / lt;
      if (row_valid) {
        uint16_t* orow = p.out + static_cast<int64_t>(t0 + i0 + pos_local) * out_stride +
                         static_cast<int64_t>(head) * D;
        // register i of tile mt is d = 32mt + 8(i/4) + 4*lhalf + i%4
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t w[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int ir = 4 * q + 2 * e;
              const float* x1 = &xo[(rg * S::O_TILES * 16 + mt * 16 + ir) * 64 + lane];
              const float v0 = (o[mt][ir] * a0 + x1[0] * a1) * inv;
              const float v1 = (o[mt][ir + 1] * a0 + x1[64] * a1) * inv;
              w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v0))) |
                     (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v1))) << 16);
            }
            *reinterpret_cast<uint2*>(orow + 32 * mt + 8 * q + 4 * lhalf) = make_uint2(w[0], w[1]);
          }
      }
    }
    __syncthreads();  // LDS is reused by the next item
  }
}

template <int D>
constexpr size_t prefill_smem() {
  return 4 * static_cast<size_t>(PrefillShape<D>::BUF);
}
// the merge area (O of four row groups over the K buffers) must fit
static_assert(4 * 4 * 16 * 64 * sizeof(float) <= 2 * PrefillShape<128>::BUF, "merge area");

template <int D>
hipError_t launch_prefill_t(const AttnParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(prefill_kernel<D>, dim3(grid), dim3(kPrefillThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

size_t prefill_lds_bytes(int head_size) {
  return head_size == 128 ? prefill_smem<128>() : prefill_smem<64>();
}

hipError_t launch_prefill(const AttnParams& p, int head_size, int grid, hipStream_t s) {
  if (head_size == 128) return launch_prefill_t<128>(p, grid, s);
  if (head_size == 64) return launch_prefill_t<64>(p, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace pa

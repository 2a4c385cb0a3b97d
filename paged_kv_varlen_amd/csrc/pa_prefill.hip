// Causal varlen (chunked) prefill attention on gfx950 matrix cores.
//
// Rows are sequences with more than one new token.  A sequence's new tokens
// are cut into half-tiles of P = 64 / G positions; a work item is (sequence,
// half-tile pair t, kv head) and the workgroup owns 128 rows: rows 0..63 are
// half-tile t, rows 64..127 half-tile nt-1-t (nt half-tiles in the sequence),
// each row a (new-token position, query head) pair of one GQA group, laid out
// position-major (row f = position f / G, head f % G), so every K/V byte
// staged in LDS serves all G query heads of the group.  Under the causal mask
// a late half-tile sees more keys than an early one, and the pair's total is
// the same for every t, so all items cost about the same.
//
// Eight waves: a wave owns 32 rows (a "row group") and the keys of one half
// ("kv group") of every 64-key step; the two kv groups keep separate
// online-softmax states and are merged once, in LDS, at the end of the item
// (fixed order: group 0 then group 1).  Waves w and w+4 share a SIMD, so they
// get row groups of different halves: when the early half-tile has run out
// of keys each SIMD still has one busy wave.
//
// K/V staging: a ring of four LDS buffers, each holding the K and V rows of
// one 64-key step.  Step j's rows are fetched during step j-3 with direct
// global->LDS loads (global_load_lds_dwordx4: lane i's 16 bytes land at
// M0 + 16 i), each wave fetching 8 rows of K and of V after its products of
// the step, so that the load path (about 64 bytes per clock per CU) streams
// while the matrix cores work on the next step.  A step ends with a wait for the loads of the next
// step only (the two later steps stay in flight) and one barrier.  Page ids
// come from a window of cache slots (one per 16 keys, from block_table) kept
// in LDS.  Keys
// past the history read a zeroed page of the workspace instead of the cache.
// K and V rows stay row-major (2*D bytes); their 16-byte chunks are
// XOR-swizzled per row so that the reads below hit distinct LDS banks.
//
// Per step and wave (32 keys x 32 rows):
//   * S^T = K Q^T with v_mfma_f32_32x32x16_{f16,bf16} (fp32 accumulate): a
//     lane holds 16 keys of one query row, so the row max needs a single
//     exchange with lane^32.  All K and V fragments of the step are read from
//     LDS before the first product, so the step waits for one LDS round trip;
//   * keys after a row's position are masked only on steps that cross the
//     diagonal (bottom-right causal offset: new row i of sequence b is at
//     past_b + i, "WS2 CP-Aware Attention Contract", Mode-Specific Metadata);
//   * online softmax in fp32 on base-2 scores (running sums rescaled only
//     when the max grows by more than 2^8), P rounded to the data type
//     (fp16 or bf16);
//   * O^T += V^T P^T with the same MFMA.  P^T comes straight from the S^T
//     registers; the V^T operand is read from the row-major V tile with the
//     LDS transpose read ds_read_b64_tr_b16 (within 16 lanes, lanes 4r..4r+3
//     supply 16 consecutive halves of "row" r and lane i receives element i
//     of rows 0..3), which yields 4 consecutive keys of one head-dim column
//     per lane, in the key order of the P^T registers.
// O is divided by the row sum and rounded to the data type once, at the final
// write.
//
// Head size 256 (PrefillShape): four waves, one per SIMD, each with a row
// group and all keys of a step (two 32-key sub-steps), and a ring of two
// steps; everything else as above.
//
// INT8 / INT4 caches: the ring holds the cached codes (one byte or half a
// byte per element, rows of D or D/2 bytes, unswizzled) and each step turns
// them into data-type rows of a stage buffer, in the swizzled layout above
// (exact: |code| <= 127), so
// the products run as for 16-bit caches.  The scores then use the codes of K,
// so each query row is multiplied by the kv head's K scales (rounded to the
// data type) once per item; O is multiplied by the V scales at the final
// write.
//
// Items are spread over up to eight queues by kv head and a workgroup serves
// first the queue of the XCD it runs on (workgroup id mod 8), so each XCD's
// L2 holds the K/V of few heads; when its queue is empty it helps the others.
#include <type_traits>
#include <utility>

#include "pa_elem.h"
#include "pa_internal.h"
#include "pa_merge.h"

namespace pa {

namespace {

typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
#define PA_LDS __attribute__((address_space(3)))
#define PA_GLOBAL __attribute__((address_space(1)))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kGroupKeys = kPrefillKeys / 2;  // keys per kv group per step
constexpr int kSlotWindow = 2048;             // 16-key cache slots held in LDS

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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

// maximum of 16 scores: the IEEE maximum (NaN-propagating, like any product
// of a NaN) compiles to gfx950's three-input v_maximum3_f32 and, unlike
// fmaxf, needs no canonicalisation of the matrix-core results first
__device__ inline float max16(const f32x16_t& v) {
  float r = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) r = __builtin_elementwise_maximum(r, v[i]);
  return r;
}
__device__ inline float swap_halves_maximum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8)
template <int N>
__device__ inline void wait_fills() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// direct global->LDS load of LB bytes per lane (lane i's bytes land at
// dst + LB * i).  The size is a literal in each branch: the host pass rejects
// a size that is only known at template instantiation.
template <int LB>
__device__ inline void fill_lds(const char* src, char* dst) {
  static_assert(LB == 16 || LB == 4, "direct load size");
  if constexpr (LB == 16)
    __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)src, (PA_LDS void*)dst, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)src, (PA_LDS void*)dst, 4, 0, 0);
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maximum): this
// wave's LDS writes are done, the fills in flight are not waited for
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// workgroup barrier without the memory fence of __syncthreads() (which would
// also wait for every fill in flight); the empty asm statements keep the
// compiler from moving memory accesses across it
__device__ inline void plain_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Head sizes up to 128: eight waves, two kv groups, a ring of four steps.
// Head size 256: the Q and O of a 32-row group take 192 registers, so a wave
// needs a SIMD of its own (four waves, up to 512 registers each); each wave
// then takes all 64 keys of a step as two 32-key sub-steps (one kv group),
// and a ring of two steps (64 KB each) fits in LDS.
template <int D, int KQ = 0>
struct PrefillShape {
  static constexpr bool QNT = KQ != 0;               // the caches hold codes (INT8 or INT4)
  static constexpr bool WIDE = D > 128;
  static constexpr int WAVES = WIDE ? 4 : 8;         // waves per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KVG = WIDE ? 1 : 2;           // kv groups (waves sharing a row group)
  static constexpr int SUBS = 2 / KVG;               // 32-key sub-steps per wave and step
  static constexpr int RING = WIDE ? 2 : 4;          // LDS buffers per tensor
  static constexpr int ROWB = D * 2;                 // bytes per key row (data type)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 64 / CPR;     // rows per 1 KB direct load
  static constexpr int WAVE_ROWS = kPrefillKeys / WAVES;  // rows of K (and V) each wave fetches
  static constexpr int BUF = kPrefillKeys * ROWB;    // bytes per K (or V) step, data type
  // cached rows as fetched: ROWC bytes each (quantized: codes), LB bytes per lane
  // and direct load (4 when a wave's rows are under 1 KB)
  static constexpr int ROWC = cache_row_bytes(D, KQ);
  static constexpr int LB = WAVE_ROWS * ROWC >= 1024 ? 16 : 4;
  static constexpr int LOADS = WAVE_ROWS * ROWC / (64 * LB);  // direct loads per wave per tensor
  static constexpr int CBUF = kPrefillKeys * ROWC;   // bytes per ring buffer
  // quantized: the converted K and V rows of the step, and the kv-group merge
  // area (one buffer of O per row group)
  static constexpr int STAGE = QNT ? (KVG == 2 ? 4 : 2) * BUF : 16;
  static constexpr int QK_STEPS = D / 16;            // MFMA k-steps over the head dim
  static constexpr int O_TILES = D / 32;             // 32-wide d tiles of O^T
  // steps per slot window: 4 slots per step, RING - 1 steps fetched ahead,
  // and a whole number of ring turns
  static constexpr int CHUNK = (kSlotWindow / 4 - (RING - 1)) / RING * RING;
  static_assert(4 * (CHUNK + RING - 1) <= kSlotWindow && CHUNK % RING == 0, "slot window");
  // chunk swizzles (in 16-byte chunks) of K and V rows; rows of 256 and 512
  // bytes both start on bank 0, so they share one
  static __device__ int k_swz(int row) { return D >= 128 ? (row & 15) : (row & 7); }
  static __device__ int v_swz(int row) { return D >= 128 ? ((row & 3) << 2) : 0; }
};

template <int D, bool BF16, int KQ>
__global__ __launch_bounds__(PrefillShape<D>::THREADS) void prefill_kernel(AttnParams p) {
  using S = PrefillShape<D, KQ>;
  constexpr bool QNT = S::QNT;
  using E = Elem<BF16>;
  typedef typename E::x8 x8;
  typedef typename E::x4 x4;
  constexpr int ROWB = S::ROWB, CPR = S::CPR;
  constexpr int kRing = S::RING;
  constexpr int kChunk = S::CHUNK;
  static_assert(S::LOADS >= 1 && S::LOADS * 64 * S::LB == S::WAVE_ROWS * S::ROWC, "loads per wave");
  // quantized, two kv groups: two stages (step parity); step j converts the
  // codes of step j + 1 while the products of step j run
  constexpr bool kAhead = QNT && S::KVG == 2;
  static_assert(!kAhead || S::STAGE >= 4 * S::BUF, "two stages");
  // 16-bit caches up to head size 128: software-pipelined steps (pstep)
  constexpr bool kPipe = !QNT && !S::WIDE;

  // one LDS object per ring buffer and tensor: the compiler can then see that
  // a fill of one buffer never aliases reads of another and does not make
  // those reads wait for the fill
  __shared__ __align__(16) char k_lds0[S::CBUF];
  __shared__ __align__(16) char k_lds1[S::CBUF];
  __shared__ __align__(16) char k_lds2[kRing > 2 ? S::CBUF : 16];
  __shared__ __align__(16) char k_lds3[kRing > 2 ? S::CBUF : 16];
  __shared__ __align__(16) char a_lds0[S::CBUF];
  __shared__ __align__(16) char a_lds1[S::CBUF];
  __shared__ __align__(16) char a_lds2[kRing > 2 ? S::CBUF : 16];
  __shared__ __align__(16) char a_lds3[kRing > 2 ? S::CBUF : 16];
  __shared__ __align__(16) char stage[S::STAGE];
  __shared__ int slot_lds[kSlotWindow];
  __shared__ int lds_item;
  auto kbuf = [&](int b) -> char* { return b == 0 ? k_lds0 : b == 1 ? k_lds1 : b == 2 ? k_lds2 : k_lds3; };
  auto vbuf = [&](int b) -> char* { return b == 0 ? a_lds0 : b == 1 ? a_lds1 : b == 2 ? a_lds2 : a_lds3; };
  // the K and V rows the products of ring buffer b's step read (data type,
  // swizzled); with two stages, a step's parity is that of its ring buffer
  auto kread = [&](int b) -> char* { return QNT ? stage + (kAhead ? (b & 1) * 2 * S::BUF : 0) : kbuf(b); };
  auto vread = [&](int b) -> char* { return QNT ? kread(b) + S::BUF : vbuf(b); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // eight waves: w and w+4 run on one SIMD, same kv group, row groups r and
  // r+2; four waves: one row group each, all keys
  const int rg = S::WIDE ? wave : (wave & 1) + 2 * (wave >> 2);  // row group (rows 32*rg .. +31)
  const int kvg = S::WIDE ? 0 : (wave >> 1) & 1;                  // kv group
  const int half = rg >> 1;                     // half-tile of the pair
  const int lrow = lane & 31;   // MFMA column owned by this lane
  const int lhalf = lane >> 5;  // which k-half of the MFMA operand
  const int G = p.group;
  const int P = p.prefill_positions;  // positions per half-tile
  const int bs = p.block_size;
  const int64_t kv_row = static_cast<int64_t>(p.kv_heads) * D;
  const int64_t out_stride = static_cast<int64_t>(p.num_heads) * D;
  const float c = fabsf(p.scale_log2);
  const bool negate_q = p.scale_log2 < 0.f;  // fold the sign into Q (exact)

  // decode segments cut by a wave boundary: one wave per segment.  The first
  // task's sequence record is read together with the control block (the
  // record array always holds batch + 1 entries).
  {
    const int U = p.decode_units;
    const int first = static_cast<int>(blockIdx.x) * S::WAVES + wave;
    const int4 sq0 = p.dec_seq[min(first / U, p.batch)];
    const int segments = p.ws_ctrl[kCtrlDecodeSeqs] * U;
    const int T = p.ws_ctrl[kCtrlDecodeTiles];
    const int nw = static_cast<int>(gridDim.x) * S::WAVES;
    for (int task = first; task < segments; task += nw)
      merge_segment_any<D, BF16>(p, task, T, lane, task == first ? sq0 : p.dec_seq[task / U]);
  }

  const int nq = prefill_queue_count(p.kv_heads);
  const int hq = p.kv_heads / nq;
  const int per_queue = p.ws_ctrl[kCtrlPrefillItems] * hq;
  if (per_queue == 0) return;  // no multi-token sequence in this call
  const int home = static_cast<int>(blockIdx.x % 8) % nq;
  // one wave of each SIMD runs ahead, so that its softmax (VALU) overlaps the
  // other wave's matrix products
  if (wave >= 4) __builtin_amdgcn_s_setprio(1);

  // per-lane LDS byte offsets (everything else is an immediate).  The
  // swizzles permute chunks within 16-chunk (256-byte) halves of a row, so
  // for head size 256 fragment kk + 8 (d tile mt + 4) sits 256 bytes after
  // fragment kk (d tile mt): one register serves both.
  constexpr int KOFF = S::QK_STEPS < 8 ? S::QK_STEPS : 8;
  constexpr int VOFF = S::O_TILES < 4 ? S::O_TILES : 4;
  int koff[KOFF];  // K fragment kk of row kvg*32 + lrow
#pragma unroll
  for (int kk = 0; kk < KOFF; ++kk) {
    const int row = kvg * kGroupKeys + lrow;
    koff[kk] = row * ROWB + (((2 * kk + lhalf) ^ S::k_swz(row)) << 4);
  }
  int voff[VOFF];  // transpose-read address of d tile mt (keys kvg*32 + ...)
  {
    const int grp = lane >> 4, i = lane & 15, r = i >> 2, q = i & 3;
    const int row = kvg * kGroupKeys + 4 * (grp >> 1) + r;
#pragma unroll
    for (int mt = 0; mt < VOFF; ++mt) {
      const int chunk = 4 * mt + 2 * (grp & 1) + (q >> 1);
      voff[mt] = row * ROWB + ((chunk ^ S::v_swz(row)) << 4) + ((q & 1) << 3);
    }
  }

  // loader: direct load i of a wave covers 64 * LB bytes of its WAVE_ROWS
  // rows; byte offsets (from the wave's first row) of this lane's piece for
  // each load (16-bit rows: a swizzled 16-byte chunk; codes: bytes in order),
  // and of the same piece in the zero page
  const int lrow0 = lane / CPR;
  const int lchunk = lane % CPR;
  auto load_row = [&](int i) -> int {  // row (within the wave's) of this lane's piece of load i
    return QNT ? (64 * S::LB * i + S::LB * lane) / S::ROWC : S::ROWS_PER_LOAD * i + lrow0;
  };
  uint32_t offk[S::LOADS], offv[S::LOADS];
#pragma unroll
  for (int i = 0; i < S::LOADS; ++i) {
    const int rl = load_row(i);
    const int trow = S::WAVE_ROWS * wave + rl;  // row within the step's 64
    if constexpr (QNT) {
      offk[i] = offv[i] = static_cast<uint32_t>(rl * p.kv_heads * S::ROWC + (64 * S::LB * i + S::LB * lane) % S::ROWC);
    } else {
      offk[i] = static_cast<uint32_t>((rl * static_cast<int>(kv_row) + (lchunk ^ S::k_swz(trow)) * 8) * 2);
      offv[i] = static_cast<uint32_t>((rl * static_cast<int>(kv_row) + (lchunk ^ S::v_swz(trow)) * 8) * 2);
    }
  }

  // The first item of every workgroup is static: workgroup b takes item
  // rank(b) of its home queue, rank(b) counting the workgroups of that home
  // below b (nq divides 8).  Later items come from the queue counters (zeroed
  // by the plan), offset by the number of static items of the queue, so a
  // call with at most one item per workgroup needs no atomic at all.
  const int gd = static_cast<int>(gridDim.x);
  auto static_items = [&](int q) {  // workgroups whose home queue is q
    const int rem = gd % 8;
    return (gd / 8) * (8 / nq) + (q < rem ? (rem - 1 - q) / nq + 1 : 0);
  };
  int queue = home, tried = 0;
  bool first_item = true;
  auto fetch = [&]() -> int {  // next item of this workgroup, or -1
    if (first_item) {
      first_item = false;
      const int j = static_cast<int>(blockIdx.x / 8) * (8 / nq) + static_cast<int>(blockIdx.x % 8) / nq;
      if (j < per_queue) return j;
    }
    while (tried < nq) {
      const int base = static_items(queue);
      if (base < per_queue) {  // (uniform) the queue has items beyond the static ones
        if (tid == 0) lds_item = atomicAdd(&p.ws_ctrl[kCtrlPrefillQueue0 + queue], 1) + base;
        // LDS traffic only: no wait for the previous item's output stores
        wait_lds();
        plain_barrier();
        // (uniform: every lane reads the same value, which the compiler
        // cannot see; from here on the item's values live in scalar registers)
        const int j = __builtin_amdgcn_readfirstlane(lds_item);
        wait_lds();
        plain_barrier();
        if (j < per_queue) return j;
      }
      queue = queue + 1 == nq ? 0 : queue + 1;
      ++tried;
    }
    return -1;
  };

  for (int j = fetch(); j >= 0; j = fetch()) {
    const int2 bt = p.items[j / hq];
    const int kvh = queue + nq * (j % hq);
    const int b = bt.x, pair = bt.y;
    const int t0 = p.cum[b];
    const int qlen = p.cum[b + 1] - t0;
    const int past = p.past[b];
    const int L = past + qlen;
    const int nt = (qlen + P - 1) / P;  // half-tiles of this sequence
    const int tb = nt - 1 - pair;       // half-tile of rows 64..127 (none if == pair)
    // keys [0, kv_end) are visible to some row of the item
    const int kv_end = past + min((tb > pair ? tb : pair) * P + P, qlen);
    const int nsteps = (kv_end + kPrefillKeys - 1) / kPrefillKeys;
    const int i0 = (half == 0 ? pair : tb) * P;  // this wave's half-tile
    const int i1 = min(i0 + P, qlen);

    // this lane's query row
    const int fh = (rg & 1) * 32 + lrow;  // row within the half-tile
    const int pos_local = fh / G;
    const int g = fh % G;
    const bool half_valid = half == 0 || tb > pair;
    const bool row_valid = half_valid && (fh < P * G) && (i0 + pos_local < i1);
    const int row_pos = past + i0 + (row_valid ? pos_local : 0);
    const int head = kvh * G + g;
    // positions spanned by this wave's valid rows (none: wave_last = -1)
    const int fh0 = (rg & 1) * 32;
    const bool wave_valid = half_valid && fh0 < P * G && i0 + fh0 / G < i1;
    const int wave_first = past + i0 + fh0 / G;
    const int wave_last = wave_valid ? past + min(i0 + min(fh0 + 31, P * G - 1) / G, i1 - 1) : -1;

    const int32_t* btab = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
    // cache slot (block_table[k / bs] * bs + k % bs) of every 16th key k <
    // min(L, nsteps * 64), for 16-key groups [gbase, gbase + kSlotWindow);
    // a wave's 8 rows of a step never cross a page (bs is a multiple of 16)
    const int ngroups = (min(L, nsteps * kPrefillKeys) + 15) / 16;
    // the first window's block-table reads, issued before the query loads so
    // that writing the window waits for them alone
    // (head size 256: the old order, its registers are needed by the ring)
    constexpr int kWinPer = S::WIDE ? 1 : kSlotWindow / S::THREADS;  // window entries per thread
    int win0[kWinPer];
    if constexpr (!S::WIDE) {
      const int n = min(kSlotWindow, ngroups);
#pragma unroll
      for (int r = 0; r < kWinPer; ++r) {
        const int i = tid + r * S::THREADS;
        win0[r] = i < n ? btab[(16 * i) / bs] * bs + (16 * i) % bs : 0;
      }
    }
    asm volatile("" ::: "memory");

    x8 qf[S::QK_STEPS];
    uint4 qraw[S::QK_STEPS];
    {
      const uint16_t* qrow = p.q + static_cast<int64_t>(t0 + i0 + (row_valid ? pos_local : 0)) * p.q_stride +
                             static_cast<int64_t>(head) * D;
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) {
        qraw[kk] = make_uint4(0u, 0u, 0u, 0u);
        if (row_valid) qraw[kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * lhalf);
      }
    }
    // the query row, finished once its loads landed (the first fills are in
    // flight by then)
    auto finish_q = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) {
        uint4 raw = qraw[kk];
        if constexpr (QNT) {  // q_d * ks_d, d = 16 kk + 8 lhalf + e, rounded to the data type
          const float4* ks = reinterpret_cast<const float4*>(p.k_scale + static_cast<int64_t>(kvh) * D + 16 * kk +
                                                             8 * lhalf);
          const float4 s0 = ks[0], s1 = ks[1];
          const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          x8 qx = __builtin_bit_cast(x8, raw);
#pragma unroll
          for (int e = 0; e < 8; ++e) qx[e] = E::round(static_cast<float>(qx[e]) * sv[e]);
          raw = __builtin_bit_cast(uint4, qx);
        }
        if (negate_q) {
          raw.x ^= 0x80008000u; raw.y ^= 0x80008000u; raw.z ^= 0x80008000u; raw.w ^= 0x80008000u;
        }
        qf[kk] = __builtin_bit_cast(x8, raw);
      }
    };
    // (head size 256: finished at once, its registers are needed by the ring)
    if constexpr (S::WIDE) finish_q();

    f32x16_t o[S::O_TILES];
#pragma unroll
    for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] = f32x16_t{};
    float m = kNegInf, l = 0.f;
    f32x16_t s_pipe = f32x16_t{};  // pipelined steps: S of the step computed next

    const char* kbytes = reinterpret_cast<const char*>(p.key_cache) + static_cast<int64_t>(kvh) * S::ROWC;
    const char* vbytes = reinterpret_cast<const char*>(p.value_cache) + static_cast<int64_t>(kvh) * S::ROWC;
    const uint32_t row_bytes = static_cast<uint32_t>(p.kv_heads * S::ROWC);  // bytes of a cache slot
    int gbase = 0;
    auto fill_window = [&](int first) {
      gbase = first;
      const int n = min(kSlotWindow, ngroups - first);
      for (int i = tid; i < n; i += S::THREADS) {
        const int key = 16 * (first + i);
        slot_lds[i] = btab[key / bs] * bs + key % bs;
      }
      __syncthreads();
    };

    // direct global->LDS fills of this wave's 8 rows of step s (ring buffer
    // BUF), loads i0 .. i1-1
    // (slot16: the window entry of the wave's rows, read ahead by slot_of)
    auto slot_of = [&](int s) -> int { return slot_lds[((s * kPrefillKeys + S::WAVE_ROWS * wave) >> 4) - gbase]; };
    auto issue = [&](auto buf_tag, int s, int slot16, int i_first, int i_last) __attribute__((always_inline)) {
      constexpr int buf = decltype(buf_tag)::value;
      const int jw = s * kPrefillKeys + S::WAVE_ROWS * wave;  // first key of the wave's rows
      if (jw + S::WAVE_ROWS <= L) {  // the usual case: all 8 rows are history
        const uint32_t slot = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(slot16) + (jw & 15));
        const uint64_t at = static_cast<uint64_t>(slot) * row_bytes;
        const char* kb = kbytes + at;
        const char* vb = vbytes + at;
        for (int i = i_first; i < i_last; ++i) {
          const int dst = S::WAVE_ROWS * wave * S::ROWC + 64 * S::LB * i;
          fill_lds<S::LB>(kb + offk[i], kbuf(buf) + dst);
          fill_lds<S::LB>(vb + offv[i], vbuf(buf) + dst);
        }
      } else {
        // rows past the history: read the zero page (rows < L read as usual)
        const int slot = jw < L ? __builtin_amdgcn_readfirstlane(slot16) + (jw & 15) : 0;
        const char* zb = reinterpret_cast<const char*>(p.zeros);
        for (int i = i_first; i < i_last; ++i) {
          const int rl = load_row(i);
          const bool hist = jw + rl < L;
          const int64_t at = static_cast<int64_t>(slot) * row_bytes;
          const uint32_t zk = offk[i] - static_cast<uint32_t>(rl) * row_bytes;  // chunk offset alone
          const uint32_t zv = offv[i] - static_cast<uint32_t>(rl) * row_bytes;
          const char* ks = hist ? kbytes + at + offk[i] : zb + zk;
          const char* vs = hist ? vbytes + at + offv[i] : zb + zv;
          const int dst = S::WAVE_ROWS * wave * S::ROWC + 64 * S::LB * i;
          fill_lds<S::LB>(ks, kbuf(buf) + dst);
          fill_lds<S::LB>(vs, vbuf(buf) + dst);
        }
      }
    };

    // one step of this wave: S (32 keys x 32 rows), softmax over the 32 keys,
    // PV (four accumulators in turn).  The K fragments of the step are all
    // read before the first product and the V fragments before the softmax,
    // so the step waits for one LDS round trip, not one per product.
    // (sub: the 32-key sub-step of a wave that takes all keys of a step; its
    // rows sit 32 rows further into the buffer, swizzled alike)
    auto compute = [&](auto buf_tag, auto sub_tag, int jk, bool masked) __attribute__((always_inline)) {
      constexpr int buf = decltype(buf_tag)::value;
      constexpr int so = decltype(sub_tag)::value * kGroupKeys * ROWB;
      // K fragments in batches of at most 8 (one batch up to head size 128)
      f32x16_t s = f32x16_t{};
      static_for<S::QK_STEPS / KOFF>([&](auto kb) __attribute__((always_inline)) {
        constexpr int k0 = decltype(kb)::value * KOFF;
        x8 kf[KOFF];
#pragma unroll
        for (int kk = 0; kk < KOFF; ++kk)
          kf[kk] = *reinterpret_cast<const x8*>(kread(buf) + so + 256 * decltype(kb)::value + koff[kk]);
        asm volatile("" ::: "memory");  // keep the reads ahead of the products
#pragma unroll
        for (int kk = 0; kk < KOFF; ++kk) s = E::mfma_32x32x16(kf[kk], qf[k0 + kk], s);
      });
      // V^T fragments, read while the products and the softmax run: the
      // transpose read of rows key0..key0+3 (key0 = 16ks + 4*lhalf, then +8)
      // gives each lane the 4 keys of its d column, in the key order of the
      // P^T registers
      // (head size 256: only the first 16 keys' fragments here, the rest
      // after the softmax, to bound the registers in flight)
      constexpr int VPRE = S::O_TILES > 4 ? 1 : 2;
      auto read_v = [&](int ks, int mt) __attribute__((always_inline)) -> x8 {
        char* vb = vread(buf) + so + voff[mt % VOFF] + 256 * (mt / VOFF) + 16 * ks * ROWB;
        const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PA_LDS fp16x4_t*)vb);
        const fp16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PA_LDS fp16x4_t*)(vb + 8 * ROWB));
        return __builtin_shufflevector(__builtin_bit_cast(x4, lo), __builtin_bit_cast(x4, hi), 0, 1, 2, 3, 4, 5, 6,
                                       7);
      };
      x8 va[VPRE][S::O_TILES];
#pragma unroll
      for (int ks = 0; ks < VPRE; ++ks)
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) va[ks][mt] = read_v(ks, mt);
      asm volatile("" ::: "memory");
      // register i holds key jk + 8(i/4) + 4*lhalf + i%4
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = jk + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          if (key > row_pos) s[i] = kNegInf;
        }
      }
      // row max as a tree (short dependency chain)
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = fmaxf(s[i], s[i + 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i) t8[i] = fmaxf(t8[i], t8[i + 4]);
      float mx = fmaxf(fmaxf(t8[0], t8[2]), fmaxf(t8[1], t8[3]));
      mx = swap_halves_max(mx) * c;
      const bool grow = mx > m + 8.f;
      if (__ballot(grow) != 0) {  // wave-uniform branch; other lanes scale by 1
        const float alpha = grow ? fast_exp2(m - mx) : 1.f;
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] *= alpha;
        m = grow ? mx : m;
      }
      // P^T operand of 16-key k-step ks = registers 8ks..8ks+7, i.e. keys
      // 16ks + 4*lhalf + 0..3 and 16ks + 8 + 4*lhalf + 0..3.  A row that has
      // seen no key yet (m = -inf) has only masked scores here.
      const float mref = m == kNegInf ? 0.f : m;
      x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ks][e] = E::round(fast_exp2(fmaf(s[8 * ks + e], c, -mref)));
      // row sum of exactly the rounded weights the MFMA multiplies (v_dot2 with 1)
      // (two partial sums: shorter dependency chains; fixed order)
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        la = E::sum2(typename E::x2{pb[0][e], pb[0][e + 1]}, la);
        lb = E::sum2(typename E::x2{pb[1][e], pb[1][e + 1]}, lb);
      }
      l += la + lb;
      // O^T[d][row] += V^T[d][key] P^T[key][row]
#pragma unroll
      for (int ks = 0; ks < VPRE; ++ks)
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt)
          o[mt] = E::mfma_32x32x16(va[ks][mt], pb[ks], o[mt]);
      if constexpr (VPRE == 1) {
        x8 vb[S::O_TILES];
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) vb[mt] = read_v(1, mt);
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] = E::mfma_32x32x16(vb[mt], pb[1], o[mt]);
      }
    };

    // Software-pipelined step (16-bit caches, head sizes up to 128).  S of
    // step j is already in registers (computed by the previous step); this
    // step reads K of step j + 1, runs the softmax of step j while those
    // reads land, computes S of step j + 1 on the matrix cores, then reads V
    // of step j and accumulates O += P V.  A wave thus keeps the products of
    // the next step queued behind the vector work of this one.  (The next
    // step's S is computed even on a wave's last step, from whatever ring
    // buffer buf + 1 holds, and then unused.)
    auto pstep = [&](auto buf_tag, int jk, bool masked, f32x16_t& s) __attribute__((always_inline)) {
      constexpr int buf = decltype(buf_tag)::value;
      constexpr int nbuf = (buf + 1) % kRing;
      x8 kf[S::QK_STEPS];
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) kf[kk] = *reinterpret_cast<const x8*>(kbuf(nbuf) + koff[kk]);
      // register i of S holds key jk + 8(i/4) + 4*lhalf + i%4
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = jk + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          if (key > row_pos) s[i] = kNegInf;
        }
      }
      const float mx = swap_halves_maximum(max16(s)) * c;
      const bool grow = mx > m + 8.f;
      if (__ballot(grow) != 0) {  // wave-uniform branch; other lanes scale by 1
        const float alpha = grow ? fast_exp2(m - mx) : 1.f;
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] *= alpha;
        m = grow ? mx : m;
      }
      const float mref = m == kNegInf ? 0.f : m;  // a row that has seen no key yet
      x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ks][e] = E::round(fast_exp2(fmaf(s[8 * ks + e], c, -mref)));
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        la = E::sum2(typename E::x2{pb[0][e], pb[0][e + 1]}, la);
        lb = E::sum2(typename E::x2{pb[1][e], pb[1][e + 1]}, lb);
      }
      l += la + lb;
      f32x16_t sn = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) sn = E::mfma_32x32x16(kf[kk], qf[kk], sn);
      x8 va[2][S::O_TILES];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) {
          char* vb = vbuf(buf) + voff[mt] + 16 * ks * ROWB;
          const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PA_LDS fp16x4_t*)vb);
          const fp16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PA_LDS fp16x4_t*)(vb + 8 * ROWB));
          va[ks][mt] = __builtin_shufflevector(__builtin_bit_cast(x4, lo), __builtin_bit_cast(x4, hi), 0, 1, 2, 3,
                                               4, 5, 6, 7);
        }
      s = sn;
      // O^T[d][row] += V^T[d][key] P^T[key][row]
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt) o[mt] = E::mfma_32x32x16(va[ks][mt], pb[ks], o[mt]);
    };

    // quantized: the codes of the step in ring buffer buf -> data-type rows of the
    // stage, in the layout the products read: cached chunk c (16 codes) of
    // row r becomes chunks 2c and 2c+1 of row r, swizzled
    // (into the stage that the products of ring buffer buf's step read)
    // (INT4: a 16-byte chunk holds 32 codes and becomes chunks 4c .. 4c+3)
    auto convert = [&](auto buf_tag) __attribute__((always_inline)) {
      constexpr int buf = decltype(buf_tag)::value;
      constexpr int NC = kPrefillKeys * S::ROWC / 16;  // 16-byte code chunks per tensor
      constexpr int CPRC = S::ROWC / 16;               // per row
      constexpr int TPC = 2 * D / S::ROWC;             // data-type chunks per code chunk
      auto one = [&](bool is_v, int cc) __attribute__((always_inline)) {
        const int r = cc / CPRC, k = cc % CPRC;
        const uint4 raw = *reinterpret_cast<const uint4*>((is_v ? vbuf(buf) : kbuf(buf)) + 16 * cc);
        x8 t[TPC];
        if constexpr (KQ == 4) {
          t[0] = E::from_nibbles8(raw.x);
          t[1] = E::from_nibbles8(raw.y);
          t[2] = E::from_nibbles8(raw.z);
          t[3] = E::from_nibbles8(raw.w);
        } else {
          t[0] = E::from_codes(raw.x, raw.y);
          t[1] = E::from_codes(raw.z, raw.w);
        }
        const int swz = is_v ? S::v_swz(r) : S::k_swz(r);
        char* row = (is_v ? vread(buf) : kread(buf)) + r * ROWB;
#pragma unroll
        for (int i = 0; i < TPC; ++i) *reinterpret_cast<x8*>(row + (((TPC * k + i) ^ swz) << 4)) = t[i];
      };
      if constexpr (NC >= S::THREADS) {
        static_assert(NC % S::THREADS == 0, "conversion split");
#pragma unroll
        for (int it = 0; it < NC / S::THREADS; ++it) {
          one(false, it * S::THREADS + tid);
          one(true, it * S::THREADS + tid);
        }
      } else {
        static_assert(2 * NC <= S::THREADS, "conversion split");
        if (tid < 2 * NC) one(tid >= NC, tid >= NC ? tid - NC : tid);  // (wave-uniform tensor)
      }
    };

    // Step j computes from ring buffer j % 4 and fetches step j + 3 into ring
    // buffer (j + 3) % 4, which held step j - 1 (finished by every wave at the
    // barrier that ended it).  Each step issues 2 * LOADS direct loads per
    // wave, so "step j + 1 landed" is "at most 4 * LOADS loads outstanding"
    // while steps j + 2 and j + 3 are both in flight.
    //
    // With a ring of two (head size 256) the fill of step j + 1 goes into
    // buffer (j + 1) % 2 at the start of step j (its last reader, step j - 1,
    // ended at the barrier) and lands before the barrier that ends step j.
    // With quantized caches a ring buffer's readers are the conversion at the start
    // of its step, which ends at a barrier of its own; the products read the
    // stage, which the barrier ending a step frees for the next conversion.
    auto step = [&](auto buf_tag, int jstep) __attribute__((always_inline)) {
      constexpr int buf = decltype(buf_tag)::value;
      constexpr int nbuf = (buf + kRing - 1) % kRing;
      const int s_next = jstep + kRing - 1;  // step fetched now
      const bool more = s_next < nsteps;
      const int slot16 = slot_of(s_next);  // (in the window; unused past the history)
      if constexpr (kRing == 2) {
        if (more) issue(std::integral_constant<int, nbuf>{}, s_next, slot16, 0, S::LOADS);
      }
      if constexpr (kAhead) {
        // the next step's codes (landed before the barrier that ended the
        // previous step) into the other stage, whose readers finished there
        if (jstep + 1 < nsteps) convert(std::integral_constant<int, (buf + 1) % kRing>{});
      } else if constexpr (QNT) {
        // the stage's last readers finished at the barrier that ended the
        // previous step; the codes of this step landed before it
        convert(buf_tag);
        wait_lds();
        plain_barrier();
      }
      if constexpr (kPipe) {
        const int jk = jstep * kPrefillKeys + kvg * kGroupKeys;  // first key of this wave's 32 keys
        if (jk <= wave_last) pstep(buf_tag, jk, jk + kGroupKeys - 1 > wave_first, s_pipe);
      } else {
        static_for<S::SUBS>([&](auto sub) __attribute__((always_inline)) {
          // first key of this wave's 32 keys
          const int jk = jstep * kPrefillKeys + (kvg + decltype(sub)::value) * kGroupKeys;
          if (jk <= wave_last) compute(buf_tag, sub, jk, jk + kGroupKeys - 1 > wave_first);
        });
      }
      if constexpr (kRing == 2) {
        wait_fills<0>();
      } else {
        // the fills of step j + 3, after the products: issued in one burst
        // they stream while the other waves compute and the next step runs
        if (more) issue(std::integral_constant<int, nbuf>{}, s_next, slot16, 0, S::LOADS);
        // a plain barrier: __syncthreads() would also wait for the fills
        // still in flight.  The waits go through the builtin so that the
        // compiler knows which fills have landed and adds no wait of its own.
        // (Converting one step ahead, or reading the next step's K in this
        // one: step j + 2 must have landed, only step j + 3 stays in flight;
        // the wait also covers the stage writes.)
        if (more) wait_fills<(kAhead || kPipe ? 2 : 4) * S::LOADS>();
        else wait_fills<0>();
      }
      plain_barrier();
    };

    if constexpr (S::WIDE) {
      fill_window(0);
    } else {  // the first window (LDS only: the query loads stay in flight)
#pragma unroll
      for (int r = 0; r < kWinPer; ++r)
        if (tid + r * S::THREADS < min(kSlotWindow, ngroups)) slot_lds[tid + r * S::THREADS] = win0[r];
      wait_lds();
      plain_barrier();
    }
    // steps 0..2 in flight before the first step (nested conditions: no path
    // that the compiler considers skips a step and fetches a later one)
    issue(std::integral_constant<int, 0>{}, 0, slot_of(0), 0, S::LOADS);
    if constexpr (kRing == 2) {
      wait_fills<0>();
    } else if (nsteps > 2) {
      issue(std::integral_constant<int, 1>{}, 1, slot_of(1), 0, S::LOADS);
      issue(std::integral_constant<int, 2 % kRing>{}, 2, slot_of(2), 0, S::LOADS);
      // step 0 landed (converting ahead, or pipelined: and step 1)
      wait_fills<(kAhead || kPipe ? 2 : 4) * S::LOADS>();
    } else {
      if (nsteps > 1) issue(std::integral_constant<int, 1>{}, 1, slot_of(1), 0, S::LOADS);
      wait_fills<0>();
    }
    if constexpr (!S::WIDE) finish_q();  // (loads issued before the fills: the wait above covers them)
    plain_barrier();
    if constexpr (kAhead) {  // step 0's rows, before its products
      convert(std::integral_constant<int, 0>{});
      wait_lds();
      plain_barrier();
    }
    if constexpr (kPipe) {  // S of step 0 (unused by a wave with no key)
      x8 kf[S::QK_STEPS];
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) kf[kk] = *reinterpret_cast<const x8*>(kbuf(0) + koff[kk]);
      s_pipe = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < S::QK_STEPS; ++kk) s_pipe = E::mfma_32x32x16(kf[kk], qf[kk], s_pipe);
    }
    // Steps in chunks of kChunk: the slot window holds the chunk's steps and
    // the three fetched ahead of it, and is refilled between chunks (the
    // fills already in flight read the previous window).  Within a chunk,
    // whole turns of the ring, then the last 0..3 steps: every turn runs all
    // four, so the compiler can see that the wait ending each step covers the
    // fills of the next turn's first step.
    for (int c0 = 0; c0 < nsteps; c0 += kChunk) {
      if (c0 > 0) fill_window(4 * c0);  // uniform; all waves are between barriers
      const int c1 = min(nsteps, c0 + kChunk);
      int j0 = c0;
      for (; j0 + kRing <= c1; j0 += kRing) {
        static_for<kRing>([&](auto r) __attribute__((always_inline)) { step(r, j0 + decltype(r)::value); });
      }
      // (nested so that no path skips a step and runs a later one)
      if (j0 < c1) {
        step(std::integral_constant<int, 0>{}, j0);
        if constexpr (kRing > 2) {
          if (j0 + 1 < c1) {
            step(std::integral_constant<int, 1>{}, j0 + 1);
            if (j0 + 2 < c1) step(std::integral_constant<int, 2 % kRing>{}, j0 + 2);
          }
        }
      }
    }

    // merge the two kv groups (group 0 first) and write.  Row group r's O of
    // kv group 1 goes to K buffer r ([O_TILES*16][64 lanes] floats), (m, l)
    // of all row groups to V buffer 0 (quantized: stage buffer r and the slot
    // window).  (One kv group: nothing to merge.)
    wait_fills<0>();  // (the last steps already waited)
    float* xo = reinterpret_cast<float*>(QNT ? stage + (S::KVG == 2 ? rg * S::BUF : 0) : kbuf(rg));
    float* xml = QNT ? reinterpret_cast<float*>(slot_lds) : reinterpret_cast<float*>(a_lds0);
    if constexpr (S::KVG == 2) {
      if (kvg == 1) {
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) xo[(mt * 16 + i) * 64 + lane] = o[mt][i];
        xml[(rg * 2 + 0) * 64 + lane] = m;
        xml[(rg * 2 + 1) * 64 + lane] = l;
      }
      wait_lds();  // LDS traffic only
      plain_barrier();
    }
    if (kvg == 0 && wave_valid) {
      float m1 = kNegInf, l1 = 0.f;
      if constexpr (S::KVG == 2) {
        m1 = xml[(rg * 2 + 0) * 64 + lane];
        l1 = xml[(rg * 2 + 1) * 64 + lane];
      }
      const float mm = fmaxf(m, m1);
      const float a0 = fast_exp2(m - mm), a1 = fast_exp2(m1 - mm);
      const float lt = swap_halves_sum(l * a0 + l1 * a1);
      const float inv = 1.f / lt;
      if (row_valid) {
        const int64_t tok = t0 + i0 + pos_local;
        // optional partial state: natural-log lse (both lane halves hold it)
        if (p.lse_out != nullptr && lhalf == 0)
          p.lse_out[tok * p.num_heads + head] = (mm + __log2f(lt)) * 0.6931471805599453f;
        float* orow_f = p.out_f32 == nullptr ? nullptr : p.out_f32 + tok * out_stride + static_cast<int64_t>(head) * D;
        uint16_t* orow = p.out + tok * out_stride + static_cast<int64_t>(head) * D;
        // register i of tile mt is d = 32mt + 8(i/4) + 4*lhalf + i%4
#pragma unroll
        for (int mt = 0; mt < S::O_TILES; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int ir = 4 * q + 2 * e;
              if constexpr (S::KVG == 2) {
                const float* x1 = &xo[(mt * 16 + ir) * 64 + lane];
                v[2 * e] = (o[mt][ir] * a0 + x1[0] * a1) * inv;
                v[2 * e + 1] = (o[mt][ir + 1] * a0 + x1[64] * a1) * inv;
              } else {
                v[2 * e] = o[mt][ir] * inv;
                v[2 * e + 1] = o[mt][ir + 1] * inv;
              }
            }
            if constexpr (QNT) {  // O used the codes of V: times the V scales of d = 32mt + 8q + 4lhalf + 0..3
              const float4 vs = *reinterpret_cast<const float4*>(p.v_scale + static_cast<int64_t>(kvh) * D + 32 * mt +
                                                                 8 * q + 4 * lhalf);
              v[0] *= vs.x;
              v[1] *= vs.y;
              v[2] *= vs.z;
              v[3] *= vs.w;
            }
            float sg[4] = {1.f, 1.f, 1.f, 1.f};  // output gate (the fp32 state stays ungated)
            if (p.gate != nullptr) {
              const uint2 gw = *reinterpret_cast<const uint2*>(p.gate + tok * out_stride + static_cast<int64_t>(head) * D +
                                                               32 * mt + 8 * q + 4 * lhalf);
              sg[0] = gate_sigmoid(E::value(gw.x & 0xffffu));
              sg[1] = gate_sigmoid(E::value(gw.x >> 16));
              sg[2] = gate_sigmoid(E::value(gw.y & 0xffffu));
              sg[3] = gate_sigmoid(E::value(gw.y >> 16));
            }
            uint32_t w[2];
#pragma unroll
            for (int e = 0; e < 2; ++e)
              w[e] = static_cast<uint32_t>(E::bits(v[2 * e] * sg[2 * e])) |
                     (static_cast<uint32_t>(E::bits(v[2 * e + 1] * sg[2 * e + 1])) << 16);
            *reinterpret_cast<uint2*>(orow + 32 * mt + 8 * q + 4 * lhalf) = make_uint2(w[0], w[1]);
            if (orow_f != nullptr)
              *reinterpret_cast<float4*>(orow_f + 32 * mt + 8 * q + 4 * lhalf) = make_float4(v[0], v[1], v[2], v[3]);
          }
      }
    }
    // LDS is reused by the next item (the output stores need not have landed)
    wait_lds();
    plain_barrier();
  }
}

template <int D, int KQ>
constexpr size_t prefill_smem() {
  using S = PrefillShape<D, KQ>;
  return 2 * S::RING * static_cast<size_t>(S::CBUF) + (S::RING > 2 ? 0 : 4 * 16) + S::STAGE +
         kSlotWindow * sizeof(int) + 16;
}
// the merge area (O of one row group) must fit one K buffer (quantized
// caches: one stage buffer), (m, l) of the four row groups one V buffer (the
// slot window)
static_assert(4 * 16 * 64 * sizeof(float) <= PrefillShape<128>::CBUF, "merge area");
static_assert(2 * 16 * 64 * sizeof(float) <= PrefillShape<64>::CBUF, "merge area");
static_assert(4 * 16 * 64 * sizeof(float) <= PrefillShape<128, 8>::BUF, "merge area");
static_assert(2 * 16 * 64 * sizeof(float) <= PrefillShape<64, 8>::BUF, "merge area");
static_assert(4 * 2 * 64 * sizeof(float) <= kSlotWindow * sizeof(int), "merge area");
static_assert(prefill_smem<128, 0>() <= 160 * 1024 && prefill_smem<256, 0>() <= 160 * 1024, "LDS budget");
static_assert(prefill_smem<128, 8>() <= 160 * 1024 && prefill_smem<256, 8>() <= 160 * 1024, "LDS budget");
static_assert(prefill_smem<128, 4>() <= 160 * 1024 && prefill_smem<256, 4>() <= 160 * 1024, "LDS budget");

template <int D, bool BF16>
hipError_t launch_prefill_q(const AttnParams& p, int kq, int grid, hipStream_t s) {
  const dim3 b(PrefillShape<D>::THREADS);
  if (kq == 8) hipLaunchKernelGGL((prefill_kernel<D, BF16, 8>), dim3(grid), b, 0, s, p);
  else if (kq == 4) hipLaunchKernelGGL((prefill_kernel<D, BF16, 4>), dim3(grid), b, 0, s, p);
  else hipLaunchKernelGGL((prefill_kernel<D, BF16, 0>), dim3(grid), b, 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_t(const AttnParams& p, bool bf16, int kq, int grid, hipStream_t s) {
  return bf16 ? launch_prefill_q<D, true>(p, kq, grid, s) : launch_prefill_q<D, false>(p, kq, grid, s);
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, int head_size, bool bf16, int kq, int grid, hipStream_t s) {
  if (head_size == 256) return launch_prefill_t<256>(p, bf16, kq, grid, s);
  if (head_size == 128) return launch_prefill_t<128>(p, bf16, kq, grid, s);
  if (head_size == 64) return launch_prefill_t<64>(p, bf16, kq, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace pa

// Decode attention: sequences with one new token, on gfx950 matrix cores.
//
// Operation (model-card README "com.microsoft.PagedAttention", Inputs and
// Outputs; "WS2 CP-Aware Attention Contract", Mode-Specific Metadata): the
// new token of sequence b sits at position L-1 = past[b] and attends to the
// L cached positions 0..L-1, read through block_table after this call's cache
// writes.  Query head h reads kv head h / G.
//
// Work split.  A unit is one kv head with up to 16 of its query heads; a
// segment is (decode sequence, unit) and has ceil(L / 16) tiles of 16 keys.
// Segments are laid end to end and wave w of W streams the tiles
// [floor(w T / W), floor((w + 1) T / W)), so every wave moves the same number
// of K/V bytes whatever the length mix.  A segment that is whole in one wave
// is written (rounded to the data type) directly.  A cut segment leaves one normalised partial
// (o, lse) per piece in the wave's two partial slots; the next launch merges
// them in wave order (pa_merge.h).
//
// Stream.  Each wave runs a ring of R LDS slots filled with direct
// global->LDS loads (global_load_lds_dwordx4: lane i's 16 bytes land at
// M0 + 16 i), up to R-1 tiles ahead of the tile it computes, across segment
// boundaries.  A slot holds the K and V tile (16 keys x D, row-major with
// XOR-swizzled 16-byte chunks) and, for the first tile of a piece, the
// query block of the unit.  The page ids of the sequence (64 block-table
// entries at a time) and the next sequence's record are also fetched with
// direct loads, one window ahead, so the issuing side never waits on a
// register load.  Every wait on these loads is an explicit vmcnt whose count
// comes from the number of loads issued since (loads complete in order), and
// every LDS read is an asm block that ends with its own lgkmcnt wait, so the
// compiler never has to guess (and over-wait) on the direct loads.
//
// Per tile (all heads of the unit at once):
//   S^T[key][head] = K Q^T      4 x v_mfma_f32_16x16x32_{f16,bf16} (D = 128)
//   online softmax in base 2, fp32, lazy rescale (only when the running max
//   grows by more than 2^8), P rounded to the data type (fp16 or bf16)
//   O^T[d][head] += V^T P^T     8 x v_mfma_f32_16x16x16_{f16,bf16}
// P^T is the S^T accumulator itself (lane = head + 16 * key group); the V^T
// operand comes from the transposing LDS read ds_read_b64_tr_b16.
//
// INT8 / INT4 caches (codes with per-(kv head, channel) scales): the slot holds
// code rows (and, with a piece's first tile, the kv head's two scale rows);
// the K fragments and V^T columns are read as code bytes and converted to the
// data type in registers (exact), the query is scaled by the K scales once per
// piece and the output by the V scales at its write.  The smaller slots let a
// workgroup run twice the waves.
#include <utility>

#include "pa_elem.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define PA_LDS __attribute__((address_space(3)))
#define PA_GLOBAL __attribute__((address_space(1)))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;  // natural log of 2 (lse in base e)

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      reinterpret_cast<const PA_LDS char*>(reinterpret_cast<uintptr_t>(p))));
}

// x combined with lane x^16 / x^32 (VALU lane swaps)
__device__ inline float swap16(float x, bool want_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}
__device__ inline float swap32(float x, bool want_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}

// Direct global->LDS load: each lane moves BYTES bytes; they land at
// lds + BYTES * lane.  `lds` must be wave-uniform.
template <int BYTES>
__device__ inline void dma(const void* src, uint32_t lds) {
  if constexpr (BYTES == 16)
    __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)src, (PA_LDS void*)(uintptr_t)lds, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((PA_GLOBAL void*)src, (PA_LDS void*)(uintptr_t)lds, 4, 0, 0);
}

// Wait until at most `younger` vector-memory operations are outstanding, i.e.
// every operation issued before the last `younger` ones has completed (they
// complete in order).  Rounded down to the nearest count below, so it may wait
// a little longer than needed, never shorter.
__device__ inline void wait_vm(int younger) {
  if (younger >= 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
  else if (younger >= 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  else if (younger >= 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (younger >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (younger >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (younger >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (younger >= 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (younger >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (younger >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if (younger >= 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// LDS reads that return only once the data is in the registers.
__device__ inline u32x4 lds_read_b128(uint32_t a) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
__device__ inline uint32_t lds_read_b32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
__device__ inline void lds_write_b128(uint32_t a, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// four 16-byte reads at a + O0..O3, one wait
template <int O0, int O1, int O2, int O3>
__device__ inline void lds_read4_b128(u32x4 (&v)[4], uint32_t a) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a), "n"(O0), "n"(O1), "n"(O2), "n"(O3)
      : "memory");
}
// N (2 or 4) 16-byte reads at a + i * STEP, one wait
template <int N, int STEP>
__device__ inline void lds_readn_b128(u32x4 (&v)[N], uint32_t a) {
  if constexpr (N == 4) {
    lds_read4_b128<0, STEP, 2 * STEP, 3 * STEP>(v, a);
  } else {
    static_assert(N == 2, "2 or 4 reads");
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1])
                 : "v"(a), "n"(STEP)
                 : "memory");
  }
}

template <typename F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The tile's MFMA operands: KS 16-byte K reads and DB transposing V reads at
// fixed per-lane addresses plus the slot's offset, issued back to back and
// waited for once.
template <int D>
struct TileRegs;
template <>
struct TileRegs<128> {
  u32x4 k[4];
  u32x2 v[8];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[4], const uint32_t (&va)[8]) {
    asm volatile(
        "ds_read_b128 %0, %12 offset:%24\n\t"
        "ds_read_b128 %1, %13 offset:%24\n\t"
        "ds_read_b128 %2, %14 offset:%24\n\t"
        "ds_read_b128 %3, %15 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]),
          "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]),
          "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]), "n"(OFF)
        : "memory");
  }
};
// head_size 256: the second 16 key-dims of every K read and the second 8 d
// blocks of every V read sit 256 bytes after the first (the swizzle only
// permutes chunks within 16-chunk halves), so the addresses of the first
// half serve both, with an offset.  Two blocks keep each asm statement small.
template <>
struct TileRegs<256> {
  u32x4 k[8];
  u32x2 v[16];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[8], const uint32_t (&va)[16]) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%12\n\t"
        "ds_read_b128 %1, %9 offset:%12\n\t"
        "ds_read_b128 %2, %10 offset:%12\n\t"
        "ds_read_b128 %3, %11 offset:%12\n\t"
        "ds_read_b128 %4, %8 offset:%13\n\t"
        "ds_read_b128 %5, %9 offset:%13\n\t"
        "ds_read_b128 %6, %10 offset:%13\n\t"
        "ds_read_b128 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
          "=&v"(k[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "n"(OFF), "n"(OFF + 256)
        : "memory");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
        "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
          "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
          "=&v"(v[14]), "=&v"(v[15])
        : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]),
          "n"(OFF), "n"(OFF + 256)
        : "memory");
  }
};
template <>
struct TileRegs<64> {
  u32x4 k[2];
  u32x2 v[4];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[2], const uint32_t (&va)[4]) {
    asm volatile(
        "ds_read_b128 %0, %6 offset:%12\n\t"
        "ds_read_b128 %1, %7 offset:%12\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "n"(OFF)
        : "memory");
  }
};

// Query operand reads (once per piece).
template <int KS, int OFF>
__device__ inline void read_q(u32x4 (&q)[KS], const uint32_t (&qa)[KS]) {
  if constexpr (KS == 8) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\tds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\tds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\tds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\tds_read_b128 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]), "=&v"(q[7])
        : "v"(qa[0]), "v"(qa[1]), "v"(qa[2]), "v"(qa[3]), "v"(qa[4]), "v"(qa[5]), "v"(qa[6]), "v"(qa[7]),
          "n"(OFF)
        : "memory");
  } else if constexpr (KS == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\tds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\tds_read_b128 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3])
        : "v"(qa[0]), "v"(qa[1]), "v"(qa[2]), "v"(qa[3]), "n"(OFF)
        : "memory");
  } else {
    asm volatile("ds_read_b128 %0, %2 offset:%4\n\tds_read_b128 %1, %3 offset:%4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(q[0]), "=&v"(q[1])
                 : "v"(qa[0]), "v"(qa[1]), "n"(OFF)
                 : "memory");
  }
}

// XOR swizzle (in 16-byte chunks) of key row k (0..15) of a tile: chosen so
// that the 16-byte K reads (16 keys, one chunk) and the transposing V reads
// (4 keys x 2 chunks per 16 lanes) touch distinct LDS banks.
template <int D>
__device__ inline int swz(int k) {
  if constexpr (D >= 128) {  // rows of 256 or 512 bytes: both start on bank 0
    return ((k & 7) << 1) | ((k >> 3) & 1);
  } else {
    const int x = (k >> 1) & 7;
    return ((x & 3) << 1) | (x >> 2);
  }
}

// INT8 caches: XOR swizzle (in 16-byte chunks) of code row r (0..15) of a
// tile, chosen so that the 8-byte K reads (16 keys, 16 lanes each) touch
// distinct LDS banks (every 256 bytes hold 256 / D rows); the transposing V
// reads take one whole chunk of each of 16 rows
template <int D>
__device__ inline int swz8(int r) {
  if constexpr (D == 64) return (r >> 2) & 3;
  else if constexpr (D == 128) return (r >> 1) & 7;
  else return ((r >> 2) & 3) | ((r & 3) << 2);
}

// INT8 caches: the tile's codes as operand bits, converted in registers.
// k[s]: the 8 codes of key n at d = 32 s + 8 g .. +7 (one ds_read_b64).
// v[R]: the V^T operands of blocks 2R and 2R+1 from one transposing read
// (ds_read_b64_tr_b8).  That read forms, in each group of 16 lanes, eight
// 16-byte rows (row e: the 8 bytes of lane 2e, then those of lane 2e+1) and
// hands lane l byte l of every row, row e as byte e of its result.  Row e of
// group g is the 16 codes of key 4 g + (e & 3) at d = 16 (2R + (e >> 2)) ..
// +15, so lane (n, g) receives keys 4 g .. 4 g + 3 of column d = 16 (2R + j)
// + n as bytes 4j .. 4j+3: the A operands of blocks 2R and 2R+1 as the
// 16x16x16 product reads them.  One address register per read (vt[R]).
template <int D>
struct CodeRegs;
template <>
struct CodeRegs<64> {
  u32x2 k[2];
  u32x2 v[2];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[2], const uint32_t (&vt)[8]) {
    asm volatile(
        "ds_read_b64 %0, %4 offset:%8\n\t"
        "ds_read_b64 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b8 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b8 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1])
        : "v"(ka[0]), "v"(ka[1]), "v"(vt[0]), "v"(vt[1]), "n"(OFF)
        : "memory");
  }
};
template <>
struct CodeRegs<128> {
  u32x2 k[4];
  u32x2 v[4];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[4], const uint32_t (&vt)[8]) {
    asm volatile(
        "ds_read_b64 %0, %8 offset:%16\n\t"
        "ds_read_b64 %1, %9 offset:%16\n\t"
        "ds_read_b64 %2, %10 offset:%16\n\t"
        "ds_read_b64 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b8 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b8 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b8 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b8 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(vt[0]), "v"(vt[1]), "v"(vt[2]), "v"(vt[3]), "n"(OFF)
        : "memory");
  }
};
template <>
struct CodeRegs<256> {
  u32x2 k[8];
  u32x2 v[8];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[8], const uint32_t (&vt)[8]) {
    asm volatile(
        "ds_read_b64 %0, %16 offset:%32\n\t"
        "ds_read_b64 %1, %17 offset:%32\n\t"
        "ds_read_b64 %2, %18 offset:%32\n\t"
        "ds_read_b64 %3, %19 offset:%32\n\t"
        "ds_read_b64 %4, %20 offset:%32\n\t"
        "ds_read_b64 %5, %21 offset:%32\n\t"
        "ds_read_b64 %6, %22 offset:%32\n\t"
        "ds_read_b64 %7, %23 offset:%32\n\t"
        "ds_read_b64_tr_b8 %8, %24 offset:%32\n\t"
        "ds_read_b64_tr_b8 %9, %25 offset:%32\n\t"
        "ds_read_b64_tr_b8 %10, %26 offset:%32\n\t"
        "ds_read_b64_tr_b8 %11, %27 offset:%32\n\t"
        "ds_read_b64_tr_b8 %12, %28 offset:%32\n\t"
        "ds_read_b64_tr_b8 %13, %29 offset:%32\n\t"
        "ds_read_b64_tr_b8 %14, %30 offset:%32\n\t"
        "ds_read_b64_tr_b8 %15, %31 offset:%32\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]),
          "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7]),
          "v"(vt[0]), "v"(vt[1]), "v"(vt[2]), "v"(vt[3]), "v"(vt[4]), "v"(vt[5]), "v"(vt[6]), "v"(vt[7]), "n"(OFF)
        : "memory");
  }
};

// INT4 caches: XOR swizzle (16-byte chunks) of code row r for head sizes 128
// and 256 (rows of 64 and 128 bytes), chosen like swz8 for the 4-byte K reads
// (the transposing V reads take 32 contiguous bytes of each of 16 rows); head
// size 64 (32-byte rows, 4-byte direct loads) is not swizzled
template <int D>
__device__ inline int swz4(int r) {
  if constexpr (D == 128) return (r >> 2) & 3;
  else if constexpr (D == 256) return (r >> 1) & 7;
  else return 0;
}

// INT4 caches: the tile's codes as operand bits, converted in registers.
// k[s]: the 8 codes of key n at d = 32 s + 8 g .. +7 (4 bytes, one
// ds_read_b32).  v[R]: the V^T operands of blocks 4R .. 4R+3 from one
// transposing read (ds_read_b64_tr_b4).  That read takes, in each group of 16
// lanes, one 8-byte row per lane (16 codes) and hands lane l code l of every
// row, row r as code r of its result.  Lane r of group g supplies row r = the
// 16 codes of key 4 g + k(r) at d = 16 (4R + (r >> 2)) .. +15, k(r) being r &
// 3 with its two bits swapped, so lane (n, g) receives in codes 4j .. 4j+3
// keys 4 g + {0, 2, 1, 3} of column d = 16 (4R + j) + n; the conversion
// (from_nibbles8_swapped) takes them in the order 0, 2, 1, 3, which gives keys
// 4 g .. 4 g + 3 in order: the A operand of block 4R + j as the 16x16x16
// product reads it.  One address register per read (vt[R]).
template <int D>
struct CodeRegs4;
template <>
struct CodeRegs4<64> {
  uint32_t k[2];
  u32x2 v[1];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[2], const uint32_t (&vt)[8]) {
    asm volatile(
        "ds_read_b32 %0, %3 offset:%6\n\t"
        "ds_read_b32 %1, %4 offset:%6\n\t"
        "ds_read_b64_tr_b4 %2, %5 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0])
        : "v"(ka[0]), "v"(ka[1]), "v"(vt[0]), "n"(OFF)
        : "memory");
  }
};
template <>
struct CodeRegs4<128> {
  uint32_t k[4];
  u32x2 v[2];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[4], const uint32_t (&vt)[8]) {
    asm volatile(
        "ds_read_b32 %0, %6 offset:%12\n\t"
        "ds_read_b32 %1, %7 offset:%12\n\t"
        "ds_read_b32 %2, %8 offset:%12\n\t"
        "ds_read_b32 %3, %9 offset:%12\n\t"
        "ds_read_b64_tr_b4 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b4 %5, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(vt[0]), "v"(vt[1]), "n"(OFF)
        : "memory");
  }
};
template <>
struct CodeRegs4<256> {
  uint32_t k[8];
  u32x2 v[4];
  template <int OFF>
  __device__ void read(const uint32_t (&ka)[8], const uint32_t (&vt)[8]) {
    asm volatile(
        "ds_read_b32 %0, %12 offset:%24\n\t"
        "ds_read_b32 %1, %13 offset:%24\n\t"
        "ds_read_b32 %2, %14 offset:%24\n\t"
        "ds_read_b32 %3, %15 offset:%24\n\t"
        "ds_read_b32 %4, %16 offset:%24\n\t"
        "ds_read_b32 %5, %17 offset:%24\n\t"
        "ds_read_b32 %6, %18 offset:%24\n\t"
        "ds_read_b32 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b4 %8, %20 offset:%24\n\t"
        "ds_read_b64_tr_b4 %9, %21 offset:%24\n\t"
        "ds_read_b64_tr_b4 %10, %22 offset:%24\n\t"
        "ds_read_b64_tr_b4 %11, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]),
          "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7]),
          "v"(vt[0]), "v"(vt[1]), "v"(vt[2]), "v"(vt[3]), "n"(OFF)
        : "memory");
  }
};

// per-tile flags handed from the issuing side to the computing side
constexpr int kFirst = 1 << 8;     // first tile of a piece
constexpr int kLast = 1 << 9;      // last tile of a piece
constexpr int kComplete = 1 << 10; // the piece is the whole segment
constexpr int kSecond = 1 << 11;   // partial goes to the wave's second slot

template <int D, int HS, bool BF16, int KQ>
__global__ __launch_bounds__(64 * decode_wg_waves(D, KQ, HS)) void decode_kernel(AttnParams p) {
  using E = Elem<BF16>;
  constexpr bool QNT = KQ != 0;                   // the caches hold codes (INT8 or INT4)
  constexpr bool Q4 = KQ == 4;
  constexpr int kDecodeWaves = decode_wg_waves(D, KQ, HS);
  constexpr int ROW = 2 * D;                      // bytes of one key of one kv head (data type)
  constexpr int CPR = ROW / 16;                   // 16-byte chunks per row
  constexpr int ROWC = cache_row_bytes(D, KQ);    // bytes of a cached row (codes when quantized)
  constexpr int QPI = 1024 / ROW;                 // query rows (data type) per 1 KB direct load
  // direct loads of LBK bytes per lane (4 when a tile is under 1 KB)
  constexpr int LBK = kDecodeTile * ROWC >= 1024 ? 16 : 4;
  constexpr int NK = kDecodeTile * ROWC / (64 * LBK);  // direct loads per tensor per tile
  constexpr int TB = kDecodeTile * ROW;           // bytes per tensor per tile (data type)
  constexpr int TBC = kDecodeTile * ROWC;         // bytes per tensor per tile as cached
  constexpr int QB = decode_q_bytes(D, HS);
  constexpr int NQ = QB / 1024;                   // direct loads of a query block
  constexpr int SB = QNT ? decode_scale_bytes(D) : 0;  // k and v scale rows of the unit
  constexpr int NSC = SB / 1024;                  // direct loads of the scale rows
  constexpr int SLOT = decode_slot_bytes(D, HS, KQ);
  constexpr int R = decode_ring(D, HS, KQ);
  constexpr int KS = D / 32;                      // QK MFMA steps
  constexpr int DB = D / 16;                      // PV MFMA blocks (16 dims each)
  static_assert(SLOT == 2 * TBC + QB + SB, "slot layout");
  static_assert(NK >= 1 && NK * 64 * LBK == TBC, "tile loads");
  static_assert(R >= 2, "ring");

  __shared__ __align__(1024) char ring[kDecodeWaves][R][SLOT];
  __shared__ __align__(16) int meta[kDecodeWaves][2][64];  // [0] next window, [1] next sequence
  // a piece's (token, first head, heads), handed over with its first tile
  __shared__ __align__(16) int piece[kDecodeWaves][R][4];
  __shared__ int prog[kDecodeWaves];  // tiles computed, per wave (two waves per SIMD)

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int W = p.decode_waves;
  const int w = static_cast<int>(blockIdx.x) * kDecodeWaves + wave;
  // two waves per SIMD: every wave's progress count starts at zero before any
  // wave can leave early (a wave without tiles stays at zero)
  constexpr bool kPaired = kDecodeWaves == 8;
  if constexpr (kPaired) {
    if (lane == 0) prog[wave] = 0;
    __syncthreads();
  }
  if (w >= W) return;

  // ---- this wave's share ---------------------------------------------------
  // Unit groups (PF = 8, 4 or 2): wave group vw streams the tiles of unit
  // groups, wave PF vw + par taking units PF u + par (consecutive kv heads,
  // read by one compute unit at nearly the same time).  Split pairs (SP = 2,
  // eight waves of 16-bit caches when the units cannot be grouped): the
  // plan's record vw starts pair vw's tiles; wave 2vw takes their lower half,
  // wave 2vw+1 the upper half (decode_wave_begin_sp).
  const int PF = p.decode_unit_group;
  const int SP = !QNT && kDecodeWaves == 8 ? p.decode_split : 1;  // (1 for every other shape)
  const int vw = w / (PF * SP), par = w % PF;
  const int* rec = p.dec_start + 8 * vw;
  const int rv = rec[lane & 7];
  const int g_pair = uniform(__builtin_amdgcn_readlane(rv, 3));
  const int g_next = p.dec_start[8 * (vw + 1) + 3];
  int g0 = g_pair, g1 = g_next;
  if (SP == 2) {
    const int mid = g_pair + (g_next - g_pair) / 2;
    if (w & 1) g0 = mid;
    else g1 = mid;
  }
  if (g0 >= g1) return;
  const int Bd = p.ws_ctrl[kCtrlDecodeSeqs];
  const int U = p.decode_units / PF;  // unit groups per sequence in the tile order
  const int hcc = decode_head_chunks(p.group);
  const int G = p.group;
  const int bs = p.block_size;
  const int tpp = bs / kDecodeTile;  // tiles per page
  const int MB = p.max_blocks;
  const int kv_row = p.kv_heads * D;                      // elements per cache slot
  const int64_t page_elems = static_cast<int64_t>(bs) * kv_row;
  const int tile_elems = kDecodeTile * kv_row;

  // ---- per-lane constant offsets ---------------------------------------------
  // tile loads: byte offset (from the tile's first cached row) of the LBK
  // bytes that land at lane * LBK of direct load j: row kj, 16-byte chunk c
  // (16-bit caches: swizzled by swz; INT8: swz8; INT4: swz4, none at D = 64)
  const int slot_bytes = p.kv_heads * ROWC;  // bytes of one cache slot
  uint32_t src_off[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int o = 64 * LBK * j + LBK * lane;
    const int kj = o / ROWC, pos = (o % ROWC) / 16;
    const int c = KQ == 8 ? pos ^ swz8<D>(kj) : KQ == 4 ? pos ^ swz4<D>(kj) : pos ^ swz<D>(kj);
    src_off[j] = static_cast<uint32_t>(kj * slot_bytes + (LBK == 16 ? 16 * c : o % ROWC));
  }
  const int qchunk = (lane % CPR) * 8;
  // MFMA operand addresses of ring slot 0 (slot s adds s * SLOT); quantized
  // caches: addresses of the code reads (CodeRegs, CodeRegs4) in ka and vb
  const int n = lane & 15, g = lane >> 4;
  const uint32_t ring0 = uniform(static_cast<int>(lds_addr(&ring[wave][0][0])));
  uint32_t ka[KS], va[QNT ? 1 : DB], vb[8], qa[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    ka[s] = Q4    ? ring0 + n * ROWC + 16 * (s ^ swz4<D>(n)) + 4 * g
            : QNT ? ring0 + n * D + 16 * ((2 * s + (g >> 1)) ^ swz8<D>(n)) + 8 * (g & 1)
                  : ring0 + n * ROW + 16 * ((4 * s + g) ^ swz<D>(n));
    qa[s] = ring0 + 2 * TBC + (n < QB / ROW ? n : 0) * ROW + 16 * (4 * s + g);
  }
  if constexpr (Q4) {
    // row of transposing read R (CodeRegs4): key 4g + j with j = n & 3, its
    // two bits swapped (the conversion takes the codes of a word in the order
    // 0, 2, 1, 3, 4, 6, 5, 7), codes of block 4R + (n >> 2), i.e. bytes 8 blk
    // .. +7 of the key's row (chunk blk / 2, swizzled, half blk & 1)
    const int key = 4 * g + (((n & 1) << 1) | ((n >> 1) & 1));
#pragma unroll
    for (int R = 0; R < 8; ++R) {
      const int blk = 4 * R + (n >> 2);
      vb[R] = R < DB / 4 ? ring0 + TBC + key * ROWC + 16 * ((blk >> 1) ^ swz4<D>(key)) + 8 * (blk & 1) : 0u;
    }
  } else if constexpr (QNT) {
    // half n & 1 of row n >> 1 of transposing read R (CodeRegs): key 4g + ((n
    // >> 1) & 3), the 16 codes of block 2R + (n >> 3) (one swizzled chunk)
    const int key = 4 * g + ((n >> 1) & 3);
#pragma unroll
    for (int R = 0; R < 8; ++R) {
      const int blk = 2 * R + (n >> 3);
      vb[R] = R < DB / 2 ? ring0 + TBC + key * ROWC + 16 * (blk ^ swz8<D>(key)) + 8 * (n & 1) : 0u;
    }
  } else {
    const int kv = 4 * g + (n >> 2), cc = n & 3;
#pragma unroll
    for (int blk = 0; blk < DB; ++blk)
      va[blk] = ring0 + TB + kv * ROW + 16 * ((2 * blk + (cc >> 1)) ^ swz<D>(kv)) + 8 * (cc & 1);
  }
  const uint32_t meta_w = lds_addr(&meta[wave][0][0]);
  const uint32_t piece0 = uniform(static_cast<int>(lds_addr(&piece[wave][0][0])));

  const uint32_t meta_s = lds_addr(&meta[wave][1][0]);

  int opc = 0;  // direct loads issued so far by this wave

  // ---- issuing side: cursor over (sequence d, unit u, tile i) ---------------
  int d_i = uniform(__builtin_amdgcn_readlane(rv, 0));
  int u_i = uniform(__builtin_amdgcn_readlane(rv, 1));
  int i_i = uniform(__builtin_amdgcn_readlane(rv, 2));
  int b_i = uniform(__builtin_amdgcn_readlane(rv, 4));
  int t_i = uniform(__builtin_amdgcn_readlane(rv, 5));
  int L_i = uniform(__builtin_amdgcn_readlane(rv, 6));
  int P_i = uniform(__builtin_amdgcn_readlane(rv, 7));
  int n_i = (L_i + kDecodeTile - 1) / kDecodeTile;
  if (SP == 2) {
    if (w & 1) {  // the upper half starts at g0: from the pair's sequence, forward to the one holding g0
      while (g0 >= P_i + U * n_i) {  // (the last sequence ends at T > g0)
        ++d_i;
        const int4 sq = p.dec_seq[d_i];
        b_i = uniform(sq.x);
        t_i = uniform(sq.y);
        L_i = uniform(sq.z);
        P_i = uniform(sq.w);
        n_i = (L_i + kDecodeTile - 1) / kDecodeTile;
      }
      u_i = (g0 - P_i) / n_i;
      i_i = (g0 - P_i) % n_i;
    }
  }
  int kvh_i = (PF * u_i + par) / hcc, hc_i = (PF * u_i + par) % hcc;  // of the actual unit
  int pi = i_i / tpp, ip = i_i % tpp;  // page of the tile and tile within the page
  int g_i = g0;
  // per-segment values
  int h0_i = 0, nh_i = 0, segfl = 0, seg0_i = 0;
  const char* kp = nullptr;  // K and V of the next tile to issue (this kv head)
  const char* vp = nullptr;

  // next sequence record (direct load into meta_s)
  int ns_opc = 0, ns_b = 0, ns_t = 0, ns_L = 0, ns_P = 0;
  bool ns_have = false;
  auto issue_nseq = [&](int d) __attribute__((always_inline)) {
    const int* src = reinterpret_cast<const int*>(p.dec_seq + min(d, Bd)) + (lane & 3);
    dma<4>(src, meta_s);
    ns_opc = ++opc;
    ns_have = false;
  };
  auto ensure_nseq = [&]() __attribute__((always_inline)) {
    if (!ns_have) {
      wait_vm(opc - ns_opc);
      const u32x4 v = lds_read_b128(meta_s);
      ns_b = uniform(static_cast<int>(v.x));
      ns_t = uniform(static_cast<int>(v.y));
      ns_L = uniform(static_cast<int>(v.z));
      ns_P = uniform(static_cast<int>(v.w));
      ns_have = true;
    }
  };

  // block-table window: lane j holds the page id of page wp0 + j of sequence wd
  int wcur = 0, wd = -1, wp0 = 0;
  bool nw_valid = false;
  int nw_opc = 0, nw_d = 0, nw_p0 = 0;
  auto issue_window = [&](int d, int b, int p0) __attribute__((always_inline)) {
    const int idx = min(p0 + lane, MB - 1);
    dma<4>(p.block_table + static_cast<int64_t>(b) * MB + idx, meta_w);
    nw_opc = ++opc;
    nw_d = d;
    nw_p0 = p0;
    nw_valid = true;
  };
  // prefetch the next window the cursor will need after the current one
  auto plan_window = [&]() __attribute__((always_inline)) {
    if (nw_valid) return;
    const int np = (L_i + bs - 1) / bs;
    if (wd == d_i && wp0 + kDecodeWindow < np) {
      issue_window(d_i, b_i, wp0 + kDecodeWindow);
    } else if (u_i + 1 < U) {
      if (wd != d_i || wp0 != 0) issue_window(d_i, b_i, 0);
    } else if (d_i + 1 < Bd) {
      ensure_nseq();
      issue_window(d_i + 1, ns_b, 0);
    }
  };
  // make the window hold page pi of the cursor's sequence
  auto need_window = [&]() __attribute__((always_inline)) {
    if (!(wd == d_i && pi >= wp0 && pi < wp0 + kDecodeWindow)) {
      if (!(nw_valid && nw_d == d_i && nw_p0 == pi)) issue_window(d_i, b_i, pi);
      wait_vm(opc - nw_opc);
      wcur = static_cast<int>(lds_read_b32(meta_w + 4 * lane));
      wd = d_i;
      wp0 = nw_p0;
      nw_valid = false;
    }
    plan_window();
  };
  auto set_pointers = [&]() __attribute__((always_inline)) {
    const int page = uniform(__builtin_amdgcn_readlane(wcur, pi - wp0));
    const int64_t base = (static_cast<int64_t>(page) * page_elems + ip * tile_elems + kvh_i * D) / D * ROWC;
    kp = reinterpret_cast<const char*>(p.key_cache) + base;
    vp = reinterpret_cast<const char*>(p.value_cache) + base;
  };
  auto enter_segment = [&]() __attribute__((always_inline)) {
    h0_i = kvh_i * G + kDecodeUnitHeads * hc_i;
    nh_i = min(kDecodeUnitHeads, G - kDecodeUnitHeads * hc_i);
    seg0_i = P_i + u_i * n_i;
    segfl = (seg0_i >= g0 && seg0_i + n_i <= g1 ? kComplete : 0) | (seg0_i > g0 ? kSecond : 0);
    need_window();
    set_pointers();
  };

  issue_nseq(d_i + 1);
  issue_window(d_i, b_i, pi);
  enter_segment();

  // per-slot hand-over (static indices only: these stay in scalar registers);
  // a piece's (token, first head, heads) goes through LDS with its first tile
  int m_opc[R], m_fl[R];

  auto issue = [&](auto slot_c) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_c)::value;
    const uint32_t sb = ring0 + S * SLOT;
#pragma unroll
    for (int j = 0; j < NK; ++j) dma<LBK>(kp + src_off[j], sb + 64 * LBK * j);
#pragma unroll
    for (int j = 0; j < NK; ++j) dma<LBK>(vp + src_off[j], sb + TBC + 64 * LBK * j);
    opc += 2 * NK;
    const bool first = g_i == g0 || i_i == 0;
    if (first) {  // the unit's query heads (absent heads read zeros)
      const uint16_t* qtok = p.q + static_cast<int64_t>(t_i) * p.q_stride + static_cast<int64_t>(h0_i) * D;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int hh = j * QPI + lane / CPR;
        dma<16>(hh < nh_i ? qtok + hh * D + qchunk : p.zeros + qchunk, sb + 2 * TBC + 1024 * j);
      }
      opc += NQ;
      if constexpr (QNT) {  // the kv head's scale rows: [k_scale (4D bytes) | v_scale (4D bytes) | zeros]
#pragma unroll
        for (int j = 0; j < NSC; ++j) {
          const int o = 1024 * j + 16 * lane;
          const void* src = o < 4 * D ? static_cast<const void*>(p.k_scale + kvh_i * D + o / 4)
                            : o < 8 * D ? static_cast<const void*>(p.v_scale + kvh_i * D + (o - 4 * D) / 4)
                                        : static_cast<const void*>(p.zeros);
          dma<16>(src, sb + 2 * TBC + QB + 1024 * j);
        }
        opc += NSC;
      }
      lds_write_b128(piece0 + 16 * S, u32x4{static_cast<uint32_t>(t_i), static_cast<uint32_t>(h0_i),
                                          static_cast<uint32_t>(nh_i), 0u});
    }
    const bool last = i_i == n_i - 1 || g_i == g1 - 1;
    m_opc[S] = opc;
    m_fl[S] = min(kDecodeTile, L_i - kDecodeTile * i_i) | (first ? kFirst : 0) | (last ? kLast : 0) | segfl;
    // advance the cursor
    ++g_i;
    if (++i_i == n_i) {
      if (g_i < g1) {  // next segment
        i_i = 0;
        pi = 0;
        ip = 0;
        ++u_i;
        if (u_i == U) {
          u_i = 0;
          ++d_i;
          ensure_nseq();
          b_i = ns_b;
          t_i = ns_t;
          L_i = ns_L;
          P_i = ns_P;
          n_i = (L_i + kDecodeTile - 1) / kDecodeTile;
          issue_nseq(d_i + 1);
        }
        kvh_i = (PF * u_i + par) / hcc;
        hc_i = (PF * u_i + par) % hcc;
        enter_segment();
      }
    } else if (++ip == tpp) {  // next page
      ip = 0;
      ++pi;
      if (pi == wp0 + kDecodeWindow) need_window();
      set_pointers();
    } else {
      kp += tile_elems / D * ROWC;
      vp += tile_elems / D * ROWC;
    }
  };

  // ---- computing side ---------------------------------------------------------
  f32x4_t acc[DB];
#pragma unroll
  for (int blk = 0; blk < DB; ++blk) acc[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // quantized caches: the v scale of each output value of this lane (d = 16 blk +
  // 4 g + e), read with the piece's first tile
  f32x4_t vsc[QNT ? DB : 1];
#pragma unroll
  for (int blk = 0; blk < (QNT ? DB : 1); ++blk) vsc[blk] = f32x4_t{1.f, 1.f, 1.f, 1.f};
  float m = kNegInf, l = 0.f;
  u32x4 qv[KS];
  int nh_c = 0, h0_c = 0, t_c = 0;

  auto compute = [&](auto slot_c) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_c)::value;
    wait_vm(opc - m_opc[S]);  // this tile's loads (and everything before) landed
    const int fl = m_fl[S];
    const int nvalid = fl & 0xff;
    if (fl & kFirst) {  // first tile of a piece: query operand, fresh running state
      const u32x4 pc = lds_read_b128(piece0 + 16 * S);
      t_c = uniform(static_cast<int>(pc.x));
      h0_c = uniform(static_cast<int>(pc.y));
      nh_c = uniform(static_cast<int>(pc.z));
      read_q<KS, S * SLOT>(qv, qa);
      if (n >= nh_c) {
#pragma unroll
        for (int s = 0; s < KS; ++s) qv[s] = u32x4{0u, 0u, 0u, 0u};
      }
      if constexpr (QNT) {
        // scores use the codes of K, so its per-channel scale goes into Q:
        // q_d s_d, rounded to the data type (values d = 32 s + 8 g + e)
        const uint32_t sc0 = ring0 + S * SLOT + 2 * TBC + QB;
        u32x4 ks[2 * KS];
        static_for<KS / 2>([&](auto i) __attribute__((always_inline)) {
          constexpr int b = 256 * decltype(i)::value;  // fragments 2i, 2i+1 (128 bytes each)
          u32x4 t[4];
          lds_read4_b128<b, b + 16, b + 128, b + 144>(t, sc0 + 32 * g);
#pragma unroll
          for (int k = 0; k < 4; ++k) ks[4 * decltype(i)::value + k] = t[k];
        });
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          typename E::x8 qx = __builtin_bit_cast(typename E::x8, qv[s]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            qx[e] = E::round(static_cast<float>(qx[e]) * __uint_as_float(ks[2 * s + (e >> 2)][e & 3]));
          qv[s] = __builtin_bit_cast(u32x4, qx);
        }
        static_for<DB / 4>([&](auto i) __attribute__((always_inline)) {
          constexpr int b = 256 * decltype(i)::value;  // blocks 4i .. 4i+3 (64 bytes apart)
          u32x4 t[4];
          lds_read4_b128<b, b + 64, b + 128, b + 192>(t, sc0 + 4 * D + 16 * g);
#pragma unroll
          for (int k = 0; k < 4; ++k) vsc[4 * decltype(i)::value + k] = __builtin_bit_cast(f32x4_t, t[k]);
        });
        if constexpr (Q4) {  // the d order of the INT4 K fragments: 0, 2, 1, 3, 4, 6, 5, 7
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const u32x4 q = qv[s];
            qv[s] = u32x4{__builtin_amdgcn_perm(q.y, q.x, 0x05040100u), __builtin_amdgcn_perm(q.y, q.x, 0x07060302u),
                          __builtin_amdgcn_perm(q.w, q.z, 0x05040100u), __builtin_amdgcn_perm(q.w, q.z, 0x07060302u)};
          }
        }
      }
      // acc is rescaled by exp2(-inf) = 0 below, as every lane's max grows
      m = kNegInf;
      l = 0.f;
    }
    // the tile's operands: K fragments (KS) and V^T fragments (DB)
    typename E::x8 kx[KS];
    typename E::x4 vx[DB];
    if constexpr (Q4) {  // INT4 codes -> data type in registers (exact)
      CodeRegs4<D> cr;
      cr.template read<S * SLOT>(ka, vb);
      // K fragments with their d in the order 0, 2, 1, 3, 4, 6, 5, 7 of each 8
      // (the query operand is permuted alike once per piece)
#pragma unroll
      for (int s = 0; s < KS; ++s) kx[s] = E::from_nibbles8_swapped(cr.k[s]);
      // codes 8h .. 8h+7 of read R: blocks 4R + 2h and 4R + 2h + 1, keys 4g .. 4g+3 each
#pragma unroll
      for (int R = 0; R < DB / 4; ++R)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const typename E::x8 t = E::from_nibbles8_swapped(h == 0 ? cr.v[R].x : cr.v[R].y);
          vx[4 * R + 2 * h] = typename E::x4{t[0], t[1], t[2], t[3]};
          vx[4 * R + 2 * h + 1] = typename E::x4{t[4], t[5], t[6], t[7]};
        }
    } else if constexpr (QNT) {  // INT8 codes -> data type in registers (exact)
      CodeRegs<D> cr;
      cr.template read<S * SLOT>(ka, vb);
#pragma unroll
      for (int s = 0; s < KS; ++s) kx[s] = E::from_codes(cr.k[s].x, cr.k[s].y);
      // bytes 0..3 of read R: block 2R, keys 4g .. 4g+3; bytes 4..7: block 2R+1
#pragma unroll
      for (int R = 0; R < DB / 2; ++R) {
        const typename E::x8 t = E::from_codes(cr.v[R].x, cr.v[R].y);
        vx[2 * R] = typename E::x4{t[0], t[1], t[2], t[3]};
        vx[2 * R + 1] = typename E::x4{t[4], t[5], t[6], t[7]};
      }
    } else {
      TileRegs<D> tr;
      tr.template read<S * SLOT>(ka, va);
#pragma unroll
      for (int s = 0; s < KS; ++s) kx[s] = __builtin_bit_cast(typename E::x8, tr.k[s]);
#pragma unroll
      for (int blk = 0; blk < DB; ++blk) vx[blk] = __builtin_bit_cast(typename E::x4, tr.v[blk]);
    }
    // S^T: lane = head n + 16 * key group g, element e = key 4 g + e
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) st = E::mfma_16x16x32(kx[s], __builtin_bit_cast(typename E::x8, qv[s]), st);
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = st[e] * p.scale_log2;
    if (nvalid < kDecodeTile) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * g + e >= nvalid) sc[e] = kNegInf;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = swap32(swap16(mx, true), true);  // over the 16 keys of head n
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? fast_exp2(m - mx) : 1.f;
      l *= alpha;
#pragma unroll
      for (int blk = 0; blk < DB; ++blk) acc[blk] *= alpha;
      m = grow ? mx : m;
    }
    typename E::x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) pb[e] = E::round(fast_exp2(sc[e] - m));
    // row sum of exactly the rounded weights the MFMA multiplies
    l = E::sum2(typename E::x2{pb[0], pb[1]}, l);
    l = E::sum2(typename E::x2{pb[2], pb[3]}, l);
    if (!QNT && nvalid < kDecodeTile) {
      // keys past the history may hold any bits (NaN included): zero their
      // values (codes are always finite, and their weights are 0)
      const int k0 = 4 * g;
      const uint32_t lo = (k0 < nvalid ? 0xffffu : 0u) | (k0 + 1 < nvalid ? 0xffff0000u : 0u);
      const uint32_t hi = (k0 + 2 < nvalid ? 0xffffu : 0u) | (k0 + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int blk = 0; blk < DB; ++blk) {
        u32x2 w = __builtin_bit_cast(u32x2, vx[blk]);
        w.x &= lo;
        w.y &= hi;
        vx[blk] = __builtin_bit_cast(typename E::x4, w);
      }
    }
#pragma unroll
    for (int blk = 0; blk < DB; ++blk) acc[blk] = E::mfma_16x16x16(vx[blk], pb, acc[blk]);
    if (fl & kLast) {  // last tile of the piece: normalise and write
      const float lt = swap32(swap16(l, false), false);
      const float inv = 1.f / lt;
      if (fl & kComplete) {  // whole segment here: the final output
        if (n < nh_c) {
          const int64_t row = static_cast<int64_t>(t_c) * p.num_heads + h0_c + n;
          uint16_t* o = p.out + row * D + 4 * g;
          const uint16_t* gt = p.gate == nullptr ? nullptr : p.gate + row * D + 4 * g;  // output gate
#pragma unroll
          for (int blk = 0; blk < DB; ++blk) {
            f32x4_t sg = {1.f, 1.f, 1.f, 1.f};
            if (gt != nullptr) {
              const uint2 gw = *reinterpret_cast<const uint2*>(gt + 16 * blk);
              sg = f32x4_t{gate_sigmoid(E::value(gw.x & 0xffffu)), gate_sigmoid(E::value(gw.x >> 16)),
                           gate_sigmoid(E::value(gw.y & 0xffffu)), gate_sigmoid(E::value(gw.y >> 16))};
            }
            typename E::x4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = E::round(acc[blk][e] * inv * vsc[QNT ? blk : 0][e] * sg[e]);
            *reinterpret_cast<typename E::x4*>(o + 16 * blk) = hv;
          }
          // optional partial state: fp32 output and natural-log lse
          if (p.out_f32 != nullptr) {
#pragma unroll
            for (int blk = 0; blk < DB; ++blk)
              *reinterpret_cast<f32x4_t*>(p.out_f32 + row * D + 4 * g + 16 * blk) = acc[blk] * inv * vsc[QNT ? blk : 0];
          }
          if (p.lse_out != nullptr && g == 0) p.lse_out[row] = (m + __log2f(lt)) * kLn2;
        }
      } else if (n < nh_c) {  // a piece: partial (o, lse) in the wave's slot
        const int ps = 2 * w + ((fl & kSecond) ? 1 : 0);
        float* po = p.part_o + (static_cast<int64_t>(ps) * kDecodeUnitHeads + n) * D + 4 * g;
#pragma unroll
        for (int blk = 0; blk < DB; ++blk) *reinterpret_cast<f32x4_t*>(po + 16 * blk) = acc[blk] * inv * vsc[QNT ? blk : 0];
        if (g == 0) p.part_lse[ps * kDecodeUnitHeads + n] = m + __log2f(lt);
      }
    }
  };

  // ---- the stream: tile k lives in slot k % R, issued R-1 tiles ahead --------
  const int count = g1 - g0;
  // Two waves per SIMD (quantized caches, D <= 128): the SIMD issues for the
  // older wave first when both are ready, so with equal shares the younger
  // one (waves 4..7 beside waves 0..3) would end several microseconds later,
  // alone on its SIMD.  After every tile the wave that is behind its sibling
  // takes the higher issue priority, so the two progress together.
  const uint32_t prog_a = lds_addr(&prog[0]);
  int done = 0;
  static_for<R - 1>([&](auto S) __attribute__((always_inline)) {
    if (g_i < g1) issue(S);
  });
  for (int k = 0; k < count; k += R) {
    static_for<R>([&](auto S) __attribute__((always_inline)) {
      constexpr int s = decltype(S)::value;
      if (k + s < count) {
        if (g_i < g1) issue(std::integral_constant<int, (s + R - 1) % R>{});
        compute(S);
        if constexpr (kPaired) {
          ++done;
          asm volatile("ds_write_b32 %0, %1" ::"v"(prog_a + 4 * wave), "v"(done) : "memory");
          const int sib = uniform(static_cast<int>(lds_read_b32(prog_a + 4 * (wave ^ 4))));
          if (done > sib) __builtin_amdgcn_s_setprio(0);
          else if (done < sib) __builtin_amdgcn_s_setprio(1);
        }
      }
    });
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

}

}  // namespace

template <int D, int HS, bool BF16>
void launch_decode_t(const AttnParams& p, int kq, dim3 g, hipStream_t s) {
  const dim3 b(64 * decode_wg_waves(D, kq, HS));
  if (kq == 8) hipLaunchKernelGGL((decode_kernel<D, HS, BF16, 8>), g, b, 0, s, p);
  else if (kq == 4) hipLaunchKernelGGL((decode_kernel<D, HS, BF16, 4>), g, b, 0, s, p);
  else hipLaunchKernelGGL((decode_kernel<D, HS, BF16, 0>), g, b, 0, s, p);
}

hipError_t launch_decode(const AttnParams& p, int head_size, int head_slots, bool bf16, int kq, int grid,
                         hipStream_t s) {
  const dim3 g(grid);
#define PA_DECODE(DD, HH)                                                                        \
  if (head_size == DD && head_slots == HH) {                                                     \
    if (bf16) launch_decode_t<DD, HH, true>(p, kq, g, s);                                        \
    else launch_decode_t<DD, HH, false>(p, kq, g, s);                                            \
    return hipGetLastError();                                                                    \
  }
  PA_DECODE(128, 4)
  PA_DECODE(128, 8)
  PA_DECODE(128, 16)
  PA_DECODE(64, 4)
  PA_DECODE(64, 8)
  PA_DECODE(64, 16)
  PA_DECODE(256, 4)
  PA_DECODE(256, 8)
  PA_DECODE(256, 16)
#undef PA_DECODE
  return hipErrorInvalidValue;
}

}  // namespace pa

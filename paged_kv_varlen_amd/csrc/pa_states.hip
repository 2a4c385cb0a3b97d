// Fixed-order merge of partial attention states (pa_merge_states).
//
// "WS2 CP-Aware Attention Contract", Reduction Semantics: a partial state is
// (out, attention-domain lse); states merge by the online-softmax rule, in
// fp32, in a fixed order, with one rounding (to fp16 or bf16) at the final
// write.  Row r of the
// result folds states 0, 1, .. P-1 in that order:
//   lse' = m + log(e^(lse - m) + e^(lse_p - m)), m = max(lse, lse_p),
//   out  = (e^(lse - m) out + e^(lse_p - m) out_p) / (e^(lse - m) + e^(lse_p - m)).
// States with lse = -inf hold no keys and are skipped; a row with no keys at
// all gets out = 0, lse = -inf.
//
// Memory-bound: a lane owns 4 consecutive head-dim values of one row and
// reads them (16-byte loads) from every state; consecutive lanes cover a row,
// then the next row, so each state is streamed once, coalesced.
#include "pa_elem.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kMergeThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kMergeThreads) void merge_states_kernel(MergeStatesParams p) {
  const int qpr = p.head_size / 4;  // lanes per row
  const int64_t lanes = p.rows * qpr;
  const float kNegInf = -__builtin_huge_valf();
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kMergeThreads + threadIdx.x; t < lanes;
       t += static_cast<int64_t>(gridDim.x) * kMergeThreads) {
    const int64_t row = t / qpr;
    const int q = static_cast<int>(t % qpr);
    float lse = kNegInf;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < p.states; ++s) {
      const int64_t idx = static_cast<int64_t>(s) * p.rows + row;
      const float ls = p.state_lse[idx];
      if (ls == kNegInf) continue;  // no keys in this state
      const float4 os = reinterpret_cast<const float4*>(p.state_out + idx * p.head_size)[q];
      if (lse == kNegInf) {
        lse = ls;
        o = os;
        continue;
      }
      const float m = fmaxf(lse, ls);
      const float a = expf(lse - m), b = expf(ls - m);
      const float inv = 1.f / (a + b);
      o.x = (a * o.x + b * os.x) * inv;
      o.y = (a * o.y + b * os.y) * inv;
      o.z = (a * o.z + b * os.z) * inv;
      o.w = (a * o.w + b * os.w) * inv;
      lse = m + logf(a + b);
    }
    if (p.out_f32 != nullptr) reinterpret_cast<float4*>(p.out_f32 + row * p.head_size)[q] = o;
    if (p.out != nullptr) {
      using E = Elem<BF16>;
      const typename E::x4 h = {E::round(o.x), E::round(o.y), E::round(o.z), E::round(o.w)};
      reinterpret_cast<typename E::x4*>(p.out + row * p.head_size)[q] = h;
    }
    if (p.lse != nullptr && q == 0) p.lse[row] = lse;
  }
}

}  // namespace

hipError_t launch_merge_states(const MergeStatesParams& p, hipStream_t s) {
  const int64_t lanes = p.rows * (p.head_size / 4);
  const int64_t blocks = (lanes + kMergeThreads - 1) / kMergeThreads;
  const int grid = static_cast<int>(blocks < 65536 ? blocks : 65536);
  if (p.bf16)
    hipLaunchKernelGGL(merge_states_kernel<true>, dim3(grid), dim3(kMergeThreads), 0, s, p);
  else
    hipLaunchKernelGGL(merge_states_kernel<false>, dim3(grid), dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa

// Fixed-order merge of decode segments that wave boundaries cut in pieces.
//
// "WS2 ReductionSpec" (CP-aware attention contract page): partial results
// (o_i normalised, lse_i in base 2) of one query row are combined as
// sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), M = max_i lse_i, in fp32 and
// in a fixed order (here: the order of the decode waves), with one rounding
// to the data type (fp16 or bf16) at the end.
//
// The decode kernel leaves the pieces of segment S..S+n-1 (tiles of one
// sequence and unit) in the partial slots of waves wf..wl: the first piece in
// wf's second slot when the segment starts inside wf's range, every other in
// the wave's first slot; waves whose range is empty hold none.  It runs as a
// prologue of the prefill kernel, the next launch on the stream, so every
// partial is visible without any cross-workgroup synchronisation.
#pragma once

#include "pa_elem.h"
#include "pa_internal.h"

namespace pa {

// One segment (decode sequence d = task / U, unit u = task % U) per call, all
// 64 lanes: lane = query head slot (lane % HSL) + HSL * part, with HSL the
// head slots of the group (4, 8 or 16), so that a group of four heads still
// uses every lane.  Part q of the 64 / HSL parts of a head row holds the
// head-dim elements 4 (q + (64 / HSL) i) .. +3, so each load of a piece's row
// is contiguous across the row's lanes.  sq is the sequence's record (b,
// token, L, first tile).
template <int D, bool BF16, int HSL>
__device__ inline void merge_segment(const AttnParams& p, int task, int T, int lane, int4 sq) {
  // Everything but the lane's head and part is the same on all lanes: the
  // record goes to scalar registers, so every branch below is uniform and the
  // index arithmetic scalar (32-bit: the partial area holds < 2^31 floats).
  const int L = __builtin_amdgcn_readfirstlane(sq.z);
  const int tile0 = __builtin_amdgcn_readfirstlane(sq.w);
  const int token = __builtin_amdgcn_readfirstlane(sq.y);
  const int U = p.decode_units;
  const int u = task % U;
  const int n = (L + kDecodeTile - 1) / kDecodeTile;
  // unit groups: the tile order and the wave ranges are over unit groups and
  // wave groups; unit u's pieces are in the waves of its place in the group
  const int PF = p.decode_unit_group, par = u % PF;
  const int W = p.decode_waves / PF;
  const int SP = p.decode_split;  // 2: waves halve the plan's pair ranges
  const int S = tile0 + (u / PF) * n;
  const int wf = decode_wave_of_sp(S, T, W, SP), wl = decode_wave_of_sp(S + n - 1, T, W, SP);
  if (wf == wl) return;  // written whole by its wave
  const int first_k = decode_wave_begin_sp(wf, T, W, SP) < S ? 1 : 0;
  const int hcc = decode_head_chunks(p.group);
  const int kvh = u / hcc, hc = u % hcc;
  const int nh = min(kDecodeUnitHeads, p.group - kDecodeUnitHeads * hc);
  constexpr int PARTS = 64 / HSL;  // lanes per head row
  constexpr int E4 = D / (4 * PARTS);  // float4 pieces of a row per lane
  const int hn = lane % HSL, qd = lane / HSL;
  // (with at least as many tiles as waves every range is non-empty)
  const bool every_wave_holds = T >= W;
  // partial slot of wave v's piece: the first piece in wf's second slot when
  // the segment starts inside wf's range, every other in the wave's first
  auto slot_of_piece = [&](int v) { return 2 * (PF * v + par) + (v == wf ? first_k : 0); };
  // Lanes of absent heads (hn >= nh) run along and store nothing.
  const float* lse_base = p.part_lse + hn;
  const float* o_base = p.part_o + hn * D + 4 * qd;
  // Pieces are combined in wave order with weights 2^(lse - M), M the
  // largest lse: a pass for M, then one for the weighted sum.  Each pass
  // loads a batch of pieces before it uses any (a batch is one memory round
  // trip, not one per piece), and the first batch of the sum's loads is issued
  // with the first lse batch, so a segment of up to PB pieces costs one round
  // trip; the sums still run in wave order.  Pieces are taken in windows of
  // 64 waves (more than one only when there are fewer tiles than waves), the
  // running sum rescaled to each window's larger maximum.
  constexpr int kLseBatch = 16;
  constexpr int PB = 32 / E4 > 16 ? 16 : 32 / E4;  // pieces per batch (<= 128 floats)
  float M = -__builtin_huge_valf(), wsum = 0.f;
  float4 o[E4];
#pragma unroll
  for (int e = 0; e < E4; ++e) o[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int w0 = wf; w0 <= wl; w0 += 64) {
    const int wend = min(wl, w0 + 63);
    // lane j: whether wave w0 + j holds a piece (a range of at least one tile)
    uint64_t mask = ~0ull;
    if (!every_wave_holds) {
      const int v = w0 + lane;
      mask = __ballot(v <= wend && (v == wf || decode_wave_begin_sp(v, T, W, SP) < decode_wave_begin_sp(v + 1, T, W, SP)));
    }
    auto have = [&](int v) { return v <= wend && ((mask >> ((v - w0) & 63)) & 1ull) != 0; };
    float lv[PB];
    float4 x[PB][E4];
    auto load_batch = [&](int v0) {
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int v = v0 + j;
        const bool ok = have(v);
        const int ps = slot_of_piece(min(v, wend));  // (loads at a valid piece, then a select)
        const float l = lse_base[ps * kDecodeUnitHeads];
        lv[j] = ok ? l : -__builtin_huge_valf();
        const float4* po = reinterpret_cast<const float4*>(o_base + ps * (kDecodeUnitHeads * D));
#pragma unroll
        for (int e = 0; e < E4; ++e) {
          const float4 t = po[PARTS * e];
          x[j][e] = ok ? t : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    };
    load_batch(w0);
    float Mw = -__builtin_huge_valf();
    for (int v0 = w0; v0 <= wend; v0 += kLseBatch) {
      float y[kLseBatch];
#pragma unroll
      for (int j = 0; j < kLseBatch; ++j) {
        const float l = lse_base[slot_of_piece(min(v0 + j, wend)) * kDecodeUnitHeads];
        y[j] = have(v0 + j) ? l : -__builtin_huge_valf();
      }
#pragma unroll
      for (int j = 0; j < kLseBatch; ++j) Mw = fmaxf(Mw, y[j]);
    }
    if (w0 != wf && Mw > M) {  // a later window with a larger maximum
      const float r = __builtin_amdgcn_exp2f(M - Mw);
#pragma unroll
      for (int e = 0; e < E4; ++e) o[e] = make_float4(o[e].x * r, o[e].y * r, o[e].z * r, o[e].w * r);
      wsum *= r;
    }
    M = fmaxf(M, Mw);
    for (int v0 = w0; v0 <= wend; v0 += PB) {
      if (v0 != w0) load_batch(v0);
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const float wk = __builtin_amdgcn_exp2f(lv[j] - M);  // 0 for a missing piece
#pragma unroll
        for (int e = 0; e < E4; ++e) {
          o[e].x = fmaf(wk, x[j][e].x, o[e].x);
          o[e].y = fmaf(wk, x[j][e].y, o[e].y);
          o[e].z = fmaf(wk, x[j][e].z, o[e].z);
          o[e].w = fmaf(wk, x[j][e].w, o[e].w);
        }
        wsum += wk;
      }
    }
  }
  if (hn >= nh) return;
  const float inv = 1.f / wsum;
  const int h = kvh * p.group + kDecodeUnitHeads * hc + hn;
  const int64_t row = static_cast<int64_t>(token) * p.num_heads + h;
  // optional partial state of the whole row: fp32 output and natural-log lse
  if (p.out_f32 != nullptr) {
    float4* of = reinterpret_cast<float4*>(p.out_f32 + row * D + 4 * qd);
#pragma unroll
    for (int e = 0; e < E4; ++e) of[PARTS * e] = make_float4(o[e].x * inv, o[e].y * inv, o[e].z * inv, o[e].w * inv);
  }
  if (p.lse_out != nullptr && qd == 0) p.lse_out[row] = (M + __log2f(wsum)) * 0.6931471805599453f;
  uint16_t* out = p.out + row * D + 4 * qd;
  const uint16_t* gt = p.gate == nullptr ? nullptr : p.gate + row * D + 4 * qd;  // output gate
#pragma unroll
  for (int e = 0; e < E4; ++e) {
    float sg[4] = {1.f, 1.f, 1.f, 1.f};
    if (gt != nullptr) {
      const uint2 gw = *reinterpret_cast<const uint2*>(gt + 4 * PARTS * e);
      sg[0] = gate_sigmoid(Elem<BF16>::value(gw.x & 0xffffu));
      sg[1] = gate_sigmoid(Elem<BF16>::value(gw.x >> 16));
      sg[2] = gate_sigmoid(Elem<BF16>::value(gw.y & 0xffffu));
      sg[3] = gate_sigmoid(Elem<BF16>::value(gw.y >> 16));
    }
    const float v4[4] = {o[e].x, o[e].y, o[e].z, o[e].w};
    uint32_t w2[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      w2[c] = static_cast<uint32_t>(Elem<BF16>::bits(v4[2 * c] * inv * sg[2 * c])) |
              (static_cast<uint32_t>(Elem<BF16>::bits(v4[2 * c + 1] * inv * sg[2 * c + 1])) << 16);
    }
    *reinterpret_cast<uint2*>(out + 4 * PARTS * e) = make_uint2(w2[0], w2[1]);
  }
}

// The merge of one segment with the lane layout of the group's head slots.
template <int D, bool BF16>
__device__ inline void merge_segment_any(const AttnParams& p, int task, int T, int lane, int4 sq) {
  const int hsl = decode_head_slots(p.group);
  if (hsl == 4) merge_segment<D, BF16, 4>(p, task, T, lane, sq);
  else if (hsl == 8) merge_segment<D, BF16, 8>(p, task, T, lane, sq);
  else merge_segment<D, BF16, 16>(p, task, T, lane, sq);
}

}  // namespace pa

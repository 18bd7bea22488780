// Top-k selection and softmax over one token's router logits, by one wave.
//
// "Mixture of experts: por qué un modelo enorme apenas usa sus parámetros",
// section "El router: la pieza que de verdad decide": the k highest scores
// are kept and normalised by a softmax among themselves.  Order: value
// descending, ties to the lower expert index; slot q is the q-th of that
// order.  The softmax adds exp(l - l_max) of the chosen in slot order, l_max
// the largest chosen logit.
#pragma once
#include "device.hpp"

namespace moe {

// (v, i) ranks before (w, j).
__device__ __forceinline__ bool ranks_before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// logit: the token's E logits (any memory the wave can read); every lane of
// the wave calls this.  sel: per-expert selection bias, or NULL.  With it the
// order is taken on the fp32 key logit + sel (the auxiliary-loss-free load
// balancer of the glossary "MoE (Mixture of Experts - Mezcla de Expertos)",
// section 2 item 4) and the softmax still runs over the plain logits of the
// chosen, with their maximum subtracted.  out(q, expert, weight) is called by
// exactly one lane for each slot q < k.  E <= 256, 1 <= k <= min(E, 8).
template <class Out>
__device__ __forceinline__ void topk_softmax(const float* logit, const float* sel, int E, int k,
                                             int lane, Out out) {
  if (E <= 64) {
    // one logit per lane: a lane's slot is the number of keys that rank
    // before its own, counted from scalar reads of every lane (no shuffles)
    const float v = lane < E ? logit[lane] : -__builtin_inff();
    const float key = (sel && lane < E) ? v + sel[lane] : v;
    int rank = 0;
    for (int j = 0; j < E; ++j) rank += ranks_before(lane_value(key, j), j, key, lane) ? 1 : 0;
    const bool chosen = lane < E && rank < k;
    int src[8];  // lane holding slot q
    float vmax = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      src[q] = q < k ? (int)__builtin_ctzll(__ballot(chosen && rank == q)) : 0;
      if (q < k) vmax = fmaxf(vmax, lane_value(v, src[q]));
    }
    const float ex = chosen ? expf(v - vmax) : 0.f;
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < k) tot += lane_value(ex, src[q]);
    if (chosen) out(rank, lane, ex / tot);
    return;
  }
  // up to 256 logits, 4 per lane: k rounds of a wave-wide arg-max of the keys
  float v[4];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    live[q] = e < E;
    v[q] = live[q] ? logit[e] : 0.f;
    if (sel && live[q]) v[q] += sel[e];
  }
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = 0x7fffffff;
    bool have = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (live[q] && (!have || ranks_before(v[q], e, bv, bi))) {
        bv = v[q];
        bi = e;
        have = true;
      }
    }
    // lanes with nothing left carry index INT_MAX and lose every comparison
    if (!have) bv = -__builtin_inff();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q == bi) live[q] = false;
    if (lane == j) my_i = bi;
  }
  // plain logit of slot `lane`; softmax with the chosen maximum subtracted
  const float my_v = lane < k ? logit[my_i] : -__builtin_inff();
  float vmax = -__builtin_inff();
  for (int q = 0; q < k; ++q) vmax = fmaxf(vmax, lane_value(my_v, q));
  const float ex = lane < k ? expf(my_v - vmax) : 0.f;
  float tot = 0.f;
  for (int q = 0; q < k; ++q) tot += lane_value(ex, q);  // slot order
  if (lane < k) out(lane, my_i, ex / tot);
}

}  // namespace moe

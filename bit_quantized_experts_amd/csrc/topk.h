// topk.h -- top-k selection with gate weights by one wavefront, shared by
// the route kernels (standalone selection) and the decode gate/up kernel
// (each of its workgroups selects the experts of every token itself).
//
// The router keeps about ten of 512 small experts per token and weighs them
// by a softmax over the kept logits [cnyes profile of Strata, section
// "Strata 到底是什麼？"].
#pragma once
#include "kern_common.h"

namespace {

// Selection key of (logit v, expert e): larger key = ranks earlier (logit
// descending, then index ascending).  The float's bits are mapped to an
// unsigned integer of the same order (-0.0 first folded into +0.0); the low
// word is the complement of the index.  Key 0 never occurs for a finite
// logit, so it marks an expert already taken.
DEVI uint64_t sel_key(float v, int e) {
  uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
DEVI float key_value(uint64_t k) {
  uint32_t b = (uint32_t)(k >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}
DEVI int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

// Top-k of one row of E logits by one wavefront, then the gate weights.
// Lane l holds the keys of experts l, l+64, ...; keys are unique.
//   1. Candidates: theta = the k-th largest (counted with multiplicity) of
//      the 64 lane maxima of the keys' value words (high 32 bits), rounded
//      down to a multiple of 2^16 (sign, exponent and 7 mantissa bits of the
//      logit), found from the most significant bit with ballots, two bits per
//      step (three ballots against independent thresholds), 8 steps.  At
//      least k keys have a value word >= theta (those k lane maxima), so every
//      key of the top k does too (a smaller one would rank below those k
//      keys).  The rounding only admits the few keys within 2^-7 relative of
//      the k-th lane maximum as extra candidates.
//   2. If at most 64 keys reach theta they are compacted to LDS, each is
//      ranked by counting the larger candidates, and the first k ranks are
//      the answer.  Otherwise (many equal logits) a radix search on the value
//      words finds the k-th largest value (a trial threshold is kept while at
//      least k values reach it, stopping once exactly k do); the values above
//      it and the tied ones in ascending expert index are taken, compacted
//      and ranked the same way.
// Lane r ends up with rank r (value descending, then index ascending).  Gate
// weights: m = logit of rank 0, e_r = exp64(l_r - m), S = sum of e_r in rank
// order, w_r = fp32(e_r / S).  `buf`: this wave's 96 LDS entries.  NPER >=
// ceil(E / 64).  The work is a single wavefront's dependent chain, so the
// loops stay short: 8 steps for theta and one step per candidate for the
// ranks.  Returns lane r's (expert, weight) for r < k ({-1, 0} above) and
// also stores them to idx_out / w_out unless those are null.
DEVI int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

DEVI uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int TOPK_BUF = 96;  // LDS entries per wave: 64 candidates + 32

struct TopkLane {
  int e;
  float w;
};

template <int NPER>
DEVI TopkLane topk_keys(const uint64_t (&key)[NPER], int E, int k, int32_t* idx_out, float* w_out, uint64_t* buf);

template <int NPER, typename RowT>
DEVI void topk_wave(RowT row, int E, int k, int32_t* idx_out, float* w_out, uint64_t* buf) {
  const int lane = opaque_tid() & 63;
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? sel_key(row(e), e) : 0ull;  // 0: no expert
  }
  topk_keys<NPER>(key, E, k, idx_out, w_out, buf);
}

// The same from the keys (lane l: experts l, l+64, ...; 0 = no expert).
template <int NPER>
DEVI TopkLane topk_keys(const uint64_t (&key)[NPER], int E, int k, int32_t* idx_out, float* w_out, uint64_t* buf) {
  const int lane = opaque_tid() & 63;
  // 1. theta = the largest multiple of 2^16 that at least k of the 64 lane
  // maxima of the value words reach, by a most-significant-bit-first search
  // over ballots
  uint32_t lhi = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) lhi = max(lhi, (uint32_t)(key[i] >> 32));
  // two bits per step over the high 16 bits (the three trial thresholds are
  // independent, so the dependent chain is 8 steps long)
  uint32_t theta = 0;
  for (int b = 30; b >= 16; b -= 2) {
    const uint32_t t1 = theta | (1u << b), t2 = theta | (2u << b), t3 = theta | (3u << b);
    const int c1 = (int)__builtin_popcountll(__ballot(lhi >= t1));
    const int c2 = (int)__builtin_popcountll(__ballot(lhi >= t2));
    const int c3 = (int)__builtin_popcountll(__ballot(lhi >= t3));
    theta = c3 >= k ? t3 : c2 >= k ? t2 : c1 >= k ? t1 : theta;
  }
  int c = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) c += (int)__builtin_popcountll(__ballot((uint32_t)(key[i] >> 32) >= theta));

  // 2. choose the candidate set: keys >= theta, or the exact top k
  bool exact = true;
  uint32_t tau = 0;
  int need = 0;
  if (c > 64) {
    uint32_t hv[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) hv[i] = (uint32_t)(key[i] >> 32);
    exact = false;
    for (int b = 31; b >= 0; --b) {
      const uint32_t t = tau | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) cnt += (int)__builtin_popcountll(__ballot(hv[i] >= t));
      if (cnt >= k) {
        tau = t;
        if (cnt == k) {
          exact = true;
          break;
        }
      }
    }
    if (!exact) {
      int c_gt = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) c_gt += (int)__builtin_popcountll(__ballot(hv[i] > tau));
      need = k - c_gt;
    }
  }
  const bool radix = c > 64;
  // compact the candidates to buf[0..n) in (slot, lane) order
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const uint32_t hv = (uint32_t)(key[i] >> 32);
    bool take;
    if (!radix) {
      take = hv >= theta;
    } else {
      const bool tie = !exact && hv == tau;
      const uint64_t tm = __ballot(tie);
      take = exact ? (hv >= tau) : (hv > tau || (tie && lanes_below(tm) < need));
      need -= min(need, (int)__builtin_popcountll(tm));
    }
    const uint64_t sm = __ballot(take);
    const int pos = n + lanes_below(sm);
    if (take && pos < 64) buf[pos] = key[i];
    n += (int)__builtin_popcountll(sm);
  }
  n = min(n, 64);
  // rank the candidates (lanes >= n hold 0, which is never larger); the
  // first k ranks are the result
  // (each candidate read by every lane from LDS at once, a broadcast; the
  // wavefront's own compaction stores are in order before these reads)
  const uint64_t mine = (lane < n) ? buf[lane] : 0ull;
  int rank = 0;
#pragma unroll 8
  for (int j = 0; j < n; ++j) rank += (buf[j] > mine) ? 1 : 0;
  if (lane < n && rank < k) buf[64 + rank] = mine;
  const uint64_t kr = (lane < k) ? buf[64 + lane] : 0ull;
  const float my_v = key_value(kr);
  const int my_e = key_index(kr);
  const double m = (double)__builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, my_v)));
  double ev = 0.0;
  if (lane < k) ev = moe_exp64((double)my_v - m);
  // S in rank order, the same in every lane: each lane puts its e_r in
  // buf[r] (the candidates are no longer needed) and every lane adds them
  // back from broadcast reads
  if (lane < k) buf[lane] = __builtin_bit_cast(uint64_t, ev);
  double S = 0.0;
  for (int r = 0; r < k; ++r) S += __builtin_bit_cast(double, buf[r]);
  TopkLane r{-1, 0.f};
  if (lane < k) {
    r.e = (my_e >= 0 && my_e < E) ? my_e : 0;  // (other only with non-finite logits, out of contract)
    r.w = (float)(ev / S);
    if (idx_out) idx_out[lane] = r.e;
    if (w_out) w_out[lane] = r.w;
  }
  return r;
}

}  // namespace

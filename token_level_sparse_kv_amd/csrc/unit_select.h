// Exact selection of whole units (runs of consecutive positions) by a per-unit
// score, shared by the gated-logit step (units = gated context units) and the
// block-sparse step (units = key blocks). One workgroup of NT threads (1024 for the
// selection kernels, 256 where the selection is fused into the attention) per
// (sequence, KV head):
//   * forced units are always kept; when the sequence has at most `budget` units,
//     every unit is kept;
//   * otherwise `need` more units are taken among the eligible ones, largest score
//     first, equal scores by lower unit (order-preserving u32 keys, NaN lowest), by
//     a radix select over 8-bit digits from the top: each pass histograms the keys
//     that share the digits fixed so far and fixes the digit holding the boundary;
//     it stops early once the boundary digit's keys are all taken, else after the
//     last digit it takes the lowest units among those equal to the boundary key;
//   * an ordered compaction (one block scan of packed counts) lists the kept units
//     ascending, and the kept units' positions are written out, -1 past n and past
//     the kept units.
#pragma once

#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {

constexpr int SEL_UNIT_THREADS = 1024;
constexpr int SEL_UNIT_WAVES = SEL_UNIT_THREADS / 64;

// LDS of the selector: NT threads, room for KC kept units.
template <int NT = SEL_UNIT_THREADS, int KC = SJSA_MAX_SELECT_UNITS>
struct UnitSelectSharedT {
  static constexpr int THREADS = NT;
  static constexpr int KEPT_CAP = KC;
  uint32_t hist[256];
  uint32_t wsum[NT / 64];
  uint32_t misc[4];
  int32_t kept[KC];
};
using UnitSelectShared = UnitSelectSharedT<>;

// Block-wide exclusive prefix sum of one value per thread (NT threads); total gets
// the sum. Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ uint32_t unit_block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = wsum[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Kept units of one (sequence, KV head), ascending, into sh.kept; returns how many.
// U: units of the sequence; all: keep every unit; need: eligible units to take
// (need <= the eligible units when !all); score(i): the unit's score (called for
// eligible units only); forced(i), eligible(i): predicates for i < U (disjoint).
// Every thread of the workgroup must call it. At most KEPT_CAP units are listed.
template <class SH, class ScoreF, class ForcedF, class EligF>
__device__ uint32_t select_kept_units(int U, bool all, int need, ScoreF score, ForcedF forced, EligF eligible,
                                      SH& sh) {
  constexpr int NT = SH::THREADS;
  constexpr uint32_t KC = (uint32_t)SH::KEPT_CAP;
  const int tid = threadIdx.x;
  // keep eligible unit i iff (key & mask) > prefix, or (key & mask) == prefix and
  // either the whole boundary digit is taken or it is among the first take_eq
  uint32_t prefix = 0xffffffffu, mask = 0xffffffffu, take_eq = 0;
  bool whole = false;
  if (!all && need > 0) {
    prefix = 0;
    mask = 0;
    uint32_t remaining = (uint32_t)need;
    if (tid == 0) { sh.misc[0] = 0u; sh.misc[1] = 0u; sh.misc[2] = 0u; }
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < U; i += NT) {
        if (!eligible(i)) continue;
        const uint32_t key = score_key(score(i));
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds bins 255-4l .. 252-4l; the scan runs from the top bin down.
        // remaining <= the keys sharing the prefix, so some lane reaches it.
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { c[e] = sh.hist[255 - 4 * tid - e]; sum += c[e]; }
        const uint32_t inc = wave_incl_scan(sum);
        const uint64_t hit = __ballot(inc >= remaining);
        const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 63;
        if (tid == L) {
          uint32_t before = inc - sum;
          int e = 0;
          while (e < 3 && before + c[e] < remaining) before += c[e++];
          sh.misc[0] = (uint32_t)(255 - 4 * tid - e);      // boundary digit
          sh.misc[1] = remaining - before;                 // keys to take from it
          sh.misc[2] = c[e];                               // keys in it
        }
      }
      __syncthreads();
      prefix |= sh.misc[0] << shift;
      mask |= 0xffu << shift;
      remaining = sh.misc[1];
      const uint32_t in_bin = sh.misc[2];
      __syncthreads();
      if (remaining == in_bin) { whole = true; break; }
    }
    take_eq = remaining;
  }

  // ordered compaction: one scan of (boundary-equal << 16 | kept for sure)
  uint32_t ndef = 0, neq = 0;
  for (int base = 0; base < U; base += NT) {
    const int i = base + tid;
    bool def = false, eq = false;
    if (i < U) {
      if (all || forced(i)) {
        def = true;
      } else if (need > 0 && eligible(i)) {
        const uint32_t hi = score_key(score(i)) & mask;
        def = hi > prefix || (whole && hi == prefix);
        eq = !whole && hi == prefix;
      }
    }
    uint32_t tot;
    const uint32_t ex = unit_block_excl_scan<NT>((eq ? 0x10000u : 0u) | (def ? 1u : 0u), sh.wsum, tot);
    const uint32_t eq_before = neq + (ex >> 16);
    const bool keep = def || (eq && eq_before < take_eq);
    const uint32_t slot = ndef + (ex & 0xffffu) + min(eq_before, take_eq);
    if (keep && slot < KC) sh.kept[slot] = i;
    ndef += tot & 0xffffu;
    neq += tot >> 16;
  }
  __syncthreads();
  return min(ndef + min(neq, take_eq), KC);
}

// Positions of the kept units, ascending: entry e of the list belongs to kept unit
// e / unit_size; positions >= n and entries past the kept units are -1. extra(e, s,
// valid) is called for every entry (s = kept slot) to write per-entry side data.
template <class SH, class ExtraF>
__device__ void write_kept_positions(const SH& sh, uint32_t nsel, int unit_size, float inv_unit,
                                     int64_t n, int ktok, int32_t* __restrict__ out, ExtraF extra) {
  for (int e = threadIdx.x; e < ktok; e += SH::THREADS) {
    int s = (int)((float)e * inv_unit);          // e < 2^24: off by at most one, fixed below
    s -= s * unit_size > e ? 1 : 0;
    s += (s + 1) * unit_size <= e ? 1 : 0;
    int32_t p = -1;
    if (s < (int)nsel) {
      const int64_t pos = (int64_t)sh.kept[s] * unit_size + (e - s * unit_size);
      if (pos < n) p = (int32_t)pos;
    }
    out[e] = p;
    extra(e, s, p >= 0);
  }
}

}  // namespace sjsa

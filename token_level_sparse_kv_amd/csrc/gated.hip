// Gated-logit unit selection (SAS): per (sequence, KV head), normalize the
// selector's per-unit scores into softmax gates, keep the current unit plus the
// units with the largest gates, expand the kept units into their token positions
// and give every position its log-gate logit term.
//
// Source: SAS article ("SAS：用门控稀疏注意力把上下文排序端到端对齐 LM 损失"),
// section 2.1 (the gate enters each attention logit as lambda * log g), section
// 2.2 (b) (normalized softmax gates; the current block is always kept) and
// section 2.3 (decode keeps the top units by gate and attends only over them).
//
// grid = B * H_kv workgroups of 1024 threads. With U units in the sequence (the
// last one, holding position n-1, is the current unit):
//   * gates: m = max u, S = sum 2^((u - m) log2 e), both from one pass that keeps a
//     running (max, sum) per thread and merges the pairs; the exp2-domain logit
//     term of unit i is lambda * ((u_i - m) log2 e - log2 S) = lambda * log2(e) * ln g_i;
//   * selection, when U > k_units: the k_units - 1 largest scores among the other
//     units, ties to the lower unit (order-preserving u32 keys, NaN lowest), by a
//     radix select over 8-bit digits from the top: each pass histograms the keys
//     that share the digits fixed so far and fixes the digit holding the boundary;
//     it stops early once the boundary digit's keys are all taken, else after the
//     last digit it takes the lowest units among those equal to the boundary key.
//     Scores are staged in LDS when they fit (else read from global each pass);
//   * an ordered compaction (one block scan of packed counts) lists the kept units
//     in ascending order, then the workgroup writes their positions (coalesced),
//     -1 past n and past the kept units, and the matching logit terms.
#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int GATE_THREADS = 1024;
constexpr int GATE_WAVES = GATE_THREADS / 64;
constexpr int GATE_LDS_UNITS = 8192;        // scores staged in LDS up to this many units
constexpr float GATE_LOG2E = 1.4426950408889634f;

// Block-wide exclusive prefix sum of one value per thread; total gets the sum.
// Every thread of the block must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < GATE_WAVES; ++w) {
    const uint32_t t = wsum[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

__global__ __launch_bounds__(GATE_THREADS) void gate_select_kernel(
    const float* __restrict__ u, int64_t ustride, const int32_t* __restrict__ seq_len, int n_kv_heads,
    int64_t cap, int unit_size, int k_units, float lam, int32_t* __restrict__ idx, float* __restrict__ bias,
    int ktok, float inv_unit) {
  constexpr int THREADS = GATE_THREADS, WAVES = GATE_WAVES;
  __shared__ float su[GATE_LDS_UNITS];
  __shared__ uint32_t hist[256];
  __shared__ int32_t sel_unit[SJSA_MAX_GATED_UNITS];
  __shared__ float sel_bias[SJSA_MAX_GATED_UNITS];
  __shared__ uint32_t wsum[WAVES];
  __shared__ float red[2][WAVES];
  __shared__ uint32_t misc[4];

  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int U = (int)((n + unit_size - 1) / unit_size);
  const int tid = threadIdx.x;
  const bool staged = U <= GATE_LDS_UNITS;
  const float* ug = u + (size_t)unit * ustride;
  auto score = [&](int i) -> float { return staged ? su[i] : ug[i]; };

  // stage the scores; normalized softmax gates (exp2 domain) from a running
  // (max, sum of 2^((u - max) log2 e)) per thread, merged per wave, then per block
  float tm = -INFINITY, ts = 0.f;
  for (int i = tid; i < U; i += THREADS) {
    const float x = ug[i];
    if (staged) su[i] = x;
    const float nm = fmaxf(tm, x);
    ts = ts * exp2f((tm - nm) * GATE_LOG2E) + exp2f((x - nm) * GATE_LOG2E);   // tm = -inf: ts = 0
    tm = nm;
  }
  const float wm = wave_max_f32(tm);
  float ws = wm == -INFINITY ? 0.f : ts * exp2f((tm - wm) * GATE_LOG2E);
  ws = row16_sum(ws);
  ws = readlane_f32(ws, 0) + readlane_f32(ws, 16) + readlane_f32(ws, 32) + readlane_f32(ws, 48);
  if ((tid & 63) == 0) { red[0][tid >> 6] = wm; red[1][tid >> 6] = ws; }
  __syncthreads();                              // also publishes the staged scores
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) mx = fmaxf(mx, red[0][w]);
  float sm = 0.f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) sm += red[0][w] == -INFINITY ? 0.f : red[1][w] * exp2f((red[0][w] - mx) * GATE_LOG2E);
  const float lse2 = log2f(sm);

  const int cur = U - 1;
  const bool all = U <= k_units;
  const int need = all ? 0 : k_units - 1;     // other units to take when not all
  const int cand = U - 1;                      // the other units: 0 .. U-2
  // keep unit i (i < cand) iff (key & mask) > prefix, or (key & mask) == prefix and
  // either the whole boundary digit is taken (whole) or it is among the first
  // take_eq such units
  uint32_t prefix = 0xffffffffu, mask = 0xffffffffu;
  uint32_t take_eq = 0;
  bool whole = false;
  if (need > 0) {
    prefix = 0;
    mask = 0;
    uint32_t remaining = (uint32_t)need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += THREADS) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < cand; i += THREADS) {
        const uint32_t key = score_key(score(i));
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds bins 255-4l .. 252-4l; the scan runs from the top bin down.
        // remaining <= the keys sharing the prefix, so some lane reaches it.
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { c[e] = hist[255 - 4 * tid - e]; sum += c[e]; }
        const uint32_t inc = wave_incl_scan(sum);
        const uint64_t hit = __ballot(inc >= remaining);
        const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 63;
        if (tid == L) {
          uint32_t before = inc - sum;
          int e = 0;
          while (e < 3 && before + c[e] < remaining) before += c[e++];
          misc[0] = (uint32_t)(255 - 4 * tid - e);      // boundary digit
          misc[1] = remaining - before;                 // keys to take from it
          misc[2] = c[e];                               // keys in it
        }
      }
      __syncthreads();
      prefix |= misc[0] << shift;
      mask |= 0xffu << shift;
      remaining = misc[1];
      const uint32_t in_bin = misc[2];
      __syncthreads();
      if (remaining == in_bin) { whole = true; break; }
    }
    take_eq = remaining;
  }

  // ordered compaction of the kept units: one scan of (boundary-equal << 16 | kept)
  uint32_t ndef = 0, neq = 0;
  for (int base = 0; base < U; base += THREADS) {
    const int i = base + tid;
    bool def = false, eq = false;
    if (i < U) {
      if (all || i == cur) {
        def = true;
      } else if (need > 0) {
        const uint32_t hi = score_key(score(i)) & mask;
        def = hi > prefix || (whole && hi == prefix);
        eq = !whole && hi == prefix;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((eq ? 0x10000u : 0u) | (def ? 1u : 0u), wsum, tot);
    const uint32_t eq_before = neq + (ex >> 16);
    const bool keep = def || (eq && eq_before < take_eq);
    const uint32_t slot = ndef + (ex & 0xffffu) + min(eq_before, take_eq);
    if (keep && slot < (uint32_t)SJSA_MAX_GATED_UNITS) {
      sel_unit[slot] = i;
      sel_bias[slot] = lam * ((score(i) - mx) * GATE_LOG2E - lse2);
    }
    ndef += tot & 0xffffu;
    neq += tot >> 16;
  }
  __syncthreads();
  const uint32_t nsel = min(ndef + min(neq, take_eq), (uint32_t)SJSA_MAX_GATED_UNITS);

  // positions of the kept units, ascending; -1 past n and after the kept units
  int32_t* oi = idx + (size_t)unit * ktok;
  float* ob = bias + (size_t)unit * ktok;
  for (int e = tid; e < ktok; e += THREADS) {
    int s = (int)((float)e * inv_unit);          // e < 2^24: off by at most one, fixed below
    s -= s * unit_size > e ? 1 : 0;
    s += (s + 1) * unit_size <= e ? 1 : 0;
    int32_t p = -1;
    float bb = 0.f;
    if (s < (int)nsel) {
      const int64_t pos = (int64_t)sel_unit[s] * unit_size + (e - s * unit_size);
      if (pos < n) {
        p = (int32_t)pos;
        bb = sel_bias[s];
      }
    }
    oi[e] = p;
    ob[e] = bb;
  }
}

}  // namespace

hipError_t launch_gate_select(const sjsa_shape& s, const float* gate_scores, int64_t gate_stride,
                              const int32_t* seq_len, int unit_size, int k_units, float lambda, int32_t* idx,
                              float* bias, hipStream_t st) {
  const int ktok = k_units * unit_size;
  const dim3 grid((unsigned)((int64_t)s.batch * s.n_kv_heads));
  gate_select_kernel<<<grid, dim3(GATE_THREADS), 0, st>>>(gate_scores, gate_stride, seq_len, s.n_kv_heads,
                                                          s.capacity, unit_size, k_units, lambda, idx, bias, ktok,
                                                          1.0f / (float)unit_size);
  return hipGetLastError();
}

}  // namespace sjsa

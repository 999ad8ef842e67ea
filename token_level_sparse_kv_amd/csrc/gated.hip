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
// grid = B * H_kv workgroups of 256 threads. With U units in the sequence (the last
// one, holding position n-1, is the current unit):
//   * gates: m = max u, S = sum 2^((u - m) log2 e); the exp2-domain logit term of
//     unit i is lambda * ((u_i - m) log2 e - log2 S) = lambda * log2(e) * ln g_i;
//   * selection, when U > k_units: the k_units - 1 largest scores among the other
//     units, ties to the lower unit (order-preserving u32 keys, NaN lowest). Up to
//     GATE_RANK_MAX units are ranked by counting in LDS; more go through a 4-pass
//     8-bit radix select that finds the boundary key and how many of its equal keys
//     to take (the lowest units);
//   * an ordered compaction (block scans) lists the kept units in ascending order,
//     then the workgroup writes their positions (coalesced), -1 past n and past the
//     kept units, and the matching logit terms.
#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int GATE_THREADS = 256;
constexpr int GATE_WAVES = GATE_THREADS / 64;
constexpr int GATE_RANK_MAX = 1024;
constexpr float GATE_LOG2E = 1.4426950408889634f;

// Block-wide exclusive prefix sum of one value per thread; *total gets the sum.
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

__device__ __forceinline__ float block_max_f32(float v, float* red) {
  v = wave_max_f32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < GATE_WAVES; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum_f32(float v, float* red) {
  v = row16_sum(v);
  v = readlane_f32(v, 0) + readlane_f32(v, 16) + readlane_f32(v, 32) + readlane_f32(v, 48);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < GATE_WAVES; ++w) r += red[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(GATE_THREADS) void gate_select_kernel(
    const float* __restrict__ u, int64_t ustride, const int32_t* __restrict__ seq_len, int n_kv_heads,
    int64_t cap, int unit_size, int k_units, float lam, int32_t* __restrict__ idx, float* __restrict__ bias,
    int ktok) {
  __shared__ __align__(16) uint32_t keys[GATE_RANK_MAX];
  __shared__ uint32_t hist[256];
  __shared__ unsigned char flag[GATE_RANK_MAX];
  __shared__ int32_t sel_unit[SJSA_MAX_GATED_UNITS];
  __shared__ float sel_bias[SJSA_MAX_GATED_UNITS];
  __shared__ uint32_t wsum[GATE_WAVES];
  __shared__ float red[GATE_WAVES];
  __shared__ uint32_t misc[2];

  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int U = (int)((n + unit_size - 1) / unit_size);
  const float* uu = u + (size_t)unit * ustride;
  const int tid = threadIdx.x;

  // normalized softmax gates (exp2 domain)
  float mx = -INFINITY;
  for (int i = tid; i < U; i += GATE_THREADS) mx = fmaxf(mx, uu[i]);
  mx = block_max_f32(mx, red);
  float sm = 0.f;
  for (int i = tid; i < U; i += GATE_THREADS) sm += exp2f((uu[i] - mx) * GATE_LOG2E);
  sm = block_sum_f32(sm, red);
  const float lse2 = log2f(sm);

  const int cur = U - 1;
  const bool all = U <= k_units;
  const int need = all ? 0 : k_units - 1;     // other units to take when not all
  const int cand = U - 1;                      // the other units
  const bool counting = !all && cand <= GATE_RANK_MAX;
  uint32_t T = 0xffffffffu;                    // radix path: keys > T are taken ...
  int take_eq = 0;                             // ... and the first take_eq keys == T

  if (counting && need > 0) {
    // rank of unit i = units with a larger key, or an equal key and a lower index
    const int cand4 = (cand + 3) & ~3;
    for (int i = tid; i < cand4; i += GATE_THREADS) keys[i] = i < cand ? score_key(uu[i]) : 0u;
    __syncthreads();
    for (int i = tid; i < cand; i += GATE_THREADS) {
      const uint32_t ki = keys[i];
      uint32_t rank = 0;
      for (int j = 0; j < cand4; j += 4) {
        const uint4 kj = *reinterpret_cast<const uint4*>(&keys[j]);
        // padding keys are 0 and lie past i: they never count
        rank += (kj.x > ki || (kj.x == ki && j < i)) ? 1u : 0u;
        rank += (kj.y > ki || (kj.y == ki && j + 1 < i)) ? 1u : 0u;
        rank += (kj.z > ki || (kj.z == ki && j + 2 < i)) ? 1u : 0u;
        rank += (kj.w > ki || (kj.w == ki && j + 3 < i)) ? 1u : 0u;
      }
      flag[i] = rank < (uint32_t)need ? 1 : 0;
    }
    __syncthreads();
  } else if (!all && need > 0) {
    uint32_t prefix = 0, mask = 0;
    int remaining = need;
    if (tid == 0) { misc[0] = 0u; misc[1] = 0u; }
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += GATE_THREADS) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < cand; i += GATE_THREADS) {
        const uint32_t key = score_key(uu[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds bins 255-4l .. 252-4l; the scan runs from the top bin down
        uint32_t c[4], s = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { c[e] = hist[255 - 4 * tid - e]; s += c[e]; }
        const uint32_t inc = wave_incl_scan(s);
        const uint64_t hit = __ballot(inc >= (uint32_t)remaining);
        const int L = __ffsll((long long)hit) - 1;      // remaining <= cand keys: some lane hits
        if (tid == L) {
          uint32_t before = inc - s;
          for (int e = 0; e < 4; ++e) {
            if (before + c[e] >= (uint32_t)remaining) {
              misc[0] = (uint32_t)(255 - 4 * tid - e);
              misc[1] = (uint32_t)remaining - before;
              break;
            }
            before += c[e];
          }
        }
      }
      __syncthreads();
      prefix |= misc[0] << shift;
      mask |= 0xffu << shift;
      remaining = (int)misc[1];
      __syncthreads();
    }
    T = prefix;
    take_eq = remaining;
  }

  // ordered compaction of the kept units
  uint32_t nsel = 0, neq = 0;
  for (int base = 0; base < U; base += GATE_THREADS) {
    const int i = base + tid;
    bool keep = false, eq = false;
    uint32_t key = 0;
    if (i < U) {
      if (all || i == cur) {
        keep = true;
      } else if (counting) {
        keep = need > 0 && flag[i] != 0;
      } else {
        key = score_key(uu[i]);
        keep = key > T;
        eq = key == T && need > 0;
      }
    }
    uint32_t tot_eq;
    const uint32_t eq_rank = neq + block_excl_scan(eq ? 1u : 0u, wsum, tot_eq);
    neq += tot_eq;
    keep = keep || (eq && eq_rank < (uint32_t)take_eq);
    uint32_t tot_sel;
    const uint32_t slot = nsel + block_excl_scan(keep ? 1u : 0u, wsum, tot_sel);
    nsel += tot_sel;
    if (keep && slot < (uint32_t)SJSA_MAX_GATED_UNITS) {
      sel_unit[slot] = i;
      sel_bias[slot] = lam * ((uu[i] - mx) * GATE_LOG2E - lse2);
    }
  }
  __syncthreads();
  nsel = min(nsel, (uint32_t)SJSA_MAX_GATED_UNITS);

  // positions of the kept units, ascending; -1 past n and after the kept units
  int32_t* oi = idx + (size_t)unit * ktok;
  float* ob = bias + (size_t)unit * ktok;
  for (int e = tid; e < ktok; e += GATE_THREADS) {
    const int s = e / unit_size;
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
  gate_select_kernel<<<dim3((unsigned)((int64_t)s.batch * s.n_kv_heads)), dim3(GATE_THREADS), 0, st>>>(
      gate_scores, gate_stride, seq_len, s.n_kv_heads, s.capacity, unit_size, k_units, lambda, idx,
      bias, ktok);
  return hipGetLastError();
}

}  // namespace sjsa

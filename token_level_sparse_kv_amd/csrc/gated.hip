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
//   * selection (unit_select.h), when U > k_units: the current unit is forced and
//     the k_units - 1 largest scores among the other units are taken (ties to the
//     lower unit); scores are staged in LDS when they fit (else read from global);
//   * the kept units' positions are written out with each position's logit term.
#include "unit_select.h"

namespace sjsa {
namespace {

constexpr int GATE_LDS_UNITS = 8192;        // scores staged in LDS up to this many units
constexpr float GATE_LOG2E = 1.4426950408889634f;

__global__ __launch_bounds__(SEL_UNIT_THREADS) void gate_select_kernel(
    const float* __restrict__ u, int64_t ustride, const int32_t* __restrict__ seq_len, int n_kv_heads,
    int64_t cap, int unit_size, int k_units, float lam, int32_t* __restrict__ idx, float* __restrict__ bias,
    int ktok, float inv_unit) {
  __shared__ float su[GATE_LDS_UNITS];
  __shared__ UnitSelectShared sh;
  __shared__ float sel_bias[SJSA_MAX_SELECT_UNITS];
  __shared__ float red[2][SEL_UNIT_WAVES];

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
  for (int i = tid; i < U; i += SEL_UNIT_THREADS) {
    const float x = ug[i];
    if (staged) su[i] = x;
    const float nm = fmaxf(tm, x);
    // a score of -inf (gate 0) adds nothing; skipping it while nothing else has
    // been seen also keeps (-inf) - (-inf) out of the sum (tm = -inf: ts = 0)
    if (nm != -INFINITY) {
      ts = ts * exp2f((tm - nm) * GATE_LOG2E) + exp2f((x - nm) * GATE_LOG2E);
      tm = nm;
    }
  }
  const float wm = wave_max_f32(tm);
  float ws = wm == -INFINITY ? 0.f : ts * exp2f((tm - wm) * GATE_LOG2E);
  ws = row16_sum(ws);
  ws = readlane_f32(ws, 0) + readlane_f32(ws, 16) + readlane_f32(ws, 32) + readlane_f32(ws, 48);
  if ((tid & 63) == 0) { red[0][tid >> 6] = wm; red[1][tid >> 6] = ws; }
  __syncthreads();                              // also publishes the staged scores
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < SEL_UNIT_WAVES; ++w) mx = fmaxf(mx, red[0][w]);
  float sm = 0.f;
#pragma unroll
  for (int w = 0; w < SEL_UNIT_WAVES; ++w)
    sm += red[0][w] == -INFINITY ? 0.f : red[1][w] * exp2f((red[0][w] - mx) * GATE_LOG2E);
  const float lse2 = log2f(sm);

  // the current unit (the last) is forced; the others compete
  const int cur = U - 1;
  const bool all = U <= k_units;
  const uint32_t nsel = select_kept_units(
      U, all, k_units - 1, score, [&](int i) { return i == cur; }, [&](int i) { return i < cur; }, sh);
  for (int s = tid; s < (int)nsel; s += SEL_UNIT_THREADS)
    // lambda = 0 drops the gate term (also for a gate of 0, where lambda * ln g is 0 * -inf)
    sel_bias[s] = lam == 0.f ? 0.f : lam * ((score(sh.kept[s]) - mx) * GATE_LOG2E - lse2);
  __syncthreads();

  float* ob = bias + (size_t)unit * ktok;
  write_kept_positions(sh, nsel, unit_size, inv_unit, n, ktok, idx + (size_t)unit * ktok,
                       [&](int e, int s, bool valid) { ob[e] = valid ? sel_bias[s] : 0.f; });
}

}  // namespace

hipError_t launch_gate_select(const sjsa_shape& s, const float* gate_scores, int64_t gate_stride,
                              const int32_t* seq_len, int unit_size, int k_units, float lambda, int32_t* idx,
                              float* bias, hipStream_t st) {
  const int ktok = k_units * unit_size;
  const dim3 grid((unsigned)((int64_t)s.batch * s.n_kv_heads));
  gate_select_kernel<<<grid, dim3(SEL_UNIT_THREADS), 0, st>>>(gate_scores, gate_stride, seq_len, s.n_kv_heads,
                                                              s.capacity, unit_size, k_units, lambda, idx, bias, ktok,
                                                              1.0f / (float)unit_size);
  return hipGetLastError();
}

}  // namespace sjsa

// Gather-free indexed attention over each KV head's selected positions.
//
// Source: JSSA article, section 原理详解(二) (gather-free indexed attention): one
// launch per layer; the kernel resolves every KV head's own index set and maps
// each query head to its KV head's set; K and V are read in place, never copied
// to a staging buffer. One token's K (or V) row is contiguous along head_dim, so
// each indexed read is a full burst (section 不规则索引本身不是障碍): here a
// 256-byte row is read by 16 lanes with 16 bytes each.
//
// grid = (nsplit, B * H_kv), 256 threads = 16 row slots of 16 lanes (G = 8 without
// logit terms uses the MFMA form below instead). A workgroup
// handles `chunk` consecutive entries of its unit's index list; each slot walks
// its share of rows, U rows at a time (nontemporal loads: every row is read once),
// computing the G logits per row (lane t holds head dims 8t..8t+7, dotted as bf16
// pairs; DPP row reductions finish the dots: at G = 4 one transposed reduction
// leaves each lane one of the batch's 16 logits), and keeps an online softmax
// (reference m, sum l, accumulator acc) per query head in the exp2 domain (logits
// scaled by sm_scale*log2(e)); the reference is raised only when a logit exceeds it
// by more than RESCALE_SLACK, so most iterations skip the rescale. Slots are
// combined in LDS; with one split the workgroup writes the output directly,
// otherwise it writes its
// (m, l, acc) partial and merge_kernel (one workgroup per (unit, query head),
// launched next on the same stream) combines the partials in split order with a
// log-sum-exp merge.
#include <utility>

#include "sjsa_device.h"
#include "sjsa_internal.h"
#include "unit_select.h"

namespace sjsa {
namespace {

constexpr int ATT_THREADS = 256;
constexpr int SLOTS = ATT_THREADS / 16;
constexpr int ATT_U = 4;             // rows in flight per slot
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.f;  // log2 units a logit may exceed the softmax reference by

// Softmax weight 2^x for x <= RESCALE_SLACK: the hardware exp2 alone (results below
// 2^-126 come out as 0, which changes no sum of weights that holds one weight >= 1).
__device__ __forceinline__ float weight_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int DPP_ROW_HALF_MIRROR = 0x141;   // lane t of a row reads lane t ^ 7
// Lane i of each DPP row, broadcast to the whole row (row_newbcast:i).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(I >= 0 && I < 16, "a row has 16 lanes");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + I, 0xF, 0xF, true));
}
// out[i] = lane i's v, for lanes 0 .. sizeof...(I) - 1 of the row.
template <int... I>
__device__ __forceinline__ void row_bcast_all(float v, float* out, std::integer_sequence<int, I...>) {
  ((out[I] = row_bcast<I>(v)), ...);
}
// out[g] = lane 4g's v (the first lane of quad g), for g < sizeof...(I) <= 4.
template <int... I>
__device__ __forceinline__ void row_bcast_heads(float v, float* out, std::integer_sequence<int, I...>) {
  ((out[I] = row_bcast<(4 * I) & 15>(v)), ...);
}

// Transposed sum over the 16 lanes of a DPP row; lane t gets the full sum of value t.
// Lane t keeps its share of value i ^ ((t >> 2) << 2) in slot i (its caller permutes
// the upper two index bits by the lane's own), so the first two exchange rounds
// (partners t ^ 8 and t ^ 7, whose t >> 2 differs from the lane's in bit 1, resp.
// bit 0) add the partner's upper half of the slots to the lane's lower half without
// selects; the
// last two (partners t ^ 2 and t ^ 1) keep the half whose index bit matches the
// lane's. 15 additions instead of the 64 of sixteen full row sums.
__device__ __forceinline__ float row16_transpose_sum(const float (&v)[16], int t) {
  float b[8], c[4], d[2];
  const bool h1 = (t & 2) != 0, h0 = (t & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = v[i] + dpp<DPP_ROW_ROR8>(v[i + 8]);
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = b[i] + dpp<DPP_ROW_HALF_MIRROR>(b[i + 4]);
#pragma unroll
  for (int i = 0; i < 2; ++i) d[i] = (h1 ? c[i + 2] : c[i]) + dpp<DPP_QUAD_XOR2>(h1 ? c[i] : c[i + 2]);
  return (h0 ? d[1] : d[0]) + dpp<DPP_QUAD_XOR1>(h0 ? d[0] : d[1]);
}

// Gated-logit selection run by every attention workgroup of a unit (GATE form):
// the unit scores u, the unit size, the budget in units, lambda, and where the
// index list goes.
struct GateArgs {
  const float* u = nullptr;
  int64_t ustride = 0;
  int unit_size = 1;
  int k_units = 1;
  float lam = 0.f;
  int32_t* idx_out = nullptr;
};
constexpr int GATE_FUSED_MAX_UNITS = GATE_FUSED_UNITS_MAX;   // unit scores staged in LDS by the GATE form
constexpr int GATE_FUSED_MAX_KEPT = GATE_FUSED_KEPT_MAX;     // kept units the GATE form can list
constexpr float GATE_LOG2E = 1.4426950408889634f;

struct GateShared {
  UnitSelectSharedT<ATT_THREADS, GATE_FUSED_MAX_KEPT> sel;
  float su[GATE_FUSED_MAX_UNITS];
  float red[2][ATT_THREADS / 64];
};

// BIAS: every index entry carries an additive exp2-domain logit term (bias, laid out
// like idx), as the gated-logit variant needs.
// GATE (with BIAS): the workgroup first makes its unit's gated selection itself (the
// same gates, selection and logit terms as gate_select_kernel, here with 256
// threads; every split of the unit repeats it, which costs less than a launch and a
// round trip of the index list), keeps its own chunk of the positions and their
// terms in LDS and writes that chunk of the index list.
template <int G, int U, bool BIAS, bool GATE = false>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ bias, const int32_t* __restrict__ seq_len,
    int n_kv_heads, int64_t cap, int k, int chunk, int nsplit, float qscale, float* __restrict__ partials,
    void* __restrict__ out, int out_f32, GateArgs ga) {
  static_assert(!GATE || BIAS, "the gated selection gives every entry a logit term");
  constexpr int ACC_BYTES = SLOTS * G * HEAD_DIM * 4;
  constexpr int RAW_BYTES = GATE && sizeof(GateShared) > ACC_BYTES ? sizeof(GateShared) : ACC_BYTES;
  __shared__ int32_t sidx[1024];
  __shared__ float sbias[BIAS ? 1024 : 1];
  __shared__ uint32_t sq2[G][HEAD_DIM / 2];     // query heads as packed bf16 pairs
  __shared__ float sm_m[SLOTS][G];
  __shared__ float sm_l[SLOTS][G];
  __shared__ __attribute__((aligned(16))) unsigned char sraw[RAW_BYTES];   // slot combine (GATE: selection first)
  auto sm_acc = reinterpret_cast<float (*)[G][HEAD_DIM]>(sraw);

  const int unit = blockIdx.y;
  const int split = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int tid = threadIdx.x;
  const int slot = tid >> 4;
  const int t = tid & 15;

  const int first = split * chunk;
  const int cnt = max(0, min(chunk, k - first));
  const int32_t* ids = idx + (size_t)unit * k + first;
  const float* bss = (BIAS && !GATE) ? bias + (size_t)unit * k + first : nullptr;
  const uint16_t* Kb = K + (size_t)unit * cap * HEAD_DIM + t * 8;
  const uint16_t* Vb = V + (size_t)unit * cap * HEAD_DIM + t * 8;

  // loads are unconditional (an invalid entry reads row 0, which always exists, and
  // gets zero weight), so the compiler can keep every load of a batch in flight;
  // each selected row is read once, so the loads are nontemporal
  const uint32_t cap_u = (uint32_t)min(cap, (int64_t)INT32_MAX);
  const uint32_t n_u = (uint32_t)min(n, (int64_t)INT32_MAX);
  auto load_rows = [&](const int32_t (&j)[U], u32x4 (&kw)[U], u32x4 (&vw)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t row = (uint32_t)j[u] < cap_u ? (uint32_t)j[u] : 0u;
      kw[u] = ld16_stream(Kb + (size_t)row * HEAD_DIM);
      vw[u] = ld16_stream(Vb + (size_t)row * HEAD_DIM);
    }
  };
  int32_t j0[U];
  float b0[U];
  u32x4 kw0[U], vw0[U];
  if constexpr (GATE) {
    // ---- the unit's gated selection (as gate_select_kernel): normalized softmax
    // gates from a running (max, sum of 2^((u - max) log2 e)) per thread; the current
    // unit (the last) forced and the k_units - 1 largest other scores taken; this
    // workgroup's chunk of the kept positions and their logit terms into LDS
    GateShared& gs = *reinterpret_cast<GateShared*>(sraw);
    const int nu = (int)((n + ga.unit_size - 1) / ga.unit_size);
    const float* ug = ga.u + (size_t)unit * ga.ustride;
    float tm = -INFINITY, ts = 0.f;
    for (int i = tid; i < nu; i += ATT_THREADS) {
      const float x = ug[i];
      gs.su[i] = x;
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
    if ((tid & 63) == 0) { gs.red[0][tid >> 6] = wm; gs.red[1][tid >> 6] = ws; }
    __syncthreads();                            // also publishes the staged scores
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < ATT_THREADS / 64; ++w) mx = fmaxf(mx, gs.red[0][w]);
    float sm = 0.f;
#pragma unroll
    for (int w = 0; w < ATT_THREADS / 64; ++w)
      sm += gs.red[0][w] == -INFINITY ? 0.f : gs.red[1][w] * exp2f((gs.red[0][w] - mx) * GATE_LOG2E);
    const float lse2 = log2f(sm);
    const int cur = nu - 1;
    const uint32_t nsel = select_kept_units(
        nu, nu <= ga.k_units, ga.k_units - 1, [&](int i) { return gs.su[i]; }, [&](int i) { return i == cur; },
        [&](int i) { return i < cur; }, gs.sel);
    int32_t* iout = ga.idx_out + (size_t)unit * k + first;
    for (int i = tid; i < cnt; i += ATT_THREADS) {
      const int e = first + i;
      const int sl = e / ga.unit_size;
      int32_t p = -1;
      float bt = 0.f;
      if (sl < (int)nsel) {
        const int ku = gs.sel.kept[sl];
        const int64_t pos = (int64_t)ku * ga.unit_size + (e - sl * ga.unit_size);
        if (pos < n) {
          p = (int32_t)pos;
          // lambda = 0 drops the gate term (also for a gate of 0: 0 * -inf)
          bt = ga.lam == 0.f ? 0.f : ga.lam * ((gs.su[ku] - mx) * GATE_LOG2E - lse2);
        }
      }
      sidx[i] = p;
      sbias[i] = bt;
      iout[i] = p;
    }
    __syncthreads();                            // the chunk is staged; sraw is free again
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j0[u] = slot * U + u < cnt ? sidx[slot * U + u] : -1;
      b0[u] = slot * U + u < cnt ? sbias[slot * U + u] : 0.f;
    }
    load_rows(j0, kw0, vw0);
  } else {
    // the slot's first batch of rows is requested straight from the index list, before
    // the workgroup stages the list and the queries in LDS
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j0[u] = slot * U + u < cnt ? ids[slot * U + u] : -1;
      b0[u] = (BIAS && slot * U + u < cnt) ? bss[slot * U + u] : 0.f;
    }
    load_rows(j0, kw0, vw0);

    for (int i = tid; i < cnt; i += ATT_THREADS) {
      sidx[i] = ids[i];
      if constexpr (BIAS) sbias[i] = bss[i];
    }
  }
  // query heads kept in LDS as bf16 pairs (read per use: fewer registers, more
  // waves in flight); the exp2-domain scale is applied to each finished dot
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(q + (size_t)unit * G * HEAD_DIM);
  for (int i = tid; i < G * HEAD_DIM / 2; i += ATT_THREADS) sq2[i / (HEAD_DIM / 2)][i % (HEAD_DIM / 2)] = q2[i];
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  __syncthreads();

  auto consume = [&](const int32_t (&j)[U], const float (&bj)[U], const u32x4 (&kw)[U], const u32x4 (&vw)[U]) {
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ok[u] = j[u] >= 0 && (int64_t)j[u] < n;
    // logits: per query head, its q slice (8 bf16) is read from LDS once and dotted
    // with the U packed K rows by bf16 pair dot products (fp32 accumulation); the row
    // reduction runs for every row (a DPP row is one slot) and invalid rows are
    // masked afterwards
    float z[U][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(&sq2[g][t * 4]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float a = dot2_bf16(qv.x, kw[u].x, 0.f);
        a = dot2_bf16(qv.y, kw[u].y, a);
        a = dot2_bf16(qv.z, kw[u].z, a);
        a = dot2_bf16(qv.w, kw[u].w, a);
        a = row16_sum(a);
        z[u][g] = ok[u] ? (BIAS ? fmaf(a, qscale, bj[u]) : a * qscale) : -INFINITY;
      }
    }
    // online softmax with a lazy reference: the running reference m only moves (and
    // the accumulators are rescaled) when a logit exceeds it by more than
    // RESCALE_SLACK (weights stay <= 2^RESCALE_SLACK); with no valid logit yet
    // (m = -inf) the reference point is 0 and every weight comes out 0
    float p[U][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = z[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, z[u][g]);
      if (mx > m[g] + RESCALE_SLACK) {
        const float sc = exp2f(m[g] - mx);
        l[g] *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= sc;
        m[g] = mx;
      }
      const float ref = m[g] == -INFINITY ? 0.f : m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u][g] = weight_exp2(z[u][g] - ref);
        l[g] += p[u][g];
      }
    }
    // weighted V rows: each V row is unpacked once and added into the G accumulators
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      vf[0] = bf_lo(vw[u].x); vf[1] = bf_hi(vw[u].x); vf[2] = bf_lo(vw[u].y); vf[3] = bf_hi(vw[u].y);
      vf[4] = bf_lo(vw[u].z); vf[5] = bf_hi(vw[u].z); vf[6] = bf_lo(vw[u].w); vf[7] = bf_hi(vw[u].w);
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
      }
    }
  };

  // G * U = 16: lane t of a slot owns the logit of query head t / U and row t % U
  // (value t = g * U + u). Its dot partials are summed with the transposed row
  // reduction (slot i holds value i ^ ((t >> 2) << 2): head (i >> 2) ^ (t >> 2), row
  // i & 3), the softmax bookkeeping runs once per logit (the head's reference is kept
  // by each of its lanes, the running sum as per-lane shares), and each weight is
  // broadcast from its lane for the V accumulation.
  constexpr bool TR = G * U == 16;
  static_assert(!TR || (G == 4 && U == 4), "the lane layout covers 4 heads of 4 rows");
  const int tg = t / U, tu = t % U;
  float m_t = -INFINITY, l_t = 0.f;
  auto consume_tr = [&](int base, const int32_t (&j)[U], const u32x4 (&kw)[U], const u32x4 (&vw)[U]) {
    float a[16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(&sq2[(g ^ tg) & (G - 1)][t * 4]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x = dot2_bf16(qv.x, kw[u].x, 0.f);
        x = dot2_bf16(qv.y, kw[u].y, x);
        x = dot2_bf16(qv.z, kw[u].z, x);
        a[(g * U + u) & 15] = dot2_bf16(qv.w, kw[u].w, x);
      }
    }
    const float dot = row16_transpose_sum(a, t);
    // which rows of the batch are valid, as a bit mask (an index into a register
    // array would go through scratch memory); the lane's term comes from LDS
    uint32_t okm = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) okm |= (uint32_t)j[u] < n_u ? 1u << u : 0u;
    const bool ok = ((okm >> tu) & 1u) != 0u;
    float z;
    if constexpr (BIAS) z = ok ? fmaf(dot, qscale, sbias[base + tu]) : -INFINITY;
    else z = ok ? dot * qscale : -INFINITY;
    // the head's greatest logit of the batch: its U logits fill a quad of lanes
    float mx = fmaxf(z, dpp<DPP_QUAD_XOR1>(z));
    mx = fmaxf(mx, dpp<DPP_QUAD_XOR2>(mx));
    const bool raise = mx > m_t + RESCALE_SLACK;
    if (__ballot(raise) != 0) {
      const float sc = raise ? weight_exp2(m_t - mx) : 1.f;
      l_t *= sc;
      m_t = raise ? mx : m_t;
      float scg[G];                             // head g's factor, from lane g * U
      row_bcast_heads(sc, scg, std::make_integer_sequence<int, (G < 16 ? G : 16)>{});
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= scg[g];
      }
    }
    const float ref = m_t == -INFINITY ? 0.f : m_t;
    const float pt = weight_exp2(z - ref);
    l_t += pt;
    float p[16];                                // the batch's weights, from their lanes
    row_bcast_all(pt, p, std::make_integer_sequence<int, 16>{});
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      vf[0] = bf_lo(vw[u].x); vf[1] = bf_hi(vw[u].x); vf[2] = bf_lo(vw[u].y); vf[3] = bf_hi(vw[u].y);
      vf[4] = bf_lo(vw[u].z); vf[5] = bf_hi(vw[u].z); vf[6] = bf_lo(vw[u].w); vf[7] = bf_hi(vw[u].w);
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p[(g * U + u) & 15], vf[e], acc[g][e]);
      }
    }
  };
  auto step = [&](int base, const int32_t (&j)[U], const float (&bj)[U], const u32x4 (&kw)[U],
                  const u32x4 (&vw)[U]) {
    if constexpr (TR) consume_tr(base, j, kw, vw);
    else consume(j, bj, kw, vw);
  };

  if (slot * U < cnt) step(slot * U, j0, b0, kw0, vw0);
  for (int base = slot * U + SLOTS * U; base < cnt; base += SLOTS * U) {
    int32_t j[U];
    float bj[U];
    u32x4 kw[U], vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j[u] = base + u < cnt ? sidx[base + u] : -1;
      bj[u] = (BIAS && base + u < cnt) ? sbias[base + u] : 0.f;
    }
    load_rows(j, kw, vw);
    step(base, j, bj, kw, vw);
  }
  if constexpr (TR) {
    // the head's running sum: its shares fill a quad of lanes; lane g * U then
    // writes head g's reference and sum
    float lt = l_t + dpp<DPP_QUAD_XOR1>(l_t);
    lt += dpp<DPP_QUAD_XOR2>(lt);
    if (tu == 0) { sm_m[slot][tg] = m_t; sm_l[slot][tg] = lt; }
  }

  // ---- combine the 16 slots of this workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (!TR && t == 0) { sm_m[slot][g] = m[g]; sm_l[slot][g] = l[g]; }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[slot][g][t * 8 + e] = acc[g][e];
  }
  __syncthreads();

  const bool direct = nsplit == 1;
  float* part = partials + ((size_t)unit * nsplit + split) * G * PART_STRIDE;
  for (int o = tid; o < G * HEAD_DIM; o += ATT_THREADS) {
    const int g = o / HEAD_DIM, dim = o - g * HEAD_DIM;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) M = fmaxf(M, sm_m[s][g]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const float ms = sm_m[s][g];
        if (ms == -INFINITY) continue;
        const float w = exp2f(ms - M);
        L = fmaf(sm_l[s][g], w, L);
        A = fmaf(sm_acc[s][g][dim], w, A);
      }
    }
    if (direct) {
      const float r = L > 0.f ? A / L : 0.f;
      const size_t oi = ((size_t)unit * G + g) * HEAD_DIM + dim;
      if (out_f32) reinterpret_cast<float*>(out)[oi] = r;
      else reinterpret_cast<uint16_t*>(out)[oi] = (uint16_t)f32_to_bf16_rne(r);
    } else {
      part[g * PART_STRIDE + dim] = A;
      if (dim == 0) { part[g * PART_STRIDE + HEAD_DIM] = M; part[g * PART_STRIDE + HEAD_DIM + 1] = L; }
    }
  }
}

// MFMA form of the same computation, used for G = 8 (v_mfma_f32_16x16x16_bf16; lane
// l of a wave holds A[l%16][4*(l/16)+v], B[4*(l/16)+v][l%16] and D[4*(l/16)+v][l%16],
// v = 0..3). With 8 heads the per-row dot products and reductions of the vector form
// need about 210 VGPRs (2 waves per SIMD); here the 16-wide tiles are half used and
// the kernel keeps 4 waves per SIMD.
// grid = (nsplit, B * H_kv), 256 threads = 4 waves; wave w takes groups w, w+4, ...
// of 16 consecutive entries of the workgroup's chunk. Per group:
//  * S = K Q^T (16 keys x 16 columns, the first G columns being the query heads) in
//    8 steps over d; lane l loads 4 x 16 bytes of key row l%16, which directly form
//    its A operands once d is ordered so that step s, k-row 4q+v covers dim
//    32(s/2) + 8q + 4(s%2) + v; the queries are laid out the same way as B;
//  * softmax bookkeeping per head on the D layout (the 4 keys of a lane, then
//    across the 4 lane rows), with the lazily moved reference as above;
//  * O += P V: D's layout already is P's A layout (head l%16, keys 4(l/16)+v); V is
//    staged through a per-wave LDS tile and read back as key columns; O columns
//    are dims in the order dim(t, c) = 32(t/2) + 2c + (t%2) for tile t, column c.
template <int G>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void attend_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ seq_len, int n_kv_heads, int64_t cap,
    int k, int chunk, int nsplit, float qscale, float* __restrict__ partials,
    void* __restrict__ out, int out_f32) {
  static_assert(G <= 16, "the query heads fill at most the 16 MFMA columns");
  constexpr int NW = ATT_THREADS / 64;
  constexpr int KG = 16;                    // keys per MFMA group
  constexpr int PITCH = HEAD_DIM + 8;       // LDS V row pitch in bf16 (272 bytes: conflict-free column reads)
  __shared__ int32_t sidx[1024];
  __shared__ uint16_t sv[NW][KG * PITCH];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_o[NW][G][HEAD_DIM];

  const int unit = blockIdx.y;
  const int split = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q4 = lane >> 4;  // A/B/D row-in-16 and 4-row group of this lane

  const int first = split * chunk;
  const int cnt = max(0, min(chunk, k - first));
  const int32_t* ids = idx + (size_t)unit * k + first;
  for (int i = tid; i < cnt; i += ATT_THREADS) sidx[i] = ids[i];

  // B operands of S = K Q^T: column r is query head r (zero past G)
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  s16x4 qb[8];
  {
    const uint16_t* qh = q + ((size_t)unit * G + min(r, G - 1)) * HEAD_DIM;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint2 w = *reinterpret_cast<const uint2*>(qh + 32 * (s / 2) + 8 * q4 + 4 * (s % 2));
      const u32x2 x = {r < G ? w.x : 0u, r < G ? w.y : 0u};
      qb[s] = __builtin_bit_cast(s16x4, x);
    }
  }
  f32x4 O[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;          // per head r (identical in the 4 lane rows)
  __syncthreads();

  const uint16_t* Kb = K + (size_t)unit * cap * HEAD_DIM + 8 * q4;
  const uint16_t* Vb = V + (size_t)unit * cap * HEAD_DIM + 8 * q4;
  uint16_t* tile = sv[wave];
  for (int e0 = wave * KG; e0 < cnt; e0 += NW * KG) {
    // key row r of the group: 4 x 16 bytes each of K and V (unconditional loads; an
    // invalid entry reads row 0 and gets zero weight)
    const int32_t jr = e0 + r < cnt ? sidx[e0 + r] : -1;
    const int64_t row = (jr >= 0 && (int64_t)jr < cap) ? jr : 0;
    u32x4 kc[4], vc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kc[c] = ld16_stream(Kb + (size_t)row * HEAD_DIM + 32 * c);
#pragma unroll
    for (int c = 0; c < 4; ++c) vc[c] = ld16_stream(Vb + (size_t)row * HEAD_DIM + 32 * c);
    bool ok[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = e0 + 4 * q4 + v;
      const int32_t j = e < cnt ? sidx[e] : -1;
      ok[v] = j >= 0 && (int64_t)j < n && r < G;
    }
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 kw = kc[s / 2];
      const u32x2 h = (s % 2) ? u32x2{kw.z, kw.w} : u32x2{kw.x, kw.y};
      S = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, h), qb[s], S, 0, 0, 0);
    }
    // V rows into the wave's LDS tile (row r, dims 32c + 8q4 ..)
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(tile + r * PITCH + 32 * c + 8 * q4) = vc[c];

    // softmax bookkeeping for head r over the group's keys 4q4+v
    float z[4];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      z[v] = ok[v] ? S[v] * qscale : -INFINITY;
      mx = fmaxf(mx, z[v]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool raise = mx > m + RESCALE_SLACK;
    if (__ballot(raise) != 0ull) {          // some head's reference moves: rescale
      const float sc = raise ? exp2f(m - mx) : 1.f;
      if (raise) m = mx;
      lsum *= sc;
      // O rows are heads 4q4+v; head h's factor is in lane h
      float f[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int qq = 0; qq < (G + 3) / 4; ++qq) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (q4 == qq) f[v] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), 4 * qq + v));
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int v = 0; v < 4; ++v) O[t][v] *= f[v];
      }
    }
    // the weights enter the PV product as bf16 pairs hi + lo (hi = bf16(p), lo =
    // bf16(p - hi)), which keeps them to about 16 significant bits
    const float ref = m == -INFINITY ? 0.f : m;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float pv = weight_exp2(z[v] - ref);
      lsum += pv;
      ph[v] = f32_to_bf16_rne(pv);
      pl[v] = f32_to_bf16_rne(pv - __uint_as_float(ph[v] << 16));
    }
    const s16x4 pa_hi = __builtin_bit_cast(s16x4, u32x2{ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16)});
    const s16x4 pa_lo = __builtin_bit_cast(s16x4, u32x2{pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16)});

    // the tile's writes are wave-private: order them before the column reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
      uint32_t w[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) w[v] = *reinterpret_cast<const uint32_t*>(tile + (4 * q4 + v) * PITCH + 32 * t2 + 2 * r);
      const u32x2 lo = {(w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16)};
      const u32x2 hi = {(w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u)};
      const s16x4 vlo = __builtin_bit_cast(s16x4, lo), vhi = __builtin_bit_cast(s16x4, hi);
      O[2 * t2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, vlo, O[2 * t2], 0, 0, 0);
      O[2 * t2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, vlo, O[2 * t2], 0, 0, 0);
      O[2 * t2 + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, vhi, O[2 * t2 + 1], 0, 0, 0);
      O[2 * t2 + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, vhi, O[2 * t2 + 1], 0, 0, 0);
    }
    // the next group rewrites the tile only after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // ---- combine the waves of this workgroup
  if (q4 == 0 && r < G) { sm_m[wave][r] = m; sm_l[wave][r] = lsum; }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * q4 + v;
      if (h < G) sm_o[wave][h][32 * (t / 2) + 2 * r + (t % 2)] = O[t][v];
    }
  }
  __syncthreads();

  const bool direct = nsplit == 1;
  float* part = partials + ((size_t)unit * nsplit + split) * G * PART_STRIDE;
  for (int o = tid; o < G * HEAD_DIM; o += ATT_THREADS) {
    const int g = o / HEAD_DIM, dim = o - g * HEAD_DIM;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NW; ++s) M = fmaxf(M, sm_m[s][g]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int s = 0; s < NW; ++s) {
        const float ms = sm_m[s][g];
        if (ms == -INFINITY) continue;
        const float w = exp2f(ms - M);
        L = fmaf(sm_l[s][g], w, L);
        A = fmaf(sm_o[s][g][dim], w, A);
      }
    }
    if (direct) {
      const float res = L > 0.f ? A / L : 0.f;
      const size_t oi = ((size_t)unit * G + g) * HEAD_DIM + dim;
      if (out_f32) reinterpret_cast<float*>(out)[oi] = res;
      else reinterpret_cast<uint16_t*>(out)[oi] = (uint16_t)f32_to_bf16_rne(res);
    } else {
      part[g * PART_STRIDE + dim] = A;
      if (dim == 0) { part[g * PART_STRIDE + HEAD_DIM] = M; part[g * PART_STRIDE + HEAD_DIM + 1] = L; }
    }
  }
}

// Combine the nsplit partials of one (unit, query head) in split order; one thread
// per output dim. Partial s holds the running maximum m_s (exp2 domain), the sum
// l_s and the unnormalized output acc_s; the merge keeps a running (m, l, acc)
// and rescales by 2^(m_old - m_new) as each partial comes in (log-sum-exp merge),
// then out = acc / l.
template <int G, int MU>
__global__ __launch_bounds__(HEAD_DIM) void merge_kernel(const float* __restrict__ partials, int nsplit,
                                                         void* __restrict__ out, int out_f32) {
  const int unit = blockIdx.x / G;
  const int g = blockIdx.x - unit * G;
  const int dim = threadIdx.x;
  const float* pu = partials + ((size_t)unit * nsplit * G + g) * PART_STRIDE;
  const size_t sstride = (size_t)G * PART_STRIDE;
  float m = -INFINITY, l = 0.f, a = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += MU) {
    float ms[MU], ls[MU], as[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int s = min(s0 + u, nsplit - 1);
      const float* ps = pu + (size_t)s * sstride;
      ms[u] = s0 + u < nsplit ? ps[HEAD_DIM] : -INFINITY;
      ls[u] = ps[HEAD_DIM + 1];
      as[u] = ps[dim];
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const float mn = fmaxf(m, ms[u]);
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float so = exp2f(m - ref), sn = exp2f(ms[u] - ref);
      l = fmaf(l, so, ls[u] * sn);
      a = fmaf(a, so, as[u] * sn);
      m = mn;
    }
  }
  const float r = l > 0.f ? a / l : 0.f;
  const size_t oi = ((size_t)unit * G + g) * HEAD_DIM + dim;
  if (out_f32) reinterpret_cast<float*>(out)[oi] = r;
  else reinterpret_cast<uint16_t*>(out)[oi] = (uint16_t)f32_to_bf16_rne(r);
}

}  // namespace

namespace {

template <int G>
void launch_attend_g(const Layout& L, const uint16_t* q, const uint16_t* K, const uint16_t* V, const int32_t* idx,
                     const float* bias, int k, const int32_t* seq_len, int n_kv_heads, int64_t cap, float qscale,
                     float* partials, void* out, int out_f32, hipStream_t st, const GateArgs* gate) {
  const dim3 grid((unsigned)L.nsplit, (unsigned)L.units), block(ATT_THREADS);
  if (gate) {
    attend_kernel<G, ATT_U, true, true><<<grid, block, 0, st>>>(q, K, V, gate->idx_out, nullptr, seq_len, n_kv_heads,
                                                                cap, k, L.chunk, L.nsplit, qscale, partials, out,
                                                                out_f32, *gate);
  } else if (bias) {
    attend_kernel<G, ATT_U, true><<<grid, block, 0, st>>>(q, K, V, idx, bias, seq_len, n_kv_heads, cap, k, L.chunk,
                                                          L.nsplit, qscale, partials, out, out_f32, GateArgs{});
  } else if constexpr (G == 8) {
    attend_mfma_kernel<G><<<grid, block, 0, st>>>(q, K, V, idx, seq_len, n_kv_heads, cap, k, L.chunk, L.nsplit,
                                                  qscale, partials, out, out_f32);
  } else {
    attend_kernel<G, ATT_U, false><<<grid, block, 0, st>>>(q, K, V, idx, nullptr, seq_len, n_kv_heads, cap, k,
                                                           L.chunk, L.nsplit, qscale, partials, out, out_f32,
                                                           GateArgs{});
  }
  const dim3 mgrid((unsigned)(L.units * G));
  if (L.nsplit > 8) merge_kernel<G, 32><<<mgrid, dim3(HEAD_DIM), 0, st>>>(partials, L.nsplit, out, out_f32);
  else if (L.nsplit > 1) merge_kernel<G, 8><<<mgrid, dim3(HEAD_DIM), 0, st>>>(partials, L.nsplit, out, out_f32);
}

}  // namespace

hipError_t launch_attend(const sjsa_shape& s, const Layout& L, const uint16_t* q, const uint16_t* K,
                         const uint16_t* V, const int32_t* idx, int k, const int32_t* seq_len,
                         float sm_scale, void* out, unsigned char* ws, hipStream_t st, const float* bias,
                         const GatedSelect* gsel) {
  GateArgs ga;
  if (gsel) {
    ga.u = gsel->gate_scores;
    ga.ustride = gsel->gate_stride;
    ga.unit_size = gsel->unit_size;
    ga.k_units = gsel->k_units;
    ga.lam = gsel->lambda;
    ga.idx_out = gsel->idx;
  }
  const GateArgs* gate = gsel ? &ga : nullptr;
  float* partials = reinterpret_cast<float*>(ws + L.off_partials);
  const float qscale = sm_scale * LOG2E;
  const int out_f32 = (s.flags & SJSA_FLAG_OUT_F32) ? 1 : 0;
  switch (s.group) {
    case 1: launch_attend_g<1>(L, q, K, V, idx, bias, k, seq_len, s.n_kv_heads, s.capacity, qscale, partials, out,
                               out_f32, st, gate); break;
    case 2: launch_attend_g<2>(L, q, K, V, idx, bias, k, seq_len, s.n_kv_heads, s.capacity, qscale, partials, out,
                               out_f32, st, gate); break;
    case 4: launch_attend_g<4>(L, q, K, V, idx, bias, k, seq_len, s.n_kv_heads, s.capacity, qscale, partials, out,
                               out_f32, st, gate); break;
    case 8: launch_attend_g<8>(L, q, K, V, idx, bias, k, seq_len, s.n_kv_heads, s.capacity, qscale, partials, out,
                               out_f32, st, gate); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sjsa

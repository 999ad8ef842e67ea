// Per-(sequence, KV head) top-k selection over the fp32 scores.
//
// Source: JSSA article, section JSSA 的整体结构 (top-k token positions per KV head,
// shared by its query heads) and section 组件级拆解 (top-k selection is the stage
// that dominates at small batch). Ranking: larger score first; equal scores go to
// the lower position; -0 equals +0; NaN ranks below everything. Output: the
// min(k, n) selected positions in ascending order, then -1.
//
// One 1024-thread workgroup per unit, working on order-preserving u32 keys:
//  1. First radix digit (top 12 key bits): the histogram comes from the score
//     kernel (or is built here in one pass). A block scan finds the bin b1 that
//     holds the k-th largest key: cntA keys lie in higher bins, cntC in b1.
//  2. Fast path (cntA <= A_CAP, cntC <= C_CAP): one ordered pass over the scores
//     compacts the positions above b1 (list A) and the (key, position) pairs in b1
//     (list C) into LDS, in position order, with wavefront ballots. The rest is
//     LDS-only: two 10-bit radix rounds over C give the exact threshold key T and
//     how many keys equal to T are taken (the lowest positions first); C is
//     compacted to the selected positions, and A and C are merged by rank.
//  3. Fallback (large k or a degenerate score distribution): the remaining two
//     digits are resolved by histogram passes over the scores, then one ordered
//     ballot-compaction pass writes the result directly.
#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int EPT = 4;                          // consecutive positions per thread (one float4)
constexpr int SUB = SEL_THREADS * EPT;          // positions per sub-chunk
constexpr int SUPER = 4;                        // sub-chunks loaded ahead together
constexpr int A_CAP = 8192;
constexpr int C_CAP = 12288;

struct SelShared {
  uint32_t hist[HIST_BINS];
  int32_t listA[A_CAP];
  uint32_t ckey[C_CAP];
  int32_t cpos[C_CAP];
  uint32_t wtot[2][SEL_WAVES];
  uint32_t wcnt[2][2][SUPER][SEL_WAVES];   // [buffer][list A/C][sub-chunk][wave]
  uint32_t scan[SEL_WAVES];
  int32_t misc[8];
};

// Block-wide inclusive scan of one u32 per thread; returns the inclusive value and
// writes the block total to *total. Contains two barriers.
__device__ uint32_t block_incl_scan(uint32_t v, uint32_t* scan_lds, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane == 63) scan_lds[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t t = scan_lds[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return inc + before;
}

// Given a histogram of `nbins` bins (LDS) and need >= 1, find the bin b with
// count(bins > b) < need <= count(bins >= b). Results go to misc[0] (bin) and
// misc[1] (count above the bin), misc[2] (count in the bin). All threads call.
__device__ void find_bucket(const uint32_t* hist, int nbins, uint32_t need, SelShared& sh) {
  const int per = nbins / SEL_THREADS;         // 4 or 1 bins per thread
  const int lo = threadIdx.x * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[lo + i];
  uint32_t total;
  const uint32_t inc = block_incl_scan(local, sh.scan, &total);
  // keys in bins above this thread's range
  uint32_t above = total - inc;
  if (above < need && need <= above + local) {
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = hist[lo + i];
      if (above + c >= need) {
        sh.misc[0] = lo + i;
        sh.misc[1] = (int32_t)above;
        sh.misc[2] = (int32_t)c;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
}

// Unconditional float4 load of positions pos..pos+3 of a score row: positions at or
// past n are clamped to the last float4 that starts inside the row (the row is
// allocated up to a multiple of 4), and callers mask them out. Keeping every load
// unconditional lets the compiler overlap a whole batch of them.
__device__ __forceinline__ f32x4 load4(const float* row, int64_t pos, int64_t last4) {
  return *reinterpret_cast<const f32x4*>(row + min(pos, last4));
}

// Ordered compaction helper: ranks of the flagged elements of one sub-chunk (each
// thread holds EPT consecutive positions; lanes, then waves, are in position order).
// Returns this thread's first output slot relative to the sub-chunk start for the
// flag vector `f`, and the sub-chunk total through wave totals in wtot[which].
__device__ __forceinline__ uint32_t ballot_rank(const bool (&f)[EPT], uint32_t* wtot_row, uint32_t* total) {
  const int wave = threadIdx.x >> 6;
  const uint64_t lt = lanemask_lt();
  uint32_t below = 0, wave_cnt = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint64_t m = __ballot(f[e]);
    below += __popcll(m & lt);
    wave_cnt += __popcll(m);
  }
  if ((threadIdx.x & 63) == 0) wtot_row[wave] = wave_cnt;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t t = wtot_row[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  *total = tot;
  return before + below;
}

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const float* __restrict__ scores, int64_t stride, const int32_t* __restrict__ seq_len,
    int n_kv_heads, int64_t cap, int k, int32_t* __restrict__ idx,
    uint32_t* __restrict__ ghist, int have_hist) {
  __shared__ SelShared sh;
  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int tid = threadIdx.x;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int kk = (int)min((int64_t)k, n);
  int32_t* out = idx + (size_t)unit * k;
  const float* row = scores + (size_t)unit * stride;

  for (int i = kk + tid; i < k; i += SEL_THREADS) out[i] = -1;
  if (kk == 0) return;
  const int64_t last4 = ((n - 1) >> 2) << 2;     // last float4 start inside the row

  // ---- first digit: histogram of the top 12 key bits
  if (have_hist) {
    const uint32_t* gh = ghist + (size_t)unit * HIST_BINS;
    for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = gh[i];
  } else {
    for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = 0u;
    __syncthreads();
    for (int64_t c = (int64_t)tid * EPT; c < n; c += SUB) {
      const f32x4 v = load4(row, c, last4);
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (c + e < n) atomicAdd(&sh.hist[score_key(v[e]) >> HIST_SHIFT], 1u);
    }
  }
  __syncthreads();
  find_bucket(sh.hist, HIST_BINS, (uint32_t)kk, sh);
  const uint32_t b1 = (uint32_t)sh.misc[0];
  const int cntA = sh.misc[1];
  const int cntC = sh.misc[2];
  uint32_t need = (uint32_t)(kk - cntA);          // 1 <= need <= cntC

  if (cntA <= A_CAP && cntC <= C_CAP) {
    // ---- fast path, pass A: ordered compaction of lists A and C into LDS.
    // A super-chunk is SUPER sub-chunks of SUB positions; in sub-chunk s thread t holds
    // positions c0 + s*SUB + 4t .. +3, so position order is (s, wave, lane, e). Each
    // wave publishes its A and C counts per sub-chunk (double-buffered, one barrier
    // per super-chunk); every thread then derives its output slots. The next
    // super-chunk's loads are in flight while the current one is classified.
    uint32_t baseA = 0, baseC = 0;
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t lt = lanemask_lt();
    f32x4 cur[SUPER];
#pragma unroll
    for (int s = 0; s < SUPER; ++s) cur[s] = load4(row, (int64_t)s * SUB + tid * EPT, last4);
    int it = 0;
    for (int64_t c0 = 0; c0 < n; c0 += (int64_t)SUPER * SUB, ++it) {
      f32x4 nxt[SUPER];
#pragma unroll
      for (int s = 0; s < SUPER; ++s) nxt[s] = load4(row, c0 + (int64_t)(SUPER + s) * SUB + tid * EPT, last4);
      const int buf = it & 1;
      uint32_t key[SUPER][EPT];
      uint32_t fa[SUPER], fc[SUPER];                 // flag bits per element e
      uint32_t ra[SUPER], rc[SUPER];                 // flagged elements in lower lanes
#pragma unroll
      for (int s = 0; s < SUPER; ++s) {
        const int64_t p0 = c0 + (int64_t)s * SUB + tid * EPT;
        fa[s] = 0u;
        fc[s] = 0u;
        ra[s] = 0u;
        rc[s] = 0u;
        uint32_t wa = 0u, wc = 0u;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          key[s][e] = score_key(cur[s][e]);
          const uint32_t bin = key[s][e] >> HIST_SHIFT;
          const bool valid = p0 + e < n;
          const bool a = valid && bin > b1;
          const bool c = valid && bin == b1;
          fa[s] |= (uint32_t)a << e;
          fc[s] |= (uint32_t)c << e;
          const uint64_t ma = __ballot(a), mc = __ballot(c);
          ra[s] += __popcll(ma & lt);
          rc[s] += __popcll(mc & lt);
          wa += __popcll(ma);
          wc += __popcll(mc);
        }
        if (lane == 0) { sh.wcnt[buf][0][s][wave] = wa; sh.wcnt[buf][1][s][wave] = wc; }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < SUPER; ++s) {
        uint32_t beforeA = 0, beforeC = 0, totA = 0, totC = 0;
#pragma unroll
        for (int w = 0; w < SEL_WAVES; ++w) {
          const uint32_t xa = sh.wcnt[buf][0][s][w], xc = sh.wcnt[buf][1][s][w];
          beforeA += (w < wave) ? xa : 0u;
          beforeC += (w < wave) ? xc : 0u;
          totA += xa;
          totC += xc;
        }
        uint32_t oa = baseA + beforeA + ra[s], oc = baseC + beforeC + rc[s];
        const int64_t p0 = c0 + (int64_t)s * SUB + tid * EPT;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          if ((fa[s] >> e) & 1u) { if (oa < A_CAP) sh.listA[oa] = (int32_t)(p0 + e); ++oa; }
          if ((fc[s] >> e) & 1u) {
            if (oc < C_CAP) { sh.ckey[oc] = key[s][e]; sh.cpos[oc] = (int32_t)(p0 + e); }
            ++oc;
          }
        }
        baseA += totA;
        baseC += totC;
      }
#pragma unroll
      for (int s = 0; s < SUPER; ++s) cur[s] = nxt[s];
    }
    __syncthreads();

    // ---- resolve the threshold inside list C (LDS only)
    uint32_t T = 0;
    uint32_t needT = need;                 // keys equal to T to take (lowest positions)
    const bool take_all_c = (need == (uint32_t)cntC);
    if (!take_all_c) {
      uint32_t prefix = 0;                 // resolved bits 19..10 (as a 10-bit digit)
      for (int round = 0; round < 2; ++round) {
        const int shift = round == 0 ? 10 : 0;
        for (int i = tid; i < 1024; i += SEL_THREADS) sh.hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < cntC; i += SEL_THREADS) {
          const uint32_t key = sh.ckey[i];
          if (round == 0 || ((key >> 10) & 1023u) == prefix) atomicAdd(&sh.hist[(key >> shift) & 1023u], 1u);
        }
        __syncthreads();
        find_bucket(sh.hist, 1024, needT, sh);
        const uint32_t d = (uint32_t)sh.misc[0];
        needT -= (uint32_t)sh.misc[1];
        if (round == 0) prefix = d;
        else T = (b1 << HIST_SHIFT) | (prefix << 10) | d;
      }
    }

    // ---- compact C in place to the selected positions (position order kept)
    uint32_t baseS = 0, baseEq = 0;
    for (int c0 = 0; c0 < cntC; c0 += SUB) {
      const int i0 = c0 + tid * EPT;
      bool sel[EPT], eq[EPT];
      int32_t pos[EPT];
      uint32_t key[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const bool valid = i0 + e < cntC;
        key[e] = valid ? sh.ckey[i0 + e] : 0u;
        pos[e] = valid ? sh.cpos[i0 + e] : 0;
        eq[e] = valid && !take_all_c && key[e] == T;
      }
      uint32_t totEq;
      const uint32_t req = ballot_rank(eq, sh.wtot[0], &totEq);
      uint32_t r = baseEq + req;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const bool valid = i0 + e < cntC;
        if (take_all_c) sel[e] = valid;
        else if (eq[e]) { sel[e] = r < needT; ++r; }
        else sel[e] = valid && key[e] > T;
      }
      uint32_t totS;
      const uint32_t rs = ballot_rank(sel, sh.wtot[1], &totS);
      __syncthreads();     // every thread has read its C entries before any is overwritten
      uint32_t o = baseS + rs;
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (sel[e]) { if (o < C_CAP) sh.cpos[o] = pos[e]; ++o; }
      baseS += totS;
      baseEq += totEq;
      __syncthreads();
    }
    const int nS = kk - cntA;

    // ---- merge lists A (cntA) and C-selected (nS), both ascending, by rank
    for (int i = tid; i < cntA; i += SEL_THREADS) {
      const int32_t x = sh.listA[i];
      int lo = 0, hi = nS;
      while (lo < hi) { const int mid = (lo + hi) >> 1; if (sh.cpos[mid] < x) lo = mid + 1; else hi = mid; }
      if (i + lo < kk) out[i + lo] = x;
    }
    for (int i = tid; i < nS; i += SEL_THREADS) {
      const int32_t x = sh.cpos[i];
      int lo = 0, hi = cntA;
      while (lo < hi) { const int mid = (lo + hi) >> 1; if (sh.listA[mid] < x) lo = mid + 1; else hi = mid; }
      if (i + lo < kk) out[i + lo] = x;
    }
    return;
  }

  // ---- fallback: resolve the lower 20 bits with passes over the scores
  uint32_t prefix = b1 << HIST_SHIFT;
  uint32_t mask = 0xfff00000u;
  for (int round = 0; round < 2; ++round) {
    const int shift = round == 0 ? 10 : 0;
    for (int i = tid; i < 1024; i += SEL_THREADS) sh.hist[i] = 0u;
    __syncthreads();
    for (int64_t c = (int64_t)tid * EPT; c < n; c += SUB) {
      const f32x4 v = load4(row, c, last4);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint32_t key = score_key(v[e]);
        if (c + e < n && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 1023u], 1u);
      }
    }
    __syncthreads();
    find_bucket(sh.hist, 1024, need, sh);
    need -= (uint32_t)sh.misc[1];
    prefix |= (uint32_t)sh.misc[0] << shift;
    mask |= 1023u << shift;
  }
  const uint32_t T = prefix;
  const uint32_t needT = need;
  uint32_t baseS = 0, baseEq = 0;
  for (int64_t c0 = 0; c0 < n; c0 += SUB) {
    const int64_t p0 = c0 + tid * EPT;
    const f32x4 v = load4(row, p0, last4);
    bool eq[EPT], sel[EPT];
    uint32_t key[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      key[e] = score_key(v[e]);
      eq[e] = (p0 + e < n) && key[e] == T;
    }
    uint32_t totEq;
    const uint32_t req = ballot_rank(eq, sh.wtot[0], &totEq);
    uint32_t r = baseEq + req;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (eq[e]) { sel[e] = r < needT; ++r; }
      else sel[e] = (p0 + e < n) && key[e] > T;
    }
    uint32_t totS;
    const uint32_t rs = ballot_rank(sel, sh.wtot[1], &totS);
    uint32_t o = baseS + rs;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (sel[e]) { if (o < (uint32_t)kk) out[o] = (int32_t)(p0 + e); ++o; }
    baseS += totS;
    baseEq += totEq;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_select(const sjsa_shape& s, const Layout& L, const float* scores, int64_t stride,
                         const int32_t* seq_len, int k, int32_t* idx, unsigned char* ws, hipStream_t st) {
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.off_hist);
  const int have_hist = scores == nullptr ? 1 : 0;
  const float* src = scores ? scores : reinterpret_cast<const float*>(ws + L.off_scores);
  const int64_t sstride = scores ? stride : L.score_stride;
  select_kernel<<<dim3((unsigned)L.units), dim3(SEL_THREADS), 0, st>>>(
      src, sstride, seq_len, s.n_kv_heads, s.capacity, k, idx, hist, have_hist);
  return hipGetLastError();
}

}  // namespace sjsa

// Per-(sequence, KV head) top-k selection.
//
// Source: JSSA article, section JSSA 的整体结构 (top-k token positions per KV head,
// shared by its query heads) and section 组件级拆解 (top-k selection is the stage
// that dominates at small batch). Ranking: larger score first; equal scores go to
// the lower position; -0 equals +0; NaN ranks below everything. Output: the
// min(k, n) selected positions in ascending order, then -1.
//
// Scores are compared as order-preserving u32 keys. One 1024-thread workgroup per
// unit, three paths:
//  * take-all: k >= n, positions 0..n-1.
//  * candidates (the usual case): the scan kept, per tile and in position order,
//    every row whose key reached the unit's sampled threshold. If their count c
//    satisfies k <= c <= CAND_CAP (and no tile overflowed), the exact top k is
//    among them: the tiles are gathered into LDS in order, radix rounds over the
//    offsets key - (least candidate key), at most 12 bits each and usually two,
//    find the exact k-th key T and how many keys equal to T are taken (lowest
//    positions first), and one ordered ballot compaction writes the ascending
//    result.
//  * dense: exact selection over a full score row. Used for caller-provided
//    scores, and when the sampled threshold misjudged the distribution (fewer than
//    k candidates, more than fit in LDS, or more than a scan wave could stage);
//    the unit's scores are then recomputed first with arithmetic bit-identical to
//    the scan's. The first radix digit's histogram locates the bin b1 of the k-th
//    key; one ordered pass compacts the positions above b1 (list A) and the (key,
//    position) pairs in b1 (list C) into LDS; C is resolved exactly and merged with
//    A by rank. If A or C would not fit, the remaining digits are resolved by
//    passes over the row and a final ordered pass writes the result.
#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int EPT = 4;                          // consecutive positions per thread (one float4)
constexpr int SUB = SEL_THREADS * EPT;          // positions per sub-chunk
constexpr int STEPS = 4;                        // float4 loads per lane per super-chunk
constexpr int WAVE_SPAN = STEPS * 64 * EPT;     // contiguous positions per wave per super-chunk
constexpr int SUPER_SPAN = SEL_WAVES * WAVE_SPAN;
constexpr int LDS_WORDS = 32768;                // list storage (128 KB)
constexpr int A_CAP = 8192;                     // dense path: listA | ckey | cpos
constexpr int C_CAP = 12288;
constexpr int CAND_CAP = LDS_WORDS / 2;         // candidate path: ckey | cpos
static_assert(A_CAP + 2 * C_CAP == LDS_WORDS, "dense lists fill the list storage");

constexpr int HIST2_BINS = 2048;                // second histogram (candidate path, second radix digit)
constexpr int HIST1_BITS = 12;                  // candidate path: first digit of the relative keys
static_assert(1 << HIST1_BITS <= HIST_BINS && HIST1_BITS < CAND_KEY_BITS, "first digit fits sh.hist");

struct SelShared {
  uint32_t hist[HIST_BINS];
  uint32_t buf[LDS_WORDS];
  uint32_t hist2[HIST2_BINS];
  uint32_t toff[144];                // candidate path: tile output offsets of a chunk
  float qh[64];                      // candidate path: q_hat, for exact scores at the boundary
  uint32_t wtot[2][2 * SEL_WAVES];   // [buffer][A totals of waves | C totals of waves]
  uint32_t scan[SEL_WAVES];
  uint32_t scan2[SEL_WAVES];
  int32_t misc[8];
  uint32_t spare[64];                // hist_add's sink: one word per lane of a wave
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

// Given a histogram of `nbins` bins (LDS, nbins a power of two <= HIST_BINS) and
// 1 <= need <= total count, find the bin b with count(bins > b) < need <=
// count(bins >= b). Results: misc[0] = b, misc[1] = count above b, misc[2] = count
// in b. All threads call.
__device__ void find_bucket(const uint32_t* hist, int nbins, uint32_t need, SelShared& sh) {
  const int per = (nbins + SEL_THREADS - 1) / SEL_THREADS;     // 4, 1 or (small nbins) 1
  const int lo = threadIdx.x * per;
  const int cnt = max(0, min(per, nbins - lo));
  uint32_t local = 0;
  for (int i = 0; i < cnt; ++i) local += hist[lo + i];
  uint32_t total;
  const uint32_t inc = block_incl_scan(local, sh.scan, &total);
  uint32_t above = total - inc;                // keys in bins above this thread's range
  if (above < need && need <= above + local) {
    for (int i = cnt - 1; i >= 0; --i) {
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
// past n are clamped to the last float4 that starts inside the row (rows are
// allocated up to a multiple of 4) and are masked by the callers. Keeping every
// load unconditional lets the compiler overlap a whole batch of them.
__device__ __forceinline__ f32x4 load4(const float* row, int64_t pos, int64_t last4) {
  return *reinterpret_cast<const f32x4*>(row + min(pos, last4));
}

// Counts each lane with `on` into hist[bin] (LDS), one atomic per lane, with no
// branch (a branch in a loop that keeps loads in flight makes the compiler wait on
// them early). The counted lanes of the wave that share the bin of its first active
// lane add their number through the first of them; the other lanes add 0 to their
// own word of `spare`. Without this a run of equal keys (a constant score row,
// duplicated cache rows) sends every lane of every wave to one LDS address, where
// the atomics are done one at a time.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t* spare, uint32_t bin, bool on) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(bin);
  const bool in_same = on && bin == b0;
  const uint64_t same = __ballot(in_same);
  const uint32_t lead = same != 0 ? (uint32_t)__builtin_ctzll(same) : 64u;
  const bool counts = on && (!in_same || lane == lead);
  const uint32_t v = !counts ? 0u : (in_same ? (uint32_t)__popcll(same) : 1u);
  atomicAdd(counts ? &hist[bin] : &spare[lane], v);
}

// Ordered compaction helper: ranks of the flagged elements of one sub-chunk (each
// thread holds NE consecutive positions; lanes, then waves, are in position order).
// Returns this thread's first output slot relative to the sub-chunk start and the
// sub-chunk total (through per-wave totals in wtot_row). One barrier.
template <int NE>
__device__ __forceinline__ uint32_t ballot_rank(const bool (&f)[NE], uint32_t* wtot_row, uint32_t* total) {
  const int wave = threadIdx.x >> 6;
  const uint64_t lt = lanemask_lt();
  uint32_t below = 0, wave_cnt = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
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

// Exact resolution of the threshold inside an LDS key list: the keys all share the
// bits selected by `mask` (value `prefix`, the first 12-bit digit); `need` of them
// are to be taken. The remaining 20 bits are resolved 10 at a time. Returns T;
// *needT receives how many keys equal to T are taken.
__device__ uint32_t lds_threshold(const uint32_t* keys, int cnt, uint32_t prefix, uint32_t mask, uint32_t need,
                                  SelShared& sh, uint32_t* needT) {
  const int tid = threadIdx.x;
  for (int round = 0; round < 2; ++round) {
    const int shift = round == 0 ? 10 : 0;
    for (int i = tid; i < 1024; i += SEL_THREADS) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < cnt; i += SEL_THREADS) {
      const uint32_t key = keys[i];
      hist_add(sh.hist, sh.spare, (key >> shift) & 1023u, (key & mask) == prefix);
    }
    __syncthreads();
    find_bucket(sh.hist, 1024, need, sh);
    need -= (uint32_t)sh.misc[1];
    prefix |= (uint32_t)sh.misc[0] << shift;
    mask |= 1023u << shift;
  }
  *needT = need;
  return prefix;
}

// find_bucket with two barriers (the wave totals go through sh.scan2, which the
// next call rewrites only after two more barriers).
__device__ void find_bucket_fast(const uint32_t* hist, int nbins, uint32_t need, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (nbins + SEL_THREADS - 1) / SEL_THREADS;
  const int lo = threadIdx.x * per;
  const int cnt = max(0, min(per, nbins - lo));
  uint32_t local = 0;
  for (int i = 0; i < cnt; ++i) local += hist[lo + i];
  const uint32_t inc = wave_incl_scan(local);
  if (lane == 63) sh.scan2[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t t = sh.scan2[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  uint32_t above = tot - (inc + before);       // keys in bins above this thread's range
  if (above < need && need <= above + local) {
    for (int i = cnt - 1; i >= 0; --i) {
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

// Exact threshold of an LDS key list whose keys all lie in [kmin, kmax]: the keys
// are ranked by their offset key - kmin, whose significant bits are resolved from
// the top, 12 at a time in sh.hist and 11 in sh.hist2 for the second round (both
// must be zero on entry, so that the first two rounds need no clearing pass), so
// the first histogram spreads the keys over up to 4096 bins whatever part of the
// key range they occupy. With `prebuilt` the caller has already counted the keys
// into sh.hist by their top 12 bits of [kmin, kmax] (the first round's digit). When
// the bin holding rank `need` is taken whole, the
// threshold stops there. Returns T and *needT such that the selection is: keys
// above T, plus the first needT keys equal to T; *all_eq is set when that takes
// every key equal to T.
__device__ uint32_t lds_threshold_range(const uint32_t* keys, int cnt, uint32_t kmin, uint32_t kmax,
                                        uint32_t need, SelShared& sh, uint32_t* needT, bool* all_eq,
                                        bool prebuilt = false) {
  *all_eq = false;
  const int tid = threadIdx.x;
  int hi = 32 - __clz(kmax - kmin);           // significant bits of the offsets
  uint32_t prefix = 0;                        // resolved bits hi.. of the k-th offset
  for (int round = 0; hi > 0; ++round) {
    const bool second = round == 1;
    const int shift = max(hi - (second ? 11 : 12), 0);
    const int nb = 1 << (hi - shift);
    uint32_t* hist = second ? sh.hist2 : sh.hist;
    if (round >= 2) {                         // rare: a third round reuses sh.hist
      for (int i = tid; i < nb; i += SEL_THREADS) hist[i] = 0u;
      __syncthreads();
    }
    const uint64_t want = (uint64_t)prefix >> hi;
    if (!(prebuilt && round == 0)) {
      // KU keys per thread per batch: all their LDS reads are issued before any atomic
      constexpr int KU = 8;
      for (int i0 = tid; i0 < cnt; i0 += KU * SEL_THREADS) {
        uint32_t off[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) off[u] = keys[min(i0 + u * SEL_THREADS, cnt - 1)] - kmin;
#pragma unroll
        for (int u = 0; u < KU; ++u)
          if (i0 + u * SEL_THREADS < cnt && ((uint64_t)off[u] >> hi) == want)
            atomicAdd(&hist[(off[u] >> shift) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
    }
    find_bucket_fast(hist, nb, need, sh);
    const uint32_t bin = (uint32_t)sh.misc[0];
    const uint32_t above = (uint32_t)sh.misc[1];
    const uint32_t inbin = (uint32_t)sh.misc[2];
    need -= above;
    prefix |= bin << shift;
    hi = shift;
    if (hi > 0 && inbin == need) {            // every key of the bin is taken
      const uint32_t lo_key = kmin + prefix;  // smallest key the bin can hold
      if (lo_key == 0u) { *needT = 0xffffffffu; return 0u; }
      *needT = 0u;
      return lo_key - 1u;
    }
    if (hi == 0) *all_eq = inbin == need;     // the last bin holds one key value
  }
  *needT = need;
  return kmin + prefix;
}

// Ordered compaction of an LDS (key, position) list in position order: keep keys
// above T, and the first needT keys equal to T. With to_lds the kept positions are
// written back into pos_l[] (in place); otherwise to out[]. Returns the kept count.
constexpr int CEPT = 8;                         // list entries per thread per compaction pass
constexpr int CSUB = SEL_THREADS * CEPT;

__device__ uint32_t compact_list(const uint32_t* key_l, int32_t* pos_l, int cnt, uint32_t T, uint32_t needT,
                                 bool take_all, bool to_lds, int32_t* out, SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t baseS = 0, baseEq = 0;
  for (int c0 = 0; c0 < cnt; c0 += CSUB) {
    const int i0 = c0 + tid * CEPT;
    bool sel[CEPT], eq[CEPT];
    int32_t pos[CEPT];
    uint32_t key[CEPT];
#pragma unroll
    for (int e = 0; e < CEPT; ++e) {
      const bool valid = i0 + e < cnt;
      key[e] = valid ? key_l[i0 + e] : 0u;
      pos[e] = valid ? pos_l[i0 + e] : 0;
      eq[e] = valid && !take_all && key[e] == T;
    }
    uint32_t totEq;
    const uint32_t req = ballot_rank(eq, sh.wtot[0], &totEq);
    uint32_t r = baseEq + req;
#pragma unroll
    for (int e = 0; e < CEPT; ++e) {
      const bool valid = i0 + e < cnt;
      if (take_all) sel[e] = valid;
      else if (eq[e]) { sel[e] = r < needT; ++r; }
      else sel[e] = valid && key[e] > T;
    }
    uint32_t totS;
    const uint32_t rs = ballot_rank(sel, sh.wtot[1], &totS);
    __syncthreads();     // every thread has read its entries before any is overwritten
    uint32_t o = baseS + rs;
#pragma unroll
    for (int e = 0; e < CEPT; ++e) {
      if (sel[e]) {
        if (to_lds) pos_l[o] = pos[e];
        else out[o] = pos[e];
        ++o;
      }
    }
    baseS += totS;
    baseEq += totEq;
    __syncthreads();
  }
  return baseS;
}

// Ranks for a strided ordered compaction: element e of thread t in a pass is list
// entry e*SEL_THREADS + t, so consecutive lanes touch consecutive LDS words (no bank
// conflicts) and the list order is (e, wave, lane). A ballot per e gives the order
// inside a wave; the counts of every (e, wave) are scanned by wave 0 in that order.
// rank[e] receives the output slot of flagged element e relative to the pass start,
// *total the pass's flagged count. `table` needs NE*SEL_WAVES + 1 words. Two barriers.
template <int NE>
__device__ __forceinline__ void strided_rank(const bool (&f)[NE], uint32_t (&rank)[NE], uint32_t* table,
                                             uint32_t* total) {
  static_assert(NE * SEL_WAVES == 128, "wave 0 scans two counts per lane");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t lt = lanemask_lt();
  uint64_t m[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) m[e] = __ballot(f[e]);
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < NE; ++e) table[e * SEL_WAVES + wave] = (uint32_t)__popcll(m[e]);
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t a = table[2 * lane], c = table[2 * lane + 1];
    const uint32_t incl = wave_incl_scan(a + c);
    table[2 * lane] = incl - (a + c);
    table[2 * lane + 1] = incl - c;
    if (lane == 63) table[NE * SEL_WAVES] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NE; ++e) rank[e] = table[e * SEL_WAVES + wave] + (uint32_t)__popcll(m[e] & lt);
  *total = table[NE * SEL_WAVES];
}

// Ordered compaction of the candidate list: keep keys above T, and the first needT
// keys equal to T (all of them when all_eq). out[0 .. kept) receives the kept
// positions in list order (slots at or past `limit` are not written). Returns the
// kept count.
__device__ __forceinline__ uint32_t compact_candidates(const uint32_t* key_l, const int32_t* pos_l, int cnt, uint32_t T,
                                       uint32_t needT, bool all_eq, int32_t* out, uint32_t limit,
                                       SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t* table = sh.hist;
  uint32_t* table2 = sh.hist + 256;
  uint32_t baseS = 0, baseEq = 0;
  for (int c0 = 0; c0 < cnt; c0 += CSUB) {
    bool sel[CEPT], eq[CEPT];
    int32_t pos[CEPT];
#pragma unroll
    for (int e = 0; e < CEPT; ++e) {
      const int i = c0 + e * SEL_THREADS + tid;
      const bool valid = i < cnt;
      const uint32_t key = valid ? key_l[i] : 0u;
      pos[e] = valid ? pos_l[i] : 0;
      eq[e] = valid && key == T;
      sel[e] = valid && key > T;
    }
    if (all_eq) {
#pragma unroll
      for (int e = 0; e < CEPT; ++e) sel[e] = sel[e] || eq[e];
    } else if (needT > 0) {
      uint32_t req[CEPT], totEq;
      strided_rank(eq, req, table2, &totEq);
#pragma unroll
      for (int e = 0; e < CEPT; ++e) sel[e] = sel[e] || (eq[e] && baseEq + req[e] < needT);
      baseEq += totEq;
    }
    uint32_t rs[CEPT], totS;
    strided_rank(sel, rs, table, &totS);
#pragma unroll
    for (int e = 0; e < CEPT; ++e)
      if (sel[e] && baseS + rs[e] < limit) out[baseS + rs[e]] = pos[e];
    baseS += totS;
    // the next pass's strided_rank rewrites table only after its first barrier
  }
  return baseS;
}

// Exact top-kk of a dense score row of n >= kk >= 1 entries -> out[0..kk). With
// hist_ready the caller has already counted the row's keys by their top 12 bits into
// sh.hist (the first radix digit).
__device__ __forceinline__ void select_dense(const float* row, int64_t n, int kk, int32_t* out, SelShared& sh,
                                             bool hist_ready = false) {
  const int tid = threadIdx.x;
  const int64_t last4 = ((n - 1) >> 2) << 2;     // last float4 start inside the row
  int32_t* listA = reinterpret_cast<int32_t*>(sh.buf);
  uint32_t* ckey = sh.buf + A_CAP;
  int32_t* cpos = reinterpret_cast<int32_t*>(sh.buf + A_CAP + C_CAP);

  // first digit: histogram of the top 12 key bits
  if (!hist_ready) {
    for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = 0u;
    __syncthreads();
    constexpr int HU = 8;                         // float4 loads in flight per thread
    for (int64_t c0 = (int64_t)tid * EPT; c0 < n; c0 += (int64_t)SUB * HU) {
      f32x4 v[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u) v[u] = load4(row, c0 + (int64_t)u * SUB, last4);
#pragma unroll
      for (int u = 0; u < HU; ++u) {
#pragma unroll
        for (int e = 0; e < EPT; ++e)
          hist_add(sh.hist, sh.spare, score_key(v[u][e]) >> HIST_SHIFT, c0 + (int64_t)u * SUB + e < n);
      }
    }
    __syncthreads();
  }
  find_bucket(sh.hist, HIST_BINS, (uint32_t)kk, sh);
  const uint32_t b1 = (uint32_t)sh.misc[0];
  const int cntA = sh.misc[1];
  const int cntC = sh.misc[2];
  uint32_t need = (uint32_t)(kk - cntA);          // 1 <= need <= cntC

  if (cntA <= A_CAP && cntC <= C_CAP) {
    // Pass A: ordered compaction of lists A and C into LDS. A super-chunk is
    // SEL_WAVES * WAVE_SPAN positions; wave w owns the contiguous range
    // c0 + w*WAVE_SPAN .. +WAVE_SPAN, read as STEPS coalesced float4 loads per lane
    // (step i, lane l: positions +i*256 + 4l .. +3). Inside a wave, ballots give each
    // flagged element its rank in position order (step, lane, e); across waves the
    // per-wave totals are published once per super-chunk (double-buffered, one
    // barrier) and scanned by a DPP row scan read back with readlane. The next
    // super-chunk's loads are in flight while the current one is classified.
    uint32_t baseA = 0, baseC = 0;
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t lt = lanemask_lt();
    f32x4 cur[STEPS];
#pragma unroll
    for (int i = 0; i < STEPS; ++i) cur[i] = load4(row, (int64_t)wave * WAVE_SPAN + i * 256 + lane * EPT, last4);
    int it = 0;
    for (int64_t c0 = 0; c0 < n; c0 += SUPER_SPAN, ++it) {
      const int64_t wbase = c0 + (int64_t)wave * WAVE_SPAN;
      f32x4 nxt[STEPS];
#pragma unroll
      for (int i = 0; i < STEPS; ++i) nxt[i] = load4(row, wbase + SUPER_SPAN + i * 256 + lane * EPT, last4);
      const int buf = it & 1;
      uint32_t key[STEPS][EPT];
      uint32_t fa[STEPS], fc[STEPS];      // flag bits per element e
      uint32_t ra[STEPS], rc[STEPS];      // rank of this lane's first flagged element within the wave
      uint32_t wa = 0u, wc = 0u;          // wave totals so far
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        const int64_t p0 = wbase + i * 256 + lane * EPT;
        fa[i] = 0u;
        fc[i] = 0u;
        uint32_t la = 0u, lc = 0u, sa = 0u, sc = 0u;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          key[i][e] = score_key(cur[i][e]);
          const uint32_t bin = key[i][e] >> HIST_SHIFT;
          const bool valid = p0 + e < n;
          const bool a = valid && bin > b1;
          const bool c = valid && bin == b1;
          fa[i] |= (uint32_t)a << e;
          fc[i] |= (uint32_t)c << e;
          const uint64_t ma = __ballot(a), mc = __ballot(c);
          la += __popcll(ma & lt);
          lc += __popcll(mc & lt);
          sa += __popcll(ma);
          sc += __popcll(mc);
        }
        ra[i] = wa + la;
        rc[i] = wc + lc;
        wa += sa;
        wc += sc;
      }
      if (lane == 0) { sh.wtot[buf][wave] = wa; sh.wtot[buf][SEL_WAVES + wave] = wc; }
      __syncthreads();
      // lanes 0..15 scan the A totals of waves 0..15, lanes 16..31 the C totals
      const uint32_t scan = row16_incl_scan(lane < 32 ? sh.wtot[buf][lane] : 0u);
      const uint32_t totA = __builtin_amdgcn_readlane(scan, 15);
      const uint32_t totC = __builtin_amdgcn_readlane(scan, 31);
      const uint32_t beforeA = wave == 0 ? 0u : __builtin_amdgcn_readlane(scan, wave - 1);
      const uint32_t beforeC = wave == 0 ? 0u : __builtin_amdgcn_readlane(scan, 16 + wave - 1);
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        uint32_t oa = baseA + beforeA + ra[i], oc = baseC + beforeC + rc[i];
        const int64_t p0 = wbase + i * 256 + lane * EPT;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          if ((fa[i] >> e) & 1u) { if (oa < A_CAP) listA[oa] = (int32_t)(p0 + e); ++oa; }
          if ((fc[i] >> e) & 1u) {
            if (oc < C_CAP) { ckey[oc] = key[i][e]; cpos[oc] = (int32_t)(p0 + e); }
            ++oc;
          }
        }
      }
      baseA += totA;
      baseC += totC;
#pragma unroll
      for (int i = 0; i < STEPS; ++i) cur[i] = nxt[i];
    }
    __syncthreads();

    // resolve the threshold inside list C (LDS only) and keep the selected C entries
    const bool take_all_c = need == (uint32_t)cntC;
    uint32_t T = 0, needT = need;
    if (!take_all_c)
      T = lds_threshold(ckey, cntC, b1 << HIST_SHIFT, 0xfff00000u, need, sh, &needT);
    compact_list(ckey, cpos, cntC, T, needT, take_all_c, true, nullptr, sh);
    const int nS = kk - cntA;

    // merge lists A (cntA) and C-selected (nS), both ascending, by rank
    for (int i = tid; i < cntA; i += SEL_THREADS) {
      const int32_t x = listA[i];
      int lo = 0, hi = nS;
      while (lo < hi) { const int mid = (lo + hi) >> 1; if (cpos[mid] < x) lo = mid + 1; else hi = mid; }
      if (i + lo < kk) out[i + lo] = x;
    }
    for (int i = tid; i < nS; i += SEL_THREADS) {
      const int32_t x = cpos[i];
      int lo = 0, hi = cntA;
      while (lo < hi) { const int mid = (lo + hi) >> 1; if (listA[mid] < x) lo = mid + 1; else hi = mid; }
      if (i + lo < kk) out[i + lo] = x;
    }
    return;
  }

  // the lists would not fit: resolve the lower 20 bits with passes over the row
  // (HU float4 loads in flight per thread, as in the first digit's pass)
  constexpr int HU = 8;
  uint32_t prefix = b1 << HIST_SHIFT;
  uint32_t mask = 0xfff00000u;
  int rounds = 2;
  if (cntC > C_CAP) {
    // a crowded boundary bin: first its least and greatest keys. When they are equal
    // (a constant row, for one) that key is the threshold; when the bin is also the
    // whole row, every score ties and the selection is the first kk positions.
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int64_t c0 = (int64_t)tid * EPT; c0 < n; c0 += (int64_t)SUB * HU) {
      f32x4 v[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u) v[u] = load4(row, c0 + (int64_t)u * SUB, last4);
#pragma unroll
      for (int u = 0; u < HU; ++u) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          const uint32_t key = score_key(v[u][e]);
          const bool in = c0 + (int64_t)u * SUB + e < n && (key & mask) == prefix;
          kmin = in ? min(kmin, key) : kmin;
          kmax = in ? max(kmax, key) : kmax;
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if ((tid & 63) == 0) { sh.scan[tid >> 6] = kmin; sh.scan2[tid >> 6] = kmax; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < SEL_WAVES; ++w) { kmin = min(kmin, sh.scan[w]); kmax = max(kmax, sh.scan2[w]); }
    __syncthreads();
    if (kmin == kmax) {
      if (cntA == 0 && (int64_t)cntC == n) {
        for (int i = tid; i < kk; i += SEL_THREADS) out[i] = i;
        return;
      }
      prefix = kmin;
      rounds = 0;
    }
  }
  for (int round = 0; round < rounds; ++round) {
    const int shift = round == 0 ? 10 : 0;
    for (int i = tid; i < 1024; i += SEL_THREADS) sh.hist[i] = 0u;
    __syncthreads();
    for (int64_t c0 = (int64_t)tid * EPT; c0 < n; c0 += (int64_t)SUB * HU) {
      f32x4 v[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u) v[u] = load4(row, c0 + (int64_t)u * SUB, last4);
#pragma unroll
      for (int u = 0; u < HU; ++u) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          const uint32_t key = score_key(v[u][e]);
          hist_add(sh.hist, sh.spare, (key >> shift) & 1023u,
                   c0 + (int64_t)u * SUB + e < n && (key & mask) == prefix);
        }
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
  // ordered selection, one sub-chunk per step; each step first issues the next
  // sub-chunk's load, which is in flight while this one is ranked (a deeper queue
  // gains nothing: the loop's global stores make the compiler wait on every load at
  // its head)
  f32x4 next = load4(row, (int64_t)tid * EPT, last4);
  for (int64_t c0 = 0; c0 < n; c0 += SUB) {
    const int64_t p0 = c0 + tid * EPT;
    const f32x4 v = next;
    next = load4(row, p0 + SUB, last4);
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
    for (int e = 0; e < EPT; ++e) {
      if (sel[e]) { if (o < (uint32_t)kk) out[o] = (int32_t)(p0 + e); ++o; }
    }
    baseS += totS;
    baseEq += totEq;
    __syncthreads();
  }
}

// Recompute a unit's dense scores over rows [row0, row1) into row[] with the scan's
// lane layout and arithmetic, so every key is bit-identical to the scan's: a wave-wide
// 16-byte load covers 64 / LPR consecutive rows (LPR lanes per row), the chunk dots are
// summed by the same transposed reduction, after which each lane holds one row's score.
// Each wave keeps RU such groups of 64 rows in flight (LOADS loads per lane), and waves
// take consecutive 64*RU-row blocks in turn. The keys are also counted by their first
// radix digit (top 12 bits) into sh.hist, for select_dense. Scores are staged in the
// list storage (LDS) and written out once per STAGE rows with coalesced 16-byte stores:
// a store in the load loop would hold up the next loads, which wait on one in-order
// counter with it.
template <int R, int KB>
__device__ void recompute_scores(const unsigned char* kproj_unit, const float* qhat_unit, int64_t row0, int64_t row1,
                                 float* row, SelShared& sh) {
  constexpr int LPR = R * KB / 16;                 // lanes per projected row (16 bytes each)
  constexpr int VPC = 16 / KB;                     // values per 16-byte chunk
  constexpr int RPL = 64 / LPR;                    // rows per wave-wide load
  constexpr int LOADS = KB == 2 ? 16 : 8;          // 16-byte loads in flight per lane (FP8: its
                                                   // decode needs more registers)
  constexpr int RU = LPR >= LOADS ? 1 : LOADS / LPR;   // 64-row groups in flight per wave
  constexpr int STEP = SEL_WAVES * RU * 64;        // rows of one pass of all waves
  constexpr int STAGE = LDS_WORDS;                 // rows staged in LDS between writes
  static_assert(STAGE % STEP == 0, "a stage holds whole passes");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = lane % LPR, rs = lane / LPR;
  float* stage = reinterpret_cast<float*>(sh.buf);
  float qh[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) qh[e] = qhat_unit[p * VPC + e];
  for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = 0u;
  __syncthreads();
  const unsigned char* base = kproj_unit + p * 16;
  const int64_t last = row1 - 1;
  for (int64_t s0 = row0; s0 < row1; s0 += STAGE) {
    const int64_t s1 = min(s0 + STAGE, row1);
    for (int64_t g0 = s0 + (int64_t)wave * RU * 64; g0 < s1; g0 += STEP) {
      u32x4 w[RU][LPR];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
#pragma unroll
        for (int i = 0; i < LPR; ++i)              // rows past the range read its last row
          w[u][i] = ld16_stream(base + (size_t)min(g0 + u * 64 + i * RPL + rs, last) * R * KB);
      }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        float d[LPR];
#pragma unroll
        for (int i = 0; i < LPR; ++i) d[i] = dot_chunk<KB>(qh, w[u][i]);
        const float sc = transpose_reduce<LPR>(d, p);
        const int64_t j = g0 + u * 64 + p * RPL + rs;
        if (j < s1) stage[j - s0] = sc;
        hist_add(sh.hist, sh.spare, score_key(sc) >> HIST_SHIFT, j < s1);
      }
    }
    __syncthreads();
    // the staged scores to row[s0, s1): 16-byte stores where the row is 16-byte aligned
    // (s0 is a multiple of 4096 and the row starts 256-byte aligned), then the tail
    const int len = (int)(s1 - s0);
    const int len4 = len & ~3;
    for (int i = tid * 4; i < len4; i += SEL_THREADS * 4)
      *reinterpret_cast<f32x4*>(row + s0 + i) = *reinterpret_cast<const f32x4*>(stage + i);
    for (int i = len4 + tid; i < len; i += SEL_THREADS) row[s0 + i] = stage[i];
    __syncthreads();
  }
}

// grid = (B * H_kv, parts). scores != nullptr (parts = 1): dense selection over caller
// scores (stride `stride`). Otherwise (1 <= parts <= EXACT_WGS, see select_parts):
// take-all, the candidate path (part 0 alone), or the exact path: every part recomputes
// its share of the unit's scores and the last part to finish runs the dense selection.
template <int R, int KB>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const float* __restrict__ scores, int64_t stride, const int32_t* __restrict__ seq_len,
    int n_kv_heads, int64_t cap, int k, int32_t* __restrict__ idx, const unsigned char* __restrict__ kproj,
    const float* __restrict__ qhat, const uint32_t* __restrict__ tlow, const uint32_t* __restrict__ cand,
    const uint64_t* __restrict__ counts, float* __restrict__ dense, int64_t dense_stride, int64_t ntile_cap,
    int64_t cand_stride, uint32_t* __restrict__ epoch, uint32_t* __restrict__ arrive,
    uint32_t* __restrict__ parthist) {
  __shared__ SelShared sh;
  const int unit = blockIdx.x;
  const int part = blockIdx.y;                    // 0: the unit's selector; > 0: exact-path helpers
  const int b = unit / n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // Candidates. Scan tile x (rows [x*TR, +TR)) left its candidates, in
  // position order, at entries [x*TR, ...) as (the key relative to the
  // threshold, cand_rel, in CAND_KEY_BITS bits; the row offset in the tile); counts[x]
  // holds their number (TILE_OVERFLOW when it could not keep them all) and their
  // greatest key. Every candidate key is at least the scan's threshold key, so no
  // relative key wraps. The gather counts the relative keys by their first digit as
  // it places them. Tiles are
  // gathered in chunks of CHUNK_T; wave w owns TPW consecutive tiles of a chunk and
  // loads their first SPEC*64 entries unconditionally (entries past the count are
  // never used) together with the counts, so one memory round trip serves a chunk
  // (64 tiles of 2048 rows, or 32 of 4096, cover a 131072-row sequence).
  // The first chunk's loads are issued before the sequence length is known (tiles
  // clamped to the capacity), so they overlap the kernel's first load; later chunks
  // clamp to the sequence.
  constexpr int TR = tile_rows(R * KB);
  constexpr int TPW = 8192 / TR;
  constexpr int SPEC = TR >= 4096 ? 5 : (TR >= 2048 ? 3 : 2);
  constexpr int CHUNK_T = SEL_WAVES * TPW;
  const uint64_t* cnt_u = counts + (size_t)unit * ntile_cap;
  const uint32_t* cand_u = cand + (size_t)unit * cand_stride;
  uint64_t cw = 0;
  uint32_t v[TPW][SPEC];
  auto load_chunk = [&](int64_t t0, int64_t tiles) {
    cw = cnt_u[min(t0 + min(tid, CHUNK_T - 1), tiles - 1)];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t t = min(t0 + wave * TPW + i, tiles - 1);
#pragma unroll
      for (int e = 0; e < SPEC; ++e) v[i][e] = __builtin_nontemporal_load(cand_u + t * TR + 64 * e + lane);
    }
  };
  const bool cand_path = scores == nullptr;
  const bool helper = part > 0;
  uint32_t tkey = 0, tshift = 0;
  if (cand_path && !helper) {
    // one more step of this unit done on this workspace: the next prep publishes
    // under a new tag
    if (tid == 0) epoch[unit] += 1u;
    tkey = tlow[unit * 2];
    tshift = tlow[unit * 2 + 1] >> TLOW_SHIFT_POS;
    load_chunk(0, (cap + TR - 1) / TR);            // the scan's tiles at capacity
    if (tid < R) sh.qh[tid] = qhat[(size_t)unit * QHAT_STRIDE + tid];
    if (tid == 0) sh.misc[6] = 0;                 // boundary entry counter (read after many barriers)
  }

  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int kk = (int)min((int64_t)k, n);
  int32_t* out = idx + (size_t)unit * k;

  if (!helper)
    for (int i = kk + tid; i < k; i += SEL_THREADS) out[i] = -1;
  if (kk == 0) return;
  if (!cand_path) {
    select_dense(scores + (size_t)unit * stride, n, kk, out, sh);
    return;
  }
  if ((int64_t)kk == n) {
    if (!helper)
      for (int i = tid; i < kk; i += SEL_THREADS) out[i] = i;
    return;
  }
  const int64_t ntiles = (n + TR - 1) / TR;
  // a tile that could not keep its candidates counts OVF_MARK in the chunk's scan (a
  // tile holds at most TR candidates, so a chunk's marks and counts cannot collide)
  constexpr uint32_t OVF_MARK = 1u << 24;
  static_assert(CHUNK_T * TR < OVF_MARK && (uint64_t)CHUNK_T * OVF_MARK < (1ull << 32), "marks apart");
  uint32_t total = 0;
  bool exact = false;                             // block-uniform: take the exact path
  if (helper) {
    // the same decision as part 0's gather, from the count words alone: the exact path
    // when a tile overflowed, or the candidates exceed the lists or fall short of kk
    for (int64_t t0 = 0; t0 < ntiles && !exact; t0 += CHUNK_T) {
      const bool own = tid < CHUNK_T && t0 + tid < ntiles;
      const uint32_t c = own ? (uint32_t)cnt_u[t0 + tid] : 0u;
      uint32_t chunk_total;
      block_incl_scan(c == TILE_OVERFLOW ? OVF_MARK : c, sh.scan, &chunk_total);
      if (chunk_total >= OVF_MARK || total + chunk_total > (uint32_t)CAND_CAP) exact = true;
      total += chunk_total;
    }
    if (!exact && total >= (uint32_t)kk) return;   // part 0 selects from the candidates
  }

  uint32_t* ckey = sh.buf;
  int32_t* cpos = reinterpret_cast<int32_t*>(sh.buf + CAND_CAP);
  uint32_t* toff = sh.toff;                       // CHUNK_T + 1 output offsets
  static_assert(CHUNK_T + 1 <= 144, "toff holds a chunk's offsets");
  // the threshold's first two histograms start from zero
  for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = 0u;
  for (int i = tid; i < HIST2_BINS; i += SEL_THREADS) sh.hist2[i] = 0u;
  for (int64_t t0 = 0; t0 < ntiles && !helper; t0 += CHUNK_T) {
    if (t0 > 0) load_chunk(t0, ntiles);
    const uint32_t c = (uint32_t)cw;
    const bool own = tid < CHUNK_T && t0 + tid < ntiles;
    uint32_t chunk_total;
    const uint32_t incl = block_incl_scan(own ? (c == TILE_OVERFLOW ? OVF_MARK : c) : 0u, sh.scan, &chunk_total);
    // an overflowed tile, or more candidates than the lists hold: the exact path,
    // decided from the counts alone, before any candidate is placed
    if (chunk_total >= OVF_MARK || total + chunk_total > (uint32_t)CAND_CAP) {
      exact = true;
      break;
    }
    if (tid < CHUNK_T) toff[tid + 1] = incl;
    if (tid == 0) toff[0] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tl = wave * TPW + i;
      const uint32_t o = toff[tl];
      const uint32_t ct = toff[tl + 1] - o;       // 0 for tiles past the end
#pragma unroll
      for (int e = 0; e < SPEC; ++e) {
        const uint32_t j = (uint32_t)(64 * e + lane);
        const uint32_t dst = total + o + j;
        if (j < ct && dst < (uint32_t)CAND_CAP) {
          ckey[dst] = v[i][e] >> CAND_ROW_BITS;
          cpos[dst] = (int32_t)((t0 + tl) * TR + (v[i][e] & CAND_ROW_MASK));
          atomicAdd(&sh.hist[v[i][e] >> (32 - HIST1_BITS)], 1u);
        }
      }
      for (uint32_t j = SPEC * 64 + lane; j < ct; j += 64) {     // tiles with many candidates
        const uint32_t dst = total + o + j;
        if (dst < (uint32_t)CAND_CAP) {
          const uint32_t x = __builtin_nontemporal_load(cand_u + (t0 + tl) * TR + j);
          ckey[dst] = x >> CAND_ROW_BITS;
          cpos[dst] = (int32_t)((t0 + tl) * TR + (x & CAND_ROW_MASK));
          atomicAdd(&sh.hist[x >> (32 - HIST1_BITS)], 1u);
        }
      }
    }
    total += chunk_total;
    __syncthreads();
  }

  if (!helper && !exact && total >= (uint32_t)kk) {
    // threshold on the relative keys over their whole range [0, CAND_REL_MAX]: the
    // gather has counted them by their top HIST1_BITS bits already
    uint32_t needT;
    bool all_eq;
    uint32_t T = lds_threshold_range(ckey, (int)total, 0u, CAND_REL_MAX, (uint32_t)kk, sh, &needT, &all_eq, true);
    if (needT == 0xffffffffu) all_eq = true;
    const unsigned char* kp_unit = kproj + (size_t)unit * cap * R * KB;
    int nb = 0;                                   // entries on the boundary relative key T
    if (!all_eq && needT > 0) {
      // only some entries of the boundary relative key T are taken: list them
      uint32_t* bidx = sh.hist2;
      for (int i = tid; i < (int)total; i += SEL_THREADS)
        if (ckey[i] == T) {
          const int at = atomicAdd(&sh.misc[6], 1);
          if (at < HIST2_BINS) bidx[at] = (uint32_t)i;
        }
      __syncthreads();
      nb = sh.misc[6];
    }
    if (!all_eq && needT > 0 && nb <= 64) {
      // few boundary entries (the usual case): wave 0 recomputes their exact keys
      // (arithmetic bit-identical to the scan) and ranks them (larger key first, then
      // lower list index, i.e. lower position); the taken ones are lifted above T
      if (wave == 0) {
        const uint32_t* bidx = sh.hist2;
        int li = 0x7fffffff;
        uint32_t ex = 0u;
        if (lane < nb) {
          li = (int)bidx[lane];
          ex = score_key(row_score<R, KB>(sh.qh, kp_unit + (size_t)cpos[li] * R * KB));
        }
        uint32_t rank = 0;
        for (int j = 0; j < nb; ++j) {
          const uint32_t exj = readlane_u32(ex, j);
          const int lij = (int)readlane_u32((uint32_t)li, j);
          rank += (exj > ex || (exj == ex && lij < li)) ? 1u : 0u;
        }
        if (lane < nb && rank < needT) ckey[li] = T + 1u;
      }
      __syncthreads();
      needT = 0;                                  // keep the keys above T
    } else if (!all_eq && needT > 0 && T < CAND_REL_MAX) {
      // many boundary entries: recompute their exact keys and rank on full keys, each
      // entry's key becoming (relative key, the exact key's offset inside the boundary's
      // 2^shift-key range scaled to CAND_ROW_BITS bits, or 0 off the boundary)
      for (int i = tid; i < (int)total; i += SEL_THREADS) {
        const uint32_t kt = ckey[i];
        uint32_t low = 0;
        if (kt == T) {
          const uint32_t ex = score_key(row_score<R, KB>(sh.qh, kp_unit + (size_t)cpos[i] * R * KB));
          low = ((ex - tkey - (T << tshift)) & ((1u << tshift) - 1u)) << (CAND_ROW_BITS - tshift);
        }
        ckey[i] = (kt << CAND_ROW_BITS) | low;
      }
      for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = 0u;
      for (int i = tid; i < HIST2_BINS; i += SEL_THREADS) sh.hist2[i] = 0u;
      __syncthreads();
      const uint32_t lo = T << CAND_ROW_BITS;
      T = lds_threshold_range(ckey, (int)total, lo, lo | CAND_ROW_MASK, needT, sh, &needT, &all_eq);
    } else if (!all_eq && needT > 0) {
      // many boundary entries on the saturated relative key (their exact keys may lie
      // anywhere above its range): those entries take their exact keys, every other
      // entry 0, below them all (entries under the boundary are never taken, and none
      // lies above it); the needT largest exact keys are then taken, equal keys by
      // list order, i.e. by position
      for (int i = tid; i < (int)total; i += SEL_THREADS)
        ckey[i] = ckey[i] == T ? score_key(row_score<R, KB>(sh.qh, kp_unit + (size_t)cpos[i] * R * KB)) : 0u;
      for (int i = tid; i < HIST_BINS; i += SEL_THREADS) sh.hist[i] = 0u;
      for (int i = tid; i < HIST2_BINS; i += SEL_THREADS) sh.hist2[i] = 0u;
      __syncthreads();
      T = lds_threshold_range(ckey, (int)total, 0u, 0xffffffffu, needT, sh, &needT, &all_eq);
      if (needT == 0xffffffffu) all_eq = true;
    }
    // compact in place in LDS, then write the result with coalesced stores
    compact_candidates(ckey, cpos, (int)total, T, needT, all_eq, out, (uint32_t)kk, sh);
    return;
  }
  // Exact path (the sampled threshold misjudged this unit, a scan tile overflowed, or
  // k exceeds the candidate lists): every part recomputes its share of the unit's
  // scores (bit-identical to the scan) into the dense row and counts their first radix
  // digit; the part that finishes last adds the other parts' counts and selects over
  // the whole row. The hand-over is an arrival counter (reset by the prep each step):
  // each part's stores are released before it arrives, and the last one acquires
  // them, so no part ever waits for another.
  float* row = dense + (size_t)unit * dense_stride;
  const int parts = (int)gridDim.y;
  const int64_t blk = (int64_t)SEL_THREADS * 4;  // part boundaries on 4096-row multiples
  const int64_t nblk = (n + blk - 1) / blk;
  const int64_t r0 = min(n, nblk * part / parts * blk), r1 = min(n, nblk * (part + 1) / parts * blk);
  recompute_scores<R, KB>(kproj + (size_t)unit * cap * R * KB, qhat + (size_t)unit * QHAT_STRIDE, r0, r1, row, sh);
  if (parts > 1) {
    uint32_t* ph = parthist + ((size_t)unit * parts + part) * HIST_BINS;
    for (int i = tid; i < HIST_BINS; i += SEL_THREADS) ph[i] = sh.hist[i];
    // the workgroup's rows and counts, made visible to thread 0 by the barrier, are
    // released at agent scope by thread 0's fence (one L2 write-back per workgroup)
    // before it arrives; the last part's thread 0 acquires them, and the barrier
    // passes them on to its other threads
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t before = atomicAdd(arrive + unit, 1u);
      if (before == (uint32_t)parts - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      sh.misc[7] = (int32_t)before;
    }
    __syncthreads();
    if (sh.misc[7] != parts - 1) return;          // another part is still recomputing
    for (int i = tid; i < HIST_BINS; i += SEL_THREADS) {
      uint32_t c = sh.hist[i];
      for (int q = 0; q < parts; ++q)
        if (q != part) c += parthist[((size_t)unit * parts + q) * HIST_BINS + i];
      sh.hist[i] = c;
    }
    __syncthreads();
  }
  select_dense(row, n, kk, out, sh, true);
}

// Workgroups per unit of the selection launch: the selector, and exact-path helpers.
// On the candidate path a helper only reads its unit's count words and exits: free
// while the selectors (one per unit, each filling a CU's LDS) leave CUs idle, which run
// the helpers in short rounds beside them, but extra rounds after the selectors once
// these fill the GPU (512 units of the 128K decode step: 35 us with three helpers per
// unit, 27 us with none). So a unit gets as many helpers as about three rounds on the
// idle CUs hold: all EXACT_WGS - 1 up to half as many units as CUs, none from one unit
// per CU on (the exact path then recomputes the unit in one workgroup).
int select_parts(int64_t units) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return EXACT_WGS;                            // the error is reported after the launch
  if (units >= cus) return 1;
  const int64_t p = 1 + 3 * (cus - units) / units;
  return (int)(p < EXACT_WGS ? p : EXACT_WGS);
}

}  // namespace

hipError_t launch_select(const sjsa_shape& s, const Layout& L, const float* scores, int64_t stride,
                         const void* kproj, const int32_t* seq_len, int k, int32_t* idx, unsigned char* ws,
                         hipStream_t st) {
  const float* qhat = reinterpret_cast<const float*>(ws + L.off_qhat);
  const uint32_t* cand = reinterpret_cast<const uint32_t*>(ws + L.off_cand);
  const uint64_t* counts = reinterpret_cast<const uint64_t*>(ws + L.off_counts);
  const uint32_t* tlow = reinterpret_cast<const uint32_t*>(ws + L.off_tlow);
  float* dense = reinterpret_cast<float*>(ws + L.off_scores);
  uint32_t* epoch = reinterpret_cast<uint32_t*>(ws + L.off_epoch);
  uint32_t* arrive = reinterpret_cast<uint32_t*>(ws + L.off_arrive);
  uint32_t* parthist = reinterpret_cast<uint32_t*>(ws + L.off_parthist);
  const dim3 grid((unsigned)L.units, scores ? 1u : (unsigned)select_parts(L.units)), block(SEL_THREADS);
  const unsigned char* kp = static_cast<const unsigned char*>(kproj);
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
#define SJSA_SEL(RR, KB)                                                                                \
  select_kernel<RR, KB><<<grid, block, 0, st>>>(scores, stride, seq_len, s.n_kv_heads, s.capacity, k, idx, \
                                                kp, qhat, tlow, cand, counts, dense, L.score_stride,      \
                                                L.ntile_cap, L.cand_stride, epoch, arrive, parthist)
  switch (s.rank) {
    case 16: if (fp8) SJSA_SEL(16, 1); else SJSA_SEL(16, 2); break;
    case 32: if (fp8) SJSA_SEL(32, 1); else SJSA_SEL(32, 2); break;
    case 64: if (fp8) SJSA_SEL(64, 1); else SJSA_SEL(64, 2); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_SEL
  return hipGetLastError();
}

}  // namespace sjsa

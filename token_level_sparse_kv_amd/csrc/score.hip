// Scoring prep and the full-context score scan.
//
// Source: JSSA article, section 打分误差的定义: selection uses the mean query of
// the G query heads of a KV head, and the projected score of key k is
// s_hat = q_bar^T M^T M k = (M q_bar) . (M k) = q_hat . Kproj_j. Section 原理详解(二)
// notes that scoring still scans every candidate position; only the attention
// becomes sparse. Section 组件级拆解 names the stages: scoring prep, candidate
// scoring, top-k selection, sparse attention.
//
// prep  (one workgroup per (b, h)): q_bar in fp32 (sum in head order, then divide
//       by G), q_hat = M_h q_bar (fp32), and the unit's candidate threshold, placed
//       from the scores of sample rows (one adjacent pair in each of 1024 strata).
// scan  (one workgroup per tile of a unit, about 128 KB of rows): streams Kproj rows with
//       128-bit coalesced loads, each lane holding 8 of a row's r values; the
//       partial dots of the r/8 lanes of a row are reduced with DPP lane moves in a
//       transposed pattern, so that after the reduction each lane owns the full
//       score of one row. Rows whose score key reaches the threshold are kept as
//       candidates for the top-k stage (and, on request, every score is stored).
//
// The two run as separate kernels (prep_kernel, score_kernel) or as one
// (prep_scan_kernel): its first B*H_kv workgroups do the prep of one unit each and
// publish q_hat, the threshold and the appended token's projected row as tagged
// 64-bit words; the scan workgroups read q_hat as soon as it is published, stream
// and score their whole tile, and only then need the threshold, so the prep runs
// under the scan's memory stream instead of before it.
#include "key_proj.h"

namespace sjsa {
namespace {

constexpr int SCORE_THREADS = 256;
constexpr int SCORE_WAVES = SCORE_THREADS / 64;
constexpr int GROUP_ROWS = 64;       // rows covered by r/8 wave-wide 16-byte loads
constexpr int SCORE_UNROLL = 2;      // groups per segment
constexpr int SEGS_MAX = TILE_ROWS_MAX / SEG_ROWS;
constexpr int STASH = TILE_ROWS_MAX / SCORE_WAVES;    // keys of one wave's rows of a tile
// rows scored by the prep to place the threshold: more samples give a tighter
// threshold (fewer candidates) but cost the prep about as much time as the later
// stages save (measured with 4096 at the 128K batch-16 shape)
constexpr int PREP_SAMPLES = 2048;
// Sample batches per load pass: one for bf16 rows (two make the fused kernel spill at 8
// waves per SIMD) and for FP8 rows of rank 64 (spills at 6 waves); two for FP8 rows of
// rank 16 or 32, whose fused kernel runs at 7 waves with registers to spare, which at
// small batch, where the prep's chain of sample loads decides the launch, took the step
// from 45-47 to 43 us at batch 1 and from 51 to 49 us at batch 2.
template <int R, int KB>
constexpr int prep_pass() { return KB == 1 && R <= 32 ? 2 : 1; }
constexpr int PREP_BINS = 4096;      // linear score bins of the threshold histogram
constexpr uint32_t TAG_MULT = 0x9E3779B1u;
constexpr uint32_t TAG_ADD = 0x7F4A7C15u;
// A scan wave waits at most sjsa_shape.fused_wait_us for a published word (200 us
// when the field is 0, far above a prep's duration); past it the tile reports
// TILE_OVERFLOW and the selection recomputes the unit exactly. The device's
// real-time counter runs at 100 MHz.
constexpr int32_t DEFAULT_WAIT_US = 200;
constexpr uint64_t TICKS_PER_US = 100;

static_assert(SEG_ROWS == GROUP_ROWS * SCORE_UNROLL, "one wave iteration covers one segment");
static_assert(SEGS_MAX <= 64, "one wave scans the segment counts");

// Tag of the words one launch publishes for a unit: a function of the unit's step
// count on this workspace, which the selection that follows every fused launch
// advances by one, so words left by the previous launch (or an earlier replay of a
// captured graph) never carry the current tag. Distinct counts give distinct tags.
__device__ __forceinline__ uint32_t launch_tag(const uint32_t* epoch, int unit) {
  return (epoch[unit] + 1u) * TAG_MULT + TAG_ADD;
}

__device__ __forceinline__ void publish(uint64_t* w, uint32_t tag, uint32_t v) {
  __hip_atomic_store(w, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide wait for tagged words: lane l < nw reads w[l] until every one of them
// carries `tag` (its value then goes to v) or `deadline` passes (returns false; the
// outcome is uniform over the wave).
__device__ __forceinline__ bool poll_words(const uint64_t* w, int nw, uint32_t tag, uint64_t deadline,
                                           uint32_t& v) {
  const int lane = threadIdx.x & 63;
  for (;;) {
    const uint64_t x = lane < nw ? __hip_atomic_load(w + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : (uint64_t)tag << 32;
    if (!__any((uint32_t)(x >> 32) != tag)) {
      v = (uint32_t)x;
      return true;
    }
    if (__builtin_readsteadycounter() > deadline) return false;
    __builtin_amdgcn_s_sleep(8);
  }
}

struct PrepShared {
  uint32_t hist[PREP_BINS];
  uint32_t qraw[8][64];      // the G query rows (bf16 pairs)
  float qh[64];
  float red[2 * SCORE_WAVES];
  uint32_t scan[SCORE_WAVES];
  uint32_t misc[4];
  uint32_t row[32];          // the appended token's projected row
};

struct ScanShared {
  uint32_t stash[SCORE_WAVES][STASH];   // a wave's keys, then its candidates (compacted in place)
  uint32_t segcnt[SEGS_MAX];
  uint32_t segoff[SEGS_MAX + 1];
  uint32_t sstart[SEGS_MAX];
  uint32_t overflow[SCORE_WAVES];
  uint32_t wmax[SCORE_WAVES];
  alignas(16) uint32_t words[SCORE_WAVES][64];  // published words, as each wave read them
};

union ScoreShared {
  PrepShared p;
  ScanShared s;
};

// Block-wide (SCORE_THREADS) inclusive scan of one u32 per thread; the block total
// goes to *total. Two barriers.
__device__ uint32_t prep_block_scan(uint32_t v, uint32_t* scan_lds, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) scan_lds[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SCORE_WAVES; ++w) {
    const uint32_t t = scan_lds[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return inc + before;
}

// MurmurHash3's 32-bit finalizer (fmix32): a bijective avalanche mix of a 32-bit word.
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// Row of sample s (0 <= s < min(NS, n)): every row when n <= NS; else the samples
// come in adjacent pairs (2j, 2j + 1 share a 128-byte cache line whenever a projected
// row is at most 64 bytes), one pair in each of NS/2 equal strata of the sequence
// (stratum i holds the pairs floor(i n / NS) .. floor((i+1) n / NS) - 1), at an offset
// inside its stratum drawn from `seed` (which changes from unit to unit and step to
// step): stratified like evenly spaced samples, but a fixed arrangement of the keys
// cannot keep its largest scores out of the sample step after step.
template <int NS>
__device__ __forceinline__ int64_t sample_row(int s, int64_t n, uint32_t seed) {
  if (n <= NS) return s;
  const int64_t i = s >> 1;
  const int64_t a = (i * n) / NS, w = ((i + 1) * n) / NS - a;      // w >= 1 pairs in the stratum
  const uint32_t h = fmix32(seed ^ ((uint32_t)i * 0x9E3779B9u));
  const int64_t j = (int64_t)(((uint64_t)h * (uint64_t)w) >> 32);  // uniform in [0, w)
  return 2 * (a + j) + (s & 1);
}

struct PrepArgs {
  const uint16_t* q;
  const float* M;
  const unsigned char* kproj;
  const int32_t* seq_len;
  int k;
  float* qhat;
  uint32_t* tlow;
  uint32_t* arrive;           // the unit's exact-path arrival counter, reset here each step
  const uint32_t* epoch;      // the unit's step count (seeds the sample positions)
  int n_kv_heads;
  int group;
  int64_t cap;
};

// Prep of one unit (b, h), 256 threads.
//  * q_bar in fp32 (sum in head order, then divide by G) and q_hat = M_h q_bar: output
//    i is split over 16 lanes of 8 channels each (fp32 partial dots, DPP row sum).
//  * Threshold for the scan: the scores of NS rows (pairs of adjacent rows, one pair
//    per stratum at a drawn offset, see sample_row; all rows when n <= NS) are
//    binned linearly between their least and
//    greatest finite value (+inf in the top bin, -inf and NaN left out); the bin
//    that holds the sample of rank m (see below) is found, and the least key in it
//    becomes the unit's candidate threshold, so at least m samples reach it. The
//    exact top k is among the rows that reach it unless the sample misjudges the
//    distribution, a case the select stage detects and handles exactly: the
//    threshold only decides how much work the select stage does, never its result.
//  * tlow[2u + 1]: bit 0 set when k >= n (every position is selected; the scan has no
//    work); bits TLOW_SHIFT_POS.. the shift of the candidates' relative keys (see
//    cand_rel), set so that the sampled keys' range above the threshold fills them.
// With APPEND the unit's new token (decode: one token per sequence at slot pos[b]) is
// appended first: threads 0..31 copy its K and V rows and all threads compute its
// projected row with the KeyProj layout (bit-identical to the append kernel). A sample
// that lands on that slot may read the row before or after the write; either way only
// the threshold moves, never the result.
// PUBLISH: q_hat, the appended row and the threshold are also published as tagged
// words (sync) for the scan workgroups of the same launch.
template <int R, int KB, bool APPEND, bool PUBLISH>
__device__ __forceinline__ void prep_body(PrepShared& sh, int unit, const PrepArgs& a, const PrepAppend& ap,
                                          uint64_t* sync, uint32_t tag) {
  constexpr int LPR = R * KB / 16;                    // 16-byte words per Kproj row
  constexpr int VPC = 16 / KB;                        // values per 16-byte word
  constexpr int RPL = 64 / LPR;                       // samples per wave-wide load
  constexpr int NS = PREP_SAMPLES;
  constexpr int BATCHES = NS / SCORE_THREADS;         // 64-sample batches per wave (= samples per lane)
  constexpr int OUTS = R * 16 / SCORE_THREADS;        // q_hat outputs per thread
  constexpr int RW = R * KB / 4;                      // 32-bit words of a projected row
  constexpr int PREP_PASS = prep_pass<R, KB>();
  static_assert(BATCHES % PREP_PASS == 0 && R * 16 % SCORE_THREADS == 0, "prep work divides evenly");
  const int b = unit / a.n_kv_heads;
  const int h = unit - b * a.n_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t* sw = sync + (size_t)unit * SYNC_WORDS;

  // the query rows: thread (g, part) of the first 128 loads 16 bytes of head g (heads
  // past G repeat the last; they are never read)
  const int part = tid & 15;
  u32x4 qw = {0u, 0u, 0u, 0u};
  if (tid < 128) qw = ld16(a.q + ((size_t)unit * a.group + min(tid >> 4, a.group - 1)) * HEAD_DIM + part * 8);
  // this thread's slices of the basis rows of its q_hat outputs (loaded up front where
  // the registers allow, so that q_hat, which the scan workgroups wait for, follows
  // the first barrier at once)
  constexpr bool EARLY_M = OUTS <= 2;
  auto m_slice = [&](int o) {
    return reinterpret_cast<const f32x4*>(a.M + ((size_t)h * R + tid / 16 + o * (SCORE_THREADS / 16)) * HEAD_DIM +
                                          part * 8);
  };
  f32x4 mq[EARLY_M ? OUTS : 1][2];
  if constexpr (EARLY_M) {
#pragma unroll
    for (int o = 0; o < OUTS; ++o) {
      mq[o][0] = m_slice(o)[0];
      mq[o][1] = m_slice(o)[1];
    }
  }

  if constexpr (APPEND) {
    using KP = KeyProj<R>;
    static_assert(KP::THREADS == SCORE_THREADS, "one projection output per lane group");
    const int64_t apos = ap.pos[b];
    const bool in_range = apos >= 0 && apos < a.cap;
    f32x4 amv[KP::CH / 4];
    u32x4 akv[KP::CH / 8];
    KP::load_basis(a.M + (size_t)h * R * HEAD_DIM, tid, amv);
    KP::load_key(ap.k_new + (size_t)unit * HEAD_DIM, tid, akv);
    if (tid < 32 && in_range) {
      const int cp = tid & 15;
      const bool is_v = tid >= 16;
      const u32x4 x = ld16((is_v ? ap.v_new : ap.k_new) + (size_t)unit * HEAD_DIM + cp * 8);
      *reinterpret_cast<u32x4*>((is_v ? ap.V : ap.K) + ((size_t)unit * a.cap + apos) * HEAD_DIM + cp * 8) = x;
    }
    const float acc = KP::dot(amv, akv);             // whole waves: the DPP combine needs them
    if (tid % KP::TPO == 0) {
      const int i = tid / KP::TPO;
      const uint32_t bits = KP::template encode<KB>(acc);
      if (in_range) {
        unsigned char* row = ap.Kproj + ((size_t)unit * a.cap + apos) * R * KB;
        if constexpr (KB == 2) reinterpret_cast<uint16_t*>(row)[i] = (uint16_t)bits;
        else row[i] = (unsigned char)bits;
      }
      if constexpr (PUBLISH) {
        if constexpr (KB == 2) reinterpret_cast<uint16_t*>(sh.row)[i] = (uint16_t)bits;
        else reinterpret_cast<unsigned char*>(sh.row)[i] = (unsigned char)bits;
      }
    }
  }
  if (tid < 128) {
    sh.qraw[tid >> 4][part * 4 + 0] = qw.x;
    sh.qraw[tid >> 4][part * 4 + 1] = qw.y;
    sh.qraw[tid >> 4][part * 4 + 2] = qw.z;
    sh.qraw[tid >> 4][part * 4 + 3] = qw.w;
  }
  for (int i = tid; i < PREP_BINS; i += SCORE_THREADS) sh.hist[i] = 0u;
  if (tid == 0) {
    sh.misc[0] = 0xffffffffu;
    sh.misc[2] = 0u;
    a.arrive[unit] = 0u;      // the selection launch that follows counts its exact-path workgroups here
  }
  __syncthreads();
  if constexpr (APPEND && PUBLISH) {
    if (tid < RW) publish(sw + SYNC_ROW + tid, tag, sh.row[tid]);
  }

  // q_bar for channels 8*part .. 8*part + 7 (every lane of a 16-lane row computes it)
  float qbar[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qbar[c] = 0.f;
  for (int g = 0; g < a.group; ++g) {
    const uint32_t* w = &sh.qraw[g][part * 4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qbar[2 * c] += bf_lo(w[c]);
      qbar[2 * c + 1] += bf_hi(w[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) qbar[c] = qbar[c] / (float)a.group;
#pragma unroll
  for (int o = 0; o < OUTS; ++o) {
    const int i = tid / 16 + o * (SCORE_THREADS / 16);
    const f32x4 m0 = EARLY_M ? mq[EARLY_M ? o : 0][0] : m_slice(o)[0];
    const f32x4 m1 = EARLY_M ? mq[EARLY_M ? o : 0][1] : m_slice(o)[1];
    float acc = m0.x * qbar[0];
    acc = fmaf(m0.y, qbar[1], acc);
    acc = fmaf(m0.z, qbar[2], acc);
    acc = fmaf(m0.w, qbar[3], acc);
    acc = fmaf(m1.x, qbar[4], acc);
    acc = fmaf(m1.y, qbar[5], acc);
    acc = fmaf(m1.z, qbar[6], acc);
    acc = fmaf(m1.w, qbar[7], acc);
    acc = row16_sum(acc);
    if (part == 0) {
      a.qhat[(size_t)unit * QHAT_STRIDE + i] = acc;
      sh.qh[i] = acc;
      if constexpr (PUBLISH) publish(sw + i, tag, __float_as_uint(acc));
    }
  }

  const int64_t n = min((int64_t)max(a.seq_len[b], 0), a.cap);
  const int64_t kk = min((int64_t)a.k, n);
  if (!(kk < n)) {        // take every position (also n = 0): no threshold needed
    if (tid == 0) {
      a.tlow[unit * 2] = 0u;
      a.tlow[unit * 2 + 1] = 1u;
      if constexpr (PUBLISH) {
        publish(sw + SYNC_THR, tag, 0u);
        publish(sw + SYNC_THR + 1, tag, 0u);
      }
    }
    return;
  }
  __syncthreads();                                    // sh.qh complete
  const int S = (int)min((int64_t)NS, n);
  const uint32_t seed = fmix32((uint32_t)unit * 0x632BE5ABu + a.epoch[unit] * 0x85157AF5u);

  // sample s sits in row sample_row(s) (one adjacent pair per stratum); wave-wide loads as in the scan: in
  // batch t a wave covers samples sb .. sb + 63 (sb = 64 * (wave + t * waves)), load
  // i reading 16 bytes (lane column p) of sample sb + i * RPL + rs, so the LPR lanes
  // of a sample read its row contiguously; the lane is left the score of sample
  // sb + p * RPL + rs by the transposed reduction
  const int p = lane % LPR, rs = lane / LPR;
  float qh[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) qh[e] = sh.qh[p * VPC + e];
  const unsigned char* base = a.kproj + (size_t)unit * a.cap * R * KB + p * 16;
  float sc[BATCHES];
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int t0 = 0; t0 < BATCHES; t0 += PREP_PASS) {
    u32x4 w[PREP_PASS][LPR];
#pragma unroll
    for (int t = 0; t < PREP_PASS; ++t) {
#pragma unroll
      for (int i = 0; i < LPR; ++i) {
        const int sidx = min(64 * (wave + (t0 + t) * SCORE_WAVES) + i * RPL + rs, S - 1);   // clamped: not binned
        w[t][i] = ld16_stream(base + sample_row<NS>(sidx, n, seed) * R * KB);
      }
    }
#pragma unroll
    for (int t = 0; t < PREP_PASS; ++t) {
      float d[LPR];
#pragma unroll
      for (int i = 0; i < LPR; ++i) d[i] = dot_chunk<KB>(qh, w[t][i]);
      const float s = transpose_reduce<LPR>(d, p);
      sc[t0 + t] = s;
      const int sid = 64 * (wave + (t0 + t) * SCORE_WAVES) + p * RPL + rs;
      if (sid < S && __builtin_isfinite(s)) {
        lo = fminf(lo, s);
        hi = fmaxf(hi, s);
      }
    }
    __builtin_amdgcn_sched_barrier(0);                // one pass of loads in flight at a time
  }
  // the greatest sampled key (NaN, +-inf included) sets the unit's candidate key shift
  uint32_t kmx = 0u;
#pragma unroll
  for (int t = 0; t < BATCHES; ++t)
    if (64 * (wave + t * SCORE_WAVES) + p * RPL + rs < S) kmx = max(kmx, score_key(sc[t]));
  kmx = wave_max_u32(kmx);
  lo = wave_min_f32(lo);
  hi = wave_max_f32(hi);
  if (lane == 0) { sh.red[wave] = lo; sh.red[SCORE_WAVES + wave] = hi; atomicMax(&sh.misc[2], kmx); }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < SCORE_WAVES; ++v) {
    lo = fminf(lo, sh.red[v]);
    hi = fmaxf(hi, sh.red[SCORE_WAVES + v]);
  }
  const float scale = hi > lo ? (float)PREP_BINS / (hi - lo) : 0.f;
  // bin of sample t of this lane (-1: not binned)
  auto bin_of = [&](int t) {
    const float x = sc[t];
    const int sid = 64 * (wave + t * SCORE_WAVES) + p * RPL + rs;
    if (sid >= S || x != x || x == -__builtin_inff()) return -1;
    const float f = (x - lo) * scale;                         // +inf -> top bin
    return f > 0.f ? (int)fminf(f, (float)(PREP_BINS - 1)) : 0;
  };
#pragma unroll
  for (int t = 0; t < BATCHES; ++t) {
    const int bt = bin_of(t);
    if (bt >= 0) atomicAdd(&sh.hist[bt], 1u);
  }
  __syncthreads();
  // the number of samples at or above the true k-th key is Binomial(S, kk/n): taking
  // the sample of rank mean + 5 sd + 4 keeps the threshold below that key except with
  // probability ~1e-7, while about kk + 5 sd n/S rows reach it
  const double pk = (double)kk / (double)n;
  const double mu = (double)S * pk;
  int64_t m = (int64_t)ceil(mu + 5.0 * sqrt(mu * (1.0 - pk)) + 4.0);
  m = m < 1 ? 1 : (m > S ? S : m);
  constexpr int BPT = PREP_BINS / SCORE_THREADS;
  const int b0 = tid * BPT;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += sh.hist[b0 + i];
  uint32_t total;
  const uint32_t inc = prep_block_scan(local, sh.scan, &total);
  uint32_t above = total - inc;                 // samples in bins above this thread's bins
  const uint32_t mm = (uint32_t)m;
  if (above < mm && mm <= above + local) {
    for (int i = BPT - 1; i >= 0; --i) {
      const uint32_t c = sh.hist[b0 + i];
      if (above + c >= mm) { sh.misc[1] = (uint32_t)(b0 + i); break; }
      above += c;
    }
  }
  __syncthreads();
  if (total >= mm) {
    const int bsel = (int)sh.misc[1];
#pragma unroll
    for (int t = 0; t < BATCHES; ++t)
      if (bin_of(t) == bsel) atomicMin(&sh.misc[0], score_key(sc[t]));
  }
  __syncthreads();
  // fewer than m binned samples (most scores NaN or -inf): every row is a candidate
  if (tid == 0) {
    const uint32_t thr = total >= mm ? sh.misc[0] : 0u;
    // candidate keys are stored as (key - thr) >> shift in CAND_KEY_BITS bits: the
    // shift that fits four times the sampled range above the threshold (keys of rows
    // beyond that saturate); at most CAND_ROW_BITS, where no key saturates, which is
    // also the shift when the threshold is 0
    const uint32_t range = sh.misc[2] > thr ? sh.misc[2] - thr : 0u;
    const int bits = range ? 32 - __clz(range) : 0;
    const uint32_t shift =
        total >= mm ? (uint32_t)min(CAND_ROW_BITS, max(0, bits + CAND_HEADROOM - CAND_KEY_BITS)) : (uint32_t)CAND_ROW_BITS;
    a.tlow[unit * 2] = thr;
    a.tlow[unit * 2 + 1] = shift << TLOW_SHIFT_POS;
    if constexpr (PUBLISH) {
      publish(sw + SYNC_THR, tag, thr);
      publish(sw + SYNC_THR + 1, tag, shift);
    }
  }
}

struct ScanArgs {
  const unsigned char* kproj;
  const float* qhat;
  const uint32_t* tlow;
  const int32_t* seq_len;
  int k;
  float* scores;
  uint32_t* cand;
  uint64_t* counts;
  int n_kv_heads;
  int64_t cap;
  int64_t stride;
  int64_t ntile;             // tiles per unit
  int64_t ntile_cap;         // count words per unit
  int64_t cand_stride;
};

// Scan of tile `tile` (rows [tile*TR, +TR), TR = tile_rows(R*KB)) of one unit, 256 threads.
// A segment is the SEG_ROWS = 128 rows one wave covers in one iteration
// (SCORE_UNROLL groups of 64); the waves take the tile's segments in turn (wave w:
// segments w, w + 4, ...), so the workgroup streams one contiguous region. Loads are
// 128-bit and coalesced, each lane holding 8 of a row's r values; the partial dots of
// the r/8 lanes of a row are reduced with DPP lane moves in a transposed pattern,
// after which lane (rs, p) owns the score of group row p*RPL + rs.
//
// Each wave first scores all its rows into a private LDS stash (one key per row);
// then it takes the threshold (and the unit's key shift) and keeps the rows whose key
// reaches it as candidates, 32-bit entries (the key relative to the threshold in 20
// bits, the row's offset in its tile; see cand_entry) in position order: with a ballot of the flags in lane order, the number
// of flagged rows before a row is the popcount of the ballot under a per-lane mask of
// the lanes that hold earlier rows (earlier lane columns, and this column above this
// lane). The candidates are compacted in place over the stash (a segment's entries
// land no later than its own keys, which are read first). At the end the workgroup
// writes the tile's candidates, in position order, to its region of the candidate
// buffer (entries [x*TR, ...) for tile x), and to counts[x] their number (low
// word; TILE_OVERFLOW when a published word did not arrive in time) and their
// greatest key (high word; 0 when there are none); writes in the middle of the
// stream cost far more HBM time than their size. With WRITE_DENSE every score is
// also stored.
// POLL: q_hat and the threshold come from the unit's prep in the same launch (tagged
// words); apos (may be null) gives the slot of each sequence's appended token, whose
// projected row is taken from the published words rather than from memory.
template <int R, int KB, bool WRITE_DENSE, bool POLL>
__device__ __forceinline__ void scan_body(ScanShared& sh, int unit, int tile, const ScanArgs& a,
                                          const uint64_t* sync, uint32_t tag, const int32_t* apos_b,
                                          uint64_t wait_ticks) {
  static_assert(!(WRITE_DENSE && POLL), "dense scores come from the two-launch form");
  constexpr int LPR = R * KB / 16;      // lanes per Kproj row (16 bytes each)
  constexpr int VPC = 16 / KB;          // values per 16-byte word
  constexpr int RPL = 64 / LPR;         // rows per wave-wide load
  constexpr int RW = R * KB / 4;        // 32-bit words of a projected row
  constexpr int TR = tile_rows(R * KB);
  constexpr int SEGS = TR / SEG_ROWS;   // segments per tile
  const int b = unit / a.n_kv_heads;
  const int n = (int)min((int64_t)max(a.seq_len[b], 0), a.cap);      // cap < 2^30
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg0 = tile * SEGS;
  if (seg0 * SEG_ROWS >= n) return;            // the whole tile lies past the end
  const bool take_all = POLL ? a.k >= n : (a.tlow[unit * 2 + 1] & 1u) != 0u;
  if (take_all && !WRITE_DENSE) return;
  const int p = lane % LPR;
  const int rs = lane / LPR;
  // lanes holding rows before this lane's row p*RPL + rs
  uint64_t col0 = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) col0 |= 1ull << (i * LPR);
  const uint64_t earlier = col0 * ((1ull << p) - 1) | ((col0 << p) & ((1ull << (LPR * rs)) - 1));

  const uint64_t* sw = sync + (size_t)unit * SYNC_WORDS;
  uint64_t deadline = 0;
  int apos = -1;
  float qh[VPC];
  if constexpr (POLL) {
    deadline = __builtin_readsteadycounter() + wait_ticks;
    if (apos_b) {
      const int64_t ap = apos_b[b];
      if (ap >= (int64_t)tile * TR && ap < (int64_t)(tile + 1) * TR && ap < a.cap) apos = (int)ap;
    }
  } else {
#pragma unroll
    for (int e = 0; e < VPC; ++e) qh[e] = a.qhat[(size_t)unit * QHAT_STRIDE + p * VPC + e];
  }

  const unsigned char* base = a.kproj + (size_t)unit * a.cap * R * KB + p * 16;
  float* srow = a.scores + (size_t)unit * a.stride;
  uint32_t* stash = sh.stash[wave];
  const int last = n - 1;
  bool ok = true;                          // published words arrived
  // loads of the segment starting at row g0: rows past the end are clamped to the last
  // valid row (never reported), so every load is unconditional and the whole batch
  // stays in flight
  auto load_seg = [&](int g0, u32x4 (&w)[SCORE_UNROLL][LPR]) {
#pragma unroll
    for (int u = 0; u < SCORE_UNROLL; ++u) {
#pragma unroll
      for (int i = 0; i < LPR; ++i)
        w[u][i] = ld16_stream(base + (size_t)min(g0 + u * GROUP_ROWS + i * RPL + rs, last) * R * KB);
    }
  };
  // scores of the segment into stash slot `slot` (its keys, one per row)
  auto score_seg = [&](int g0, int slot, const u32x4 (&w)[SCORE_UNROLL][LPR]) {
#pragma unroll
    for (int u = 0; u < SCORE_UNROLL; ++u) {
      float d[LPR];
#pragma unroll
      for (int i = 0; i < LPR; ++i) d[i] = dot_chunk<KB>(qh, w[u][i]);
      const float s = transpose_reduce<LPR>(d, p);
      if (WRITE_DENSE) {
        const int row = g0 + u * GROUP_ROWS + p * RPL + rs;
        if (row < n) srow[row] = s;
      }
      stash[SEG_ROWS * slot + GROUP_ROWS * u + lane] = score_key(s);
    }
  };
  int nseg = 0;
  int j = wave;
  if constexpr (POLL) {
    // first segment: q_hat is polled while its loads are in flight
    const int g0 = (seg0 + j) * SEG_ROWS;
    if (g0 < n) {
      u32x4 w[SCORE_UNROLL][LPR];
      load_seg(g0, w);
      uint32_t v;
      ok = wait_ticks != 0 && poll_words(sw, R, tag, deadline, v);   // 0: never take them
      if (ok) {
        if (lane < R) sh.words[wave][lane] = v;
#pragma unroll
        for (int e = 0; e < VPC; ++e) qh[e] = __uint_as_float(sh.words[wave][p * VPC + e]);
        score_seg(g0, 0, w);
        nseg = 1;
        j += SCORE_WAVES;
      }
    }
  }
  if (ok) {
    for (; j < SEGS; j += SCORE_WAVES, ++nseg) {
      const int g0 = (seg0 + j) * SEG_ROWS;
      if (g0 >= n) break;
      u32x4 w[SCORE_UNROLL][LPR];
      load_seg(g0, w);
      score_seg(g0, nseg, w);
    }
  }

  if constexpr (POLL) {
    // the appended token's row (if it falls in a segment this wave scored): its key
    // from the published bytes, not from memory, which the prep may not have written
    // yet. The chunk dots of lanes 0..LPR-1 are added in the balanced tree of the
    // transposed reduction, so the key is the one the scan would have computed.
    const int ja = apos - seg0 * SEG_ROWS;               // row offset in the tile (< 0: none)
    const int jseg = ja >> 7;                            // segment of the tile (SEG_ROWS = 128)
    if (ok && ja >= 0 && apos < n && (jseg & (SCORE_WAVES - 1)) == wave) {
      uint32_t v;
      ok = poll_words(sw + SYNC_ROW, RW, tag, deadline, v);
      if (ok) {
        if (lane < RW) sh.words[wave][lane] = v;
        const u32x4 chunk = *reinterpret_cast<const u32x4*>(&sh.words[wave][4 * p]);
        float x = dot_chunk<KB>(qh, chunk);
        if constexpr (LPR >= 2) x += dpp<DPP_QUAD_XOR1>(x);
        if constexpr (LPR >= 4) x += dpp<DPP_QUAD_XOR2>(x);
        if constexpr (LPR >= 8) x += swz_xor4(x);
        const int r_in = ja & (SEG_ROWS - 1);            // row in its segment
        const int u = r_in / GROUP_ROWS, rg = r_in % GROUP_ROWS;
        const int owner = (rg % RPL) * LPR + rg / RPL;   // the lane whose score is that row's
        if (lane == 0) stash[SEG_ROWS * (jseg / SCORE_WAVES) + GROUP_ROWS * u + owner] = score_key(x);
      }
    }
  }
  uint32_t tkey = 0, tshift = 0;           // the threshold key and the candidate key shift
  if (ok && !take_all && nseg > 0) {
    if constexpr (POLL) {
      uint32_t v;
      ok = poll_words(sw + SYNC_THR, 2, tag, deadline, v);
      tkey = readlane_u32(v, 0);
      tshift = readlane_u32(v, 1);
    } else {
      tkey = a.tlow[unit * 2];
      tshift = a.tlow[unit * 2 + 1] >> TLOW_SHIFT_POS;
    }
  }
  uint32_t wcount = 0;                     // candidates of this wave so far
  uint32_t kmax = 0;                       // greatest candidate key seen by this lane
  int filtered = 0;
  if (ok && !take_all) {
    for (; filtered < nseg; ++filtered) {
      const int j = wave + filtered * SCORE_WAVES;
      const int g0 = (seg0 + j) * SEG_ROWS;
      uint32_t key[SCORE_UNROLL];
#pragma unroll
      for (int u = 0; u < SCORE_UNROLL; ++u) key[u] = stash[SEG_ROWS * filtered + GROUP_ROWS * u + lane];
      uint32_t count = 0;
#pragma unroll
      for (int u = 0; u < SCORE_UNROLL; ++u) {
        const int row = g0 + u * GROUP_ROWS + p * RPL + rs;
        const bool c = row < n && key[u] >= tkey;
        const uint64_t m = __ballot(c);
        if (c) {
          stash[wcount + count + (uint32_t)__popcll(m & earlier)] =
              cand_entry(cand_rel(key[u], tkey, tshift), row - seg0 * SEG_ROWS);   // offset in the tile
          kmax = max(kmax, key[u]);
        }
        count += (uint32_t)__popcll(m);
      }
      if (lane == 0) sh.segcnt[j] = count;
      wcount += count;
    }
  }
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    for (int j = wave + filtered * SCORE_WAVES; j < SEGS; j += SCORE_WAVES) sh.segcnt[j] = 0u;
    sh.overflow[wave] = ok ? 0u : 1u;
    sh.wmax[wave] = kmax;
  }
  __syncthreads();
  // the tile's candidates in position order: segment jj's entries start at
  // segoff[jj] (the counts of segments 0 .. jj-1) in the output and at sstart[jj]
  // (the counts of the same wave's earlier segments) in its wave's stash
  if (wave == 0) {
    const uint32_t c = lane < SEGS ? sh.segcnt[lane] : 0u;
    const uint32_t inc = wave_incl_scan(c);
    if (lane < SEGS) {
      sh.segoff[lane + 1] = inc;
      uint32_t st = 0;
      for (int q = lane % SCORE_WAVES; q < lane; q += SCORE_WAVES) st += sh.segcnt[q];
      sh.sstart[lane] = st;
    }
    if (lane == 0) sh.segoff[0] = 0u;
  }
  __syncthreads();
  bool ovf = false;
#pragma unroll
  for (int v = 0; v < SCORE_WAVES; ++v) ovf = ovf || sh.overflow[v] != 0u;
  const uint32_t tot = sh.segoff[SEGS];
  if (!ovf) {
    // every thread writes entries e, e + 256, ...: coalesced, streamed past the caches
    uint32_t* wtile = a.cand + (size_t)unit * a.cand_stride + (size_t)tile * TR;
    for (uint32_t e = threadIdx.x; e < tot; e += SCORE_THREADS) {
      int lo = 0, hi = SEGS;                     // the segment holding entry e
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.segoff[mid] <= e) lo = mid; else hi = mid;
      }
      __builtin_nontemporal_store(sh.stash[lo % SCORE_WAVES][sh.sstart[lo] + (e - sh.segoff[lo])], wtile + e);
    }
  }
  if (threadIdx.x == 0) {
    uint32_t tmax = 0;
#pragma unroll
    for (int v = 0; v < SCORE_WAVES; ++v) tmax = max(tmax, sh.wmax[v]);
    a.counts[(size_t)unit * a.ntile_cap + tile] = ((uint64_t)tmax << 32) | (ovf ? TILE_OVERFLOW : tot);
  }
}

// grid = B * H_kv
template <int R, int KB, bool APPEND>
__global__ __launch_bounds__(SCORE_THREADS) void prep_kernel(PrepArgs a, PrepAppend ap) {
  __shared__ PrepShared sh;
  prep_body<R, KB, APPEND, false>(sh, blockIdx.x, a, ap, nullptr, 0u);
}

// grid = (ntile_cap, B * H_kv)
template <int R, int KB, bool WRITE_DENSE>
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(ScanArgs a) {
  __shared__ ScanShared sh;
  scan_body<R, KB, WRITE_DENSE, false>(sh, blockIdx.y, blockIdx.x, a, nullptr, 0u, nullptr, 0u);
}

// Waves per SIMD the fused kernel is compiled for: the most at which both roles fit
// their registers without spilling (8, as the scan alone runs, for bf16 rows with
// r <= 32); left to the compiler, the prep role's registers would set a lower one.
template <int R, int KB>
constexpr int fused_waves() { return R <= 32 ? (KB == 2 ? 8 : 7) : (KB == 2 ? 5 : 6); }

// grid = B*H_kv + B*H_kv * ntile, one-dimensional: workgroups [0, units) are the
// preps (dispatched first), then the scan tiles unit by unit.
template <int R, int KB, bool APPEND>
__global__ __launch_bounds__(SCORE_THREADS) __attribute__((amdgpu_waves_per_eu(fused_waves<R, KB>()))) void prep_scan_kernel(PrepArgs pa, PrepAppend ap, ScanArgs sa,
                                                                  uint64_t* sync, const uint32_t* epoch,
                                                                  int units, uint64_t wait_ticks) {
  __shared__ ScoreShared sh;
  const int64_t bid = blockIdx.x;
  if (bid < units) {
    const int unit = (int)bid;
    prep_body<R, KB, APPEND, true>(sh.p, unit, pa, ap, sync, launch_tag(epoch, unit));
  } else {
    const int64_t id = bid - units;
    const int unit = (int)(id / sa.ntile);
    const int tile = (int)(id - (int64_t)unit * sa.ntile);
    scan_body<R, KB, false, true>(sh.s, unit, tile, sa, sync, launch_tag(epoch, unit),
                                  APPEND ? ap.pos : nullptr, wait_ticks);
  }
}

PrepArgs prep_args(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                   const unsigned char* kproj, const int32_t* seq_len, int k, unsigned char* ws) {
  PrepArgs a;
  a.q = q;
  a.M = M;
  a.kproj = kproj;
  a.seq_len = seq_len;
  a.k = k;
  a.qhat = reinterpret_cast<float*>(ws + L.off_qhat);
  a.tlow = reinterpret_cast<uint32_t*>(ws + L.off_tlow);
  a.arrive = reinterpret_cast<uint32_t*>(ws + L.off_arrive);
  a.epoch = reinterpret_cast<const uint32_t*>(ws + L.off_epoch);
  a.n_kv_heads = s.n_kv_heads;
  a.group = s.group;
  a.cap = s.capacity;
  return a;
}

ScanArgs scan_args(const sjsa_shape& s, const Layout& L, const unsigned char* kproj, const int32_t* seq_len,
                   int k, unsigned char* ws) {
  ScanArgs a;
  a.kproj = kproj;
  a.qhat = reinterpret_cast<const float*>(ws + L.off_qhat);
  a.tlow = reinterpret_cast<const uint32_t*>(ws + L.off_tlow);
  a.seq_len = seq_len;
  a.k = k;
  a.scores = reinterpret_cast<float*>(ws + L.off_scores);
  a.cand = reinterpret_cast<uint32_t*>(ws + L.off_cand);
  a.counts = reinterpret_cast<uint64_t*>(ws + L.off_counts);
  a.n_kv_heads = s.n_kv_heads;
  a.cap = s.capacity;
  a.stride = L.score_stride;
  a.ntile = L.ntile;
  a.ntile_cap = L.ntile_cap;
  a.cand_stride = L.cand_stride;
  return a;
}

}  // namespace

hipError_t launch_prep(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                       const void* kproj_v, const int32_t* seq_len, int k, unsigned char* ws, hipStream_t st,
                       const PrepAppend* ap) {
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
  const PrepArgs a = prep_args(s, L, q, M, static_cast<const unsigned char*>(kproj_v), seq_len, k, ws);
  const dim3 grid((unsigned)L.units), block(SCORE_THREADS);
  const PrepAppend none{};
#define SJSA_PREP2(RR, KB)                                                             \
  if (ap) prep_kernel<RR, KB, true><<<grid, block, 0, st>>>(a, *ap);                   \
  else prep_kernel<RR, KB, false><<<grid, block, 0, st>>>(a, none)
#define SJSA_PREP(RR) if (fp8) { SJSA_PREP2(RR, 1); } else { SJSA_PREP2(RR, 2); }
  switch (s.rank) {
    case 16: SJSA_PREP(16); break;
    case 32: SJSA_PREP(32); break;
    case 64: SJSA_PREP(64); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_PREP
#undef SJSA_PREP2
  return hipGetLastError();
}

hipError_t launch_score(const sjsa_shape& s, const Layout& L, const void* kproj_v, const int32_t* seq_len,
                        unsigned char* ws, hipStream_t st) {
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
  const ScanArgs a = scan_args(s, L, static_cast<const unsigned char*>(kproj_v), seq_len, 0, ws);
  const dim3 grid((unsigned)L.ntile, (unsigned)L.units), block(SCORE_THREADS);
  const bool dense = (s.flags & SJSA_FLAG_WRITE_SCORES) != 0;
#define SJSA_SCAN2(RR, KB, DD) score_kernel<RR, KB, DD><<<grid, block, 0, st>>>(a)
#define SJSA_SCAN(RR)                                              \
  if (fp8) {                                                       \
    if (dense) SJSA_SCAN2(RR, 1, true); else SJSA_SCAN2(RR, 1, false); \
  } else {                                                         \
    if (dense) SJSA_SCAN2(RR, 2, true); else SJSA_SCAN2(RR, 2, false); \
  }
  switch (s.rank) {
    case 16: SJSA_SCAN(16); break;
    case 32: SJSA_SCAN(32); break;
    case 64: SJSA_SCAN(64); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_SCAN
#undef SJSA_SCAN2
  return hipGetLastError();
}

hipError_t launch_prep_scan(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                            const void* kproj_v, const int32_t* seq_len, int k, unsigned char* ws, hipStream_t st,
                            const PrepAppend* ap) {
  const int64_t blocks = L.units * (L.ntile + 1);
  if ((s.flags & SJSA_FLAG_WRITE_SCORES) != 0 || blocks > 0x7fffffff) {
    hipError_t e = launch_prep(s, L, q, M, kproj_v, seq_len, k, ws, st, ap);
    return e == hipSuccess ? launch_score(s, L, kproj_v, seq_len, ws, st) : e;
  }
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
  const unsigned char* kproj = static_cast<const unsigned char*>(kproj_v);
  const PrepArgs pa = prep_args(s, L, q, M, kproj, seq_len, k, ws);
  const ScanArgs sa = scan_args(s, L, kproj, seq_len, k, ws);
  uint64_t* sync = reinterpret_cast<uint64_t*>(ws + L.off_sync);
  const uint32_t* epoch = reinterpret_cast<const uint32_t*>(ws + L.off_epoch);
  const dim3 grid((unsigned)blocks), block(SCORE_THREADS);
  const PrepAppend none{};
  const int units = (int)L.units;
  const int32_t wait_us = s.fused_wait_us == 0 ? DEFAULT_WAIT_US : (s.fused_wait_us < 0 ? 0 : s.fused_wait_us);
  const uint64_t wait = (uint64_t)wait_us * TICKS_PER_US;
#define SJSA_PS2(RR, KB)                                                                                     \
  if (ap) prep_scan_kernel<RR, KB, true><<<grid, block, 0, st>>>(pa, *ap, sa, sync, epoch, units, wait); \
  else prep_scan_kernel<RR, KB, false><<<grid, block, 0, st>>>(pa, none, sa, sync, epoch, units, wait)
#define SJSA_PS(RR) if (fp8) { SJSA_PS2(RR, 1); } else { SJSA_PS2(RR, 2); }
  switch (s.rank) {
    case 16: SJSA_PS(16); break;
    case 32: SJSA_PS(32); break;
    case 64: SJSA_PS(64); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_PS
#undef SJSA_PS2
  return hipGetLastError();
}

}  // namespace sjsa

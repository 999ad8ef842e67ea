// Scoring prep and the full-context score scan.
//
// Source: JSSA article, section 打分误差的定义: selection uses the mean query of
// the G query heads of a KV head, and the projected score of key k is
// s_hat = q_bar^T M^T M k = (M q_bar) . (M k) = q_hat . Kproj_j. Section 原理详解(二)
// notes that scoring still scans every candidate position; only the attention
// becomes sparse. Section 组件级拆解 names the stages: scoring prep, candidate
// scoring, top-k selection, sparse attention.
//
// prep_kernel  (one workgroup per (b, h)): q_bar in fp32 (sum in head order, then
//              divide by G), q_hat = M_h q_bar (fp32), and the unit's candidate
//              threshold, placed from the scores of evenly spaced sample rows.
// score_kernel (grid = tiles x units): streams Kproj rows with 128-bit coalesced
//              loads, each lane holding 8 of a row's r values; the partial dots of
//              the r/8 lanes of a row are reduced with DPP lane moves in a
//              transposed pattern, so that after the reduction each lane owns the
//              full score of one row. Rows whose score key reaches the threshold
//              are kept as candidates for the top-k stage (and, on request, every
//              score is stored).
#include "key_proj.h"

namespace sjsa {
namespace {

constexpr int PREP_THREADS = 512;
constexpr int PREP_WAVES = PREP_THREADS / 64;
constexpr int SCORE_THREADS = 256;
constexpr int SCORE_WAVES = SCORE_THREADS / 64;
constexpr int GROUP_ROWS = 64;       // rows covered by r/8 wave-wide 16-byte loads
// rows scored by the prep kernel to place the threshold: more samples give a tighter
// threshold (fewer candidates) but cost the prep kernel about as much time as the
// later stages save (measured with 4096 at the 128K batch-16 shape)
template <int R>
constexpr int samples_for() { return 2048; }
constexpr int PREP_BINS = 4096;      // linear score bins of the threshold histogram

// Block-wide (PREP_THREADS) inclusive scan of one u32 per thread; the block total
// goes to *total. Two barriers.
__device__ uint32_t prep_block_scan(uint32_t v, uint32_t* scan_lds, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) scan_lds[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < PREP_WAVES; ++w) {
    const uint32_t t = scan_lds[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return inc + before;
}

// Row of sample s (0 <= s < min(NS, n)): every row when n <= NS; else the samples
// come in adjacent pairs (2i, 2i + 1 share a 128-byte cache line whenever a
// projected row is at most 64 bytes), the pairs evenly spaced over the sequence.
template <int NS>
__device__ __forceinline__ int64_t sample_row(int s, int64_t n) {
  if (n <= NS) return s;
  return 2 * (((int64_t)(s >> 1) * n) / NS) + (s & 1);
}

// One workgroup per (b, h).
//  * q_bar in fp32 (sum in head order, then divide by G) and q_hat = M_h q_bar: output
//    i is split over 16 lanes of 8 channels each (fp32 partial dots, DPP row sum).
//  * Threshold for the scan: the scores of NS rows (NS = samples_for<R>(), evenly
//    spaced pairs of adjacent rows; all rows when n <= NS) are binned linearly
//    between their least and greatest finite value (+inf in the top bin, -inf and
//    NaN left out); the bin that holds the sample of rank m (see below) is found,
//    and the least key in it becomes the unit's candidate threshold, so at least m
//    samples reach it. The exact top k is among
//    the rows that reach it unless the sample misjudges the distribution, a case the
//    select stage detects and handles exactly: the threshold only decides how much
//    work the select stage does, never its result.
//  * mode: 1 when k >= n (every position is selected and the scan has no work).
// The sample rows are loaded first, so their latency overlaps the q_hat work.
//
// With APPEND the workgroup first appends its unit's new token (decode: one token
// per sequence at slot pos[b]): threads 256..287 copy its K and V rows and threads
// 0..255 write its projected row with the KeyProj layout (bit-identical to the
// append kernel). A sample that lands on that slot may read the row before or
// after the write; either way only the threshold moves, never the result.
template <int R, int KB, bool APPEND>
__global__ __launch_bounds__(PREP_THREADS) void prep_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ M, const unsigned char* kproj,
    const int32_t* __restrict__ seq_len, int k, float* __restrict__ qhat, uint32_t* __restrict__ tlow,
    int n_kv_heads, int group, int64_t cap, PrepAppend ap) {
  constexpr int LPR = R * KB / 16;                    // 16-byte words per Kproj row
  constexpr int VPC = 16 / KB;                        // values per 16-byte word
  constexpr int RPL = 64 / LPR;                       // samples per wave-wide load
  constexpr int NS = samples_for<R>();
  constexpr int BATCHES = NS / PREP_THREADS;          // 64-sample batches per wave (= samples per lane)
  constexpr int OUTS = (R * 16 + PREP_THREADS - 1) / PREP_THREADS;   // q_hat outputs per thread
  __shared__ float sqh[R];
  __shared__ uint32_t shist[PREP_BINS];
  __shared__ float sred[2 * PREP_WAVES];
  __shared__ uint32_t sscan[PREP_WAVES];
  __shared__ uint32_t smisc[4];
  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int h = unit - b * n_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  using KP = KeyProj<R>;
  static_assert(KP::THREADS + 32 <= PREP_THREADS, "projection and row copies fit the workgroup");
  f32x4 amv[KP::CH / 4];
  u32x4 akv[KP::CH / 8];
  int64_t apos = -1;
  if constexpr (APPEND) {
    apos = ap.pos[b];
    const uint16_t* krow = ap.k_new + (size_t)unit * HEAD_DIM;
    if (tid < KP::THREADS) {
      KP::load_basis(M + (size_t)h * R * HEAD_DIM, tid, amv);
      KP::load_key(krow, tid, akv);
    } else if (tid < KP::THREADS + 32 && apos >= 0 && apos < cap) {
      const int part = tid & 15;
      const bool is_v = (tid - KP::THREADS) >= 16;
      const u32x4 x = ld16((is_v ? ap.v_new : ap.k_new) + (size_t)unit * HEAD_DIM + part * 8);
      *reinterpret_cast<u32x4*>((is_v ? ap.V : ap.K) + ((size_t)unit * cap + apos) * HEAD_DIM + part * 8) = x;
    }
  }

  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int64_t kk = min((int64_t)k, n);
  const bool sampling = kk < n;                       // uniform over the workgroup
  const int S = (int)min((int64_t)NS, n);

  // sample s sits in row pos(s) (evenly spaced); wave-wide loads as in the scan: in
  // batch t a wave covers samples sb .. sb + 63 (sb = 64 * (wave + t * PREP_WAVES)),
  // load i reading 16 bytes (lane column p) of sample sb + i * RPL + rs, so the LPR
  // lanes of a sample read its row contiguously
  const int p = lane % LPR, rs = lane / LPR;
  u32x4 w[BATCHES][LPR];
  if (sampling) {
    const unsigned char* base = kproj + (size_t)unit * cap * R * KB + p * 16;
#pragma unroll
    for (int t = 0; t < BATCHES; ++t) {
#pragma unroll
      for (int i = 0; i < LPR; ++i) {
        const int sidx = min(64 * (wave + t * PREP_WAVES) + i * RPL + rs, S - 1);   // clamped: not binned
        const int64_t pos = sample_row<NS>(sidx, n);
        w[t][i] = ld16_stream(base + pos * R * KB);
      }
    }
  }

  // q_bar for channels 8*part .. 8*part + 7 (every lane of a 16-lane row computes it)
  const int part = tid & 15;
  float qbar[8];
  {
    const uint16_t* qg = q + (size_t)unit * group * HEAD_DIM + part * 8;
    u32x4 qw[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) qw[g] = ld16(qg + (size_t)min(g, group - 1) * HEAD_DIM);
#pragma unroll
    for (int c = 0; c < 8; ++c) qbar[c] = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < group) {
        qbar[0] += bf_lo(qw[g].x); qbar[1] += bf_hi(qw[g].x);
        qbar[2] += bf_lo(qw[g].y); qbar[3] += bf_hi(qw[g].y);
        qbar[4] += bf_lo(qw[g].z); qbar[5] += bf_hi(qw[g].z);
        qbar[6] += bf_lo(qw[g].w); qbar[7] += bf_hi(qw[g].w);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) qbar[c] = qbar[c] / (float)group;
  }
#pragma unroll
  for (int o = 0; o < OUTS; ++o) {
    const int i = tid / 16 + o * (PREP_THREADS / 16);
    const f32x4* m4 = reinterpret_cast<const f32x4*>(M + ((size_t)h * R + min(i, R - 1)) * HEAD_DIM + part * 8);
    const f32x4 m0 = m4[0], m1 = m4[1];
    float acc = m0.x * qbar[0];
    acc = fmaf(m0.y, qbar[1], acc);
    acc = fmaf(m0.z, qbar[2], acc);
    acc = fmaf(m0.w, qbar[3], acc);
    acc = fmaf(m1.x, qbar[4], acc);
    acc = fmaf(m1.y, qbar[5], acc);
    acc = fmaf(m1.z, qbar[6], acc);
    acc = fmaf(m1.w, qbar[7], acc);
    acc = row16_sum(acc);
    if (part == 0 && i < R) {
      qhat[(size_t)unit * QHAT_STRIDE + i] = acc;
      sqh[i] = acc;
    }
  }
  if constexpr (APPEND) {
    if (tid < KP::THREADS) {                          // whole waves: the DPP combine needs them
      const float acc = KP::dot(amv, akv);
      if (tid % KP::TPO == 0 && apos >= 0 && apos < cap)
        KP::template store<KB>(ap.Kproj + ((size_t)unit * cap + apos) * R * KB, tid / KP::TPO, acc);
    }
  }
  for (int i = tid; i < PREP_BINS; i += PREP_THREADS) shist[i] = 0u;
  if (tid == 0) smisc[0] = 0xffffffffu;
  __syncthreads();
  if (!sampling) {        // take every position (also n = 0): no threshold needed
    if (tid == 0) { tlow[unit * 2] = 0u; tlow[unit * 2 + 1] = 1u; }
    return;
  }

  // lane (rs, p) scores its VPC columns of the LPR rows of a batch; the transposed
  // reduction leaves it the score of sample sb + p * RPL + rs
  float qh[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) qh[e] = sqh[p * VPC + e];
  float sc[BATCHES];
  int sid[BATCHES];
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < BATCHES; ++t) {
    float a[LPR];
#pragma unroll
    for (int i = 0; i < LPR; ++i) a[i] = dot_chunk<KB>(qh, w[t][i]);
    sc[t] = transpose_reduce<LPR>(a, p);
    sid[t] = 64 * (wave + t * PREP_WAVES) + p * RPL + rs;
    if (sid[t] < S && __builtin_isfinite(sc[t])) {
      lo = fminf(lo, sc[t]);
      hi = fmaxf(hi, sc[t]);
    }
  }
  lo = wave_min_f32(lo);
  hi = wave_max_f32(hi);
  if (lane == 0) { sred[wave] = lo; sred[PREP_WAVES + wave] = hi; }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < PREP_WAVES; ++v) {
    lo = fminf(lo, sred[v]);
    hi = fmaxf(hi, sred[PREP_WAVES + v]);
  }
  const float scale = hi > lo ? (float)PREP_BINS / (hi - lo) : 0.f;
  int bin[BATCHES];
#pragma unroll
  for (int t = 0; t < BATCHES; ++t) {
    const float x = sc[t];
    bin[t] = -1;
    if (sid[t] < S && !(x != x) && x != -__builtin_inff()) {
      const float f = (x - lo) * scale;                       // +inf -> top bin; NaN -> bin 0
      bin[t] = f > 0.f ? (int)fminf(f, (float)(PREP_BINS - 1)) : 0;
      atomicAdd(&shist[bin[t]], 1u);
    }
  }
  __syncthreads();
  // the number of samples at or above the true k-th key is Binomial(S, kk/n): taking
  // the sample of rank mean + 5 sd + 4 keeps the threshold below that key except with
  // probability ~1e-7, while about kk + 5 sd n/S rows reach it
  const double pk = (double)kk / (double)n;
  const double mu = (double)S * pk;
  int64_t m = (int64_t)ceil(mu + 5.0 * sqrt(mu * (1.0 - pk)) + 4.0);
  m = m < 1 ? 1 : (m > S ? S : m);
  constexpr int BPT = PREP_BINS / PREP_THREADS;
  const int b0 = tid * BPT;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += shist[b0 + i];
  uint32_t total;
  const uint32_t inc = prep_block_scan(local, sscan, &total);
  uint32_t above = total - inc;                 // samples in bins above this thread's bins
  const uint32_t mm = (uint32_t)m;
  if (above < mm && mm <= above + local) {
    for (int i = BPT - 1; i >= 0; --i) {
      const uint32_t c = shist[b0 + i];
      if (above + c >= mm) { smisc[1] = (uint32_t)(b0 + i); break; }
      above += c;
    }
  }
  __syncthreads();
  if (total >= mm) {
    const int bsel = (int)smisc[1];
#pragma unroll
    for (int t = 0; t < BATCHES; ++t)
      if (bin[t] == bsel) atomicMin(&smisc[0], score_key(sc[t]));
  }
  __syncthreads();
  // fewer than m binned samples (most scores NaN or -inf): every row is a candidate
  if (tid == 0) { tlow[unit * 2] = total >= mm ? smisc[0] : 0u; tlow[unit * 2 + 1] = 0u; }
}

// grid = (ceil(cap / TILE_ROWS), B * H_kv). A segment is the SEG_ROWS = 128 rows
// one wave covers in one iteration (UNROLL groups of 64); the waves of a workgroup
// take the tile's segments in turn (wave w: segments w, w + 4, ...), so the
// workgroup streams one contiguous region. Loads are 128-bit and coalesced, each
// lane holding 8 of a row's r values; the partial dots of the r/8 lanes of a row
// are reduced with DPP lane moves in a transposed pattern, after which lane (rs, p)
// owns the score of group row p*RPL + rs.
//
// Rows whose key reaches the unit's threshold are candidates, kept as 32-bit entries
// (the key's top 20 bits, the row's offset in its tile; see cand_entry) in position
// order: with a ballot of the flags in lane order, the number of
// flagged rows before a row is the popcount of the ballot under a per-lane mask of
// the lanes that hold earlier rows (earlier lane columns, and this column above this
// lane). Each wave packs the candidates of its segments back to back into a
// wave-private LDS stage and records each segment's count. At the end the
// workgroup writes the tile's candidates, in position order, to its region of the
// candidate buffer (entries [x*TILE_ROWS, ...) for tile x), and to counts[x] their
// number (low word; TILE_OVERFLOW when a wave had more than CAND_STAGE) and their
// greatest key (high word; 0 when there are none); writes in the
// middle of the stream cost far more HBM time than their size. With WRITE_DENSE
// every score is also stored.
template <int R, int KB, int UNROLL, bool WRITE_DENSE>
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(
    const unsigned char* __restrict__ kproj, const float* __restrict__ qhat, const uint32_t* __restrict__ tlow,
    const int32_t* __restrict__ seq_len, float* __restrict__ scores, uint32_t* __restrict__ cand,
    uint64_t* __restrict__ counts, int n_kv_heads, int64_t cap, int64_t stride, int64_t ntile_cap,
    int64_t cand_stride) {
  constexpr int LPR = R * KB / 16;      // lanes per Kproj row (16 bytes each)
  constexpr int VPC = 16 / KB;          // values per 16-byte word
  constexpr int RPL = 64 / LPR;         // rows per wave-wide load
  static_assert(GROUP_ROWS * UNROLL == SEG_ROWS, "one wave iteration covers one segment");
  static_assert(TILE_ROWS / SEG_ROWS <= 64, "one wave scans the segment counts");
  constexpr int SEGS_PER_TILE = TILE_ROWS / SEG_ROWS;
  __shared__ uint32_t stage[SCORE_WAVES][CAND_STAGE];
  __shared__ uint32_t segcnt[SEGS_PER_TILE];
  __shared__ uint32_t segoff[SEGS_PER_TILE + 1];
  __shared__ uint32_t sstart[SEGS_PER_TILE];
  __shared__ uint32_t overflow[SCORE_WAVES];
  __shared__ uint32_t wmax[SCORE_WAVES];
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int n = (int)min((int64_t)max(seq_len[b], 0), cap);      // cap < 2^30
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg0 = blockIdx.x * SEGS_PER_TILE;
  if (seg0 * SEG_ROWS >= n) return;            // the whole tile lies past the end
  const bool take_all = tlow[unit * 2 + 1] != 0u;
  if (take_all && !WRITE_DENSE) return;
  const uint32_t tkey = tlow[unit * 2];
  const int p = lane % LPR;
  const int rs = lane / LPR;
  // lanes holding rows before this lane's row p*RPL + rs
  uint64_t col0 = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) col0 |= 1ull << (i * LPR);
  const uint64_t earlier = col0 * ((1ull << p) - 1) | ((col0 << p) & ((1ull << (LPR * rs)) - 1));

  float qh[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) qh[e] = qhat[(size_t)unit * QHAT_STRIDE + p * VPC + e];

  const unsigned char* base = kproj + (size_t)unit * cap * R * KB + p * 16;
  float* srow = scores + (size_t)unit * stride;
  const int last = n - 1;
  uint32_t wcount = 0;                     // candidates of this wave so far
  uint32_t kmax = 0;                       // greatest candidate key seen by this lane

  int j = wave;
  for (; j < SEGS_PER_TILE; j += SCORE_WAVES) {
    const int g0 = (seg0 + j) * SEG_ROWS;
    if (g0 >= n) break;
    u32x4 w[UNROLL][LPR];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
      for (int i = 0; i < LPR; ++i) {
        // rows past the end are clamped to the last valid row (never reported), so
        // every load is unconditional and the whole batch stays in flight
        const int row = min(g0 + u * GROUP_ROWS + i * RPL + rs, last);
        w[u][i] = ld16_stream(base + (size_t)row * R * KB);
      }
    }
    uint32_t count = 0;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float a[LPR];
#pragma unroll
      for (int i = 0; i < LPR; ++i) a[i] = dot_chunk<KB>(qh, w[u][i]);
      const float s = transpose_reduce<LPR>(a, p);
      const int row = g0 + u * GROUP_ROWS + p * RPL + rs;
      const bool valid = row < n;
      if (WRITE_DENSE && valid) srow[row] = s;
      const uint32_t key = score_key(s);
      const bool c = valid && !take_all && key >= tkey;
      const uint64_t m = __ballot(c);
      if (c) {
        const uint32_t at = wcount + count + (uint32_t)__popcll(m & earlier);
        if (at < (uint32_t)CAND_STAGE) stage[wave][at] = cand_entry(key, row);
        kmax = max(kmax, key);
      }
      count += (uint32_t)__popcll(m);
    }
    if (lane == 0) segcnt[j] = count;
    wcount += count;
  }
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    for (; j < SEGS_PER_TILE; j += SCORE_WAVES) segcnt[j] = 0u;    // segments past the end
    overflow[wave] = wcount > (uint32_t)CAND_STAGE ? 1u : 0u;
    wmax[wave] = kmax;
  }
  __syncthreads();
  // the tile's candidates in position order: segment jj's entries start at
  // segoff[jj] (the counts of segments 0 .. jj-1) in the output and at sstart[jj]
  // (the counts of the same wave's earlier segments) in its wave's stage
  if (wave == 0) {
    const uint32_t c = lane < SEGS_PER_TILE ? segcnt[lane] : 0u;
    const uint32_t inc = wave_incl_scan(c);
    if (lane < SEGS_PER_TILE) {
      segoff[lane + 1] = inc;
      uint32_t st = 0;
      for (int q = lane % SCORE_WAVES; q < lane; q += SCORE_WAVES) st += segcnt[q];
      sstart[lane] = st;
    }
    if (lane == 0) segoff[0] = 0u;
  }
  __syncthreads();
  bool ovf = false;
#pragma unroll
  for (int v = 0; v < SCORE_WAVES; ++v) ovf = ovf || overflow[v] != 0u;
  const uint32_t tot = segoff[SEGS_PER_TILE];
  if (!ovf) {
    // every thread writes entries e, e + 256, ...: coalesced, streamed past the caches
    uint32_t* wtile = cand + (size_t)unit * cand_stride + (size_t)blockIdx.x * TILE_ROWS;
    for (uint32_t e = threadIdx.x; e < tot; e += SCORE_THREADS) {
      int lo = 0, hi = SEGS_PER_TILE;            // the segment holding entry e
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (segoff[mid] <= e) lo = mid; else hi = mid;
      }
      __builtin_nontemporal_store(stage[lo % SCORE_WAVES][sstart[lo] + (e - segoff[lo])], wtile + e);
    }
  }
  if (threadIdx.x == 0) {
    uint32_t tmax = 0;
#pragma unroll
    for (int v = 0; v < SCORE_WAVES; ++v) tmax = max(tmax, wmax[v]);
    counts[(size_t)unit * ntile_cap + blockIdx.x] = ((uint64_t)tmax << 32) | (ovf ? TILE_OVERFLOW : tot);
  }
}

constexpr int SCORE_UNROLL = 2;

}  // namespace

hipError_t launch_prep(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                       const void* kproj_v, const int32_t* seq_len, int k, unsigned char* ws, hipStream_t st,
                       const PrepAppend* ap) {
  const unsigned char* kproj = static_cast<const unsigned char*>(kproj_v);
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
  float* qhat = reinterpret_cast<float*>(ws + L.off_qhat);
  uint32_t* tlow = reinterpret_cast<uint32_t*>(ws + L.off_tlow);
  const dim3 grid((unsigned)L.units), block(PREP_THREADS);
  const PrepAppend none{};
#define SJSA_PREP2(RR, KB)                                                                              \
  if (ap) prep_kernel<RR, KB, true><<<grid, block, 0, st>>>(q, M, kproj, seq_len, k, qhat, tlow, s.n_kv_heads, \
                                                              s.group, s.capacity, *ap);                   \
  else prep_kernel<RR, KB, false><<<grid, block, 0, st>>>(q, M, kproj, seq_len, k, qhat, tlow, s.n_kv_heads,  \
                                                            s.group, s.capacity, none)
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
  const unsigned char* kproj = static_cast<const unsigned char*>(kproj_v);
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
  const float* qhat = reinterpret_cast<const float*>(ws + L.off_qhat);
  const uint32_t* tlow = reinterpret_cast<const uint32_t*>(ws + L.off_tlow);
  float* scores = reinterpret_cast<float*>(ws + L.off_scores);
  uint32_t* cand = reinterpret_cast<uint32_t*>(ws + L.off_cand);
  uint64_t* counts = reinterpret_cast<uint64_t*>(ws + L.off_counts);
  const dim3 grid((unsigned)((s.capacity + TILE_ROWS - 1) / TILE_ROWS), (unsigned)L.units), block(SCORE_THREADS);
  const bool dense = (s.flags & SJSA_FLAG_WRITE_SCORES) != 0;
#define SJSA_SCAN2(RR, KB, DD)                                                                     \
  score_kernel<RR, KB, SCORE_UNROLL, DD><<<grid, block, 0, st>>>(kproj, qhat, tlow, seq_len, scores, cand, \
                                                             counts, s.n_kv_heads, s.capacity,       \
                                                             L.score_stride, L.ntile_cap, L.cand_stride)
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

}  // namespace sjsa

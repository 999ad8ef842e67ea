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
//              divide by G), q_hat = M_h q_bar (fp32), and clears this unit's
//              first-digit histogram for the scan.
// score_kernel (grid = tiles x units): streams Kproj rows with 128-bit coalesced
//              loads, each lane holding 8 of a row's r values; the partial dots of
//              the r/8 lanes of a row are reduced with DPP lane moves in a
//              transposed pattern, so that after the reduction each lane owns the
//              full score of one row. Scores are written as fp32, and a histogram
//              of their top 12 key bits is accumulated for the top-k stage.
#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int PREP_THREADS = 256;
constexpr int SCORE_THREADS = 256;
constexpr int SCORE_WAVES = SCORE_THREADS / 64;
constexpr int GROUP_ROWS = 64;       // rows covered by r/8 wave-wide 16-byte loads
constexpr int SAMPLES = 2048;        // rows scored by the prep kernel to place the threshold

// Radix select over `cnt` u32 keys in LDS with PREP_THREADS threads: the key of
// rank m (1 = largest). Three rounds of 11, 11 and 10 bits; in each round a
// histogram of the keys that match the bits resolved so far is built, and the bin
// holding rank m is found with a block scan. hist needs 2048 words, scratch 8.
__device__ uint32_t lds_kth_largest(const uint32_t* keys, int cnt, uint32_t m, uint32_t* hist,
                                    uint32_t* scratch) {
  constexpr int NW = PREP_THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, mask = 0;
  for (int round = 0; round < 3; ++round) {
    const int sh = round == 0 ? 21 : (round == 1 ? 10 : 0);
    const int nb = round == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += PREP_THREADS) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < cnt; i += PREP_THREADS) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    const int per = nb / PREP_THREADS;
    const int lo = tid * per;
    uint32_t local = 0;
    for (int i = 0; i < per; ++i) local += hist[lo + i];
    const uint32_t inc = wave_incl_scan(local);
    if (lane == 63) scratch[2 + wave] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t t = scratch[2 + w];
      before += w < wave ? t : 0u;
      total += t;
    }
    uint32_t above = total - (inc + before);      // keys in bins above this thread's range
    if (above < m && m <= above + local) {
      for (int i = per - 1; i >= 0; --i) {
        const uint32_t c = hist[lo + i];
        if (above + c >= m) { scratch[0] = (uint32_t)(lo + i); scratch[1] = above; break; }
        above += c;
      }
    }
    __syncthreads();
    const uint32_t bsel = scratch[0];
    m -= scratch[1];
    prefix |= bsel << sh;
    mask |= (uint32_t)(nb - 1) << sh;
    __syncthreads();
  }
  return prefix;
}

// One workgroup per (b, h).
//  * q_bar in fp32 (sum in head order, then divide by G) and q_hat = M_h q_bar.
//  * Threshold for the scan: the scores of SAMPLES evenly spaced rows (all rows when
//    n <= SAMPLES) are ranked, and the key of rank m (see below) becomes the unit's
//    candidate threshold. The exact top k is among the rows that reach it unless the
//    sample misjudges the distribution, a case the select stage detects and handles
//    exactly.
//  * mode: 1 when k >= n (every position is selected and the scan has no work).
template <int R>
__global__ __launch_bounds__(PREP_THREADS) void prep_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ M, const uint16_t* __restrict__ kproj,
    const int32_t* __restrict__ seq_len, int k, float* __restrict__ qhat, uint32_t* __restrict__ tlow,
    int n_kv_heads, int group, int64_t cap) {
  __shared__ float sq[HEAD_DIM];
  __shared__ float sM[R * (HEAD_DIM + 1)];
  __shared__ float sqh[R];
  __shared__ uint32_t skey[SAMPLES];
  __shared__ uint32_t shist[2048];
  __shared__ uint32_t sscratch[8];
  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int h = unit - b * n_kv_heads;
  const int tid = threadIdx.x;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int64_t kk = min((int64_t)k, n);
  // stage M_h (r x d) in LDS with a padded row stride (conflict-free column reads);
  // all of a thread's loads are issued before any is stored
  constexpr int MV = R * HEAD_DIM / 4 / PREP_THREADS;    // float4 loads per thread
  {
    const f32x4* m4 = reinterpret_cast<const f32x4*>(M + (size_t)h * R * HEAD_DIM);
    f32x4 mv[MV];
#pragma unroll
    for (int i = 0; i < MV; ++i) mv[i] = m4[tid + i * PREP_THREADS];
#pragma unroll
    for (int i = 0; i < MV; ++i) {
      const int e = (tid + i * PREP_THREADS) * 4;
      const int j = e / HEAD_DIM, c = e - j * HEAD_DIM;
      float* dst = sM + j * (HEAD_DIM + 1) + c;
      dst[0] = mv[i].x; dst[1] = mv[i].y; dst[2] = mv[i].z; dst[3] = mv[i].w;
    }
  }
  if (tid < HEAD_DIM) {
    // q[b, h*G + g, tid] for every head g (G <= 8), all loads issued before the sum,
    // which runs in head order
    const uint16_t* qg = q + (size_t)unit * group * HEAD_DIM + tid;
    uint32_t qb[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) qb[g] = qg[(size_t)min(g, group - 1) * HEAD_DIM];
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < group) acc += __uint_as_float(qb[g] << 16);
    sq[tid] = acc / (float)group;
  }
  __syncthreads();
  if (tid < R) {
    const float* mr = sM + tid * (HEAD_DIM + 1);
    float acc = 0.f;
    for (int c = 0; c < HEAD_DIM; ++c) acc = fmaf(mr[c], sq[c], acc);
    qhat[(size_t)unit * QHAT_STRIDE + tid] = acc;
    sqh[tid] = acc;
  }
  __syncthreads();
  if (kk >= n) {          // take every position (also n = 0): no threshold needed
    if (tid == 0) { tlow[unit * 2] = 0u; tlow[unit * 2 + 1] = 1u; }
    return;
  }
  const int S = (int)min((int64_t)SAMPLES, n);
  float qreg[R];
#pragma unroll
  for (int i = 0; i < R; ++i) qreg[i] = sqh[i];
  const uint16_t* base = kproj + (size_t)unit * cap * R;
  // all sample rows of a thread are loaded before any is scored (positions past S
  // are clamped to sample S-1 and not stored), so the loads overlap
  constexpr int PER = SAMPLES / PREP_THREADS;
  float sc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sidx = min(tid + i * PREP_THREADS, S - 1);
    const int64_t pos = (n <= SAMPLES) ? sidx : (int64_t)sidx * n / SAMPLES;
    sc[i] = row_score<R>(qreg, base + pos * R);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (tid + i * PREP_THREADS < S) skey[tid + i * PREP_THREADS] = score_key(sc[i]);
  __syncthreads();
  // the number of samples at or above the true k-th key is Binomial(S, kk/n): taking
  // the sample of rank mean + 5 sd + 4 keeps the threshold below that key except with
  // probability ~1e-7, while about kk + 5 sd n/S rows reach it
  const double pk = (double)kk / (double)n;
  const double mu = (double)S * pk;
  int64_t m = (int64_t)ceil(mu + 5.0 * sqrt(mu * (1.0 - pk)) + 4.0);
  m = m < 1 ? 1 : (m > S ? S : m);
  const uint32_t t = lds_kth_largest(skey, S, (uint32_t)m, shist, sscratch);
  if (tid == 0) { tlow[unit * 2] = t; tlow[unit * 2 + 1] = 0u; }
}

// grid = (ceil(cap / TILE_ROWS), B * H_kv). A segment is the SEG_ROWS = 128 rows one
// wave covers in one iteration (UNROLL groups of 64); the waves of a workgroup take
// the tile's segments in turn (wave w: segments w, w + 4, ...), so the workgroup
// streams one contiguous region. Loads are 128-bit and coalesced, each lane holding
// 8 of a row's r values; the partial dots of the r/8 lanes of a row are reduced with
// DPP lane moves in a transposed pattern, after which lane (rs, p) owns the score of
// group row p*RPL + rs.
//
// Rows whose key reaches the unit's threshold are candidates, kept as (key, row)
// pairs in position order: with a ballot of the flags in lane order, the number of
// flagged rows before a row is the popcount of the ballot under a per-lane mask of
// the lanes that hold earlier rows (earlier lane columns, and this column above this
// lane). Each wave packs the candidates of its segments back to back, first into a
// wave-private LDS stage, and writes them out once at the end into its region of the
// candidate buffer (tile x, wave w: entries [x*TILE_ROWS + w*TILE_ROWS/4, +TILE_ROWS/4));
// writes in the middle of the stream cost far more HBM time than their size. Each
// segment's count goes to counts[]. With WRITE_DENSE every score is also stored.
template <int R, int UNROLL, bool WRITE_DENSE>
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(
    const uint16_t* __restrict__ kproj, const float* __restrict__ qhat, const uint32_t* __restrict__ tlow,
    const int32_t* __restrict__ seq_len, float* __restrict__ scores, uint64_t* __restrict__ cand,
    uint32_t* __restrict__ counts, int n_kv_heads, int64_t cap, int64_t stride, int64_t nseg_cap,
    int64_t cand_stride) {
  constexpr int LPR = R / 8;            // lanes per Kproj row (16 bytes each)
  constexpr int RPL = 64 / LPR;         // rows per wave-wide load
  static_assert(GROUP_ROWS * UNROLL == SEG_ROWS, "one wave iteration covers one segment");
  constexpr int SEGS_PER_TILE = TILE_ROWS / SEG_ROWS;
  constexpr int WAVE_REGION = TILE_ROWS / SCORE_WAVES;
  __shared__ uint64_t stage[SCORE_WAVES][CAND_STAGE];
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int n = (int)min((int64_t)max(seq_len[b], 0), cap);      // cap < 2^30
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg0 = blockIdx.x * SEGS_PER_TILE;
  if ((seg0 + wave) * SEG_ROWS >= n) return;   // this wave has no segment below n
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

  float qh[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qh[e] = qhat[(size_t)unit * QHAT_STRIDE + p * 8 + e];

  const uint16_t* base = kproj + (size_t)unit * cap * R + p * 8;
  float* srow = scores + (size_t)unit * stride;
  uint64_t* wreg = cand + (size_t)unit * cand_stride + (size_t)blockIdx.x * TILE_ROWS + (size_t)wave * WAVE_REGION;
  uint32_t* cnt_unit = counts + (size_t)unit * nseg_cap;
  const int last = n - 1;
  uint32_t wcount = 0;                     // candidates of this wave so far

  for (int j = wave; j < SEGS_PER_TILE; j += SCORE_WAVES) {
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
        w[u][i] = ld16_stream(base + (size_t)row * R);
      }
    }
    uint32_t count = 0;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float a[LPR];
#pragma unroll
      for (int i = 0; i < LPR; ++i) a[i] = dot8_bf16(qh, w[u][i]);
      const float s = transpose_reduce<LPR>(a, p);
      const int row = g0 + u * GROUP_ROWS + p * RPL + rs;
      const bool valid = row < n;
      if (WRITE_DENSE && valid) srow[row] = s;
      const uint32_t key = score_key(s);
      const bool c = valid && !take_all && key >= tkey;
      const uint64_t m = __ballot(c);
      if (c) {
        const uint32_t at = wcount + count + (uint32_t)__popcll(m & earlier);
        const uint64_t v = ((uint64_t)key << 32) | (uint64_t)(uint32_t)row;
        if (at < (uint32_t)CAND_STAGE) stage[wave][at] = v;
        else wreg[at] = v;                // stage full (more than CAND_STAGE candidates)
      }
      count += (uint32_t)__popcll(m);
    }
    if (lane == 0) cnt_unit[seg0 + j] = count;
    wcount += count;
  }
  // the stage is wave-private: order this wave's LDS writes before its reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t nst = min(wcount, (uint32_t)CAND_STAGE);
  for (uint32_t i = lane; i < nst; i += 64) wreg[i] = stage[wave][i];
}

constexpr int SCORE_UNROLL = 2;

}  // namespace

hipError_t launch_prep(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                       const uint16_t* kproj, const int32_t* seq_len, int k, unsigned char* ws, hipStream_t st) {
  float* qhat = reinterpret_cast<float*>(ws + L.off_qhat);
  uint32_t* tlow = reinterpret_cast<uint32_t*>(ws + L.off_tlow);
  const dim3 grid((unsigned)L.units), block(PREP_THREADS);
  switch (s.rank) {
    case 16: prep_kernel<16><<<grid, block, 0, st>>>(q, M, kproj, seq_len, k, qhat, tlow, s.n_kv_heads, s.group, s.capacity); break;
    case 32: prep_kernel<32><<<grid, block, 0, st>>>(q, M, kproj, seq_len, k, qhat, tlow, s.n_kv_heads, s.group, s.capacity); break;
    case 64: prep_kernel<64><<<grid, block, 0, st>>>(q, M, kproj, seq_len, k, qhat, tlow, s.n_kv_heads, s.group, s.capacity); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score(const sjsa_shape& s, const Layout& L, const uint16_t* kproj, const int32_t* seq_len,
                        unsigned char* ws, hipStream_t st) {
  const float* qhat = reinterpret_cast<const float*>(ws + L.off_qhat);
  const uint32_t* tlow = reinterpret_cast<const uint32_t*>(ws + L.off_tlow);
  float* scores = reinterpret_cast<float*>(ws + L.off_scores);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + L.off_cand);
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.off_counts);
  const dim3 grid((unsigned)((s.capacity + TILE_ROWS - 1) / TILE_ROWS), (unsigned)L.units), block(SCORE_THREADS);
  const bool dense = (s.flags & SJSA_FLAG_WRITE_SCORES) != 0;
#define SJSA_SCAN(RR, DD)                                                                          \
  score_kernel<RR, SCORE_UNROLL, DD><<<grid, block, 0, st>>>(kproj, qhat, tlow, seq_len, scores, cand, \
                                                             counts, s.n_kv_heads, s.capacity,       \
                                                             L.score_stride, L.nseg_cap, L.cand_stride)
  switch (s.rank) {
    case 16: if (dense) SJSA_SCAN(16, true); else SJSA_SCAN(16, false); break;
    case 32: if (dense) SJSA_SCAN(32, true); else SJSA_SCAN(32, false); break;
    case 64: if (dense) SJSA_SCAN(64, true); else SJSA_SCAN(64, false); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_SCAN
  return hipGetLastError();
}

}  // namespace sjsa

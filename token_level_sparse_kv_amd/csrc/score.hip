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

template <int R>
__global__ __launch_bounds__(PREP_THREADS) void prep_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ M, float* __restrict__ qhat,
    uint32_t* __restrict__ hist, int n_kv_heads, int group) {
  __shared__ float sq[HEAD_DIM];
  const int unit = blockIdx.x;
  const int h = unit % n_kv_heads;
  const int tid = threadIdx.x;
  if (tid < HEAD_DIM) {
    const uint16_t* qg = q + (size_t)unit * group * HEAD_DIM + tid;   // q[b, h*G + g, tid]
    float acc = 0.f;
    for (int g = 0; g < group; ++g) acc += __uint_as_float((uint32_t)qg[(size_t)g * HEAD_DIM] << 16);
    sq[tid] = acc / (float)group;
  }
  // clear this unit's histogram for the scan
  u32x4* hz = reinterpret_cast<u32x4*>(hist + (size_t)unit * HIST_BINS);
  for (int i = tid; i < HIST_BINS / 4; i += PREP_THREADS) hz[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  if (tid < R) {
    const float* mr = M + ((size_t)h * R + tid) * HEAD_DIM;
    float acc = 0.f;
    for (int c = 0; c < HEAD_DIM; ++c) acc = fmaf(mr[c], sq[c], acc);
    qhat[(size_t)unit * QHAT_STRIDE + tid] = acc;
  }
}

// After the reduction lane p (p = lane % LPR) holds the full sum for load index p.
// Stage with lane distance m: of the values still held, a lane keeps those whose
// load index has bit log2(m) equal to its own, and adds the partner's copy.
template <int LPR>
__device__ __forceinline__ float transpose_reduce(float (&a)[LPR], int p) {
  if constexpr (LPR == 1) {
    return a[0];
  } else {
    float b[LPR / 2];
    const bool odd = p & 1;
#pragma unroll
    for (int t = 0; t < LPR / 2; ++t) {
      const float keep = odd ? a[2 * t + 1] : a[2 * t];
      const float send = odd ? a[2 * t] : a[2 * t + 1];
      b[t] = keep + dpp<DPP_QUAD_XOR1>(send);
    }
    if constexpr (LPR == 2) {
      return b[0];
    } else {
      float c[LPR / 4];
      const bool b1 = (p >> 1) & 1;
#pragma unroll
      for (int t = 0; t < LPR / 4; ++t) {
        const float keep = b1 ? b[2 * t + 1] : b[2 * t];
        const float send = b1 ? b[2 * t] : b[2 * t + 1];
        c[t] = keep + dpp<DPP_QUAD_XOR2>(send);
      }
      if constexpr (LPR == 4) {
        return c[0];
      } else {
        const bool b2 = (p >> 2) & 1;
        const float keep = b2 ? c[1] : c[0];
        const float send = b2 ? c[0] : c[1];
        return keep + swz_xor4(send);
      }
    }
  }
}

// grid = (ceil(cap / tile_rows), B * H_kv)
template <int R, int UNROLL>
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(
    const uint16_t* __restrict__ kproj, const float* __restrict__ qhat,
    const int32_t* __restrict__ seq_len, float* __restrict__ scores, uint32_t* __restrict__ hist,
    int n_kv_heads, int64_t cap, int64_t stride, int tile_rows) {
  constexpr int LPR = R / 8;            // lanes per Kproj row (16 bytes each)
  constexpr int RPL = 64 / LPR;         // rows per wave-wide load
  __shared__ uint32_t lh[HIST_BINS];

  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int64_t row0 = (int64_t)blockIdx.x * tile_rows;
  if (row0 >= n) return;
  const int64_t row_end = min(row0 + (int64_t)tile_rows, n);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p = lane % LPR;
  const int rs = lane / LPR;

  float qh[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qh[e] = qhat[(size_t)unit * QHAT_STRIDE + p * 8 + e];
  for (int i = tid; i < HIST_BINS; i += SCORE_THREADS) lh[i] = 0u;
  __syncthreads();

  const uint16_t* base = kproj + (size_t)unit * cap * R + p * 8;
  float* srow = scores + (size_t)unit * stride;

  for (int64_t g0 = row0 + (int64_t)wave * GROUP_ROWS * UNROLL; g0 < row_end;
       g0 += (int64_t)SCORE_WAVES * GROUP_ROWS * UNROLL) {
    u32x4 w[UNROLL][LPR];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
      for (int i = 0; i < LPR; ++i) {
        // rows past the end are clamped to the last valid row (their score is not stored),
        // so every load is unconditional and the whole batch stays in flight
        const int64_t row = min(g0 + u * GROUP_ROWS + i * RPL + rs, row_end - 1);
        w[u][i] = ld16_stream(base + row * R);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float a[LPR];
#pragma unroll
      for (int i = 0; i < LPR; ++i) a[i] = dot8_bf16(qh, w[u][i]);
      const float s = transpose_reduce<LPR>(a, p);
      const int64_t row = g0 + u * GROUP_ROWS + p * RPL + rs;
      if (row < row_end) {
        srow[row] = s;
        atomicAdd(&lh[score_key(s) >> HIST_SHIFT], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = hist + (size_t)unit * HIST_BINS;
  for (int i = tid; i < HIST_BINS; i += SCORE_THREADS) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

constexpr int SCORE_UNROLL = 2;
constexpr int SCORE_TILE_ROWS = 4096;

}  // namespace

hipError_t launch_prep(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                       unsigned char* ws, hipStream_t st) {
  float* qhat = reinterpret_cast<float*>(ws + L.off_qhat);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.off_hist);
  const dim3 grid((unsigned)L.units), block(PREP_THREADS);
  switch (s.rank) {
    case 16: prep_kernel<16><<<grid, block, 0, st>>>(q, M, qhat, hist, s.n_kv_heads, s.group); break;
    case 32: prep_kernel<32><<<grid, block, 0, st>>>(q, M, qhat, hist, s.n_kv_heads, s.group); break;
    case 64: prep_kernel<64><<<grid, block, 0, st>>>(q, M, qhat, hist, s.n_kv_heads, s.group); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score(const sjsa_shape& s, const Layout& L, const uint16_t* kproj, const int32_t* seq_len,
                        unsigned char* ws, hipStream_t st) {
  const float* qhat = reinterpret_cast<const float*>(ws + L.off_qhat);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.off_hist);
  float* scores = reinterpret_cast<float*>(ws + L.off_scores);
  const int tile = SCORE_TILE_ROWS;
  const dim3 grid((unsigned)((s.capacity + tile - 1) / tile), (unsigned)L.units), block(SCORE_THREADS);
  switch (s.rank) {
    case 16: score_kernel<16, SCORE_UNROLL><<<grid, block, 0, st>>>(kproj, qhat, seq_len, scores, hist, s.n_kv_heads, s.capacity, L.score_stride, tile); break;
    case 32: score_kernel<32, SCORE_UNROLL><<<grid, block, 0, st>>>(kproj, qhat, seq_len, scores, hist, s.n_kv_heads, s.capacity, L.score_stride, tile); break;
    case 64: score_kernel<64, SCORE_UNROLL><<<grid, block, 0, st>>>(kproj, qhat, seq_len, scores, hist, s.n_kv_heads, s.capacity, L.score_stride, tile); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sjsa

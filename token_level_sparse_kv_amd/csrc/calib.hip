// Calibration of the scoring basis: second moments accumulated on the GPU during
// a dense prefill, then the closed-form basis on the host.
//
// Source: JSSA article, section 校准:一次前向 + 一次特征分解 (one dense prefill per
// calibration sequence accumulates, per layer and KV head, the second moments of the
// group-mean query and of the key; then one eigendecomposition per layer and KV
// head), section 迹归一化 (each moment normalized to unit trace) and section 闭式谱解
// (the basis rows are the top-r eigenvectors of the sum of the normalized moments).
//
// calib_mfma_kernel: grid (nwg_q + nwg_k, H_kv), 512 threads, one workgroup per CU (its
// LDS). Workgroups [0, nwg_q) accumulate the group-mean query's moment (fp32 sum of the
// G bf16 heads in head order, divided by G), the rest the bf16 key's; each takes a
// contiguous slice of the B*T positions. Only the upper triangle of the symmetric
// 128 x 128 moment is formed: its 36 tiles of 16 x 16 (tile row bi <= tile column bj),
// each a sum over positions p of x_p[16 bi ..] x_p[16 bj ..]^T on the matrix cores:
//  * keys: v_mfma_f32_16x16x32_bf16, 32 positions per instruction; products of two
//    bf16 values are exact in fp32;
//  * mean queries: v_mfma_f32_16x16x4_f32, 4 positions per instruction.
// Waves 4-7 load the rows (128 query or 256 key positions per stage) and write them
// transposed (dim-major) into a double-buffered LDS stage, so a lane's operand fragment
// (one dim x 4 or 8 positions of the instruction's K) is one 16-byte read; waves 0-3
// take 9 tiles each, chosen so a wave reads one fragment per 16-dim block it touches
// (4 or 6) and reuses it across its tiles. The fp32 tile sums are folded into fp64
// sums held in the multiplying lanes' registers every 256 key positions and every
// 128 query positions (whose products are rounded), so no element's fp32 run exceeds
// 256 rounding steps. At the end each workgroup writes its fp64 tiles to the workspace;
// calib_reduce_kernel adds them in workgroup order (deterministic) into the caller's
// fp64 accumulators, mirroring the upper triangle into the lower one.
#include <math.h>
#include <string.h>

#include <vector>

#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int CAL_THREADS = 512;          // waves 0-3 multiply, waves 4-7 load and stage
constexpr int CAL_MMA_THREADS = 256;
constexpr int CAL_TILES = 36;             // upper-triangle 16 x 16 tiles of a 128 x 128 moment
constexpr int CAL_TPW = CAL_TILES / (CAL_MMA_THREADS / 64);   // tiles per product wave
constexpr int CAL_PK = 256;               // key positions staged at a time
constexpr int CAL_FOLD_Q = 128;           // query positions per fp32 run
constexpr int CAL_FOLD_K = 256;           // key positions per fp32 run
// query positions staged at a time: 128 KB of query rows per stage up to G = 4
template <int G>
constexpr int cal_pq() { return G <= 4 ? 128 : 64; }
constexpr int cal_ldf(int p) { return p + 4; }   // fp32 row pitch of staged queries (floats)
constexpr int cal_ldb(int p) { return p + 8; }   // bf16 row pitch of staged keys (halves)
constexpr int CAL_STAGE_BYTES = HEAD_DIM * cal_ldf(128) * 4 > HEAD_DIM * cal_ldb(CAL_PK) * 2
                                    ? HEAD_DIM * cal_ldf(128) * 4
                                    : HEAD_DIM * cal_ldb(CAL_PK) * 2;
static_assert(CAL_TILES % (CAL_MMA_THREADS / 64) == 0, "tiles split evenly over the product waves");
static_assert(CAL_FOLD_K % CAL_PK == 0 && CAL_FOLD_Q % 64 == 0, "runs hold whole stages");

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Tile t of the upper triangle, row-major over (bi, bj), bi <= bj < 8.
__host__ __device__ constexpr int tile_index(int bi, int bj) { return bi * 8 - bi * (bi - 1) / 2 + (bj - bi); }

// The four product waves' tiles, 9 each, chosen so that a wave's tiles touch few
// 16-dim blocks: one operand fragment per block is read from LDS per instruction step
// and reused by all the wave's tiles in that block (4 or 6 reads per 9 products instead
// of 18). Wave 0: the upper triangle of blocks 0..3 without (3, 3); wave 1: that of
// blocks 4..7 without (7, 7); wave 2: blocks 0..3 x 4..5 and (3, 3); wave 3: blocks
// 0..3 x 6..7 and (7, 7).
template <int W>
struct WaveTiles;
template <>
struct WaveTiles<0> {
  static constexpr int nb = 4;
  static constexpr int blk[6] = {0, 1, 2, 3, 0, 0};
  static constexpr int ta[CAL_TPW] = {0, 0, 0, 0, 1, 1, 1, 2, 2};
  static constexpr int tb[CAL_TPW] = {0, 1, 2, 3, 1, 2, 3, 2, 3};
};
template <>
struct WaveTiles<1> {
  static constexpr int nb = 4;
  static constexpr int blk[6] = {4, 5, 6, 7, 0, 0};
  static constexpr int ta[CAL_TPW] = {0, 0, 0, 0, 1, 1, 1, 2, 2};
  static constexpr int tb[CAL_TPW] = {0, 1, 2, 3, 1, 2, 3, 2, 3};
};
template <>
struct WaveTiles<2> {
  static constexpr int nb = 6;
  static constexpr int blk[6] = {0, 1, 2, 3, 4, 5};
  static constexpr int ta[CAL_TPW] = {0, 1, 2, 3, 0, 1, 2, 3, 3};
  static constexpr int tb[CAL_TPW] = {4, 4, 4, 4, 5, 5, 5, 5, 3};
};
template <>
struct WaveTiles<3> {
  static constexpr int nb = 6;
  static constexpr int blk[6] = {0, 1, 2, 3, 6, 7};
  static constexpr int ta[CAL_TPW] = {0, 1, 2, 3, 0, 1, 2, 3, 5};
  static constexpr int tb[CAL_TPW] = {4, 4, 4, 4, 5, 5, 5, 5, 5};
};

struct CalShared {
  __attribute__((aligned(16))) float stage[2][CAL_STAGE_BYTES / 4];   // staged positions, dim-major (double buffer)
};

constexpr bool wave_tiles_cover_once() {
  int seen[CAL_TILES] = {};
  const int* tabs[4][3] = {{WaveTiles<0>::blk, WaveTiles<0>::ta, WaveTiles<0>::tb},
                           {WaveTiles<1>::blk, WaveTiles<1>::ta, WaveTiles<1>::tb},
                           {WaveTiles<2>::blk, WaveTiles<2>::ta, WaveTiles<2>::tb},
                           {WaveTiles<3>::blk, WaveTiles<3>::ta, WaveTiles<3>::tb}};
  for (int w = 0; w < 4; ++w)
    for (int u = 0; u < CAL_TPW; ++u) {
      const int bi = tabs[w][0][tabs[w][1][u]], bj = tabs[w][0][tabs[w][2][u]];
      if (bi > bj) return false;
      ++seen[tile_index(bi, bj)];
    }
  for (int t = 0; t < CAL_TILES; ++t)
    if (seen[t] != 1) return false;
  return true;
}
static_assert(wave_tiles_cover_once(), "the waves' tiles are the upper triangle, each once");

// One stage's products for wave W: per instruction step, one fragment per block of the
// wave (lane (lg, li): dim 16 blk + li at the step's positions 4 lg .. 4 lg + 3 for the
// fp32 queries, 8 lg .. 8 lg + 7 for the bf16 keys), then the wave's 9 tiles.
template <int W, bool IS_Q, int P>
__device__ __forceinline__ void calib_products(const float* XF, const uint16_t* XB, int li, int lg,
                                               f32x4_t (&acc)[CAL_TPW]) {
  using WT = WaveTiles<W>;
  if constexpr (IS_Q) {
    constexpr int LD = cal_ldf(P);
#pragma unroll 1
    for (int c0 = 0; c0 < P; c0 += 16) {
      f32x4_t f[WT::nb];
#pragma unroll
      for (int b = 0; b < WT::nb; ++b)
        f[b] = *reinterpret_cast<const f32x4_t*>(&XF[(16 * WT::blk[b] + li) * LD + c0 + 4 * lg]);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
        for (int u = 0; u < CAL_TPW; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(f[WT::ta[u]][s4], f[WT::tb[u]][s4], acc[u], 0, 0, 0);
      }
    }
  } else {
    constexpr int LD = cal_ldb(P);
#pragma unroll 2
    for (int c0 = 0; c0 < P; c0 += 32) {
      bf16x8_t f[WT::nb];
#pragma unroll
      for (int b = 0; b < WT::nb; ++b)
        f[b] = *reinterpret_cast<const bf16x8_t*>(&XB[(16 * WT::blk[b] + li) * LD + c0 + 8 * lg]);
#pragma unroll
      for (int u = 0; u < CAL_TPW; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[WT::ta[u]], f[WT::tb[u]], acc[u], 0, 0, 0);
    }
  }
}

// One workgroup's slice: IS_Q selects the mean query's moment (G heads per position)
// or the key's. Waves 0-3 multiply (9 tiles each) and keep the fp64 sums of their
// tiles in registers (lane (lg, li) owns rows 4 lg + v, column li of each tile);
// waves 4-7 load the next stage while the current one is multiplied and then write it,
// transposed, into the other half of a double-buffered LDS stage; one barrier per stage
// hands a buffer from the loaders to the multipliers. A stage is large (128 KB of query
// rows at G = 4, 64 KB of key rows), so one stage of loads in flight keeps the CU's
// share of the HBM stream busy. Loader thread lt stages the 8-dim chunk c = lt / 16 of
// the position groups j = lt % 16 + 16 i (4 consecutive positions each); a load
// instruction of a wave so reads 64 bytes of each of 16 rows, the four loader waves
// the rest of those rows, and each LDS write (4 positions of one dim) falls on its own
// banks.
template <int G, bool IS_Q>
__device__ __forceinline__ void calib_body(CalShared& sh, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k, int n_kv_heads, int64_t T, int64_t rows,
                                           int wg, int64_t chunk, double* __restrict__ out) {
  constexpr int P = IS_Q ? cal_pq<G>() : CAL_PK;  // positions per stage
  constexpr int NG = P / 64;                    // position groups per loader thread
  constexpr int NH = IS_Q ? G : 1;              // head rows loaded per position
  constexpr int LDF = cal_ldf(P), LDB = cal_ldb(P);
  constexpr int FOLD = IS_Q ? CAL_FOLD_Q : CAL_FOLD_K;
  static_assert(FOLD % P == 0 && HEAD_DIM * (IS_Q ? LDF * 4 : LDB * 2) <= CAL_STAGE_BYTES, "stage fits");
  const int h = blockIdx.y;
  const int64_t r0 = (int64_t)wg * chunk;
  const int64_t r1 = min(r0 + chunk, rows);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave >= CAL_MMA_THREADS / 64;
  const int lt = tid - CAL_MMA_THREADS;         // loader thread index
  const int n_q_heads = n_kv_heads * G;
  const int li = lane & 15, lg = lane >> 4;
  const int c = (lt >> 4) & 15;
  const int64_t nst = r1 > r0 ? (r1 - r0 + P - 1) / P : 0;

  u32x4 raw[NG][4][NH];                         // [group][position in group][head]
  // (sequence, position) of a row from the stage's first row by one division per stage:
  // a stage spans fewer than T rows unless T < P
  auto load_stage = [&](int64_t base) {
    const int64_t b0 = base / T, t0 = base - b0 * T;
    const int64_t last = r1 - 1 - base;          // rows past the slice read its last row (unused)
#pragma unroll
    for (int i = 0; i < NG; ++i) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int64_t off = 4 * ((lt & 15) + 16 * i) + s4;
        int64_t t = t0 + (off < last ? off : last), b = b0;
        if (t >= T) {
          if (T >= P) {
            t -= T;
            ++b;
          } else {
            const int64_t w = t / T;
            b += w;
            t -= w * T;
          }
        }
        if constexpr (IS_Q) {
#pragma unroll
          for (int g = 0; g < G; ++g)
            raw[i][s4][g] = ld16(q + (((size_t)b * n_q_heads + (size_t)h * G + g) * T + t) * HEAD_DIM + 8 * c);
        } else {
          raw[i][s4][0] = ld16(k + (((size_t)b * n_kv_heads + h) * T + t) * HEAD_DIM + 8 * c);
        }
      }
    }
  };
  auto store_stage = [&](int64_t base, float* XF) {
    uint16_t* XB = reinterpret_cast<uint16_t*>(XF);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int p0 = 4 * ((lt & 15) + 16 * i);
      bool valid[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) valid[s4] = base + p0 + s4 < r1;
      if constexpr (IS_Q) {
        float v[4][8];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[s4][e] = 0.f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const u32x4 w = raw[i][s4][g];
            v[s4][0] += bf_lo(w.x); v[s4][1] += bf_hi(w.x); v[s4][2] += bf_lo(w.y); v[s4][3] += bf_hi(w.y);
            v[s4][4] += bf_lo(w.z); v[s4][5] += bf_hi(w.z); v[s4][6] += bf_lo(w.w); v[s4][7] += bf_hi(w.w);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f32x4_t o;
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) o[s4] = valid[s4] ? v[s4][e] / (float)G : 0.f;
          *reinterpret_cast<f32x4_t*>(&XF[(8 * c + e) * LDF + p0]) = o;
        }
      } else {
        uint32_t w[4][4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const u32x4 x = raw[i][s4][0];
          w[s4][0] = valid[s4] ? x.x : 0u; w[s4][1] = valid[s4] ? x.y : 0u;
          w[s4][2] = valid[s4] ? x.z : 0u; w[s4][3] = valid[s4] ? x.w : 0u;
        }
        // dims 8 c + 2 e (low halves) and 8 c + 2 e + 1 (high halves), positions p0 .. p0 + 3
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint2 lo = make_uint2((w[0][e] & 0xffffu) | (w[1][e] << 16), (w[2][e] & 0xffffu) | (w[3][e] << 16));
          const uint2 hi = make_uint2((w[0][e] >> 16) | (w[1][e] & 0xffff0000u),
                                      (w[2][e] >> 16) | (w[3][e] & 0xffff0000u));
          *reinterpret_cast<uint2*>(&XB[(8 * c + 2 * e) * LDB + p0]) = lo;
          *reinterpret_cast<uint2*>(&XB[(8 * c + 2 * e + 1) * LDB + p0]) = hi;
        }
      }
    }
  };

  // The two roles run separate loops with one barrier per stage each (the same count);
  // stage s sits in buffer s & 1. Loads past the last stage repeat the last one (never
  // multiplied), so every iteration issues the same loads.
  if (loader) {
    if (nst > 0) {
      load_stage(r0);
      store_stage(r0, sh.stage[0]);
      load_stage(r0 + min((int64_t)1, nst - 1) * P);
    }
    __syncthreads();
    for (int64_t st = 0; st < nst; ++st) {
      store_stage(r0 + min(st + 1, nst - 1) * P, sh.stage[(st + 1) & 1]);
      load_stage(r0 + min(st + 2, nst - 1) * P);
      __syncthreads();
    }
  } else {
    f32x4_t acc[CAL_TPW];
    double sum[CAL_TPW][4];
#pragma unroll
    for (int u = 0; u < CAL_TPW; ++u) {
      acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) sum[u][v] = 0.0;
    }
    auto fold = [&]() {
#pragma unroll
      for (int u = 0; u < CAL_TPW; ++u) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sum[u][v] += (double)acc[u][v];
        acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    };
    __syncthreads();
    int staged = 0;                             // positions in the current fp32 run
    for (int64_t st = 0; st < nst; ++st) {
      const float* XF = sh.stage[st & 1];
      const uint16_t* XB = reinterpret_cast<const uint16_t*>(XF);
      switch (wave) {
        case 0: calib_products<0, IS_Q, P>(XF, XB, li, lg, acc); break;
        case 1: calib_products<1, IS_Q, P>(XF, XB, li, lg, acc); break;
        case 2: calib_products<2, IS_Q, P>(XF, XB, li, lg, acc); break;
        default: calib_products<3, IS_Q, P>(XF, XB, li, lg, acc); break;
      }
      // fp32 runs of at most 128 query positions (rounded products) or 256 key positions
      staged += P;
      if (staged == FOLD) { fold(); staged = 0; }
      __syncthreads();
    }
    fold();
    // the wave's tiles' fp64 sums, each element written by the lane that owns it
    auto write = [&](auto wt) {
      using WT = decltype(wt);
#pragma unroll
      for (int u = 0; u < CAL_TPW; ++u) {
        double* o = out + tile_index(WT::blk[WT::ta[u]], WT::blk[WT::tb[u]]) * 256 + (4 * lg) * 16 + li;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v * 16] = sum[u][v];
      }
    };
    switch (wave) {
      case 0: write(WaveTiles<0>{}); break;
      case 1: write(WaveTiles<1>{}); break;
      case 2: write(WaveTiles<2>{}); break;
      default: write(WaveTiles<3>{}); break;
    }
  }
}

template <int G>
__global__ __launch_bounds__(CAL_THREADS) void calib_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int n_kv_heads, int64_t T, int64_t rows,
    int nwg_q, int64_t chunk_q, int64_t chunk_k, double* __restrict__ part) {
  __shared__ CalShared sh;
  double* out = part + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * CAL_TILES * 256;
  if ((int)blockIdx.x < nwg_q)
    calib_body<G, true>(sh, q, k, n_kv_heads, T, rows, (int)blockIdx.x, chunk_q, out);
  else
    calib_body<G, false>(sh, q, k, n_kv_heads, T, rows, (int)blockIdx.x - nwg_q, chunk_k, out);
}

// grid (CAL_TILES, H_kv, 2), 256 threads: thread e of workgroup (t, h, mat) sums tile
// t's element e over the workgroups' partial tiles, in workgroup order (deterministic),
// and adds the sum to the caller's accumulator at (i, j) and, off the diagonal tiles,
// at (j, i) as well (the lower triangle mirrors the upper one).
__global__ __launch_bounds__(256) void calib_reduce_kernel(const double* __restrict__ part, int nwg_q, int nwg_k,
                                                           double* __restrict__ SQ, double* __restrict__ SK) {
  const int t = blockIdx.x, h = blockIdx.y, mat = blockIdx.z, e = threadIdx.x;
  int bi = 0, r = t;
  while (r >= 8 - bi) { r -= 8 - bi; ++bi; }
  const int bj = bi + r;
  const int i = 16 * bi + e / 16, j = 16 * bj + e % 16;
  const int nwg = nwg_q + nwg_k;
  const int w0 = mat == 0 ? 0 : nwg_q, w1 = mat == 0 ? nwg_q : nwg;
  const double* p = part + ((size_t)h * nwg) * CAL_TILES * 256 + (size_t)t * 256 + e;
  constexpr int RU = 32;                         // partials loaded at once
  double s = 0.0;
  for (int w = w0; w < w1; w += RU) {
    double x[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) x[u] = p[(size_t)min(w + u, w1 - 1) * CAL_TILES * 256];
#pragma unroll
    for (int u = 0; u < RU; ++u)
      if (w + u < w1) s += x[u];
  }
  double* dst = (mat == 0 ? SQ : SK) + (size_t)h * HEAD_DIM * HEAD_DIM;
  dst[i * HEAD_DIM + j] += s;
  if (bi != bj) dst[j * HEAD_DIM + i] += s;
}

}  // namespace

// Workgroups per KV head: one workgroup fits a CU, so about 256 in all, seven eighths
// of them for the mean queries (G head rows per position, converted and multiplied in
// fp32; at G = 4 and 8 KV heads the 28 : 4 split beat 24 : 8, 26 : 6, 27 : 5 and
// 29 : 3); never more than one per 256 positions.
void calib_groups(const sjsa_shape& s, int64_t rows, int* nwg_q, int* nwg_k) {
  auto limit = [&](int64_t want) {
    const int64_t by_rows = (rows + 255) / 256;
    const int64_t n = want < by_rows ? want : by_rows;
    return (int)(n < 1 ? 1 : n);
  };
  const int64_t per_head = (256 + s.n_kv_heads - 1) / s.n_kv_heads;
  const int64_t q_share = per_head * 7 / 8;
  *nwg_q = limit(q_share);
  *nwg_k = limit(per_head - q_share);
}

size_t calib_part_bytes(const sjsa_shape& s, int64_t rows) {
  int nq, nk;
  calib_groups(s, rows, &nq, &nk);
  return (size_t)s.n_kv_heads * (nq + nk) * CAL_TILES * 256 * sizeof(double);
}

hipError_t launch_calib(const sjsa_shape& s, const uint16_t* q, const uint16_t* k, int64_t T, double* SQ,
                        double* SK, unsigned char* ws, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * T;
  int nwg_q, nwg_k;
  calib_groups(s, rows, &nwg_q, &nwg_k);
  const int64_t chunk_q = ((rows + nwg_q - 1) / nwg_q + 127) / 128 * 128;   // whole query stages
  const int64_t chunk_k = ((rows + nwg_k - 1) / nwg_k + CAL_PK - 1) / CAL_PK * CAL_PK;
  double* part = reinterpret_cast<double*>(ws);
  const dim3 grid((unsigned)(nwg_q + nwg_k), (unsigned)s.n_kv_heads);
  switch (s.group) {
#define SJSA_CAL(GG) \
    case GG: calib_mfma_kernel<GG><<<grid, dim3(CAL_THREADS), 0, st>>>(q, k, s.n_kv_heads, T, rows, nwg_q, chunk_q, \
                                                                    chunk_k, part); break;
    SJSA_CAL(1) SJSA_CAL(2) SJSA_CAL(4) SJSA_CAL(8)
#undef SJSA_CAL
    default: return hipErrorInvalidValue;
  }
  calib_reduce_kernel<<<dim3(CAL_TILES, (unsigned)s.n_kv_heads, 2), dim3(256), 0, st>>>(
      part, nwg_q, nwg_k, SQ, SK);
  return hipGetLastError();
}

// Host: eigenvalues and eigenvectors of a symmetric d x d matrix by cyclic Jacobi
// rotations (fp64). On return A's diagonal holds the eigenvalues and the columns of V
// the eigenvectors. Sweeps stop once the off-diagonal mass is below 1e-30 of the
// total (or after 100 sweeps).
void jacobi_eigen(std::vector<double>& A, std::vector<double>& V, int d) {
  V.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) V[(size_t)i * d + i] = 1.0;
  auto a = [&](int i, int j) -> double& { return A[(size_t)i * d + j]; };
  double total = 0.0;
  for (size_t i = 0; i < A.size(); ++i) total += A[i] * A[i];
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q2 = p + 1; q2 < d; ++q2) off += 2.0 * a(p, q2) * a(p, q2);
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int p = 0; p < d; ++p) {
      for (int r = p + 1; r < d; ++r) {
        const double apr = a(p, r);
        if (apr == 0.0) continue;
        const double theta = (a(r, r) - a(p, p)) / (2.0 * apr);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int i = 0; i < d; ++i) {            // columns p, r
          const double aip = a(i, p), air = a(i, r);
          a(i, p) = c * aip - s * air;
          a(i, r) = s * aip + c * air;
        }
        for (int j = 0; j < d; ++j) {            // rows p, r
          const double apj = a(p, j), arj = a(r, j);
          a(p, j) = c * apj - s * arj;
          a(r, j) = s * apj + c * arj;
        }
        a(p, r) = 0.0;
        a(r, p) = 0.0;
        for (int i = 0; i < d; ++i) {
          const double vip = V[(size_t)i * d + p], vir = V[(size_t)i * d + r];
          V[(size_t)i * d + p] = c * vip - s * vir;
          V[(size_t)i * d + r] = s * vip + c * vir;
        }
      }
    }
  }
}

}  // namespace sjsa

using namespace sjsa;

extern "C" {

size_t sjsa_calib_workspace_size(const sjsa_shape* shape, int64_t n_tokens) {
  if (!shape || shape->batch < 1 || shape->n_kv_heads < 1 || shape->head_dim != HEAD_DIM || n_tokens < 1) return 0;
  if (shape->group != 1 && shape->group != 2 && shape->group != 4 && shape->group != 8) return 0;
  return calib_part_bytes(*shape, (int64_t)shape->batch * n_tokens);
}

int sjsa_calib_accumulate(const sjsa_shape* shape, const void* q, const void* k, int64_t n_tokens, double* SQ,
                          double* SK, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape) return SJSA_ERR_NULL;
  if (shape->batch < 1 || shape->n_kv_heads < 1 || n_tokens < 1) return SJSA_ERR_DIMS;
  if ((int64_t)shape->batch * n_tokens > ((int64_t)1 << 40)) return SJSA_ERR_DIMS;
  if (shape->head_dim != HEAD_DIM) return SJSA_ERR_UNSUPPORTED;
  if (shape->group != 1 && shape->group != 2 && shape->group != 4 && shape->group != 8) return SJSA_ERR_UNSUPPORTED;
  if (!q || !k || !SQ || !SK || !workspace) return SJSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) % 16 ||
      (reinterpret_cast<uintptr_t>(SQ) | reinterpret_cast<uintptr_t>(SK) | reinterpret_cast<uintptr_t>(workspace)) % 8)
    return SJSA_ERR_ALIGN;
  if (workspace_bytes < sjsa_calib_workspace_size(shape, n_tokens)) return SJSA_ERR_WORKSPACE;
  const hipError_t e = launch_calib(*shape, (const uint16_t*)q, (const uint16_t*)k, n_tokens, SQ, SK,
                                    (unsigned char*)workspace, (hipStream_t)stream);
  return e == hipSuccess ? SJSA_OK : SJSA_ERR_HIP;
}

int sjsa_calib_basis(const double* SQ, const double* SK, int32_t n_kv_heads, int32_t d, int32_t r, float* M,
                     double* eigenvalues) {
  if (!SQ || !SK || !M) return SJSA_ERR_NULL;
  if (n_kv_heads < 1 || d < 1 || d > 4096 || r < 1 || r > d) return SJSA_ERR_DIMS;
  std::vector<double> A((size_t)d * d), V;
  std::vector<int> order(d);
  for (int h = 0; h < n_kv_heads; ++h) {
    const double* sq = SQ + (size_t)h * d * d;
    const double* sk = SK + (size_t)h * d * d;
    double tq = 0.0, tk = 0.0;
    for (int i = 0; i < d; ++i) { tq += sq[(size_t)i * d + i]; tk += sk[(size_t)i * d + i]; }
    if (!(tq > 0.0) || !(tk > 0.0)) return SJSA_ERR_DIMS;       // no samples, or not finite
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        // symmetrized sum of the trace-normalized moments
        const size_t ij = (size_t)i * d + j, ji = (size_t)j * d + i;
        A[ij] = 0.5 * ((sq[ij] + sq[ji]) / tq + (sk[ij] + sk[ji]) / tk);
      }
    jacobi_eigen(A, V, d);
    for (int i = 0; i < d; ++i) order[i] = i;
    // descending eigenvalues; equal ones keep index order
    for (int i = 1; i < d; ++i) {
      const int o = order[i];
      const double w = A[(size_t)o * d + o];
      int j = i - 1;
      while (j >= 0 && A[(size_t)order[j] * d + order[j]] < w) { order[j + 1] = order[j]; --j; }
      order[j + 1] = o;
    }
    for (int i = 0; i < r; ++i) {
      const int c = order[i];
      // sign: the component of largest magnitude is positive (first one on ties)
      int arg = 0;
      for (int j = 1; j < d; ++j)
        if (fabs(V[(size_t)j * d + c]) > fabs(V[(size_t)arg * d + c])) arg = j;
      const double sgn = V[(size_t)arg * d + c] < 0 ? -1.0 : 1.0;
      for (int j = 0; j < d; ++j) M[((size_t)h * r + i) * d + j] = (float)(sgn * V[(size_t)j * d + c]);
    }
    if (eigenvalues)
      for (int i = 0; i < d; ++i) eigenvalues[(size_t)h * d + i] = A[(size_t)order[i] * d + order[i]];
  }
  return SJSA_OK;
}

}  // extern "C"

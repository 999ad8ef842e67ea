// Calibration of the scoring basis: second moments accumulated on the GPU during
// a dense prefill, then the closed-form basis on the host.
//
// Source: JSSA article, section 校准:一次前向 + 一次特征分解 (one dense prefill per
// calibration sequence accumulates, per layer and KV head, the second moments of the
// group-mean query and of the key; then one eigendecomposition per layer and KV
// head), section 迹归一化 (each moment normalized to unit trace) and section 闭式谱解
// (the basis rows are the top-r eigenvectors of the sum of the normalized moments).
//
// calib_partial_kernel: grid (nwg, H_kv, 2), 256 threads. Workgroup w of (head h,
// matrix m) takes a contiguous slice of the B*T positions; m = 0 stages the
// group-mean query of each position (fp32 sum of the G bf16 heads in head order,
// divided by G), m = 1 the bf16 key, 32 positions at a time in LDS. Thread (ty, tx)
// owns the 8x8 output block rows 8ty.., columns 8tx..; it accumulates x_i x_j in
// fp32 and folds the fp32 sums into fp64 every 256 positions, so the fp32 rounding
// covers at most 256 products per element. The fp64 partials go to the workspace
// and calib_reduce_kernel adds them, in workgroup order, into the caller's fp64
// accumulators (deterministic).
#include <math.h>
#include <string.h>

#include <vector>

#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int CAL_THREADS = 256;
constexpr int CAL_ROWS = 32;          // positions staged per LDS tile
constexpr int CAL_FOLD_TILES = 8;     // fp32 sums folded into fp64 every 8 tiles (256 positions)
constexpr int CAL_LD = HEAD_DIM + 4;  // padded LDS row

template <int G>
__global__ __launch_bounds__(CAL_THREADS) void calib_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int n_kv_heads, int64_t T, int64_t rows,
    int64_t chunk, double* __restrict__ part) {
  __shared__ float X[CAL_ROWS][CAL_LD];
  const int h = blockIdx.y;
  const int mat = blockIdx.z;
  const int wg = blockIdx.x;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int64_t r0 = (int64_t)wg * chunk;
  const int64_t r1 = min(r0 + chunk, rows);
  const int n_q_heads = n_kv_heads * G;

  float a32[8][8];
  double a64[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) { a32[i][j] = 0.f; a64[i][j] = 0.0; }

  int tiles = 0;
  for (int64_t base = r0; base < r1; base += CAL_ROWS) {
    // stage 32 positions: 16 lanes x 8 values per position row
    for (int c = tid; c < CAL_ROWS * 16; c += CAL_THREADS) {
      const int rr = c >> 4, part8 = (c & 15) * 8;
      const int64_t r = base + rr;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (r < r1) {
        const int64_t b = r / T, t = r - b * T;
        if (mat == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const u32x4 w = ld16(q + (((size_t)b * n_q_heads + (size_t)h * G + g) * T + t) * HEAD_DIM + part8);
            v[0] += bf_lo(w.x); v[1] += bf_hi(w.x); v[2] += bf_lo(w.y); v[3] += bf_hi(w.y);
            v[4] += bf_lo(w.z); v[5] += bf_hi(w.z); v[6] += bf_lo(w.w); v[7] += bf_hi(w.w);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] / (float)G;
        } else {
          const u32x4 w = ld16(k + (((size_t)b * n_kv_heads + h) * T + t) * HEAD_DIM + part8);
          v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
          v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) X[rr][part8 + e] = v[e];
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < CAL_ROWS; ++rr) {
      float xi[8], xj[8];
      const float4 i0 = *reinterpret_cast<const float4*>(&X[rr][8 * ty]);
      const float4 i1 = *reinterpret_cast<const float4*>(&X[rr][8 * ty + 4]);
      const float4 j0 = *reinterpret_cast<const float4*>(&X[rr][8 * tx]);
      const float4 j1 = *reinterpret_cast<const float4*>(&X[rr][8 * tx + 4]);
      xi[0] = i0.x; xi[1] = i0.y; xi[2] = i0.z; xi[3] = i0.w; xi[4] = i1.x; xi[5] = i1.y; xi[6] = i1.z; xi[7] = i1.w;
      xj[0] = j0.x; xj[1] = j0.y; xj[2] = j0.z; xj[3] = j0.w; xj[4] = j1.x; xj[5] = j1.y; xj[6] = j1.z; xj[7] = j1.w;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) a32[i][j] = fmaf(xi[i], xj[j], a32[i][j]);
    }
    __syncthreads();
    if (++tiles == CAL_FOLD_TILES) {
      tiles = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) { a64[i][j] += (double)a32[i][j]; a32[i][j] = 0.f; }
    }
  }
  double* out = part + (((size_t)h * 2 + mat) * gridDim.x + wg) * HEAD_DIM * HEAD_DIM;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) out[(size_t)(8 * ty + i) * HEAD_DIM + 8 * tx + j] = a64[i][j] + (double)a32[i][j];
}

// grid (HEAD_DIM * HEAD_DIM / 256, H_kv, 2): acc[h][i][j] += sum over workgroups.
__global__ __launch_bounds__(256) void calib_reduce_kernel(const double* __restrict__ part, int nwg,
                                                           double* __restrict__ SQ, double* __restrict__ SK) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, mat = blockIdx.z;
  const double* p = part + ((size_t)h * 2 + mat) * nwg * HEAD_DIM * HEAD_DIM + e;
  double s = 0.0;
  for (int w = 0; w < nwg; ++w) s += p[(size_t)w * HEAD_DIM * HEAD_DIM];
  double* dst = (mat == 0 ? SQ : SK) + (size_t)h * HEAD_DIM * HEAD_DIM + e;
  *dst += s;
}

}  // namespace

int calib_groups(const sjsa_shape& s, int64_t rows) {
  const int64_t per_matrix = (512 + 2 * s.n_kv_heads - 1) / (2 * s.n_kv_heads);
  const int64_t by_rows = (rows + 255) / 256;
  int64_t n = per_matrix < by_rows ? per_matrix : by_rows;
  return (int)(n < 1 ? 1 : n);
}

hipError_t launch_calib(const sjsa_shape& s, const uint16_t* q, const uint16_t* k, int64_t T, double* SQ,
                        double* SK, unsigned char* ws, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * T;
  const int nwg = calib_groups(s, rows);
  const int64_t chunk = (rows + nwg - 1) / nwg;
  double* part = reinterpret_cast<double*>(ws);
  const dim3 grid((unsigned)nwg, (unsigned)s.n_kv_heads, 2);
  switch (s.group) {
    case 1: calib_partial_kernel<1><<<grid, dim3(CAL_THREADS), 0, st>>>(q, k, s.n_kv_heads, T, rows, chunk, part); break;
    case 2: calib_partial_kernel<2><<<grid, dim3(CAL_THREADS), 0, st>>>(q, k, s.n_kv_heads, T, rows, chunk, part); break;
    case 4: calib_partial_kernel<4><<<grid, dim3(CAL_THREADS), 0, st>>>(q, k, s.n_kv_heads, T, rows, chunk, part); break;
    case 8: calib_partial_kernel<8><<<grid, dim3(CAL_THREADS), 0, st>>>(q, k, s.n_kv_heads, T, rows, chunk, part); break;
    default: return hipErrorInvalidValue;
  }
  calib_reduce_kernel<<<dim3(HEAD_DIM * HEAD_DIM / 256, (unsigned)s.n_kv_heads, 2), dim3(256), 0, st>>>(
      part, nwg, SQ, SK);
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
  const int nwg = calib_groups(*shape, (int64_t)shape->batch * n_tokens);
  return (size_t)shape->n_kv_heads * 2 * nwg * HEAD_DIM * HEAD_DIM * sizeof(double);
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

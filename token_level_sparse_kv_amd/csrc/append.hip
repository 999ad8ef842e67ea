// Cache append: write the new tokens' K and V rows and their projected scoring
// rows Kproj = bf16_rne(M_h k_new) (fp32 dot over d).
// Source: JSSA article, section 投影打分缓存与校准成本 (the scoring cache Kproj =
// K M^T is kept next to the original KV cache) and section 组件级拆解 (projecting
// each new key is the pipeline's cheapest stage).
#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr int APPEND_THREADS = 256;
constexpr int APPEND_ROWS = 64;                 // token rows per workgroup
constexpr int LDS_ROW = HEAD_DIM + 1;           // padded LDS row (no bank conflicts)

// grid = (ceil(n_new / APPEND_ROWS), B * H_kv)
template <int R>
__global__ __launch_bounds__(APPEND_THREADS) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int n_new,
    const float* __restrict__ M, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ K, uint16_t* __restrict__ V, uint16_t* __restrict__ Kproj,
    int n_kv_heads, int64_t cap) {
  __shared__ float sM[R * LDS_ROW];
  __shared__ float sk[APPEND_ROWS * LDS_ROW];

  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int h = unit - b * n_kv_heads;
  const int t0 = blockIdx.x * APPEND_ROWS;
  const int rows = min(APPEND_ROWS, n_new - t0);
  const int64_t p0 = (int64_t)pos[b] + t0;
  const int tid = threadIdx.x;

  const float* Mh = M + (size_t)h * R * HEAD_DIM;
  for (int i = tid; i < R * HEAD_DIM; i += APPEND_THREADS) {
    const int j = i / HEAD_DIM, c = i - j * HEAD_DIM;
    sM[j * LDS_ROW + c] = Mh[i];
  }

  // K / V rows: 16 lanes x 16 bytes per 256-byte row.
  const size_t src_base = ((size_t)unit * n_new + t0) * HEAD_DIM;
  for (int i = tid; i < APPEND_ROWS * 16; i += APPEND_THREADS) {
    const int r = i >> 4, part = i & 15;
    if (r < rows) {
      const u32x4 kw = ld16(k_new + src_base + (size_t)r * HEAD_DIM + part * 8);
      const u32x4 vw = ld16(v_new + src_base + (size_t)r * HEAD_DIM + part * 8);
      const int64_t p = p0 + r;
      if (p >= 0 && p < cap) {
        const size_t dst = ((size_t)unit * cap + p) * HEAD_DIM + part * 8;
        *reinterpret_cast<u32x4*>(K + dst) = kw;
        *reinterpret_cast<u32x4*>(V + dst) = vw;
      }
      float* dstk = sk + r * LDS_ROW + part * 8;
      dstk[0] = bf_lo(kw.x); dstk[1] = bf_hi(kw.x);
      dstk[2] = bf_lo(kw.y); dstk[3] = bf_hi(kw.y);
      dstk[4] = bf_lo(kw.z); dstk[5] = bf_hi(kw.z);
      dstk[6] = bf_lo(kw.w); dstk[7] = bf_hi(kw.w);
    }
  }
  __syncthreads();

  // Kproj rows: one (row, output) pair per thread iteration, fp32 dot in channel order.
  for (int o = tid; o < APPEND_ROWS * R; o += APPEND_THREADS) {
    const int r = o / R, j = o - r * R;
    if (r >= rows) continue;
    const int64_t p = p0 + r;
    if (p < 0 || p >= cap) continue;
    const float* mr = sM + j * LDS_ROW;
    const float* kr = sk + r * LDS_ROW;
    float acc = 0.f;
#pragma unroll 16
    for (int c = 0; c < HEAD_DIM; ++c) acc = fmaf(mr[c], kr[c], acc);
    Kproj[((size_t)unit * cap + p) * R + j] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

}  // namespace

hipError_t launch_append(const sjsa_shape& s, const uint16_t* k_new, const uint16_t* v_new, int n_new,
                         const float* M, const int32_t* pos, uint16_t* K, uint16_t* V, uint16_t* Kproj,
                         hipStream_t st) {
  const dim3 grid((n_new + APPEND_ROWS - 1) / APPEND_ROWS, s.batch * s.n_kv_heads);
  const dim3 block(APPEND_THREADS);
  switch (s.rank) {
    case 16: append_kernel<16><<<grid, block, 0, st>>>(k_new, v_new, n_new, M, pos, K, V, Kproj, s.n_kv_heads, s.capacity); break;
    case 32: append_kernel<32><<<grid, block, 0, st>>>(k_new, v_new, n_new, M, pos, K, V, Kproj, s.n_kv_heads, s.capacity); break;
    case 64: append_kernel<64><<<grid, block, 0, st>>>(k_new, v_new, n_new, M, pos, K, V, Kproj, s.n_kv_heads, s.capacity); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sjsa

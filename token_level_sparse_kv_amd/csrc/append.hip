// Cache append: write the new tokens' K and V rows and their projected scoring
// rows Kproj = M_h k_new (fp32 dot over d, rounded to bf16 or, with
// SJSA_FLAG_KPROJ_FP8, to FP8 E4M3).
// Source: JSSA article, section 投影打分缓存与校准成本 (the scoring cache Kproj =
// K M^T is kept next to the original KV cache) and section 组件级拆解 (projecting
// each new key is the pipeline's cheapest stage).
#include "key_proj.h"

namespace sjsa {
namespace {

constexpr int APPEND_THREADS = 256;
constexpr int APPEND_ROWS = 64;                 // token rows per workgroup

// grid = (ceil(n_new / APPEND_ROWS), B * H_kv). Threads copy the workgroup's K and
// V rows (16 bytes each), then project them with the KeyProj layout, each thread
// holding its basis slice in registers for all the workgroup's rows, so a projected
// row's bits do not depend on how many tokens one call appends.
template <int R, int KB>
__global__ __launch_bounds__(APPEND_THREADS) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int n_new,
    const float* __restrict__ M, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ K, uint16_t* __restrict__ V, unsigned char* __restrict__ Kproj,
    int n_kv_heads, int64_t cap) {
  using KP = KeyProj<R>;
  static_assert(KP::THREADS == APPEND_THREADS, "one projection layout");
  constexpr int TPO = KP::TPO, CH = KP::CH;
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int h = unit - b * n_kv_heads;
  const int t0 = blockIdx.x * APPEND_ROWS;
  const int rows = min(APPEND_ROWS, n_new - t0);
  const int64_t p0 = (int64_t)pos[b] + t0;
  const int tid = threadIdx.x;
  const size_t src0 = ((size_t)unit * n_new + t0) * HEAD_DIM;

  for (int w = tid; w < rows * 32; w += APPEND_THREADS) {
    const int r = w >> 5, part = w & 15;
    const int64_t p = p0 + r;
    if (p < 0 || p >= cap) continue;
    const bool is_v = (w >> 4) & 1;
    const size_t off = (size_t)r * HEAD_DIM + part * 8;
    const u32x4 x = ld16((is_v ? v_new : k_new) + src0 + off);
    *reinterpret_cast<u32x4*>((is_v ? V : K) + ((size_t)unit * cap + p) * HEAD_DIM + part * 8) = x;
  }

  const int i = tid / TPO, part = tid % TPO;
  f32x4 mv[CH / 4];
  KP::load_basis(M + (size_t)h * R * HEAD_DIM, tid, mv);
  for (int r = 0; r < rows; ++r) {
    u32x4 kv[CH / 8];
    KP::load_key(k_new + src0 + (size_t)r * HEAD_DIM, tid, kv);
    const float acc = KP::dot(mv, kv);
    const int64_t p = p0 + r;
    if (part == 0 && p >= 0 && p < cap) KP::template store<KB>(Kproj + ((size_t)unit * cap + p) * R * KB, i, acc);
  }
}

}  // namespace

hipError_t launch_append(const sjsa_shape& s, const uint16_t* k_new, const uint16_t* v_new, int n_new,
                         const float* M, const int32_t* pos, uint16_t* K, uint16_t* V, void* Kproj_v,
                         hipStream_t st) {
  unsigned char* Kproj = static_cast<unsigned char*>(Kproj_v);
  const bool fp8 = (s.flags & SJSA_FLAG_KPROJ_FP8) != 0;
  const dim3 block(APPEND_THREADS);
  const dim3 grid((n_new + APPEND_ROWS - 1) / APPEND_ROWS, s.batch * s.n_kv_heads);
#define SJSA_APPEND(RR)                                                                                          \
  if (fp8) append_kernel<RR, 1><<<grid, block, 0, st>>>(k_new, v_new, n_new, M, pos, K, V, Kproj, s.n_kv_heads, \
                                                         s.capacity);                                            \
  else append_kernel<RR, 2><<<grid, block, 0, st>>>(k_new, v_new, n_new, M, pos, K, V, Kproj, s.n_kv_heads,      \
                                                     s.capacity)
  switch (s.rank) {
    case 16: SJSA_APPEND(16); break;
    case 32: SJSA_APPEND(32); break;
    case 64: SJSA_APPEND(64); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_APPEND
  return hipGetLastError();
}

}  // namespace sjsa

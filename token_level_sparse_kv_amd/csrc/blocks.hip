// Block-sparse decode (NSA-style block selection over a block-key cache, with an
// optional INT4 form of that cache).
//
// Sources: the NSA tutorial page ("稀疏注意力:每个 query 只挑一部分历史去读"): a
// block's summary key exists once the block is complete; the block score is the
// softmax of q . key / sqrt(head_size) over the visible blocks, summed over the
// query heads that share a K/V head, which then select together; the current
// block, the first block and the local blocks are always selected. The
// SpotAttention abstract page: the selector's key cache can be held in INT4.
//
// Kernels:
//   * block_keys_kernel: the key of a complete block is the mean of its keys (fp32
//     sum in row order, divided by the block size, rounded to bf16); optionally also
//     its INT4 form: per group of 64 elements, scale = fp16(absmax / 7) and codes
//     clamp(rint(x / scale), -7, 7), two codes per byte (low nibble first);
//   * block_score_kernel: per (sequence, KV head) and 64 blocks, the exp2-domain
//     logits z[g][j] = sm_scale * log2(e) * q_g . key_j of every query head over the
//     complete blocks, plus each tile's per-head (max, sum of 2^(z - max));
//   * block_select_kernel: merges the tiles' (max, sum) into each head's softmax,
//     scores s_j = sum_g 2^(z[g][j] - max_g) / sum_g, keeps the forced blocks plus
//     the best others (unit_select.h) and writes the kept blocks' positions; the
//     attention kernel then reads those rows in place.
#include "unit_select.h"

namespace sjsa {
namespace {

constexpr float BLK_LOG2E = 1.4426950408889634f;
constexpr int BLK_TILE = 64;              // blocks per scoring workgroup
constexpr int BLK_SLOTS = 16;             // 16-lane row slots per scoring workgroup
constexpr int BLK_LDS_SCORES = 8192;      // block scores staged in LDS up to this many blocks
constexpr int INT4_GROUP = 64;

// Copy of new K and V rows into the caches (rows outside [0, cap) are skipped).
__global__ __launch_bounds__(256) void kv_rows_kernel(const uint16_t* __restrict__ k_new,
                                                      const uint16_t* __restrict__ v_new, int n_new,
                                                      const int32_t* __restrict__ pos, uint16_t* __restrict__ K,
                                                      uint16_t* __restrict__ V, int n_kv_heads, int64_t cap) {
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int t0 = blockIdx.x * 64;
  const int rows = min(64, n_new - t0);
  const int64_t p0 = (int64_t)pos[b] + t0;
  const size_t src0 = ((size_t)unit * n_new + t0) * HEAD_DIM;
  for (int w = threadIdx.x; w < rows * 32; w += 256) {
    const int r = w >> 5, part = w & 15;
    const int64_t p = p0 + r;
    if (p < 0 || p >= cap) continue;
    const bool is_v = (w >> 4) & 1;
    const u32x4 x = ld16((is_v ? v_new : k_new) + src0 + (size_t)r * HEAD_DIM + part * 8);
    *reinterpret_cast<u32x4*>((is_v ? V : K) + ((size_t)unit * cap + p) * HEAD_DIM + part * 8) = x;
  }
}

// grid = (blocks to consider, B * H_kv), 128 threads (thread c owns dimension c).
// pos == nullptr: block j = blockIdx.x, kept if it is complete (j < floor(n_b / bs)).
// pos != nullptr: block j = floor(pos_b / bs) + blockIdx.x, kept if its last row lies
// in the rows [pos_b, pos_b + n_new) just written and inside the capacity.
__global__ __launch_bounds__(HEAD_DIM) void block_keys_kernel(
    const uint16_t* __restrict__ K, const int32_t* __restrict__ seq_len, const int32_t* __restrict__ pos,
    int n_new, int n_kv_heads, int64_t cap, int bs, int64_t nblk_cap, uint16_t* __restrict__ Kc,
    unsigned char* __restrict__ Kq, uint16_t* __restrict__ Ks) {
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  int64_t j;
  if (pos == nullptr) {
    j = blockIdx.x;
    const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
    if (j >= n / bs) return;
  } else {
    const int64_t p0 = pos[b];
    if (p0 < 0) return;
    j = p0 / bs + blockIdx.x;
    const int64_t end = (j + 1) * bs;            // one past the block's last row
    if (end <= p0 || end > p0 + n_new || j >= nblk_cap) return;
  }
  const int c = threadIdx.x;
  const uint16_t* kr = K + ((size_t)unit * cap + (size_t)j * bs) * HEAD_DIM + c;
  float sum = 0.f;
  for (int r = 0; r < bs; ++r) sum += __uint_as_float((uint32_t)kr[(size_t)r * HEAD_DIM] << 16);
  const uint32_t kb = f32_to_bf16_rne(sum / (float)bs);
  const size_t row = (size_t)unit * nblk_cap + j;
  if (Kc) Kc[row * HEAD_DIM + c] = (uint16_t)kb;
  if (Kq) {
    // one wave per group of 64 elements (HEAD_DIM = 2 groups)
    const float x = __uint_as_float(kb << 16);
    const float absmax = wave_max_f32(fabsf(x));
    const _Float16 sh = (_Float16)fminf(absmax / 7.f, 65504.f);
    const float scale = (float)sh;
    const int code = scale > 0.f ? (int)fminf(fmaxf(rintf(x / scale), -7.f), 7.f) : 0;
    const int other = __shfl_xor(code, 1);
    if ((c & 1) == 0) Kq[row * (HEAD_DIM / 2) + c / 2] = (unsigned char)((code & 0xF) | ((other & 0xF) << 4));
    if ((c & 63) == 0) Ks[row * (HEAD_DIM / INT4_GROUP) + c / INT4_GROUP] = __builtin_bit_cast(uint16_t, sh);
  }
}

// grid = (ceil(nblk_cap / BLK_TILE), B * H_kv), 256 threads = 16 slots of 16 lanes;
// lane t of a slot holds dimensions 8t .. 8t+7 of a block key. INT4: the key is
// codes (4 bytes per lane) times its group's scale.
template <int G, bool INT4>
__global__ __launch_bounds__(256) void block_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc, const unsigned char* __restrict__ Kq,
    const uint16_t* __restrict__ Ks, const int32_t* __restrict__ seq_len, int n_kv_heads, int64_t cap, int bs,
    int64_t nblk_cap, float qscale, float* __restrict__ z, int64_t zstride, float* __restrict__ ms,
    int ntile) {
  __shared__ float sq[G][HEAD_DIM];
  __shared__ float smax[BLK_SLOTS][G];
  __shared__ float ssum[BLK_SLOTS][G];
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int64_t m = n / bs;                     // complete blocks
  const int tid = threadIdx.x, slot = tid >> 4, t = tid & 15;
  const int64_t j0 = (int64_t)blockIdx.x * BLK_TILE;
  for (int i = tid; i < G * HEAD_DIM; i += 256)
    sq[i / HEAD_DIM][i % HEAD_DIM] = __uint_as_float((uint32_t)q[(size_t)unit * G * HEAD_DIM + i] << 16);
  __syncthreads();
  float mx[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; sm[g] = 0.f; }
#pragma unroll
  for (int r = 0; r < BLK_TILE / BLK_SLOTS; ++r) {
    const int64_t j = j0 + r * BLK_SLOTS + slot;
    const bool ok = j < m;
    const size_t row = (size_t)unit * nblk_cap + (ok ? j : 0);
    float kv[8];
    if (INT4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(Kq + row * (HEAD_DIM / 2) + t * 4);
      const float scale = (float)__builtin_bit_cast(_Float16, Ks[row * (HEAD_DIM / INT4_GROUP) + t / 8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int code = ((int)(w << (28 - 4 * e))) >> 28;      // sign-extended nibble e
        kv[e] = (float)code * scale;
      }
    } else {
      const u32x4 w = ld16(Kc + row * HEAD_DIM + t * 8);
      kv[0] = bf_lo(w.x); kv[1] = bf_hi(w.x); kv[2] = bf_lo(w.y); kv[3] = bf_hi(w.y);
      kv[4] = bf_lo(w.z); kv[5] = bf_hi(w.z); kv[6] = bf_lo(w.w); kv[7] = bf_hi(w.w);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(sq[g][t * 8 + e], kv[e], a);
      a = row16_sum(a) * qscale;
      if (ok) {
        if (t == g) z[((size_t)unit * G + g) * zstride + j] = a;
        const float nm = fmaxf(mx[g], a);
        sm[g] = sm[g] * exp2f(mx[g] - nm) + exp2f(a - nm);
        mx[g] = nm;
      }
    }
  }
  if (t == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { smax[slot][g] = mx[g]; ssum[slot][g] = sm[g]; }
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int s = 0; s < BLK_SLOTS; ++s) M = fmaxf(M, smax[s][tid]);
    float S = 0.f;
    if (M != -INFINITY)
      for (int s = 0; s < BLK_SLOTS; ++s)
        if (smax[s][tid] != -INFINITY) S += ssum[s][tid] * exp2f(smax[s][tid] - M);
    float* o = ms + (((size_t)unit * ntile + blockIdx.x) * G + tid) * 2;
    o[0] = M;
    o[1] = S;
  }
}

// grid = B * H_kv, SEL_UNIT_THREADS threads.
template <int G>
__global__ __launch_bounds__(SEL_UNIT_THREADS) void block_select_kernel(
    const float* __restrict__ z, int64_t zstride, const float* __restrict__ ms, int ntile,
    const int32_t* __restrict__ seq_len, int n_kv_heads, int64_t cap, int bs, int k_blocks, int n_init,
    int n_local, int32_t* __restrict__ idx, int ktok, float inv_bs) {
  __shared__ float ss[BLK_LDS_SCORES];
  __shared__ UnitSelectShared sh;
  __shared__ float head_m[G], head_s[G];
  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int m = (int)(n / bs);                       // complete blocks (scored)
  const int nb = (int)((n + bs - 1) / bs);           // all blocks
  const int tid = threadIdx.x;
  if (tid < G) {
    // each head's softmax normaliser from the tiles' (max, sum) pairs, in tile order
    float M = -INFINITY, S = 0.f;
    const int tiles = (m + BLK_TILE - 1) / BLK_TILE;
    for (int i = 0; i < tiles; ++i) {
      const float* p = ms + (((size_t)unit * ntile + i) * G + tid) * 2;
      const float tm = p[0], ts = p[1];
      if (tm == -INFINITY) continue;
      const float nm = fmaxf(M, tm);
      S = S * exp2f(M - nm) + ts * exp2f(tm - nm);
      M = nm;
    }
    head_m[tid] = M;
    head_s[tid] = S > 0.f ? 1.f / S : 0.f;
  }
  __syncthreads();
  const bool staged = m <= BLK_LDS_SCORES;
  const float* zu = z + (size_t)unit * G * zstride;
  auto score_of = [&](int j) -> float {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) s += exp2f(zu[(size_t)g * zstride + j] - head_m[g]) * head_s[g];
    return s;
  };
  if (staged) {
    for (int j = tid; j < m; j += SEL_UNIT_THREADS) ss[j] = score_of(j);
    __syncthreads();
  }
  auto score = [&](int j) -> float { return staged ? ss[j] : score_of(j); };

  const int cur = nb - 1;
  const int lo_local = cur - n_local + 1;
  auto forced = [&](int j) { return j < n_init || j >= lo_local; };
  auto eligible = [&](int j) { return j < m && !forced(j); };
  const int a_cnt = min(n_init, nb);
  const int l_cnt = n_local > 0 ? cur - max(lo_local, 0) + 1 : 0;
  const int overlap = n_local > 0 ? max(0, a_cnt - max(lo_local, 0)) : 0;
  const int nforced = a_cnt + l_cnt - overlap;
  const bool all = nb <= k_blocks;
  const uint32_t nsel = select_kept_units(nb, all, max(k_blocks - nforced, 0), score, forced, eligible, sh);
  write_kept_positions(sh, nsel, bs, inv_bs, n, ktok, idx + (size_t)unit * ktok, [](int, int, bool) {});
}

}  // namespace

hipError_t launch_kv_rows(const sjsa_shape& s, const uint16_t* k_new, const uint16_t* v_new, int n_new,
                          const int32_t* pos, uint16_t* K, uint16_t* V, hipStream_t st) {
  const dim3 grid((unsigned)((n_new + 63) / 64), (unsigned)((int64_t)s.batch * s.n_kv_heads));
  kv_rows_kernel<<<grid, dim3(256), 0, st>>>(k_new, v_new, n_new, pos, K, V, s.n_kv_heads, s.capacity);
  return hipGetLastError();
}

hipError_t launch_block_keys(const sjsa_shape& s, int bs, const uint16_t* K, const int32_t* seq_len,
                             const int32_t* pos, int n_new, uint16_t* Kc, unsigned char* Kq, uint16_t* Ks,
                             hipStream_t st) {
  const int64_t nblk_cap = s.capacity / bs;
  if (nblk_cap == 0) return hipGetLastError();
  const int64_t gx = pos ? (int64_t)n_new / bs + 1 : nblk_cap;
  const dim3 grid((unsigned)gx, (unsigned)((int64_t)s.batch * s.n_kv_heads));
  block_keys_kernel<<<grid, dim3(HEAD_DIM), 0, st>>>(K, seq_len, pos, n_new, s.n_kv_heads, s.capacity, bs, nblk_cap,
                                                     Kc, Kq, Ks);
  return hipGetLastError();
}

hipError_t launch_block_select(const sjsa_shape& s, const BlockLayout& L, int bs, const uint16_t* q,
                               const uint16_t* Kc, const unsigned char* Kq, const uint16_t* Ks,
                               const int32_t* seq_len, int k_blocks, int n_init, int n_local, float sm_scale,
                               int32_t* idx, unsigned char* ws, hipStream_t st) {
  float* z = reinterpret_cast<float*>(ws + L.off_z);
  float* ms = reinterpret_cast<float*>(ws + L.off_ms);
  const int64_t units = (int64_t)s.batch * s.n_kv_heads;
  const int ktok = k_blocks * bs;
  const float qscale = sm_scale * BLK_LOG2E;
  if (L.ntile > 0) {
    const dim3 grid((unsigned)L.ntile, (unsigned)units);
#define SJSA_BSCORE(GG)                                                                                          \
  if (Kc)                                                                                                        \
    block_score_kernel<GG, false><<<grid, dim3(256), 0, st>>>(q, Kc, Kq, Ks, seq_len, s.n_kv_heads, s.capacity,   \
                                                               bs, L.nblk_cap, qscale, z, L.zstride, ms, L.ntile); \
  else                                                                                                           \
    block_score_kernel<GG, true><<<grid, dim3(256), 0, st>>>(q, Kc, Kq, Ks, seq_len, s.n_kv_heads, s.capacity,    \
                                                              bs, L.nblk_cap, qscale, z, L.zstride, ms, L.ntile)
    switch (s.group) {
      case 1: SJSA_BSCORE(1); break;
      case 2: SJSA_BSCORE(2); break;
      case 4: SJSA_BSCORE(4); break;
      case 8: SJSA_BSCORE(8); break;
      default: return hipErrorInvalidValue;
    }
#undef SJSA_BSCORE
  }
  const dim3 grid((unsigned)units);
#define SJSA_BSEL(GG)                                                                                              \
  block_select_kernel<GG><<<grid, dim3(SEL_UNIT_THREADS), 0, st>>>(z, L.zstride, ms, L.ntile, seq_len,            \
                                                                   s.n_kv_heads, s.capacity, bs, k_blocks, n_init, \
                                                                   n_local, idx, ktok, 1.0f / (float)bs)
  switch (s.group) {
    case 1: SJSA_BSEL(1); break;
    case 2: SJSA_BSEL(2); break;
    case 4: SJSA_BSEL(4); break;
    case 8: SJSA_BSEL(8); break;
    default: return hipErrorInvalidValue;
  }
#undef SJSA_BSEL
  return hipGetLastError();
}

}  // namespace sjsa

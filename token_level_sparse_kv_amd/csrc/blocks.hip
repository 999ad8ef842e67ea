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
//   * block_score_mfma_kernel: per (sequence, KV head) and 64 blocks, the exp2-domain
//     logits z[g][j] = sm_scale * log2(e) * q_g . key_j of every query head over the
//     complete blocks (an MFMA product), plus each tile's per-head (max, sum of
//     2^(z - max));
//   * block_select_kernel: merges the tiles' (max, sum) into each head's softmax,
//     scores s_j = sum_g 2^(z[g][j] - max_g) / sum_g, keeps the forced blocks plus
//     the best others (unit_select.h) and writes the kept blocks' positions; the
//     attention kernel then reads those rows in place.
#include "unit_select.h"

namespace sjsa {
namespace {

constexpr float BLK_LOG2E = 1.4426950408889634f;
constexpr int BLK_TILE = 64;              // blocks per scoring workgroup
constexpr int BLK_LDS_SCORES = 8192;      // block scores staged in LDS up to this many blocks
constexpr int INT4_GROUP = 64;

typedef short s16x4 __attribute__((ext_vector_type(4)));

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

// grid = (ceil(nblk_cap / BLK_TILE), B * H_kv), 256 threads. The logits of a tile
// are a matrix product, Z = Q Kc^T per 16 blocks, on v_mfma_f32_16x16x16_bf16 (16
// heads, zero past G, by 16 blocks; bf16 products are exact, sums in fp32); wave w of
// the workgroup takes the tile's w-th group of 16 blocks. Lane l feeds head l % 16 (A) and block l % 16 (B) with contraction
// indices 4*(l/16)..+3 of each of 8 chunks, and receives heads 4*(l/16)..+3 of block
// l % 16 (D). The contraction order is a permutation of the dimensions chosen so a
// lane reads whole runs of its block's key: 32 consecutive dimensions (64 bytes) of a
// bf16 key, or two runs of 16 (8 bytes of codes each), one per INT4 scale group,
// whose partial products are accumulated and scaled separately.
template <int G, bool INT4>
__global__ __launch_bounds__(256) void block_score_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc, const unsigned char* __restrict__ Kq,
    const uint16_t* __restrict__ Ks, const int32_t* __restrict__ seq_len, int n_kv_heads, int64_t cap, int bs,
    int64_t nblk_cap, float qscale, float* __restrict__ z, int64_t zstride, float* __restrict__ ms,
    int ntile) {
  static_assert(BLK_TILE == 4 * 16, "four waves of 16 blocks per tile");
  __shared__ float wmax[4][G], wsum[4][G];
  const int unit = blockIdx.y;
  const int b = unit / n_kv_heads;
  const int64_t n = min((int64_t)max(seq_len[b], 0), cap);
  const int64_t m = n / bs;                     // complete blocks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, col = lane & 15;
  const int64_t blk = (int64_t)blockIdx.x * BLK_TILE + wave * 16 + col;
  const bool ok = blk < m;
  const size_t row = (size_t)unit * nblk_cap + (ok ? blk : 0);

  auto dim_of = [&](int c, int v) { return INT4 ? 64 * (c >> 2) + 16 * gq + 4 * (c & 3) + v : 32 * gq + 4 * c + v; };
  s16x4 a[8];
  const uint16_t* qh = q + ((size_t)unit * G + (col < G ? col : 0)) * HEAD_DIM;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) a[c][v] = col < G ? (short)qh[dim_of(c, v)] : (short)0;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!INT4) {
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = ld16(Kc + row * HEAD_DIM + 32 * gq + 8 * i);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 x = w[c >> 1];
      const uint32_t lo = (c & 1) ? x.z : x.x, hi = (c & 1) ? x.w : x.y;
      s16x4 bv;
      bv[0] = (short)(lo & 0xffffu); bv[1] = (short)(lo >> 16); bv[2] = (short)(hi & 0xffffu); bv[3] = (short)(hi >> 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[c], bv, acc, 0, 0, 0);
    }
  } else {
    const unsigned char* cr = Kq + row * (HEAD_DIM / 2);
    const uint2 p0 = *reinterpret_cast<const uint2*>(cr + 8 * gq);          // dims 16gq .. 16gq+15
    const uint2 p1 = *reinterpret_cast<const uint2*>(cr + 32 + 8 * gq);     // dims 64+16gq ..
    const uint16_t sc0 = Ks[row * (HEAD_DIM / INT4_GROUP)], sc1 = Ks[row * (HEAD_DIM / INT4_GROUP) + 1];
    f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint2 p = c < 4 ? p0 : p1;
      const uint32_t word = ((c & 3) < 2) ? p.x : p.y;
      s16x4 bv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int nib = 4 * (c & 1) + v;                              // nibble within the 32-bit word
        const int code = ((int)(word << (28 - 4 * nib))) >> 28;      // sign-extended
        bv[v] = (short)(__float_as_uint((float)code) >> 16);          // small integers are exact in bf16
      }
      if (c < 4) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[c], bv, acc, 0, 0, 0);
      else acc1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[c], bv, acc1, 0, 0, 0);
    }
    const float s0 = (float)__builtin_bit_cast(_Float16, sc0), s1 = (float)__builtin_bit_cast(_Float16, sc1);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = acc[v] * s0 + acc1[v] * s1;
  }
  // logits of heads 4*gq + v for this lane's block; each head's (max, sum) over the
  // wave's 16 blocks by row reductions (a DPP row is the 16 blocks of one head group)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * gq + v;
    const float zz = ok ? acc[v] * qscale : -INFINITY;
    if (h < G && ok) z[((size_t)unit * G + h) * zstride + blk] = zz;
    const float mx = row16_max(zz);
    const float e = mx == -INFINITY ? 0.f : exp2f(zz - mx);
    const float sm = row16_sum(e);
    if (col == 0 && h < G) { wmax[wave][h] = mx; wsum[wave][h] = sm; }
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wmax[w][tid]);
    float S = 0.f;
    if (M != -INFINITY)
      for (int w = 0; w < 4; ++w)
        if (wmax[w][tid] != -INFINITY) S += wsum[w][tid] * exp2f(wmax[w][tid] - M);
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
  const int lane = tid & 63, wave = tid >> 6;
  static_assert(G <= SEL_UNIT_THREADS / 64, "one wave per query head");
  if (wave < G) {
    // head `wave`'s softmax normaliser from the tiles' (max, sum) pairs: lane l
    // merges tiles l, l + 64, ... in order (all of a wave's loads in flight at
    // once), then the wave combines its lanes (max, then sum rescaled to it)
    float M = -INFINITY, S = 0.f;
    const int tiles = (m + BLK_TILE - 1) / BLK_TILE;
    for (int i = lane; i < tiles; i += 64) {
      const float* p = ms + (((size_t)unit * ntile + i) * G + wave) * 2;
      const float tm = p[0], ts = p[1];
      if (tm == -INFINITY) continue;
      const float nm = fmaxf(M, tm);
      S = S * exp2f(M - nm) + ts * exp2f(tm - nm);
      M = nm;
    }
    const float wm = wave_max_f32(M);
    float ws = M == -INFINITY ? 0.f : S * exp2f(M - wm);
    ws = row16_sum(ws);
    ws = (readlane_f32(ws, 0) + readlane_f32(ws, 16)) + (readlane_f32(ws, 32) + readlane_f32(ws, 48));
    if (lane == 0) {
      head_m[wave] = wm;
      head_s[wave] = ws > 0.f ? 1.f / ws : 0.f;
    }
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
    block_score_mfma_kernel<GG, false><<<grid, dim3(256), 0, st>>>(q, Kc, Kq, Ks, seq_len, s.n_kv_heads,         \
                                                                    s.capacity, bs, L.nblk_cap, qscale, z,        \
                                                                    L.zstride, ms, L.ntile);                      \
  else                                                                                                           \
    block_score_mfma_kernel<GG, true><<<grid, dim3(256), 0, st>>>(q, Kc, Kq, Ks, seq_len, s.n_kv_heads,          \
                                                                   s.capacity, bs, L.nblk_cap, qscale, z,         \
                                                                   L.zstride, ms, L.ntile)
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

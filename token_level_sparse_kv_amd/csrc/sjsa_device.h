// Device-side helpers shared by the gfx950 kernels of libsjsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sjsa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 halves of a 32-bit word (little endian: element 2i in the low half).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bit pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map of an fp32 score to a u32 key: a larger score gives a
// larger key; -0 and +0 share one key; every NaN maps to 0, below -inf (0x007fffff).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0u;
  if (mag == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-lane moves with DPP (within rows of 16 lanes). quad_perm [a,b,c,d] is
// encoded as a | b<<2 | c<<4 | d<<6; row_ror:n is 0x120 + n.
constexpr int DPP_QUAD_XOR1 = 0xB1;   // [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Lane xor 4 inside groups of 32 (ds_swizzle bitmask mode: and 0x1f, or 0, xor 4).
__device__ __forceinline__ float swz_xor4(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same value.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<DPP_ROW_ROR8>(v);
  v += dpp<DPP_ROW_ROR4>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_QUAD_XOR1>(v);
  return v;
}

// Max over the 16 lanes of a DPP row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
  v = fmaxf(v, dpp<DPP_ROW_ROR4>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
  return v;
}

constexpr int DPP_ROW_SHR1 = 0x111;
constexpr int DPP_ROW_SHR2 = 0x112;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHR8 = 0x118;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Inclusive prefix sum inside each DPP row of 16 lanes (lanes shifted in from
// outside the row read 0).
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v) {
  v += dpp_u32<DPP_ROW_SHR1>(v);
  v += dpp_u32<DPP_ROW_SHR2>(v);
  v += dpp_u32<DPP_ROW_SHR4>(v);
  v += dpp_u32<DPP_ROW_SHR8>(v);
  return v;
}

// 128-bit global loads; the nontemporal form streams data that is read once.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Dot of 8 fp32 values with the 8 bf16 values packed in a 128-bit word.
__device__ __forceinline__ float dot8_bf16(const float* q, u32x4 w) {
  float a = q[0] * bf_lo(w.x);
  a = fmaf(q[1], bf_hi(w.x), a);
  a = fmaf(q[2], bf_lo(w.y), a);
  a = fmaf(q[3], bf_hi(w.y), a);
  a = fmaf(q[4], bf_lo(w.z), a);
  a = fmaf(q[5], bf_hi(w.z), a);
  a = fmaf(q[6], bf_lo(w.w), a);
  a = fmaf(q[7], bf_hi(w.w), a);
  return a;
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// a.lo*b.lo + a.hi*b.hi + c for two packed bf16 pairs, fp32 accumulation
// (v_dot2c_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Dot of 16 fp32 values with the 16 OCP FP8 E4M3 values packed in a 128-bit word
// (hardware decoding, two values per instruction; sum in element order).
__device__ __forceinline__ float dot16_fp8(const float* q, u32x4 w) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], true);
    a = i == 0 ? q[0] * lo[0] : fmaf(q[4 * i], lo[0], a);
    a = fmaf(q[4 * i + 1], lo[1], a);
    a = fmaf(q[4 * i + 2], hi[0], a);
    a = fmaf(q[4 * i + 3], hi[1], a);
  }
  return a;
}

// Dot of the q slice with one 16-byte chunk of a projected row: 8 bf16 values
// (KB = 2 bytes per element) or 16 fp8 values (KB = 1).
template <int KB>
__device__ __forceinline__ float dot_chunk(const float* q, u32x4 w) {
  if constexpr (KB == 2) return dot8_bf16(q, w);
  else return dot16_fp8(q, w);
}

// OCP FP8 E4M3 code of an fp32 value: nearest, ties to even, saturating at +-448,
// NaN to 0x7F (the hardware conversion rounds to nearest even; the clamp makes it
// saturate).
__device__ __forceinline__ uint32_t f32_to_fp8_sat(float f) {
  if (f != f) return 0x7Fu;
  const float c = fminf(fmaxf(f, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.f, 0, false) & 0xFFu;
}

// Wave-wide (64 lanes) inclusive prefix sum of a u32: DPP scans inside the four rows
// of 16 lanes, then each row adds the totals of the rows before it (read from lanes
// 15, 31 and 47). Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v = row16_incl_scan(v);
  const uint32_t t0 = readlane_u32(v, 15), t1 = readlane_u32(v, 31), t2 = readlane_u32(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// Wave-wide min / max (the result is uniform). Every lane must be active.
__device__ __forceinline__ float wave_min_f32(float v) {
  v = fminf(v, dpp<DPP_ROW_ROR8>(v));
  v = fminf(v, dpp<DPP_ROW_ROR4>(v));
  v = fminf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fminf(v, dpp<DPP_QUAD_XOR1>(v));
  return fminf(fminf(readlane_f32(v, 0), readlane_f32(v, 16)), fminf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_ROW_ROR8>(v));
  v = max(v, dpp_u32<DPP_ROW_ROR4>(v));
  v = max(v, dpp_u32<DPP_QUAD_XOR2>(v));
  v = max(v, dpp_u32<DPP_QUAD_XOR1>(v));
  return max(max(readlane_u32(v, 0), readlane_u32(v, 16)), max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Wave-level transposed reduction: lanes p = lane % LPR of a row hold partial sums
// a[i] for LPR consecutive loads i; afterwards lane p holds the full sum of load
// index p. At the stage with lane distance 2^j a lane keeps the loads whose index
// has bit j equal to its own and adds its partner's copy (quad DPP moves for
// distances 1 and 2, a swizzle for 4).
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

// Score of one projected row by one lane from its 16-byte chunks (r*KB/16 of them,
// KB = bytes per stored element): the chunk dots are summed in the balanced tree the
// transposed wave reduction uses, so identical rows get bit-identical scores
// whichever code path computes them. q holds q_hat (r fp32).
template <int R, int KB>
__device__ __forceinline__ float row_score_words(const float* q, const u32x4 (&w)[R * KB / 16]) {
  constexpr int LPR = R * KB / 16;
  constexpr int VPC = 16 / KB;                 // values per chunk
  float a[LPR];
#pragma unroll
  for (int i = 0; i < LPR; ++i) a[i] = dot_chunk<KB>(q + VPC * i, w[i]);
  if constexpr (LPR == 1) {
    return a[0];
  } else if constexpr (LPR == 2) {
    return a[0] + a[1];
  } else if constexpr (LPR == 4) {
    return (a[0] + a[1]) + (a[2] + a[3]);
  } else {
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  }
}

template <int R, int KB>
__device__ __forceinline__ float row_score(const float* q, const unsigned char* rowp) {
  u32x4 w[R * KB / 16];
#pragma unroll
  for (int i = 0; i < R * KB / 16; ++i) w[i] = ld16(rowp + 16 * i);
  return row_score_words<R, KB>(q, w);
}

}  // namespace sjsa

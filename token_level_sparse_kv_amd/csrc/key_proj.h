// Projection of one new key row onto the scoring basis, Kproj = M_h k (fp32 dot over
// d, rounded to the cache format: bf16 or FP8 E4M3), shared by the append kernel
// and the fused append in the prep kernel so that a projected row's bits do not
// depend on which call wrote it.
//
// 256 threads: output i of the projected row is split over TPO = 256 / R lanes,
// lane `part` owning channels part*CH .. part*CH + CH - 1 (CH = d / TPO) of basis
// row i; each lane's partial dot runs in channel order and the TPO partials are
// combined with DPP lane moves (the full dot ends in lane part == 0 and its
// partners).
#pragma once

#include "sjsa_device.h"
#include "sjsa_internal.h"

namespace sjsa {

template <int R>
struct KeyProj {
  static constexpr int THREADS = 256;
  static constexpr int TPO = THREADS / R;       // lanes per output (16, 8 or 4)
  static constexpr int CH = HEAD_DIM / TPO;     // channels per lane (8, 16 or 32)

  // basis slice of thread t (t < THREADS): row t / TPO, channels (t % TPO) * CH ..
  __device__ static void load_basis(const float* Mh, int t, f32x4 (&mv)[CH / 4]) {
    const f32x4* m4 = reinterpret_cast<const f32x4*>(Mh + (size_t)(t / TPO) * HEAD_DIM + (t % TPO) * CH);
#pragma unroll
    for (int c = 0; c < CH / 4; ++c) mv[c] = m4[c];
  }
  // key slice of thread t: channels (t % TPO) * CH .. of the row at krow
  __device__ static void load_key(const uint16_t* krow, int t, u32x4 (&kv)[CH / 8]) {
#pragma unroll
    for (int c = 0; c < CH / 8; ++c) kv[c] = ld16(krow + (t % TPO) * CH + c * 8);
  }
  // element i of a projected row in the cache format: bf16 (KB = 2, nearest even) or
  // OCP FP8 E4M3 (KB = 1, nearest even, saturating)
  template <int KB>
  __device__ static uint32_t encode(float v) {
    if constexpr (KB == 2) return f32_to_bf16_rne(v);
    else return f32_to_fp8_sat(v);
  }
  template <int KB>
  __device__ static void store(unsigned char* row, int i, float v) {
    if constexpr (KB == 2) reinterpret_cast<uint16_t*>(row)[i] = (uint16_t)encode<KB>(v);
    else row[i] = (unsigned char)encode<KB>(v);
  }
  // combined dot (valid in the lane with t % TPO == 0); every lane of the wave calls
  __device__ static float dot(const f32x4 (&mv)[CH / 4], const u32x4 (&kv)[CH / 8]) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CH / 8; ++c) {
      const f32x4 m0 = mv[2 * c], m1 = mv[2 * c + 1];
      acc = fmaf(m0.x, bf_lo(kv[c].x), acc);
      acc = fmaf(m0.y, bf_hi(kv[c].x), acc);
      acc = fmaf(m0.z, bf_lo(kv[c].y), acc);
      acc = fmaf(m0.w, bf_hi(kv[c].y), acc);
      acc = fmaf(m1.x, bf_lo(kv[c].z), acc);
      acc = fmaf(m1.y, bf_hi(kv[c].z), acc);
      acc = fmaf(m1.z, bf_lo(kv[c].w), acc);
      acc = fmaf(m1.w, bf_hi(kv[c].w), acc);
    }
    if constexpr (TPO == 16) {
      acc = row16_sum(acc);
    } else {
      acc += dpp<DPP_QUAD_XOR1>(acc);
      acc += dpp<DPP_QUAD_XOR2>(acc);
      if constexpr (TPO == 8) acc += swz_xor4(acc);
    }
    return acc;
  }
};

}  // namespace sjsa

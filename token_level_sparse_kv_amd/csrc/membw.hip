// Read-bandwidth ceiling of the GPU, for the benchmark's roofline: a plain streaming
// read of a device buffer with 16-byte nontemporal loads, the access the score scan
// makes, and nothing else. Built as its own library (libsjsa_membw.so); the decode
// path does not use it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int THREADS = 256;
constexpr int UNROLL = 8;

// Workgroup w reads the 16-byte words [w*per_wg, min((w+1)*per_wg, n16)), each thread
// UNROLL words per iteration (256 apart, so every load instruction is coalesced).
// The words are folded with XOR and stored only when the result equals a value no
// input here produces, so the loads cannot be removed.
__global__ __launch_bounds__(THREADS) void read_kernel(const u32x4* __restrict__ p, size_t n16, size_t per_wg,
                                                       unsigned* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * per_wg;
  const size_t end = base + per_wg < n16 ? base + per_wg : n16;
  unsigned acc = 0;
  for (size_t i = base + threadIdx.x; i < end; i += (size_t)THREADS * UNROLL) {
    u32x4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t j = i + (size_t)u * THREADS;
      w[u] = j < end ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) at device pointer p with `workgroups` workgroups;
// sink: `workgroups` device u32 words. Returns 0, or -1 on a bad argument or launch error.
extern "C" int sjsa_membw_read(const void* p, size_t bytes, int workgroups, unsigned* sink, void* stream) {
  if (!p || !sink || workgroups < 1 || bytes % 16 != 0) return -1;
  const size_t n16 = bytes / 16;
  const size_t per = (n16 + (size_t)workgroups - 1) / (size_t)workgroups;
  read_kernel<<<workgroups, THREADS, 0, (hipStream_t)stream>>>((const u32x4*)p, n16, per, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

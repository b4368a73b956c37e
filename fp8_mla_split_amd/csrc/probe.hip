// Streaming HBM read of a device buffer, for benchmarks: the read rate the decode kernel's
// KV traffic is compared with, measured on the same GPU in the same run.  Not part of the
// decode path.
//
// Every lane loads 16 bytes per access, eight accesses in flight before any is used, and
// folds them into one word by XOR so that no load can be dropped; one word per workgroup is
// written.  The grid strides over the buffer in 32 KiB blocks (256 lanes x 8 x 16 B).
#include "internal.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int64_t kProbeChunk = (int64_t)kProbeThreads * kProbeUnroll * 16;  // 32 KiB

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src,
                                                                   int64_t chunks,
                                                                   uint32_t* __restrict__ out) {
  asm volatile("" ::"s"(src), "s"(chunks), "s"(out));
  uint32_t acc = 0;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const u32x4* p = src + c * (kProbeChunk / 16) + threadIdx.x;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) v[j] = __builtin_nontemporal_load(p + j * kProbeThreads);
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // one word per workgroup: each wave folds its lanes, the four waves meet in LDS
  __shared__ uint32_t wave_acc[kProbeThreads / 64];
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) wave_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = wave_acc[0] ^ wave_acc[1] ^ wave_acc[2] ^ wave_acc[3];
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, int grid,
                             hipStream_t s) {
  clear_last_error();
  read_probe_kernel<<<grid, kProbeThreads, 0, s>>>((const u32x4*)src, bytes / kProbeChunk, out);
  return hipGetLastError();
}

int64_t read_probe_chunk_bytes() { return kProbeChunk; }

}  // namespace mla

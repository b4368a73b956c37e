// Saturating fp32 -> E4M3 quantisation (the "prep" step; see the saturating-conversion item of
// the MLA section of the arex-research.com Vera Rubin / Kimi K3 write-up: without saturation
// the conversion cannot use the packed hardware instruction, with it overflow clamps to +-448).
//
// gfx950's v_cvt_pk_fp8_f32 converts two fp32 values to OCP E4M3 with round-to-nearest-even,
// including subnormals and the sign of zero, but it is not saturating: quotients above 464
// become NaN.  We therefore clamp to +-448 first (every value in (448, 464) rounds to 448
// anyway) and write NaN inputs explicitly as 0x7F | sign.  The quotient is an IEEE-rounded
// fp32 division (__fdiv_rn), not a reciprocal multiply, so ties at E4M3 midpoints resolve the
// same way as for the exact quotient rounded to fp32.
//
// HBM-bound: 4 B read + 1 B written per element.  Each thread converts 16 consecutive
// elements per iteration (four 16-B loads, one 16-B store); the grid strides over the array.
// Tensors under 2^21 elements (one step's Q) take four elements per thread instead.
#include "internal.h"

namespace mla {
namespace {

__device__ __forceinline__ float clamp448(float t) { return fminf(fmaxf(t, -448.0f), 448.0f); }

__device__ __forceinline__ uint32_t nan_code(float t) {
  return 0x7Fu | ((__float_as_uint(t) >> 31) << 7);
}

// Four quotients -> four codes packed little-endian in one dword.
__device__ __forceinline__ uint32_t encode4(float t0, float t1, float t2, float t3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(t0), clamp448(t1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(t2), clamp448(t3), w, true);
  uint32_t out = (uint32_t)w;
  const float t[4] = {t0, t1, t2, t3};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (t[i] != t[i]) out = (out & ~(0xFFu << (8 * i))) | (nan_code(t[i]) << (8 * i));
  }
  return out;
}

__device__ __forceinline__ uint8_t encode1(float t) {
  if (t != t) return (uint8_t)nan_code(t);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(t), 0.0f, 0, false) & 0xFF);
}

// Workgroups of kThreads threads; stride = grid * kThreads comes in as an argument, so the
// kernel reads nothing but its arguments (all fetched in one batch) before its first load.
constexpr int kThreads = 256;
constexpr int64_t kSmallN = int64_t(1) << 21;  // below this, four elements per thread

__global__ __launch_bounds__(kThreads) void quantize_vec16(const float4* __restrict__ src,
                                                           uint4* __restrict__ dst, int64_t n16,
                                                           int64_t stride, float scale) {
  asm volatile("" ::"s"(src), "s"(dst), "s"(n16), "s"(stride), "s"(scale));
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const float4 a = src[4 * i + 0], b = src[4 * i + 1], c = src[4 * i + 2], d = src[4 * i + 3];
    uint4 o;
    o.x = encode4(__fdiv_rn(a.x, scale), __fdiv_rn(a.y, scale), __fdiv_rn(a.z, scale),
                  __fdiv_rn(a.w, scale));
    o.y = encode4(__fdiv_rn(b.x, scale), __fdiv_rn(b.y, scale), __fdiv_rn(b.z, scale),
                  __fdiv_rn(b.w, scale));
    o.z = encode4(__fdiv_rn(c.x, scale), __fdiv_rn(c.y, scale), __fdiv_rn(c.z, scale),
                  __fdiv_rn(c.w, scale));
    o.w = encode4(__fdiv_rn(d.x, scale), __fdiv_rn(d.y, scale), __fdiv_rn(d.z, scale),
                  __fdiv_rn(d.w, scale));
    dst[i] = o;
  }
}

// Four elements per thread (one 16-byte load, one 4-byte store): for small tensors such as
// one step's Q, where spreading the divisions over more threads shortens the kernel (it is
// latency-bound there, not bandwidth-bound).
__global__ __launch_bounds__(kThreads) void quantize_vec4(const float4* __restrict__ src,
                                                          uint32_t* __restrict__ dst, int64_t n4,
                                                          int64_t stride, float scale) {
  asm volatile("" ::"s"(src), "s"(dst), "s"(n4), "s"(stride), "s"(scale));
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    const float4 a = src[i];
    dst[i] = encode4(__fdiv_rn(a.x, scale), __fdiv_rn(a.y, scale), __fdiv_rn(a.z, scale),
                     __fdiv_rn(a.w, scale));
  }
}

// Element-wise variant for unaligned buffers and for the tail after the vector blocks.
__global__ __launch_bounds__(kThreads) void quantize_scalar(const float* __restrict__ src,
                                                            uint8_t* __restrict__ dst,
                                                            int64_t begin, int64_t n,
                                                            int64_t stride, float scale) {
  asm volatile("" ::"s"(src), "s"(dst), "s"(begin), "s"(n), "s"(stride), "s"(scale));
  for (int64_t i = begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    dst[i] = encode1(__fdiv_rn(src[i], scale));
}

}  // namespace

hipError_t launch_quantize(const float* src, uint8_t* dst, int64_t n, float scale,
                           hipStream_t s) {
  const bool aligned = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  int64_t done = 0;
  if ((uintptr_t)src % 16 == 0 && (uintptr_t)dst % 4 == 0 && n >= 4 && n < kSmallN) {
    const int64_t n4 = n / 4;
    const int grid = (int)((n4 + kThreads - 1) / kThreads);
    quantize_vec4<<<grid, kThreads, 0, s>>>((const float4*)src, (uint32_t*)dst, n4,
                                            (int64_t)grid * kThreads, scale);
    done = n4 * 4;
  } else if (aligned && n >= 16) {
    const int64_t n16 = n / 16;
    const int64_t want = (n16 + kThreads - 1) / kThreads;
    const int grid = (int)(want < 8192 ? want : 8192);
    quantize_vec16<<<grid, kThreads, 0, s>>>((const float4*)src, (uint4*)dst, n16,
                                             (int64_t)grid * kThreads, scale);
    done = n16 * 16;
  }
  if (done < n) {
    const int64_t rest = n - done;
    const int64_t want = (rest + kThreads - 1) / kThreads;
    const int grid = (int)(want < 8192 ? want : 8192);
    quantize_scalar<<<grid, kThreads, 0, s>>>(src, dst, done, n, (int64_t)grid * kThreads,
                                              scale);
  }
  return hipGetLastError();
}

}  // namespace mla

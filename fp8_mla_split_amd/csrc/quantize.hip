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
//
// The same encode serves the other entry points below: the append of a decode step's new KV
// rows straight into their paged cache slots (fp32 or bf16 rows, optionally with RoPE applied
// to their rope columns first), and the quantisation whose per-tensor scale (amax / 448) is
// taken from the data on the device in two passes.
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

// bf16 sources hold the upper halves of fp32 patterns.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- Appending a decode step's new KV rows to the paged FP8 cache ----------------------
// New token t of request b (of T) is logical position n = seq_lens[b] - T + t and goes to row
// n % P of page page_table[b, n / P].  One thread per 16 columns of a 576-wide row (36 per
// row: 64 or 32 source bytes, one 16-B store), or per column where a buffer is not 16-byte
// aligned.  Sources are fp32 or bf16 (the upper half of an fp32 pattern, widened exactly).
// Positions past the page table and page ids outside the pool are skipped, so a bad
// device-side length or table entry cannot write outside the pool.
// RoPE on the way in (the Muse Spark Open page's kernel-work item that fuses RoPE with the
// KV-cache write): rope pair (512 + 2i, 513 + 2i) of a new row is the complex number
// x0 + i x1, multiplied by cos + i sin of its position's angle i (cos_t / sin_t: fp32
// [positions, 32]).  Each product and sum is rounded on its own (no fused multiply-add), so
// the rotated value, whose rounding decides its E4M3 code, is the same on every compiler.
__device__ __forceinline__ void rope_pair(float& x0, float& x1, float c, float s) {
  const float r0 = __fsub_rn(__fmul_rn(x0, c), __fmul_rn(x1, s));
  const float r1 = __fadd_rn(__fmul_rn(x0, s), __fmul_rn(x1, c));
  x0 = r0;
  x1 = r1;
}

struct RopeTables {
  const float* cos_t;  // NULL: no rotation
  const float* sin_t;
  int64_t positions;
};

template <bool Vec, bool Bf16, bool kRope>
__global__ __launch_bounds__(kThreads) void kv_append(const void* __restrict__ src,
                                                      uint8_t* __restrict__ pool,
                                                      const int32_t* __restrict__ page_table,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int t_new, int page_size, int max_pages,
                                                      int64_t num_pages, int64_t units,
                                                      int64_t stride, float scale,
                                                      RopeTables rope) {
  constexpr int kPer = Vec ? 16 : 1;
  constexpr int kUnitsPerRow = kD / kPer;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
    const int64_t row = u / kUnitsPerRow;
    const int c = (int)(u - row * kUnitsPerRow);
    const int b = (int)(row / t_new), t = (int)(row - (int64_t)b * t_new);
    const int64_t n = (int64_t)seq_lens[b] - t_new + t;
    if (n < 0 || n >= (int64_t)max_pages * page_size) continue;
    if (kRope && n >= rope.positions) continue;  // no angle for it: not written
    const int64_t page = page_table[(int64_t)b * max_pages + n / page_size];
    if (page < 0 || page >= num_pages) continue;
    uint8_t* d = pool + (page * page_size + n % page_size) * kD + c * kPer;
    const int64_t e0 = row * kD + c * kPer;  // first source element
    if constexpr (Vec) {
      float x[16];
      if constexpr (Bf16) {
        const uint4* w = (const uint4*)((const uint16_t*)src + e0);
        const uint4 a = w[0], bb = w[1];
        const uint32_t ws[8] = {a.x, a.y, a.z, a.w, bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          x[2 * k] = bf16_lo(ws[k]);
          x[2 * k + 1] = bf16_hi(ws[k]);
        }
      } else {
        const float4* x4 = (const float4*)((const float*)src + e0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 a = x4[k];
          x[4 * k] = a.x; x[4 * k + 1] = a.y; x[4 * k + 2] = a.z; x[4 * k + 3] = a.w;
        }
      }
      if constexpr (kRope) {
        if (c >= kDv / 16) {  // columns 16c .. 16c + 15 are rope pairs 8 (c - 32) ..
          const int64_t a0 = n * 32 + 8 * (c - kDv / 16);
          const float4 c0 = *(const float4*)(rope.cos_t + a0),
                       c1 = *(const float4*)(rope.cos_t + a0 + 4);
          const float4 s0 = *(const float4*)(rope.sin_t + a0),
                       s1 = *(const float4*)(rope.sin_t + a0 + 4);
          const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) rope_pair(x[2 * k], x[2 * k + 1], cs[k], sn[k]);
        }
      }
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = encode4(__fdiv_rn(x[4 * k], scale), __fdiv_rn(x[4 * k + 1], scale),
                       __fdiv_rn(x[4 * k + 2], scale), __fdiv_rn(x[4 * k + 3], scale));
      *(uint4*)d = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      auto elem = [&](int64_t e) __attribute__((always_inline)) {
        return Bf16 ? __uint_as_float((uint32_t)((const uint16_t*)src)[e] << 16)
                    : ((const float*)src)[e];
      };
      float x = elem(e0);
      if constexpr (kRope) {
        if (c >= kDv) {  // rope column: rotate it with its pair partner
          const int j = c - kDv, i = j >> 1;
          const int64_t ep = row * kD + kDv + 2 * i;
          float x0 = elem(ep), x1 = elem(ep + 1);
          rope_pair(x0, x1, rope.cos_t[n * 32 + i], rope.sin_t[n * 32 + i]);
          x = (j & 1) ? x1 : x0;
        }
      }
      *d = encode1(__fdiv_rn(x, scale));
    }
  }
}

// ---- Per-tensor scale taken from the data (amax / 448), then the same encode ----------
// Pass 1 writes one maximum per workgroup; pass 2 has every workgroup fold those maxima
// (at most kAmaxBlocks words, from L2), derive the scale and quantise its share.  No atomics
// and nothing to clear beforehand, so both passes can be replayed in a captured graph.
// Magnitudes are compared as the bit patterns of |x| (sign cleared): for non-negative IEEE
// values the unsigned order is the numeric order, and every NaN pattern sorts above +inf,
// so the result is NaN whenever the tensor holds one, as max|x| is.
constexpr int kAmaxBlocks = 1024;


__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t abs_bits_word(uint32_t w, bool bf16) {
  return bf16 ? umax(w & 0x7FFF0000u, (w & 0x7FFFu) << 16) : (w & 0x7FFFFFFFu);
}

__device__ __forceinline__ uint32_t abs_bits_16b(const uint4& v, bool bf16) {
  return umax(umax(abs_bits_word(v.x, bf16), abs_bits_word(v.y, bf16)),
              umax(abs_bits_word(v.z, bf16), abs_bits_word(v.w, bf16)));
}

__device__ __forceinline__ float load_elem(const void* src, int64_t i, bool bf16) {
  return bf16 ? __uint_as_float((uint32_t)((const uint16_t*)src)[i] << 16)
              : ((const float*)src)[i];
}

// Largest value of a workgroup (all threads return it).
__device__ __forceinline__ uint32_t block_umax(uint32_t m) {
  __shared__ uint32_t red[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = umax(m, red[w]);
  return m;
}

// src: 16-byte aligned when vec (16-B words = 4 fp32 or 8 bf16 values, four words in flight
// per thread); the elements after the last whole word are read one at a time.
template <bool Bf16>
__global__ __launch_bounds__(kThreads) void amax_partial(const void* __restrict__ src,
                                                         int64_t n, int vec,
                                                         uint32_t* __restrict__ partial) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  int64_t done = 0;
  if (vec) {
    constexpr int kPerWord = Bf16 ? 8 : 4;
    const int64_t nw = n / kPerWord;
    const uint4* w = (const uint4*)src;
    int64_t i = tid;
    for (; i + 3 * stride < nw; i += 4 * stride) {
      const uint4 a = w[i], b = w[i + stride], c = w[i + 2 * stride], d = w[i + 3 * stride];
      m = umax(m, umax(umax(abs_bits_16b(a, Bf16), abs_bits_16b(b, Bf16)),
                       umax(abs_bits_16b(c, Bf16), abs_bits_16b(d, Bf16))));
    }
    for (; i < nw; i += stride) m = umax(m, abs_bits_16b(w[i], Bf16));
    done = nw * kPerWord;
  }
  for (int64_t i = done + tid; i < n; i += stride)
    m = umax(m, __float_as_uint(load_elem(src, i, Bf16)) & 0x7FFFFFFFu);
  m = block_umax(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Pass 2.  Per = elements per thread and iteration: 16 (16-B stores), 4 (4-B stores; small
// tensors, where more threads shorten the latency-bound kernel) or 1 (unaligned buffers).
template <bool Bf16, int Per>
__global__ __launch_bounds__(kThreads) void quantize_from_amax(
    const void* __restrict__ src, uint8_t* __restrict__ dst, int64_t n, int64_t stride,
    const uint32_t* __restrict__ partial, int nparts, float* __restrict__ scale_out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) m = umax(m, partial[i]);
  const float amax = __uint_as_float(block_umax(m));
  const float scale = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = scale;
  const int64_t groups = n / Per;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
    float x[Per];
    if constexpr (Per == 1) {
      x[0] = load_elem(src, g, Bf16);
    } else if constexpr (Bf16) {
      uint32_t w[Per / 2];
      if constexpr (Per == 16) {
        const uint4 a = ((const uint4*)src)[2 * g], b = ((const uint4*)src)[2 * g + 1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
      } else {
        const uint2 a = ((const uint2*)src)[g];
        w[0] = a.x; w[1] = a.y;
      }
#pragma unroll
      for (int k = 0; k < Per / 2; ++k) {
        x[2 * k] = bf16_lo(w[k]);
        x[2 * k + 1] = bf16_hi(w[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < Per / 4; ++k) {
        const float4 a = ((const float4*)src)[(Per / 4) * g + k];
        x[4 * k] = a.x; x[4 * k + 1] = a.y; x[4 * k + 2] = a.z; x[4 * k + 3] = a.w;
      }
    }
    if constexpr (Per == 1) {
      dst[g] = encode1(__fdiv_rn(x[0], scale));
    } else {
      uint32_t o[Per / 4];
#pragma unroll
      for (int k = 0; k < Per / 4; ++k)
        o[k] = encode4(__fdiv_rn(x[4 * k], scale), __fdiv_rn(x[4 * k + 1], scale),
                       __fdiv_rn(x[4 * k + 2], scale), __fdiv_rn(x[4 * k + 3], scale));
      if constexpr (Per == 16)
        ((uint4*)dst)[g] = make_uint4(o[0], o[1], o[2], o[3]);
      else
        ((uint32_t*)dst)[g] = o[0];
    }
  }
  // elements after the last whole group
  if (blockIdx.x == 0)
    for (int64_t i = groups * Per + threadIdx.x; i < n; i += kThreads)
      dst[i] = encode1(__fdiv_rn(load_elem(src, i, Bf16), scale));
}

int grid_for(int64_t units, int64_t cap) {
  const int64_t want = (units + kThreads - 1) / kThreads;
  return (int)(want < 1 ? 1 : (want < cap ? want : cap));
}

template <bool Bf16>
hipError_t launch_dynamic_t(const void* src, uint8_t* dst, int64_t n, float* scale_out,
                            uint32_t* partial, hipStream_t s) {
  clear_last_error();
  const int esz = Bf16 ? 2 : 4;
  const bool src16 = (uintptr_t)src % 16 == 0;
  const int64_t words = src16 ? n * esz / 16 : n;
  const int ablocks = grid_for((words + 3) / 4, kAmaxBlocks);
  amax_partial<Bf16><<<ablocks, kThreads, 0, s>>>(src, n, src16 ? 1 : 0, partial);
  if (src16 && (uintptr_t)dst % 4 == 0 && n < kSmallN) {
    const int grid = grid_for(n / 4, 8192);
    quantize_from_amax<Bf16, 4><<<grid, kThreads, 0, s>>>(src, dst, n, (int64_t)grid * kThreads,
                                                          partial, ablocks, scale_out);
  } else if (src16 && (uintptr_t)dst % 16 == 0) {
    const int grid = grid_for(n / 16, 8192);
    quantize_from_amax<Bf16, 16><<<grid, kThreads, 0, s>>>(src, dst, n, (int64_t)grid * kThreads,
                                                           partial, ablocks, scale_out);
  } else {
    const int grid = grid_for(n, 8192);
    quantize_from_amax<Bf16, 1><<<grid, kThreads, 0, s>>>(src, dst, n, (int64_t)grid * kThreads,
                                                          partial, ablocks, scale_out);
  }
  return hipGetLastError();
}

}  // namespace

int64_t dynamic_quantize_workspace_bytes() { return (int64_t)kAmaxBlocks * 4; }

hipError_t launch_quantize_dynamic(const void* src, bool bf16, uint8_t* dst, int64_t n,
                                   float* scale_out, void* workspace, hipStream_t s) {
  return bf16 ? launch_dynamic_t<true>(src, dst, n, scale_out, (uint32_t*)workspace, s)
              : launch_dynamic_t<false>(src, dst, n, scale_out, (uint32_t*)workspace, s);
}

hipError_t launch_kv_append(const void* src, bool bf16, uint8_t* pool, int64_t num_pages,
                            const int32_t* page_table, const int32_t* seq_lens, int batch,
                            int t_new, int page_size, int max_pages, float scale,
                            const float* rope_cos, const float* rope_sin, int64_t rope_positions,
                            hipStream_t s) {
  clear_last_error();
  const bool rope = rope_cos != nullptr;
  // the vector path loads a rope unit's eight angles as two 16-byte words per table
  const bool vec = (uintptr_t)src % 16 == 0 && (uintptr_t)pool % 16 == 0 &&
                   (!rope || ((uintptr_t)rope_cos % 16 == 0 && (uintptr_t)rope_sin % 16 == 0));
  const int64_t units = (int64_t)batch * t_new * (vec ? kD / 16 : kD);
  const int grid = grid_for(units, 8192);
  const int64_t stride = (int64_t)grid * kThreads;
  const RopeTables tables{rope_cos, rope_sin, rope_positions};
#define MLA_APPEND(V, B, R)                                                                 \
  kv_append<V, B, R><<<grid, kThreads, 0, s>>>(src, pool, page_table, seq_lens, t_new,      \
                                               page_size, max_pages, num_pages, units, stride, \
                                               scale, tables)
  if (rope) {
    if (vec && bf16) MLA_APPEND(true, true, true);
    else if (vec) MLA_APPEND(true, false, true);
    else if (bf16) MLA_APPEND(false, true, true);
    else MLA_APPEND(false, false, true);
  } else {
    if (vec && bf16) MLA_APPEND(true, true, false);
    else if (vec) MLA_APPEND(true, false, false);
    else if (bf16) MLA_APPEND(false, true, false);
    else MLA_APPEND(false, false, false);
  }
#undef MLA_APPEND
  return hipGetLastError();
}

hipError_t launch_quantize(const float* src, uint8_t* dst, int64_t n, float scale,
                           hipStream_t s) {
  clear_last_error();
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

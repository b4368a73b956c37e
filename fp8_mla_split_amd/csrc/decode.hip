// Split-KV partial attention for MLA decode over an FP8 (OCP E4M3) KV cache, gfx950.
//
// Cited pages: [A] the arex-research.com Vera Rubin / Kimi K3 write-up, section "Kimi K3 的
// MLA：更深的流水线、更快的 split-KV 归约" (items: deeper pipeline, faster split-KV reduction,
// 64-way split, saturating FP8 conversion); [B] the ai.newsbites.today summary, section
// "MLAアテンションのパイプライン深化".  They state that long-context MLA decode waits mostly
// on KV reads from HBM and is made faster by keeping more reads in flight (a deeper staging
// pipeline), and that at low batch one request's KV is split over many workgroups whose
// partial results a second kernel merges.  Their stage counts are tuned for a 227/327 KiB
// shared-memory part with 212 SMs; the layout below is designed for gfx950 instead.
//
// Work decomposition.  A workgroup is four wavefronts, one per SIMD (the 512-register budget
// of a lone wave holds the 32x512 fp32 output accumulator in AGPRs).  It owns 32*RG query
// rows (rows = (query token, head) pairs of one request) and one chunk of that request's
// tokens.  Wave w works on row block w / TL and takes every TL-th tile of the chunk
// (TL = 4 / RG), so with RG = 1 the four waves stream four different tiles and share nothing
// but the LDS ring; their partial (max, sum, O) are merged in LDS at the end.
//
// KV staging.  A tile is 32 tokens x 576 bytes.  Tiles go HBM -> LDS with buffer_load ... lds
// (16 bytes per lane, no VGPR round trip) into an 8-slot ring (151 KiB of the CU's 160 KiB):
// 8 / TL stages of TL tiles, so 8/TL - 1 stages are in flight while one is consumed.  Rows
// are stored with a 592-byte pitch (37 x 16 B); the 64-bank LDS then serves both read
// patterns below without conflicts.  The buffer resource of each tile is bounded by the
// number of valid rows, so rows past the end of the sequence arrive as zeros: no NaN bytes
// from a page's unused tail can reach the P.V product (0 x NaN).  The DMA is issued with
// inline asm and waited on with explicit vmcnt counts because the compiler, when it sees the
// intrinsic, waits for every outstanding LDS DMA before any LDS read and so removes the
// pipelining this staging exists for.
//
// Math per tile (per wave, 32 rows x 32 tokens), all on FP8 MFMA v_mfma_scale_f32_32x32x64:
//  * S^T = K . Q^T: tokens along M, rows along N, 576 = 9 x 64 channels along K.  Q stays in
//    registers for the whole kernel.  Computing the transpose puts each lane's 16 scores for
//    one row exactly where the P.V step needs them as its A operand (no data movement).
//    MFMA token m reads LDS row perm_row(m); the permutation makes the transposed V reads
//    below touch 8 rows of one parity, which is what keeps them conflict-free.
//  * Online softmax in base 2 against a fixed reference max mu per row (the max of the row's
//    first tile with a visible position), so the 256-register O is never rescaled.  Each
//    tile's probabilities are instead normalised per row by 2^-e (e = floor of the tile max
//    above mu) before the FP8 cast, and the MFMA's per-lane E8M0 scale multiplies them back
//    by 2^e.  If a row's true max ends up more than kHeadroom above mu (fp32 range at
//    risk), the workgroup recomputes its chunk once with mu = the true max.
//  * P is encoded as hi = e4m3(p) and lo = e4m3(p - hi), both in the same units; one
//    32x32x64 MFMA takes [hi | lo] for 32 tokens against [V | V], i.e. P.V with about
//    7 bits of P mantissa.  (A single e4m3 P costs ~3e-3 normalised L1 error against the
//    fp64 oracle at 128K context, more than the 2e-3 budget.)
//  * V (the first 512 columns of the same tile) is read transposed with ds_read_b64_tr_b8.
#include "internal.h"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPitch = 592;                 // LDS bytes per KV row (576 + one 16-B pad)
constexpr int kTileBytes = kTile * kPitch;  // 18944
constexpr int kSlot = kTileBytes + 512;     // guard for the half-used last DMA instruction
constexpr int kSlots = 8;
constexpr int kLds = kSlots * kSlot;        // 155648 bytes
constexpr int kDmaPerTile = 19;             // ceil(32 rows * 37 chunks / 64 lanes)
constexpr float kHeadroom = 64.0f;          // log2 range of a pass above its reference max
constexpr float kLog2PScale = 7.807354922057604f;  // log2(224): p in [0, 448)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMergeStride = 264;           // floats per row in the merge buffer

// MFMA token index -> LDS row of the tile: bits (b4 b3 b2 b1 b0) -> (b4 b3 b1 b0 b2).
__device__ __forceinline__ int perm_row(int m) {
  return (m & 0x18) | ((m & 3) << 1) | ((m >> 2) & 1);
}
// Token index held in register r of a 32x32 MFMA result by lanes of half gg.
__device__ __forceinline__ int tok_of(int gg, int r) { return 8 * (r >> 2) + 4 * gg + (r & 3); }

__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff,
                                      __amdgpu_buffer_rsrc_t rsrc) {
  // one wait state between the M0 write and the LDS DMA that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// FP8 x FP8 32x32x64 MFMA with explicit register classes.  The compiler, left to itself,
// puts every MFMA accumulator of this kernel into AGPRs; the 16 score registers then evict
// part of the 256-register O accumulator and Q gets spilled.  Issuing the instruction from
// asm pins the scores to VGPRs and O to AGPRs.  The "memory" clobber keeps the LDS
// fragment reads where the source places them (one MFMA ahead), which bounds how many
// fragment registers are live at once.  Hazards the compiler cannot see through the
// asm are covered explicitly: s_nop 1 before each MFMA covers a VALU write of an operand
// just before it, and mfma_drain() (24 wait states, more than the 16-pass instruction's
// requirement) separates the last MFMA of a chain from any non-MFMA reader of its result.
__device__ __forceinline__ f32x16 mfma_qk_first(const i32x8& a, const i32x8& b) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
               : "=&v"(d)
               : "v"(a), "v"(b), "v"(127)
               : "memory");
  return d;
}
__device__ __forceinline__ void mfma_qk(f32x16& d, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
               : "+v"(d)
               : "v"(a), "v"(b), "v"(127)
               : "memory");
}
__device__ __forceinline__ void mfma_pv(f32x16& acc, const i32x8& a, const i32x8& b, int scale_a) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc)
               : "v"(a), "v"(b), "v"(scale_a), "v"(127)
               : "memory");
}
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ i32x4 lds_read16(const uint8_t* lds, uint32_t addr) {
  return *(const i32x4*)(lds + addr);
}

__device__ __forceinline__ i32x2 lds_read_tr8(uint8_t* lds, uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(lds + addr));
}

template <int RG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const DecodeParams p) {
  constexpr int TL = 4 / RG;               // tile lanes (waves sharing a row block)
  constexpr int NST = kSlots / TL;         // ring stages
  constexpr int LOADS = (TL * kDmaPerTile) / 4;  // DMA instructions per wave per stage (min)
  constexpr int VMC = (NST - 2) * LOADS;

  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rg = wave / TL, tl = wave % TL;
  const int n = lane & 31, gg = lane >> 5;

  // ---- workgroup -> (request, split, row group); the G row groups of one split share an
  // XCD (workgroups are dealt to the 8 XCDs round-robin) so their KV reads meet in one L2.
  const int G = p.groups, S = p.num_splits, M = p.rows;
  const int id = blockIdx.x;
  const int kx = id >> 3;
  const int g = kx % G;
  const int u = (kx / G) * 8 + (id & 7);
  if (u >= p.batch * S) return;
  const int b = u / S, s = u - b * S;

  int L = p.seq_lens[b];
  const int Lmax = p.max_pages * p.page_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int ntiles_all = (L + kTile - 1) / kTile;
  const int per = (ntiles_all + S - 1) / S;
  const int t_begin = s * per;
  const int ntiles = max(min(t_begin + per, ntiles_all) - t_begin, 0);

  const int row0 = g * 32 * RG;
  const int64_t prow = (int64_t)(b * S + s) * M;  // first partial row of this (b, s)
  if (ntiles == 0) {
    for (int i = threadIdx.x; i < 32 * RG; i += 256)
      if (row0 + i < M) p.partial_lse[prow + row0 + i] = -INFINITY;
    return;
  }

  const int wrow0 = row0 + rg * 32;
  const int R = wrow0 + n;  // this lane's query row (score and P layout)
  const bool row_ok = R < M;
  // last visible position of the row (bottom-right causal); rows past M are never stored
  const int lim = row_ok ? L - p.q_tokens + R / p.heads : 0x7FFFFFFF;
  const int lim_min = L - p.q_tokens + wrow0 / p.heads;

  // ---- Q fragments (B operand of S^T = K . Q^T), kept for the whole kernel
  i32x8 qf[9];
  const uint8_t* qsrc = p.q8 + ((int64_t)b * M + (row_ok ? R : 0)) * kD + 32 * gg;
  auto load_q = [&]() {
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const i32x4 lo = *(const i32x4*)(qsrc + 64 * c);
      const i32x4 hi = *(const i32x4*)(qsrc + 64 * c + 16);
      qf[c] = row_ok ? (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}
                     : (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
  };
  load_q();

  // ---- DMA of one stage (TL tiles).  Stages past the chunk load nothing (resource with 0
  // records -> zeros) so every wave issues the same count and the vmcnt arithmetic holds.
  const int P = p.page_size;
  // LDS byte address of the ring (M0 of the DMA takes an LDS address, not a flat pointer)
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);
  // The page table is never written while the kernel runs; reading it through the constant
  // address space lets the compiler use scalar loads, which wait on lgkmcnt and so do not
  // force a vmcnt(0) drain of the in-flight KV DMA.
  const __attribute__((address_space(4))) int32_t* page_table =
      (const __attribute__((address_space(4))) int32_t*)p.page_table;
  auto issue_stage = [&](int st) {
#pragma unroll
    for (int j = 0; j < TL; ++j) {
      const int ti = st * TL + j;
      const int slot = (st % NST) * TL + j;
      const uint8_t* base = p.kv;
      int nrec = 0;
      if (ti < ntiles) {
        const int T0 = (t_begin + ti) * kTile;
        const int page = page_table[(int64_t)b * p.max_pages + T0 / P];  // scalar load
        base = p.kv + ((int64_t)page * P + (T0 % P)) * kD;
        nrec = min(kTile, L - T0) * kD;
      }
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, 0x00020000);
      // instruction q = 19 j + k of the stage belongs to wave q % 4.  The lane id is routed
      // through an opaque move so the per-lane offsets are recomputed here (4 VALU each)
      // instead of being hoisted out of the tile loop into ~19 permanently live VGPRs.
      int lane_v;
      asm volatile("v_mov_b32 %0, %1" : "=v"(lane_v) : "v"(lane));
      for (int k = ((wave - kDmaPerTile * j) % 4 + 4) % 4; k < kDmaPerTile; k += 4) {
        const uint32_t pch = 64u * k + (uint32_t)lane_v;  // 16-B chunk index in the slot
        const uint32_t row = (pch * 1772u) >> 16;         // pch / 37 for pch < 1216
        const uint32_t voff = 16u * (pch - row);          // row * 576 + col * 16
        dma16(lds_base + (uint32_t)(slot * kSlot + k * 1024), voff, rsrc);
      }
    }
  };

  const int G16 = lane >> 4, i16 = lane & 15;
  const uint32_t vcol = 16 * (G16 & 1) + 8 * (i16 & 1);
  const uint32_t vrow0 = perm_row(tok_of(gg, i16 >> 1)) * kPitch + vcol;
  const uint32_t vrow1 = perm_row(tok_of(gg, 8 + (i16 >> 1))) * kPitch + vcol;
  const uint32_t krow = perm_row(n) * kPitch + 32 * gg;
  const int nsteps = (ntiles + TL - 1) / TL;

  // ---- per-row softmax state (score layout: lane holds row n; lanes n and n+32 agree).
  // The reference max mu of a row is the max of its first tile with a visible position; it
  // never moves during a pass, so the AGPR-resident O is never rescaled.  Each tile's
  // probabilities are normalised by 2^-e (e = floor(tile max - mu)) before the FP8 cast and
  // the MFMA multiplies them back by 2^e.  With e <= kHeadroom, O and l stay far below the
  // fp32 range (O <= 448 * 448 * 2^kHeadroom * tokens).  If some row's true max exceeds its
  // mu by more than that, the whole workgroup recomputes its chunk once with mu = true max.
  float mu = -INFINITY;     // reference max (log2 units)
  float m_true = -INFINITY; // running true max
  float l_run = 0.f;        // this lane's share of sum 2^(x - mu) * 224
  f32x16 o[16];

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = (f32x16){0.f};
    l_run = 0.f;
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
      if (st < nsteps) issue_stage(st);

    for (int st = 0; st < nsteps; ++st) {
      if (st + NST - 2 < nsteps) wait_vmcnt<VMC>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (st + NST - 1 < nsteps) issue_stage(st + NST - 1);

      const int ti = st * TL + tl;
      if (ti >= ntiles) continue;
      const uint32_t tb = (uint32_t)(((st % NST) * TL + tl) * kSlot);

      // S^T = K . Q^T (tokens x rows), one fragment read ahead of each MFMA
      f32x16 sacc;
      i32x4 a0 = lds_read16(lds, tb + krow);
      i32x4 a1 = lds_read16(lds, tb + krow + 16);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const i32x8 a = (i32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        if (c < 8) {
          a0 = lds_read16(lds, tb + krow + 64 * (c + 1));
          a1 = lds_read16(lds, tb + krow + 64 * (c + 1) + 16);
        }
        if (c == 0) sacc = mfma_qk_first(a, qf[0]);
        else mfma_qk(sacc, a, qf[c]);
      }
      mfma_drain();

      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = sacc[r] * p.c2;
      const int T0 = (t_begin + ti) * kTile;
      if (T0 + kTile - 1 > lim_min) {  // tail or causal tile: mask per element
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (T0 + perm_row(tok_of(gg, r)) > lim) x[r] = -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (mu == -INFINITY) mu = mx;  // first tile with a visible position (pass 0)
      m_true = fmaxf(m_true, mx);

      const float mref = mu == -INFINITY ? 0.f : mu;
      const float ef = fminf(fmaxf(floorf(mx - mref), -126.0f), 127.0f);
      const float off = mref + ef - kLog2PScale;
      float pv[16];
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(x[r] - off);  // in [0, 448); 0 where masked
        lsum += pv[r];
      }
      l_run += ldexpf(lsum, (int)ef);
      const int escale = 127 + (int)ef;

      // P as hi + lo e4m3 bytes: bytes 0..15 of the A operand are hi(p_r), 16..31 lo(p_r)
      i32x8 pa;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q], pv[4 * q + 1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q + 2], pv[4 * q + 3], w, true);
        const f32x2 d01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const f32x2 d23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        int w2 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q] - d01[0], pv[4 * q + 1] - d01[1], 0,
                                                 false);
        w2 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q + 2] - d23[0], pv[4 * q + 3] - d23[1], w2,
                                             true);
        pa[q] = w;
        pa[4 + q] = w2;
      }

      // O += P . V over the 16 blocks of 32 value columns; B = [V | V] for [hi | lo]
      i32x2 v0 = lds_read_tr8(lds, tb + vrow0);
      i32x2 v1 = lds_read_tr8(lds, tb + vrow1);
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const i32x8 vb = (i32x8){v0[0], v0[1], v1[0], v1[1], v0[0], v0[1], v1[0], v1[1]};
        if (d < 15) {
          v0 = lds_read_tr8(lds, tb + vrow0 + 32 * (d + 1));
          v1 = lds_read_tr8(lds, tb + vrow1 + 32 * (d + 1));
        }
        mfma_pv(o[d], pa, vb, escale);
      }
    }
    mfma_drain();
    // all waves are past their last read of the ring; decide whether to recompute
    const bool over = mu != -INFINITY && m_true > mu + kHeadroom;
    if (!__syncthreads_or(over)) break;
    mu = m_true;  // second pass: reference = true max, so every e <= 0
  }

  // ---- merge the TL waves of each row block, normalise, write partial O and lse
  __syncthreads();  // the ring is free from here on
  float* st_m = (float*)lds;        // [4 waves][32]
  float* st_l = st_m + 4 * 32;
  float* st_f = st_l + 4 * 32;
  const float l_row = l_run + __shfl_xor(l_run, 32);
  if (lane < 32) {
    st_m[wave * 32 + n] = mu;
    st_l[wave * 32 + n] = l_row;
  }
  __syncthreads();
  float Mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < TL; ++t) Mx = fmaxf(Mx, st_m[(rg * TL + t) * 32 + n]);
  float Ls = 0.f;
#pragma unroll
  for (int t = 0; t < TL; ++t) {
    const float mt = st_m[(rg * TL + t) * 32 + n];
    if (mt != -INFINITY) Ls += st_l[(rg * TL + t) * 32 + n] * exp2f(mt - Mx);
  }
  const float f = (mu != -INFINITY && Ls > 0.f) ? exp2f(mu - Mx) * p.kv_scale / Ls : 0.f;
  if (lane < 32) st_f[wave * 32 + n] = f;
  if (tl == 0 && lane < 32 && row_ok)
    p.partial_lse[prow + R] = Ls > 0.f ? (Mx + log2f(Ls) - kLog2PScale) * kLn2 : -INFINITY;
  __syncthreads();

  // per-register factors: register r of every block holds row 8(r/4) + 4gg + r%4
  float fr[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *(const float4*)(st_f + wave * 32 + 8 * q + 4 * gg);
    fr[4 * q] = v.x;
    fr[4 * q + 1] = v.y;
    fr[4 * q + 2] = v.z;
    fr[4 * q + 3] = v.w;
  }

  float* out = p.partial_o + prow * kDv;
  if constexpr (TL == 1) {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const f32x16 v = o[d];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wrow0 + tok_of(gg, r);
        if (row < M) out[(int64_t)row * kDv + 32 * d + n] = v[r] * fr[r];
      }
    }
  } else {
    float* mbuf = (float*)(lds + 4096);  // [4 waves][32 rows][kMergeStride]
    float* mine = mbuf + wave * 32 * kMergeStride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) __syncthreads();  // previous half fully read
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const f32x16 v = o[8 * half + dd];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          mine[tok_of(gg, r) * kMergeStride + 32 * dd + n] = v[r] * fr[r];
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < RG * 32 * 64; idx += 256) {
        const int rgi = idx / (32 * 64);
        const int rem = idx - rgi * 32 * 64;
        const int row = rem >> 6, c4 = rem & 63;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int t = 0; t < TL; ++t) {
          const float4 v =
              *(const float4*)(mbuf + ((rgi * TL + t) * 32 + row) * kMergeStride + 4 * c4);
          acc.x += v.x;
          acc.y += v.y;
          acc.z += v.z;
          acc.w += v.w;
        }
        const int grow = row0 + rgi * 32 + row;
        if (grow < M) *(float4*)(out + (int64_t)grow * kDv + 256 * half + 4 * c4) = acc;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int rows_per_group, hipStream_t s) {
  const int64_t units = (int64_t)p.batch * p.num_splits;
  const int64_t blocks = ((units + 7) / 8) * 8 * p.groups;
  switch (rows_per_group) {
    case 32: decode_kernel<1><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    case 64: decode_kernel<2><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    case 128: decode_kernel<4><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla

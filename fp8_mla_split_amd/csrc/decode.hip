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
// Work decomposition.  A workgroup is four wavefronts, one per SIMD (a lone wave's 512
// registers hold a 32x512 fp32 output accumulator in AGPRs).  It owns 128 query rows
// (rows = (query token, head) pairs of one request; wave w takes rows 32w .. 32w+31) and one
// chunk of that request's tokens; every wave reads every KV tile of the chunk from LDS, so
// each KV byte crosses HBM and L2 once per 128 rows.
//
// KV staging.  A tile is 32 tokens x 576 bytes; a step is two tiles (64 tokens).  Tiles go
// HBM -> LDS with buffer_load ... lds (16 bytes per lane, no VGPR round trip) into an
// 8-tile ring (152 KiB of the CU's 160 KiB) = 4 step slots.  While the waves work on steps
// i and i + 1, steps i + 2 and i + 3 are in flight.  Rows are stored with a 592-byte pitch
// (37 x 16 B); the 64-bank LDS then serves both read patterns below without conflicts.
// The buffer resource of each tile is bounded by the number of valid rows, so rows past
// the end of the sequence arrive as zeros: no NaN bytes from a page's unused tail can reach
// the P.V product (0 x NaN).  The query rows are staged through the same ring (in its last
// four tile slots, before the ring starts) and then held in registers.  Every DMA is issued
// from inline asm and waited on with explicit vmcnt counts: the compiler does not track
// them, so none of its own waits drain the ring, and the kernel issues no compiler-visible
// global load before the main loop for the same reason.  M0 is written only by these asm
// statements (the compiler uses it for nothing else in this kernel).
//
// Math per step (per wave, 32 rows x 64 tokens), all on FP8 MFMA v_mfma_scale_f32_32x32x64:
//  * S^T = K . Q^T per tile: tokens along M, rows along N, 576 = 9 x 64 channels along K;
//    the two tiles' chains are interleaved.  Computing the transpose puts each lane's 16
//    scores for one row exactly where the P.V step needs them as its A operand.  MFMA
//    token m reads LDS row perm_row(m), so register r of lane half gg holds tile token
//    2r + gg; the permutation makes the transposed V reads below conflict-free.
//  * Online softmax in base 2 against a fixed reference max mu per row (the max of the row's
//    first step with a visible position), so the 256-register O is never rescaled.  Each
//    step's probabilities are normalised per row by 2^-e (e = floor of the row's step max
//    above mu) before the FP8 cast, and the MFMA's E8M0 scale multiplies them back by 2^e.
//    The two lanes that hold a row (n and n + 32) use the same e.  If a row's true max ends
//    up more than kHeadroom above mu (fp32 range at risk), the workgroup recomputes its
//    chunk once with mu = the true max.
//  * P is encoded as hi = e4m3(p) and lo = e4m3(p - hi), both in the same units, and
//    O += hi . V + lo . V as two MFMAs over the step's 64 tokens that share one V operand
//    (P.V with about 7 bits of P mantissa; a single e4m3 P costs several times the 2e-3
//    normalised-L1 budget against the fp64 oracle).
//  * V (the first 512 columns of the same tiles) is read transposed with ds_read_b64_tr_b8.
//  * Software pipeline: the 18 QK MFMAs of step i+1 are issued before the 32 PV MFMAs of
//    step i, the softmax of step i+1 is issued in the gaps between those PV MFMAs, the DMA
//    of step i+3 between the QK MFMAs, and the per-step barrier right after the last PV
//    MFMA, so the matrix pipe keeps working through it.
#include <type_traits>

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
constexpr int kSlots = 8;                   // tile slots; a step takes two
constexpr int kStepSlots = kSlots / 2;
constexpr int kLds = kSlots * kSlot;        // 155648 bytes
constexpr int kLmin = 8;                    // fewest DMA instructions a wave issues per step
constexpr int kQSlot = 4;                   // the 128 query rows are staged in tile slots 4..7
constexpr int kQDma = 72;                   // 128 rows x 576 B / 1 KiB per DMA instruction
constexpr int kRows = 128;                  // query rows per workgroup
constexpr float kHeadroom = 64.0f;          // log2 range of a pass above its reference max
constexpr float kLog2PScale = 7.807354922057604f;  // log2(224): p in [0, 448)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKAhead = 2;                  // QK MFMA pairs whose K fragments are in flight
constexpr int kVAhead = 2;                  // PV blocks whose V fragments are in flight

// MFMA token index -> LDS row of the tile: bits (b4 b3 b2 b1 b0) -> (b4 b3 b1 b0 b2).
__device__ __forceinline__ int perm_row(int m) {
  return (m & 0x18) | ((m & 3) << 1) | ((m >> 2) & 1);
}
// Token index held in register r of a 32x32 MFMA result by lanes of half gg.
__device__ __forceinline__ int tok_of(int gg, int r) { return 8 * (r >> 2) + 4 * gg + (r & 3); }

// 16 bytes per lane, global -> LDS at M0 + 16 * lane, with M0 = lds_addr + IMM (the
// constant part of the address stays out of the register file).  One wait state separates
// the M0 write from the DMA that reads it.
template <int IMM>
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff,
                                      __amdgpu_buffer_rsrc_t rsrc) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "n"(IMM)
               : "memory", "m0", "scc");
}
// As dma16, with the constant part in an SGPR.
__device__ __forceinline__ void dma16_s(uint32_t lds_addr, uint32_t voff,
                                        __amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(off)
               : "memory", "m0", "scc");
}

// FP8 x FP8 32x32x64 MFMA with explicit register classes: the scores live in VGPRs and O in
// AGPRs (left to itself the compiler puts every accumulator in AGPRs, which then do not
// hold O).  The "memory" clobber keeps the LDS fragment reads where the source places them.
// Hazards the compiler cannot see through the asm are covered explicitly: s_nop 1 before
// each MFMA covers a VALU write of an operand just before it, and at least 24 wait states
// separate the last MFMA of a chain from any non-MFMA reader of its result (mfma_drain2,
// which takes the accumulators as operands: the compiler treats an asm output as ready at
// once and would otherwise copy it straight after the MFMA).
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
__device__ __forceinline__ void mfma_drain2(f32x16& a, f32x16& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b)::"memory");
}
__device__ __forceinline__ void mfma_drain_acc(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc)::"memory");
}
// Orders later reads of acc after the preceding asm (no wait states of its own).
__device__ __forceinline__ void acc_fence(f32x16& acc) { asm volatile("" : "+a"(acc)); }

// (value of lane n, value of lane n + 32) in every lane n and n + 32, by one
// v_permlane32_swap (no LDS traffic).
__device__ __forceinline__ f32x2 row_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return (f32x2){__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// One accumulator block, copied to VGPRs where it is used.  The empty asm keeps the compiler
// from hoisting the copies of all 256 accumulator registers to one place, which would need
// more VGPRs than a wave has.
__device__ __forceinline__ f32x16 from_acc(const f32x16& a) {
  f32x16 v;
  asm volatile("" : "=v"(v) : "0"(a));
  return v;
}
// Keeps the compiler from moving instructions across this point (used to interleave the
// softmax VALU work with the PV MFMAs in source order).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

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

__device__ __forceinline__ i32x8 cat8(const i32x4& a, const i32x4& b) {
  return (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Softmax state of one lane: its row's reference max, the running true max and its share of
// the row's sum of 2^(x - mu) * 224.
struct RowState {
  float mu, m_true, l_run;
};

// One step's scores and probabilities (tile a in sa, tile b in sb).
struct StepTile {
  f32x16 sa, sb;  // raw scores, then probabilities in place
  float off;      // exp2 argument offset
  float psum;
  int ef;
  i32x8 hi, lo;   // P bytes: [tile a | tile b]
};

// K fragments of one QK MFMA pair (tile a, tile b).
struct KPair {
  i32x4 a0, a1, b0, b1;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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

  // Wave-uniform scalars come from the constant address space (scalar loads, lgkmcnt).
  const __attribute__((address_space(4))) int32_t* seq_lens =
      (const __attribute__((address_space(4))) int32_t*)p.seq_lens;
  const __attribute__((address_space(4))) int32_t* page_table =
      (const __attribute__((address_space(4))) int32_t*)p.page_table;
  int L = seq_lens[b];
  const int Lmax = p.max_pages * p.page_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int ntiles_all = (L + kTile - 1) / kTile;
  const int per = (ntiles_all + S - 1) / S;
  const int t_begin = s * per;
  const int ntiles = max(min(t_begin + per, ntiles_all) - t_begin, 0);

  const int row0 = g * kRows;
  const int64_t prow = (int64_t)(b * S + s) * M;  // first partial row of this (b, s)
  if (ntiles == 0) {
    for (int i = threadIdx.x; i < kRows; i += 256)
      if (row0 + i < M) p.partial_lse[prow + row0 + i] = -INFINITY;
    return;
  }

  const int wrow0 = row0 + wave * 32;
  const int R = wrow0 + n;  // this lane's query row (score and P layout)
  const bool row_ok = R < M;
  // last visible position of the row (bottom-right causal); rows past M are never stored
  const int lim = row_ok ? L - p.q_tokens + R / p.heads : 0x7FFFFFFF;
  const int lim_min = L - p.q_tokens + wrow0 / p.heads;
  const int nsteps = (ntiles + 1) / 2;
  const int P = p.page_size;

  // ---- DMA lane offsets.  Of a tile's 19 DMA instructions, wave w issues k = w + 4 i
  // (i < 4, and i = 4 for waves 0..2): LDS bytes 1024 w + 4096 i of the slot.  Chunk
  // pch = 64k + lane of the tile is row pch / 37, 16-byte column pch % 37 of the LDS tile;
  // column 36 is the pad (it receives the next row's first 16 bytes, or zeros).
  uint32_t voff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t pch = 64u * (uint32_t)(wave + 4 * i) + (uint32_t)lane;
    const uint32_t row = pch / 37u;
    voff[i] = 16u * (pch - row);
  }
  const uint32_t wave_lds = lds_base + (uint32_t)wave * 1024u;

  // Page of tile ti of the chunk (scalar load); tiles past the chunk map to a valid entry
  // and load nothing.
  auto page_of = [&](int ti) __attribute__((always_inline)) -> int {
    const int t = min(ti, ntiles - 1);
    return page_table[(int64_t)b * p.max_pages + ((t_begin + t) * kTile) / P];
  };
  auto issue_tile = [&](int ti, int page, uint32_t slot_lds, auto jc)
      __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    const uint8_t* base = p.kv;
    int nrec = 0;
    if (ti < ntiles) {
      const int T0 = (t_begin + ti) * kTile;
      base = p.kv + ((int64_t)page * P + (T0 % P)) * kD;
      nrec = min(kTile, L - T0) * kD;
    }
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, 0x00020000);
    dma16<j * kSlot + 0 * 4096>(slot_lds, voff[0], rsrc);
    dma16<j * kSlot + 1 * 4096>(slot_lds, voff[1], rsrc);
    dma16<j * kSlot + 2 * 4096>(slot_lds, voff[2], rsrc);
    dma16<j * kSlot + 3 * 4096>(slot_lds, voff[3], rsrc);
    if (wave < 3) dma16<j * kSlot + 4 * 4096>(slot_lds, voff[4], rsrc);
  };
  // Both tiles of step st into its step slot.  Every step is issued, also past the end of
  // the chunk (those load nothing and write zeros into a free slot), so the number of DMA
  // instructions in flight behind any step is fixed and every wait below is a constant.
  auto issue_step = [&](int st, int pg0, int pg1) __attribute__((always_inline)) {
    const uint32_t slot_lds = wave_lds + (uint32_t)((st % kStepSlots) * 2 * kSlot);
    issue_tile(2 * st, pg0, slot_lds, std::integral_constant<int, 0>{});
    issue_tile(2 * st + 1, pg1, slot_lds, std::integral_constant<int, 1>{});
  };

  const int G16 = lane >> 4, i16 = lane & 15;
  const uint32_t vcol = 16 * (G16 & 1) + 8 * (i16 & 1);
  const uint32_t vrow0 = perm_row(tok_of(gg, i16 >> 1)) * kPitch + vcol;
  const uint32_t vrow1 = perm_row(tok_of(gg, 8 + (i16 >> 1))) * kPitch + vcol;
  const uint32_t krow = perm_row(n) * kPitch + 32 * gg;
  const float c2 = p.c2;

  auto step_base = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)((st % kStepSlots) * 2 * kSlot);
  };

  i32x8 qf[9];  // Q fragments (B operand of S^T = K . Q^T), staged once per pass

  auto read_kpair = [&](uint32_t sb, int c) __attribute__((always_inline)) -> KPair {
    KPair k;
    k.a0 = lds_read16(lds, sb + krow + 64 * c);
    k.a1 = lds_read16(lds, sb + krow + 64 * c + 16);
    k.b0 = lds_read16(lds, sb + kSlot + krow + 64 * c);
    k.b1 = lds_read16(lds, sb + kSlot + krow + 64 * c + 16);
    return k;
  };

  RowState rs{-INFINITY, -INFINITY, 0.f};

  // Softmax of one step in 17 pieces that the caller interleaves with MFMAs (piece 0 must
  // come at least 24 wait states after the last MFMA that wrote t.sa / t.sb).  A tile that
  // this wave does not own (past the chunk, or past the loop) is masked whole.
  auto softmax_piece = [&](StepTile& t, int st, int piece) __attribute__((always_inline)) {
    if (piece == 0) {
      // mask the tail / causal positions: register r holds tile token 2 r + gg, visible
      // while T0 + 2 r + gg <= lim, i.e. while r <= c
      const int T0a = (t_begin + 2 * st) * kTile;
      const int T0b = T0a + kTile;
      const bool va = 2 * st < ntiles, vb = 2 * st + 1 < ntiles;
      if (!va || T0a + kTile - 1 > lim_min) {
        const int c = va ? (lim - T0a - gg) >> 1 : -1;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r > c) t.sa[r] = -INFINITY;
      }
      if (!vb || T0b + kTile - 1 > lim_min) {
        const int c = vb ? (lim - T0b - gg) >> 1 : -1;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r > c) t.sb[r] = -INFINITY;
      }
      float m = fmaxf(fmaxf(t.sa[0], t.sa[1]), t.sa[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, t.sa[r]), t.sa[r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) m = fmaxf(fmaxf(m, t.sb[r]), t.sb[r + 1]);
      m = fmaxf(m, t.sa[15]);
      const f32x2 both = row_pair(m);
      const float mx = fmaxf(both[0], both[1]) * c2;  // the row's max; c2 > 0
      if (rs.mu == -INFINITY) rs.mu = mx;  // first step with a visible position
      rs.m_true = fmaxf(rs.m_true, mx);
      const float mref = rs.mu == -INFINITY ? 0.f : rs.mu;
      const float ef = fminf(fmaxf(floorf(mx - mref), -126.0f), 127.0f);
      t.ef = (int)ef;
      t.off = mref + ef - kLog2PScale;
    } else if (piece <= 8) {  // p = 2^(c2 s - off), in [0, 448); 0 where masked
      const int q = piece - 1;  // values 4q .. 4q + 3 of [sa | sb]
      float sum = q == 0 ? 0.f : t.psum;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (q < 4) {
          t.sa[4 * q + r] = __builtin_amdgcn_exp2f(fmaf(t.sa[4 * q + r], c2, -t.off));
          sum += t.sa[4 * q + r];
        } else {
          t.sb[4 * (q - 4) + r] = __builtin_amdgcn_exp2f(fmaf(t.sb[4 * (q - 4) + r], c2, -t.off));
          sum += t.sb[4 * (q - 4) + r];
        }
      }
      t.psum = sum;
      if (q == 7) rs.l_run += ldexpf(sum, t.ef);
    } else {  // pieces 9..16: P bytes 4q .. 4q+3 as hi and lo e4m3
      const int q = piece - 9;
      const f32x16& v = q < 4 ? t.sa : t.sb;
      const int o = 4 * (q & 3);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[o], v[o + 1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[o + 2], v[o + 3], w, true);
      const f32x2 d01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const f32x2 d23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      int w2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[o] - d01[0], v[o + 1] - d01[1], 0, false);
      w2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[o + 2] - d23[0], v[o + 3] - d23[1], w2, true);
      t.hi[q] = w;
      t.lo[q] = w2;
    }
  };

  f32x16 o[16];
  i32x8 phi, plo;  // P of the step whose PV comes next, and its per-row exponent
  int ef = 0;

  // O += [hi | lo] . V of step st over the 16 blocks of 32 value columns, one V fragment
  // (64 tokens x 32 columns) per block shared by the hi and lo MFMAs.  With kNext, the
  // next step's softmax fills the gaps between these MFMAs.
  auto pv_step = [&](int st, StepTile& nx, auto with_next) __attribute__((always_inline)) {
    constexpr bool kNext = decltype(with_next)::value;
    const uint32_t sb = step_base(st);
    const int escale = 127 + ef;
    i32x2 va[16][4];
#pragma unroll
    for (int d = 0; d < kVAhead; ++d) {
      va[d][0] = lds_read_tr8(lds, sb + vrow0 + 32 * d);
      va[d][1] = lds_read_tr8(lds, sb + vrow1 + 32 * d);
      va[d][2] = lds_read_tr8(lds, sb + kSlot + vrow0 + 32 * d);
      va[d][3] = lds_read_tr8(lds, sb + kSlot + vrow1 + 32 * d);
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      if (d + kVAhead < 16) {
        const int e = d + kVAhead;
        va[e][0] = lds_read_tr8(lds, sb + vrow0 + 32 * e);
        va[e][1] = lds_read_tr8(lds, sb + vrow1 + 32 * e);
        va[e][2] = lds_read_tr8(lds, sb + kSlot + vrow0 + 32 * e);
        va[e][3] = lds_read_tr8(lds, sb + kSlot + vrow1 + 32 * e);
      }
      const i32x8 vb = (i32x8){va[d][0][0], va[d][0][1], va[d][1][0], va[d][1][1],
                               va[d][2][0], va[d][2][1], va[d][3][0], va[d][3][1]};
      mfma_pv(o[d], phi, vb, escale);
      if constexpr (kNext) {
        sched_fence();
        if (d == 0) mfma_drain2(nx.sa, nx.sb);  // the QK chains' results are read from here
        if (2 * d < 17) softmax_piece(nx, st + 1, 2 * d);
        sched_fence();
      }
      mfma_pv(o[d], plo, vb, escale);
      if constexpr (kNext) {
        if (2 * d + 1 < 17) {
          sched_fence();
          softmax_piece(nx, st + 1, 2 * d + 1);
          sched_fence();
        }
      }
    }
  };

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = (f32x16){0.f};
    rs.l_run = 0.f;

    // ---- stage the workgroup's 128 query rows (contiguous in q8) in tile slots 4..7 with
    // steps 0 and 1 in flight beside them.  Each pass stages them again, so the Q fragments
    // are live within a pass only.
    {
      const int qrows = min(kRows, M - row0);
      const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.q8 + ((int64_t)b * M + row0) * kD), 0, qrows * kD, 0x00020000);
      // instruction i = wave + 4 j moves bytes [1024 i, 1024 (i + 1)) of the rows
      const uint32_t qvoff = (uint32_t)wave * 1024u + 16u * (uint32_t)lane;
#pragma unroll
      for (int j = 0; j < kQDma / 4; ++j)
        dma16_s(wave_lds, qvoff + 4096u * j, qrsrc, kQSlot * kSlot + 4096 * j);
    }
    issue_step(0, page_of(0), page_of(1));
    issue_step(1, page_of(2), page_of(3));
    wait_vmcnt<2 * kLmin>();  // this wave's Q chunks have landed
    __syncthreads();
    {
      const uint32_t qrow = (uint32_t)(kQSlot * kSlot + (wave * 32 + n) * kD + 32 * gg);
#pragma unroll
      for (int c = 0; c < 9; ++c)
        qf[c] = cat8(lds_read16(lds, qrow + 64 * c), lds_read16(lds, qrow + 64 * c + 16));
    }
    __syncthreads();  // the Q slots are free from here on
    issue_step(2, page_of(4), page_of(5));

    // ---- step 0: scores and probabilities, not overlapped with anything
    wait_vmcnt<2 * kLmin>();
    __syncthreads();
    {
      StepTile t;
      const uint32_t sb = step_base(0);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const KPair k = read_kpair(sb, c);
        if (c == 0) {
          t.sa = mfma_qk_first(cat8(k.a0, k.a1), qf[0]);
          t.sb = mfma_qk_first(cat8(k.b0, k.b1), qf[0]);
        } else {
          mfma_qk(t.sa, cat8(k.a0, k.a1), qf[c]);
          mfma_qk(t.sb, cat8(k.b0, k.b1), qf[c]);
        }
      }
      mfma_drain2(t.sa, t.sb);
#pragma unroll
      for (int piece = 0; piece < 17; ++piece) softmax_piece(t, 0, piece);
      phi = t.hi;
      plo = t.lo;
      ef = t.ef;
    }
    // step 1 visible to every wave before the loop reads it
    wait_vmcnt<kLmin>();
    __syncthreads();
    int pg0 = page_of(6), pg1 = page_of(7);  // pages of the next step to issue (3)

    for (int st = 0; st + 1 < nsteps; ++st) {
      // step st + 1 is visible and step slot (st - 1) % 4 is free: barrier at the end of the
      // previous iteration, or just above
      StepTile t;
      const uint32_t sb1 = step_base(st + 1);
      KPair kp[9];
#pragma unroll
      for (int c = 0; c < kKAhead; ++c) kp[c] = read_kpair(sb1, c);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        if (c + kKAhead < 9) kp[c + kKAhead] = read_kpair(sb1, c + kKAhead);
        if (c == 0) {
          t.sa = mfma_qk_first(cat8(kp[0].a0, kp[0].a1), qf[0]);
          t.sb = mfma_qk_first(cat8(kp[0].b0, kp[0].b1), qf[0]);
        } else {
          mfma_qk(t.sa, cat8(kp[c].a0, kp[c].a1), qf[c]);
          mfma_qk(t.sb, cat8(kp[c].b0, kp[c].b1), qf[c]);
        }
        if (c == 1) issue_step(st + 3, pg0, pg1);  // into the slot that step st - 1 left
      }
      pv_step(st, t, std::true_type{});
      phi = t.hi;
      plo = t.lo;
      ef = t.ef;
      // step st + 2 landed for every wave, and every wave is past its reads of step st
      wait_vmcnt<kLmin>();
      __syncthreads();
      pg0 = page_of(2 * (st + 4));
      pg1 = page_of(2 * (st + 4) + 1);
    }
    {
      StepTile unused;
      pv_step(nsteps - 1, unused, std::false_type{});  // landed before the last barrier
    }
    mfma_drain_acc(o[15]);
#pragma unroll
    for (int d = 0; d < 15; ++d) acc_fence(o[d]);
    wait_vmcnt<0>();  // the steps past the chunk have landed too
    // all waves are past their last read of the ring; decide whether to recompute
    const bool over = rs.mu != -INFINITY && rs.m_true > rs.mu + kHeadroom;
    if (!__syncthreads_or(over)) break;
    // second pass: reference = the row's true max, so every exponent is <= 0
    rs.mu = rs.m_true;
  }

  // ---- normalise, write partial O (fp16, in units of kv_scale: |O| <= 448) and lse
  const float mu = rs.mu;
  const f32x2 lpair = row_pair(rs.l_run);
  const float Ls = lpair[0] + lpair[1];  // both halves of the row
  const float f = (mu != -INFINITY && Ls > 0.f) ? 1.0f / Ls : 0.f;
  if (lane < 32 && row_ok)
    p.partial_lse[prow + R] = Ls > 0.f ? (mu + log2f(Ls) - kLog2PScale) * kLn2 : -INFINITY;

  // per-register factors: register r of every block holds row 8(r/4) + 4gg + r%4, i.e. the
  // factor of lane tok_of(gg, r) (lanes n and n + 32 hold the same value)
  float fr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) fr[r] = __shfl(f, tok_of(gg, r));

  // register r of block d is row wrow0 + tok_of(gg, r), column 32 d + n
  _Float16* wout = (_Float16*)p.partial_o + (prow + wrow0) * kDv + n;
  if (wrow0 + 32 <= M) {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const f32x16 v = from_acc(o[d]);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        wout[tok_of(gg, r) * kDv + 32 * d] = (_Float16)(v[r] * fr[r]);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const f32x16 v = from_acc(o[d]);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (wrow0 + tok_of(gg, r) < M)
          wout[tok_of(gg, r) * kDv + 32 * d] = (_Float16)(v[r] * fr[r]);
    }
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int rows_per_group, hipStream_t s) {
  if (rows_per_group != kRows) return hipErrorInvalidValue;
  const int64_t units = (int64_t)p.batch * p.num_splits;
  const int64_t blocks = ((units + 7) / 8) * 8 * p.groups;
  decode_kernel<<<(unsigned)blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace mla

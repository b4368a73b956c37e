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
// registers hold a 32x512 fp32 output accumulator in AGPRs).  It owns 32*RG query rows
// (rows = (query token, head) pairs of one request; RG = 2 or 4) and one chunk of that
// request's tokens.  Wave w works on row block w / TL and takes every TL-th tile of the chunk
// (TL = 4 / RG): with RG = 4 all four waves read every tile, with RG = 2 two pairs of waves
// take alternate tiles.  Waves that share a row block merge (max, sum, O) in LDS at the end.
//
// KV staging.  A tile is 32 tokens x 576 bytes.  Tiles go HBM -> LDS with buffer_load ... lds
// (16 bytes per lane, no VGPR round trip) into an 8-slot ring (152 KiB of the CU's 160 KiB),
// grouped in stages of TL tiles.  While the waves work on stages st and st + 1, stages up to
// st + NST - 1 are in flight (6 tiles for RG = 4, 4 for RG = 2).  Rows are stored with a
// 592-byte pitch (37 x 16 B); the 64-bank LDS then serves both read patterns below without
// conflicts.  The buffer resource of each tile is bounded by the number of valid rows, so
// rows past the end of the sequence arrive as zeros: no NaN bytes from a page's unused tail
// can reach the P.V product (0 x NaN).  The query rows are staged through the same ring (in
// its last RG slots, before the ring starts) and then held in registers.  Every DMA is issued
// from inline asm and waited on with explicit vmcnt counts: the compiler does not track them,
// so none of its own waits drain the ring, and the kernel issues no compiler-visible global
// load before the main loop for the same reason.
//
// Math per tile (per wave, 32 rows x 32 tokens), all on FP8 MFMA v_mfma_scale_f32_32x32x64:
//  * S^T = K . Q^T: tokens along M, rows along N, 576 = 9 x 64 channels along K.  Computing
//    the transpose puts each lane's 16 scores for one row exactly where the P.V step needs
//    them as its A operand (no data movement).  MFMA token m reads LDS row perm_row(m); the
//    permutation makes the transposed V reads below touch 8 rows of one parity, which keeps
//    them conflict-free.
//  * Online softmax in base 2 against a fixed reference max mu per row (the max of the row's
//    first tile with a visible position), so the 256-register O is never rescaled.  Each
//    tile's probabilities are normalised per row by 2^-e (e = floor of the row's tile max
//    above mu) before the FP8 cast, and the MFMA's per-lane E8M0 scale multiplies them back
//    by 2^e.  The two lanes that hold a row (n and n + 32) must use the same e: each holds
//    16 K-elements of both 32-element scale blocks of the row, and a block's scale is read
//    from one of them.  If a row's true max ends up more than kHeadroom above mu (fp32 range
//    at risk), the workgroup recomputes its chunk once with mu = the true max.
//  * P is encoded as hi = e4m3(p) and lo = e4m3(p - hi), both in the same units; one
//    32x32x64 MFMA takes [hi | lo] for 32 tokens against [V | V], i.e. P.V with about
//    7 bits of P mantissa.  (A single e4m3 P costs ~3e-3 normalised L1 error against the
//    fp64 oracle at 128K context, more than the 2e-3 budget.)
//  * V (the first 512 columns of the same tile) is read transposed with ds_read_b64_tr_b8.
//  * Software pipeline: the 9 QK MFMAs of tile i+1 are issued before the 16 PV MFMAs of tile
//    i, and the softmax of tile i+1 (about 100 VALU instructions per lane) is issued in the
//    gaps between those PV MFMAs, so the matrix pipe is not left idle while the VALU works.
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

// As dma16, for the unrolled Q staging loop whose offsets are compile-time after unrolling.
__device__ __forceinline__ void dma16_q(uint32_t lds_addr, uint32_t voff,
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
// separate the last MFMA of a chain from any non-MFMA reader of its result (mfma_drain,
// which takes the accumulator as an operand: the compiler treats an asm output as ready
// at once and would otherwise copy it straight after the MFMA).
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
// 24 wait states after the last MFMA that wrote acc, before anything reads it.  acc is an
// operand so that no read or copy of it can be placed ahead of the wait states.
__device__ __forceinline__ void mfma_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc)::"memory");
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

// Softmax state of one lane: its row's reference max, the running true max and its share of
// the row's sum of 2^(x - mu) * 224.
struct RowState {
  float mu, m_true, l_run;
};

// One tile's probabilities, in pieces that the caller interleaves with MFMAs.
struct SoftmaxTile {
  f32x16 s;   // raw scores
  float off;  // exp2 argument offset
  float psum;
  int ef;
  float pv[16];
  i32x8 pa;
};

template <int RG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const DecodeParams p) {
  constexpr int TL = 4 / RG;               // waves sharing a row block
  constexpr int NST = kSlots / TL;         // stages in the ring
  constexpr int LMIN = 4 * TL;             // fewest DMA instructions a wave issues per stage
  constexpr int QSLOT = kSlots - RG;       // the query rows are staged in the last RG slots
  constexpr int P0 = QSLOT / TL;           // stages that fit beside them
  constexpr int QDMA = 18 * RG;            // 32*RG rows x 576 B / 1 KiB per DMA instruction
  static_assert(RG == 2 || RG == 4, "row blocks per workgroup");
  static_assert(NST >= 4 && P0 >= 1 && P0 <= NST - 1, "ring layout");
  static_assert(32 * RG * kD <= RG * kSlot, "staged Q fits its slots");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rb = wave / TL, tl = wave % TL;
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

  const int row0 = g * 32 * RG;
  const int64_t prow = (int64_t)(b * S + s) * M;  // first partial row of this (b, s)
  if (ntiles == 0) {
    for (int i = threadIdx.x; i < 32 * RG; i += 256)
      if (row0 + i < M) p.partial_lse[prow + row0 + i] = -INFINITY;
    return;
  }

  const int wrow0 = row0 + rb * 32;
  const int R = wrow0 + n;  // this lane's query row (score and P layout)
  const bool row_ok = R < M;
  // last visible position of the row (bottom-right causal); rows past M are never stored
  const int lim = row_ok ? L - p.q_tokens + R / p.heads : 0x7FFFFFFF;
  const int lim_min = L - p.q_tokens + wrow0 / p.heads;
  const int nsteps = (ntiles + TL - 1) / TL;
  const int P = p.page_size;

  // ---- DMA lane offsets.  Of a tile's 19 DMA instructions, wave w issues k = w, w+4, ...
  // Chunk pch = 64k + lane of the tile is row pch / 37, 16-byte column pch % 37 of the LDS
  // tile; column 36 is the pad (it receives the next row's first 16 bytes, or zeros).
  uint32_t voff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t pch = 64u * (uint32_t)(wave + 4 * i) + (uint32_t)lane;
    const uint32_t row = pch / 37u;
    voff[i] = 16u * (pch - row);
  }

  // this wave's share of a tile: instructions k = wave + 4 i (i < 4, and i = 4 for waves
  // 0..2), i.e. LDS bytes wave * 1024 + i * 4096 of the slot
  const uint32_t wave_lds = lds_base + (uint32_t)wave * 1024u;
  auto issue_tile = [&](int st, uint32_t slot_lds, auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    const int ti = st * TL + j;
    const uint8_t* base = p.kv;
    int nrec = 0;
    if (ti < ntiles) {
      const int T0 = (t_begin + ti) * kTile;
      const int page = page_table[(int64_t)b * p.max_pages + T0 / P];
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
  auto issue_stage = [&](int st) __attribute__((always_inline)) {
    const uint32_t slot_lds = wave_lds + (uint32_t)((st % NST) * TL * kSlot);
    issue_tile(st, slot_lds, std::integral_constant<int, 0>{});
    if constexpr (TL == 2) issue_tile(st, slot_lds, std::integral_constant<int, 1>{});
  };

  const int G16 = lane >> 4, i16 = lane & 15;
  const uint32_t vcol = 16 * (G16 & 1) + 8 * (i16 & 1);
  const uint32_t vrow0 = perm_row(tok_of(gg, i16 >> 1)) * kPitch + vcol;
  const uint32_t vrow1 = perm_row(tok_of(gg, 8 + (i16 >> 1))) * kPitch + vcol;
  const uint32_t krow = perm_row(n) * kPitch + 32 * gg;
  const float c2 = p.c2;

  auto tile_base = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(((st % NST) * TL + tl) * kSlot);
  };

  i32x8 qf[9];  // Q fragments (B operand of S^T = K . Q^T), staged once per pass

  // S^T = K . Q^T of this wave's tile of stage st (tokens x rows), one fragment read ahead
  auto qk = [&](int st) __attribute__((always_inline)) -> f32x16 {
    const uint32_t tb = tile_base(st) + krow;
    f32x16 acc;
    i32x4 a0 = lds_read16(lds, tb);
    i32x4 a1 = lds_read16(lds, tb + 16);
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const i32x8 a = (i32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      if (c < 8) {
        a0 = lds_read16(lds, tb + 64 * (c + 1));
        a1 = lds_read16(lds, tb + 64 * (c + 1) + 16);
      }
      if (c == 0) acc = mfma_qk_first(a, qf[0]);
      else mfma_qk(acc, a, qf[c]);
    }
    return acc;
  };

  RowState rs{-INFINITY, -INFINITY, 0.f};

  // Softmax of one tile, in 9 pieces that the caller interleaves with MFMAs (piece 0 must
  // come at least 24 wait states after the last MFMA that wrote t.s).  A tile that this wave
  // does not own (past the chunk, or past the loop) is masked whole: p = 0, no state change.
  auto softmax_piece = [&](SoftmaxTile& t, int st, bool valid, int piece)
      __attribute__((always_inline)) {
    switch (piece) {
      case 0: {  // mask the tail / causal positions, lane max, reference max, exponent
        const int T0 = (t_begin + st * TL + tl) * kTile;
        if (!valid) {
#pragma unroll
          for (int r = 0; r < 16; ++r) t.s[r] = -INFINITY;
        } else if (T0 + kTile - 1 > lim_min) {
          // register r holds tile token perm_row(tok_of(gg, r)) = 2 r + gg, visible while
          // T0 + 2 r + gg <= lim, i.e. while r <= c
          const int c = (lim - T0 - gg) >> 1;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (r > c) t.s[r] = -INFINITY;
        }
        float m = fmaxf(fmaxf(t.s[0], t.s[1]), t.s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, t.s[r]), t.s[r + 1]);
        m = fmaxf(m, t.s[15]);
        // the row's max over both lanes that hold it (lanes n and n + 32)
        const f32x2 both = row_pair(m);
        const float mx = fmaxf(both[0], both[1]) * c2;  // c2 > 0
        if (rs.mu == -INFINITY) rs.mu = mx;  // first tile with a visible position
        rs.m_true = fmaxf(rs.m_true, mx);
        const float mref = rs.mu == -INFINITY ? 0.f : rs.mu;
        const float ef = fminf(fmaxf(floorf(mx - mref), -126.0f), 127.0f);
        t.ef = (int)ef;
        t.off = mref + ef - kLog2PScale;
        break;
      }
      case 1:
      case 2:
      case 3:
      case 4: {  // p = 2^(c2 s - off), in [0, 448); 0 where masked
        const int r0 = 4 * (piece - 1);
        float sum = piece == 1 ? 0.f : t.psum;
#pragma unroll
        for (int r = r0; r < r0 + 4; ++r) {
          t.pv[r] = __builtin_amdgcn_exp2f(fmaf(t.s[r], c2, -t.off));
          sum += t.pv[r];
        }
        t.psum = sum;
        if (piece == 4) rs.l_run += ldexpf(sum, t.ef);
        break;
      }
      default: {  // pieces 5..8: P as hi + lo e4m3 bytes (A operand bytes 0..15 hi, 16..31 lo)
        const int q = piece - 5;
        const float* pv = t.pv;
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q], pv[4 * q + 1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q + 2], pv[4 * q + 3], w, true);
        const f32x2 d01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const f32x2 d23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        int w2 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q] - d01[0], pv[4 * q + 1] - d01[1], 0,
                                                 false);
        w2 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * q + 2] - d23[0], pv[4 * q + 3] - d23[1], w2,
                                             true);
        t.pa[q] = w;
        t.pa[4 + q] = w2;
        break;
      }
    }
  };

  f32x16 o[16];

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = (f32x16){0.f};
    rs.l_run = 0.f;
    // ---- stage the workgroup's query rows (contiguous in q8) in the last RG slots, with the
    // first P0 KV stages in flight beside them.  Each pass stages them again, so the Q
    // fragments are live within a pass only.
    {
      const int qrows = min(32 * RG, M - row0);
      const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.q8 + ((int64_t)b * M + row0) * kD), 0, qrows * kD, 0x00020000);
      // instruction i = wave + 4 j moves bytes [1024 i, 1024 (i + 1)) of the rows
      const uint32_t qvoff = (uint32_t)wave * 1024u + 16u * (uint32_t)lane;
      static_assert(QDMA % 4 == 0, "every wave issues the same number of Q chunks");
#pragma unroll
      for (int j = 0; j < QDMA / 4; ++j)
        dma16_q(wave_lds, qvoff + 4096u * j, qrsrc, QSLOT * kSlot + 4096 * j);
    }
    // Every stage is issued, also past the end of the chunk (those load nothing and write
    // zeros into a free slot), so the number of DMA instructions in flight behind any stage
    // is fixed and every wait below is a constant.
#pragma unroll
    for (int st = 0; st < P0; ++st) issue_stage(st);
    wait_vmcnt<P0 * LMIN>();  // this wave's Q chunks have landed
    __syncthreads();

    // Q fragments (B operand of S^T = K . Q^T), in registers for the whole pass
    {
      const uint32_t qrow = (uint32_t)(QSLOT * kSlot + (rb * 32 + n) * kD + 32 * gg);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const i32x4 lo = lds_read16(lds, qrow + 64 * c);
        const i32x4 hi = lds_read16(lds, qrow + 64 * c + 16);
        qf[c] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    __syncthreads();  // the Q slots are free from here on
#pragma unroll
    for (int st = P0; st < NST - 1; ++st) issue_stage(st);

    // first tile: scores and probabilities, not overlapped with anything
    wait_vmcnt<(NST - 2) * LMIN>();
    __syncthreads();
    i32x8 pa;  // P of the tile whose PV comes next, and its per-row exponent
    int ef;
    {
      SoftmaxTile t;
      t.s = qk(0);
      mfma_drain(t.s);
#pragma unroll
      for (int piece = 0; piece < 9; ++piece) softmax_piece(t, 0, tl < ntiles, piece);
      pa = t.pa;
      ef = t.ef;
    }

    // O += P . V of stage st over the 16 blocks of 32 value columns; B = [V | V] for
    // [hi | lo].  With a next tile, its softmax fills the gaps between these MFMAs.
    auto pv_tile = [&](int st, SoftmaxTile& nx, bool next_valid, auto with_next)
        __attribute__((always_inline)) {
      constexpr bool kNext = decltype(with_next)::value;
      const uint32_t tb = tile_base(st);
      const int escale = 127 + ef;
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
        if constexpr (kNext) {
          sched_fence();
          if (d == 0) mfma_drain(nx.s);  // the QK chain's result is read from here on
          if (d < 9) softmax_piece(nx, st + 1, next_valid, d);
          sched_fence();
        }
      }
    };

    for (int st = 0; st + 1 < nsteps; ++st) {
      wait_vmcnt<(NST - 3) * LMIN>();
      // stage st + 1 is visible to every wave, and every wave is done with stage st - 1
      __syncthreads();
      issue_stage(st + NST - 1);
      SoftmaxTile t;
      t.s = qk(st + 1);
      pv_tile(st, t, (st + 1) * TL + tl < ntiles, std::true_type{});
      pa = t.pa;
      ef = t.ef;
    }
    {
      SoftmaxTile unused;
      pv_tile(nsteps - 1, unused, false, std::false_type{});  // landed before the last barrier
    }
    mfma_drain_acc(o[15]);
#pragma unroll
    for (int d = 0; d < 15; ++d) acc_fence(o[d]);
    wait_vmcnt<0>();  // the stages past the chunk have landed too
    // all waves are past their last read of the ring; decide whether to recompute
    const bool over = rs.mu != -INFINITY && rs.m_true > rs.mu + kHeadroom;
    if (!__syncthreads_or(over)) break;
    // second pass: reference = the row's true max, so every exponent is <= 0
    rs.mu = rs.m_true;
  }

  // ---- merge the TL waves of each row block, normalise, write partial O and lse
  __syncthreads();  // the ring is free from here on
  float* st_m = (float*)lds;        // [4 waves][32]
  float* st_l = st_m + 4 * 32;
  float* st_f = st_l + 4 * 32;
  const float mu = rs.mu;
  const float l_row = rs.l_run + __shfl_xor(rs.l_run, 32);
  if (lane < 32) {
    st_m[wave * 32 + n] = mu;
    st_l[wave * 32 + n] = l_row;
  }
  __syncthreads();
  float Mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < TL; ++t) Mx = fmaxf(Mx, st_m[(rb * TL + t) * 32 + n]);
  float Ls = 0.f;
#pragma unroll
  for (int t = 0; t < TL; ++t) {
    const float mt = st_m[(rb * TL + t) * 32 + n];
    if (mt != -INFINITY) Ls += st_l[(rb * TL + t) * 32 + n] * exp2f(mt - Mx);
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
    // register r of block d is row wrow0 + tok_of(gg, r), column 32 d + n
    float* wout = out + (int64_t)wrow0 * kDv + n;
    if (wrow0 + 32 <= M) {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const f32x16 v = from_acc(o[d]);
#pragma unroll
        for (int r = 0; r < 16; ++r) wout[tok_of(gg, r) * kDv + 32 * d] = v[r] * fr[r];
      }
    } else {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const f32x16 v = from_acc(o[d]);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (wrow0 + tok_of(gg, r) < M) wout[tok_of(gg, r) * kDv + 32 * d] = v[r] * fr[r];
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
        const f32x16 v = from_acc(o[8 * half + dd]);
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
    case 64: decode_kernel<2><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    case 128: decode_kernel<4><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla

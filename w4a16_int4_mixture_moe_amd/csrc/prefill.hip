// Prefill-side W4A16 MoE GEMM tiles for gfx950: 128 routed rows x 256 weight
// rows per workgroup (four waves, two workgroups per CU), or 256 routed rows x
// 256 weight rows (eight waves, one workgroup per CU; an expert of up to 256
// rows then streams its weights once).  The description below is the
// 128-row tile's; the 256-row one gives each wave two weight tiles of all
// sixteen token tiles instead of four of eight, which leaves registers for a
// software-pipelined step (see pf_mainloop).
//
// Why a separate kernel.  Large routed blocks are MFMA-bound, and on gfx950
// what limits the MFMA rate in this GEMM is the LDS and register traffic per
// MFMA, not the MFMA unit.  Each wave here owns four 16-row weight tiles
// (64 weight rows) and all eight 16-row token tiles of the block, so every
// activation fragment read from LDS feeds four MFMAs, and the dequantised
// weights (VALU work, subtract-then-scale of the Chord post's "H200 and
// Blackwell indexed decode" section) are amortised over 128 rows.  The
// accumulators (4 x 8 MFMA tiles, 128 registers) stay in ordinary VGPRs and
// the whole wave fits 256 registers, so two workgroups (two waves per SIMD)
// share a CU.  (One eight-wave workgroup of 512 weight rows per CU, which
// stages each activation chunk once for twice the weight rows, measured 3-19 %
// slower: its eight waves meet at every chunk barrier together, where two
// independent workgroups cover each other's waits.)  That needs the
// activation staging to cost no registers: the
// block's rows are copied HBM -> LDS with global_load_lds_dwordx4 (16 bytes
// per lane, straight into LDS), one 128-wide K chunk ahead of the MFMAs,
// double buffered.
//
// LDS layout.  A staged chunk is 128 rows x 256 bytes (128 bf16 of K).  The
// LDS-DMA writes each instruction's 64 lanes to 1 KB of consecutive LDS (four
// rows), so rows cannot be padded; instead the sixteen 16-byte granules of
// row r are permuted, granule q at position q ^ swz(r) with
// swz(r) = (r % 4) ^ (12 if bit 2 of r is set).  The MFMA operand read of
// lane l (row 16 t + l % 16, granule 4 (l / 16) + j) is then free of bank
// conflicts.  Measured on MI355X with SQ_LDS_BANK_CONFLICT (a wave's
// ds_read_b128 takes 4 LDS cycles when linear): q ^ swz(r) 4 cycles;
// q ^ (r % 16), q ^ (r % 8), and 272-byte padded rows 8 cycles each.  gfx950
// serves the 64 lanes of a b128 read 16 at a time, and the lanes that share
// a cycle are not a run of 16 consecutive lanes (that model would make
// q ^ (r % 16) conflict-free); swz was chosen to be conflict-free under every
// lane grouping and 64-bank mapping consistent with a set of measured read
// patterns, and measured so.
//
// Arithmetic is that of moe_gemm_kernel: the same packed weights and scales,
// dequant8, v_mfma_f32_16x16x32_bf16 with the weights as the A operand, K
// chunks in order and the four 32-wide MFMA steps of a chunk in order, so the
// outputs are bit-identical to the general kernel's tile configurations
// (only the tile whose waves split K sums in another order).  K must be a
// multiple of 128 (the DMA copies whole chunks; other K use the general
// kernel).
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_common.hpp"

namespace w4a16 {

namespace {

// Tile shapes: MT token tiles per block (BM = 16 MT rows), NR weight tiles
// per wave, NW waves per workgroup; every wave covers all MT token tiles, so
// a wave holds NR x MT accumulator tiles (128 registers in both shapes) and
// two waves run per SIMD.
template <int MT_, int NR_, int NW_>
struct PfCfg {
  static constexpr int MT = MT_, NR = NR_, NW = NW_, BM = 16 * MT_;
  static constexpr int kPerCU = 8 / NW_;   // resident workgroups per CU
};
// 128 rows x 256 weight rows, two workgroups per CU
using PfNarrow = PfCfg<8, 4, 4>;
// 256 rows x 256 weight rows, one workgroup per CU: each dequantised weight
// fragment feeds 16 token tiles (half the dequantisation and weight traffic
// per MFMA of the narrow tile) and an expert of up to 256 rows reads its
// weights once; LDS holds two 64 KB chunks
using PfWide = PfCfg<16, 2, 8>;

template <int BM>
struct PfSmem {
  uint16_t xs[2][BM * kChunk];      // two staged chunks, granules permuted by row
  int row[BM];                      // activation row per block row, -1 = padding
  int out[BM];                      // output row per block row, -1 = not stored
  float w[BM];                      // top-k weight per block row (weighted epilogue)
  // byte offsets of the LDS-DMA source rows, in the order the DMA reads them:
  // entry 8 g + k is block row g + (BM / 8) k (see pf_mainloop)
  uint32_t xoff[BM];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(3))) char* lds_cptr_t;
typedef const __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst wave-uniform).  (Kept out of templates: the host pass
// rejects the builtin's pointer arguments inside one.)
__device__ __forceinline__ void dma16(gptr_t src, lds_ptr_t dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// acc += this wave's 16 NR weight rows x the block's first 16 NA rows over
// all K.  SHORT: K is at most two chunks.  resident (SHORT only): the block's
// activation rows are already in LDS from the previous N tile (two chunks
// fill both buffers); nothing is staged.
template <class C, int NA, bool SHORT>
__device__ __forceinline__ void pf_mainloop(const GemmParams& p, PfSmem<C::BM>& sm, int expert, int nt,
                                            f32x4_t (&acc)[C::NR][C::MT], bool resident) {
  constexpr int NR = C::NR, NW = C::NW;
  static_assert(NA >= 1 && NA <= C::MT && (4 * NA) % NW == 0, "active tile count");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int KC = p.KC;

  // LDS-DMA of a chunk: instruction i (of 4 NA) writes block rows 4 i .. 4 i + 3;
  // this wave issues i = wave + NW k, k < 4 NA / NW.  Lane l lands at row
  // 4 i + l / 16, position l % 16, so it loads granule (l % 16) ^ swz(row)
  // of that row, the same granule for every k (4 NW k leaves row % 16 alone).
  // The per-lane source offsets of rows g + 4 NW k (g = 4 wave + l / 16,
  // k < 8; 8 x 4 NW = BM rows) sit in LDS as 8 consecutive words per g, so a
  // lane fetches its offsets with two 16-byte reads and one wait (read one by
  // one, each DMA waited on its own LDS round trip).
  static_assert(8 * 4 * NW == C::BM, "eight DMA rows per lane cover the block");
  constexpr int KX = 4 * NA / NW;        // DMA instructions per wave per chunk (<= 8)
  if (!resident) {
    const int fallback_row = sm.row[0];   // always valid
    for (int i = tid; i < C::BM; i += NW * kWave) {
      const int r = sm.row[i];
      sm.xoff[(i % (4 * NW)) * 8 + i / (4 * NW)] = (uint32_t)(r >= 0 ? r : fallback_row) * (uint32_t)(p.K * 2);
    }
  }
  __syncthreads();
  // row % 16 = (4 wave + l / 16) % 16: swz = l / 16 ^ (12 if wave is odd)
  const uint32_t gran = (uint32_t)(((lane & 15) ^ (lane >> 4) ^ ((wave & 1) * 12)) * 16);
  const int xrow = 4 * wave + (lane >> 4);
  const gptr_t xbase = uniform_ptr(p.a);
  auto issue_x = [&](int c, int buf) {
    if (resident) return;
    const gptr_t base = xbase + (int64_t)c * (kChunk * 2) + gran;
    const u32x4_t* xq = reinterpret_cast<const u32x4_t*>(&sm.xoff[xrow * 8]);
    uint32_t xo[8];
    const u32x4_t lo = xq[0];
#pragma unroll
    for (int k = 0; k < 4; ++k) xo[k] = lo[k];
    if constexpr (KX > 4) {
      const u32x4_t hi = xq[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) xo[4 + k] = hi[k];
    }
#pragma unroll
    for (int k = 0; k < KX; ++k)
      dma16(base + xo[k], (lds_ptr_t)(reinterpret_cast<char*>(&sm.xs[buf][0]) + (wave + NW * k) * 1024));
  };

  // weights and scales: a ring of two chunks per wave, as in moe_gemm_kernel
  const int rt_base = nt * (NW * NR) + wave * NR;
  gptr_t wbase[NR];
  gptr_t sbase[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rt = min(rt_base + r, p.NT - 1);
    const int64_t tile = (int64_t)expert * p.w_tiles + rt;
    wbase[r] = uniform_ptr(p.packed_w + tile * p.KC * kWave);
    sbase[r] = uniform_ptr(p.packed_s + tile * ((p.KC + 1) / 2) * kWave);
  }
  const uint32_t woff = (uint32_t)lane * 16u;
  const uint32_t soff = (uint32_t)lane * 4u;
  auto issue_w = [&](int c, u32x4_t (&w)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = gload_u32x4(wbase[r] + (int64_t)c * (kWave * 16) + woff);
  };
  // the scale words of a chunk pair (low half: even chunk, high half: odd)
  auto issue_s = [&](int c, uint32_t (&sc)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) sc[r] = gload_u32(sbase[r] + (int64_t)(c >> 1) * (kWave * 4) + soff);
  };

  const DequantMasks masks = make_dequant_masks();
  // weights and scales of the current chunk and of the next one (a ring of
  // two register sets: the second wave on each SIMD covers the rest of the
  // load latency)
  u32x4_t wr[2][NR];
  uint32_t sr[2][NR];               // scale words of the current and the next chunk pair

  // prologue: chunk 0 to LDS, weights and scales of chunk 0 in flight
  issue_x(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_w(0, wr[0]);
  issue_s(0, sr[0]);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<2 * NR>();             // this wave's DMA of chunk 0 has landed
  __syncthreads();                  // ... and every wave's

  // one chunk at ring position P: DMA of chunk c + 1 into the other LDS
  // buffer and the weights of chunk c + 1 into the other register set, then
  // dequant + MFMAs of chunk c, then wait for the DMA and synchronise.
  // has_next: chunk c + 1 exists.
  //
  // P = c % 2 and Q = (c / 2) % 2 are compile-time constants, so every ring
  // index below is static (a run-time index puts the ring in scratch memory).
  // P: the LDS buffer and weight register set of chunk c, and which half of
  // the pair's scale word holds its scales (low for P = 0); Q: the scale
  // register set of the chunk pair.
  auto chunk = [&](auto P_, auto Q_, int c, bool has_next) {
    constexpr int P = decltype(P_)::value;
    constexpr int Q = decltype(Q_)::value;
    if (has_next) {
      issue_x(c + 1, P ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(c + 1, wr[P ^ 1]);
      if (P == 1) issue_s(c + 1, sr[Q ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const char* xs = reinterpret_cast<const char*>(&sm.xs[P][0]);
    const uint32_t rowoff = (uint32_t)(lane & 15) * 256u;
    // this wave's weight fragments of 32-K step j, dequantised
    auto dequant_step = [&](int j, bf16x8_t (&A)[NR]) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t word = sr[Q][r];
        const float sv = __builtin_bit_cast(float, P ? (word & 0xFFFF0000u) : (word << 16));
        A[r] = dequant8(wr[P][r][j], sv, -1032.0f * sv, 0.0625f * sv, -72.0f * sv, masks);
      }
    };
    // the activation fragment of token tile t at step j
    auto goff = [&](int j) {
      return (uint32_t)((((lane >> 4) * 4 + j) ^ (lane & 3) ^ (((lane >> 2) & 1) * 12)) * 16);
    };
    auto operand = [&](int j, int t) {
      return *reinterpret_cast<const bf16x8_t*>(xs + t * 4096 + rowoff + goff(j));
    };
    if constexpr (NR == 2) {
      // two weight tiles per wave leave registers for a pipeline: the
      // fragments of the next two token tiles are read while the MFMAs of
      // the current two run, and the next step's weights are dequantised
      // under the current step's MFMAs (the order of every accumulator's
      // MFMAs is unchanged).  Measured on MI355X against reading each pair
      // and waiting for it: gate/up EP8 prefill 540 -> 518 us, EP32 145 ->
      // 135 us.  (Loading the weights two chunks ahead gained 1 % more: it
      // needs a barrier without __syncthreads' wait for every load, and the
      // compiler then waits for all loads wherever a register load is used
      // after an LDS-DMA was issued, so it was not kept.)
      // LDS byte address of this lane's row of step j in chunk c's buffer,
      // opaque to the optimiser: the token tiles' offsets (t x 4 KB) then stay
      // in the reads' immediate field (a folded 64 KB buffer offset would
      // overflow it and cost an address register per tile and step)
      uint32_t xb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xb[j] = (uint32_t)(uintptr_t)(lds_cptr_t)xs + rowoff + goff(j);
        __asm__ volatile("" : "+v"(xb[j]));
      }
      auto operand2 = [&](int j, int t) {
        return *reinterpret_cast<const lds_bf16x8_t*>((lds_cptr_t)(uintptr_t)xb[j] + t * 4096);
      };
      bf16x8_t A[NR], An[NR];
      dequant_step(0, A);
      bf16x8_t B0 = operand2(0, 0), B1 = operand2(0, 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int tp = 0; tp < NA / 2; ++tp) {
          bf16x8_t N0 = B0, N1 = B1;
          if (tp + 1 < NA / 2) {
            N0 = operand2(j, 2 * tp + 2);
            N1 = operand2(j, 2 * tp + 3);
          } else if (j < 3) {
            N0 = operand2(j + 1, 0);
            N1 = operand2(j + 1, 1);
          }
          // weight tile r of the next step under pair min(r, NA / 2 - 1): one
          // per pair, the rest under the last pair when there are fewer pairs
          // than tiles
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (j < 3 && tp == (r < NA / 2 ? r : NA / 2 - 1)) {
              const uint32_t word = sr[Q][r];
              const float sv = __builtin_bit_cast(float, P ? (word & 0xFFFF0000u) : (word << 16));
              An[r] = dequant8(wr[P][r][j + 1], sv, -1032.0f * sv, 0.0625f * sv, -72.0f * sv, masks);
            }
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            acc[r][2 * tp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B0, acc[r][2 * tp], 0, 0, 0);
            acc[r][2 * tp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B1, acc[r][2 * tp + 1], 0, 0, 0);
          }
          B0 = N0;
          B1 = N1;
          // one pair per scheduling region (a wider one lets the scheduler
          // hoist later pairs' reads and dequant work, which spills)
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j < 3)
#pragma unroll
          for (int r = 0; r < NR; ++r) A[r] = An[r];
      }
    } else {
      // four weight tiles per wave: registers for one activation fragment
      // read ahead (the next token tile's, under the current one's four
      // MFMAs), not for the next step's dequant.  Measured against reading
      // each fragment where it is used: TP8 T = 4096 gate/up 320 -> 306 us,
      // grouped contiguous / masked 880 / 962 -> 858 / 940 us; the N-tile-loop
      // form (SHORT) spills with it and stays as it was (its down + combine
      // 486 against 501 us)
      if constexpr (!SHORT) {
        bf16x8_t B = operand(0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8_t A[NR];
          dequant_step(j, A);
#pragma unroll
          for (int t = 0; t < NA; ++t) {
            bf16x8_t Bn = B;
            if (t + 1 < NA)
              Bn = operand(j, t + 1);
            else if (j < 3)
              Bn = operand(j + 1, 0);
#pragma unroll
            for (int r = 0; r < NR; ++r)
              acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B, acc[r][t], 0, 0, 0);
            B = Bn;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8_t A[NR];
          dequant_step(j, A);
#pragma unroll
          for (int t = 0; t < NA; ++t) {
            const bf16x8_t B = operand(j, t);
#pragma unroll
            for (int r = 0; r < NR; ++r)
              acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B, acc[r][t], 0, 0, 0);
          }
          // keep each 32-K step's operands to itself (more registers than
          // two waves per SIMD leave otherwise)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (has_next) {
      // the DMA of chunk c + 1 was issued before its weights (and, after an
      // odd chunk, the next pair's scales)
      if (P == 1)
        wait_vmcnt<2 * NR>();
      else
        wait_vmcnt<NR>();
    }
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (SHORT) {
    chunk(I0{}, I0{}, 0, KC > 1);
    if (KC > 1) chunk(I1{}, I0{}, 1, false);
  } else {
    int c = 0;
    for (; c + 4 < KC; c += 4) {
      chunk(I0{}, I0{}, c, true);
      chunk(I1{}, I0{}, c + 1, true);
      chunk(I0{}, I1{}, c + 2, true);
      chunk(I1{}, I1{}, c + 3, true);
    }
    // the last one to four chunks (c is a multiple of four here)
    if (c < KC) chunk(I0{}, I0{}, c, c + 1 < KC);
    if (c + 1 < KC) chunk(I1{}, I0{}, c + 1, c + 2 < KC);
    if (c + 2 < KC) chunk(I0{}, I1{}, c + 2, c + 3 < KC);
    if (c + 3 < KC) chunk(I1{}, I1{}, c + 3, false);
  }
}

// go(integral_constant<2 k>) for the smallest even 2 k >= na, 2 <= 2 k <= MT.
template <int MT, int K2 = 2, class F>
__device__ __forceinline__ void dispatch_even(int na, F&& go) {
  if constexpr (K2 >= MT) {
    go(std::integral_constant<int, MT>{});
  } else {
    if (na <= K2)
      go(std::integral_constant<int, K2>{});
    else
      dispatch_even<MT, K2 + 2>(na, go);
  }
}

// The block's tiles: the main loop specialised for its active token tiles
// (a prefix, rounded up to an even count: at most one tile of padding rows
// multiplied), then the epilogue.
// N tiles nt0 .. nt1 - 1 of the block, one after another.  LOOP (a kernel
// of its own, so the registers of the one-tile kernels are unaffected): more
// than one tile, K fits the two LDS buffers and the later tiles reuse the
// staged rows.
template <class C, int EPI, bool LOOP>
__device__ __forceinline__ void pf_run(const GemmParams& p, PfSmem<C::BM>& sm, int expert, int nt0, int nt1,
                                       uint32_t tmask) {
  const int na = 32 - __clz(tmask);
  auto go = [&](auto NA_) {
    constexpr int NA = decltype(NA_)::value;
    auto tile = [&](int nt, bool resident) {
      f32x4_t acc[C::NR][C::MT];
#pragma unroll
      for (int r = 0; r < C::NR; ++r)
#pragma unroll
        for (int t = 0; t < C::MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pf_mainloop<C, NA, LOOP>(p, sm, expert, nt, acc, resident);
      epilogue<C::MT, C::NR, C::NW, EPI>(p, sm, nt, (1u << NA) - 1u, acc);
    };
    if constexpr (LOOP) {
      for (int nt = nt0; nt < nt1; ++nt) tile(nt, nt != nt0);
    } else {
      tile(nt0, false);
    }
  };
  // active tiles rounded up to an even count (the DMA splits the rows of
  // 4 NA / NW instructions per wave); in the 256-row tile, rounding to a
  // multiple of four instead issued 14 % more MFMAs than the valid rows need
  // and measured 5-6 % slower (EP8 / EP16 prefill gate/up 522 / 341 against
  // 495 / 319 us)
  dispatch_even<C::MT>(na, go);
}

// One workgroup per (routed block, group of n_loop consecutive N tiles);
// n_loop > 1 only when K fits the two LDS buffers.
// (Template arguments are the tile's sizes rather than its PfCfg so that the
// kernel's name in a trace reads like the general kernel's.)
template <int MT, int NR, int NW, int ROUTE, int EPI, bool LOOP>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void moe_gemm_prefill_kernel(const GemmParams p, int n_loop) {
  using C = PfCfg<MT, NR, NW>;
  __shared__ __attribute__((aligned(16))) PfSmem<C::BM> sm;
  // work item (routed block, N-tile group), block-major (consecutive
  // workgroups, the N tiles of one block, go to different XCDs) unless the
  // block has few groups (block_of).  Measured against orders that keep a
  // block's sixteen N tiles on one XCD (its activation rows then come from
  // HBM once): all sixteen side by side there, 4.8x slower (one L2 serving
  // the same lines to sixteen CUs at once); spread over time (N-tile-major),
  // 1-8 % slower.
  const int groups = (p.n_tiles + n_loop - 1) / n_loop;
  int mb, g;
  if (!block_of(p, blockIdx.x, groups, mb, g)) return;
  const int nt0 = g * n_loop;
  const int expert = setup_rows<C::MT, C::NW, ROUTE, EPI>(p, mb, sm);
  if (expert < 0) return;
  __syncthreads();
  pf_run<C, EPI, LOOP>(p, sm, expert, nt0, min(nt0 + n_loop, p.n_tiles), active_tiles<C::MT>(sm));
}

typedef void (*PfKernel)(const GemmParams, int);

template <class C, bool LOOP>
PfKernel pick_prefill_of(int route, int epi) {
  if (route == kRouteIndexed) {
    if (epi == kEpiStore) return moe_gemm_prefill_kernel<C::MT, C::NR, C::NW, kRouteIndexed, kEpiStore, LOOP>;
    if (epi == kEpiWeighted) return moe_gemm_prefill_kernel<C::MT, C::NR, C::NW, kRouteIndexed, kEpiWeighted, LOOP>;
    if (epi == kEpiSilu) return moe_gemm_prefill_kernel<C::MT, C::NR, C::NW, kRouteIndexed, kEpiSilu, LOOP>;
    return nullptr;
  }
  if (epi != kEpiStore) return nullptr;
  if (route == kRouteContiguous) return moe_gemm_prefill_kernel<C::MT, C::NR, C::NW, kRouteContiguous, kEpiStore, LOOP>;
  if (route == kRouteMasked) return moe_gemm_prefill_kernel<C::MT, C::NR, C::NW, kRouteMasked, kEpiStore, LOOP>;
  return nullptr;
}

// The prefill tile of a configuration (m_tiles, nr, waves), or nullptr; the
// N-tile loop exists for the narrow tile only.
PfKernel pick_prefill(int m_tiles, int nr, int waves, int route, int epi, bool loop) {
  if (m_tiles == PfNarrow::MT && nr == PfNarrow::NR && waves == PfNarrow::NW)
    return loop ? pick_prefill_of<PfNarrow, true>(route, epi) : pick_prefill_of<PfNarrow, false>(route, epi);
  if (m_tiles == PfWide::MT && nr == PfWide::NR && waves == PfWide::NW && !loop)
    return pick_prefill_of<PfWide, false>(route, epi);
  return nullptr;
}

}  // namespace

bool prefill_applies(int route, int epilogue, int m_tiles, int nr, int waves, int stages, const GemmParams& p) {
  return stages == 2 && p.K % kChunk == 0 && p.split <= 1 &&
         pick_prefill(m_tiles, nr, waves, route, epilogue, false) != nullptr;
}

// N tiles per workgroup.  With K of at most two chunks (K <= 256, the down
// projection of a TP8 share) a block's 128 activation rows (64 KB at K = 256)
// outweigh an N tile's weights (36 KB with scales), and every N tile's
// workgroup fetches them again; a workgroup that keeps them in LDS and runs
// several N tiles fetches them once.  As many tiles per workgroup as keep the
// grid at kPfLoopMinWorkgroups or more (the routed-block bound counts every
// block).  Measured on MI355X, TP8 T = 4096 down + combine in four passes of
// seven N tiles: one tile per workgroup 541 us; 2, 3, 7 tiles 513, 501,
// 515 us; 4 tiles (two workgroups per block) 684 us.
constexpr int64_t kPfLoopMinWorkgroups = 1536;

int prefill_n_loop(const GemmParams& p, int m_tiles) {
  if (p.KC > 2 || m_tiles != PfNarrow::MT) return 1;
  int best = 1;
  for (int l = 2; l <= p.n_tiles; ++l)
    if ((int64_t)p.grid_blocks * ((p.n_tiles + l - 1) / l) >= kPfLoopMinWorkgroups) best = l;
  return best;
}

hipError_t launch_gemm_prefill(int route, int epilogue, int m_tiles, int nr, int waves, const GemmParams& p,
                               hipStream_t stream) {
  const int n_loop = prefill_n_loop(p, m_tiles);
  const PfKernel k = pick_prefill(m_tiles, nr, waves, route, epilogue, n_loop > 1);
  if (k == nullptr || p.K % kChunk) return hipErrorInvalidValue;
  const int groups = (p.n_tiles + n_loop - 1) / n_loop;
  GemmParams q = p;
  q.xcd_group = xcd_group_for(1, groups);
  const int64_t grid = grid_of(q, groups);
  if (grid <= 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(waves * kWave), 0, stream, q, n_loop);
  return hipGetLastError();
}

}  // namespace w4a16

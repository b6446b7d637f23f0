// W4A16 MoE expert GEMM for gfx950: BF16 activations x INT4 weights with
// BF16 group-32 scales, FP32 accumulation in v_mfma_f32_16x16x32_bf16.
//
// Operand orientation.  The dequantised weights are the MFMA "A" operand
// (16 weight rows x 32 K) and the routed activation rows are the "B" operand
// (32 K x 16 token rows), so the wide operand is always filled with weight
// rows however few tokens an expert received.  This is the gfx950 form of the
// operand swap the Chord W4A16 MoE post uses for decode (section "H200 and
// Blackwell indexed decode": dequantised weights in the MMA M operand); here
// it is the only orientation, and large token counts simply loop over more
// 16-row token tiles per weight fragment, so every weight element is
// dequantised once per workgroup however many rows share it.
//
// Tile: one routed block of BM = 16 * MT rows (one expert) times BN = NW * NR
// * 16 weight rows; each wave owns NR 16-row weight tiles and every token
// tile of the block.  Per 128-wide K chunk:
//   - activations: BM rows x 256 B staged global -> registers -> LDS
//     (double buffered, rows padded to 272 B; on gfx950 the operand reads
//     of this layout are 2-way bank-conflicted, 8 LDS cycles per wave read
//     against 4 for a conflict-free one, measured with
//     SQ_LDS_BANK_CONFLICT; the kernels this template serves are bound by
//     their weight stream, and the prefill tile, where the reads matter
//     more, uses a conflict-free permutation of unpadded rows);
//   - weights: one 16-byte load per lane per weight tile straight from HBM
//     into registers (the packed layout is the operand layout) plus the
//     lane's one bf16 scale, both requested two or three chunks ahead;
//   - dequant (dequant8) -> 4 MFMAs per (weight tile, active token tile).
// Token tiles without a valid row are skipped (wave-uniform).  Summation
// order per output: chunks in K order, and inside a chunk the hardware's
// order over its 32 K; with one workgroup per tile this is independent of
// BM, NR, NW, so the output bits do not depend on the tile configuration.
//
// Two schedules (the post gates stream-K by shape, section "H200 prefill and
// TP8"; its decode section reports a semi-static tile schedule beating a
// fully dynamic one):
//   classic   one workgroup per (routed block, N tile);
//   stream-K  as many workgroups as the device keeps resident, each taking
//             an equal contiguous range of (tile, chunk pair) units, so a grid of
//             1.5 "waves" of tiles no longer idles half the machine at the
//             end; a tile cut by a range boundary leaves fp32 partials
//             (one slot per contributor) that streamk_fixup_kernel sums in
//             range order -- deterministic for a given device and config.
//
// Row sources (the post's two families, sections "Two kernel families" and
// "Grouped SM90 kernels"):
//   indexed     block b -> expert_ids[b]; row i -> sorted_ids[b*BM + i],
//               a sentinel (>= T*k) marks padding; activation row =
//               slot / a_row_div; output row = slot.
//   contiguous  block b covers rows b*BM.. of A; expert = m_indices of its
//               first row (-1: whole block is padding); rows whose m_index
//               differs are skipped.
//   masked      block b -> (group g, rows r0..r0+BM) of A[g]; rows at or past
//               masked_m[g] skipped; output row g*max_m + r.
// Epilogues: bf16 store (round to nearest even) or, for the top-k combine,
// fp32 partial = topk_weight(slot) * acc stored per slot (staged through LDS
// so whole rows are written at once, when the tile is at most 128 columns);
// launch_combine then sums a token's local slots in j order and rounds once.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_common.hpp"

namespace w4a16 {

template <int MT>
struct TileSmem {
  uint16_t xs[2][16 * MT][kChunk + 8];  // staged activation chunk, 272-byte rows
  int row[16 * MT];                     // activation row per block row, -1 = padding
  int out[16 * MT];                     // output row per block row, -1 = not stored
  float w[16 * MT];                     // top-k weight per block row (weighted epilogue)
  int last;                             // split-K: this workgroup reduces the tile
};

#ifndef W4A16_PIPELINED_DEQUANT
#define W4A16_PIPELINED_DEQUANT 1
#endif
constexpr bool kPipelinedDequant = W4A16_PIPELINED_DEQUANT != 0;

// acc += this wave's weight tiles x the block's rows over K chunks [c0, c1).
// Starts and ends with the workgroup synchronised.  The active token tiles
// are always a prefix (valid rows come first in every layout); the loop
// processes exactly tiles [0, NA), NA fixed at compile time, so it loads,
// reads and multiplies only those, without per-tile branches.
template <int MT, int NR, int NW, int D, int NA>
__device__ __forceinline__ void mainloop(const GemmParams& p, TileSmem<MT>& sm, int expert, int nt,
                                         int c0, int c1, f32x4_t (&acc)[NR][MT]) {
  constexpr int NTHR = NW * kWave;
  constexpr int ROWS_PER_PASS = NTHR / 16;          // staged rows covered by one piece index
  static_assert(ROWS_PER_PASS == 16 || ROWS_PER_PASS == 32, "four or eight waves");
  constexpr int PPT = (16 * MT + ROWS_PER_PASS - 1) / ROWS_PER_PASS;   // pieces per thread
  static_assert(NA >= 1 && NA <= MT, "active tile count");
  auto active = [&](int t) { return t < NA; };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // Activation staging.  Piece i of this thread is row (tid / 16) +
  // i * ROWS_PER_PASS, 16 bytes at column 8 * (tid % 16); its token tile is
  // wave-uniform (a wave covers 4 consecutive rows), so pieces of inactive
  // tiles, or past the block (eight waves, one tile), are skipped with a
  // scalar branch.  Padding rows read the block's first row (always valid)
  // instead; their LDS columns only feed output columns never stored.
  // Addressing: every stream is (wave-uniform base in SGPRs) + (per-lane
  // 32-bit byte offset fixed for the whole loop) + (uniform chunk offset), so
  // the per-chunk address update is scalar and loads use the saddr form.
  const int fallback_row = sm.row[0];
  const int xcol = (tid & 15) * 8;
  const gptr_t xbase = uniform_ptr(p.a);
  auto piece_row = [&](int i) { return (tid >> 4) + i * ROWS_PER_PASS; };
  // wave-uniform: the tile of piece i, and whether the piece is loaded
  auto piece_tile = [&](int i) { return ROWS_PER_PASS == 16 ? i : 2 * i + (wave >> 2); };
  auto piece_on = [&](int i) { return piece_tile(i) < NA; };
  uint32_t xoff[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int r = sm.row[min(piece_row(i), 16 * MT - 1)];
    xoff[i] = (uint32_t)((r >= 0 ? r : fallback_row) * p.K + xcol) * 2u;
  }

  // this wave's weight tiles (clamped so loads stay in bounds; tiles past N
  // compute throw-away values that are never stored)
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
  const uint32_t woff = (uint32_t)lane * 16u;   // one 16-byte fragment set per lane
  const uint32_t soff = (uint32_t)lane * 4u;    // one pair of bf16 scales per lane

  const int K = p.K;
  // `tail`: chunk c may be the ragged last one; a piece past K then reads
  // column 0 of its row (in bounds) and store_x replaces it by zeros.  No
  // select on the loaded value, so its destination is never rewritten
  // before it lands.
  auto issue_x = [&](int c, u32x4_t (&xr)[PPT], bool tail) {
    const gptr_t base = xbase + (int64_t)c * (kChunk * 2);
    const bool kin = !tail || c * kChunk + xcol < K;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (piece_on(i)) xr[i] = gload_u32x4(kin ? base + xoff[i] : xbase + xoff[i]);
  };
  auto store_x = [&](int buf, int c, const u32x4_t (&xr)[PPT], bool tail) {
    const bool kin = !tail || c * kChunk + xcol < K;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (piece_on(i)) {
        const u32x4_t v = kin ? xr[i] : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(&sm.xs[buf][piece_row(i)][xcol]) = v;
      }
  };
  // weights of chunk c and, for an even chunk (withs), the scale word of
  // its chunk pair, which the odd chunk after it reuses: a range starts on
  // an even chunk (split-K slices and stream-K units are whole chunk
  // pairs), so even ring positions hold even chunks
  auto issue_w = [&](int c, u32x4_t (&w)[NR], uint32_t (&sc)[NR], auto withs) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      w[r] = gload_u32x4(wbase[r] + (int64_t)c * (kWave * 16) + woff);
      if constexpr (decltype(withs)::value) sc[r] = gload_u32(sbase[r] + (int64_t)(c >> 1) * (kWave * 4) + soff);
    }
  };
  using WithS = std::integral_constant<bool, true>;
  using NoS = std::integral_constant<bool, false>;

  // Weights and scales: a ring of D register sets (the config's prefetch
  // stages); chunk c0 + m*D + P uses set P, and the set is refilled with
  // chunk c + D as soon as chunk c has been dequantised, so weights have
  // about D chunk times to arrive from HBM.  Activations come from L2
  // (every N tile of a block reads the same rows): one register set,
  // requested at the top of a chunk and written to the other LDS buffer at
  // its end, before the barrier.  (A second set, for two chunks of
  // distance, measured no faster and costs registers.)
  static_assert(D == 2 || D == 4, "the loop body below unrolls two or four chunks");
  const DequantMasks masks = make_dequant_masks();
  // 128-bit vector registers (not the 4-field struct): each loop-carried
  // value stays one register tuple that the allocator can keep in place
  u32x4_t xr[PPT];
  u32x4_t wr[D][NR];
  uint32_t sr[D][NR];   // scale words: even ring positions only
  uint32_t spair[NR];   // the current pair's word, kept for its odd chunk

  // c0 < c1 (both callers).  Unconditional, clamped (a set past the range
  // re-reads the last chunk and is never used) and in ring order: the waits
  // inside the loop are computed for the worst entry path, so a conditional
  // or reordered load here would make every chunk wait for the newest loads.
  issue_x(c0, xr, true);
#pragma unroll
  for (int i = 0; i < D; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i % 2 == 0)
      issue_w(min(c0 + i, c1 - 1), wr[i], sr[i], WithS{});
    else
      issue_w(min(c0 + i, c1 - 1), wr[i], sr[i], NoS{});
  }
  __builtin_amdgcn_sched_barrier(0);
  store_x(0, c0, xr, true);
  __syncthreads();

  // one chunk at ring position P (c - c0 = P mod D).  STEADY: chunks c + 1
  // and c + D exist and c + 1 is not the ragged last chunk, so every
  // prefetch and store is unconditional (no register phis, no selects)
  // Scale constants of chunk c for a weight set: s, -1032 s, s / 16, -72 s
  // (the word holds the scales of chunks c & ~1 (low half) and c | 1 (high))
  auto scale_consts = [&](const uint32_t (&sc)[NR], int c, float (&k)[NR][4]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float sv = __builtin_bit_cast(float, (c & 1) ? (sc[r] & 0xFFFF0000u) : (sc[r] << 16));
      k[r][0] = sv;
      k[r][1] = -1032.0f * sv;
      k[r][2] = 0.0625f * sv;
      k[r][3] = -72.0f * sv;
    }
  };
  auto dequant_set = [&](const u32x4_t (&w)[NR], int j, const float (&k)[NR][4], bf16x8_t (&A)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) A[r] = dequant8(w[r][j], k[r][0], k[r][1], k[r][2], k[r][3], masks);
  };
  auto mfmas = [&](int buf, int j, const bf16x8_t (&A)[NR]) {
    bf16x8_t B[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (active(t))
        B[t] = *reinterpret_cast<const bf16x8_t*>(&sm.xs[buf][16 * t + (lane & 15)][32 * (lane >> 4) + 8 * j]);
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (active(t))
#pragma unroll
        for (int r = 0; r < NR; ++r)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B[t], acc[r][t], 0, 0, 0);
  };
  // refill weight set P with chunk c + D once its last word is dequantised
  // (A holds that word's operands).  The empty asm and the scheduling
  // barrier keep the loads below that dequant: moved above it, old and new
  // values overlap, the new ones land in other registers and the loop
  // back-edge copies them over, which waits for the loads just issued and
  // serialises the prefetch.  The second barrier keeps them above the
  // chunk's activation store, whose wait (for the newest activation load)
  // would otherwise cover them too.
  auto refill = [&](auto P_, int c, const bf16x8_t (&A)[NR]) {
    constexpr int P = decltype(P_)::value;
#pragma unroll
    for (int r = 0; r < NR; ++r) asm volatile("" ::"v"(A[r]));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (P % 2 == 0)
      issue_w(c + D, wr[P], sr[P], WithS{});
    else
      issue_w(c + D, wr[P], sr[P], NoS{});
    __builtin_amdgcn_sched_barrier(0);
  };
  // an even chunk hands its pair's scale word to the odd chunk after it,
  // before its refill overwrites the word (a copy of a value that arrived
  // long ago: it waits for nothing)
  auto keep_pair = [&](auto P_) {
    constexpr int P = decltype(P_)::value;
    if constexpr (P % 2 == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) spair[r] = sr[P][r];
    }
  };
  // the scale word of the chunk at ring position P
  auto word_of = [&](auto P_) -> const uint32_t(&)[NR] {
    constexpr int P = decltype(P_)::value;
    if constexpr (P % 2 == 0)
      return sr[P];
    else
      return spair;
  };

  // Pipelined form: fragment j + 1 is dequantised
  // before fragment j's MFMAs are issued, so the VALU work of one overlaps
  // the matrix work of the other inside a wave; the last fragment of a chunk
  // dequantises the first one of the next chunk (its weights are already
  // resident).  Acur / kcur carry that across chunks.
  constexpr bool PIPE = kPipelinedDequant;
  bf16x8_t Acur[NR];
  float kcur[NR][4];
  if constexpr (PIPE) {
    scale_consts(sr[0], c0, kcur);
    dequant_set(wr[0], 0, kcur, Acur);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) spair[r] = 0u;

  // one chunk at ring position P (c - c0 = P mod D).  STEADY: chunks c + 1
  // and c + D exist and c + 1 is not the ragged last chunk, so every
  // prefetch and store is unconditional (no register phis, no selects)
  auto chunk = [&](auto P_, auto STEADY_, int c) {
    constexpr int P = decltype(P_)::value;
    constexpr bool STEADY = decltype(STEADY_)::value;
    const int buf = (c - c0) & 1;                   // LDS buffer holding chunk c
    if (STEADY || c + 1 < c1) issue_x(c + 1, xr, !STEADY);
    if constexpr (PIPE) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t Anext[NR];
        if (j < 3) {
          dequant_set(wr[P], j + 1, kcur, Anext);
          if (j == 2) keep_pair(P_);
          if (j == 2 && (STEADY || c + D < c1)) refill(P_, c, Anext);
        } else if (STEADY || c + 1 < c1) {
          using PN = std::integral_constant<int, (P + 1) % D>;
          scale_consts(word_of(PN{}), c + 1, kcur);
          dequant_set(wr[PN::value], 0, kcur, Anext);
        }
        mfmas(buf, j, Acur);
#pragma unroll
        for (int r = 0; r < NR; ++r) Acur[r] = Anext[r];
      }
    } else {
      float k[NR][4];
      scale_consts(word_of(P_), c, k);
      keep_pair(P_);
      // one 8-wide K fragment at a time: dequantise it, read the matching
      // activation fragments, issue its MFMAs
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t A[NR];
        dequant_set(wr[P], j, k, A);
        if (j == 3 && (STEADY || c + D < c1)) refill(P_, c, A);
        mfmas(buf, j, A);
      }
    }
    if (STEADY || c + 1 < c1) store_x(buf ^ 1, c + 1, xr, !STEADY);
    __syncthreads();
  };
  using Steady = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2 % D>;
  using I3 = std::integral_constant<int, 3 % D>;
  int c = c0;
  for (; c + 2 * D - 1 < c1; c += D) {
    chunk(I0{}, Steady{}, c);
    chunk(I1{}, Steady{}, c + 1);
    if constexpr (D > 2) {
      chunk(I2{}, Steady{}, c + 2);
      chunk(I3{}, Steady{}, c + 3);
    }
  }
  // the last up to 2D - 1 chunks (c - c0 is a multiple of D here)
  for (int m = 0; m < 2; ++m, c += D) {
    if (c < c1) chunk(I0{}, Tail{}, c);
    if (c + 1 < c1) chunk(I1{}, Tail{}, c + 1);
    if constexpr (D > 2) {
      if (c + 2 < c1) chunk(I2{}, Tail{}, c + 2);
      if (c + 3 < c1) chunk(I3{}, Tail{}, c + 3);
    }
  }
}

// One tile's K range [c0, c1): zeroed accumulators, the main loop
// specialised for the block's active token tiles (a workgroup-uniform
// prefix), then finish(acc, mask).  One- and two-tile blocks run exactly
// their active tiles; four- and eight-tile blocks round the count up to an
// even one, so the extra tile (rows that are all padding: they read the
// block's first row and are never stored) costs at most one tile of MFMAs,
// where testing tiles inside the loop made it wait for every outstanding
// load at each test.  Each path owns its
// accumulators and finishes on its own: merging them into one array before
// a shared epilogue makes the allocator rotate them between registers with
// moves inside the loop, each of which waits for an MFMA.
template <int MT, int NR, int NW, int D, typename Finish>
__device__ __forceinline__ void run_tile(const GemmParams& p, TileSmem<MT>& sm, int expert, int nt,
                                         uint32_t tmask, int c0, int c1, Finish&& finish) {
  auto go = [&](auto na) {
    constexpr int NA = decltype(na)::value;
    f32x4_t acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mainloop<MT, NR, NW, D, NA>(p, sm, expert, nt, c0, c1, acc);
    finish(acc, (1u << NA) - 1u);
  };
  if constexpr (MT == 1) {
    go(std::integral_constant<int, 1>{});
  } else if constexpr (MT == 2) {
    if (tmask == 1u)
      go(std::integral_constant<int, 1>{});
    else
      go(std::integral_constant<int, 2>{});
  } else if constexpr (MT == 4) {
    if (tmask < 4u)
      go(std::integral_constant<int, 2>{});
    else
      go(std::integral_constant<int, 4>{});
  } else {
    static_assert(MT == 8 || MT == 16, "token tiles per block: 1, 2, 4, 8 or 16");
    constexpr int Q = MT / 4;                        // active tiles rounded up to a multiple of Q
    const int na = 32 - __clz(tmask);               // tmask is a prefix
    if (na <= Q)
      go(std::integral_constant<int, Q>{});
    else if (na <= 2 * Q)
      go(std::integral_constant<int, 2 * Q>{});
    else if (na <= 3 * Q)
      go(std::integral_constant<int, 3 * Q>{});
    else
      go(std::integral_constant<int, 4 * Q>{});
  }
}

// Stream-K partial slots: slot s holds NR * MT float4 per thread, laid out
// [(r * MT + t)][thread] so each (r, t) is one coalesced 16 * NTHR-byte store.
template <int MT, int NR, int NW>
__device__ __forceinline__ float4* partial_slot(const GemmParams& p, int64_t slot) {
  constexpr int NTHR = NW * kWave;
  return reinterpret_cast<float4*>(p.sk_partial) + slot * (int64_t)(NR * MT * NTHR);
}

// Weighted epilogue through LDS: the tile's fp32 partials (times the slot's
// top-k weight) are first placed in the idle activation buffers, rows padded
// by 16 bytes, then written row by row, each wave storing two 512-byte row
// runs per instruction instead of sixteen 64-byte pieces.
template <int MT, int NR, int NW>
__device__ __forceinline__ void epilogue_weighted_staged(const GemmParams& p, TileSmem<MT>& sm, int nt,
                                                         uint32_t tmask, const f32x4_t (&acc)[NR][MT]) {
  constexpr int BN = 16 * NR * NW;
  constexpr int LD = BN + 4;
  static_assert(16 * MT * LD * 4 <= (int)sizeof(sm.xs), "staged tile fits the activation buffers");
  constexpr int NTHR = NW * kWave;
  float* tile = reinterpret_cast<float*>(&sm.xs[0][0][0]);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  __syncthreads();                                   // every wave is done reading the buffers
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (!((tmask >> t) & 1u)) continue;
      const int i = 16 * t + (lane & 15);
      const float w = sm.w[i];
      const f32x4_t v = acc[r][t];
      *reinterpret_cast<float4*>(tile + i * LD + (wave * NR + r) * 16 + 4 * (lane >> 4)) =
          make_float4(w * v[0], w * v[1], w * v[2], w * v[3]);
    }
  __syncthreads();
  const int n0 = nt * BN;
  const int rows = 16 * (32 - __clz(tmask));
  for (int idx = threadIdx.x; idx < rows * (BN / 4); idx += NTHR) {
    const int i = idx / (BN / 4);
    const int c = 4 * (idx - i * (BN / 4));
    const int orow = sm.out[i];
    if (orow == -1 || n0 + c >= p.N) continue;
    const float4 v = *reinterpret_cast<const float4*>(tile + i * LD + c);
    if (orow < 0) {               // the token's only local slot: its combined output
      uint2 o;
      o.x = pack_bf16x2(v.x, v.y);
      o.y = pack_bf16x2(v.z, v.w);
      *reinterpret_cast<uint2*>(p.direct_out + (int64_t)(-orow - 2) * p.direct_ld + n0 + c) = o;
      continue;
    }
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (int64_t)orow * p.N + n0 + c) = v;
  }
}

// Split-K reduce (the post gates splitting by shape, section "H200 prefill
// and TP8"; here a plain split of K into p.split slices for grids that would
// leave the machine underfilled).  Every slice's workgroup stores its fp32
// accumulators, then counts its arrival on the tile's counter; the last to
// arrive sums all slices in slice order 0, 1, ..., so the result does not
// depend on which workgroup came last, resets the counter for the next call
// and returns true with the sum in tot.  No workgroup waits for another.
//
// Coherence without whole-cache maintenance: the eight XCDs' L2 caches are
// not coherent with each other, and an agent-scope fence writes back or
// invalidates a whole L2 (measured: TP8 T = 16 gate/up 51 -> 349 us with a
// fence per workgroup).  So the slices are written and read with agent-scope
// relaxed atomic accesses, which the gfx950 code generator issues with the
// device-coherence cache bit (write-through / re-fetch at the coherence
// point); each workgroup waits for its stores' completion before it counts
// its arrival, and the counter is itself an agent-scope atomic.
template <int MT, int NR, int NW>
__device__ __forceinline__ bool split_reduce(const GemmParams& p, TileSmem<MT>& sm, int tile, int s, uint32_t tmask,
                                             const f32x4_t (&acc)[NR][MT], f32x4_t (&tot)[NR][MT]) {
  constexpr int NTHR = NW * kWave;
  constexpr int SLICE = NR * MT * NTHR * 2;          // 64-bit words per slice
  uint64_t* base = reinterpret_cast<uint64_t*>(p.split_partial) + (int64_t)tile * p.split * SLICE;
  uint64_t* mine = base + (int64_t)s * SLICE;
  auto pair = [](float a, float b) {
    return (uint64_t)__builtin_bit_cast(uint32_t, a) | ((uint64_t)__builtin_bit_cast(uint32_t, b) << 32);
  };
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if ((tmask >> t) & 1u) {
        const f32x4_t v = acc[r][t];
        uint64_t* d = mine + 2 * ((r * MT + t) * NTHR + threadIdx.x);
        __hip_atomic_store(d, pair(v[0], v[1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d + 1, pair(v[2], v[3]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);                     // this thread's slice stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();                                    // ... for every thread of the workgroup
  if (threadIdx.x == 0) {
    const uint32_t before = __hip_atomic_fetch_add(p.split_count + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before == (uint32_t)p.split - 1u;
    if (last) __hip_atomic_store(p.split_count + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = last;
  }
  __syncthreads();
  if (!sm.last) return false;
  auto lo = [](uint64_t w) { return __builtin_bit_cast(float, (uint32_t)w); };
  auto hi = [](uint64_t w) { return __builtin_bit_cast(float, (uint32_t)(w >> 32)); };
  for (int q = 0; q < p.split; ++q) {
    const uint64_t* src = base + (int64_t)q * SLICE;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if ((tmask >> t) & 1u) {
          f32x4_t v;
          if (q == s) {
            v = acc[r][t];
          } else {
            const uint64_t* d = src + 2 * ((r * MT + t) * NTHR + threadIdx.x);
            const uint64_t w0 = __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t w1 = __hip_atomic_load(d + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v = f32x4_t{lo(w0), hi(w0), lo(w1), hi(w1)};
          }
          tot[r][t] = q == 0 ? v : tot[r][t] + v;
        }
  }
  return true;
}

template <int MT, int NR, int NW, int D, int ROUTE, int EPI>
__global__ __launch_bounds__(NW * kWave) void moe_gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) TileSmem<MT> sm;
  // workgroup -> (tile, K slice); consecutive workgroups are the slices of
  // one tile, then the N tiles of one routed block
  int tile = blockIdx.x, s = 0;
  const int S = p.split;
  if (S > 1) {
    tile = blockIdx.x / S;
    s = blockIdx.x - tile * S;
  }
  const bool split = S > 1 && tile < p.split_tiles;   // else slice 0 runs the whole K
  if (S > 1 && !split && s != 0) return;
  int mb, nt;
  if (!block_of(p, tile, p.n_tiles, mb, nt)) return;
  const int expert = setup_rows<MT, NW, ROUTE, EPI>(p, mb, sm);
  if (expert < 0) return;
  __syncthreads();
  const uint32_t tmask = active_tiles<MT>(sm);
  // slices of whole chunk pairs (the main loop's ranges start on an even
  // chunk); split <= (KC + 1) / 2, so none is empty
  const int KC2 = (p.KC + 1) / 2;
  const int c0 = split ? 2 * (int)((int64_t)s * KC2 / S) : 0;
  const int c1 = split ? min(p.KC, 2 * (int)((int64_t)(s + 1) * KC2 / S)) : p.KC;
  auto store = [&](const f32x4_t(&acc)[NR][MT], uint32_t tm) {
    if constexpr (EPI == kEpiWeighted && 16 * NR * NW <= 128)
      epilogue_weighted_staged<MT, NR, NW>(p, sm, nt, tm, acc);
    else
      epilogue<MT, NR, NW, EPI>(p, sm, nt, tm, acc);
  };
  run_tile<MT, NR, NW, D>(p, sm, expert, nt, tmask, c0, c1, [&](const f32x4_t(&acc)[NR][MT], uint32_t tm) {
    if (split) {
      f32x4_t tot[NR][MT];
      if (split_reduce<MT, NR, NW>(p, sm, tile, s, tm, acc, tot)) store(tot, tm);
    } else {
      store(acc, tm);
    }
  });
}

// Few routed rows (block_m 16) and a grid too small for the machine: one
// 16-row weight tile of one routed block per workgroup (two, gate and up,
// for the fused SiLU epilogue), its NW waves splitting K (wave w takes
// chunks [w KC / NW, (w + 1) KC / NW)).  Each wave keeps a batch of chunks of
// weights, scales and activation fragments in flight straight into
// registers (no LDS staging: the B operand of lane l is 64 contiguous bytes
// of its token row per chunk), and the waves' partial sums meet in LDS,
// summed in wave order, so no global split-K reduction (slices, arrival
// counter, second pass) sits on the path.  The product is the MFMA
// kernel's: bf16 weights dequantised by dequant8, fp32 accumulation, one
// rounding at the store; only the order of the K sums differs from the
// other tiles (per wave, then over waves).  Indexed routing; per-slot,
// weighted or fused SiLU epilogue.
template <int NT, int NW>
struct KwSmem {
  int row[16];
  int out[16];
  float w[16];
  f32x4_t red[NW][NT][kWave];
};

template <int NW, int EPI>
__global__ __launch_bounds__(NW * kWave) void moe_gemm_kwave_kernel(const GemmParams p) {
  constexpr int NT = EPI == kEpiSilu ? 2 : 1;     // weight tiles per workgroup
  constexpr int KB = 8 / NT;                       // chunks in flight per wave
  __shared__ __attribute__((aligned(16))) KwSmem<NT, NW> sm;
  int mb, nt;
  if (!block_of(p, blockIdx.x, p.n_tiles, mb, nt)) return;
  const int expert = setup_rows<1, NW, kRouteIndexed, EPI>(p, mb, sm);
  if (expert < 0) return;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int KC = p.KC;
  const int c0 = (int)((int64_t)wave * KC / NW), c1 = (int)((int64_t)(wave + 1) * KC / NW);
  gptr_t wbase[NT], sbase[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const int64_t tile = (int64_t)expert * p.w_tiles + min(NT * nt + r, p.NT - 1);
    wbase[r] = uniform_ptr(p.packed_w + tile * KC * kWave) + lane * 16;
    sbase[r] = uniform_ptr(p.packed_s + tile * ((KC + 1) / 2) * kWave) + lane * 4;
  }
  // B operand: lane l supplies token row l % 16 at K 32 (l / 16) .. + 31 of
  // each chunk, the same K positions its weight words cover (step j: bytes
  // 16 j .. 16 j + 15 of those 64)
  const int arow = sm.row[lane & 15];
  const gptr_t abase = uniform_ptr(p.a) + (int64_t)max(arow, 0) * p.K * 2 + (lane >> 4) * 64;
  const DequantMasks masks = make_dequant_masks();
  f32x4_t acc[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int cb = c0; cb < c1; cb += KB) {
    u32x4_t w[KB][NT];
    uint32_t sw[KB][NT];
    bf16x8_t x[KB][4];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int c = min(cb + i, c1 - 1);          // past c1: a repeated load, not used
#pragma unroll
      for (int r = 0; r < NT; ++r) {
        w[i][r] = gload_u32x4(wbase[r] + (int64_t)c * (kWave * 16));
        sw[i][r] = gload_u32(sbase[r] + (int64_t)(c >> 1) * (kWave * 4));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[i][j] = arow >= 0 ? __builtin_bit_cast(bf16x8_t, gload_u32x4(abase + (int64_t)c * (kChunk * 2) + 16 * j))
                            : bf16x8_t{};
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int c = cb + i;
      if (c >= c1) break;
#pragma unroll
      for (int r = 0; r < NT; ++r) {
        const float sv = __builtin_bit_cast(float, (c & 1) ? (sw[i][r] & 0xFFFF0000u) : (sw[i][r] << 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t A = dequant8(w[i][r][j], sv, -1032.0f * sv, 0.0625f * sv, -72.0f * sv, masks);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, x[i][j], acc[r], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NT; ++r) sm.red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave != 0) return;
  f32x4_t tot[NT][1];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    tot[r][0] = sm.red[0][r][lane];
#pragma unroll
    for (int v = 1; v < NW; ++v) tot[r][0] += sm.red[v][r][lane];
  }
  epilogue<1, NT, 1, EPI>(p, sm, nt, 1u, tot);
}

// Work partition shared by the stream-K kernel and its fix-up: `units`
// (tile, chunk pair) units split into ranges of `per` units, one per
// workgroup (whole pairs: the main loop's ranges start on an even chunk).
struct SkPartition {
  int64_t units, per;
};

template <int MT, int ROUTE>
__device__ __forceinline__ SkPartition sk_partition(const GemmParams& p, int64_t workgroups) {
  const int64_t units = (int64_t)live_blocks<MT, ROUTE>(p) * p.n_tiles * ((p.KC + 1) / 2);
  return SkPartition{units, (units + workgroups - 1) / workgroups};
}

template <int MT, int NR, int NW, int D, int ROUTE, int EPI>
__global__ __launch_bounds__(NW * kWave) void moe_gemm_streamk_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) TileSmem<MT> sm;
  constexpr int NTHR = NW * kWave;
  const SkPartition part = sk_partition<MT, ROUTE>(p, gridDim.x);
  const int64_t g = blockIdx.x;
  const int64_t end = min(part.units, (g + 1) * part.per);
  const int KC = p.KC;
  const int KC2 = (KC + 1) / 2;
  bool first = true;
  for (int64_t u = g * part.per; u < end;) {
    const int64_t item = u / KC2;
    const int q0 = (int)(u - item * KC2);
    const int q1 = (int)min((int64_t)KC2, q0 + (end - u));
    const int c0 = 2 * q0;
    const int c1 = min(KC, 2 * q1);
    const int mb = (int)(item / p.n_tiles);
    const int nt = (int)(item - (int64_t)mb * p.n_tiles);
    __syncthreads();                       // previous tile's LDS readers are done
    const int expert = setup_rows<MT, NW, ROUTE, EPI>(p, mb, sm);
    __syncthreads();
    if (expert >= 0) {
      const uint32_t tmask = active_tiles<MT>(sm);
      run_tile<MT, NR, NW, D>(p, sm, expert, nt, tmask, c0, c1, [&](const f32x4_t(&acc)[NR][MT], uint32_t tm) {
        if (c0 == 0 && c1 == KC) {
          epilogue<MT, NR, NW, EPI>(p, sm, nt, tm, acc);
        } else {
          // a range holds at most two cut tiles: its first and its last
          float4* slot = partial_slot<MT, NR, NW>(p, 2 * g + (first ? 0 : 1));
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t)
              if ((tm >> t) & 1u) {
                const f32x4_t v = acc[r][t];
                slot[(r * MT + t) * NTHR + threadIdx.x] = make_float4(v[0], v[1], v[2], v[3]);
              }
        }
      });
    }
    first = false;
    u += q1 - q0;
  }
}

// One workgroup per range boundary: if the boundary cuts a tile and is the
// first boundary inside it, sum that tile's partials in range order (the
// order of the K chunks they cover) and write its outputs.
template <int MT, int NR, int NW, int ROUTE, int EPI>
__global__ __launch_bounds__(NW * kWave) void streamk_fixup_kernel(const GemmParams p, int sk_grid) {
  __shared__ __attribute__((aligned(16))) TileSmem<MT> sm;
  constexpr int NTHR = NW * kWave;
  const SkPartition part = sk_partition<MT, ROUTE>(p, sk_grid);
  const int KC2 = (p.KC + 1) / 2;                  // units (chunk pairs) per tile
  const int64_t g = (int64_t)blockIdx.x + 1;       // boundary between ranges g-1 and g
  const int64_t b = g * part.per;
  if (b >= part.units || b % KC2 == 0) return;     // boundary at a tile edge: nothing cut
  const int64_t item = b / KC2;
  if ((g - 1) * part.per > item * KC2) return;     // an earlier boundary inside this tile owns it
  const int mb = (int)(item / p.n_tiles);
  const int nt = (int)(item - (int64_t)mb * p.n_tiles);
  const int expert = setup_rows<MT, NW, ROUTE, EPI>(p, mb, sm);
  if (expert < 0) return;
  __syncthreads();
  const uint32_t tmask = active_tiles<MT>(sm);
  f32x4_t acc[NR][MT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t h0 = item * KC2 / part.per, h1 = ((item + 1) * KC2 - 1) / part.per;
  for (int64_t h = h0; h <= h1; ++h) {
    const int64_t slot = (h * part.per) / KC2 == item ? 2 * h : 2 * h + 1;
    const float4* src = partial_slot<MT, NR, NW>(p, slot);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if ((tmask >> t) & 1u) {
          const float4 v = src[(r * MT + t) * NTHR + threadIdx.x];
          acc[r][t][0] += v.x;
          acc[r][t][1] += v.y;
          acc[r][t][2] += v.z;
          acc[r][t][3] += v.w;
        }
  }
  epilogue<MT, NR, NW, EPI>(p, sm, nt, tmask, acc);
}

// Top-k combine: out[t, n] = bf16(sum over local j, in j order, of
// partial[t*k + j, n]); tokens with no local slot get 0.  One thread per
// 8 columns of a token.  For topk <= KMAX every load (the token's ids, then
// the partial rows of its local slots) is issued before the first add, so
// the slots' latencies overlap instead of adding up; the sum still runs in
// j order and skips non-local slots (an add of zero would turn -0 into +0).
// token_local != nullptr: tokens with exactly one local slot were stored by
// the GEMM and are left alone.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial,
                                                      const int32_t* __restrict__ topk_ids,
                                                      int32_t T, int32_t topk, int32_t first,
                                                      int32_t E_loc, int32_t N,
                                                      uint16_t* __restrict__ out, int32_t ldo,
                                                      const uint8_t* __restrict__ token_local) {
  const int n8 = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * n8) return;
  const int64_t t = idx / n8;
  const int n = (int)(idx - t * n8) * 8;
  if (token_local != nullptr && token_local[t] == 1) return;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const float4& u, const float4& v) {
    a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w;
    a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
  };
  if (topk <= KMAX) {
    // the id loads are unconditional (clamped index) so they issue together
    int32_t id[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) id[j] = topk_ids[t * topk + (j < topk ? j : topk - 1)];
    bool loc[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) loc[j] = j < topk && (unsigned)(id[j] - first) < (unsigned)E_loc;
    float4 u[KMAX], v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j]) {
        const float4* src = reinterpret_cast<const float4*>(partial + (t * topk + j) * (int64_t)N + n);
        u[j] = src[0];
        v[j] = src[1];
      }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j]) add(u[j], v[j]);
  } else {
    for (int j = 0; j < topk; ++j) {
      const int e = topk_ids[t * topk + j] - first;
      if ((unsigned)e >= (unsigned)E_loc) continue;
      const float4* src = reinterpret_cast<const float4*>(partial + (t * topk + j) * (int64_t)N + n);
      add(src[0], src[1]);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(a[0], a[1]);
  o.y = pack_bf16x2(a[2], a[3]);
  o.z = pack_bf16x2(a[4], a[5]);
  o.w = pack_bf16x2(a[6], a[7]);
  *reinterpret_cast<uint4*>(out + t * ldo + n) = o;
}

// Zero `words` 32-bit words (a kernel, not hipMemsetAsync, so the call can
// sit in a captured HIP graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, int64_t words, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, words);
  return hipGetLastError();
}

hipError_t launch_combine(const float* partial, const int32_t* topk_ids, int32_t T, int32_t topk,
                          int32_t first, int32_t E_loc, int32_t cols, uint16_t* out, int32_t ldo,
                          const uint8_t* token_local, hipStream_t stream) {
  const int64_t threads = (int64_t)T * (cols / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (topk <= 8)
    hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, stream, partial, topk_ids, T, topk, first, E_loc, cols,
                       out, ldo, token_local);
  else
    hipLaunchKernelGGL(combine_kernel<16>, grid, dim3(256), 0, stream, partial, topk_ids, T, topk, first, E_loc, cols,
                       out, ldo, token_local);
  return hipGetLastError();
}

// Local slots of each token (saturated at 255), one thread per token.
__global__ __launch_bounds__(256) void token_local_kernel(const int32_t* __restrict__ topk_ids, int32_t T,
                                                          int32_t topk, int32_t first, int32_t E_loc,
                                                          uint8_t* __restrict__ cnt) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int c = 0;
  for (int j = 0; j < topk; ++j) c += (unsigned)(topk_ids[t * topk + j] - first) < (unsigned)E_loc;
  cnt[t] = (uint8_t)min(c, 255);
}

hipError_t launch_token_local(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t first, int32_t E_loc,
                              uint8_t* cnt, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(token_local_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream, topk_ids, T, topk,
                     first, E_loc, cnt);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch
typedef void (*GemmKernel)(const GemmParams);
typedef void (*FixupKernel)(const GemmParams, int);

struct KernelSet {
  GemmKernel classic = nullptr;
  GemmKernel streamk = nullptr;
  FixupKernel fixup = nullptr;
};

template <int MT, int NR, int NW, int D, int ROUTE, int EPI>
static KernelSet make_set() {
  KernelSet s;
  s.classic = moe_gemm_kernel<MT, NR, NW, D, ROUTE, EPI>;
  s.streamk = moe_gemm_streamk_kernel<MT, NR, NW, D, ROUTE, EPI>;
  s.fixup = streamk_fixup_kernel<MT, NR, NW, ROUTE, EPI>;
  return s;
}

// one workgroup per tile only (no stream-K form)
template <int MT, int NR, int NW, int D, int ROUTE, int EPI>
static KernelSet make_classic() {
  KernelSet s;
  s.classic = moe_gemm_kernel<MT, NR, NW, D, ROUTE, EPI>;
  return s;
}

template <int MT, int NR, int NW, int D>
static KernelSet pick(int route, int epi) {
  if (route == kRouteIndexed) {
    if (epi == kEpiSilu) {
      if constexpr (NR % 2 == 0) return make_classic<MT, NR, NW, D, kRouteIndexed, kEpiSilu>();
      return KernelSet{};
    }
    return epi == kEpiWeighted ? make_set<MT, NR, NW, D, kRouteIndexed, kEpiWeighted>()
                               : make_set<MT, NR, NW, D, kRouteIndexed, kEpiStore>();
  }
  if (epi != kEpiStore) return KernelSet{};
  if (route == kRouteContiguous) return make_set<MT, NR, NW, D, kRouteContiguous, kEpiStore>();
  if (route == kRouteMasked) return make_set<MT, NR, NW, D, kRouteMasked, kEpiStore>();
  return KernelSet{};
}

// Built tile configurations (MT, NR, waves, stages): every (MT, NR) with four
// waves and two prefetch stages; four stages for the decode tiles (MT <= 2,
// NR = 2); eight waves (twice the weight rows per staged activation chunk)
// for MT = 1, 2 and 8 with NR = 2.
static KernelSet find_kernels(int route, int epi, int m_tiles, int nr, int waves, int stages) {
  // one weight tile per workgroup, waves splitting K (moe_gemm_kwave_kernel)
  if (m_tiles == 1 && nr == 1 && waves == kKwWaves && stages == 2 && route == kRouteIndexed) {
    KernelSet k;
    if (epi == kEpiStore) k.classic = moe_gemm_kwave_kernel<kKwWaves, kEpiStore>;
    if (epi == kEpiWeighted) k.classic = moe_gemm_kwave_kernel<kKwWaves, kEpiWeighted>;
    if (epi == kEpiSilu) k.classic = moe_gemm_kwave_kernel<kKwWaves, kEpiSilu>;
    return k;
  }
#define W4A16_CASE(MT_, NR_, NW_, D_) \
  if (m_tiles == MT_ && nr == NR_ && waves == NW_ && stages == D_) return pick<MT_, NR_, NW_, D_>(route, epi);
  W4A16_CASE(1, 2, 4, 2) W4A16_CASE(2, 2, 4, 2) W4A16_CASE(4, 2, 4, 2) W4A16_CASE(8, 2, 4, 2)
  W4A16_CASE(1, 4, 4, 2) W4A16_CASE(2, 4, 4, 2) W4A16_CASE(4, 4, 4, 2) W4A16_CASE(8, 4, 4, 2)
  W4A16_CASE(1, 2, 4, 4) W4A16_CASE(2, 2, 4, 4)
  W4A16_CASE(1, 2, 8, 2) W4A16_CASE(2, 2, 8, 2) W4A16_CASE(8, 2, 8, 2) W4A16_CASE(16, 2, 8, 2)
#undef W4A16_CASE
  return KernelSet{};
}

bool gemm_config_supported(int route, int epilogue, int m_tiles, int nr, int waves, int stages) {
  return find_kernels(route, epilogue, m_tiles, nr, waves, stages).classic != nullptr;
}

// The N tiles of a block share an XCD (block_of) when K is not split and a
// block has 2 .. kXcdGroupMaxTiles of them.
int xcd_group_for(int split, int per_block) { return split <= 1 && per_block >= 2 && per_block <= kXcdGroupMaxTiles; }

hipError_t launch_gemm(int route, int epilogue, int m_tiles, int nr, int waves, int stages,
                       const GemmParams& p, hipStream_t stream) {
  if (prefill_applies(route, epilogue, m_tiles, nr, waves, stages, p))
    return launch_gemm_prefill(route, epilogue, m_tiles, nr, waves, p, stream);
  const KernelSet k = find_kernels(route, epilogue, m_tiles, nr, waves, stages);
  if (k.classic == nullptr) return hipErrorInvalidValue;
  // Block-major order spreads a block's N tiles over the XCDs (round robin);
  // blocks with few N tiles keep them on one XCD instead (block_of).
  GemmParams q = p;
  q.xcd_group = xcd_group_for(p.split, p.n_tiles);
  // decode tiles (at most 32 rows) of a block with 32 or more N tiles: groups
  // of kXcdDecodeGroup N tiles per XCD, so the block's activation rows land in
  // min(8, n_tiles / 16) L2s instead of all eight (measured on MI355X, EP8
  // decode gate/up: 2% faster, HBM bytes 1.089x -> 1.030x the weight and
  // scale bytes).  Not the K-split tile (nr 1): it runs on small grids, where
  // rounding up to whole groups leaves workgroups idle (T = 1: 0.5 us slower).
  if (nr > 1 && p.split <= 1 && m_tiles <= 2 && q.n_tiles >= 2 * kXcdDecodeGroup &&
      q.n_tiles % kXcdDecodeGroup == 0)
    q.xcd_group = kXcdDecodeGroup;
  const int64_t grid = grid_of(q, q.n_tiles) * std::max(q.split, 1);
  if (grid <= 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  if (q.split > 1 && (q.split > (q.KC + 1) / 2 || (q.split_tiles > 0 && (!q.split_partial || !q.split_count))))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k.classic, dim3((unsigned)grid), dim3(waves * kWave), 0, stream, q);
  return hipGetLastError();
}

size_t split_slice_bytes(int m_tiles, int nr, int waves) { return (size_t)nr * m_tiles * waves * kWave * 16; }

int streamk_workgroups(int route, int epilogue, int m_tiles, int nr, int waves, int stages) {
  const KernelSet k = find_kernels(route, epilogue, m_tiles, nr, waves, stages);
  if (k.streamk == nullptr) return 0;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k.streamk),
                                                   waves * kWave, 0) != hipSuccess)
    return 0;
  return cus * std::max(per_cu, 1);
}

size_t streamk_partial_bytes(int m_tiles, int nr, int waves, int workgroups) {
  return (size_t)2 * workgroups * (size_t)(nr * m_tiles * waves * kWave) * 16;
}

hipError_t launch_gemm_streamk(int route, int epilogue, int m_tiles, int nr, int waves, int stages,
                               const GemmParams& p, int workgroups, hipStream_t stream) {
  const KernelSet k = find_kernels(route, epilogue, m_tiles, nr, waves, stages);
  if (k.streamk == nullptr || workgroups <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k.streamk, dim3((unsigned)workgroups), dim3(waves * kWave), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || workgroups < 2) return e;
  hipLaunchKernelGGL(k.fixup, dim3((unsigned)(workgroups - 1)), dim3(waves * kWave), 0, stream, p,
                     workgroups);
  return hipGetLastError();
}

}  // namespace w4a16

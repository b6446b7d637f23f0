// Routed-block bookkeeping shared by the W4A16 and MXFP4 GEMM kernels:
// which rows a block reads and writes (the row sources of the Chord W4A16
// MoE post, sections "Two kernel families" and "Grouped SM90 kernels"), and
// the epilogues that store a tile's fp32 accumulators.  `Smem` is any
// shared-memory struct with the per-block tables
//   int row[16 * MT];    activation row per block row, -1 = padding
//   int out[16 * MT];    output row per block row, -1 = not stored
//   float w[16 * MT];    top-k weight per block row (weighted epilogue)
#pragma once
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

// Number of routed blocks with work (indexed: from the device-side padded
// total; grouped: the launch's block count).
template <int MT, int ROUTE>
__device__ __forceinline__ int live_blocks(const GemmParams& p) {
  if constexpr (ROUTE == kRouteIndexed)
    return min(*p.num_tokens_padded / (16 * MT), p.grid_blocks);
  else
    return p.grid_blocks;
}

// Routed block mb and per-block item j (N tile, or group of N tiles) of work
// item w, for `per` items per block.  Block-major by default: consecutive
// items are one block's, and the hardware's round-robin dispatch sends
// consecutive workgroups to different XCDs, so each XCD fetches the block's
// activation rows into its own L2.  p.xcd_group: items of one block are 8
// apart, i.e. on one XCD, which then fetches the rows once (1: all `per`
// items of a block; > 1: groups of xcd_group items, so a block spans
// per / xcd_group XCDs); w runs over groups of 8 (block, group) pairs x the
// group's items (the launcher rounds the grid up to whole groups) and items
// past the last block return false.  Group sizes are measured choices: an
// early decode kernel ran 3x slower with all 32 N tiles of a block on one XCD
// (its workgroups asked one L2 for the same lines at once); the current one
// takes groups of 16 at no cost.
__device__ __forceinline__ bool block_of(const GemmParams& p, int w, int per, int& mb, int& j) {
  if (!p.xcd_group) {
    mb = w / per;
    j = w - mb * per;
    return true;
  }
  // groups of tq consecutive items of a block share an XCD (tq = per: the
  // whole block; xcd_group > 1: tq = xcd_group, dividing per)
  const int tq = p.xcd_group == 1 ? per : p.xcd_group;
  const int parts = per / tq;
  const int k = w >> 3;
  const int g = k / tq;
  const int t = k - g * tq;
  const int q = g * 8 + (w & 7);
  mb = q / parts;
  j = (q - mb * parts) * tq + t;
  return mb < p.grid_blocks;
}

// Grid of a launch with `per` items per routed block (see block_of).
inline int64_t grid_of(const GemmParams& p, int per) {
  if (!p.xcd_group) return (int64_t)p.grid_blocks * per;
  const int tq = p.xcd_group == 1 ? per : p.xcd_group;
  return ((int64_t)p.grid_blocks * (per / tq) + 7) / 8 * 8 * tq;
}

// Fill the block's row tables; returns the block's expert (wave-uniform) or
// -1 when the block has no work.  The caller synchronises afterwards.
template <int MT, int NW, int ROUTE, int EPI, typename Smem>
__device__ __forceinline__ int setup_rows(const GemmParams& p, int mb, Smem& sm) {
  constexpr int BM = 16 * MT;
  constexpr int NTHR = NW * kWave;
  const int tid = threadIdx.x;
  int expert;
  if constexpr (ROUTE == kRouteIndexed) {
    if (mb * BM >= *p.num_tokens_padded) return -1;
    expert = p.expert_ids[mb >> p.expert_shift];
    if ((unsigned)expert >= (unsigned)p.E) return -1;   // -1 (unused block) or foreign id
    // tiles smaller than the routing's blocks: an expert's padding sits at the
    // end of its segment, so a tile whose first row is padding has no rows
    if (p.expert_shift && (unsigned)p.sorted_ids[mb * BM] >= (unsigned)p.sentinel) return -1;
    for (int i = tid; i < BM; i += NTHR) {
      const int pos = mb * BM + i;                         // sorted position
      const int s = p.sorted_ids[pos];
      const bool v = (unsigned)s < (unsigned)p.sentinel;
      // activation row: the slot's token (a_row_div = topk), the slot (1),
      // or the sorted position itself (0: rows already in sorted order)
      sm.row[i] = v ? (p.a_row_div > 0 ? s / p.a_row_div : pos) : -1;
      sm.out[i] = v ? (EPI == kEpiSilu || EPI == kEpiSiluMx ? pos : s) : -1;
      if constexpr (EPI == kEpiWeighted) {
        sm.w[i] = v ? p.slot_weight[s] : 0.f;
        // a token with one local slot: out = -(token + 2), stored directly as bf16
        if (v && p.token_local != nullptr) {
          const int t = s / p.topk;
          if (p.token_local[t] == 1) sm.out[i] = -(t + 2);
        }
      }
    }
  } else if constexpr (ROUTE == kRouteContiguous) {
    const int r0 = mb * BM;
    expert = p.m_indices[r0];
    if ((unsigned)expert >= (unsigned)p.E) return -1;   // padding block (-1) or foreign id
    for (int i = tid; i < BM; i += NTHR) {
      const bool v = p.m_indices[r0 + i] == expert;
      sm.row[i] = v ? r0 + i : -1;
      sm.out[i] = sm.row[i];
    }
  } else {
    const int g = mb / p.blocks_per_group;
    const int r0 = (mb - g * p.blocks_per_group) * BM;
    const int cnt = min(p.masked_m[g], p.max_m);
    if (r0 >= cnt) return -1;
    expert = g;
    for (int i = tid; i < BM; i += NTHR) {
      const int r = r0 + i;
      const bool v = r < cnt;
      sm.row[i] = v ? g * p.max_m + r : -1;
      sm.out[i] = sm.row[i];
    }
  }
  return __builtin_amdgcn_readfirstlane(expert);
}

// Wave-uniform mask of token tiles holding at least one valid row.
template <int MT, typename Smem>
__device__ __forceinline__ uint32_t active_tiles(const Smem& sm) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t tmask = 0;
#pragma unroll
  for (int t = 0; t < MT; ++t)
    if (__ballot(sm.row[16 * t + (lane & 15)] >= 0)) tmask |= 1u << t;
  return tmask;
}

// Output feature tile of packed tile `rt` (gate/up interleaved weights store
// gate tile t at 2t and up tile t at 2t + 1).
__device__ __forceinline__ int logical_tile(const GemmParams& p, int rt) {
  return p.gated ? (rt & 1 ? p.NT / 2 + (rt >> 1) : rt >> 1) : rt;
}

// silu(g) * u in fp32 for bf16-rounded g and u (the values the per-slot
// gate/up output holds), rounded once to bf16 by the caller
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Write the tile's outputs.  Lane holds rows n = 16*tile + 4*(lane/16) + v
// (v = 0..3) of token column lane % 16 of each token tile.
template <int MT, int NR, int NW, int EPI, typename Smem>
__device__ __forceinline__ void epilogue(const GemmParams& p, const Smem& sm, int nt,
                                         uint32_t tmask, const f32x4_t (&acc)[NR][MT]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rt_base = nt * (NW * NR) + wave * NR;
  const int nr_valid = min(NR, p.NT - rt_base);
  if constexpr (EPI == kEpiSilu) {
    // tiles come in (gate, up) pairs: packed tiles rt_base + r and + r + 1
    // (rt_base and NT are even) hold gate and up tile (rt_base + r) / 2
    static_assert(NR % 2 == 0, "gate and up tiles in pairs");
    const int NI = p.N / 2;
#pragma unroll
    for (int r = 0; r < NR; r += 2) {
      if (r >= nr_valid) continue;
      const int n = ((rt_base + r) >> 1) * kRowTile + 4 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (!((tmask >> t) & 1u)) continue;
        const int i = 16 * t + (lane & 15);
        const int orow = sm.out[i];
        if (orow < 0) continue;
        const f32x4_t g = acc[r][t], u = acc[r + 1][t];
        float y[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t gu = pack_bf16x2(g[v], u[v]);       // the per-slot bf16 outputs
          y[v] = silu_mul(bf16_bits_to_float(gu & 0xFFFFu), bf16_bits_to_float(gu >> 16));
        }
        uint2 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + (int64_t)orow * NI + n) = o;
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r >= nr_valid) continue;
    const int n = logical_tile(p, rt_base + r) * kRowTile + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (!((tmask >> t) & 1u)) continue;
      const int i = 16 * t + (lane & 15);
      const int orow = sm.out[i];
      if (EPI == kEpiWeighted ? orow == -1 : orow < 0) continue;
      const f32x4_t v = acc[r][t];
      if constexpr (EPI == kEpiWeighted) {
        const float w = sm.w[i];
        if (orow < 0) {            // the token's only local slot: its combined output
          uint2 o;
          o.x = pack_bf16x2(w * v[0], w * v[1]);
          o.y = pack_bf16x2(w * v[2], w * v[3]);
          *reinterpret_cast<uint2*>(p.direct_out + (int64_t)(-orow - 2) * p.direct_ld + n) = o;
          continue;
        }
      }
      if constexpr (EPI == kEpiStore) {
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + (int64_t)orow * p.N + n) = o;
      } else {
        const float w = sm.w[i];
        float4 o = make_float4(w * v[0], w * v[1], w * v[2], w * v[3]);
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (int64_t)orow * p.N + n) = o;
      }
    }
  }
}

}  // namespace w4a16

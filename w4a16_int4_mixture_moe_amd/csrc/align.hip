// Routing align for the indexed MoE GEMM: a stable counting sort of routed
// slots by local expert, padded per expert to a multiple of block_m with a
// sentinel slot id.
//
// Chord W4A16 MoE post (vLLM x Novita AI), section "Two kernel families": the
// indexed family consumes sorted_ids / expert_ids / num_tokens_padded; section
// "vLLM integration": the buffers are over-allocated so no count is read back
// to the host and the call stays graph-capturable; section "Grouped SM90
// kernels", Figure 3: indexed routing puts its padding in sentinel indices.
//
// One workgroup of 16 or 8 waves.  Wave w owns a contiguous range of slots, so the
// order of slots inside an expert segment is ascending by construction:
//   pass 1  each wave counts its slots per expert (LDS atomics), 16 loads in
//           flight per lane (one workgroup has to keep many requests out to
//           read the ids at more than a trickle);
//   scan    per expert, exclusive prefix over waves, then an exclusive scan of
//           the padded expert totals gives segment starts;
//   fill    sentinels inside segment tails and after the padded total,
//           expert_ids per block, the padded total itself;
//   pass 2  each wave walks its range 64 slots at a time; lanes routed to the
//           same expert find each other (a per-wave table of lane masks in
//           LDS, or one ballot per expert-id bit), take consecutive
//           positions in lane order, and the group's lowest lane advances
//           the wave's cursor for that expert.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

constexpr int kAlignBatch = 16;                // slot ids in flight per lane

// kAlignWaves waves: 16, or 8 when the per-wave tables of many experts would
// not fit the default LDS allocation.  kMaskMatch: pass 2 finds the lanes of
// a sub-tile routed to the same expert through a per-wave table of 64-bit
// lane masks in LDS (one atomic OR per lane, one read back); otherwise with
// one ballot per expert-id bit (no table; for more than 512 local experts).
template <int kAlignWaves, bool kMaskMatch>
__global__ __launch_bounds__(kAlignWaves * kWave) void align_kernel(
    const int32_t* __restrict__ topk_ids, int32_t total, int32_t first, int32_t E_loc,
    int32_t bm, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ ntp_out, int64_t capacity) {
  constexpr int kAlignThreads = kAlignWaves * kWave;
  extern __shared__ unsigned long long smem64[];
  // [kAlignWaves][E_loc] lane masks (kMaskMatch only), 8-byte aligned first
  unsigned long long* lanes_of = smem64;
  int* cnt = reinterpret_cast<int*>(smem64 + (kMaskMatch ? kAlignWaves * E_loc : 0));
                                              // [kAlignWaves][E_loc]: counts, then cursors
  int* seg = cnt + kAlignWaves * E_loc;       // [E_loc + 1]: padded segment starts
  int* num = seg + E_loc + 1;                 // [E_loc]: slots per expert

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;

  for (int i = tid; i < kAlignWaves * E_loc; i += kAlignThreads) {
    cnt[i] = 0;
    if constexpr (kMaskMatch) lanes_of[i] = 0ull;
  }
  __syncthreads();

  const int per = ((total + kAlignWaves - 1) / kAlignWaves + kWave - 1) & ~(kWave - 1);
  const int beg = min(w * per, total);
  const int end = min(beg + per, total);

  // pass 1: per-wave expert histogram
  for (int s0 = beg; s0 < end; s0 += kAlignBatch * kWave) {
    int id[kAlignBatch];
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int s = s0 + u * kWave + lane;
      id[u] = s < end ? topk_ids[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int e = id[u] - first;
      if (id[u] >= 0 && (unsigned)e < (unsigned)E_loc) atomicAdd(&cnt[w * E_loc + e], 1);
    }
  }
  __syncthreads();

  // per expert: exclusive prefix over waves, total count
  for (int e = tid; e < E_loc; e += kAlignThreads) {
    int run = 0;
    for (int v = 0; v < kAlignWaves; ++v) {
      const int c = cnt[v * E_loc + e];
      cnt[v * E_loc + e] = run;
      run += c;
    }
    num[e] = run;
  }
  __syncthreads();

  // exclusive scan of padded totals (wave 0; each lane a run of experts)
  if (w == 0) {
    const int per_lane = (E_loc + kWave - 1) / kWave;
    const int e0 = min(lane * per_lane, E_loc);
    const int e1 = min(e0 + per_lane, E_loc);
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += (num[e] + bm - 1) / bm * bm;
    int incl = mine;
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    int run = incl - mine;
    for (int e = e0; e < e1; ++e) {
      seg[e] = run;
      run += (num[e] + bm - 1) / bm * bm;
    }
    if (lane == kWave - 1) seg[E_loc] = incl;
  }
  __syncthreads();

  const int ntp = seg[E_loc];
  const int sentinel = total;
  for (int i = tid; i < kAlignWaves * E_loc; i += kAlignThreads) cnt[i] += seg[i % E_loc];
  for (int e = tid; e < E_loc; e += kAlignThreads) {
    const int o = seg[e], n = num[e], o_end = seg[e + 1];
    for (int q = o + n; q < o_end; ++q) sorted_ids[q] = sentinel;
    for (int b = o / bm; b < o_end / bm; ++b) expert_ids[b] = e;
  }
  for (int64_t q = ntp + tid; q < capacity; q += kAlignThreads) sorted_ids[q] = sentinel;
  for (int64_t b = ntp / bm + tid; b < capacity / bm; b += kAlignThreads) expert_ids[b] = -1;
  if (tid == 0) *ntp_out = ntp;
  __syncthreads();

  // pass 2: stable scatter
  const int nbits = 32 - __clz(max(E_loc - 1, 1));
  const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  // ids of the next kAlignBatch sub-tiles are requested together, then
  // consumed in order
  for (int s0 = beg; s0 < end; s0 += kAlignBatch * kWave) {
    int id8[kAlignBatch];
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int s = s0 + u * kWave + lane;
      id8[u] = s < end ? topk_ids[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int base = s0 + u * kWave;
      if (base >= end) break;
      const int s = base + lane;
      const int e = id8[u] - first;
      const bool loc = (s < end) && id8[u] >= 0 && ((unsigned)e < (unsigned)E_loc);
      uint64_t peers;
      if constexpr (kMaskMatch) {
        // every lane ORs its bit into its expert's mask; the wave's LDS
        // operations complete in order, so the read-back sees all of them
        if (loc) atomicOr(&lanes_of[w * E_loc + e], 1ull << lane);
        __builtin_amdgcn_wave_barrier();
        peers = loc ? lanes_of[w * E_loc + e] : 0ull;
      } else {
        peers = __ballot(loc);
        for (int b = 0; b < nbits; ++b) {
          const bool bit = loc && ((e >> b) & 1);
          const uint64_t m = __ballot(bit);
          peers &= bit ? m : ~m;
        }
      }
      int cur = 0;
      if (loc) {
        cur = cnt[w * E_loc + e];
        sorted_ids[cur + __popcll(peers & lanes_below)] = s;
      }
      // every lane has read its cursor (and mask) before any lane of this
      // wave updates them
      __builtin_amdgcn_wave_barrier();
      if (loc && (peers & lanes_below) == 0) {
        cnt[w * E_loc + e] = cur + __popcll(peers);
        if constexpr (kMaskMatch) lanes_of[w * E_loc + e] = 0ull;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

hipError_t launch_align(const int32_t* topk_ids, int32_t total_slots, int32_t first, int32_t E_loc,
                        int32_t block_m, int32_t* sorted_ids, int32_t* expert_ids,
                        int32_t* num_tokens_padded, int64_t capacity, hipStream_t stream) {
  // LDS: lane masks 8 B and counters 4 B per (wave, expert), plus 8 B per
  // expert: <= 27 KB (16 waves, <= 128 experts), <= 53 KB (8 waves, <= 512),
  // <= 41 KB (8 waves, ballot matching, <= 1024)
  auto lds = [&](int waves, bool masks) {
    return (masks ? 8 * (size_t)waves * E_loc : 0) + sizeof(int) * ((size_t)waves * E_loc + 2 * (size_t)E_loc + 1);
  };
  if (E_loc <= 128)
    hipLaunchKernelGGL((align_kernel<16, true>), dim3(1), dim3(16 * kWave), lds(16, true), stream, topk_ids,
                       total_slots, first, E_loc, block_m, sorted_ids, expert_ids, num_tokens_padded, capacity);
  else if (E_loc <= 512)
    hipLaunchKernelGGL((align_kernel<8, true>), dim3(1), dim3(8 * kWave), lds(8, true), stream, topk_ids,
                       total_slots, first, E_loc, block_m, sorted_ids, expert_ids, num_tokens_padded, capacity);
  else
    hipLaunchKernelGGL((align_kernel<8, false>), dim3(1), dim3(8 * kWave), lds(8, false), stream, topk_ids,
                       total_slots, first, E_loc, block_m, sorted_ids, expert_ids, num_tokens_padded, capacity);
  return hipGetLastError();
}

}  // namespace w4a16

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
// G workgroups of 16 or 8 waves (G = 1 below kAlignMultiMin slots).
// Workgroup g owns a contiguous chunk of the slots and wave w a contiguous
// range of that chunk, so the order of slots inside an expert segment is
// ascending by construction:
//   pass 1  every workgroup counts all slots per expert (LDS atomics, 16
//           loads in flight per lane; past the first workgroup the ids come
//           from L2): its own waves' slots per wave, the slots of earlier and
//           later chunks in two totals, so each workgroup knows every
//           segment and where its own slots start in each, with no
//           communication between workgroups;
//   scan    per expert, exclusive prefix over earlier chunks and waves, then
//           an exclusive scan of the padded expert totals gives segment
//           starts;
//   fill    sentinels inside segment tails and after the padded total,
//           expert_ids per block, the padded total itself (experts and tail
//           positions dealt round robin over the workgroups);
//   pass 2  each wave walks its range 64 slots at a time; lanes routed to the
//           same expert find each other (a per-wave table of lane masks in
//           LDS, or one ballot per expert-id bit), take consecutive
//           positions in lane order, and the group's lowest lane advances
//           the wave's cursor for that expert.
// With G workgroups the scatter and fill are split G ways; the count is not
// (every workgroup reads all ids), which is what bounds a large align.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

constexpr int kAlignBatch = 16;                // slot ids in flight per lane
constexpr int kAlignMultiMin = 16384;          // slots from which several workgroups share the work
constexpr int kAlignSlotsPerGroup = 2048;
constexpr int kAlignMaxGroups = 64;

// kAlignWaves waves: 16, or 8 when the per-wave tables of many experts would
// not fit the default LDS allocation.  kMaskMatch: pass 2 finds the lanes of
// a sub-tile routed to the same expert through a per-wave table of 64-bit
// lane masks in LDS (one atomic OR per lane, one read back); otherwise with
// one ballot per expert-id bit (no table; for more than 512 local experts).
// kMulti: launched as several workgroups (otherwise exactly one, and the
// chunk bookkeeping compiles away).
template <int kAlignWaves, bool kMaskMatch, bool kMulti>
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
  int* pre = num + E_loc;                     // [E_loc]: slots of earlier chunks
  int* post = pre + E_loc;                    // [E_loc]: slots of later chunks

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int G = kMulti ? (int)gridDim.x : 1;
  const int g = kMulti ? (int)blockIdx.x : 0;

  for (int i = tid; i < kAlignWaves * E_loc; i += kAlignThreads) {
    cnt[i] = 0;
    if constexpr (kMaskMatch) lanes_of[i] = 0ull;
  }
  if constexpr (kMulti)
    for (int e = tid; e < E_loc; e += kAlignThreads) {
      pre[e] = 0;
      post[e] = 0;
    }
  __syncthreads();

  // this workgroup's chunk and this wave's range of it (multiples of 64
  // slots, so a 64-slot tile never straddles two owners)
  const int chunk = ((total + G - 1) / G + kWave - 1) & ~(kWave - 1);
  const int cbeg = min(g * chunk, total);
  const int cend = min(cbeg + chunk, total);
  const int per = ((cend - cbeg + kAlignWaves - 1) / kAlignWaves + kWave - 1) & ~(kWave - 1);
  const int beg = min(cbeg + w * per, cend);
  const int end = min(beg + per, cend);

  // pass 1: expert histogram
  if constexpr (!kMulti) {
    // one workgroup: each wave counts its own range
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
  } else {
    // all slots, tile by tile (64 slots each), counted for the owning wave
    // of this workgroup or as earlier / later chunks
    const int ntiles = (total + kWave - 1) / kWave;
    for (int t0 = w * kAlignBatch; t0 < ntiles; t0 += kAlignWaves * kAlignBatch) {
      int id[kAlignBatch];
#pragma unroll
      for (int u = 0; u < kAlignBatch; ++u) {
        const int s = (t0 + u) * kWave + lane;
        id[u] = s < total ? topk_ids[s] : -1;
      }
#pragma unroll
      for (int u = 0; u < kAlignBatch; ++u) {
        const int tb = (t0 + u) * kWave;                      // wave-uniform
        int* dst = tb < cbeg ? pre : tb >= cend ? post : cnt + ((tb - cbeg) / max(per, kWave)) * E_loc;
        const int e = id[u] - first;
        if (id[u] >= 0 && (unsigned)e < (unsigned)E_loc) atomicAdd(&dst[e], 1);
      }
    }
  }
  __syncthreads();

  // per expert: exclusive prefix over earlier chunks and this chunk's
  // waves, total count
  for (int e = tid; e < E_loc; e += kAlignThreads) {
    int run = kMulti ? pre[e] : 0;
    for (int v = 0; v < kAlignWaves; ++v) {
      const int c = cnt[v * E_loc + e];
      cnt[v * E_loc + e] = run;
      run += c;
    }
    num[e] = kMulti ? run + post[e] : run;
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
  for (int e = g + G * tid; e < E_loc; e += G * kAlignThreads) {
    const int o = seg[e], n = num[e], o_end = seg[e + 1];
    for (int q = o + n; q < o_end; ++q) sorted_ids[q] = sentinel;
    for (int b = o / bm; b < o_end / bm; ++b) expert_ids[b] = e;
  }
  const int64_t stride = (int64_t)G * kAlignThreads;
  const int64_t first_q = (int64_t)g * kAlignThreads + tid;
  for (int64_t q = ntp + first_q; q < capacity; q += stride) sorted_ids[q] = sentinel;
  for (int64_t b = ntp / bm + first_q; b < capacity / bm; b += stride) expert_ids[b] = -1;
  if (g == 0 && tid == 0) *ntp_out = ntp;
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
  // LDS: lane masks 8 B and counters 4 B per (wave, expert), plus 16 B per
  // expert: 26 KiB + 4 B at most (16 waves, <= 128 experts), 56 KiB + 4 B (8 waves,
  // <= 512), 48 KiB + 4 B (8 waves, ballot matching, <= 1024)
  auto lds = [&](int waves, bool masks) {
    return (masks ? 8 * (size_t)waves * E_loc : 0) + sizeof(int) * ((size_t)waves * E_loc + 4 * (size_t)E_loc + 1);
  };
  // one workgroup up to kAlignMultiMin slots (its count and scatter are
  // latency-bound, and more workgroups would each count everything again),
  // then one per kAlignSlotsPerGroup slots
  const int groups = total_slots < kAlignMultiMin
                         ? 1
                         : std::min(kAlignMaxGroups, (total_slots + kAlignSlotsPerGroup - 1) / kAlignSlotsPerGroup);
  auto go = [&](auto kernel, int waves, bool masks) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)groups), dim3(waves * kWave), lds(waves, masks), stream, topk_ids,
                       total_slots, first, E_loc, block_m, sorted_ids, expert_ids, num_tokens_padded, capacity);
  };
  const bool multi = groups > 1;
  if (E_loc <= 128)
    multi ? go(align_kernel<16, true, true>, 16, true) : go(align_kernel<16, true, false>, 16, true);
  else if (E_loc <= 512)
    multi ? go(align_kernel<8, true, true>, 8, true) : go(align_kernel<8, true, false>, 8, true);
  else
    multi ? go(align_kernel<8, false, true>, 8, false) : go(align_kernel<8, false, false>, 8, false);
  return hipGetLastError();
}

}  // namespace w4a16

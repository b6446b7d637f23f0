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
// Workgroup tile: one routed block of BM = 16 * MT rows (one expert) times
// BN = NW * NR * 16 weight rows; each wave owns NR 16-row weight tiles and
// every token tile of the block.  Per 128-wide K chunk:
//   - activations: BM rows x 256 B staged global -> registers -> LDS
//     (double buffered, rows padded to 272 B so the 16-byte operand reads
//     of 16 different rows fall in different LDS banks);
//   - weights: one 16-byte load per lane per weight tile straight from HBM
//     into registers (the packed layout is the operand layout), issued one
//     chunk ahead; the lane's bf16 scale rides along;
//   - dequant (dequant8) -> 4 MFMAs per (weight tile, token tile).
// Token tiles without a valid row are skipped (wave-uniform), so padding rows
// of a block cost neither MFMA work nor activation loads past the first
// check.  Summation order per output: chunks in K order, and inside a chunk
// the hardware's order over its 32 K -- independent of BM, NR, NW, so the
// output bits do not depend on the tile configuration.
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
// fp32 partial = topk_weight(slot) * acc stored per slot; launch_combine then
// sums a token's local slots in j order and rounds once.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

template <int MT, int NR, int NW, int ROUTE, int EPI>
__global__ __launch_bounds__(NW * kWave) void moe_gemm_kernel(const GemmParams p) {
  constexpr int BM = 16 * MT;
  constexpr int NTHR = NW * kWave;
  constexpr int XROW = kChunk + 8;                 // bf16 per staged row (272 B)
  constexpr int PIECES = BM * (kChunk / 8);        // 16-byte pieces per chunk
  static_assert(PIECES % NTHR == 0, "block rows must cover the workgroup's threads");
  constexpr int PPT = PIECES / NTHR;               // pieces per thread
  constexpr int ROWS_PER_PASS = NTHR / 16;         // staged rows covered by one piece index

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][XROW];
  __shared__ int s_row[BM];
  __shared__ int s_out[BM];
  __shared__ float s_w[EPI == kEpiWeighted ? BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
  const int mb = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x - mb * p.n_tiles;

  // ---------------------------------------------------------------- rows
  int expert;
  if constexpr (ROUTE == kRouteIndexed) {
    if (mb * BM >= *p.num_tokens_padded) return;
    expert = p.expert_ids[mb];
    if ((unsigned)expert >= (unsigned)p.E) return;   // -1 (unused block) or foreign id
    for (int i = tid; i < BM; i += NTHR) {
      const int s = p.sorted_ids[(int64_t)mb * BM + i];
      const bool v = (unsigned)s < (unsigned)p.sentinel;
      s_row[i] = v ? s / p.a_row_div : -1;
      s_out[i] = v ? s : -1;
      if constexpr (EPI == kEpiWeighted) s_w[i] = v ? p.slot_weight[s] : 0.f;
    }
  } else if constexpr (ROUTE == kRouteContiguous) {
    const int r0 = mb * BM;
    expert = p.m_indices[r0];
    if ((unsigned)expert >= (unsigned)p.E) return;   // padding block (-1) or foreign id
    for (int i = tid; i < BM; i += NTHR) {
      const bool v = p.m_indices[r0 + i] == expert;
      s_row[i] = v ? r0 + i : -1;
      s_out[i] = s_row[i];
    }
  } else {
    const int g = mb / p.blocks_per_group;
    const int r0 = (mb - g * p.blocks_per_group) * BM;
    const int cnt = min(p.masked_m[g], p.max_m);
    if (r0 >= cnt) return;
    expert = g;
    for (int i = tid; i < BM; i += NTHR) {
      const int r = r0 + i;
      const bool v = r < cnt;
      s_row[i] = v ? g * p.max_m + r : -1;
      s_out[i] = s_row[i];
    }
  }
  expert = __builtin_amdgcn_readfirstlane(expert);
  __syncthreads();

  // wave-uniform mask of token tiles holding at least one valid row
  uint32_t tmask = 0;
#pragma unroll
  for (int t = 0; t < MT; ++t)
    if (__ballot(s_row[16 * t + (lane & 15)] >= 0)) tmask |= 1u << t;

  // Activation staging.  Piece i of this thread is row (tid / 16) +
  // i * ROWS_PER_PASS, 16 bytes at column 8 * (tid % 16); the row's token
  // tile is wave-uniform, so inactive tiles are skipped with a scalar branch.
  // Padding rows read the block's first row (always valid) instead; their
  // LDS columns only feed output columns that are never stored.
  const int fallback_row = s_row[0];
  const int xcol = (tid & 15) * 8;
  const uint16_t* xsrc[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int row = (tid >> 4) + i * ROWS_PER_PASS;
    const int r = s_row[row];
    xsrc[i] = p.a + (int64_t)(r >= 0 ? r : fallback_row) * p.K + xcol;
  }
  auto piece_tile = [&](int i) { return (wave * kWave) / 256 + i * (ROWS_PER_PASS / 16); };

  // this wave's weight tiles (clamped so loads stay in bounds; tiles past N
  // compute throw-away values that are never stored)
  const int rt_base = nt * (NW * NR) + wave * NR;
  const int nr_valid = min(NR, p.NT - rt_base);
  const uint4* wptr[NR];
  const uint16_t* sptr[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rt = min(rt_base + r, p.NT - 1);
    const int64_t tile = ((int64_t)expert * p.NT + rt) * p.KC;
    wptr[r] = p.packed_w + tile * kWave + lane;
    sptr[r] = p.packed_s + tile * kWave + lane;
  }

  const int K = p.K;
  const int KC = p.KC;
  auto issue_x = [&](int c, uint4 (&xr)[PPT]) {
    // ragged K: a piece past K reads column 0 of its row instead (in bounds)
    // and is replaced by zeros when stored; no select here, so the load's
    // destination is never rewritten before it lands
    const int64_t off = (c * kChunk + xcol < K) ? (int64_t)c * kChunk : 0;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if ((tmask >> piece_tile(i)) & 1u) xr[i] = *reinterpret_cast<const uint4*>(xsrc[i] + off);
  };
  // `tail`: the chunk may be the ragged last one, pieces past K become zeros
  auto store_x = [&](int buf, int c, const uint4 (&xr)[PPT], bool tail) {
    const bool kin = !tail || c * kChunk + xcol < K;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if ((tmask >> piece_tile(i)) & 1u) {
        const uint4 v = kin ? xr[i] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&xs[buf][(tid >> 4) + i * ROWS_PER_PASS][xcol]) = v;
      }
  };
  auto issue_w = [&](int c, uint4 (&w)[NR], uint32_t (&sc)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      w[r] = wptr[r][(int64_t)c * kWave];
      sc[r] = sptr[r][(int64_t)c * kWave];
    }
  };

  f32x4_t acc[NR][MT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Two register sets: chunk c uses set c % 2.  At the top of chunk c the
  // activation pieces of chunk c + 2 are requested into the set whose data
  // (chunk c) already sits in LDS; weights and scales of chunk c + 2 are
  // requested as soon as chunk c's have been dequantised; chunk c + 1's
  // activations (requested one chunk earlier) are written to the other LDS
  // buffer before the barrier.  So every global load has about two chunk
  // times to land, and the barrier never waits on HBM.
  const DequantMasks masks = make_dequant_masks();
  uint4 xr[2][PPT];
  uint4 wr[2][NR];
  uint32_t sr[2][NR];

  issue_x(0, xr[0]);
  issue_w(0, wr[0], sr[0]);
  if (KC > 1) {
    issue_x(1, xr[1]);
    issue_w(1, wr[1], sr[1]);
  }
  store_x(0, 0, xr[0], true);
  __syncthreads();

  // one chunk; STEADY: chunks c + 1 and c + 2 exist and c + 1 is not the
  // ragged last chunk, so every prefetch and store is unconditional (no
  // register phis, no selects)
  auto chunk = [&](auto P_, auto STEADY_, int c) {
    constexpr int P = decltype(P_)::value;
    constexpr bool STEADY = decltype(STEADY_)::value;
    const bool pf = STEADY || c + 2 < KC;
    if (pf) issue_x(c + 2, xr[P]);
    bf16x8_t A[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float s = bf16_bits_to_float(sr[P][r] & 0xFFFFu);
      const float c0 = -1032.0f * s, s16 = 0.0625f * s, c1 = -72.0f * s;
      A[r][0] = dequant8(wr[P][r].x, s, c0, s16, c1, masks);
      A[r][1] = dequant8(wr[P][r].y, s, c0, s16, c1, masks);
      A[r][2] = dequant8(wr[P][r].z, s, c0, s16, c1, masks);
      A[r][3] = dequant8(wr[P][r].w, s, c0, s16, c1, masks);
    }
    if (pf) issue_w(c + 2, wr[P], sr[P]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t B[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if ((tmask >> t) & 1u)
          B[t] = *reinterpret_cast<const bf16x8_t*>(
              &xs[P][16 * t + (lane & 15)][32 * (lane >> 4) + 8 * j]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if ((tmask >> t) & 1u)
#pragma unroll
          for (int r = 0; r < NR; ++r)
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r][j], B[t], acc[r][t], 0, 0, 0);
    }
    if (STEADY || c + 1 < KC) store_x(P ^ 1, c + 1, xr[P ^ 1], !STEADY);
    __syncthreads();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using Steady = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  int c = 0;
  for (; c + 3 < KC; c += 2) {
    chunk(I0{}, Steady{}, c);
    chunk(I1{}, Steady{}, c + 1);
  }
  // the last one to three chunks (c is even here)
  if (c < KC) chunk(I0{}, Tail{}, c);
  if (c + 1 < KC) chunk(I1{}, Tail{}, c + 1);
  if (c + 2 < KC) chunk(I0{}, Tail{}, c + 2);

  // ---------------------------------------------------------------- epilogue
  // lane holds rows n = 16*tile + 4*(lane/16) + v (v = 0..3) of token
  // column lane % 16 of each token tile.
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r >= nr_valid) continue;
    const int n = (rt_base + r) * kRowTile + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (!((tmask >> t) & 1u)) continue;
      const int i = 16 * t + (lane & 15);
      const int orow = s_out[i];
      if (orow < 0) continue;
      const f32x4_t v = acc[r][t];
      if constexpr (EPI == kEpiStore) {
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + (int64_t)orow * p.N + n) = o;
      } else {
        const float w = s_w[i];
        float4 o = make_float4(w * v[0], w * v[1], w * v[2], w * v[3]);
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (int64_t)orow * p.N + n) = o;
      }
    }
  }
}

// Top-k combine: out[t, n] = bf16(sum over local j, in j order, of
// partial[t*k + j, n]); tokens with no local slot get 0.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial,
                                                      const int32_t* __restrict__ topk_ids,
                                                      int32_t T, int32_t topk, int32_t first,
                                                      int32_t E_loc, int32_t N,
                                                      uint16_t* __restrict__ out) {
  const int n8 = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * n8) return;
  const int64_t t = idx / n8;
  const int n = (int)(idx - t * n8) * 8;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const int e = topk_ids[t * topk + j] - first;
    if ((unsigned)e >= (unsigned)E_loc) continue;
    const float4* src = reinterpret_cast<const float4*>(partial + (t * topk + j) * (int64_t)N + n);
    const float4 u = src[0], v = src[1];
    a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w;
    a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
  }
  uint4 o;
  o.x = pack_bf16x2(a[0], a[1]);
  o.y = pack_bf16x2(a[2], a[3]);
  o.z = pack_bf16x2(a[4], a[5]);
  o.w = pack_bf16x2(a[6], a[7]);
  *reinterpret_cast<uint4*>(out + t * N + n) = o;
}

hipError_t launch_combine(const float* partial, const int32_t* topk_ids, int32_t T, int32_t topk,
                          int32_t first, int32_t E_loc, int32_t N, uint16_t* out,
                          hipStream_t stream) {
  const int64_t threads = (int64_t)T * (N / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     partial, topk_ids, T, topk, first, E_loc, N, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch
typedef void (*GemmKernel)(const GemmParams);

template <int MT, int NR, int NW>
static GemmKernel pick_kernel(int route, int epi) {
  if (route == kRouteIndexed)
    return epi == kEpiWeighted ? moe_gemm_kernel<MT, NR, NW, kRouteIndexed, kEpiWeighted>
                               : moe_gemm_kernel<MT, NR, NW, kRouteIndexed, kEpiStore>;
  if (epi != kEpiStore) return nullptr;
  if (route == kRouteContiguous) return moe_gemm_kernel<MT, NR, NW, kRouteContiguous, kEpiStore>;
  if (route == kRouteMasked) return moe_gemm_kernel<MT, NR, NW, kRouteMasked, kEpiStore>;
  return nullptr;
}

static GemmKernel find_kernel(int route, int epi, int m_tiles, int nr, int waves) {
  if (waves != 4) return nullptr;
#define W4A16_CASE(MT_, NR_) \
  if (m_tiles == MT_ && nr == NR_) return pick_kernel<MT_, NR_, 4>(route, epi);
  W4A16_CASE(1, 2) W4A16_CASE(2, 2) W4A16_CASE(4, 2) W4A16_CASE(8, 2)
  W4A16_CASE(1, 4) W4A16_CASE(2, 4) W4A16_CASE(4, 4) W4A16_CASE(8, 4)
#undef W4A16_CASE
  return nullptr;
}

bool gemm_config_supported(int route, int epilogue, int m_tiles, int nr, int waves) {
  return find_kernel(route, epilogue, m_tiles, nr, waves) != nullptr;
}

hipError_t launch_gemm(int route, int epilogue, int m_tiles, int nr, int waves,
                       const GemmParams& p, int64_t grid_blocks, hipStream_t stream) {
  GemmKernel k = find_kernel(route, epilogue, m_tiles, nr, waves);
  if (k == nullptr) return hipErrorInvalidValue;
  const int64_t grid = grid_blocks * p.n_tiles;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(waves * kWave), 0, stream, p);
  return hipGetLastError();
}

}  // namespace w4a16

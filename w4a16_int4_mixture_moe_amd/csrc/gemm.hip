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
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

template <int MT, int NR, int NW, int ROUTE, int EPI>
__global__ __launch_bounds__(NW * kWave) void moe_gemm_kernel(const GemmParams p) {
  constexpr int BM = 16 * MT;
  constexpr int NTHR = NW * kWave;
  constexpr int XROW = kChunk + 8;                 // bf16 per staged row (272 B)
  constexpr int PIECES = BM * (kChunk / 8);        // 16-byte pieces per chunk
  constexpr int PPT = (PIECES + NTHR - 1) / NTHR;  // pieces per thread

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][XROW];
  __shared__ int s_row[BM];
  __shared__ int s_out[BM];
  __shared__ float s_w[EPI == kEpiWeighted ? BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
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
  __syncthreads();

  // wave-uniform mask of token tiles holding at least one valid row
  uint32_t tmask = 0;
#pragma unroll
  for (int t = 0; t < MT; ++t)
    if (__ballot(s_row[16 * t + (lane & 15)] >= 0)) tmask |= 1u << t;

  // this thread's activation pieces: row pointer (nullptr = zero fill)
  const uint16_t* xsrc[PPT];
  int xrow[PPT], xcol[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int q = tid + i * NTHR;
    xrow[i] = q >> 4;
    xcol[i] = (q & 15) * 8;
    const int r = (q < PIECES) ? s_row[q >> 4] : -1;
    xsrc[i] = r >= 0 ? p.a + (int64_t)r * p.K + xcol[i] : nullptr;
  }

  // this wave's weight tiles (clamped for loads; tiles past N do no work)
  const int rt_base = nt * (NW * NR) + wave * NR;
  const int nr_valid = min(NR, p.NT - rt_base);
  const uint4* wptr[NR];
  const uint16_t* sptr[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rt = min(rt_base + r, p.NT - 1);
    const int64_t tile = (int64_t)expert * p.NT + rt;
    wptr[r] = p.packed_w + tile * p.KC * kWave + lane;
    sptr[r] = p.packed_s + (tile * kWave + lane) * p.SC;
  }

  const int K = p.K;
  const int KC = p.KC;
  auto load_x = [&](int c, uint4 (&xr)[PPT]) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int kk = c * kChunk + xcol[i];
      if (xsrc[i] != nullptr && kk < K)
        xr[i] = *reinterpret_cast<const uint4*>(xsrc[i] + (int64_t)c * kChunk);
      else
        xr[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf, const uint4 (&xr)[PPT]) {
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (tid + i * NTHR < PIECES)
        *reinterpret_cast<uint4*>(&xs[buf][xrow[i]][xcol[i]]) = xr[i];
  };

  f32x4_t acc[NR][MT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 xr[PPT];
  uint4 wcur[NR], wnxt[NR];
  uint32_t scur[NR], snxt[NR];

  load_x(0, xr);
  store_x(0, xr);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    wcur[r] = wptr[r][0];
    scur[r] = sptr[r][0];
  }
  __syncthreads();

  for (int c = 0; c < KC; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < KC;
    if (more) {
      load_x(c + 1, xr);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        wnxt[r] = wptr[r][(int64_t)(c + 1) * kWave];
        snxt[r] = sptr[r][c + 1];
      }
    }

    float sc[NR], c0[NR], s16[NR], c1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      sc[r] = bf16_bits_to_float(scur[r]);
      c0[r] = -1032.0f * sc[r];
      s16[r] = 0.0625f * sc[r];
      c1[r] = -72.0f * sc[r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t A[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t d = j == 0 ? wcur[r].x : j == 1 ? wcur[r].y : j == 2 ? wcur[r].z : wcur[r].w;
        A[r] = dequant8(d, sc[r], c0[r], s16[r], c1[r]);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (!((tmask >> t) & 1u)) continue;
        const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(
            &xs[buf][16 * t + (lane & 15)][32 * (lane >> 4) + 8 * j]);
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (r < nr_valid)
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B, acc[r][t], 0, 0, 0);
      }
    }

    if (more) store_x(buf ^ 1, xr);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      wcur[r] = wnxt[r];
      scur[r] = snxt[r];
    }
  }

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

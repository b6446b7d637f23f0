// A4W4 path for gfx950: MXFP4 activations x MXFP4 weights (FP4 E2M1 codes,
// one E8M0 scale per 32 consecutive K) in v_mfma_scale_f32_16x16x128_f8f6f4,
// routed like the W4A16 GEMM (indexed sorted_ids / expert_ids).
//
// The AMD Kimi K3 post ("Blick hinter die Kulissen der Kimi-K3-Optimierung",
// technical note "Experten-Routing und Praezision") describes A4W4 as the
// MoE activations going from eight to four bits while the weights stay
// 4-bit, with MXFP4 model weights on MI355X; the formats are those of the OCP
// Microscaling specification (E2M1 elements, E8M0 block scales).
//
// Operand layout of the scaled FP4 MFMA (16 x 16 x 128; checked on the
// device): lane l holds row l % 16 of its operand and the 32 consecutive K of
// block l / 16 of the 128, element i in nibble i of the lane's 128-bit value
// (low nibble first), and that block's E8M0 scale in byte 0 of its scale
// register.  A row of MXFP4 codes stored two per byte (element 2i in the low
// nibble) therefore already holds, for every lane, exactly the 16 bytes it
// needs: bytes 64 c + 16 (l / 16) of the row for K chunk c.  So
//   - activations need no staging: each lane loads its 16 bytes and its one
//     scale byte straight from the quantised rows (L2), no LDS, no barrier;
//   - weights are re-tiled once (mx_pack_kernel) to [E][N/16][K/128][64]
//     16-byte lane fragments plus [E][N/16][K/128][64] scale bytes, so a
//     wave's tile stream is contiguous;
//   - there is nothing to dequantise: one MFMA per (weight tile, token tile,
//     chunk).
// Activation quantisation (mx_quant_kernel) is the OCP conversion: shared
// exponent floor(log2 max|v|) - 2 clamped to E8M0's range (a zero block takes
// code 0), elements rounded to the nearest E2M1 value, ties to even, clamped
// at 6, sign from the input's sign bit (gfx950's FP4 conversion instruction
// does the rounding).
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_common.hpp"

namespace w4a16 {

// ------------------------------------------------------------ quantisation

// One thread per 32-element block: 64 bytes of bf16 in, 16 bytes of codes
// and one scale byte out.  slot_ids != NULL: row r is routed slot r and is
// converted only when slot_ids[r] names a local expert (first <= id <
// first + E_loc); other rows are left as they are.
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ x, int64_t blocks,
                                                        int32_t kb, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        const int32_t* __restrict__ slot_ids, int32_t first,
                                                        int32_t E_loc) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= blocks) return;
  const int64_t row = i / kb;
  if (slot_ids != nullptr && (unsigned)(slot_ids[row] - first) >= (unsigned)E_loc) return;
  const int b = (int)(i - row * kb);
  const uint4* src = reinterpret_cast<const uint4*>(x + row * (int64_t)kb * 32 + b * 32);
  uint32_t v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = src[q];
    v[4 * q] = u.x;
    v[4 * q + 1] = u.y;
    v[4 * q + 2] = u.z;
    v[4 * q + 3] = u.w;
  }
  // max |v| as a bit pattern: for finite bf16 the magnitude bits order like
  // the values, and only the exponent field is needed
  uint32_t amax = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) amax = max(amax, max(v[q] & 0x7FFFu, (v[q] >> 16) & 0x7FFFu));
  // floor(log2 amax) = exponent field - 127 for a normal amax; subnormal and
  // zero blocks clamp to code 0 either way, so code = max(field - 2, 0)
  const int field = (int)(amax >> 7);
  const uint32_t code = (uint32_t)max(field - 2, 0);
  const float inv = __builtin_bit_cast(float, (254u - code) << 23);    // 2^(127 - code), exact
  // y = v * 2^(127 - code) is exact (denormals are kept), and gfx950's
  // v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds a pair of floats to E2M1
  // exactly as the conversion asks: nearest, ties to the even code, clamped
  // at 6, sign kept for results that round to zero (checked on the device
  // against a CPU reference at every tie, past the clamp and at -0); the
  // byte selector packs four pairs into one word, element 2i in the low
  // nibble of byte i.
  // one pair of bf16 values (a packed word) into byte B of `word`
  auto pair = [&](auto b_, uint32_t word, uint32_t pv) {
    constexpr int B = decltype(b_)::value;
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, __builtin_bit_cast(float, pv << 16) * inv,
                                                    __builtin_bit_cast(float, pv & 0xFFFF0000u) * inv, 1.0f, B);
  };
  uint32_t out[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = pair(std::integral_constant<int, 0>{}, 0u, v[4 * w]);
    word = pair(std::integral_constant<int, 1>{}, word, v[4 * w + 1]);
    word = pair(std::integral_constant<int, 2>{}, word, v[4 * w + 2]);
    out[w] = pair(std::integral_constant<int, 3>{}, word, v[4 * w + 3]);
  }
  *reinterpret_cast<uint4*>(codes + i * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  scales[i] = (uint8_t)code;
}

hipError_t launch_mx_quant(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                           const int32_t* slot_ids, int32_t first, int32_t E_loc, hipStream_t stream) {
  const int64_t blocks = rows * (K / 32);
  if (blocks == 0) return hipSuccess;
  const int64_t grid = (blocks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, blocks, K / 32, codes,
                     scales, slot_ids, first, E_loc);
  return hipGetLastError();
}

// ------------------------------------------------------------ weight packing

// One thread per (expert, tile, chunk, lane): row n = 16 tile + lane % 16,
// block 4 chunk + lane / 16 -> the row's 16 code bytes of that block and its
// scale byte.
__global__ __launch_bounds__(256) void mx_pack_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ s,
                                                       int32_t E, int32_t N, int32_t K, int32_t gate_up,
                                                       uint4* __restrict__ pw, uint8_t* __restrict__ ps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KC = K / 128, NT = N / 16;
  const int64_t total = (int64_t)E * NT * KC * kWave;
  if (i >= total) return;
  const int lane = (int)(i % kWave);
  const int64_t q = i / kWave;
  const int c = (int)(q % KC);
  const int64_t et = q / KC;                    // expert * NT + tile
  const int t = (int)(et % NT);
  const int64_t e = et / NT;
  const int64_t n = e * N + source_row(t, lane & 15, N, gate_up);
  const int b = 4 * c + (lane >> 4);
  pw[i] = *reinterpret_cast<const uint4*>(w + n * (K / 2) + 16 * b);
  ps[i] = s[n * (K / 32) + b];
}

hipError_t launch_mx_pack(const uint8_t* w, const uint8_t* s, int32_t E, int32_t N, int32_t K, int32_t gate_up,
                          uint4* pw, uint8_t* ps, hipStream_t stream) {
  const int64_t total = (int64_t)E * (N / 16) * (K / 128) * kWave;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mx_pack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, s, E, N, K, gate_up, pw, ps);
  return hipGetLastError();
}

// ------------------------------------------------------------ GEMM

template <int MT>
struct MxSmem {
  int row[16 * MT];
  int out[16 * MT];
  float w[16 * MT];
};

// Blocks of four or eight token tiles stage each chunk's activation
// fragments once per workgroup in LDS (double buffered), laid out as the
// lanes read them: frag[buf][t][lane] is lane `lane`'s 16-byte operand of
// token tile t and sc[buf][t][lane] its scale byte.
template <int MT>
struct MxStagedSmem : MxSmem<MT> {
  u32x4_t frag[2][MT][kWave];
  uint32_t sc[2][MT][kWave];
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// 128 K of one weight tile (A) against 128 K of one token tile (B); only the
// low four dwords of each operand carry FP4 data
__device__ __forceinline__ f32x4_t mx_mfma(const u32x4_t& w, uint32_t ws, const u32x4_t& x, uint32_t xs,
                                           const f32x4_t& acc) {
  const i32x8_t A = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  const i32x8_t B = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, 0, (int)ws, 0, (int)xs);
}

__device__ __forceinline__ uint32_t gload_u8(gptr_t p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) uint8_t*>(p);
}

// acc += this wave's NR weight tiles x the block's first NA token tiles over
// all K chunks.  A ring of D stages, each holding one chunk's weight and
// activation fragments and scales: chunk c lives in stage c mod D and the
// stage is refilled with chunk c + D right after its MFMAs are issued, so
// every load has D - 1 chunks of MFMAs and loads ahead of its use.  Loads
// past the last chunk re-read the last chunk (never used), so every stage is
// filled unconditionally and in the same order on every path.
template <int MT, int NR, int NW, int D, int NA>
__device__ __forceinline__ void mx_mainloop(const GemmParams& p, const MxSmem<MT>& sm, int expert, int nt,
                                            f32x4_t (&acc)[NR][MT]) {
  static_assert(NA >= 1 && NA <= MT, "active token tiles");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int KC = p.KC;

  // activation rows: 16-byte fragment and scale byte of (row, block l/16)
  const gptr_t abase = uniform_ptr(p.a);
  const gptr_t asbase = uniform_ptr(p.a_scale);
  const uint32_t kb = (uint32_t)p.K / 2, ks = (uint32_t)p.K / 32;
  const int fallback_row = sm.row[0];
  uint32_t aoff[NA], asoff[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const int r = sm.row[16 * t + (lane & 15)];
    const uint32_t row = (uint32_t)(r >= 0 ? r : fallback_row);     // padding reads a valid row
    aoff[t] = row * kb + 16u * (uint32_t)(lane >> 4);
    asoff[t] = row * ks + (uint32_t)(lane >> 4);
  }
  // weight tiles (clamped: tiles past N compute values never stored)
  const int rt_base = nt * (NW * NR) + wave * NR;
  gptr_t wbase[NR], sbase[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rt = min(rt_base + r, p.NT - 1);
    const int64_t tile = (int64_t)expert * p.w_tiles + rt;
    wbase[r] = uniform_ptr(p.packed_w + tile * KC * kWave);
    sbase[r] = uniform_ptr(reinterpret_cast<const uint8_t*>(p.packed_s) + tile * KC * kWave);
  }
  const uint32_t woff = (uint32_t)lane * 16u;

  u32x4_t wr[D][NR], xr[D][NA];
  uint32_t wsr[D][NR], xsr[D][NA];
  auto issue = [&](int st, int c) {
    c = min(c, KC - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      wr[st][r] = gload_u32x4((wbase[r] + (int64_t)c * (kWave * 16)) + woff);
      wsr[st][r] = gload_u8((sbase[r] + (int64_t)c * kWave) + (uint32_t)lane);
    }
    const gptr_t ac = abase + (int64_t)c * 64, asc = asbase + (int64_t)c * 4;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      xr[st][t] = gload_u32x4(ac + aoff[t]);
      xsr[st][t] = gload_u8(asc + asoff[t]);
    }
  };
  auto compute = [&](int st) {
#pragma unroll
    for (int t = 0; t < NA; ++t)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r][t] = mx_mfma(wr[st][r], wsr[st][r], xr[st][t], xsr[st][t], acc[r][t]);
  };

#pragma unroll
  for (int st = 0; st < D; ++st) {
    __builtin_amdgcn_sched_barrier(0);
    issue(st, st);
  }
  __builtin_amdgcn_sched_barrier(0);
  int c = 0;
  for (; c + D <= KC; c += D) {
#pragma unroll
    for (int st = 0; st < D; ++st) {
      compute(st);
      // the refill stays after this stage's MFMAs, which read its registers
      __builtin_amdgcn_sched_barrier(0);
      issue(st, c + st + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int st = 0; st < D; ++st)
    if (c + st < KC) compute(st);
}

// The same product for blocks of four or eight token tiles: every wave of
// the workgroup multiplies the same activation fragments, so loading them
// per wave (as above) reads each one NW times through the L1; here the
// workgroup loads each fragment once per chunk into LDS (thread i takes
// fragments i, i + NW * 64, ...), and the waves read it from there.  Chunk c:
// request the fragments of chunk c + 1, multiply chunk c from LDS buffer
// c & 1 with weight stage c mod D, refill that stage with chunk c + D, store
// chunk c + 1 into the other buffer, barrier.
template <int MT, int NR, int NW, int D, int NA>
__device__ __forceinline__ void mx_mainloop_staged(const GemmParams& p, MxStagedSmem<MT>& sm, int expert, int nt,
                                                   f32x4_t (&acc)[NR][MT]) {
  static_assert(NA >= 1 && NA <= MT, "active token tiles");
  constexpr int NTHR = NW * kWave;
  constexpr int FPT = (NA * kWave + NTHR - 1) / NTHR;     // fragments per thread
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int KC = p.KC;

  const gptr_t abase = uniform_ptr(p.a);
  const gptr_t asbase = uniform_ptr(p.a_scale);
  const uint32_t kb = (uint32_t)p.K / 2, ks = (uint32_t)p.K / 32;
  const int fallback_row = sm.row[0];
  // fragment f = tid + i * NTHR: token tile f / 64, lane f % 64 of that tile;
  // wave-uniform whether it exists (NTHR is a multiple of 64)
  uint32_t goff[FPT], gsoff[FPT];
#pragma unroll
  for (int i = 0; i < FPT; ++i) {
    const int f = min(tid + i * NTHR, NA * kWave - 1);
    const int t = f / kWave, l = f % kWave;
    const int r = sm.row[16 * t + (l & 15)];
    const uint32_t row = (uint32_t)(r >= 0 ? r : fallback_row);
    goff[i] = row * kb + 16u * (uint32_t)(l >> 4);
    gsoff[i] = row * ks + (uint32_t)(l >> 4);
  }
  // every thread has all its fragments when NA * 64 is a multiple of the
  // workgroup size (known at compile time: no branch around the loads)
  constexpr bool ALL_ON = (NA * kWave) % NTHR == 0;
  auto frag_on = [&](int i) { return ALL_ON || i * NTHR + wave * kWave < NA * kWave; };

  const int rt_base = nt * (NW * NR) + wave * NR;
  gptr_t wbase[NR], sbase[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rt = min(rt_base + r, p.NT - 1);
    const int64_t tile = (int64_t)expert * p.w_tiles + rt;
    wbase[r] = uniform_ptr(p.packed_w + tile * KC * kWave);
    sbase[r] = uniform_ptr(reinterpret_cast<const uint8_t*>(p.packed_s) + tile * KC * kWave);
  }
  const uint32_t woff = (uint32_t)lane * 16u;

  u32x4_t wr[D][NR];
  uint32_t wsr[D][NR];
  u32x4_t xr[FPT];
  uint32_t xsr[FPT];
  auto issue_w = [&](int st, int c) {
    c = min(c, KC - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      wr[st][r] = gload_u32x4((wbase[r] + (int64_t)c * (kWave * 16)) + woff);
      wsr[st][r] = gload_u8((sbase[r] + (int64_t)c * kWave) + (uint32_t)lane);
    }
  };
  auto issue_x = [&](int c) {
    c = min(c, KC - 1);
    const gptr_t ac = abase + (int64_t)c * 64, asc = asbase + (int64_t)c * 4;
#pragma unroll
    for (int i = 0; i < FPT; ++i)
      if (frag_on(i)) {
        xr[i] = gload_u32x4(ac + goff[i]);
        xsr[i] = gload_u8(asc + gsoff[i]);
      }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FPT; ++i)
      if (frag_on(i)) {
        const int f = tid + i * NTHR;
        sm.frag[buf][f / kWave][f % kWave] = xr[i];
        sm.sc[buf][f / kWave][f % kWave] = xsr[i];
      }
  };
  auto compute = [&](int buf, int st) {
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const u32x4_t B = sm.frag[buf][t][lane];
      const uint32_t bs = sm.sc[buf][t][lane];
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r][t] = mx_mfma(wr[st][r], wsr[st][r], B, bs, acc[r][t]);
    }
  };

  issue_x(0);
#pragma unroll
  for (int st = 0; st < D; ++st) {
    __builtin_amdgcn_sched_barrier(0);
    issue_w(st, st);
  }
  __builtin_amdgcn_sched_barrier(0);
  store_x(0);
  __syncthreads();
  // STEADY: chunk c + 1 exists, so the store is unconditional and the loop
  // body is one basic block (a branch there lets the compiler sink the
  // MFMAs past the stores and the barrier into the next block)
  auto chunk = [&](auto steady_, int c, int st) {
    constexpr bool STEADY = decltype(steady_)::value;
    const int buf = c & 1;
    issue_x(c + 1);                          // clamped: past the end it re-reads the last chunk, never stored
    __builtin_amdgcn_sched_barrier(0);
    compute(buf, st);
    __builtin_amdgcn_sched_barrier(0);
    issue_w(st, c + D);
    __builtin_amdgcn_sched_barrier(0);
    if (STEADY || c + 1 < KC) store_x(buf ^ 1);
    __syncthreads();
  };
  using Steady = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  int c = 0;
  for (; c + D < KC; c += D) {
#pragma unroll
    for (int st = 0; st < D; ++st) chunk(Steady{}, c + st, st);
  }
#pragma unroll
  for (int st = 0; st < D; ++st)
    if (c + st < KC) chunk(Tail{}, c + st, st);
}

// Fused activation for the A4W4 chain: a wave's four packed tiles of a
// gate/up-interleaved weight (gate t, up t, gate t + 1, up t + 1, t even)
// hold output columns [16 t, 16 t + 32) of the activation, one whole MXFP4
// block per token.  Each lane forms bf16(silu(g) * u) from the bf16-rounded
// per-slot values (as the bf16 path's fused epilogue does) for its 8 of the
// token's 32 values; the four lanes of a token (lane % 16 equal) combine
// their maxima with two cross-lane shuffles; each lane rounds its 8 values
// with the FP4 conversion (the quantiser's steps) and stores its 4 code
// bytes, the first lane the block's scale.  Rows go to sorted positions.
template <int MT, int NR, int NW, typename Smem>
__device__ __forceinline__ void mx_silu_epilogue(const GemmParams& p, const Smem& sm, int nt, uint32_t tmask,
                                                 const f32x4_t (&acc)[NR][MT]) {
  static_assert(NR == 4, "four packed tiles per wave: one 32-column block");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rt_base = nt * (NW * NR) + wave * NR;
  if (rt_base >= p.NT) return;                    // NT % 4 == 0: all four tiles exist
  const int blk = rt_base / 4;                    // activation block of 32 columns
  const int g = lane >> 4;
  const int64_t row_bytes = p.N / 4;              // N / 2 activation columns, two per byte
  const int64_t row_scales = p.N / 64;
  uint8_t* codes = static_cast<uint8_t*>(p.out);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (!((tmask >> t) & 1u)) continue;           // wave-uniform
    float y[2][4];
    uint32_t amax = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t gu = pack_bf16x2(acc[2 * h][t][v], acc[2 * h + 1][t][v]);
        const uint32_t a = pack_bf16x2(silu_mul(bf16_bits_to_float(gu & 0xFFFFu), bf16_bits_to_float(gu >> 16)), 0.f);
        y[h][v] = bf16_bits_to_float(a & 0xFFFFu);
        amax = max(amax, a & 0x7FFFu);
      }
    // every lane takes part in the shuffles; padding rows are dropped below
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
    const uint32_t code = (uint32_t)max((int)(amax >> 7) - 2, 0);
    const float inv = __builtin_bit_cast(float, (254u - code) << 23);
    const int orow = sm.out[16 * t + (lane & 15)];
    if (orow < 0) continue;
    uint8_t* dst = codes + (int64_t)orow * row_bytes + 16 * blk + 2 * g;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[h][0] * inv, y[h][1] * inv, 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[h][2] * inv, y[h][3] * inv, 1.0f, 1);
      *reinterpret_cast<uint16_t*>(dst + 8 * h) = (uint16_t)w;
    }
    if (g == 0) p.out_scale[(int64_t)orow * row_scales + blk] = (uint8_t)code;
  }
}

template <int MT, int NR, int NW, int D, int EPI>
__global__ __launch_bounds__(NW * kWave) void mx_gemm_kernel(const GemmParams p) {
  constexpr bool STAGED = MT >= 4;
  __shared__ std::conditional_t<STAGED, MxStagedSmem<MT>, MxSmem<MT>> sm;
  int mb, nt;
  if (!block_of(p, blockIdx.x, p.n_tiles, mb, nt)) return;
  const int expert = setup_rows<MT, NW, kRouteIndexed, EPI>(p, mb, sm);
  if (expert < 0) return;
  __syncthreads();
  const uint32_t tmask = active_tiles<MT>(sm);
  // token tiles run: the active prefix, rounded up to an even count for
  // four- and eight-tile blocks (an extra tile of padding rows reads a valid
  // row and is never stored)
  auto go = [&](auto na) {
    constexpr int NA = decltype(na)::value;
    f32x4_t acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (STAGED)
      mx_mainloop_staged<MT, NR, NW, D, NA>(p, sm, expert, nt, acc);
    else
      mx_mainloop<MT, NR, NW, D, NA>(p, sm, expert, nt, acc);
    if constexpr (EPI == kEpiSiluMx)
      mx_silu_epilogue<MT, NR, NW>(p, sm, nt, (1u << NA) - 1u, acc);
    else
      epilogue<MT, NR, NW, EPI>(p, sm, nt, (1u << NA) - 1u, acc);
  };
  const int na = 32 - __clz(tmask);
  if constexpr (MT == 1) {
    go(std::integral_constant<int, 1>{});
  } else if constexpr (MT == 2) {
    if (na <= 1) go(std::integral_constant<int, 1>{});
    else go(std::integral_constant<int, 2>{});
  } else if constexpr (MT == 4) {
    if (na <= 2) go(std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, 4>{});
  } else {
    static_assert(MT == 8, "token tiles per block: 1, 2, 4 or 8");
    if (na <= 2) go(std::integral_constant<int, 2>{});
    else if (na <= 4) go(std::integral_constant<int, 4>{});
    else if (na <= 6) go(std::integral_constant<int, 6>{});
    else go(std::integral_constant<int, 8>{});
  }
}

// Few routed rows (block_m 16) and a grid too small for the machine: one
// 16-row weight tile per workgroup (four, gate t / up t / gate t+1 / up t+1,
// for the fused SiLU and quantisation epilogue, which needs one whole
// 32-column activation block per token), its NW waves splitting K (wave w
// takes chunks [w KC / NW, (w + 1) KC / NW)).  Each wave loads a batch of
// its chunks' weight and activation fragments and scale bytes straight into
// registers (the activation rows need no staging, as above), and the waves'
// partial sums meet in LDS, summed in wave order.  The W4A16 K-split tile's
// scheme, on the scaled FP4 MFMA.
template <int NW, int NT>
struct MxKwSmem : MxSmem<1> {
  f32x4_t red[NW][NT][kWave];
};

template <int NW, int EPI>
__global__ __launch_bounds__(NW * kWave) void mx_kwave_kernel(const GemmParams p) {
  constexpr int NT = EPI == kEpiSiluMx ? 4 : 1;   // weight tiles per workgroup
  constexpr int KB = 8 / NT;                       // chunks in flight per wave
  __shared__ MxKwSmem<NW, NT> sm;
  const int mb = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x - mb * p.n_tiles;
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
    sbase[r] = uniform_ptr(reinterpret_cast<const uint8_t*>(p.packed_s) + tile * KC * kWave) + lane;
  }
  // B operand: lane l supplies token row l % 16, block l / 16 of each chunk
  const int r16 = sm.row[lane & 15];
  const int64_t row = r16 >= 0 ? r16 : sm.row[0];  // padding reads a valid row, never stored
  const gptr_t abase = uniform_ptr(p.a) + row * (p.K / 2) + 16 * (lane >> 4);
  const gptr_t asbase = uniform_ptr(p.a_scale) + row * (p.K / 32) + (lane >> 4);
  f32x4_t acc[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int cb = c0; cb < c1; cb += KB) {
    u32x4_t w[KB][NT], x[KB];
    uint32_t ws[KB][NT], xs[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int c = min(cb + i, c1 - 1);          // past c1: a repeated load, not used
#pragma unroll
      for (int r = 0; r < NT; ++r) {
        w[i][r] = gload_u32x4(wbase[r] + (int64_t)c * (kWave * 16));
        ws[i][r] = gload_u8(sbase[r] + (int64_t)c * kWave);
      }
      x[i] = gload_u32x4(abase + (int64_t)c * 64);
      xs[i] = gload_u8(asbase + (int64_t)c * 4);
    }
    __builtin_amdgcn_sched_barrier(0);            // the whole batch in flight before the first MFMA
    // every MFMA of the batch is issued (a conditional one would let the
    // compiler sink its loads behind the branch, one round trip per chunk);
    // past c1 the activation operand is zero (FP4 has no Inf or NaN, so the
    // products are exact zeros)
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const u32x4_t xb = cb + i < c1 ? x[i] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < NT; ++r) acc[r] = mx_mfma(w[i][r], ws[i][r], xb, xs[i], acc[r]);
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
  if constexpr (EPI == kEpiSiluMx)
    mx_silu_epilogue<1, NT, 1>(p, sm, nt, 1u, tot);
  else
    epilogue<1, NT, 1, EPI>(p, sm, nt, 1u, tot);
}

typedef void (*MxKernel)(const GemmParams);

// N tiles of an A4W4 decode block kept together on one XCD (launch_mx_gemm)
constexpr int kMxXcdGroup = 8;

template <int MT, int NR, int NW, int D>
static MxKernel mx_pick(int epi) {
  if (epi == kEpiStore) return mx_gemm_kernel<MT, NR, NW, D, kEpiStore>;
  if (epi == kEpiWeighted) return mx_gemm_kernel<MT, NR, NW, D, kEpiWeighted>;
  if constexpr (NR == 4)
    if (epi == kEpiSiluMx) return mx_gemm_kernel<MT, NR, NW, D, kEpiSiluMx>;
  return nullptr;
}

// Built tile configurations (MT, NR, waves, stages): four waves; NR = 2 or 4
// weight tiles per wave; four stages for the decode tiles (MT <= 2), two for
// the larger blocks; and the K-split tile (MT 1, NR 1, kKwWaves waves).
static MxKernel find_mx_kernel(int epi, int m_tiles, int nr, int waves, int stages) {
  if (nr == 1) {  // the K-split tile: block_m 16, kKwWaves waves (stages do not apply)
    if (m_tiles != 1 || waves != kKwWaves) return nullptr;
    if (epi == kEpiStore) return mx_kwave_kernel<kKwWaves, kEpiStore>;
    if (epi == kEpiWeighted) return mx_kwave_kernel<kKwWaves, kEpiWeighted>;
    if (epi == kEpiSiluMx) return mx_kwave_kernel<kKwWaves, kEpiSiluMx>;
    return nullptr;
  }
#define W4A16_MX_CASE(MT_, NR_, NW_, D_) \
  if (m_tiles == MT_ && nr == NR_ && waves == NW_ && stages == D_) return mx_pick<MT_, NR_, NW_, D_>(epi);
  W4A16_MX_CASE(1, 2, 4, 4) W4A16_MX_CASE(2, 2, 4, 4) W4A16_MX_CASE(4, 2, 4, 2) W4A16_MX_CASE(8, 2, 4, 2)
  W4A16_MX_CASE(1, 4, 4, 4) W4A16_MX_CASE(2, 4, 4, 4) W4A16_MX_CASE(4, 4, 4, 2) W4A16_MX_CASE(8, 4, 4, 2)
#undef W4A16_MX_CASE
  return nullptr;
}

bool mx_gemm_config_supported(int epilogue, int m_tiles, int nr, int waves, int stages) {
  return find_mx_kernel(epilogue, m_tiles, nr, waves, stages) != nullptr;
}

hipError_t launch_mx_gemm(int epilogue, int m_tiles, int nr, int waves, int stages, const GemmParams& p,
                          hipStream_t stream) {
  const MxKernel k = find_mx_kernel(epilogue, m_tiles, nr, waves, stages);
  if (k == nullptr) return hipErrorInvalidValue;
  // decode tiles (at most 32 rows) of a block with 16 or more N tiles:
  // groups of kMxXcdGroup N tiles per XCD (block_of), so the block's
  // activation rows reach fewer L2s (measured on MI355X, A4W4 gate/up, same
  // run: EP8 decode 139.5 -> 138.3 us, K3-like decode 312.5 -> 309.8 us);
  // other tiles, and the K-split tile, block-major
  GemmParams q = p;
  q.xcd_group = nr > 1 && m_tiles <= 2 && p.n_tiles >= 2 * kMxXcdGroup && p.n_tiles % kMxXcdGroup == 0
                    ? kMxXcdGroup
                    : 0;
  const int64_t grid = grid_of(q, q.n_tiles);
  if (grid <= 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(waves * kWave), 0, stream, q);
  return hipGetLastError();
}

}  // namespace w4a16

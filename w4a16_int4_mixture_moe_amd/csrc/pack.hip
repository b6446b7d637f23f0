// INT4 weight packer: codes [E, N, K] (one per byte) and bf16 scales
// [E, N, K/32] into the MFMA-operand layout documented in w4a16_moe.h.
//
// The Chord W4A16 MoE post prepacks weights once at load (section "Indexed
// kernels") into a layout tied to its kernel profile; here a single layout,
// made of whole v_mfma_f32_16x16x32_bf16 operand fragments, serves every
// kernel variant: word j of lane l = 16 g + i of (tile, chunk c) holds row
// 16 tile + i, K = 128 c + 32 g + 8 j .. + 7, so one 16-byte load per lane
// brings one full scale group of one row.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

__global__ __launch_bounds__(256) void pack_w_kernel(const uint8_t* __restrict__ codes, int32_t N,
                                                     int32_t K, int32_t NT, int32_t KC,
                                                     int32_t gate_up, int64_t total_words,
                                                     uint32_t* __restrict__ packed_w) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_words) return;
  const int j = (int)(idx & 3);
  const int l = (int)((idx >> 2) & 63);
  int64_t rest = idx >> 8;
  const int c = (int)(rest % KC);
  rest /= KC;
  const int tile = (int)(rest % NT);
  const int64_t e = rest / NT;
  const int n = source_row(tile, l & 15, N, gate_up);
  const int k0 = c * kChunk + (l >> 4) * kGroup + j * 8;
  const uint8_t* src = codes + (e * N + n) * (int64_t)K;
  uint32_t word = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int kk = k0 + q;
    const uint32_t code = kk < K ? (uint32_t)(src[kk] & 0xF) : 8u;
    word |= code << (4 * (q >> 1) + 16 * (q & 1));
  }
  packed_w[idx] = word;
}

__global__ __launch_bounds__(256) void pack_s_kernel(const uint16_t* __restrict__ scales,
                                                     int32_t N, int32_t K, int32_t NT,
                                                     int32_t KC, int32_t gate_up, int64_t total,
                                                     uint32_t* __restrict__ packed_s) {
  // output word index = ((e * NT + tile) * KC2 + m) * 64 + lane; the word
  // holds the lane's scale for chunk 2m (low half) and 2m + 1 (high half)
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int KC2 = (KC + 1) / 2;
  const int l = (int)(idx & 63);
  int64_t rest = idx >> 6;
  const int m = (int)(rest % KC2);
  rest /= KC2;
  const int tile = (int)(rest % NT);
  const int64_t e = rest / NT;
  const int n = source_row(tile, l & 15, N, gate_up);
  const int G = K / kGroup;
  const uint16_t* row = scales + (e * N + n) * (int64_t)G;
  const int g0 = 4 * (2 * m) + (l >> 4), g1 = g0 + 4;
  const uint32_t lo = g0 < G ? row[g0] : 0u, hi = g1 < G ? row[g1] : 0u;
  packed_s[idx] = lo | (hi << 16);
}

hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, int32_t E, int32_t N,
                       int32_t K, int32_t KC, int32_t gate_up, uint32_t* packed_w,
                       uint32_t* packed_s, hipStream_t stream) {
  const int32_t NT = N / kRowTile;
  const int64_t words = (int64_t)E * NT * KC * 256;
  const int64_t sents = (int64_t)E * NT * ((KC + 1) / 2) * 64;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                     codes, N, K, NT, KC, gate_up, words, packed_w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(pack_s_kernel, dim3((unsigned)((sents + 255) / 256)), dim3(256), 0, stream,
                     scales, N, K, NT, KC, gate_up, sents, packed_s);
  return hipGetLastError();
}

}  // namespace w4a16

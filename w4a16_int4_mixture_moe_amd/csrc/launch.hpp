// Host-side launchers of the gfx950 kernels (internal to the library; the
// public entry points in api.cpp validate arguments before calling these).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// ---- routing align (align.hip)
hipError_t launch_align(const int32_t* topk_ids, int32_t total_slots, int32_t first, int32_t E_loc,
                        int32_t block_m, int32_t* sorted_ids, int32_t* expert_ids,
                        int32_t* num_tokens_padded, int64_t capacity, hipStream_t stream);

// ---- packer (pack.hip)
hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, int32_t E, int32_t N,
                       int32_t K, int32_t KC, int32_t gate_up, uint32_t* packed_w,
                       uint32_t* packed_s, hipStream_t stream);

// ---- GEMM (gemm.hip)
enum RouteKind : int { kRouteIndexed = 0, kRouteContiguous = 1, kRouteMasked = 2 };
// kEpiSilu: gate/up pairs of tiles -> bf16(silu(g) * u) at sorted positions;
// kEpiSiluMx (MXFP4 kernels): the same activation quantised to MXFP4 rows
enum EpilogueKind : int { kEpiStore = 0, kEpiWeighted = 1, kEpiSilu = 2, kEpiSiluMx = 3 };

struct GemmParams {
  const uint4* packed_w;        // [E][NT][KC][64][4 words]
  const uint32_t* packed_s;     // [E][NT][KC2][64], bf16 scale pairs (MXFP4: [E][NT][KC][64] E8M0 bytes)
  const uint16_t* a;            // bf16 activations, row stride K (MXFP4: E2M1 codes, two per byte, row stride K/2 bytes)
  const uint8_t* a_scale;       // MXFP4 activations: E8M0 scales, row stride K/32 bytes
  int32_t E, N, K, NT, KC;      // N, NT: the output columns (16-row weight tiles) this call covers
  int32_t w_tiles;              // 16-row tiles per expert in packed_w / packed_s (>= NT: a call may
                                // cover a column range, packed_w / packed_s then point at its first tile)
  int32_t n_tiles;              // workgroup tiles along N
  int32_t xcd_group;            // 1: a block's N tiles run on one XCD (see block_of), else block-major
  // indexed
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  int32_t expert_shift;         // log2(routing block_m / tile rows): tile b reads expert_ids[b >> shift]
  const int32_t* num_tokens_padded;
  int32_t sentinel;             // T * topk
  int32_t a_row_div;            // topk (rows per token), 1 (rows per slot), 0 (rows per sorted position)
  int32_t gated;                // packed tiles alternate gate / up (output columns remapped)
  const float* slot_weight;     // weighted epilogue: topk weights, one per slot
  // weighted epilogue, optional (token_local != nullptr): local slots per
  // token (saturated at 255); the rows of tokens with exactly one local slot
  // are stored as bf16(w * acc) to direct_out[token * direct_ld + column]
  // instead of as fp32 partials (their combine is that one term)
  const uint8_t* token_local;
  int32_t topk;
  uint16_t* direct_out;
  int32_t direct_ld;
  // contiguous
  const int32_t* m_indices;
  // masked
  const int32_t* masked_m;
  int32_t max_m;
  int32_t blocks_per_group;
  // output: bf16 [rows][N] (store) or fp32 [rows][N] (weighted); kEpiSiluMx:
  // E2M1 codes [rows][N/4] bytes (N/2 activation columns, two per byte)
  void* out;
  uint8_t* out_scale;           // kEpiSiluMx: E8M0 scales [rows][N/64]
  // routed blocks (all kinds; for indexed the live count comes from
  // num_tokens_padded on the device, this is the capacity bound)
  int32_t grid_blocks;
  // stream-K: fp32 partial tiles, two slots per persistent workgroup
  float* sk_partial;
  // split-K: `split` workgroups per tile, each over an equal share of the K
  // chunks; tiles with index below split_tiles leave their fp32 slices in
  // split_partial ([tile][slice][NR * MT * threads] float4) and count their
  // arrival in split_count[tile] (zero at entry, reset to zero by the last
  // arriver); tiles past split_tiles run whole in their slice-0 workgroup
  int32_t split;
  int32_t split_tiles;
  float* split_partial;
  uint32_t* split_count;
};

// XCD-grouped block order (block_of in tile_common.hpp) for blocks with
// 2 .. kXcdGroupMaxTiles N tiles (or N-tile groups) and K not split.
constexpr int kXcdGroupMaxTiles = 4;
// N tiles of a decode block kept together on one XCD (see launch_gemm)
constexpr int kXcdDecodeGroup = 16;
// waves of the K-split tile (nr = 1: one 16-row weight tile per workgroup,
// its waves splitting K; moe_gemm_kwave_kernel)
constexpr int kKwWaves = 8;
int xcd_group_for(int split, int per_block);

// m_tiles: 16-row token tiles per block (block_m / 16); nr: 16-row weight
// tiles per wave; waves: waves per workgroup; stages: chunks of weights in
// flight per wave (2 or 3).
bool gemm_config_supported(int route, int epilogue, int m_tiles, int nr, int waves, int stages);

// One workgroup per (routed block, N tile), full K each; with p.split > 1,
// p.split workgroups per tile, each over a share of K, reduced in slice order.
hipError_t launch_gemm(int route, int epilogue, int m_tiles, int nr, int waves, int stages,
                       const GemmParams& p, hipStream_t stream);

// The prefill tiles (prefill.hip): 128 or 256 routed rows x 256 weight rows
// per workgroup, activations staged by LDS-DMA.  Serve the (m_tiles 8, nr 4,
// waves 4) and (m_tiles 16, nr 2, waves 8) configurations with stages 2 when
// K is a multiple of 128 and K is not split; launch_gemm dispatches to them.
bool prefill_applies(int route, int epilogue, int m_tiles, int nr, int waves, int stages, const GemmParams& p);
hipError_t launch_gemm_prefill(int route, int epilogue, int m_tiles, int nr, int waves, const GemmParams& p,
                               hipStream_t stream);

// Stream-K: `workgroups` persistent workgroups each take an equal contiguous
// range of (tile, 128-K chunk) units; tiles cut by a range boundary leave
// fp32 partials in p.sk_partial that a fix-up kernel sums in range order.
hipError_t launch_gemm_streamk(int route, int epilogue, int m_tiles, int nr, int waves, int stages,
                               const GemmParams& p, int workgroups, hipStream_t stream);

// Persistent workgroups for stream-K on the current device (resident
// workgroups per CU x CUs), and the partial-tile bytes they need.
int streamk_workgroups(int route, int epilogue, int m_tiles, int nr, int waves, int stages);
size_t streamk_partial_bytes(int m_tiles, int nr, int waves, int workgroups);

// Bytes of one K slice of one tile in split_partial.
size_t split_slice_bytes(int m_tiles, int nr, int waves);

// ---- zero fill of 32-bit words, graph-capturable (gemm.hip)
hipError_t launch_zero_words(uint32_t* p, int64_t words, hipStream_t stream);

// ---- combine of weighted per-slot partials (gemm.hip): partial [T*topk][cols]
// fp32 -> out[t * ldo + c] bf16 for c < cols; token_local != nullptr: tokens
// with exactly one local slot are skipped (the GEMM stored them)
hipError_t launch_combine(const float* partial, const int32_t* topk_ids, int32_t T, int32_t topk,
                          int32_t first, int32_t E_loc, int32_t cols, uint16_t* out, int32_t ldo,
                          const uint8_t* token_local, hipStream_t stream);
// local slots of each token: cnt[t] = min(#{j : first <= ids[t*topk + j] < first + E_loc}, 255)
hipError_t launch_token_local(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t first, int32_t E_loc,
                              uint8_t* cnt, hipStream_t stream);

// ---- A4W4: MXFP4 activations x MXFP4 weights (mx.hip)
// bf16 [rows][K] -> E2M1 codes [rows][K/2] (two per byte, low nibble first)
// and E8M0 scales [rows][K/32]; K % 32 == 0.  slot_ids != NULL: only rows r
// with first <= slot_ids[r] < first + E_loc are converted.
hipError_t launch_mx_quant(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                           const int32_t* slot_ids, int32_t first, int32_t E_loc, hipStream_t stream);
// codes [E][N][K/2] + scales [E][N][K/32] -> packed [E][N/16][K/128][64]
// 16-byte fragments + [E][N/16][K/128][64] scale bytes; K % 128 == 0.
// gate_up: tiles of the gate rows [0, N/2) and up rows [N/2, N) alternate.
hipError_t launch_mx_pack(const uint8_t* w, const uint8_t* s, int32_t E, int32_t N, int32_t K, int32_t gate_up,
                          uint4* pw, uint8_t* ps, hipStream_t stream);
// Indexed routing only; epilogue kEpiStore, kEpiWeighted or kEpiSiluMx.
bool mx_gemm_config_supported(int epilogue, int m_tiles, int nr, int waves, int stages);
hipError_t launch_mx_gemm(int epilogue, int m_tiles, int nr, int waves, int stages, const GemmParams& p,
                          hipStream_t stream);

}  // namespace w4a16

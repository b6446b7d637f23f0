// C ABI of the W4A16 MoE expert GEMM (declared in include/w4a16_moe.h):
// argument validation, tile-configuration selection and kernel dispatch.
// Every check runs on the host before anything is enqueued; no entry point
// allocates device memory.
#include "w4a16_moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <random>
#include <string>
#include <tuple>
#include <vector>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

w4a16_status fail(w4a16_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

w4a16_status hip_fail(hipError_t e, const char* what) {
  return fail(W4A16_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

uint64_t desc_checksum(const w4a16_weight_desc& d) {
  // FNV-1a over every field before `check`
  const unsigned char* b = reinterpret_cast<const unsigned char*>(&d);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < offsetof(w4a16_weight_desc, check); ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

w4a16_weight_desc make_desc(int32_t E, int32_t N, int32_t K, int32_t flags) {
  w4a16_weight_desc d;
  std::memset(&d, 0, sizeof d);
  d.magic = W4A16_DESC_MAGIC;
  d.version = W4A16_DESC_VERSION;
  d.E = E;
  d.N = N;
  d.K = K;
  d.flags = flags;
  d.K_pad = (int32_t)round_up(K, 128);
  const int64_t KC = d.K_pad / 128;
  d.chunks = (int32_t)KC;
  d.group = 32;
  const int64_t NT = N / 16;
  d.w_bytes = (uint64_t)E * NT * KC * 1024;
  d.s_bytes = (flags & W4A16_DESC_MXFP4) ? (uint64_t)E * NT * KC * 64          // one E8M0 byte per lane
                                         : (uint64_t)E * NT * ((KC + 1) / 2) * 64 * 4;
  d.check = desc_checksum(d);
  return d;
}

w4a16_status check_shape(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_ARG, "E, N, K must be positive (got %d, %d, %d)", E, N, K);
  if (K % 32) return fail(W4A16_ERR_SHAPE, "K = %d is not a multiple of the scale group 32", K);
  if (N % 16) return fail(W4A16_ERR_SHAPE, "N = %d is not a multiple of 16", N);
  if ((int64_t)K * 2 > INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "K = %d too large", K);
  return W4A16_OK;
}

w4a16_status check_desc(const w4a16_weight_desc* d) {
  if (d == nullptr) return fail(W4A16_ERR_ARG, "weight descriptor is NULL");
  if (d->magic != W4A16_DESC_MAGIC || d->version != W4A16_DESC_VERSION)
    return fail(W4A16_ERR_LAYOUT, "weight descriptor has a wrong magic/version (not from w4a16_weight_desc_init?)");
  if (d->check != desc_checksum(*d)) return fail(W4A16_ERR_LAYOUT, "weight descriptor checksum mismatch (corrupted)");
  w4a16_status st = check_shape(d->E, d->N, d->K);
  if (st != W4A16_OK) return fail(W4A16_ERR_LAYOUT, "weight descriptor shape invalid: %s", g_last_error.c_str());
  const bool flags_ok = d->flags == 0 || (d->flags == W4A16_DESC_GATE_UP && d->N % 32 == 0) ||
                        (d->flags == W4A16_DESC_MXFP4 && d->K % 128 == 0) ||
                        (d->flags == (W4A16_DESC_MXFP4 | W4A16_DESC_GATE_UP) && d->K % 128 == 0 && d->N % 64 == 0);
  if (!flags_ok) return fail(W4A16_ERR_LAYOUT, "weight descriptor flags invalid");
  const w4a16_weight_desc ref = make_desc(d->E, d->N, d->K, d->flags);
  if (std::memcmp(&ref, d, sizeof ref) != 0) return fail(W4A16_ERR_LAYOUT, "weight descriptor fields inconsistent");
  return W4A16_OK;
}

// An INT4 (W4A16) weight descriptor: valid, and not an MXFP4 one.
w4a16_status check_int4_desc(const w4a16_weight_desc* d) {
  w4a16_status st = check_desc(d);
  if (st != W4A16_OK) return st;
  if (d->flags & W4A16_DESC_MXFP4)
    return fail(W4A16_ERR_LAYOUT, "an MXFP4 weight descriptor is used by the w4a16_mxfp4_* calls only");
  return W4A16_OK;
}

w4a16_status check_mx_desc(const w4a16_weight_desc* d) {
  w4a16_status st = check_desc(d);
  if (st != W4A16_OK) return st;
  if (!(d->flags & W4A16_DESC_MXFP4))
    return fail(W4A16_ERR_LAYOUT, "not an MXFP4 weight descriptor (use w4a16_mxfp4_weight_desc_init)");
  return W4A16_OK;
}

bool valid_block_m(int32_t bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

// ---------------------------------------------------------------- selection
//
// Chord W4A16 MoE post, section "H200 prefill and TP8": block_m is chosen from
// tokens per expert tok_e = routed rows / experts; below about 80 a search
// minimises the total number of blocks on sampled routing, above it the
// padded expert rows are fitted under a maximum block_m; K is split only
// where the plain grid leaves the machine underfilled.  On gfx950 the kernel
// skips 16-row token tiles that hold no valid row, so MFMA work follows valid
// rows whatever block_m is, while every extra block of an expert re-reads and
// re-dequantises its weights.  So:
//   - decode side (tok_e < kPrefillTokE): sample per-expert counts, pick the
//     smallest block_m whose total block count is within 2 % of the minimum
//     (smaller blocks keep fewer accumulators live and more waves resident);
//   - prefill side: the padded expert rows fitted under the largest tile
//     (fit_padded_rows: the fewest blocks per expert of at most that many
//     rows, each block's rows rounded up to 16), rounded up to a built tile:
//     128 rows, or 256 where K allows the 256-row prefill tile;
//   - split_k doubles while the doubled grid stays within 4/5 of one round
//     of resident workgroups and each slice keeps kMinSliceChunks chunks
//     (measured on MI355X, gate/up K = 7168: TP8 T = 1, 32 tiles, 32.3 us
//     unsplit, 13.1 us at 8 slices; EP32 decode, 384 tiles, 47.7 -> 40.2 us
//     at 2, slower at 4; EP16 decode, 768 tiles, and TP8 T = 16, 456 tiles,
//     no faster split).
// The machine model is fixed (256 CUs, resident workgroups per CU of each
// tile from its register use), so the choice is deterministic and available
// without a device.
constexpr double kPrefillTokE = 48.0;
// Routed rows per expert from which the routing takes 256-row blocks: both
// projections run the 256-row prefill tile (an expert of up to 256 rows
// streams its weights once).  Measured on MI355X at 171 rows per expert
// (T = 8192, top-8 of 384, Zipf-skewed), against 128-row blocks: gate/up
// EP8 595 -> 544 us, EP16 384 -> 356 us, EP32 180 -> 144 us; on the
// software-pipelined 256-row tile the down + combine against 128-row tiles
// on the same routing: EP8 352 -> 344 us, EP16 221 -> 210 us, EP32 135 ->
// 133 us.  Grouped masked calls (up to 512 rows per group) were 20 % slower
// on it, so they keep 128.
constexpr double kWideTokE = 128.0;

// Rows per block when an expert's tok_e rows are split into the fewest
// blocks of at most max_rows rows, each rounded up to the 16-row token tile
// (the post's padded-rows fit, section "H200 prefill and TP8").
int fit_padded_rows(double tok_e, int max_rows) {
  const int rows = std::max(1, (int)std::ceil(tok_e));
  const int blocks = (rows + max_rows - 1) / max_rows;
  return (int)round_up((rows + blocks - 1) / blocks, 16);
}
// A4W4: above this many rows per expert the MXFP4 GEMM takes 64-row blocks
// where the W4A16 rule gives 128 (measured on MI355X, step time: EP8 / EP16
// prefill shares 5 % / 9 % faster at 64; at 85 rows per expert, TP8 T = 4096,
// 128 stays 6 % faster, since 64 would split most experts into two blocks
// that each stream the expert's weights).
constexpr double kMxHalfTileTokE = 128.0;
constexpr int kCUs = 256;
constexpr int kMinSliceChunks = 4;    // 512 K elements per slice at least
constexpr int kMaxSplit = 16;
// split-K slices are kept for at most this many tiles per call (a tile past
// it runs whole in one workgroup); the selector splits only grids below one
// round of resident workgroups, so real grids stay well under it
constexpr int kSplitTileCap = 2048;

std::mutex g_cache_mu;
typedef std::tuple<int, int, int, int, int, int, int, int> SelectKey;
std::map<SelectKey, w4a16_config> g_cache;

int64_t sampled_blocks(const std::vector<int>& counts, int bm) {
  int64_t b = 0;
  for (int c : counts) b += (c + bm - 1) / bm;
  return b;
}

// Resident workgroups per CU of the one-workgroup-per-tile kernel with this
// tile (four waves; register use of the gfx950 build: 16- and 32-row blocks
// fit four workgroups per CU, 64-row blocks three, 128-row blocks two; the
// eight-wave 256-row tile one).
int resident_per_cu(int block_m) { return block_m <= 32 ? 4 : block_m == 64 ? 3 : block_m == 128 ? 2 : 1; }

int n_tiles_of(int N, int nr, int waves) {
  const int tiles_per_wg = nr == 1 ? 1 : nr * waves;   // nr 1: the waves split K, not N
  return (N / 16 + tiles_per_wg - 1) / tiles_per_wg;
}

int chunks_of(int K) { return (K + 127) / 128; }

// split_k for a grid of `tiles` one-workgroup tiles over K
int choose_split(int64_t tiles, int block_m, int K) {
  const int64_t resident = (int64_t)kCUs * resident_per_cu(block_m);
  const int KC = chunks_of(K);
  int split = 1;
  while (split < kMaxSplit && tiles * split * 2 * 5 <= resident * 4 && KC / (2 * split) >= kMinSliceChunks)
    split *= 2;
  return split;
}

// per-expert counts of a seeded multinomial sample of the routing: each of
// T * topk slots lands on one of E_glob experts uniformly; the local ones kept
std::vector<int> sampled_counts(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc) {
  std::mt19937 rng(12345u);
  std::vector<int> counts(std::max(E_loc, 1), 0);
  std::binomial_distribution<int> bin(std::max(T, 0) * std::max(topk, 1), 1.0 / std::max(E_glob, 1));
  for (int e = 0; e < E_loc; ++e) counts[e] = bin(rng);
  return counts;
}

// Indexed config; block_m chosen by the tok_e rule, or, when the routing
// buffers already fix their block_m (force_block_m > 0), that block_m (a
// 256-row routing with K not a multiple of 128: the 128-row tile).
w4a16_config select_indexed(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N, int32_t K,
                            int32_t force_block_m) {
  w4a16_config c{};
  c.kind = W4A16_ROUTE_INDEXED;
  c.waves = 4;
  c.stages = 2;
  c.nr = 2;  // measured: two 16-row weight tiles per wave beat four at 128 rows
  const double tok_e = (double)T * topk / std::max(E_glob, 1);
  const std::vector<int> counts = sampled_counts(T, topk, E_glob, E_loc);
  if (force_block_m > 0) {
    c.block_m = force_block_m;
    if (c.block_m == 256 && K % 128) c.block_m = 128;
  } else if (tok_e >= kPrefillTokE) {
    // the fitted rows rounded up to a built tile: above 128 rows the 256-row
    // tile, whose lower bound is kWideTokE (the fit exceeds 128 rows exactly
    // when tok_e does, up to 256)
    const int max_rows = K % 128 == 0 ? 256 : 128;
    c.block_m = fit_padded_rows(tok_e, max_rows) > 128 && tok_e >= kWideTokE ? 256 : 128;
  } else {
    const int cands[3] = {16, 32, 64};
    int64_t best = INT64_MAX;
    for (int bm : cands) best = std::min(best, sampled_blocks(counts, bm));
    c.block_m = 64;
    for (int bm : cands)
      if (sampled_blocks(counts, bm) * 100 <= best * 102) {
        c.block_m = bm;
        break;
      }
  }
  // 128-row blocks with K a multiple of 128: the prefill tile (four weight
  // tiles per wave, LDS-DMA staging); measured on MI355X against two tiles
  // per wave: EP8 prefill gate/up 629 -> 604 us, down 413 -> 401 us, TP8
  // T = 4096 gate/up 378 -> 362 us, down 637 -> 616 us, bit-identical outputs
  if (c.block_m == 128 && K % 128 == 0) c.nr = 4;
  // 256-row blocks (only when the routing fixes them): the wide prefill tile,
  // two weight tiles per wave over eight waves, unsplit
  if (c.block_m == 256) {
    c.waves = 8;
    c.split_k = 1;
    return c;
  }
  const int64_t tiles = sampled_blocks(counts, c.block_m) * n_tiles_of(N, c.nr, c.waves);
  c.split_k = choose_split(tiles, c.block_m, K);
  // 16-row blocks over a short K (at most two chunks: the down projection of
  // a TP8 share): four weight tiles per wave spread each block's staging over
  // twice the weight rows, while the grid keeps two workgroups per CU.
  // Measured on MI355X, TP8 down (N = 7168, K = 256): T = 16 35.9 -> 34.3 us,
  // T = 128 107.5 -> 99.6 us; T = 1 (252 workgroups) 10.5 against 11.0 us.
  if (c.block_m == 16 && K <= 256 && c.split_k == 1 &&
      sampled_blocks(counts, 16) * n_tiles_of(N, 4, c.waves) >= 2 * (int64_t)kCUs)
    c.nr = 4;
  // A grid this small would split K four or more ways: one 16-row weight
  // tile per workgroup with its waves splitting K instead (partials meet in
  // LDS, no global reduction).  Measured on MI355X, TP8 gate/up (N = 512,
  // K = 7168): T = 1 14.6 -> 9.0 us (K split 8 ways -> waves splitting K);
  // T = 16 (split 2) 49 against 79 us and T = 128 146 against 288 us, so
  // only where the split would reach 4.
  if (c.block_m == 16 && c.split_k >= 4 && K % 128 == 0) {
    c.nr = 1;
    c.waves = w4a16::kKwWaves;
    c.split_k = 1;
  }
  return c;
}

// Contiguous grouped layout: 128-row blocks when their grid fills the
// machine, else 64 (post, section "Grouped SM90 kernels": BM128 for large
// grids, BM64 for small concatenated problems so M tiles still fill).
w4a16_config select_contiguous(int64_t m_rows, int32_t E, int32_t N, int32_t K) {
  (void)E;
  w4a16_config c{};
  c.kind = W4A16_ROUTE_CONTIGUOUS;
  c.nr = 2;
  c.waves = 4;
  c.stages = 2;
  const int64_t grid128 = (m_rows + 127) / 128 * n_tiles_of(N, K % 128 == 0 ? 4 : 2, c.waves);
  c.block_m = grid128 >= (int64_t)kCUs * resident_per_cu(128) ? 128 : 64;
  if (c.block_m == 128 && K % 128 == 0) c.nr = 4;   // the prefill tile
  c.split_k = choose_split((m_rows + c.block_m - 1) / c.block_m * n_tiles_of(N, c.nr, c.waves), c.block_m, K);
  return c;
}

// Masked grouped layout (post, section "Grouped SM90 kernels"): a group that
// spills into a second M tile re-reads all of K, so deep-K projections cover
// about 1.3 x expected_m rows; short-K ones take the leaner
// ceil(1.25 x expected_m, 8).  Rounded up to a built block (at most 128).
// Buffered K follows latency: 512 elements (four 128-K stages) for decode-size
// blocks, two stages for larger ones.
w4a16_config select_masked(int32_t max_m, int32_t E, int32_t N, int32_t K, int32_t expected_m) {
  w4a16_config c{};
  c.kind = W4A16_ROUTE_MASKED;
  c.nr = 2;
  c.waves = 4;
  const int em = std::max(1, std::min(expected_m, max_m));
  const int want = K >= 4096 ? (int)std::ceil(1.3 * em) : (int)round_up((int64_t)std::ceil(1.25 * em), 8);
  c.block_m = want <= 16 ? 16 : want <= 32 ? 32 : want <= 64 ? 64 : 128;
  c.stages = c.block_m <= 32 ? 4 : 2;
  if (c.block_m == 128 && K % 128 == 0) c.nr = 4;   // the prefill tile
  const int64_t blocks = (int64_t)E * ((std::min(em, max_m) + c.block_m - 1) / c.block_m);
  c.split_k = choose_split(blocks * n_tiles_of(N, c.nr, c.waves), c.block_m, K);
  return c;
}

const char* env_str(const char* name) {
  const char* v = std::getenv(name);
  return (v && *v) ? v : nullptr;
}

const char* const kOverrideVars[5] = {"W4A16_BLOCK_M", "W4A16_NR", "W4A16_WAVES", "W4A16_SPLIT_K", "W4A16_STAGES"};

// W4A16_BLOCK_M / W4A16_NR / W4A16_WAVES / W4A16_SPLIT_K / W4A16_STAGES override the indexed selector
// (read on every call; the memoised result is the selector's, overrides are applied on top).
// block_m is left alone when the routing already fixes it.
void apply_env_overrides(w4a16_config* c, bool block_m_free) {
  if (const char* v = env_str("W4A16_BLOCK_M"))
    if (block_m_free) c->block_m = std::atoi(v);
  if (const char* v = env_str("W4A16_NR")) c->nr = std::atoi(v);
  if (const char* v = env_str("W4A16_WAVES")) c->waves = std::atoi(v);
  if (const char* v = env_str("W4A16_SPLIT_K")) c->split_k = std::atoi(v);
  if (const char* v = env_str("W4A16_STAGES")) c->stages = std::atoi(v);
}

// the first tuning override set in the environment, or NULL
const char* env_override_present() {
  for (const char* name : kOverrideVars)
    if (env_str(name)) return name;
  return nullptr;
}

bool valid_split(int split) { return split == 0 || split == 1 || split == 2 || split == 4 || split == 8 || split == 16; }

w4a16_status check_config(const w4a16_config& c, int route, int epi, int K) {
  if (c.kind != route)
    return fail(W4A16_ERR_ARG, "config was chosen for routing kind %d, this call is kind %d (%s)", c.kind, route,
                route == W4A16_ROUTE_INDEXED ? "indexed" : "grouped calls choose their own tiles");
  if (!valid_block_m(c.block_m)) return fail(W4A16_ERR_UNSUPPORTED, "block_m %d not in {16, 32, 64, 128, 256}", c.block_m);
  if (c.combine_cols < 0 || c.combine_cols % 16)
    return fail(W4A16_ERR_ARG, "combine_cols %d: 0 (the library's choice) or a positive multiple of 16",
                c.combine_cols);
  if (!valid_split(c.split_k))
    return fail(W4A16_ERR_UNSUPPORTED, "split_k %d: 1 (one workgroup per tile), 2, 4, 8, 16 (K slices) or 0 (stream-K)",
                c.split_k);
  if (c.split_k == 0 && route != W4A16_ROUTE_INDEXED)
    return fail(W4A16_ERR_UNSUPPORTED, "stream-K (split_k = 0) is built for indexed routing only");
  if (c.split_k > 1 && c.split_k > (chunks_of(K) + 1) / 2)
    return fail(W4A16_ERR_UNSUPPORTED, "split_k %d exceeds the %d pairs of 128-K chunks of K = %d", c.split_k,
                (chunks_of(K) + 1) / 2, K);
  if (c.nr == 1 && (c.split_k != 1 || K % 128))
    return fail(W4A16_ERR_UNSUPPORTED, "nr = 1 (waves splitting K) needs split_k = 1 and K a multiple of 128");
  if (!w4a16::gemm_config_supported(route, epi, c.block_m / 16, c.nr, c.waves, c.stages))
    return fail(W4A16_ERR_UNSUPPORTED, "tile config block_m=%d nr=%d waves=%d stages=%d not built", c.block_m,
                c.nr, c.waves, c.stages);
  return W4A16_OK;
}

w4a16::GemmParams base_params(const w4a16_weight_desc* d, const void* pw, const void* ps,
                              const uint16_t* a, void* out, int nr, int waves) {
  w4a16::GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.packed_w = static_cast<const uint4*>(pw);
  p.packed_s = static_cast<const uint32_t*>(ps);
  p.a = a;
  p.E = d->E;
  p.N = d->N;
  p.K = d->K;
  p.NT = d->N / 16;
  p.w_tiles = d->N / 16;
  p.KC = d->K_pad / 128;
  p.n_tiles = n_tiles_of(d->N, nr, waves);
  p.gated = (d->flags & W4A16_DESC_GATE_UP) != 0;
  p.out = out;
  p.split = 1;
  return p;
}

// Workspace carve-up (each region 256-byte aligned):
//   [split counters, 4 B per splittable tile][split slices][combine partials, fp32 T*topk*cols]
//   [stream-K partials][local slots per token, T bytes (combine)]
struct Workspace {
  size_t counters = 0, slices = 0, combine = 0, streamk = 0, tokens = 0;
  int split_tiles = 0;
  size_t total() const { return counters + slices + combine + streamk + tokens; }
};

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

int resident_workgroups(const w4a16_config& c, int epi);

// Output columns per pass of the down projection + combine.  A pass's fp32
// per-slot partials are written by the GEMM and read back by the combine;
// when they fit the last-level cache (256 MB) the combine reads them without
// HBM write-backs competing.  Measured on MI355X: a buffer of up to 256 MB
// written by one kernel reads back at 6.5 TB/s, a 1 GB one at 4.3 TB/s; TP8
// T = 4096 (940 MB of partials) combines in 238 us in one pass, 145 us in
// four.  Every extra pass costs the GEMM a fetch of each block's activation
// rows per XCD (down GEMM 354 us in one pass, 391 us in four), so the
// library's choice is the fewest passes whose expected partials (local slots
// under uniform routing x columns x 4 bytes) stay within kCombinePassBytes,
// in whole workgroup tiles; an explicit config's combine_cols wins.
constexpr double kCombinePassBytes = 240.0 * (1 << 20);

// fp32 per-slot partials of the local slots under uniform routing
double expected_partial_bytes(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N) {
  const double local = E_glob > 0 ? std::min(1.0, (double)E_loc / E_glob) : 1.0;
  return (double)std::max(T, 0) * topk * local * N * 4.0;
}

// Partials from which tokens with one local slot bypass them (see moe_gemm_impl).
constexpr double kDirectMinBytes = 64.0 * (1 << 20);

int32_t combine_cols_of(const w4a16_config& c, int32_t N, int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc) {
  if (c.combine_cols > 0) return std::min(c.combine_cols, N);
  const double bytes = expected_partial_bytes(T, topk, E_glob, E_loc, N);
  if (bytes <= kCombinePassBytes) return N;
  const int64_t passes = (int64_t)std::ceil(bytes / kCombinePassBytes);
  const int64_t wg_n = 16 * (int64_t)c.nr * c.waves;
  const int64_t cols = ((N + passes - 1) / passes + wg_n - 1) / wg_n * wg_n;
  return (int32_t)std::min<int64_t>(cols, N);
}

// tiles: an upper bound of the call's tiles (routed blocks x N tiles);
// cols: output columns per combine pass (combine_cols_of)
Workspace workspace_layout(const w4a16_config& c, int epi, int64_t tiles, int32_t cols, int32_t T, int32_t topk,
                           bool combine) {
  Workspace w;
  if (c.split_k > 1) {
    w.split_tiles = (int)std::min<int64_t>(std::max<int64_t>(tiles, 0), kSplitTileCap);
    w.counters = al256((size_t)w.split_tiles * 4);
    w.slices = al256((size_t)w.split_tiles * c.split_k * w4a16::split_slice_bytes(c.block_m / 16, c.nr, c.waves));
  }
  if (combine) {
    w.combine = al256((size_t)T * topk * cols * sizeof(float));
    w.tokens = al256((size_t)std::max(T, 0));
  }
  if (c.split_k == 0) {
    const int wgs = resident_workgroups(c, epi);
    if (wgs > 0) w.streamk = w4a16::streamk_partial_bytes(c.block_m / 16, c.nr, c.waves, wgs);
  }
  return w;
}

void attach_split(w4a16::GemmParams& p, const w4a16_config& c, const Workspace& w, char* ws) {
  p.split = std::max(c.split_k, 1);
  if (c.split_k > 1) {
    p.split_tiles = w.split_tiles;
    p.split_count = reinterpret_cast<uint32_t*>(ws);
    p.split_partial = reinterpret_cast<float*>(ws + w.counters);
  }
}

// Upper bound of the tiles of block_m rows that hold routed rows in an
// indexed call: the align writes the experts' segments from position 0, each
// rounded up to the routing's block_m R, so num_tokens_padded is at most
// slots + (R - 1) per expert with rows, and there are at most T * topk local
// slots (so at most that many experts with rows).  Every tile past it is
// padding, so it also bounds the launch grid: the over-allocated capacity
// (one block of padding per local expert) would otherwise launch mostly
// empty workgroups -- 361 blocks for the 8 rows of one token over 384
// experts.
int64_t indexed_block_bound(const w4a16_indexed_routing& r, int32_t block_m) {
  const int64_t slots = (int64_t)r.T * r.topk;
  const int64_t b = std::max(block_m, 1);
  const int64_t per_expert = std::max<int64_t>(r.block_m / b, 1);   // tiles of one routed block
  return std::min<int64_t>(r.capacity / b, (slots + b - 1) / b + per_expert * std::min<int64_t>(r.E_loc, slots));
}

// Workgroups of this config the current device keeps resident (stream-K
// grid); 0 when no device is visible or the config is not built.
int resident_workgroups(const w4a16_config& c, int epi) {
  return w4a16::streamk_workgroups(w4a16::kRouteIndexed, epi, c.block_m / 16, c.nr, c.waves, c.stages);
}

// select_indexed, memoised per argument set (no environment overrides)
w4a16_config cached_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N, int32_t K,
                           int32_t kind, int32_t expected_m, int32_t force_block_m) {
  const SelectKey key = std::make_tuple(T, topk, E_glob, E_loc, N, K, kind * 1024 + force_block_m, expected_m);
  {
    std::lock_guard<std::mutex> g(g_cache_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second;
  }
  w4a16_config c{};
  if (kind == W4A16_ROUTE_CONTIGUOUS)
    c = select_contiguous(T, E_loc, N, K);
  else if (kind == W4A16_ROUTE_MASKED)
    c = select_masked(T, E_loc, N, K, expected_m);
  else
    c = select_indexed(T, topk, E_glob, E_loc, N, K, force_block_m);
  std::lock_guard<std::mutex> g(g_cache_mu);
  g_cache[key] = c;
  return c;
}

// An activation / output tensor the kernels address with 32-bit byte offsets.
w4a16_status check_offset_range(int64_t rows, int32_t K, const char* what) {
  if (rows > 0 && rows * (int64_t)K * 2 > ((int64_t)1 << 32))
    return fail(W4A16_ERR_SHAPE, "%s: %lld rows x K = %d x 2 bytes exceed the 4 GiB the kernels address", what,
                (long long)rows, K);
  return W4A16_OK;
}

}  // namespace

extern "C" {

const char* w4a16_last_error(void) { return g_last_error.c_str(); }

int32_t w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

w4a16_status w4a16_weight_desc_init(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out) {
  if (out == nullptr) return fail(W4A16_ERR_ARG, "out is NULL");
  w4a16_status st = check_shape(E, N, K);
  if (st != W4A16_OK) return st;
  *out = make_desc(E, N, K, 0);
  return W4A16_OK;
}

w4a16_status w4a16_weight_desc_init_gate_up(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out) {
  if (out == nullptr) return fail(W4A16_ERR_ARG, "out is NULL");
  w4a16_status st = check_shape(E, N, K);
  if (st != W4A16_OK) return st;
  if (N % 32) return fail(W4A16_ERR_SHAPE, "a gate/up weight needs N %% 32 == 0 (got %d)", N);
  *out = make_desc(E, N, K, W4A16_DESC_GATE_UP);
  return W4A16_OK;
}

w4a16_status w4a16_pack_w4(const uint8_t* codes, const uint16_t* scales,
                           const w4a16_weight_desc* desc, void* packed_w, void* packed_s,
                           w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (!codes || !scales || !packed_w || !packed_s) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(packed_w) || !aligned16(packed_s)) return fail(W4A16_ERR_ARG, "packed buffers must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(scales) & 1u) return fail(W4A16_ERR_ARG, "scales must be 2-byte aligned");
  hipError_t e = w4a16::launch_pack(codes, scales, desc->E, desc->N, desc->K, desc->chunks,
                                    desc->flags == W4A16_DESC_GATE_UP, static_cast<uint32_t*>(packed_w),
                                    static_cast<uint32_t*>(packed_s), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack_w4 launch");
  return W4A16_OK;
}

int64_t w4a16_align_capacity(int32_t T, int32_t topk, int32_t E_loc, int32_t block_m) {
  if (T < 0 || topk <= 0 || E_loc <= 0 || !valid_block_m(block_m)) return -1;
  return round_up((int64_t)T * topk + (int64_t)E_loc * (block_m - 1), block_m);
}

w4a16_status w4a16_moe_align(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E_glob,
                             int32_t first_expert, int32_t E_loc, int32_t block_m,
                             int32_t* sorted_ids, int32_t* expert_ids,
                             int32_t* num_tokens_padded, int64_t capacity, int32_t validate,
                             w4a16_stream_t stream) {
  if (!sorted_ids || !expert_ids || !num_tokens_padded || (T > 0 && !topk_ids))
    return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (T < 0 || topk <= 0 || E_glob <= 0 || E_loc <= 0 || first_expert < 0)
    return fail(W4A16_ERR_ARG, "bad sizes T=%d topk=%d E_glob=%d first=%d E_loc=%d", T, topk, E_glob, first_expert, E_loc);
  if ((int64_t)first_expert + E_loc > E_glob)
    return fail(W4A16_ERR_ARG, "local experts [%d, %d) exceed E_glob=%d", first_expert, first_expert + E_loc, E_glob);
  if (E_loc > 1024) return fail(W4A16_ERR_SHAPE, "E_loc=%d > 1024 not supported", E_loc);
  if (!valid_block_m(block_m)) return fail(W4A16_ERR_SHAPE, "block_m %d not in {16, 32, 64, 128, 256}", block_m);
  if ((int64_t)T * topk >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "T*topk too large");
  const int64_t need = w4a16_align_capacity(T, topk, E_loc, block_m);
  if (capacity < need || capacity % block_m)
    return fail(W4A16_ERR_CAPACITY, "capacity %lld < %lld needed (or not a multiple of block_m %d)",
                (long long)capacity, (long long)need, block_m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate && T > 0) {
    std::vector<int32_t> h((size_t)T * topk);
    hipError_t e = hipMemcpyAsync(h.data(), topk_ids, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "moe_align validate readback");
    for (size_t i = 0; i < h.size(); ++i)
      if (h[i] < 0 || h[i] >= E_glob)
        return fail(W4A16_ERR_ROUTING, "topk_ids[%zu] = %d outside [0, %d)", i, h[i], E_glob);
  }
  hipError_t e = w4a16::launch_align(topk_ids, T * topk, first_expert, E_loc, block_m, sorted_ids,
                                     expert_ids, num_tokens_padded, capacity, s);
  if (e != hipSuccess) return hip_fail(e, "moe_align launch");
  return W4A16_OK;
}

}  // extern "C"

namespace {

// The indexed config of a call: cfg, or the selector's choice for the
// routing's shape and block_m with environment overrides applied.
w4a16_status indexed_call_config(const w4a16_indexed_routing& r, const w4a16_weight_desc* d, const w4a16_config* cfg,
                                 w4a16_config* out) {
  if (cfg) {
    *out = *cfg;
    return W4A16_OK;
  }
  if (r.E_glob <= 0) return fail(W4A16_ERR_ARG, "routing.E_glob must be positive (it steers the config when cfg is NULL)");
  *out = cached_select(r.T, r.topk, r.E_glob, r.E_loc, d->N, d->K, W4A16_ROUTE_INDEXED, 0, r.block_m);
  apply_env_overrides(out, false);
  return W4A16_OK;
}

// An indexed call's tile rows: the routing's block_m or a divisor of it (a
// 256-row routing also serves 128-row tiles; the tiles then look their
// expert up as expert_ids[tile >> shift]).
w4a16_status check_tile_rows(const w4a16_config& c, const w4a16_indexed_routing& r) {
  if (c.block_m > r.block_m || r.block_m % c.block_m)
    return fail(W4A16_ERR_LAYOUT, "config block_m=%d does not divide the routing's block_m=%d", c.block_m, r.block_m);
  return W4A16_OK;
}

// The A4W4 calls' tile rows when cfg is NULL: the routing's block_m, except
// that a 256-row routing (which the W4A16 selector gives from 128 rows per
// expert) takes 64-row tiles, the A4W4 choice at those token counts.
int32_t mx_tile_rows(const w4a16_indexed_routing& r) { return r.block_m == 256 ? 64 : r.block_m; }

int32_t tile_shift(const w4a16_config& c, const w4a16_indexed_routing& r) {
  int32_t s = 0;
  while ((c.block_m << s) < r.block_m) ++s;
  return s;
}

// Checks shared by the indexed W4A16 calls; fills the activation rows the
// call may read.
w4a16_status check_indexed_call(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                const void* a, const void* out, const w4a16_indexed_routing* routing) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (!routing) return fail(W4A16_ERR_ARG, "routing is NULL");
  const w4a16_indexed_routing& r = *routing;
  if (!packed_w || !packed_s || !r.sorted_ids || !r.expert_ids || !r.num_tokens_padded)
    return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (r.T < 0 || r.topk <= 0 || r.capacity < 0 || r.E_loc <= 0) return fail(W4A16_ERR_ARG, "bad routing sizes");
  if (r.T > 0 && (!a || !out)) return fail(W4A16_ERR_ARG, "activations or output are NULL");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
  if (r.E_loc != desc->E)
    return fail(W4A16_ERR_LAYOUT, "routing has E_loc=%d but the packed weight holds %d experts", r.E_loc, desc->E);
  if (!valid_block_m(r.block_m)) return fail(W4A16_ERR_ARG, "routing.block_m %d not in {16, 32, 64, 128, 256}", r.block_m);
  if ((int64_t)r.T * r.topk >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "T*topk too large");
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (r.capacity / r.block_m > INT32_MAX / 2) return fail(W4A16_ERR_CAPACITY, "capacity too large");
  return W4A16_OK;
}

}  // namespace

extern "C" {

w4a16_status w4a16_indexed_config(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N, int32_t K,
                                  int32_t block_m, w4a16_config* out) {
  if (!out) return fail(W4A16_ERR_ARG, "out is NULL");
  if (!valid_block_m(block_m)) return fail(W4A16_ERR_ARG, "block_m %d not in {16, 32, 64, 128, 256}", block_m);
  if (T < 0 || topk <= 0 || E_glob <= 0 || E_loc <= 0 || N <= 0 || K <= 0)
    return fail(W4A16_ERR_ARG, "bad sizes for indexed_config");
  *out = cached_select(T, topk, E_glob, E_loc, N, K, W4A16_ROUTE_INDEXED, 0, block_m);
  apply_env_overrides(out, false);
  return W4A16_OK;
}

w4a16_status w4a16_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N,
                          int32_t K, int32_t kind, int32_t expected_m, w4a16_config* out) {
  if (!out) return fail(W4A16_ERR_ARG, "out is NULL");
  if (T < 0 || E_loc <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_ARG, "bad sizes for select");
  if (kind == W4A16_ROUTE_INDEXED) {
    if (topk <= 0 || E_glob <= 0) return fail(W4A16_ERR_ARG, "bad sizes for select");
    *out = cached_select(T, topk, E_glob, E_loc, N, K, kind, 0, 0);
    apply_env_overrides(out, true);
    return W4A16_OK;
  }
  if (kind != W4A16_ROUTE_CONTIGUOUS && kind != W4A16_ROUTE_MASKED)
    return fail(W4A16_ERR_ARG, "kind %d is not a W4A16_ROUTE_* value", kind);
  if (const char* v = env_override_present())
    return fail(W4A16_ERR_ARG, "%s is set: tuning overrides apply to indexed routing only; grouped calls choose their own tiles", v);
  if (kind == W4A16_ROUTE_MASKED && expected_m <= 0) return fail(W4A16_ERR_ARG, "expected_m must be positive");
  *out = cached_select(T, 1, 1, E_loc, N, K, kind, kind == W4A16_ROUTE_MASKED ? expected_m : 0, 0);
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N,
                                int32_t K, w4a16_config* out) {
  if (!out) return fail(W4A16_ERR_ARG, "out is NULL");
  if (T < 0 || topk <= 0 || E_glob <= 0 || E_loc <= 0 || N <= 0 || K <= 0)
    return fail(W4A16_ERR_ARG, "bad sizes for select");
  w4a16_config c = cached_select(T, topk, E_glob, E_loc, N, K, W4A16_ROUTE_INDEXED, 0, 0);
  const double tok_e = (double)T * topk / E_glob;
  if (c.block_m >= 128 && tok_e >= kMxHalfTileTokE) c.block_m = 64;
  // the K-split tile where the W4A16 rule takes it (block_m 16, a grid that
  // would split K four or more ways), else four weight tiles per wave
  const bool kwave = c.nr == 1;
  c.nr = kwave ? 1 : 4;
  c.waves = kwave ? w4a16::kKwWaves : 4;
  c.split_k = 1;
  c.stages = c.block_m <= 32 ? 4 : 2;
  *out = c;
  apply_env_overrides(out, true);
  return W4A16_OK;
}

size_t w4a16_moe_gemm_workspace_bytes(const w4a16_weight_desc* desc, const w4a16_indexed_routing* routing,
                                      int32_t combine, const w4a16_config* cfg) {
  if (check_int4_desc(desc) != W4A16_OK || !routing) return 0;
  const w4a16_indexed_routing& r = *routing;
  if (r.T < 0 || r.topk <= 0 || r.E_loc <= 0 || !valid_block_m(r.block_m) || r.capacity < 0) return 0;
  w4a16_config c{};
  if (indexed_call_config(r, desc, cfg, &c) != W4A16_OK) return 0;
  const int epi = combine ? w4a16::kEpiWeighted : w4a16::kEpiStore;
  if (check_config(c, W4A16_ROUTE_INDEXED, epi, desc->K) != W4A16_OK) return 0;
  const int64_t tiles = indexed_block_bound(r, c.block_m) * n_tiles_of(desc->N, c.nr, c.waves);
  const int32_t cols = combine_cols_of(c, desc->N, r.T, r.topk, r.E_glob, r.E_loc);
  return workspace_layout(c, epi, tiles, cols, r.T, r.topk, combine != 0).total();
}

}  // extern "C"

namespace {

// The indexed GEMM with its workspace already chosen.  With no_alloc, the
// workspace is the library's own scratch array of `workspace_bytes` bytes:
// a call needing more is refused, and the split-K arrival counters are
// cleared first (the array keeps whatever the previous call on the device
// left in it).
w4a16_status moe_gemm_impl(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                           const uint16_t* a, int64_t a_rows, int32_t a_layout, const w4a16_indexed_routing* routing,
                           const float* topk_weights, uint16_t* out, const w4a16_config* cfg, void* workspace,
                           size_t workspace_bytes, w4a16_stream_t stream, bool no_alloc) {
  w4a16_status st = check_indexed_call(desc, packed_w, packed_s, a, out, routing);
  if (st != W4A16_OK) return st;
  const w4a16_indexed_routing& r = *routing;
  const bool combine = topk_weights != nullptr;
  if (combine && (desc->flags & W4A16_DESC_GATE_UP))
    return fail(W4A16_ERR_LAYOUT, "a gate/up interleaved weight cannot take the top-k combine (it belongs to the down projection)");
  if (a_layout != W4A16_A_TOKEN && a_layout != W4A16_A_SLOT && a_layout != W4A16_A_SORTED)
    return fail(W4A16_ERR_ARG, "a_layout %d is not W4A16_A_TOKEN, W4A16_A_SLOT or W4A16_A_SORTED", a_layout);
  const int64_t need_rows = a_layout == W4A16_A_TOKEN  ? (int64_t)r.T
                            : a_layout == W4A16_A_SLOT ? (int64_t)r.T * r.topk
                                                       : r.capacity;
  if (a_rows < need_rows)
    return fail(W4A16_ERR_SHAPE, "activations have %lld rows, need %lld", (long long)a_rows, (long long)need_rows);
  st = check_offset_range(need_rows, desc->K, "activations");
  if (st != W4A16_OK) return st;
  const int epi = combine ? w4a16::kEpiWeighted : w4a16::kEpiStore;
  w4a16_config c{};
  st = indexed_call_config(r, desc, cfg, &c);
  if (st != W4A16_OK) return st;
  st = check_config(c, W4A16_ROUTE_INDEXED, epi, desc->K);
  if (st != W4A16_OK) return st;
  st = check_tile_rows(c, r);
  if (st != W4A16_OK) return st;
  if (combine && !r.topk_ids) return fail(W4A16_ERR_ARG, "combine needs routing.topk_ids");
  const int64_t tiles = indexed_block_bound(r, c.block_m) * n_tiles_of(desc->N, c.nr, c.waves);
  const int32_t cols = combine ? combine_cols_of(c, desc->N, r.T, r.topk, r.E_glob, r.E_loc) : desc->N;
  const Workspace wl = workspace_layout(c, epi, tiles, cols, r.T, r.topk, combine);
  if (c.split_k == 0 && wl.streamk == 0)
    return fail(W4A16_ERR_HIP, "stream-K: could not query the device's resident workgroups");
  const size_t need = wl.total();
  if (no_alloc && need > workspace_bytes)
    return fail(W4A16_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the library's scratch array holds %zu "
                "(use w4a16_moe_gemm with a caller workspace)", need, workspace_bytes);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(W4A16_ERR_WORKSPACE, "this call needs %zu bytes of 16-byte aligned workspace, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (r.T == 0) return W4A16_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if (no_alloc && wl.counters > 0) {
    e = w4a16::launch_zero_words(reinterpret_cast<uint32_t*>(ws), (int64_t)(wl.counters / 4), s);
    if (e != hipSuccess) return hip_fail(e, "scratch counter clear launch");
  }
  float* comb = combine ? reinterpret_cast<float*>(ws + wl.counters + wl.slices) : nullptr;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, a, combine ? (void*)comb : (void*)out, c.nr, c.waves);
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = a_layout == W4A16_A_TOKEN ? r.topk : a_layout == W4A16_A_SLOT ? 1 : 0;
  p.slot_weight = topk_weights;
  p.expert_shift = tile_shift(c, r);
  p.grid_blocks = (int32_t)indexed_block_bound(r, c.block_m);
  if (c.split_k == 0) p.sk_partial = reinterpret_cast<float*>(ws + wl.counters + wl.slices + wl.combine);
  else attach_split(p, c, wl, ws);
  // Tokens with exactly one local slot: the GEMM stores bf16(w * acc) as their
  // output and the combine leaves them alone (the sum of one term), which
  // saves their fp32 round trip at the cost of a small counting launch.
  // Used where the partials are large (measured on MI355X, down + combine:
  // EP8 prefill 360-373 -> 354 us, EP16 prefill 228 -> 219 us; EP8 decode
  // 90 -> 93 us, so not there); skipped when every expert is local and
  // top-k >= 2, where no token has one.
  const bool direct = combine && !(r.first_expert == 0 && r.E_loc >= r.E_glob && r.topk >= 2) &&
                      expected_partial_bytes(r.T, r.topk, r.E_glob, r.E_loc, desc->N) >= kDirectMinBytes;
  uint8_t* token_local = combine ? reinterpret_cast<uint8_t*>(ws + wl.counters + wl.slices + wl.combine + wl.streamk)
                                 : nullptr;
  if (direct) {
    e = w4a16::launch_token_local(r.topk_ids, r.T, r.topk, r.first_expert, r.E_loc, token_local, s);
    if (e != hipSuccess) return hip_fail(e, "token count launch");
    p.token_local = token_local;
    p.topk = r.topk;
    p.direct_ld = desc->N;
  }
  // one pass per `cols` output columns (all of N without the combine): the
  // GEMM over that column range of the weights, then its combine
  const int64_t kc2 = (p.KC + 1) / 2;
  for (int32_t n0 = 0; n0 < desc->N; n0 += cols) {
    const int32_t nc = std::min(cols, desc->N - n0);
    w4a16::GemmParams q = p;
    q.packed_w = p.packed_w + (int64_t)(n0 / 16) * p.KC * 64;
    q.packed_s = p.packed_s + (int64_t)(n0 / 16) * kc2 * 64;
    q.N = nc;
    q.NT = nc / 16;
    q.n_tiles = n_tiles_of(nc, c.nr, c.waves);
    if (direct) q.direct_out = out + n0;
    if (c.split_k == 0) {
      e = w4a16::launch_gemm_streamk(w4a16::kRouteIndexed, epi, c.block_m / 16, c.nr, c.waves, c.stages, q,
                                     resident_workgroups(c, epi), s);
    } else {
      e = w4a16::launch_gemm(w4a16::kRouteIndexed, epi, c.block_m / 16, c.nr, c.waves, c.stages, q, s);
    }
    if (e != hipSuccess) return hip_fail(e, "moe_gemm launch");
    if (combine) {
      e = w4a16::launch_combine(comb, r.topk_ids, r.T, r.topk, r.first_expert, r.E_loc, nc, out + n0, desc->N,
                                direct ? token_local : nullptr, s);
      if (e != hipSuccess) return hip_fail(e, "combine launch");
    }
  }
  return W4A16_OK;
}

// The library's own scratch for w4a16_moe_gemm_noalloc: one array per GPU,
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a host-side stand-in, not a device
// address); it passes the device address hipGetSymbolAddress returns for the
// current device, looked up once per device on the first call there.
static __device__ __align__(256) unsigned char scratch[W4A16_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

w4a16_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(W4A16_ERR_HIP, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return W4A16_OK;
}

}  // namespace

extern "C" {

w4a16_status w4a16_moe_gemm(const w4a16_weight_desc* desc, const void* packed_w,
                            const void* packed_s, const uint16_t* a, int64_t a_rows,
                            int32_t a_layout, const w4a16_indexed_routing* routing,
                            const float* topk_weights, uint16_t* out,
                            const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                            w4a16_stream_t stream) {
  return moe_gemm_impl(desc, packed_w, packed_s, a, a_rows, a_layout, routing, topk_weights, out, cfg, workspace,
                       workspace_bytes, stream, false);
}

w4a16_status w4a16_moe_gemm_noalloc(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                    const uint16_t* a, int64_t a_rows, int32_t a_layout,
                                    const w4a16_indexed_routing* routing, const float* topk_weights, uint16_t* out,
                                    const w4a16_config* cfg, w4a16_stream_t stream) {
  void* ws = nullptr;
  w4a16_status st = scratch_of_current_device(&ws);
  if (st != W4A16_OK) return st;
  return moe_gemm_impl(desc, packed_w, packed_s, a, a_rows, a_layout, routing, topk_weights, out, cfg, ws,
                       W4A16_SCRATCH_BYTES, stream, true);
}

w4a16_status w4a16_moe_gate_up_silu(const w4a16_weight_desc* desc, const void* packed_w,
                                    const void* packed_s, const uint16_t* x, int64_t x_rows,
                                    const w4a16_indexed_routing* routing, uint16_t* out,
                                    const w4a16_config* cfg, w4a16_stream_t stream) {
  w4a16_status st = check_indexed_call(desc, packed_w, packed_s, x, out, routing);
  if (st != W4A16_OK) return st;
  if (desc->flags != W4A16_DESC_GATE_UP)
    return fail(W4A16_ERR_LAYOUT, "the fused SiLU gate/up call needs a weight packed with w4a16_weight_desc_init_gate_up");
  const w4a16_indexed_routing& r = *routing;
  if (x_rows < r.T) return fail(W4A16_ERR_SHAPE, "activations have %lld rows, need %d", (long long)x_rows, r.T);
  st = check_offset_range(r.T, desc->K, "activations");
  if (st != W4A16_OK) return st;
  w4a16_config c{};
  st = indexed_call_config(r, desc, cfg, &c);
  if (st != W4A16_OK) return st;
  if (!cfg) c.split_k = 1;  // the fused epilogue runs whole tiles
  if (c.split_k != 1) return fail(W4A16_ERR_UNSUPPORTED, "the fused SiLU gate/up call runs one workgroup per tile (split_k = 1)");
  if (c.nr != 1 && c.nr % 2)
    return fail(W4A16_ERR_UNSUPPORTED, "the fused SiLU gate/up call needs an even nr, or 1 (gate and up tiles in pairs)");
  st = check_config(c, W4A16_ROUTE_INDEXED, w4a16::kEpiSilu, desc->K);
  if (st != W4A16_OK) return st;
  st = check_tile_rows(c, r);
  if (st != W4A16_OK) return st;
  if (r.T == 0) return W4A16_OK;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, x, out, c.nr, c.waves);
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = r.topk;
  p.expert_shift = tile_shift(c, r);
  p.grid_blocks = (int32_t)indexed_block_bound(r, c.block_m);
  if (c.nr == 1) p.n_tiles = p.NT / 2;   // one (gate, up) tile pair per workgroup
  hipError_t e = w4a16::launch_gemm(w4a16::kRouteIndexed, w4a16::kEpiSilu, c.block_m / 16, c.nr, c.waves,
                                    c.stages, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gate_up_silu launch");
  return W4A16_OK;
}

namespace {

// The config of a grouped call: NULL -> its own selection; otherwise a config
// of its kind (an indexed config is refused by check_config).  Tuning
// overrides in the environment are refused either way.
w4a16_status grouped_call_config(int kind, const w4a16_weight_desc* d, int64_t rows, int32_t expected_m,
                                 const w4a16_config* cfg, w4a16_config* out) {
  if (const char* v = env_override_present())
    return fail(W4A16_ERR_ARG, "%s is set: tuning overrides apply to indexed routing only; grouped calls choose their own tiles", v);
  if (cfg) {
    *out = *cfg;
    return W4A16_OK;
  }
  if (kind == W4A16_ROUTE_MASKED && expected_m <= 0) return fail(W4A16_ERR_ARG, "expected_m must be positive");
  if (rows > INT32_MAX) return fail(W4A16_ERR_SHAPE, "too many rows");
  *out = cached_select((int32_t)rows, 1, 1, d->E, d->N, d->K, kind, kind == W4A16_ROUTE_MASKED ? expected_m : 0, 0);
  return W4A16_OK;
}

// routed blocks of a grouped call's grid
int64_t grouped_blocks(int kind, const w4a16_weight_desc* d, int64_t rows, const w4a16_config& c) {
  if (kind == W4A16_ROUTE_CONTIGUOUS) return rows / c.block_m;
  return (int64_t)d->E * ((rows + c.block_m - 1) / c.block_m);
}

}  // namespace

size_t w4a16_grouped_workspace_bytes(const w4a16_weight_desc* desc, int32_t kind, int64_t rows, int32_t expected_m,
                                     const w4a16_config* cfg) {
  if (check_int4_desc(desc) != W4A16_OK || rows < 0) return 0;
  if (kind != W4A16_ROUTE_CONTIGUOUS && kind != W4A16_ROUTE_MASKED) return 0;
  w4a16_config c{};
  if (grouped_call_config(kind, desc, rows, expected_m, cfg, &c) != W4A16_OK) return 0;
  if (check_config(c, kind, w4a16::kEpiStore, desc->K) != W4A16_OK) return 0;
  const int64_t tiles = grouped_blocks(kind, desc, rows, c) * n_tiles_of(desc->N, c.nr, c.waves);
  return workspace_layout(c, w4a16::kEpiStore, tiles, desc->N, 0, 1, false).total();
}

namespace {

w4a16_status launch_grouped(int kind, const w4a16_weight_desc* desc, const w4a16_config& c, w4a16::GemmParams& p,
                            int64_t rows, void* workspace, size_t workspace_bytes, hipStream_t s, const char* what) {
  const int64_t tiles = grouped_blocks(kind, desc, rows, c) * n_tiles_of(desc->N, c.nr, c.waves);
  const Workspace wl = workspace_layout(c, w4a16::kEpiStore, tiles, desc->N, 0, 1, false);
  const size_t need = wl.total();
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(W4A16_ERR_WORKSPACE, "this call needs %zu bytes of 16-byte aligned workspace, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  attach_split(p, c, wl, static_cast<char*>(workspace));
  hipError_t e = w4a16::launch_gemm(kind == W4A16_ROUTE_CONTIGUOUS ? w4a16::kRouteContiguous : w4a16::kRouteMasked,
                                    w4a16::kEpiStore, c.block_m / 16, c.nr, c.waves, c.stages, p, s);
  if (e != hipSuccess) return hip_fail(e, what);
  return W4A16_OK;
}

}  // namespace

w4a16_status w4a16_grouped_contiguous(const w4a16_weight_desc* desc, const void* packed_w,
                                      const void* packed_s, const uint16_t* a, int64_t m_rows,
                                      const int32_t* m_indices, uint16_t* out,
                                      const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                                      w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (m_rows < 0) return fail(W4A16_ERR_ARG, "m_rows < 0");
  if (m_rows > 0 && (!a || !m_indices || !out)) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!packed_w || !packed_s) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
  st = check_offset_range(m_rows, desc->K, "activations");
  if (st != W4A16_OK) return st;
  w4a16_config c{};
  st = grouped_call_config(W4A16_ROUTE_CONTIGUOUS, desc, m_rows, 0, cfg, &c);
  if (st != W4A16_OK) return st;
  st = check_config(c, W4A16_ROUTE_CONTIGUOUS, w4a16::kEpiStore, desc->K);
  if (st != W4A16_OK) return st;
  if (128 % c.block_m) return fail(W4A16_ERR_UNSUPPORTED, "contiguous layout needs block_m dividing 128");
  if (m_rows % c.block_m) return fail(W4A16_ERR_SHAPE, "m_rows=%lld is not a multiple of block_m=%d (segments are 128-row aligned)", (long long)m_rows, c.block_m);
  if (m_rows == 0) return W4A16_OK;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, a, out, c.nr, c.waves);
  p.m_indices = m_indices;
  p.grid_blocks = (int32_t)(m_rows / c.block_m);
  return launch_grouped(W4A16_ROUTE_CONTIGUOUS, desc, c, p, m_rows, workspace, workspace_bytes,
                        static_cast<hipStream_t>(stream), "grouped_contiguous launch");
}

w4a16_status w4a16_grouped_masked(const w4a16_weight_desc* desc, const void* packed_w,
                                  const void* packed_s, const uint16_t* a, int32_t max_m,
                                  const int32_t* masked_m, int32_t expected_m, uint16_t* out,
                                  const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                                  w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (max_m <= 0) return fail(W4A16_ERR_ARG, "max_m must be positive");
  if (!a || !masked_m || !out || !packed_w || !packed_s) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
  if ((int64_t)desc->E * max_m >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "E * max_m too large");
  st = check_offset_range((int64_t)desc->E * max_m, desc->K, "activations");
  if (st != W4A16_OK) return st;
  w4a16_config c{};
  st = grouped_call_config(W4A16_ROUTE_MASKED, desc, max_m, expected_m, cfg, &c);
  if (st != W4A16_OK) return st;
  st = check_config(c, W4A16_ROUTE_MASKED, w4a16::kEpiStore, desc->K);
  if (st != W4A16_OK) return st;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, a, out, c.nr, c.waves);
  p.masked_m = masked_m;
  p.max_m = max_m;
  p.blocks_per_group = (max_m + c.block_m - 1) / c.block_m;
  p.grid_blocks = desc->E * p.blocks_per_group;
  return launch_grouped(W4A16_ROUTE_MASKED, desc, c, p, max_m, workspace, workspace_bytes,
                        static_cast<hipStream_t>(stream), "grouped_masked launch");
}

// ------------------------------------------------------------ A4W4 (MXFP4)

w4a16_status w4a16_mxfp4_weight_desc_init(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out) {
  if (out == nullptr) return fail(W4A16_ERR_ARG, "out is NULL");
  w4a16_status st = check_shape(E, N, K);
  if (st != W4A16_OK) return st;
  if (K % 128) return fail(W4A16_ERR_SHAPE, "an MXFP4 weight needs K %% 128 == 0 (got %d)", K);
  *out = make_desc(E, N, K, W4A16_DESC_MXFP4);
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_weight_desc_init_gate_up(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out) {
  if (out == nullptr) return fail(W4A16_ERR_ARG, "out is NULL");
  w4a16_status st = check_shape(E, N, K);
  if (st != W4A16_OK) return st;
  if (K % 128) return fail(W4A16_ERR_SHAPE, "an MXFP4 weight needs K %% 128 == 0 (got %d)", K);
  if (N % 64) return fail(W4A16_ERR_SHAPE, "an MXFP4 gate/up weight needs N %% 64 == 0 (got %d)", N);
  *out = make_desc(E, N, K, W4A16_DESC_MXFP4 | W4A16_DESC_GATE_UP);
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_pack(const uint8_t* codes, const uint8_t* scales, const w4a16_weight_desc* desc,
                              void* packed_w, void* packed_s, w4a16_stream_t stream) {
  w4a16_status st = check_mx_desc(desc);
  if (st != W4A16_OK) return st;
  if (!codes || !scales || !packed_w || !packed_s) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(codes) || !aligned16(packed_w) || !aligned16(packed_s))
    return fail(W4A16_ERR_ARG, "codes and packed buffers must be 16-byte aligned");
  hipError_t e = w4a16::launch_mx_pack(codes, scales, desc->E, desc->N, desc->K,
                                       (desc->flags & W4A16_DESC_GATE_UP) != 0, static_cast<uint4*>(packed_w),
                                       static_cast<uint8_t*>(packed_s), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxfp4_pack launch");
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_quant(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                               w4a16_stream_t stream) {
  if (rows < 0 || K <= 0) return fail(W4A16_ERR_ARG, "bad sizes rows=%lld K=%d", (long long)rows, K);
  if (K % 32) return fail(W4A16_ERR_SHAPE, "K = %d is not a multiple of the MX block 32", K);
  if (rows == 0) return W4A16_OK;
  if (!x || !codes || !scales) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(x) || !aligned16(codes)) return fail(W4A16_ERR_ARG, "x and codes must be 16-byte aligned");
  hipError_t e = w4a16::launch_mx_quant(x, rows, K, codes, scales, nullptr, 0, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxfp4_quant launch");
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_quant_local_slots(const uint16_t* x, const int32_t* topk_ids, int32_t T, int32_t topk,
                                           int32_t first_expert, int32_t E_loc, int32_t K, uint8_t* codes,
                                           uint8_t* scales, w4a16_stream_t stream) {
  if (T < 0 || topk <= 0 || E_loc <= 0 || K <= 0)
    return fail(W4A16_ERR_ARG, "bad sizes T=%d topk=%d E_loc=%d K=%d", T, topk, E_loc, K);
  if (K % 32) return fail(W4A16_ERR_SHAPE, "K = %d is not a multiple of the MX block 32", K);
  if (T == 0) return W4A16_OK;
  if (!x || !topk_ids || !codes || !scales) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(x) || !aligned16(codes)) return fail(W4A16_ERR_ARG, "x and codes must be 16-byte aligned");
  hipError_t e = w4a16::launch_mx_quant(x, (int64_t)T * topk, K, codes, scales, topk_ids, first_expert, E_loc,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxfp4_quant_local_slots launch");
  return W4A16_OK;
}

size_t w4a16_mxfp4_moe_gemm_workspace_bytes(const w4a16_weight_desc* desc, int32_t T, int32_t topk,
                                            int32_t combine) {
  if (check_mx_desc(desc) != W4A16_OK || T < 0 || topk <= 0) return 0;
  return combine ? al256((size_t)T * topk * desc->N * sizeof(float)) : 0;
}

w4a16_status w4a16_mxfp4_moe_gemm(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                  const uint8_t* a_codes, const uint8_t* a_scales, int64_t a_rows,
                                  int32_t a_layout, const w4a16_indexed_routing* routing,
                                  const float* topk_weights, uint16_t* out, const w4a16_config* cfg,
                                  void* workspace, size_t workspace_bytes, w4a16_stream_t stream) {
  w4a16_status st = check_mx_desc(desc);
  if (st != W4A16_OK) return st;
  if (!routing) return fail(W4A16_ERR_ARG, "routing is NULL");
  const w4a16_indexed_routing& r = *routing;
  const bool combine = topk_weights != nullptr;
  if (!packed_w || !packed_s || !r.sorted_ids || !r.expert_ids || !r.num_tokens_padded)
    return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (r.T < 0 || r.topk <= 0 || r.capacity < 0) return fail(W4A16_ERR_ARG, "bad routing sizes");
  if (r.T > 0 && (!a_codes || !a_scales || !out)) return fail(W4A16_ERR_ARG, "activations or output are NULL");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a_codes) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activation codes and output must be 16-byte aligned");
  if (r.E_loc != desc->E)
    return fail(W4A16_ERR_LAYOUT, "routing has E_loc=%d but the packed weight holds %d experts", r.E_loc, desc->E);
  if (a_layout != W4A16_A_TOKEN && a_layout != W4A16_A_SLOT && a_layout != W4A16_A_SORTED)
    return fail(W4A16_ERR_ARG, "a_layout %d is not W4A16_A_TOKEN, W4A16_A_SLOT or W4A16_A_SORTED", a_layout);
  const int64_t need_rows = a_layout == W4A16_A_TOKEN  ? (int64_t)r.T
                            : a_layout == W4A16_A_SLOT ? (int64_t)r.T * r.topk
                                                       : r.capacity;
  if (a_rows < need_rows)
    return fail(W4A16_ERR_SHAPE, "activations have %lld rows, need %lld", (long long)a_rows, (long long)need_rows);
  if ((int64_t)r.T * r.topk >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "T*topk too large");
  if (a_rows * (int64_t)(desc->K / 2) >= ((int64_t)1 << 32))
    return fail(W4A16_ERR_SHAPE, "activation codes exceed 4 GiB (32-bit row offsets)");
  const int epi = combine ? w4a16::kEpiWeighted : w4a16::kEpiStore;
  w4a16_config c{};
  if (cfg) {
    c = *cfg;
  } else {
    c.block_m = mx_tile_rows(r);      // the routing buffers fix block_m
    // the K-split tile on a 16-row routing where the selector takes it
    const bool kwave = c.block_m == 16 && r.E_glob > 0 &&
                       cached_select(r.T, r.topk, r.E_glob, r.E_loc, desc->N, desc->K, W4A16_ROUTE_INDEXED, 0,
                                     r.block_m).nr == 1;
    c.nr = kwave ? 1 : 4;
    c.waves = kwave ? w4a16::kKwWaves : 4;
    c.split_k = 1;
    c.stages = c.block_m <= 32 ? 4 : 2;
    c.kind = W4A16_ROUTE_INDEXED;
    apply_env_overrides(&c, false);
  }
  if (c.kind != W4A16_ROUTE_INDEXED) return fail(W4A16_ERR_ARG, "config was chosen for a grouped routing kind");
  if (!valid_block_m(c.block_m)) return fail(W4A16_ERR_UNSUPPORTED, "block_m %d not in {16, 32, 64, 128, 256}", c.block_m);
  if (c.split_k != 1) return fail(W4A16_ERR_UNSUPPORTED, "the MXFP4 GEMM runs one workgroup per tile (split_k = 1)");
  if (!w4a16::mx_gemm_config_supported(epi, c.block_m / 16, c.nr, c.waves, c.stages))
    return fail(W4A16_ERR_UNSUPPORTED, "MXFP4 tile config block_m=%d nr=%d waves=%d stages=%d not built", c.block_m,
                c.nr, c.waves, c.stages);
  st = check_tile_rows(c, r);
  if (st != W4A16_OK) return st;
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (combine && !r.topk_ids) return fail(W4A16_ERR_ARG, "combine needs routing.topk_ids");
  const size_t need = combine ? al256((size_t)r.T * r.topk * desc->N * sizeof(float)) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(W4A16_ERR_WORKSPACE, "this call needs %zu bytes of 16-byte aligned workspace, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (r.T == 0) return W4A16_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, reinterpret_cast<const uint16_t*>(a_codes),
                                    combine ? workspace : (void*)out, c.nr, c.waves);
  p.a_scale = a_scales;
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = a_layout == W4A16_A_TOKEN ? r.topk : a_layout == W4A16_A_SLOT ? 1 : 0;
  p.slot_weight = topk_weights;
  p.expert_shift = tile_shift(c, r);
  p.grid_blocks = (int32_t)indexed_block_bound(r, c.block_m);
  hipError_t e = w4a16::launch_mx_gemm(epi, c.block_m / 16, c.nr, c.waves, c.stages, p, s);
  if (e != hipSuccess) return hip_fail(e, "mxfp4_moe_gemm launch");
  if (combine) {
    e = w4a16::launch_combine(static_cast<const float*>(workspace), r.topk_ids, r.T, r.topk, r.first_expert,
                              r.E_loc, desc->N, out, desc->N, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_gate_up_silu(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                      const uint8_t* x_codes, const uint8_t* x_scales, int64_t x_rows,
                                      const w4a16_indexed_routing* routing, uint8_t* out_codes,
                                      uint8_t* out_scales, const w4a16_config* cfg, w4a16_stream_t stream) {
  w4a16_status st = check_mx_desc(desc);
  if (st != W4A16_OK) return st;
  if (!(desc->flags & W4A16_DESC_GATE_UP))
    return fail(W4A16_ERR_LAYOUT, "the fused A4W4 gate/up call needs a weight from w4a16_mxfp4_weight_desc_init_gate_up");
  if (!routing) return fail(W4A16_ERR_ARG, "routing is NULL");
  const w4a16_indexed_routing& r = *routing;
  if (!packed_w || !packed_s || !r.sorted_ids || !r.expert_ids || !r.num_tokens_padded)
    return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (r.T < 0 || r.topk <= 0 || r.capacity < 0) return fail(W4A16_ERR_ARG, "bad routing sizes");
  if (r.T > 0 && (!x_codes || !x_scales || !out_codes || !out_scales))
    return fail(W4A16_ERR_ARG, "activations or outputs are NULL");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(x_codes) || !aligned16(out_codes))
    return fail(W4A16_ERR_ARG, "packed weights and code buffers must be 16-byte aligned");
  if (r.E_loc != desc->E)
    return fail(W4A16_ERR_LAYOUT, "routing has E_loc=%d but the packed weight holds %d experts", r.E_loc, desc->E);
  if (x_rows < r.T) return fail(W4A16_ERR_SHAPE, "activations have %lld rows, need %d", (long long)x_rows, r.T);
  if ((int64_t)r.T * r.topk >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "T*topk too large");
  if (x_rows * (int64_t)(desc->K / 2) >= ((int64_t)1 << 32))
    return fail(W4A16_ERR_SHAPE, "activation codes exceed 4 GiB (32-bit row offsets)");
  w4a16_config c{};
  if (cfg) {
    c = *cfg;
  } else {
    c.block_m = mx_tile_rows(r);
    // the K-split tile on a 16-row routing where the selector takes it
    const bool kwave = c.block_m == 16 && r.E_glob > 0 &&
                       cached_select(r.T, r.topk, r.E_glob, r.E_loc, desc->N, desc->K, W4A16_ROUTE_INDEXED, 0,
                                     r.block_m).nr == 1;
    c.nr = kwave ? 1 : 4;
    c.waves = kwave ? w4a16::kKwWaves : 4;
    c.split_k = 1;
    c.stages = c.block_m <= 32 ? 4 : 2;
    c.kind = W4A16_ROUTE_INDEXED;
    apply_env_overrides(&c, false);
  }
  if (c.kind != W4A16_ROUTE_INDEXED) return fail(W4A16_ERR_ARG, "config was chosen for a grouped routing kind");
  if (!valid_block_m(c.block_m)) return fail(W4A16_ERR_UNSUPPORTED, "block_m %d not in {16, 32, 64, 128, 256}", c.block_m);
  if (c.split_k != 1 || (c.nr != 4 && c.nr != 1))
    return fail(W4A16_ERR_UNSUPPORTED,
                "the fused A4W4 gate/up call runs one workgroup per tile with nr = 4 (or 1: the K-split tile)");
  if (!w4a16::mx_gemm_config_supported(w4a16::kEpiSiluMx, c.block_m / 16, c.nr, c.waves, c.stages))
    return fail(W4A16_ERR_UNSUPPORTED, "MXFP4 tile config block_m=%d nr=%d waves=%d stages=%d not built", c.block_m,
                c.nr, c.waves, c.stages);
  st = check_tile_rows(c, r);
  if (st != W4A16_OK) return st;
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (r.T == 0) return W4A16_OK;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, reinterpret_cast<const uint16_t*>(x_codes),
                                    out_codes, c.nr, c.waves);
  if (c.nr == 1) p.n_tiles = p.NT / 4;   // the K-split tile: four packed tiles (one activation block) each
  p.a_scale = x_scales;
  p.out_scale = out_scales;
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = r.topk;
  p.expert_shift = tile_shift(c, r);
  p.grid_blocks = (int32_t)indexed_block_bound(r, c.block_m);
  hipError_t e = w4a16::launch_mx_gemm(w4a16::kEpiSiluMx, c.block_m / 16, c.nr, c.waves, c.stages, p,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxfp4_gate_up_silu launch");
  return W4A16_OK;
}

}  // extern "C"

// C ABI of the W4A16 MoE expert GEMM (declared in include/w4a16_moe.h):
// argument validation, tile-configuration selection and kernel dispatch.
// Every check runs on the host before anything is enqueued; no entry point
// allocates device memory.
#include "w4a16_moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
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

bool valid_block_m(int32_t bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

// ---------------------------------------------------------------- selection
//
// Chord W4A16 MoE post, section "H200 prefill and TP8": block_m is chosen from
// tokens per expert tok_e = routed rows / experts; below about 80 a search
// minimises the total number of blocks on sampled routing, above it the
// padded expert rows are fitted under a maximum block_m.  On gfx950 the
// kernel skips 16-row token tiles that hold no valid row, so MFMA work
// follows valid rows whatever block_m is, while every extra block of an
// expert re-reads and re-dequantises its weights.  So:
//   - decode side (tok_e < kPrefillTokE): sample per-expert counts, pick the
//     smallest block_m whose total block count is within 2 % of the minimum
//     (smaller blocks keep fewer accumulators live and more waves resident);
//   - prefill side: block_m 128 (largest tile the accumulators allow), two
//     weight tiles per wave (measured faster than four at 128 rows).
constexpr double kPrefillTokE = 48.0;
// A4W4: above this many rows per expert the MXFP4 GEMM takes 64-row blocks
// where the W4A16 rule gives 128 (measured on MI355X, step time: EP8 / EP16
// prefill shares 5 % / 9 % faster at 64; at 85 rows per expert, TP8 T = 4096,
// 128 stays 6 % faster, since 64 would split most experts into two blocks
// that each stream the expert's weights).
constexpr double kMxHalfTileTokE = 128.0;

std::mutex g_cache_mu;
std::map<std::tuple<int, int, int, int, int, int>, w4a16_config> g_cache;

int64_t sampled_blocks(const std::vector<int>& counts, int bm) {
  int64_t b = 0;
  for (int c : counts) b += (c + bm - 1) / bm;
  return b;
}

int resident_workgroups(const w4a16_config& c, int epi);

w4a16_config select_config(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc) {
  w4a16_config c;
  c.waves = 4;
  c.split_k = 1;
  c.stages = 2;
  const double tok_e = (double)T * topk / std::max(E_glob, 1);
  // sampled routing: each of T*topk slots lands on one of E_glob experts
  // uniformly; keep the local ones (fixed seed: deterministic choice)
  std::mt19937 rng(12345u);
  std::vector<int> counts(std::max(E_loc, 1), 0);
  std::binomial_distribution<int> bin(std::max(T, 0) * std::max(topk, 1), 1.0 / std::max(E_glob, 1));
  for (int e = 0; e < E_loc; ++e) counts[e] = bin(rng);
  if (tok_e >= kPrefillTokE) {
    c.block_m = 128;
    c.nr = 2;  // measured: two 16-row weight tiles per wave beat four at 128 rows
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
    c.nr = 2;
  }
  // One workgroup per tile throughout.  Stream-K (split_k = 0) stays
  // available as an explicit config; the post gates it by shape (section
  // "H200 prefill and TP8"), but measured on MI355X against the current
  // one-workgroup kernel it no longer wins anywhere on the step: TP8 T = 1
  // 0.051 vs 0.059 ms, TP8 T = 16 0.095 vs 0.118, EP32 decode 0.089 vs
  // 0.104 (one workgroup per tile first), the down projection losing most
  // (its fix-up pass and per-segment pipeline restarts against K = 256 or
  // 2048).
  return c;
}

const char* env_str(const char* name) {
  const char* v = std::getenv(name);
  return (v && *v) ? v : nullptr;
}

// W4A16_BLOCK_M / W4A16_NR / W4A16_WAVES / W4A16_SPLIT_K / W4A16_STAGES override the selector (read on
// every call; the memoised result is the selector's, overrides are applied on top).
void apply_env_overrides(w4a16_config* c) {
  if (const char* v = env_str("W4A16_BLOCK_M")) c->block_m = std::atoi(v);
  if (const char* v = env_str("W4A16_NR")) c->nr = std::atoi(v);
  if (const char* v = env_str("W4A16_WAVES")) c->waves = std::atoi(v);
  if (const char* v = env_str("W4A16_SPLIT_K")) c->split_k = std::atoi(v);
  if (const char* v = env_str("W4A16_STAGES")) c->stages = std::atoi(v);
}

w4a16_status check_config(const w4a16_config& c, int route, int epi) {
  if (!valid_block_m(c.block_m)) return fail(W4A16_ERR_UNSUPPORTED, "block_m %d not in {16, 32, 64, 128}", c.block_m);
  if (c.split_k != 0 && c.split_k != 1)
    return fail(W4A16_ERR_UNSUPPORTED, "split_k %d: 0 (stream-K) or 1 (one workgroup per tile)", c.split_k);
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
  p.KC = d->K_pad / 128;
  const int tiles_per_wg = nr * waves;
  p.n_tiles = (p.NT + tiles_per_wg - 1) / tiles_per_wg;
  p.gated = (d->flags & W4A16_DESC_GATE_UP) != 0;
  p.out = out;
  return p;
}

// Workspace carve-up: [combine partials, fp32 T*topk*N][stream-K partial tiles]
size_t combine_region(int32_t T, int32_t topk, int32_t N, bool combine) {
  return combine ? (size_t)round_up((int64_t)T * topk * N * (int64_t)sizeof(float), 256) : 0;
}

size_t streamk_region(const w4a16_config& c, int epi) {
  if (c.split_k != 0) return 0;
  const int wgs = resident_workgroups(c, epi);
  if (wgs <= 0) return 0;
  return w4a16::streamk_partial_bytes(c.block_m / 16, c.nr, c.waves, wgs);
}

w4a16_config default_indexed_config(int32_t block_m) {
  w4a16_config c;
  c.block_m = block_m;
  c.nr = 2;
  c.waves = 4;
  c.split_k = 1;
  c.stages = 2;
  apply_env_overrides(&c);
  return c;
}

// Workgroups of this config the current device keeps resident (stream-K
// grid); 0 when no device is visible or the config is not built.
int resident_workgroups(const w4a16_config& c, int epi) {
  return w4a16::streamk_workgroups(w4a16::kRouteIndexed, epi, c.block_m / 16, c.nr, c.waves, c.stages);
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
  if (!valid_block_m(block_m)) return fail(W4A16_ERR_SHAPE, "block_m %d not in {16, 32, 64, 128}", block_m);
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

w4a16_status w4a16_indexed_config(int32_t block_m, w4a16_config* out) {
  if (!out) return fail(W4A16_ERR_ARG, "out is NULL");
  if (!valid_block_m(block_m)) return fail(W4A16_ERR_ARG, "block_m %d not in {16, 32, 64, 128}", block_m);
  *out = default_indexed_config(block_m);
  return W4A16_OK;
}

// select_config, memoised per argument set of the public call (no
// environment overrides)
w4a16_config cached_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N, int32_t K) {
  const auto key = std::make_tuple(T, topk, E_glob, E_loc, N, K);
  {
    std::lock_guard<std::mutex> g(g_cache_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second;
  }
  const w4a16_config c = select_config(T, topk, E_glob, E_loc);
  std::lock_guard<std::mutex> g(g_cache_mu);
  g_cache[key] = c;
  return c;
}

w4a16_status w4a16_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N,
                          int32_t K, w4a16_config* out) {
  if (!out) return fail(W4A16_ERR_ARG, "out is NULL");
  if (T < 0 || topk <= 0 || E_glob <= 0 || E_loc <= 0 || N <= 0 || K <= 0)
    return fail(W4A16_ERR_ARG, "bad sizes for select");
  *out = cached_select(T, topk, E_glob, E_loc, N, K);
  apply_env_overrides(out);
  return W4A16_OK;
}

w4a16_status w4a16_mxfp4_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N,
                                int32_t K, w4a16_config* out) {
  if (!out) return fail(W4A16_ERR_ARG, "out is NULL");
  if (T < 0 || topk <= 0 || E_glob <= 0 || E_loc <= 0 || N <= 0 || K <= 0)
    return fail(W4A16_ERR_ARG, "bad sizes for select");
  w4a16_config c = cached_select(T, topk, E_glob, E_loc, N, K);
  const double tok_e = (double)T * topk / E_glob;
  if (c.block_m == 128 && tok_e >= kMxHalfTileTokE) c.block_m = 64;
  c.nr = 4;
  c.waves = 4;
  c.split_k = 1;
  c.stages = c.block_m <= 32 ? 4 : 2;
  *out = c;
  apply_env_overrides(out);
  return W4A16_OK;
}

size_t w4a16_moe_gemm_workspace_bytes(const w4a16_weight_desc* desc, int32_t T, int32_t topk,
                                      int32_t combine, const w4a16_config* cfg) {
  if (check_int4_desc(desc) != W4A16_OK || T < 0 || topk <= 0) return 0;
  const w4a16_config c = cfg ? *cfg : default_indexed_config(16);
  const int epi = combine ? w4a16::kEpiWeighted : w4a16::kEpiStore;
  if (check_config(c, w4a16::kRouteIndexed, epi) != W4A16_OK) return 0;
  return combine_region(T, topk, desc->N, combine != 0) + streamk_region(c, epi);
}

w4a16_status w4a16_moe_gemm(const w4a16_weight_desc* desc, const void* packed_w,
                            const void* packed_s, const uint16_t* a, int64_t a_rows,
                            int32_t a_layout, const w4a16_indexed_routing* routing,
                            const float* topk_weights, uint16_t* out,
                            const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                            w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (!routing) return fail(W4A16_ERR_ARG, "routing is NULL");
  const w4a16_indexed_routing& r = *routing;
  const bool combine = topk_weights != nullptr;
  if (!packed_w || !packed_s || !r.sorted_ids || !r.expert_ids || !r.num_tokens_padded)
    return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (r.T < 0 || r.topk <= 0 || r.capacity < 0) return fail(W4A16_ERR_ARG, "bad routing sizes");
  if (r.T > 0 && (!a || !out)) return fail(W4A16_ERR_ARG, "activations or output are NULL");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
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
  const int epi = combine ? w4a16::kEpiWeighted : w4a16::kEpiStore;
  w4a16_config c;
  if (cfg) {
    c = *cfg;
  } else {
    c = default_indexed_config(r.block_m);   // the routing buffers fix block_m
  }
  st = check_config(c, w4a16::kRouteIndexed, epi);
  if (st != W4A16_OK) return st;
  if (c.block_m != r.block_m)
    return fail(W4A16_ERR_LAYOUT, "config block_m=%d differs from the routing's block_m=%d", c.block_m, r.block_m);
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (combine && !r.topk_ids) return fail(W4A16_ERR_ARG, "combine needs routing.topk_ids");
  const size_t comb_bytes = combine_region(r.T, r.topk, desc->N, combine);
  const size_t sk_bytes = streamk_region(c, epi);
  if (c.split_k == 0 && sk_bytes == 0)
    return fail(W4A16_ERR_HIP, "stream-K: could not query the device's resident workgroups");
  const size_t need = comb_bytes + sk_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(W4A16_ERR_WORKSPACE, "this call needs %zu bytes of 16-byte aligned workspace, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (r.T == 0) return W4A16_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, a, combine ? (void*)ws : (void*)out, c.nr, c.waves);
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = a_layout == W4A16_A_TOKEN ? r.topk : a_layout == W4A16_A_SLOT ? 1 : 0;
  p.slot_weight = topk_weights;
  p.grid_blocks = (int32_t)(r.capacity / r.block_m);
  hipError_t e;
  if (c.split_k == 0) {
    p.sk_partial = reinterpret_cast<float*>(ws + comb_bytes);
    const int wgs = resident_workgroups(c, epi);
    e = w4a16::launch_gemm_streamk(w4a16::kRouteIndexed, epi, c.block_m / 16, c.nr, c.waves, c.stages, p,
                                   wgs, s);
  } else {
    e = w4a16::launch_gemm(w4a16::kRouteIndexed, epi, c.block_m / 16, c.nr, c.waves, c.stages, p, s);
  }
  if (e != hipSuccess) return hip_fail(e, "moe_gemm launch");
  if (combine) {
    e = w4a16::launch_combine(static_cast<const float*>(workspace), r.topk_ids, r.T, r.topk,
                              r.first_expert, r.E_loc, desc->N, out, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return W4A16_OK;
}

w4a16_status w4a16_moe_gate_up_silu(const w4a16_weight_desc* desc, const void* packed_w,
                                    const void* packed_s, const uint16_t* x, int64_t x_rows,
                                    const w4a16_indexed_routing* routing, uint16_t* out,
                                    const w4a16_config* cfg, w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (desc->flags != W4A16_DESC_GATE_UP)
    return fail(W4A16_ERR_LAYOUT, "the fused SiLU gate/up call needs a weight packed with w4a16_weight_desc_init_gate_up");
  if (!routing) return fail(W4A16_ERR_ARG, "routing is NULL");
  const w4a16_indexed_routing& r = *routing;
  if (!packed_w || !packed_s || !r.sorted_ids || !r.expert_ids || !r.num_tokens_padded)
    return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (r.T < 0 || r.topk <= 0 || r.capacity < 0) return fail(W4A16_ERR_ARG, "bad routing sizes");
  if (r.T > 0 && (!x || !out)) return fail(W4A16_ERR_ARG, "activations or output are NULL");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(x) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
  if (r.E_loc != desc->E)
    return fail(W4A16_ERR_LAYOUT, "routing has E_loc=%d but the packed weight holds %d experts", r.E_loc, desc->E);
  if (x_rows < r.T) return fail(W4A16_ERR_SHAPE, "activations have %lld rows, need %d", (long long)x_rows, r.T);
  if ((int64_t)r.T * r.topk >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "T*topk too large");
  w4a16_config c = cfg ? *cfg : default_indexed_config(r.block_m);
  if (c.split_k != 1) return fail(W4A16_ERR_UNSUPPORTED, "the fused SiLU gate/up call runs one workgroup per tile (split_k = 1)");
  if (c.nr % 2) return fail(W4A16_ERR_UNSUPPORTED, "the fused SiLU gate/up call needs an even nr (gate and up tiles in pairs)");
  st = check_config(c, w4a16::kRouteIndexed, w4a16::kEpiSilu);
  if (st != W4A16_OK) return st;
  if (c.block_m != r.block_m)
    return fail(W4A16_ERR_LAYOUT, "config block_m=%d differs from the routing's block_m=%d", c.block_m, r.block_m);
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (r.T == 0) return W4A16_OK;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, x, out, c.nr, c.waves);
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = r.topk;
  p.grid_blocks = (int32_t)(r.capacity / r.block_m);
  hipError_t e = w4a16::launch_gemm(w4a16::kRouteIndexed, w4a16::kEpiSilu, c.block_m / 16, c.nr, c.waves,
                                    c.stages, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gate_up_silu launch");
  return W4A16_OK;
}

w4a16_status w4a16_grouped_contiguous(const w4a16_weight_desc* desc, const void* packed_w,
                                      const void* packed_s, const uint16_t* a, int64_t m_rows,
                                      const int32_t* m_indices, uint16_t* out,
                                      const w4a16_config* cfg, w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (m_rows < 0) return fail(W4A16_ERR_ARG, "m_rows < 0");
  if (m_rows > 0 && (!a || !m_indices || !out)) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!packed_w || !packed_s) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
  w4a16_config c;
  if (cfg) {
    c = *cfg;
  } else {
    c.block_m = 128; c.nr = 2; c.waves = 4; c.split_k = 1; c.stages = 2;
    apply_env_overrides(&c);
  }
  st = check_config(c, w4a16::kRouteContiguous, w4a16::kEpiStore);
  if (st != W4A16_OK) return st;
  if (c.split_k != 1) return fail(W4A16_ERR_UNSUPPORTED, "grouped calls run split_k = 1 only");
  if (128 % c.block_m) return fail(W4A16_ERR_UNSUPPORTED, "contiguous layout needs block_m dividing 128");
  if (m_rows % c.block_m) return fail(W4A16_ERR_SHAPE, "m_rows=%lld is not a multiple of block_m=%d (segments are 128-row aligned)", (long long)m_rows, c.block_m);
  if (m_rows >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "m_rows too large");
  if (m_rows == 0) return W4A16_OK;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, a, out, c.nr, c.waves);
  p.m_indices = m_indices;
  p.grid_blocks = (int32_t)(m_rows / c.block_m);
  hipError_t e = w4a16::launch_gemm(w4a16::kRouteContiguous, w4a16::kEpiStore, c.block_m / 16, c.nr,
                                    c.waves, c.stages, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "grouped_contiguous launch");
  return W4A16_OK;
}

w4a16_status w4a16_grouped_masked(const w4a16_weight_desc* desc, const void* packed_w,
                                  const void* packed_s, const uint16_t* a, int32_t max_m,
                                  const int32_t* masked_m, int32_t expected_m, uint16_t* out,
                                  const w4a16_config* cfg, w4a16_stream_t stream) {
  w4a16_status st = check_int4_desc(desc);
  if (st != W4A16_OK) return st;
  if (max_m <= 0) return fail(W4A16_ERR_ARG, "max_m must be positive");
  if (!a || !masked_m || !out || !packed_w || !packed_s) return fail(W4A16_ERR_ARG, "NULL pointer argument");
  if (!aligned16(packed_w) || !aligned16(packed_s) || !aligned16(a) || !aligned16(out))
    return fail(W4A16_ERR_ARG, "packed weights, activations and output must be 16-byte aligned");
  if ((int64_t)desc->E * max_m >= INT32_MAX / 2) return fail(W4A16_ERR_SHAPE, "E * max_m too large");
  w4a16_config c;
  if (cfg) {
    c = *cfg;
  } else {
    if (expected_m <= 0) return fail(W4A16_ERR_ARG, "expected_m must be positive");
    // chosen from the expected rows per group (post, section "Grouped SM90
    // kernels": masked decode picks BLOCK_M from the expected tokens per expert)
    const int want = (int)round_up(std::min(expected_m, 128), 16);
    c.block_m = want <= 16 ? 16 : want <= 32 ? 32 : want <= 64 ? 64 : 128;
    c.nr = 2;
    c.waves = 4;
    c.split_k = 1;
    c.stages = 2;
    apply_env_overrides(&c);
  }
  st = check_config(c, w4a16::kRouteMasked, w4a16::kEpiStore);
  if (st != W4A16_OK) return st;
  if (c.split_k != 1) return fail(W4A16_ERR_UNSUPPORTED, "grouped calls run split_k = 1 only");
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, a, out, c.nr, c.waves);
  p.masked_m = masked_m;
  p.max_m = max_m;
  p.blocks_per_group = (max_m + c.block_m - 1) / c.block_m;
  p.grid_blocks = desc->E * p.blocks_per_group;
  hipError_t e = w4a16::launch_gemm(w4a16::kRouteMasked, w4a16::kEpiStore, c.block_m / 16, c.nr,
                                    c.waves, c.stages, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "grouped_masked launch");
  return W4A16_OK;
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
  return combine_region(T, topk, desc->N, combine != 0);
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
  w4a16_config c;
  if (cfg) {
    c = *cfg;
  } else {
    c.block_m = r.block_m;            // the routing buffers fix block_m
    c.nr = 4;
    c.waves = 4;
    c.split_k = 1;
    c.stages = r.block_m <= 32 ? 4 : 2;
    apply_env_overrides(&c);
  }
  if (!valid_block_m(c.block_m)) return fail(W4A16_ERR_UNSUPPORTED, "block_m %d not in {16, 32, 64, 128}", c.block_m);
  if (c.split_k != 1) return fail(W4A16_ERR_UNSUPPORTED, "the MXFP4 GEMM runs one workgroup per tile (split_k = 1)");
  if (!w4a16::mx_gemm_config_supported(epi, c.block_m / 16, c.nr, c.waves, c.stages))
    return fail(W4A16_ERR_UNSUPPORTED, "MXFP4 tile config block_m=%d nr=%d waves=%d stages=%d not built", c.block_m,
                c.nr, c.waves, c.stages);
  if (c.block_m != r.block_m)
    return fail(W4A16_ERR_LAYOUT, "config block_m=%d differs from the routing's block_m=%d", c.block_m, r.block_m);
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (combine && !r.topk_ids) return fail(W4A16_ERR_ARG, "combine needs routing.topk_ids");
  const size_t need = combine_region(r.T, r.topk, desc->N, combine);
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
  p.grid_blocks = (int32_t)(r.capacity / r.block_m);
  hipError_t e = w4a16::launch_mx_gemm(epi, c.block_m / 16, c.nr, c.waves, c.stages, p, s);
  if (e != hipSuccess) return hip_fail(e, "mxfp4_moe_gemm launch");
  if (combine) {
    e = w4a16::launch_combine(static_cast<const float*>(workspace), r.topk_ids, r.T, r.topk, r.first_expert,
                              r.E_loc, desc->N, out, s);
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
  w4a16_config c;
  if (cfg) {
    c = *cfg;
  } else {
    c.block_m = r.block_m;
    c.nr = 4;
    c.waves = 4;
    c.split_k = 1;
    c.stages = r.block_m <= 32 ? 4 : 2;
    apply_env_overrides(&c);
  }
  if (!valid_block_m(c.block_m)) return fail(W4A16_ERR_UNSUPPORTED, "block_m %d not in {16, 32, 64, 128}", c.block_m);
  if (c.split_k != 1 || c.nr != 4)
    return fail(W4A16_ERR_UNSUPPORTED, "the fused A4W4 gate/up call runs one workgroup per tile with nr = 4");
  if (!w4a16::mx_gemm_config_supported(w4a16::kEpiSiluMx, c.block_m / 16, c.nr, c.waves, c.stages))
    return fail(W4A16_ERR_UNSUPPORTED, "MXFP4 tile config block_m=%d nr=%d waves=%d stages=%d not built", c.block_m,
                c.nr, c.waves, c.stages);
  if (c.block_m != r.block_m)
    return fail(W4A16_ERR_LAYOUT, "config block_m=%d differs from the routing's block_m=%d", c.block_m, r.block_m);
  if (r.capacity % r.block_m) return fail(W4A16_ERR_CAPACITY, "capacity not a multiple of block_m");
  if (r.T == 0) return W4A16_OK;
  w4a16::GemmParams p = base_params(desc, packed_w, packed_s, reinterpret_cast<const uint16_t*>(x_codes),
                                    out_codes, c.nr, c.waves);
  p.a_scale = x_scales;
  p.out_scale = out_scales;
  p.sorted_ids = r.sorted_ids;
  p.expert_ids = r.expert_ids;
  p.num_tokens_padded = r.num_tokens_padded;
  p.sentinel = r.T * r.topk;
  p.a_row_div = r.topk;
  p.grid_blocks = (int32_t)(r.capacity / r.block_m);
  hipError_t e = w4a16::launch_mx_gemm(w4a16::kEpiSiluMx, c.block_m / 16, c.nr, c.waves, c.stages, p,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxfp4_gate_up_silu launch");
  return W4A16_OK;
}

}  // extern "C"

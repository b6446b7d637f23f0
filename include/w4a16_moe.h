/*
 * w4a16_moe.h -- C ABI of the W4A16 INT4 mixture-of-experts expert GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (Chord W4A16 MoE post, "vLLM x Novita AI: Chord, a faster
 * INT4 MoE for Kimi K2.x"; summary and section "Kernel optimisation"):
 * BF16 activations times INT4 weights that carry one BF16 scale per 32
 * consecutive K elements.  A weight code q in 0..15 stands for
 * bf16_rne((q - 8) * s) -- subtract, then scale, rounded once to BF16 (section
 * "H200 and Blackwell indexed decode") -- and the products are summed in FP32
 * (section "vLLM integration": FP16 accumulation is not offered).  Every
 * output element is rounded once to BF16 (round to nearest even).
 *
 * Conventions for every call below
 *  - Tensor pointers are DEVICE pointers unless stated.  The caller allocates
 *    and owns all device memory (activations, packed weights, routing
 *    buffers, outputs, workspace); the library never allocates or frees
 *    device memory and keeps no device state.
 *  - BF16 tensors are passed as uint16_t bit patterns, row-major, no padding
 *    between rows unless a stride is given.
 *  - Calls that take a stream enqueue work on it and return without waiting,
 *    except where "synchronises" is stated.  A NULL stream is the default
 *    stream.  No call reads device memory back to the host unless stated, so
 *    the align + GEMM sequence can be captured in a HIP graph.
 *  - Arguments are checked on the host before anything is enqueued.  On a
 *    bad argument the call returns a negative w4a16_status, enqueues nothing,
 *    and w4a16_last_error() describes the problem (thread-local string, valid
 *    until the next failing call on the same thread).
 *  - Calls that overlap on one stream are ordered by it; the library itself
 *    is thread-safe (its only state is a mutex-guarded host cache).
 */
#ifndef W4A16_MOE_H
#define W4A16_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t, kept opaque so this header needs no HIP include. */
typedef void* w4a16_stream_t;

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_ARG = -1,          /* NULL pointer, negative size, misaligned pointer */
  W4A16_ERR_SHAPE = -2,        /* unsupported shape: K % 32 != 0, N % 16 != 0, ... */
  W4A16_ERR_LAYOUT = -3,       /* weight descriptor corrupt or not matching the call */
  W4A16_ERR_UNSUPPORTED = -4,  /* tile configuration not built into this library */
  W4A16_ERR_CAPACITY = -5,     /* routing buffer smaller than the worst case needs */
  W4A16_ERR_ROUTING = -6,      /* validation found an expert id outside [0, E_glob) */
  W4A16_ERR_HIP = -7,          /* the HIP runtime reported an error */
  W4A16_ERR_WORKSPACE = -8     /* workspace missing or smaller than required */
} w4a16_status;

/* Description of the last non-OK status on this thread ("" if none). */
const char* w4a16_last_error(void);

/* ABI version of this header (W4A16_ABI_VERSION). */
#define W4A16_ABI_VERSION 8
int32_t w4a16_abi_version(void);

/* ------------------------------------------------------------------------
 * Packed weights.
 *
 * Input format (Chord post, section "Grouped SM90 kernels", operator listing):
 * unsigned INT4 codes [E, N, K], here one code per byte (values 0..15; the
 * upper four bits of each byte are ignored), and BF16 scales [E, N, K/32],
 * scale index kk / 32 along K.  The post packs once at model load (section
 * "Indexed kernels": configuration and layout are fixed before packing);
 * here one packed layout serves every call and every tile configuration, so
 * nothing about the call has to be known when packing.
 *
 * Packed layout (all little-endian), with NT = N / 16, KP = K rounded up to
 * 128, KC = KP / 128, KC2 = ceil(KC / 2):
 *   packed_w : uint32 words [E][NT][KC][64 lanes][4 words]
 *     lane l = 16 * g + i holds row n = 16 * tile + i; word j of that lane
 *     holds the 8 codes of K indices kk = 128 * c + 32 * g + 8 * j + e,
 *     e = 0..7, code e at bit 4 * (e / 2) + 16 * (e % 2).  Codes for kk >= K
 *     are 8 (weight 0).  Each lane's word is exactly one MFMA operand
 *     fragment of 8 consecutive K values, and one lane's four words span one
 *     32-wide scale group.
 *   packed_s : uint32 words [E][NT][KC2][64 lanes]
 *     lane l = 16 * g + i of (tile, chunk pair m) holds the bf16 scales
 *     scale[n = 16 * tile + i][4 * c + g] for c = 2m (low half) and
 *     c = 2m + 1 (high half), 0 past K / 32: the one scale each of its
 *     chunks needs, so a wave's scales for a chunk pair are one 256-byte run.
 *   packed_w is E * NT * KC * 1024 bytes, packed_s is E * NT * KC2 * 256.
 *
 * Gate/up interleaved (flag W4A16_DESC_GATE_UP): a gate/up projection whose
 * rows [0, N/2) are the gate and [N/2, N) the up rows is packed with their
 * 16-row tiles alternating: packed tile 2i holds gate tile i, packed tile
 * 2i + 1 up tile i.  Every call on such a weight still produces output
 * columns in the logical order; the fused SiLU gate/up call needs it.
 * ---------------------------------------------------------------------- */
#define W4A16_DESC_MAGIC 0x16A4B0E5u /* arbitrary tag */
#define W4A16_DESC_VERSION 2u
#define W4A16_DESC_GATE_UP 1         /* flags: gate/up tiles interleaved */
#define W4A16_DESC_MXFP4 2           /* flags: MXFP4 weight (A4W4 calls only); may be
                                        combined with W4A16_DESC_GATE_UP */

typedef struct {
  uint32_t magic;       /* W4A16_DESC_MAGIC */
  uint32_t version;     /* W4A16_DESC_VERSION */
  int32_t E, N, K;      /* experts, output features, reduction length */
  int32_t K_pad;        /* KP above */
  int32_t chunks;       /* KC above */
  int32_t group;        /* 32 */
  int32_t flags;        /* 0, W4A16_DESC_GATE_UP, W4A16_DESC_MXFP4 or both MXFP4 bits */
  int32_t reserved;     /* 0 */
  uint64_t w_bytes;     /* size of packed_w */
  uint64_t s_bytes;     /* size of packed_s */
  uint64_t check;       /* checksum of the fields above */
} w4a16_weight_desc;

/* Fill *out for an [E, N, K] weight (host only, no device work).
 * Errors: ERR_ARG (out NULL, E/N/K <= 0), ERR_SHAPE (K % 32 or N % 16). */
w4a16_status w4a16_weight_desc_init(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out);

/* The same for a gate/up weight packed with interleaved tiles (flag
 * W4A16_DESC_GATE_UP): rows [0, N/2) gate, [N/2, N) up.
 * Errors: as above, and ERR_SHAPE when N % 32 != 0. */
w4a16_status w4a16_weight_desc_init_gate_up(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out);

/* Pack codes [E, N, K] (uint8) and scales [E, N, K/32] (bf16) into the
 * layout above.  `desc` must come from w4a16_weight_desc_init for the same
 * E, N, K; packed_w / packed_s must be 16-byte aligned and desc->w_bytes /
 * desc->s_bytes long.  Inputs are read, outputs fully written.
 * Errors: ERR_ARG, ERR_LAYOUT (bad desc), ERR_HIP. */
w4a16_status w4a16_pack_w4(const uint8_t* codes, const uint16_t* scales,
                           const w4a16_weight_desc* desc, void* packed_w, void* packed_s,
                           w4a16_stream_t stream);

/* ------------------------------------------------------------------------
 * Routing align: topk_ids -> sorted_ids / expert_ids / num_tokens_padded.
 *
 * (Chord post, section "Two kernel families": the indexed family consumes
 * these three buffers; section "vLLM integration": they are over-allocated so
 * no routed count is read back to the host; Figure 3: padding lives in
 * sentinel index values, activations are not padded.)
 *
 * Slot s = t * topk + j.  A slot is local when first_expert <= topk_ids[t][j]
 * < first_expert + E_loc; its local expert is the difference.  For each local
 * expert e in order, its slot ids ascending, then the sentinel T * topk until
 * the segment length is a multiple of block_m.  expert_ids[b] = local expert
 * of block b (rows b*block_m .. b*block_m + block_m - 1), -1 for blocks past
 * the padded total.  *num_tokens_padded = padded total (device int32).
 * sorted_ids past the padded total hold the sentinel.  Ids outside
 * [0, E_glob) are treated as not local.
 *
 * capacity = length of sorted_ids, >= w4a16_align_capacity(); expert_ids has
 * capacity / block_m entries.  block_m in {16, 32, 64, 128, 256}.  E_loc <= 1024.
 * validate != 0 synchronises: topk_ids are copied to the host and checked
 * to lie in [0, E_glob) before anything is enqueued (ERR_ROUTING otherwise).
 * Errors: ERR_ARG, ERR_SHAPE, ERR_CAPACITY, ERR_ROUTING, ERR_HIP. */
int64_t w4a16_align_capacity(int32_t T, int32_t topk, int32_t E_loc, int32_t block_m);

w4a16_status w4a16_moe_align(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E_glob,
                             int32_t first_expert, int32_t E_loc, int32_t block_m,
                             int32_t* sorted_ids, int32_t* expert_ids,
                             int32_t* num_tokens_padded, int64_t capacity, int32_t validate,
                             w4a16_stream_t stream);

/* ------------------------------------------------------------------------
 * Tile configuration and its selection.
 *
 * The post picks block_m from tokens per expert, tok_e = routed rows /
 * experts, not from total tokens (section "H200 prefill and TP8": below about
 * 80 rows per expert a search over block counts on sampled routing, above it
 * a fit of padded expert rows), and gates splitting of K by shape (same
 * section: split only where the plain grid leaves the machine underfilled).
 * The grouped calls choose their own tiles and accept no indexed config or
 * tuning override (section "Grouped SM90 kernels").  w4a16_select applies
 * these rules with gfx950 constants; a config may also be given explicitly.
 * ---------------------------------------------------------------------- */
#define W4A16_ROUTE_INDEXED 0     /* sorted_ids / expert_ids / num_tokens_padded */
#define W4A16_ROUTE_CONTIGUOUS 1  /* grouped, m_indices */
#define W4A16_ROUTE_MASKED 2      /* grouped, masked_m */

typedef struct {
  int32_t block_m;   /* rows per tile: 16, 32, 64, 128 or 256.  Indexed
                        calls: the routing's block_m or a divisor of it (a
                        tile then covers part of a routed block) */
  int32_t nr;        /* 16-row weight tiles per wave: 2 or 4; or 1: one
                        16-row weight tile per workgroup whose waves (8)
                        split K and sum their partials in LDS (block_m 16,
                        split_k 1, K a multiple of 128, indexed routing; in
                        the fused SiLU call one gate / up tile pair per
                        workgroup) */
  int32_t waves;     /* waves per workgroup: 4 (8 for some tiles) */
  int32_t split_k;   /* 1: one workgroup per (block, N tile), whole K;
                        2, 4, 8, 16: that many workgroups per tile, each over
                        an equal share of the pairs of 128-K chunks (at most
                        one slice per pair); each leaves fp32 partials in workspace
                        and the last to finish sums them in slice order
                        (results independent of timing, but not bit-identical
                        to split_k = 1);
                        0: stream-K -- the workgroups the device keeps resident
                        each take an equal share of (tile, pair of 128-K
                        chunks) units;
                        tiles cut between two workgroups are finished from
                        fp32 partials in workspace, summed in K order (results
                        then depend on the device's CU count, not on timing);
                        indexed routing only */
  int32_t stages;    /* K chunks of weights each wave keeps in flight: 2, or 4
                        for block_m <= 32 with nr = 2 */
  int32_t kind;      /* W4A16_ROUTE_*: the routing the config is for.  A call
                        given a config of another kind returns ERR_ARG */
  int32_t combine_cols; /* top-k combine only: output columns per pass.  The
                        call runs the GEMM and the combine over one range of
                        this many columns after another, so the fp32 per-slot
                        partials of a pass (T * topk * combine_cols * 4
                        bytes of workspace) can stay in the last-level cache
                        between the two.  0: the library's choice (all of N
                        when the expected local partials fit 240 MiB, else the
                        fewest passes that do, in whole workgroup tiles); else
                        a multiple of 16 (ERR_ARG otherwise).  Results do not
                        depend on it.  Selection returns 0. */
} w4a16_config;

/* The config w4a16_select gives for indexed routing aligned to block_m (the
 * routing buffers fix block_m; the rest is chosen as w4a16_select does):
 * what w4a16_moe_gemm and w4a16_moe_gate_up_silu use when their cfg is NULL.
 * A 256-row routing gives the 256-row tile (128-row tiles when K is not a
 * multiple of 128).  Host only; environment overrides W4A16_NR, W4A16_WAVES,
 * W4A16_SPLIT_K, W4A16_STAGES applied.
 * Errors: ERR_ARG. */
w4a16_status w4a16_indexed_config(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N,
                                  int32_t K, int32_t block_m, w4a16_config* out);

/* Choose a config (host only; memoised per argument set, so repeated calls
 * cost about a microsecond).
 *  kind W4A16_ROUTE_INDEXED: T tokens, top-k, E_glob model experts of which
 *    E_loc are held here, projection [N, K]; expected_m ignored.
 *    tok_e = T * topk / E_glob.  Below 48 rows per expert block_m minimises
 *    the total block count over {16, 32, 64} on a seeded multinomial sample
 *    of the routing (ties to the smaller block); from 48 on, 128 (with K a
 *    multiple of 128: the prefill tile, nr 4); from 128 on with K a
 *    multiple of 128, 256 (the 256-row tile: nr 2, eight waves, split_k
 *    1).  split_k doubles from 1 while the sampled grid (routed blocks x N tiles x
 *    split_k) stays below one round of resident workgroups on 256 CUs and
 *    each slice keeps at least four 128-K chunks; a block_m 16 grid that
 *    would split K four or more ways (K a multiple of 128) takes nr 1 with
 *    eight waves splitting K instead, split_k 1.
 *  kind W4A16_ROUTE_CONTIGUOUS: T = rows of the contiguous layout, E_loc =
 *    experts, [N, K]; topk, E_glob and expected_m ignored.  block_m 128 when
 *    the grid of 128-row blocks fills the machine, else 64.
 *  kind W4A16_ROUTE_MASKED: T = max_m, E_loc = groups, [N, K], expected_m > 0
 *    the expected rows per group; topk and E_glob ignored.  block_m covers
 *    1.3 * expected_m rows for K >= 4096 (a second M tile re-reads all of
 *    K) and ceil(1.25 * expected_m, 8) for shorter K, rounded up to a built
 *    block (at most 128); stages 4 (512 K elements in flight) for block_m
 *    <= 32, else 2.
 * Environment overrides W4A16_BLOCK_M, W4A16_NR, W4A16_WAVES,
 * W4A16_SPLIT_K, W4A16_STAGES apply to indexed configs only; a grouped
 * selection with any of them set returns ERR_ARG.
 * Errors: ERR_ARG. */
w4a16_status w4a16_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc, int32_t N,
                          int32_t K, int32_t kind, int32_t expected_m, w4a16_config* out);

/* ------------------------------------------------------------------------
 * Indexed MoE GEMM (the post's indexed family).
 * ---------------------------------------------------------------------- */
typedef struct {
  const int32_t* sorted_ids;         /* from w4a16_moe_align */
  const int32_t* expert_ids;
  const int32_t* num_tokens_padded;  /* device scalar */
  int64_t capacity;                  /* length of sorted_ids */
  int32_t block_m;                   /* a multiple of the config's block_m */
  int32_t T, topk;                   /* sentinel is T * topk */
  const int32_t* topk_ids;           /* [T, topk]; read only by the combine */
  int32_t first_expert, E_loc;       /* local expert range; read only by the combine */
  int32_t E_glob;                    /* model experts (tok_e = T * topk / E_glob for
                                        the config chosen when cfg is NULL) */
} w4a16_indexed_routing;

/* Bytes of workspace w4a16_moe_gemm needs for this weight, routing shape,
 * combine flag and config (NULL: the config the call would choose):
 *   - split_k > 1: 4 bytes of arrival counter per tile that may be split,
 *     then that many tiles' fp32 slices;
 *   - combine != 0: the fp32 per-slot partials of one pass,
 *     T * topk * cols * 4 bytes (cols: the config's combine_cols, or the
 *     library's choice for it), then T bytes of local-slot counts per token
 *     (each region rounded up to 256 bytes);
 *   - split_k = 0: two partial tiles per resident workgroup of the current
 *     device.
 * The workspace must be zero-filled once before its first use (the arrival
 * counters start at zero); every call leaves the counters at zero again, so
 * the same workspace serves any number of later calls on one stream.  The
 * other bytes are scratch of the call.  Returns 0 on bad arguments. */
size_t w4a16_moe_gemm_workspace_bytes(const w4a16_weight_desc* desc, const w4a16_indexed_routing* routing,
                                      int32_t combine, const w4a16_config* cfg);

/* Row layouts of the activations `a` (argument a_layout). */
#define W4A16_A_TOKEN 0   /* one row per token, [T, K] (gate/up input) */
#define W4A16_A_SLOT 1    /* one row per slot t * topk + j, [T * topk, K] */
#define W4A16_A_SORTED 2  /* one row per sorted position p (row p serves the
                             slot sorted_ids[p]), [capacity, K]: the output of
                             w4a16_moe_gate_up_silu, read without a gather */

/* out = routed W4A16 product.
 *  a          : bf16 activations, row stride K (desc->K), rows as a_layout
 *               says; a_rows = rows in `a`.
 *  topk_weights == NULL: per-slot output out[T * topk, N]; only local slots
 *               are written, other rows keep their contents.
 *  topk_weights != NULL (float32 [T, topk]): top-k-weighted combine,
 *               out[t] = bf16(sum over local j of w[t][j] * (a_row . W[e]^T))
 *               with fp32 products, summed in j order, one rounding; tokens
 *               without local slots get 0; every row of out[T, N] written
 *               (a token with one local slot is written by the GEMM itself:
 *               bf16 of that one product).
 *               Needs workspace (fp32 partials per slot).
 *               A weight packed with interleaved gate/up tiles
 *               (W4A16_DESC_GATE_UP) is rejected here (ERR_LAYOUT): the
 *               combine belongs to the down projection.
 *  workspace  : w4a16_moe_gemm_workspace_bytes() bytes, zero-filled before
 *               its first use (see there).
 *  cfg        : NULL: w4a16_indexed_config for the routing's shape and
 *               block_m.  A config of another routing kind: ERR_ARG.
 * Sizes: activation rows are addressed with 32-bit byte offsets, so the rows
 * the call may read (T, T * topk or capacity by a_layout) times K * 2 bytes
 * must not exceed 4 GiB (ERR_SHAPE otherwise).
 * Pointers: packed_w, packed_s, a, out, workspace 16-byte aligned.
 * Errors: ERR_ARG, ERR_LAYOUT, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP. */
w4a16_status w4a16_moe_gemm(const w4a16_weight_desc* desc, const void* packed_w,
                            const void* packed_s, const uint16_t* a, int64_t a_rows,
                            int32_t a_layout, const w4a16_indexed_routing* routing,
                            const float* topk_weights, uint16_t* out,
                            const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                            w4a16_stream_t stream);

/* w4a16_moe_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, outputs and errors as w4a16_moe_gemm, without the workspace:
 * the call uses the library's own scratch array instead, W4A16_SCRATCH_BYTES
 * per GPU (allocated with the library's code on each device it runs on and
 * held until the process ends; the call itself allocates nothing).  A call
 * needing more scratch than that (w4a16_moe_gemm_workspace_bytes) returns
 * ERR_WORKSPACE: 128 MiB covers, for example, the top-k combine of 576
 * tokens x top-8 x N = 7168.  All calls on one GPU share its array and each
 * starts by clearing the part it needs zeroed, so calls that overlap on one
 * GPU (different streams, or threads) race and give wrong results: order
 * them on one stream.  The first call on a device looks up the array's
 * device address (no device work). */
#define W4A16_SCRATCH_BYTES ((size_t)128 << 20)
w4a16_status w4a16_moe_gemm_noalloc(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                    const uint16_t* a, int64_t a_rows, int32_t a_layout,
                                    const w4a16_indexed_routing* routing, const float* topk_weights, uint16_t* out,
                                    const w4a16_config* cfg, w4a16_stream_t stream);

/* Gate/up projection with the activation between the two projections
 * fused into its epilogue, written in sorted order for the down projection.
 * (The post's layer numbers exclude the activation, section "Measurement";
 * fusing it and keeping rows in sorted order removes a launch, a pass over
 * the intermediate and the down projection's row gather.)
 *  desc       : a W4A16_DESC_GATE_UP weight, N = 2 * I.
 *  x          : bf16 token rows [x_rows, K], x_rows >= routing->T.
 *  out        : bf16 [routing->capacity, I]; for each sorted position p that
 *               holds a local slot s = sorted_ids[p] = t * topk + j:
 *               out[p][n] = bf16(silu(g) * u), g = bf16(x[t] . W_gate[n]),
 *               u = bf16(x[t] . W_up[n]) (the same bf16 values the unfused
 *               per-slot call writes), silu(g) = g / (1 + exp(-g)) in fp32.
 *               Padding positions are left unwritten (the down call never
 *               uses them).
 *  cfg        : NULL: w4a16_indexed_config for the routing's shape and
 *               block_m, without splitting; one workgroup per tile
 *               (split_k = 1), nr even or 1.  A config of another routing
 *               kind: ERR_ARG.
 * Sizes: x_rows * K * 2 bytes at most 4 GiB (ERR_SHAPE).
 * Pointers 16-byte aligned.
 * Errors: ERR_ARG, ERR_LAYOUT (not a gate/up weight), ERR_SHAPE,
 * ERR_UNSUPPORTED, ERR_HIP. */
w4a16_status w4a16_moe_gate_up_silu(const w4a16_weight_desc* desc, const void* packed_w,
                                    const void* packed_s, const uint16_t* x, int64_t x_rows,
                                    const w4a16_indexed_routing* routing, uint16_t* out,
                                    const w4a16_config* cfg, w4a16_stream_t stream);

/* ------------------------------------------------------------------------
 * Grouped layouts (the post's grouped family, section "Grouped SM90
 * kernels": contiguous prefill and masked decode; same packed weights here).
 * The grouped calls own their tile choice: cfg is NULL (the call selects
 * with w4a16_select for its kind) or a config w4a16_select returned for that
 * kind; an indexed config, or any W4A16_* tuning override in the
 * environment, returns ERR_ARG (section "Grouped SM90 kernels": grouped
 * dispatch accepts no indexed block_m or tuning override).
 * ---------------------------------------------------------------------- */

/* Contiguous: a [m_rows, K] holds each expert's rows back to back, each
 * expert's segment starting at a multiple of 128 rows; m_indices[r] is the
 * expert of row r or -1 on padding.  out[m_rows, N]: rows with
 * m_indices[r] >= 0 written as bf16(a[r] . W[m_indices[r]]^T); -1 rows are
 * left unwritten.  cfg: see above (its block_m divides 128).
 * workspace: w4a16_grouped_workspace_bytes(desc, W4A16_ROUTE_CONTIGUOUS,
 * m_rows, 0, cfg) bytes, zero-filled before first use, or NULL when that is
 * 0.  Sizes: m_rows * K * 2 bytes at most 4 GiB (ERR_SHAPE).
 * Errors: ERR_ARG, ERR_LAYOUT, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP. */
w4a16_status w4a16_grouped_contiguous(const w4a16_weight_desc* desc, const void* packed_w,
                                      const void* packed_s, const uint16_t* a, int64_t m_rows,
                                      const int32_t* m_indices, uint16_t* out,
                                      const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                                      w4a16_stream_t stream);

/* Masked: a [E, max_m, K]; masked_m[g] (device int32, E entries) valid rows
 * of group g; out flat [E * max_m, N], row g * max_m + r written for
 * r < min(masked_m[g], max_m), other rows unwritten.  expected_m (host, > 0)
 * only steers the tile choice.  cfg: see above.  workspace:
 * w4a16_grouped_workspace_bytes(desc, W4A16_ROUTE_MASKED, max_m,
 * expected_m, cfg) bytes, zero-filled before first use, or NULL when that is
 * 0.  Sizes: E * max_m * K * 2 bytes at most 4 GiB (ERR_SHAPE).
 * Errors: ERR_ARG, ERR_LAYOUT, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP. */
w4a16_status w4a16_grouped_masked(const w4a16_weight_desc* desc, const void* packed_w,
                                  const void* packed_s, const uint16_t* a, int32_t max_m,
                                  const int32_t* masked_m, int32_t expected_m, uint16_t* out,
                                  const w4a16_config* cfg, void* workspace, size_t workspace_bytes,
                                  w4a16_stream_t stream);

/* Workspace bytes of a grouped call (kind W4A16_ROUTE_CONTIGUOUS with
 * rows = m_rows, or W4A16_ROUTE_MASKED with rows = max_m and its
 * expected_m) with cfg (NULL: the call's own selection): split-K arrival
 * counters and slices when the config splits K, else 0.  Returns 0 on bad
 * arguments. */
size_t w4a16_grouped_workspace_bytes(const w4a16_weight_desc* desc, int32_t kind, int64_t rows,
                                     int32_t expected_m, const w4a16_config* cfg);

/* ------------------------------------------------------------------------
 * A4W4: MXFP4 activations x MXFP4 weights.
 *
 * The AMD Kimi K3 post ("Blick hinter die Kulissen der Kimi-K3-Optimierung",
 * technical note "Experten-Routing und Praezision") describes A4W4 as the
 * MoE activations going from eight to four bits while the weights stay
 * 4-bit, and serves MXFP4 model weights on MI355X.  MXFP4 as in the OCP
 * Microscaling specification: FP4 E2M1 elements (values 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6 and their negatives; code bit 3 is the sign), two per byte with
 * element 2i in the low nibble, and one E8M0 scale byte 2^(c - 127) per 32
 * consecutive elements along K.  Routing is the indexed routing above.
 * ---------------------------------------------------------------------- */

/* Fill *out for an MXFP4 [E, N, K] weight (flag W4A16_DESC_MXFP4; host only).
 * Packed layout, NT = N / 16, KC = K / 128:
 *   packed_w : [E][NT][KC][64 lanes][16 bytes]; lane l = 16 g + i of (tile,
 *     chunk c) holds row n = 16 tile + i, code bytes [64 c + 16 g, + 16) of
 *     that row (the 32 elements of block 4 c + g: one scaled-FP4 MFMA operand
 *     fragment);
 *   packed_s : [E][NT][KC][64 lanes] bytes, the E8M0 scale of that block.
 *   packed_w is E * N * K / 2 bytes, packed_s is E * N * K / 32.
 * Errors: ERR_ARG (out NULL, E/N/K <= 0), ERR_SHAPE (K % 128 or N % 16). */
w4a16_status w4a16_mxfp4_weight_desc_init(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out);

/* The same for an MXFP4 gate/up weight (rows [0, N/2) gate, [N/2, N) up)
 * packed with its gate and up tiles alternating (flags W4A16_DESC_MXFP4 |
 * W4A16_DESC_GATE_UP), as the fused A4W4 gate/up call needs; every other
 * call on it still sees the logical column order.
 * Errors: as above, and ERR_SHAPE when N % 64 != 0. */
w4a16_status w4a16_mxfp4_weight_desc_init_gate_up(int32_t E, int32_t N, int32_t K, w4a16_weight_desc* out);

/* Pack MXFP4 weights: codes [E, N, K/2] bytes (two per byte) and E8M0
 * scales [E, N, K/32] bytes into the layout above.  codes 16-byte aligned;
 * packed_w / packed_s 16-byte aligned and desc->w_bytes / desc->s_bytes long.
 * Errors: ERR_ARG, ERR_LAYOUT (desc not from w4a16_mxfp4_weight_desc_init), ERR_HIP. */
w4a16_status w4a16_mxfp4_pack(const uint8_t* codes, const uint8_t* scales, const w4a16_weight_desc* desc,
                              void* packed_w, void* packed_s, w4a16_stream_t stream);

/* Quantise bf16 rows x [rows, K] (K % 32 == 0) to MXFP4: codes [rows, K/2]
 * bytes and scales [rows, K/32] bytes.  Per row and per block of 32: shared
 * exponent floor(log2 max|v|) - 2 clamped to [-127, 127] (scale code 0 for a
 * block of zeros), elements rounded to the nearest E2M1 value with ties to
 * the even code, magnitudes past 6 clamped to 6, sign bit copied from the
 * input (the OCP conversion).  Inf / NaN inputs give unspecified codes.
 * x and codes 16-byte aligned.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_HIP. */
w4a16_status w4a16_mxfp4_quant(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                               w4a16_stream_t stream);

/* w4a16_mxfp4_quant on the per-slot rows x [T * topk][K] (the down
 * projection's input, row s = slot s = t * topk + j), converting only the
 * rows of slots routed to a local expert (first_expert <= topk_ids[s] <
 * first_expert + E_loc); the codes and scales of other rows are left as they
 * are.  These are the rows w4a16_mxfp4_moe_gemm with W4A16_A_SLOT reads.
 * topk_ids: device int32 [T][topk].  Errors as w4a16_mxfp4_quant, and
 * ERR_ARG for topk <= 0, E_loc <= 0 or a NULL topk_ids. */
w4a16_status w4a16_mxfp4_quant_local_slots(const uint16_t* x, const int32_t* topk_ids, int32_t T, int32_t topk,
                                           int32_t first_expert, int32_t E_loc, int32_t K, uint8_t* codes,
                                           uint8_t* scales, w4a16_stream_t stream);

/* Choose a config for the A4W4 GEMM (host only; arguments, memoisation and
 * environment overrides as w4a16_select): block_m as w4a16_select, except
 * that where it gives 128 or 256 and tokens per expert T * topk / E_glob are
 * at least 128, 64 (the MXFP4 kernel keeps more waves resident on 64-row
 * blocks and measured faster there); nr 4, waves 4, one workgroup per
 * tile, stages 4 for block_m <= 32, else 2 -- except where w4a16_select
 * gives the tile whose waves split K (block_m 16, nr 1): there the A4W4
 * K-split tile, nr 1 with eight waves.  Errors: ERR_ARG. */
w4a16_status w4a16_mxfp4_select(int32_t T, int32_t topk, int32_t E_glob, int32_t E_loc,
                                int32_t N, int32_t K, w4a16_config* out);

/* Bytes of workspace w4a16_mxfp4_moe_gemm needs (the top-k combine's fp32
 * partials; 0 without combine). */
size_t w4a16_mxfp4_moe_gemm_workspace_bytes(const w4a16_weight_desc* desc, int32_t T, int32_t topk,
                                            int32_t combine);

/* out = routed A4W4 product on MXFP4 activations (a_codes [a_rows, K/2],
 * a_scales [a_rows, K/32], rows as a_layout says: W4A16_A_TOKEN,
 * W4A16_A_SLOT, or W4A16_A_SORTED for the rows w4a16_mxfp4_gate_up_silu
 * writes) and an MXFP4 weight.  Outputs exactly as w4a16_moe_gemm:
 * per-slot bf16 rows (topk_weights NULL) or the top-k-weighted combine into
 * out[T, N] with fp32 partials summed in j order and rounded once.
 * Accumulation is fp32 (the MFMA's); each output is rounded once to bf16.
 *  cfg : NULL: block_m from the routing (64 on a 256-row routing), nr 4,
 *        four waves, stages 4 for block_m <= 32 else 2 -- or, on a 16-row
 *        routing where w4a16_mxfp4_select takes it, nr 1 with eight waves
 *        (one 16-row weight tile per workgroup, its waves splitting K);
 *        split_k must be 1.  A config's block_m divides the routing's.
 * Pointers: packed_w, packed_s, a_codes, out, workspace 16-byte aligned.
 * Errors: ERR_ARG, ERR_LAYOUT (not an MXFP4 weight, E_loc mismatch, or a
 * block_m that does not divide the routing's), ERR_SHAPE, ERR_UNSUPPORTED,
 * ERR_WORKSPACE, ERR_HIP. */
w4a16_status w4a16_mxfp4_moe_gemm(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                  const uint8_t* a_codes, const uint8_t* a_scales, int64_t a_rows,
                                  int32_t a_layout, const w4a16_indexed_routing* routing,
                                  const float* topk_weights, uint16_t* out, const w4a16_config* cfg,
                                  void* workspace, size_t workspace_bytes, w4a16_stream_t stream);

/* Fused A4W4 gate/up: the gate/up product on MXFP4 token rows (x_codes
 * [x_rows, K/2], x_scales [x_rows, K/32], x_rows >= routing->T) with a
 * W4A16_DESC_MXFP4 | W4A16_DESC_GATE_UP weight (N = 2 I), the activation
 * bf16(silu(g) * u) of its bf16-rounded per-slot values (as
 * w4a16_moe_gate_up_silu), quantised to MXFP4 by the conversion of
 * w4a16_mxfp4_quant, written for each sorted position p that holds a local
 * slot: out_codes[p] ([capacity, I/2] bytes), out_scales[p] ([capacity,
 * I/32]).  Padding positions are left unwritten; the down projection reads
 * the rows with a_layout = W4A16_A_SORTED.
 *  cfg : NULL: block_m from the routing (64 on a 256-row routing), nr 4,
 *        four waves -- or, on a 16-row routing where w4a16_mxfp4_select
 *        takes it, nr 1 with eight waves (the K-split tile, here four packed
 *        tiles, one activation block, per workgroup); nr must be 4 or 1 and
 *        split_k 1, and block_m divide the routing's.
 * Pointers: packed_w, packed_s, x_codes, out_codes 16-byte aligned.
 * Errors: ERR_ARG, ERR_LAYOUT (not an MXFP4 gate/up weight, or block_m not
 * dividing the routing's), ERR_SHAPE, ERR_UNSUPPORTED, ERR_HIP. */
w4a16_status w4a16_mxfp4_gate_up_silu(const w4a16_weight_desc* desc, const void* packed_w, const void* packed_s,
                                      const uint8_t* x_codes, const uint8_t* x_scales, int64_t x_rows,
                                      const w4a16_indexed_routing* routing, uint8_t* out_codes,
                                      uint8_t* out_scales, const w4a16_config* cfg, w4a16_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_MOE_H */

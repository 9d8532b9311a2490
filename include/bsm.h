/*
 * bsm.h - exact block-sparse masked attention for packed multimodal sequences,
 * one ring rank's share on one MI355X (gfx950).
 *
 * C ABI of libbsm.so.  Plain integers, host pointers and device pointers only.
 *
 * Conventions for every entry point
 *   - Return value: BSM_OK (0) on success, a negative BSM_E_* code otherwise.
 *     No entry point aborts, throws or exits; bsm_last_error() returns a
 *     thread-local description of the most recent failure on that thread.
 *   - Argument and shape errors are reported before anything is launched,
 *     misaligned tensor pointers among them (BSM_E_INVALID).
 *   - GPU entry points enqueue work on the caller's stream (`stream` is a
 *     hipStream_t; NULL means the default stream) and never synchronize.
 *     Faults inside a kernel surface at the caller's next synchronization;
 *     with the environment variable BSM_DEBUG_SYNC=1 every entry point
 *     synchronizes its stream and reports such faults as BSM_E_HIP.
 *   - The library never allocates device memory.  Every device buffer is
 *     allocated by the caller, who keeps ownership.  Host plans are owned by
 *     the library and released with bsm_plan_free / bsm_dplan_free.
 *   - Tensor layouts (all contiguous device memory, 16-byte aligned; the fp32
 *     row arrays m, l, LSE and delta need only 4-byte alignment):
 *       Q, O, dO          bf16  [rows, Hq, d]     token-major
 *       K, V              bf16  [keys, Hkv, d]
 *       dQ                fp32  [rows, Hq, d]
 *       O_acc             fp32  tile-blocked, ceil(rows / 128) * 128 * Hq * d
 *                               floats (bsm_state_unpack reads it out)
 *       dK, dV            fp32  [keys, Hkv, d]
 *       m, l, LSE, delta  fp32  [Hq, rows]        head-major
 *     d must be 128.  Query head h reads key/value head h / (Hq / Hkv).
 *
 * Terms (MARBLE, "exact sequence parallelism for packed multimodal masks"):
 *   ring of R ranks; at step s rank r holds the key/value shard of rank
 *   j = (r - s) mod R (section 03, "Block classification", ring submasks);
 *   tiles are 128 query tokens x 128 key tokens.
 */
#ifndef BSM_H
#define BSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
enum {
  BSM_OK = 0,
  BSM_E_INVALID = -1,      /* bad argument, shape or metadata               */
  BSM_E_UNSUPPORTED = -2,  /* valid but not supported (e.g. d != 128)       */
  BSM_E_NOMEM = -3,        /* host allocation failed / caller buffer small  */
  BSM_E_HIP = -4           /* a HIP runtime call or kernel launch failed    */
};

/* Window value for global (non-sliding-window) layers. */
#define BSM_WINDOW_INF 0x7fffffff

/* Token orders (MARBLE section 04, "Layout transforms"). */
enum {
  BSM_ORDER_CONTIGUOUS = 0, /* shard r = tokens [r*N/R, (r+1)*N/R); tiles are
                               `block`-token pieces of a shard, last ragged   */
  BSM_ORDER_PTRR = 1,       /* processing-time round robin over blocks        */
  BSM_ORDER_EXPLICIT = 2    /* caller-given permutation of blocks             */
};

/* Tile classes (MARBLE section 03, "Block classification"). */
enum { BSM_TILE_EMPTY = 0, BSM_TILE_PARTIAL = 1, BSM_TILE_FULL = 2 };

/* Flags of the forward entry points. */
enum {
  BSM_FWD_KEEP_STATE = 1,  /* never finalize: always store (O_acc, m, l),
                              even on a tile's last step; O and LSE untouched */
  BSM_FWD_STEP_ONLY = 2    /* accuracy controls: ignore the carried state and
                              treat every tile as on its first and last step,
                              so the call's result covers this step's keys
                              only (with KEEP_STATE: their unnormalized
                              O_acc, m, l; without: normalized bf16 O, LSE) */
};

/* Thread-local text of the last failure on the calling thread ("" if none). */
const char* bsm_last_error(void);

/* Library version, e.g. 100 for 0.1.0. */
int32_t bsm_version(void);

/* ====================================================================== *
 *  Host planner (pure CPU).                                               *
 * ====================================================================== */

typedef struct bsm_plan bsm_plan;

/*
 * Per-token metadata of one packed sequence, in its ORIGINAL order
 * (MARBLE section 01, the four tracks and the mask_mod code block):
 *   sample[i]  sample id >= 0; each sample is one contiguous run, ids
 *              non-decreasing (a negative id is BSM_E_INVALID: padding tokens
 *              need a sample id of their own)
 *   seg[i]     id of the bidirectional span / group, -1 for causal tokens
 *   noise[i]   id of the generated (noise) span, -1 otherwise
 *   pos[i]     original position, >= 0; positions need not rise with the
 *              index: a layout transform (bsm_vision_group_order) permutes
 *              tokens, each keeping its original position
 * A query q may attend a key k iff
 *   ((0 <= pos[q]-pos[k] < window) or (seg[q] == seg[k] and seg[k] >= 0))
 *   and (noise[k] < 0 or noise[q] == noise[k]) and sample[q] == sample[k].
 * All pointers are host memory, read during the call only.
 */
typedef struct {
  int64_t n;                 /* tokens, 1 <= n <= 2^30                        */
  const int32_t* sample;
  const int32_t* seg;
  const int32_t* noise;
  const int32_t* pos;
  int32_t window;            /* >= 1; BSM_WINDOW_INF for global layers        */
  int32_t ranks;             /* ring degree R, 1..64                          */
  int32_t block;             /* tile / PTRR block tokens; 128 for the kernels */
  int32_t order;             /* BSM_ORDER_*                                   */
  const int32_t* explicit_block_perm; /* ORDER_EXPLICIT: new block i is original
                                         block explicit_block_perm[i]; else NULL */
  int32_t threads;           /* planner threads; <= 0: all hardware threads   */
} bsm_plan_desc;

/*
 * Build the plan (MARBLE section 03: "Block classification" and "PTRR";
 * section 04 "Planning cost": built once per packed batch from metadata only,
 * reused by every layer, forward and backward).
 *   - Validates the tracks (BSM_E_INVALID on violation).
 *   - Classifies every (query tile, key tile) pair exactly: the number of
 *     legal token pairs among the tile's valid tokens decides EMPTY (0),
 *     FULL (all) or PARTIAL.  Per-tile summaries only skip work; they never
 *     decide a class that enumeration would decide differently.
 *   - PTRR: tile cost = exact legal pairs of the tile's queries over all keys;
 *     sort by cost descending, ties by ascending original index; deal in
 *     rounds of R, even rounds to ranks 0..R-1, odd rounds to R-1..0; each
 *     rank keeps its tiles in ascending original order.
 *   ORDER_PTRR / ORDER_EXPLICIT need n % (block * ranks) == 0;
 *   ORDER_CONTIGUOUS needs n % ranks == 0.
 * On success *out owns a new plan (free with bsm_plan_free).
 */
int bsm_plan_build(const bsm_plan_desc* desc, bsm_plan** out);
void bsm_plan_free(bsm_plan* plan);

typedef struct {
  int64_t n;
  int32_t ranks;
  int32_t block;
  int32_t order;
  int32_t window;
  int64_t shard_tokens;      /* n / ranks                                      */
  int32_t tiles_per_shard;   /* ceil(shard_tokens / block)                     */
  int32_t tiles_total;       /* ranks * tiles_per_shard                        */
  int32_t busiest_rank;      /* most legal pairs, ties -> lowest rank          */
  int32_t reserved;
  int64_t total_pairs;       /* legal pairs of the whole sequence              */
  int64_t candidate_pairs;   /* tile pairs whose samples overlap               */
  int64_t full_tiles;        /* tile pairs classified FULL (all ranks/steps)   */
  int64_t partial_tiles;     /* tile pairs classified PARTIAL                  */
  double build_seconds;      /* wall time of bsm_plan_build                    */
  int64_t interval_keys;     /* keys whose legal queries form one pos range    */
} bsm_plan_info;

int bsm_plan_get_info(const bsm_plan* plan, bsm_plan_info* out);

/* Token permutation: new_to_orig[new] = original index (host int32[n]). */
int bsm_plan_permutation(const bsm_plan* plan, int32_t* new_to_orig);

/* Per ORIGINAL tile: cost (legal pairs, int64[tiles_total]) and owner rank
 * (int32[tiles_total]).  Either pointer may be NULL. */
int bsm_plan_block_cost(const bsm_plan* plan, int64_t* cost, int32_t* owner);

/* Tile map of rank r at step s: map[a * tiles_per_shard + b] = class of
 * (query tile a of rank r, key tile b of shard (r - s) mod R), host
 * uint8[tiles_per_shard^2]; *pairs (may be NULL) = legal token pairs. */
int bsm_plan_step_map(const bsm_plan* plan, int32_t r, int32_t s, uint8_t* map,
                      int64_t* pairs);

/* pairs[r * R + s] = legal pairs of rank r at step s (host int64[R*R]). */
int bsm_plan_pairs(const bsm_plan* plan, int64_t* pairs);

/*
 * Chunked ring layout (MARBLE section 03, "Chunked ring attention").  The
 * sequence (the plan's tiles in the original order) is cut into R*k
 * contiguous chunks, k a power of two in [min_chunks, max_chunks] dividing
 * the tiles per shard.  Chunks are dealt to ranks by the PTRR rule once in the
 * order of work (strategy 0) and once in sequence order (strategy 1), then
 * improved by up to `swaps` rounds of greedy pairwise swaps (only when
 * R*k <= 64).  The layout minimizing
 *   C = sum_s max_r W[r][(r - s) mod R] + tau * R * k
 * wins; W[r][j] is the legal pairs between rank r's queries and rank j's keys
 * and tau the fixed cost of one range in one step, in pairs.  block_perm
 * (host int32[tiles_total]) receives its explicit block order (new position ->
 * original block; ranks in order, each rank's blocks ascending), to rebuild the
 * plan with BSM_ORDER_EXPLICIT.  Needs n % (block * ranks) == 0.
 */
typedef struct {
  int32_t chunks_per_rank;   /* k of the chosen layout                        */
  int32_t strategy;          /* 0: dealt in order of work, 1: sequence order  */
  double cost;               /* C                                             */
  double step_max_sum;       /* sum over steps of the slowest rank's pairs    */
  double range_term;         /* tau * R * k                                   */
} bsm_chunk_info;

int bsm_plan_chunk_order(const bsm_plan* plan, int32_t min_chunks, int32_t max_chunks, double tau,
                         int32_t swaps, int32_t* block_perm, bsm_chunk_info* out);

/*
 * Sparse fetch (MARBLE section 04, "Sparse all-to-all and strategy selection":
 * instead of the ring, each rank pulls only the remote 128-token key/value
 * blocks its queries can see, then runs one pass over its local and fetched
 * keys): needed[j * tps + b] = 1
 * when some query tile of rank r has a legal pair with key tile b of shard
 * j != r (host uint8[ranks * tiles_per_shard]); *tiles (may be NULL) = their
 * count.  The bytes a rank avoids are the remote tiles with needed = 0.
 */
int bsm_plan_fetch_set(const bsm_plan* plan, int32_t r, uint8_t* needed, int64_t* tiles);

/*
 * Key intervals (MARBLE section 03, "Block classification": a partial tile can
 * test one range per key in a chosen coordinate).  The coordinate is the token
 * index in the caller's order (the order of the tracks given to
 * bsm_plan_build).  For every key k, when the queries k is legal for are
 * exactly the tokens with index in [lo[k], hi[k]) (the union of its causal
 * window and the tokens of its seg id, within its sample and restricted to
 * the tokens of its noise id, is one run of indices), lo/hi receive that
 * range; otherwise lo[k] = 0, hi[k] = -1 and the kernels keep the four-track
 * predicate for its tiles.  A key may also get no range when its noise span
 * lies partly outside its seg and holds more than 4096 tokens (the planner
 * does not scan such spans).  Host int32[n] each.
 */
int bsm_plan_key_intervals(const bsm_plan* plan, int32_t* lo, int32_t* hi);

/*
 * Vision-group token order (MARBLE section 04, "Layout transforms": for
 * vision-group sequences all text goes first and the group spans after it in
 * reverse, so that each key's visible queries form one range).  Per sample (a
 * contiguous run of one sample id), the tokens of group spans (runs of a seg
 * id >= 0 that occurs in two or more runs of the sample) move after the rest:
 * the other tokens keep their order, then the group spans follow in reverse
 * order of their first token, each span's tokens in their order.  The caller
 * permutes tracks and activations once with new_to_orig (position i of the
 * new order holds token new_to_orig[i]) and plans the permuted sequence; each
 * token keeps its position track, so the mask is unchanged.  Host pointers;
 * sample ids >= 0, contiguous and non-decreasing, seg ids >= -1, else
 * BSM_E_INVALID.
 */
int bsm_vision_group_order(int64_t n, const int32_t* sample, const int32_t* seg, int32_t* new_to_orig);

/*
 * Dense calls (MARBLE section 03, "Chunked ring attention": for long, mostly
 * dense samples each ring step runs as a few dense calls, full, causal or
 * reverse causal over runs of tokens, instead of one masked block-sparse
 * call).  The calls of rank r at step s cover every legal pair between rank
 * r's query shard and key shard (r - s) mod R exactly once and no illegal one.
 * Dense calls need positions that rise with the token index (BSM_E_UNSUPPORTED
 * otherwise, e.g. after a vision-group order).
 * A call pairs query rows [q0, q0 + q_len) of the query shard with key rows
 * [k0, k0 + k_len) of the key shard (plan order, local to each shard) and
 * computes the pairs whose positions satisfy `kind`:
 *   BSM_CALL_FULL         every pair
 *   BSM_CALL_CAUSAL       0 <= pos_q - pos_k < W (W: the plan's window)
 *   BSM_CALL_REVERSE      pos_k > pos_q
 *   BSM_CALL_PAST_WINDOW  pos_q - pos_k >= W (finite windows only)
 * The families behind them: each sample's queries against its clean
 * (noise < 0) keys, causal; each seg's queries against the seg's clean keys,
 * the rest of the seg (reverse, past window); each noise span's queries
 * against the span's keys, full when the whole span has one seg >= 0, else
 * causal plus the per-seg rest.
 * *count receives the number of calls; with calls != NULL and capacity >=
 * *count they are written to calls (host memory), with a smaller capacity the
 * call fails with BSM_E_NOMEM.
 */
typedef enum {
  BSM_CALL_FULL = 0,
  BSM_CALL_CAUSAL = 1,
  BSM_CALL_REVERSE = 2,
  BSM_CALL_PAST_WINDOW = 3
} bsm_call_kind;

typedef struct {
  int32_t q0, q_len;         /* query rows of rank r's shard                  */
  int32_t k0, k_len;         /* key rows of shard (r - s) mod R               */
  int32_t kind;              /* bsm_call_kind                                 */
} bsm_call;

int bsm_plan_dense_calls(const bsm_plan* plan, int32_t r, int32_t s, bsm_call* calls,
                         int64_t capacity, int64_t* count);

/* ====================================================================== *
 *  Device plan: one rank's lists, packed into caller-owned device memory. *
 * ====================================================================== */

typedef struct bsm_dplan bsm_dplan;

/* Bytes the device plan of rank r needs (256-byte aligned sections). */
int bsm_dplan_bytes(const bsm_plan* plan, int32_t r, int64_t* bytes);

/*
 * Pack rank r's device plan (permuted tracks, per-step forward row lists and
 * backward column lists, the merged single-pass list) on the host and copy it
 * into `dev` (caller device memory of >= bsm_dplan_bytes bytes) on `stream`;
 * the call synchronizes `stream` before it returns (a plan is uploaded once per
 * packed batch, outside any timed loop).  Requires block == 128.  `dev` must
 * stay allocated while the handle is used.  *out: new handle (host memory,
 * free with bsm_dplan_free, which does not touch `dev`).
 */
int bsm_dplan_upload(const bsm_plan* plan, int32_t r, void* dev, int64_t bytes,
                     void* stream, bsm_dplan** out);
void bsm_dplan_free(bsm_dplan* dplan);

/*
 * Dense-call device plan of rank r (MARBLE section 03, "Chunked ring
 * attention"): its forward lists run the calls of bsm_plan_dense_calls, each
 * as pieces of its key run cut at key-tile edges, for every query tile it
 * meets, tested by row range and one position compare (pieces every pair of
 * which satisfies the relation run unmasked).  Its backward lists hold the
 * same pieces per key tile, tested by key range and one compare.  Same
 * memory rules as bsm_dplan_bytes / bsm_dplan_upload.  bsm_fwd_step,
 * bsm_fwd_single and bsm_bwd_step accept the handle with the same arguments
 * and results; bsm_fwd_fetched refuses it with BSM_E_UNSUPPORTED.  Needs
 * every position below 2^31 - 1 (BSM_E_UNSUPPORTED).
 */
int bsm_dplan_calls_bytes(const bsm_plan* plan, int32_t r, int64_t* bytes);
int bsm_dplan_calls_upload(const bsm_plan* plan, int32_t r, void* dev, int64_t bytes,
                           void* stream, bsm_dplan** out);

/* What a device plan holds per step (MARBLE section 03, "Block classification":
 * for every ring step the blocks the rank computes), for callers that skip
 * steps without work and size workspaces. */
typedef struct {
  int32_t rank;
  int32_t ranks;
  int64_t shard_tokens;
  int32_t tiles_per_shard;
  int32_t window;
  int64_t fwd_items[64];     /* query tiles with work at step s               */
  int64_t bwd_items[64];     /* key tiles with work at step s                 */
  int64_t step_pairs[64];    /* legal pairs at step s                         */
  int64_t single_items;      /* query tiles with work in the merged list      */
  int64_t fetch_tiles;       /* remote key tiles the rank needs (sparse fetch) */
  int64_t fetch_rows;        /* rows of the compact key/value buffer          */
  int32_t dense_calls;       /* 1: a dense-call device plan                   */
  int32_t bwd_workspace_slots; /* max over steps of the split dK/dV work's
                                  workspace slots (each Hkv * 128 KiB)      */
  int64_t fwd_chain0_items[64]; /* of fwd_items[s], those in chain 0 (the
                                   rest are chain 1; bsm_fwd_step_chain)     */
} bsm_dplan_info;

int bsm_dplan_get_info(const bsm_dplan* dplan, bsm_dplan_info* out);

/* ====================================================================== *
 *  Forward.                                                               *
 * ====================================================================== */

typedef struct {
  int32_t hq;     /* query heads                                          */
  int32_t hkv;    /* key/value heads, hq % hkv == 0                        */
  int32_t d;      /* head dim, must be 128                                 */
  float scale;    /* softmax scale, usually 1/sqrt(d)                      */
} bsm_heads;

/*
 * One ring step of the online forward (MARBLE section 03, "Exact ring
 * attention accumulation"): for every query tile of the rank with a
 * non-empty list at step s and every query head, fold the listed key tiles of
 * shard j = (r - s) mod R into the fp32 running state.
 *   q      bf16 [S, Hq, d]   the rank's query shard in plan order
 *   k, v   bf16 [S, Hkv, d]  shard j in plan order
 *   o_acc  fp32, ceil(S / 128) * 128 * Hq * d floats: the unnormalized
 *                            accumulator (carried state) in the kernel's
 *                            tile-blocked order, each (query tile, head)
 *                            one contiguous 64 KiB run; bsm_state_unpack
 *                            converts it to [S, Hq, d]
 *   m      fp32 [Hq, S]      reference of the row in base-2 units
 *                            (scale*log2(e)*q.k): the row max at the last
 *                            rescale, -inf before the first legal key; o_acc
 *                            and l are scaled by 2^-m, and later scores exceed
 *                            m by less than 12 (every 2^(x - m) < 2^12)
 *   l      fp32 [Hq, S]      running row sum of 2^(x - m)
 *   o      bf16 [S, Hq, d]   written at a tile's last non-empty step
 *   lse    fp32 [Hq, S]      natural-log LSE, written with o
 * A tile's first non-empty step initializes the state in-kernel (m = -inf,
 * l = 0, O_acc = 0), so the state buffers need no clearing; later steps read
 * it; the last non-empty step writes O = O_acc / l (bf16, round to nearest
 * even) and LSE = ln 2 * (m + log2 l) instead of storing the state, unless
 * flags has BSM_FWD_KEEP_STATE.  Rows with no legal key get O = 0 and
 * LSE = -inf.  Steps without work return BSM_OK without a launch.  S is the
 * plan's shard_tokens; rows of a ragged last tile beyond S are never touched.
 * Every bf16 tensor must be under 4 GiB (the kernels use 32-bit byte
 * offsets), else BSM_E_UNSUPPORTED.
 */
int bsm_fwd_step(const bsm_dplan* dplan, int32_t s, const bsm_heads* heads,
                 const void* q, const void* k, const void* v,
                 float* o_acc, float* m, float* l, void* o, float* lse,
                 int32_t flags, void* stream);

/*
 * The items of one chain of ring step s (MARBLE section 03, "Exact ring
 * attention accumulation"; the order in which a rank's query tiles meet the
 * ring's steps is free, only each tile's own steps are ordered).  The device
 * plan splits the rank's query tiles into two chains (0 and 1) by whole
 * samples, balanced by list entries; bsm_dplan_info.fwd_chain0_items[s] of
 * the fwd_items[s] tiles are chain 0's.  A tile's state is touched only by
 * its own chain, so the calls of chain 0 (steps in order) and those of chain
 * 1 (steps in order) may run on two streams side by side; calling both
 * chains of a step has the effect of bsm_fwd_step, bitwise (each tile runs
 * the same list in the same order).  chain not 0 or 1 returns BSM_E_INVALID;
 * a chain without items at step s returns BSM_OK without a launch.  Other
 * arguments, flags and errors as for bsm_fwd_step.
 */
int bsm_fwd_step_chain(const bsm_dplan* dplan, int32_t s, int32_t chain, const bsm_heads* heads,
                       const void* q, const void* k, const void* v,
                       float* o_acc, float* m, float* l, void* o, float* lse,
                       int32_t flags, void* stream);

/*
 * Single pass over all R shards at once (the one-GPU result the ring must
 * equal): k_all, v_all bf16 [N, Hkv, d] hold all shards in plan order
 * (shard j at rows [j*S, (j+1)*S)).  Tiles are visited in the same order as
 * the ring visits them, with the state kept in registers, so the result is
 * bitwise identical to the R ring steps.  With BSM_FWD_KEEP_STATE it stores
 * (o_acc, m, l) instead of (o, lse); otherwise o_acc, m, l may be NULL.
 * k_all and v_all must each be under 4 GiB, else BSM_E_UNSUPPORTED.
 */
int bsm_fwd_single(const bsm_dplan* dplan, const bsm_heads* heads,
                   const void* q, const void* k_all, const void* v_all,
                   float* o_acc, float* m, float* l, void* o, float* lse,
                   int32_t flags, void* stream);

/*
 * One pass over the rank's local shard and the fetched remote tiles (sparse
 * fetch).  k_fetch, v_fetch bf16 [fetch_rows, Hkv, d] hold the compact
 * buffer: rows [0, S) = the rank's own shard j = r in plan order, then every
 * needed remote tile (bsm_plan_fetch_set) at 128 rows each, in ring step
 * order s = 1..R-1 (shard j = (r - s) mod R), ascending tile b; rows of a
 * ragged tile past its valid rows are never read.  Tiles are visited in the
 * single pass's order, so the result is bitwise that of bsm_fwd_single.
 * Other arguments and flags as for bsm_fwd_single.
 */
int bsm_fwd_fetched(const bsm_dplan* dplan, const bsm_heads* heads, const void* q,
                    const void* k_fetch, const void* v_fetch, float* o_acc, float* m, float* l,
                    void* o, float* lse, int32_t flags, void* stream);

/*
 * Accuracy controls (MARBLE section 03, "Exact ring attention accumulation":
 * the fp32 carry of (O_acc, m, l) against per-step merges).  A ring can also
 * finish every step (BSM_FWD_STEP_ONLY) and merge the step's normalized
 * partial into a running result:
 *   lse = ln(e^lse_run + e^lse_s),  O = O_run e^(lse_run - lse) + O_s e^(lse_s - lse).
 * bsm_fwd_merge_bf16: o_run, o_s bf16 [rows, Hq, d]; lse_run, lse_s fp32
 *   [Hq, rows] (natural log); the merged O is rounded to bf16 every step.
 * bsm_fwd_merge_fp32: o_run fp32 [rows, Hq, d] normalized; the step is given
 *   as its unnormalized fp32 (acc_s tile-blocked as o_acc, m_s, l_s) from
 *   BSM_FWD_STEP_ONLY | BSM_FWD_KEEP_STATE; o_bf16 (may be NULL) receives RNE
 *   bf16 of the merged O.
 * Rows the step did not reach must read lse_s = -inf (bf16) or l_s = 0
 * (fp32): the caller fills them before the step; they keep the running values.
 * Start from lse_run = -inf (o_run is then ignored).  Stream-ordered on
 * `stream`; rows >= 1; heads as for the forward.
 */
int bsm_fwd_merge_bf16(const bsm_heads* heads, int64_t rows, void* o_run, float* lse_run,
                       const void* o_s, const float* lse_s, void* stream);
int bsm_fwd_merge_fp32(const bsm_heads* heads, int64_t rows, float* o_run, float* lse_run,
                       const float* acc_s, const float* m_s, const float* l_s, void* o_bf16,
                       void* stream);

/*
 * The carried accumulator of bsm_fwd_step / bsm_fwd_single in row order
 * (MARBLE section 03, "Exact ring attention accumulation": the fp32 O_acc that
 * stays in HBM between ring steps, here laid out tile by tile for the kernels):
 * out fp32 [rows, Hq, d] from o_acc (tile-blocked, ceil(rows / 128) * 128 *
 * Hq * d floats).  Stream-ordered on `stream`; rows >= 1.
 */
int bsm_state_unpack(const bsm_heads* heads, int64_t rows, const float* o_acc, float* out,
                     void* stream);

/* ====================================================================== *
 *  Backward.                                                              *
 * ====================================================================== */

/*
 * Backward preparation (MARBLE section 03, "Exact ring attention
 * accumulation": every backward step runs against the final output and LSE):
 * delta[h][i] = sum_c dO[i][h][c] * O[i][h][c] in fp32 (the row term of the
 * softmax backward), from the bf16 O the forward wrote.  rows >= 1.
 */
int bsm_bwd_prep(const bsm_heads* heads, int64_t rows, const void* o, const void* dout,
                 float* delta, void* stream);

/*
 * One ring step of the backward (MARBLE section 03: each step runs the
 * attention backward against the FINAL LSE; the fp32 dQ accumulator is carried
 * across steps, and each key shard's fp32 dK/dV accumulator travels with it).
 *   q, dout         bf16 [S, Hq, d]    the rank's queries and output gradient
 *   k, v            bf16 [S, Hkv, d]   shard j = (r - s) mod R
 *   lse, delta      fp32 [Hq, S]       from the forward / bsm_bwd_prep
 *   dq_acc          fp32 [S, Hq, d]    carried: a query tile's first step with
 *                                      work overwrites, later steps add
 *   dk, dv          fp32 [S, Hkv, d]   shard j's accumulators: this call ADDS
 *                                      the rank's contribution (caller clears
 *                                      them before the first contribution)
 * With grouped heads, dk/dv of a key/value head sum over its query heads.
 * Every bf16 tensor must be under 4 GiB, else BSM_E_UNSUPPORTED.
 */
int bsm_bwd_step(const bsm_dplan* dplan, int32_t s, const bsm_heads* heads,
                 const void* q, const void* k, const void* v, const void* dout,
                 const float* lse, const float* delta,
                 float* dq_acc, float* dk, float* dv, void* stream);

/*
 * bsm_bwd_step with a caller workspace, for layouts whose dK/dV launch would
 * last as long as its few longest column lists (one workgroup per key tile
 * and key/value head; MARBLE section 03 balances ring steps across ranks, this
 * balances one step's work across the GPU).  When the step has fewer than
 * twice as many (key tile, kv head) units as the device has CUs and its plan
 * splits lists (bsm_dplan_info.bwd_workspace_slots > 0), each long list is cut
 * into sub-tile ranges: the first adds into dk/dv, the others write their
 * partial sums to workspace slots, and a reduction then adds the slots into
 * dk/dv in slot order (deterministic; sums in a different order than the
 * unsplit call, so results differ from it by rounding).  workspace: device
 * memory of at least bwd_workspace_slots * Hkv * 131072 bytes, clobbered; NULL
 * behaves as bsm_bwd_step.  Calls in stream order may share one workspace;
 * calls that can run concurrently (other streams) need their own.  A smaller workspace_bytes than the step needs
 * returns BSM_E_INVALID before any launch.  Other arguments as bsm_bwd_step.
 */
int bsm_bwd_step_ws(const bsm_dplan* dplan, int32_t s, const bsm_heads* heads,
                    const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, const float* delta, float* dq_acc, float* dk, float* dv,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * bsm_bwd_step_ws with the step's two updates on two streams: the dQ product
 * on dq_stream, the dK/dV products (and the split reduction) on kv_stream.
 * MARBLE section 03 ("Exact ring attention accumulation") carries dQ across
 * steps in the query rank and sends each key shard's dK/dV along the ring, so
 * within a step the two updates write different buffers and read only the
 * step's inputs.  Issuing every step's dQ update on one stream and every
 * step's dK/dV update on another keeps each chain in step order and lets the
 * GPU run the two side by side (one fills the CUs the other's tail leaves
 * idle).  The caller orders q, k, v, dout, lse and delta before both streams
 * and joins the streams before reading dq_acc, dk or dv.  Results equal
 * bsm_bwd_step_ws bit for bit.  workspace is used on kv_stream only.  Equal
 * streams make it bsm_bwd_step_ws.  Other arguments as bsm_bwd_step_ws.
 */
int bsm_bwd_step_streams(const bsm_dplan* dplan, int32_t s, const bsm_heads* heads,
                         const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, const float* delta, float* dq_acc, float* dk, float* dv,
                         void* workspace, int64_t workspace_bytes, void* dq_stream, void* kv_stream);

/*
 * Backward of the sparse-fetch pass (MARBLE section 04, "Sparse all-to-all and
 * strategy selection": the fetched blocks' dK and dV go back to their owners
 * with the inverse all-to-all and are accumulated there in fp32).  One pass
 * over the rank's queries and the compact buffer of bsm_fwd_fetched, against
 * the final LSE:
 *   q, dout            bf16 [S, Hq, d]
 *   k_fetch, v_fetch   bf16 [fetch_rows, Hkv, d], laid out as for
 *                      bsm_fwd_fetched; rows of a ragged tile past its valid
 *                      rows are never read
 *   lse, delta         fp32 [Hq, S] (forward LSE, bsm_bwd_prep)
 *   dq                 fp32 [S, Hq, d], written for every query tile with work
 *   dk_fetch, dv_fetch fp32 [fetch_rows, Hkv, d]: this call ADDS the rank's
 *                      contribution of every compact row (caller clears);
 *                      padding rows are never written
 * Results equal the ring backward's up to the order of the fp32 sums.  A
 * dense-call device plan returns BSM_E_UNSUPPORTED.
 */
int bsm_bwd_fetched(const bsm_dplan* dplan, const bsm_heads* heads, const void* q,
                    const void* k_fetch, const void* v_fetch, const void* dout,
                    const float* lse, const float* delta, float* dq, float* dk_fetch,
                    float* dv_fetch, void* stream);

/*
 * The way back of the sparse fetch on one device: for every row c of the
 * compact buffer that holds a shard row (not padding), dk_all[src] +=
 * dk_fetch[c] and dv_all[src] += dv_fetch[c] in fp32, src being that row's
 * position in the shards concatenated in plan order (dk_all, dv_all fp32
 * [R * S, Hkv, d]).  Across devices this is the inverse all-to-all followed
 * by each owner's fp32 add; every shard row receives at most one compact row,
 * so the adds never collide.  Stream-ordered; BSM_E_UNSUPPORTED for a
 * dense-call device plan.
 */
int bsm_fetched_accumulate(const bsm_dplan* dplan, const bsm_heads* heads, const float* dk_fetch,
                           const float* dv_fetch, float* dk_all, float* dv_all, void* stream);

/*
 * bsm_bwd_step_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split dK/dV partial sums go to a
 * static device array of the library, 64 MiB per device, resident from the
 * library's load until the process ends; its address is looked up once per
 * device, on the first call with that device current.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine) and writes
 * every scratch slot it reads within the same call, so no clearing is needed
 * and nothing carries over between calls.  All calls on one device share the
 * array: calls that can overlap on one device (other streams, other host
 * threads without ordering) race and must be serialized by the caller.  A step
 * whose split needs more than 64 MiB (bwd_workspace_slots * Hkv * 131072
 * bytes) returns BSM_E_UNSUPPORTED before any launch; bsm_bwd_step_ws takes
 * such steps.  Arguments and results as bsm_bwd_step_ws on one stream.
 */
int bsm_bwd_step_noalloc(const bsm_dplan* dplan, int32_t s, const bsm_heads* heads,
                         const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, const float* delta, float* dq_acc, float* dk, float* dv,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSM_H */

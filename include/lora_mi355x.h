/*
 * lora_mi355x.h -- C ABI of the heterogeneous-adapter LoRA apply on MI355X (gfx950).
 *
 * The operation (per token i with adapter id a_i):
 *     y_i <- y_i + s_{a_i} * B_{a_i} (A_{a_i} x_i)        (a_i < 0: y_i untouched)
 * A_a (rank r_a x d_in) is the shrink matrix, B_a (d_out x r_a) the expand
 * matrix and s_a the per-adapter scale (alpha / r by default).  Sources:
 *   - S-LoRA paper explainer (0h-n0.github.io/posts/paper-2311-04928):
 *       section "BGMVカーネル" -- the BGMV equation (one launch applies a
 *       different adapter per request, ranks may differ inside a batch) and
 *       its reference loop (negative adapter id = no adapter, scale after the
 *       expand, y accumulated in place);
 *       section "Unified Paging" -- adapters live in fixed-size pages of one
 *       pool shared with KV-cache blocks.
 *   - Multi-LoRA serving article (produtoramaxvision.com.br): SGMV section --
 *       Y = X W0 + (alpha/r)((X A) B), A = shrink, B = expand, an index vector
 *       maps every token to its adapter's place in VRAM, shrink then expand;
 *       unified paged pool section -- fixed-size pages, waste only in the last
 *       page of each adapted layer.
 *
 * Conventions for every entry point:
 *   - All functions return lora_status; LORA_OK is 0.  On failure nothing is
 *     launched and no pool state changes; lora_last_error() returns a
 *     thread-local message.  No C++ exception crosses this boundary.
 *   - Pointers named *_dev are device pointers (HBM), *_host are host pointers.
 *     The caller owns every buffer it passes in; the library never frees them.
 *   - `stream` is a hipStream_t (NULL: the null stream).  Compute entry points
 *     (lora_bgmv_*, lora_sgmv_*, lora_apply) are stream-ordered: they neither
 *     allocate memory nor wait for the device.  Set-up calls (pool creation,
 *     upload, evict, page-table build, plan create/build/prepare) may do both.
 *   - x rows are d_in elements of the pool's activation dtype (act_dtype:
 *     the page dtype, except 16-bit activations on FP8 pools), y rows d_out
 *     elements of y_dtype (act_dtype or LORA_F32), both dense row-major,
 *     16-byte aligned base pointers.  v (the shrink output) is fp32 [n][v_ld].
 *   - Adapter ids on the device should lie in [-1, max_adapters) and name
 *     adapters resident in the slice used.  The kernels treat any id outside
 *     [0, max_adapters) like -1 (the token is skipped) and a non-resident
 *     adapter as contributing nothing; no error is reported from the device.
 *     Host-side ids (lora_plan_build) are checked.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* LORA_FP8_E4M3: OCP 8-bit float codes (sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities) for quantised adapter pages, with fp32 scales
 * per rank: A = diag(a_scale) A_codes, B = B_codes diag(b_scale) (the FP8
 * adapters of the serving article's trade-offs section, which halve the bytes
 * that uploads and gathers move). */
typedef enum { LORA_F32 = 0, LORA_F16 = 1, LORA_BF16 = 2, LORA_FP8_E4M3 = 3 } lora_dtype;

typedef enum {
  LORA_OK = 0,
  LORA_E_ARG = -1,          /* bad argument (null, out of range, misaligned, shape) */
  LORA_E_NOMEM = -2,        /* pool has too few free pages, or a device allocation failed */
  LORA_E_NOT_RESIDENT = -3, /* an id names an adapter that is not uploaded */
  LORA_E_RANK = -4,         /* rank < 1 or > max_rank, or too large for one page */
  LORA_E_STATE = -5,        /* wrong state: stale page table, double upload/evict, ... */
  LORA_E_HIP = -6,          /* a HIP runtime call failed (message has the HIP error) */
  LORA_E_UNSUPPORTED = -7   /* valid request this build does not implement */
} lora_status;

typedef struct lora_pool lora_pool; /* opaque, library-owned */
typedef struct lora_plan lora_plan; /* opaque, library-owned */
typedef struct lora_dplan lora_dplan; /* opaque, library-owned: a plan built on the device */

#define LORA_MAX_SLICES 16
#define LORA_MAX_RANK 128
#define LORA_MAX_IO 8

/* Pool flags */
#define LORA_POOL_POISON 1u    /* fill the whole pool with quiet NaNs at creation and
                                  refill pages with NaNs when they are freed/evicted */
#define LORA_POOL_HOST_ONLY 2u /* no device: the pool is a host image (layout tests) */

/*
 * Unified page pool (S-LoRA explainer, "Unified Paging"; serving article,
 * unified paged pool section).  The pool is n_pages pages of page_elems
 * elements of `dtype`.  Pages are handed out from a free list that is a
 * permutation of all page ids (seeded shuffle; shuffle_seed 0 = in order), to
 * adapter uploads and to other users (lora_pool_alloc_pages, e.g. KV blocks).
 *
 * Layout of one uploaded adapter slice (rank r, dims d_in x d_out):
 *   r_s = r rounded up to a multiple of 16 bytes' worth of elements (4 for
 *         fp32, 8 for fp16/bf16, 16 for FP8)
 *   A   : r rows of d_in elements; row k occupies ceil(d_in/P) pages, element j
 *         in page a_pages[k*ceil(d_in/P) + j/P] at position j % P.
 *   B   : d_out rows of r_s elements (columns r..r_s-1 are zero), packed
 *         rpp = floor(P / r_s) rows per page: row m at page b_pages[m / rpp],
 *         position (m % rpp) * r_s.  The tail of each page is unused.
 */
typedef struct {
  int32_t page_elems;        /* P: elements per page, P * elt a multiple of 16 bytes */
  int32_t dtype;             /* lora_dtype of pages and activations x              */
  int64_t n_pages;           /* pool capacity in pages, < 2^31                      */
  int32_t max_adapters;      /* adapter ids live in [0, max_adapters)               */
  int32_t max_rank;          /* 1..LORA_MAX_RANK; also the minimum v_ld             */
  int32_t n_slices;          /* adapted projections, 1..LORA_MAX_SLICES             */
  const int32_t* slice_d_in; /* [n_slices], multiples of 8                          */
  const int32_t* slice_d_out;/* [n_slices], multiples of 8                          */
  uint64_t shuffle_seed;     /* free-list permutation seed (0: sequential)          */
  uint32_t flags;            /* LORA_POOL_* */
  void* pages_dev;           /* caller-owned device buffer of n_pages*P*elt bytes, or
                                NULL: the library allocates (and frees) it            */
  int32_t act_dtype;         /* lora_dtype of x (and of 16-bit y): equal to dtype for
                                f32/f16/bf16 pools; LORA_F16 or LORA_BF16 for
                                LORA_FP8_E4M3 pools (whose slices need d_in % 16 == 0) */
} lora_pool_desc;

lora_status lora_pool_create(const lora_pool_desc* desc, lora_pool** out);
lora_status lora_pool_destroy(lora_pool* pool);

/* Free pages left, pool base pointer (device, or host for HOST_ONLY pools). */
lora_status lora_pool_info(const lora_pool* pool, int64_t* free_pages, void** pages_base);

/* Pages for other users of the unified pool (KV-cache blocks).  Allocation is
 * all-or-nothing (LORA_E_NOMEM leaves the pool unchanged).  Freeing a page that
 * is free or belongs to an adapter is LORA_E_STATE. */
lora_status lora_pool_alloc_pages(lora_pool* pool, int64_t n, int32_t* page_ids_host);
lora_status lora_pool_free_pages(lora_pool* pool, int64_t n, const int32_t* page_ids_host);

/* Upload one adapter slice: A_host [rank][d_in], B_host [d_out][rank] in the pool
 * dtype, scale stored as given (fp32).  The pages are taken from the free list
 * and written on `stream`; the call returns after the copies finish, so the host
 * buffers may be reused at once.  Uploading a resident slice is LORA_E_STATE.
 * Invalidates the device page table until lora_page_table_build.  FP8 pools
 * take lora_pool_upload_scaled instead (LORA_E_ARG here). */
lora_status lora_pool_upload(lora_pool* pool, int32_t adapter, int32_t slice, int32_t rank,
                             float scale, const void* A_host, const void* B_host,
                             void* stream);
/* Upload of a quantised adapter slice to an FP8 pool: A_host [rank][d_in] and
 * B_host [d_out][rank] FP8 E4M3 codes, a_scale_host [rank] (row k of A is
 * a_scale[k] * codes) and b_scale_host [rank] (column k of B is codes *
 * b_scale[k]), fp32.  Otherwise as lora_pool_upload; LORA_E_ARG on other
 * pools or with a NULL scale array. */
lora_status lora_pool_upload_scaled(lora_pool* pool, int32_t adapter, int32_t slice,
                                    int32_t rank, float scale, const void* A_host,
                                    const float* a_scale_host, const void* B_host,
                                    const float* b_scale_host, void* stream);
/* Return an adapter slice's pages to the free list (refilled with NaN under
 * LORA_POOL_POISON).  Evicting a non-resident slice is LORA_E_STATE. */
lora_status lora_pool_evict(lora_pool* pool, int32_t adapter, int32_t slice, void* stream);

/* Push the adapter table (rank, scale, page-list offsets per slice x adapter)
 * and the page-id lists to the device (index vector of the serving article's
 * SGMV section).  Compute entry points refuse to run on a stale table. */
lora_status lora_page_table_build(lora_pool* pool, void* stream);

/* Host copy of one adapter slice's table entry: rank (0 = not resident), scale,
 * and its page lists (a_pages: rank*ceil(d_in/P) ids, b_pages: ceil(d_out/rpp)
 * ids).  Pass NULL page buffers to query the counts only. */
lora_status lora_pool_export_entry(const lora_pool* pool, int32_t adapter, int32_t slice,
                                   int32_t* rank, float* scale, int32_t* n_a_pages,
                                   int32_t* a_pages_host, int32_t* n_b_pages,
                                   int32_t* b_pages_host);
/* Host copy of a quantised adapter slice's scales: a_scale [rank], b_scale
 * [rank] (LORA_E_ARG on pools that are not FP8, LORA_E_NOT_RESIDENT if the
 * slice is not uploaded). */
lora_status lora_pool_export_scales(const lora_pool* pool, int32_t adapter, int32_t slice,
                                    float* a_scale_host, float* b_scale_host);
/* Copy pages [first, first+count) of the pool to host memory (synchronous). */
lora_status lora_pool_read_pages(const lora_pool* pool, int64_t first, int64_t count,
                                 void* dst_host);

/* ---------------------------------------------------------------------------
 * Host adapter store and on-demand residency (S-LoRA explainer, "Unified
 * Paging": every adapter lives in host memory and is paged into the pool when
 * a request needs it, least recently used adapters leaving first; serving
 * article, unified paged pool section: loads on dedicated streams overlapped
 * with compute).
 * ------------------------------------------------------------------------- */
typedef struct lora_store lora_store; /* opaque, library-owned */
typedef struct {
  int64_t uploads;         /* adapter slices loaded into the pool */
  int64_t evictions;       /* adapter slices evicted */
  int64_t bytes_uploaded;  /* page bytes copied host -> device */
  int32_t resident;        /* adapters resident in every slice */
  int32_t registered;      /* adapters registered in every slice */
} lora_store_stats;

/* A store for a device pool.  The pool must outlive the store. */
lora_status lora_store_create(lora_pool* pool, lora_store** out);
lora_status lora_store_destroy(lora_store* store);
/* Register one adapter slice (copied into pinned host memory as page images,
 * so the host buffers may be reused at once).  Arguments as lora_pool_upload
 * (a_scale/b_scale NULL) or, on FP8 pools, lora_pool_upload_scaled.  Nothing
 * is loaded: the adapter becomes resident through lora_store_ensure. */
lora_status lora_store_add(lora_store* store, int32_t adapter, int32_t slice, int32_t rank,
                           float scale, const void* A_host, const float* a_scale_host,
                           const void* B_host, const float* b_scale_host);
/* Make the listed adapters (negative ids ignored) resident in every slice
 * for the launches that follow.  Missing adapters are loaded on upload_stream
 * (no host wait: work already enqueued on compute_stream keeps running); if the
 * pool lacks free pages, store adapters outside the list are evicted, least
 * recently used first, and their pages are overwritten only after
 * compute_stream has passed this call (pages not reused are refilled with NaN
 * under LORA_POOL_POISON and rejoin the free list when that is done).  A new
 * page table is written into the inactive half of the pool's double-buffered
 * table and compute_stream waits for it: launches enqueued on compute_stream
 * after this call see the new residency, launches enqueued before it keep the
 * table they were given.  Launches on other streams must be ordered by the
 * caller.  Plans built before a call that changed residency are refused
 * (rebuild them).  Host waits: for the previous call's copies, and, when a
 * request needs more staging than any before it, for the reallocation of the
 * store's device staging buffer.  Errors: LORA_E_NOT_RESIDENT (an adapter not
 * in the store), LORA_E_NOMEM (the list does not fit the pool, or staging
 * memory cannot be allocated), with the pool unchanged; LORA_E_HIP from a
 * runtime call after the loads were enqueued leaves the pool unusable
 * (destroy it). */
lora_status lora_store_ensure(lora_store* store, int32_t n, const int32_t* adapters_host,
                              void* upload_stream, void* compute_stream);
lora_status lora_store_get_stats(const lora_store* store, lora_store_stats* out);

/* One adapted projection in a multi-slice launch: its slice index, its input
 * x [n][d_in] and its output y [n][d_out] (accumulated in place).  x_group:
 * 0, or a positive id that entries reading one and the same x share (q, k and
 * v of a layer, gate and up of an MLP): their x_dev and d_in must be equal
 * (LORA_E_ARG otherwise).  When a batch has at least one (group, token) pair
 * per compute unit, lora_bgmv_apply reads a token's x once and dots it
 * against the A rows of every slice of the group in one block; smaller
 * batches run one block per (slice, token), a token's blocks sharing one L2.
 * The results are those of separate x, bit for bit. */
typedef struct {
  int32_t slice;
  int32_t x_group;
  const void* x_dev;
  void* y_dev;
} lora_io;

/* ---------------------------------------------------------------------------
 * BGMV: decode form, one token per request, ids on the device (S-LoRA
 * explainer, "BGMVカーネル").
 * ------------------------------------------------------------------------- */
/* v[i][k] = sum_j A_{a_i}[k][j] x[i][j] for k < r_{a_i}; v[i][k] = 0 for
 * r_{a_i} <= k < v_ld and for tokens with a negative id.  v_ld >= max_rank. */
lora_status lora_bgmv_shrink(lora_pool* pool, int32_t slice, const void* x_dev,
                             const int32_t* ids_dev, int32_t n, float* v_dev, int32_t v_ld,
                             void* stream);
/* y[i][m] += s * sum_k B_{a_i}[m][k] v[i][k], s = token_scale_dev[i] if given,
 * else the adapter's stored scale.  One RNE rounding at the store. */
lora_status lora_bgmv_expand(lora_pool* pool, int32_t slice, const float* v_dev, int32_t v_ld,
                             const int32_t* ids_dev, int32_t n, const float* token_scale_dev,
                             void* y_dev, int32_t y_dtype, void* stream);
/* Fused shrink + expand in one launch for up to LORA_MAX_IO slices (v never
 * leaves the chip).  All io entries share ids and n.  Entries with a common
 * x_group may run as one block per (group, token) with x read once (see
 * lora_io). */
lora_status lora_bgmv_apply(lora_pool* pool, int32_t n_io, const lora_io* io_host,
                            const int32_t* ids_dev, int32_t n, int32_t y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * SGMV: tokens grouped into segments that share an adapter (serving article,
 * SGMV section), including heterogeneous ranks (explainer, BGMV section) and
 * rank bands (serving article, FAQ on mixed ranks).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t n_tokens;     /* tokens in the batch                                 */
  int32_t n_groups;     /* distinct adapters (incl. the no-adapter group)        */
  int32_t n_items;      /* work items                                            */
  int32_t n_mfma_items; /* items that run on bf16/fp16 MFMA tiles                */
  int32_t mfma_tokens;  /* tokens covered by MFMA items                          */
  int32_t l_long;       /* group length from which MFMA tiles are used           */
} lora_plan_stats;

/* Plan for up to max_tokens tokens (perm and item buffers allocated here).
 * A plan is used by one stream and one host thread at a time: its set-up calls
 * and the compute calls that use it are issued in order on one stream. */
lora_status lora_plan_create(lora_pool* pool, int32_t max_tokens, lora_plan** out);
lora_status lora_plan_destroy(lora_plan* plan);
/* Build the plan of one batch from host ids [n] (any order, -1 = no adapter):
 * stable counting sort by adapter -> groups; on fp16/bf16 pools groups of at
 * least l_long tokens become MFMA tiles of up to 64 tokens (l_long <= 0: 1, i.e.
 * every group), the others -- and every group of an fp32 pool -- short items of
 * <= 4 tokens on the vector ALUs; items ordered MFMA first, then by rank band,
 * largest first.  Every id >= 0 must be < max_adapters and resident in every
 * slice (LORA_E_NOT_RESIDENT otherwise).  The plan is copied to the device on
 * `stream`; the host ids may be reused on return.  Building drops the launch
 * shapes prepared for the previous batch.  The SGMV calls below launch one
 * kernel per item kind present in the plan. */
lora_status lora_plan_build(lora_plan* plan, const int32_t* ids_host, int32_t n,
                            int32_t l_long, void* stream);
/* Prepare one launch shape of a built plan: the slices of a planned call, in
 * the order the call lists them (only io[k].slice is read; the split calls use
 * one-slice shapes).  On 16-bit pools with MFMA tiles this builds, on the host,
 * the block-range tables and split-K contribution lists of that shape and
 * copies them to the device on `stream` (the plan keeps up to 8 shapes, least
 * recently used replaced first); otherwise it does nothing.  Every planned
 * compute call needs its shape prepared after the last lora_plan_build
 * (LORA_E_STATE otherwise).  May allocate and synchronise. */
lora_status lora_plan_prepare(lora_plan* plan, int32_t n_io, const lora_io* io_host,
                              void* stream);
/* Bytes of caller-owned device workspace that lora_apply and lora_sgmv_shrink
 * need for this prepared launch shape: the split-K partial tiles of the MFMA
 * tiles, 16 bytes per (token block x 16-rank block x 64 lanes) per
 * contribution (a few MB at the configured workloads); 0 without MFMA tiles.
 * The workspace needs no initial contents; calls that share one workspace must
 * not overlap.  LORA_E_STATE if the shape is not prepared. */
lora_status lora_workspace_size(const lora_plan* plan, int32_t n_io, const lora_io* io_host,
                                size_t* bytes);
lora_status lora_plan_get_stats(const lora_plan* plan, lora_plan_stats* out);
/* Host copy of the plan: perm [n_tokens] (token indices, grouped by adapter)
 * and items [n_items][4] = {adapter, start in perm, count, kind (0 short,
 * 1 MFMA tile)}.  Either pointer may be NULL. */
lora_status lora_plan_export(const lora_plan* plan, int32_t* perm_host, int32_t* items_host);

/* Shrink for a planned batch: v[i][.] as lora_bgmv_shrink (rows indexed by the
 * original token index).  MFMA tiles: two launches (block ranges, then the sum
 * of the partial tiles of every tile that several ranges share, in block
 * order); the partial tiles go to workspace_dev (16-byte aligned, at least
 * lora_workspace_size bytes for the one-slice shape {slice}, else LORA_E_ARG;
 * may be NULL when that size is 0). */
lora_status lora_sgmv_shrink(lora_pool* pool, const lora_plan* plan, int32_t slice,
                             const void* x_dev, float* v_dev, int32_t v_ld, void* workspace_dev,
                             size_t ws_bytes, void* stream);
/* Expand for a planned batch: y[i] += s B v[i].  Needs the one-slice shape
 * {slice} prepared; uses no workspace. */
lora_status lora_sgmv_expand(lora_pool* pool, const lora_plan* plan, int32_t slice,
                             const float* v_dev, int32_t v_ld, void* y_dev, int32_t y_dtype,
                             void* stream);
/* Fused shrink + expand for a planned (mixed prefill + decode) batch, for up to
 * LORA_MAX_IO slices; v is never materialized.  x_group is checked as for
 * lora_bgmv_apply; each slice's shrink reads x itself.  Short items: one launch, v in
 * LDS.  MFMA tiles: two launches on `stream` (shrink ranges keep partial tiles
 * in workspace_dev; the expand sums them while loading V).  The launch shape
 * (the io slices in this order) must be prepared; workspace_dev as for
 * lora_sgmv_shrink, sized by lora_workspace_size for this shape. */
lora_status lora_apply(lora_pool* pool, const lora_plan* plan, int32_t n_io,
                       const lora_io* io_host, int32_t y_dtype, void* workspace_dev,
                       size_t ws_bytes, void* stream);

/* lora_apply for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels, with the partial tiles in a static device array of the library
 * (16 MiB per GPU, held until the process ends) instead of a caller workspace.
 * A launch shape whose lora_workspace_size exceeds 16 MiB is LORA_E_ARG.  The
 * launch shape must be prepared as for lora_apply.  Every call on one GPU
 * shares that GPU's array: calls on one GPU that overlap in time (other
 * streams, other threads) race on it and must be serialised by the caller. */
lora_status lora_apply_noalloc(lora_pool* pool, const lora_plan* plan, int32_t n_io,
                               const lora_io* io_host, int32_t y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Decode with device ids, grouped on the device (S-LoRA paper explainer,
 * section "BGMVカーネル": one launch sequence for a batch whose tokens carry
 * their own adapters and ranks; multi-LoRA serving article, SGMV section: the
 * index vector sends tokens to adapters, tokens of one adapter form one
 * segment).
 * ------------------------------------------------------------------------- */
/* Bytes of caller-owned device workspace that lora_bgmv_apply_planned needs
 * for n tokens over the slices of io (only io[k].slice is read): the plan and
 * a bound on its split-K partial tiles (about 10 MB for 256 tokens, two
 * slices, rank <= 64).  LORA_E_UNSUPPORTED on pools the MFMA tiles cannot
 * take (FP8 or fp32 pages, fewer than 16 B rows per page, A rows over more
 * than 8 pages). */
lora_status lora_bgmv_planned_workspace_size(lora_pool* pool, int32_t n_io,
                                             const lora_io* io_host, int32_t n,
                                             size_t* bytes);
/* y_i += s_a B_a (A_a x_i) for every token i of the slices of io, like
 * lora_bgmv_apply, with ids_dev [n] on the device (ids outside [0,
 * max_adapters): the token is skipped; an adapter not resident in a slice
 * leaves that slice's row untouched).  One workgroup sorts the tokens by
 * adapter into tiles of at most 64 tokens and lays out the block ranges of
 * the planned MFMA kernels in the workspace, then the fused shrink and expand
 * launches run from it: three launches on `stream`, no host wait, no
 * allocation (graph-capturable).  n <= 1024; 16-bit pools only.  workspace_dev:
 * 256-byte aligned, at least lora_bgmv_planned_workspace_size bytes (else
 * LORA_E_ARG), no initial contents; calls sharing a workspace must not
 * overlap. */
lora_status lora_bgmv_apply_planned(lora_pool* pool, int32_t n_io, const lora_io* io_host,
                                    const int32_t* ids_dev, int32_t n, int32_t y_dtype,
                                    void* workspace_dev, size_t ws_bytes, void* stream);

/* A device plan kept between calls, for the layers of a model whose LoRA calls
 * share one decode step's ids: built once per step from the ids on the device,
 * applied to every launch whose slices have the shapes it was created for.
 * lora_dplan_create: for up to max_tokens tokens over slices with the shapes
 * (d_in, d_out) of io[k].slice, in this order; allocates the plan's device
 * workspace (the same size as lora_bgmv_planned_workspace_size), so it may
 * allocate and synchronise; refusals as for lora_bgmv_planned_workspace_size.
 * lora_dplan_destroy waits for the device. */
lora_status lora_dplan_create(lora_pool* pool, int32_t max_tokens, int32_t n_io,
                              const lora_io* io_host, lora_dplan** out);
lora_status lora_dplan_destroy(lora_dplan* dplan);
/* The planning launch of lora_bgmv_apply_planned alone, on `stream`: groups
 * the n (<= max_tokens) ids by adapter.  A token takes part when its adapter
 * is resident in at least one slice of io (same shapes as at creation, else
 * LORA_E_ARG).  Stream-ordered, no allocation, no wait. */
lora_status lora_dplan_build(lora_dplan* dplan, int32_t n_io, const lora_io* io_host,
                             const int32_t* ids_dev, int32_t n, void* stream);
/* The MFMA launches of lora_bgmv_apply_planned from the last build, on
 * `stream` (stream-ordered after that build), for slices with the plan's
 * shapes in the plan's order (other layers' slices included: LORA_E_ARG
 * otherwise).  An adapter not resident in a slice leaves that slice's rows
 * untouched.  LORA_E_STATE before a build or after any residency change of
 * the pool since it.  Calls reading one plan may run one after another; a
 * build while earlier applies of the plan are in flight on another stream
 * races with them. */
lora_status lora_dplan_apply(lora_pool* pool, const lora_dplan* dplan, int32_t n_io,
                             const lora_io* io_host, int32_t y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Debug / verification of the page-table resolution done inside the kernels.
 * ------------------------------------------------------------------------- */
/* For token i: a_off[i][k*npa + c] = byte offset (from the pool base) of page
 * chunk c of A row k (k < max_rank; -1 past the rank or for id < 0), and
 * b_off[i][m] = byte offset of B row m (m < d_out; -1 for id < 0).  Computed by
 * the device resolver the compute kernels use. */
lora_status lora_debug_resolve(lora_pool* pool, int32_t slice, const int32_t* ids_dev,
                               int32_t n, int64_t* a_off_dev, int64_t* b_off_dev,
                               void* stream);
/* Gather one adapter slice through the device page table into dense
 * A [rank][d_in] and B [d_out][rank] (pool dtype). */
lora_status lora_debug_gather(lora_pool* pool, int32_t slice, int32_t adapter, void* A_dev,
                              void* B_dev, void* stream);

/* Decode n stored elements of `dtype` (src_dev, 16-byte aligned, n * element
 * bytes a multiple of 16) to fp32 dst_dev with the decoder the compute kernels
 * use. */
lora_status lora_debug_decode(int32_t dtype, const void* src_dev, int64_t n, float* dst_dev,
                              void* stream);

/* Profiling: per-block timeline of the last lora_bgmv_apply launch that ran
 * one block per (slice, token) unit, in a library built with
 * LORA_BLOCK_TIMELINE (build.py --timeline); LORA_E_UNSUPPORTED in other
 * builds.  Copies up to `bytes` (a multiple of 64) into host memory: per block
 * index, 8 uint64 words {start, end} (100 MHz constant clock), the hardware
 * wave id register of the block's first wave (compute unit, shader array and
 * engine fields), slice (-1: past the batch), rank (0: skipped token), token,
 * row split, 1.  Records of blocks that did not run in that launch keep older
 * contents.  Waits for the copy. */
lora_status lora_debug_block_timeline(void* host, size_t bytes);

/* Message of the last failing call on this thread ("" if none). */
const char* lora_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LORA_MI355X_H */

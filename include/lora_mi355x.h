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
 *     are stream-ordered and never synchronise the host.
 *   - x rows are d_in elements of the pool dtype, y rows d_out elements of
 *     y_dtype (the pool dtype or LORA_F32), both dense row-major, 16-byte
 *     aligned base pointers.  v (the shrink output) is fp32 [n][v_ld].
 *   - Adapter ids on the device must lie in [-1, max_adapters) and name
 *     adapters resident in the slice used; this is a contract the kernels do
 *     not check (a non-resident adapter contributes nothing).  Host-side ids
 *     (lora_plan_build) are checked.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LORA_F32 = 0, LORA_F16 = 1, LORA_BF16 = 2 } lora_dtype;

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
 *         fp32, 8 for fp16/bf16)
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
 * Invalidates the device page table until lora_page_table_build. */
lora_status lora_pool_upload(lora_pool* pool, int32_t adapter, int32_t slice, int32_t rank,
                             float scale, const void* A_host, const void* B_host,
                             void* stream);
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
/* Copy pages [first, first+count) of the pool to host memory (synchronous). */
lora_status lora_pool_read_pages(const lora_pool* pool, int64_t first, int64_t count,
                                 void* dst_host);

/* One adapted projection in a multi-slice launch: its slice index, its input
 * x [n][d_in] and its output y [n][d_out] (accumulated in place). */
typedef struct {
  int32_t slice;
  int32_t reserved;
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
 * leaves the chip).  All io entries share ids and n. */
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
 * On 16-bit pools the MFMA tiles also need, per launch shape (the slices of a
 * call), block-range tables and split-K contribution lists -- built on the
 * host at the first call of that shape after lora_plan_build and copied on the
 * call's stream; the plan keeps four shapes -- and a workspace of partial
 * tiles (16 bytes per token block x rank block x 64 per contribution, a few
 * MB), grown at first use (growing synchronizes the device).  A plan is used
 * by one stream and one host thread at a time: calls that use the same plan
 * must not overlap (they share its workspace and layout cache). */
lora_status lora_plan_create(lora_pool* pool, int32_t max_tokens, lora_plan** out);
lora_status lora_plan_destroy(lora_plan* plan);
/* Build the plan of one batch from host ids [n] (any order, -1 = no adapter):
 * stable counting sort by adapter -> groups; on fp16/bf16 pools groups of at
 * least l_long tokens become MFMA tiles of up to 64 tokens (l_long <= 0: 1, i.e.
 * every group), the others -- and every group of an fp32 pool -- short items of
 * <= 4 tokens on the vector ALUs; items ordered MFMA first, then by rank band,
 * largest first.  Every id >= 0 must be < max_adapters and resident in every
 * slice (LORA_E_NOT_RESIDENT otherwise).  The plan is copied to the device on
 * `stream`; the host ids may be reused on return.  The SGMV calls below launch
 * one kernel per item kind present in the plan. */
lora_status lora_plan_build(lora_plan* plan, const int32_t* ids_host, int32_t n,
                            int32_t l_long, void* stream);
lora_status lora_plan_get_stats(const lora_plan* plan, lora_plan_stats* out);
/* Host copy of the plan: perm [n_tokens] (token indices, grouped by adapter)
 * and items [n_items][4] = {adapter, start in perm, count, kind (0 short,
 * 1 MFMA tile)}.  Either pointer may be NULL. */
lora_status lora_plan_export(const lora_plan* plan, int32_t* perm_host, int32_t* items_host);

/* Shrink for a planned batch: v[i][.] as lora_bgmv_shrink (rows indexed by the
 * original token index).  MFMA tiles: two launches (block ranges, then the sum
 * of the partial tiles of every tile that several ranges share, in block
 * order). */
lora_status lora_sgmv_shrink(lora_pool* pool, const lora_plan* plan, int32_t slice,
                             const void* x_dev, float* v_dev, int32_t v_ld, void* stream);
/* Expand for a planned batch: y[i] += s B v[i]. */
lora_status lora_sgmv_expand(lora_pool* pool, const lora_plan* plan, int32_t slice,
                             const float* v_dev, int32_t v_ld, void* y_dev, int32_t y_dtype,
                             void* stream);
/* Fused shrink + expand for a planned (mixed prefill + decode) batch, for up to
 * LORA_MAX_IO slices; v is never materialized.  Short items: one launch, v in
 * LDS.  MFMA tiles: two launches on `stream` (shrink ranges keep partial tiles
 * in the plan's workspace; the expand sums them while loading V). */
lora_status lora_apply(lora_pool* pool, const lora_plan* plan, int32_t n_io,
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

/* Message of the last failing call on this thread ("" if none). */
const char* lora_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LORA_MI355X_H */

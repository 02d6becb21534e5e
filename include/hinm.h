/*
 * hinm.h - C ABI of libhinm: hierarchical N:M (HiNM) sparse weight x dense
 * activation product for AMD Instinct MI355X (gfx950).
 *
 * The operation (FlexHiNM-GP paper notes, one-line summary, "整体框架" and key
 * designs 1, 2 and 4): every output-channel tile of a weight W [cout x cin] is
 * cut into three regions of whole column vectors - dense (4:4), 2:4 (top two of
 * every four consecutive entries along the input dimension, 2-bit positions as
 * in the 2:4 structured-sparsity article, section 3) and pruned (0:4).  The
 * sizes of the regions follow the closed form
 *     t_s = v_s + (1 - v_s) * p_s / 2,   p_s = 2 (t_s - v_s) / (1 - v_s)
 * where t_s is the target sparsity and v_s the pruned-vector fraction.  The
 * input channels of each tile are permuted (PermLLM summary, problem
 * definition: W_hat = W P); the product gathers rows of X through per-tile
 * kept-vector indices that already include the permutation, so the result is
 *     Y = (W (.) M) X,    Y [cout x batch], X [cin x batch].
 *
 * Conventions shared by every entry point
 *   - All matrices are row-major.  W, X and Y hold bf16 values (raw 16-bit
 *     patterns, passed as void*), importance holds fp32.  Accumulation is fp32.
 *   - Device pointers are device memory owned by the caller; the library never
 *     allocates or frees device memory and keeps no device state.  Host
 *     pointers are marked "host".
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Functions return a hinm_status and never throw.  On failure a message is
 *     available from hinm_last_error() in the calling thread.  Argument errors
 *     are detected on the host before anything is launched.
 *   - Functions are re-entrant; calls that share output or workspace buffers
 *     must not overlap in time.
 */
#ifndef HINM_H_
#define HINM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HINM_ABI_VERSION 2

/* Version of the packed-buffer layout described at hinm_packed_t and
 * hinm_tpacked_t.  A stored packed weight carries it; a different value
 * means the bytes must be packed again from the weight. */
#define HINM_FORMAT_VERSION 1

/* K-block sizes of the packed layout: 32 dense columns; 64 positions
 * (16 groups of 4) of the 2:4 region. */
#define HINM_KB_DENSE 32
#define HINM_KB_24 64

typedef enum {
  HINM_OK = 0,
  HINM_EINVAL = 1,      /* null pointer, non-finite or out-of-range t_s / v_s        */
  HINM_ESHAPE = 2,      /* sizes: cout % tile_rows, cin % 4, tile_rows % 16, ld < n  */
  HINM_EPERM = 3,       /* a perm row is not a permutation of 0..cin-1 (device check) */
  HINM_EIMPORTANCE = 4, /* importance has a negative or non-finite entry (device)    */
  HINM_EALIGN = 5,      /* a pointer is not aligned as documented                    */
  HINM_EWORKSPACE = 6,  /* workspace missing or smaller than required                */
  HINM_EHIP = 7,        /* a HIP runtime call or kernel launch failed                */
  HINM_EDEVICE = 8      /* no usable gfx950 device                                   */
} hinm_status;

/* Region counts and buffer sizes of one weight.  Plain data, computed on the
 * host by hinm_plan; identical in every output tile. */
typedef struct {
  int32_t abi_version;  /* HINM_ABI_VERSION                                          */
  int32_t cout, cin;    /* W is cout x cin                                           */
  int32_t tile_rows;    /* rows per output-channel tile (R)                          */
  int32_t n_tiles;      /* cout / tile_rows                                          */
  int32_t z;            /* zeros per row: floor(t_s * cin + 1/2)                     */
  int32_t groups;       /* 2:4 groups per tile row: n_24 / 4                         */
  int32_t n_dense;      /* dense (4:4) vectors per tile                              */
  int32_t n_24;         /* 2:4 vectors per tile                                      */
  int32_t n_pruned;     /* pruned (0:4) vectors per tile                             */
  int32_t n_dense_pad;  /* n_dense rounded up to HINM_KB_DENSE                       */
  int32_t n_24_pad;     /* n_24 rounded up to HINM_KB_24                             */
  int32_t kb_dense;     /* HINM_KB_DENSE                                             */
  int32_t kb_24;        /* HINM_KB_24                                                */
  double t_s, v_s;      /* the arguments                                             */
  double p_s;           /* 2 (t_s - v_s) / (1 - v_s), informational                  */
  int64_t bytes_val_dense; /* n_tiles * n_dense_pad * tile_rows * 2                  */
  int64_t bytes_idx_dense; /* n_tiles * n_dense_pad * 4                              */
  int64_t bytes_val_24;    /* n_tiles * (n_24_pad / 2) * tile_rows * 2               */
  int64_t bytes_meta_24;   /* n_tiles * (n_24_pad / 64) * tile_rows * 8              */
  int64_t bytes_idx_24;    /* n_tiles * n_24_pad * 4                                 */
} hinm_plan_t;

/* A packed weight: the plan plus five caller-owned device buffers (each at
 * least 16-byte aligned, sized by the plan; a buffer of size 0 may be NULL).
 *   val_dense  bf16   [n_tiles][n_dense_pad/32][tile_rows][32]
 *              val_dense[t][kb][r][k] = W[t*R + r][idx_dense[t][32*kb + k]]
 *   idx_dense  int32  [n_tiles][n_dense_pad]   dense columns in permuted order
 *   val_24     bf16   [n_tiles][n_24_pad/64][tile_rows][32]
 *              two kept values per group, group g of block kb at [2g, 2g+1],
 *              lower in-group position first
 *   meta_24    uint64 [n_tiles][n_24_pad/64][tile_rows]
 *              group g's nibble (i0 | i1 << 2, i0 < i1, positions 0..3 within
 *              the group) at bits 4g..4g+3
 *   idx_24     int32  [n_tiles][n_24_pad]      2:4 columns in permuted order;
 *              group q of a tile is idx_24[t][4q .. 4q+3]
 * Padding: indices -1, values +0, nibbles 0x4. */
typedef struct {
  hinm_plan_t plan;
  void* val_dense;
  int32_t* idx_dense;
  void* val_24;
  uint64_t* meta_24;
  int32_t* idx_24;
  uint32_t flags;     /* HINM_PACKED_* bits describing the index lists (set by hinm_pack; 0 = none known) */
  uint32_t reserved;  /* 0 */
} hinm_packed_t;

/* flags bit: every perm row kept each column inside its aligned block of 64
 * positions (a block-diagonal permutation with blocks of 64, PermLLM
 * summary, block-wise permutation; NULL perm included), so every tile's
 * index lists walk X in windows of 64 rows, in the same order.  The product
 * then orders its batch > 64 work items in pairs of token blocks per tile
 * (the X rows that tiles read at one time stay near each other in the L2
 * cache) - the same bits of Y.  hinm_translate_indices clears it unless its
 * map is block-diagonal too.  A caller that builds hinm_packed_t itself may
 * leave flags 0. */
#define HINM_PACKED_WINDOWED 1u

/* Per-tile region counts (FlexHiNM-GP notes, "整体框架": the ratio of the
 * three regions is decided inside each output-channel tile).  t_s is shared,
 * so every row keeps cin - z entries; each tile has its own v_s and so its
 * own dense / 2:4 / pruned counts.  The K-blocks of the tiles are laid end
 * to end in the packed buffers, and a tile table locates them.  Plain data,
 * computed on the host by hinm_plan_tiles. */
typedef struct {
  int32_t abi_version;     /* HINM_ABI_VERSION                                        */
  int32_t cout, cin, tile_rows, n_tiles;
  int32_t z;               /* zeros per row, as in hinm_plan_t                        */
  int32_t max_n_dense_pad; /* largest per-tile n_dense rounded up to HINM_KB_DENSE    */
  int32_t max_n_24_pad;    /* largest per-tile n_24 rounded up to HINM_KB_24          */
  int32_t dense_blocks;    /* total dense K-blocks (32 columns) over the tiles        */
  int32_t blocks_24;       /* total 2:4 K-blocks (64 positions) over the tiles        */
  double t_s;
  int64_t bytes_val_dense; /* dense_blocks * tile_rows * 32 * 2                       */
  int64_t bytes_idx_dense; /* dense_blocks * 32 * 4                                   */
  int64_t bytes_val_24;    /* blocks_24 * tile_rows * 32 * 2                          */
  int64_t bytes_meta_24;   /* blocks_24 * tile_rows * 8                               */
  int64_t bytes_idx_24;    /* blocks_24 * 64 * 4                                      */
  int64_t bytes_tiles;     /* n_tiles * 4 * 4                                         */
} hinm_tplan_t;

/* A packed weight with per-tile counts.  Buffers as in hinm_packed_t with
 * the tile axis folded into the block axis: tile t's dense blocks are
 * blocks tiles[t][0] .. tiles[t][0] + ceil(tiles[t][1] / 32) - 1 of
 * val_dense [dense_blocks][tile_rows][32] and of idx_dense
 * [dense_blocks * 32]; its 2:4 blocks start at block tiles[t][2] of val_24
 * [blocks_24][tile_rows][32], meta_24 [blocks_24][tile_rows] and idx_24
 * [blocks_24 * 64].  `tiles` (device, caller-owned, filled by the caller
 * from the table hinm_plan_tiles returns) is int32 [n_tiles][4]: first
 * dense block, n_dense, first 2:4 block, n_24. */
typedef struct {
  hinm_tplan_t plan;
  const int32_t* tiles;
  void* val_dense;
  int32_t* idx_dense;
  void* val_24;
  uint64_t* meta_24;
  int32_t* idx_24;
} hinm_tpacked_t;

/* Library ABI version (HINM_ABI_VERSION of the build). */
int hinm_abi_version(void);

/* Launch-shape options of the product (for tuning and for tests that run
 * every kernel variant; the defaults are the measured best).  They are
 * process-wide.  Each starts from its environment variable, read once, at
 * the first call that uses any option; afterwards only hinm_set_option
 * changes them.  An unset or invalid variable gives the default.
 *   HINM_OPT_DECODE_PATH      env HINM_DECODE_PATH=rows16 -> 1: batch <= 64
 *                             runs the 16-row kernel without a K split
 *                             (default 0: the split kernel when tile_rows %
 *                             64 == 0)
 *   HINM_OPT_DECODE_WGS       env HINM_DECODE_WGS: about how many
 *                             workgroups the batch <= 64 kernel splits K over
 *                             (default 256; 1 .. 2^20).  With the default,
 *                             a launch whose row blocks times splits fall
 *                             between 256 and 512 gives its last row blocks
 *                             twice the splits, so that 512 workgroups run
 *                             (two share a compute unit at batch <= 32).  A
 *                             different split count may change the last bits
 *                             of Y.
 *   HINM_OPT_PREFILL_NT       env HINM_PREFILL_NT: token block of the
 *                             batch > 64 kernel, 128 or 256 (default 0:
 *                             256 from batch 1024; from 256 to 1023, 256
 *                             when it takes fewer rounds of the persistent
 *                             grid, or as many with at least as many
 *                             workgroups and >= 120 K units per tile (a
 *                             2:4 block counting two); else 128)
 *   HINM_OPT_PREFILL_SPLITS   env HINM_PREFILL_SPLITS: K split of each
 *                             batch > 64 work item, 1, 2 or 4 (default 0: 2
 *                             or 4 up to 128 items; 2 with 225 to 256 items
 *                             on a K range of >= 120 units; between 256 and
 *                             512 items of 128 tokens in two or more token
 *                             blocks, the first items of each XCD whole and
 *                             the rest in two halves; else 1.  Cut in
 *                             two, an item's K range is cut by cost (a
 *                             dense block one unit, a 2:4 block two); in
 *                             four, by block count.  A different split may
 *                             change the last bits of Y)
 *   HINM_OPT_PREFILL_PATH     env HINM_PREFILL_PATH=staged -> 1: the
 *                             batch > 64 kernel gathers X through registers
 *                             instead of straight into LDS (same bits of Y)
 *   HINM_OPT_PREFILL_PER_XCD  env HINM_PREFILL_PER_XCD: persistent
 *                             workgroups per XCD of the batch > 64 kernel
 *                             (default 0: 64; 1 .. 1024)
 *   HINM_OPT_PREFILL_TB_GROUP env HINM_PREFILL_TB_GROUP: the batch > 64
 *                             kernel orders its (token block, row block)
 *                             items in groups of this many token blocks,
 *                             row-block major inside a group, so an XCD
 *                             takes fewer tiles over more token blocks
 *                             (default 0: 2 for a weight whose flags hold
 *                             HINM_PACKED_WINDOWED, else 1, token-block
 *                             major; 1 .. 64; same bits of Y)
 *   HINM_OPT_PREFILL_STAGGER  env HINM_PREFILL_STAGGER: 0 (default): the
 *                             batch > 64 kernel starts tile t's dense and
 *                             2:4 K loops, in token block tb, at block
 *                             t * n / n_tiles + ((3 tb) mod 8) * n / 8 (mod
 *                             n) of its n and wraps around, so tiles whose
 *                             index lists walk X in the same order
 *                             (block-diagonal or identity perms) do not read
 *                             the same rows at the same time, and XCDs on
 *                             different token blocks do not read a tile's
 *                             packed values at the same time; 1: every tile
 *                             from its first block.  Either order is
 *                             deterministic; they add the products in
 *                             different orders.
 * A change applies to products launched afterwards; a workspace sized under
 * other settings may then be too small (HINM_EWORKSPACE). */
typedef enum {
  HINM_OPT_DECODE_PATH = 1,
  HINM_OPT_DECODE_WGS = 2,
  HINM_OPT_PREFILL_NT = 3,
  HINM_OPT_PREFILL_SPLITS = 4,
  HINM_OPT_PREFILL_PATH = 5,
  HINM_OPT_PREFILL_PER_XCD = 6,
  HINM_OPT_PREFILL_TB_GROUP = 7,
  HINM_OPT_PREFILL_STAGGER = 8,
  HINM_OPT_COUNT = 9
} hinm_option;

/* Sets an option (host only).  Errors: HINM_EINVAL (unknown option or value
 * out of its range; the option is then unchanged). */
int hinm_set_option(int option, int64_t value);

/* Current value of an option into *value (host).  Errors: HINM_EINVAL. */
int hinm_get_option(int option, int64_t* value);

/* Region counts for a cout x cin weight (FlexHiNM-GP notes, key design 1).
 * Host only, touches no device.  Requires cout, cin > 0, tile_rows % 16 == 0,
 * cout % tile_rows == 0, cin % 4 == 0 (pad the input dimension as the N:M
 * article's section 2 does), 0 <= t_s < 1 and
 * max(0, 2 t_s - 1) <= v_s <= t_s, so that p_s lies in [0, 1].
 * Counts: z = floor(t_s*cin + 1/2); g = floor((t_s - v_s)*cin/2 + 1/2)
 * clamped to [0, floor(min(z, cin - z)/2)]; n_24 = 4g; n_pruned = z - 2g;
 * n_dense = cin - z - 2g.  Every row keeps cin - z entries.
 * `out` (host) receives the plan.  Errors: HINM_EINVAL, HINM_ESHAPE. */
int hinm_plan(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double v_s,
              hinm_plan_t* out);

/* Device scratch that hinm_pack needs, in bytes (host only). */
int hinm_pack_workspace_bytes(const hinm_plan_t* plan, size_t* bytes);

/* Pack a weight (FlexHiNM-GP notes, key designs 1, 2 and 4; 2:4 article,
 * section 3; PermLLM summary, mask on the permuted importance):
 *   1. score every column vector of every tile: the float64 sum of its
 *      importance over the tile's rows, rows in ascending order from +0.0;
 *   2. rank columns by (-score, column): the first n_dense are dense, the
 *      next n_24 are 2:4, the rest pruned;
 *   3. list dense and 2:4 columns in the tile's permuted order perm[t][0..];
 *   4. in every 2:4 group of 4 listed columns and every row keep the two
 *      entries with the largest importance (ties: lower position);
 *   5. write the packed buffers of `out` (layout above).
 * Inputs (device): w_bf16 [cout][ldw], importance fp32 [cout][ldi] (finite,
 * >= 0), perm int32 [n_tiles][cin] or NULL for the identity; perm[t][j] is
 * the original column at position j of tile t.  `plan` (host) comes from
 * hinm_plan; `out` (host) holds the plan copy and the output pointers, which
 * the caller allocates from the plan's sizes.  workspace (device, 256-byte
 * aligned) of hinm_pack_workspace_bytes bytes.
 * Synchronous: returns after the work on `stream` has finished, because a bad
 * perm or importance is detected on the device (HINM_EPERM, HINM_EIMPORTANCE;
 * the outputs are then unspecified).  Other errors: HINM_EINVAL, HINM_ESHAPE,
 * HINM_EALIGN, HINM_EWORKSPACE, HINM_EHIP. */
int hinm_pack(const hinm_plan_t* plan, const void* w_bf16, int64_t ldw, const float* importance,
              int64_t ldi, const int32_t* perm, hinm_packed_t* out, void* workspace,
              size_t workspace_bytes, void* stream);

/* Device scratch that hinm_spmm needs for a batch, in bytes (host only).
 * Zero when the product runs without a split of the reduction dimension. */
int hinm_spmm_workspace_bytes(const hinm_plan_t* plan, int64_t batch, size_t* bytes);

/* Y = (W (.) M) X for a packed weight (FlexHiNM-GP notes, key design 4: the
 * kernel gathers X rows through the precomputed indices, with the input
 * permutation folded in).  X (device) bf16 [cin][ldx], ldx >= batch; Y
 * (device) bf16 [cout][ldy], ldy >= batch, every element of Y[:, 0:batch] is
 * written (rounded to nearest even from the fp32 accumulator), nothing else.
 * X and Y must be 2-byte aligned.  X rows are gathered with 16-byte loads
 * whatever the layout; rows that are not 16-byte aligned (X not 16-byte
 * aligned, or ldx % 8 != 0) cost more, as most loads then straddle cache
 * lines.  workspace (device, 256-byte aligned) of at least
 * hinm_spmm_workspace_bytes(plan, batch) bytes, may be NULL when that is 0.
 * The workspace must be zero-filled before its first use; every call that
 * returns HINM_OK leaves it ready for the next one (its arrival counters are
 * back at zero when the work on `stream` completes).  Calls sharing one
 * workspace must be ordered (same stream, or synchronised).
 * batch == 0 is a no-op.  Asynchronous on `stream`; no host synchronisation.
 * Partial sums of a split reduction dimension are added in split order, so
 * the same inputs give bitwise-identical Y on every call.
 * The launch shape follows the process-wide options of hinm_set_option;
 * the workspace size asked for must come from the same settings.
 * Errors (host-side checks only): HINM_EINVAL, HINM_ESHAPE, HINM_EALIGN,
 * HINM_EWORKSPACE, HINM_EHIP (launch failure). */
int hinm_spmm(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx,
              void* y_bf16, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Several packed weights multiplied by one X, in one launch where possible:
 *     Y_g = (W_g (.) M_g) X,   g = 0 .. n-1
 * (FlexHiNM-GP notes, key design 4: each product gathers X rows through its
 * weight's precomputed indices).  This is the product hinm_spmm computes,
 * once per weight; weights that read the same activations (the q, k and v
 * projections of a transformer layer, or gate and up) then share one launch,
 * so at small batches the weights' rows together fill the device without
 * splitting the reduction dimension, and no launch waits for another's tail.
 * packed (host) [n] pointers to packed weights with equal cin and tile_rows
 * (1 <= n <= 8; region counts may differ); y (host) [n] device pointers,
 * Y_g bf16 [cout_g][ldy[g]]; ldy (host) [n], each >= batch.  X, workspace,
 * stream, rounding and errors as hinm_spmm; the workspace comes from
 * hinm_spmm_group_workspace_bytes.  With tile_rows % 64 == 0 one launch runs
 * the group (the split count follows the group's total rows, so the last
 * bits of Y_g may differ from hinm_spmm's at batch <= 64); otherwise the
 * weights run one launch each on `stream`.  Deterministic. */
int hinm_spmm_group_workspace_bytes(int n, const hinm_packed_t* const* packed, int64_t batch, size_t* bytes);
int hinm_spmm_group(int n, const hinm_packed_t* const* packed, const void* x_bf16, int64_t batch, int64_t ldx,
                    void* const* y_bf16, const int64_t* ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device array that holds hinm_spmm_noalloc's scratch: 64 KiB
 * of arrival counters and 32 MiB of partial sums, one copy on every device
 * the library runs on, held until the process ends.  Every launch shape the
 * default options choose fits: the split decode (batch <= 64) needs at most
 * 4 MiB of partials, the K split of larger batches (at most 512 workgroups
 * of 256 threads x up to 64 floats) and the generic kernel's split at most
 * 32 MiB. */
#define HINM_NOALLOC_SCRATCH_BYTES ((size_t)65536 + ((size_t)32 << 20))

/* hinm_spmm without a workspace argument and without any device allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc.  The scratch
 * of the split reduction lives in a static device array of
 * HINM_NOALLOC_SCRATCH_BYTES that the library holds on each device; the
 * first call on a device takes its address and clears its counters (a fill
 * kernel on `stream`).  Every call on one device shares that array, so calls
 * that overlap in time on one device (different streams, or work queued
 * from another thread) race on it and give wrong results; calls on one
 * stream are safe.  The array keeps the last call's partial sums; its
 * counters are back at zero whenever no call is in flight.
 * A product whose scratch need (hinm_spmm_workspace_bytes) exceeds
 * HINM_NOALLOC_SCRATCH_BYTES - possible only under options that force more
 * splits (hinm_set_option) - is refused with HINM_EWORKSPACE before
 * anything is launched.  Arguments, result bits and other errors as
 * hinm_spmm. */
int hinm_spmm_noalloc(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx, void* y_bf16,
                      int64_t ldy, void* stream);

/* hinm_spmm with the output-channel permutation fused into the write-out
 * (FlexHiNM-GP notes, key design 2: the output channels of a tile are
 * permuted before pruning, and the permutation is undone where the data
 * moves anyway; highlights: permutation at no run-time cost).  Row r of the
 * product (W's row order, which is the order the weight was packed in) is
 * written to Y row out_rows[r]:  Y[out_rows[r]][n] = ((W (.) M) X)[r][n].
 * out_rows (device) int32 [cout], 4-byte aligned, a permutation of
 * 0..cout-1; an entry outside [0, cout) leaves nothing written for that row
 * (the device does not check that out_rows is a permutation; rows that two
 * entries name receive one of the two results).  All other arguments,
 * errors and guarantees as hinm_spmm; out_rows == NULL is HINM_EINVAL. */
int hinm_spmm_rows(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx, void* y_bf16,
                   int64_t ldy, const int32_t* out_rows, void* workspace, size_t workspace_bytes, void* stream);

/* Cross-layer index translation (FlexHiNM-GP notes, key design 2: the
 * translation between one layer's output order and the next layer's input
 * order is folded into the HiNM index lists; key design 4: the kernel
 * gathers X rows through those indices).  Every non-negative entry i of
 * packed->idx_dense and packed->idx_24 becomes map[i]; pads (-1) stay.  Use
 * map[c] = the position at which the activations hold input channel c, so
 * that a product over activations stored in that order equals the product
 * over activations in channel order, bit for bit.
 * map (device) int32 [cin], 4-byte aligned, must be a permutation of
 * 0..cin-1; it is checked on the device first and nothing is written if it
 * is not (HINM_EPERM).  workspace (device, 256-byte aligned, >= 256 bytes).
 * Synchronous (returns after the work on `stream` has finished).  Errors:
 * HINM_EINVAL, HINM_EPERM, HINM_EALIGN, HINM_EWORKSPACE, HINM_EHIP,
 * HINM_EDEVICE. */
int hinm_translate_indices(hinm_packed_t* packed, const int32_t* map, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Device scratch that hinm_boundary_search needs, in bytes (host only; the
 * same for every t_s). */
int hinm_boundary_workspace_bytes(int64_t cout, int64_t cin, int32_t tile_rows, size_t* bytes);

/* Boundary search for v_s (FlexHiNM-GP notes, key design 1): with t_s fixed,
 * the closed form leaves v_s as the only free parameter; the search starts
 * at v_s = t_s and lowers it by `step` while the retained importance
 *     R_total(v) = R_dense(v) + R_24(v)
 * does not decrease, stopping at the first strict decrease.  R_dense sums
 * the vector scores (as in hinm_pack, step 1) of the dense columns of every
 * tile; R_24 sums, over every row and every 2:4 group (as in hinm_pack,
 * steps 2-4, with the region counts of v), the two largest importances of
 * the group.  Grid: v_k = t_s - step*k for k = 0, 1, ... while
 * v_k >= max(0, 2 t_s - 1) - 1e-12, the last point clamped to that bound.
 * The result is n_pruned / cin of the plan at the last v before the
 * decrease (so hinm_plan reproduces the same counts from it).  Sums are
 * float64 in a fixed order (per tile and per row on the device, then the
 * tiles and rows in ascending order on the host): the same inputs give the
 * same trace on every call.
 * Inputs (device): importance fp32 [cout][ldi] (finite, >= 0), perm int32
 * [n_tiles][cin] or NULL.  Outputs (host): *v_s_out; the first trace_cap
 * grid points visited and their R_total in trace_v / trace_r (may be NULL
 * when trace_cap == 0), their number in *trace_len (may be NULL).
 * workspace (device, 256-byte aligned) of hinm_boundary_workspace_bytes.
 * Synchronous.  Errors: HINM_EINVAL (also a non-positive step), HINM_ESHAPE,
 * HINM_EPERM, HINM_EIMPORTANCE, HINM_EALIGN, HINM_EWORKSPACE, HINM_EHIP,
 * HINM_EDEVICE. */
int hinm_boundary_search(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double step,
                         const float* importance, int64_t ldi, const int32_t* perm, void* workspace,
                         size_t workspace_bytes, double* v_s_out, double* trace_v, double* trace_r,
                         int32_t trace_cap, int32_t* trace_len, void* stream);

/* Per-tile plan (host only).  v_s (host) [n_tiles]: tile t's v_s, each in
 * [max(0, 2 t_s - 1), t_s]; tile t's counts are those of hinm_plan at
 * (t_s, v_s[t]).  out (host) receives the shared fields and the buffer
 * sizes; tiles_out (host) int32 [n_tiles][4] the tile table (copy it to the
 * device for hinm_pack_tiles / hinm_spmm_tiles).  Errors as hinm_plan. */
int hinm_plan_tiles(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, const double* v_s, hinm_tplan_t* out,
                    int32_t* tiles_out);

/* Device scratch for hinm_pack_tiles, in bytes (host only). */
int hinm_pack_tiles_workspace_bytes(const hinm_tplan_t* plan, size_t* bytes);

/* hinm_pack with per-tile counts: the same five steps, tile t cut at its
 * own n_dense / n_24 (read from out->tiles).  Same inputs, guarantees and
 * errors as hinm_pack; out holds the plan copy, the device tile table and
 * the output buffers sized by the plan. */
int hinm_pack_tiles(const hinm_tplan_t* plan, const void* w_bf16, int64_t ldw, const float* importance, int64_t ldi,
                    const int32_t* perm, hinm_tpacked_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* Device scratch that hinm_spmm_tiles needs for a batch, in bytes (host only). */
int hinm_spmm_tiles_workspace_bytes(const hinm_tplan_t* plan, int64_t batch, size_t* bytes);

/* Y = (W (.) M) X for a packed weight with per-tile counts; as hinm_spmm.
 * Each tile runs its own number of K-blocks.  Requires tile_rows % 64 == 0
 * and buffers below 2^31 bytes (HINM_ESHAPE otherwise). */
int hinm_spmm_tiles(const hinm_tpacked_t* packed, const void* x_bf16, int64_t batch, int64_t ldx, void* y_bf16,
                    int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* The boundary search run inside each tile on its own (FlexHiNM-GP notes,
 * "整体框架": the region ratio is decided per tile; key design 1: the
 * search).  Tile t follows hinm_boundary_search's grid and stop rule on its
 * own retained importance R_t(v) = R_dense(t) + R_24(t); the grid goes on
 * while any tile has not stopped.  Outputs (host): v_s_tiles [n_tiles]
 * (n_pruned / cin of each tile's plan), points_tiles [n_tiles] (grid points
 * each tile visited; may be NULL).  Other arguments, workspace and errors as
 * hinm_boundary_search. */
int hinm_boundary_search_tiles(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double step,
                               const float* importance, int64_t ldi, const int32_t* perm, void* workspace,
                               size_t workspace_bytes, double* v_s_tiles, int32_t* points_tiles, void* stream);

/* In-tile input-channel gyro permutation (FlexHiNM-GP notes, key design 2:
 * channels are reordered so that important weights land where the structure
 * keeps them; the in-tile input step is rounds of drawing vectors from each
 * tile, a balanced K-means of them and a Hungarian assignment on a pruning
 * cost matrix).  It rewrites perm so that the 2:4 groups of plan's regions
 * drop less importance; the dense and pruned sets and their positions in
 * perm do not change.  One round, per tile, with G = plan->groups 2:4 groups
 * (group q = entries 4q..4q+3 of the tile's 2:4 list in perm order):
 *   1. the column at position sample[r][t][q] (0..3) of every group q is
 *      taken out, leaving a hole;
 *   2. its importance vector (float64 over the tile's rows) is clustered
 *      into N = ceil(G / cluster_size) clusters of sizes floor(G / N) or one
 *      more (the first G mod N clusters), centroids starting at the vectors
 *      of groups init[r][t][0..N-1] (distinct); each of kmeans_iters
 *      assignment steps gives every vector the cluster of the first
 *      (squared distance, group, cluster) triple in increasing order whose
 *      cluster has room, and centroids move to their members' mean between
 *      steps;
 *   3. inside every cluster the drawn columns go back into its holes by a
 *      minimum-cost assignment (Hungarian algorithm, lowest column index on
 *      equal reduced costs), the cost of a group being its pruning cost: per
 *      row the two smallest of its four importances, over the tile's rows.
 * No round raises a tile's pruning cost (putting every column back is one
 * assignment).  Distances, centroids and costs are float64 sums in a fixed
 * order, so the result is a function of the inputs alone.
 * importance (device) fp32 [cout][ldi] as for hinm_pack; perm (device) int32
 * [n_tiles][cin], in/out, each row a permutation of 0..cin-1 (checked on the
 * device, HINM_EPERM).  sample (host) uint8 [rounds][n_tiles][G]; init
 * (host) int32 [rounds][n_tiles][N]; both may be NULL when rounds == 0 or
 * G == 0.  cost_trace (host) float64 [rounds + 1][n_tiles] or NULL: the
 * pruning cost of every tile before the first round and after each round.
 * workspace (device, 256-byte aligned) of hinm_gyro_workspace_bytes.
 * Synchronous on `stream`.  Errors: HINM_EINVAL (counts, sample or init out
 * of range), HINM_ESHAPE, HINM_EALIGN, HINM_EPERM, HINM_EIMPORTANCE,
 * HINM_EWORKSPACE, HINM_EHIP. */
int hinm_gyro_workspace_bytes(const hinm_plan_t* plan, int32_t cluster_size, size_t* bytes);
int hinm_gyro_permute(const hinm_plan_t* plan, const float* importance, int64_t ldi, int32_t* perm, int32_t rounds,
                      int32_t cluster_size, int32_t kmeans_iters, const uint8_t* sample, const int32_t* init,
                      double* cost_trace, void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* hinm_status_str(int status);

/* Detail of the last failure in the calling thread ("" if none). */
const char* hinm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HINM_H_ */

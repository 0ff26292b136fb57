/*
 * thd_cp.h -- C ABI of the THD context-parallel layout transform (MI355X, gfx950).
 *
 * Packed variable-length batches ("THD": tokens x heads x dim, documents laid
 * end to end and described by a boundary list cu_seqlens) are sharded over cp
 * context-parallel ranks in one of two token layouts:
 *
 *   zigzag     every padded document of length L is cut into 2*cp chunks of
 *              L/(2*cp) tokens; rank r keeps chunk r and chunk 2*cp-1-r of
 *              every document, documents in order, the earlier chunk first
 *              (ring slice, page "Packed Sequence 与上下文并行", §2.4 and the
 *              worked example of §3.5);
 *   contiguous rank r keeps tokens [r*T/cp, (r+1)*T/cp) of the packed stream
 *              (Ulysses slice, same page §2.5).
 *
 * Both layouts are unions of global token intervals, so the route between them
 * is an interval intersection (Relax PR #273 "fla mcore chunkwise cp stage 3",
 * §2.1).  This library builds that route on the GPU from the padded boundary
 * list and applies it to row-major activations.  On one GPU the cross-rank
 * exchange is emulated: a buffer holds every rank's share, rank 0 first
 * ("emulated global rows": row = rank * T/cp + local row), and the swap is one
 * global row permutation.
 *
 * Conventions for every call:
 *  - pointers are device pointers unless the argument says "host";
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream); every
 *    call is stream-ordered and returns without waiting for the GPU, except
 *    the two marked SYNC;
 *  - boundary lists are int32 [n_slots + 1], non-decreasing, starting at 0;
 *    an empty slot (a repeated boundary) is allowed anywhere;
 *  - the call must be made with the route's device current;
 *  - return value: THD_OK (0), THD_IDENTITY (1, nothing written), or a
 *    negative THD_ERR_* code.  Argument errors are detected on the host and
 *    returned at once; errors that depend on boundary values are detected on
 *    the GPU and written to a device status word (see thd_route_status).
 *  - no call allocates or frees memory except thd_route_create/destroy, and
 *    no call synchronises except thd_route_status and thd_route_copy_out.
 */
#ifndef THD_CP_H
#define THD_CP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return and status codes ------------------------------------------ */
#define THD_OK                  0
#define THD_IDENTITY            1   /* swap is the identity: nothing written, use `in` */
#define THD_ERR_ARG            -1   /* null pointer, negative size, cp < 1, ...        */
#define THD_ERR_DIRECTION      -2   /* direction is neither of the two values below    */
#define THD_ERR_NOT_BUILT      -3   /* route never built                               */
#define THD_ERR_ALIAS          -4   /* input and output byte ranges overlap            */
#define THD_ERR_CAPACITY       -5   /* n_slots / cp_size / total_tokens above create() */
#define THD_ERR_SHAPE          -6   /* rows differs from the route's total_tokens      */
#define THD_ERR_HIP            -7   /* a HIP runtime call or kernel launch failed      */
#define THD_ERR_DEVICE         -8   /* current device differs from the route's device  */
/* Written on the device, in this precedence (first rule that fails wins): */
#define THD_ERR_CU_START      -10   /* cu[0] != 0                                      */
#define THD_ERR_CU_MONOTONE   -11   /* cu[i+1] < cu[i] for some i                      */
#define THD_ERR_CU_TOTAL      -12   /* cu[n_slots] != total_tokens                     */
#define THD_ERR_CU_DIVISIBLE  -13   /* a slot length is not a multiple of 2*cp_size    */
#define THD_ERR_REAL_GT_PADDED -14  /* roll: real length above padded length           */
#define THD_ERR_INTEGRITY     -15   /* route self-check failed (internal error)        */
#define THD_ERR_PACK_DOCS     -16   /* pack: more documents than max_docs              */
#define THD_ERR_PACK_CAPACITY -17   /* pack: padded documents longer than capacity     */

/* ---- directions ---------------------------------------------------------- */
#define THD_ZIGZAG_TO_CONTIGUOUS 0
#define THD_CONTIGUOUS_TO_ZIGZAG 1

/* ---- limits -------------------------------------------------------------- */
#define THD_MAX_CP        1024
#define THD_MAX_SHIFT     8
#define THD_MAX_BATCH     16
#define THD_PACK_MAX_SEQ  2147479552   /* 2^31 - 4096 tokens per packed row */
#define THD_PACK_STATIC_BYTES 1048576   /* device scratch of thd_pack_noalloc (1 MiB per GPU) */

typedef struct thd_route thd_route;   /* opaque; owns one device workspace */

/*
 * thd_route_create -- allocate a route able to hold any batch with at most
 * `max_slots` slots, `max_cp` ranks and `max_tokens` tokens (all >= 1,
 * max_cp <= THD_MAX_CP, max_tokens <= INT32_MAX).  The workspace lives on the
 * current device: (2*max_cp*max_slots + max_cp) runs in each of two orders
 * (8 B each), a max_cp^2 split matrix, two row directories of
 * ceil(max_tokens/16) + 1 entries of 16 B, 3*max_slots int32 of scratch and a
 * 64-byte header.  *out (host) receives the handle.  The only call that
 * allocates device memory.  Returns THD_OK, THD_ERR_ARG or THD_ERR_HIP.
 */
int thd_route_create(int32_t max_slots, int32_t max_cp, int64_t max_tokens, thd_route** out);

/* thd_route_destroy -- free the workspace (waits for the device to finish
 * using it).  NULL is ignored. */
void thd_route_destroy(thd_route* route);

/*
 * thd_build_route -- build the zigzag <-> contiguous route for one batch.
 *
 * cu_seqlens_padded: device int32 [n_slots + 1], the padded boundaries.  The
 * route depends only on these boundaries and cp_size (Relax PR #273, §1 and
 * §2.1), so one build serves every layer, both directions and the recompute
 * replay of a micro-batch; rebuild it for the next micro-batch.
 *
 * The build validates the boundaries (codes THD_ERR_CU_START ..
 * THD_ERR_CU_DIVISIBLE, in that precedence), drops empty slots, lays out the
 * 2*cp zigzag segments of every document, cuts them at the contiguous ranks'
 * borders and writes the maximal runs (in zigzag-row order and in token
 * order) plus the cp x cp split matrix, then a row directory: for every 16th
 * output row of each direction, the input row feeding it, the end of its run,
 * the run's index and which of the 16 rows start a run.  Launches, by the
 * route's size (segments = 2*cp*n_slots): above 1024 segments with cp <= 64
 * and the documents in LDS, one launch of ceil(segments / own) + 1
 * workgroups (own = 128 segments each, more when that would take over 255
 * workgroups) that place every segment's runs at slots given in closed form,
 * each also writing the directory entries whose rows start in its segments
 * from a copy of their runs in LDS (while the entries of one direction
 * average at most 2048 per workgroup; past that the directory takes a
 * second, grid-wide launch);
 * otherwise, up to 16384 segments when the route fits in
 * 150 KiB of LDS, one launch of ceil(total_tokens / 16384) workgroups, at
 * most 512, each building the route in its own LDS and writing an equal share
 * of the directory; larger routes take one single-workgroup build launch (in
 * LDS, or in the route's workspace when LDS is too small) and the directory
 * launch.  Results and the status word stay on the device.
 *
 * cp_size == 1: the route is the identity; nothing is launched and the
 * boundaries are not read (the swap short-circuits for one rank before any
 * validation, Relax PR #273 §2.6).  cp_size above the route's max_cp, n_slots
 * above max_slots or total_tokens above max_tokens: THD_ERR_CAPACITY.
 * Rebuilding while swaps that use the route are still queued on another
 * stream is a race the caller must avoid.
 */
int thd_build_route(thd_route* route, const int32_t* cu_seqlens_padded, int32_t n_slots,
                    int32_t cp_size, int64_t total_tokens, void* stream);

/*
 * thd_swap -- apply the route to `rows` rows of `row_bytes` bytes each.
 *
 * THD_ZIGZAG_TO_CONTIGUOUS: `in` is the emulated zigzag buffer, `out` receives
 * the emulated contiguous buffer (token order); THD_CONTIGUOUS_TO_ZIGZAG is
 * the inverse.  Both buffers are row-major [rows, row_bytes] with the token
 * dimension outermost (Relax PR #273 §2.6 moves it there first).  Rows are
 * copied bit for bit; no arithmetic is done on them.  `in` and `out` must not
 * overlap (THD_ERR_ALIAS): an in-place permutation is not supported.
 * `rows` must equal the route's total_tokens (THD_ERR_SHAPE); any
 * row_bytes >= 1 works, 16-byte multiples with 16-byte aligned pointers take
 * the widest path.
 *
 * Returns THD_IDENTITY without launching when the route is the identity
 * (cp_size == 1 or total_tokens == 0): the caller keeps `in` (zero copy, as
 * the pages' identity route does).  If the route's device status is an error,
 * the kernel writes nothing.  One kernel launch otherwise.
 *
 * The work is a bandwidth-bound copy of 2 * rows * row_bytes bytes.  Row
 * sizes that are powers of two or multiples of 128 bytes, with 16-byte
 * aligned buffers, run within 1-3 % of the fastest plain copy of the same
 * bytes (thd_copy); other row sizes or alignments are moved in narrower
 * units, 2-6 % below it.
 */
int thd_swap(const thd_route* route, int32_t direction, const void* in, void* out,
             int64_t rows, int64_t row_bytes, void* stream);

/*
 * thd_swap_batch -- thd_swap for n_tensors tensors (1..THD_MAX_BATCH) in one
 * kernel launch: the tokens, labels, loss mask, position ids and valid mask
 * of a packed batch all take the same route ("Packed Sequence 与上下文并行"
 * §2.4 slices every per-token stream with one index), as do the several
 * activations of one layer.
 *
 * ins, outs, row_bytes: host arrays of n_tensors entries; ins[i] and outs[i]
 * are device buffers of rows x row_bytes[i] bytes, row-major, token dimension
 * outermost.  No output may overlap any input or any other output
 * (THD_ERR_ALIAS).  Other rules as thd_swap; THD_IDENTITY when the route is
 * the identity (nothing written, callers keep their inputs).
 */
int thd_swap_batch(const thd_route* route, int32_t direction, int32_t n_tensors, const void* const* ins,
                   void* const* outs, const int64_t* row_bytes, int64_t rows, void* stream);

/*
 * thd_roll_labels -- document-aware label shift, MTP roll and valid-token mask
 * in one pass ("Packed Sequence 与上下文并行" §1.3, §1.6, §2.2).
 *
 * ids:               device int64 [total_tokens], the packed token stream
 *                    in natural (contiguous) order.
 * cu_seqlens_padded: device int32 [n_slots + 1], padded boundaries (positions).
 * cu_seqlens:        device int32 [n_slots + 1], real (unpadded) boundaries;
 *                    NULL means no slot has pads.  The pads of a slot are the
 *                    tail of its padded range.
 * max_shift:         J in 1..THD_MAX_SHIFT.  Shift 1 is the next-token label,
 *                    shift k+1 the target of MTP depth k.
 * shifted:           device int64 [J][total_tokens] (output).
 * mask:              device uint8 [J + 1][total_tokens] (output).
 * status:            device int32 word or NULL; receives THD_OK or the first
 *                    failing rule: THD_ERR_CU_START, THD_ERR_CU_MONOTONE (either
 *                    list), THD_ERR_CU_TOTAL (padded list), then
 *                    THD_ERR_REAL_GT_PADDED.  On such an error nothing else is
 *                    written.
 *
 * For position t of slot s, with e = cu_seqlens_padded[s] + real length of s:
 * mask[0][t] = (t < e); for j = 1..J, when t + j < e, shifted[j-1][t] =
 * ids[t + j] and mask[j][t] = 1, else shifted[j-1][t] = fill and mask[j][t] =
 * 0.  No target ever comes from another document or from a pad.  Outputs must
 * not overlap each other or ids (THD_ERR_ALIAS).  One kernel launch.
 */
int thd_roll_labels(const int64_t* ids, const int32_t* cu_seqlens_padded, const int32_t* cu_seqlens,
                    int32_t n_slots, int64_t total_tokens, int32_t max_shift, int64_t fill,
                    int64_t* shifted, uint8_t* mask, int32_t* status, void* stream);

/*
 * thd_roll_labels_zigzag -- thd_roll_labels with its outputs written in the
 * emulated zigzag layout of `route`, i.e. the roll followed by the c->z slice
 * of every output stream, in one pass: row t of each natural-order stream
 * lands on the zigzag row that holds token t ("Packed Sequence 与上下文并行"
 * §2.2 rolls labels at pack time and §2.4 slices them with the tokens).
 *
 * The route must have been built from the same cu_seqlens_padded and
 * total_tokens (THD_ERR_SHAPE if total_tokens or n_slots differs from the
 * last build's, THD_ERR_NOT_BUILT if never built).  Identity route (cp_size
 * 1, or no tokens): same as thd_roll_labels.  If the route's status is an
 * error, that code is written to `status` and nothing else is written.
 * Other arguments, errors and outputs as thd_roll_labels.
 */
int thd_roll_labels_zigzag(const thd_route* route, const int64_t* ids, const int32_t* cu_seqlens_padded,
                           const int32_t* cu_seqlens, int32_t n_slots, int64_t total_tokens, int32_t max_shift,
                           int64_t fill, int64_t* shifted, uint8_t* mask, int32_t* status, void* stream);

/*
 * thd_pack_workspace_bytes -- device workspace thd_pack needs for a
 * [batch, seq] token matrix (host-only arithmetic; -1 for negative sizes or
 * seq > THD_PACK_MAX_SEQ).  About 40 bytes per 1024-token chunk of a row.
 */
int64_t thd_pack_workspace_bytes(int32_t batch, int32_t seq);

/*
 * thd_pack -- pack [batch, seq] token rows into one padded THD stream on the
 * device ("Packed Sequence 与上下文并行" §2.2 steps (1)-(3), worked example
 * §3.1-§3.4), with every output shape fixed by the arguments so that the route
 * build, the swaps and the roll can follow without the host reading anything.
 *
 * tokens:    device int64 [batch][seq], row-major.
 * Documents: in each row the valid part ends after the last token that is not
 *            pad_id; inside it every eod_id token closes a document (the EOD is
 *            its last token) and the tokens after the last EOD form one more
 *            document.  pad_id tokens before the valid end stay in their
 *            document.  Rows in order, documents left to right.
 * align:     each document is padded at its end to a multiple of align (the
 *            pages use TP*CP*2, or TP*CP*16 with FP8; a multiple of 2*cp_size
 *            is what the route needs).
 * capacity:  token budget of the packed stream, a multiple of align, at most
 *            INT32_MAX.  packed: device int64 [capacity]; positions holding no
 *            token get pad_value.
 * max_docs:  document slots.  cu_seqlens / cu_seqlens_padded: device int32
 *            [max_docs + 2] (real / padded boundaries, n_slots = max_docs + 1):
 *            slot k < n_docs is document k, slot n_docs is the trailing
 *            pad-only slot up to capacity (real length 0), later slots are
 *            empty (a repeated boundary).
 * workspace: device buffer of at least thd_pack_workspace_bytes(batch, seq).
 * status:    device int32 or NULL: THD_OK, THD_ERR_PACK_DOCS or
 *            THD_ERR_PACK_CAPACITY (THD_ERR_PACK_DOCS when both apply); on
 *            an error nothing but status is written.
 *
 * Host errors: THD_ERR_ARG (negative sizes, seq > THD_PACK_MAX_SEQ, align < 1,
 * capacity not a multiple of align, pad_id == eod_id, null pointers,
 * workspace too small),
 * THD_ERR_ALIAS (outputs overlapping each other, the tokens or the workspace).
 * Stream-ordered kernel launches: two for batches of up to 256 chunks of
 * 1024 tokens (a chunk pass, then a write pass whose every workgroup runs
 * the scan over all chunks itself), three beyond (a one-workgroup scan
 * launch between them).
 */
int thd_pack(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id, int32_t align,
             int64_t capacity, int32_t max_docs, int64_t pad_value, void* workspace, int64_t workspace_bytes,
             int64_t* packed, int32_t* cu_seqlens, int32_t* cu_seqlens_padded, int32_t* status, void* stream);

/*
 * thd_pack_noalloc -- thd_pack for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, outputs and
 * errors as thd_pack, minus the workspace: the pack runs in a device scratch
 * array of THD_PACK_STATIC_BYTES inside the library, one per GPU, held until
 * the process ends.  It allocates nothing and frees nothing.
 *
 * Size limit: batches whose thd_pack_workspace_bytes(batch, seq) exceeds
 * THD_PACK_STATIC_BYTES (about 23,700 chunks of 1024 tokens, i.e. about 24
 * million tokens in [batch, seq]) return THD_ERR_CAPACITY before any device
 * work.  The first call on a device looks up that device's scratch address
 * (hipGetSymbolAddress, host only); make one call before capturing a graph
 * if the capture mode forbids runtime calls.  THD_ERR_HIP if the lookup
 * fails.
 *
 * Every call on one GPU shares that GPU's scratch: calls whose work
 * overlaps on one GPU (on different streams, or from different threads,
 * with no ordering between them) race and may produce wrong outputs.
 * Calls ordered on one stream are safe.  Nothing in the scratch has to
 * start at zero.  Stream-ordered, the same launches as thd_pack.
 */
int thd_pack_noalloc(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id,
                     int32_t align, int64_t capacity, int32_t max_docs, int64_t pad_value, int64_t* packed,
                     int32_t* cu_seqlens, int32_t* cu_seqlens_padded, int32_t* status, void* stream);

/*
 * thd_route_status -- SYNC.  Waits for `stream`, then stores the status word
 * written by the last build into *host_status (host): THD_OK or one of
 * THD_ERR_CU_* / THD_ERR_INTEGRITY.  For an identity route it stores THD_OK
 * without touching the device.  Opt-in: the hot path never calls it.
 */
int thd_route_status(const thd_route* route, void* stream, int32_t* host_status);

/*
 * thd_route_copy_out -- SYNC.  Waits for `stream`, then copies the route to
 * host memory for inspection: *host_n_runs = number of runs; if the pointers
 * are non-NULL and `capacity` >= that number, host_runs_by_src and
 * host_runs_by_dst (host int32 [capacity][3]) receive the runs as
 * (zigzag row, contiguous row, length) triples in emulated global rows, sorted
 * by zigzag row and by contiguous row respectively, and host_split (host
 * int32 [cp][cp]) the split matrix: split[s][d] rows go from zigzag rank s to
 * contiguous rank d.  An identity route, or one whose status is an error,
 * reports 0 runs.  THD_ERR_CAPACITY if `capacity` is too small (only
 * *host_n_runs is written then); THD_ERR_INTEGRITY if the device reports more
 * runs than the route can hold (nothing is written).
 */
int thd_route_copy_out(const thd_route* route, void* stream, int32_t* host_n_runs, int32_t capacity,
                       int32_t* host_runs_by_src, int32_t* host_runs_by_dst, int32_t* host_split);

/*
 * thd_route_info -- host-only query of the last build's shape: cp_size,
 * total_tokens, n_slots and whether it was built (each pointer may be NULL).
 */
int thd_route_info(const thd_route* route, int32_t* cp_size, int64_t* total_tokens,
                   int32_t* n_slots, int32_t* built);

/*
 * thd_copy -- plain streaming copy of `bytes` bytes from `in` to `out`
 * (device pointers, non-overlapping): no route, no permutation.  It moves
 * the bytes in 4 KiB tiles with the same units and non-temporal loads as
 * thd_swap, in the form that streams a plain copy fastest on MI355X (16-byte
 * units: 256 threads per tile, one word per lane, XCD-chunked order with
 * chunks of 256 tiles, and tiles of whole 128-byte lines stored with the
 * write-through cache policy), so a swap's bandwidth can be set beside that
 * of a copy of the same bytes in the same run: the ceiling a row permutation
 * is measured against.
 * Stream-ordered, one launch; THD_ERR_ARG for a negative size or a null
 * pointer (bytes > 0), THD_ERR_ALIAS for overlapping buffers; 0 bytes is
 * THD_OK with no launch.
 */
int thd_copy(const void* in, void* out, int64_t bytes, void* stream);

/* thd_strerror -- static text for a return or status code. */
const char* thd_strerror(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* THD_CP_H */

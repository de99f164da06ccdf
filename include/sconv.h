/*
 * sconv.h -- C ABI of libsconv: paged depthwise causal short convolution
 * for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns an int status: SCONV_OK (0) or one of the
 *   SCONV_ERR_* codes below.  On error, sconv_last_error() returns a
 *   thread-local message; nothing is launched.
 * - Every buffer is a caller-owned DEVICE pointer (hipMalloc / torch).  The
 *   library allocates nothing, never synchronizes and never reads device data
 *   on the host: each call enqueues one kernel on `stream` (NULL = the null
 *   stream; sconv_fused_insert_conv_gather may enqueue two) and returns.
 *   This makes every call capturable in a hipGraph; grids depend on host
 *   scalars only.
 * - Strides are in ELEMENTS.  Only host scalars are validated.  Properties of
 *   device data (index ranges, monotone offsets, distinct slots) are the
 *   caller's contract and are stated per function; breaking them is
 *   undefined behaviour.
 * - Floating tensors of one call share one element type (sconv_dtype_t):
 *   x, weight, bias, cache / state pool and out.  Arithmetic is fp32.
 * - SCONV_ERR_HIP reports a launch error taken from hipGetLastError().
 */
#ifndef SCONV_H
#define SCONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque HIP stream handle (identical to the one in hip_runtime_api.h). */
typedef struct ihipStream_t* hipStream_t;

enum {
  SCONV_OK = 0,
  SCONV_ERR_INVALID = 1,     /* bad host scalar, shape, stride or pointer */
  SCONV_ERR_UNSUPPORTED = 2, /* valid request the library does not cover */
  SCONV_ERR_HIP = 3          /* the HIP runtime reported a launch error   */
};

typedef enum { SCONV_F32 = 0, SCONV_BF16 = 1 } sconv_dtype_t;
typedef enum { SCONV_ACT_NONE = 0, SCONV_ACT_SILU = 1 } sconv_act_t;

/* Message describing the last failed call on this thread ("" if none). */
const char* sconv_last_error(void);

/* Library version string. */
const char* sconv_version(void);

/*
 * Load the library's GPU code on the current device without launching
 * anything.  Every entry point otherwise loads it at its first launch; a
 * caller whose first call is captured into a hipGraph calls sconv_init
 * first, so that the capture records launches only.  Idempotent.
 * SCONV_ERR_HIP if the runtime cannot load the code (no gfx950 device).
 */
int sconv_init(void);

/*
 * sconv_seq_metadata -- per-token request index and request start row.
 *
 * Source: vLLM page "vllm.models.inkling.nvidia.ops.sconv", function
 * sconv_seq_metadata (docstring and wrapper source): one launch replaces the
 * search-and-gather chain that builds the static per-token buffers.
 *
 * For rows t < num_actual_tokens:
 *     seq_idx_out[t]     = the request r whose rows [qsl[r], qsl[r+1]) hold t
 *                          (empty requests never match; rows at or beyond
 *                          qsl[num_reqs] get num_reqs - 1)
 *     query_start_out[t] = qsl[r]
 * For rows num_actual_tokens <= t < num_padded_tokens both are 0 (such rows
 * must carry slot_mapping == -1 in sconv_fused_insert_conv).
 *
 *   query_start_loc  int32 [num_reqs + 1], non-decreasing, qsl[0] == 0 (device)
 *   seq_idx_out      int32 [seq_idx_len]     (device, written)
 *   query_start_out  int32 [query_start_len] (device, written)
 *
 * Errors (SCONV_ERR_INVALID): num_padded_tokens < num_actual_tokens, either
 * output shorter than num_padded_tokens, num_actual_tokens < 0, or
 * num_reqs < 1 while num_actual_tokens > 0.  num_padded_tokens == 0 is a
 * successful no-op.
 */
int sconv_seq_metadata(const int32_t* query_start_loc, int32_t num_reqs,
                       int64_t num_actual_tokens, int64_t num_padded_tokens,
                       int32_t* seq_idx_out, int64_t seq_idx_len,
                       int32_t* query_start_out, int64_t query_start_len,
                       hipStream_t stream);

/*
 * sconv_fused_insert_conv -- single-launch insert + depthwise causal conv
 * over a paged cache, for one conv stream.
 *
 * Source: vLLM page "vllm.models.inkling.nvidia.ops.sconv", module
 * description and function fused_sconv (signature, docstring, wrapper
 * source).
 *
 * Layout:
 *   x          [T, C] row stride x_row_stride, channels contiguous,
 *              C = H * ws, channel c = h*ws + j (head-major)
 *   weight     [C, W] strides (w_stride_c, w_stride_k); 1 <= W <= 4
 *   cache      [num_blocks, H, N, D] strides (cs0, cs1, cs2, 1); this stream
 *              owns columns [off_s, off_s + ws) of every head
 *   positions  int64 [T]  absolute position of each row
 *   block_table int32 [num_reqs, max_blocks] row stride bt_row_stride
 *   seq_idx    int32 [T]  request of each row     (sconv_seq_metadata)
 *   slot_mapping int64 [T] flat cache slot, < 0 = PAD
 *   query_start int32 [T] first row of the row's request
 *   out        [T, C] row stride out_row_stride (written, same dtype as x)
 *
 * For each row t with slot_mapping[t] >= 0, channel c, tap k in [0, W):
 *   lag = W-1-k, src = positions[t] - lag, and the tap value is
 *     0                                   if src < 0,
 *     x[t - lag, c]                       if t - lag >= query_start[t],
 *     cache[bt[seq_idx[t], src / N], h, src % N, off_s + j]   otherwise;
 *   out[t, c] = act(sum_k weight[c, k] * tap_k) (+ x[t, c] if use_residual)
 *   and x[t, :] is copied bit for bit to cache[slot / N, h, slot % N,
 *   off_s + j].  PAD rows produce no output (out row untouched) and no
 *   write, but their input still serves as a tap for later rows of their
 *   request.
 *
 * Device-data contract: rows of a request are contiguous with consecutive
 * positions; every block-table entry that is read lies in [0, num_blocks);
 * non-PAD slots are distinct and none of them is read as a pre-forward tap
 * in the same call (the cache is read and written in one launch).
 *
 * Host errors (SCONV_ERR_INVALID): T < 0, H, N, ws < 1, off_s < 0,
 * off_s + ws > D, W outside [1, 4], strides smaller than the row they span,
 * unknown dtype or activation, NULL pointer with T > 0, out overlapping x or
 * cache.  T == 0 is a successful no-op.
 */
int sconv_fused_insert_conv(const void* x, int64_t x_row_stride,
                            const void* weight, int64_t w_stride_c, int64_t w_stride_k,
                            void* cache, int64_t num_blocks, int32_t H, int32_t N,
                            int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
                            const int64_t* positions, const int32_t* block_table,
                            int64_t bt_row_stride, int32_t max_blocks,
                            const int32_t* seq_idx, const int64_t* slot_mapping,
                            const int32_t* query_start, void* out,
                            int64_t out_row_stride, int64_t T, int32_t off_s,
                            int32_t ws, int32_t W, int32_t dtype, int32_t activation,
                            int32_t use_residual, hipStream_t stream);

/*
 * sconv_fused_insert_conv_qsl -- the same insert + conv, with the per-row
 * request search folded into the launch.
 *
 * Source: vLLM page "vllm.models.inkling.nvidia.ops.sconv", fused_sconv and
 * sconv_seq_metadata: it computes exactly what sconv_seq_metadata followed
 * by sconv_fused_insert_conv computes, in one launch.  Every argument is as
 * in sconv_fused_insert_conv except that seq_idx / query_start are replaced
 * by the request row offsets:
 *
 *   query_start_loc  int32 [num_reqs + 1], non-decreasing, qsl[0] == 0 (device)
 *
 * Each non-PAD row t belongs to the last request r with qsl[r] <= t (rows
 * past qsl[num_reqs] clamp to the last request), and query_start = qsl[r].
 * How the launch finds r (the result is the same either way):
 *   - When every request may hold the same k <= 8 rows (T <= num_reqs,
 *     k = 1; or T a multiple of num_reqs, k = T / num_reqs) and W > 1, row
 *     t first tries request g = t / k, kept when qsl[g] <= t < qsl[g+1].
 *     With k = 1 (decode) and one-row tiles, the rows that keep it take
 *     their block-table entries from row t of block_table, read in
 *     advance (its first min(max_blocks, 256) entries: every row
 *     [0, num_reqs) of block_table must be readable).
 *     A row that misses its guess searches the offsets in device memory.
 *   - Other launches read the offsets whole into registers up to 512
 *     requests, and above that search them in device memory once per row
 *     tile.
 * The launch allocates nothing.
 *
 * Errors: as sconv_fused_insert_conv, plus SCONV_ERR_INVALID for
 * num_reqs < 1 (or a NULL query_start_loc) with T > 0.
 */
int sconv_fused_insert_conv_qsl(const void* x, int64_t x_row_stride,
                                const void* weight, int64_t w_stride_c, int64_t w_stride_k,
                                void* cache, int64_t num_blocks, int32_t H, int32_t N,
                                int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
                                const int64_t* positions, const int32_t* block_table,
                                int64_t bt_row_stride, int32_t max_blocks,
                                const int32_t* query_start_loc, int32_t num_reqs,
                                const int64_t* slot_mapping, void* out,
                                int64_t out_row_stride, int64_t T, int32_t off_s,
                                int32_t ws, int32_t W, int32_t dtype, int32_t activation,
                                int32_t use_residual, hipStream_t stream);

/*
 * sconv_stream_t -- one conv stream of a layer, for
 * sconv_fused_insert_conv_streams.  Fields as the same-named arguments of
 * sconv_fused_insert_conv: x and out [T, H*ws] rows of their row strides,
 * weight [H*ws, W], and the stream's columns [off_s, off_s + ws) of every
 * head of the shared cache.  activation and use_residual are per stream.
 * All pointers are device pointers owned by the caller; the array itself is
 * host memory, read during the call only.
 */
typedef struct sconv_stream {
  const void* x;
  int64_t x_row_stride;
  const void* weight;
  int64_t w_stride_c, w_stride_k;
  void* out;
  int64_t out_row_stride;
  int32_t off_s, ws;
  int32_t activation, use_residual;
} sconv_stream_t;

/*
 * sconv_fused_insert_conv_streams -- the insert + conv of up to four conv
 * streams of one layer in a single launch.
 *
 * Source: vLLM page "vllm.models.inkling.nvidia.ops.sconv", module
 * description (a layer's four conv streams -- K, V, attention output, MLP
 * output -- share one paged cache, each in its own column sub-range of
 * every head) and fused_sconv.  The result is exactly that of calling
 * sconv_fused_insert_conv once per stream, in any order: streams touch
 * disjoint cache columns, and each reads only its own pre-forward taps.
 *
 *   streams      host array [num_streams], 1 <= num_streams <= 4; their
 *                column ranges must be pairwise disjoint
 *   per-row request: either seq_idx and query_start (as filled by
 *                sconv_seq_metadata; query_start_loc NULL), or
 *                query_start_loc [num_reqs + 1] searched inside the launch
 *                (seq_idx and query_start NULL), as in
 *                sconv_fused_insert_conv_qsl
 *   all other arguments as in sconv_fused_insert_conv, shared by the streams
 *
 * The 16-byte-lane kernels run when every stream meets their alignment
 * (else all streams take the one-channel kernels).
 *
 * Device-data contract: as sconv_fused_insert_conv, for every stream.
 *
 * Host errors (SCONV_ERR_INVALID): num_streams outside [1, 4], overlapping
 * column ranges, both or neither per-row request forms, any stream failing
 * the checks of sconv_fused_insert_conv, any stream's out overlapping the
 * cache or another stream's x or out.  T == 0 is a successful no-op.
 */
int sconv_fused_insert_conv_streams(const sconv_stream_t* streams, int32_t num_streams,
                                    void* cache, int64_t num_blocks, int32_t H, int32_t N,
                                    int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
                                    const int64_t* positions, const int32_t* block_table,
                                    int64_t bt_row_stride, int32_t max_blocks,
                                    const int32_t* seq_idx, const int32_t* query_start,
                                    const int32_t* query_start_loc, int32_t num_reqs,
                                    const int64_t* slot_mapping, int64_t T, int32_t W,
                                    int32_t dtype, hipStream_t stream);

/*
 * sconv_fused_plan_t / sconv_fused_plan -- the launch a fused call would
 * make, without making it.
 *
 * For callers that size, tune or check launches ahead of time (and for the
 * library's own host tests): sconv_fused_plan takes exactly the arguments of
 * sconv_fused_insert_conv_streams (without the stream), runs the same host
 * checks with the same error codes, and on success fills *plan with the
 * kernel configuration and grid that call would enqueue.  Nothing is
 * launched and no pointer is dereferenced, so stand-in addresses of the
 * right alignment suffice.  The single-stream entry points plan like one
 * stream of it (sconv_fused_insert_conv: seq_idx and query_start;
 * sconv_fused_insert_conv_qsl: query_start_loc).  T == 0 gives an all-zero
 * plan (nothing to launch).
 */
typedef struct sconv_fused_plan {
  int32_t lane_elems;        /* channels per lane: 16 bytes' worth, or 1 */
  int32_t rows_per_tile;     /* consecutive rows of one wave's tile */
  int32_t request_mode;      /* 0 per-row buffers, 1 offsets in registers,
                                2 device-memory search, 3 request guess */
  int32_t rows_per_request;  /* rows per request the guess assumes */
  int32_t bt_row_entries;    /* block-table entries of the guessed row read
                                ahead per wave (0: none); >= 1 whenever
                                request_mode == 3 and rows_per_tile == 1 */
  int32_t stream_x_loads;    /* input rows loaded as streaming reads */
  int32_t stream_hist_loads; /* history rows loaded as streaming reads */
  int32_t tile_major;        /* wave order: 0 slab-major, 1 tile-major */
  int32_t wg_threads;        /* workgroup size */
  int32_t gather_mode;       /* window gather: 0 none, 1 in the conv's launch,
                                2 its own launch right after the conv's */
  int64_t waves;             /* tiles x slabs */
  int64_t workgroups;        /* grid size (with the gather's, if in it) */
  int32_t early_inserts;     /* cache inserts issued behind the history loads
                                (one-stream decode launches that fit the chip
                                in one wave generation) */
} sconv_fused_plan_t;

/*
 * sconv_window_gather_t -- the arguments of gather_intermediate_conv_window
 * (same names, meaning, layout and contract; the element type is the
 * fused call's), for sconv_fused_insert_conv_gather and sconv_fused_plan.
 */
typedef struct sconv_window_gather {
  const void* src;                /* [seq_len, conv_dim] rows (batch 0) */
  int64_t seq_len;
  int32_t conv_dim;
  int64_t src_stride_s, src_stride_c;
  const int32_t* abs_positions;   /* int32 [max_count] */
  const int32_t* real_count;      /* int32 [1], read on the device */
  int32_t max_count;
  void* out;                      /* [max_count, conv_dim, d_conv] */
  int64_t out_slot_stride;
  int32_t d_conv;
} sconv_window_gather_t;

/* `gather` may be NULL (a plain fused call). */
int sconv_fused_plan(const sconv_stream_t* streams, int32_t num_streams, void* cache,
                     int64_t num_blocks, int32_t H, int32_t N, int32_t D, int64_t cs0,
                     int64_t cs1, int64_t cs2, const int64_t* positions,
                     const int32_t* block_table, int64_t bt_row_stride, int32_t max_blocks,
                     const int32_t* seq_idx, const int32_t* query_start,
                     const int32_t* query_start_loc, int32_t num_reqs,
                     const int64_t* slot_mapping, int64_t T, int32_t W, int32_t dtype,
                     const sconv_window_gather_t* gather, sconv_fused_plan_t* plan);

/*
 * sconv_fused_insert_conv_gather -- a speculative-decode step in one launch:
 * the insert + conv of sconv_fused_insert_conv_streams and the conditional
 * window gather of gather_intermediate_conv_window.
 *
 * Sources: vLLM page "vllm.models.inkling.nvidia.ops.sconv", fused_sconv;
 * Megatron-core page "core.ssm.ops.intermediate_extraction",
 * scatter_intermediate_conv (parameters) and its kernel.  The results are
 * exactly those of the two calls in turn: the gather reads only its source
 * rows (usually the conv's x), which the conv never writes.
 *
 * The conv's workgroups come first in the grid and the gather's after them
 * (one per live-or-dead slot and channel block, the count read on the
 * device as in gather_intermediate_conv_window), so gather workgroups run
 * in the room the conv's resident waves leave.  Configurations without a
 * combined kernel (see sconv_fused_plan_t.gather_mode) launch the gather
 * right after the conv on the same stream, with the same results.
 *
 *   streams ... dtype   as sconv_fused_insert_conv_streams
 *   gather              as gather_intermediate_conv_window (host struct,
 *                       read during the call); max_count == 0 or
 *                       conv_dim == 0: no gather
 *
 * Host errors (SCONV_ERR_INVALID / _UNSUPPORTED): those of both calls; the
 * gather's out overlapping its source, the cache, any stream's x, weight
 * or out, or the conv's per-row metadata (positions, slot_mapping,
 * seq_idx, query_start, query_start_loc); the gather's source overlapping
 * the cache or any stream's out.  (The block table is not checked: its
 * row count is known only to the caller.)
 */
int sconv_fused_insert_conv_gather(const sconv_stream_t* streams, int32_t num_streams,
                                   void* cache, int64_t num_blocks, int32_t H, int32_t N,
                                   int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
                                   const int64_t* positions, const int32_t* block_table,
                                   int64_t bt_row_stride, int32_t max_blocks,
                                   const int32_t* seq_idx, const int32_t* query_start,
                                   const int32_t* query_start_loc, int32_t num_reqs,
                                   const int64_t* slot_mapping, int64_t T, int32_t W,
                                   int32_t dtype, const sconv_window_gather_t* gather,
                                   hipStream_t stream);

/*
 * causal_conv1d_varlen_fwd -- causal depthwise conv over packed
 * variable-length sequences, with a slot-indexed state pool.
 *
 * Source: leeroopedia page "Implementation:Sgl project Sglang Mamba Ops",
 * causal_conv1d_fwd (Signature, I/O Contract, Usage Examples).
 *
 *   x        [dim, total_T] strides (x_stride_c, x_stride_t) (device)
 *   weight   [dim, W] strides (w_stride_c, w_stride_k); bias [dim] or NULL
 *   conv_states [num_slots, dim, W-1] strides (st_stride_slot, st_stride_c,
 *            st_stride_k), oldest input first (read and written)
 *   query_start_loc int32 [batch+1] sequence b = tokens [qsl[b], qsl[b+1])
 *   cache_indices   int32 [batch] state slot of each sequence (NULL: b);
 *            a sequence whose slot equals pad_slot_id is skipped entirely
 *   has_initial_state uint8 [batch] (NULL: all 0); 0 = history is zeros and
 *            the slot is not read
 *   out      [dim, total_T] strides (out_stride_c, out_stride_t); may be x
 *            itself (in-place), otherwise must not overlap it
 *
 * For each non-PAD sequence, with u the state (oldest first) followed by the
 * sequence's inputs:  out[c, t] = act(bias[c] + sum_k weight[c, k] *
 * u[t - (W-1) + k]), and the slot receives the last W-1 entries of u (a bit
 * copy).
 *
 * Device-data contract: offsets non-decreasing within [0, total_T]; non-PAD
 * slots distinct and in [0, num_slots).
 *
 * Host errors (SCONV_ERR_INVALID): batch, dim, total_T < 0, W outside
 * [1, 4], NULL required pointer, unknown dtype or activation, partial overlap
 * of out and x.  batch == 0 or dim == 0 is a successful no-op.
 */
int causal_conv1d_varlen_fwd(const void* x, int64_t x_stride_c, int64_t x_stride_t,
                             const void* weight, int64_t w_stride_c, int64_t w_stride_k,
                             const void* bias, void* conv_states, int64_t num_slots,
                             int64_t st_stride_slot, int64_t st_stride_c,
                             int64_t st_stride_k, const int32_t* query_start_loc,
                             int32_t batch, const int32_t* cache_indices,
                             const uint8_t* has_initial_state, void* out,
                             int64_t out_stride_c, int64_t out_stride_t, int32_t dim,
                             int64_t total_T, int32_t W, int32_t dtype,
                             int32_t activation, int32_t pad_slot_id, hipStream_t stream);

/*
 * causal_conv1d_update -- one decode step against the state pool.
 *
 * Source: leeroopedia page "Implementation:Sgl project Sglang Mamba Ops",
 * causal_conv1d_update (Signature, I/O Contract).
 *
 *   x        [batch, dim] row stride x_stride_b, channels contiguous
 *   conv_states as in causal_conv1d_varlen_fwd (read and written)
 *   cache_seqlens: NULL (shift state, below) or int32 [batch]: the state's
 *            W-1 columns are then a ring, exactly as in
 *            causal_conv1d_update_tokens with seqlen 1 and state_len W-1
 *            (ignored when W == 1, which keeps no state)
 *   conv_state_indices int32 [batch] (NULL: b); pad_slot_id skips a row
 *   out      [batch, dim] row stride out_stride_b; may be x itself
 *
 * window = state[slot, c, 0..W-2] followed by x[b, c];
 * out[b, c] = act(bias[c] + sum_k weight[c, k] * window[k]);
 * state[slot, c, :] = window[1..W-1]  (bit copies).
 *
 * Host errors (SCONV_ERR_INVALID): batch, dim < 0, W outside [1, 4], NULL
 * required pointer, unknown dtype or activation, partial overlap of out and x.
 */
int causal_conv1d_update(const void* x, int64_t x_stride_b, void* conv_states,
                         int64_t num_slots, int64_t st_stride_slot, int64_t st_stride_c,
                         int64_t st_stride_k, const void* weight, int64_t w_stride_c,
                         int64_t w_stride_k, const void* bias,
                         const int32_t* cache_seqlens, const int32_t* conv_state_indices,
                         void* out, int64_t out_stride_b, int32_t batch, int32_t dim,
                         int32_t W, int32_t dtype, int32_t activation,
                         int32_t pad_slot_id, hipStream_t stream);

/*
 * causal_conv1d_update_tokens -- seqlen new tokens per row against the state
 * pool, with a shift or a ring state.
 *
 * Source: sglang page "Implementation:Sgl project Sglang Mamba Ops",
 * causal_conv1d_update (Signature, I/O Contract), which lists cache_seqlens
 * without semantics; the ring reading below is this library's, chosen to
 * match the absolute-position taps of sconv_fused_insert_conv.
 *
 *   x        [batch, dim, seqlen] strides (x_stride_b, x_stride_c, x_stride_t)
 *   conv_states [num_slots, dim, state_len] strides (st_stride_slot,
 *            st_stride_c, st_stride_k); W-1 <= state_len <= 8 (read and written)
 *   cache_seqlens NULL, or int32 [batch] >= 0: position of x[b, :, 0]
 *   conv_state_indices int32 [batch] (NULL: b); pad_slot_id skips a row
 *   out      [batch, dim, seqlen] strides (out_stride_*); may be x itself
 *
 * Shift state (cache_seqlens NULL): the state holds the last state_len
 * inputs, oldest first.  Token i convolves the W entries ending at it in
 * state ++ x[b, c, :]; afterwards the state holds the last state_len
 * entries of state ++ x[b, c, :].
 * Ring state: the input at position p lives in column p % state_len.  Token
 * i at position q = cache_seqlens[b] + i reads lag l from x if q - l >=
 * cache_seqlens[b], from the ring if 0 <= q - l < cache_seqlens[b], and
 * zero if q - l < 0; afterwards column (cache_seqlens[b] + i) % state_len
 * holds x[b, c, i].  cache_seqlens is read only.
 * In both: out[b, c, i] = act(bias[c] + sum_k weight[c, k] * tap_k).
 *
 * Device-data contract: state slots of non-PAD rows are distinct and in
 * [0, num_slots).
 *
 * Host errors (SCONV_ERR_INVALID): batch, dim or seqlen < 0, W outside
 * [1, 4], state_len < W-1 (or < 1 with a ring), NULL required pointer,
 * unknown dtype or activation, partial overlap of out and x.
 * SCONV_ERR_UNSUPPORTED: state_len above 8.
 */
int causal_conv1d_update_tokens(const void* x, int64_t x_stride_b, int64_t x_stride_c,
                                int64_t x_stride_t, int32_t seqlen, void* conv_states,
                                int64_t num_slots, int32_t state_len, int64_t st_stride_slot,
                                int64_t st_stride_c, int64_t st_stride_k, const void* weight,
                                int64_t w_stride_c, int64_t w_stride_k, const void* bias,
                                const int32_t* cache_seqlens, const int32_t* conv_state_indices,
                                void* out, int64_t out_stride_b, int64_t out_stride_c,
                                int64_t out_stride_t, int32_t batch, int32_t dim, int32_t W,
                                int32_t dtype, int32_t activation, int32_t pad_slot_id,
                                hipStream_t stream);

/*
 * gather_intermediate_conv_window -- conditional gather of the length-d_conv
 * input window before each slot's position, written transposed.
 *
 * Source: Megatron-core page "core.ssm.ops.intermediate_extraction", module
 * description, _scatter_intermediate_conv_kernel and scatter_intermediate_conv.
 *
 *   src            [seq_len, conv_dim] strides (src_stride_s, src_stride_c):
 *                  batch row 0 of the pre-conv input (device)
 *   abs_positions  int32 [max_count] window end of each slot (device)
 *   real_count_dev int32 [1] number of live slots, read ON THE DEVICE when
 *                  the kernel runs (clamped into [0, max_count]); the grid is
 *                  sized by max_count, so the call is graph-replay safe
 *   out            [max_count, conv_dim, d_conv], slot stride out_slot_stride,
 *                  dense inside a slot
 *
 * For slot i < n: out[i, c, k] = src[clamp(abs_positions[i] - d_conv + k,
 * 0, seq_len - 1), c]  (bit copies).  Slots i >= n are not written.
 *
 * Host errors (SCONV_ERR_INVALID): seq_len < 1, conv_dim < 0, max_count < 0,
 * NULL pointer, unknown dtype.  SCONV_ERR_UNSUPPORTED: d_conv outside [1, 4],
 * max_count above 65535 (each slot is one row of the launch grid).
 */
int gather_intermediate_conv_window(const void* src, int64_t seq_len, int32_t conv_dim,
                                    int64_t src_stride_s, int64_t src_stride_c,
                                    const int32_t* abs_positions,
                                    const int32_t* real_count_dev, int32_t max_count,
                                    void* out, int64_t out_slot_stride, int32_t d_conv,
                                    int32_t dtype, hipStream_t stream);

/*
 * gather_intermediate_ssm_state -- conditional gather of whole SSM-state
 * rows, with the live slot count read on the device.
 *
 * Source: Megatron-core page "core.ssm.ops.intermediate_extraction", module
 * description, _scatter_intermediate_ssm_kernel and scatter_intermediate_ssm.
 *
 *   states         [num_chunks, state_flat] row stride states_row_stride:
 *                  one layer's chunk-scan states, each flattened (device)
 *   chunk_indices  int64 [max_count] source row of each slot (device)
 *   real_count_dev int32 [1] number of live slots, read ON THE DEVICE when
 *                  the kernel runs (clamped into [0, max_count]); the grid is
 *                  sized by max_count, so the call is graph-replay safe
 *   out            [max_count, state_flat] row stride out_row_stride
 *
 * For slot i < n: out[i, :] = states[chunk_indices[i], :] (bit copies).
 * Slots i >= n are not written and cost no memory traffic.
 *
 * Device-data contract: chunk_indices[i] lies in [0, num_chunks) for every
 * live slot.
 *
 * Host errors (SCONV_ERR_INVALID): num_chunks < 1, state_flat < 0,
 * max_count < 0, a row stride smaller than state_flat, NULL pointer, unknown
 * dtype, out overlapping states.  SCONV_ERR_UNSUPPORTED: max_count above
 * 65535 (each slot is one row of the launch grid).  state_flat == 0 or
 * max_count == 0 is a successful no-op.
 */
int gather_intermediate_ssm_state(const void* states, int64_t num_chunks, int64_t state_flat,
                                  int64_t states_row_stride, const int64_t* chunk_indices,
                                  const int32_t* real_count_dev, int32_t max_count, void* out,
                                  int64_t out_row_stride, int32_t dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SCONV_H */

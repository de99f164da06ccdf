/*
 * sconv_oracle.h -- plain, slow CPU oracle for the paged depthwise causal
 * short convolution and its companion ops.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library
 * against a literal reading of the source pages.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or helper with
 * the GPU library.
 *
 * Arithmetic: every product and sum is formed in double precision, in the
 * tap order k = 0 .. W-1, and rounded once to the output type
 * (float: C cast, round-to-nearest-even; bfloat16: the helper
 * oracle_round_bf16 below, round-to-nearest-even).  Element type ORC_F64
 * keeps results unrounded so that identities can be checked exactly.
 *
 * Index arguments are element strides (not bytes).  Every function returns 0
 * on success and a negative code when an index it is asked to follow leaves
 * the buffer it was told about (the caller's input broke a precondition).
 */
#ifndef SCONV_ORACLE_H
#define SCONV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };
enum { ORC_ACT_NONE = 0, ORC_ACT_SILU = 1 };

enum {
  ORC_OK = 0,
  ORC_ERR_ARGS = -1,      /* nonsensical scalar argument            */
  ORC_ERR_REQ = -2,       /* seq_idx outside [0, num_reqs)          */
  ORC_ERR_BT_COL = -3,    /* logical block outside [0, max_blocks)  */
  ORC_ERR_BLOCK = -4,     /* physical block outside [0, num_blocks) */
  ORC_ERR_ROW = -5,       /* x row outside [0, T)                   */
  ORC_ERR_SLOT = -6,      /* state slot outside [0, num_slots)      */
  ORC_ERR_CHUNK = -7,     /* state row outside [0, num_chunks)      */
};

/* bfloat16 helpers (bit patterns held in uint16_t). */
double oracle_bf16_to_double(uint16_t bits);
uint16_t oracle_round_bf16(double v);
/* v * sigmoid(v), evaluated in double. */
double oracle_silu(double v);

/*
 * Per-token request index and request start row.  Page: vLLM
 * "vllm.models.inkling.nvidia.ops.sconv", function sconv_seq_metadata.
 * Rows t < num_actual get the request r whose row range
 * [qsl[r], qsl[r+1]) holds t (rows past qsl[num_reqs] clamp to the last
 * request), and query_start = qsl[r]; rows in [num_actual, num_padded) get 0.
 */
int oracle_seq_metadata(const int32_t* qsl, int32_t num_reqs, int64_t num_actual,
                        int64_t num_padded, int32_t* seq_idx_out,
                        int32_t* query_start_out);

/*
 * Insert + depthwise causal conv over the paged cache.  Page: vLLM
 * "vllm.models.inkling.nvidia.ops.sconv", module description and
 * function fused_sconv.
 *   x       [T, C]   row stride x_rs, unit channel stride, C = H*ws
 *   w       [C, W]   strides (w_sc, w_sk)
 *   cache_in / cache_out  [num_blocks, H, N, D] strides (cs0, cs1, cs2, 1);
 *           cache_in is the snapshot read for taps, cache_out receives the
 *           slot writes (the caller initialises it as a copy of cache_in).
 *   out     [T, C]   row stride out_rs; PAD rows (slot < 0) are not written.
 */
int oracle_fused_insert_conv(const void* x, int64_t x_rs, const void* w, int64_t w_sc,
                             int64_t w_sk, const void* cache_in, void* cache_out,
                             int64_t num_blocks, int32_t H, int32_t N, int32_t D,
                             int64_t cs0, int64_t cs1, int64_t cs2,
                             const int64_t* positions, const int32_t* block_table,
                             int64_t bt_rs, int32_t num_reqs, int32_t max_blocks,
                             const int32_t* seq_idx, const int64_t* slot_mapping,
                             const int32_t* query_start, void* out, int64_t out_rs,
                             int64_t T, int32_t off_s, int32_t ws, int32_t W,
                             int dtype, int act, int residual);

/*
 * Varlen causal conv1d over channel-major packed sequences with a
 * slot-indexed state pool.  Page: leeroopedia "Implementation:Sgl project
 * Sglang Mamba Ops", causal_conv1d_fwd (Signature, I/O Contract).
 *   x, out  [dim, total_T] strides (c, t)
 *   w       [dim, W]       strides (w_sc, w_sk);  bias [dim] or NULL
 *   st_in / st_out  [num_slots, dim, W-1] strides (slot, c, k): snapshot
 *           and destination of the state pool
 *   cache_indices[b] (NULL: b), has_init[b] (NULL: all false)
 */
int oracle_causal_conv1d_varlen_fwd(const void* x, int64_t x_sc, int64_t x_st,
                                    const void* w, int64_t w_sc, int64_t w_sk,
                                    const void* bias, const void* st_in, void* st_out,
                                    int64_t num_slots, int64_t ss_slot, int64_t ss_c,
                                    int64_t ss_k, const int32_t* qsl, int32_t batch,
                                    const int32_t* cache_indices,
                                    const uint8_t* has_init, void* out, int64_t o_sc,
                                    int64_t o_st, int32_t dim, int64_t total_T,
                                    int32_t W, int dtype, int act, int32_t pad_slot_id);

/*
 * One decode step of the causal conv against the state pool.  Page:
 * leeroopedia "Implementation:Sgl project Sglang Mamba Ops",
 * causal_conv1d_update.
 *   x, out  [batch, dim] row strides x_rs / out_rs, unit channel stride
 *   st_in / st_out as above; conv_state_indices[b] (NULL: b)
 */
int oracle_causal_conv1d_update(const void* x, int64_t x_rs, const void* st_in,
                                void* st_out, int64_t num_slots, int64_t ss_slot,
                                int64_t ss_c, int64_t ss_k, const void* w, int64_t w_sc,
                                int64_t w_sk, const void* bias,
                                const int32_t* conv_state_indices, void* out,
                                int64_t out_rs, int32_t batch, int32_t dim, int32_t W,
                                int dtype, int act, int32_t pad_slot_id);

/*
 * Multi-token state update, with an optional ring-buffer state.  Page:
 * sglang "Implementation:Sgl project Sglang Mamba Ops", Signature and I/O
 * Contract of causal_conv1d_update (cache_seqlens is listed there without
 * semantics; the reading below is ours).
 *   x     [batch, dim, seqlen] strides (x_sb, x_sc, x_st)
 *   state [num_slots, dim, state_len] strides (ss_slot, ss_c, ss_k),
 *         state_len >= W-1; st_out must start as a copy of st_in
 *   out   [batch, dim, seqlen] strides (out_sb, out_sc, out_st)
 * Without cache_seqlens the state is the last state_len inputs, oldest
 * first; token i convolves the W taps ending at it in state ++ x, and the
 * state becomes the last state_len entries of state ++ x.  With
 * cache_seqlens[b] = s (the position of x[b, :, 0]) the state is a ring:
 * the input at position p sits in column p % state_len; taps before
 * position 0 are zero, taps at positions >= s come from x, earlier ones
 * from the ring; afterwards column (s + i) % state_len holds x[b, :, i].
 */
int oracle_causal_conv1d_update_tokens(
    const void* x, int64_t x_sb, int64_t x_sc, int64_t x_st, int32_t seqlen, const void* st_in,
    void* st_out, int64_t num_slots, int32_t state_len, int64_t ss_slot, int64_t ss_c,
    int64_t ss_k, const void* w, int64_t w_sc, int64_t w_sk, const void* bias,
    const int32_t* cache_seqlens, const int32_t* conv_state_indices, void* out, int64_t out_sb,
    int64_t out_sc, int64_t out_st, int32_t batch, int32_t dim, int32_t W, int dtype, int act,
    int32_t pad_slot_id);

/*
 * Conditional gather of the length-d_conv window ending before each slot's
 * position, written transposed.  Page: Megatron-core
 * "core.ssm.ops.intermediate_extraction", scatter_intermediate_conv and its
 * kernel description.
 *   src  [seq_len, conv_dim] strides (src_ss, src_sc)   (batch row 0)
 *   out  [max_count, conv_dim, d_conv], slot stride out_ss, dense inside
 *   real_count: host copy of the device count; slots >= it are untouched.
 */
int oracle_gather_conv_window(const void* src, int64_t seq_len, int32_t conv_dim,
                              int64_t src_ss, int64_t src_sc, const int32_t* abs_positions,
                              int32_t real_count, int32_t max_count, void* out,
                              int64_t out_ss, int32_t d_conv, int dtype);

/*
 * Conditional gather of whole SSM-state rows.  Page: Megatron-core
 * "core.ssm.ops.intermediate_extraction", scatter_intermediate_ssm and the
 * description of its kernel.
 *   states [num_chunks, state_flat] row stride states_rs
 *   chunk_indices int64 [max_count]: source row of each slot
 *   out    [max_count, state_flat] row stride out_rs
 *   real_count: host copy of the device count; slots >= it are untouched.
 */
int oracle_gather_ssm_state(const void* states, int64_t num_chunks, int64_t state_flat,
                            int64_t states_rs, const int64_t* chunk_indices,
                            int32_t real_count, int32_t max_count, void* out, int64_t out_rs,
                            int dtype);

/*
 * The fused op and the varlen op with their outer loop split over
 * `nthreads` host threads (1..256): rows for the fused op, channels for the
 * varlen op.  Same arguments, same results bit for bit; used to time the
 * oracle on every host core.
 */
int oracle_fused_insert_conv_mt(const void* x, int64_t x_rs, const void* w, int64_t w_sc,
                                int64_t w_sk, const void* cache_in, void* cache_out,
                                int64_t num_blocks, int32_t H, int32_t N, int32_t D,
                                int64_t cs0, int64_t cs1, int64_t cs2,
                                const int64_t* positions, const int32_t* block_table,
                                int64_t bt_rs, int32_t num_reqs, int32_t max_blocks,
                                const int32_t* seq_idx, const int64_t* slot_mapping,
                                const int32_t* query_start, void* out, int64_t out_rs,
                                int64_t T, int32_t off_s, int32_t ws, int32_t W,
                                int dtype, int act, int residual, int32_t nthreads);
int oracle_causal_conv1d_varlen_fwd_mt(const void* x, int64_t x_sc, int64_t x_st,
                                       const void* w, int64_t w_sc, int64_t w_sk,
                                       const void* bias, const void* st_in, void* st_out,
                                       int64_t num_slots, int64_t ss_slot, int64_t ss_c,
                                       int64_t ss_k, const int32_t* qsl, int32_t batch,
                                       const int32_t* cache_indices,
                                       const uint8_t* has_init, void* out, int64_t o_sc,
                                       int64_t o_st, int32_t dim, int64_t total_T,
                                       int32_t W, int dtype, int act, int32_t pad_slot_id,
                                       int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif

/*
 * sconv_oracle.c -- plain, slow CPU oracle (see sconv_oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.
 *
 * Each function is the definition written out as nested loops in the order
 * the pages describe the computation: no blocking, no fusion, no reordering.
 * Readings of points the pages leave open are marked "Reading:".
 */
#include "sconv_oracle.h"

#include <math.h>
#include <pthread.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element access.                                                     */
/* ------------------------------------------------------------------ */

double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16; /* bfloat16 is the top half of a float */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bfloat16 (8 significant bits, float's
 * exponent range), ties to even, with gradual underflow and overflow to
 * infinity.  Works on the value, not on float bits, so there is exactly one
 * rounding step between the double result and the stored bfloat16. */
uint16_t oracle_round_bf16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(v);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);              /* 2^(e-1) <= a < 2^e */
  int E = e - 1;             /* unbiased exponent */
  if (E < -126) E = -126;    /* subnormal range: fixed quantum */
  double q = ldexp(1.0, E - 7);          /* spacing of bfloat16 values here */
  double r = nearbyint(a / q) * q;       /* default mode: ties to even */
  const double max_bf16 = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
  if (r > max_bf16) return (uint16_t)(sign | 0x7F80u);
  float f = (float)r;        /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

static size_t elem_size(int dtype) {
  return dtype == ORC_F32 ? 4 : dtype == ORC_BF16 ? 2 : 8;
}

static double ld(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)p)[i];
  if (dtype == ORC_BF16) return oracle_bf16_to_double(((const uint16_t*)p)[i]);
  return ((const double*)p)[i];
}

static void st(void* p, int dtype, int64_t i, double v) {
  if (dtype == ORC_F32)
    ((float*)p)[i] = (float)v; /* C conversion: round to nearest even */
  else if (dtype == ORC_BF16)
    ((uint16_t*)p)[i] = oracle_round_bf16(v);
  else
    ((double*)p)[i] = v;
}

/* Bit-for-bit copy of one element (cache and state writes are copies). */
static void copy_elem(void* dst, int64_t di, const void* src, int64_t si, int dtype) {
  size_t es = elem_size(dtype);
  memcpy((char*)dst + (size_t)di * es, (const char*)src + (size_t)si * es, es);
}

static void store_zero(void* dst, int64_t di, int dtype) {
  size_t es = elem_size(dtype);
  memset((char*)dst + (size_t)di * es, 0, es);
}

static int valid_dtype(int dtype) {
  return dtype == ORC_F32 || dtype == ORC_BF16 || dtype == ORC_F64;
}

static double activate(double v, int act) {
  return act == ORC_ACT_SILU ? oracle_silu(v) : v;
}

/* ------------------------------------------------------------------ */
/* sconv_seq_metadata                                                  */
/* ------------------------------------------------------------------ */

int oracle_seq_metadata(const int32_t* qsl, int32_t num_reqs, int64_t num_actual,
                        int64_t num_padded, int32_t* seq_idx_out,
                        int32_t* query_start_out) {
  if (num_actual < 0 || num_padded < num_actual) return ORC_ERR_ARGS;
  if (num_actual > 0 && num_reqs < 1) return ORC_ERR_ARGS;
  for (int64_t t = 0; t < num_actual; ++t) {
    /* The request whose row range [qsl[r], qsl[r+1]) contains row t.
     * An empty request has an empty range and never matches. */
    int32_t r = -1;
    for (int32_t rr = 0; rr < num_reqs; ++rr) {
      if ((int64_t)qsl[rr] <= t && t < (int64_t)qsl[rr + 1]) {
        r = rr;
        break;
      }
    }
    /* Reading: a row past the last request's end is clamped to the last
     * request, as a sorted search followed by a clamp would do; a row before
     * qsl[0] (never the case when qsl[0] == 0) goes to request 0. */
    if (r < 0) r = (t >= (int64_t)qsl[num_reqs]) ? num_reqs - 1 : 0;
    seq_idx_out[t] = r;
    query_start_out[t] = qsl[r];
  }
  for (int64_t t = num_actual; t < num_padded; ++t) {
    seq_idx_out[t] = 0;      /* padded rows are zero-filled */
    query_start_out[t] = 0;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* fused insert + depthwise causal conv over the paged cache           */
/* ------------------------------------------------------------------ */

/* Rows [t_begin, t_end) of oracle_fused_insert_conv (arguments checked by
 * the caller).  Each row reads only x, the snapshot cache_in and its own
 * metadata, and writes only its own out row and its own slot, so disjoint
 * row ranges are independent. */
static int fused_rows(const void* x, int64_t x_rs, const void* w, int64_t w_sc,
                      int64_t w_sk, const void* cache_in, void* cache_out,
                      int64_t num_blocks, int32_t H, int32_t N, int32_t D,
                      int64_t cs0, int64_t cs1, int64_t cs2,
                      const int64_t* positions, const int32_t* block_table,
                      int64_t bt_rs, int32_t num_reqs, int32_t max_blocks,
                      const int32_t* seq_idx, const int64_t* slot_mapping,
                      const int32_t* query_start, void* out, int64_t out_rs,
                      int64_t T, int32_t off_s, int32_t ws, int32_t W,
                      int dtype, int act, int residual, int64_t t_begin, int64_t t_end) {
  (void)D;
  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t slot = slot_mapping[t];
    /* Reading: a negative slot is PAD -- no cache write and no output. */
    if (slot < 0) continue;
    const int64_t pos = positions[t];
    const int32_t r = seq_idx[t];
    const int64_t q = query_start[t];
    if (r < 0 || r >= num_reqs) return ORC_ERR_REQ;

    for (int32_t h = 0; h < H; ++h) {
      for (int32_t j = 0; j < ws; ++j) {
        const int64_t c = (int64_t)h * ws + j; /* head-major channel */
        double acc = 0.0;
        /* Reading: weight column k multiplies the input at position
         * pos - (W-1) + k, so the last column meets the current token. */
        for (int32_t k = 0; k < W; ++k) {
          const int64_t lag = W - 1 - k;
          const int64_t src = pos - lag;
          double v;
          if (src < 0) {
            v = 0.0; /* Reading: taps before position 0 are zero. */
          } else if (t - lag >= q) {
            /* Tap inside this forward: the input row lag rows earlier. */
            const int64_t row = t - lag;
            if (row < 0 || row >= T) return ORC_ERR_ROW;
            v = ld(x, dtype, row * x_rs + c);
          } else {
            /* Tap from before this forward: the paged cache snapshot. */
            const int64_t lblk = src / N;
            if (lblk >= max_blocks) return ORC_ERR_BT_COL;
            const int64_t pblk = block_table[(int64_t)r * bt_rs + lblk];
            if (pblk < 0 || pblk >= num_blocks) return ORC_ERR_BLOCK;
            v = ld(cache_in, dtype,
                   pblk * cs0 + (int64_t)h * cs1 + (src % N) * cs2 + off_s + j);
          }
          acc += ld(w, dtype, c * w_sc + (int64_t)k * w_sk) * v;
        }
        double y = activate(acc, act);
        /* Reading: the residual is the raw input, added after the
         * activation. */
        if (residual) y += ld(x, dtype, t * x_rs + c);
        st(out, dtype, t * out_rs + c, y);
      }
    }

    /* Insert: this token's input goes to its flat slot, stream sub-range
     * [off_s, off_s + ws) of every head. */
    const int64_t blk = slot / N;
    const int64_t off = slot % N;
    if (blk >= num_blocks) return ORC_ERR_BLOCK;
    for (int32_t h = 0; h < H; ++h)
      for (int32_t j = 0; j < ws; ++j)
        copy_elem(cache_out, blk * cs0 + (int64_t)h * cs1 + off * cs2 + off_s + j, x,
                  t * x_rs + (int64_t)h * ws + j, dtype);
  }
  return ORC_OK;
}

int oracle_fused_insert_conv(const void* x, int64_t x_rs, const void* w, int64_t w_sc,
                             int64_t w_sk, const void* cache_in, void* cache_out,
                             int64_t num_blocks, int32_t H, int32_t N, int32_t D,
                             int64_t cs0, int64_t cs1, int64_t cs2,
                             const int64_t* positions, const int32_t* block_table,
                             int64_t bt_rs, int32_t num_reqs, int32_t max_blocks,
                             const int32_t* seq_idx, const int64_t* slot_mapping,
                             const int32_t* query_start, void* out, int64_t out_rs,
                             int64_t T, int32_t off_s, int32_t ws, int32_t W,
                             int dtype, int act, int residual) {
  if (!valid_dtype(dtype) || T < 0 || H < 1 || N < 1 || ws < 1 || W < 1 ||
      off_s < 0 || off_s + ws > D)
    return ORC_ERR_ARGS;
  return fused_rows(x, x_rs, w, w_sc, w_sk, cache_in, cache_out, num_blocks, H, N, D, cs0, cs1,
                    cs2, positions, block_table, bt_rs, num_reqs, max_blocks, seq_idx,
                    slot_mapping, query_start, out, out_rs, T, off_s, ws, W, dtype, act,
                    residual, 0, T);
}

/* ------------------------------------------------------------------ */
/* varlen causal conv1d with a state pool                              */
/* ------------------------------------------------------------------ */

/* Channels [c_begin, c_end) of oracle_causal_conv1d_varlen_fwd, for every
 * sequence (arguments checked by the caller).  A (sequence, channel) pair
 * reads only its own inputs and state row and writes only its own outputs
 * and state row, so disjoint channel ranges are independent. */
static int varlen_channels(const void* x, int64_t x_sc, int64_t x_st,
                           const void* w, int64_t w_sc, int64_t w_sk,
                           const void* bias, const void* st_in, void* st_out,
                           int64_t num_slots, int64_t ss_slot, int64_t ss_c,
                           int64_t ss_k, const int32_t* qsl, int32_t batch,
                           const int32_t* cache_indices,
                           const uint8_t* has_init, void* out, int64_t o_sc,
                           int64_t o_st, int64_t total_T,
                           int32_t W, int dtype, int act, int32_t pad_slot_id,
                           int32_t c_begin, int32_t c_end) {
  const int32_t S = W - 1; /* state length */

  for (int32_t b = 0; b < batch; ++b) {
    const int64_t slot = cache_indices ? cache_indices[b] : b;
    if (slot == pad_slot_id) continue; /* padded sequence: untouched */
    if (slot < 0 || slot >= num_slots) return ORC_ERR_SLOT;
    const int64_t start = qsl[b];
    const int64_t L = (int64_t)qsl[b + 1] - start;
    if (start < 0 || L < 0 || start + L > total_T) return ORC_ERR_ROW;
    /* Reading: without an initial state the history is zeros and the pool
     * slot is not read. */
    const int init = has_init ? (has_init[b] != 0) : 0;

    for (int32_t c = c_begin; c < c_end; ++c) {
      /* Logical input u(i): x for i >= 0, the initial state (oldest first)
       * for -S <= i < 0. */
#define U_VAL(i)                                                                  \
  ((i) >= 0 ? ld(x, dtype, (int64_t)c * x_sc + (start + (i)) * x_st)              \
            : (init ? ld(st_in, dtype, slot * ss_slot + (int64_t)c * ss_c +       \
                                           (int64_t)(S + (i)) * ss_k)             \
                    : 0.0))
      for (int64_t i = 0; i < L; ++i) {
        double acc = bias ? ld(bias, dtype, c) : 0.0;
        for (int32_t k = 0; k < W; ++k) {
          const int64_t ui = i - S + k;
          acc += ld(w, dtype, (int64_t)c * w_sc + (int64_t)k * w_sk) * U_VAL(ui);
        }
        st(out, dtype, (int64_t)c * o_sc + (start + i) * o_st, activate(acc, act));
      }
      /* Final state: the last S logical inputs, copied bit for bit. */
      for (int32_t m = 0; m < S; ++m) {
        const int64_t ui = L - S + m;
        const int64_t di = slot * ss_slot + (int64_t)c * ss_c + (int64_t)m * ss_k;
        if (ui >= 0)
          copy_elem(st_out, di, x, (int64_t)c * x_sc + (start + ui) * x_st, dtype);
        else if (init)
          copy_elem(st_out, di, st_in,
                    slot * ss_slot + (int64_t)c * ss_c + (int64_t)(S + ui) * ss_k, dtype);
        else
          store_zero(st_out, di, dtype);
      }
#undef U_VAL
    }
  }
  return ORC_OK;
}

int oracle_causal_conv1d_varlen_fwd(const void* x, int64_t x_sc, int64_t x_st,
                                    const void* w, int64_t w_sc, int64_t w_sk,
                                    const void* bias, const void* st_in, void* st_out,
                                    int64_t num_slots, int64_t ss_slot, int64_t ss_c,
                                    int64_t ss_k, const int32_t* qsl, int32_t batch,
                                    const int32_t* cache_indices,
                                    const uint8_t* has_init, void* out, int64_t o_sc,
                                    int64_t o_st, int32_t dim, int64_t total_T,
                                    int32_t W, int dtype, int act, int32_t pad_slot_id) {
  if (!valid_dtype(dtype) || batch < 0 || dim < 0 || W < 1 || total_T < 0)
    return ORC_ERR_ARGS;
  return varlen_channels(x, x_sc, x_st, w, w_sc, w_sk, bias, st_in, st_out, num_slots,
                         ss_slot, ss_c, ss_k, qsl, batch, cache_indices, has_init, out, o_sc,
                         o_st, total_T, W, dtype, act, pad_slot_id, 0, dim);
}

/* ------------------------------------------------------------------ */
/* single decode step against the state pool                           */
/* ------------------------------------------------------------------ */

int oracle_causal_conv1d_update(const void* x, int64_t x_rs, const void* st_in,
                                void* st_out, int64_t num_slots, int64_t ss_slot,
                                int64_t ss_c, int64_t ss_k, const void* w, int64_t w_sc,
                                int64_t w_sk, const void* bias,
                                const int32_t* conv_state_indices, void* out,
                                int64_t out_rs, int32_t batch, int32_t dim, int32_t W,
                                int dtype, int act, int32_t pad_slot_id) {
  if (!valid_dtype(dtype) || batch < 0 || dim < 0 || W < 1) return ORC_ERR_ARGS;
  const int32_t S = W - 1;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t slot = conv_state_indices ? conv_state_indices[b] : b;
    if (slot == pad_slot_id) continue;
    if (slot < 0 || slot >= num_slots) return ORC_ERR_SLOT;
    for (int32_t c = 0; c < dim; ++c) {
      /* Window: the stored state (oldest first) followed by the new input. */
      double acc = bias ? ld(bias, dtype, c) : 0.0;
      for (int32_t k = 0; k < W; ++k) {
        const double v =
            k < S ? ld(st_in, dtype, slot * ss_slot + (int64_t)c * ss_c + (int64_t)k * ss_k)
                  : ld(x, dtype, (int64_t)b * x_rs + c);
        acc += ld(w, dtype, (int64_t)c * w_sc + (int64_t)k * w_sk) * v;
      }
      st(out, dtype, (int64_t)b * out_rs + c, activate(acc, act));
      /* The state moves one step: window entries 1 .. W-1. */
      for (int32_t m = 0; m < S; ++m) {
        const int64_t di = slot * ss_slot + (int64_t)c * ss_c + (int64_t)m * ss_k;
        if (m + 1 < S)
          copy_elem(st_out, di, st_in,
                    slot * ss_slot + (int64_t)c * ss_c + (int64_t)(m + 1) * ss_k, dtype);
        else
          copy_elem(st_out, di, x, (int64_t)b * x_rs + c, dtype);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* multi-token update, shift or ring state                             */
/* ------------------------------------------------------------------ */

int oracle_causal_conv1d_update_tokens(
    const void* x, int64_t x_sb, int64_t x_sc, int64_t x_st, int32_t seqlen, const void* st_in,
    void* st_out, int64_t num_slots, int32_t state_len, int64_t ss_slot, int64_t ss_c,
    int64_t ss_k, const void* w, int64_t w_sc, int64_t w_sk, const void* bias,
    const int32_t* cache_seqlens, const int32_t* conv_state_indices, void* out, int64_t out_sb,
    int64_t out_sc, int64_t out_st, int32_t batch, int32_t dim, int32_t W, int dtype, int act,
    int32_t pad_slot_id) {
  if (!valid_dtype(dtype) || batch < 0 || dim < 0 || W < 1 || seqlen < 0 ||
      state_len < W - 1 || (cache_seqlens && state_len < 1))
    return ORC_ERR_ARGS;
  const int64_t L = state_len;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t slot = conv_state_indices ? conv_state_indices[b] : b;
    if (slot == pad_slot_id) continue;
    if (slot < 0 || slot >= num_slots) return ORC_ERR_SLOT;
    const int64_t s = cache_seqlens ? cache_seqlens[b] : 0;
    if (s < 0) return ORC_ERR_ARGS;
    for (int32_t c = 0; c < dim; ++c) {
      const int64_t sbase = slot * ss_slot + (int64_t)c * ss_c;
      const int64_t xbase = (int64_t)b * x_sb + (int64_t)c * x_sc;
      for (int32_t i = 0; i < seqlen; ++i) {
        double acc = bias ? ld(bias, dtype, c) : 0.0;
        for (int32_t k = 0; k < W; ++k) {
          const int64_t lag = W - 1 - k;
          double v;
          if (!cache_seqlens) {
            /* Shift state: index j of the sequence state ++ x. */
            const int64_t j = L + i - lag;
            v = j < L ? ld(st_in, dtype, sbase + j * ss_k)
                      : ld(x, dtype, xbase + (j - L) * x_st);
          } else {
            /* Ring state: absolute positions. */
            const int64_t pos = s + i - lag;
            if (pos < 0)
              v = 0.0;
            else if (pos >= s)
              v = ld(x, dtype, xbase + (pos - s) * x_st);
            else
              v = ld(st_in, dtype, sbase + (pos % L) * ss_k);
          }
          acc += ld(w, dtype, (int64_t)c * w_sc + (int64_t)k * w_sk) * v;
        }
        st(out, dtype, (int64_t)b * out_sb + (int64_t)c * out_sc + (int64_t)i * out_st,
           activate(acc, act));
      }
      if (!cache_seqlens) {
        /* Column m of the new state is entry seqlen + m of state ++ x. */
        for (int64_t m = 0; m < L; ++m) {
          const int64_t j = seqlen + m;
          if (j < L)
            copy_elem(st_out, sbase + m * ss_k, st_in, sbase + j * ss_k, dtype);
          else
            copy_elem(st_out, sbase + m * ss_k, x, xbase + (j - L) * x_st, dtype);
        }
      } else {
        /* Each new input lands in its ring column, in order. */
        for (int32_t i = 0; i < seqlen; ++i)
          copy_elem(st_out, sbase + ((s + i) % L) * ss_k, x, xbase + (int64_t)i * x_st, dtype);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* conditional gather of conv windows                                  */
/* ------------------------------------------------------------------ */

int oracle_gather_conv_window(const void* src, int64_t seq_len, int32_t conv_dim,
                              int64_t src_ss, int64_t src_sc, const int32_t* abs_positions,
                              int32_t real_count, int32_t max_count, void* out,
                              int64_t out_ss, int32_t d_conv, int dtype) {
  if (!valid_dtype(dtype) || seq_len < 1 || conv_dim < 0 || max_count < 0 || d_conv < 1)
    return ORC_ERR_ARGS;
  /* Reading: a count outside [0, max_count] is clamped into it. */
  int64_t n = real_count;
  if (n < 0) n = 0;
  if (n > max_count) n = max_count;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t p = abs_positions[i];
    for (int32_t c = 0; c < conv_dim; ++c) {
      for (int32_t k = 0; k < d_conv; ++k) {
        /* Window [p - d_conv, p), each row index clamped into the sequence. */
        int64_t row = p - d_conv + k;
        if (row < 0) row = 0;
        if (row > seq_len - 1) row = seq_len - 1;
        copy_elem(out, i * out_ss + (int64_t)c * d_conv + k, src,
                  row * src_ss + (int64_t)c * src_sc, dtype);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* conditional gather of SSM-state rows                                */
/* ------------------------------------------------------------------ */

int oracle_gather_ssm_state(const void* states, int64_t num_chunks, int64_t state_flat,
                            int64_t states_rs, const int64_t* chunk_indices,
                            int32_t real_count, int32_t max_count, void* out, int64_t out_rs,
                            int dtype) {
  if (!valid_dtype(dtype) || num_chunks < 1 || state_flat < 0 || max_count < 0)
    return ORC_ERR_ARGS;
  /* Reading: as for the conv windows, a count outside [0, max_count] is
     clamped into it. */
  int64_t n = real_count;
  if (n < 0) n = 0;
  if (n > max_count) n = max_count;
  for (int64_t i = 0; i < n; ++i) {
    /* Slot i receives the whole state row chosen by its index. */
    const int64_t r = chunk_indices[i];
    if (r < 0 || r >= num_chunks) return ORC_ERR_CHUNK;
    for (int64_t e = 0; e < state_flat; ++e)
      copy_elem(out, i * out_rs + e, states, r * states_rs + e, dtype);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* The same two ops split across host threads (CPU baseline only)      */
/* ------------------------------------------------------------------ */

/* The bodies above, unchanged, run on disjoint ranges of their outer loop:
 * rows for the fused op, channels for the varlen op.  Each range touches
 * only its own outputs (see fused_rows and varlen_channels), so the result
 * equals the single-threaded call bit for bit.  The first failing range's
 * code is returned. */
#define ORC_MAX_THREADS 256

typedef struct {
  const void* x; int64_t x_rs; const void* w; int64_t w_sc, w_sk;
  const void* cache_in; void* cache_out; int64_t num_blocks; int32_t H, N, D;
  int64_t cs0, cs1, cs2; const int64_t* positions; const int32_t* block_table;
  int64_t bt_rs; int32_t num_reqs, max_blocks; const int32_t* seq_idx;
  const int64_t* slot_mapping; const int32_t* query_start; void* out; int64_t out_rs, T;
  int32_t off_s, ws, W; int dtype, act, residual;
  int64_t lo, hi; int rc;
} fused_job;

static void* fused_worker(void* arg) {
  fused_job* j = (fused_job*)arg;
  j->rc = fused_rows(j->x, j->x_rs, j->w, j->w_sc, j->w_sk, j->cache_in, j->cache_out,
                     j->num_blocks, j->H, j->N, j->D, j->cs0, j->cs1, j->cs2, j->positions,
                     j->block_table, j->bt_rs, j->num_reqs, j->max_blocks, j->seq_idx,
                     j->slot_mapping, j->query_start, j->out, j->out_rs, j->T, j->off_s, j->ws,
                     j->W, j->dtype, j->act, j->residual, j->lo, j->hi);
  return NULL;
}

int oracle_fused_insert_conv_mt(const void* x, int64_t x_rs, const void* w, int64_t w_sc,
                                int64_t w_sk, const void* cache_in, void* cache_out,
                                int64_t num_blocks, int32_t H, int32_t N, int32_t D,
                                int64_t cs0, int64_t cs1, int64_t cs2,
                                const int64_t* positions, const int32_t* block_table,
                                int64_t bt_rs, int32_t num_reqs, int32_t max_blocks,
                                const int32_t* seq_idx, const int64_t* slot_mapping,
                                const int32_t* query_start, void* out, int64_t out_rs,
                                int64_t T, int32_t off_s, int32_t ws, int32_t W,
                                int dtype, int act, int residual, int32_t nthreads) {
  if (!valid_dtype(dtype) || T < 0 || H < 1 || N < 1 || ws < 1 || W < 1 ||
      off_s < 0 || off_s + ws > D || nthreads < 1 || nthreads > ORC_MAX_THREADS)
    return ORC_ERR_ARGS;
  fused_job jobs[ORC_MAX_THREADS];
  pthread_t tid[ORC_MAX_THREADS];
  int started[ORC_MAX_THREADS];
  for (int32_t i = 0; i < nthreads; ++i) {
    fused_job j = {x, x_rs, w, w_sc, w_sk, cache_in, cache_out, num_blocks, H, N, D,
                   cs0, cs1, cs2, positions, block_table, bt_rs, num_reqs, max_blocks,
                   seq_idx, slot_mapping, query_start, out, out_rs, T, off_s, ws, W,
                   dtype, act, residual, T * i / nthreads, T * (i + 1) / nthreads, ORC_OK};
    jobs[i] = j;
    started[i] = pthread_create(&tid[i], NULL, fused_worker, &jobs[i]) == 0;
    if (!started[i]) fused_worker(&jobs[i]); /* no thread: run the range here */
  }
  int rc = ORC_OK;
  for (int32_t i = 0; i < nthreads; ++i) {
    if (started[i]) pthread_join(tid[i], NULL);
    if (rc == ORC_OK) rc = jobs[i].rc;
  }
  return rc;
}

typedef struct {
  const void* x; int64_t x_sc, x_st; const void* w; int64_t w_sc, w_sk;
  const void* bias; const void* st_in; void* st_out; int64_t num_slots, ss_slot, ss_c, ss_k;
  const int32_t* qsl; int32_t batch; const int32_t* cache_indices; const uint8_t* has_init;
  void* out; int64_t o_sc, o_st, total_T; int32_t W; int dtype, act; int32_t pad_slot_id;
  int32_t lo, hi; int rc;
} varlen_job;

static void* varlen_worker(void* arg) {
  varlen_job* j = (varlen_job*)arg;
  j->rc = varlen_channels(j->x, j->x_sc, j->x_st, j->w, j->w_sc, j->w_sk, j->bias, j->st_in,
                          j->st_out, j->num_slots, j->ss_slot, j->ss_c, j->ss_k, j->qsl,
                          j->batch, j->cache_indices, j->has_init, j->out, j->o_sc, j->o_st,
                          j->total_T, j->W, j->dtype, j->act, j->pad_slot_id, j->lo, j->hi);
  return NULL;
}

int oracle_causal_conv1d_varlen_fwd_mt(const void* x, int64_t x_sc, int64_t x_st,
                                       const void* w, int64_t w_sc, int64_t w_sk,
                                       const void* bias, const void* st_in, void* st_out,
                                       int64_t num_slots, int64_t ss_slot, int64_t ss_c,
                                       int64_t ss_k, const int32_t* qsl, int32_t batch,
                                       const int32_t* cache_indices,
                                       const uint8_t* has_init, void* out, int64_t o_sc,
                                       int64_t o_st, int32_t dim, int64_t total_T,
                                       int32_t W, int dtype, int act, int32_t pad_slot_id,
                                       int32_t nthreads) {
  if (!valid_dtype(dtype) || batch < 0 || dim < 0 || W < 1 || total_T < 0 || nthreads < 1 ||
      nthreads > ORC_MAX_THREADS)
    return ORC_ERR_ARGS;
  varlen_job jobs[ORC_MAX_THREADS];
  pthread_t tid[ORC_MAX_THREADS];
  int started[ORC_MAX_THREADS];
  for (int32_t i = 0; i < nthreads; ++i) {
    varlen_job j = {x, x_sc, x_st, w, w_sc, w_sk, bias, st_in, st_out, num_slots, ss_slot,
                    ss_c, ss_k, qsl, batch, cache_indices, has_init, out, o_sc, o_st, total_T,
                    W, dtype, act, pad_slot_id, (int32_t)((int64_t)dim * i / nthreads),
                    (int32_t)((int64_t)dim * (i + 1) / nthreads), ORC_OK};
    jobs[i] = j;
    started[i] = pthread_create(&tid[i], NULL, varlen_worker, &jobs[i]) == 0;
    if (!started[i]) varlen_worker(&jobs[i]);
  }
  int rc = ORC_OK;
  for (int32_t i = 0; i < nthreads; ++i) {
    if (started[i]) pthread_join(tid[i], NULL);
    if (rc == ORC_OK) rc = jobs[i].rc;
  }
  return rc;
}

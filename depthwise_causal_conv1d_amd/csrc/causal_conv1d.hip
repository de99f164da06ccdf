// causal_conv1d.hip -- causal depthwise conv over packed variable-length
// sequences with a slot-indexed state pool (prefill), and its one-token
// decode step, for gfx950.
//
// Source: leeroopedia page "Implementation:Sgl project Sglang Mamba Ops",
// causal_conv1d_fwd and causal_conv1d_update (Signature, I/O Contract).
//
// Prefill decomposition: x is channel-major, so a channel's tokens are
// contiguous.  One wave64 owns one (sequence, channel) pair and walks the
// sequence front to back in chunks of 64*VEC tokens (16 bytes per lane).
// The W-1 inputs a lane needs before its own vector come from the lane
// below through a cross-lane shift, and from the previous chunk's last lane
// through a carry kept in registers; the state (or zeros) stands in for the
// inputs before the sequence start.  Because each element is read before the
// wave writes anything it still needs, out may be x itself (in place), with
// no grid-wide ordering.  The final W-1 inputs are read before any write and
// become the slot's new state at the end.  The weights, bias and state of
// the wave's channel are scalars.
#include "sconv_device.h"
#include "sconv_host.h"

namespace sconv {

// Build-time tuning knobs (defaults chosen by measurement on MI355X).
#ifndef SCONV_VARLEN_GROUP
#define SCONV_VARLEN_GROUP 4       // chunks loaded together per wave
#endif
#ifndef SCONV_VARLEN_EXTRA_LDS
#define SCONV_VARLEN_EXTRA_LDS 0   // unused dynamic LDS bytes per workgroup (fewer per CU)
#endif
#ifndef SCONV_VARLEN_NT_LOADS
#define SCONV_VARLEN_NT_LOADS 1    // streaming loads of the inputs (read once)
#endif
#ifndef SCONV_VARLEN_NT_STORES
#define SCONV_VARLEN_NT_STORES 1   // streaming stores of the outputs
#endif
#ifndef SCONV_UPDATE_TOKENS_VEC
#define SCONV_UPDATE_TOKENS_VEC 1  // vector-lane kernel for packed multi-token updates
#endif
// Channels per lane of the packed update kernels.  These launches are small
// (a decode batch): two channels per lane keep enough waves in flight to
// use every CU, where 16-byte lanes left most of them idle (measured on
// MI355X at 8..256 rows of 8192 channels).
#ifndef SCONV_UPDATE_LANE_CHANNELS
#define SCONV_UPDATE_LANE_CHANNELS 2
#endif

struct VarlenParams {
  const void* x;
  const void* w;
  const void* bias;
  void* states;
  const int32_t* qsl;
  const int32_t* cache_indices;
  const uint8_t* has_init;
  void* out;
  int64_t x_sc, x_st, w_sc, w_sk, ss_slot, ss_c, ss_k, o_sc, o_st, total_T;
  int64_t num_pairs;
  int32_t batch, dim, silu, pad_slot_id;
};

__device__ __forceinline__ float lane_shift_up(float v, int d) {
  return __shfl_up(v, (unsigned)d, 64);
}
__device__ __forceinline__ float read_lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Raw bits of VEC elements at tokens [tk, tk+VEC) of a row, zero bits for
// tokens outside [lo, hi).  One 16-byte load when the whole vector is inside.
template <typename D, int VEC>
__device__ __forceinline__ Pack<D, VEC> load_span(const typename D::storage* row, int64_t stride,
                                                  int64_t tk, int64_t lo, int64_t hi) {
  Pack<D, VEC> pk;
  if (tk >= lo && tk + VEC <= hi) {
    if constexpr (VEC > 1) {
#if SCONV_VARLEN_NT_LOADS
      pk.load_nt(row + tk);
#else
      pk.load(row + tk);
#endif
    } else {
      pk.load(row + tk * stride);
    }
  } else {
    typename Pack<D, VEC>::Elems v;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int64_t tok = tk + e;
      v.e[e] = (tok >= lo && tok < hi) ? row[tok * stride] : (typename D::storage)0;
    }
    pk.raw = __builtin_bit_cast(typename Pack<D, VEC>::raw_t, v);
  }
  return pk;
}

template <typename D, int VEC, int W>
__global__ __launch_bounds__(256) void varlen_fwd_kernel(const VarlenParams p) {
  using S = typename D::storage;
  using P = Pack<D, VEC>;
  constexpr int SL = W - 1;                 // state length
  constexpr int SA = SL > 0 ? SL : 1;       // array extent
  constexpr int kChunk = 64 * VEC;
  static_assert(VEC == 1 || VEC >= SL, "lane shift assumes VEC == 1 or VEC >= W-1");
  const S* x = static_cast<const S*>(p.x);  // may alias out
  S* out = static_cast<S*>(p.out);
  S* st = static_cast<S*>(p.states);
  const S* __restrict__ wt = static_cast<const S*>(p.w);
  const S* __restrict__ bias = static_cast<const S*>(p.bias);

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * (blockDim.x >> 6) +
                       uniform(threadIdx.x >> 6);
  if (wave >= p.num_pairs) return;
  const int b = (int)(wave / p.dim);
  const int c = (int)(wave - (int64_t)b * p.dim);
  const int64_t slot = p.cache_indices ? (int64_t)p.cache_indices[b] : (int64_t)b;
  if (slot == p.pad_slot_id) return;
  const int64_t start = p.qsl[b];
  const int64_t end = p.qsl[b + 1];
  const int64_t L = end - start;
  const bool init = p.has_init ? p.has_init[b] != 0 : false;

  float wk[W];
#pragma unroll
  for (int k = 0; k < W; ++k) wk[k] = load_as_float<D>(wt + (int64_t)c * p.w_sc + k * p.w_sk);
  const float bc = bias ? load_as_float<D>(bias + c) : 0.f;

  // Initial state (oldest first), as values and as raw bits.
  S* srow = st + slot * p.ss_slot + (int64_t)c * p.ss_c;
  S sraw[SA];
  float s0[SA];
#pragma unroll
  for (int m = 0; m < SA; ++m) {
    sraw[m] = (S)0;
    if (m < SL && init) sraw[m] = srow[m * p.ss_k];
    s0[m] = to_float<D>(sraw[m]);
  }
  // Final state: the last SL logical inputs, read before anything is written.
  const S* xrow = x + (int64_t)c * p.x_sc;
  S fin[SA];
#pragma unroll
  for (int m = 0; m < SA; ++m) {
    const int64_t i = L - SL + m;  // logical index, >= -SL
    fin[m] = (m < SL) ? (i >= 0 ? xrow[(start + i) * p.x_st] : pick(sraw, (int)(SL + i))) : (S)0;
  }

  S* orow = out + (int64_t)c * p.o_sc;
  // Chunks start on a VEC-aligned token so that full vectors are 16-byte
  // aligned (row bases are aligned by the launcher).
  int64_t base = start & ~(int64_t)(VEC - 1);
  float carry[SA];
#pragma unroll
  for (int m = 0; m < SA; ++m) {
    const int64_t i = base - start - SL + m;  // < 0
    carry[m] = (m < SL && i >= -SL) ? pick(s0, (int)(SL + i)) : 0.f;
  }

  // Chunks are processed in groups of G; the next group's loads are issued
  // before the current group is computed, so up to 2G chunks are in flight.
  constexpr int G = SCONV_VARLEN_GROUP;
  P buf[G];
#pragma unroll
  for (int u = 0; u < G; ++u)
    buf[u] = load_span<D, VEC>(xrow, p.x_st, base + u * kChunk + lane * VEC, start, end);
  for (; base < end; base += G * kChunk) {
    P cur[G];
#pragma unroll
    for (int u = 0; u < G; ++u) cur[u] = buf[u];
    if (base + G * kChunk < end) {
#pragma unroll
      for (int u = 0; u < G; ++u)
        buf[u] = load_span<D, VEC>(xrow, p.x_st, base + (G + u) * kChunk + lane * VEC, start, end);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t cb = base + u * kChunk;
      if (cb >= end) break;
      const int64_t tk = cb + lane * VEC;
      float f[VEC];
      cur[u].to_float(f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int64_t i = tk + e - start;
        if (i < 0) f[e] = (i >= -SL) ? pick(s0, (int)(SL + i)) : 0.f;
      }
      // prev[m]: input at token tk - SL + m.
      float prev[SA];
#pragma unroll
      for (int m = 0; m < SL; ++m) {
        const int d = SL - m;
        if constexpr (VEC == 1) {
          const float v = lane_shift_up(f[0], d);
          prev[m] = lane >= d ? v : pick(carry, SL + lane - d);
        } else {
          const float v = lane_shift_up(f[VEC - d], 1);
          prev[m] = lane >= 1 ? v : carry[m];
        }
      }
      if (SL == 0) prev[0] = 0.f;
      // Carry for the next chunk: the last SL inputs of this one.
#pragma unroll
      for (int m = 0; m < SL; ++m) {
        if constexpr (VEC == 1) carry[m] = read_lane63(lane_shift_up(f[0], SL - 1 - m));
        else carry[m] = read_lane63(f[VEC - SL + m]);
      }

      float y[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float acc = bc;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const int o = e - SL + k;  // offset from tk
          const float v = o >= 0 ? f[o < 0 ? 0 : o] : prev[SL + o < 0 ? 0 : SL + o];
          acc = __builtin_fmaf(wk[k], v, acc);
        }
        y[e] = p.silu ? silu(acc) : acc;
      }
      P o;
      o.from_float(y);
      if (tk >= start && tk + VEC <= end) {
        if constexpr (VEC > 1) {
#if SCONV_VARLEN_NT_STORES
          o.store_nt(orow + tk);
#else
          o.store(orow + tk);
#endif
        } else {
          o.store(orow + tk * p.o_st);
        }
      } else {
        typename P::Elems v = __builtin_bit_cast(typename P::Elems, o.raw);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int64_t tok = tk + e;
          if (tok >= start && tok < end) orow[tok * p.o_st] = v.e[e];
        }
      }
    }
  }

  // New state: lanes 0 .. SL-1 write one element each.
#pragma unroll
  for (int m = 0; m < SL; ++m)
    if (lane == m) srow[m * p.ss_k] = fin[m];
}

// ---------------------------------------------------------------- decode update

struct UpdateParams {
  // Small fields first (they come in with the first scalar load).
  int32_t batch, dim, silu, pad_slot_id;
  int32_t has_bias, has_idx, threads, nvec;  // nvec: lane vectors per row
  const void* x;
  void* states;
  const void* w;
  const void* bias;
  const int32_t* idx;
  void* out;
  int64_t x_rs, ss_slot, ss_c, ss_k, w_sc, w_sk, out_rs;
};

// Element `flat` of a run of lane vectors (compile-time index).
template <typename D, int VEC, int N>
__device__ __forceinline__ typename D::storage elem_at(const Pack<D, VEC> (&a)[N], int flat) {
  return __builtin_bit_cast(typename Pack<D, VEC>::Elems, a[flat / VEC].raw).e[flat % VEC];
}

// Keep a loaded value's load ahead of this point: without it the compiler
// sinks loads whose only use is under the store branch behind that branch.
template <typename T>
__device__ __forceinline__ void loaded_here(const T& v) {
  asm volatile("" ::"v"(v));
}

// One thread per (row, VEC channels): window = state ++ x, one dot product,
// state shifted by one.  Loads are unconditional from valid addresses (a
// PAD row reads slot 0 and stores nothing; a missing bias reads the weights
// and is replaced by zero), so the only dependent step is index -> state.
// The vector-lane kernels take packed [dim, W] weights and the packed
// [slot, dim, W-1] state layout and move each as W (W-1) lane vectors: the
// VEC channels' taps are contiguous, flat index e*W + k (e*(W-1) + m).  The
// one-channel kernels read any strides, one element per vector.
template <typename D, int VEC, int W>
__global__ __launch_bounds__(256) void update_kernel(const UpdateParams p) {
  using S = typename D::storage;
  using P = Pack<D, VEC>;
  constexpr int SL = W - 1;
  constexpr int SA = SL > 0 ? SL : 1;
  const S* x = static_cast<const S*>(p.x);
  S* out = static_cast<S*>(p.out);
  S* st = static_cast<S*>(p.states);
  const S* __restrict__ wt = static_cast<const S*>(p.w);
  // Bias, or the stand-in: each channel's first weight.
  const S* bbase = p.has_bias ? static_cast<const S*>(p.bias) : wt;
  const int64_t bstride = p.has_bias ? 1 : (VEC > 1 ? W : p.w_sc);
  // Fetch every kernel argument in the first batch of scalar loads.
  asm volatile("" ::"s"(p.idx), "s"(p.x), "s"(p.w), "s"(bbase), "s"(p.states), "s"(p.x_rs),
               "s"(p.ss_slot), "s"(p.out), "s"(p.out_rs));

  // The host bounds batch * nvec below 2^31, so 32-bit index math suffices.
  const uint32_t gid = blockIdx.x * (uint32_t)p.threads + threadIdx.x;
  uint32_t b = gid / (uint32_t)p.nvec;
  const bool live = b < (uint32_t)p.batch;
  int c0 = (int)(gid - b * (uint32_t)p.nvec) * VEC;
  if (!live) {
    b = p.batch - 1;
    c0 = 0;
  }

  // Independent loads: state index first, then input, weights, bias.
  int32_t slot_in = (int32_t)b;
  if (p.has_idx) slot_in = p.idx[b];
  P xv, bv, wv[W], sv[SA];
  xv.load(x + (int64_t)b * p.x_rs + c0);
#pragma unroll
  for (int k = 0; k < W; ++k) {
    if constexpr (VEC > 1)
      wv[k].load(wt + (int64_t)c0 * W + k * VEC);
    else
      wv[k].load(wt + (int64_t)c0 * p.w_sc + (int64_t)k * p.w_sk);
  }
  bv.load(bbase + (int64_t)c0 * bstride);

  // Dependent: the state of this thread's channels.
  const bool pad = slot_in == p.pad_slot_id;
  S* srow = st + (int64_t)(pad ? 0 : slot_in) * p.ss_slot;
#pragma unroll
  for (int m = 0; m < SL; ++m) {
    if constexpr (VEC > 1)
      sv[m].load(srow + (int64_t)c0 * SL + m * VEC);
    else
      sv[m].load(srow + (int64_t)c0 * p.ss_c + (int64_t)m * p.ss_k);
  }
  loaded_here(xv.raw);
  loaded_here(bv.raw);
#pragma unroll
  for (int k = 0; k < W; ++k) loaded_here(wv[k].raw);
#pragma unroll
  for (int m = 0; m < SL; ++m) loaded_here(sv[m].raw);

  float xf[VEC], bf[VEC], y[VEC];
  xv.to_float(xf);
  bv.to_float(bf);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float acc = p.has_bias ? bf[e] : 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const float v = k < SL ? to_float<D>(elem_at(sv, e * SL + (k < SL ? k : 0))) : xf[e];
      acc = __builtin_fmaf(to_float<D>(elem_at(wv, e * W + k)), v, acc);
    }
    y[e] = p.silu ? silu(acc) : acc;
  }
  if (!live || pad) return;
  P o;
  o.from_float(y);
  o.store(out + (int64_t)b * p.out_rs + c0);

  // Shifted state: window entries 1 .. W-1 (no state when W = 1; SA is SL
  // whenever the loop runs).
  const typename P::Elems xe = __builtin_bit_cast(typename P::Elems, xv.raw);
#pragma unroll
  for (int m = 0; m < SL; ++m) {
    typename P::Elems v;
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      const int flat = m * VEC + q, e = flat / SA, j = flat % SA;
      v.e[q] = j + 1 < SL ? elem_at(sv, e * SL + j + 1) : xe.e[e];
    }
    P pk;
    pk.raw = __builtin_bit_cast(typename P::raw_t, v);
    if constexpr (VEC > 1)
      pk.store(srow + (int64_t)c0 * SL + m * VEC);
    else
      pk.store(srow + (int64_t)c0 * p.ss_c + (int64_t)m * p.ss_k);
  }
}

// ---------------------------------------------------------------- multi-token update

struct UpdTokParams {
  const void* x;
  void* out;
  void* states;
  const void* w;
  const void* bias;  // or the weights as a stand-in (value unused)
  const int32_t* idx;
  const int32_t* seqlens;
  int64_t x_sb, x_sc, x_st, out_sb, out_sc, out_st;
  int64_t ss_slot, ss_c, ss_k, w_sc, w_sk;
  int32_t batch, dim, seqlen, L;
  int32_t silu, pad_slot_id, has_bias, has_idx, ring, threads;
  int32_t nvec;  // lane vectors per row (vector-lane kernel)
};

// One thread per (row, channel).  win[LMAX - l] holds the input at lag l
// (l = 1..LMAX) before the current token: loaded straight from the state
// column that holds it (shift state: column L - l; ring state: the column
// of position s - l), then shifted by one per token.  Taps are win slots
// and state columns are addresses, so no register array is indexed at run
// time.  The weights, the bias and the first tokens are loaded before the
// state index, so only index -> state is a dependent step.  A thread reads
// each x[i] before it writes out[i], so out may be x.
template <typename D, int W, int LMAX>
__global__ __launch_bounds__(256) void update_tokens_kernel(const UpdTokParams p) {
  using S = typename D::storage;
  static_assert(W - 1 <= LMAX, "the window holds every tap");
  constexpr int kChunk = 8;  // tokens loaded together
  asm volatile("" ::"s"(p.x), "s"(p.out), "s"(p.states), "s"(p.w), "s"(p.bias), "s"(p.idx),
               "s"(p.seqlens), "s"(p.x_sb), "s"(p.x_st), "s"(p.ss_slot), "s"(p.ss_c),
               "s"(p.ss_k));
  const S* x = static_cast<const S*>(p.x);
  S* out = static_cast<S*>(p.out);
  S* st = static_cast<S*>(p.states);
  const S* __restrict__ wt = static_cast<const S*>(p.w);
  const S* __restrict__ bs = static_cast<const S*>(p.bias);

  const uint32_t gid = blockIdx.x * (uint32_t)p.threads + threadIdx.x;
  uint32_t b = gid / (uint32_t)p.dim;
  const bool live = b < (uint32_t)p.batch;
  int c = (int)(gid - b * (uint32_t)p.dim);
  if (!live) {
    b = p.batch - 1;
    c = 0;
  }
  // Independent of the state: weights, bias, the first chunk of tokens.
  S wr[W];
#pragma unroll
  for (int k = 0; k < W; ++k) wr[k] = wt[(int64_t)c * p.w_sc + (int64_t)k * p.w_sk];
  const S br = bs[p.has_bias ? c : 0];
  const S* xrow = x + (int64_t)b * p.x_sb + (int64_t)c * p.x_sc;
  S* orow = out + (int64_t)b * p.out_sb + (int64_t)c * p.out_sc;
  S xc[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u) xc[u] = xrow[(int64_t)(u < p.seqlen ? u : p.seqlen - 1) * p.x_st];

  // State index and ring position, then the state columns.
  int32_t slot_in = (int32_t)b;
  if (p.has_idx) slot_in = p.idx[b];
  int32_t s0 = p.L;  // shift state: its columns are positions 0 .. L-1
  if (p.ring) s0 = p.seqlens[b];
  const bool pad = slot_in == p.pad_slot_id;
  S* srow = st + (int64_t)(pad ? 0 : slot_in) * p.ss_slot + (int64_t)c * p.ss_c;
  const int L = p.L;
  // Ring column of position s0 - l, l = 1..L: (r - l) mod L, r = s0 mod L.
  const int r0 = (p.ring && L > 0) ? (int)((uint32_t)s0 % (uint32_t)L) : 0;
  S win[LMAX];
#pragma unroll
  for (int j = 0; j < LMAX; ++j) {
    const int l = LMAX - j;  // lag of this slot; slots with l > L are never read
    int col = p.ring ? r0 - l : L - l;
    if (col < 0) col += L;
    win[j] = srow[(int64_t)(l <= L && col >= 0 ? col : 0) * p.ss_k];
  }
  float wk[W];
#pragma unroll
  for (int k = 0; k < W; ++k) wk[k] = to_float<D>(wr[k]);
  const float bias = p.has_bias ? to_float<D>(br) : 0.f;

  for (int i0 = 0; i0 < p.seqlen; i0 += kChunk) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int i = i0 + u < p.seqlen ? i0 + u : p.seqlen - 1;  // clamped: a valid row
        xc[u] = xrow[(int64_t)i * p.x_st];
      }
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = i0 + u;
      if (i >= p.seqlen) break;
      const S xi = xc[u];
      float acc = bias;
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int l = W - 1 - k;
        float v = to_float<D>(l == 0 ? xi : win[LMAX - (l > 0 ? l : 1)]);
        if (p.ring && s0 + i - l < 0) v = 0.f;  // before position 0
        acc = __builtin_fmaf(wk[k], v, acc);
      }
      const float y = p.silu ? silu(acc) : acc;
      if (live && !pad) {
        S o;
        if constexpr (sizeof(S) == 2) o = __builtin_bit_cast(uint16_t, (__bf16)y);
        else o = y;
        orow[(int64_t)i * p.out_st] = o;
      }
#pragma unroll
      for (int j = 0; j + 1 < LMAX; ++j) win[j] = win[j + 1];
      win[LMAX - 1] = xi;
    }
  }
  if (!live || pad) return;
  // The last L inputs back into the state: win[LMAX - l] is the input at
  // position s0 + seqlen - l, ring column (r1 - l) mod L.
  const int r1 = (p.ring && L > 0) ? (int)((uint32_t)(s0 + p.seqlen) % (uint32_t)L) : 0;
#pragma unroll
  for (int l = 1; l <= LMAX; ++l) {
    if (l > L) break;
    int col = p.ring ? r1 - l : L - l;
    if (col < 0) col += L;
    srow[(int64_t)col * p.ss_k] = win[LMAX - l];
  }
}

// The same update with vector lanes, for the packed layout: x and out with
// contiguous channels, weights [dim, W] and states [slot, dim, W-1] packed.
// A lane owns VEC channels of one row.  Each token of x and out is one lane
// vector; the lane's W-1 state columns are W-1 vectors (element e*(W-1) +
// column of channel e) and its taps W vectors (element e*W + k).  The
// window wl[l-1] holds the raw inputs at lag l, taken from the column of
// each lag: a per-lane choice among W-1 columns (rows, and with them the
// ring rotation, can change inside a wave), made with selects on values
// already in registers.  Values stay raw bits until used, so a state
// written back is an exact copy of the inputs it holds.
template <typename D, int VEC, int W>
__global__ __launch_bounds__(256) void update_tokens_vec_kernel(const UpdTokParams p) {
  using S = typename D::storage;
  using P = Pack<D, VEC>;
  using E = typename P::Elems;
  constexpr int L = W - 1;
  static_assert(L >= 1, "the packed kernel has a state");
  constexpr int kChunk = 4;  // tokens loaded together
  asm volatile("" ::"s"(p.x), "s"(p.out), "s"(p.states), "s"(p.w), "s"(p.bias), "s"(p.idx),
               "s"(p.seqlens), "s"(p.x_sb), "s"(p.x_st), "s"(p.ss_slot));
  const S* x = static_cast<const S*>(p.x);
  S* out = static_cast<S*>(p.out);
  S* st = static_cast<S*>(p.states);
  const S* __restrict__ wt = static_cast<const S*>(p.w);
  const S* __restrict__ bs = static_cast<const S*>(p.bias);

  // The host bounds batch * nvec below 2^31.
  const uint32_t gid = blockIdx.x * (uint32_t)p.threads + threadIdx.x;
  uint32_t b = gid / (uint32_t)p.nvec;
  const bool live = b < (uint32_t)p.batch;
  int c0 = (int)(gid - b * (uint32_t)p.nvec) * VEC;
  if (!live) {
    b = p.batch - 1;
    c0 = 0;
  }
  // Independent of the state: taps, bias (or the weights as a stand-in),
  // the first tokens.
  P wv[W], bv;
#pragma unroll
  for (int k = 0; k < W; ++k) wv[k].load(wt + (int64_t)c0 * W + k * VEC);
  bv.load(bs + (p.has_bias ? c0 : 0));
  const S* xrow = x + (int64_t)b * p.x_sb + c0;
  S* orow = out + (int64_t)b * p.out_sb + c0;
  P xc[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u)
    xc[u].load(xrow + (int64_t)(u < p.seqlen ? u : p.seqlen - 1) * p.x_st);

  // State index and ring position, then the state columns.
  int32_t slot_in = (int32_t)b;
  if (p.has_idx) slot_in = p.idx[b];
  int32_t s0 = L;  // shift state: its columns are positions 0 .. L-1
  if (p.ring) s0 = p.seqlens[b];
  const bool pad = slot_in == p.pad_slot_id;
  S* srow = st + (int64_t)(pad ? 0 : slot_in) * p.ss_slot + (int64_t)c0 * L;
  P sv[L];
#pragma unroll
  for (int m = 0; m < L; ++m) sv[m].load(srow + m * VEC);

  float wk[W][VEC], bias[VEC];
  bv.to_float(bias);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (!p.has_bias) bias[e] = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k][e] = to_float<D>(elem_at(wv, e * W + k));
  }
  // Lag l sits in column (r0 - l) mod L of a ring (r0 = s0 mod L), in
  // column L - l of a shift state.
  const int r0 = p.ring ? (int)((uint32_t)s0 % (uint32_t)L) : 0;
  E wl[L];
#pragma unroll
  for (int l = 1; l <= L; ++l) {
    int col = p.ring ? r0 - l : L - l;
    if (col < 0) col += L;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      S v = elem_at(sv, e * L);
#pragma unroll
      for (int q = 1; q < L; ++q) v = col == q ? elem_at(sv, e * L + q) : v;
      wl[l - 1].e[e] = v;
    }
  }

  for (int i0 = 0; i0 < p.seqlen; i0 += kChunk) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int i = i0 + u < p.seqlen ? i0 + u : p.seqlen - 1;  // clamped: a valid row
        xc[u].load(xrow + (int64_t)i * p.x_st);
      }
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = i0 + u;
      if (i >= p.seqlen) break;
      const E xe = __builtin_bit_cast(E, xc[u].raw);
      float y[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float acc = bias[e];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const int l = W - 1 - k;
          float v = to_float<D>(l == 0 ? xe.e[e] : wl[l > 0 ? l - 1 : 0].e[e]);
          if (l > 0 && p.ring && s0 + i - l < 0) v = 0.f;  // before position 0
          acc = __builtin_fmaf(wk[k][e], v, acc);
        }
        y[e] = p.silu ? silu(acc) : acc;
      }
      if (live && !pad) {
        P o;
        o.from_float(y);
        o.store(orow + (int64_t)i * p.out_st);
      }
#pragma unroll
      for (int l = L; l >= 2; --l) wl[l - 1] = wl[l - 2];
      wl[0] = xe;
    }
  }
  if (!live || pad) return;
  // New state: column q receives the input at lag l(q) after the last
  // token, the lag whose column is q: (r1 - q) mod L in (0, L] for a ring
  // (r1 = (s0 + seqlen) mod L), L - q for a shift state.
  const int r1 = p.ring ? (int)((uint32_t)(s0 + p.seqlen) % (uint32_t)L) : 0;
  E so[L];
#pragma unroll
  for (int q = 0; q < L; ++q) {
    int lq = p.ring ? r1 - q : L - q;
    if (lq <= 0) lq += L;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      S v = wl[0].e[e];
#pragma unroll
      for (int l = 2; l <= L; ++l) v = lq == l ? wl[l - 1].e[e] : v;
      const int flat = e * L + q;
      so[flat / VEC].e[flat % VEC] = v;
    }
  }
#pragma unroll
  for (int m = 0; m < L; ++m) {
    P pk;
    pk.raw = __builtin_bit_cast(typename P::raw_t, so[m]);
    pk.store(srow + m * VEC);
  }
}

template <typename D, int VEC>
static void launch_upd_tok_vec(int W, const UpdTokParams& p, uint32_t g, uint32_t th,
                               hipStream_t s) {
  switch (W) {
    case 2: hipLaunchKernelGGL((update_tokens_vec_kernel<D, VEC, 2>), dim3(g), dim3(th), 0, s, p); break;
    case 3: hipLaunchKernelGGL((update_tokens_vec_kernel<D, VEC, 3>), dim3(g), dim3(th), 0, s, p); break;
    default: hipLaunchKernelGGL((update_tokens_vec_kernel<D, VEC, 4>), dim3(g), dim3(th), 0, s, p); break;
  }
}

template <typename D, int LMAX>
static void launch_upd_tok(int W, const UpdTokParams& p, uint32_t g, uint32_t th, hipStream_t s) {
  switch (W) {
    case 1: hipLaunchKernelGGL((update_tokens_kernel<D, 1, LMAX>), dim3(g), dim3(th), 0, s, p); break;
    case 2: hipLaunchKernelGGL((update_tokens_kernel<D, 2, LMAX>), dim3(g), dim3(th), 0, s, p); break;
    case 3: hipLaunchKernelGGL((update_tokens_kernel<D, 3, LMAX>), dim3(g), dim3(th), 0, s, p); break;
    default: hipLaunchKernelGGL((update_tokens_kernel<D, 4, LMAX>), dim3(g), dim3(th), 0, s, p); break;
  }
}

// Shared by causal_conv1d_update_tokens and the ring form of
// causal_conv1d_update.
static int update_tokens_launch(
    const char* fn, const void* x, int64_t x_sb, int64_t x_sc, int64_t x_st, int32_t seqlen,
    void* conv_states, int64_t num_slots, int32_t state_len, int64_t ss_slot, int64_t ss_c,
    int64_t ss_k, const void* weight, int64_t w_sc, int64_t w_sk, const void* bias,
    const int32_t* cache_seqlens, const int32_t* conv_state_indices, void* out, int64_t out_sb,
    int64_t out_sc, int64_t out_st, int32_t batch, int32_t dim, int32_t W, int32_t dtype,
    int32_t activation, int32_t pad_slot_id, hipStream_t stream) {
  if (batch < 0 || dim < 0 || seqlen < 0)
    return fail(SCONV_ERR_INVALID, "%s: batch, dim and seqlen must be >= 0", fn);
  if (W < 1 || W > 4) return fail(SCONV_ERR_INVALID, "%s: W=%d outside [1, 4]", fn, W);
  if (!valid_dtype(dtype)) return fail(SCONV_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (!valid_act(activation))
    return fail(SCONV_ERR_INVALID, "%s: unknown activation %d", fn, activation);
  if (state_len < W - 1 || state_len < 0)
    return fail(SCONV_ERR_INVALID, "%s: state_len=%d shorter than W-1", fn, state_len);
  if (cache_seqlens && state_len < 1)
    return fail(SCONV_ERR_INVALID, "%s: a ring state needs state_len >= 1", fn);
  if (state_len > 8)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: state_len=%d above 8", fn, state_len);
  if (batch == 0 || dim == 0 || seqlen == 0) return SCONV_OK;
  if (!x || !weight || !out || (state_len > 0 && !conv_states))
    return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
  if (state_len > 0 && !conv_state_indices && num_slots < batch)
    return fail(SCONV_ERR_INVALID, "%s: state pool has fewer slots than rows", fn);
  if (w_sc < 1 || w_sk < 1 || x_sb < 0 || x_sc < 0 || x_st < 0 || out_sb < 0 || out_sc < 0 ||
      out_st < 0 || (state_len > 0 && (num_slots < 1 || ss_slot < 1 || ss_c < 1 || ss_k < 1)))
    return fail(SCONV_ERR_INVALID, "%s: strides too small", fn);
  const bool inplace = out == x;
  if (inplace && (out_sb != x_sb || out_sc != x_sc || out_st != x_st))
    return fail(SCONV_ERR_INVALID, "%s: in-place call needs identical strides", fn);
  const int64_t es = elem_size(dtype);
  if (!inplace) {
    const int64_t xb = ((int64_t)(batch - 1) * x_sb + (int64_t)(dim - 1) * x_sc +
                        (int64_t)(seqlen - 1) * x_st + 1) * es;
    const int64_t ob = ((int64_t)(batch - 1) * out_sb + (int64_t)(dim - 1) * out_sc +
                        (int64_t)(seqlen - 1) * out_st + 1) * es;
    if (overlap(x, xb, out, ob)) return fail(SCONV_ERR_INVALID, "%s: out partially overlaps x", fn);
  }
  // Vector lanes for the packed layout (state_len = W-1, channels
  // contiguous, every row start and row step a whole number of vectors).
  constexpr int kLC = SCONV_UPDATE_LANE_CHANNELS;
  const int64_t lb = kLC * es;  // bytes per lane vector
  const bool vec = SCONV_UPDATE_TOKENS_VEC && W >= 2 && state_len == W - 1 && x_sc == 1 &&
                   out_sc == 1 && dim % kLC == 0 && x_sb % kLC == 0 && x_st % kLC == 0 &&
                   out_sb % kLC == 0 && out_st % kLC == 0 && aligned_to(x, lb) &&
                   aligned_to(out, lb) && w_sc == W && w_sk == 1 && aligned_to(weight, lb) &&
                   (!bias || aligned_to(bias, lb)) && ss_k == 1 && ss_c == state_len &&
                   ss_slot % kLC == 0 && aligned_to(conv_states, lb);
  const int64_t threads_total = (int64_t)batch * (vec ? dim / kLC : dim);
  if (threads_total + 256 > INT32_MAX)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: batch * dim too large", fn);
  UpdTokParams p = {};
  p.x = x; p.out = out; p.states = conv_states; p.w = weight;
  p.bias = bias ? bias : weight; p.idx = conv_state_indices; p.seqlens = cache_seqlens;
  p.x_sb = x_sb; p.x_sc = x_sc; p.x_st = x_st;
  p.out_sb = out_sb; p.out_sc = out_sc; p.out_st = out_st;
  p.ss_slot = ss_slot; p.ss_c = ss_c; p.ss_k = ss_k; p.w_sc = w_sc; p.w_sk = w_sk;
  p.batch = batch; p.dim = dim; p.seqlen = seqlen; p.L = state_len;
  p.silu = activation == SCONV_ACT_SILU; p.pad_slot_id = pad_slot_id;
  p.has_bias = bias != nullptr; p.has_idx = conv_state_indices != nullptr;
  p.ring = cache_seqlens != nullptr;
  if (state_len == 0) {  // W == 1: no state to read or write
    p.states = const_cast<void*>(weight); p.ss_slot = 0; p.ss_c = 0; p.ss_k = 0;
  }
  const uint32_t th = threads_total >= 256 * 512 ? 256 : 64;
  p.threads = (int32_t)th;
  p.nvec = vec ? dim / kLC : dim;
  const int64_t grid = cdiv(threads_total, th);
  if (vec) {
    if (dtype == SCONV_BF16) launch_upd_tok_vec<Bf16, kLC>(W, p, (uint32_t)grid, th, stream);
    else launch_upd_tok_vec<F32, kLC>(W, p, (uint32_t)grid, th, stream);
    return check_launch(fn);
  }
  if (dtype == SCONV_BF16) {
    if (state_len <= 4) launch_upd_tok<Bf16, 4>(W, p, (uint32_t)grid, th, stream);
    else launch_upd_tok<Bf16, 8>(W, p, (uint32_t)grid, th, stream);
  } else {
    if (state_len <= 4) launch_upd_tok<F32, 4>(W, p, (uint32_t)grid, th, stream);
    else launch_upd_tok<F32, 8>(W, p, (uint32_t)grid, th, stream);
  }
  return check_launch(fn);
}

// ---------------------------------------------------------------- dispatch

template <typename D, int VEC>
static void launch_varlen(int W, const VarlenParams& p, uint32_t g, hipStream_t s) {
  switch (W) {
    case 1: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 1>), dim3(g), dim3(256), SCONV_VARLEN_EXTRA_LDS, s, p); break;
    case 2: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 2>), dim3(g), dim3(256), SCONV_VARLEN_EXTRA_LDS, s, p); break;
    case 3: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 3>), dim3(g), dim3(256), SCONV_VARLEN_EXTRA_LDS, s, p); break;
    default: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 4>), dim3(g), dim3(256), SCONV_VARLEN_EXTRA_LDS, s, p); break;
  }
}

template <typename D, int VEC>
static void launch_update(int W, const UpdateParams& p, uint32_t g, uint32_t th, hipStream_t s) {
  switch (W) {
    case 1: hipLaunchKernelGGL((update_kernel<D, VEC, 1>), dim3(g), dim3(th), 0, s, p); break;
    case 2: hipLaunchKernelGGL((update_kernel<D, VEC, 2>), dim3(g), dim3(th), 0, s, p); break;
    case 3: hipLaunchKernelGGL((update_kernel<D, VEC, 3>), dim3(g), dim3(th), 0, s, p); break;
    default: hipLaunchKernelGGL((update_kernel<D, VEC, 4>), dim3(g), dim3(th), 0, s, p); break;
  }
}

}  // namespace sconv

extern "C" int causal_conv1d_varlen_fwd(
    const void* x, int64_t x_stride_c, int64_t x_stride_t, const void* weight,
    int64_t w_stride_c, int64_t w_stride_k, const void* bias, void* conv_states,
    int64_t num_slots, int64_t st_stride_slot, int64_t st_stride_c, int64_t st_stride_k,
    const int32_t* query_start_loc, int32_t batch, const int32_t* cache_indices,
    const uint8_t* has_initial_state, void* out, int64_t out_stride_c, int64_t out_stride_t,
    int32_t dim, int64_t total_T, int32_t W, int32_t dtype, int32_t activation,
    int32_t pad_slot_id, hipStream_t stream) {
  using namespace sconv;
  clear_error();
  const char* fn = "causal_conv1d_varlen_fwd";
  if (batch < 0 || dim < 0 || total_T < 0)
    return fail(SCONV_ERR_INVALID, "%s: batch, dim and total_T must be >= 0", fn);
  if (W < 1 || W > 4) return fail(SCONV_ERR_INVALID, "%s: W=%d outside [1, 4]", fn, W);
  if (!valid_dtype(dtype)) return fail(SCONV_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (!valid_act(activation))
    return fail(SCONV_ERR_INVALID, "%s: unknown activation %d", fn, activation);
  if (batch == 0 || dim == 0) return SCONV_OK;
  if (!x || !weight || !out || !query_start_loc || (W > 1 && !conv_states))
    return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
  if (W > 1 && (num_slots < 1 || (!cache_indices && num_slots < batch)))
    return fail(SCONV_ERR_INVALID, "%s: state pool has fewer slots than needed", fn);
  if (x_stride_c < 1 || x_stride_t < 1 || out_stride_c < 1 || out_stride_t < 1 ||
      w_stride_c < 1 || w_stride_k < 1 ||
      (W > 1 && (st_stride_slot < 1 || st_stride_c < 1 || st_stride_k < 1)))
    return fail(SCONV_ERR_INVALID, "%s: strides must be >= 1", fn);
  const int64_t es = elem_size(dtype);
  const bool inplace = out == x;
  if (inplace && (out_stride_c != x_stride_c || out_stride_t != x_stride_t))
    return fail(SCONV_ERR_INVALID, "%s: in-place call needs identical strides", fn);
  if (!inplace && total_T > 0) {
    const int64_t xb = ((int64_t)(dim - 1) * x_stride_c + (total_T - 1) * x_stride_t + 1) * es;
    const int64_t ob = ((int64_t)(dim - 1) * out_stride_c + (total_T - 1) * out_stride_t + 1) * es;
    if (overlap(x, xb, out, ob))
      return fail(SCONV_ERR_INVALID, "%s: out partially overlaps x", fn);
  }
  const int vec16 = (int)(16 / es);
  const bool vec = x_stride_t == 1 && out_stride_t == 1 && x_stride_c % vec16 == 0 &&
                   out_stride_c % vec16 == 0 && aligned16(x) && aligned16(out);
  VarlenParams p;
  p.x = x; p.w = weight; p.bias = bias; p.states = conv_states; p.qsl = query_start_loc;
  p.cache_indices = cache_indices; p.has_init = has_initial_state; p.out = out;
  p.x_sc = x_stride_c; p.x_st = x_stride_t; p.w_sc = w_stride_c; p.w_sk = w_stride_k;
  p.ss_slot = st_stride_slot; p.ss_c = st_stride_c; p.ss_k = st_stride_k;
  p.o_sc = out_stride_c; p.o_st = out_stride_t; p.total_T = total_T;
  p.num_pairs = (int64_t)batch * dim;
  p.batch = batch; p.dim = dim; p.silu = activation == SCONV_ACT_SILU;
  p.pad_slot_id = pad_slot_id;
  const int64_t grid = cdiv(p.num_pairs, 4);
  if (grid > INT32_MAX) return fail(SCONV_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (dtype == SCONV_BF16) {
    if (vec) launch_varlen<Bf16, 8>(W, p, (uint32_t)grid, stream);
    else launch_varlen<Bf16, 1>(W, p, (uint32_t)grid, stream);
  } else {
    if (vec) launch_varlen<F32, 4>(W, p, (uint32_t)grid, stream);
    else launch_varlen<F32, 1>(W, p, (uint32_t)grid, stream);
  }
  return check_launch(fn);
}

extern "C" int causal_conv1d_update(const void* x, int64_t x_stride_b, void* conv_states,
                                    int64_t num_slots, int64_t st_stride_slot,
                                    int64_t st_stride_c, int64_t st_stride_k,
                                    const void* weight, int64_t w_stride_c, int64_t w_stride_k,
                                    const void* bias, const int32_t* cache_seqlens,
                                    const int32_t* conv_state_indices, void* out,
                                    int64_t out_stride_b, int32_t batch, int32_t dim, int32_t W,
                                    int32_t dtype, int32_t activation, int32_t pad_slot_id,
                                    hipStream_t stream) {
  using namespace sconv;
  clear_error();
  const char* fn = "causal_conv1d_update";
  if (batch < 0 || dim < 0) return fail(SCONV_ERR_INVALID, "%s: batch and dim must be >= 0", fn);
  if (W < 1 || W > 4) return fail(SCONV_ERR_INVALID, "%s: W=%d outside [1, 4]", fn, W);
  if (!valid_dtype(dtype)) return fail(SCONV_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (!valid_act(activation))
    return fail(SCONV_ERR_INVALID, "%s: unknown activation %d", fn, activation);
  if (cache_seqlens && W > 1)  // ring state of W-1 columns, one token (W = 1 has no state)
    return update_tokens_launch(fn, x, x_stride_b, 1, 0, 1, conv_states, num_slots, W - 1,
                                st_stride_slot, st_stride_c, st_stride_k, weight, w_stride_c,
                                w_stride_k, bias, cache_seqlens, conv_state_indices, out,
                                out_stride_b, 1, 0, batch, dim, W, dtype, activation,
                                pad_slot_id, stream);
  if (batch == 0 || dim == 0) return SCONV_OK;
  if (!x || !weight || !out || (W > 1 && !conv_states))
    return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
  if (W > 1 && !conv_state_indices && num_slots < batch)
    return fail(SCONV_ERR_INVALID, "%s: state pool has fewer slots than rows", fn);
  if (x_stride_b < dim || out_stride_b < dim || w_stride_c < 1 || w_stride_k < 1 ||
      (W > 1 && (num_slots < 1 || st_stride_slot < 1 || st_stride_c < 1 || st_stride_k < 1)))
    return fail(SCONV_ERR_INVALID, "%s: strides too small", fn);
  const int64_t es = elem_size(dtype);
  const bool inplace = out == x;
  if (inplace && out_stride_b != x_stride_b)
    return fail(SCONV_ERR_INVALID, "%s: in-place call needs identical strides", fn);
  if (!inplace) {
    const int64_t xb = ((int64_t)(batch - 1) * x_stride_b + dim) * es;
    const int64_t ob = ((int64_t)(batch - 1) * out_stride_b + dim) * es;
    if (overlap(x, xb, out, ob))
      return fail(SCONV_ERR_INVALID, "%s: out partially overlaps x", fn);
  }
  // Vector lanes need packed weights and states, aligned rows and bias.
  constexpr int kLC = SCONV_UPDATE_LANE_CHANNELS;
  const int64_t lb = kLC * es;  // bytes per lane vector
  const bool vec = dim % kLC == 0 && x_stride_b % kLC == 0 && out_stride_b % kLC == 0 &&
                   aligned_to(x, lb) && aligned_to(out, lb) && w_stride_c == W &&
                   w_stride_k == 1 && aligned_to(weight, lb) && (!bias || aligned_to(bias, lb)) &&
                   (W == 1 || (st_stride_k == 1 && st_stride_c == W - 1 &&
                               st_stride_slot % kLC == 0 && aligned_to(conv_states, lb)));
  const int VEC = vec ? kLC : 1;
  UpdateParams p = {};
  p.x = x; p.states = conv_states; p.w = weight; p.bias = bias; p.idx = conv_state_indices;
  p.out = out; p.x_rs = x_stride_b; p.ss_slot = st_stride_slot; p.ss_c = st_stride_c;
  p.ss_k = st_stride_k; p.w_sc = w_stride_c; p.w_sk = w_stride_k; p.out_rs = out_stride_b;
  p.nvec = (int32_t)cdiv(dim, VEC);
  p.batch = batch; p.dim = dim; p.silu = activation == SCONV_ACT_SILU;
  p.pad_slot_id = pad_slot_id;
  p.has_bias = bias != nullptr;
  p.has_idx = conv_state_indices != nullptr;
  const int64_t threads_total = (int64_t)p.nvec * batch;
  if (threads_total + 256 > INT32_MAX) return fail(SCONV_ERR_UNSUPPORTED, "%s: batch * dim too large", fn);
  const uint32_t th = threads_total >= 256 * 512 ? 256 : 64;
  p.threads = (int32_t)th;
  const int64_t grid = cdiv(threads_total, th);
  if (dtype == SCONV_BF16) {
    if (vec) launch_update<Bf16, kLC>(W, p, (uint32_t)grid, th, stream);
    else launch_update<Bf16, 1>(W, p, (uint32_t)grid, th, stream);
  } else {
    if (vec) launch_update<F32, kLC>(W, p, (uint32_t)grid, th, stream);
    else launch_update<F32, 1>(W, p, (uint32_t)grid, th, stream);
  }
  return check_launch(fn);
}

extern "C" int causal_conv1d_update_tokens(
    const void* x, int64_t x_stride_b, int64_t x_stride_c, int64_t x_stride_t, int32_t seqlen,
    void* conv_states, int64_t num_slots, int32_t state_len, int64_t st_stride_slot,
    int64_t st_stride_c, int64_t st_stride_k, const void* weight, int64_t w_stride_c,
    int64_t w_stride_k, const void* bias, const int32_t* cache_seqlens,
    const int32_t* conv_state_indices, void* out, int64_t out_stride_b, int64_t out_stride_c,
    int64_t out_stride_t, int32_t batch, int32_t dim, int32_t W, int32_t dtype,
    int32_t activation, int32_t pad_slot_id, hipStream_t stream) {
  using namespace sconv;
  clear_error();
  return update_tokens_launch("causal_conv1d_update_tokens", x, x_stride_b, x_stride_c,
                              x_stride_t, seqlen, conv_states, num_slots, state_len,
                              st_stride_slot, st_stride_c, st_stride_k, weight, w_stride_c,
                              w_stride_k, bias, cache_seqlens, conv_state_indices, out,
                              out_stride_b, out_stride_c, out_stride_t, batch, dim, W, dtype,
                              activation, pad_slot_id, stream);
}

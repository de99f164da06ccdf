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
#ifndef SCONV_VARLEN_NT_STORES
#define SCONV_VARLEN_NT_STORES 1   // streaming stores of the outputs
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
      pk.load(row + tk);
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
  const void* x;
  void* states;
  const void* w;
  const void* bias;
  const int32_t* idx;
  void* out;
  int64_t x_rs, ss_slot, ss_c, ss_k, w_sc, w_sk, out_rs;
  int64_t nvec;  // lane vectors per row
  int32_t batch, dim, silu, pad_slot_id, state_packed;
};

// One thread per (row, VEC channels): window = state ++ x, one dot product,
// state shifted by one.  The VEC*(W-1) state elements of a thread are
// contiguous in the usual [slot, dim, W-1] layout and move as 16-byte chunks.
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
  const S* __restrict__ bias = static_cast<const S*>(p.bias);

  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = gid / p.nvec;
  if (b >= p.batch) return;
  const int c0 = (int)(gid - b * p.nvec) * VEC;
  const int64_t slot = p.idx ? (int64_t)p.idx[b] : b;
  if (slot == p.pad_slot_id) return;

  P xv;
  xv.load(x + b * p.x_rs + c0);
  typename P::Elems xe = __builtin_bit_cast(typename P::Elems, xv.raw);
  float xf[VEC];
  xv.to_float(xf);

  S* srow = st + slot * p.ss_slot;
  struct StateElems { S e[VEC * SA]; } sr;  // [e][m] flattened, m fastest
  constexpr int kChunkE = 16 / (int)sizeof(S);
  constexpr bool kChunked = VEC > 1 && SL > 0 && (VEC * SL) % kChunkE == 0;
  if constexpr (kChunked) {
    if (p.state_packed) {
#pragma unroll
      for (int ch = 0; ch < VEC * SL / kChunkE; ++ch) {
        Pack<D, kChunkE> pk;
        pk.load(srow + (int64_t)c0 * SL + ch * kChunkE);
        typename Pack<D, kChunkE>::Elems v = __builtin_bit_cast(typename Pack<D, kChunkE>::Elems, pk.raw);
#pragma unroll
        for (int q = 0; q < kChunkE; ++q) sr.e[ch * kChunkE + q] = v.e[q];
      }
    }
  }
  if (!kChunked || !p.state_packed) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int m = 0; m < SL; ++m)
        sr.e[e * SA + m] = srow[(int64_t)(c0 + e) * p.ss_c + m * p.ss_k];
  }

  float y[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float acc = bias ? load_as_float<D>(bias + c0 + e) : 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const float v = k < SL ? to_float<D>(sr.e[e * SA + (k < SL ? k : 0)]) : xf[e];
      acc = __builtin_fmaf(load_as_float<D>(wt + (int64_t)(c0 + e) * p.w_sc + k * p.w_sk), v, acc);
    }
    y[e] = p.silu ? silu(acc) : acc;
  }
  P o;
  o.from_float(y);
  o.store(out + b * p.out_rs + c0);

  // Shifted state: window entries 1 .. W-1.
  StateElems ns;
#pragma unroll
  for (int e = 0; e < VEC; ++e)
#pragma unroll
    for (int m = 0; m < SL; ++m)
      ns.e[e * SA + m] = (m + 1 < SL) ? sr.e[e * SA + m + 1] : xe.e[e];
  if constexpr (kChunked) {
    if (p.state_packed) {
#pragma unroll
      for (int ch = 0; ch < VEC * SL / kChunkE; ++ch) {
        typename Pack<D, kChunkE>::Elems v;
#pragma unroll
        for (int q = 0; q < kChunkE; ++q) v.e[q] = ns.e[ch * kChunkE + q];
        Pack<D, kChunkE> pk;
        pk.raw = __builtin_bit_cast(typename Pack<D, kChunkE>::raw_t, v);
        pk.store(srow + (int64_t)c0 * SL + ch * kChunkE);
      }
    }
  }
  if (!kChunked || !p.state_packed) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int m = 0; m < SL; ++m)
        srow[(int64_t)(c0 + e) * p.ss_c + m * p.ss_k] = ns.e[e * SA + m];
  }
}

// ---------------------------------------------------------------- dispatch

template <typename D, int VEC>
static void launch_varlen(int W, const VarlenParams& p, uint32_t g, hipStream_t s) {
  switch (W) {
    case 1: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 1>), dim3(g), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 2>), dim3(g), dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 3>), dim3(g), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((varlen_fwd_kernel<D, VEC, 4>), dim3(g), dim3(256), 0, s, p); break;
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
  if (cache_seqlens)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: cache_seqlens (circular states) not supported", fn);
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
  const int vec16 = (int)(16 / es);
  const bool vec = dim % vec16 == 0 && x_stride_b % vec16 == 0 && out_stride_b % vec16 == 0 &&
                   aligned16(x) && aligned16(out);
  const int VEC = vec ? vec16 : 1;
  UpdateParams p;
  p.x = x; p.states = conv_states; p.w = weight; p.bias = bias; p.idx = conv_state_indices;
  p.out = out; p.x_rs = x_stride_b; p.ss_slot = st_stride_slot; p.ss_c = st_stride_c;
  p.ss_k = st_stride_k; p.w_sc = w_stride_c; p.w_sk = w_stride_k; p.out_rs = out_stride_b;
  p.nvec = cdiv(dim, VEC);
  p.batch = batch; p.dim = dim; p.silu = activation == SCONV_ACT_SILU;
  p.pad_slot_id = pad_slot_id;
  p.state_packed = st_stride_k == 1 && st_stride_c == W - 1 && aligned16(conv_states) &&
                   st_stride_slot % vec16 == 0;
  const int64_t threads_total = p.nvec * batch;
  const uint32_t th = threads_total >= 256 * 512 ? 256 : 64;
  const int64_t grid = cdiv(threads_total, th);
  if (grid > INT32_MAX) return fail(SCONV_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (dtype == SCONV_BF16) {
    if (vec) launch_update<Bf16, 8>(W, p, (uint32_t)grid, th, stream);
    else launch_update<Bf16, 1>(W, p, (uint32_t)grid, th, stream);
  } else {
    if (vec) launch_update<F32, 4>(W, p, (uint32_t)grid, th, stream);
    else launch_update<F32, 1>(W, p, (uint32_t)grid, th, stream);
  }
  return check_launch(fn);
}

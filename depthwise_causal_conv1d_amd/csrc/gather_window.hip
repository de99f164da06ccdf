// gather_window.hip -- conditional gather of each slot's length-d_conv input
// window, written transposed, with the live slot count read on the device.
//
// Source: Megatron-core page "core.ssm.ops.intermediate_extraction", module
// description and scatter_intermediate_conv: the grid is sized for the
// largest slot count when a graph is captured, each workgroup reads the real
// count from a fixed device address when it runs, and workgroups of dead
// slots leave before touching memory.  The window [pos - d_conv, pos) is
// clamped into the sequence and stored as (conv_dim, d_conv) per slot.
//
// Each lane owns VEC channels of one slot: it loads the d_conv source rows
// as 16-byte vectors and writes its VEC*d_conv output elements, which are
// contiguous in the transposed layout, as 16-byte chunks.
#include "sconv_device.h"
#include "sconv_host.h"

#ifndef SCONV_GATHER_LDS_STORES
#define SCONV_GATHER_LDS_STORES 1  // stores staged through LDS as 1 KB runs
#endif
#ifndef SCONV_GATHER_NT_STORES_LDS
#define SCONV_GATHER_NT_STORES_LDS 1  // streaming stores for the 1 KB runs
#endif
// Neighbouring slots' windows overlap, so source rows are read again
// through L2: streaming reads measured 25% slower (4.9 -> 6.1 us on the
// 512-slot spec-decode extraction).
#ifndef SCONV_GATHER_NT_LOADS
#define SCONV_GATHER_NT_LOADS 0  // streaming reads of the source rows
#endif


namespace sconv {

struct GatherParams {
  const void* src;
  const int32_t* pos;
  const int32_t* real_count;
  void* out;
  int64_t seq_len, src_ss, src_sc, out_ss;
  int32_t conv_dim, max_count, cblocks, out_chunked, threads;
};

template <typename D, int VEC, int DC>
__global__ __launch_bounds__(256) void gather_window_kernel(const GatherParams p) {
  using S = typename D::storage;
  const S* __restrict__ src = static_cast<const S*>(p.src);
  S* __restrict__ out = static_cast<S*>(p.out);
  const int slot = (int)blockIdx.y;  // grid: (channel blocks, max_count)
  const int cb = (int)blockIdx.x;
  // The live count and this slot's position are fetched together (slot <
  // max_count, so its entry is always readable): one round trip, not two.
  // Every kernel argument comes in the first scalar batch, and both values
  // are in registers before the early exit (else the position load would be
  // sunk below it).
  asm volatile("" ::"s"(p.src), "s"(p.out), "s"(p.seq_len), "s"(p.src_ss), "s"(p.out_ss),
               "s"(p.conv_dim), "s"(p.threads), "s"(p.max_count));
  int n = *p.real_count;
  const int64_t pend = p.pos[slot];
  asm volatile("" ::"v"(n), "v"(pend));
  n = n < 0 ? 0 : (n > p.max_count ? p.max_count : n);
  if (slot >= n) return;  // dead slot: no input or output traffic
  int c0 = (cb * p.threads + (int)threadIdx.x) * VEC;
  const bool lane_live = c0 < p.conv_dim;
#if SCONV_GATHER_LDS_STORES
  constexpr int kChunkE0 = 16 / (int)sizeof(S);
  constexpr bool kLdsPath = VEC > 1 && (VEC * DC) % kChunkE0 == 0;
#else
  constexpr bool kLdsPath = false;
#endif
  if constexpr (!kLdsPath) {
    if (!lane_live) return;
  } else {
    if (!lane_live) c0 = 0;  // loads a valid row; stores nothing
  }

  struct OutElems { S e[VEC * DC]; } oe;  // [c][k], k fastest
#pragma unroll
  for (int k = 0; k < DC; ++k) {
    int64_t row = pend - DC + k;
    row = row < 0 ? 0 : (row > p.seq_len - 1 ? p.seq_len - 1 : row);
    Pack<D, VEC> pk;
    if constexpr (VEC > 1) {
#if SCONV_GATHER_NT_LOADS
      pk.load_nt(src + row * p.src_ss + c0);
#else
      pk.load(src + row * p.src_ss + c0);
#endif
    } else {
      pk.raw = __builtin_bit_cast(typename Pack<D, 1>::raw_t, src[row * p.src_ss + (int64_t)c0 * p.src_sc]);
    }
    typename Pack<D, VEC>::Elems v = __builtin_bit_cast(typename Pack<D, VEC>::Elems, pk.raw);
#pragma unroll
    for (int e = 0; e < VEC; ++e) oe.e[e * DC + k] = v.e[e];
  }

  constexpr int kChunkE = 16 / (int)sizeof(S);
#if SCONV_GATHER_LDS_STORES
  if constexpr (kLdsPath) {
    if (p.out_chunked) {
      // The wave's output is one contiguous run of 64 * VEC * DC elements
      // (the lanes' channels are consecutive).  Each lane parks its VEC*DC
      // elements in LDS and reads back the 16-byte chunks it stores, so
      // every store instruction writes 1 KB of consecutive bytes.
      constexpr int kPer = VEC * DC / kChunkE;  // chunks per lane
      using Chunk = typename Pack<D, kChunkE>::raw_t;
      __shared__ Chunk lds[256 / 64][64 * kPer];
      Chunk* wl = lds[threadIdx.x >> 6];
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int ch = 0; ch < kPer; ++ch) {
        typename Pack<D, kChunkE>::Elems v;
#pragma unroll
        for (int q = 0; q < kChunkE; ++q) v.e[q] = oe.e[ch * kChunkE + q];
        wl[lane * kPer + ch] = __builtin_bit_cast(Chunk, v);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Live lanes are a prefix of the wave; so are their chunks.
      const int wave_c0 = (cb * p.threads + (int)(threadIdx.x & ~63)) * VEC;
      const int live = (p.conv_dim - wave_c0) / VEC;  // live lanes (may exceed 64)
      const int nchunks = (live < 64 ? live : 64) * kPer;
      S* wdst = out + (int64_t)slot * p.out_ss + (int64_t)wave_c0 * DC;
      Chunk back[kPer];  // read every chunk first (always in the LDS array), then store
#pragma unroll
      for (int r = 0; r < kPer; ++r) back[r] = wl[r * 64 + lane];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int idx = r * 64 + lane;
        if (idx < nchunks) {
          Pack<D, kChunkE> pk;
          pk.raw = back[r];
#if SCONV_GATHER_NT_STORES_LDS
          pk.store_nt(wdst + (int64_t)idx * kChunkE);
#else
          pk.store(wdst + (int64_t)idx * kChunkE);
#endif
        }
      }
      return;
    }
    if (!lane_live) return;
  }
#endif
  S* dst = out + (int64_t)slot * p.out_ss + (int64_t)c0 * DC;
  constexpr bool kChunked = (VEC * DC) % kChunkE == 0;
  if constexpr (kChunked) {
    if (p.out_chunked) {
#pragma unroll
      for (int ch = 0; ch < VEC * DC / kChunkE; ++ch) {
        typename Pack<D, kChunkE>::Elems v;
#pragma unroll
        for (int q = 0; q < kChunkE; ++q) v.e[q] = oe.e[ch * kChunkE + q];
        Pack<D, kChunkE> pk;
        pk.raw = __builtin_bit_cast(typename Pack<D, kChunkE>::raw_t, v);
        pk.store(dst + ch * kChunkE);
      }
      return;
    }
  }
#pragma unroll
  for (int q = 0; q < VEC * DC; ++q) dst[q] = oe.e[q];
}

template <typename D, int VEC>
static void launch_gather(int dc, const GatherParams& p, dim3 g, uint32_t th, hipStream_t s) {
  switch (dc) {
    case 1: hipLaunchKernelGGL((gather_window_kernel<D, VEC, 1>), g, dim3(th), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gather_window_kernel<D, VEC, 2>), g, dim3(th), 0, s, p); break;
    case 3: hipLaunchKernelGGL((gather_window_kernel<D, VEC, 3>), g, dim3(th), 0, s, p); break;
    default: hipLaunchKernelGGL((gather_window_kernel<D, VEC, 4>), g, dim3(th), 0, s, p); break;
  }
}

// ---------------------------------------------------------------- SSM-state rows

struct SsmGatherParams {
  const void* states;
  const int64_t* idx;
  const int32_t* real_count;
  void* out;
  int64_t states_rs, out_rs;  // row strides in units of T
  int64_t nvec;               // units of T per row
  int32_t max_count, threads;
};

// Measured on the 96-slot, 2 MiB-row extraction: 2 units per thread with
// streaming reads 67 us (6.0 TB/s); 4 units 71 us, 1 unit 69 us, ordinary
// reads 3-5% slower, 8 units 103 us.
#ifndef SCONV_SSM_GATHER_UNROLL
#define SCONV_SSM_GATHER_UNROLL 2  // units of T per thread
#endif
#ifndef SCONV_SSM_GATHER_NT_LOADS
#define SCONV_SSM_GATHER_NT_LOADS 1  // streaming reads of the source rows (read once)
#endif

// One workgroup per (column block, slot): the live count and the slot's
// source row are fetched in one round trip, dead slots leave at once, and
// live ones copy U units of T per thread (T = 16 bytes when the rows allow
// it), with streaming reads and stores.
template <typename T, int U>
__global__ __launch_bounds__(256) void gather_ssm_kernel(const SsmGatherParams p) {
  const int slot = (int)blockIdx.y;  // grid: (column blocks, max_count)
  asm volatile("" ::"s"(p.states), "s"(p.out), "s"(p.states_rs), "s"(p.out_rs), "s"(p.nvec),
               "s"(p.threads), "s"(p.max_count));
  int n = *p.real_count;
  const int64_t r = p.idx[slot];
  asm volatile("" ::"v"(n), "v"(r));
  n = n < 0 ? 0 : (n > p.max_count ? p.max_count : n);
  if (slot >= n) return;  // dead slot: no traffic
  const T* __restrict__ src = static_cast<const T*>(p.states) + r * p.states_rs;
  T* __restrict__ dst = static_cast<T*>(p.out) + (int64_t)slot * p.out_rs;
  const int64_t base = (int64_t)blockIdx.x * p.threads * U + threadIdx.x;
  T v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * p.threads;
#if SCONV_SSM_GATHER_NT_LOADS
    if (i < p.nvec) v[u] = __builtin_nontemporal_load(src + i);
#else
    if (i < p.nvec) v[u] = src[i];
#endif
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * p.threads;
    if (i < p.nvec) __builtin_nontemporal_store(v[u], dst + i);
  }
}

template <typename T>
static void launch_ssm(const SsmGatherParams& p, hipStream_t s) {
  constexpr int U = SCONV_SSM_GATHER_UNROLL;
  const dim3 grid((uint32_t)cdiv(p.nvec, (int64_t)p.threads * U), (uint32_t)p.max_count);
  hipLaunchKernelGGL((gather_ssm_kernel<T, U>), grid, dim3(p.threads), 0, s, p);
}

}  // namespace sconv

extern "C" int gather_intermediate_ssm_state(const void* states, int64_t num_chunks,
                                             int64_t state_flat, int64_t states_row_stride,
                                             const int64_t* chunk_indices,
                                             const int32_t* real_count_dev, int32_t max_count,
                                             void* out, int64_t out_row_stride, int32_t dtype,
                                             hipStream_t stream) {
  using namespace sconv;
  clear_error();
  const char* fn = "gather_intermediate_ssm_state";
  if (!valid_dtype(dtype)) return fail(SCONV_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (num_chunks < 1) return fail(SCONV_ERR_INVALID, "%s: num_chunks < 1", fn);
  if (state_flat < 0 || max_count < 0)
    return fail(SCONV_ERR_INVALID, "%s: state_flat and max_count must be >= 0", fn);
  if (max_count > 65535)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: max_count above 65535 (one grid row per slot)", fn);
  if (states_row_stride < state_flat || out_row_stride < state_flat)
    return fail(SCONV_ERR_INVALID, "%s: row strides smaller than state_flat", fn);
  if (state_flat == 0 || max_count == 0) return SCONV_OK;
  if (!states || !chunk_indices || !real_count_dev || !out)
    return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
  const int64_t es = elem_size(dtype);
  const int64_t s_bytes = ((num_chunks - 1) * states_row_stride + state_flat) * es;
  const int64_t o_bytes = ((int64_t)(max_count - 1) * out_row_stride + state_flat) * es;
  if (overlap(out, o_bytes, states, s_bytes))
    return fail(SCONV_ERR_INVALID, "%s: out overlaps states", fn);
  SsmGatherParams p;
  p.states = states; p.idx = chunk_indices; p.real_count = real_count_dev; p.out = out;
  p.max_count = max_count;
  p.threads = 256;
  const bool vec = (state_flat * es) % 16 == 0 && (states_row_stride * es) % 16 == 0 &&
                   (out_row_stride * es) % 16 == 0 && aligned16(states) && aligned16(out);
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  if (vec) {
    const int64_t per = 16 / es;
    p.nvec = state_flat / per; p.states_rs = states_row_stride / per;
    p.out_rs = out_row_stride / per;
    launch_ssm<u4>(p, stream);
  } else {
    p.nvec = state_flat; p.states_rs = states_row_stride; p.out_rs = out_row_stride;
    if (es == 2) launch_ssm<uint16_t>(p, stream);
    else launch_ssm<uint32_t>(p, stream);
  }
  return check_launch(fn);
}

extern "C" int gather_intermediate_conv_window(const void* src, int64_t seq_len,
                                               int32_t conv_dim, int64_t src_stride_s,
                                               int64_t src_stride_c,
                                               const int32_t* abs_positions,
                                               const int32_t* real_count_dev, int32_t max_count,
                                               void* out, int64_t out_slot_stride,
                                               int32_t d_conv, int32_t dtype,
                                               hipStream_t stream) {
  using namespace sconv;
  clear_error();
  const char* fn = "gather_intermediate_conv_window";
  if (!valid_dtype(dtype)) return fail(SCONV_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (seq_len < 1) return fail(SCONV_ERR_INVALID, "%s: seq_len < 1", fn);
  if (conv_dim < 0 || max_count < 0)
    return fail(SCONV_ERR_INVALID, "%s: conv_dim and max_count must be >= 0", fn);
  if (d_conv < 1 || d_conv > 4)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: d_conv=%d outside [1, 4]", fn, d_conv);
  if (max_count > 65535)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: max_count above 65535 (one grid row per slot)", fn);
  if (conv_dim == 0 || max_count == 0) return SCONV_OK;
  if (!src || !abs_positions || !real_count_dev || !out)
    return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
  if (src_stride_s < 1 || src_stride_c < 1 || out_slot_stride < (int64_t)conv_dim * d_conv)
    return fail(SCONV_ERR_INVALID, "%s: strides too small", fn);
  const int64_t es = elem_size(dtype);
  const int vec16 = (int)(16 / es);
  const bool vec = src_stride_c == 1 && conv_dim % vec16 == 0 && src_stride_s % vec16 == 0 &&
                   aligned16(src);
  const int VEC = vec ? vec16 : 1;
  GatherParams p;
  p.src = src; p.pos = abs_positions; p.real_count = real_count_dev; p.out = out;
  p.seq_len = seq_len; p.src_ss = src_stride_s; p.src_sc = src_stride_c;
  p.out_ss = out_slot_stride; p.conv_dim = conv_dim; p.max_count = max_count;
  p.out_chunked = aligned16(out) && out_slot_stride % vec16 == 0 && vec;
  const uint32_t th = (int64_t)conv_dim >= 256 * VEC ? 256 : 64;
  p.cblocks = (int32_t)cdiv(conv_dim, (int64_t)th * VEC);
  p.threads = (int32_t)th;
  const dim3 grid((uint32_t)p.cblocks, (uint32_t)max_count);
  if (dtype == SCONV_BF16) {
    if (vec) launch_gather<Bf16, 8>(d_conv, p, grid, th, stream);
    else launch_gather<Bf16, 1>(d_conv, p, grid, th, stream);
  } else {
    if (vec) launch_gather<F32, 4>(d_conv, p, grid, th, stream);
    else launch_gather<F32, 1>(d_conv, p, grid, th, stream);
  }
  return check_launch(fn);
}

// gather_window.hip -- conditional gathers with the live slot count read on
// the device: length-d_conv input windows written transposed (the body is
// in gather_window.h), and whole SSM-state rows.
//
// Source: Megatron-core page "core.ssm.ops.intermediate_extraction", module
// description, scatter_intermediate_conv and scatter_intermediate_ssm.
#include "gather_window.h"

namespace sconv {

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
#ifndef SCONV_SSM_GATHER_EXTRA_LDS
#define SCONV_SSM_GATHER_EXTRA_LDS 0  // unused dynamic LDS bytes per workgroup (fewer per CU)
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
  hipLaunchKernelGGL((gather_ssm_kernel<T, U>), grid, dim3(p.threads), SCONV_SSM_GATHER_EXTRA_LDS, s, p);
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

namespace sconv {

int gather_window_setup(const char* fn, const void* src, int64_t seq_len, int32_t conv_dim,
                        int64_t src_stride_s, int64_t src_stride_c,
                        const int32_t* abs_positions, const int32_t* real_count_dev,
                        int32_t max_count, void* out, int64_t out_slot_stride, int32_t d_conv,
                        int32_t dtype, uint32_t threads, GatherParams* p, int* vec_out,
                        bool* empty) {
  *empty = true;
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
  p->src = src; p->pos = abs_positions; p->real_count = real_count_dev; p->out = out;
  p->seq_len = seq_len; p->src_ss = src_stride_s; p->src_sc = src_stride_c;
  p->out_ss = out_slot_stride; p->conv_dim = conv_dim; p->max_count = max_count;
  p->out_chunked = aligned16(out) && out_slot_stride % vec16 == 0 && vec;
  const uint32_t th = threads ? threads : ((int64_t)conv_dim >= 256 * VEC ? 256 : 64);
  p->cblocks = (int32_t)cdiv(conv_dim, (int64_t)th * VEC);
  p->threads = (int32_t)th;
  *vec_out = VEC;
  *empty = false;
  return SCONV_OK;
}

void gather_window_launch(const GatherParams& p, int vec, int d_conv, int32_t dtype,
                          hipStream_t stream) {
  const dim3 grid((uint32_t)p.cblocks, (uint32_t)p.max_count);
  const uint32_t th = (uint32_t)p.threads;
  if (dtype == SCONV_BF16) {
    if (vec > 1) launch_gather<Bf16, 8>(d_conv, p, grid, th, stream);
    else launch_gather<Bf16, 1>(d_conv, p, grid, th, stream);
  } else {
    if (vec > 1) launch_gather<F32, 4>(d_conv, p, grid, th, stream);
    else launch_gather<F32, 1>(d_conv, p, grid, th, stream);
  }
}

}  // namespace sconv

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
  GatherParams p;
  int vec = 1;
  bool empty = true;
  const int rc = gather_window_setup(fn, src, seq_len, conv_dim, src_stride_s, src_stride_c,
                                     abs_positions, real_count_dev, max_count, out,
                                     out_slot_stride, d_conv, dtype, 0, &p, &vec, &empty);
  if (rc != SCONV_OK || empty) return rc;
  gather_window_launch(p, vec, d_conv, dtype, stream);
  return check_launch(fn);
}

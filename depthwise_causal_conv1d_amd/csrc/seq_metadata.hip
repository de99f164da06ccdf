// seq_metadata.hip -- per-token request index and request start row.
//
// Source: vLLM page "vllm.models.inkling.nvidia.ops.sconv", function
// sconv_seq_metadata.  One launch fills both static per-token buffers that
// the fused conv reads, in place of a search / clamp / gather / copy chain.
//
// Each thread owns one row.  The request offsets are staged once per
// workgroup in LDS when they fit (they usually do: a few KB), and the
// request is found by a binary search for the last offset <= row, which
// skips empty requests and clamps rows past the end to the last request.
#include "sconv_device.h"
#include "sconv_host.h"

namespace sconv {

constexpr int kMetaBlock = 256;
constexpr int kMetaLdsMax = 8192;  // offsets staged in LDS (32 KB)

__global__ __launch_bounds__(kMetaBlock) void seq_metadata_kernel(
    const int32_t* __restrict__ qsl, int32_t num_reqs, int64_t num_actual,
    int64_t num_padded, int32_t* __restrict__ seq_idx, int32_t* __restrict__ query_start) {
  __shared__ int32_t s_qsl[kMetaLdsMax];
  const int64_t row0 = (int64_t)blockIdx.x * kMetaBlock;
  const int64_t t = row0 + threadIdx.x;
  // Stage only if this workgroup has a real row to search for.
  const bool staged = (num_reqs < kMetaLdsMax) && (row0 < num_actual);
  if (staged) {
    for (int i = threadIdx.x; i < num_reqs; i += kMetaBlock) s_qsl[i] = qsl[i];
    __syncthreads();
  }
  if (t >= num_padded) return;
  int32_t r = 0, q = 0;
  if (t < num_actual) {
    // Largest r in [0, num_reqs) with qsl[r] <= t (r = 0 if none).
    int32_t lo = 0, hi = num_reqs;
    if (staged) {
      while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if ((int64_t)s_qsl[mid] <= t) lo = mid; else hi = mid;
      }
      q = s_qsl[lo];
    } else {
      while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if ((int64_t)qsl[mid] <= t) lo = mid; else hi = mid;
      }
      q = qsl[lo];
    }
    r = lo;
  }
  seq_idx[t] = r;
  query_start[t] = q;
}

}  // namespace sconv

extern "C" int sconv_seq_metadata(const int32_t* query_start_loc, int32_t num_reqs,
                                  int64_t num_actual_tokens, int64_t num_padded_tokens,
                                  int32_t* seq_idx_out, int64_t seq_idx_len,
                                  int32_t* query_start_out, int64_t query_start_len,
                                  hipStream_t stream) {
  using namespace sconv;
  clear_error();
  if (num_actual_tokens < 0)
    return fail(SCONV_ERR_INVALID, "sconv_seq_metadata: num_actual_tokens < 0");
  if (num_padded_tokens < num_actual_tokens)
    return fail(SCONV_ERR_INVALID,
                "sconv_seq_metadata: num_padded_tokens (%lld) is below num_actual_tokens (%lld)",
                (long long)num_padded_tokens, (long long)num_actual_tokens);
  if (num_padded_tokens > seq_idx_len)
    return fail(SCONV_ERR_INVALID,
                "sconv_seq_metadata: seq_idx_out holds %lld entries, %lld rows requested",
                (long long)seq_idx_len, (long long)num_padded_tokens);
  if (num_padded_tokens > query_start_len)
    return fail(SCONV_ERR_INVALID,
                "sconv_seq_metadata: query_start_out holds %lld entries, %lld rows requested",
                (long long)query_start_len, (long long)num_padded_tokens);
  if (num_actual_tokens > 0 && num_reqs < 1)
    return fail(SCONV_ERR_INVALID, "sconv_seq_metadata: num_reqs < 1 with actual tokens");
  if (num_padded_tokens == 0) return SCONV_OK;
  if (!seq_idx_out || !query_start_out || (num_actual_tokens > 0 && !query_start_loc))
    return fail(SCONV_ERR_INVALID, "sconv_seq_metadata: NULL pointer");
  const int64_t blocks = cdiv(num_padded_tokens, kMetaBlock);
  if (blocks > INT32_MAX)
    return fail(SCONV_ERR_UNSUPPORTED, "sconv_seq_metadata: too many tokens");
  hipLaunchKernelGGL(seq_metadata_kernel, dim3((uint32_t)blocks), dim3(kMetaBlock), 0, stream,
                     query_start_loc, num_reqs, num_actual_tokens, num_padded_tokens,
                     seq_idx_out, query_start_out);
  return check_launch("sconv_seq_metadata");
}

// Load the library's GPU code on the current device.  Launches otherwise
// load it on first use; a caller that captures its first call into a
// hipGraph calls this beforehand so that nothing but the launch itself
// happens inside the capture.  Asking for a kernel's attributes loads the
// code object holding every kernel of the library.
extern "C" int sconv_init(void) {
  sconv::clear_error();
  hipFuncAttributes attr;
  const hipError_t e =
      hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&sconv::seq_metadata_kernel));
  if (e != hipSuccess)
    return sconv::fail(SCONV_ERR_HIP, "sconv_init: %s", hipGetErrorString(e));
  return SCONV_OK;
}

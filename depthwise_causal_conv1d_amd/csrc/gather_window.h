// gather_window.h -- the conditional window gather's device body and host
// set-up, shared by its own entry point and by the fused launch that runs
// it in the same grid as the conv.
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
#pragma once

#include "sconv_device.h"
#include "sconv_host.h"

#ifndef SCONV_GATHER_LDS_STORES
#define SCONV_GATHER_LDS_STORES 1  // stores staged through LDS as 1 KB runs
#endif
#ifndef SCONV_GATHER_NT_STORES_LDS
#define SCONV_GATHER_NT_STORES_LDS 1  // streaming stores for the 1 KB runs
#endif
// Neighbouring slots' windows overlap, so source rows are read again
// through L2: in the gather's own launch streaming reads measured slower
// (5.14 -> 6.42 us with all 512 slots of the spec-decode extraction live).
// Inside the conv's launch they measured faster (15.90 -> 15.73 us per
// speculative step): there the conv's streaming input reads have already
// passed the rows by.
#ifndef SCONV_GATHER_NT_LOADS
#define SCONV_GATHER_NT_LOADS 0  // streaming reads of the source rows (own launch)
#endif
#ifndef SCONV_FUSED_GATHER_NT_LOADS
#define SCONV_FUSED_GATHER_NT_LOADS 1  // the same, in the conv's launch
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

// Checked host set-up of one gather: parameters for workgroups of `threads`
// (0: the gather's own choice) and lane width VEC (16 bytes, or 1 element).
// Returns SCONV_OK, an error status, or SCONV_OK with *empty set when there
// is nothing to launch.
int gather_window_setup(const char* fn, const void* src, int64_t seq_len, int32_t conv_dim,
                        int64_t src_stride_s, int64_t src_stride_c,
                        const int32_t* abs_positions, const int32_t* real_count_dev,
                        int32_t max_count, void* out, int64_t out_slot_stride, int32_t d_conv,
                        int32_t dtype, uint32_t threads, GatherParams* p, int* vec, bool* empty);

// Enqueue the gather's own kernel for a set-up from gather_window_setup.
void gather_window_launch(const GatherParams& p, int vec, int d_conv, int32_t dtype,
                          hipStream_t stream);




// LDS a gather workgroup stages its stores in: per wave, 64 lanes x up to
// four 16-byte chunks (bf16 lanes of 8 channels x d_conv <= 4 taps).  One
// array serves every d_conv, so a kernel holding several bodies reserves it
// once: kGatherLdsWave chunks per wave of the workgroup.
typedef uint32_t GatherChunk __attribute__((ext_vector_type(4)));
constexpr int kGatherLdsWave = 64 * 4;
constexpr int kGatherLdsChunks = (256 / 64) * kGatherLdsWave;  // the gather's own 256-thread groups

// The gather of one (channel block, slot) workgroup, staging through `lds`
// (kGatherLdsWave chunks for each of its waves).  It uses neither
// workgroup barriers nor the grid shape, so a larger kernel can run it in
// some of its workgroups.
// NTL: source rows loaded as streaming reads.
template <typename D, int VEC, int DC, bool NTL = SCONV_GATHER_NT_LOADS>
__device__ __forceinline__ void gather_window_body(const GatherParams& p, int slot, int cb,
                                                   GatherChunk* lds) {
  using S = typename D::storage;
  const S* __restrict__ src = static_cast<const S*>(p.src);
  S* __restrict__ out = static_cast<S*>(p.out);
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
      if constexpr (NTL) pk.load_nt(src + row * p.src_ss + c0);
      else pk.load(src + row * p.src_ss + c0);
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
      static_assert(sizeof(Chunk) == sizeof(GatherChunk) && kPer <= 4, "LDS staging layout");
      Chunk* wl = reinterpret_cast<Chunk*>(lds) + (threadIdx.x >> 6) * kGatherLdsWave;
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

template <typename D, int VEC, int DC>
__global__ __launch_bounds__(256) void gather_window_kernel(const GatherParams p) {
  __shared__ GatherChunk lds[kGatherLdsChunks];
  // grid: (channel blocks, max_count)
  gather_window_body<D, VEC, DC>(p, (int)blockIdx.y, (int)blockIdx.x, lds);
}

}  // namespace sconv

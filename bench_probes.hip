// bench_probes.hip -- reference kernels that measure what one MI355X can do
// for the memory patterns of the short-convolution kernels, so that their
// timings can be read against the machine rather than against the nominal
// 8 TB/s alone.  Measurement only: nothing in libsconv uses them, and they
// compute nothing of the convolution.
//
// Streaming ceilings (bytes moved linearly, 16 bytes per lane, streaming
// loads; each workgroup of 256 threads owns `per` consecutive vectors, and a
// lane handles U of them per pass (1, 2 or 4, all of a pass's loads issued
// before its stores); stores streaming or ordinary):
//   probe_read        read n vectors
//   probe_write       write n vectors
//   probe_copy        read n, write n
//   probe_read_write2 read n, write n linearly and n more in pieces of
//                     `piece` bytes at a stride of `row` bytes (piece == row:
//                     linear).  The fused prefill moves its bytes this way:
//                     x read linearly, out written linearly, and each
//                     stream's cache inserts as ws-column pieces of every
//                     head's D-column cache row.
// The best shape differs by pattern and size, so a ceiling is the best of
// several (u, per, store form, occupancy) runs; occupancy is lowered by
// `lds` bytes of dynamic LDS per workgroup, which the kernels do not use.
//   probe_prefill_layout  the mixed prefill's own traffic: one 1 KiB slab of
//                     one 8 KiB x row per wave, read, written to out and, as
//                     four 256-byte pieces, to the [blocks, 32, 16, 512]
//                     cache, in slab-major order with each XCD on one
//                     contiguous range of workgroups; optionally with the
//                     conv's other loads: 3 halo rows (x rows of the
//                     previous waves) and 4 filter-tap vectors per lane.
// Latency floors at the decode launch shape (one wave per workgroup):
//   probe_empty       an empty kernel
//   probe_load_store  one 16-byte load per lane, then its store
//   probe_chain       dependent loads, then a store: optionally a per-wave
//                     metadata word, then a 256-entry table row (as the
//                     decode kernel reads its block-table row), then
//                     `pieces` loads in the decode kernel's history-tap
//                     pattern from the block the row names; `pieces` = 0
//                     stops after the row.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4 v, u32x4* p) { __builtin_nontemporal_store(v, p); }

template <bool NT>
__device__ __forceinline__ void st(u32x4 v, u32x4* p) {
  if constexpr (NT) st_nt(v, p);
  else *p = v;
}

// Workgroup g owns vectors [g*per, min((g+1)*per, n)); a pass of a lane
// takes U vectors at a stride of the workgroup size.
template <int U>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* src, int64_t n, int64_t per,
                                                        u32x4* sink, int flag) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = a + threadIdx.x; i < b; i += (int64_t)U * kThreads) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t k = i + (int64_t)j * kThreads;
      if (k < b) acc ^= ld_nt(src + k);
    }
  }
  if (flag) sink[threadIdx.x] = acc;  // flag is 0: keeps the loads
}

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* dst, int64_t n, int64_t per) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  const u32x4 v = {blockIdx.x, threadIdx.x, 1u, 2u};
  for (int64_t i = a + threadIdx.x; i < b; i += (int64_t)U * kThreads) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t k = i + (int64_t)j * kThreads;
      if (k < b) st<NT>(v, dst + k);
    }
  }
}

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* src, u32x4* dst, int64_t n,
                                                        int64_t per) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  for (int64_t i = a + threadIdx.x; i < b; i += (int64_t)U * kThreads) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t k = i + (int64_t)j * kThreads;
      v[j] = k < b ? ld_nt(src + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t k = i + (int64_t)j * kThreads;
      if (k < b) st<NT>(v[j], dst + k);
    }
  }
}

// Vector k of the second write goes to piece k / pv (pv vectors per piece)
// at row stride rv vectors: offset (k / pv) * rv + k % pv.
template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void read_write2_kernel(const u32x4* src, u32x4* dst_a,
                                                               u32x4* dst_b, int64_t n,
                                                               int64_t per, int32_t pv,
                                                               int32_t rv) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  for (int64_t i = a + threadIdx.x; i < b; i += (int64_t)U * kThreads) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t k = i + (int64_t)j * kThreads;
      v[j] = k < b ? ld_nt(src + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t k = i + (int64_t)j * kThreads;
      if (k < b) {
        st<NT>(v[j], dst_a + k);
        st<NT>(v[j], dst_b + (k / pv) * rv + k % pv);
      }
    }
  }
}

// The mixed prefill's traffic (one stream launch, C = 4096 bf16: 8 slabs of
// 1 KiB per 8 KiB x row; cache [T/16 blocks][32 heads][16 slots][1 KiB],
// slot t for row t).  Workgroup = 4 waves = 4 consecutive rows of one
// slab; workgroups slab-major, renumbered so that XCD x (blockIdx % 8)
// runs the x-th eighth of them.  The grid is a multiple of 8.
template <int HALO, int WTS>
__global__ __launch_bounds__(kThreads) void prefill_layout_kernel(const u32x4* __restrict__ x,
                                                                  const u32x4* __restrict__ w,
                                                                  u32x4* __restrict__ out,
                                                                  u32x4* __restrict__ cache,
                                                                  int32_t T, int32_t ntiles) {
  const uint32_t G = gridDim.x;
  const uint32_t wg = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int32_t slab = (int32_t)(wg / (uint32_t)ntiles), tile = (int32_t)(wg % (uint32_t)ntiles);
  const int32_t t = tile * 4 + (int32_t)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t col = slab * 64 + lane;
  const u32x4 v = x[(int64_t)t * 512 + col];
  u32x4 acc = v;
#pragma unroll
  for (int m = 1; m <= HALO; ++m) acc ^= x[(int64_t)(t - m >= 0 ? t - m : 0) * 512 + col];
#pragma unroll
  for (int k = 0; k < WTS; ++k) acc ^= w[col * 4 + k];
  st_nt(acc, out + (int64_t)t * 512 + col);
  const int64_t head = slab * 4 + (lane >> 4);
  st_nt(v, cache + (((int64_t)(t >> 4) * 32 + head) * 16 + (t & 15)) * 64 + (lane & 15));
}

__global__ void empty_kernel() {}

// Wave w (one per workgroup) loads 64 x 16 bytes at src + w*64 and stores
// them at dst + w*64.
__global__ __launch_bounds__(64) void load_store_kernel(const u32x4* src, u32x4* dst) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  dst[i] = src[i];
}

// Wave w: meta[w] (a row index) -> that row of `table` (256 int32 entries,
// four per lane, as the decode kernel reads its block-table row) -> the
// block named by the row's entry 0 (entries 64, 128 and 192 are 0 by the
// caller's contract, so the XOR below is entry 0) -> `pieces` loads laid out
// as the decode kernel's history taps: lane L reads 16 bytes at block *
// 8192 + (L/4)*256 + p*16 + L%4 vectors, i.e. 16 pieces of 64 bytes at a
// 4 KiB stride, piece p one 256-byte row further -> store at dst + w*64.
// With meta NULL the row is row0 + w, known without a load (the decode
// kernel reads its block-table row alongside its metadata).
__global__ __launch_bounds__(64) void chain_kernel(const int32_t* meta, int32_t row0,
                                                   const int32_t* table, const u32x4* data,
                                                   u32x4* dst, int pieces) {
  const int w = blockIdx.x, lane = threadIdx.x;
  const int32_t row = meta ? __builtin_amdgcn_readfirstlane(meta[w]) : row0 + w;
  const int32_t* r = table + (int64_t)row * 256;
  int32_t e0 = r[lane], e1 = r[64 + lane], e2 = r[128 + lane], e3 = r[192 + lane];
  u32x4 acc = {(uint32_t)e0, (uint32_t)e1, (uint32_t)e2, (uint32_t)e3};
  const int32_t blk = __builtin_amdgcn_readfirstlane(e0 ^ e1 ^ e2 ^ e3);
  const int64_t at = (int64_t)blk * 8192 + (lane >> 2) * 256 + (lane & 3);
  for (int p = 0; p < pieces; ++p) acc ^= __builtin_nontemporal_load(data + at + p * 16);
  dst[(int64_t)w * 64 + lane] = acc;
}

// Workgroups for n vectors at `per` each; 0 when the shape is not one the
// kernels are built for.
int grid_for(int64_t n, int64_t per, int32_t u) {
  if (n < 1 || per < 1 || !(u == 1 || u == 2 || u == 4)) return 0;
  const int64_t g = (n + per - 1) / per;
  return g <= 0x7fffffff ? (int)g : 0;
}

}  // namespace

extern "C" {

// Instantiations by lane depth and store form.
#define BY_SHAPE(NT_, LAUNCH)                       \
  if (u == 1 && (NT_) == 1) { LAUNCH(1, true) }     \
  else if (u == 1) { LAUNCH(1, false) }             \
  else if (u == 2 && (NT_) == 1) { LAUNCH(2, true) } \
  else if (u == 2) { LAUNCH(2, false) }             \
  else if ((NT_) == 1) { LAUNCH(4, true) }          \
  else { LAUNCH(4, false) }

// Every streaming probe: n16 vectors of 16 bytes; each workgroup of 256
// threads owns per16 of them; u (1, 2 or 4) vectors per lane and pass; nt
// selects streaming (1) or ordinary (0) stores; lds bytes of dynamic LDS
// per workgroup (0 up to 160 KiB) limit how many workgroups share a CU.
// Returns -1 for a shape outside these, else the launch status.

// sink holds 256 vectors (never written).
int probe_read(const void* src, int64_t n16, void* sink, int64_t per16, int32_t u,
               uint32_t lds, hipStream_t s) {
  const int g = grid_for(n16, per16, u);
  if (!g) return -1;
  if (u == 1) hipLaunchKernelGGL(read_kernel<1>, dim3(g), dim3(kThreads), lds, s, (const u32x4*)src, n16, per16, (u32x4*)sink, 0);
  else if (u == 2) hipLaunchKernelGGL(read_kernel<2>, dim3(g), dim3(kThreads), lds, s, (const u32x4*)src, n16, per16, (u32x4*)sink, 0);
  else hipLaunchKernelGGL(read_kernel<4>, dim3(g), dim3(kThreads), lds, s, (const u32x4*)src, n16, per16, (u32x4*)sink, 0);
  return (int)hipGetLastError();
}

int probe_write(void* dst, int64_t n16, int64_t per16, int32_t u, int32_t nt, uint32_t lds,
                hipStream_t s) {
  const int g = grid_for(n16, per16, u);
  if (!g) return -1;
#define L_(U, NT) hipLaunchKernelGGL((write_kernel<U, NT>), dim3(g), dim3(kThreads), lds, s, (u32x4*)dst, n16, per16);
  BY_SHAPE(nt, L_)
#undef L_
  return (int)hipGetLastError();
}

int probe_copy(const void* src, void* dst, int64_t n16, int64_t per16, int32_t u, int32_t nt,
               uint32_t lds, hipStream_t s) {
  const int g = grid_for(n16, per16, u);
  if (!g) return -1;
#define L_(U, NT) hipLaunchKernelGGL((copy_kernel<U, NT>), dim3(g), dim3(kThreads), lds, s, (const u32x4*)src, (u32x4*)dst, n16, per16);
  BY_SHAPE(nt, L_)
#undef L_
  return (int)hipGetLastError();
}

// dst_b must hold (n16 / (piece/16)) * (row/16) vectors; piece and row are
// multiples of 16 bytes with piece <= row, and n16 a multiple of piece/16.
int probe_read_write2(const void* src, void* dst_a, void* dst_b, int64_t n16, int32_t piece,
                      int32_t row, int64_t per16, int32_t u, int32_t nt, uint32_t lds,
                      hipStream_t s) {
  if (piece < 16 || row < piece || piece % 16 || row % 16 || n16 % (piece / 16)) return -1;
  const int g = grid_for(n16, per16, u);
  if (!g) return -1;
  const int32_t pv = piece / 16, rv = row / 16;
#define L_(U, NT) hipLaunchKernelGGL((read_write2_kernel<U, NT>), dim3(g), dim3(kThreads), lds, s, (const u32x4*)src, (u32x4*)dst_a, (u32x4*)dst_b, n16, per16, pv, rv);
  BY_SHAPE(nt, L_)
#undef L_
  return (int)hipGetLastError();
}

// x and out hold T * 512 vectors, cache T * 2048, w 2048; T a positive
// multiple of 16; halo 0 or 3, wts 0 or 4.
int probe_prefill_layout(const void* x, const void* w, void* out, void* cache, int32_t T,
                         int32_t halo, int32_t wts, uint32_t lds, hipStream_t s) {
  if (T < 16 || T % 16 || (halo != 0 && halo != 3) || (wts != 0 && wts != 4)) return -1;
  const int32_t ntiles = T / 4;
  const dim3 g((uint32_t)ntiles * 8), b(kThreads);
#define L_(H, K)                                                                          \
  hipLaunchKernelGGL((prefill_layout_kernel<H, K>), g, b, lds, s, (const u32x4*)x,        \
                     (const u32x4*)w, (u32x4*)out, (u32x4*)cache, T, ntiles);
  if (halo == 0 && wts == 0) { L_(0, 0) }
  else if (halo == 0) { L_(0, 4) }
  else if (wts == 0) { L_(3, 0) }
  else { L_(3, 4) }
#undef L_
  return (int)hipGetLastError();
}

int probe_empty(int32_t waves, hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(waves), dim3(64), 0, s);
  return (int)hipGetLastError();
}

// src and dst hold waves * 64 vectors each.
int probe_load_store(const void* src, void* dst, int32_t waves, hipStream_t s) {
  hipLaunchKernelGGL(load_store_kernel, dim3(waves), dim3(64), 0, s, (const u32x4*)src,
                     (u32x4*)dst);
  return (int)hipGetLastError();
}

// meta (or NULL: rows row0 .. row0 + waves - 1) holds `waves` row indices
// into table (rows of 256 entries); entry 0 of each row names a block of
// data (8192 vectors each) and its entries 64, 128 and 192 are 0;
// pieces <= 16; dst holds waves * 64 vectors.
int probe_chain(const void* meta, int32_t row0, const void* table, const void* data,
                void* dst, int32_t waves, int32_t pieces, hipStream_t s) {
  if (pieces < 0 || pieces > 16) return -1;
  hipLaunchKernelGGL(chain_kernel, dim3(waves), dim3(64), 0, s, (const int32_t*)meta, row0,
                     (const int32_t*)table, (const u32x4*)data, (u32x4*)dst, pieces);
  return (int)hipGetLastError();
}

}  // extern "C"

// bench_probes.hip -- reference kernels that measure what one MI355X can do
// for the memory patterns of the short-convolution kernels, so that their
// timings can be read against the machine rather than against the nominal
// 8 TB/s alone.  Measurement only: nothing in libsconv uses them, and they
// compute nothing of the convolution.
//
// Streaming ceilings (bytes moved linearly, 16 bytes per lane, streaming
// loads and stores, 32768 workgroups of 256 threads by default):
//   probe_read        read n vectors
//   probe_write       write n vectors
//   probe_copy        read n, write n
//   probe_read_write2 read n, write n linearly and n more in pieces of
//                     `piece` bytes at a stride of `row` bytes (piece == row:
//                     linear).  The fused prefill moves its bytes this way:
//                     x read linearly, out written linearly, and each
//                     stream's cache inserts as ws-column pieces of every
//                     head's D-column cache row.
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

// Workgroup g owns vectors [g*per, min((g+1)*per, n)); lanes stride by the
// workgroup size, two vectors in flight per lane.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* src, int64_t n, int64_t per,
                                                        u32x4* sink, int flag) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = a + threadIdx.x; i < b; i += 2 * kThreads) {
    const u32x4 v0 = ld_nt(src + i);
    const u32x4 v1 = i + kThreads < b ? ld_nt(src + i + kThreads) : u32x4{0, 0, 0, 0};
    acc ^= v0 ^ v1;
  }
  if (flag) sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;  // flag is 0: keeps the loads
}

__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* dst, int64_t n, int64_t per) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  const u32x4 v = {blockIdx.x, threadIdx.x, 1u, 2u};
  for (int64_t i = a + threadIdx.x; i < b; i += kThreads) st_nt(v, dst + i);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* src, u32x4* dst, int64_t n,
                                                        int64_t per) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  for (int64_t i = a + threadIdx.x; i < b; i += 2 * kThreads) {
    const u32x4 v0 = ld_nt(src + i);
    const bool two = i + kThreads < b;
    const u32x4 v1 = two ? ld_nt(src + i + kThreads) : u32x4{0, 0, 0, 0};
    st_nt(v0, dst + i);
    if (two) st_nt(v1, dst + i + kThreads);
  }
}

// Vector i of the second write goes to piece i / pv (pv vectors per piece)
// at row stride rv vectors: offset (i / pv) * rv + i % pv.
__global__ __launch_bounds__(kThreads) void read_write2_kernel(const u32x4* src, u32x4* dst_a,
                                                               u32x4* dst_b, int64_t n,
                                                               int64_t per, int32_t pv,
                                                               int32_t rv) {
  const int64_t a = (int64_t)blockIdx.x * per, b = a + per < n ? a + per : n;
  for (int64_t i = a + threadIdx.x; i < b; i += 2 * kThreads) {
    const u32x4 v0 = ld_nt(src + i);
    const bool two = i + kThreads < b;
    const u32x4 v1 = two ? ld_nt(src + i + kThreads) : u32x4{0, 0, 0, 0};
    st_nt(v0, dst_a + i);
    st_nt(v0, dst_b + (i / pv) * rv + i % pv);
    if (two) {
      const int64_t k = i + kThreads;
      st_nt(v1, dst_a + k);
      st_nt(v1, dst_b + (k / pv) * rv + k % pv);
    }
  }
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

int grid_for(int64_t n, int64_t groups, int64_t* per) {
  *per = (n + groups - 1) / groups;
  if (*per < 1) *per = 1;
  return (int)((n + *per - 1) / *per);
}

}  // namespace

extern "C" {

int probe_read(const void* src, int64_t n16, void* sink, int32_t groups, hipStream_t s) {
  int64_t per;
  const int g = grid_for(n16, groups, &per);
  hipLaunchKernelGGL(read_kernel, dim3(g), dim3(kThreads), 0, s, (const u32x4*)src, n16, per,
                     (u32x4*)sink, 0);
  return (int)hipGetLastError();
}

int probe_write(void* dst, int64_t n16, int32_t groups, hipStream_t s) {
  int64_t per;
  const int g = grid_for(n16, groups, &per);
  hipLaunchKernelGGL(write_kernel, dim3(g), dim3(kThreads), 0, s, (u32x4*)dst, n16, per);
  return (int)hipGetLastError();
}

int probe_copy(const void* src, void* dst, int64_t n16, int32_t groups, hipStream_t s) {
  int64_t per;
  const int g = grid_for(n16, groups, &per);
  hipLaunchKernelGGL(copy_kernel, dim3(g), dim3(kThreads), 0, s, (const u32x4*)src, (u32x4*)dst,
                     n16, per);
  return (int)hipGetLastError();
}

// dst_b must hold (n16 / (piece/16)) * (row/16) vectors; piece and row are
// multiples of 16 bytes with piece <= row, and n16 a multiple of piece/16.
int probe_read_write2(const void* src, void* dst_a, void* dst_b, int64_t n16, int32_t piece,
                      int32_t row, int32_t groups, hipStream_t s) {
  if (piece < 16 || row < piece || piece % 16 || row % 16 || n16 % (piece / 16)) return -1;
  int64_t per;
  const int g = grid_for(n16, groups, &per);
  hipLaunchKernelGGL(read_write2_kernel, dim3(g), dim3(kThreads), 0, s, (const u32x4*)src,
                     (u32x4*)dst_a, (u32x4*)dst_b, n16, per, piece / 16, row / 16);
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

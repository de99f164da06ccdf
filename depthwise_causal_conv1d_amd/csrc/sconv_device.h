// sconv_device.h -- device-side building blocks shared by the libsconv
// kernels: element types, 16-byte lane vectors, fp32 conversions, SiLU, and
// the XCD-aware workgroup order.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sconv {

// ---------------------------------------------------------------- element types

struct Bf16 {
  using storage = uint16_t;
  static constexpr int kVec16 = 8;  // elements per 16-byte lane vector
};
struct F32 {
  using storage = float;
  static constexpr int kVec16 = 4;
};

template <int BYTES> struct RawT;
template <> struct RawT<16> { typedef uint32_t type __attribute__((ext_vector_type(4))); };
template <> struct RawT<8> { typedef uint32_t type __attribute__((ext_vector_type(2))); };
template <> struct RawT<4> { typedef uint32_t type; };
template <> struct RawT<2> { typedef uint16_t type; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

// One lane's VEC consecutive elements, kept as raw bits so that cache and
// state writes are exact copies of what was read.
template <typename D, int VEC>
struct Pack {
  using S = typename D::storage;
  static constexpr int kBytes = VEC * (int)sizeof(S);
  using raw_t = typename RawT<kBytes>::type;
  struct Elems { S e[VEC]; };
  raw_t raw;

  __device__ __forceinline__ void load(const S* p) {
    raw = *reinterpret_cast<const raw_t*>(p);
  }
  __device__ __forceinline__ void store(S* p) const {
    *reinterpret_cast<raw_t*>(p) = raw;
  }
  // Streaming load: these bytes are read once.
  __device__ __forceinline__ void load_nt(const S* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const raw_t*>(p));
  }
  // Streaming store: nothing will read these bytes again in this kernel.
  __device__ __forceinline__ void store_nt(S* p) const {
    __builtin_nontemporal_store(raw, reinterpret_cast<raw_t*>(p));
  }
  __device__ __forceinline__ void zero() { raw = raw_t{}; }

  __device__ __forceinline__ void to_float(float (&f)[VEC]) const {
    Elems v = __builtin_bit_cast(Elems, raw);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if constexpr (sizeof(S) == 2)
        f[e] = bf16_bits_to_float(v.e[e]);
      else
        f[e] = v.e[e];
    }
  }

  // Round fp32 values to the element type (round to nearest even).
  __device__ __forceinline__ void from_float(const float (&f)[VEC]) {
    Elems v;
    if constexpr (sizeof(S) == 2) {
      if constexpr (VEC == 1) {
        v.e[0] = __builtin_bit_cast(uint16_t, (__bf16)f[0]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; e += 2) {
          bf16x2 b = __builtin_convertvector((f32x2){f[e], f[e + 1]}, bf16x2);
          uint32_t w = __builtin_bit_cast(uint32_t, b);
          v.e[e] = (uint16_t)(w & 0xFFFFu);
          v.e[e + 1] = (uint16_t)(w >> 16);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) v.e[e] = f[e];
    }
    raw = __builtin_bit_cast(raw_t, v);
  }
};

template <typename D>
__device__ __forceinline__ float to_float(typename D::storage v) {
  if constexpr (sizeof(typename D::storage) == 2)
    return bf16_bits_to_float(v);
  else
    return v;
}

template <typename D>
__device__ __forceinline__ float load_as_float(const typename D::storage* p) {
  return to_float<D>(*p);
}

// v * sigmoid(v) with the hardware exp2 and reciprocal (about 1 ulp each).
// v -> -inf gives -0 (or NaN at -inf itself, as the definition does).
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// a[idx] for a run-time idx in [0, N), as a chain of selects over constant
// indices: an array indexed by a run-time value would be demoted to scratch
// or LDS memory.
template <typename T, int N>
__device__ __forceinline__ T pick(const T (&a)[N], int idx) {
  T r = a[0];
#pragma unroll
  for (int q = 1; q < N; ++q) {
    // An empty statement makes each element an opaque register value: a
    // select between two reads of the array would otherwise be folded into
    // one read at a computed index, which keeps the array in memory.
    T v = a[q];
    asm("" : "+v"(v));
    r = idx == q ? v : r;
  }
  return r;
}

// ---------------------------------------------------------------- launch order

// Workgroups are handed to the 8 XCDs round-robin (workgroup g runs on XCD
// g % 8), and each XCD has its own L2.  Renumber so that each XCD walks one
// contiguous run of logical workgroups, in order: neighbouring tiles, which
// share halo rows, then meet in the same L2.  A bijection on [0, G).
// Branch-free: XCD x owns the run starting at x*per + min(x, rem).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t g, uint32_t G) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = G / kXcd, rem = G % kXcd;
  const uint32_t xcd = g % kXcd, idx = g / kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Make a value the compiler cannot prove wave-uniform live in a scalar
// register (it is uniform by construction at every call site).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace sconv

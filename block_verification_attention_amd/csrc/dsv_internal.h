// Internal helpers of libdsv (device code for gfx950 and host-side checks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "dsv.h"

namespace dsv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> f32 (storage is raw uint16 bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite and infinite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Order-preserving float -> uint32 map used for argmax / top-2 keys.
// -0.0 is folded onto +0.0 so that the two compare equal.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((int)(uint32_t)v, m);
  uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((int)(uint32_t)v, src);
  uint32_t hi = __shfl((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Global-memory accesses through address-space-qualified pointers.  Pointers that reach a
// kernel inside a by-value parameter struct are generic to the compiler, which then emits
// flat instructions for them; a flat load also counts against the LDS counter, so every LDS
// wait would wait for outstanding HBM loads too.  T is a scalar or an ext_vector_type.
template <class T>
using global_t = __attribute__((address_space(1))) T;
template <class T>
__device__ __forceinline__ T gload(const void *ptr) {
  return *(const global_t<T> *)ptr;
}
template <class T>
__device__ __forceinline__ T gload_stream(const void *ptr) {  // read once: non-temporal
  return __builtin_nontemporal_load((const global_t<T> *)ptr);
}
template <class T>
__device__ __forceinline__ void gstore(void *ptr, T v) {
  *(global_t<T> *)ptr = v;
}
template <class T>
__device__ __forceinline__ void gstore_stream(void *ptr, T v) {  // read once later: non-temporal
  __builtin_nontemporal_store(v, (global_t<T> *)ptr);
}

__device__ __forceinline__ void status_or(int32_t *status, int32_t bits) {
  if (status) atomicOr(status, bits);
}

// Flat-buffer packer rule (DScale Sec. III-C, Fig. 6): a request is well formed when its length
// lies in [0, W] and its context and segment base are not negative; its effective length is
// then k, else 0 (it takes no slots).  Offsets are the exclusive sums of effective lengths.
__device__ __forceinline__ bool pack_request_ok(int k, int ctx, int64_t kv_base, int W) {
  return k >= 0 && k <= W && ctx >= 0 && kv_base >= 0;
}
__device__ __forceinline__ int pack_effective_length(int k, int ctx, int64_t kv_base, int W) {
  return pack_request_ok(k, ctx, kv_base, W) ? k : 0;
}

// Writes the slots [off, off + k) of request i (k <= W <= DSV_MAX_W): the request's tokens
// are loaded together first, so the writes wait for one memory round trip, not one per slot.
__device__ __forceinline__ void write_request_slots(int i, int k, int off, int W, int c, int64_t kb,
                                                    const int32_t *__restrict__ block_tokens,
                                                    int32_t *__restrict__ slot_req,
                                                    int32_t *__restrict__ slot_tok,
                                                    int32_t *__restrict__ slot_pos,
                                                    int64_t *__restrict__ slot_cache_loc) {
  int32_t tok[DSV_MAX_W];
#pragma unroll
  for (int j = 0; j < DSV_MAX_W; ++j) tok[j] = j < k ? block_tokens[(int64_t)i * W + j] : 0;
#pragma unroll
  for (int j = 0; j < DSV_MAX_W; ++j) {
    if (j < k) {
      const int s = off + j;
      slot_req[s] = i;
      slot_tok[s] = tok[j];
      slot_pos[s] = c + j;
      slot_cache_loc[s] = kb + c + j;
    }
  }
}


}  // namespace dsv

// Host-side launch check: returns DSV_ERR_HIP from the enclosing function on failure.
#define DSV_LAUNCH_CHECK()                              \
  do {                                                  \
    if (hipGetLastError() != hipSuccess) return DSV_ERR_HIP; \
  } while (0)

namespace dsv {
// Host-side aliasing check.  A Span is the byte range [p, p + bytes) an argument covers (a
// null p or zero bytes cover nothing).
struct Span {
  const void *p;
  size_t bytes;
};
inline bool spans_overlap(const Span &a, const Span &b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
  return x >= y ? x - y < b.bytes : y - x < a.bytes;
}
// Product of non-negative counts, saturating at INT64_MAX (a negative factor gives -1).
inline int64_t mul_sat(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x < 0) return -1;
    if (x != 0 && r > INT64_MAX / x) return INT64_MAX;
    r *= x;
  }
  return r;
}
// A 1-D launch of `blocks` workgroups of `threads` work-items: at most 2^32 - 1 work-items
// (the dispatch's grid size is 32-bit) and a block index that fits an int.
inline bool launch_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= INT32_MAX && blocks * threads <= (int64_t)UINT32_MAX;
}
// Sum of non-negative counts, saturating at INT64_MAX.
inline int64_t add_sat(int64_t a, int64_t b) { return a > INT64_MAX - b ? INT64_MAX : a + b; }
// Bytes of n elements of elem bytes (none for n <= 0; saturating at SIZE_MAX).
inline size_t span_bytes(int64_t n, size_t elem) {
  if (n <= 0) return 0;
  return (uint64_t)n > SIZE_MAX / elem ? SIZE_MAX : (size_t)n * elem;
}
// True when an output shares a byte with another output or with an input, or a read-write
// buffer (shared) with an output or an input.  Inputs may share bytes with each other, and
// read-write buffers with each other (two views of one allocation, such as K and V pools
// interleaved by head).
template <size_t NO, size_t NI, size_t NS = 1>
inline bool outputs_alias(const Span (&out)[NO], const Span (&in)[NI],
                          const Span (&shared)[NS] = {{nullptr, 0}}) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = i + 1; j < NO; ++j)
      if (spans_overlap(out[i], out[j])) return true;
    for (size_t j = 0; j < NI; ++j)
      if (spans_overlap(out[i], in[j])) return true;
  }
  for (size_t s = 0; s < NS; ++s) {
    for (size_t i = 0; i < NO; ++i)
      if (spans_overlap(shared[s], out[i])) return true;
    for (size_t j = 0; j < NI; ++j)
      if (spans_overlap(shared[s], in[j])) return true;
  }
  return false;
}
}  // namespace dsv

// Shared device helpers for the gfx950 (CDNA4) kernels: element formats,
// 16-byte chunk loads, MFMA wrappers and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ll {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Compile-time index (register-ring slots and unrolled loop parities).
template <int I>
using ic = std::integral_constant<int, I>;
// Calls f(ic<I>{}), ..., f(ic<N-1>{}): a loop whose index is a compile-time
// constant in the body.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// ---------------------------------------------------------------------------
// Scalar conversions.  float -> bf16/f16 round to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Element traits.  T is the storage type; a 16-byte chunk holds PER16 elements.
template <int DT> struct Elt;
template <> struct Elt<DT_F32> {
  typedef float T;
  static constexpr int PER16 = 4;
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elt<DT_BF16> {
  typedef uint16_t T;
  static constexpr int PER16 = 8;
  static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elt<DT_F16> {
  typedef uint16_t T;
  static constexpr int PER16 = 8;
  static __device__ __forceinline__ float to_f32(uint16_t v) { return f16_to_f32(v); }
  static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_f16(v); }
};

// ---------------------------------------------------------------------------
// 16-byte chunks <-> fp32 lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming load (non-temporal hint) for data read once per call: weights in
// decode, KV-cache rows.  Measured 2-8% faster than plain loads there.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Unpack a chunk of PER16 elements to floats (f[0..PER16)).
template <int DT>
__device__ __forceinline__ void unpack16(u32x4 c, float* f) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c[i]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(c[i] << 16);
      f[2 * i + 1] = __uint_as_float(c[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_to_f32(c[i] & 0xffffu);
      f[2 * i + 1] = f16_to_f32(c[i] >> 16);
    }
  }
}

// Two floats to two 16-bit elements of one 32-bit word (a in the low half),
// rounded to nearest even: one v_cvt_pk_{bf16,f16}_f32.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  if constexpr (DT == DT_BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// Pack PER16 floats into one chunk.
template <int DT>
__device__ __forceinline__ u32x4 pack16(const float* f) {
  u32x4 c;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(f[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
  }
  return c;
}

// Store n (1..8) consecutive floats as elements of format DT.
template <int DT>
__device__ __forceinline__ void store_n(typename Elt<DT>::T* p, const float* f, int n) {
  for (int i = 0; i < n; ++i) p[i] = Elt<DT>::from_f32(f[i]);
}

// Store 4 consecutive values (8-byte store for 16-bit formats, 16-byte for f32).
template <int DT>
__device__ __forceinline__ void store4(typename Elt<DT>::T* p, float a, float b, float c, float d) {
  if constexpr (DT == DT_F32) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    u32x2 v;
    v[0] = pack2<DT>(a, b);
    v[1] = pack2<DT>(c, d);
    *reinterpret_cast<u32x2*>(p) = v;
  }
}

template <int DT>
__device__ __forceinline__ void load4(const typename Elt<DT>::T* p, float* f) {
  if constexpr (DT == DT_F32) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
    f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
  } else {
    u32x2 v = *reinterpret_cast<const u32x2*>(p);
    f[0] = Elt<DT>::to_f32(v[0] & 0xffffu);
    f[1] = Elt<DT>::to_f32(v[0] >> 16);
    f[2] = Elt<DT>::to_f32(v[1] & 0xffffu);
    f[3] = Elt<DT>::to_f32(v[1] >> 16);
  }
}

// ---------------------------------------------------------------------------
// MFMA on one 16-byte chunk per lane.
//   16-bit formats: v_mfma_f32_16x16x32_{bf16,f16}; the chunk is the lane's
//   8-element k-slice.  f32: four v_mfma_f32_16x16x4_f32, one per element.
// Lane layout (16x16 result): lane l holds column l%16, rows (l/16)*4 + 0..3.
// A operand lane l: row l%16; B operand lane l: column l%16; both hold the k
// elements of k-group l/16.  Any k order works as long as A and B agree.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x4 mfma16_chunk(u32x4 a, u32x4 b, f32x4 acc) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]),
                                                 acc, 0, 0, 0);
    return acc;
  }
}

// 16x16x16 bf16/f16 MFMA: the same 16x16 result layout as above; A lane l:
// row l%16, B lane l: column l%16, each with the 4 k-elements of k-group l/16
// (one 8-byte register pair).
template <int DT>
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 acc) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, a),
                                                     __builtin_bit_cast(v4i16, b), acc, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), acc, 0, 0, 0);
  }
}

// 32x32x16 bf16/f16 MFMA: lane l holds column l%32 and rows
// (r/4)*8 + (l/32)*4 + r%4 of the result, r = 0..15; A lane l: row l%32,
// B lane l: column l%32, each with the 8 k-elements of k-group l/32.
template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 acc) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (global_load_lds_dwordx4): lane l of a wave writes
// bytes [16 l, 16 l + 16) of the LDS destination, read from its own global
// address, so no registers stage the data and no ds_write is issued.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds, 16, 0, 0);
}
// Same with the non-temporal cache policy (streamed data read once).
__device__ __forceinline__ void dma16_stream(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds, 16, 0, 2);
}

// ds_read_b64_tr_b16 at LDS byte address addr, as inline assembly: within each
// group of 16 lanes, lane i = 4e + q points at 4 16-bit elements (row R + e,
// cols C + 4q .. +3) and lane j receives rows R .. R+3 of col C + j.  The
// compiler does not track this read: the caller waits for it (lgkmcnt) before
// using the result.  (For the builtin the compiler cannot tell the read from
// reads of rows a global_load_lds still has in flight, and waits for every
// outstanding load first.)
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
// s_waitcnt lgkmcnt(N) only: at most N LDS/scalar-memory operations still
// outstanding (LDS operations of one wave complete in order).
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace ll

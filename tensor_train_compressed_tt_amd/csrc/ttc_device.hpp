// Device-side helpers shared by the HIP kernels: element types, the MFMA
// fragments used for gfx950, guarded 16-byte row loads and bf16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// bf16 activations are carried as raw 16-bit patterns.
struct bf16_t {
  unsigned short bits;
};
// fp8 activations: OCP e4m3 (4 exponent bits, bias 7, 3 mantissa bits,
// largest finite 448), the format of gfx950's fp8 conversions and MFMAs,
// carried as raw bytes.
struct fp8_t {
  unsigned char bits;
};
typedef unsigned char u8x16 __attribute__((ext_vector_type(16)));
typedef long i64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __uint_as_float(((unsigned int)b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even (gfx950 converts in hardware:
// one v_cvt_pk_bf16_f32 per pair of values).
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  return __builtin_bit_cast(unsigned short, (__bf16)f);
}
// two values packed low, high
__device__ __forceinline__ unsigned int f32x2_to_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2));
}

// One MFMA "k-step": each lane supplies 16 bytes of one row of A and of one
// column of B.  Lane l = 16*g + c holds row/column c and the 16-byte group g,
// so a k-step spans 4 groups x (16 bytes / element size) k-values.  The order
// of k inside a step is the same for both operands, so any assignment of
// memory columns to (g, element) pairs gives the same dot products.
template <typename T>
struct Mma;

template <>
struct Mma<bf16_t> {
  static constexpr int EPV = 8;    // elements per lane per k-step
  static constexpr int KSTEP = 32; // k-values per k-step
  typedef u16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0}; }
  __device__ __forceinline__ static unsigned short from_f32(float f) { return f32_to_bf16(f); }
};

template <>
struct Mma<float> {
  static constexpr int EPV = 4;
  static constexpr int KSTEP = 16;
  typedef f32x4 frag;
  // four 16x16x4 fp32 MFMAs; MFMA e takes element e of every lane
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static frag zero() { return frag{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ static float from_f32(float f) { return f; }
};

// fp8: a k-step is 4 groups x 16 bytes = 64 k-values; the 16 bytes of a lane
// feed two 16x16x32 fp8 MFMAs (elements 0..7, then 8..15), the same split
// for both operands, so the dot products are those of the k-step.
template <>
struct Mma<fp8_t> {
  static constexpr int EPV = 16;
  static constexpr int KSTEP = 64;
  typedef u8x16 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    const i64x2 a2 = __builtin_bit_cast(i64x2, a), b2 = __builtin_bit_cast(i64x2, b);
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], c, 0, 0, 0);
    return c;
  }
  // one 32-wide k-step: the MFMA on the low eight bytes of each lane only
  // (lane group g holds k = 8g .. 8g + 7); the rank-contracting products of a
  // rank tile of 32
  __device__ __forceinline__ static f32x4 mma_k32(frag a, frag b, f32x4 c) {
    const i64x2 a2 = __builtin_bit_cast(i64x2, a), b2 = __builtin_bit_cast(i64x2, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}; }
  // round to nearest even (hardware conversion); values beyond the format's
  // range are not expected (activations and operands are O(1))
  __device__ __forceinline__ static unsigned char from_f32(float f) {
    return (unsigned char)(__builtin_amdgcn_cvt_pk_fp8_f32(f, f, 0, false) & 0xff);
  }
};

// four values -> four e4m3 bytes (little-endian order), round to nearest even
__device__ __forceinline__ unsigned f32x4_to_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// storage element of an activation type
template <typename T> struct Elem;
template <> struct Elem<bf16_t> { typedef unsigned short type; };
template <> struct Elem<float> { typedef float type; };
template <> struct Elem<fp8_t> { typedef unsigned char type; };

template <typename T>
__device__ __forceinline__ float elem_to_f32(typename Elem<T>::type v);
template <>
__device__ __forceinline__ float elem_to_f32<bf16_t>(unsigned short v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float elem_to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float elem_to_f32<fp8_t>(unsigned char v) { return __builtin_amdgcn_cvt_f32_fp8((int)v, 0); }

// Load the 16-byte group of row `row` starting at column `col` of a row-major
// matrix (leading dimension ld elements).  Elements outside [0,nrows) x
// [0,ncols) read as zero.  `vec` says that rows are 16-byte aligned.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag(const typename Elem<T>::type* __restrict__ base,
                                                           int64_t row, int64_t nrows, int64_t col,
                                                           int64_t ncols, int64_t ld, bool vec) {
  typedef typename Mma<T>::frag frag;
  constexpr int EPV = Mma<T>::EPV;
  if (row >= nrows || col >= ncols) return Mma<T>::zero();
  const typename Elem<T>::type* p = base + row * ld + col;
  if (vec && col + EPV <= ncols) return *reinterpret_cast<const frag*>(p);
  frag f = Mma<T>::zero();
#pragma unroll
  for (int e = 0; e < EPV; ++e)
    if (col + e < ncols) f[e] = p[e];
  return f;
}

// Branch-free variant for 16-byte-aligned rows whose length is a multiple of
// the group size: the address is clamped into the matrix and the value
// replaced by zero when out of range, so consecutive calls issue their loads
// back to back instead of waiting at a branch each.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag_v(const typename Elem<T>::type* __restrict__ base,
                                                             int64_t row, int64_t nrows, int64_t col,
                                                             int64_t ncols, int64_t ld) {
  typedef typename Mma<T>::frag frag;
  const bool ok = row < nrows && col < ncols;
  const frag f = *reinterpret_cast<const frag*>(base + (ok ? row * ld + col : 0));
  return ok ? f : Mma<T>::zero();
}

// compile-time choice between the two
template <typename T, bool VEC>
__device__ __forceinline__ typename Mma<T>::frag ld_frag(const typename Elem<T>::type* __restrict__ base,
                                                         int64_t row, int64_t nrows, int64_t col, int64_t ncols,
                                                         int64_t ld) {
  if constexpr (VEC)
    return load_frag_v<T>(base, row, nrows, col, ncols, ld);
  else
    return load_frag<T>(base, row, nrows, col, ncols, ld, false);
}

// Buffer loads.  A raw buffer resource over `bytes` bytes returns zero, with no
// memory access, for a load at a byte offset at or beyond `bytes`.  A guarded
// load is then one unconditional instruction whose offset is swapped for
// kNoOff when the element is out of range: no branch, so the compiler knows
// how many loads were issued after any other and waits for exactly the one
// it needs instead of draining all outstanding loads.  Resources are at most
// 2^31 - 1 bytes, so kNoOff plus any instruction offset is out of range.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kNoOff = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  // third descriptor word of an untyped 32-bit-format buffer on gfx9-class GPUs
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag buf_frag(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(typename Mma<T>::frag, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
#ifndef TTC_STREAM_HINTS
#define TTC_STREAM_HINTS 1
#endif
constexpr int kStreamLoadPolicy = TTC_STREAM_HINTS ? 2 : 0;  // nt
// The same load for the last read of a streamed activation in the step (dY in
// the dY pass, x in the dX pass): non-temporal, so that the lines need not
// stay in the caches after this read.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag buf_frag_last(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(typename Mma<T>::frag,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamLoadPolicy));
}

// Stores through a buffer resource: a store at an out-of-range offset is
// dropped, so guarded stores need no branch either.
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t off, unsigned short v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t off, unsigned char v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store32(rsrc_t r, uint32_t off, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, uint2 v) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_f32x4(rsrc_t r, uint32_t off, f32x4 v) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, 0);
}
// 16-byte store of a streamed output (a layer's Y or dX): written once and not
// read again by the pass that follows, so it carries the non-temporal cache
// policy bit and does not displace the operands the next kernels re-read
// from the caches.
constexpr int kStreamStorePolicy = TTC_STREAM_HINTS ? 2 : 0;  // nt
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 v) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)off, 0, kStreamStorePolicy);
}

// Same from LDS (always in range, 16-byte aligned).
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag lds_frag(const typename Elem<T>::type* p) {
  return *reinterpret_cast<const typename Mma<T>::frag*>(p);
}

// Eight e4m3 values in the low half of a fragment, the upper half zero: the
// operand of one 32-wide k-step (Mma::mma_k32), 8-byte aligned.
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag lds_frag_lo8(const typename Elem<T>::type* p) {
  static_assert(sizeof(typename Elem<T>::type) == 1, "one-byte activations only");
  const u32x2v v = *reinterpret_cast<const u32x2v*>(p);
  return __builtin_bit_cast(typename Mma<T>::frag, u32x4v{v.x, v.y, 0u, 0u});
}
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag buf_frag_lo8(rsrc_t r, uint32_t off) {
  static_assert(sizeof(typename Elem<T>::type) == 1, "one-byte activations only");
  const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return __builtin_bit_cast(typename Mma<T>::frag, u32x4v{v.x, v.y, 0u, 0u});
}
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag_lo8(const typename Elem<T>::type* __restrict__ base,
                                                               int64_t row, int64_t nrows, int64_t col, int64_t ld) {
  static_assert(sizeof(typename Elem<T>::type) == 1, "one-byte activations only");
  const bool ok = row < nrows;
  const u32x2v v = *reinterpret_cast<const u32x2v*>(base + (ok ? row * ld + col : 0));
  return ok ? __builtin_bit_cast(typename Mma<T>::frag, u32x4v{v.x, v.y, 0u, 0u}) : Mma<T>::zero();
}

// Column fragment from LDS: EPV consecutive rows of one column.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag lds_col_frag(const typename Elem<T>::type* p, int ld) {
  typename Mma<T>::frag f;
#pragma unroll
  for (int e = 0; e < Mma<T>::EPV; ++e) f[e] = p[e * ld];
  return f;
}

// Column fragments of a 16-column tile of a row-major LDS tile, one per lane:
// lane 16g + i gets EPV consecutive rows, from row EPV*g on, of column i.  `p`
// is the tile's first column in its first row (row 0 of block g = 0; the
// caller adds EPV*g rows).
//
// bf16 uses gfx950's transposing LDS read (ds_read_b64_tr_b16).  Inside each
// block of 16 lanes it hands lane i, as its result j (j = 0..3), element
// i mod 4 of the 64-bit word read by lane 4j + i/4.  So lane 4j + q of the
// block reads row j at columns 4q..4q+3, and lane i ends up with rows 0..3
// of column i; a second read four rows further down gives rows 4..7.  Two
// LDS reads per fragment instead of eight 16-bit reads and the packing.
#ifndef TTC_LDS_TR
#define TTC_LDS_TR 1
#endif
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag lds_colT_frag(const typename Elem<T>::type* p, int ld) {
#if TTC_LDS_TR
  if constexpr (sizeof(typename Elem<T>::type) == 2) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int i = threadIdx.x & 15;
    const typename Elem<T>::type* q = p + (i >> 2) * ld + 4 * (i & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)q);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(q + 4 * ld));
    return __builtin_bit_cast(typename Mma<T>::frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#endif
  return lds_col_frag<T>(p + (threadIdx.x & 15), ld);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Work-group barrier that orders LDS accesses only.  __syncthreads() is a
// work-group release/acquire fence over all address spaces, which on gfx950
// waits for every outstanding global load and store of the wave first; a
// barrier that only hands LDS tiles between waves must not drain the
// prefetched loads and the pending stores of a streaming kernel.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace ttc

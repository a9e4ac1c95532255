// common.hpp -- device helpers shared by the libssd kernels (gfx950 / CDNA4).
//
// Fragment convention for the 16x16 matrix-core tiles used everywhere:
//   A operand (16 x K):  lane L holds row  L % 16, k = (L / 16) * 8 + 0..7
//   B operand (K x 16):  lane L holds col  L % 16, k = (L / 16) * 8 + 0..7
//   accumulator (16x16): lane L holds col  L % 16, rows (L / 16) * 4 + 0..3
// i.e. one K-block of 32 per lane-quad of 8 consecutive k values.  For bf16
// operands that is exactly one v_mfma_f32_16x16x32_bf16.  For fp32 operands the
// same eight values feed eight v_mfma_f32_16x16x4_f32, instruction i taking the
// i-th value of every lane: both operands use the same k assignment, so the
// sum over k is unchanged.
//
// Precision: inputs x, B, C are exact in their storage type.  Operands derived
// in fp32 (decay-weighted CB, decay-scaled x, carried states) are split into a
// bf16 "hi" part and a bf16 "lo" remainder and multiplied in two passes, which
// keeps ~16 significant bits instead of bf16's 8 (one pass would lose accuracy
// the output's dynamic range cannot absorb).  Accumulation is always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ scalars

__device__ __forceinline__ float bf16_to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f32_to_bf16(float v) { return (bf16)v; }  // round to nearest even

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 v) { return (float)v; }

// A value's bits in a 32-bit register (bf16 zero-extended) and back to fp32.
__device__ __forceinline__ uint32_t raw_bits(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t raw_bits(bf16 v) {
  return (uint32_t)__builtin_bit_cast(unsigned short, v);
}
template <typename T> __device__ __forceinline__ float from_bits(uint32_t r);
template <> __device__ __forceinline__ float from_bits<float>(uint32_t r) { return __uint_as_float(r); }
template <> __device__ __forceinline__ float from_bits<bf16>(uint32_t r) { return __uint_as_float(r << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
// 2^x: the hardware exponential itself.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(u) = log(1 + e^u); for u > 20 the correction log1p(e^-u) is below
// 2.1e-9 relative and u itself is returned.
__device__ __forceinline__ float softplus_f32(float u) {
  return u > 20.0f ? u : log1pf(__expf(u));
}

__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ------------------------------------------------------------------ vectors

// Eight consecutive elements of type T from memory, widened to fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ f32x8 load(const bf16* p) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (float)v[i];
    return r;
  }
  static __device__ __forceinline__ void store(bf16* p, f32x8 v) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = o;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ f32x8 load(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[i + 4] = b[i]; }
    return r;
  }
  static __device__ __forceinline__ void store(float* p, f32x8 v) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[i + 4]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  }
};

// Packed bf16 pairs: a dword holds two bf16, element 2i in the low half.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {  // (a.lo16, b.lo16)
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {  // (a.hi16, b.hi16)
  return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t bf16_bits(bf16 v) {
  return (uint32_t)__builtin_bit_cast(unsigned short, v);
}
__device__ __forceinline__ uint32_t pack2(bf16 a, bf16 b) {
  return bf16_bits(a) | (bf16_bits(b) << 16);
}
__device__ __forceinline__ float bf16_lo_f32(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// ------------------------------------------------------------------ fragments

// bf16 path: exact operand (one register quad) and split operand (hi + lo).
struct FragBF { bf16x8 v; };
struct FragSplit { bf16x8 hi, lo; };
// fp32 path: eight fp32 values.
struct FragF32 { f32x8 v; };

// Two fp32 values rounded (to nearest even) to a packed bf16 pair in one
// conversion: the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// hi = bf16(a), lo = bf16(a - hi), per pair of elements.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16_lo_f32(hi), b - bf16_hi_f32(hi));
}

__device__ __forceinline__ FragSplit split_f32x8(f32x8 a) {
  u32x4 hi, lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h, l;
    split_pair(a[2 * i], a[2 * i + 1], h, l);
    hi[i] = h;
    lo[i] = l;
  }
  FragSplit f;
  f.hi = __builtin_bit_cast(bf16x8, hi);
  f.lo = __builtin_bit_cast(bf16x8, lo);
  return f;
}

__device__ __forceinline__ void mma(f32x4& acc, const FragBF& a, const FragBF& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const FragSplit& a, const FragBF& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.v, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const FragBF& a, const FragSplit& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.lo, acc, 0, 0, 0);
}
// Both operands split: hi.hi + hi.lo + lo.hi (the lo.lo term is below fp32
// rounding of the sum's leading terms), ~16 significant bits on each side.
__device__ __forceinline__ void mma(f32x4& acc, const FragSplit& a, const FragSplit& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const FragF32& a, const FragF32& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// Operand policy per input type: how an exact input fragment and an fp32-derived
// fragment are represented, loaded and built.
template <typename T> struct Prec;
template <> struct Prec<bf16> {
  using Exact = FragBF;
  using Derived = FragSplit;
  static __device__ __forceinline__ Exact load_exact(const bf16* p) {
    Exact f; f.v = *reinterpret_cast<const bf16x8*>(p); return f;
  }
  static __device__ __forceinline__ Exact zero_exact() {
    Exact f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = (bf16)0.0f;
    return f;
  }
  static __device__ __forceinline__ Derived derive(f32x8 v) { return split_f32x8(v); }
};
template <> struct Prec<float> {
  using Exact = FragF32;
  using Derived = FragF32;
  static __device__ __forceinline__ Exact load_exact(const float* p) {
    Exact f; f.v = Vec8<float>::load(p); return f;
  }
  static __device__ __forceinline__ Exact zero_exact() {
    Exact f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = 0.0f;
    return f;
  }
  static __device__ __forceinline__ Derived derive(f32x8 v) { Derived f; f.v = v; return f; }
};

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// ------------------------------------------------------------------ LDS transpose reads

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 4a + b receives element b of the 8-byte words addressed by lanes
// a, a + 4, a + 8 and a + 12 of the group (in that order; layout checked on
// the hardware).  So if lane l of a group addresses row k0 + l / 4, columns
// col0 + 4 (l % 4) .. + 3 of a row-major [k][col] bf16 tile, lane c of the
// group receives column col0 + c of rows k0 .. k0 + 3: four consecutive k of
// one column, half of a 16x16x32 matrix-core operand fragment.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Operand fragment (8 bf16 along k for column col0 + lane % 16) from a
// row-major [k][col] bf16 tile in LDS with row pitch ld (elements, a multiple
// of 4): k = k0 .. k0 + 3, then k1 .. k1 + 3 (k0, k1 chosen per lane group).
__device__ __forceinline__ bf16x8 lds_frag_tr(const bf16* tile, int ld, int k0, int k1,
                                              int col0) {
  const int l = threadIdx.x % 16;
  const bf16* c = tile + col0 + 4 * (l % 4);
  const u32x2 lo = lds_read_tr16(c + (k0 + l / 4) * ld);
  const u32x2 hi = lds_read_tr16(c + (k1 + l / 4) * ld);
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// threadIdx.x passed through an empty asm statement, so that the per-lane
// addresses derived from it are recomputed where they are used instead of
// being hoisted out of a long loop and kept live across all of it (which can
// exhaust the register file and force spills).  Emits no instruction.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ------------------------------------------------------------------ wave scan

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    float o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP lane moves
// (row shifts within each 16-lane row, then row broadcasts across rows); no
// LDS traffic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf,
                                                    false));
}
__device__ __forceinline__ float wave_inclusive_sum_dpp(float v) {
  // row_shr:1, 2, 4, 8 (lanes without a source receive 0)
  v += dpp_f32<0x111, 0xf>(v);
  v += dpp_f32<0x112, 0xf>(v);
  v += dpp_f32<0x114, 0xf>(v);
  v += dpp_f32<0x118, 0xf>(v);
  // row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3
  v += dpp_f32<0x142, 0xa>(v);
  v += dpp_f32<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ double wave_inclusive_sum_f64(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    double o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// ------------------------------------------------------------------ XCD placement

// MI355X has 8 accelerator complex dies (XCDs), each with its own L2.  The
// dispatcher hands consecutive workgroup ids to the XCDs in turn, so a linear
// block id L runs on XCD L % 8.  This maps L to a logical work item such that
// consecutive logical items share an XCD (and its L2): items [x * per, (x+1) *
// per) run on XCD x.  Ids of an incomplete last round keep their own number.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / kNumXcd;
  if (L >= per * kNumXcd) return L;
  return (L % kNumXcd) * per + L / kNumXcd;
}

// ------------------------------------------------------------------ geometry

// Problem geometry passed by value to every kernel.
struct Geo {
  int b, T, H, P, G, N, C;
  int nc;        // ceil(T / C) chunks per sequence (batch mode)
  int K;         // logical chunk slots
  int nseq;      // sequences (batch mode: b)
  int hpg;       // heads per group
  int Hs;        // heads of the (sequence, head, P, N) initial/final state tensors:
                 // H, or more when a pass covers only some of the heads
  const int32_t* meta;  // packed-mode chunk table, NULL in batch mode
};

struct Chunk {
  int b;      // batch row of the chunk's tokens
  int t0;     // first token (within the batch row)
  int len;    // tokens in the chunk (1..C)
  int seq;    // sequence id (batch row in batch mode)
};

// Chunk table header size and accessors (see the layout in ssd.h).
constexpr int kMetaHeader = 4;

// The chunk table is built by an earlier kernel and only read by the kernels
// that walk it, so it is read through the constant address space: at uniform
// indices these are scalar loads, which do not queue behind the vector loads a
// kernel has in flight.
typedef __attribute__((address_space(4))) const int32_t MetaWord;
__device__ __forceinline__ int32_t meta_word(const int32_t* meta, int i) {
  return ((const MetaWord*)meta)[i];
}

__device__ __forceinline__ bool get_chunk(const Geo& g, int j, Chunk& c) {
  if (g.meta) {
    if (j >= meta_word(g.meta, 0)) return false;
    const int e = kMetaHeader + 3 * j;
    c.seq = meta_word(g.meta, e); c.t0 = meta_word(g.meta, e + 1); c.len = meta_word(g.meta, e + 2);
    c.b = 0;
    return true;
  }
  if (j >= g.K) return false;
  c.b = j / g.nc;
  const int cc = j - c.b * g.nc;
  c.t0 = cc * g.C;
  c.len = min(g.C, g.T - c.t0);
  c.seq = c.b;
  return true;
}

// Range of logical chunks [first, last) of sequence i.
__device__ __forceinline__ void seq_chunks(const Geo& g, int i, int& first, int& last) {
  if (g.meta) {
    const int fc = kMetaHeader + 3 * g.K;
    first = meta_word(g.meta, fc + i); last = meta_word(g.meta, fc + i + 1);
  } else {
    first = i * g.nc; last = first + g.nc;
  }
}

// Strided tensor argument as the kernels see it.
struct TArg {
  const void* p;
  int64_t s0, s1, s2;   // batch, token, head/group strides (elements)
};

// base + off elements with the offset in 32-bit arithmetic: a uniform base
// stays in scalar registers and the per-lane part is one 32-bit vector
// register (the scalar-base form of the global loads and stores).  The byte
// offset must fit in 32 bits.
template <typename T>
__device__ __forceinline__ const T* at(const T* base, uint32_t off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off * (uint32_t)sizeof(T));
}
template <typename T>
__device__ __forceinline__ T* at(T* base, uint32_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off * (uint32_t)sizeof(T));
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const TArg& a, int b, int t, int hg) {
  return reinterpret_cast<const T*>(a.p) + (int64_t)b * a.s0 + (int64_t)t * a.s1 +
         (int64_t)hg * a.s2;
}
template <typename T>
__device__ __forceinline__ T* row_ptr_mut(const TArg& a, int b, int t, int hg) {
  return reinterpret_cast<T*>(const_cast<void*>(a.p)) + (int64_t)b * a.s0 +
         (int64_t)t * a.s1 + (int64_t)hg * a.s2;
}

}  // namespace ssd

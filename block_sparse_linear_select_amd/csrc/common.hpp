// Device-side building blocks shared by the gfx950 kernels: operand
// fragments for 16x16x32 matrix-core steps, conversions and small wave
// utilities.  Everything here is written for CDNA4 wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;     // tokens per tile (query and key)
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16_t { uint16_t bits; };   // storage type of a bfloat16 element
struct fp8_t { uint8_t bits; };     // storage type of an OCP E4M3FN element

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bfloat16 bits (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair with the hardware round-to-nearest-even
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// OCP E4M3FN code -> float with the gfx950 conversion instruction (exact
// for every finite code; the two NaN codes do not occur in valid inputs).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }
// byte `sel` (0..3) of a word of four codes
template <int SEL>
__device__ __forceinline__ float e4m3_byte(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL); }

// ---------------------------------------------------------------------------
// Fragments.  A fragment is what one lane holds of a 16 x 32 operand of a
// 16x16x32 step: lane l holds row (l % 16) and the 8 contraction indices
// k = 8*(l/16) + s, s = 0..7.  The accumulator of a step is 16x16 float with
// lane l holding column (l % 16), rows 4*(l/16) + i, i = 0..3.
// For bf16 the step is one v_mfma_f32_16x16x32_bf16; for float it is eight
// v_mfma_f32_16x16x4_f32 steps, step s contracting index 8*(l/16) + s.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  u32x4 w;  // 8 bf16, element s in the low/high half of word s/2
  __device__ __forceinline__ void zero() { w = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ void set_pair(int j, float a, float b) { w[j] = pack_bf16x2(a, b); }
};

template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = 0.f;
  }
  __device__ __forceinline__ void set_pair(int j, float a, float b) { v[2 * j] = a; v[2 * j + 1] = b; }
};

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.w),
                                              __builtin_bit_cast(bf16x8_t, b.w), c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

// Position of element (rank row rr, column e) of an r x d state inside its
// readout A fragments (rows: d, contraction: r in chunks of 32): fragment
// (e / 16, rr / 32), lane e % 16 + 16 g, slot s, where within a 32-row chunk
// row 16 h + 4 g + i sits at slot 4 h + i -- the order in which the readout
// packs its rotated features into B fragments.
template <int D, int R>
__host__ __device__ __forceinline__ int sp_frag_index(int rr, int e) {
  constexpr int NRC = (R + 31) / 32;
  const int rc = rr >> 5, rem = rr & 31;
  const int s = 4 * (rem >> 4) + (rem & 3), g = (rem >> 2) & 3;
  const int lane = (e & 15) + 16 * g, db = e >> 4;
  return ((db * NRC + rc) * 64 + lane) * 8 + s;
}

// Load 8 consecutive elements (one fragment's worth) from memory of type T.
__device__ __forceinline__ void load8(Frag<bf16_t>& f, const bf16_t* p) {
  f.w = *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void load8(Frag<float>& f, const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
  float4 a = q[0], b = q[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Raw 8-element chunk of the storage type, kept in registers between a
// global load and an LDS store.
template <typename T> struct Chunk8;
template <> struct Chunk8<bf16_t> { u32x4 w; };
template <> struct Chunk8<float> { float4 a, b; };
template <> struct Chunk8<fp8_t> { uint2 w; };

__device__ __forceinline__ void gload8(Chunk8<bf16_t>& c, const bf16_t* p) { c.w = *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void gload8(Chunk8<float>& c, const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
  c.a = q[0]; c.b = q[1];
}
__device__ __forceinline__ void gload8(Chunk8<fp8_t>& c, const fp8_t* p) { c.w = *reinterpret_cast<const uint2*>(p); }
// Bounds-checked buffer loads of one chunk: a buffer view covers the valid
// part of a tensor, and any element offset past it reads as zero.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, bounds-checked (gfx9-family dword 3)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, nbytes, kBufferFlags);
}
__device__ __forceinline__ void bload8(Chunk8<bf16_t>& c, __amdgpu_buffer_rsrc_t r, int elem) {
  c.w = __builtin_amdgcn_raw_buffer_load_b128(r, elem * 2, 0, 0);
}
__device__ __forceinline__ void bload8(Chunk8<fp8_t>& c, __amdgpu_buffer_rsrc_t r, int elem) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, elem, 0, 0);
  c.w = make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void bload8(Chunk8<float>& c, __amdgpu_buffer_rsrc_t r, int elem) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, elem * 4, 0, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, elem * 4 + 16, 0, 0);
  c.a = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]));
  c.b = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
}

__device__ __forceinline__ void zero8(Chunk8<bf16_t>& c) { c.w = u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void zero8(Chunk8<float>& c) { c.a = make_float4(0, 0, 0, 0); c.b = c.a; }
__device__ __forceinline__ void zero8(Chunk8<fp8_t>& c) { c.w = make_uint2(0, 0); }

// Element e (0..7) of a chunk as float.
__device__ __forceinline__ float elem(const Chunk8<bf16_t>& c, int e) {
  uint32_t w = c.w[e >> 1];
  return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}
__device__ __forceinline__ float elem(const Chunk8<float>& c, int e) {
  switch (e) {
    case 0: return c.a.x; case 1: return c.a.y; case 2: return c.a.z; case 3: return c.a.w;
    case 4: return c.b.x; case 5: return c.b.y; case 6: return c.b.z; default: return c.b.w;
  }
}
__device__ __forceinline__ float elem(const Chunk8<fp8_t>& c, int e) {
  const uint32_t w = (e < 4) ? c.w.x : c.w.y;
  switch (e & 3) {
    case 0: return e4m3_byte<0>(w);
    case 1: return e4m3_byte<1>(w);
    case 2: return e4m3_byte<2>(w);
    default: return e4m3_byte<3>(w);
  }
}

// Position of key `key` (0..63) of a tile staged transposed for a
// contraction over keys: within each 32-key chunk, key 16h + 4g + i sits at
// 8g + 4h + i, so that lane group g reads its eight slots as one run.
__device__ __forceinline__ int vt_pos_a(int key) {
  int c = key >> 5, kk = key & 31;
  int h = kk >> 4, g = (kk >> 2) & 3, i = kk & 3;
  return 32 * c + 8 * g + 4 * h + i;
}

__device__ __forceinline__ void st4o(bf16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st4o(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void st4v(bf16_t* dst, float a, float b, float c, float d) { st4o(dst, a, b, c, d); }
__device__ __forceinline__ void st4v(float* dst, float a, float b, float c, float d) { st4o(dst, a, b, c, d); }

__device__ __forceinline__ void lds_row(bf16_t* dst, const Chunk8<bf16_t>& c) { *reinterpret_cast<u32x4*>(dst) = c.w; }
__device__ __forceinline__ void lds_row(float* dst, const Chunk8<float>& c) {
  reinterpret_cast<float4*>(dst)[0] = c.a;
  reinterpret_cast<float4*>(dst)[1] = c.b;
}

// ---------------------------------------------------------------------------
// wave utilities
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_xor(float x, int m) { return __shfl_xor(x, m, kWave); }

// max / sum over the four 16-lane groups that share a column
__device__ __forceinline__ float group4_max(float x) {
  x = fmaxf(x, wave_xor(x, 16));
  return fmaxf(x, wave_xor(x, 32));
}
__device__ __forceinline__ float group4_sum(float x) {
  x += wave_xor(x, 16);
  return x + wave_xor(x, 32);
}

// elu(x) + 1, without a branch: the exponential of x is always formed (one
// transcendental op) and selected for x <= 0.
__device__ __forceinline__ float elu1(float x) {
  const float e = __expf(x);  // taken only for x <= 0 (for large x it overflows and is not selected)
  return x > 0.f ? x + 1.f : e;
}

// Block order of the query-tile kernels.  The hardware hands block i to XCD
// i % 8.  All eight XCDs work on the same head at a time, so the key/value
// tiles in use stay within one or two heads (~40 MB at 720P) and remain
// resident in the 256 MB MALL; inside a head, XCD x takes the contiguous x-th
// eighth of the query tiles, so neighbouring query tiles, which keep many of
// the same key tiles, share that XCD's L2.  Grid: 8 * heads * ceil(T / 8)
// blocks; returns the (b*H + h) * T + a row, or -1 for padding blocks.
__device__ __forceinline__ int head_interleaved_row(int i, int T) {
  const int per = (T + 7) / 8;
  const int xcd = i & 7, j = i >> 3;
  const int head = j / per, a = xcd * per + j % per;
  return a < T ? head * T + a : -1;
}

// Marks a value as wave-uniform (kept in a scalar register), so that buffer
// descriptors and addresses derived from it need no per-lane handling.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

}  // namespace hsa

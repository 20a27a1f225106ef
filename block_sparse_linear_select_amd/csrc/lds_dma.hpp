// LDS-direct staging and small matrix-core helpers shared by the query-tile
// kernels and the FP8 projection: buffer_load ... lds issued from an asm
// statement (the kernels count these loads themselves), the barrier that
// goes with it, and the 16x16x128 FP8 matrix-core step.
#pragma once
#include <type_traits>
#include "common.hpp"

namespace hsa {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void* lds_void_t;

// s_waitcnt immediate that waits for all but n vector-memory operations
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Workgroup barrier for the LDS-direct pipeline.  __syncthreads() also
// orders memory, which makes the compiler wait for every load still writing
// LDS, including the one just issued for the other buffer.  Here each wave
// waits for its own loads of the buffer it is about to publish (s_waitcnt
// before the call), finishes its own LDS reads, and the asm statement keeps
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are complete
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer descriptor as four scalar registers (base, stride 0, num_records,
// flags) for the LDS-direct loads below.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc_regs(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)p, (int)((p >> 32) & 0xFFFF), nbytes, kBufferFlags};
}

// One 16-byte-per-lane LDS-direct load: M0 = LDS destination of lane 0 (lane
// l writes 16 bytes at M0 + 16 l), voff = the lane's byte offset in the
// buffer.  Written as an asm statement so that the compiler, which does not
// see its LDS write, inserts no waits for it before unrelated LDS reads (it
// would wait for every such load before a transposing read, whose memory
// operand carries no alias information); the kernels wait on vmcnt
// themselves before publishing a buffer.  s_nop covers the M0 hazard.
// M0 is saved and restored around the load (the compiler keeps no value of
// its own there across the statement); `imm` is a compile-time byte offset
// added to the LDS destination.
template <int IMM = 0>
__device__ __forceinline__ void lds_dma16(const i32x4_t& rs, const uint8_t* lds_dst, int voff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(lds_void_t)(lds_dst);
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %2, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(voff), "s"(m0v), "s"(rs), "n"(IMM) : "memory", "scc");
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Swizzles of a staged tile with RG 16-byte granules per row (RB = 16 RG
// bytes): rows sharing a 256-byte bank set get distinct granule positions
// (K) or distinct granule pairs (V).
template <int RG> __device__ __forceinline__ int swz_k(int row) { return (row / (16 / RG)) & (RG - 1); }
template <int RG> __device__ __forceinline__ int swz_v(int row) { return 2 * ((row / (16 / RG)) & (RG / 2 - 1)); }

// One wave's share of the LDS-direct loads of a 64-row tile (RB bytes per
// row) moved by NW waves: load i of wave w fills LDS bytes
// [1024 (NI w + i), +1024) with NI = RB / (16 NW).
// off[i] = the lane's byte offset within the tile of the granule it moves.
template <int RB, bool V, int NW = 2>
__device__ __forceinline__ void dma_offsets(int w, int lane, int* off) {
  constexpr int RG = RB / 16, NI = 64 * RB / 1024 / NW;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int lin = 1024 * (NI * w + i) + 16 * lane;
    const int row = lin / RB, pos = (lin % RB) / 16;
    const int gr = pos ^ (V ? swz_v<RG>(row) : swz_k<RG>(row));
    off[i] = row * RB + 16 * gr;
  }
}
template <int RB, int NW = 2>
__device__ __forceinline__ void dma_tile(const i32x4_t& rs, int col, const int* off, uint8_t* dst, int w) {
  constexpr int NI = 64 * RB / 1024 / NW;
  const int base = col * 64 * RB;  // out-of-range columns fall outside the buffer and load zeros
  static_for<0, NI>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    lds_dma16<1024 * i>(rs, dst + 1024 * NI * w, base + off[i]);
  });
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma_fp8(const i32x8_t& a, const i32x8_t& b, const f32x4& c) {
  // formats 0/0 = E4M3 for both operands, unit (2^0) block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8_t cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

}  // namespace hsa

// Device helpers for the gfx950 (CDNA4) attention kernels: vector types, bf16
// conversion, the 32x32x16 bf16 MFMA, the swizzled LDS layout of K/V tiles,
// direct global->LDS tile loads and the transposing LDS read of V.
//
// Lane layouts used throughout (64-lane wavefront; checked on gfx950):
//   v_mfma_f32_32x32x16_bf16, C[32x32] += A[32x16] * B[16x32]:
//     A: lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]
//     B: lane l holds B[8*(l/32) .. 8*(l/32)+7][l % 32]
//     C: lane l, register j holds C[8*(j/4) + 4*(l/32) + j%4][l % 32]
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lane s supplies the address
//     of 4 consecutive 16-bit elements; lane l receives element l%4 of the chunks of
//     lanes l/4, 4+l/4, 8+l/4, 12+l/4.  With lane s pointing at row r0 + s/4,
//     column c0 + 4*(s%4) of a row-major tile, lane l receives column c0 + l of rows
//     r0 .. r0+3: a 4x16 transpose.
//   global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e2d2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define E2D2_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform value (moves it to a scalar register).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Pack 8 fp32 values (round to nearest even) into bf16x8.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// ---------------------------------------------------------------------------------
// K/V tile layout in LDS: `rows` rows of D bf16, each row split into CH = D/8 chunks
// of 16 bytes; logical chunk c of row r is stored at physical chunk c ^ swz(r).  The
// XOR pattern keeps the MFMA reads of K (16 lanes, 16 rows, one chunk) and the
// transposing reads of V (8 rows, 4 chunks) spread over the LDS banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;
  else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

// Element offset of (row, col) in a swizzled tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r))) << 3) + (col & 7);
}

// Direct global->LDS load of rows [row0, row0 + ROWS) of a [n_rows][D] bf16 matrix
// into a swizzled LDS tile.  Rows at or past n_rows read row n_rows - 1 instead (their
// scores are masked off; their values stay finite).  The calling waves split the
// 16-byte slots: wave w issues instructions w, w + n_waves, ...; each instruction
// fills 64 consecutive slots (1 KiB).  `tile` and the wave index must be uniform.
template <int D, int ROWS>
__device__ __forceinline__ void load_tile_lds(const __bf16* __restrict__ src, int row0,
                                              int n_rows, __bf16 E2D2_LDS* tile, int wave,
                                              int n_waves, int lane) {
  constexpr int CH = D / 8;
  constexpr int NI = ROWS * CH / 64;
  static_assert(ROWS * CH % 64 == 0, "tile must be a whole number of 1 KiB slices");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i % n_waves != wave) continue;
    const int slot = i * 64 + lane;
    const int r = slot / CH;
    const int pc = slot % CH;
    const int lc = pc ^ swz<D>(r);
    int g = row0 + r;
    g = g < n_rows ? g : n_rows - 1;
    __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)g * D + lc * 8),
                                     (E2D2_LDS void*)(tile + i * 512), 16, 0, 0);
  }
}

// MFMA A-operand read of K for S^T = K Q^T: lane l gets K[row0 + l%32][col0 + 8*(l/32) ..+7].
template <int D>
__device__ __forceinline__ bf16x8 read_k_frag(const __bf16 E2D2_LDS* tile, int row0, int col0,
                                              int lane) {
  const int r = row0 + (lane & 31);
  const int col = col0 + ((lane >> 5) << 3);
  return *(const bf16x8 E2D2_LDS*)(tile + tile_off<D>(r, col));
}

// MFMA A-operand read of V^T for O^T += V^T P^T, for the 16 keys [key0, key0 + 16)
// and the 32 head dims [d0, d0 + 32): lane l gets V[k][d0 + l%32] for the eight keys
// k = key0 + 4*(l/32) + {0,1,2,3} and key0 + 8 + 4*(l/32) + {0,1,2,3}, which is the
// key order of the P^T operand taken from the S^T accumulator.
template <int D>
__device__ __forceinline__ bf16x8 read_vt_frag(const __bf16 E2D2_LDS* tile, int key0, int d0,
                                               int lane) {
  const int g = lane >> 5;
  const int s = lane & 15;
  const int col = d0 + (((lane >> 4) & 1) << 4) + ((s & 3) << 2);
  const int r_a = key0 + (g << 2) + (s >> 2);
  const int r_b = r_a + 8;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 E2D2_LDS*)(tile + tile_off<D>(r_a, col)));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 E2D2_LDS*)(tile + tile_off<D>(r_b, col)));
  // Whole-vector reinterpretation (element-wise casts of the 16-bit lanes were
  // mis-assembled into the MFMA operand by the compiler).
  const bf16x4 ab = __builtin_bit_cast(bf16x4, a);
  const bf16x4 bb = __builtin_bit_cast(bf16x4, b);
  const bf16x8 out = __builtin_shufflevector(ab, bb, 0, 1, 2, 3, 4, 5, 6, 7);
  return out;
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace e2d2

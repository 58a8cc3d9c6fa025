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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
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

// Max of x over the lane pair (l, l ^ 32), which hold the two halves of one query row in
// the 32x32 accumulator layout.  v_permlane32_swap gives every lane the values
// of lanes l % 32 and l % 32 + 32 (checked on gfx950), combined in that fixed order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// v_mfma_f32_16x16x32_bf16, C[16x16] += A[16x32] * B[32x16] (checked on gfx950):
//   A: lane l holds A[l % 16][8*(l/16) .. 8*(l/16)+7]
//   B: lane l holds B[8*(l/16) .. 8*(l/16)+7][l % 16]
//   C: lane l, register r holds C[4*(l/16) + r][l % 16]
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Max / sum over the four lanes l % 16 + 16 g (g = 0..3), which hold one row of the
// 16x16 layout: v_permlane32_swap, then v_permlane16_swap; every lane gets its group's
// values in lane order (checked on gfx950), so all four compute the same result.
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

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

// Softmax numerators of one 32-key block of S^T: p = 2^(s * c + negm) for the lane's
// 16 scores, packed to bf16 as the two B operands of O^T += V^T P^T (pb[h] holds
// registers 8h .. 8h+7).  Returns acc plus the sum of the packed values (v_dot2 with
// ones, two per instruction), so the denominator adds exactly the rounded p's that the
// numerator multiplies.
__device__ __forceinline__ float exp_pack(const f32x16& s, float c, float negm, bf16x8 (&pb)[2],
                                          float acc) {
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = fast_exp2(fmaf(s[8 * h + j], c, negm));
    const bf16x8 v = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    pb[h] = v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x2 pr = {v[2 * k], v[2 * k + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
  }
  return acc;
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


// Buffer resource over `bytes` bytes at `base` (raw, unswizzled, 32-bit records).  Loads
// past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Direct buffer->LDS loads of a ROWS x D bf16 tile into the swizzled layout, split
// over NWAVES waves.  Per lane, the byte offsets inside a tile do not depend on the
// tile, so they are computed once (init); per tile only the scalar row offset
// changes.  Rows past the buffer's end read as zero.
template <int D, int ROWS, int NWAVES>
struct TileLoader {
  static constexpr int CH = D / 8;
  static constexpr int NI = ROWS * CH / 64;  // 1 KiB instructions per tile
  static constexpr int NPW = NI / NWAVES;    // per wave
  static_assert(NI % NWAVES == 0 && ROWS * CH % 64 == 0, "tile does not split evenly");
  uint32_t voff[NPW];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const int slot = (wave + k * NWAVES) * 64 + lane;
      const int r = slot / CH;
      const int lc = (slot % CH) ^ swz<D>(r);
      voff[k] = (uint32_t)(r * D + lc * 8) * 2u;
    }
  }
  // tile: LDS destination (uniform); row0: first row of the tile in the buffer.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int row0, char E2D2_LDS* tile,
                                       int wave) const {
#pragma unroll
    for (int k = 0; k < NPW; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void E2D2_LDS*)(tile + (wave + k * NWAVES) * 1024),
                                               16, (int)voff[k], row0 * D * 2, 0, 0);
  }
};

// Per-lane byte offsets of the K operand reads (S^T = K Q^T): koff[cc] addresses
// K[l % 32][16 cc + 8 (l / 32) ..+7] in a swizzled tile; the 32-key block kb sits
// 64 * D * kb bytes further (rows 32 apart share the swizzle).
template <int D>
__device__ __forceinline__ void k_offsets(int lane, uint32_t (&koff)[D / 16]) {
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc)
    koff[cc] = 2u * (uint32_t)tile_off<D>(lane & 31, cc * 16 + ((lane >> 5) << 3));
}




// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------------
// Transposing LDS reads of V in one asm block that also waits for them.  Written as
// inline asm (not the builtin) because the compiler cannot tell these reads apart from
// the in-flight global_load_lds writes of later tiles and would otherwise wait for ALL
// outstanding vector-memory loads before each of them, which serialises the prefetch.
// The tiles read here are complete: the caller waited for their loads (wait_vmem) and
// passed a workgroup barrier where other waves loaded them.  Each asm block ends with
// s_waitcnt lgkmcnt(0), so its outputs are valid when it completes.
//
// tr_reads<O0, O1>: for each of the N byte addresses a[i] (LDS), reads 8 bytes at
// a[i] + O0 and at a[i] + O1; o[2i] gets the first, o[2i+1] the second.
template <int O0, int O1>
__device__ __forceinline__ void tr_reads(const uint32_t (&a)[2], long (&o)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "i"(O0), "i"(O1)
      : "memory");
}
template <int O0, int O1>
__device__ __forceinline__ void tr_reads(const uint32_t (&a)[4], long (&o)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(O0), "i"(O1)
      : "memory");
}
template <int O0, int O1>
__device__ __forceinline__ void tr_reads(const uint32_t (&a)[8], long (&o)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%25\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:%25\n\t"
      "ds_read_b64_tr_b16 %6, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]),
        "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
        "v"(a[7]), "i"(O0), "i"(O1)
      : "memory");
}

// Transposing reads at one offset: o[i] = 8 bytes at a[i] + O (N in {2, 4, 8}).
template <int O>
__device__ __forceinline__ void tr_reads1(const uint32_t (&a)[2], long (&o)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:%4\n\t"
      "ds_read_b64_tr_b16 %1, %3 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1])
      : "v"(a[0]), "v"(a[1]), "i"(O)
      : "memory");
}
template <int O>
__device__ __forceinline__ void tr_reads1(const uint32_t (&a)[4], long (&o)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
      "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
      "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(O)
      : "memory");
}
template <int O>
__device__ __forceinline__ void tr_reads1(const uint32_t (&a)[8], long (&o)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
        "v"(a[7]), "i"(O)
      : "memory");
}

// Batched 16-byte LDS reads (the K operands of S^T = K Q^T), in one asm block that
// waits for them, so one LDS round trip covers a whole batch of MFMAs instead of one
// each.  kreadN<OFF>: o[i] = 16 bytes at a[i] + OFF.
template <int OFF>
__device__ __forceinline__ void kread8(const uint32_t (&a)[8], bf16x8 (&o)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%16\n\t"
      "ds_read_b128 %1, %9 offset:%16\n\t"
      "ds_read_b128 %2, %10 offset:%16\n\t"
      "ds_read_b128 %3, %11 offset:%16\n\t"
      "ds_read_b128 %4, %12 offset:%16\n\t"
      "ds_read_b128 %5, %13 offset:%16\n\t"
      "ds_read_b128 %6, %14 offset:%16\n\t"
      "ds_read_b128 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
        "v"(a[7]), "i"(OFF)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void kread4(const uint32_t (&a)[4], bf16x8 (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void kread2(const uint32_t (&a)[2], bf16x8 (&o)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n\t"
      "ds_read_b128 %1, %3 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1])
      : "v"(a[0]), "v"(a[1]), "i"(OFF)
      : "memory");
}


// S^T = K Q^T for the 32-key blocks of a K tile at LDS byte address kbase whose mask
// `want` is set (bit kb = block kb; NB blocks of 32 keys, 64*D bytes apart).  The K
// operands of a block are read in one batch, then its MFMAs issue back to back; the
// next block's reads overlap the previous block's MFMAs.
// BASE: a compile-time byte offset added to kbase through the instructions' offset field.
template <int D, int KB, int BASE = 0>
__device__ __forceinline__ void kread_block(uint32_t kbase, const uint32_t (&koff)[D / 16],
                                            bf16x8 (&kf)[D / 16]) {
  constexpr int NC = D / 16;
  constexpr int OFF = BASE + KB * 64 * D;
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  uint32_t a[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) a[cc] = kbase + koff[cc];
  if constexpr (NC == 8) kread8<OFF>(a, kf);
  else if constexpr (NC == 4) kread4<OFF>(a, kf);
  else kread2<OFF>(a, kf);
}
template <int D, int NB, int BASE = 0>
__device__ __forceinline__ void qk_blocks(uint32_t kbase, const uint32_t (&koff)[D / 16],
                                          const bf16x8 (&qf)[D / 16], f32x16 (&sc)[NB],
                                          int want) {
  constexpr int NC = D / 16;
  bf16x8 kf[NC];
  if (want & 1) {
    kread_block<D, 0, BASE>(kbase, koff, kf);
    f32x16 acc = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) acc = mfma32(kf[cc], qf[cc], acc);
    sc[0] = acc;
  }
  if constexpr (NB > 1) {
    if (want & 2) {
      kread_block<D, 1, BASE>(kbase, koff, kf);
      f32x16 acc = zero16();
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) acc = mfma32(kf[cc], qf[cc], acc);
      sc[1] = acc;
    }
  }
}

__device__ __forceinline__ bf16x8 join_bf16(long lo, long hi) {
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane byte offsets, inside a swizzled V tile, of the two transposing reads that
// give lane l its V^T operand for keys [0, 16) and head dims [32*db, 32*db + 32); the
// operands of keys [16j, 16j + 16) sit 32*D*j bytes further (rows 16 apart share the
// swizzle).  Lane l receives V[k][32*db + l%32] for the eight keys k = 4*(l/32) +
// {0,1,2,3} and 8 + 4*(l/32) + {0,1,2,3} of the 16, the key order of the P^T operand
// taken from the 32x32 S^T accumulator.
template <int D>
__device__ __forceinline__ void vt_offsets(int lane, uint32_t (&offA)[D / 32],
                                           uint32_t (&offB)[D / 32]) {
  const int g = lane >> 5;
  const int s = lane & 15;
  const int r_a = (g << 2) + (s >> 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int col = db * 32 + (((lane >> 4) & 1) << 4) + ((s & 3) << 2);
    offA[db] = 2u * (uint32_t)tile_off<D>(r_a, col);
    offB[db] = 2u * (uint32_t)tile_off<D>(r_a + 8, col);
  }
}


// V^T operands of a 32-key tile: vf[j][db] covers keys [16j, 16j + 16), j = 0, 1.
template <int D, int BASE = 0>
__device__ __forceinline__ void read_vt_tile32(uint32_t vbase, const uint32_t (&offA)[D / 32],
                                               const uint32_t (&offB)[D / 32],
                                               bf16x8 (&vf)[2][D / 32]) {
  constexpr int NDB = D / 32;
  constexpr int OFF = 32 * D;
  static_assert(BASE >= 0 && BASE + OFF < 65536, "LDS offset field is 16 bits");
  if constexpr (NDB == 1) {
    const uint32_t a[2] = {vbase + offA[0], vbase + offB[0]};
    long o[4];
    tr_reads<BASE, BASE + OFF>(a, o);
    vf[0][0] = join_bf16(o[0], o[2]);
    vf[1][0] = join_bf16(o[1], o[3]);
  } else if constexpr (NDB == 2) {
    const uint32_t a[4] = {vbase + offA[0], vbase + offB[0], vbase + offA[1], vbase + offB[1]};
    long o[8];
    tr_reads<BASE, BASE + OFF>(a, o);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      vf[0][db] = join_bf16(o[4 * db], o[4 * db + 2]);
      vf[1][db] = join_bf16(o[4 * db + 1], o[4 * db + 3]);
    }
  } else {
    const uint32_t a[8] = {vbase + offA[0], vbase + offB[0], vbase + offA[1], vbase + offB[1],
                           vbase + offA[2], vbase + offB[2], vbase + offA[3], vbase + offB[3]};
    long o[16];
    tr_reads<BASE, BASE + OFF>(a, o);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      vf[0][db] = join_bf16(o[4 * db], o[4 * db + 2]);
      vf[1][db] = join_bf16(o[4 * db + 1], o[4 * db + 3]);
    }
  }
}

// O^T += V^T P^T for one 32-key block whose V rows start at LDS byte address
// vbase + BASE; pb holds the block's P^T operands (exp_pack).
template <int D, int BASE>
__device__ __forceinline__ void pv_block(uint32_t vbase, const uint32_t (&offA)[D / 32],
                                         const uint32_t (&offB)[D / 32], const bf16x8 (&pb)[2],
                                         f32x16 (&o)[D / 32]) {
  bf16x8 vf[2][D / 32];
  read_vt_tile32<D, BASE>(vbase, offA, offB, vf);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = mfma32(vf[h][db], pb[h], o[db]);
}

// A compile-time int carried as a value (selects a template branch from a loop body).
template <int N>
struct IntC {
  static constexpr int value = N;
};


// LDS byte address of an LDS pointer.
__device__ __forceinline__ uint32_t lds_addr(const void E2D2_LDS* p) {
  return (uint32_t)(uintptr_t)p;
}


// ---------------------------------------------------------------------------------
// Direct-to-LDS loads issued from inline asm, and LDS operand reads left to the
// compiler.  With the builtin buffer_load ... lds the compiler sees an LDS write in
// flight and waits for every outstanding load (s_waitcnt vmcnt(0)) before any LDS read
// it can see, which serialises the prefetch.  Issued from asm (no output registers: the
// loads write LDS only), the loads are invisible to it; the caller waits for the stage
// it reads with wait_vmem and crosses a barrier.  The reads are then plain LDS loads
// (or the ds_read_b64_tr_b16 builtin) that the compiler schedules against the MFMAs
// with partial lgkmcnt waits.

// Raw buffer descriptor words (base, byte size; reads past the size return zero).
typedef int BufDesc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ BufDesc buf_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  BufDesc r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)((a >> 32) & 0xFFFFu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}
// 16 (dma_lds16) or 4 (dma_lds4) bytes per lane from buffer offset voff + soff into
// LDS at lds + 16 * lane (4 * lane); lds and soff wave-uniform.
// Each call sets m0 (the LDS base of a buffer_load ... lds) itself, with the one wait
// state the ISA requires between an SALU write of m0 and a load that reads it, and
// leaves m0 changed.  The compiler reserves m0 and cannot be told of that (a clobber of a
// reserved register is not honoured), so these helpers go only into kernels where the
// compiler emits no m0 user of its own: no builtin LDS-DMA (TileLoader), no m0-indexed
// register access.  The build enforces this on the generated AMD assembly of every
// kernel (masked_attention_amd/build.py, check_m0) and fails when a kernel holding these
// blocks has any other m0 access.
__device__ __forceinline__ void dma_lds16(BufDesc d, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(d), "s"(soff), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma_lds4(BufDesc d, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(d), "s"(soff), "s"(lds) : "memory");
}
// TileLoader's layout and work split, loads issued with dma_lds16.
template <int D, int ROWS, int NWAVES>
struct TileDma {
  static constexpr int CH = D / 8;
  static constexpr int NI = ROWS * CH / 64;
  static constexpr int NPW = NI / NWAVES;
  static_assert(NI % NWAVES == 0 && ROWS * CH % 64 == 0, "tile does not split evenly");
  uint32_t voff[NPW];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const int slot = (wave + k * NWAVES) * 64 + lane;
      const int r = slot / CH;
      const int lc = (slot % CH) ^ swz<D>(r);
      voff[k] = (uint32_t)(r * D + lc * 8) * 2u;
    }
  }
  __device__ __forceinline__ void load(BufDesc d, int row0, char E2D2_LDS* tile, int wave) const {
#pragma unroll
    for (int k = 0; k < NPW; ++k)
      dma_lds16(d, voff[k], (uint32_t)(row0 * D * 2), lds_addr(tile + (wave + k * NWAVES) * 1024));
  }
};
// 16 bytes at base + off + OFF (compiler-scheduled).
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(const char E2D2_LDS* base, uint32_t off) {
  return *(const bf16x8 E2D2_LDS*)(base + off + OFF);
}
// ds_read_b64_tr_b16 at base + off + OFF (compiler-scheduled).
template <int OFF>
__device__ __forceinline__ long lds_read_tr(const char E2D2_LDS* base, uint32_t off) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 E2D2_LDS*)(base + off + OFF));
  return __builtin_bit_cast(long, v);
}
// V^T operands of one 16-key half H of a 32-key block (vt_offsets' key order) with
// compiler-scheduled reads: vf[db] covers head dims [32*db, 32*db + 32).
template <int D, int BASE, int H>
__device__ __forceinline__ void read_vt_half32_lds(const char E2D2_LDS* base,
                                                   const uint32_t (&offA)[D / 32],
                                                   const uint32_t (&offB)[D / 32],
                                                   bf16x8 (&vf)[D / 32]) {
  constexpr int O = BASE + H * 32 * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vf[db] = join_bf16(lds_read_tr<O>(base, offA[db]), lds_read_tr<O>(base, offB[db]));
}

}  // namespace e2d2

// Denoising-step attention of E2D2 on gfx950, and the KV-cache append.
//
// Pages cited, by title and section:
//   [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
//             Inference", Paper-Notes page, 方法详解 §3 采样算法: every denoising step of
//             a block calls only the light decoder, whose queries (the S tokens of the
//             [MASK] block) attend the encoder's KV cache of the clean prefix plus the
//             block itself; once the block is finished it goes through the encoder,
//             which appends its KV to the cache.
//   [Summary] ai.info "AI summary" page, "Methodology in Plain English": the decoder
//             runs many times against an unchanged encoder cache.
//
// The step is bound by HBM: it streams the whole cache once per step while the
// queries are few.  Design:
//   * One workgroup serves one (batch, kv head) and up to two 32-row column blocks of
//     the queries that read that kv head (grouped query heads share one K/V stream),
//     so every cached K/V byte is read from HBM once per step.
//   * The key axis (cache rows [0, C), then the block's own S keys) is cut into
//     32-key tiles.  The 4 waves of a workgroup take every 4th tile and stream them
//     independently (no barrier in the loop) through a wave-private, double-buffered
//     LDS stage filled by buffer_load_dwordx4 ... lds, so each wave keeps one tile in
//     flight while it computes the other.
//   * Per tile: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with an
//     online base-2 softmax with lazy rescaling, as in the training kernel; only
//     ragged tile ends mask.
//   * The 4 waves' partial (max, sum, O) are merged in LDS, in a fixed order.  When
//     there are too few (batch, kv head) items to fill the GPU, the key axis is also
//     split over workgroups; each split writes its partial to the workspace and a
//     small combine kernel merges them (same fixed order, so results are
//     deterministic).
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace e2d2 {
namespace {

constexpr int kTN = 32;     // keys per tile
constexpr int kNQB = 2;     // column blocks (32 query rows each) per workgroup
constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(256) void denoise_bf16_kernel(DenoiseParams p) {
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = kTN * D;            // elements of one K or V tile
  constexpr int NI = kTN * (D / 8) / 64;   // load instructions per K (or V) tile
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  // ---- work item
  int w = blockIdx.x;
  const int split = w % p.n_split;
  w /= p.n_split;
  const int qg = w % p.n_qgroups;
  const int bhk = w / p.n_qgroups;
  const int b = bhk / p.Hkv;
  const int hk = bhk % p.Hkv;
  const int S = p.S, C = p.C;

  // column blocks served by this workgroup
  int cb_valid[kNQB], cb_hq[kNQB], cb_r0[kNQB];
#pragma unroll
  for (int i = 0; i < kNQB; ++i) {
    const int cbg = qg * kNQB + i;
    cb_valid[i] = cbg < p.ncb;
    const int hh = cb_valid[i] ? cbg / p.nrc : 0;
    cb_hq[i] = hk * p.g + hh;
    cb_r0[i] = cb_valid[i] ? (cbg % p.nrc) * 32 : 0;
  }

  // ---- key tiles of this split
  const int t_begin = (int)((long long)p.n_tiles * split / p.n_split);
  const int t_end = (int)((long long)p.n_tiles * (split + 1) / p.n_split);

  const size_t kv_bh = (size_t)b * p.Hkv + hk;
  const __amdgpu_buffer_rsrc_t rkc = make_rsrc(p.k_cache + kv_bh * (size_t)p.cap * D, (uint32_t)C * D * 2u);
  const __amdgpu_buffer_rsrc_t rvc = make_rsrc(p.v_cache + kv_bh * (size_t)p.cap * D, (uint32_t)C * D * 2u);
  const __amdgpu_buffer_rsrc_t rkb = make_rsrc(p.k_blk + kv_bh * (size_t)S * D, (uint32_t)S * D * 2u);
  const __amdgpu_buffer_rsrc_t rvb = make_rsrc(p.v_blk + kv_bh * (size_t)S * D, (uint32_t)S * D * 2u);
  TileLoader<D, kTN, 1> loader;  // each wave loads its own tiles
  loader.init(0, lane);

  char E2D2_LDS* my = (char E2D2_LDS*)smem_raw + wave * (2 * 2 * TILE * 2);  // [stage][K, V]
  auto issue = [&](int t, int stage) {
    char E2D2_LDS* kt = my + stage * 2 * TILE * 2;
    if (t < p.n_tiles_cache) {
      loader.load(rkc, t * kTN, kt, 0);
      loader.load(rvc, t * kTN, kt + TILE * 2, 0);
    } else {
      loader.load(rkb, (t - p.n_tiles_cache) * kTN, kt, 0);
      loader.load(rvb, (t - p.n_tiles_cache) * kTN, kt + TILE * 2, 0);
    }
  };
  uint32_t offA[NDB], offB[NDB];
  vt_offsets<D>(lane, offA, offB);
  uint32_t koff[NC];
  k_offsets<D>(lane, koff);
  const uint32_t my0 = lds_addr(my);

  // ---- queries
  bf16x8 qf[kNQB][NC];
#pragma unroll
  for (int i = 0; i < kNQB; ++i) {
    const int r = cb_r0[i] + (lane & 31);
    const bool ok = cb_valid[i] && r < S;
    const __bf16* qrow =
        p.q + (((size_t)b * p.Hq + cb_hq[i]) * S + (ok ? r : 0)) * D + ((lane >> 5) << 3);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      bf16x8 v = *(const bf16x8*)(qrow + cc * 16);
      if (!ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)0.f;
      }
      qf[i][cc] = v;
    }
  }

  f32x16 o[kNQB][NDB];
  float m[kNQB], l[kNQB];  // m: running max in use, base-2 units; l: lane-partial sum
#pragma unroll
  for (int i = 0; i < kNQB; ++i) {
    m[i] = -1e30f;
    l[i] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[i][db] = zero16();
  }
  const float c = p.c;
  const int nq = cb_valid[1] ? 2 : 1;

  // ---- stream this wave's tiles: t_begin + wave, + 4, ...
  const int first = t_begin + wave;
  const int n_my = first < t_end ? (t_end - first + kWaves - 1) / kWaves : 0;
  if (n_my > 0) issue(first, 0);
  for (int i = 0; i < n_my; ++i) {
    const int t = first + i * kWaves;
    if (i + 1 < n_my) {
      issue(t + kWaves, (i + 1) & 1);
      wait_vmem<2 * NI>();
    } else {
      wait_vmem<0>();
    }
    const bool cache = t < p.n_tiles_cache;
    const int k0 = (cache ? t : t - p.n_tiles_cache) * kTN;
    const int n = cache ? C : S;
    const bool ragged = k0 + kTN > n;

    // K operands once per tile, then S^T of every column block back to back.
    const uint32_t kb_addr = my0 + (uint32_t)((i & 1) * 2 * TILE * 2);
    bf16x8 kf[NC];
    kread_block<D, 0>(kb_addr, koff, kf);
    f32x16 sc[kNQB];
#pragma unroll
    for (int qi = 0; qi < kNQB; ++qi) {
      if (qi >= nq) break;
      f32x16 acc = zero16();
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) acc = mfma32(kf[cc], qf[qi][cc], acc);
      sc[qi] = acc;
    }
    bf16x8 vf[2][NDB];
    read_vt_tile32<D>(kb_addr + (uint32_t)(TILE * 2), offA, offB, vf);

#pragma unroll
    for (int qi = 0; qi < kNQB; ++qi) {
      if (qi >= nq) break;
      if (ragged) {
        const int kr = k0 + ((lane >> 5) << 2);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (kr + ((j >> 2) << 3) + (j & 3) >= n) sc[qi][j] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[qi][j]);
      // lazy, per-row rescale: keep the running max unless the row max grew by > 2^8
      const float rmax = pair_max(mx);
      const bool need = rmax * c > m[qi] + 8.f;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        if (need) {
          const float m_new = rmax * c;
          const float alpha = fast_exp2(m[qi] - m_new);
          l[qi] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[qi][db][j] *= alpha;
          m[qi] = m_new;
        }
      }
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(fmaf(sc[qi][j], c, -m[qi]));
        sc[qi][j] = e;
        rs += e;
      }
      l[qi] += rs;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 pb = to_bf16x8(sc[qi][h * 8], sc[qi][h * 8 + 1], sc[qi][h * 8 + 2],
                                    sc[qi][h * 8 + 3], sc[qi][h * 8 + 4], sc[qi][h * 8 + 5],
                                    sc[qi][h * 8 + 6], sc[qi][h * 8 + 7]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[qi][db] = mfma32(vf[h][db], pb, o[qi][db]);
      }
    }
  }

  // ---- merge the 4 waves' partials in LDS (fixed order)
  __syncthreads();  // every wave is done with its stream buffers
  float* mw = (float*)smem_raw;                  // [wave][cb][32]   max (base-2 units)
  float* lw = mw + kWaves * kNQB * 32;           // [wave][cb][64]   lane-partial sums
  float* ow = lw + kWaves * kNQB * 64;           // [wave][cb*32 + row][D]
  const int row = lane & 31;
#pragma unroll
  for (int qi = 0; qi < kNQB; ++qi) {
    const float ms = n_my > 0 ? m[qi] : -INFINITY;
    if (lane < 32) mw[(wave * kNQB + qi) * 32 + row] = ms;
    lw[(wave * kNQB + qi) * 64 + lane] = n_my > 0 ? l[qi] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < kNQB; ++qi) {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, mw[(v * kNQB + qi) * 32 + row]);
    const float mine = mw[(wave * kNQB + qi) * 32 + row];
    const float f = mine == -INFINITY ? 0.f : fast_exp2(mine - M);
    float* dst = ow + ((size_t)wave * kNQB * 32 + qi * 32 + row) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = db * 32 + jg * 8 + ((lane >> 5) << 2);
        f32x4 v;
        v[0] = o[qi][db][jg * 4 + 0] * f;
        v[1] = o[qi][db][jg * 4 + 1] * f;
        v[2] = o[qi][db][jg * 4 + 2] * f;
        v[3] = o[qi][db][jg * 4 + 3] * f;
        *(f32x4*)(dst + d) = v;
      }
  }
  __syncthreads();

  // every thread: rows r = 0..63 of the workgroup, head dims in steps of 4
  if (p.visits != nullptr && threadIdx.x == 0)
    atomicAdd(p.visits, (unsigned long long)(t_end - t_begin) * nq);
  const size_t unit = ((size_t)b * p.Hkv + hk) * p.n_qgroups + qg;
  for (int e = threadIdx.x; e < kNQB * 32 * (D / 4); e += 256) {
    const int r = e / (D / 4);
    const int d = (e % (D / 4)) * 4;
    const int qi = r >> 5, rr = r & 31;
    const int grow = cb_r0[qi] + rr;
    if (!cb_valid[qi] || grow >= S) continue;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, mw[(v * kNQB + qi) * 32 + rr]);
    float lt = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = mw[(v * kNQB + qi) * 32 + rr];
      const float f = mv == -INFINITY ? 0.f : fast_exp2(mv - M);
      lt += (lw[(v * kNQB + qi) * 64 + rr] + lw[(v * kNQB + qi) * 64 + rr + 32]) * f;
      const f32x4 x = *(const f32x4*)(ow + ((size_t)v * kNQB * 32 + r) * D + d);
      acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
    }
    if (p.n_split == 1) {
      const float inv = 1.f / lt;
      bf16x4 ov;
      ov[0] = (__bf16)(acc[0] * inv);
      ov[1] = (__bf16)(acc[1] * inv);
      ov[2] = (__bf16)(acc[2] * inv);
      ov[3] = (__bf16)(acc[3] * inv);
      const size_t orow = ((size_t)b * p.Hq + cb_hq[qi]) * S + grow;
      *(bf16x4*)(p.o + orow * D + d) = ov;
      if (d == 0 && p.lse != nullptr) p.lse[orow] = (M + __log2f(lt)) * 0.6931471805599453f;
    } else {
      const size_t prow = (unit * p.n_split + split) * (kNQB * 32) + r;
      *(f32x4*)(p.ws_o + prow * D + d) = acc;
      if (d == 0) {
        p.ws_ml[prow * 2 + 0] = M;
        p.ws_ml[prow * 2 + 1] = lt;
      }
    }
  }
}

// Merge of the split partials: one workgroup per (batch, kv head, query group).
template <int D>
__global__ __launch_bounds__(256) void denoise_combine_kernel(DenoiseParams p) {
  const int unit = blockIdx.x;
  const int qg = unit % p.n_qgroups;
  const int bhk = unit / p.n_qgroups;
  const int b = bhk / p.Hkv, hk = bhk % p.Hkv;
  const int S = p.S;
  for (int e = threadIdx.x; e < kNQB * 32 * (D / 4); e += 256) {
    const int r = e / (D / 4);
    const int d = (e % (D / 4)) * 4;
    const int qi = r >> 5, rr = r & 31;
    const int cbg = qg * kNQB + qi;
    if (cbg >= p.ncb) continue;
    const int grow = (cbg % p.nrc) * 32 + rr;
    if (grow >= S) continue;
    const int hq = hk * p.g + cbg / p.nrc;
    float M = -INFINITY;
    for (int s = 0; s < p.n_split; ++s)
      M = fmaxf(M, p.ws_ml[(((size_t)unit * p.n_split + s) * (kNQB * 32) + r) * 2]);
    float lt = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.n_split; ++s) {
      const size_t prow = ((size_t)unit * p.n_split + s) * (kNQB * 32) + r;
      const float ms = p.ws_ml[prow * 2];
      const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      lt += p.ws_ml[prow * 2 + 1] * f;
      const f32x4 x = *(const f32x4*)(p.ws_o + prow * D + d);
      acc[0] += x[0] * f; acc[1] += x[1] * f; acc[2] += x[2] * f; acc[3] += x[3] * f;
    }
    const float inv = 1.f / lt;
    bf16x4 ov;
    ov[0] = (__bf16)(acc[0] * inv);
    ov[1] = (__bf16)(acc[1] * inv);
    ov[2] = (__bf16)(acc[2] * inv);
    ov[3] = (__bf16)(acc[3] * inv);
    const size_t orow = ((size_t)b * p.Hq + hq) * S + grow;
    *(bf16x4*)(p.o + orow * D + d) = ov;
    if (d == 0 && p.lse != nullptr) p.lse[orow] = (M + __log2f(lt)) * 0.6931471805599453f;
  }
}

template <int D>
size_t denoise_smem() {
  const size_t stream = (size_t)kWaves * 2 * 2 * kTN * D * sizeof(__bf16);
  const size_t merge = (size_t)kWaves * kNQB * (32 + 64) * sizeof(float) +
                       (size_t)kWaves * kNQB * 32 * D * sizeof(float);
  return stream > merge ? stream : merge;
}

template <int D>
hipError_t launch_denoise_d(const DenoiseParams& p, hipStream_t stream) {
  const size_t smem = denoise_smem<D>();
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)denoise_bf16_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  const long long units = (long long)p.B * p.Hkv * p.n_qgroups;
  hipLaunchKernelGGL(denoise_bf16_kernel<D>, dim3((unsigned)(units * p.n_split)), dim3(256),
                     smem, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL(denoise_combine_kernel<D>, dim3((unsigned)units), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Bitwise copy of the new block's K and V rows into the caches, 16 bytes per lane.
__global__ __launch_bounds__(256) void kv_append_kernel(int row_bytes, int S, int BH,
                                                        char* k_cache, char* v_cache,
                                                        long long cache_len, long long cap,
                                                        const char* k_new, const char* v_new) {
  const int per_row = row_bytes / 16;
  const long long per_tensor = (long long)BH * S * per_row;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * per_tensor;
       i += (long long)gridDim.x * blockDim.x) {
    const bool is_v = i >= per_tensor;
    const long long j = is_v ? i - per_tensor : i;
    const int ch = (int)(j % per_row);
    const long long rs = j / per_row;  // (bh, s)
    const int s = (int)(rs % S);
    const long long bh = rs / S;
    const char* src = (is_v ? v_new : k_new) + (rs * per_row + ch) * 16;
    char* dst = (is_v ? v_cache : k_cache) + ((bh * cap + cache_len + s) * per_row + ch) * 16;
    *(int4*)dst = *(const int4*)src;
  }
}

}  // namespace

int denoise_splits(int B, int Hkv, int n_qgroups, int n_tiles) {
  const long long units = (long long)B * Hkv * n_qgroups;
  const long long target = 256;  // one workgroup per compute unit
  if (units >= target || n_tiles <= 2 * kWaves) return 1;
  long long s = (target + units - 1) / units;
  const long long max_s = n_tiles / (2 * kWaves);  // keep >= 2 tiles per wave
  if (s > max_s) s = max_s;
  return s < 1 ? 1 : (int)s;
}

hipError_t launch_denoise_bf16(const DenoiseParams& p, int d, hipStream_t stream) {
  if ((long long)p.B * p.Hkv * p.n_qgroups == 0) return hipSuccess;
  switch (d) {
    case 32: return launch_denoise_d<32>(p, stream);
    case 64: return launch_denoise_d<64>(p, stream);
    case 128: return launch_denoise_d<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kv_append(int elem_bytes, int B, int Hkv, int S, int d, void* k_cache,
                            void* v_cache, long long cache_len, long long cap, const void* k_new,
                            const void* v_new, hipStream_t stream) {
  const int row_bytes = d * elem_bytes;
  const long long total = 2ll * B * Hkv * S * (row_bytes / 16);
  if (total == 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, row_bytes, S,
                     B * Hkv, (char*)k_cache, (char*)v_cache, cache_len, cap,
                     (const char*)k_new, (const char*)v_new);
  return hipGetLastError();
}

}  // namespace e2d2

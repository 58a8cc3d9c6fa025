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
//     32-key tiles.  The 8 waves of a workgroup form 4 pairs; pair p takes every 4th
//     tile (p, p + 4, ...) and streams it through its own double-buffered LDS ring
//     filled by buffer_load_dwordx4 ... lds (each wave of the pair loads half of the
//     tile), and each wave of the pair computes one of the two column blocks against
//     it.  One workgroup barrier per round (all pairs step together) publishes the
//     round's tiles and frees the other stage; the next round's tiles are in flight
//     while the current one is computed.  One column block per wave keeps the
//     accumulators within 256 registers, so two waves share each SIMD.
//   * Per tile: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with an
//     online base-2 softmax with lazy rescaling, as in the training kernel; only
//     ragged tile ends mask.
//   * The 4 pairs' partial (max, sum, O) are merged in LDS, in a fixed order.  When
//     there are too few (batch, kv head) items to fill the GPU, the key axis is also
//     split over workgroups; each split writes its partial to the workspace and a
//     small combine kernel merges them (same fixed order, so results are
//     deterministic).
#include <mutex>

#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace e2d2 {
namespace {

constexpr int kTN = 32;     // keys per tile
constexpr int kNQB = 2;     // column blocks (32 query rows each) per workgroup
constexpr int kPairs = 4;   // key lanes: lane pair p streams tiles p, p + 4, ... of its split
constexpr int kWaves = kPairs * kNQB;  // wave = 2 * pair + column block
constexpr int kThreads = kWaves * 64;
constexpr float kBound = 65536.f;      // lane sum of a block's numerators forcing a rescale
constexpr float kNegBig = -1e30f;      // "no key yet" running max
// Row pitch (floats) of the partial O rows merged in LDS: padded by 4 so that the 32
// rows one wave writes (one per lane) spread over the banks instead of sharing one.
template <int D>
constexpr int kOPitch = D + 4;

template <int D>
__global__ __launch_bounds__(kThreads) void denoise_bf16_kernel(DenoiseParams p) {
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = kTN * D;            // elements of one K or V tile
  constexpr int RING = 2 * 2 * TILE * 2;   // bytes of a pair's ring: 2 stages x (K, V)
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int pair = wave >> 1;
  const int qi = wave & 1;  // this wave's column block within the workgroup

  // ---- work item
  int w = blockIdx.x;
  const int split = w % p.n_split;
  w /= p.n_split;
  const int qg = w % p.n_qgroups;
  const int bhk = w / p.n_qgroups;
  const int b = bhk / p.Hkv;
  const int hk = bhk % p.Hkv;
  const int S = p.S;
  // this sequence's cache length (per-sequence lengths live on the device, so one
  // captured launch serves every step of a decode loop)
  const int C = p.lens != nullptr ? min(max(p.lens[b], 0), p.C) : p.C;
  const int tiles_c = (C + kTN - 1) / kTN;  // cache tiles of this sequence (<= n_tiles_cache)

  // this wave's column block: 32 query rows of one query head of the kv head's group
  const int cbg = qg * kNQB + qi;
  const bool cb_valid = cbg < p.ncb;
  const int cb_hq = hk * p.g + (cb_valid ? cbg / p.nrc : 0);
  const int cb_r0 = cb_valid ? (cbg % p.nrc) * 32 : 0;

  // ---- key tiles of this split; pair p takes tiles t_begin + p + 4 r
  const int t_begin = (int)((long long)p.n_tiles * split / p.n_split);
  const int t_end = (int)((long long)p.n_tiles * (split + 1) / p.n_split);
  const int rounds = (t_end - t_begin + kPairs - 1) / kPairs;

  const size_t kv_bh = (size_t)b * p.Hkv + hk;
  const __amdgpu_buffer_rsrc_t rkc = make_rsrc(p.k_cache + kv_bh * (size_t)p.cap * D, (uint32_t)C * D * 2u);
  const __amdgpu_buffer_rsrc_t rvc = make_rsrc(p.v_cache + kv_bh * (size_t)p.cap * D, (uint32_t)C * D * 2u);
  const __amdgpu_buffer_rsrc_t rkb = make_rsrc(p.k_blk + kv_bh * (size_t)S * D, (uint32_t)S * D * 2u);
  const __amdgpu_buffer_rsrc_t rvb = make_rsrc(p.v_blk + kv_bh * (size_t)S * D, (uint32_t)S * D * 2u);
  TileLoader<D, kTN, 2> loader;  // the two waves of a pair load half of each tile
  loader.init(qi, lane);

  char E2D2_LDS* ring = (char E2D2_LDS*)smem_raw + pair * RING;
  // tile t holds keys of this sequence: a cache tile below its length, or an own-block tile
  auto live = [&](int t) { return t < p.n_tiles_cache ? t < tiles_c : true; };
  auto issue = [&](int t, int stage) {
    char E2D2_LDS* kt = ring + stage * 2 * TILE * 2;
    if (t < p.n_tiles_cache) {
      loader.load(rkc, t * kTN, kt, qi);
      loader.load(rvc, t * kTN, kt + TILE * 2, qi);
    } else {
      loader.load(rkb, (t - p.n_tiles_cache) * kTN, kt, qi);
      loader.load(rvb, (t - p.n_tiles_cache) * kTN, kt + TILE * 2, qi);
    }
  };
  uint32_t offA[NDB], offB[NDB];
  vt_offsets<D>(lane, offA, offB);
  uint32_t koff[NC];
  k_offsets<D>(lane, koff);
  const uint32_t ring0 = lds_addr(ring);

  // ---- queries of this wave's column block
  bf16x8 qf[NC];
  {
    const int r = cb_r0 + (lane & 31);
    const bool ok = cb_valid && r < S;
    const __bf16* qrow = p.q + (((size_t)b * p.Hq + cb_hq) * S + (ok ? r : 0)) * D + ((lane >> 5) << 3);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      bf16x8 v = *(const bf16x8*)(qrow + cc * 16);
      if (!ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)0.f;
      }
      qf[cc] = v;
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = zero16();
  float m = kNegBig;  // running max in use, base-2 units
  float l = 0.f;      // lane-partial sum of the bf16 numerators
  const float c = p.c;

  // One tile from ring stage STG (a constant: the LDS reads carry it in their offset).
  auto tile = [&](int t, auto stg) {
    constexpr int KOFF = decltype(stg)::value * 2 * TILE * 2;
    constexpr int VOFF = KOFF + TILE * 2;
    const bool cache = t < p.n_tiles_cache;
    const int k0 = (cache ? t : t - p.n_tiles_cache) * kTN;
    const int n = cache ? C : S;
    f32x16 sc[1];
    qk_blocks<D, 1, KOFF>(ring0, koff, qf, sc, 1);
    if (k0 + kTN > n) {  // ragged end of the cache or of the block
      const int kr = k0 + ((lane >> 5) << 2);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kr + ((j >> 2) << 3) + (j & 3) >= n) sc[0][j] = -INFINITY;
    }
    bf16x8 pb[2];
    float rs = exp_pack(sc[0], c, -m, pb, 0.f);
    if (__builtin_amdgcn_ballot_w64(rs > kBound) != 0) {
      // rare: a row's numerators outgrew the bound (its first keys, or a new max)
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[0][j]);
      const float rmax = pair_max(mx);
      const bool need = pair_max(rs > kBound ? 1.f : 0.f) > 0.f;
      if (need) {
        const float m_new = rmax * c;
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        m = m_new;
      }
      rs = exp_pack(sc[0], c, -m, pb, 0.f);
    }
    l += rs;
    pv_block<D, VOFF>(ring0, offA, offB, pb, o);
  };

  // ---- rounds: all pairs step together; one barrier per round makes the pair's
  //      tile (loaded half by each wave) visible and frees the other stage
  const int first = t_begin + pair;
  if (first < t_end && live(first)) issue(first, 0);
  int done = 0;  // tiles this wave computed
  auto round = [&](int r, auto stg) {
    constexpr int STG = decltype(stg)::value;
    const int t = first + r * kPairs;
    wait_vmem<0>();  // this wave's part of round r landed (nothing else is in flight)
    __syncthreads();
    if (t + kPairs < t_end && live(t + kPairs)) issue(t + kPairs, 1 - STG);
    if (t < t_end && live(t) && cb_valid) {
      tile(t, IntC<STG>{});
      ++done;
    }
  };
  for (int r = 0; r < rounds; r += 2) {
    round(r, IntC<0>{});
    if (r + 1 < rounds) round(r + 1, IntC<1>{});
  }
  const bool had = done > 0;

  // ---- merge the 4 pairs' partials per column block in LDS (fixed order)
  __syncthreads();  // every wave is done with the rings
  float* mw = (float*)smem_raw;             // [pair][cb][32]   max (base-2 units)
  float* lw = mw + kPairs * kNQB * 32;      // [pair][cb][64]   lane-partial sums
  float* ow = lw + kPairs * kNQB * 64;      // [pair][cb*32 + row][D]
  const int row = lane & 31;
  {
    const float ms = had ? m : -INFINITY;
    if (lane < 32) mw[(pair * kNQB + qi) * 32 + row] = ms;
    lw[(pair * kNQB + qi) * 64 + lane] = had ? l : 0.f;
  }
  __syncthreads();
  {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kPairs; ++v) M = fmaxf(M, mw[(v * kNQB + qi) * 32 + row]);
    const float mine = mw[(pair * kNQB + qi) * 32 + row];
    const float f = mine == -INFINITY ? 0.f : fast_exp2(mine - M);
    float* dst = ow + ((size_t)pair * kNQB * 32 + qi * 32 + row) * kOPitch<D>;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = db * 32 + jg * 8 + ((lane >> 5) << 2);
        f32x4 v;
        v[0] = o[db][jg * 4 + 0] * f;
        v[1] = o[db][jg * 4 + 1] * f;
        v[2] = o[db][jg * 4 + 2] * f;
        v[3] = o[db][jg * 4 + 3] * f;
        *(f32x4*)(dst + d) = v;
      }
  }
  __syncthreads();

  // every thread: rows r = 0..63 of the workgroup, head dims in steps of 4
  if (p.visits != nullptr && lane == 0 && done > 0) atomicAdd(p.visits, (unsigned long long)done);
  const size_t unit = ((size_t)b * p.Hkv + hk) * p.n_qgroups + qg;
  for (int e = threadIdx.x; e < kNQB * 32 * (D / 4); e += kThreads) {
    const int r = e / (D / 4);
    const int d = (e % (D / 4)) * 4;
    const int cq = r >> 5, rr = r & 31;
    const int cg = qg * kNQB + cq;
    if (cg >= p.ncb) continue;
    const int grow = (cg % p.nrc) * 32 + rr;
    if (grow >= S) continue;
    const int hq = hk * p.g + cg / p.nrc;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kPairs; ++v) M = fmaxf(M, mw[(v * kNQB + cq) * 32 + rr]);
    float lt = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < kPairs; ++v) {
      const float mv = mw[(v * kNQB + cq) * 32 + rr];
      const float f = mv == -INFINITY ? 0.f : fast_exp2(mv - M);
      lt += (lw[(v * kNQB + cq) * 64 + rr] + lw[(v * kNQB + cq) * 64 + rr + 32]) * f;
      const f32x4 x = *(const f32x4*)(ow + ((size_t)v * kNQB * 32 + r) * kOPitch<D> + d);
      acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
    }
    if (p.n_split == 1) {
      const float inv = 1.f / lt;
      bf16x4 ov;
      ov[0] = (__bf16)(acc[0] * inv);
      ov[1] = (__bf16)(acc[1] * inv);
      ov[2] = (__bf16)(acc[2] * inv);
      ov[3] = (__bf16)(acc[3] * inv);
      const size_t orow = ((size_t)b * p.Hq + hq) * S + grow;
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
  const size_t stream = (size_t)kPairs * 2 * 2 * kTN * D * sizeof(__bf16);
  const size_t merge = (size_t)kPairs * kNQB * (32 + 64) * sizeof(float) +
                       (size_t)kPairs * kNQB * 32 * kOPitch<D> * sizeof(float);
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
  hipLaunchKernelGGL(denoise_bf16_kernel<D>, dim3((unsigned)(units * p.n_split)), dim3(kThreads),
                     smem, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL(denoise_combine_kernel<D>, dim3((unsigned)units), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Bitwise copy of the new block's K and V rows into the caches, 16 bytes per lane.
// Workgroup = (sequence-head bh, 256 16-byte chunks of its S rows); row s of bh goes to
// cache row len + s, with len = cache_len, or lens[b] when lens is given (a sequence
// whose length is outside [0, max_len] is left untouched).  Chunks per row are a power
// of two, so the index arithmetic is shifts and masks.
__global__ __launch_bounds__(256) void kv_append_kernel(int per_row_log2, int S, int Hkv,
                                                        int blocks_per_bh, int4* k_cache,
                                                        int4* v_cache, long long cache_len,
                                                        long long max_len, long long cap,
                                                        const int4* k_new, const int4* v_new,
                                                        const int* lens) {
  const int bh = blockIdx.x / blocks_per_bh;  // uniform
  const int j = (blockIdx.x - bh * blocks_per_bh) * 256 + threadIdx.x;
  if (j >= (S << per_row_log2)) return;
  long long len = cache_len;
  if (lens != nullptr) {
    len = lens[bh / Hkv];
    if (len < 0 || len > max_len) return;
  }
  const int s = j >> per_row_log2;
  const int ch = j & ((1 << per_row_log2) - 1);
  const size_t src = (((size_t)bh * S + s) << per_row_log2) + ch;
  const size_t dst = (((size_t)bh * cap + len + s) << per_row_log2) + ch;
  k_cache[dst] = k_new[src];
  v_cache[dst] = v_new[src];
}

hipError_t launch_append(int elem_bytes, int B, int Hkv, int S, int d, void* k_cache,
                         void* v_cache, long long cache_len, const int* lens, long long max_len,
                         long long cap, const void* k_new, const void* v_new, hipStream_t stream) {
  const int per_row = d * elem_bytes / 16;
  int log2 = 0;
  while ((1 << log2) < per_row) ++log2;
  if ((1 << log2) != per_row) return hipErrorInvalidValue;
  const long long bh = (long long)B * Hkv;
  const long long bpb = (((long long)S << log2) + 255) / 256;
  if (bh * bpb == 0) return hipSuccess;
  if (bh * bpb > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)(bh * bpb)), dim3(256), 0, stream, log2, S,
                     Hkv, (int)bpb, (int4*)k_cache, (int4*)v_cache, cache_len, max_len, cap,
                     (const int4*)k_new, (const int4*)v_new, lens);
  return hipGetLastError();
}

// Device scratch of the allocation-free denoise call: the split partials (ws_o, ws_ml)
// live here instead of in a caller workspace.  Its size covers every shape: a split is
// used only when units = B * Hkv * query groups < 256, with at most ceil(256 / units)
// splits, so units * splits <= 510 and the workspace holds at most 510 * 64 rows of
// d + 2 <= 130 floats (16.97 MB).  Each GPU the library runs on holds its own copy until
// the process ends.
constexpr size_t kScratchBytes = (size_t)17 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t denoise_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // The host-side name `scratch` is not a device address: the runtime gives the
    // address of this device's copy.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

int denoise_splits(int B, int Hkv, int n_qgroups, int n_tiles) {
  const long long units = (long long)B * Hkv * n_qgroups;
  const long long target = 256;  // one workgroup per compute unit
  if (units >= target || n_tiles <= 2 * kPairs) return 1;
  long long s = (target + units - 1) / units;
  const long long max_s = n_tiles / (2 * kPairs);  // keep >= 2 tiles per key lane
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
  return launch_append(elem_bytes, B, Hkv, S, d, k_cache, v_cache, cache_len, nullptr, cache_len,
                       cap, k_new, v_new, stream);
}

hipError_t launch_kv_append_varlen(int elem_bytes, int B, int Hkv, int S, int d, void* k_cache,
                                   void* v_cache, const int* lens, long long max_len, long long cap,
                                   const void* k_new, const void* v_new, hipStream_t stream) {
  return launch_append(elem_bytes, B, Hkv, S, d, k_cache, v_cache, 0, lens, max_len, cap, k_new,
                       v_new, stream);
}

}  // namespace e2d2

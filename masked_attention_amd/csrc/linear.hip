// Projections of a decoder layer's attention sublayer on gfx950: C = A W^T in bf16
// with fp32 accumulation.
//
// Pages cited, by title and section:
//   [Notes] "Encoder-Decoder Diffusion Language Models for Efficient Training and
//           Inference", Paper-Notes page: 方法详解 §3 采样算法 (each denoising step runs
//           only the small decoder on the block's tokens), §2 两种连接方式 (the decoder
//           layer attends over the encoder's KV cache plus its own block).
//
// One launch computes C[m][n] = sum_k A(m, k) W[n][k] for m < M = B*S (the block's
// tokens), n < N, k < K, where
//   * A(m, k) is gathered: row m = (b, s) of a [B, S, K] activation, or, for the output
//     projection, column k = (h, c) of per-head [B, H, S, w] attention output;
//   * W is an nn.Linear-style [N][K] weight (K contiguous);
//   * C is scattered: column n falls in one of up to three segments (the query, key
//     and value heads of a stacked projection), each written per head as
//     [B, H_seg, S, w], or, with one segment of one "head" of width N, as [B, S, N].
// Tiling: a workgroup of 4 waves owns a (64 NBW) x (64 MBW) tile of C^T (n x m); each
// wave owns NBW x MBW blocks of 32 x 32.  The k axis is walked 64 at a time through a
// 3-deep ring of swizzled LDS stages filled straight from memory (buffer_load ... lds),
// the W and A rows of a stage read with the same swizzle as the attention K tiles.
// Blocks of C^T come from v_mfma_f32_32x32x16_bf16 with W rows as the A operand, so a
// lane holds 4 consecutive n of one m per register group: 8-byte bf16 stores.
#include "device_common.h"
#include "kernels.h"

namespace e2d2 {
namespace {

constexpr int kKS = 64;       // k per stage
constexpr int kLStages = 3;   // ring depth
constexpr int kLWaves = 4;
constexpr int kLThreads = kLWaves * 64;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every record: loads return 0

template <int NBW, int MBW>
struct LinGeo {
  static constexpr int NT = 64 * NBW;            // n rows of W per workgroup
  static constexpr int MT = 64 * MBW;            // m rows of A per workgroup
  static constexpr int W_BYTES = NT * kKS * 2;   // one stage of W
  static constexpr int A_BYTES = MT * kKS * 2;
  static constexpr int STAGE = W_BYTES + A_BYTES;
  static constexpr int NLW = NT * 8 / kLThreads;  // 16-byte loads per thread per stage (W)
  static constexpr int NLA = MT * 8 / kLThreads;  // (A)
  static_assert(NT * 8 % kLThreads == 0 && MT * 8 % kLThreads == 0, "stage does not split");
};

template <int NBW, int MBW>
__global__ __launch_bounds__(kLThreads, 1) void linear_bf16_kernel(LinearParams p) {
  using G = LinGeo<NBW, MBW>;
  constexpr int NLW = G::NLW, NLA = G::NLA, STAGE = G::STAGE;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  char E2D2_LDS* lds_b = (char E2D2_LDS*)smem_raw;
  const uint32_t lds0 = lds_addr(lds_b);

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n_tiles_n = (p.N + G::NT - 1) / G::NT;
  const int n0 = (blockIdx.x % n_tiles_n) * G::NT;
  const int m0 = (blockIdx.x / n_tiles_n) * G::MT;
  const int nk = (p.K + kKS - 1) / kKS;

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);

  // Per-lane load slots.  Load i of this lane fills LDS slot (wave + 4 i) * 64 + lane
  // of the W (or A) part of a stage: row r = slot / 8, physical chunk slot % 8, which
  // holds logical chunk lc = (slot % 8) ^ swz(r), i.e. k = k0 + 8 lc.
  uint32_t w_base[NLW];
  int w_col[NLW];
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int slot = (wave + i * kLWaves) * 64 + lane;
    const int r = slot >> 3;
    const int lc = (slot & 7) ^ swz<kKS>(r);
    const int n = n0 + r;
    w_col[i] = lc * 8;
    w_base[i] = n < p.N ? (uint32_t)((n * p.K + lc * 8) * 2) : kOOB;
  }
  uint32_t a_row[NLA];  // byte offset of row m's element k = 0 (before the head split)
  int a_col[NLA];
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int slot = (wave + i * kLWaves) * 64 + lane;
    const int r = slot >> 3;
    const int lc = (slot & 7) ^ swz<kKS>(r);
    const int m = m0 + r;
    a_col[i] = lc * 8;
    if (m < p.M) {
      const int b = m / p.S, s = m - (m / p.S) * p.S;
      a_row[i] = (uint32_t)((b * p.a_sb + s * p.a_ss) * 2);
    } else {
      a_row[i] = kOOB;
    }
  }
  // Issue stage kt (k0 = 64 kt) into ring slot kt % 3.
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * kKS;
    const int kv = p.K - k0;  // valid k in this stage: lanes with col >= kv read zero
    char E2D2_LDS* st = lds_b + (kt % kLStages) * STAGE;
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const uint32_t off = w_col[i] < kv ? w_base[i] + (uint32_t)(k0 * 2) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (void E2D2_LDS*)(st + (wave + i * kLWaves) * 1024), 16, (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      uint32_t off = kOOB;
      if (a_col[i] < kv && a_row[i] != kOOB) {
        const int k = k0 + a_col[i];
        const int kk = p.a_heads ? ((k >> p.a_log2w) * p.a_sh + (k & ((1 << p.a_log2w) - 1))) : k;
        off = a_row[i] + (uint32_t)(kk * 2);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (void E2D2_LDS*)(st + G::W_BYTES + (wave + i * kLWaves) * 1024), 16, (int)off, 0, 0,
          0);
    }
  };

  // This wave's 32-row blocks: W rows [32 (NBW wn + nb)), A rows [32 (MBW wm + mb)).
  const int wn = wave & 1, wm = wave >> 1;
  uint32_t koff[4];
  k_offsets<kKS>(lane, koff);
  const uint32_t wbase = lds0 + (uint32_t)(wn * NBW * 32 * kKS * 2);
  const uint32_t abase = lds0 + (uint32_t)(G::W_BYTES + wm * MBW * 32 * kKS * 2);

  f32x16 acc[NBW][MBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) acc[nb][mb] = zero16();

  constexpr int NL = NLW + NLA;  // loads per thread per stage
  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  auto step = [&](int kt, auto stg) __attribute__((always_inline)) {
    constexpr int OFF = decltype(stg)::value * STAGE;
    // stage kt landed; stage kt+1 may still be in flight
    if (kt + 1 < nk) wait_vmem<NL>();
    else wait_vmem<0>();
    __syncthreads();
    if (kt + 2 < nk) issue(kt + 2);
    // (stage offsets exceed the 16-bit LDS offset field: added to the base instead)
    const uint32_t wst = wbase + (uint32_t)OFF, ast = abase + (uint32_t)OFF;
    bf16x8 wf[NBW][4], af[MBW][4];
    kread_block<kKS, 0>(wst, koff, wf[0]);
    if constexpr (NBW == 2) kread_block<kKS, 1>(wst, koff, wf[1]);
    kread_block<kKS, 0>(ast, koff, af[0]);
    if constexpr (MBW == 2) kread_block<kKS, 1>(ast, koff, af[1]);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[nb][mb] = mfma32(wf[nb][cc], af[mb][cc], acc[nb][mb]);
  };
  for (int kt = 0; kt < nk; kt += kLStages) {
    step(kt, IntC<0>{});
    if (kt + 1 < nk) step(kt + 1, IntC<1>{});
    if (kt + 2 < nk) step(kt + 2, IntC<2>{});
  }

  // ---- epilogue: register j of block (nb, mb) holds C^T[n][m] with
  //      n = n0 + 32 (NBW wn + nb) + 8 (j / 4) + 4 (lane / 32) + j % 4,
  //      m = m0 + 32 (MBW wm + mb) + lane % 32.
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int m = m0 + 32 * (MBW * wm + mb) + (lane & 31);
    if (m >= p.M) continue;
    const int b = m / p.S, s = m - (m / p.S) * p.S;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int n = n0 + 32 * (NBW * wn + nb) + 8 * jg + 4 * (lane >> 5);
        if (n >= p.N) continue;
        const int seg = n < p.c_n0[1] ? 0 : (n < p.c_n0[2] ? 1 : 2);
        const int nn = n - p.c_n0[seg];
        const int h = nn / p.c_w, c = nn - (nn / p.c_w) * p.c_w;
        __bf16* dst = p.c[seg] + (((size_t)b * p.c_h[seg] + h) * p.S + s) * (size_t)p.c_w + c;
        bf16x4 v;
        v[0] = (__bf16)acc[nb][mb][4 * jg + 0];
        v[1] = (__bf16)acc[nb][mb][4 * jg + 1];
        v[2] = (__bf16)acc[nb][mb][4 * jg + 2];
        v[3] = (__bf16)acc[nb][mb][4 * jg + 3];
        *(bf16x4*)dst = v;
      }
    }
  }
}

template <int NBW, int MBW>
hipError_t launch_linear_t(const LinearParams& p, hipStream_t stream) {
  using G = LinGeo<NBW, MBW>;
  const size_t smem = (size_t)kLStages * G::STAGE;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)linear_bf16_kernel<NBW, MBW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  const long long grid = (long long)((p.N + G::NT - 1) / G::NT) * ((p.M + G::MT - 1) / G::MT);
  hipLaunchKernelGGL((linear_bf16_kernel<NBW, MBW>), dim3((unsigned)grid), dim3(kLThreads), smem,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

// 128 x 128 tiles while they give at least one workgroup per CU (256), else 128 x 64.
hipError_t launch_linear_bf16(const LinearParams& p, hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const long long t128 = (long long)((p.N + 127) / 128) * ((p.M + 127) / 128);
  if (t128 >= 256) return launch_linear_t<2, 2>(p, stream);
  return launch_linear_t<2, 1>(p, stream);
}

}  // namespace e2d2

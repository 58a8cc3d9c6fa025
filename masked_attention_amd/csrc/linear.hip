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
// Tiling: a workgroup of WN x WM waves owns a (32 NBW WN) x (32 MBW WM) tile of C^T
// (n x m); each wave owns NBW x MBW blocks of 32 x 32, formed by
// v_mfma_f32_32x32x16_bf16 with W rows as the A operand.  The k axis is walked 64 at
// a time through an ST-deep ring of swizzled LDS stages (the swizzle of the attention
// K tiles) filled straight from memory by buffer_load_dwordx4 ... lds; ST - 1 stages
// are in flight while one is multiplied.  A step issues its refill halfway through its
// products (measured on MI355X: 2.1% off the decoder-layer step against issuing it
// right after the barrier).  The loads are issued from inline asm and
// their completion is waited for explicitly (s_waitcnt vmcnt) before a bare
// s_barrier: the compiler then neither drains every prefetch at the barrier nor
// before each LDS read, and it schedules the plain C++ LDS reads of the operands
// against the MFMAs itself.  The C tile is staged through LDS on the way out, so the
// global stores are 16 contiguous bytes per lane along n.
#include "device_common.h"
#include "kernels.h"

namespace e2d2 {
namespace {

constexpr int kKS = 64;                  // k per stage
constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every record: loads return 0

// Workgroup shape: WN x WM waves, each owning NBW x MBW blocks of 32 x 32 of C^T; an
// ST-deep ring of k stages.
template <int NBW, int MBW, int WN, int WM, int ST>
struct LinGeo {
  static constexpr int WAVES = WN * WM;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NT = 32 * NBW * WN;       // n rows of W per workgroup
  static constexpr int MT = 32 * MBW * WM;       // m rows of A per workgroup
  static constexpr int W_BYTES = NT * kKS * 2;   // one stage of W
  static constexpr int A_BYTES = MT * kKS * 2;
  static constexpr int STAGE = W_BYTES + A_BYTES;
  static constexpr int NLW = NT * 8 / THREADS;   // 16-byte loads per thread per stage (W)
  static constexpr int NLA = MT * 8 / THREADS;   // (A)
  static_assert(NT * 8 % THREADS == 0 && MT * 8 % THREADS == 0, "stage does not split");
  static_assert(ST >= 2 && ST <= 4, "ring depth");
  static constexpr int CP = NT + 8;              // bf16 row pitch of the C tile staged in LDS
  static constexpr int C_BYTES = MT * CP * 2;
  static constexpr int LDS = ST * STAGE > C_BYTES ? ST * STAGE : C_BYTES;
};

// Wait until at most n (0 <= n < 4, run time) groups of G loads of this wave remain.
template <int G>
__device__ __forceinline__ void wait_groups(int n) {
  if (n >= 3) wait_vmem<3 * G>();
  else if (n == 2) wait_vmem<2 * G>();
  else if (n == 1) wait_vmem<G>();
  else wait_vmem<0>();
}

template <int NBW, int MBW, int WN, int WM, int ST>
__global__ __launch_bounds__(64 * WN * WM, 1) void linear_bf16_kernel(
    LinearParams p) {
  using G = LinGeo<NBW, MBW, WN, WM, ST>;
  constexpr int NLW = G::NLW, NLA = G::NLA, STAGE = G::STAGE, WAVES = G::WAVES;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  char E2D2_LDS* lds_b = (char E2D2_LDS*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n_tiles_n = (p.N + G::NT - 1) / G::NT;
  const int n0 = (blockIdx.x % n_tiles_n) * G::NT;
  const int m0 = (blockIdx.x / n_tiles_n) * G::MT;
  const int nk = (p.K + kKS - 1) / kKS;

  const BufDesc rw = buf_desc(p.w, p.w_bytes);
  const BufDesc ra = buf_desc(p.a, p.a_bytes);

  // Per-lane load slots.  Load i of this lane fills LDS slot (wave + WAVES i) * 64 +
  // lane of the W (or A) part of a stage: row r = slot / 8, physical chunk slot % 8,
  // which holds logical chunk lc = (slot % 8) ^ swz(r), i.e. k = k0 + 8 lc.
  uint32_t w_base[NLW];
  int w_col[NLW];
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int slot = (wave + i * WAVES) * 64 + lane;
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
    const int slot = (wave + i * WAVES) * 64 + lane;
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
  // Issue stage kt (k0 = 64 kt) into ring slot SL = kt % ST (a constant).
  auto issue = [&](int kt, auto slc) __attribute__((always_inline)) {
    constexpr int SL = decltype(slc)::value;
    const int k0 = kt * kKS;
    const int kv = p.K - k0;  // valid k in this stage: lanes with col >= kv read zero
    char E2D2_LDS* st = lds_b + SL * STAGE;
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const uint32_t off = w_col[i] < kv ? w_base[i] + (uint32_t)(k0 * 2) : kOOB;
      dma_lds16(rw, off, 0, lds_addr(st + (wave + i * WAVES) * 1024));
    }
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      uint32_t off = kOOB;
      if (a_col[i] < kv && a_row[i] != kOOB) {
        const int k = k0 + a_col[i];
        const int kk = p.a_heads ? ((k >> p.a_log2w) * p.a_sh + (k & ((1 << p.a_log2w) - 1))) : k;
        off = a_row[i] + (uint32_t)(kk * 2);
      }
      dma_lds16(ra, off, 0, lds_addr(st + G::W_BYTES + (wave + i * WAVES) * 1024));
    }
  };

  // This wave's 32-row blocks: W rows 32 (NBW wn + nb) .., A rows 32 (MBW wm + mb) ..
  const int wn = wave % WN, wm = wave / WN;
  uint32_t koff[4];
  k_offsets<kKS>(lane, koff);
  const int wofs = wn * NBW * 32 * kKS * 2;
  const int aofs = G::W_BYTES + wm * MBW * 32 * kKS * 2;

  f32x16 acc[NBW][MBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) acc[nb][mb] = zero16();

  constexpr int NL = NLW + NLA;  // loads per thread per stage
  if (0 < nk) issue(0, IntC<0>{});
  if (ST > 2 && 1 < nk) issue(1, IntC<1>{});
  if (ST > 3 && 2 < nk) issue(2, IntC<2 % ST>{});
  auto step = [&](int kt, auto stg) __attribute__((always_inline)) {
    // stage kt landed; the stages issued after it (up to ST - 2) may still be in flight
    wait_groups<NL>(min(ST - 2, nk - 1 - kt));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    constexpr int SL = decltype(stg)::value;
    const char E2D2_LDS* stb = lds_b + SL * STAGE;
    bf16x8 wf[NBW][4], af[MBW][4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        wf[nb][cc] = *(const bf16x8 E2D2_LDS*)(stb + wofs + nb * 4096 + koff[cc]);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
        af[mb][cc] = *(const bf16x8 E2D2_LDS*)(stb + aofs + mb * 4096 + koff[cc]);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[nb][mb] = mfma32(wf[nb][cc], af[mb][cc], acc[nb][mb]);
      if (cc == 1) {
        // Refill the slot read in the previous step (every wave left it before the
        // barrier above) once half of this step's products are issued: issued right
        // after the barrier, the loads of all waves delay the first products.
        __builtin_amdgcn_sched_barrier(0);
        if (kt + ST - 1 < nk) issue(kt + ST - 1, IntC<(SL + ST - 1) % ST>{});
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int kt = 0; kt < nk; kt += ST) {
    step(kt, IntC<0>{});
    if (kt + 1 < nk) step(kt + 1, IntC<1>{});
    if constexpr (ST > 2) {
      if (kt + 2 < nk) step(kt + 2, IntC<2 % ST>{});
    }
    if constexpr (ST > 3) {
      if (kt + 3 < nk) step(kt + 3, IntC<3 % ST>{});
    }
  }

  // ---- epilogue: register j of block (nb, mb) holds C^T[n][m] with
  //      n = n0 + 32 (NBW wn + nb) + 8 (j / 4) + 4 (lane / 32) + j % 4,
  //      m = m0 + 32 (MBW wm + mb) + lane % 32.
  //      The tile goes through LDS as C[m][n] (bf16, row pitch CP) so that the global
  //      stores are 16 contiguous bytes per lane along n.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // stages no longer read
  __bf16 E2D2_LDS* ct = (__bf16 E2D2_LDS*)lds_b;
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int ml = 32 * (MBW * wm + mb) + (lane & 31);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int nl = 32 * (NBW * wn + nb) + 8 * jg + 4 * (lane >> 5);
        bf16x4 v;
        v[0] = (__bf16)acc[nb][mb][4 * jg + 0];
        v[1] = (__bf16)acc[nb][mb][4 * jg + 1];
        v[2] = (__bf16)acc[nb][mb][4 * jg + 2];
        v[3] = (__bf16)acc[nb][mb][4 * jg + 3];
        *(bf16x4 E2D2_LDS*)(ct + ml * G::CP + nl) = v;
      }
    }
  }
  __syncthreads();
  constexpr int CPR = G::NT / 8;  // 16-byte chunks per tile row
  for (int ch = threadIdx.x; ch < G::MT * CPR; ch += G::THREADS) {
    const int r = ch / CPR, cq = ch - (ch / CPR) * CPR;
    const int m = m0 + r, n = n0 + 8 * cq;
    if (m >= p.M || n >= p.N) continue;
    const bf16x8 v = *(const bf16x8 E2D2_LDS*)(ct + r * G::CP + 8 * cq);
    const int b = m / p.S, s = m - (m / p.S) * p.S;
    const int seg = n < p.c_n0[1] ? 0 : (n < p.c_n0[2] ? 1 : 2);
    const int nn = n - p.c_n0[seg];
    const int h = nn / p.c_w, c = nn - (nn / p.c_w) * p.c_w;
    *(bf16x8*)(p.c[seg] + (((size_t)b * p.c_h[seg] + h) * p.S + s) * (size_t)p.c_w + c) = v;
  }
}

template <int NBW, int MBW, int WN, int WM, int ST>
hipError_t launch_linear_t(const LinearParams& p, hipStream_t stream) {
  using G = LinGeo<NBW, MBW, WN, WM, ST>;
  const size_t smem = G::LDS;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)linear_bf16_kernel<NBW, MBW, WN, WM, ST>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  const long long grid = (long long)((p.N + G::NT - 1) / G::NT) * ((p.M + G::MT - 1) / G::MT);
  hipLaunchKernelGGL((linear_bf16_kernel<NBW, MBW, WN, WM, ST>), dim3((unsigned)grid),
                     dim3(G::THREADS), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bf16(const LinearParams& p, hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const long long t128 = (long long)((p.N + 127) / 128) * ((p.M + 127) / 128);
  // 8 waves and a 4-deep ring; 128 x 128 tiles while they give at least one workgroup
  // per CU (256), else 128 x 64 (measured on MI355X at the denoise workload's
  // projections: 1024 x 4096 x 2048 and 1024 x 2048 x 2048).
  if (t128 >= 256) return launch_linear_t<2, 1, 2, 4, 4>(p, stream);
  return launch_linear_t<1, 1, 4, 2, 4>(p, stream);
}

}  // namespace e2d2

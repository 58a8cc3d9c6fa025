// Training-forward attention of E2D2 on gfx950: encoder block-causal attention,
// fused decoder self+cross attention over [clean | noised] keys, or both in one grid.
//
// Pages cited, by title and section:
//   [Notes] "Encoder-Decoder Diffusion Language Models for Efficient Training and
//           Inference", Paper-Notes page: 方法详解 §2 两种连接方式 (self- and
//           cross-attention fused into one call), §4 训练算法 (the encoder mask and the
//           decoder's 2L-key mask; the FLOPs table whose halved attention term is what
//           skipping masked tiles realises).
//
// bf16 kernel, one workgroup = 4 waves = 128 query rows of one (batch, query head, kind):
//   * Each wave owns 32 query rows and keeps their Q fragments in registers.
//   * The key axis is walked one 64-key tile at a time, source by source (clean
//     context keys, then, for the decoder, the noised keys of the own blocks), over
//     exactly the tiles that hold an allowed pair (schedule.h).  K and V tiles go from
//     HBM straight into a 2-deep ring of swizzled LDS stages (buffer_load ... lds);
//     tile t+1 is in flight while tile t is computed, and other workgroups on the CU
//     (4 at d <= 64, 2 at d = 128) fill the gaps.
//   * Scores are formed transposed, S^T = K Q^T, per 32-key x 32-query block as four
//     16x16 tiles of v_mfma_f32_16x16x32_bf16 (measured on MI355X: 1.94 against 1.58
//     PFLOP/s for v_mfma_f32_32x32x16_bf16 with random bf16 operands at full load, and
//     half as long accumulator chains).  Lane l (c = l % 16, g = l / 16) holds, for the
//     query rows wq0 + c and wq0 + 16 + c, the keys 4g + r and 16 + 4g + r (r < 4) of
//     the block; a row's 32 keys sit in the four lanes c + 16 g, and its reductions
//     (only when rescaling and at the end) are two lane swaps.
//   * Online softmax in base 2 with the scale folded in (p = 2^(s*c - m), c =
//     scale*log2 e), p packed to bf16 and summed with v_dot2 (the denominator adds the
//     same rounded values the PV MFMA multiplies).  Rescaling is lazy: a row keeps its
//     running max until a lane's block sum of p exceeds 2^16, then takes the block's
//     max (the same softmax; p stays far inside bf16 and fp32 range).  The decision is
//     per row, so a row's arithmetic depends on its own keys only.  A wave's first
//     block takes each row's max directly.
//   * O^T += V^T P^T per 32-key block on 16x16 tiles of head dims x queries: the B
//     operand is the lane's own 8 numerators, the A operand V^T comes from two
//     transposing LDS reads (keys 4g .. 4g+3 and 16+4g .. 16+4g+3, the same order).
//   * Within a tile, each wave classifies its 32x32 key blocks: empty blocks are
//     skipped (no MFMA), full blocks skip the mask, the rest mask per element (one bit
//     extract and one bit select per score from a per-lane key mask).
//   * Epilogue: O = O^T / l in bf16, LSE = (m + log2 l) ln 2 in fp32.
//   * Work order: query tiles are issued from the last (most keys) to the first;
//     when the number of (head, kind) items per tile level is a multiple of 8, each of
//     the 8 XCDs gets a fixed contiguous set of heads so that a head's K/V tiles stay
//     in one XCD's L2, and the encoder and decoder items of a head run side by side.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace e2d2 {
namespace {

constexpr int kBN = 64;           // keys per tile
constexpr float kBound = 65536.f; // lane sum of a tile's numerators that forces a rescale
constexpr float kNegBig = -1e30f; // "no key yet" running max (finite: no inf - inf)

// Workgroup shape per head dimension (measured on MI355X).  128 query rows (4 waves of
// 32) per workgroup and a 2-deep ring of 64-key K/V tiles; LDS and registers decide how
// many workgroups share a CU:
//   d <= 64: <= 128 VGPRs and 32 KiB of LDS (d = 64), four workgroups per CU, so one
//     wave's softmax overlaps another's MFMAs.  (Measured: 256-row workgroups with a
//     4-deep ring at two per CU, and 3-deep rings at three per CU, are slower.)
//   d = 128: <= 256 VGPRs and 64 KiB of LDS, two workgroups per CU.  (Measured 1.07 vs
//     1.55 ms on the B2 Hq16/8 L8192 S64 forward against one workgroup per CU with a
//     4-deep ring and S^T of tile t+1 software-pipelined beside the softmax of tile t,
//     and 1.11 ms for 256-row workgroups at one per CU.)
template <int D>
struct LoopCfg {
  static constexpr int kBM = 128;
  static constexpr int kWaves = kBM / 32;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kStages = 2;
  static constexpr int kBlocksPerCU = D > 64 ? 2 : 4;
};

template <int D>
struct Geo {
  static constexpr int TILE = kBN * D;  // bf16 elements of one K or V tile
  static constexpr int STAGE = 2 * TILE;
};

// ---------------------------------------------------------------------------------
// Per wave and 32x32 key-query block (layouts checked on gfx950):
//   S^T tile (kh, qh) = K[kh*16 .. +16] Q[qh*16 .. +16]^T: A = K rows (lane: key c,
//     dims 8g .. 8g+7 of each 32-dim step), B = Q^T (lane: query c, the same dims);
//     C: lane l, register r = S^T[kh*16 + 4g + r][qh*16 + c].
//   O^T tile (dt, qh) += V^T[dt*16 .. +16][keys] P^T[keys][qh*16 .. +16] over the
//     block's 32 keys in the lane order 4g + r, 16 + 4g + r: B = the lane's 8
//     numerators of row qh*16 + c, A = V^T (lane: dim dt*16 + c, the same 8 keys).

template <int D>
__global__ __launch_bounds__(LoopCfg<D>::kThreads, LoopCfg<D>::kBlocksPerCU) void train_fwd_bf16_kernel(TrainParams p) {
  using G = Geo<D>;
  constexpr int kStages = LoopCfg<D>::kStages;
  constexpr int kBM = LoopCfg<D>::kBM;
  constexpr int kWaves = LoopCfg<D>::kWaves;
  constexpr int TILE = G::TILE, STAGE = G::STAGE;
  constexpr int NK = D / 32;   // 32-dim k-steps of S^T
  constexpr int NDT = D / 16;  // 16-dim tiles of O^T
  static_assert(kStages == 2, "two-stage ring");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;

  // ---- work item (as in train_fwd_bf16_kernel)
  const int BH = p.B * p.Hq;
  const int per_level = BH * p.n_kinds;
  const int w = blockIdx.x;
  int level, rem;
  if (p.xcd_groups) {
    const int per_xcd = per_level >> 3;
    const int local = w >> 3;
    level = local / per_xcd;
    rem = (w & 7) * per_xcd + local % per_xcd;
  } else {
    level = w / per_level;
    rem = w % per_level;
  }
  const int slot = rem % p.n_kinds;
  const int bh = rem / p.n_kinds;
  const int qtile = p.n_qtiles - 1 - level;
  const int kind = p.kinds[slot];
  const int b = bh / p.Hq;
  const int hq = bh % p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);
  const int S = p.S;
  const int L = p.lens != nullptr ? min(max(p.lens[b], 0), p.L) : p.L;

  const int q0 = qtile * kBM;
  if (q0 >= L) return;
  const int r_last = min(q0 + kBM, L) - 1;
  const int nsrc = num_sources(kind);
  const TileRange tr0 = visited_tiles(kind, 0, q0, r_last, S, L, 0, kBN);
  const TileRange tr1 = nsrc > 1 ? visited_tiles(kind, 1, q0, r_last, S, L, 0, kBN) : TileRange{0, 0};
  const int n0 = tr0.last - tr0.first;
  const int ntot = n0 + (tr1.last - tr1.first);

  const size_t kv_off = ((size_t)b * p.Hkv + hk) * (size_t)p.kv_rows * D;
  const uint32_t kv_bytes = (uint32_t)L * D * 2u;
  const __amdgpu_buffer_rsrc_t rk0 = make_rsrc(p.k[0] + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv0 = make_rsrc(p.v[0] + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t rk1 = make_rsrc(p.k[1] + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv1 = make_rsrc(p.v[1] + kv_off, kv_bytes);
  TileLoader<D, kBN, kWaves> loader;
  loader.init(wave, lane);
  char E2D2_LDS* lds_b = (char E2D2_LDS*)smem_raw;

  auto tsrc = [&](int t) { return t < n0 ? 0 : 1; };
  auto tnum = [&](int t) { return t < n0 ? tr0.first + t : tr1.first + (t - n0); };
  auto issue = [&](int t) {
    char E2D2_LDS* kt = lds_b + (t % kStages) * STAGE * 2;
    const int row0 = tnum(t) * kBN;
    if (t < n0) {
      loader.load(rk0, row0, kt, wave);
      loader.load(rv0, row0, kt + TILE * 2, wave);
    } else {
      loader.load(rk1, row0, kt, wave);
      loader.load(rv1, row0, kt + TILE * 2, wave);
    }
  };
  if (0 < ntot) issue(0);

  // ---- per-wave rows; the lane's two query rows qr[0] = wq0 + c, qr[1] = wq0 + 16 + c
  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < L;
  const int wr1 = min(wq0 + 32, L) - 1;
  int qr[2];
  bool rok[2];
  Interval iv[2][2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    qr[qh] = wq0 + qh * 16 + c16;
    rok[qh] = qr[qh] < L;
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      iv[qh][sidx] = row_interval(kind, sidx, rok[qh] ? qr[qh] : 0, S, L, 0);
      if (!rok[qh]) iv[qh][sidx] = Interval{0, 0};
    }
  }
  Interval wu[2] = {{0, 0}, {0, 0}}, wc[2] = {{0, 0}, {0, 0}};
  if (wave_live) {
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      if (sidx < nsrc) {
        wu[sidx] = union_interval(kind, sidx, wq0, wr1, S, L, 0);
        wc[sidx] = common_interval(kind, sidx, wq0, wr1, S, L, 0);
      }
    }
  }
  auto classify_tile = [&](int t, int (&cls)[2]) {
    const int src = tsrc(t);
    const Interval u = src ? wu[1] : wu[0];
    const Interval cm = src ? wc[1] : wc[0];
    const int kt0 = tnum(t) * kBN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = kt0 + kb * 32;
      const int k1 = min(k0 + 32, L);
      int cl;
      if (k1 <= u.lo || k0 >= u.hi || k1 <= k0) cl = 0;
      else if (cm.lo <= k0 && k1 <= cm.hi && k1 - k0 == 32) cl = 2;
      else cl = 1;
      cls[kb] = cl;
    }
  };

  // queries: qf[qh][kk] = Q[qr[qh]][kk*32 + 8g .. +7]
  const size_t q_off = ((size_t)b * p.Hq + hq) * (size_t)p.L * D;
  bf16x8 qf[2][NK];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const __bf16* qrow = p.q[slot] + q_off + (size_t)(rok[qh] ? qr[qh] : 0) * D + (g4 << 3);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      bf16x8 v = *(const bf16x8*)(qrow + kk * 32);
      if (!rok[qh]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)0.f;
      }
      qf[qh][kk] = v;
    }
  }
  // LDS byte offsets: K operand of key half kh, k-step kk (row kh*16 + c, col kk*32 + 8g);
  // V^T reads of dim tile dt (row 4g + c/4, col dt*16 + 4 (c % 4)); rows 16 further sit
  // 32*D bytes further, rows 32 further 64*D (the swizzle uses row bits 0..3)
  uint32_t kof[2][NK];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kof[kh][kk] = 2u * (uint32_t)tile_off<D>(kh * 16 + c16, kk * 32 + 8 * g4);
  uint32_t vof[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    vof[dt] = 2u * (uint32_t)tile_off<D>(4 * g4 + (c16 >> 2), dt * 16 + 4 * (c16 & 3));
  const uint32_t lds0 = lds_addr(lds_b);

  f32x4 o[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt][0] = o[dt][1] = zero4();
  float ms[2] = {kNegBig, kNegBig};  // running max per row, base-2 units
  float l[2] = {0.f, 0.f};           // lane-partial sums
  const float c = p.c;
  bool started = false;              // wave-uniform

  // S^T of block kb (tile stage at byte offset KOFF): sc[kh][qh]
  auto qk = [&](auto koffc, auto kbc, f32x4 (&sc)[2][2]) {
    constexpr int OFF = decltype(koffc)::value + decltype(kbc)::value * 64 * D;
    bf16x8 kf[2 * NK];
    uint32_t a[2 * NK];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) a[kh * NK + kk] = lds0 + kof[kh][kk];
    if constexpr (2 * NK == 8) kread8<OFF>(a, kf);
    else if constexpr (2 * NK == 4) kread4<OFF>(a, kf);
    else kread2<OFF>(a, kf);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc = mfma16(kf[kh * NK + kk], qf[qh][kk], acc);
        sc[kh][qh] = acc;
      }
  };
  // mask of a partly allowed block: bit k of bits[qh] (after the lane's shift by 4g)
  // says whether key k0 + 4g + k of row qr[qh] is allowed
  auto mask = [&](int t, int kb, f32x4 (&sc)[2][2]) {
    const int src = tsrc(t);
    const int k0 = tnum(t) * kBN + kb * 32;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int a = min(max(iv[qh][src].lo - k0, 0), 32);
      const int e = min(max(iv[qh][src].hi - k0, 0), 32);
      uint32_t bits = e <= a ? 0u : (e - a >= 32 ? 0xffffffffu : ((1u << (e - a)) - 1u) << a);
      bits >>= 4 * g4;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = kh * 16 + r;
          const uint32_t keep = (uint32_t)((int32_t)(bits << (31 - off)) >> 31);
          sc[kh][qh][r] = __uint_as_float((__float_as_uint(sc[kh][qh][r]) & keep) | (~keep & 0xff800000u));
        }
    }
  };
  // numerators of row half qh against its running max: 8 values, packed (key order
  // 4g + r, then 16 + 4g + r), lane sum returned
  auto expq = [&](const f32x4 (&sc)[2][2], int qh, bf16x8& pb) {
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    const float nm = -ms[qh];
    float e[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e[r] = fast_exp2(fmaf(sc[0][qh][r], c, nm));
      e[4 + r] = fast_exp2(fmaf(sc[1][qh][r], c, nm));
    }
    pb = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x2 pr = {pb[2 * k], pb[2 * k + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
    return acc;
  };
  auto row_max = [&](const f32x4 (&sc)[2][2], int qh) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fmaxf(sc[0][qh][r], sc[1][qh][r]));
    return quad_max(mx);
  };
  // online softmax of one block (lazy rescale as in train_fwd_bf16_kernel, per row)
  auto softmax = [&](const f32x4 (&sc)[2][2], bf16x8 (&pb)[2]) {
    if (!started) {
      started = true;
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const float rmax = row_max(sc, qh);
        if (rmax > -INFINITY) ms[qh] = rmax * c;
        l[qh] = expq(sc, qh, pb[qh]);
      }
      return;
    }
    float rs[2];
    rs[0] = expq(sc, 0, pb[0]);
    rs[1] = expq(sc, 1, pb[1]);
    if (__builtin_amdgcn_ballot_w64(rs[0] > kBound || rs[1] > kBound) != 0) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const float rmax = row_max(sc, qh);
        const bool need = quad_max(rs[qh] > kBound ? 1.f : 0.f) > 0.f;
        if (need) {
          const float m_new = rmax * c;
          const float alpha = fast_exp2(ms[qh] - m_new);
          l[qh] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[dt][qh][r] *= alpha;
          ms[qh] = m_new;
        }
        rs[qh] = expq(sc, qh, pb[qh]);
      }
    }
    l[0] += rs[0];
    l[1] += rs[1];
  };
  // O^T += V^T P^T for block kb (V tile at byte offset VOFF)
  auto pv = [&](auto voffc, auto kbc, const bf16x8 (&pb)[2]) {
    constexpr int OFF = decltype(voffc)::value + decltype(kbc)::value * 64 * D;
    uint32_t a[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) a[dt] = lds0 + vof[dt];
    long lo[NDT], hi[NDT];
    tr_reads1<OFF>(a, lo);
    tr_reads1<OFF + 32 * D>(a, hi);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x8 vt = join_bf16(lo[dt], hi[dt]);
      o[dt][0] = mfma16(vt, pb[0], o[dt][0]);
      o[dt][1] = mfma16(vt, pb[1], o[dt][1]);
    }
  };

  {
    const Interval cm = common_interval(kind, 0, q0, r_last, S, L, 0);
    const int nf = max(0, min(min(cm.hi / kBN, tr0.last) - tr0.first, n0));
    auto tile = [&](int t, auto stg) {
      constexpr int KOFF = decltype(stg)::value * STAGE * 2;
      constexpr int VOFF = KOFF + TILE * 2;
      wait_vmem<0>();
      __syncthreads();
      if (t + 1 < ntot) issue(t + 1);
      int cls[2];
      if (t < nf) {
        cls[0] = cls[1] = wave_live ? 2 : 0;
      } else {
        classify_tile(t, cls);
      }
      if (cls[0]) {
        f32x4 sc[2][2];
        qk(IntC<KOFF>{}, IntC<0>{}, sc);
        if (cls[0] == 1) mask(t, 0, sc);
        bf16x8 pb[2];
        softmax(sc, pb);
        pv(IntC<VOFF>{}, IntC<0>{}, pb);
      }
      if (cls[1]) {
        f32x4 sc[2][2];
        qk(IntC<KOFF>{}, IntC<1>{}, sc);
        if (cls[1] == 1) mask(t, 1, sc);
        bf16x8 pb[2];
        softmax(sc, pb);
        pv(IntC<VOFF>{}, IntC<1>{}, pb);
      }
    };
    for (int t = 0; t < ntot; t += 2) {
      tile(t, IntC<0>{});
      if (t + 1 < ntot) tile(t + 1, IntC<1>{});
    }
  }

  // ---- epilogue: O = O^T / l (lane: dims dt*16 + 4g .. +3 of row qr[qh]), LSE
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const float l_tot = quad_sum(l[qh]);
    if (rok[qh]) {
      const float inv = 1.f / l_tot;
      __bf16* orow = p.o[slot] + q_off + (size_t)qr[qh] * D + 4 * g4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bf16x4 v;
        v[0] = (__bf16)(o[dt][qh][0] * inv);
        v[1] = (__bf16)(o[dt][qh][1] * inv);
        v[2] = (__bf16)(o[dt][qh][2] * inv);
        v[3] = (__bf16)(o[dt][qh][3] * inv);
        *(bf16x4*)(orow + dt * 16) = v;
      }
      if (p.lse[slot] != nullptr && g4 == 0)
        p.lse[slot][((size_t)b * p.Hq + hq) * p.L + qr[qh]] = (ms[qh] + __log2f(l_tot)) * 0.6931471805599453f;
    }
  }
  if (p.visits != nullptr && threadIdx.x == 0) atomicAdd(p.visits, (unsigned long long)ntot);
}

// ---------------------------------------------------------------------------------
// fp32 path: one wave per 64 query rows (one row per lane), 64-key fp32 tiles in LDS,
// scores and P*V on the vector ALU in fp32, exp in fp32.  Serves every kind with two
// key sources described by (pointer, allocated rows, length) per source.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(F32Params p) {
  constexpr int BN = 64;
  __shared__ float ks[BN][D];  // every lane reads the same key row: broadcast, no padding
  __shared__ float vs[BN][D];
  const int lane = threadIdx.x;

  const int per_level = p.B * p.Hq * p.n_kinds;
  const int level = blockIdx.x / per_level;
  const int rem = blockIdx.x % per_level;
  const int slot = rem % p.n_kinds;
  const int bh = rem / p.n_kinds;
  const int qtile = p.n_qtiles - 1 - level;
  const int kind = p.kinds[slot];
  const int b = bh / p.Hq, hq = bh % p.Hq, hk = hq / (p.Hq / p.Hkv);
  const int L = p.L, S = p.S, C = p.C;
  const int Lq = query_len(kind, L, S);
  const int q0 = qtile * 64;
  if (q0 >= Lq) return;
  const int r_last = min(q0 + 64, Lq) - 1;
  const int qi = q0 + lane;
  const bool row_ok = qi < Lq;

  float q[D];
  const float* qrow = p.q[slot] + (((size_t)b * p.Hq + hq) * Lq + (row_ok ? qi : 0)) * D;
#pragma unroll
  for (int j = 0; j < D; ++j) q[j] = row_ok ? qrow[j] : 0.f;
  float o[D];
#pragma unroll
  for (int j = 0; j < D; ++j) o[j] = 0.f;
  // Running max in base-2 units (max score times c) and the sum relative to it.  The
  // rescale factor is 2^(old - new) of two stored values, so it is exactly 1 whenever
  // the max did not change (recomputing old * c there could leave a rounding residue
  // that would reweight earlier keys against later ones at every sub-block).
  float mb = -INFINITY, l = 0.f;
  const float c = p.c;
  int visits = 0;

  for (int src = 0; src < num_sources(kind); ++src) {
    const int n = source_len(kind, src, L, S, C);
    const TileRange tr = visited_tiles(kind, src, q0, r_last, S, L, C, BN);
    Interval iv = row_interval(kind, src, row_ok ? qi : 0, S, L, C);
    if (!row_ok) iv = Interval{0, 0};
    const int nalloc = p.src_rows[slot][src];
    const float* kb = p.kf[slot][src] + ((size_t)b * p.Hkv + hk) * (size_t)nalloc * D;
    const float* vb = p.vf[slot][src] + ((size_t)b * p.Hkv + hk) * (size_t)nalloc * D;
    for (int t = tr.first; t < tr.last; ++t) {
      ++visits;
      __syncthreads();
      for (int e = lane; e < BN * D; e += 64) {
        const int r = e / D, col = e % D;
        const int g = min(t * BN + r, n - 1);
        ks[r][col] = kb[(size_t)g * D + col];
        vs[r][col] = vb[(size_t)g * D + col];
      }
      __syncthreads();
      // Rounding error is kept well under 1e-5 relative at thousands of keys: four
      // partial sums per dot product, and the 16 keys of a sub-block are summed on
      // their own before one fused multiply-add folds them into the running O and l.
      for (int sub = 0; sub < BN; sub += 16) {
        float s[16];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * BN + sub + r;
          float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < D; ++j) a[j & 3] = fmaf(q[j], ks[sub + r][j], a[j & 3]);
          const float acc = (a[0] + a[1]) + (a[2] + a[3]);
          s[r] = (key >= iv.lo && key < iv.hi) ? acc : -INFINITY;
          mx = fmaxf(mx, s[r]);
        }
        const float mb_new = fmaxf(mb, mx * c);
        const float base = mb_new == -INFINITY ? 0.f : mb_new;
        const float alpha = exp2f(mb - base);
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = exp2f(fmaf(s[r], c, -base));  // the numerator, in place
          ls += s[r];
        }
        l = fmaf(l, alpha, ls);
#pragma unroll
        for (int j = 0; j < D; ++j) {
          float part = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) part = fmaf(s[r], vs[sub + r][j], part);
          o[j] = fmaf(o[j], alpha, part);
        }
        mb = mb_new;
      }
    }
  }
  if (row_ok) {
    float* orow = p.o[slot] + (((size_t)b * p.Hq + hq) * Lq + qi) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int j = 0; j < D; ++j) orow[j] = o[j] * inv;
    if (p.lse[slot] != nullptr)
      p.lse[slot][((size_t)b * p.Hq + hq) * Lq + qi] = mb * 0.6931471805599453f + logf(l);
  }
  if (p.visits != nullptr && lane == 0) atomicAdd(p.visits, (unsigned long long)visits);
}

template <int D>
hipError_t launch_train_bf16_d(const TrainParams& p, int grid, hipStream_t stream) {
  const size_t smem = (size_t)LoopCfg<D>::kStages * Geo<D>::STAGE * sizeof(__bf16);
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)train_fwd_bf16_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(train_fwd_bf16_kernel<D>, dim3(grid), dim3(LoopCfg<D>::kThreads), smem, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32_d(const F32Params& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(attn_f32_kernel<D>, dim3(grid), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int train_tile_bm(int d) {
  return d == 64 ? LoopCfg<64>::kBM : (d == 32 ? LoopCfg<32>::kBM : LoopCfg<128>::kBM);
}
int train_tile_bn() { return kBN; }

hipError_t launch_train_bf16(const TrainParams& p, int d, hipStream_t stream) {
  const int grid = p.n_qtiles * p.B * p.Hq * p.n_kinds;
  if (grid == 0) return hipSuccess;
  switch (d) {
    case 32: return launch_train_bf16_d<32>(p, grid, stream);
    case 64: return launch_train_bf16_d<64>(p, grid, stream);
    case 128: return launch_train_bf16_d<128>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_f32(const F32Params& p, int d, hipStream_t stream) {
  const int grid = p.n_qtiles * p.B * p.Hq * p.n_kinds;
  if (grid == 0) return hipSuccess;
  switch (d) {
    case 32: return launch_f32_d<32>(p, grid, stream);
    case 64: return launch_f32_d<64>(p, grid, stream);
    case 128: return launch_f32_d<128>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace e2d2

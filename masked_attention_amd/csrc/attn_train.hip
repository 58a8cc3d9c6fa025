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
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so a
//     lane holds 16 keys of ONE query row: row reductions are in-lane plus, when
//     needed, one exchange with lane l^32.
//   * Online softmax in base 2 with the scale folded in (p = 2^(s*c - m), c =
//     scale*log2 e), p packed to bf16 and summed with v_dot2 (the denominator adds the
//     same rounded values the PV MFMA multiplies).  Rescaling is lazy: a row keeps its
//     running max until a lane's block sum of p exceeds 2^16, then takes the block's
//     max (the same softmax; p stays far inside bf16 and fp32 range).  The decision is
//     per row, so a row's arithmetic depends on its own keys only.
//   * O^T += V^T P^T per 32-key block, V^T from the transposing LDS read.
//   * Within a tile, each wave classifies its 32x32 key blocks: empty blocks are
//     skipped (no MFMA), full blocks skip the mask, the rest mask per element.
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
  static constexpr int NC = D / 16;   // MFMA k-steps over the head dim for S^T
  static constexpr int NDB = D / 32;  // 32-wide head-dim blocks of O^T
  static constexpr int TILE = kBN * D;  // bf16 elements of one K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NIW = 2 * (kBN * (D / 8) / 64) / LoopCfg<D>::kWaves;  // loads per wave per tile
};

template <int D>
__global__ __launch_bounds__(LoopCfg<D>::kThreads, LoopCfg<D>::kBlocksPerCU) void train_fwd_bf16_kernel(TrainParams p) {
  using G = Geo<D>;
  constexpr int kStages = LoopCfg<D>::kStages;
  constexpr int kBM = LoopCfg<D>::kBM;
  constexpr int kWaves = LoopCfg<D>::kWaves;
  constexpr int NC = G::NC, NDB = G::NDB, TILE = G::TILE, STAGE = G::STAGE, NIW = G::NIW;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  // ---- work item: query tiles from the last (most keys) to the first; heads grouped
  //      per XCD when the item count of a tile level is a multiple of 8
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
  // this sequence's length: all L rows, or (per-sequence lengths on the device) its own
  // prefix of them; the row stride of q, o and lse stays p.L
  const int L = p.lens != nullptr ? min(max(p.lens[b], 0), p.L) : p.L;

  const int q0 = qtile * kBM;
  if (q0 >= L) return;  // the whole query tile lies past this sequence's end
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

  // tile index -> (source, key-tile number in that source)
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

  // first tiles in flight before the per-row setup below
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < ntot) issue(i);

  // ---- per-wave rows and per-lane query row
  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < L;
  const int wr1 = min(wq0 + 32, L) - 1;
  const int qi = wq0 + (lane & 31);
  const bool row_ok = qi < L;
  Interval iv[2];
#pragma unroll
  for (int sidx = 0; sidx < 2; ++sidx) {
    iv[sidx] = row_interval(kind, sidx, row_ok ? qi : 0, S, L, 0);
    if (!row_ok) iv[sidx] = Interval{0, 0};
  }
  // Classification of the two 32-key blocks of tile t for this wave:
  // 0 = no allowed pair (skipped), 1 = partly allowed (masked), 2 = all allowed.
  // The keys the wave's rows allow at all (union) and allow in every row (common) are
  // fixed per source, so a block is classified with four compares.
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

  const size_t q_off = ((size_t)b * p.Hq + hq) * (size_t)p.L * D;
  bf16x8 qf[NC];
  {
    const __bf16* qrow = p.q[slot] + q_off + (size_t)(row_ok ? qi : 0) * D + ((lane >> 5) << 3);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      bf16x8 v = *(const bf16x8*)(qrow + cc * 16);
      if (!row_ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)0.f;
      }
      qf[cc] = v;
    }
  }
  uint32_t offA[NDB], offB[NDB];
  vt_offsets<D>(lane, offA, offB);
  uint32_t koff[NC];
  k_offsets<D>(lane, koff);
  const uint32_t lds0 = lds_addr(lds_b);

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = zero16();
  float ms = kNegBig;  // running max in use, in base-2 units (raw max * c)
  float l = 0.f;       // lane-partial running sum, relative to ms
  const float c = p.c;

  // Element mask of the partly allowed blocks of tile t.  The lane's 16 keys are
  // kr + {0..3, 8..11, 16..19, 24..27}; bit k of `bits` says whether key kr + k is
  // allowed, so each score takes one bit extract and one bit select.
  auto mask = [&](int t, const int (&cls)[2], f32x16 (&sc)[2]) {
    const int src = tsrc(t);
    const int kt0 = tnum(t) * kBN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (cls[kb] == 1) {
        const int kr = kt0 + kb * 32 + ((lane >> 5) << 2);
        const int a = min(max(iv[src].lo - kr, 0), 32);
        const int e = min(max(iv[src].hi - kr, 0), 32);
        const uint32_t bits =
            e <= a ? 0u : (e - a >= 32 ? 0xffffffffu : ((1u << (e - a)) - 1u) << a);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = ((j >> 2) << 3) + (j & 3);
          const uint32_t keep = (uint32_t)((int32_t)(bits << (31 - off)) >> 31);
          sc[kb][j] = __uint_as_float((__float_as_uint(sc[kb][j]) & keep) | (~keep & 0xff800000u));
        }
      }
    }
  };
  // Numerators of one 32-key block against the running max (online softmax, base 2),
  // packed to bf16, their lane sum added to l.  Rescaling is lazy and needs no row max
  // on the common path: when a lane's sum exceeds kBound (the row's first keys, or
  // scores that outgrew the running max), the row takes its max over the block,
  // rescales O and l, and the block's numerators are formed again.  The decision is
  // per row (the lane pair), so a row's arithmetic depends on its own keys only.  Each
  // block's P^T is accumulated right after its numerators, so one block's P is live.
  // The wave's first block starts from O = 0 and l = 0: each row takes its max over
  // the block at once (rows with no allowed key there keep the "no key yet" max).
  bool started = false;  // wave-uniform
  auto block_softmax = [&](const f32x16& sblk, bf16x8 (&pbk)[2]) {
    if (!started) {
      started = true;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sblk[j]);
      const float rmax = pair_max(mx);
      if (rmax > -INFINITY) ms = rmax * c;
      l = exp_pack(sblk, c, -ms, pbk, 0.f);
      return;
    }
    float rs = exp_pack(sblk, c, -ms, pbk, 0.f);
    if (__builtin_amdgcn_ballot_w64(rs > kBound) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sblk[j]);
      const float rmax = pair_max(mx);
      const bool need = pair_max(rs > kBound ? 1.f : 0.f) > 0.f;
      if (need) {
        const float m_new = rmax * c;
        const float alpha = fast_exp2(ms - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        ms = m_new;
      }
      rs = exp_pack(sblk, c, -ms, pbk, 0.f);
    }
    l += rs;
  };
  {
    // ---- one tile at a time through a kStages-deep ring: tiles t+1 .. t+kStages-1 are
    //      in flight while tile t is computed.  Unrolled by kStages so the stage of each
    //      tile is a constant that the LDS reads carry in their offset field.  Tiles
    //      [0, nf) are full for every row of the workgroup (keys of blocks before the
    //      first row's block) and skip classification and masks.
    static_assert(kStages >= 2 && kStages <= 4, "unrolled for 2..4 stages");
    const Interval cm = common_interval(kind, 0, q0, r_last, S, L, 0);
    const int nf = max(0, min(min(cm.hi / kBN, tr0.last) - tr0.first, n0));
    auto tile = [&](int t, auto stg) {
      constexpr int KOFF = decltype(stg)::value * STAGE * 2;
      constexpr int VOFF = KOFF + TILE * 2;
      // Tile t must have landed; the tiles issued after it (up to kStages - 2 of them)
      // may stay in flight.  The barrier then makes every wave's part of tile t visible
      // and frees the stage of tile t-1 for tile t+kStages-1.
      if constexpr (kStages >= 4) {
        if (t + 2 < ntot) wait_vmem<2 * NIW>();
        else if (t + 1 < ntot) wait_vmem<NIW>();
        else wait_vmem<0>();
      } else if constexpr (kStages == 3) {
        if (t + 1 < ntot) wait_vmem<NIW>();
        else wait_vmem<0>();
      } else {
        wait_vmem<0>();
      }
      __syncthreads();
      if (t + kStages - 1 < ntot) issue(t + kStages - 1);
      int cls[2];
      if (t < nf) {
        cls[0] = cls[1] = wave_live ? 2 : 0;
      } else {
        classify_tile(t, cls);
      }
      const int want = (cls[0] ? 1 : 0) | (cls[1] ? 2 : 0);
      if (!want) return;
      f32x16 sc[2];
      qk_blocks<D, 2, KOFF>(lds0, koff, qf, sc, want);
      if (t >= nf) mask(t, cls, sc);
      if (cls[0]) {
        bf16x8 pb[2];
        block_softmax(sc[0], pb);
        pv_block<D, VOFF>(lds0, offA, offB, pb, o);
      }
      if (cls[1]) {
        bf16x8 pb[2];
        block_softmax(sc[1], pb);
        pv_block<D, VOFF + 64 * D>(lds0, offA, offB, pb, o);
      }
    };
    for (int t = 0; t < ntot; t += kStages) {
      tile(t, IntC<0>{});
      if (t + 1 < ntot) tile(t + 1, IntC<1>{});
      if constexpr (kStages > 2) {
        if (t + 2 < ntot) tile(t + 2, IntC<2 % kStages>{});
      }
      if constexpr (kStages > 3) {
        if (t + 3 < ntot) tile(t + 3, IntC<3 % kStages>{});
      }
    }
  }

  // ---- epilogue
  const float l_tot = pair_sum(l);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    __bf16* orow = p.o[slot] + q_off + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = db * 32 + jg * 8 + ((lane >> 5) << 2);
        bf16x4 v;
        v[0] = (__bf16)(o[db][jg * 4 + 0] * inv);
        v[1] = (__bf16)(o[db][jg * 4 + 1] * inv);
        v[2] = (__bf16)(o[db][jg * 4 + 2] * inv);
        v[3] = (__bf16)(o[db][jg * 4 + 3] * inv);
        *(bf16x4*)(orow + d) = v;
      }
    if (p.lse[slot] != nullptr && lane < 32)
      p.lse[slot][((size_t)b * p.Hq + hq) * p.L + qi] =
          (ms + __log2f(l_tot)) * 0.6931471805599453f;
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

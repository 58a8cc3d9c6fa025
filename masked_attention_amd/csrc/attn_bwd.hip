// Backward of the E2D2 training attentions on gfx950: gradients of the encoder's
// block-causal attention and of the decoder's fused attention over [clean | noised]
// keys, from the forward's O and LSE.
//
// Pages cited, by title and section:
//   [Notes] "Encoder-Decoder Diffusion Language Models for Efficient Training and
//           Inference", Paper-Notes page: 方法详解 §4 训练算法 (one encoder pass and one
//           decoder pass per training step; the loss is the decoder's, so its gradient
//           flows back through both attentions, and the clean keys/values feed both).
//
// For one (batch, query head), with p_ij = exp(s_ij - lse_i) on allowed pairs and the
// upstream gradient do_i:  dv_j = sum_i p_ij do_i,  dp_ij = <do_i, v_j>,
// ds_ij = p_ij (dp_ij - delta_i) with delta_i = <do_i, o_i>,  dq_i = scale sum_j ds_ij
// k_j,  dk_j = scale sum_i ds_ij q_i.  Two launches, no atomics (deterministic):
//   1. dQ: query-stationary, the forward's schedule: a workgroup owns 128 query rows
//      of one (batch, query head, kind) and walks the key tiles holding an allowed
//      pair.  It first forms delta_i = <do_i, o_i> and lse_i * log2(e) of its rows
//      (fp32, also written to the workspace for launch 2).  Per 32x32 block, as four
//      16x16 tiles of v_mfma_f32_16x16x32_bf16 (the forward's layout): S^T = K Q^T and
//      dP^T = V dO^T (K and V rows from LDS, Q and dO in registers), P^T = 2^(S^T c -
//      lse), dS^T = P^T (dP^T - delta), then dQ^T += K^T dS^T with K^T from the
//      transposing LDS read.  (The dK/dV kernel stays on 32x32x16: at one wave per
//      SIMD, d = 128, the 16x16 form measured 4.06 against 3.90 ms for the backward.)
//   2. dK/dV: key-stationary: a workgroup owns 128 keys of one (batch, kv head, key
//      source) and walks the 64-row query tiles that allow any of them -- every query
//      head of the group, and for the clean keys both the encoder's and the decoder's
//      queries -- so each key's gradient is summed in one place.  Per 32x32 block, in
//      three phases fenced against the scheduler (described at the block loop):
//      S = Q K^T and dP = dO V^T (Q, dO rows from LDS, K and V in registers), then P
//      and dS, then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from the
//      transposing read.
//   Query and key tiles are staged through a 2-deep LDS ring with buffer_load ... lds,
//   as in the forward; partial 32x32 blocks are masked per element from the closed-
//   form row / column intervals (schedule.h), empty ones are skipped.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace e2d2 {
namespace {

// Wait for every outstanding vector-memory operation, as an instruction the compiler's
// wait-count pass sees (vmcnt 0; expcnt and lgkmcnt left at their maxima, 7 and 15).
// Needed after registers are loaded in a kernel's prologue when the main loop issues
// its LDS-DMA loads from asm: without it the pass still counts the prologue loads as
// outstanding inside the loop and places vmcnt waits at their first uses there, which
// the hardware then applies to the loop's own in-flight prefetch.
__device__ __forceinline__ void drain_vmem_visible() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A compile-time bool carried as a value.
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

constexpr int kTK = 64;     // keys per K/V tile (dQ) and query rows per Q/dO tile (dK/dV)
constexpr int kRows = 128;  // query rows (dQ) or keys (dK/dV) per workgroup: 4 waves x 32
constexpr int kWaves = 4;

template <int D>
struct BwdGeo {
  static constexpr int NC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int TILE = kTK * D;  // bf16 elements of one 64-row tile
  static constexpr int STAGE = 2 * TILE;
};

// ---- 1. dQ (and delta, lse * log2(e))
template <int D>
__global__ __launch_bounds__(256, D > 64 ? 2 : 3) void bwd_dq_kernel(BwdParams p) {
  using G = BwdGeo<D>;
  constexpr int NC = G::NC, NDB = G::NDB, TILE = G::TILE, STAGE = G::STAGE;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  // work item, as in the forward: query tiles from the last to the first; when the
  // items of a tile level split evenly over the 8 XCDs (workgroups are dealt to them
  // round-robin), each XCD keeps a fixed contiguous set of heads, so a head's K/V tiles
  // are fetched into one XCD's L2 only
  const int BH = p.B * p.Hq;
  const int per_level = BH * p.n_kinds;
  const int w = blockIdx.x;
  int level, rem;
  if ((per_level & 7) == 0) {
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
  const int kind = slot ? p.kinds[1] : p.kinds[0];
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);
  const int L = p.L, S = p.S;
  const int q0 = (p.n_qtiles - 1 - level) * kRows;
  const int r_last = min(q0 + kRows, L) - 1;
  const int nsrc = num_sources(kind);
  const TileRange tr0 = visited_tiles(kind, 0, q0, r_last, S, L, 0, kTK);
  const TileRange tr1 = nsrc > 1 ? visited_tiles(kind, 1, q0, r_last, S, L, 0, kTK) : TileRange{0, 0};
  const int n0 = tr0.last - tr0.first;
  const int ntot = n0 + (tr1.last - tr1.first);

  const size_t kv_off = ((size_t)b * p.Hkv + hk) * (size_t)L * D;
  const uint32_t kv_bytes = (uint32_t)L * D * 2u;
  const __amdgpu_buffer_rsrc_t rk0 = make_rsrc(p.k[0] + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv0 = make_rsrc(p.v[0] + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t rk1 = make_rsrc(p.k[1] + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv1 = make_rsrc(p.v[1] + kv_off, kv_bytes);
  TileLoader<D, kTK, kWaves> loader;
  loader.init(wave, lane);
  char E2D2_LDS* lds_b = (char E2D2_LDS*)smem_raw;
  auto tsrc = [&](int t) { return t < n0 ? 0 : 1; };
  auto tnum = [&](int t) { return t < n0 ? tr0.first + t : tr1.first + (t - n0); };
  auto issue = [&](int t) {
    char E2D2_LDS* kt = lds_b + (t & 1) * STAGE * 2;
    const int row0 = tnum(t) * kTK;
    if (t < n0) {
      loader.load(rk0, row0, kt, wave);
      loader.load(rv0, row0, kt + TILE * 2, wave);
    } else {
      loader.load(rk1, row0, kt, wave);
      loader.load(rv1, row0, kt + TILE * 2, wave);
    }
  };
  if (ntot > 0) issue(0);

  // per-wave rows; lane l (c = l % 16, g = l / 16) serves the query rows wq0 + c and
  // wq0 + 16 + c, and in a 32-key block the keys 4g + r and 16 + 4g + r (r < 4), as the
  // 16x16 tiles of v_mfma_f32_16x16x32_bf16 lay them out (see attn_train.hip)
  const int c16 = lane & 15, g4 = lane >> 4;
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
    for (int sidx = 0; sidx < 2; ++sidx)
      if (sidx < nsrc) {
        wu[sidx] = union_interval(kind, sidx, wq0, wr1, S, L, 0);
        wc[sidx] = common_interval(kind, sidx, wq0, wr1, S, L, 0);
      }
  }
  auto classify_tile = [&](int t, int (&cls)[2]) {
    const int src = tsrc(t);
    const Interval u = src ? wu[1] : wu[0];
    const Interval cm = src ? wc[1] : wc[0];
    const int kt0 = tnum(t) * kTK;
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

  // Q and dO of the lane's rows as S^T / dP^T operands (dims kk*32 + 8g .. +7); lse
  // and delta per row
  constexpr int NK = D / 32, NDT = D / 16;
  const size_t row_base = ((size_t)b * p.Hq + hq) * (size_t)L;
  bf16x8 qf[2][NK], df[2][NK];
  float dlt[2], lse2[2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const size_t q_row = row_base + (rok[qh] ? qr[qh] : 0);
    const __bf16* qrow = (slot ? p.q[1] : p.q[0]) + q_row * D + (g4 << 3);
    const __bf16* drow = (slot ? p.dO[1] : p.dO[0]) + q_row * D + (g4 << 3);
    const __bf16* orow = (slot ? p.o[1] : p.o[0]) + q_row * D + (g4 << 3);
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      qf[qh][kk] = *(const bf16x8*)(qrow + kk * 32);
      df[qh][kk] = *(const bf16x8*)(drow + kk * 32);
      const bf16x8 ov = *(const bf16x8*)(orow + kk * 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)ov[j], (float)df[qh][kk][j], part);
    }
    // delta = <dO, O> of the row (its four lanes hold quarters) and lse * log2(e); both
    // also go to the workspace for the dK/dV kernel.  Rows past L: lse = +inf makes
    // every p zero.
    dlt[qh] = quad_sum(part);
    lse2[qh] = (slot ? p.lse[1] : p.lse[0])[q_row] * kLog2e;
    if (rok[qh] && g4 == 0) {
      (slot ? p.delta[1] : p.delta[0])[q_row] = dlt[qh];
      (slot ? p.lse2[1] : p.lse2[0])[q_row] = lse2[qh];
    }
    if (!rok[qh]) {
      dlt[qh] = 0.f;
      lse2[qh] = INFINITY;
    }
  }
  // LDS byte offsets: K/V operand rows kh*16 + c, cols kk*32 + 8g; K^T reads of dim tile
  // dt (row 4g + c/4, col dt*16 + 4 (c % 4)); rows 16 further sit 32*D bytes further
  uint32_t kof[2 * NK];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kof[kh * NK + kk] = 2u * (uint32_t)tile_off<D>(kh * 16 + c16, kk * 32 + 8 * g4);
  uint32_t tof[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    tof[dt] = 2u * (uint32_t)tile_off<D>(4 * g4 + (c16 >> 2), dt * 16 + 4 * (c16 & 3));
  const uint32_t lds0 = lds_addr(lds_b);
  const float c = p.c;

  f32x4 dq[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dq[dt][0] = dq[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 2 NK operand rows of a 32-key block at LDS byte offset OFF
  auto rows = [&](auto offc, bf16x8 (&f)[2 * NK]) __attribute__((always_inline)) {
    constexpr int OFF = decltype(offc)::value;
    uint32_t a[2 * NK];
#pragma unroll
    for (int i = 0; i < 2 * NK; ++i) a[i] = lds0 + kof[i];
    if constexpr (2 * NK == 8) kread8<OFF>(a, f);
    else if constexpr (2 * NK == 4) kread4<OFF>(a, f);
    else kread2<OFF>(a, f);
  };
  // one 32-key block kb of the tile in stage STG
  auto block = [&](int t, auto kbc, int cl, auto stg) __attribute__((always_inline)) {
    constexpr int KOFF = decltype(stg)::value * STAGE * 2 + decltype(kbc)::value * 64 * D;
    constexpr int VOFF = KOFF + TILE * 2;
    f32x4 st[2][2], dpt[2][2];
    {
      bf16x8 kf[2 * NK];
      rows(IntC<KOFF>{}, kf);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) acc = mfma16(kf[kh * NK + kk], qf[qh][kk], acc);
          st[kh][qh] = acc;
        }
      rows(IntC<VOFF>{}, kf);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) acc = mfma16(kf[kh * NK + kk], df[qh][kk], acc);
          dpt[kh][qh] = acc;
        }
    }
    if (cl == 1) {
      const int src = tsrc(t);
      const int k0 = tnum(t) * kTK + decltype(kbc)::value * 32;
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
            const uint32_t keep = (uint32_t)((int32_t)(bits << (31 - (kh * 16 + r))) >> 31);
            st[kh][qh][r] = __uint_as_float((__float_as_uint(st[kh][qh][r]) & keep) | (~keep & 0xff800000u));
          }
      }
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float e[8];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pj = fast_exp2(fmaf(st[kh][qh][r], c, -lse2[qh]));
          e[kh * 4 + r] = pj * (dpt[kh][qh][r] - dlt[qh]);
        }
      dsb[qh] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
    // dQ^T += K^T dS^T: K^T of the block's keys in the lane order 4g + r, 16 + 4g + r
    uint32_t a[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) a[dt] = lds0 + tof[dt];
    long lo[NDT], hi[NDT];
    tr_reads1<KOFF>(a, lo);
    tr_reads1<KOFF + 32 * D>(a, hi);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x8 kt = join_bf16(lo[dt], hi[dt]);
      dq[dt][0] = mfma16(kt, dsb[0], dq[dt][0]);
      dq[dt][1] = mfma16(kt, dsb[1], dq[dt][1]);
    }
  };
  auto tile = [&](int t, auto stg) __attribute__((always_inline)) {
    wait_vmem<0>();   // tile t is the only load in flight
    __syncthreads();  // tile t visible; everyone is done with the other stage
    if (t + 1 < ntot) issue(t + 1);
    int cls[2];
    classify_tile(t, cls);
    if (cls[0]) block(t, IntC<0>{}, cls[0], stg);
    if (cls[1]) block(t, IntC<1>{}, cls[1], stg);
  };
  for (int t = 0; t < ntot; t += 2) {
    tile(t, IntC<0>{});
    if (t + 1 < ntot) tile(t + 1, IntC<1>{});
  }

  // dQ = scale * dQ^T: the lane holds dims dt*16 + 4g .. +3 of its two rows
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    if (!rok[qh]) continue;
    __bf16* out = (slot ? p.dq[1] : p.dq[0]) + (row_base + qr[qh]) * D + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      bf16x4 v;
      v[0] = (__bf16)(dq[dt][qh][0] * p.scale);
      v[1] = (__bf16)(dq[dt][qh][1] * p.scale);
      v[2] = (__bf16)(dq[dt][qh][2] * p.scale);
      v[3] = (__bf16)(dq[dt][qh][3] * p.scale);
      *(bf16x4*)(out + dt * 16) = v;
    }
  }
}

// ---- 2. dK / dV
//
// Query-tile stream of a key workgroup: for each kind slot reading this key source,
// for each query head of the kv head's group, the 64-row query tiles [qt0, qt1) that
// hold a row allowing any of the workgroup's keys.
struct QStream {
  int n_slots;           // kind slots reading this source (0, 1 or 2)
  int slot0, slot1;      // kind slot of stream slot 0 / 1 (0: decoder, 1: encoder)
  int kind0, kind1;
  int qt00, qt01;        // first query tile of stream slot 0 / 1
  int nqt0, nqt1;        // query tiles per head
  int per0;              // g * nqt0
  int ntot;
};

template <int D>
__global__ __launch_bounds__(256, D > 64 ? 1 : 2) void bwd_dkv_kernel(BwdParams p) {
  using G = BwdGeo<D>;
  constexpr int NC = G::NC, NDB = G::NDB, TILE = G::TILE;
  constexpr int SPAD = 2 * 64 * 4;            // lse2 and delta of the 64 rows, fp32
  constexpr int STAGE_B = 2 * TILE * 2 + SPAD;  // bytes: Q tile, dO tile, lse2, delta
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int L = p.L, S = p.S;
  const int g = p.Hq / p.Hkv;

  // work item: (level, b, hk); levels 0..n_ktiles-1 are the clean keys' tiles in
  // increasing key order (most queries first), then the noised keys' tiles
  // (batch, kv head) units grouped per XCD as in the dQ kernel: the key tiles of a unit,
  // which all stream the same Q / dO tiles, share one XCD's L2
  const int BK = p.B * p.Hkv;
  const int w = blockIdx.x;
  int level, bk;
  if ((BK & 7) == 0) {
    const int per_xcd = BK >> 3;
    const int local = w >> 3;
    level = local / per_xcd;
    bk = (w & 7) * per_xcd + local % per_xcd;
  } else {
    level = w / BK;
    bk = w % BK;
  }
  const int b = bk / p.Hkv, hk = bk % p.Hkv;
  const int src = level < p.n_ktiles ? 0 : 1;
  const int k0 = (src ? level - p.n_ktiles : level) * kRows;
  const int k_last = min(k0 + kRows, L) - 1;

  // query stream: the kind slots that read this key source and allow some of its
  // keys, each over the query tiles of every head of the group
  QStream qs = {};
  {
    int n = 0;
    for (int s = 0; s < p.n_kinds; ++s) {
      const int kind = s ? p.kinds[1] : p.kinds[0];
      if (src == 1 && kind != kDec) continue;
      const Interval u = col_union(kind, src, k0, k_last, S, L);
      if (u.hi <= u.lo) continue;
      const int qt0 = u.lo / kTK;
      const int nqt = (u.hi + kTK - 1) / kTK - qt0;
      if (n == 0) {
        qs.slot0 = s; qs.kind0 = kind; qs.qt00 = qt0; qs.nqt0 = nqt;
      } else {
        qs.slot1 = s; qs.kind1 = kind; qs.qt01 = qt0; qs.nqt1 = nqt;
      }
      ++n;
    }
    qs.n_slots = n;
    qs.per0 = n > 0 ? g * qs.nqt0 : 0;
    qs.ntot = qs.per0 + (n > 1 ? g * qs.nqt1 : 0);
  }
  const int ntot = qs.ntot;
  // stream index u -> (stream slot, query head, query tile)
  auto locate = [&](int u, int& ss, int& hq, int& qt) {
    ss = u >= qs.per0 ? 1 : 0;
    const int w = ss ? u - qs.per0 : u;
    const int nq = ss ? qs.nqt1 : qs.nqt0;
    hq = hk * g + w / nq;
    qt = (ss ? qs.qt01 : qs.qt00) + w % nq;
  };

  TileDma<D, kTK, kWaves> loader;
  loader.init(wave, lane);
  char E2D2_LDS* lds_b = (char E2D2_LDS*)smem_raw;
  const uint32_t q_bytes = (uint32_t)L * D * 2u;
  auto issue = [&](int u) {
    int ss, hq, qt;
    locate(u, ss, hq, qt);
    const int sl = ss ? qs.slot1 : qs.slot0;
    char E2D2_LDS* st = lds_b + (u & 1) * STAGE_B;
    const size_t row_base = ((size_t)b * p.Hq + hq) * (size_t)L;
    const BufDesc rq = buf_desc((sl ? p.q[1] : p.q[0]) + row_base * D, q_bytes);
    const BufDesc rd = buf_desc((sl ? p.dO[1] : p.dO[0]) + row_base * D, q_bytes);
    loader.load(rq, qt * kTK, st, wave);
    loader.load(rd, qt * kTK, st + TILE * 2, wave);
    if (wave < 2) {  // the 64 rows' lse2 (wave 0) and delta (wave 1), 4 bytes per lane
      const float* src_f = wave == 0 ? (sl ? p.lse2[1] : p.lse2[0]) : (sl ? p.delta[1] : p.delta[0]);
      dma_lds4(buf_desc(src_f + row_base, (uint32_t)L * 4u), (uint32_t)(lane * 4),
               (uint32_t)(qt * kTK * 4), lds_addr(st + 2 * TILE * 2 + wave * 256));
    }
  };
  if (ntot > 0) issue(0);

  // this wave's 32 keys: K and V rows as the B operands of S = Q K^T and dP = dO V^T
  const int kw0 = k0 + wave * 32;
  const bool wave_live = kw0 < L;
  const int kw1 = min(kw0 + 32, L);  // keys [kw0, kw1)
  const int kj = kw0 + (lane & 31);
  const bool key_ok = kj < L;
  const size_t kv_row = ((size_t)b * p.Hkv + hk) * (size_t)L + (key_ok ? kj : 0);
  bf16x8 kf[NC], vf[NC];
  {
    const __bf16* krow = (src ? p.k[1] : p.k[0]) + kv_row * D + ((lane >> 5) << 3);
    const __bf16* vrow = (src ? p.v[1] : p.v[0]) + kv_row * D + ((lane >> 5) << 3);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      kf[cc] = *(const bf16x8*)(krow + cc * 16);
      vf[cc] = *(const bf16x8*)(vrow + cc * 16);
    }
  }
  // rows allowing this lane's key, and the wave's union / common rows, per stream slot
  Interval civ[2] = {{0, 0}, {0, 0}}, cu[2] = {{0, 0}, {0, 0}}, ccm[2] = {{0, 0}, {0, 0}};
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    if (n < qs.n_slots && wave_live) {
      const int kind = n ? qs.kind1 : qs.kind0;
      if (key_ok) civ[n] = col_interval(kind, src, kj, S, L);
      cu[n] = col_union(kind, src, kw0, kw1 - 1, S, L);
      ccm[n] = col_common(kind, src, kw0, kw1 - 1, S, L);
    }
  }
  // the K / V registers have landed before the loop, so no wait for them sits inside it
  drain_vmem_visible();
  uint32_t koff[NC];
  k_offsets<D>(lane, koff);
  uint32_t offA[NDB], offB[NDB];
  vt_offsets<D>(lane, offA, offB);
  const float c = p.c;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  // Per 32-row query block the work runs in three phases, fenced so the compiler keeps
  // their order:
  //   A  S = Q K^T and dP = dO V^T (Q, dO rows as A operands, K and V in registers),
  //      with this block's transposed operands (dO^T, Q^T) and row statistics (lse,
  //      delta) read from LDS in between the products;
  //   B  P = 2^(S c - lse) and dS = P (dP - delta), packed to bf16 (VALU only);
  //   C  dV^T += dO^T P and dK^T += Q^T dS, with the Q / dO rows of the tile's next
  //      block read in between.
  // At one or two waves per SIMD nothing else hides LDS latency, so every read is
  // issued a whole phase before its first use instead of one product before it.
  const char E2D2_LDS* ldsc = (const char E2D2_LDS*)smem_raw;
  constexpr int NDS_A = 8 + 8 * NDB;  // LDS reads of phase A: lse, delta, dO^T, Q^T
  // Q and dO rows of query block QB of the tile in stage STG
  auto load_rows = [&](auto qbc, auto stg, bf16x8 (&qr)[NC], bf16x8 (&dr)[NC])
      __attribute__((always_inline)) {
    constexpr int QOFF = decltype(stg)::value * STAGE_B + decltype(qbc)::value * 64 * D;
    constexpr int DOFF = QOFF + TILE * 2;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qr[cc] = lds_read16<QOFF>(ldsc, koff[cc]);
      dr[cc] = lds_read16<DOFF>(ldsc, koff[cc]);
    }
  };
  // query block QB of the tile in stage STG (stream slot ss, query tile qt); qr / dr hold
  // its rows; with NEXT, the rows of block QB + 1 are read into them in phase C
  auto block = [&](auto qbc, int cl, int ss, int qt, auto stg, bf16x8 (&qr)[NC],
                   bf16x8 (&dr)[NC], auto nextc) __attribute__((always_inline)) {
    constexpr int QB = decltype(qbc)::value;
    constexpr int STG = decltype(stg)::value;
    constexpr bool NEXT = decltype(nextc)::value;
    constexpr int QOFF = STG * STAGE_B;
    constexpr int DOFF = QOFF + TILE * 2;
    constexpr int SOFF = QOFF + 2 * TILE * 2;
    // this lane's 16 query rows: QB * 32 + 8 (j / 4) + 4 (lane / 32) + j % 4
    const float E2D2_LDS* lse_t = (const float E2D2_LDS*)(smem_raw + SOFF);
    const float E2D2_LDS* dlt_t = lse_t + 64;
    const int rb = QB * 32 + ((lane >> 5) << 2);

    // ---- phase A
    f32x4 lq[4], dq4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lq[i] = *(const f32x4 E2D2_LDS*)(lse_t + rb + 8 * i);
      dq4[i] = *(const f32x4 E2D2_LDS*)(dlt_t + rb + 8 * i);
    }
    bf16x8 tdo[2][NDB], tq[2][NDB];
    read_vt_half32_lds<D, DOFF + QB * 64 * D, 0>(ldsc, offA, offB, tdo[0]);
    read_vt_half32_lds<D, QOFF + QB * 64 * D, 0>(ldsc, offA, offB, tq[0]);
    read_vt_half32_lds<D, DOFF + QB * 64 * D, 1>(ldsc, offA, offB, tdo[1]);
    read_vt_half32_lds<D, QOFF + QB * 64 * D, 1>(ldsc, offA, offB, tq[1]);
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      s = mfma32(qr[cc], kf[cc], s);
      dp = mfma32(dr[cc], vf[cc], dp);
    }
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) {
      constexpr int PER = NDS_A / (2 * NC), EXTRA = NDS_A % (2 * NC);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product, then its share of reads
      if (i < EXTRA) __builtin_amdgcn_sched_group_barrier(0x100, PER + 1, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase B
    if (cl == 1) {
      // rows [r.lo, r.hi) allow this lane's key: a 32-bit row mask of the block, shifted
      // to the lane's row set; register j holds block row 8 (j / 4) + j % 4 of that set
      const Interval r = ss ? civ[1] : civ[0];
      const int r0 = qt * kTK + QB * 32;
      const int a = min(max(r.lo - r0, 0), 32);
      const int e = min(max(r.hi - r0, 0), 32);
      uint32_t bits = e <= a ? 0u : (e - a >= 32 ? 0xffffffffu : ((1u << (e - a)) - 1u) << a);
      bits >>= (lane >> 5) << 2;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int off = ((j >> 2) << 3) + (j & 3);
        const uint32_t keep = (uint32_t)((int32_t)(bits << (31 - off)) >> 31);
        s[j] = __uint_as_float((__float_as_uint(s[j]) & keep) | (~keep & 0xff800000u));
      }
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float e[8], f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lj = lq[2 * h + (j >> 2)][j & 3];
        const float dj = dq4[2 * h + (j >> 2)][j & 3];
        const float pj = fast_exp2(fmaf(s[8 * h + j], c, -lj));
        e[j] = pj;
        f[j] = pj * (dp[8 * h + j] - dj);
      }
      pb[h] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      dsb[h] = to_bf16x8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase C
    if constexpr (NEXT) load_rows(IntC<QB + 1>{}, stg, qr, dr);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = mfma32(tdo[h][db], pb[h], dv[db]);
        dk[db] = mfma32(tq[h][db], dsb[h], dk[db]);
      }
    if constexpr (NEXT) {
#pragma unroll
      for (int i = 0; i < 4 * NDB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto tile = [&](int u, auto stg) __attribute__((always_inline)) {
    wait_vmem<0>();   // tile u is the only load in flight
    __syncthreads();  // tile u visible; everyone is done with the other stage
    if (u + 1 < ntot) issue(u + 1);
    if (!wave_live) return;
    int ss, hq, qt;
    locate(u, ss, hq, qt);
    const Interval un = ss ? cu[1] : cu[0];
    const Interval cm = ss ? ccm[1] : ccm[0];
    int cls[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r0 = qt * kTK + qb * 32;
      const int r1 = min(r0 + 32, L);
      int cl;
      if (r1 <= un.lo || r0 >= un.hi || r1 <= r0) cl = 0;
      else if (cm.lo <= r0 && r1 <= cm.hi && r1 - r0 == 32 && kw1 - kw0 == 32) cl = 2;
      else cl = 1;
      cls[qb] = cl;
    }
    bf16x8 qr[NC], dr[NC];
    if (cls[0]) {
      load_rows(IntC<0>{}, stg, qr, dr);
      if (cls[1]) {
        block(IntC<0>{}, cls[0], ss, qt, stg, qr, dr, BoolC<true>{});
        block(IntC<1>{}, cls[1], ss, qt, stg, qr, dr, BoolC<false>{});
      } else {
        block(IntC<0>{}, cls[0], ss, qt, stg, qr, dr, BoolC<false>{});
      }
    } else if (cls[1]) {
      load_rows(IntC<1>{}, stg, qr, dr);
      block(IntC<1>{}, cls[1], ss, qt, stg, qr, dr, BoolC<false>{});
    }
  };
  for (int u = 0; u < ntot; u += 2) {
    tile(u, IntC<0>{});
    if (u + 1 < ntot) tile(u + 1, IntC<1>{});
  }

  // dK = scale * dK^T, dV = dV^T, rows of this lane's key
  if (key_ok) {
    __bf16* ko = (src ? p.dk[1] : p.dk[0]) + kv_row * D;
    __bf16* vo = (src ? p.dv[1] : p.dv[0]) + kv_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = db * 32 + jg * 8 + ((lane >> 5) << 2);
        bf16x4 a, v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = (__bf16)(dk[db][jg * 4 + i] * p.scale);
          v[i] = (__bf16)(dv[db][jg * 4 + i]);
        }
        *(bf16x4*)(ko + d) = a;
        *(bf16x4*)(vo + d) = v;
      }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  using G = BwdGeo<D>;
  {
    const size_t smem = 2 * (size_t)G::STAGE * sizeof(__bf16);
    if (smem > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)bwd_dq_kernel<D>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
    }
    const int grid = p.n_qtiles * p.B * p.Hq * p.n_kinds;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(grid), dim3(256), smem, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const size_t smem = 2 * ((size_t)2 * G::TILE * sizeof(__bf16) + 2 * 64 * 4);
    if (smem > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)bwd_dkv_kernel<D>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
    }
    const int grid = 2 * p.n_ktiles * p.B * p.Hkv;
    hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3(grid), dim3(256), smem, stream, p);
    return hipGetLastError();
  }
}

}  // namespace

int bwd_tile_rows() { return kRows; }

hipError_t launch_train_bwd_bf16(const BwdParams& p, int d, hipStream_t stream) {
  if (p.B == 0 || p.Hq == 0 || p.L == 0) return hipSuccess;
  switch (d) {
    case 32: return launch_bwd_d<32>(p, stream);
    case 64: return launch_bwd_d<64>(p, stream);
    case 128: return launch_bwd_d<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace e2d2

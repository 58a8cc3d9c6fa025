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
//      (fp32, also written to the workspace for launch 2).  Per 32x32 block: S^T =
//      K Q^T and dP^T = V dO^T on the MFMA (K and V rows from LDS, Q and dO in
//      registers), P^T = 2^(S^T c - lse), dS^T = P^T (dP^T - delta), then dQ^T += K^T
//      dS^T with K^T from the transposing LDS read.
//   2. dK/dV: key-stationary: a workgroup owns 128 keys of one (batch, kv head, key
//      source) and walks the 64-row query tiles that allow any of them -- every query
//      head of the group, and for the clean keys both the encoder's and the decoder's
//      queries -- so each key's gradient is summed in one place.  Per 32x32 block:
//      S = Q K^T and dP = dO V^T (Q, dO rows from LDS, K and V in registers), then
//      dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from the transposing read.
//   Query and key tiles are staged through a 2-deep LDS ring with buffer_load ... lds,
//   as in the forward; partial 32x32 blocks are masked per element from the closed-
//   form row / column intervals (schedule.h), empty ones are skipped.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace e2d2 {
namespace {

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

  // work item, as in the forward: query tiles from the last to the first
  const int BH = p.B * p.Hq;
  const int per_level = BH * p.n_kinds;
  const int level = blockIdx.x / per_level;
  const int rem = blockIdx.x % per_level;
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

  // per-wave rows and per-lane query row
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

  // Q and dO rows of this lane's query as S^T / dP^T operands; lse and delta
  const size_t q_row = ((size_t)b * p.Hq + hq) * (size_t)L + (row_ok ? qi : 0);
  bf16x8 qf[NC], df[NC];
  {
    const __bf16* qrow = (slot ? p.q[1] : p.q[0]) + q_row * D + ((lane >> 5) << 3);
    const __bf16* drow = (slot ? p.dO[1] : p.dO[0]) + q_row * D + ((lane >> 5) << 3);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qf[cc] = *(const bf16x8*)(qrow + cc * 16);
      df[cc] = *(const bf16x8*)(drow + cc * 16);
    }
  }
  // delta = <dO, O> of this lane's row (the pair of lanes l, l^32 holds it in halves),
  // and lse * log2(e); both also go to the workspace for the dK/dV kernel.  Rows past
  // L: lse = +inf makes every p zero.
  float dlt, lse2;
  {
    const __bf16* orow = (slot ? p.o[1] : p.o[0]) + q_row * D + ((lane >> 5) << 3);
    float part = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const bf16x8 ov = *(const bf16x8*)(orow + cc * 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)ov[j], (float)df[cc][j], part);
    }
    dlt = pair_sum(part);
    lse2 = (slot ? p.lse[1] : p.lse[0])[q_row] * kLog2e;
    if (row_ok && lane < 32) {
      (slot ? p.delta[1] : p.delta[0])[q_row] = dlt;
      (slot ? p.lse2[1] : p.lse2[0])[q_row] = lse2;
    }
    if (!row_ok) {
      dlt = 0.f;
      lse2 = INFINITY;
    }
  }
  uint32_t koff[NC];
  k_offsets<D>(lane, koff);
  uint32_t offA[NDB], offB[NDB];
  vt_offsets<D>(lane, offA, offB);
  const uint32_t lds0 = lds_addr(lds_b);
  const float c = p.c;

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();

  // one 32-key block kb of the tile in stage STG
  auto block = [&](int t, int kb, int cl, auto stg) __attribute__((always_inline)) {
    constexpr int KOFF = decltype(stg)::value * STAGE * 2;
    bf16x8 kf[NC];
    if (kb == 0) kread_block<D, 0, KOFF>(lds0, koff, kf);
    else kread_block<D, 1, KOFF>(lds0, koff, kf);
    f32x16 st = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) st = mfma32(kf[cc], qf[cc], st);
    if (kb == 0) kread_block<D, 0, KOFF + TILE * 2>(lds0, koff, kf);
    else kread_block<D, 1, KOFF + TILE * 2>(lds0, koff, kf);
    f32x16 dpt = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) dpt = mfma32(kf[cc], df[cc], dpt);
    if (cl == 1) {
      const Interval r = tsrc(t) ? iv[1] : iv[0];
      const int kr = tnum(t) * kTK + kb * 32 + ((lane >> 5) << 2);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kr + ((j >> 2) << 3) + (j & 3);
        if (key < r.lo || key >= r.hi) st[j] = -INFINITY;
      }
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = fast_exp2(fmaf(st[8 * h + j], c, -lse2));
        e[j] = pj * (dpt[8 * h + j] - dlt);
      }
      dsb[h] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
    bf16x8 kt[2][NDB];
    if (kb == 0) read_vt_tile32<D, KOFF>(lds0, offA, offB, kt);
    else read_vt_tile32<D, KOFF + 64 * D>(lds0, offA, offB, kt);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = mfma32(kt[h][db], dsb[h], dq[db]);
  };
  auto tile = [&](int t, auto stg) __attribute__((always_inline)) {
    wait_vmem<0>();   // tile t is the only load in flight
    __syncthreads();  // tile t visible; everyone is done with the other stage
    if (t + 1 < ntot) issue(t + 1);
    int cls[2];
    classify_tile(t, cls);
    if (cls[0]) block(t, 0, cls[0], stg);
    if (cls[1]) block(t, 1, cls[1], stg);
  };
  for (int t = 0; t < ntot; t += 2) {
    tile(t, IntC<0>{});
    if (t + 1 < ntot) tile(t + 1, IntC<1>{});
  }

  // dQ = scale * dQ^T, rows of this lane's query
  if (row_ok) {
    __bf16* out = (slot ? p.dq[1] : p.dq[0]) + q_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = db * 32 + jg * 8 + ((lane >> 5) << 2);
        bf16x4 v;
        v[0] = (__bf16)(dq[db][jg * 4 + 0] * p.scale);
        v[1] = (__bf16)(dq[db][jg * 4 + 1] * p.scale);
        v[2] = (__bf16)(dq[db][jg * 4 + 2] * p.scale);
        v[3] = (__bf16)(dq[db][jg * 4 + 3] * p.scale);
        *(bf16x4*)(out + d) = v;
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
  const int BK = p.B * p.Hkv;
  const int level = blockIdx.x / BK;
  const int bk = blockIdx.x % BK;
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

  // rows of a 32-row block (KB) of the tile at LDS offset BASE, times the registers w:
  // the S = Q K^T (or dP = dO V^T) block.  The LDS reads of this kernel are left to
  // the compiler (its loads are issued from asm, see TileDma), which overlaps them
  // with the MFMAs: at one or two waves per SIMD nothing else hides their latency.
  const char E2D2_LDS* ldsc = (const char E2D2_LDS*)smem_raw;
  auto rows_dot = [&](auto kbc, auto basec, const bf16x8 (&w)[NC]) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value, BASE = decltype(basec)::value;
    constexpr int OFF = BASE + KB * 64 * D;
    f32x16 acc = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) acc = mfma32(lds_read16<OFF>(ldsc, koff[cc]), w[cc], acc);
    return acc;
  };
  // query block qb (32 rows) of the tile in stage STG, stream slot ss, query tile qt
  auto block = [&](auto qbc, int cl, int ss, int qt, auto stg) __attribute__((always_inline)) {
    constexpr int QB = decltype(qbc)::value;
    constexpr int QOFF = decltype(stg)::value * STAGE_B;
    constexpr int DOFF = QOFF + TILE * 2;
    constexpr int SOFF = QOFF + 2 * TILE * 2;
    f32x16 s = rows_dot(IntC<QB>{}, IntC<QOFF>{}, kf);
    const f32x16 dp = rows_dot(IntC<QB>{}, IntC<DOFF>{}, vf);
    // this lane's 16 query rows: QB * 32 + 8 (j / 4) + 4 (lane / 32) + j % 4
    const float E2D2_LDS* lse_t = (const float E2D2_LDS*)(smem_raw + SOFF);
    const float E2D2_LDS* dlt_t = lse_t + 64;
    const int rb = QB * 32 + ((lane >> 5) << 2);
    if (cl == 1) {
      const Interval r = ss ? civ[1] : civ[0];
      const int q_r = qt * kTK + rb;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int q = q_r + ((j >> 2) << 3) + (j & 3);
        if (q < r.lo || q >= r.hi) s[j] = -INFINITY;
      }
    }
    // per 16-row half h: P and dS of registers 8h .. 8h+7, then dV^T += dO^T P and
    // dK^T += Q^T dS for those 16 query rows
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 l0 = *(const f32x4 E2D2_LDS*)(lse_t + rb + 16 * h);
      const f32x4 l1 = *(const f32x4 E2D2_LDS*)(lse_t + rb + 16 * h + 8);
      const f32x4 d0 = *(const f32x4 E2D2_LDS*)(dlt_t + rb + 16 * h);
      const f32x4 d1 = *(const f32x4 E2D2_LDS*)(dlt_t + rb + 16 * h + 8);
      float e[8], f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lj = j < 4 ? l0[j] : l1[j - 4];
        const float dj = j < 4 ? d0[j] : d1[j - 4];
        const float pj = fast_exp2(fmaf(s[8 * h + j], c, -lj));
        e[j] = pj;
        f[j] = pj * (dp[8 * h + j] - dj);
      }
      const bf16x8 pb = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      const bf16x8 dsb = to_bf16x8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
      bf16x8 tf[NDB];
      if (h == 0) read_vt_half32_lds<D, DOFF + QB * 64 * D, 0>(ldsc, offA, offB, tf);
      else read_vt_half32_lds<D, DOFF + QB * 64 * D, 1>(ldsc, offA, offB, tf);
#pragma unroll
      for (int db = 0; db < NDB; ++db) dv[db] = mfma32(tf[db], pb, dv[db]);
      if (h == 0) read_vt_half32_lds<D, QOFF + QB * 64 * D, 0>(ldsc, offA, offB, tf);
      else read_vt_half32_lds<D, QOFF + QB * 64 * D, 1>(ldsc, offA, offB, tf);
#pragma unroll
      for (int db = 0; db < NDB; ++db) dk[db] = mfma32(tf[db], dsb, dk[db]);
    }
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
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r0 = qt * kTK + qb * 32;
      const int r1 = min(r0 + 32, L);
      int cl;
      if (r1 <= un.lo || r0 >= un.hi || r1 <= r0) cl = 0;
      else if (cm.lo <= r0 && r1 <= cm.hi && r1 - r0 == 32 && kw1 - kw0 == 32) cl = 2;
      else cl = 1;
      if (cl) {
        if (qb == 0) block(IntC<0>{}, cl, ss, qt, stg);
        else block(IntC<1>{}, cl, ss, qt, stg);
      }
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

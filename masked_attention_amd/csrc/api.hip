// C-ABI entry points: argument validation (before anything touches the GPU), tile
// schedule sizing and kernel dispatch.  Declarations and contracts: include/e2d2_attn.h.
#include <math.h>
#include <stdint.h>

#include "../../include/e2d2_attn.h"
#include "kernels.h"
#include "schedule.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr long long kMaxLen = 1ll << 24;  // per-head rows (sequence, cache capacity)

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool scale_ok(float s) { return isfinite(s) && s > 0.f; }
// One (batch, head) slice of `rows` rows is addressed with 32-bit byte offsets (buffer
// resources) on the GPU: keep it below 2 GiB.
bool slice_ok(long long rows, int d) { return rows * d * 2 < (1ll << 31); }
int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

e2d2_status hip_status(hipError_t e) {
  if (e == hipSuccess) return E2D2_OK;
  g_last_hip_error = (int)e;
  return E2D2_ERR_HIP;
}

// Shared shape checks of the training calls.
e2d2_status check_train_shape(int dtype, int B, int Hq, int Hkv, int L, int d, int S,
                              float scale) {
  if (dtype != E2D2_F32 && dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return E2D2_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || S <= 0) return E2D2_ERR_SHAPE;
  if (Hq % Hkv != 0 || L > kMaxLen || !scale_ok(scale)) return E2D2_ERR_SHAPE;
  if (!slice_ok(L, d)) return E2D2_ERR_SHAPE;
  const int bm = dtype == E2D2_BF16 ? e2d2::train_tile_bm(d) : e2d2::kF32TileBM;
  if ((long long)B * Hq * 2 * cdiv(L, bm) > INT32_MAX) return E2D2_ERR_SHAPE;
  return E2D2_OK;
}

// Denoise query grouping: 32-row chunks per head and 2 column blocks per workgroup.
struct DenoiseShape {
  int g, nrc, ncb, n_qgroups, n_tiles_cache, n_tiles, n_split;
};
DenoiseShape denoise_shape(int B, int Hq, int Hkv, int S, long long C) {
  DenoiseShape s;
  s.g = Hq / Hkv;
  s.nrc = cdiv(S, 32);
  s.ncb = s.g * s.nrc;
  s.n_qgroups = cdiv(s.ncb, 2);
  s.n_tiles_cache = cdiv(C, e2d2::kDenoiseTileBN);
  s.n_tiles = s.n_tiles_cache + cdiv(S, e2d2::kDenoiseTileBN);
  s.n_split = e2d2::denoise_splits(B, Hkv, s.n_qgroups, s.n_tiles);
  return s;
}

size_t denoise_ws_bytes(int dtype, int B, int Hq, int Hkv, int S, int d, long long C) {
  if (dtype != E2D2_BF16) return 0;
  const DenoiseShape s = denoise_shape(B, Hq, Hkv, S, C);
  if (s.n_split == 1) return 0;
  const size_t rows = (size_t)B * Hkv * s.n_qgroups * s.n_split * 64;
  const size_t o_bytes = rows * d * sizeof(float);
  const size_t ml_bytes = rows * 2 * sizeof(float);
  return ((o_bytes + 255) & ~(size_t)255) + ml_bytes;
}

void fill_f32_common(e2d2::F32Params& p, int B, int Hq, int Hkv, int L, int S, long long C,
                     float scale, unsigned long long* visits) {
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.L = L;
  p.S = S;
  p.C = (int)C;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.visits = visits;
}

}  // namespace

extern "C" {

int e2d2_abi_version(void) { return E2D2_ABI_VERSION; }

const char* e2d2_status_string(int status) {
  switch (status) {
    case E2D2_OK: return "ok";
    case E2D2_ERR_NULL: return "a required pointer is NULL";
    case E2D2_ERR_SHAPE: return "invalid size, head grouping, scale or alignment";
    case E2D2_ERR_UNSUPPORTED: return "unsupported dtype, head dimension or kind";
    case E2D2_ERR_CAPACITY: return "cache_len + S exceeds cache_cap";
    case E2D2_ERR_WORKSPACE: return "workspace too small";
    case E2D2_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int e2d2_last_hip_error(void) { return g_last_hip_error; }

e2d2_status e2d2_attn_encoder_blockcausal(int dtype, int B, int Hq, int Hkv, int L, int d, int S,
                                          float scale, const void* q, const void* k,
                                          const void* v, void* o, float* lse,
                                          unsigned long long* dbg_tile_visits, void* stream) {
  e2d2_status st = check_train_shape(dtype, B, Hq, Hkv, L, d, S, scale);
  if (st != E2D2_OK) return st;
  if (!q || !k || !v || !o) return E2D2_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned4(lse)) || (dbg_tile_visits && ((uintptr_t)dbg_tile_visits & 7u)))
    return E2D2_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == E2D2_BF16) {
    e2d2::TrainParams p = {};
    p.q[0] = (const __bf16*)q;
    p.o[0] = (__bf16*)o;
    p.lse[0] = lse;
    p.k[0] = p.k[1] = (const __bf16*)k;
    p.v[0] = p.v[1] = (const __bf16*)v;
    p.kinds[0] = p.kinds[1] = e2d2::kEnc;
    p.n_kinds = 1;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.S = S;
    p.kv_rows = L;
    p.n_qtiles = cdiv(L, e2d2::train_tile_bm(d));
    p.xcd_groups = (B * Hq) % 8 == 0;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    p.visits = dbg_tile_visits;
    return hip_status(e2d2::launch_train_bf16(p, d, s));
  }
  e2d2::F32Params p = {};
  fill_f32_common(p, B, Hq, Hkv, L, S, 0, scale, dbg_tile_visits);
  p.q[0] = (const float*)q;
  p.o[0] = (float*)o;
  p.lse[0] = lse;
  p.kf[0][0] = p.kf[0][1] = (const float*)k;
  p.vf[0][0] = p.vf[0][1] = (const float*)v;
  p.src_rows[0][0] = p.src_rows[0][1] = L;
  p.kinds[0] = p.kinds[1] = e2d2::kEnc;
  p.n_kinds = 1;
  p.n_qtiles = cdiv(L, e2d2::kF32TileBM);
  return hip_status(e2d2::launch_attn_f32(p, d, s));
}

e2d2_status e2d2_attn_encoder_blockcausal_varlen(int dtype, int B, int Hq, int Hkv, int L, int d,
                                                 int S, float scale, const void* q, const void* k,
                                                 const void* v, long long kv_rows,
                                                 const int* lens, void* o, float* lse,
                                                 unsigned long long* dbg_tile_visits,
                                                 void* stream) {
  e2d2_status st = check_train_shape(dtype, B, Hq, Hkv, L, d, S, scale);
  if (st != E2D2_OK) return st;
  if (dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (kv_rows < L || kv_rows > kMaxLen || !slice_ok(kv_rows, d)) return E2D2_ERR_SHAPE;
  if (!q || !k || !v || !o || !lens) return E2D2_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lens) ||
      (lse && !aligned4(lse)) || (dbg_tile_visits && ((uintptr_t)dbg_tile_visits & 7u)))
    return E2D2_ERR_SHAPE;
  e2d2::TrainParams p = {};
  p.q[0] = (const __bf16*)q;
  p.o[0] = (__bf16*)o;
  p.lse[0] = lse;
  p.k[0] = p.k[1] = (const __bf16*)k;
  p.v[0] = p.v[1] = (const __bf16*)v;
  p.kinds[0] = p.kinds[1] = e2d2::kEnc;
  p.n_kinds = 1;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.S = S;
  p.kv_rows = (int)kv_rows;
  p.lens = lens;
  p.n_qtiles = cdiv(L, e2d2::train_tile_bm(d));
  p.xcd_groups = (B * Hq) % 8 == 0;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.visits = dbg_tile_visits;
  return hip_status(e2d2::launch_train_bf16(p, d, (hipStream_t)stream));
}

e2d2_status e2d2_attn_train_fwd(int dtype, int B, int Hq, int Hkv, int L, int d, int S, float scale,
                                const void* q_dec, const void* k_ctx, const void* v_ctx,
                                const void* k_dec, const void* v_dec, void* o_dec, float* lse_dec,
                                const void* q_enc, void* o_enc, float* lse_enc,
                                unsigned long long* dbg_tile_visits, void* stream) {
  e2d2_status st = check_train_shape(dtype, B, Hq, Hkv, L, d, S, scale);
  if (st != E2D2_OK) return st;
  if (!q_dec || !k_ctx || !v_ctx || !k_dec || !v_dec || !o_dec) return E2D2_ERR_NULL;
  const bool with_enc = q_enc != nullptr;
  if (with_enc && !o_enc) return E2D2_ERR_NULL;
  if (!with_enc && (o_enc || lse_enc)) return E2D2_ERR_NULL;
  if (!aligned16(q_dec) || !aligned16(k_ctx) || !aligned16(v_ctx) || !aligned16(k_dec) ||
      !aligned16(v_dec) || !aligned16(o_dec) || (lse_dec && !aligned4(lse_dec)) ||
      (with_enc && (!aligned16(q_enc) || !aligned16(o_enc) || (lse_enc && !aligned4(lse_enc)))) ||
      (dbg_tile_visits && ((uintptr_t)dbg_tile_visits & 7u)))
    return E2D2_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == E2D2_BF16) {
    e2d2::TrainParams p = {};
    p.q[0] = (const __bf16*)q_dec;
    p.o[0] = (__bf16*)o_dec;
    p.lse[0] = lse_dec;
    p.q[1] = (const __bf16*)q_enc;
    p.o[1] = (__bf16*)o_enc;
    p.lse[1] = lse_enc;
    p.k[0] = (const __bf16*)k_ctx;
    p.v[0] = (const __bf16*)v_ctx;
    p.k[1] = (const __bf16*)k_dec;
    p.v[1] = (const __bf16*)v_dec;
    p.kinds[0] = e2d2::kDec;
    p.kinds[1] = e2d2::kEnc;
    p.n_kinds = with_enc ? 2 : 1;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.S = S;
    p.kv_rows = L;
    p.n_qtiles = cdiv(L, e2d2::train_tile_bm(d));
    p.xcd_groups = (B * Hq * p.n_kinds) % 8 == 0;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    p.visits = dbg_tile_visits;
    return hip_status(e2d2::launch_train_bf16(p, d, s));
  }
  e2d2::F32Params p = {};
  fill_f32_common(p, B, Hq, Hkv, L, S, 0, scale, dbg_tile_visits);
  p.q[0] = (const float*)q_dec;
  p.o[0] = (float*)o_dec;
  p.lse[0] = lse_dec;
  p.q[1] = (const float*)q_enc;
  p.o[1] = (float*)o_enc;
  p.lse[1] = lse_enc;
  for (int sl = 0; sl < 2; ++sl) {
    p.kf[sl][0] = (const float*)k_ctx;
    p.vf[sl][0] = (const float*)v_ctx;
    p.kf[sl][1] = (const float*)k_dec;
    p.vf[sl][1] = (const float*)v_dec;
    p.src_rows[sl][0] = p.src_rows[sl][1] = L;
  }
  p.kinds[0] = e2d2::kDec;
  p.kinds[1] = e2d2::kEnc;
  p.n_kinds = with_enc ? 2 : 1;
  p.n_qtiles = cdiv(L, e2d2::kF32TileBM);
  return hip_status(e2d2::launch_attn_f32(p, d, s));
}

size_t e2d2_attn_train_bwd_workspace_bytes(int dtype, int B, int Hq, int L, int with_enc) {
  if (dtype != E2D2_BF16 || B <= 0 || Hq <= 0 || L <= 0 || L > kMaxLen) return 0;
  const size_t rows = (size_t)B * Hq * L;
  // delta and lse*log2(e) per query row and kind, each array padded to 256 bytes
  const size_t arr = (rows * sizeof(float) + 255) & ~(size_t)255;
  return arr * 2 * (with_enc ? 2 : 1);
}

e2d2_status e2d2_attn_train_bwd(int dtype, int B, int Hq, int Hkv, int L, int d, int S,
                                float scale, const void* q_dec, const void* k_ctx,
                                const void* v_ctx, const void* k_dec, const void* v_dec,
                                const void* o_dec, const float* lse_dec, const void* do_dec,
                                const void* q_enc, const void* o_enc, const float* lse_enc,
                                const void* do_enc, void* dq_dec, void* dk_ctx, void* dv_ctx,
                                void* dk_dec, void* dv_dec, void* dq_enc, void* workspace,
                                size_t workspace_bytes, void* stream) {
  e2d2_status st = check_train_shape(dtype, B, Hq, Hkv, L, d, S, scale);
  if (st != E2D2_OK) return st;
  if (dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (!q_dec || !k_ctx || !v_ctx || !k_dec || !v_dec || !o_dec || !lse_dec || !do_dec ||
      !dq_dec || !dk_ctx || !dv_ctx || !dk_dec || !dv_dec)
    return E2D2_ERR_NULL;
  const bool with_enc = q_enc != nullptr;
  if (with_enc && (!o_enc || !lse_enc || !do_enc || !dq_enc)) return E2D2_ERR_NULL;
  if (!with_enc && (o_enc || lse_enc || do_enc || dq_enc)) return E2D2_ERR_NULL;
  const void* a16[] = {q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, do_dec, dq_dec, dk_ctx, dv_ctx,
                       dk_dec, dv_dec};
  for (const void* x : a16)
    if (!aligned16(x)) return E2D2_ERR_SHAPE;
  if (!aligned4(lse_dec)) return E2D2_ERR_SHAPE;
  if (with_enc && (!aligned16(q_enc) || !aligned16(o_enc) || !aligned16(do_enc) ||
                   !aligned16(dq_enc) || !aligned4(lse_enc)))
    return E2D2_ERR_SHAPE;
  const size_t need = e2d2_attn_train_bwd_workspace_bytes(dtype, B, Hq, L, with_enc ? 1 : 0);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return E2D2_ERR_WORKSPACE;
  const int rows_per_tile = e2d2::bwd_tile_rows();
  if ((long long)cdiv(L, rows_per_tile) * B * Hq * 2 > INT32_MAX) return E2D2_ERR_SHAPE;
  e2d2::BwdParams p = {};
  p.q[0] = (const __bf16*)q_dec;
  p.o[0] = (const __bf16*)o_dec;
  p.dO[0] = (const __bf16*)do_dec;
  p.lse[0] = lse_dec;
  p.dq[0] = (__bf16*)dq_dec;
  p.q[1] = (const __bf16*)q_enc;
  p.o[1] = (const __bf16*)o_enc;
  p.dO[1] = (const __bf16*)do_enc;
  p.lse[1] = lse_enc;
  p.dq[1] = (__bf16*)dq_enc;
  p.k[0] = (const __bf16*)k_ctx;
  p.v[0] = (const __bf16*)v_ctx;
  p.k[1] = (const __bf16*)k_dec;
  p.v[1] = (const __bf16*)v_dec;
  p.dk[0] = (__bf16*)dk_ctx;
  p.dv[0] = (__bf16*)dv_ctx;
  p.dk[1] = (__bf16*)dk_dec;
  p.dv[1] = (__bf16*)dv_dec;
  const size_t rows = (size_t)B * Hq * L;
  const size_t arr = (rows * sizeof(float) + 255) & ~(size_t)255;
  char* ws = (char*)workspace;
  p.delta[0] = (float*)ws;
  p.lse2[0] = (float*)(ws + arr);
  p.delta[1] = with_enc ? (float*)(ws + 2 * arr) : nullptr;
  p.lse2[1] = with_enc ? (float*)(ws + 3 * arr) : nullptr;
  p.kinds[0] = e2d2::kDec;
  p.kinds[1] = e2d2::kEnc;
  p.n_kinds = with_enc ? 2 : 1;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.S = S;
  p.n_qtiles = cdiv(L, rows_per_tile);
  p.n_ktiles = cdiv(L, rows_per_tile);
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  return hip_status(e2d2::launch_train_bwd_bf16(p, d, (hipStream_t)stream));
}

size_t e2d2_attn_denoise_workspace_bytes(int dtype, int B, int Hq, int Hkv, int S, int d,
                                         long long cache_len) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || !head_dim_ok(d) || Hq % Hkv != 0 ||
      cache_len < 0 || cache_len > kMaxLen)
    return 0;
  return denoise_ws_bytes(dtype, B, Hq, Hkv, S, d, cache_len);
}

namespace {

// Shared by the uniform and the per-sequence denoise calls (lens == NULL: every
// sequence has cache_len rows; else sequence b has lens[b], at most cache_len).
e2d2_status denoise_step(int dtype, int B, int Hq, int Hkv, int S, int d, float scale,
                         const void* q_blk, const void* k_cache, const void* v_cache,
                         const int* lens, long long cache_len, long long cache_cap,
                         const void* k_blk, const void* v_blk, void* o_blk, float* lse_blk,
                         void* workspace, size_t workspace_bytes,
                         unsigned long long* dbg_tile_visits, void* stream,
                         bool launch = true, bool own_scratch = false) {
  if (dtype != E2D2_F32 && dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (lens != nullptr && dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return E2D2_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || Hq % Hkv != 0 || !scale_ok(scale))
    return E2D2_ERR_SHAPE;
  if (cache_len < 0 || cache_cap < 0 || cache_len > cache_cap || cache_cap > kMaxLen ||
      S > kMaxLen || !slice_ok(cache_cap, d) || !slice_ok(S, d))
    return E2D2_ERR_SHAPE;
  if (!q_blk || !k_blk || !v_blk || !o_blk) return E2D2_ERR_NULL;
  if (cache_len > 0 && (!k_cache || !v_cache)) return E2D2_ERR_NULL;
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o_blk) ||
      (cache_len > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) ||
      (lse_blk && !aligned4(lse_blk)) || (dbg_tile_visits && ((uintptr_t)dbg_tile_visits & 7u)))
    return E2D2_ERR_SHAPE;
  if (dtype == E2D2_BF16) {
    const DenoiseShape sh = denoise_shape(B, Hq, Hkv, S, cache_len);
    if ((long long)B * Hkv * sh.n_qgroups * sh.n_split > INT32_MAX) return E2D2_ERR_SHAPE;
  } else if ((long long)B * Hq * cdiv(S, e2d2::kF32TileBM) > INT32_MAX) {
    return E2D2_ERR_SHAPE;
  }
  const size_t need = denoise_ws_bytes(dtype, B, Hq, Hkv, S, d, cache_len);
  if (own_scratch && need > 0) {
    // the library's own device scratch (no allocation): its address on this device
    size_t have = 0;
    const hipError_t e = e2d2::denoise_scratch(&workspace, &have);
    if (e != hipSuccess) return hip_status(e);
    if (need > have) return E2D2_ERR_WORKSPACE;
    workspace_bytes = have;
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return E2D2_ERR_WORKSPACE;
  if (!launch) return E2D2_OK;
  hipStream_t s = (hipStream_t)stream;
  // An empty cache has no rows to read; any non-NULL pointer stands in.
  const void* kc = cache_len > 0 ? k_cache : k_blk;
  const void* vc = cache_len > 0 ? v_cache : v_blk;
  if (dtype == E2D2_BF16) {
    const DenoiseShape sh = denoise_shape(B, Hq, Hkv, S, cache_len);
    e2d2::DenoiseParams p = {};
    p.q = (const __bf16*)q_blk;
    p.k_cache = (const __bf16*)kc;
    p.v_cache = (const __bf16*)vc;
    p.k_blk = (const __bf16*)k_blk;
    p.v_blk = (const __bf16*)v_blk;
    p.o = (__bf16*)o_blk;
    p.lse = lse_blk;
    p.lens = lens;
    if (need > 0) {
      const size_t rows = (size_t)B * Hkv * sh.n_qgroups * sh.n_split * 64;
      p.ws_o = (float*)workspace;
      p.ws_ml = (float*)((char*)workspace + ((rows * d * sizeof(float) + 255) & ~(size_t)255));
    }
    p.cap = cache_len > 0 ? cache_cap : 0;
    p.C = (int)cache_len;
    p.S = S;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.g = sh.g;
    p.nrc = sh.nrc;
    p.ncb = sh.ncb;
    p.n_qgroups = sh.n_qgroups;
    p.n_split = sh.n_split;
    p.n_tiles = sh.n_tiles;
    p.n_tiles_cache = sh.n_tiles_cache;
    p.c = scale * 1.4426950408889634f;
    p.visits = dbg_tile_visits;
    return hip_status(e2d2::launch_denoise_bf16(p, d, s));
  }
  e2d2::F32Params p = {};
  fill_f32_common(p, B, Hq, Hkv, 0, S, cache_len, scale, dbg_tile_visits);
  p.q[0] = (const float*)q_blk;
  p.o[0] = (float*)o_blk;
  p.lse[0] = lse_blk;
  p.kf[0][0] = (const float*)kc;
  p.vf[0][0] = (const float*)vc;
  p.src_rows[0][0] = cache_len > 0 ? (int)cache_cap : 0;
  p.kf[0][1] = (const float*)k_blk;
  p.vf[0][1] = (const float*)v_blk;
  p.src_rows[0][1] = S;
  p.kinds[0] = p.kinds[1] = e2d2::kDenoise;
  p.n_kinds = 1;
  p.n_qtiles = cdiv(S, e2d2::kF32TileBM);
  return hip_status(e2d2::launch_attn_f32(p, d, s));
}

}  // namespace

e2d2_status e2d2_attn_denoise_step(int dtype, int B, int Hq, int Hkv, int S, int d, float scale,
                                   const void* q_blk, const void* k_cache, const void* v_cache,
                                   long long cache_len, long long cache_cap, const void* k_blk,
                                   const void* v_blk, void* o_blk, float* lse_blk, void* workspace,
                                   size_t workspace_bytes, unsigned long long* dbg_tile_visits,
                                   void* stream) {
  return denoise_step(dtype, B, Hq, Hkv, S, d, scale, q_blk, k_cache, v_cache, nullptr, cache_len,
                      cache_cap, k_blk, v_blk, o_blk, lse_blk, workspace, workspace_bytes,
                      dbg_tile_visits, stream);
}

e2d2_status e2d2_attn_denoise_step_noalloc(int dtype, int B, int Hq, int Hkv, int S, int d,
                                           float scale, const void* q_blk, const void* k_cache,
                                           const void* v_cache, long long cache_len,
                                           long long cache_cap, const void* k_blk,
                                           const void* v_blk, void* o_blk, float* lse_blk,
                                           unsigned long long* dbg_tile_visits, void* stream) {
  return denoise_step(dtype, B, Hq, Hkv, S, d, scale, q_blk, k_cache, v_cache, nullptr, cache_len,
                      cache_cap, k_blk, v_blk, o_blk, lse_blk, nullptr, 0, dbg_tile_visits, stream,
                      true, true);
}

e2d2_status e2d2_attn_denoise_step_varlen(int dtype, int B, int Hq, int Hkv, int S, int d,
                                          float scale, const void* q_blk, const void* k_cache,
                                          const void* v_cache, const int* cache_lens,
                                          long long max_cache_len, long long cache_cap,
                                          const void* k_blk, const void* v_blk, void* o_blk,
                                          float* lse_blk, void* workspace, size_t workspace_bytes,
                                          unsigned long long* dbg_tile_visits, void* stream) {
  if (cache_lens == nullptr) return E2D2_ERR_NULL;
  if (((uintptr_t)cache_lens & 3u) != 0) return E2D2_ERR_SHAPE;
  if (max_cache_len > 0 && (!k_cache || !v_cache)) return E2D2_ERR_NULL;
  return denoise_step(dtype, B, Hq, Hkv, S, d, scale, q_blk, k_cache, v_cache, cache_lens,
                      max_cache_len, cache_cap, k_blk, v_blk, o_blk, lse_blk, workspace,
                      workspace_bytes, dbg_tile_visits, stream);
}

e2d2_status e2d2_decoder_layer_denoise_step(int dtype, int B, int Hq, int Hkv, int S, int d,
                                            int Dm, float scale, const void* x,
                                            const void* w_qkv, const void* w_o,
                                            const void* k_cache, const void* v_cache,
                                            long long cache_len, long long cache_cap,
                                            void* q_blk, void* k_blk, void* v_blk, void* o_blk,
                                            float* lse_blk, void* y, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (dtype != E2D2_BF16 || !head_dim_ok(d)) return E2D2_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || Dm <= 0 || Hq % Hkv != 0 || Dm % 8 != 0)
    return E2D2_ERR_SHAPE;
  if (!x || !w_qkv || !w_o || !y) return E2D2_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(w_o) || !aligned16(y))
    return E2D2_ERR_SHAPE;
  // Every operand of the projections is addressed with 32-bit byte offsets.
  const long long M = (long long)B * S;
  const long long n_qkv = (long long)(Hq + 2 * Hkv) * d;
  const long long k_o = (long long)Hq * d;
  const long long lim = 1ll << 31;
  if (M * Dm * 2 >= lim || n_qkv * Dm * 2 >= lim || Dm * k_o * 2 >= lim || M * k_o * 2 >= lim)
    return E2D2_ERR_SHAPE;
  // the attention's own checks (pointers, cache, workspace), before anything launches
  e2d2_status st = denoise_step(dtype, B, Hq, Hkv, S, d, scale, q_blk, k_cache, v_cache, nullptr,
                                cache_len, cache_cap, k_blk, v_blk, o_blk, lse_blk, workspace,
                                workspace_bytes, nullptr, stream, false);
  if (st != E2D2_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  int log2d = 0;
  while ((1 << log2d) < d) ++log2d;

  // q, k, v = x W_qkv^T, written per head
  e2d2::LinearParams lp = {};
  lp.a = (const __bf16*)x;
  lp.w = (const __bf16*)w_qkv;
  lp.c[0] = (__bf16*)q_blk;
  lp.c[1] = (__bf16*)k_blk;
  lp.c[2] = (__bf16*)v_blk;
  lp.c_n0[0] = 0;
  lp.c_n0[1] = Hq * d;
  lp.c_n0[2] = (Hq + Hkv) * d;
  lp.c_h[0] = Hq;
  lp.c_h[1] = lp.c_h[2] = Hkv;
  lp.c_w = d;
  lp.a_sb = S * Dm;
  lp.a_ss = Dm;
  lp.a_sh = 0;
  lp.a_heads = 0;
  lp.M = (int)M;
  lp.N = (int)n_qkv;
  lp.K = Dm;
  lp.S = S;
  lp.a_bytes = (unsigned)(M * Dm * 2);
  lp.w_bytes = (unsigned)(n_qkv * Dm * 2);
  hipError_t e = e2d2::launch_linear_bf16(lp, s);
  if (e != hipSuccess) return hip_status(e);

  st = denoise_step(dtype, B, Hq, Hkv, S, d, scale, q_blk, k_cache, v_cache, nullptr, cache_len,
                    cache_cap, k_blk, v_blk, o_blk, lse_blk, workspace, workspace_bytes, nullptr,
                    stream);
  if (st != E2D2_OK) return st;

  // y = concat_h(o) W_o^T, o read per head
  e2d2::LinearParams op = {};
  op.a = (const __bf16*)o_blk;
  op.w = (const __bf16*)w_o;
  op.c[0] = op.c[1] = op.c[2] = (__bf16*)y;
  op.c_n0[0] = 0;
  op.c_n0[1] = op.c_n0[2] = Dm;
  op.c_h[0] = op.c_h[1] = op.c_h[2] = 1;
  op.c_w = Dm;
  op.a_sb = Hq * S * d;
  op.a_ss = d;
  op.a_sh = S * d;
  op.a_heads = 1;
  op.a_log2w = log2d;
  op.M = (int)M;
  op.N = Dm;
  op.K = (int)k_o;
  op.S = S;
  op.a_bytes = (unsigned)(M * k_o * 2);
  op.w_bytes = (unsigned)(Dm * k_o * 2);
  return hip_status(e2d2::launch_linear_bf16(op, s));
}

e2d2_status e2d2_kv_cache_append_varlen(int dtype, int B, int Hkv, int S, int d, void* k_cache,
                                        void* v_cache, const int* cache_lens,
                                        long long max_cache_len, long long cache_cap,
                                        const void* k_new, const void* v_new, void* stream) {
  if (dtype != E2D2_F32 && dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return E2D2_ERR_UNSUPPORTED;
  if (B <= 0 || Hkv <= 0 || S <= 0 || max_cache_len < 0 || cache_cap <= 0 ||
      cache_cap > kMaxLen)
    return E2D2_ERR_SHAPE;
  if (max_cache_len + S > cache_cap) return E2D2_ERR_CAPACITY;
  if (!k_cache || !v_cache || !k_new || !v_new || !cache_lens) return E2D2_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
      ((uintptr_t)cache_lens & 3u) != 0)
    return E2D2_ERR_SHAPE;
  return hip_status(e2d2::launch_kv_append_varlen(dtype == E2D2_BF16 ? 2 : 4, B, Hkv, S, d,
                                                  k_cache, v_cache, cache_lens, max_cache_len,
                                                  cache_cap, k_new, v_new, (hipStream_t)stream));
}

e2d2_status e2d2_kv_cache_append(int dtype, int B, int Hkv, int S, int d, void* k_cache,
                                 void* v_cache, long long cache_len, long long cache_cap,
                                 const void* k_new, const void* v_new, void* stream) {
  if (dtype != E2D2_F32 && dtype != E2D2_BF16) return E2D2_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return E2D2_ERR_UNSUPPORTED;
  if (B <= 0 || Hkv <= 0 || S <= 0 || cache_len < 0 || cache_cap <= 0 || cache_cap > kMaxLen)
    return E2D2_ERR_SHAPE;
  if (cache_len + S > cache_cap) return E2D2_ERR_CAPACITY;
  if (!k_cache || !v_cache || !k_new || !v_new) return E2D2_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return E2D2_ERR_SHAPE;
  return hip_status(e2d2::launch_kv_append(dtype == E2D2_BF16 ? 2 : 4, B, Hkv, S, d, k_cache,
                                           v_cache, cache_len, cache_cap, k_new, v_new,
                                           (hipStream_t)stream));
}

e2d2_status e2d2_attn_tile_shape(int kind, int dtype, int d, int* bm, int* bn) {
  if (!bm || !bn) return E2D2_ERR_NULL;
  if ((dtype != E2D2_F32 && dtype != E2D2_BF16) || !head_dim_ok(d)) return E2D2_ERR_UNSUPPORTED;
  if (kind == E2D2_KIND_ENC || kind == E2D2_KIND_DEC) {
    *bm = dtype == E2D2_BF16 ? e2d2::train_tile_bm(d) : e2d2::kF32TileBM;
    *bn = dtype == E2D2_BF16 ? e2d2::train_tile_bn() : e2d2::kF32TileBN;
    return E2D2_OK;
  }
  if (kind == E2D2_KIND_DENOISE) {
    *bm = dtype == E2D2_BF16 ? e2d2::kDenoiseTileBM : e2d2::kF32TileBM;
    *bn = dtype == E2D2_BF16 ? e2d2::kDenoiseTileBN : e2d2::kF32TileBN;
    return E2D2_OK;
  }
  return E2D2_ERR_UNSUPPORTED;
}

e2d2_status e2d2_attn_count_tiles(int kind, int B, int Hq, int L, int S, long long cache_len,
                                  int bm, int bn, unsigned long long* visited,
                                  unsigned long long* full) {
  if (!visited || !full) return E2D2_ERR_NULL;
  if (kind != E2D2_KIND_ENC && kind != E2D2_KIND_DEC && kind != E2D2_KIND_DENOISE)
    return E2D2_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || S <= 0 || bm <= 0 || bn <= 0 || S > kMaxLen) return E2D2_ERR_SHAPE;
  if (kind != E2D2_KIND_DENOISE && (L <= 0 || L > kMaxLen)) return E2D2_ERR_SHAPE;
  if (kind == E2D2_KIND_DENOISE && (cache_len < 0 || cache_len > kMaxLen)) return E2D2_ERR_SHAPE;
  const int C = kind == E2D2_KIND_DENOISE ? (int)cache_len : 0;
  const int Lm = kind == E2D2_KIND_DENOISE ? 0 : L;
  const int Lq = e2d2::query_len(kind, Lm, S);
  unsigned long long v = 0, f = 0;
  for (int q0 = 0; q0 < Lq; q0 += bm) {
    const int r1 = (q0 + bm < Lq ? q0 + bm : Lq) - 1;
    for (int src = 0; src < e2d2::num_sources(kind); ++src) {
      const e2d2::TileRange tr = e2d2::visited_tiles(kind, src, q0, r1, S, Lm, C, bn);
      v += (unsigned long long)(tr.last - tr.first);
      for (int t = tr.first; t < tr.last; ++t)
        f += e2d2::tile_full(kind, src, q0, r1, S, Lm, C, bn, t) ? 1ull : 0ull;
    }
  }
  *visited = v * (unsigned long long)B * Hq;
  *full = f * (unsigned long long)B * Hq;
  return E2D2_OK;
}

}  // extern "C"

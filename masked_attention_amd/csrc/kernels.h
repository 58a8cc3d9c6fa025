// Launch parameters and launchers of the HIP kernels behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace e2d2 {

// Training forward, bf16.  Grid item = (query tile, batch, query head, kind slot).
// Slot s computes kind kinds[s] with queries q[s] into o[s], lse[s].  Key source 0 is
// (k[0], v[0]) (clean keys), source 1 is (k[1], v[1]) (noised keys, decoder only).
struct TrainParams {
  const __bf16* q[2];
  __bf16* o[2];
  float* lse[2];
  const __bf16* k[2];
  const __bf16* v[2];
  int kinds[2];
  int n_kinds;
  int B, Hq, Hkv, L, S;
  int kv_rows;      // rows per (batch, kv head) of the K/V buffers (L, or a cache capacity)
  const int* lens;  // per-sequence lengths [B] on the device (clamped to [0, L]), or NULL: all L
  int n_qtiles;
  int xcd_groups;  // 1: (B*Hq*n_kinds) % 8 == 0, heads grouped per XCD
  float scale;     // softmax scale
  float c;         // scale * log2(e)
  unsigned long long* visits;
};

// fp32 path for every kind.  Source `src` of slot `s` is kf[s][src], vf[s][src] with
// src_rows[s][src] rows allocated per (batch, kv head).
struct F32Params {
  const float* q[2];
  float* o[2];
  float* lse[2];
  const float* kf[2][2];
  const float* vf[2][2];
  int src_rows[2][2];
  int kinds[2];
  int n_kinds;
  int B, Hq, Hkv, L, S, C;
  int n_qtiles;
  float scale, c;
  unsigned long long* visits;
};

// Denoising step, bf16.  Grid item = (batch, kv head, query group, split).
struct DenoiseParams {
  const __bf16* q;
  const __bf16* k_cache;
  const __bf16* v_cache;
  const __bf16* k_blk;
  const __bf16* v_blk;
  __bf16* o;
  float* lse;
  float* ws_o;   // [units][n_split][64][d] unnormalised partial O (n_split > 1)
  float* ws_ml;  // [units][n_split][64][2] partial (max, sum) in base-2 units
  const int* lens;  // per-sequence cache lengths [B] on the device (clamped to [0, C]), or NULL: all C
  long long cap;
  int C, S, B, Hq, Hkv;  // C: the cache length, or with lens the largest one allowed
  int g;          // query heads per kv head
  int nrc;        // 32-row chunks per head: ceil(S / 32)
  int ncb;        // column blocks per kv head: g * nrc
  int n_qgroups;  // ceil(ncb / 2)
  int n_split;
  int n_tiles;    // key tiles of 32: ceil(C/32) + ceil(S/32)
  int n_tiles_cache;
  float c;        // scale * log2(e)
  unsigned long long* visits;
};

// Training backward, bf16.  Slot s (0: decoder, 1: encoder when n_kinds == 2) has
// queries q[s], forward output o[s], its LSE lse[s], upstream gradient dO[s] and
// query gradient dq[s]; key source 0 is (k[0], v[0]) (clean context, read by both
// kinds), source 1 is (k[1], v[1]) (noised block, decoder only), with gradients
// dk[src], dv[src].  delta[s], lse2[s]: fp32 [B][Hq][L] workspace rows.
struct BwdParams {
  const __bf16* q[2];
  const __bf16* o[2];
  const __bf16* dO[2];
  const float* lse[2];
  __bf16* dq[2];
  const __bf16* k[2];
  const __bf16* v[2];
  __bf16* dk[2];
  __bf16* dv[2];
  float* delta[2];
  float* lse2[2];
  int kinds[2];
  int n_kinds;
  int B, Hq, Hkv, L, S;
  int n_qtiles;  // query tiles of bwd_tile_rows() rows (dQ)
  int n_ktiles;  // key tiles of bwd_tile_rows() keys per source (dK/dV)
  float scale;
  float c;       // scale * log2(e)
};

// C = A W^T for the projections of a decoder layer, bf16 in and out, fp32 accumulate.
// Row m < M = B*S is (b, s) = (m / S, m % S).  A(m, k) is element
//   (b a_sb + s a_ss) + (a_heads ? (k >> a_log2w) a_sh + (k & (2^a_log2w - 1)) : k)
// of a; W is [N][K].  Column n belongs to segment seg (c_n0[seg] <= n < c_n0[seg+1],
// c_n0[0] = 0, unused boundaries = N); with nn = n - c_n0[seg], h = nn / c_w and
// c = nn % c_w, C(m, n) goes to c[seg][((b c_h[seg] + h) S + s) c_w + c].
// a_bytes, w_bytes: sizes of the A and W buffers (reads past them return zero).
struct LinearParams {
  const __bf16* a;
  const __bf16* w;
  __bf16* c[3];
  int c_n0[3];
  int c_h[3];
  int c_w;
  int a_sb, a_ss, a_sh;
  int a_heads, a_log2w;
  int M, N, K, S;
  unsigned a_bytes, w_bytes;
};
hipError_t launch_linear_bf16(const LinearParams& p, hipStream_t stream);

int train_tile_bm(int d);
int bwd_tile_rows();
hipError_t launch_train_bwd_bf16(const BwdParams& p, int d, hipStream_t stream);
int train_tile_bn();
constexpr int kF32TileBM = 64;
constexpr int kF32TileBN = 64;
constexpr int kDenoiseTileBM = 32;
constexpr int kDenoiseTileBN = 32;

hipError_t launch_train_bf16(const TrainParams& p, int d, hipStream_t stream);
hipError_t launch_attn_f32(const F32Params& p, int d, hipStream_t stream);
hipError_t launch_denoise_bf16(const DenoiseParams& p, int d, hipStream_t stream);
// Denoise split sizing shared by the workspace query and the launch.
int denoise_splits(int B, int Hkv, int n_qgroups, int n_tiles);
// Device address (on the current device) and size of the library's own denoise scratch
// buffer, looked up once per device.
hipError_t denoise_scratch(void** ptr, size_t* bytes);
hipError_t launch_kv_append(int elem_bytes, int B, int Hkv, int S, int d, void* k_cache,
                            void* v_cache, long long cache_len, long long cap,
                            const void* k_new, const void* v_new, hipStream_t stream);
// Per-sequence variant: sequence b appends at row lens[b] (device array); a sequence
// whose lens[b] is outside [0, max_len] is left untouched.
hipError_t launch_kv_append_varlen(int elem_bytes, int B, int Hkv, int S, int d, void* k_cache,
                                   void* v_cache, const int* lens, long long max_len, long long cap,
                                   const void* k_new, const void* v_new, hipStream_t stream);

}  // namespace e2d2

// Block-sparse tile schedule of the E2D2 attention masks: closed-form allowed-key
// intervals per query row and per query tile, and the key tiles a query tile visits.
// Used by the host entry points (tile counts, launch sizing) and by the kernels.
//
// Pages cited, by title and section:
//   [Notes] "Encoder-Decoder Diffusion Language Models for Efficient Training and
//           Inference", Paper-Notes page, 方法详解 §3 采样算法 and §4 训练算法.
//   [BD3]   "Block Diffusion: Interpolating Between Autoregressive and Diffusion
//           Language Models", xllm-io review, 三 技术架构 (块级分解).
//
// Every mask row allows one contiguous interval of keys per key source:
//   ENC      (one source, clean keys [0, L)):   [0, end(i))        blk(j) <= blk(i)
//   DEC src0 (clean context keys [0, L)):       [0, start(i))      blk(j) <  blk(i)
//   DEC src1 (noised keys [0, L)):              [start(i), end(i)) blk(j) == blk(i)
//   DENOISE src0 (cache keys [0, C)):           [0, C)
//   DENOISE src1 (own-block keys [0, S)):       [0, S)
// with start(i) = blk(i) * S and end(i) = min(start(i) + S, L).  Both bounds are
// non-decreasing in i, so over query rows r0..r1 the union of the row intervals is
// [lo(r0), hi(r1)) and the keys every row allows are [lo(r1), hi(r0)).  Every key in
// the union is allowed by some row of r0..r1 (the rows cover every block between
// blk(r0) and blk(r1)), so a key tile is visited exactly when it overlaps the union,
// and it is full exactly when it lies inside the common interval.  Tiles that hold no
// allowed pair are never visited: this is where the halved attention FLOPs of the
// FLOPs table ([Notes] §4) turn into halved work.
#pragma once

#if defined(__HIPCC__)
#define E2D2_HD __host__ __device__ __forceinline__
#else
#define E2D2_HD inline
#endif

namespace e2d2 {

enum Kind : int { kEnc = 0, kDec = 1, kDenoise = 2 };

struct Interval {
  int lo, hi;  // keys [lo, hi); empty when hi <= lo
};

E2D2_HD int block_start(int i, int S) { return (i / S) * S; }
E2D2_HD int block_end(int i, int S, int L) {
  const int e = (i / S) * S + S;
  return e < L ? e : L;
}

// Number of key sources of a kind.
E2D2_HD int num_sources(int kind) { return kind == kEnc ? 1 : 2; }

// Length of key source `src` (L for ENC/DEC; C or S for DENOISE).
E2D2_HD int source_len(int kind, int src, int L, int S, int C) {
  if (kind == kDenoise) return src == 0 ? C : S;
  return L;
}

// Number of query rows of one head (L for ENC/DEC, S for DENOISE).
E2D2_HD int query_len(int kind, int L, int S) { return kind == kDenoise ? S : L; }

// Allowed keys of query row i in source src.
E2D2_HD Interval row_interval(int kind, int src, int i, int S, int L, int C) {
  if (kind == kEnc) return {0, block_end(i, S, L)};
  if (kind == kDec) {
    if (src == 0) return {0, block_start(i, S)};
    return {block_start(i, S), block_end(i, S, L)};
  }
  return {0, src == 0 ? C : S};
}

// Keys allowed by at least one of the rows r0..r1 (inclusive, r0 <= r1).
E2D2_HD Interval union_interval(int kind, int src, int r0, int r1, int S, int L, int C) {
  const Interval a = row_interval(kind, src, r0, S, L, C);
  const Interval b = row_interval(kind, src, r1, S, L, C);
  return {a.lo, b.hi};
}

// Keys allowed by every one of the rows r0..r1 (inclusive, r0 <= r1).
E2D2_HD Interval common_interval(int kind, int src, int r0, int r1, int S, int L, int C) {
  const Interval a = row_interval(kind, src, r0, S, L, C);
  const Interval b = row_interval(kind, src, r1, S, L, C);
  return {b.lo, a.hi};
}

// Key tiles [first, last) of size bn, inside source src, that query rows r0..r1 visit.
struct TileRange {
  int first, last;
};
E2D2_HD TileRange visited_tiles(int kind, int src, int r0, int r1, int S, int L, int C, int bn) {
  const Interval u = union_interval(kind, src, r0, r1, S, L, C);
  if (u.hi <= u.lo) return {0, 0};
  return {u.lo / bn, (u.hi + bn - 1) / bn};
}

// Whether key tile t (keys [t*bn, min((t+1)*bn, source length))) is full for r0..r1.
E2D2_HD bool tile_full(int kind, int src, int r0, int r1, int S, int L, int C, int bn, int t) {
  const Interval c = common_interval(kind, src, r0, r1, S, L, C);
  const int n = source_len(kind, src, L, S, C);
  const int k0 = t * bn;
  const int k1 = (t + 1) * bn < n ? (t + 1) * bn : n;
  return c.lo <= k0 && k1 <= c.hi;
}

// Classification of a block of keys [k0, k1) against query rows r0..r1:
// 0 = no allowed pair, 1 = some pairs allowed, 2 = every pair allowed.
E2D2_HD int classify(int kind, int src, int r0, int r1, int S, int L, int C, int k0, int k1) {
  const Interval u = union_interval(kind, src, r0, r1, S, L, C);
  if (k1 <= u.lo || k0 >= u.hi || k1 <= k0) return 0;
  const Interval c = common_interval(kind, src, r0, r1, S, L, C);
  return (c.lo <= k0 && k1 <= c.hi) ? 2 : 1;
}

// ---- The transposed view, for the backward pass: which query rows allow key j.
// By the same masks, every key allows one contiguous interval of query rows:
//   ENC      (key j of the clean keys):    [start(j), L)        blk(i) >= blk(j)
//   DEC src0 (clean context key j):        [start(j) + S, L)    blk(i) >  blk(j)
//   DEC src1 (noised key j):               [start(j), end(j))   blk(i) == blk(j)
// (clamped to [0, L]); both bounds are non-decreasing in j, so over keys k0..k1 the
// union is [lo(k0), hi(k1)) and the rows every key allows are [lo(k1), hi(k0)).
E2D2_HD Interval col_interval(int kind, int src, int j, int S, int L) {
  const int st = block_start(j, S);
  if (kind == kEnc) return {st, L};
  if (src == 0) return {st + S < L ? st + S : L, L};
  return {st, block_end(j, S, L)};
}
E2D2_HD Interval col_union(int kind, int src, int k0, int k1, int S, int L) {
  return {col_interval(kind, src, k0, S, L).lo, col_interval(kind, src, k1, S, L).hi};
}
E2D2_HD Interval col_common(int kind, int src, int k0, int k1, int S, int L) {
  return {col_interval(kind, src, k1, S, L).lo, col_interval(kind, src, k0, S, L).hi};
}

}  // namespace e2d2

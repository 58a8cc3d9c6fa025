/* e2d2_attn.h -- C ABI of the MI355X (gfx950) attention hot path of E2D2, the
 * encoder-decoder block diffusion language model.
 *
 * Pages cited, by title and section:
 *   [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
 *             Inference", Paper-Notes page (zhaoyang97.github.io).
 *   [Summary] ai.info "AI summary" page on the same paper.
 *   [BD3]     "Block Diffusion: Interpolating Between Autoregressive and Diffusion
 *             Language Models", xllm-io review.
 *
 * Conventions shared by every call
 *   - Tensors are dense, row-major [B][H][N][d] with d contiguous and no padding;
 *     query tensors have Hq heads, key/value tensors Hkv heads, Hq % Hkv == 0, and
 *     query head hq reads key/value head hq / (Hq / Hkv).
 *   - dtype E2D2_BF16: q, k, v and o are bfloat16; E2D2_F32: all float32.  LSE
 *     outputs are always float32 [B][Hq][N_q], natural log of the sum of
 *     exp(scale * q.k) over the allowed keys of the row.  Any LSE pointer may be NULL
 *     (not written).
 *   - Blocks hold S consecutive positions from position 0; the last block may be
 *     shorter ([BD3] 三 技术架构, 块级分解).  blk(i) = floor(i / S).
 *   - Every data pointer is a DEVICE pointer, except where noted.  `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream).
 *   - Every call validates its arguments on the host first and, on error, returns
 *     the status WITHOUT launching anything or touching device memory.  On success
 *     the work is enqueued on `stream` and the call returns at once; faults during
 *     execution surface at the caller's next synchronisation.
 *   - The library allocates, frees and synchronises no device memory, keeps no
 *     pointer after a call returns and holds no mutable global state; calls are
 *     thread-safe.  The caller owns every buffer, including the KV cache and its
 *     length.  Outputs must not alias inputs.
 *   - Results are deterministic: identical inputs and arguments give bitwise
 *     identical outputs (no floating-point atomics).
 *   - dbg_tile_visits: optional device counter (unsigned long long).  When non-NULL
 *     the kernels ADD the number of (batch, query head, query tile, key tile) tiles
 *     they visited, a tile being visited when it holds at least one allowed
 *     (query, key) pair; key tiles are laid out separately inside each key source.
 *     Pass NULL when timing.
 */
#ifndef E2D2_ATTN_H
#define E2D2_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define E2D2_ABI_VERSION 1

typedef enum {
  E2D2_OK = 0,
  E2D2_ERR_NULL = 1,        /* a required pointer is NULL */
  E2D2_ERR_SHAPE = 2,       /* a size is <= 0 (or < 0 where 0 is allowed), Hq % Hkv != 0,
                               or a size exceeds the supported range */
  E2D2_ERR_UNSUPPORTED = 3, /* the (dtype, d) pair or the kind is not built */
  E2D2_ERR_CAPACITY = 4,    /* cache_len + S exceeds cache_cap */
  E2D2_ERR_WORKSPACE = 5,   /* workspace smaller than e2d2_attn_denoise_workspace_bytes */
  E2D2_ERR_HIP = 6          /* a HIP launch failed; see e2d2_last_hip_error */
} e2d2_status;

typedef enum { E2D2_F32 = 0, E2D2_BF16 = 1 } e2d2_dtype;

typedef enum {
  E2D2_KIND_ENC = 0,     /* encoder block-causal mask */
  E2D2_KIND_DEC = 1,     /* decoder mask over [clean | noised] keys */
  E2D2_KIND_DENOISE = 2  /* denoising step over [cache | own block] keys */
} e2d2_kind;

/* Version of this header's ABI (E2D2_ABI_VERSION). */
int e2d2_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* e2d2_status_string(int status);

/* hipError_t of the last call on this thread that returned E2D2_ERR_HIP (0 if none). */
int e2d2_last_hip_error(void);

/* Supported head dimensions: d in {32, 64, 128} for both dtypes. */

/* Encoder block-causal attention over L clean tokens ([Notes] 方法详解 §4 训练算法:
 * a clean token attends the tokens of its own block and of every earlier block).
 * Row i attends keys j with blk(j) <= blk(i).
 *   q [B][Hq][L][d]; k, v [B][Hkv][L][d]; o [B][Hq][L][d]; lse [B][Hq][L] or NULL.
 *   scale multiplies q.k before the softmax (1/sqrt(d) usually). */
e2d2_status e2d2_attn_encoder_blockcausal(int dtype, int B, int Hq, int Hkv, int L, int d,
                                          int S, float scale, const void* q, const void* k,
                                          const void* v, void* o, float* lse,
                                          unsigned long long* dbg_tile_visits, void* stream);

/* Prompt encoding for a batch of prompts of different lengths ([Notes] 方法详解 §3
 * 采样算法: sampling starts by running the encoder over the prompt to build its KV
 * cache).  Sequence b's prompt holds lens[b] tokens and is blocked like the training
 * encoder (blocks of S from position 0, the last one possibly shorter): its row i
 * attends its keys j < lens[b] with blk(j) <= blk(i).
 *   q, o [B][Hq][L][d]: rows [0, lens[b]) of sequence b are read / written, the rest of
 *   o and lse is left untouched; lse [B][Hq][L] or NULL.
 *   k, v [B][Hkv][kv_rows][d], kv_rows >= L: rows [0, lens[b]) hold the prompt's keys
 *   and values.  With kv_rows = the cache capacity these are the KV-cache buffers of
 *   e2d2_attn_denoise_step: a projection writes the prompt's K/V straight into the
 *   cache, this call reads them there, and no append follows.
 *   lens: device array of B int32 (4-byte aligned), read when the kernel runs (a
 *   captured HIP graph stays valid while the caller updates it on the device); each
 *   length is clamped to [0, L].  L is the host bound that sizes the launch.
 * bf16 only (fp32: E2D2_ERR_UNSUPPORTED).  Errors as e2d2_attn_encoder_blockcausal,
 * plus E2D2_ERR_NULL for a NULL lens and E2D2_ERR_SHAPE for kv_rows < L. */
e2d2_status e2d2_attn_encoder_blockcausal_varlen(int dtype, int B, int Hq, int Hkv, int L, int d,
                                                 int S, float scale, const void* q, const void* k,
                                                 const void* v, long long kv_rows,
                                                 const int* lens, void* o, float* lse,
                                                 unsigned long long* dbg_tile_visits,
                                                 void* stream);

/* Training forward of the fused decoder self+cross attention ([Notes] §4 训练算法 and
 * §2 两种连接方式): noised query i attends, under ONE softmax, the clean context keys
 * j of strictly earlier blocks (blk(j) < blk(i)) and the noised keys j of its own
 * block (blk(j) == blk(i)) -- 2L keys in all, ordered [clean | noised].
 *   q_dec [B][Hq][L][d]; k_ctx, v_ctx, k_dec, v_dec [B][Hkv][L][d];
 *   o_dec [B][Hq][L][d]; lse_dec [B][Hq][L] or NULL.
 * k_ctx/v_ctx are the clean-context keys/values the decoder conditions on: the
 * encoder's own K/V in the shared-KV-cache wiring, or the decoder's projection of
 * the encoder output in the last-hidden-state wiring.
 * Optional, same launch: when q_enc is non-NULL the encoder block-causal attention
 * of (q_enc, k_ctx, v_ctx) is computed too, into o_enc [B][Hq][L][d] (required then)
 * and lse_enc (may be NULL); pass q_enc = o_enc = lse_enc = NULL for the decoder only. */
e2d2_status e2d2_attn_train_fwd(int dtype, int B, int Hq, int Hkv, int L, int d, int S,
                                float scale, const void* q_dec, const void* k_ctx,
                                const void* v_ctx, const void* k_dec, const void* v_dec,
                                void* o_dec, float* lse_dec, const void* q_enc, void* o_enc,
                                float* lse_enc, unsigned long long* dbg_tile_visits,
                                void* stream);

/* Bytes of device workspace e2d2_attn_train_bwd needs (with_enc: 1 when the encoder's
 * gradients are computed too).  0 for unsupported arguments.  Host-only. */
size_t e2d2_attn_train_bwd_workspace_bytes(int dtype, int B, int Hq, int L, int with_enc);

/* Backward of e2d2_attn_train_fwd ([Notes] §4 训练算法: a training step backpropagates
 * the decoder's loss through the decoder attention and, through the clean context
 * keys/values both attentions read, into the encoder).  Gradients of the same fused
 * attention, from the forward's outputs:
 *   inputs: q_dec, k_ctx, v_ctx, k_dec, v_dec as in the forward; o_dec and lse_dec
 *   (required) from the forward; do_dec [B][Hq][L][d] the gradient of o_dec.  With
 *   q_enc (then o_enc, lse_enc, do_enc and dq_enc are all required; else all NULL)
 *   the encoder's block-causal attention over (q_enc, k_ctx, v_ctx) is included.
 *   outputs (overwritten, not accumulated): dq_dec [B][Hq][L][d]; dk_ctx, dv_ctx
 *   [B][Hkv][L][d] summing the encoder's and the decoder's gradients and every query
 *   head of a grouped kv head; dk_dec, dv_dec [B][Hkv][L][d]; dq_enc.
 *   workspace: device scratch of e2d2_attn_train_bwd_workspace_bytes(...) bytes,
 *   contents ignored on entry; calls sharing it must be ordered on one stream.
 * bf16 only (fp32: E2D2_ERR_UNSUPPORTED).  Deterministic (no atomics).  Errors as the
 * forward, plus E2D2_ERR_WORKSPACE. */
e2d2_status e2d2_attn_train_bwd(int dtype, int B, int Hq, int Hkv, int L, int d, int S,
                                float scale, const void* q_dec, const void* k_ctx,
                                const void* v_ctx, const void* k_dec, const void* v_dec,
                                const void* o_dec, const float* lse_dec, const void* do_dec,
                                const void* q_enc, const void* o_enc, const float* lse_enc,
                                const void* do_enc, void* dq_dec, void* dk_ctx, void* dv_ctx,
                                void* dk_dec, void* dv_dec, void* dq_enc, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Bytes of device workspace e2d2_attn_denoise_step needs for these sizes (0 when the
 * call needs none; a NULL workspace is then accepted).  Host-only, no GPU needed. */
size_t e2d2_attn_denoise_workspace_bytes(int dtype, int B, int Hq, int Hkv, int S, int d,
                                         long long cache_len);

/* One denoising step ([Notes] §3 采样算法; [Summary] "Methodology in Plain English"):
 * the S queries of the current [MASK] block attend every cached clean key
 * (rows [0, cache_len) of the cache) and every key of their own block, with no mask.
 * The same call is the encoder's update of a finished block ([Notes] §3: the finished
 * block goes through the encoder, which extends the KV cache): with q_blk the encoder
 * queries of the block's S clean tokens and k_blk, v_blk the encoder's keys/values of
 * the block, its rows equal the training encoder's rows of that block (a clean token
 * sees its own block and every earlier one); k_blk, v_blk are then what
 * e2d2_kv_cache_append adds to the cache.
 *   q_blk [B][Hq][S][d]; k_cache, v_cache [B][Hkv][cache_cap][d] (rows beyond
 *   cache_len are not read); k_blk, v_blk [B][Hkv][S][d] this step's own-block K/V;
 *   o_blk [B][Hq][S][d]; lse_blk [B][Hq][S] or NULL.
 *   cache_len >= 0 (0 = empty cache) and cache_len <= cache_cap.
 *   workspace: device scratch of at least e2d2_attn_denoise_workspace_bytes(...)
 *   bytes, owned by the caller, contents ignored on entry; calls that share one
 *   workspace must be ordered on one stream. */
e2d2_status e2d2_attn_denoise_step(int dtype, int B, int Hq, int Hkv, int S, int d, float scale,
                                   const void* q_blk, const void* k_cache, const void* v_cache,
                                   long long cache_len, long long cache_cap, const void* k_blk,
                                   const void* v_blk, void* o_blk, float* lse_blk,
                                   void* workspace, size_t workspace_bytes,
                                   unsigned long long* dbg_tile_visits, void* stream);

/* e2d2_attn_denoise_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step and arguments without the workspace.  When the step splits its key axis, the
 * partial results go to a scratch buffer the library owns, a fixed 17 MiB array in
 * device memory that every GPU the library runs on holds until the process ends (it
 * covers the largest workspace e2d2_attn_denoise_workspace_bytes returns for any
 * shape; a larger need would return E2D2_ERR_WORKSPACE).  Its address on the current
 * device is looked up on the first call there, so that call must not itself be under
 * stream capture.  Nothing is allocated or freed.  Every call on one GPU shares that
 * GPU's scratch, so calls that may overlap on one GPU (different streams, no ordering
 * between them) race and corrupt each other's results; calls ordered on one stream do
 * not.  The scratch's contents are ignored on entry.  Errors as e2d2_attn_denoise_step,
 * plus E2D2_ERR_HIP when the scratch cannot be located. */
e2d2_status e2d2_attn_denoise_step_noalloc(int dtype, int B, int Hq, int Hkv, int S, int d,
                                           float scale, const void* q_blk, const void* k_cache,
                                           const void* v_cache, long long cache_len,
                                           long long cache_cap, const void* k_blk,
                                           const void* v_blk, void* o_blk, float* lse_blk,
                                           unsigned long long* dbg_tile_visits, void* stream);

/* KV-cache append after a block is finished ([Notes] §3 采样算法: the finished block
 * goes through the encoder, which updates the KV cache): copies k_new, v_new
 * [B][Hkv][S][d] into rows [cache_len, cache_len + S) of k_cache, v_cache
 * [B][Hkv][cache_cap][d].  Needs cache_len + S <= cache_cap (else
 * E2D2_ERR_CAPACITY).  The caller then advances its cache length by S.  Bitwise copy. */
e2d2_status e2d2_kv_cache_append(int dtype, int B, int Hkv, int S, int d, void* k_cache,
                                 void* v_cache, long long cache_len, long long cache_cap,
                                 const void* k_new, const void* v_new, void* stream);

/* One denoising step for a batch whose sequences sit at different points of the
 * sampling loop ([Notes] §3 采样算法: each sequence's cache grows by one block per
 * finished block, so in a batch decoded together the cached lengths differ).  Same as
 * e2d2_attn_denoise_step, except that sequence b attends rows [0, cache_lens[b]) of
 * its cache:
 *   cache_lens: device array of B int32 (4-byte aligned), read by the kernel when it
 *   runs, so a captured HIP graph of this call stays valid while the caller updates
 *   the lengths on the device; each length is clamped to [0, max_cache_len].
 *   max_cache_len: host bound on every length (0 <= max_cache_len <= cache_cap); it
 *   sizes the launch and the workspace (e2d2_attn_denoise_workspace_bytes with
 *   cache_len = max_cache_len).
 *   bf16 only (fp32: E2D2_ERR_UNSUPPORTED).  Errors as e2d2_attn_denoise_step, plus
 *   E2D2_ERR_NULL for a NULL cache_lens. */
e2d2_status e2d2_attn_denoise_step_varlen(int dtype, int B, int Hq, int Hkv, int S, int d,
                                          float scale, const void* q_blk, const void* k_cache,
                                          const void* v_cache, const int* cache_lens,
                                          long long max_cache_len, long long cache_cap,
                                          const void* k_blk, const void* v_blk, void* o_blk,
                                          float* lse_blk, void* workspace, size_t workspace_bytes,
                                          unsigned long long* dbg_tile_visits, void* stream);

/* KV-cache append for sequences of different lengths ([Notes] §3 采样算法): sequence b's
 * k_new, v_new rows go to rows [cache_lens[b], cache_lens[b] + S) of its cache.
 *   cache_lens: device array of B int32 read when the kernel runs; a sequence whose
 *   length is outside [0, max_cache_len] is left untouched (the call cannot report
 *   it).  Needs max_cache_len + S <= cache_cap (else E2D2_ERR_CAPACITY).  The caller
 *   then advances the lengths it appended to by S.  Bitwise copy. */
e2d2_status e2d2_kv_cache_append_varlen(int dtype, int B, int Hkv, int S, int d, void* k_cache,
                                        void* v_cache, const int* cache_lens,
                                        long long max_cache_len, long long cache_cap,
                                        const void* k_new, const void* v_new, void* stream);

/* Attention sublayer of one decoder layer in a denoising step ([Notes] §3 采样算法:
 * every step of a block calls only the small decoder on the block's S noised tokens;
 * 方法详解 §2 两种连接方式: with the shared KV cache the decoder layer attends over an
 * encoder layer's cached clean keys/values plus its own block).  Three launches on
 * `stream`, in order:
 *   1. q_blk, k_blk, v_blk = per-head slices of x W_qkv^T;
 *   2. o_blk, lse_blk = e2d2_attn_denoise_step of q_blk over the cache rows
 *      [0, cache_len) and the block's own k_blk, v_blk;
 *   3. y = concat_h(o_blk) W_o^T.
 * bf16 only (fp32: E2D2_ERR_UNSUPPORTED); d in {32, 64, 128}; fp32 accumulation, every
 * stored tensor rounded to bf16 (nearest even).  Layouts (all row-major, contiguous):
 *   x      [B][S][Dm]                hidden states of the block's tokens; Dm % 8 == 0
 *   w_qkv  [(Hq + 2 Hkv) d][Dm]      rows: query heads 0.., then key heads, then value
 *                                     heads, d consecutive rows per head (nn.Linear
 *                                     [out][in] layout)
 *   w_o    [Dm][Hq d]                column h d + c multiplies o_blk[b][h][s][c]
 *   k_cache, v_cache, cache_len, cache_cap, lse_blk, workspace: as
 *                                     e2d2_attn_denoise_step (workspace sized by
 *                                     e2d2_attn_denoise_workspace_bytes)
 *   q_blk, o_blk [B][Hq][S][d]; k_blk, v_blk [B][Hkv][S][d]; y [B][S][Dm]: written
 *                                     (the caller owns them; they must not overlap
 *                                     each other or the inputs).
 * Errors: E2D2_ERR_SHAPE also when an operand of the projections reaches 2 GiB;
 * otherwise as e2d2_attn_denoise_step.  All checks precede the first launch. */
e2d2_status e2d2_decoder_layer_denoise_step(int dtype, int B, int Hq, int Hkv, int S, int d,
                                            int Dm, float scale, const void* x,
                                            const void* w_qkv, const void* w_o,
                                            const void* k_cache, const void* v_cache,
                                            long long cache_len, long long cache_cap,
                                            void* q_blk, void* k_blk, void* v_blk, void* o_blk,
                                            float* lse_blk, void* y, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* Query/key tile shape (bm query rows of one head, bn keys) the kernels use for a
 * kind, dtype and head dimension.  Host-only; bm and bn are host pointers. */
e2d2_status e2d2_attn_tile_shape(int kind, int dtype, int d, int* bm, int* bn);

/* Tiles the block-sparse schedule visits (holding >= 1 allowed pair) and, of those,
 * the full ones (every pair allowed), summed over B * Hq heads, for query tiles of
 * bm rows and key tiles of bn keys laid out per key source.  ENC and DEC use L; DEC
 * counts both of its sources; DENOISE uses S query rows and cache_len + S keys (L
 * ignored).  Host-only; visited and full are host pointers. */
e2d2_status e2d2_attn_count_tiles(int kind, int B, int Hq, int L, int S, long long cache_len,
                                  int bm, int bn, unsigned long long* visited,
                                  unsigned long long* full);

#ifdef __cplusplus
}
#endif

#endif /* E2D2_ATTN_H */

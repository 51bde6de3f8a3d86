/*
 * attn.h -- C ABI of libattn.so: exact grouped-query scaled-dot-product
 * attention on AMD Instinct MI355X (gfx950), prefill and single-token decode.
 *
 * What is computed (all entry points):
 *   for batch b, query head h (KV head h / G with G = Hq / Hkv, consecutive
 *   query heads sharing one KV head), query row i:
 *     s_ij  = scale * <q_i, k_j>                 over the visible keys j
 *     lse_i = ln sum_j exp(s_ij)                 (natural log)
 *     out_i = sum_j exp(s_ij - lse_i) * v_j
 *   The Lq x Lk score table is never written to memory: keys are consumed in
 *   tiles with a running row maximum and row sum (an online softmax), which
 *   gives the same result up to rounding order.
 *
 * Sources (pages, by title):
 *   "어텐션 구현 고르기, SDPA·FlashAttention 메모리와 GPU 비용"
 *     (tool.smithlab.co.kr) -- section "어텐션 구현 종류와 차이 한눈에 보기"
 *     (all implementations compute the same values; flash kernels take
 *     fp16/bf16 and head dim up to 256), section "eager 어텐션 메모리, 길이에
 *     따라 얼마나 커지나" (the tiled method keeps only per-row max and sum
 *     statistics, memory linear in length, no approximation), section
 *     "is_causal 마스크 정렬, KV 캐시와 쓸 때의 함정" (causal mask anchored at
 *     the bottom-right corner when there are fewer queries than keys; a
 *     single decode query attends to the whole cache with no mask);
 *   "Как NVIDIA учит нейросети думать быстрее: оптимизация внимания для
 *     длинных контекстов" (iphoneandroid24.ru) -- section "Параметр первый:
 *     размер группы (group size)" (G query heads share one KV head), section
 *     "Параметр второй: размерность головы" (head dims 64/128/256), section
 *     "Параметр четвёртый: параллелизм…" (a long KV cache split into parts
 *     whose partial results are merged).
 *
 * Conventions shared by every entry point:
 *   - Element types: q, k, v, kcache, vcache and out are bfloat16 (passed as
 *     void*); lse is float32; kv_lens is int32.  Arithmetic: fp32
 *     accumulation and fp32 softmax statistics.
 *   - Layouts are dense and row-major (last index fastest):
 *       prefill q/out [B][Hq][Lq][D], k/v [B][Hkv][Lk][D], lse [B][Hq][Lq];
 *       decode q/out [B][Hq][D], kcache/vcache [B][Hkv][Lmax][D],
 *       kv_lens [B], lse [B][Hq].
 *   - Every pointer is device memory owned by the caller, 16-byte aligned.
 *     Inputs are read only; outputs are written only.  Inputs and outputs
 *     must not overlap.
 *   - D must be 64, 128 or 256; Hq must be a multiple of Hkv.
 *   - scale multiplies q.k in fp32 (pass 1/sqrt(D) for the usual scaling);
 *     it must be finite; 0 gives uniform weights.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: they enqueue work and return.  Argument errors are
 *     reported before anything is enqueued; device faults show up at the
 *     caller's next synchronisation.
 *   - Errors are returned as negative attn_status codes; nothing is thrown
 *     across the ABI; the library keeps no state between calls apart from
 *     HIP's stream-ordered memory pool (partials of attn_decode and of a
 *     key-split attn_prefill) and cached device properties.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,     /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,    /* a negative size, Lk = 0 with Lq > 0, causal with Lq > Lk,
                             Lmax < 1, T outside 1..Lmax, Lmax * D >= 2^30 (decode: one
                             sequence's rows of one KV head must stay below 2 GiB), or a
                             size whose element count overflows */
  ATTN_ERR_HEADDIM = -3,  /* D not in {64, 128, 256} */
  ATTN_ERR_GQA = -4,      /* Hq < 1, Hkv < 1 or Hq % Hkv != 0 */
  ATTN_ERR_SCALE = -5,    /* scale is NaN or infinite */
  ATTN_ERR_HIP = -6,      /* a HIP call or kernel launch failed */
  ATTN_ERR_SPLIT = -7,    /* decode split_keys not 0 and not a positive multiple of 128, or
                             prefill splits outside 0..64 */
  ATTN_ERR_WORKSPACE = -8, /* workspace given but smaller than the matching *_workspace_bytes() */
  ATTN_ERR_KERNEL = -9,    /* attn_decode_multi_ex: kernel not 0, 1 or 2, or kernel 2 asked for a
                              shape that kernel does not serve */
  ATTN_ERR_SCRATCH = -10   /* attn_decode_noalloc: the sizes need more partials than its static
                              scratch holds (attn_decode_noalloc_max_bytes()) */
} attn_status;

/*
 * attn_prefill -- causal or full attention of Lq query rows over Lk keys.
 *
 * Pages: the cost guide's sections on the tiled method and on is_causal
 * alignment (above).  causal != 0 applies the bottom-right-aligned mask:
 * query row i sees key j iff j <= i + (Lk - Lq).  That is the only causal
 * alignment offered; with Lq == Lk it is the usual lower triangle, and with
 * Lq < Lk (chunked prefill, several new rows over a cache) each row sees the
 * cache plus the new rows up to itself.  causal with Lq > Lk is rejected
 * (ATTN_ERR_SHAPE): such rows would see no key.
 *
 *   q   [B][Hq][Lq][D] bf16      k, v [B][Hkv][Lk][D] bf16
 *   out [B][Hq][Lq][D] bf16      lse  [B][Hq][Lq] fp32, may be NULL
 *
 * B == 0 or Lq == 0 is an empty call: ATTN_OK, nothing is read, written or
 * enqueued, and the pointers may be NULL (the other arguments are still
 * checked).
 *
 * When the grid of query blocks is small (less than two rounds of the
 * device's resident workgroups, e.g. a chunk of a few hundred rows over a
 * long cache), the keys of each query block are cut into several ranges
 * processed by separate workgroups (as many as make the grid fill whole
 * rounds best, at least 8 key tiles each, at most 32), and a second kernel
 * merges their normalised partial outputs
 * and log-sum-exps (the same merge as the decode's; see attn_prefill_ex).
 * The partials then live in a workspace taken from HIP's stream-ordered
 * allocator on `stream` and released on it.
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_prefill(const void *q, const void *k, const void *v, void *out, float *lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, float scale,
                 void *stream);

/*
 * attn_prefill_ex -- attn_prefill with three extra controls:
 *   window     0: no window.  > 0 (needs causal, else ATTN_ERR_SHAPE): sliding
 *              window, row i sees only its `window` most recent visible keys,
 *              j in [i + (Lk - Lq) - window + 1, i + (Lk - Lq)] (the local
 *              attention the NVIDIA page names for cutting the effective KV
 *              length, section "Параметр третий: длина последовательности").
 *              Tiles outside every row's window are skipped.  window >= Lk is
 *              the plain causal mask.  Negative: ATTN_ERR_SHAPE.
 *   splits     0: choose the number of key ranges per query block as
 *              attn_prefill does; 1..64: use exactly that many (else
 *              ATTN_ERR_SPLIT).  Results agree for every count up to fp32
 *              rounding of the merge.
 *   workspace  caller-owned device buffer of workspace_bytes for the partials
 *              (needed only with more than one range); NULL takes it from the
 *              stream-ordered allocator.  If non-NULL it must hold at least
 *              attn_prefill_workspace_bytes(...) bytes (else
 *              ATTN_ERR_WORKSPACE) and must not be used by other work until
 *              this call's kernels have finished on `stream`.
 * Validation order: as attn_prefill (the window is checked with the sizes),
 * with the splits check after the size checks and before the empty-call
 * return.
 */
int attn_prefill_ex(const void *q, const void *k, const void *v, void *out, float *lse,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, int window, float scale,
                    int splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_prefill_splits -- the number of key ranges attn_prefill_ex uses for
 * these sizes and splits on the current device; 0 for an empty call, invalid
 * arguments, or splits == 0 with no device available.
 */
int attn_prefill_splits(int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, int window, int splits);

/*
 * attn_prefill_workspace_bytes -- bytes of workspace attn_prefill_ex needs
 * for these sizes and splits (0 when a single range is used, for an empty
 * call and for invalid arguments).  Layout: B*Hq*Lq*n fp32 log-sum-exps, then
 * B*Hq*Lq*n*D fp32 outputs (n ranges), each part 256-byte aligned.
 */
size_t attn_prefill_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal,
                                    int window, int splits);

/*
 * attn_decode -- one new query row per sequence over a ragged KV cache.
 *
 * Pages: the cost guide's is_causal section (the new token's K/V are already
 * in the cache and the single query attends to all cached keys with no mask)
 * and the NVIDIA page's parallelism section (KV split into parts, partial
 * results merged).  Sequence b uses keys [0, n_b) of its cache rows, with
 * n_b = min(kv_lens[b], Lmax) (negative lengths count as 0); the rows past
 * n_b are never read.  n_b == 0 gives out = 0.
 *
 *   q       [B][Hq][D] bf16           out [B][Hq][D] bf16
 *   kcache, vcache [B][Hkv][Lmax][D] bf16
 *   kv_lens [B] int32, device memory (read on the device only)
 *
 * The cached keys of all (sequence, KV head) pairs are laid end to end and cut
 * into equal ranges, one per wave of the device (a balanced split that does
 * not depend on the length mix); a pair split between waves gets its partial
 * outputs and log-sum-exps merged by a final kernel.  A small planner kernel
 * turns kv_lens into block counts on the device first.  The partials live in
 * a workspace taken from HIP's stream-ordered allocator on `stream` and
 * released on it.  B == 0 is an empty call (ATTN_OK; pointers may be NULL).
 */
int attn_decode(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens,
                void *out, int B, int Hq, int Hkv, int Lmax, int D, float scale, void *stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, semantics and results (bit for bit) as
 * attn_decode, but the partial outputs and log-sum-exps live in one static
 * device array of the library (attn_decode_noalloc_max_bytes() = 64 MiB),
 * which each GPU the library runs on holds from the library's load until the
 * process ends.  The call allocates nothing and enqueues no memset; on the
 * first call on a device it looks up that device's copy of the array.
 *
 * Limit: the partials of these sizes -- (W + B * Hkv * ceil(G / 64)) slots of
 * min(G, 64) rows of D + 1 fp32 values, W the wave count attn_decode_ex
 * reports with split_keys = 0 (2048 at G <= 16 and D = 128 on an MI355X),
 * plus (B + 1) int64 -- must fit in it, else ATTN_ERR_SCRATCH before anything
 * is enqueued (the ragged 64-sequence decode at Qwen3-8B heads needs 5 MB).
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (on different streams, or from different threads) race and give wrong
 * results; calls ordered on one stream are safe.  Nothing in the array needs
 * to start at zero (each call writes every partial before it reads it).
 */
int attn_decode_noalloc(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens,
                        void *out, int B, int Hq, int Hkv, int Lmax, int D, float scale, void *stream);

/* attn_decode_noalloc_max_bytes -- the size of attn_decode_noalloc's static scratch. */
size_t attn_decode_noalloc_max_bytes(void);

/*
 * attn_decode_ex -- attn_decode with two extra controls:
 *   lse        [B][Hq] fp32 output (natural log; -inf where n_b == 0), may be NULL;
 *   split_keys 0: one key range per resident wave of the device; otherwise a
 *              positive multiple of 128 (else ATTN_ERR_SPLIT): enough ranges
 *              that none would exceed split_keys keys if every sequence had
 *              Lmax keys (at most 4096 ranges).  Results agree for every
 *              split up to fp32 rounding of the merge.
 * The partials live in a workspace taken from HIP's stream-ordered allocator
 * on `stream`, as for attn_decode (attn_decode_multi_ex takes a caller's).
 * Validation as attn_decode, with the split_keys check after the size checks
 * and before the empty-call return.
 */
int attn_decode_ex(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens,
                   void *out, float *lse, int B, int Hq, int Hkv, int Lmax, int D, float scale,
                   int split_keys, void *stream);

/*
 * attn_decode_multi -- T new query rows per sequence over the ragged cache
 * (verification of T speculated tokens, or a short chunk appended to a cache).
 *
 * Pages: the cost guide's is_causal section (with fewer queries than keys
 * the causal mask is anchored at the bottom-right corner) and its use_cache
 * section (the new tokens' K/V are already in the cache).  The T new tokens
 * of sequence b are its last T cached positions: with n_b = min(kv_lens[b],
 * Lmax), row t (0 <= t < T) sees keys [0, n_b - T + t].  This is
 * attn_prefill with Lq = T, causal, over each sequence's n_b keys; T = 1 is
 * attn_decode.  A row that sees no key (n_b < T - t, including empty
 * sequences) gets out = 0 and lse = -inf.
 *
 *   q, out  [B][Hq][T][D] bf16        lse [B][Hq][T] fp32, may be NULL
 *   kcache, vcache [B][Hkv][Lmax][D] bf16, kv_lens [B] int32 (device)
 *
 * window > 0: sliding window, row t sees only keys [n_b - T + t - window + 1,
 * n_b - T + t] (keys before the earliest window start are not read at all);
 * 0: no window; negative: ATTN_ERR_SHAPE.  With T = 1 this is a windowed
 * single-token decode.
 *
 * The G * T rows of one KV head (G = Hq / Hkv) share every K/V read, in
 * groups of up to 64 rows.  1 <= T <= Lmax (else ATTN_ERR_SHAPE).  Key ranges
 * are chosen as attn_decode does.  workspace: NULL takes the partials from
 * the stream-ordered allocator; otherwise a caller-owned device buffer of at
 * least attn_decode_multi_workspace_bytes(...) bytes (else
 * ATTN_ERR_WORKSPACE), not used by other work until this call's kernels have
 * finished on `stream`.
 *
 * Groups of 33 to 64 rows over a large cache (at least 32768 32-key blocks
 * by the shapes, D 64 or 128, bf16 caches) take a second kernel with 32-row
 * matrix blocks and K/V staged through LDS; results agree to rounding.
 */
int attn_decode_multi(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens,
                      void *out, float *lse, int B, int Hq, int Hkv, int T, int window, int Lmax, int D,
                      float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_q8 -- attn_decode_multi over int8 (q8_0-style) K and V caches.
 *
 * Pages: the Attention Slack page (Gemma-4 26B) runs llama.cpp's flash
 * attention with both caches stored as q8_0 (its llama-server service
 * configuration); the pages do not define the format.  The format read here:
 * every row of D elements is cut into D / 32 blocks of 32 consecutive
 * elements; block j of a row holds one fp16 scale s_j and 32 int8 codes c_i,
 * and element i of the block is x = s_j * c_i (computed in fp32 and rounded
 * to bf16, nearest even, before it enters the products; scores, softmax
 * statistics and accumulators are fp32 as in attn_decode).
 *
 *   q, out          [B][Hq][T][D] bf16       lse [B][Hq][T] fp32, may be NULL
 *   kq, vq          [B][Hkv][Lmax][D] int8   (codes -128..127; -128 is legal)
 *   kscale, vscale  [B][Hkv][Lmax][D / 32] fp16 (IEEE binary16 bits)
 *   kv_lens         [B] int32 (device)
 *
 * Everything else -- T, window, the causal limits, empty sequences, lengths
 * above Lmax, workspace and its size (attn_decode_multi_workspace_bytes with
 * the same sizes) and the status codes -- is as attn_decode_multi.  Codes and
 * scales of positions at or past a sequence's length (or before its window)
 * are never read.  A NULL kscale or vscale with B > 0 is ATTN_ERR_NULL.
 */
int attn_decode_q8(const void *q, const void *kq, const void *kscale, const void *vq, const void *vscale,
                   const int32_t *kv_lens, void *out, float *lse, int B, int Hq, int Hkv, int T, int window,
                   int Lmax, int D, float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_multi_workspace_bytes -- bytes of workspace attn_decode_multi
 * needs for these sizes; 0 for an empty call and for invalid arguments.
 */
size_t attn_decode_multi_workspace_bytes(int B, int Hq, int Hkv, int T, int Lmax, int D);

/*
 * attn_decode_multi_ex -- attn_decode_multi with the key-range size of
 * attn_decode_ex (split_keys) and an explicit choice of main kernel, for tests
 * and tuning:
 *   kernel  0: chosen as attn_decode_multi does;
 *           1: the kernel for row groups of up to 64 rows with K/V streamed
 *              into registers (every shape);
 *           2: the wide-group kernel (32-row matrix blocks, K/V staged through
 *              LDS), whatever the cache size; only for groups of 33 to 64
 *              rows (G * T > 32), D 64 or 128 (else ATTN_ERR_KERNEL);
 *           anything else: ATTN_ERR_KERNEL.
 * All three give the same results up to rounding order.  Everything else,
 * including the workspace and its size, is as attn_decode_multi; validation
 * order: as attn_decode_multi, then split_keys, then kernel, then the
 * workspace size.
 */
int attn_decode_multi_ex(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens,
                         void *out, float *lse, int B, int Hq, int Hkv, int T, int window, int Lmax, int D,
                         float scale, int split_keys, int kernel, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * attn_decode_waves -- the number of key ranges (waves) attn_decode_ex uses
 * for these sizes and split_keys on the current device; 0 for invalid
 * arguments or when no device is available.
 */
int attn_decode_waves(int B, int Hq, int Hkv, int Lmax, int D, int split_keys);

/*
 * attn_backward -- gradients dq, dk, dv of attn_prefill(_ex) from its out and
 * lse and the upstream gradient dout.
 *
 * Pages: the cost guide, section "eager 어텐션 메모리, 길이에 따라 얼마나
 * 커지나" (training keeps a score table per layer for the backward pass; the
 * tiled method keeps only per-row statistics, from which the weights are
 * recomputed here).  The gradients are those of the forward definition:
 * with p_ij = exp(scale <q_i, k_j> - lse_i) over the visible keys,
 *   dv_j = sum_i p_ij dout_i,   ds_ij = p_ij (<dout_i, v_j> - <dout_i, out_i>),
 *   dq_i = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i,
 * with dk and dv of a KV head summed over its G = Hq / Hkv query heads.
 *
 *   q, out, dout, dq  [B][Hq][Lq][D] bf16     lse [B][Hq][Lq] fp32 (natural log,
 *                                              as attn_prefill writes it)
 *   k, v, dk, dv      [B][Hkv][Lk][D] bf16
 *
 * causal and window as attn_prefill_ex (the same mask must be given as in
 * the forward call that produced out and lse).  D is 64, 128 or 256 (else
 * ATTN_ERR_HEADDIM).  Every row must see a key: Lk = 0 with Lq > 0, Lq = 0
 * with Lk > 0 and causal with Lq > Lk are ATTN_ERR_SHAPE; B = 0 or
 * Lq = Lk = 0 is an empty call (ATTN_OK, nothing touched, pointers may be
 * NULL).  Every pointer is required otherwise (ATTN_ERR_NULL).  dq, dk and dv
 * are fully overwritten (not accumulated into) and must not overlap the
 * inputs.  Accumulation is fp32; the three outputs are rounded to bf16.
 *
 * workspace: NULL (taken from HIP's stream-ordered allocator on `stream` and
 * released there) or at least attn_backward_workspace_bytes(B, Hq, Lq) bytes
 * of device memory (else ATTN_ERR_WORKSPACE), 256-byte aligned, not used by
 * other work until the call's kernels have finished.  The call does not
 * synchronise: a pre-pass and the dk/dv kernel are enqueued on `stream`, and
 * the dq kernel, which needs only the pre-pass, on a stream of the library's
 * own (one per device, created on the first call) that waits for the
 * pre-pass through an event; `stream` then waits for the dq kernel through a
 * second event, so all of the call's work is ordered before whatever is
 * enqueued on `stream` afterwards.
 */
int attn_backward(const void *q, const void *k, const void *v, const void *out, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Lq, int Lk,
                  int D, int causal, int window, float scale, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * attn_backward_workspace_bytes -- bytes of workspace attn_backward needs
 * (two fp32 values per query row); 0 for an empty call or invalid sizes.
 */
size_t attn_backward_workspace_bytes(int B, int Hq, int Lq);

/* attn_status_string -- static, NUL-terminated text for a status code. */
const char *attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */

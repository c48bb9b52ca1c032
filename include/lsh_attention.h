/*
 * lsh_attention.h — C ABI of the MI355X (gfx950) multi-round LSH-attention forward.
 *
 * The forward pass of Reformer's LSH attention with shared query/key vectors,
 * split into its four steps.  Each step is one call; the calls run their HIP
 * kernels asynchronously on the caller's stream and never synchronise it.
 *
 * Passages followed (page title, section):
 *   [ULT] Ultralytics glossary "Reformer" (Spanish / Arabic editions), section on
 *         LSH attention: angular hashing by the position of the largest entry of
 *         [xR, -xR] for a random R; tokens sorted by bucket; the sorted sequence
 *         cut into equal chunks; each token attends to its own chunk and the one
 *         before it; several hash rounds.
 *   [MOD] modulabs-hub notes on "Reformer: The Efficient Transformer", sections
 *         "Locality sensitive hashing" (n_buckets/2 random columns, concatenated
 *         with their negation), "LSH attention" (the query itself removed because
 *         shared QK makes it its own best match; causal attention to earlier
 *         positions only; sorting and equal chunks), "Multi-round LSH attention".
 *   [AIS] ai-scholar.tech article on Reformer: the scaled dot-product attention
 *         formula; section on LSH attention (sort by bucket, equal chunks, attend
 *         to each chunk and the previous one).
 *
 * Conventions shared by every call
 *   B = batch, H = heads, L = seq_len, d = d_head, nb = n_buckets, n_r = n_rounds,
 *   c = chunk.  Tensors are dense, row-major, last index fastest, and live in
 *   device memory (pointers from hipMalloc or a framework allocator on the
 *   current device).  The caller allocates and owns every buffer; the library
 *   allocates nothing, draws no random numbers and keeps no mutable global state,
 *   so calls on different streams may run concurrently.
 *   `stream` is the HIP stream the kernels run on (NULL = the default stream).
 *   dtype LSH_BF16: qk, v, R, o_rounds and o hold bfloat16; products are exact and
 *   accumulate in fp32; outputs are rounded to nearest even.  dtype LSH_F32: all
 *   float32.
 *
 * Errors
 *   Every call checks its arguments on the host before any HIP call and returns
 *   a status; nothing is launched unless it returns LSH_OK.
 *   LSH_ERR_INVALID_ARG  null or non-16-byte-aligned pointer; a size <= 0;
 *                        n_buckets odd; L % chunk != 0; L / chunk > 32767;
 *                        L > 2^30; scale not finite; causal not 0/1; a buffer
 *                        larger than 2^62 bytes.
 *   LSH_ERR_UNSUPPORTED  d_head not 64 or 128; dtype not LSH_F32/LSH_BF16;
 *                        n_buckets > 32768; n_rounds > 16; chunk not 32, 64 or
 *                        128 (attention only); a flag bit other than the
 *                        LSH_FLAG_* values below.
 *   LSH_ERR_WORKSPACE    workspace smaller than lsh_sort_workspace_bytes().
 *   LSH_ERR_HIP          a kernel launch failed (hipGetLastError).
 *   Faults inside a kernel surface asynchronously at the caller's next
 *   synchronisation of `stream`.  lsh_last_error() names the failed check
 *   (per thread).
 */
#ifndef LSH_ATTENTION_H
#define LSH_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

/* hipStream_t.  hipcc defines the platform macro itself; a plain C or C++
 * compiler building host code against this header adds -D__HIP_PLATFORM_AMD__
 * and -I/opt/rocm/include, as for any HIP API host code. */
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lsh_status {
    LSH_OK = 0,
    LSH_ERR_INVALID_ARG = 1,
    LSH_ERR_UNSUPPORTED = 2,
    LSH_ERR_WORKSPACE = 3,
    LSH_ERR_HIP = 4
} lsh_status;

enum { LSH_F32 = 0, LSH_BF16 = 1 };

/*
 * Variant flags (lsh_config.flags, OR-ed).  They change step 3 only; the
 * other steps accept and ignore them.  0 is the method as described above.
 *   LSH_FLAG_NO_DUP_CORRECTION  drop the -log N_ij term: every round is plain
 *        softmax over its window, and the combine no longer equals attention
 *        over the union of the rounds' windows.
 *   LSH_FLAG_WRAP_LOOKBACK      chunk 0 of a round also attends to the last
 *        chunk of that round (look-back around the end of the sorted order);
 *        with a single chunk it attends to itself once.  N_ij counts the rounds
 *        with (cid[i,r'] - cid[j,r']) mod (L / c) in {0, 1}.
 *   LSH_FLAG_SAME_BUCKET        inside the window, only keys in the query's
 *        bucket of that round are attended ([MOD] "LSH attention": the set
 *        P_i), and N_ij counts the rounds where j is in the window and in i's
 *        bucket.  lsh_sort then writes window ids instead of chunk ids:
 *        cid[b,h,pos,r] = slot / c + 2 * (number of non-empty buckets below the
 *        position's bucket in round r), stored as an unsigned 16-bit value;
 *        two ids differ by 0 or 1 exactly when the buckets are equal and the
 *        chunks differ by 0 or 1.  Needs L/c - 1 + 2 (min(nb, L) - 1) <= 65534
 *        and cannot be combined with LSH_FLAG_WRAP_LOOKBACK (LSH_ERR_UNSUPPORTED).
 * Every call of one forward pass must get the same flags.  The pages leave
 * these points open (they describe look-back to the previous chunk; [MOD]'s
 * per-bucket set P_i and the chunk windows of [AIS] and [ULT] disagree; the
 * duplicate-count term is the reading under which the rounds' outputs merge
 * to attention over their union).
 */
enum { LSH_FLAG_NO_DUP_CORRECTION = 1, LSH_FLAG_WRAP_LOOKBACK = 2, LSH_FLAG_SAME_BUCKET = 4 };

typedef struct lsh_config {
    int32_t batch;      /* B >= 1 */
    int32_t heads;      /* H >= 1 */
    int32_t seq_len;    /* L >= 1, L % chunk == 0 */
    int32_t d_head;     /* 64 or 128 */
    int32_t n_buckets;  /* even, 2 .. 32768 */
    int32_t n_rounds;   /* 1 .. 16 hash rounds, each with its own R */
    int32_t chunk;      /* c >= 1; attention supports 32, 64, 128 */
    int32_t causal;     /* 1: a query never attends to a later position */
    float scale;        /* score = scale * <qk_i, qk_j>; usually 1/sqrt(d_head) */
    int32_t dtype;      /* LSH_F32 or LSH_BF16 */
    int32_t flags;      /* LSH_FLAG_* bits, 0 for the method as described */
} lsh_config;

/*
 * Step 1 — angular LSH hash.  [ULT]; [MOD] "Locality sensitive hashing".
 *   buckets[b,h,r,i] = index of the largest entry of [p, -p], p = qk[b,h,i,:] · R[r]
 *   (p has nb/2 entries; an index k >= nb/2 means entry k - nb/2 of -p).
 *   Exact ties of |p| go to the lowest column; a zero vector gets bucket 0.
 *   qk       [B, H, L, d]        dtype
 *   R        [n_r, d, nb/2]      dtype; one random matrix per round, shared by
 *                                every batch row and head
 *   buckets  [B, H, n_r, L]      int32 out, values in [0, nb)
 */
lsh_status lsh_hash(const lsh_config* cfg, const void* qk, const void* R,
                    int32_t* buckets, hipStream_t stream);

/* Bytes of device workspace lsh_sort needs for `cfg` (0 if cfg is invalid). */
size_t lsh_sort_workspace_bytes(const lsh_config* cfg);

/*
 * Step 2 — sort by bucket.  [AIS] LSH section; [ULT]; [MOD] "LSH attention".
 *   For every (b, h, r): a stable sort of positions 0..L-1 by bucket, i.e. the
 *   lexicographic order of (round, bucket, position).
 *   buckets    [B, H, n_r, L]   int32 in, values in [0, nb) (not checked)
 *   perm       [B, H, n_r, L]   int32 out: perm[b,h,r,slot] = position
 *   cid        [B, H, L, n_r]   int16 out: cid[b,h,pos,r] = slot(pos) / chunk
 *   workspace  device scratch of at least lsh_sort_workspace_bytes(cfg) bytes
 *              (per-tile bucket counters and per-round bucket totals); its
 *              contents on entry do not matter.
 */
lsh_status lsh_sort(const lsh_config* cfg, const int32_t* buckets, int32_t* perm,
                    int16_t* cid, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Step 2 without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same inputs, outputs and results as lsh_sort; the
 * counters live in a static device array of LSH_SORT_NOALLOC_MAX_BYTES that
 * the library holds on every GPU it runs on until the process ends.  The call
 * allocates nothing.  Every call on one GPU shares that GPU's array, so calls
 * whose executions overlap on one GPU (different streams, or several host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  Errors as lsh_sort, and LSH_ERR_WORKSPACE when the configuration
 * needs more than LSH_SORT_NOALLOC_MAX_BYTES (lsh_sort_workspace_bytes(cfg)
 * tells how much).
 */
#define LSH_SORT_NOALLOC_MAX_BYTES (64u << 20)
lsh_status lsh_sort_noalloc(const lsh_config* cfg, const int32_t* buckets, int32_t* perm,
                            int16_t* cid, hipStream_t stream);

/*
 * Step 3 — chunked attention, one output per round.  [AIS] formula and LSH
 * section; [ULT]; [MOD] "LSH attention".
 *   In round r, the query at sorted slot s (chunk k = s / c) attends to the keys
 *   in chunks k-1 and k of that round's sorted order (chunk 0: only itself,
 *   unless LSH_FLAG_WRAP_LOOKBACK).  For query i and key j:
 *       s_ij = scale * <qk_i, qk_j> - log N_ij - 1e5 * [j == i]
 *   where N_ij = number of rounds r' with cid[i,r'] - cid[j,r'] in {0, 1} (the
 *   rounds whose window for i holds j; the term is absent with
 *   LSH_FLAG_NO_DUP_CORRECTION); keys j > i are dropped when causal.
 *       lse_i = logsumexp_j s_ij,   o_i = sum_j exp(s_ij - lse_i) v_j.
 *   qk, v     [B, H, L, d]          dtype
 *   perm      [B, H, n_r, L]        int32, from lsh_sort
 *   cid       [B, H, L, n_r]        int16, from lsh_sort
 *   o_rounds  [B, H, n_r, L, d]     dtype out, rows in original position order
 *   lse       [B, H, n_r, L]        float32 out, original position order
 */
lsh_status lsh_chunk_attn(const lsh_config* cfg, const void* qk, const void* v,
                          const int32_t* perm, const int16_t* cid, void* o_rounds,
                          float* lse, hipStream_t stream);

/*
 * Step 4 — combine the rounds.  [MOD] "Multi-round LSH attention"; [ULT].
 *   LSE_i = logsumexp_r lse[r,i];  o_i = sum_r exp(lse[r,i] - LSE_i) o_rounds[r,i].
 *   o_rounds [B, H, n_r, L, d] dtype;  lse [B, H, n_r, L] float32;
 *   o        [B, H, L, d]      dtype out.
 */
lsh_status lsh_combine_rounds(const lsh_config* cfg, const void* o_rounds,
                              const float* lse, void* o, hipStream_t stream);

/*
 * Backward of steps 3-4: gradients with respect to qk and v (bfloat16, chunk 64;
 * the method as above and every variant flag).  The pages print no
 * backward pass; this is the chain rule through the forward defined above.
 * After the combine, query i's output is one softmax over all (round, key)
 * pairs of its windows ([MOD] "Multi-round LSH attention" merges the rounds by
 * their logsumexp):
 *   o_i = sum_r sum_j P_ijr v_j,   P_ijr = exp(s_ijr - LSE_i),   LSE_i = logsumexp_r lse_ir.
 * With Delta_i = <d_o_i, o_i> and dS_ijr = P_ijr (<d_o_i, v_j> - Delta_i):
 *   d_v[j]  = sum of P_ijr d_o_i over the (i, r) whose window holds j
 *   d_qk[i] = scale * (sum_{r, j} dS_ijr qk_j  +  sum_{r, i'} dS_i'ir qk_i')
 *             (i as a query, and i as a key of the queries i').
 * The buckets are piecewise constant in qk and carry no gradient.
 *   qk, v [B, H, L, d] and perm, cid, lse as passed to / written by steps 2-3;
 *   o    [B, H, L, d]  the combined forward output (lsh_combine_rounds);
 *   d_o  [B, H, L, d]  bf16 in: the loss gradient at o;
 *   d_qk, d_v [B, H, L, d] float32 out (overwritten).
 *   workspace  device scratch of at least lsh_backward_workspace_bytes(cfg)
 *              bytes (combined lse and Delta, and per-round partial gradients:
 *              about 6 * B*H*n_rounds*L*d bytes); its contents on entry do not
 *              matter.
 * Errors as above, and LSH_ERR_UNSUPPORTED for dtype LSH_F32 or chunk other
 * than 64; LSH_ERR_WORKSPACE.
 */
size_t lsh_backward_workspace_bytes(const lsh_config* cfg);
lsh_status lsh_attn_backward(const lsh_config* cfg, const void* qk, const void* v,
                             const int32_t* perm, const int16_t* cid, const float* lse,
                             const void* o, const void* d_o, float* d_qk, float* d_v,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Projections of the LSH-attention layer around steps 1-4 (bfloat16 only).
 * [MOD] "LSH attention": queries and keys share one projection; [AIS]
 * experiment set-up: d_model 1024 and 8 heads.  Weights are stored like a
 * linear layer's, [out, in]; products accumulate in fp32; outputs are rounded to
 * nearest even.
 *   lsh_project_in:   qk[b,h,i,c] = sum_k x[b,i,k] * w_qk[h*d + c, k]
 *                     v[b,h,i,c]  = sum_k x[b,i,k] * w_v[h*d + c, k]
 *     x [B, L, d_model];  w_qk, w_v [H*d, d_model];  qk, v [B, H, L, d] out
 *     (the layout steps 1-4 take).
 *   lsh_project_out:  y[b,i,n] = sum_{h,c} o[b,h,i,c] * w_o[n, h*d + c]
 *     o [B, H, L, d] (from lsh_combine_rounds);  w_o [d_model, H*d];
 *     y [B, L, d_model] out.
 * Errors as above, and: d_model not a positive multiple of 64 or above 65536,
 * or B*L >= 2^31 (LSH_ERR_INVALID_ARG); dtype not LSH_BF16 (LSH_ERR_UNSUPPORTED).
 */
lsh_status lsh_project_in(const lsh_config* cfg, int32_t d_model, const void* x, const void* w_qk,
                          const void* w_v, void* qk, void* v, hipStream_t stream);
lsh_status lsh_project_out(const lsh_config* cfg, int32_t d_model, const void* o, const void* w_o,
                           void* y, hipStream_t stream);

/*
 * The Reformer block's pieces (bfloat16, fp32 accumulation, outputs rounded to
 * nearest even).  [ULT] "Capas reversibles y división en fragmentos", [MOD]
 * "Reversible Transformer" and "Chunking": the activations are two halves,
 *   y1 = x1 + Attention(x2),   y2 = x2 + FeedForward(y1),
 * and the backward pass recomputes the inputs from the outputs,
 *   x2 = y2 - FeedForward(y1),  x1 = y1 - Attention(x2).
 * The feed-forward layer acts on each position alone and runs over chunks of
 * positions (its hidden layer is several times wider than the model; [AIS]:
 * d_ff 4096 at d_model 1024).  The pages do not write it out; it is the
 * transformer's position-wise form FeedForward(x) = relu(x w1^T + b1) w2^T + b2.
 *
 *   lsh_project_out_add:  y = residual + sign * (lsh_project_out's product):
 *     the attention half of the block (sign +1), or of its inverse (sign -1).
 *     residual, y [B, L, d_model]; y may be the same buffer as residual.
 *   lsh_ffn:  y[m, :] = residual[m, :] + sign * FeedForward(x[m, :]) for the
 *     rows m < rows of x, residual and y [rows, d_model] (row-major), computed
 *     chunk_rows rows at a time: one chunk's hidden activations relu(x w1^T +
 *     b1) are rounded to bf16 in `hidden` (at least lsh_ffn_workspace_bytes()
 *     bytes) and multiplied by w2 before the next chunk.  w1 [d_ff, d_model],
 *     b1 [d_ff], w2 [d_model, d_ff], b2 [d_model].  y may be the same buffer
 *     as residual, or as x.
 * Errors: as above for lsh_project_out_add (plus sign not finite); lsh_ffn:
 * rows not in (0, 2^31), d_model or d_ff not a positive multiple of 64 at most
 * 65536, chunk_rows not positive, sign not finite, a null or misaligned pointer
 * (LSH_ERR_INVALID_ARG); hidden too small (LSH_ERR_WORKSPACE).
 */
lsh_status lsh_project_out_add(const lsh_config* cfg, int32_t d_model, const void* o,
                               const void* w_o, const void* residual, float sign, void* y,
                               hipStream_t stream);
size_t lsh_ffn_workspace_bytes(int64_t rows, int32_t d_ff, int32_t chunk_rows);
lsh_status lsh_ffn(int64_t rows, int32_t d_model, int32_t d_ff, int32_t chunk_rows, const void* x,
                   const void* w1, const void* b1, const void* w2, const void* b2,
                   const void* residual, float sign, void* y, void* hidden, size_t hidden_bytes,
                   hipStream_t stream);

/* Static description of a status code. */
const char* lsh_status_string(lsh_status status);

/* Message describing the last non-OK status returned on the calling thread. */
const char* lsh_last_error(void);

/*
 * Device-side bounds checks (debug build).  Not a step of the method.
 * The kernels clamp or skip every index they take from caller data: positions
 * read from perm (chunk attention and its backward), bucket ids (sort) and the
 * sorted slots the sort computes from them.  So out-of-range values never
 * reach memory outside the buffers; they only make the results meaningless.
 * The debug library (liblsh_attention_debug.so, built with LSH_DEVICE_CHECKS)
 * also counts every such value on the device.
 *   count   host out: failed checks since the last reset, summed over the
 *           library's kernels (one bad value may fail more than one check);
 *           always 0 in the release library, which has no checks.
 *   reset   nonzero: clear the counters after reading them.
 * Reads the counters of the current device synchronously (hipMemcpyFromSymbol),
 * so call it after the kernels of interest have finished.  Errors: count NULL
 * (LSH_ERR_INVALID_ARG); a failed copy (LSH_ERR_HIP).
 */
lsh_status lsh_debug_check_failures(unsigned long long* count, int reset);

#ifdef __cplusplus
}
#endif

#endif /* LSH_ATTENTION_H */

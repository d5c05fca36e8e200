/*
 * fa.h - exact tiled attention (forward and backward) for AMD MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention as defined on the
 * FlashAttention-2 overview page (lshu.cn/news/55956): section 2.1 gives the
 * standard definition (score matrix Q K^T, softmax of each row, weighted sum
 * of V), section 2.2 the tiled, IO-aware way of computing it (Q/K/V tiles
 * streamed from HBM, online softmax with a running row max and row sum, no
 * N x N matrix in HBM, double-buffered on-chip tiles), section 3.3 the call
 * flash_attn_func(q, k, v, dropout_p, softmax_scale, causal) on tensors laid
 * out (batch, seqlen, nheads, headdim) with num_kv_heads for K and V, and
 * section 4.2 (question 4) the causal upper-triangular mask.  The install
 * guide page (yfxerp.com/news/195771, section 1) names the sliding window
 * (window_size) and the backward that recomputes the scores instead of
 * storing them; its section 3.3 gives the head_dim contract (a multiple of 8,
 * not too small).  The same
 * overview page's section 3.2 names packed variable-length batches.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout (row-major, head dimension contiguous, no other strides):
 *   q, o, dout, dq : [batch, seqlen_q, heads,    head_dim]
 *   k, v, dk, dv   : [batch, seqlen_k, kv_heads, head_dim]
 *   lse            : [batch, heads, seqlen_q] float32
 * Packed variable-length batches (cu_seqlens_q and cu_seqlens_k both
 * non-null): sequence b holds rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of
 *   q, o, dout, dq : [total_q, heads,    head_dim]
 *   k, v, dk, dv   : [total_k, kv_heads, head_dim]
 *   lse            : [heads, total_q] float32
 * and seqlen_q / seqlen_k give the longest sequence of each.  cu_seqlens_*
 * are device arrays of batch+1 non-decreasing int32 prefix sums starting at
 * 0 (not checked on the device).
 * Padded batches (fixed layout, seqused_q and/or seqused_k non-null; the
 * padded-batch test the overview page names in section 3.2): sequence b uses
 * only its first seqused_q[b] query rows and seqused_k[b] key rows (device
 * int32[batch], clamped to 0 .. seqlen) and is computed exactly as that
 * shorter sequence, bottom-right alignment included.  The rows past them are
 * written as a sequence without them defines them: O = 0 and LSE = -inf
 * (fa_fwd), dQ = 0, dK = dV = 0 (fa_bwd).  Not combined with cu_seqlens
 * (FA_ERR_INVALID_ARG).
 *
 * Visible keys of query row i in a sequence of Lq queries and Lk keys, with
 * p = i + Lk - Lq (bottom-right alignment; p = i when Lq = Lk):
 *   key j is visible iff 0 <= j < Lk, (causal == 0 or j <= p),
 *   (window_left < 0 or j >= p - window_left) and
 *   (window_right < 0 or j <= p + window_right).
 * The conditions combine as an intersection, so with causal = 1 a
 * window_right > 0 is accepted and has no effect (causal already bounds the
 * keys at p).
 * A row with no visible key gets O = 0 and LSE = -inf (and zero gradient).
 * GQA / MQA: query head h reads kv head h / (heads / kv_heads).
 * Sizes: heads * head_dim must stay below 2^23 (offsets inside a tile of up
 * to 256 rows are 32-bit) and batch * heads below 2^31; FA_ERR_INVALID_ARG
 * otherwise.
 *
 * LSE[i] = ln(sum over visible j of exp(softmax_scale * q_i . k_j)).
 *
 * Dropout (the dropout_p argument of the attention call, overview page
 * section 3.3): with T = floor((1 - dropout_p) * 256 + 1/2), computed from
 * the float dropout_p, each softmax probability P_ij is kept and scaled by
 * 256 / T, or set to 0, before the weighted sum of V: O_i = sum_j P_ij M_ij
 * (256 / T) v_j.  LSE stays that of the undropped softmax.  Element
 * (sequence b, query head h, query row i, key j; i and j counted inside the
 * sequence) is kept iff byte (j mod 4) of word (i mod 4) of the
 * Philox4x32-10 block (Salmon et al., SC 2011) at counter (j / 4, i / 4, h,
 * b) with key (dropout_seed low 32 bits, high 32 bits) is below T.  The
 * backward given the same dropout_p and dropout_seed differentiates exactly
 * that function.  dropout_p = 0 (T = 256) is plain attention; T = 0 drops
 * everything (O = 0).
 *
 * Arithmetic: 16-bit inputs (fp16 or bf16, same type for every tensor),
 * products on the matrix cores with fp32 accumulation, softmax statistics
 * in fp32, P rounded to the input type before P.V, outputs rounded to
 * nearest even.  Every entry point except fa_bwd / fa_bwd_stage with
 * deterministic = 0 gives the same bytes for the same call on the same
 * inputs (no atomics); see fa_bwd.
 *
 * Pointers: device pointers, 16-byte aligned (lse 4-byte aligned).  A
 * tensor with no elements may be passed as NULL: the query-side tensors
 * (q, o, lse, dout, dq) when batch * seqlen_q == 0, the key-side ones
 * (k, v, dk, dv) when batch * seqlen_k == 0.  The caller owns every
 * buffer; the library allocates nothing, frees nothing and keeps no
 * pointer after returning.  Inputs are never written, outputs are fully
 * overwritten (no zeroing needed) and must not alias inputs or each other.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the null
 * stream) and the call returns without waiting.  Execution errors surface at
 * the caller's next synchronisation.
 *
 * Errors: every argument check runs before any HIP call, so a bad call
 * returns its code on any host.  The device check (FA_ERR_ARCH) is the
 * first HIP call; on a host without a gfx950 device it returns that code.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad scale   */
    FA_ERR_UNSUPPORTED = 2, /* head_dim not a multiple of 8 in [8, 256] (FP8: of 16
                               in [16, 128]), or dtype                             */
    FA_ERR_ARCH = 3,        /* no HIP device, or the current device is not gfx950 */
    FA_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace_size() call */
    FA_ERR_LAUNCH = 5       /* a kernel launch was rejected by the runtime        */
};

enum fa_dtype { FA_DTYPE_F16 = 0, FA_DTYPE_BF16 = 1 };

/*
 * Forward: O = softmax(softmax_scale * Q K^T restricted to visible keys) V,
 * and LSE, in one fused pass per query tile (overview page, sections 2.2
 * "tiled fusion" and "online softmax").
 *   q, k, v        in : see layout above
 *   o              out: like q
 *   lse            out: float32, see layout above
 *   cu_seqlens_q/k in : both NULL (fixed length) or both device int32[batch+1]
 *   seqused_q/k    in : NULL, or device int32[batch] (padded batches, above)
 *   batch >= 0, heads >= 1, kv_heads >= 1 with heads % kv_heads == 0,
 *   seqlen_q >= 0, seqlen_k >= 0, head_dim a multiple of 8 from 8 to 256
 *   (run in tiles 64, 128 or 256 wide; a head_dim below the tile width costs the
 *   tile width's arithmetic),
 *   causal in {0, 1}, window_left >= -1, window_right >= -1 (-1 = unbounded),
 *   softmax_scale finite and >= 0 (callers wanting the default pass
 *   1/sqrt(head_dim)), dtype one of fa_dtype.
 *   dropout_p in [0, 1), dropout_seed any 64-bit value: see "Dropout" below.
 * Returns FA_OK or an fa_status code; nothing is enqueued on error.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
           const int32_t* seqused_q, const int32_t* seqused_k,
           int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
           int head_dim, int causal, int window_left, int window_right,
           float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, void* stream);

/*
 * FP8 forward (overview page, section 5.2: attention on FP8 matrix cores with
 * float8_e4m3fn inputs).  q, k, v hold one byte per element, codes of the
 * 8-bit E4M3 format (OCP 8-bit floating point, E4M3 without infinities:
 * bias 7, largest value 448, 0x7F / 0xFF NaN), in the layouts above; the
 * value of an element is its tensor's descale times the code's value.
 * Computes the attention of those dequantised tensors:
 *   scores      softmax_scale * descale_q * descale_k * (q8 . k8), fp32
 *               (the matrix cores' FP8 dot products: not exactly rounded,
 *               observed within 2^-14 of the sum of the products' magnitudes)
 *   LSE         natural log of the sum of exp(score) over visible keys
 *   O           descale_v * sum_j P_ij v8_j / l_i, with the probabilities P
 *               rounded to E4M3 (nearest even) before the product and l_i
 *               their unrounded fp32 sum; stored as out_dtype (fa_dtype)
 * The rounding of P is the one approximation: each rounded P_ij lies within
 * 2^-4 P_ij + 2^-14 of P_ij (P relative to the row's largest probability),
 * so |O_ic - exact| <= (2^-4 sum_j P_ij |v_jc| + 2^-14 sum_j |v_jc| / L_i) / l_i
 * plus the score error and the output rounding, L_i being the row's sum of
 * exp(score - max score).
 *   head_dim a multiple of 16 from 16 to 128 (FA_ERR_UNSUPPORTED otherwise;
 *   run in tiles 64 or 128 wide); descales finite and
 *   >= 0; no dropout, no backward.  Everything else as for fa_fwd (masks,
 *   GQA, packed and padded batches, empty rows, alignment, errors).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
               const int32_t* seqused_q, const int32_t* seqused_k,
               int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
               int head_dim, int causal, int window_left, int window_right, float softmax_scale,
               float descale_q, float descale_k, float descale_v, int out_dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (the workspace is
 * part of the backward's contract as laid down for this library, not a
 * quantity the pages define): two float32 arrays of batch * heads *
 * seqlen_q entries, the per-row term D_i = dO_i . O_i and LSE_i * log2(e),
 * and, when deterministic = 0 and head_dim <= 128, before them a float32 dQ
 * accumulator of batch * seqlen_q * heads rows of 64 (head_dim <= 64) or
 * 128 values, padded to a multiple of 256 bytes.  For packed batches pass
 * the same batch and seqlen_q as to fa_bwd (batch * seqlen_q must be at
 * least total_q).  deterministic is 0 or 1.  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int batch, int heads, int seqlen_q, int head_dim, int dtype, int deterministic);

/*
 * Backward: given the forward's inputs, its O and LSE, and dout = dL/dO,
 * writes dq, dk, dv (same dtype and layout as q, k, v).  The scores are
 * recomputed from Q, K and the saved LSE (install guide page, section 1);
 * the N x N matrices are never stored.  Three kernels run in order on
 * `stream`: the row term D_i = dO_i . O_i, a pass over key tiles that
 * accumulates dK and dV (summing the query heads of a GQA group inside the
 * workgroup), and a dQ stage:
 *   deterministic = 1 (or head_dim > 128): a separate pass over query tiles
 *     accumulates dQ in registers; the same call gives the same bytes.
 *   deterministic = 0, head_dim <= 128: the key-tile pass also forms dQ from
 *     the same scores and adds each tile's part into a float32 accumulator
 *     in the workspace with atomic adds, and the last kernel rounds it to
 *     dq.  Five matrix products per visible pair instead of seven; the
 *     order of the float32 additions varies from call to call, so dq may
 *     differ in its last bits between calls (dk, dv do not).
 *   workspace / workspace_bytes: device memory of at least
 *   fa_bwd_workspace_size(batch, heads, seqlen_q, head_dim, dtype,
 *   deterministic) bytes, 16-byte aligned, owned by the caller; its contents
 *   on entry do not matter.
 * All other arguments as for fa_fwd, which must have produced o and lse
 * with the same arguments (dropout_p and dropout_seed included).
 * Packed batches: the query-side tensors must hold exactly
 * cu_seqlens_q[batch] rows (not checked on the device).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
           const int32_t* seqused_q, const int32_t* seqused_k,
           int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
           int head_dim, int causal, int window_left, int window_right,
           float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, int deterministic,
           void* stream);

/*
 * One stage of fa_bwd, for callers that schedule or time the three kernels
 * themselves: stage 0 writes D_i = dO_i . O_i into the workspace (and
 * clears the dQ accumulator on the atomic path), stage 1 writes dk and dv
 * (atomic path: and adds dQ into the accumulator), stage 2 writes dq.
 * fa_bwd is exactly stages 0, 1, 2 in this order on one stream.  With
 * deterministic = 1 stages 1 and 2 only read what stage 0 wrote and are
 * independent of each other; on the atomic path stage 2 reads what stage 1
 * added.  Arguments as for fa_bwd; a stage outside 0..2 returns
 * FA_ERR_INVALID_ARG.
 */
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 const int32_t* seqused_q, const int32_t* seqused_k,
                 int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                 int head_dim, int causal, int window_left, int window_right,
                 float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, int deterministic,
                 void* stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (work being captured into a HIP graph, serving loops,
 * harnesses that forbid allocation).  The workspace is a 16 MiB array inside
 * the library, one per device, held until the process ends; the call
 * allocates nothing.  Runs the deterministic path (deterministic = 1).
 * Limit: batch * heads * seqlen_q <= 2^21 (two float32 per query row and
 * head), FA_ERR_WORKSPACE beyond it.  All calls on one device share the
 * array, so calls that overlap on one GPU (other streams or threads) race:
 * the caller orders them.  Arguments and errors otherwise as for fa_bwd.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   const int32_t* seqused_q, const int32_t* seqused_k,
                   int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                   int head_dim, int causal, int window_left, int window_right,
                   float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, void* stream);

/*
 * Decode over a key/value cache (the KV-cache call named on the overview
 * page, section 3.3, for incremental inference): the same exact attention
 * as fa_fwd for a few new query tokens per sequence against a long cache.
 * The visible keys of all sequences are divided evenly over many waves,
 * whatever the sequence lengths, and the partial results are merged by
 * their LSE (overview page, section 2.2, online softmax: partial results
 * over disjoint key sets combine exactly through their row max and row
 * sum).
 *   q, o      : [batch, seqlen_q, heads, head_dim], the new tokens
 *   k_cache,
 *   v_cache   : [batch, seqlen_k, kv_heads, head_dim]; seqlen_k is the
 *               cache capacity.  Rows 0 .. cache_seqlens[b]-1 of sequence b
 *               are its keys; they already include the new tokens' own keys
 *               (the caller appends them), so query token t of sequence b
 *               sits at position cache_seqlens[b] - seqlen_q + t (bottom-right
 *               alignment, as in fa_fwd).
 *   lse       : [batch, heads, seqlen_q] float32
 *   cache_seqlens: device int32[batch], or NULL for "every sequence holds
 *               seqlen_k keys"; values are clamped to 0 .. seqlen_k on the
 *               device.  Rows past a sequence's length are never used.
 *   workspace : device memory of at least fa_fwd_kvcache_workspace_size()
 *               bytes, 16-byte aligned, owned by the caller; contents on
 *               entry do not matter.  It holds the partial O (float32) and
 *               LSE of every piece of work and the per-sequence prefix sums.
 *   num_splits: work division.  The query rows of a kv head (its query heads
 *               times seqlen_q) form blocks of 32; a segment is one
 *               (sequence, kv head, row block).  num_splits > 0 asks for
 *               num_splits waves per segment on average (batch * kv_heads *
 *               row blocks * num_splits waves in all); 0 gives about 512
 *               waves (two per CU), rounded down to a multiple of kv_heads.
 *               Capped at one wave per 32-key step of every segment at full
 *               capacity, and at 65536.
 * Sizes: batch * heads * seqlen_q and batch * ceil(heads / kv_heads *
 * seqlen_q / 32) * ceil(seqlen_k / 32) must stay below 2^31
 * (FA_ERR_INVALID_ARG otherwise).
 * All other arguments, the visibility rule, GQA, the empty-row convention
 * and the arithmetic are those of fa_fwd, except that P is rounded to 16
 * bits against each piece's own running max and the pieces are merged in
 * float32, so O is not bit-identical to fa_fwd's (both are within rounding
 * of the exact result).  Two kernels run on `stream`: the split pass and
 * the merge.  Returns FA_OK or an fa_status code; nothing is enqueued on
 * error.
 */
size_t fa_fwd_kvcache_workspace_size(int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                                     int head_dim, int num_splits);

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   const int32_t* cache_seqlens, void* workspace, size_t workspace_bytes,
                   int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                   int head_dim, int causal, int window_left, int window_right,
                   float softmax_scale, int dtype, int num_splits, void* stream);

/* The number of waves fa_fwd_kvcache's split pass uses for these sizes (0 for
 * invalid sizes). */
int fa_fwd_kvcache_splits(int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k, int head_dim,
                          int num_splits);

/* Static text for a status code ("unknown status" for others).  Part of
 * this library's contract, like the status codes themselves; the pages
 * define no error reporting. */
const char* fa_strerror(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

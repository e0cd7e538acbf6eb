/*
 * attn.h — C ABI of libattn.so: fused, tiled softmax-attention forward for AMD MI355X (gfx950).
 *
 *   O = softmax(scale · Q·Kᵀ + mask) · V, computed tile by tile with an online (running max /
 *   running sum) softmax, so the score matrix S and the weights P never reach HBM.
 *
 * Sources of the operation (cited by page title and section):
 *   - "Resumen Técnico: FlashMLA-ETAP", section "Mecanismo Central": the standard flow
 *     S = Q·Kᵀ, P = softmax(S), O = P·V that every entry point computes.
 *   - "Activar Flash Attention con llama.cpp para optimizar la inferencia", section
 *     "¿Qué es Flash Attention y por qué es crucial para llama.cpp?": tiling with iterative,
 *     local updates in on-chip memory instead of materialising the intermediates in HBM.
 *   - Same page, FAQ entry on Grouped Query Attention: K/V shared by groups of query heads.
 *   - "Resumen Técnico: FlashMLA-ETAP", sections "Planteamiento del Problema" and "Detalles de
 *     Implementación": MLA decode — 16 query heads, head dim 576 over one jointly compressed
 *     latent KV, very short queries against a KV context of up to 64K.
 *   - MInference article (7minutos.es), paragraphs on the A-shape, vertical-slash and
 *     block-sparse patterns and the dynamically built sparse indices; "SparseAccelerate:
 *     Acelerando Modelos de Lenguaje", section "Patrones de Atención Dispersa Dinámicos".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors. Q is [B, Lq, Hq, Dqk], K is [B, Lk, Hkv, Dqk], V is [B, Lk, Hkv, Dv], O is
 *   [B, Lq, Hq, Dv], all bfloat16, described by attn_tensor_t: a DEVICE pointer plus element
 *   strides for the batch, sequence and head dimensions; the head-dim stride is 1. The data
 *   pointer must be 16-byte aligned and every stride a multiple of 8 elements; the sequence
 *   stride of Q, K and V may not exceed 2^24 elements (ATTN_ERR_UNSUPPORTED). Contiguous
 *   [B, L, H, D] has stride_h = D, stride_l = H·D, stride_b = L·H·D.
 * LSE. Optional fp32 log-sum-exp of each query row, natural log of Σ_j exp(scale·q·k_j) over
 *   the visible keys, DEVICE pointer, contiguous [B, Hq, Lq]. Pass NULL to skip it. A row with
 *   no visible key gets O = 0 and LSE = -inf.
 * Scale. Any finite float. A negative scale reverses the order of the scores (the kernels
 *   negate Q as they load it and use |scale|); scale 0 weighs every visible key equally, so O is
 *   the mean of the visible value rows and LSE = ln(number of visible keys).
 * GQA. Hq must be a multiple of Hkv; query head h reads KV head h / (Hq / Hkv).
 * MLA. Pass v with the same data pointer and strides as k and Dv = 512 < Dqk = 576: V is then
 *   the first 512 columns of the latent K, read from the same memory (no copy).
 * Causal masking is aligned bottom-right: query row i sees key j iff j <= i + Lk - Lq. With
 *   Lq = 1 the single query sees the whole cache. Rows with i + Lk - Lq < 0 see nothing.
 * Arithmetic. bf16 inputs, fp32 accumulation (MFMA) and fp32 softmax statistics; O is
 *   rounded to bf16 with round-to-nearest-even.
 * Streams. `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *   asynchronously; the library never synchronises. Calls on one stream run in order.
 * Ownership. The caller allocates and owns every buffer (including split-KV partials). The
 *   library allocates no device memory, keeps no pointer after returning, and is re-entrant.
 * Errors. Every entry point returns ATTN_OK (0) or a negative attn_status. On an error nothing
 *   is launched and no output is written; attn_last_error() then holds a message (per thread).
 *   Asynchronous device faults surface at the caller's next synchronisation.
 */
#ifndef SPARSE_ATTN_AMD_ATTN_H_
#define SPARSE_ATTN_AMD_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_tensor {
  void* data;         /* device pointer to bf16 elements (const for inputs) */
  int64_t stride_b;   /* element stride between batch entries */
  int64_t stride_l;   /* element stride between sequence positions */
  int64_t stride_h;   /* element stride between heads; the head-dim stride is 1 */
} attn_tensor_t;

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,  /* a size, stride, alignment, pointer or scale is invalid */
  ATTN_ERR_UNSUPPORTED = -2,  /* valid arguments that the library has no kernel for */
  ATTN_ERR_WORKSPACE = -3,    /* split-KV partial buffers missing */
  ATTN_ERR_LAUNCH = -4        /* the HIP runtime refused the launch (message in last_error) */
} attn_status_t;

/*
 * attn_fwd — dense attention forward (prefill; any Lq, Lk).
 * Passage: "Resumen Técnico: FlashMLA-ETAP", section "Mecanismo Central" (S = Q·Kᵀ,
 * P = softmax(S), O = P·V), computed tile by tile as in "Activar Flash Attention con
 * llama.cpp para optimizar la inferencia", section "¿Qué es Flash Attention y por qué es
 * crucial para llama.cpp?"; causal GQA as in that page's FAQ entry on Grouped Query Attention.
 * Supported head dims: (Dqk, Dv) = (64, 64) or (128, 128).
 * Errors: INVALID_ARG if any of B, Hq, Hkv, Lq, Lk < 1, Hq % Hkv != 0, scale not finite, a
 * NULL q/k/v/o pointer, misalignment; UNSUPPORTED for other head dims; LAUNCH on HIP failure.
 */
int attn_fwd(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o, float* lse,
             int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv, int causal, float scale,
             void* stream);

/*
 * Split-KV decode: attn_fwd_splitkv writes per-split partials, attn_combine_lse merges them.
 * Passage: "Resumen Técnico: FlashMLA-ETAP", section "Planteamiento del Problema" (one or two
 * query tokens against a KV context of up to 64K, bound by the bandwidth of reading it) and
 * section "Mecanismo Central" (the attention each split computes over its keys). The pages do
 * not describe splitting the keys; the split and the log-sum-exp merge are this library's way
 * of spreading one decode step over the whole GPU, and the merge is exact: it equals attention
 * over all keys up to rounding.
 * Split s covers keys [s·C, min((s+1)·C, Lk)) with C = 64·ceil(ceil(Lk / S) / 64); a split
 * with no visible key writes O_s = 0 and LSE_s = -inf (weight 0 in the merge). The merge is
 * M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln Σ w_s, O = Σ w_s O_s / Σ w_s.
 * Sizes: o_part is fp32 [S, B, Hq, Lq, Dv], lse_part is fp32 [S, B, Hq, Lq], both contiguous
 * DEVICE buffers owned by the caller. num_splits must lie in [1, ceil(Lk / 64)].
 * Supported head dims: (64, 64), (128, 128) and the MLA latent (576, 512).
 * Any Lq is accepted. With D = 64 or 128 and at least 128 query rows, or 64 over at least 8192
 * keys (a query chunk against a longer cache: chunked prefill), the partials come from the
 * prefill kernel run over each split's keys; otherwise from the decode kernel (up to 32 query
 * columns of a KV head per workgroup). Both write the same partials.
 */

/* Split count the library would pick for MI355X (256 CUs): one round of one workgroup per CU
 * (for D = 128 when the work units fit that round; otherwise, and with more than 16 query
 * columns per KV head, one round of two per CU), or whole rounds when one round cannot be filled
 * exactly, each split at least one 64-key tile (two for the latent shape), at most 256 splits,
 * none empty; for query chunks of at least 128 rows, one round of two 128-row prefill
 * workgroups per CU with splits of at least 1024 keys. Pure function of its arguments; returns
 * a value in [1, ceil(Lk/64)], or ATTN_ERR_INVALID_ARG for sizes < 1. */
int attn_splitkv_num_splits(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv);

/* Bytes of o_part plus lse_part for these sizes (0 on invalid sizes). */
size_t attn_splitkv_workspace_bytes(int B, int Hq, int Lq, int Dv, int num_splits);

/* attn_fwd_splitkv — the partials of every split (passages as above).
 * Errors: as attn_fwd, plus INVALID_ARG for num_splits out of range and WORKSPACE when
 * o_part or lse_part is NULL or not 16-byte aligned. */
int attn_fwd_splitkv(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v,
                     float* o_part, float* lse_part, int num_splits,
                     int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv, int causal,
                     float scale, void* stream);

/* attn_combine_lse — merges the partials into O (bf16, strided like attn_fwd's O) and LSE
 * (fp32 [B, Hq, Lq] or NULL) with the formula above: the softmax over all keys of
 * "Mecanismo Central", rebuilt from per-split maxima and sums. Errors: INVALID_ARG for sizes < 1, NULL or misaligned pointers, Dv not in
 * {64, 128, 512}; WORKSPACE when o_part or lse_part is NULL. */
int attn_combine_lse(const float* o_part, const float* lse_part, int num_splits,
                     attn_tensor_t o, float* lse, int B, int Hq, int Lq, int Dv, void* stream);

/*
 * attn_fwd_decode — split-KV decode and its LSE combine in one call: attn_fwd_splitkv with
 * num_splits = attn_splitkv_num_splits(...) followed by attn_combine_lse, on one stream, with
 * the partials in the caller's workspace. When that count is 1, the split kernel writes O and
 * LSE itself and no combine is launched (same values bit for bit; for a query chunk of at least
 * 128 rows that kernel is attn_fwd's). Arguments as attn_fwd; o is bf16 strided like attn_fwd's,
 * lse fp32 [B, Hq, Lq] or NULL.
 * workspace: DEVICE buffer of at least attn_decode_workspace_bytes(...) bytes, 256-byte
 * aligned, owned by the caller; its contents on entry do not matter. Calls that overlap on
 * one workspace race.
 * Errors: as attn_fwd, plus WORKSPACE for a missing, short or misaligned workspace.
 */
int attn_fwd_decode(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                    float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                    int causal, float scale, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace bytes of attn_fwd_decode for these sizes (0 on invalid sizes). */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv);

/* Size of the library's per-device scratch array used by attn_fwd_decode_noalloc (16 MiB). */
#define ATTN_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * attn_fwd_decode_noalloc — attn_fwd_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc. It
 * computes exactly what attn_fwd_decode computes (same kernels, same split count, bitwise the
 * same O and LSE), but the split-KV partials go to a scratch array that the library holds in
 * device memory, ATTN_DECODE_SCRATCH_BYTES per GPU, kept from the first call on that GPU until
 * the process ends. The call allocates nothing; the caller still passes inputs and outputs as
 * for attn_fwd_decode.
 * The scratch belongs to the GPU that runs `stream` (the current device for the NULL stream);
 * its address is looked up once per GPU, on that GPU's first call.
 * Concurrency: every call on one GPU shares that GPU's scratch, which keeps the last call's
 * partials. Calls on one stream are ordered and safe; calls that overlap on one GPU (on
 * different streams, or from several host threads without ordering) race and may return
 * wrong results.
 * Errors: as attn_fwd_decode, with WORKSPACE when these sizes need more than one split and
 * attn_decode_workspace_bytes(...) exceeds ATTN_DECODE_SCRATCH_BYTES (use attn_fwd_decode
 * with a workspace then), and LAUNCH when the scratch address cannot be looked up. A call
 * with one split needs no partials and takes any size.
 */
int attn_fwd_decode_noalloc(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                            float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                            int causal, float scale, void* stream);

/*
 * attn_fwd_blocksparse — attention over a per-query-head union of listed key blocks and
 * vertical key columns (the block-sparse / A-shape / vertical-slash index lists), with the
 * causal mask applied on top when `causal` is set. Each key is counted once even when it is
 * both inside a listed block and listed as a column.
 * Passage: MInference article (7minutos.es), paragraphs on the A-shape, vertical-slash and
 * block-sparse patterns and on the sparse indices the kernels consume; "SparseAccelerate:
 * Acelerando Modelos de Lenguaje", section "Patrones de Atención Dispersa Dinámicos".
 *
 *   blk_ptr [B·Hq·nqb + 1], blk_idx — CSR over (b, h, qb) row-major, nqb = ceil(Lq / 64):
 *       blk_idx[blk_ptr[r] .. blk_ptr[r+1]) are the key-block ids (key block kb = keys
 *       [64·kb, 64·kb + 64)) visible to the 64 query rows [64·qb, 64·qb + 64).
 *   col_ptr [B·Hq + 1], col_idx — CSR over (b, h): key positions visible to every row of
 *       that head (subject to the causal mask).
 * All four are DEVICE int32 arrays; blk_idx (col_idx) may be NULL only when every block
 * (column) list is empty. Each list must be sorted ascending without duplicates,
 * block ids in [0, ceil(Lk/64)), columns in [0, Lk). Lk may be at most 2^20. Their contents are NOT checked on the
 * device (that would need a host copy): call attn_blocksparse_check on host copies.
 * block_m and block_n must both be 64. Supported head dims: (64, 64), (128, 128).
 */
int attn_fwd_blocksparse(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                         float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                         int causal, float scale, int block_m, int block_n,
                         const int32_t* blk_ptr, const int32_t* blk_idx,
                         const int32_t* col_ptr, const int32_t* col_idx, void* stream);

/*
 * attn_fwd_vertical_slash — attn_fwd_blocksparse with per-head slash lines added to the union
 * (the vertical-slash pattern of the MInference article, paragraph on the three patterns).
 * A slash line at offset o >= 0 is the diagonal o keys below the causal one: query row i
 * sees key i + (Lk - Lq) - o when that key exists. A key visible through a listed block, a
 * listed column and a slash line at once is counted once.
 *
 *   blk_ptr, blk_idx, col_ptr, col_idx — as attn_fwd_blocksparse (pass all-zero pointer
 *       arrays for no blocks or no columns).
 *   slash_ptr [B·Hq + 1], slash_idx — CSR over (b, h): sorted unique offsets in [0, Lk).
 *       DEVICE int32; slash_idx may be NULL only when every list is empty. Offsets outside
 *       [0, Lk) are ignored on the device; attn_vertical_slash_check validates host copies.
 *   workspace — DEVICE buffer of at least attn_vertical_slash_workspace_bytes(B, Hq, Lk)
 *       bytes, 256-byte aligned, owned by the caller; it receives two per-head bitmaps (the
 *       offsets and the columns) and holds nothing between calls.
 * Lk may be at most 2^19 here.
 * Errors: as attn_fwd_blocksparse, plus INVALID_ARG when slash_ptr is NULL, UNSUPPORTED for Lk
 * above 2^19, and WORKSPACE for a missing, short or misaligned workspace.
 */
int attn_fwd_vertical_slash(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                            float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                            int causal, float scale, const int32_t* blk_ptr,
                            const int32_t* blk_idx, const int32_t* col_ptr,
                            const int32_t* col_idx, const int32_t* slash_ptr,
                            const int32_t* slash_idx, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes of attn_fwd_vertical_slash (0 for sizes < 1). */
size_t attn_vertical_slash_workspace_bytes(int B, int Hq, int Lk);

/* Validates slash lists given as HOST pointers: slash_ptr[0] = 0 and monotone, offsets sorted
 * strictly ascending inside each head, in [0, Lk). Returns ATTN_OK or ATTN_ERR_INVALID_ARG
 * with a message naming the first bad entry. Touches no GPU. */
int attn_vertical_slash_check(const int32_t* slash_ptr, const int32_t* slash_idx, int B, int Hq,
                              int Lk);

/* Validates block-sparse index lists given as HOST pointers (same layout as above):
 * monotone pointers starting at 0, sorted unique ids, ids in range. Returns ATTN_OK or
 * ATTN_ERR_INVALID_ARG with a message naming the first bad entry. Touches no GPU. */
int attn_blocksparse_check(const int32_t* blk_ptr, const int32_t* blk_idx,
                           const int32_t* col_ptr, const int32_t* col_idx,
                           int B, int Hq, int Lq, int Lk, int block_m, int block_n);

/*
 * attn_build_sparse_index — builds, from Q and K, the block-sparse index lists that
 * attn_fwd_blocksparse consumes (square causal sizes: Lq = Lk = L).
 *
 * The pages (MInference article, paragraphs on the three patterns and on dynamic sparse
 * indices; "SparseAccelerate: Acelerando Modelos de Lenguaje", section "Patrones de Atención
 * Dispersa Dinámicos") fix that the indices are built per head at run time by a fast
 * approximation, and name no estimator. This library's estimator:
 *   - blocks: each 64-row block of Q and of K is mean-pooled; causal key block kb <= qb scores
 *     scale * <mean q_qb, mean k_kb>; query block qb lists its diagonal block and the top
 *     (topk_blocks - 1) other causal blocks (ties to the lower id), i.e. min(topk_blocks, qb+1)
 *     blocks, sorted ascending;
 *   - columns: the last min(64, L) query rows each take a causal softmax over the keys; a
 *     key's importance is the sum of its probabilities over those rows; the top
 *     min(n_cols, L) keys (ties to the lower index) are listed, sorted ascending.
 * The query head of KV head j are heads j*g .. j*g+g-1 (g = Hq / Hkv).
 *
 * Outputs (DEVICE int32 arrays owned by the caller; sizes from attn_sparse_index_sizes):
 *   blk_ptr [B*Hq*ceil(L/64) + 1], blk_idx [n_blk_idx], col_ptr [B*Hq + 1], col_idx [n_col_idx]
 *   (col_idx may be NULL when n_col_idx is 0).
 * workspace: DEVICE buffer of at least attn_sparse_index_workspace_bytes bytes, 256-byte
 * aligned, owned by the caller; its contents on entry do not matter.
 * Limits: D in {64, 128}, L <= 131072, topk_blocks >= 1, n_cols >= 0, every list total below
 * 2^31. Errors: INVALID_ARG for bad sizes, scale, pointers or alignment; UNSUPPORTED for D or
 * L outside the limits; WORKSPACE for a missing or short workspace; LAUNCH for a launch
 * failure. Nothing is launched on error.
 */
int attn_build_sparse_index(attn_tensor_t q, attn_tensor_t k, int B, int Hq, int Hkv, int L, int D,
                            float scale, int topk_blocks, int n_cols, int32_t* blk_ptr,
                            int32_t* blk_idx, int32_t* col_ptr, int32_t* col_idx, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Entries of blk_idx and col_idx that attn_build_sparse_index writes for these sizes.
 * Returns ATTN_OK, or INVALID_ARG for sizes < 1 (or n_cols < 0, topk_blocks < 1). */
int attn_sparse_index_sizes(int B, int Hq, int L, int topk_blocks, int n_cols,
                            int64_t* n_blk_idx, int64_t* n_col_idx);

/* Workspace bytes attn_build_sparse_index and attn_build_vslash_index need (0 on invalid
 * sizes). */
size_t attn_sparse_index_workspace_bytes(int B, int Hq, int Hkv, int L, int D);

/*
 * attn_build_vslash_index — builds, from Q and K, the column and slash-line lists that
 * attn_fwd_vertical_slash consumes (square causal sizes: Lq = Lk = L), with the same probe as
 * attn_build_sparse_index (the last min(64, L) query rows, each with its causal softmax over
 * the keys; MInference article, paragraphs on the vertical-slash pattern and on dynamic
 * indices, which name no estimator):
 *   - columns: as attn_build_sparse_index;
 *   - slash lines: line o (probe row r meets key r - o) scores the sum over probe rows of
 *     their probability on that key; the top min(n_slash, L) offsets (ties to the lower
 *     offset) are listed, sorted ascending.
 * Outputs (DEVICE int32, caller-owned): col_ptr [B*Hq + 1], col_idx [B*Hq*min(n_cols, L)],
 * slash_ptr [B*Hq + 1], slash_idx [B*Hq*min(n_slash, L)] (an index array may be NULL when
 * its size is 0). workspace: as attn_build_sparse_index (attn_sparse_index_workspace_bytes).
 * Limits: D in {64, 128}, L <= 131072, n_cols >= 0, n_slash >= 0. Errors: INVALID_ARG for bad
 * sizes, scale, pointers or alignment; UNSUPPORTED for D or L beyond the limits; WORKSPACE;
 * LAUNCH. Deterministic: every reduction runs in a fixed order.
 */
int attn_build_vslash_index(attn_tensor_t q, attn_tensor_t k, int B, int Hq, int Hkv, int L,
                            int D, float scale, int n_cols, int n_slash, int32_t* col_ptr,
                            int32_t* col_idx, int32_t* slash_ptr, int32_t* slash_idx,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Message of the last failed call on this thread ("" if none). Valid until the next call. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_AMD_ATTN_H_ */

/*
 * fa.h - exact IO-aware attention on one AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfa.so. Plain pointers and sizes only.
 *
 * The operation is exact scaled dot-product attention,
 *     O = softmax(scale * Q K^T) V,
 * computed tile by tile with the running row max / row sum rescaling of the
 * online softmax, so the N x N score matrix is never written to device
 * memory (marketmaker.cc article "Flash attention and the sequence-length
 * question", sections "Flash 注意力算法" (the algorithm, tiling into row and
 * column blocks) and "在线softmax递归" (online softmax recurrence); Ultralytics
 * glossary page "Flash Attention", section "Come funziona Flash Attention").
 * The forward keeps one number per query row for the backward, the natural
 * log-sum-exp LSE; the backward recomputes the probability tiles from Q, K
 * and LSE instead of storing them (marketmaker.cc article, section
 * "向后传递：重新计算而不是存储" (backward: recompute instead of store)).
 *
 * Common conventions
 *  - Tensors are dense, contiguous [B, H, N, d] with d innermost (the
 *    (batch, heads, seq, head_dim) shape of the marketmaker.cc article,
 *    section "集成是八行"). Every tensor pointer is a device pointer, 16-byte
 *    aligned. The caller owns every buffer; the library allocates no device
 *    memory and keeps no global mutable state, so calls are re-entrant.
 *  - d must be 64 or 128. B, H, N >= 0; a call with B*H*N == 0 returns
 *    FA_OK at once and does not inspect the pointers. One head's slab must
 *    be under 2 GiB at 4 bytes per element (N * d * 4 < 2^31, so
 *    N <= 4,194,303 at d = 128); larger N returns FA_ERR_UNSUPPORTED.
 *  - scale must be finite and > 0 (usually 1/sqrt(d)).
 *  - causal (0 or 1): key j is hidden from query i when j > i (top-left
 *    aligned; queries and keys share the length N). Key blocks wholly in a
 *    query block's future are skipped, never loaded (marketmaker.cc article,
 *    section "因果掩盖是交易获得折扣的地方" (causal masking)).
 *  - kv_len: NULL, or a device int32 array [B]; keys j >= kv_len[b] are
 *    hidden from every query row of every head of batch b. Values are
 *    clamped to [0, N]. Every query row is computed, padded ones included.
 *  - A query row with no visible key gets O = 0 and LSE = -inf (no NaN).
 *  - stream: a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued asynchronously; FA_OK means "enqueued". A device fault shows
 *    at the caller's next synchronisation. On the device side a call only
 *    launches kernels on that stream (no allocation, copy, memset or
 *    synchronisation), so it may be recorded under HIP stream capture. The
 *    only host memory a call reads is read during the call itself (the
 *    counts of the planned block-sparse calls, the mask of fa_sparse_plan).
 *  - Argument validation happens on the host before any HIP call, so every
 *    FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED / FA_ERR_WORKSPACE return has
 *    launched nothing.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, scale, flag */
  FA_ERR_UNSUPPORTED = -2, /* d not in {64,128}, or unsupported dtype pair */
  FA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than required */
  FA_ERR_HIP = -4,         /* the kernel launch itself failed */
  FA_ERR_TOO_LARGE = -5    /* problem exceeds fa_bwd_noalloc's built-in scratch */
} fa_status_t;

/*
 * Forward: O and LSE.
 *   q, k, v  [B,H,N,d] in in_dtype (FA_BF16, FA_F16 or FA_F32).
 *   o        [B,H,N,d] in o_dtype: in_dtype, or FA_F32 for bf16/fp16 inputs
 *            (an fp32 copy of the same kernel's output, used to judge
 *            accuracy apart from the output's own rounding).
 *   lse      [B,H,N] fp32: LSE_i = log(sum_j exp(scale * q_i . k_j)) over
 *            the visible keys j, natural log.
 * bf16/fp16 inputs run QK^T and PV on MFMA with fp32 accumulation; the
 * probabilities are rounded to the input type before PV. fp32 inputs are
 * computed entirely in fp32.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const int* kv_len, void* stream, int in_dtype, int o_dtype);

/*
 * Bytes of device workspace fa_bwd needs: one fp32 per query row
 * (D_i = sum_c dO_ic * O_ic), i.e. B*H*N*4. Returns 0 for negative sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward: dQ, dK, dV of L = sum(dO * O) for the forward above.
 *   q, k, v, dout     [B,H,N,d] in dtype.
 *   o                 [B,H,N,d] in o_dtype: dtype, or FA_F32 for 16-bit
 *                     inputs: the forward's output, in the type it was
 *                     written in. The backward forms D_i = sum_c dO_ic O_ic
 *                     from it, so an fp32 O keeps O's 16-bit rounding out
 *                     of D; that rounding is what limits dQ and dK on rows
 *                     with one or two visible keys, where dS = P (dP - D)
 *                     is a difference of nearly equal terms. Other o_dtype
 *                     values return FA_ERR_UNSUPPORTED.
 *   lse               [B,H,N] fp32 from fa_fwd with the same arguments.
 *   dq, dk, dv        [B,H,N,d] in dtype (written, not accumulated).
 *   workspace         device buffer of at least fa_bwd_workspace_bytes(),
 *                     16-byte aligned, owned by the caller; its contents on
 *                     entry are ignored. It receives D_i (see fa_bwd_dsum
 *                     below for how D_i is formed).
 * Deterministic: the same inputs give bit-identical gradients.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           const int* kv_len, void* workspace, size_t workspace_bytes,
           void* stream, int dtype, int o_dtype);

/*
 * The backward as its stages, for callers that want to time them. fa_bwd
 * enqueues exactly fa_bwd_dq, then fa_bwd_dkdv, on one stream. Arguments
 * mean what they mean for fa_bwd; dsum is the fp32 [B,H,N] array
 * D_i = sum_c dO_ic * O_ic (the workspace of fa_bwd).
 *   fa_bwd_dq:   reads q, k, v, o, dout, lse; writes dq and dsum (it forms
 *                D_i for its own rows; dsum 4-byte aligned).
 *   fa_bwd_dkdv: reads q, k, v, dout, lse, dsum; writes dk, dv. dsum must
 *                hold D_i, from fa_bwd_dq or fa_bwd_dsum, before it runs.
 *   fa_bwd_dsum: reads o, dout; writes dsum. D_i = rowsum(dO * O) on its
 *                own, for a caller that wants dK/dV without dQ. It sums in
 *                the order fa_bwd_dq does, so on every row that sees more
 *                than one 64-key tile either order of stages gives fa_bwd's
 *                bits. On a row whose visible keys lie in one 64-key tile
 *                fa_bwd_dq forms D_i instead as sum_j P_ij dP_ij from the P
 *                and dP it computes (equal in exact arithmetic, and free of
 *                O's rounding, which dominates dS = P (dP - D) on rows of
 *                one or two keys); fa_bwd_dsum cannot, having no Q, K, V.
 * Errors as for fa_bwd (no FA_ERR_WORKSPACE: dsum is a plain argument).
 */
int fa_bwd_dsum(const void* o, const void* dout, float* dsum, int B, int H,
                int N, int d, void* stream, int dtype, int o_dtype);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                const float* lse, const float* dsum, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                const int* kv_len, void* stream, int dtype);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, float* dsum, void* dq,
              int B, int H, int N, int d, float scale, int causal,
              const int* kv_len, void* stream, int dtype, int o_dtype);

/*
 * The backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * fa_bwd without the workspace argument. Its D_i array (one fp32 per query
 * row) lives in a fixed device array built into the library,
 * FA_NOALLOC_MAX_ROWS floats (16 MiB), which every device the library runs
 * on holds from the module's load until the process ends. The call
 * allocates nothing and launches the same kernels as fa_bwd, so its
 * results are fa_bwd's bit for bit.
 *   Arguments, results and errors as for fa_bwd, and:
 *   - B*H*N > FA_NOALLOC_MAX_ROWS returns FA_ERR_TOO_LARGE (nothing launched).
 *   - stream must be NULL or a stream of the current device, else
 *     FA_ERR_INVALID_ARG.
 *   - The first call on a device looks the array up (hipGetSymbolAddress)
 *     with that device current and keeps its address; a failed lookup
 *     returns FA_ERR_HIP.
 * Every call on one device shares that device's array and leaves its last
 * contents there; nothing in it needs to start at any value (each call
 * writes every D_i it reads). Calls that overlap on one device (different
 * streams, or several host threads without ordering) race on it; calls
 * ordered on one stream do not.
 */
#define FA_NOALLOC_MAX_ROWS (1 << 22)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk,
                   void* dv, int B, int H, int N, int d, float scale, int causal,
                   const int* kv_len, void* stream, int dtype, int o_dtype);

/*
 * Attention over part of the keys, and the merge of such parts: the pieces
 * of ring attention (Ultralytics glossary page "Flash Attention", section
 * "Flash Attention e termini correlati": each device keeps its query block
 * and visits the others' key/value blocks) and of a key-split forward. A
 * part's result is exact attention over its keys; parts over disjoint key
 * sets combine exactly by the online-softmax recurrence (marketmaker.cc
 * article, section "在线softmax递归") applied to whole results:
 *     m = max_p LSE_p,  w_p = exp(LSE_p - m),
 *     O = sum_p w_p O_p / sum_p w_p,  LSE = m + ln sum_p w_p.
 * These entry points take fp16/bf16 inputs only (FA_F32 inputs return
 * FA_ERR_UNSUPPORTED); partial results are fp32.
 *
 * fa_fwd_partial: queries q [B,H,Nq,d] at global positions q_pos0 + i,
 * keys k, v [B,H,Nk,d] at global positions k_pos0 + j. With causal = 1 a
 * key is hidden when its position is after the query's (k_pos0 + j >
 * q_pos0 + i); kv_len (NULL or device int32 [B]) hides local keys
 * j >= kv_len[b]. Writes o_part fp32 [B,H,Nq,d] (normalised over the part's
 * visible keys) and lse_part fp32 [B,H,Nq]; a row with no visible key in
 * the part gets 0 and -inf. Nq, Nk >= 0 (Nk = 0 gives every row 0 / -inf,
 * and k, v may then be NULL),
 * |q_pos0|, |k_pos0| < 2^29 (else FA_ERR_INVALID_ARG), Nk * d * 4 < 2^31.
 * B*H*Nq == 0 returns FA_OK at once.
 */
int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                   float* lse_part, int B, int H, int Nq, int Nk, int d,
                   float scale, int causal, int q_pos0, int k_pos0,
                   const int* kv_len, void* stream, int in_dtype);

/*
 * fa_merge: out = merge(a, b) for `rows` rows of d (64 or 128) elements:
 * o_a, o_b fp32 [rows, d]; lse_a, lse_b fp32 [rows] (-inf marks an empty
 * part); o [rows, d] in o_dtype (FA_F32, FA_F16 or FA_BF16) and lse fp32
 * [rows]. With o_dtype = FA_F32, o and lse may be o_a and lse_a (an
 * accumulator merged in place, as a ring step does); otherwise outputs must
 * not overlap the inputs. rows == 0 returns FA_OK at once.
 */
int fa_merge(const float* o_a, const float* lse_a, const float* o_b,
             const float* lse_b, void* o, float* lse, long long rows, int d,
             void* stream, int o_dtype);

/*
 * Key-split forward: the same O and LSE as fa_fwd (same arguments and
 * conventions), computed as num_splits (1..16) parts over consecutive key
 * ranges, one launch for all parts, then one merge launch. Splitting gives
 * a short, wide problem (few heads, or B = 1) more workgroups to run.
 * Keys are split in runs of ceil(N / num_splits) rounded up to a multiple
 * of 64; fewer parts are used when the runs cover N sooner (one part runs
 * fa_fwd's path and needs no workspace). The workspace holds the parts:
 * fa_fwd_split_workspace_bytes(B, H, N, d, num_splits) bytes, 16-byte
 * aligned, owned by the caller, contents on entry ignored.
 */
size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int num_splits);
int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal,
                 const int* kv_len, int num_splits, void* workspace,
                 size_t workspace_bytes, void* stream, int in_dtype, int o_dtype);

/*
 * Grouped-query attention: H query heads share Hkv key/value heads, query
 * head h of a batch using K/V head h / (H / Hkv). The tiled computation is
 * unchanged by how many K/V heads there are (delect.ru glossary page
 * "FlashAttention", section "Что подтверждено"); each query head's result
 * is plain attention against its K/V head, so Hkv == H is fa_fwd / fa_bwd.
 *   q, o, dout, dq  [B,H,N,d];  k, v, dk, dv  [B,Hkv,N,d];  lse [B,H,N].
 *   Hkv >= 1 and H % Hkv == 0, else FA_ERR_INVALID_ARG.
 * dK and dV of a K/V head are the sums over its H / Hkv query heads, in
 * fp32, rounded once to dtype. When B * Hkv is too small to fill the chip,
 * a group's query heads are shared among several workgroups that write
 * fp32 partial sums to the workspace, added in a fixed order by a second
 * launch; the result is deterministic either way. The workspace of
 * fa_bwd_gqa is fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d) bytes (0 for
 * invalid sizes), 16-byte aligned, owned by the caller, contents on entry
 * ignored. Everything else is as for fa_fwd / fa_bwd. fp16/bf16 only
 * (FA_F32 returns FA_ERR_UNSUPPORTED).
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               const int* kv_len, void* stream, int in_dtype, int o_dtype);
size_t fa_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d);
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               const int* kv_len, void* workspace, size_t workspace_bytes,
               void* stream, int dtype, int o_dtype);

/*
 * Block-sparse attention: attention restricted to the (query block, key
 * block) pairs a block mask keeps; the tiles of dropped blocks are never
 * loaded or computed. The pages present this as a separate variant that
 * approximates full attention (Ultralytics glossary page "Flash
 * Attention", section "Flash Attention e termini correlati"; delect.ru
 * glossary page "FlashAttention", section "Что подтверждено"). On the kept
 * pairs the result is exact: key j is visible to query i when the mask
 * keeps block pair (i / 128, j / 128) and kv_len and causal (as for fa_fwd)
 * allow it; a row with no visible key gets O = 0, LSE = -inf and zero
 * gradients.
 *   block_mask  device uint8; entry (b, h, I, J) at
 *               block_mask[b * mask_stride_b + h * mask_stride_h + I * nb + J],
 *               nb = ceil(N / 128), blocks of 128 queries by 128 keys;
 *               nonzero keeps the pair. Strides are element counts >= 0 (0
 *               shares one mask among batches or heads).
 * Other arguments and the workspace (fa_bwd_workspace_bytes) are as for
 * fa_fwd / fa_bwd. fp16/bf16 only (FA_F32 returns FA_ERR_UNSUPPORTED).
 * nb <= 4096 (N <= 524288), else FA_ERR_UNSUPPORTED; a NULL mask or a
 * negative stride returns FA_ERR_INVALID_ARG.
 */
int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal,
                  const int* kv_len, const unsigned char* block_mask,
                  long long mask_stride_b, long long mask_stride_h, void* stream,
                  int in_dtype, int o_dtype);
int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  int B, int H, int N, int d, float scale, int causal,
                  const int* kv_len, const unsigned char* block_mask,
                  long long mask_stride_b, long long mask_stride_h, void* workspace,
                  size_t workspace_bytes, void* stream, int dtype, int o_dtype);

/*
 * Block-sparse attention with long mask lines cut into pieces. In
 * fa_fwd_sparse one workgroup computes a query block over every kept key
 * block of its mask row, and in fa_bwd_sparse one workgroup computes a key
 * block's dK, dV over every kept query block of its mask column (and one a
 * query block's dQ over its row), so a line with many kept blocks (a global
 * token, the first block of a sink pattern) is one long serial job.
 * fa_sparse_plan reads a HOST copy of the mask (same layout and strides as
 * the device mask) and cuts every line with more than 8 kept blocks into
 * pieces of at most 8, longest first: columns count the query blocks from
 * the diagonal on when causal, rows the key blocks up to the diagonal.
 * The planned entry points run one workgroup per piece; pieces of a cut
 * line write fp32 partial results to the workspace and a second launch
 * combines them in piece order (deterministic): partial O with its LSE for
 * the forward (rescaled to the common maximum, the online-softmax merge),
 * partial sums for dK, dV and dQ. Lines that are not cut are written as by
 * fa_fwd_sparse / fa_bwd_sparse, bit for bit.
 *   fa_sparse_plan: counts[8] = {column items, cut columns, column slots,
 *   row items, cut rows, row slots, 0, 0}; with plan NULL only the counts,
 *   else plan (int32, plan_ints entries) holds the column items, the cut
 *   columns, the row items and the cut rows in that order, 4 ints each
 *   (FA_ERR_INVALID_ARG if plan_ints is smaller than 4 x the sum of counts
 *   0, 1, 3, 4). Host memory only, no HIP call.
 *   fa_fwd_sparse_planned / fa_bwd_sparse_planned: the arguments of
 *   fa_fwd_sparse / fa_bwd_sparse plus the plan copied to device memory
 *   (4-byte aligned) and the host array counts; workspace of
 *   fa_{fwd,bwd}_sparse_planned_workspace_bytes(B, H, N, d, counts) bytes
 *   (the forward needs none when no row is cut). The plan must come from
 *   the same mask, strides, B, H, N and causal: it is not checked on the
 *   device.
 */
int fa_sparse_plan(const unsigned char* host_mask, long long mask_stride_b,
                   long long mask_stride_h, int B, int H, int N, int causal, int* plan,
                   long long plan_ints, int* counts);
size_t fa_fwd_sparse_planned_workspace_bytes(int B, int H, int N, int d, const int* counts);
int fa_fwd_sparse_planned(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal,
                          const int* kv_len, const unsigned char* block_mask,
                          long long mask_stride_b, long long mask_stride_h,
                          const int* plan, const int* counts, void* workspace,
                          size_t workspace_bytes, void* stream, int in_dtype, int o_dtype);
size_t fa_bwd_sparse_planned_workspace_bytes(int B, int H, int N, int d, const int* counts);
int fa_bwd_sparse_planned(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk,
                          void* dv, int B, int H, int N, int d, float scale, int causal,
                          const int* kv_len, const unsigned char* block_mask,
                          long long mask_stride_b, long long mask_stride_h,
                          const int* plan, const int* counts, void* workspace,
                          size_t workspace_bytes, void* stream, int dtype, int o_dtype);

/*
 * FP8 forward with incoherent processing (marketmaker.cc article, section
 * "FA3：料斗力学", item 3: FP8 attention is spoiled by outliers, so the
 * vectors are rotated at random before a block-wise quantisation, which
 * spreads an outlier over all coordinates). An approximation of the
 * attention above; two steps:
 *
 * fa_fp8_quantize: every row of q and k is multiplied elementwise by
 * signs (device int8 [d], entries +1 or -1; NULL = no rotation) and put
 * through the unnormalised Walsh-Hadamard transform in fp32, then
 * quantised to OCP FP8 e4m3 (bias 7, largest 448): one fp32 scale per block
 * of 128 query rows (q_scale [B,H,ceil(N/128)]) and of 64 key rows
 * (k_scale [B,H,ceil(N/64)]), scale = amax / 448, code = round-to-nearest-
 * even of clamp(x * (448 / amax), -448, 448) (all in fp32; an all-zero
 * block has scale 0 and zero codes). V is not rotated: one scale per head
 * (v_scale [B,H]), codes stored transposed in vt8 [B,H,d,Np], Np = N
 * rounded up to 64, zero codes in the padding. q8, k8: [B,H,N,d] codes.
 * v_amax: device scratch of B*H*ceil(N/64) floats. q, k, v fp16/bf16.
 *
 * fa_fwd_fp8: attention on those codes, S and P V on the FP8 matrix cores
 * with fp32 accumulation, online softmax in fp32; P is quantised to e4m3
 * as 256 p per 64-key tile against the running row max, the running sum
 * adds the unquantised p. rotated (0 or 1) says whether the codes come
 * from a rotation (the scores then carry 1/d, the rotation's factor).
 * Writes o [B,H,N,d] in o_dtype (FA_F32, FA_F16, FA_BF16) and lse [B,H,N]
 * as fa_fwd does; scale, causal and kv_len as for fa_fwd.
 *
 * fa_fwd_fp8_incoherent: both steps on one stream with the codes and
 * scales in a caller-owned workspace of fa_fwd_fp8_workspace_bytes() bytes
 * (16-byte aligned, contents on entry ignored); o_dtype is in_dtype or
 * FA_F32. signs NULL runs the same path without the rotation.
 * Errors as for fa_fwd; code buffers 16-byte aligned, scales 4-byte.
 */
int fa_fp8_quantize(const void* q, const void* k, const void* v,
                    const signed char* signs, unsigned char* q8,
                    unsigned char* k8, unsigned char* vt8, float* q_scale,
                    float* k_scale, float* v_scale, float* v_amax, int B,
                    int H, int N, int d, void* stream, int in_dtype);
int fa_fwd_fp8(const unsigned char* q8, const unsigned char* k8,
               const unsigned char* vt8, const float* q_scale,
               const float* k_scale, const float* v_scale, int rotated,
               void* o, float* lse, int B, int H, int N, int d, float scale,
               int causal, const int* kv_len, void* stream, int o_dtype);
size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N, int d);
int fa_fwd_fp8_incoherent(const void* q, const void* k, const void* v,
                          const signed char* signs, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal,
                          const int* kv_len, void* workspace,
                          size_t workspace_bytes, void* stream, int in_dtype,
                          int o_dtype);

/* Static, human-readable text for a status code. Never NULL. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

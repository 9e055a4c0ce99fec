/*
 * fa.h — C ABI of the gfx950 (MI355X) exact tiled attention library, libfa.so.
 *
 * The library computes exact softmax attention
 *
 *     O = softmax(scale * Q K^T  [+ causal or block-sparse mask]) V
 *
 * tile by tile with the online softmax, so the N x N score matrix never
 * reaches device memory. The forward pass writes only O and the per-row
 * log-sum-exp; the backward pass recomputes the probabilities block by block
 * from Q, K, V and that log-sum-exp.
 *
 * Passages that define the operations (page title, then section):
 *   - "FlashAttention: exact attention made fast by counting memory traffic",
 *     "The method": tiling with running row statistics, exact result,
 *     backward by recomputation from the output and the statistics, and the
 *     block-sparse extension.
 *   - "FlashAttention and IO-aware exact attention", "Core ideas": online
 *     softmax, tiling and fusion with one log-sum-exp kept per row, backward
 *     by recomputation; "How to approach it": causal masking.
 *   - "Flash Attention — Revolutionizing Transformer Efficiency Through
 *     Memory-Aware Algorithms", "The Memory Wall Problem" ([N, d] operands,
 *     S = QK^T, softmax, O = PV) and "Online Softmax Algorithm".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory. Every tensor pointer is DEVICE memory owned by the caller; the
 *   library never allocates, frees or keeps a pointer after a call returns.
 * Layout. q, k, v, o, dO, dq, dk, dv are contiguous [B, H, N, d] row-major
 *   arrays (d fastest), in the element type `dtype` (FA_BF16: bfloat16 bits;
 *   FA_F32: IEEE float). lse and the backward's row term are float [B, H, N].
 * lse. Natural log of sum_j exp(scale * q_i . k_j) over the keys j visible to
 *   query i; -inf for a row with no visible key (its O row is 0).
 * Masks. FA_MASK_NONE: every key visible. FA_MASK_CAUSAL: key j visible to
 *   query i iff j <= i (query and key sequences both have length N).
 *   FA_MASK_BLOCK_SPARSE: block_mask is a device uint8 array of
 *   ceil(N/128) x ceil(N/128) entries, row-major (query block, key block),
 *   nonzero = keep; one mask is shared by every (batch, head); the masks are
 *   not combined. block_mask is read only for FA_MASK_BLOCK_SPARSE and may
 *   be NULL otherwise. The library never reads mask contents on the host.
 * Supported. d in {64, 128}; dtype FA_BF16 (bf16 in and out, fp32
 *   accumulation, probabilities rounded to bf16 before the P.V product) or
 *   FA_F32 (fp32 throughout). Any finite scale, including negative and 0.
 * Errors. Arguments are validated on the host before anything is enqueued;
 *   on any error a negative fa_status is returned and no output is touched.
 *   Tensor pointers must be 16-byte aligned, lse 4-byte aligned. Outputs must
 *   not overlap inputs or each other. FA_OK means the work was enqueued on
 *   `stream` (asynchronous); FA_ERR_HIP means a launch failed (the HIP error
 *   is not cleared). A device fault surfaces at the caller's next
 *   synchronisation.
 * State. No global mutable state besides fa_bwd_noalloc's library-owned
 *   scratch array per GPU and the debug switch fa_debug_reverse_order (an
 *   atomic flag read when a call builds its launch); calls are thread-safe.
 *   Results are bitwise deterministic from run to run (no atomics), and do
 *   not depend on the debug switch.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* B, H or N < 1, or the element count overflows */
  FA_ERR_UNSUPPORTED = -3, /* d not in {64, 128}, a dtype the call does not take, too many split-key rows, or an unknown tile height */
  FA_ERR_MASK = -4,        /* unknown mask_kind, or block_mask NULL for a block-sparse call */
  FA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_ALIGN = -6,       /* a pointer is not aligned as stated above */
  FA_ERR_HIP = -7,         /* a kernel launch returned a HIP error */
  FA_ERR_ARG = -8,         /* non-finite scale, or an output overlaps another tensor */
  FA_ERR_SCRATCH = -9      /* fa_bwd_noalloc: B * H * N exceeds FA_BWD_NOALLOC_MAX_ROWS */
} fa_status;

typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_BLOCK_SPARSE = 2 } fa_mask_kind;
typedef enum { FA_BF16 = 0, FA_F32 = 1 } fa_dtype;

/*
 * Forward pass. Reads q, k, v [B,H,N,d]; writes o [B,H,N,d] and lse [B,H,N].
 * Each workgroup keeps one tile of queries resident and streams the visible
 * key/value tiles through on-chip memory with the online softmax ("The
 * method"; "Core ideas": online softmax, tiling and fusion).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale,
           int mask_kind, const uint8_t* block_mask, int dtype, hipStream_t stream);

/*
 * fa_fwd with the query-tile height chosen by the caller. The block size sets
 * the HBM traffic: every workgroup of block_rows queries streams the key/value
 * tiles its rows see, so K/V reads fall as 1 / block_rows while the on-chip
 * footprint grows ("FlashAttention: exact attention made fast by counting
 * memory traffic", "The decisive evidence": Fig. 2, runtime against block
 * size; "The method": Theorem 2). Exists to measure that trade-off; results
 * equal fa_fwd's up to summation order.
 *   block_rows  0 (fa_fwd's own choice), or 32, 64, 128 or 256 query rows per
 *               workgroup (one to eight 64-wide waves; 64 keys per tile).
 * bf16 only for block_rows != 0. FA_ERR_UNSUPPORTED for another value, for fp32
 * with block_rows != 0, and for 256 with the block-sparse mask (a workgroup's
 * queries must stay inside one 128-row mask block). Otherwise as fa_fwd.
 */
int fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale,
                 int mask_kind, const uint8_t* block_mask, int dtype, int block_rows, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: two float arrays with one entry per
 * query row (b, h, i), each rounded up to 256 bytes: the row term
 * D_i = sum_k dO_ik O_ik and a rescaled copy of the LSE that the loops use.
 * Returns 0 if the shape is invalid.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass. Reads q, k, v, o, lse (as written by fa_fwd with the same
 * arguments) and dO; writes dq, dk, dv [B,H,N,d]. Probabilities are
 * recomputed tile by tile from q, k and lse ("The method": backward by
 * recomputation; "Core ideas": backward by recomputation). The gradient
 * formulas are the derivative of the forward definition:
 *   dV = P^T dO; dP = dO V^T; D = rowsum(dO * O); dS = P * (dP - D);
 *   dQ = scale dS K; dK = scale dS^T Q.
 * Three kernels run in order on `stream`: the row term, then dK/dV (one
 * workgroup per key tile), then dQ (one workgroup per query tile); under a
 * causal mask over a dense batch a workgroup takes a pair of tiles whose
 * work adds up evenly.
 * workspace: caller-owned device memory of at least
 * fa_bwd_workspace_bytes(B, H, N, d) bytes, 16-byte aligned; its contents
 * on entry are ignored and on exit are unspecified.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale,
           int mask_kind, const uint8_t* block_mask, int dtype,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The three steps fa_bwd enqueues, callable one by one with the same
 * arguments and the same validation (arguments a step does not use are not
 * taken). fa_bwd_rowterm writes the row term D and the rescaled LSE into the
 * workspace;
 * fa_bwd_dkdv and fa_bwd_dq each read it and are independent of each other,
 * so they may run on two streams once the row term is complete.
 * workspace has the size and alignment fa_bwd requires; for fa_bwd_dkdv and
 * fa_bwd_dq its contents must be those fa_bwd_rowterm left.
 */
int fa_bwd_rowterm(const void* o, const void* dO, const float* lse, int B, int H, int N, int d, int dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                void* dk, void* dv, int B, int H, int N, int d, float scale,
                int mask_kind, const uint8_t* block_mask, int dtype,
                const void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
              void* dq, int B, int H, int N, int d, float scale,
              int mask_kind, const uint8_t* block_mask, int dtype,
              const void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Packed variable-length batches, unequal query and key lengths, and K/V
 * heads shared by groups of query heads (multi-query and grouped-query
 * attention). Passages: "Flash Attention — Revolutionizing Transformer
 * Efficiency Through Memory-Aware Algorithms", "Flash Attention 2 (2023)"
 * (variable sequence lengths; multi-query and grouped-query attention);
 * "Flash Attention: Speeding Up LLM Inference and Training", "Implementation:
 * Is It Hard to Adopt?" (ragged batches without padding). Each sequence is
 * the attention problem defined above on its own tokens.
 *
 * Layout. q, o, dO, dq: [total_q, H, d]; k, v, dk, dv: [total_k, Hkv, d]
 *   (token-major, d fastest), bfloat16. lse and the backward's row term:
 *   float [H, total_q].
 * Sequences. cu_seqlens_q and cu_seqlens_k are DEVICE int32 arrays of B + 1
 *   non-decreasing token offsets, the first >= 0, the last <= total_q
 *   (total_k). Sequence b owns query tokens [cu_seqlens_q[b],
 *   cu_seqlens_q[b+1]) (nq_b of them) and key tokens [cu_seqlens_k[b],
 *   cu_seqlens_k[b+1]) (nk_b). max_seqlen_q >= every nq_b and
 *   max_seqlen_k >= every nk_b: they size the launch, since the library does
 *   not read the offsets on the host. Offsets outside this contract are
 *   clamped on the device, so no access leaves the tensors, but that
 *   sequence's results are unspecified.
 * Heads. H query heads, Hkv key/value heads, H a multiple of Hkv; query
 *   head h reads K/V head h / (H / Hkv) (Hkv = H: multi-head; Hkv = 1:
 *   multi-query). dk and dv of a K/V head sum the contributions of its
 *   H / Hkv query heads.
 * Causal. Key j of a sequence is visible to its query i iff
 *   j <= i + nk_b - nq_b: the last query sees every key; with nq_b > nk_b the
 *   first nq_b - nk_b queries see none (O row 0, lse -inf, no gradient).
 *   With nq_b = nk_b this is the causal mask of the dense calls.
 * Supported. dtype FA_BF16 only (FA_F32 returns FA_ERR_UNSUPPORTED);
 *   mask_kind FA_MASK_NONE or FA_MASK_CAUSAL (FA_MASK_BLOCK_SPARSE returns
 *   FA_ERR_MASK); d in {64, 128}; 1 <= H <= 65536.
 * Untouched rows. Query-token rows of o, lse and dq, and key-token rows of dk
 *   and dv, that belong to no sequence are not written. Key tokens of a
 *   sequence with no queries get dk = dv = 0.
 * Errors, alignment (cu_seqlens 4-byte aligned), overlap rules and
 *   asynchrony are those of the dense calls; FA_ERR_SHAPE also covers
 *   B, H, Hkv, max_seqlen or total < 1 and H not a multiple of Hkv.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                  int total_q, int total_k, int d, float scale, int mask_kind,
                  int dtype, hipStream_t stream);

/* Workspace bytes fa_bwd_varlen needs (two float arrays [H, total_q], the
 * row term and the rescaled LSE, each rounded up to 256 bytes); 0 for an
 * invalid shape. */
size_t fa_bwd_varlen_workspace_bytes(int total_q, int H, int d);

/*
 * Backward of fa_fwd_varlen: reads q, k, v, o, lse (as fa_fwd_varlen wrote
 * them) and dO; writes dq [total_q, H, d], dk and dv [total_k, Hkv, d]. The
 * same three kernels as fa_bwd run in order on `stream`; workspace is
 * caller-owned device memory of at least fa_bwd_varlen_workspace_bytes()
 * bytes, 16-byte aligned, contents ignored on entry.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dO, void* dq, void* dk, void* dv,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                  int total_q, int total_k, int d, float scale, int mask_kind, int dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Split-key forward for packed batches with few queries per sequence against
 * long key sequences (decoding). Computes exactly what fa_fwd_varlen computes
 * (same layouts, heads, masks, outputs and untouched rows), organised for
 * this shape: one workgroup per (K/V head, sequence, key range) stacks the
 * queries of all H / Hkv query heads that read the K/V head, so each K/V tile
 * is read once per group, and the key range of every sequence is split over
 * `splits` workgroups. Each range's partial result is normalised over that
 * range and merged afterwards with the block-combine rule of "Flash
 * Attention — Revolutionizing Transformer Efficiency Through Memory-Aware
 * Algorithms", "Mathematical Correctness" (a row's exponential sum is the
 * sum of the blocks' sums, each scaled by exp(block max - overall max)):
 *   LSE = max_s LSE_s + ln sum_s exp(LSE_s - max_s LSE_s),
 *   O = sum_s exp(LSE_s - LSE) O_s.
 * Rounding differs from fa_fwd_varlen (fp32 partials are merged before the
 * single rounding of O to bf16).
 *
 * Limits. (H / Hkv) * max_seqlen_q <= 128, else FA_ERR_UNSUPPORTED; the other
 *   limits and status codes are those of fa_fwd_varlen.
 * Splits. num_splits = 0 lets the library choose; 1..128 forces a count;
 *   anything else is FA_ERR_ARG. fa_splitkv_splits returns the count a call
 *   with these arguments uses (or a negative status).
 * Workspace. Caller-owned device memory, 16-byte aligned, of at least
 *   fa_splitkv_workspace_bytes(total_q, H, d, splits) bytes (fp32 partial O
 *   and LSE of every range); contents ignored on entry, unspecified on exit.
 *   Two calls in flight at once need separate workspaces.
 */
int fa_splitkv_splits(int B, int Hkv, int max_seqlen_k, int num_splits);
size_t fa_splitkv_workspace_bytes(int total_q, int H, int d, int splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int* cu_seqlens_q, const int* cu_seqlens_k,
                   int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                   int total_q, int total_k, int d, float scale, int mask_kind, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 forward: the forward pass on 8-bit floating-point inputs, the variant
 * "Flash Attention — Revolutionizing Transformer Efficiency Through
 * Memory-Aware Algorithms", "Flash Attention 3 (2024)" lists (FP8 support),
 * on the gfx950 FP8 matrix instructions (twice the bf16 rate).
 *
 * Inputs. q, k: [B, H, N, d] bytes; v_t: V transposed, [B, H, d, ldv] bytes
 *   (v_t[b][h][j][n] = V[b][h][n][j]; columns N .. ldv-1 are padding and may
 *   hold anything). Every byte is an OCP E4M3 code (1 sign, 4 exponent bits
 *   with bias 7, 3 mantissa bits; largest finite 448; S.1111.111 is NaN). The
 *   represented tensors are Q = q_descale * q, K = k_descale * k,
 *   V = v_descale * v.
 * Outputs. o: bf16 [B, H, N, d]; lse: float [B, H, N], as for fa_fwd with
 *   the represented tensors.
 * Arithmetic. Scores are exact products of the codes accumulated in fp32,
 *   times scale * q_descale * k_descale. The probabilities are rounded to
 *   E4M3 for the P.V product; the row sums and the LSE use them unrounded.
 * Supported. d in {64, 128}; mask_kind FA_MASK_NONE or FA_MASK_CAUSAL
 *   (N_q = N_k); ldv >= N and a multiple of 16; finite scale and descale
 *   factors whose product is finite.
 * Errors. As for fa_fwd: FA_ERR_NULL, FA_ERR_SHAPE (also a bad ldv),
 *   FA_ERR_UNSUPPORTED (d), FA_ERR_MASK (block-sparse or unknown),
 *   FA_ERR_ARG (non-finite factor, overlapping output), FA_ERR_ALIGN
 *   (q, k, v_t, o 16-byte, lse 4-byte), FA_ERR_HIP.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v_t, void* o, float* lse,
               int B, int H, int N, int d, int ldv, float scale,
               float q_descale, float k_descale, float v_descale, int mask_kind, hipStream_t stream);

/* Static, human-readable name of a fa_status value ("unknown status" otherwise). */
const char* fa_status_string(int status);

/*
 * Debugging aid, not part of the method: while on != 0, every kernel launched
 * by a later call of this library takes its workgroups' work items (query or
 * key tiles, heads, sequences) in the reverse of the usual order. Each work
 * item (a tile, or a causal pair of tiles) is computed by one workgroup with
 * no atomics and no communication between workgroups, so results must be
 * bitwise identical in both orders;
 * a difference points at a race (e.g. an LDS buffer reused too early). The
 * setting is process-wide and takes effect at the next call. Returns the
 * previous setting (0 or 1). Never fails.
 */
int fa_debug_reverse_order(int on);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code recorded into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc. It computes exactly what fa_bwd computes
 * (the same three kernels, bitwise the same dq, dk, dv) and allocates
 * nothing: the row term and the rescaled LSE that fa_bwd keeps in the
 * caller's workspace go to a scratch array inside the library's device code,
 * one copy per GPU, allocated when the library's code is loaded on that GPU
 * and held until the process ends. Its address on the current device is
 * looked up once per device, on that device's first call.
 *   Limit. B * H * N <= FA_BWD_NOALLOC_MAX_ROWS (2^21 query rows, 16 MiB of
 *   scratch); larger problems return FA_ERR_SCRATCH (checked before any
 *   other argument) and nothing is enqueued (use fa_bwd with a workspace).
 *   Sharing. Every call on one GPU uses that GPU's single scratch array, and
 *   each call overwrites every entry it reads before reading it. Calls that
 *   can overlap in time on one GPU (other streams, other threads) race on
 *   the array and must be serialised by the caller.
 * Arguments, layout, validation and the other errors are those of fa_bwd;
 * FA_ERR_HIP also covers a failed lookup of the scratch address.
 */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 21)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale,
                   int mask_kind, const uint8_t* block_mask, int dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

/*
 * bsm.h -- C ABI of the block-sparse masked attention library for MI355X
 * (gfx950). One shared library, libbsm.so; every entry point below is
 * extern "C", takes plain pointers and sizes, and enqueues its work on the
 * caller's HIP stream.
 *
 * Sources (cited by title and section):
 *   [SF-452]  SpecForge issue #452, "flex_attention BlockMask incorrectly created
 *             with H=num_heads" -- traceback (create_block_mask returns a partial
 *             and a full block part), Problem, Expected Behavior (one head-shared
 *             block mask).
 *   [SF-905]  SpecForge PR #905, "Fix DFlash attention masking" -- Motivation
 *             (is_causal x layer-type rule), maintainer reply item #934
 *             (resolve_dflash_is_causal, left-bound-only in-block window).
 *   [SF-474]  SpecForge issue #474, "DFlash block mask currently relies on Flex
 *             Attention only" -- Suggestion 2 (dense [B,1,Q_LEN,KV_LEN] bool mask).
 *   [FSA-190] flash-sparse-attention PR #190, "Broadcastable 4D mask/bias,
 *             128-rounded key length, stride-0 broadcasting, and dbias
 *             reductions" -- Design, Changes (mha_fwd validation), Implementation
 *             Notes (swapped path, stability fix).
 *   [FSA-197] flash-sparse-attention PR #197, "Centralize dynamic mask creation
 *             for FDMA" -- Design, Changes, Implementation Notes, review
 *             suggestion on dynamic_mask.
 *
 * Conventions shared by all entry points
 *   Layout. Q is (B, Sq, H, D); K and V are (B, Sk, KVH, D); O is (B, Sq, H, D);
 *     all with element strides and the last dimension contiguous. LSE is float
 *     (B, H, Sq), contiguous. G = H / KVH; the KV head of head h is h / G.
 *   Aux tensors (mask, bias) are 4D: ({B|1}, {H|KVH|1}, {Sq|1}, K_round) with
 *     K_round = round_multiple(Sk, 128) = (Sk + 127) / 128 * 128, last dim
 *     contiguous ([FSA-190] Design). A size-1 dim broadcasts and its stride is
 *     ignored (read as 0); a stride of 0 on a dim of size > 1 is rejected (no
 *     implicit expand, [FSA-190] Changes). Keys >= Sk are never kept, whatever
 *     the tail of a mask or bias holds ([FSA-190] Implementation Notes).
 *     Mask: 1 byte per element, nonzero = keep. Bias: additive, unscaled, same
 *     dtype as Q. Mask and bias rows must start 16-byte aligned.
 *   Tiles. 128 queries x 128 keys. nQ = ceil(Sq / 128), nK = K_round / 128.
 *   Swap. When Sq == 1 and H > KVH, the library runs the head-group swap of
 *     [FSA-190] Design / Implementation Notes: the H heads of one KV group are
 *     treated as G query rows of KV head kvh, by views only. build_block_mask
 *     and masked_attn_fwd both apply it, so a block mask always lives in the
 *     iteration space of the attention kernel; block_mask_shape reports it.
 *   Ownership. The caller allocates every device buffer; the library allocates
 *     no device memory and keeps no state except a thread-local error string
 *     and the static scratch array of masked_attn_fwd_noalloc (below).
 *     Work is enqueued on `stream` with no host synchronisation, so inputs and
 *     outputs must stay alive until that stream's work completes.
 *   Errors. Every entry point returns 0 (BSM_OK) or a negative bsm_status. On a
 *     validation error nothing is enqueued and no output is touched;
 *     bsm_last_error() then describes the failure. BSM_E_HIP reports a failed
 *     kernel launch on the caller's stream.
 */
#ifndef BSM_H
#define BSM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSM_OK = 0,
  BSM_E_ARG = -1,         /* bad scalar argument or NULL pointer */
  BSM_E_SHAPE = -2,       /* sizes violate the 4D / GQA / DFlash contract */
  BSM_E_STRIDE = -3,      /* non-contiguous last dim, illegal 0 stride, misalignment */
  BSM_E_DTYPE = -4,       /* dtype not allowed for this argument */
  BSM_E_UNSUPPORTED = -5, /* valid request outside what the library implements */
  BSM_E_HIP = -6          /* HIP launch error */
} bsm_status;

typedef enum {
  BSM_BOOL = 0, /* 1 byte per element, nonzero = keep */
  BSM_BF16 = 1,
  BSM_F32 = 2
} bsm_dtype;

/* A 4D device tensor view: element sizes and element strides. */
typedef struct {
  const void* data;
  int32_t dtype;     /* bsm_dtype */
  int32_t reserved;  /* must be 0 */
  int64_t size[4];
  int64_t stride[4];
} bsm_tensor4;

typedef struct {
  int64_t B, H, KVH, Sq, Sk, D;
} bsm_geom;

/* DFlash draft-block predicate ([SF-452] Problem; [SF-905] Motivation, #934).
 * Keys: ctx_len C context tokens, then num_blocks NB draft blocks of
 * block_size bs tokens (Sk = C + NB*bs). Queries: the NB*bs draft tokens.
 * Draft block j sees context keys k < E_j = clamp((j+1)*S + ctx_end_offset, 0, C)
 * with S = ctx_per_block (0 -> C / NB, which requires C % NB == 0), and the
 * draft tokens of its own block (token i sees i' <= i if in-block attention is
 * causal). is_causal: -1 absent, 0, 1; layer_type: 0 full-attention,
 * 1 sliding-attention. Causality = resolve_dflash_is_causal(is_causal,
 * layer_type). On sliding layers a key is visible only if
 * pos_q - pos_k < sliding_window (left bound only), with pos(context c) = c and
 * pos(draft token i of block j) = E_j + i. The mask is the same for every batch
 * entry and head. Inference (the default mask of spec_generate, [SF-905]
 * Modifications, #935): one block drafted after ctx_len cached tokens is
 * num_blocks = 1 with ctx_per_block = ctx_len, so it sees the whole cache. */
typedef struct {
  int64_t ctx_len, num_blocks, block_size, ctx_per_block, ctx_end_offset;
  int32_t is_causal;
  int32_t layer_type;
  int64_t sliding_window;
} bsm_dflash;

/* Block mask ([SF-452] traceback: partial and full block parts). Four int32
 * device arrays: kv_num_blocks / full_kv_num_blocks of shape (Bm, Hm, nQm),
 * kv_indices / full_kv_indices of shape (Bm, Hm, nQm, nK), contiguous.
 * For query tile qt, kv_indices lists the partial key tiles (some but not all
 * pairs kept) and full_kv_indices the full ones (all pairs kept), ascending,
 * padded with -1. Tiles in neither list are empty and never visited. */
typedef struct {
  int32_t* kv_num_blocks;
  int32_t* kv_indices;
  int32_t* full_kv_num_blocks;
  int32_t* full_kv_indices;
  int64_t Bm, Hm, nQm, nK;
} bsm_block_mask;

/* Kept-key list of a dense mask over a short query block: at most 32 rows per
 * (b, h) in the attention's iteration space, as under the seqlen_q == 1
 * head-group swap ([FSA-190] Design), where the rows are the G heads of a KV
 * group. For a dynamic top-k mask ([FSA-197] Design: window_size keys kept per
 * row) the union over the rows is a small part of the keys, and attention that
 * is given the list reads only those keys' K / V rows. For each (bm, hm) of the
 * mask's dims in the iteration space, with R rows (row r reads mask row r, or
 * row 0 when the mask broadcasts over queries):
 *   num_keys[bm, hm]        = number of keys j < Sk kept by at least one row;
 *   key_indices[bm, hm, p]  = those keys in ascending order, p < num_keys;
 *   row_bits[bm, hm, p]     = sum of 2^r over the rows r that keep that key.
 * Arrays: int32 (Bm, Hm), int32 (Bm, Hm, K) and uint32 (Bm, Hm, K),
 * contiguous, K = K_round; key_indices and row_bits 16-byte aligned. Entries
 * at p >= num_keys are left unspecified. */
typedef struct {
  int32_t* num_keys;
  int32_t* key_indices;
  uint32_t* row_bits;
  int64_t Bm, Hm, R, K;
} bsm_key_list;

typedef struct {
  bsm_tensor4 q, k, v;       /* bf16 or f32, all the same dtype */
  void* o;                   /* output, q's dtype, sizes (B, Sq, H, D) */
  int64_t o_stride[4];
  float* lse;                /* nullable; float (B, H, Sq) contiguous, natural log */
  float softmax_scale;       /* <= 0 selects 1 / sqrt(D) */
  int32_t reserved;          /* must be 0 */
  const bsm_dflash* pred;    /* nullable; DFlash predicate as the mask */
  const bsm_tensor4* mask;   /* nullable; bool aux tensor (not with pred) */
  const bsm_tensor4* bias;   /* nullable; additive aux tensor */
  const bsm_block_mask* bm;  /* nullable; NULL visits every key tile */
  const bsm_key_list* keys;  /* nullable; key-gather visit: needs mask, no bm, bf16,
                                and the list build_key_list made from that mask */
  void* workspace;           /* nullable; device scratch, 256-byte aligned, of at least */
  int64_t workspace_bytes;   /*   attn_fwd_workspace_size's bytes (key splits, staged
                                mask / bias rows) */
} bsm_attn_args;

/* In-block causality of a DFlash layer ([SF-905] Motivation; #934):
 * is_causal absent (-1) -> 0 on full-attention layers, 1 on sliding ones;
 * 0 -> 0; 1 -> 1. Returns 0 or 1, or BSM_E_ARG for any other input.
 * Host only; enqueues nothing. */
int resolve_dflash_is_causal(int32_t is_causal, int32_t layer_type);

/* Shape (Bm, Hm, nQm, nK) of the block mask build_block_mask produces for this
 * geometry and mask source (exactly one of pred / mask non-NULL), so the caller
 * can allocate the four arrays. DFlash: (1, 1, nQ, nK), shared by every batch
 * entry and head ([SF-452] Expected Behavior). Dense mask: (mask B, mask H,
 * ceil(mask Sq / 128), nK), after the swap when it applies. Host only. */
int block_mask_shape(const bsm_geom* geom, const bsm_dflash* pred,
                     const bsm_tensor4* mask, int64_t out_shape[4]);

/* Build the block mask of a DFlash predicate (pred) or of a dense bool mask
 * (mask, after the swap when it applies), exactly one non-NULL. out's
 * dimensions must equal block_mask_shape's and its four arrays must be device
 * buffers of those sizes. The DFlash path never materialises the dense mask;
 * the dense path reads the mask once. Replaces flex_attention's dense
 * create_block_mask reduction ([SF-452] traceback). */
int build_block_mask(const bsm_geom* geom, const bsm_dflash* pred,
                     const bsm_tensor4* mask, const bsm_block_mask* out,
                     hipStream_t stream);

/* Dynamic top-k keep mask over an additive bias ([FSA-197] Design,
 * Implementation Notes, review suggestion on dynamic_mask).
 * bias: bf16 or f32, 4D (Bb, Hb, Qb, round_multiple(seqlen_k, 128)), last dim
 * contiguous. premask: NULL or bool 4D with dims 1 or equal to the bias's and
 * last dim seqlen_k or the bias's (zero-copy view of a 2D (B, seqlen_k) mask as
 * (B, 1, 1, seqlen_k) is allowed); keys at or beyond its last dim count as
 * masked. Per row: invalid keys (pre-masked, or >= seqlen_k) take the bias
 * dtype's minimum finite value, the k largest values are selected (ties go to
 * the lower key index; -0 == +0), and out = selected AND valid, so a row keeps
 * exactly min(k, #valid) keys. out_mask: device, contiguous bool with the
 * bias's sizes. k < 0 is BSM_E_ARG. */
int dynamic_topk_mask(const bsm_tensor4* bias, const bsm_tensor4* premask,
                      int64_t seqlen_k, int64_t k, uint8_t* out_mask,
                      hipStream_t stream);

/* Dims (Bm, Hm, R, K) of the key list build_key_list makes from this bool
 * mask: the mask's batch and head dims in the iteration space (after the swap
 * when it applies), R = rows per (b, h) there (G under the swap, else Sq), and
 * K = K_round. R > 32 is BSM_E_UNSUPPORTED. Host only. */
int key_list_shape(const bsm_geom* geom, const bsm_tensor4* mask, int64_t out_shape[4]);

/* Build the kept-key list of a bool mask (see bsm_key_list). out's dims must
 * equal key_list_shape's. Reads the mask once; writes num_keys and the first
 * num_keys entries of key_indices and row_bits for every (bm, hm). */
int build_key_list(const bsm_geom* geom, const bsm_tensor4* mask, const bsm_key_list* out,
                   hipStream_t stream);

/* Dynamic top-k fused with what the attention needs from its mask: the same
 * selection as dynamic_topk_mask (seqlen_k = geom->Sk) over `bias`, whose mask
 * -- contiguous, the bias's sizes -- must be a valid mask for geom, and from it,
 * without a second pass over the mask:
 *   out_mask: the mask itself (nullable: not written);
 *   out_bm:   its block mask, as build_block_mask would build it (nullable);
 *   out_keys: its kept-key list, as build_key_list would build it (nullable).
 * At least one output; the mask must have at most 32 distinct rows per (b, h)
 * in the attention's iteration space (a query-broadcast mask, or the
 * seqlen_q == 1 head-group swap), and rows of at most 16384 bf16 / 8192 f32
 * keys (else BSM_E_UNSUPPORTED). The per-tile kept counts of the block mask
 * are taken while the selection is still in registers, which saves the
 * builder's read of the mask ([FSA-197] Design: the top-k mask; [SF-452]
 * traceback: the block-mask reduction). */
int dynamic_topk_fused(const bsm_geom* geom, const bsm_tensor4* bias, const bsm_tensor4* premask,
                       int64_t k, uint8_t* out_mask, const bsm_block_mask* out_bm,
                       const bsm_key_list* out_keys, hipStream_t stream);

/* Dense DFlash mask, materialised: out_mask is a device, contiguous bool array
 * (Sq, K_round) (the [B,1,Q_LEN,KV_LEN] mask of [SF-474] Suggestion 2 with the
 * batch dim dropped, keys rounded to 128, tail False). For consumers that need
 * a dense mask; the block-sparse path never calls it. */
int dflash_dense_mask(const bsm_geom* geom, const bsm_dflash* pred,
                      uint8_t* out_mask, hipStream_t stream);

/* Masked scaled-dot-product attention forward ([FSA-190] Design, Changes;
 * [SF-452]). For each (b, h, query q) with kept keys j < Sk:
 *   s_j = scale * <q, k_j> + bias[b', h', q', j],  O = softmax(s) V,
 *   LSE = log sum_j exp(s_j);
 * a row with no kept key gets O = 0 and LSE = -inf. With a block mask only its
 * listed tiles are visited (full tiles skip the mask test); it must have been
 * built by build_block_mask for the same geometry and mask source. With a key
 * list instead (keys, bf16 only, at most 32 rows per (b, h) in the iteration
 * space) only the listed keys are visited, row r keeping listed key p iff bit r
 * of its row word is set; the list must have been built by build_key_list from
 * the same mask, and listed keys outside [0, Sk) are treated as masked. Either
 * way the result is that of the dense mask. bf16 runs on
 * bf16 MFMA with float accumulation and a float online softmax, O rounded to
 * nearest even; f32 computes in float. D must be 64 or 128. */
int masked_attn_fwd(const bsm_geom* geom, const bsm_attn_args* args,
                    hipStream_t stream);

/* Bytes of optional device workspace masked_attn_fwd can use for these
 * arguments; 0 when it would use none. Two uses (bf16, no key list):
 *  - short query blocks (at most 32 query rows per (b, h) after the swap):
 *    the keys are split over several workgroups when the launch has few
 *    (b, head) pairs -- a few sequences decoding against a long KV cache. The
 *    split parts' float partial states (O, running max, row sum) are merged as
 *    in the online softmax ([FSA-190] Design: the swapped decode path of few
 *    rows);
 *  - longer queries with a dense mask and/or a bias that broadcast over the
 *    query dim (the dynamic top-k layout, [FSA-190] Changes): both are folded
 *    first into one float row per (b, head) and key -- the bias in log2 units
 *    where the mask keeps the key, -inf elsewhere -- which the attention reads
 *    tile by tile with K and V.
 * With a smaller or NULL workspace the same call runs without them; the result
 * is the same up to float rounding order. */
int attn_fwd_workspace_size(const bsm_geom* geom, const bsm_attn_args* args, int64_t* bytes);

/* Bytes of the static device scratch array of masked_attn_fwd_noalloc. */
#define BSM_NOALLOC_SCRATCH_BYTES (32LL << 20)

/* masked_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * args->workspace must be NULL and args->workspace_bytes 0. The call runs the
 * kernels masked_attn_fwd runs when given attn_fwd_workspace_size's bytes, with
 * that workspace taken from a static device array of BSM_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds on each device it runs on until the process
 * ends; results are identical to that call's. It allocates nothing and calls
 * no allocating routine.
 * Errors: a call that would need more than BSM_NOALLOC_SCRATCH_BYTES returns
 * BSM_E_UNSUPPORTED (use masked_attn_fwd with a workspace); a stream of another
 * device than the current one returns BSM_E_ARG; nothing is enqueued then.
 * The first call on a device that needs the scratch looks up that device's
 * copy of the array (loading the library's device code there if nothing has
 * yet): make it outside graph capture. All calls on one device share its one
 * array. Every byte a call reads from it is written earlier in the same call,
 * so nothing needs clearing, but calls that overlap in time on one device
 * (other streams, other host threads) race on it and corrupt each other's
 * results: order them on one stream or synchronise between them. */
int masked_attn_fwd_noalloc(const bsm_geom* geom, const bsm_attn_args* args,
                            hipStream_t stream);

/* Arguments of masked_attn_bwd: the forward's inputs, its output O and LSE,
 * the incoming gradient dL/dO, and the gradient outputs. */
typedef struct {
  bsm_tensor4 q, k, v;       /* as in bsm_attn_args */
  bsm_tensor4 o, dout;       /* forward output and dL/dO, q's dtype, (B, Sq, H, D) */
  const float* lse;          /* forward LSE, float (B, H, Sq) contiguous */
  bsm_tensor4 dq;            /* output, q's dtype, (B, Sq, H, D) */
  bsm_tensor4 dk, dv;        /* outputs, q's dtype, (B, Sk, KVH, D) */
  float softmax_scale;       /* as given to the forward; <= 0 selects 1 / sqrt(D) */
  int32_t reserved;          /* must be 0 */
  const bsm_dflash* pred;    /* mask source, bias and block mask exactly as given */
  const bsm_tensor4* mask;   /*   to the forward call that produced o and lse */
  const bsm_tensor4* bias;
  const bsm_block_mask* bm;
  const bsm_tensor4* dbias;  /* nullable; gradient of bias: bias's sizes and dtype, its
                                own strides (last dim contiguous); needs bias */
  void* workspace;           /* device scratch, 256-byte aligned, >= workspace_bytes */
  int64_t workspace_bytes;   /*   as reported by attn_bwd_workspace_size */
} bsm_attn_bwd_args;

/* Bytes of device workspace masked_attn_bwd needs for these arguments
 * (geometry, dtype and the mask / bias / block-mask descriptors are read, no
 * device data): float Delta = rowsum(dO * O) for every (b, h, q), plus a float
 * accumulator of the bias's size when dbias is requested, plus, for bf16 at
 * D = 128 with a mask and / or bias that broadcast over queries, one float row
 * per (b, head of the broadcast) and key: the bias in log2 units, -inf where
 * the mask drops a key ([FSA-190] Design: broadcast over the query dim).
 * Errors as masked_attn_bwd's checks of those descriptors. */
int attn_bwd_workspace_size(const bsm_geom* geom, const bsm_attn_bwd_args* args,
                            int64_t* bytes);

/* Masked attention backward ([FSA-190] Changes: mha_bwd; Tests: backward
 * equivalence). With the forward's P = exp(s - LSE) on kept keys (0 on masked
 * keys and on rows with LSE = -inf), dP = dO V^T, Delta = rowsum(dO * O) and
 * dS = P * (dP - Delta):
 *   dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO,
 * dK and dV summed over the G heads of each KV group, and
 *   dbias = dS summed over every (b, h, q) that reads the same bias element,
 * i.e. reduced over the dims where the bias broadcasts (batch, head groups,
 * query); dbias keys >= Sk are written as 0. Tiles are visited as in the
 * forward (the same block mask, full tiles without a mask test); the head-group
 * swap applies as in the forward. Every output element is written. Arithmetic
 * is float; outputs are rounded to q's dtype (nearest even). The workspace is
 * overwritten; dq, dk, dv and dbias must not alias any input. */
int masked_attn_bwd(const bsm_geom* geom, const bsm_attn_bwd_args* args,
                    hipStream_t stream);

/* ---- Packed variable-length sequences ([FSA-197] Changes: the integration's
 * varlen attention entry point and its pad / unpad helpers; [SF-452] traceback:
 * a block mask with one entry per batch element, Bm = B). */

/* Sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of a packed
 * Q / O of sizes (1, total_q, H, D) and key rows [cu_seqlens_k[b],
 * cu_seqlens_k[b+1]) of a packed K / V of sizes (1, total_k, KVH, D), and
 * attends to its own keys only. The cu arrays (num_seqs + 1 int32, starting at
 * 0, nondecreasing, ending at total_q / total_k) are given twice: on the
 * device for the kernels and on the host for validation and launch sizing;
 * both copies must hold the same values. */
typedef struct {
  int64_t num_seqs, H, KVH, D;
  int64_t total_q, total_k;
  const int32_t* cu_seqlens_q;       /* device */
  const int32_t* cu_seqlens_k;       /* device */
  const int32_t* cu_seqlens_q_host;  /* host */
  const int32_t* cu_seqlens_k_host;  /* host */
} bsm_varlen;

/* Per-sequence DFlash geometry: pred.ctx_len and pred.num_blocks must be 0;
 * sequence b is NB_b = Sq_b / block_size draft blocks after C_b = Sk_b - Sq_b
 * context tokens (Sq_b a multiple of block_size, Sk_b >= Sq_b), with
 * S_b = ctx_per_block, or C_b / NB_b when ctx_per_block is 0 (then NB_b must
 * divide C_b); is_causal, layer_type, sliding_window and ctx_end_offset are
 * shared. Block mask dims: (num_seqs, 1, max_b ceil(Sq_b / 128),
 * max_b ceil(Sk_b / 128)); row b lists sequence b's own tiles, its query
 * tiles past ceil(Sq_b / 128) are empty. Host only. */
int block_mask_varlen_shape(const bsm_varlen* vl, const bsm_dflash* pred, int64_t out_shape[4]);

/* Build that block mask on the device (never materialising a mask). */
int build_block_mask_varlen(const bsm_varlen* vl, const bsm_dflash* pred,
                            const bsm_block_mask* out, hipStream_t stream);

/* Masked attention forward over packed sequences: as masked_attn_fwd applied
 * to each sequence alone. args.q / o are (1, total_q, H, D), args.k / v
 * (1, total_k, KVH, D), args.lse (if not NULL) float (1, H, total_q)
 * contiguous. Mask source: args.pred with the per-sequence geometry above, or
 * none; args.bm NULL or built by build_block_mask_varlen for the same
 * sequences; args.mask, args.bias and args.keys must be NULL
 * (BSM_E_UNSUPPORTED). No head-group swap is applied. */
int masked_attn_varlen_fwd(const bsm_varlen* vl, const bsm_attn_args* args, hipStream_t stream);

/* Backward of masked_attn_varlen_fwd ([FSA-197] Changes: the varlen entry
 * point; [FSA-190] Changes: mha_bwd): dQ, dK, dV of packed sequences, each
 * sequence exactly as masked_attn_bwd on it alone. args as for masked_attn_bwd
 * with q, o, dout, dq (1, total_q, H, D), k, v, dk, dv (1, total_k, KVH, D),
 * lse float (1, H, total_q) contiguous (the forward's); mask source args.pred
 * with the per-sequence geometry of block_mask_varlen_shape, or none; args.bm
 * NULL or built by build_block_mask_varlen; args.mask, bias and dbias must be
 * NULL (BSM_E_UNSUPPORTED). A sequence with keys and no queries gets zero dK,
 * dV. args.workspace: at least masked_attn_varlen_bwd_workspace_size bytes of
 * device memory, 256-byte aligned, owned by the caller (Delta = rowsum(dO * O)
 * of every row). bf16 with D = 128 runs every sequence in one launch of each
 * kernel; other calls run the sequences one after another on stream. */
int masked_attn_varlen_bwd_workspace_size(const bsm_varlen* vl, int64_t* bytes);
int masked_attn_varlen_bwd(const bsm_varlen* vl, const bsm_attn_bwd_args* args,
                           hipStream_t stream);

/* Packing index of a padded batch: valid is a device bool array (batch,
 * seqlen) with row b at valid + b * row_stride (bytes). Writes cu_seqlens
 * (batch + 1 int32: cu_seqlens[b] = valid positions in rows 0 .. b-1) and
 * indices[i] = b * seqlen + s of the i-th valid position in row-major order
 * (int32, room for batch * seqlen entries; entries past the total are left
 * unspecified). The unpad of [FSA-197] Changes; batch * seqlen < 2^31. */
int unpad_index(const uint8_t* valid, int64_t batch, int64_t seqlen, int64_t row_stride,
                int32_t* cu_seqlens, int32_t* indices, hipStream_t stream);

/* dst row i = src row indices[i] for i < n (unpad). Rows of row_bytes bytes at
 * src + r * src_stride and dst + i * dst_stride; pointers, strides and
 * row_bytes multiples of 16; indices in [0, src rows) are the caller's
 * promise. */
int gather_rows(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
                int64_t row_bytes, const int32_t* indices, int64_t n, hipStream_t stream);

/* dst row indices[i] = src row i for i < n (pad; rows not listed are left as
 * they are, so a zero-filled dst gives the padded batch). Same layout rules. */
int scatter_rows(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
                 int64_t row_bytes, const int32_t* indices, int64_t n, hipStream_t stream);

/* Message of the last failing call on this thread ("" if none). The pointer
 * stays valid until the next call into the library on this thread. */
const char* bsm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSM_H */

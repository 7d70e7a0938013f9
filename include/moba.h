/*
 * moba.h -- C ABI of the MoBA (Mixture of Block Attention) causal prefill
 * forward library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (MoBA: Mixture of Block Attention for
 * Long-Context LLMs, README, "Trainable Block Sparse Attention" and
 * "Parameter-less Gating Mechanism"; FAQ entries from issue #27; Kimi发布MoBA
 * 突破性实现无限上下文, "MoBA：基于块的混合注意力机制" and "PyTorch实现关键要点"):
 * every sequence's keys are cut into blocks of block_size tokens (the last
 * block may be shorter) and each block is mean-pooled. For every (token,
 * query-head) row, the unscaled dot product of the query with the pooled keys
 * of the row's kv-head scores every past block of the same sequence; the
 * top-(topk-1) past blocks are kept (ties go to the lower block index), the
 * row's own block is always attended with a causal mask, and future blocks
 * never are. Softmax attention (scale 1/sqrt(head_dim) unless overridden)
 * runs over the union of those key sets, computed as one causal partial over
 * the own block and one partial per kept block, combined exactly through
 * their log-sum-exp.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout: packed variable-length "THD" tensors, contiguous and row-major:
 *   q, out: [T, Hq, D]; k, v: [T, Hkv, D]; T = cu_seqlens[num_seqs].
 *   Sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]). Blocks restart at
 *   every sequence start; nothing crosses a sequence boundary.
 * GQA: query head h reads kv-head h / (Hq / Hkv).
 * cu_seqlens: num_seqs+1 int32 entries, cu[0] = 0, non-decreasing (empty
 *   sequences allowed). Two copies are passed: cu_seqlens_host (host memory,
 *   read during the call for validation and launch sizes) and cu_seqlens_dev
 *   (device memory, read by the kernels). They must hold the same values.
 * Device pointers: q, k, v, out, workspace, sel_out, lse_out, kbar_out and
 *   every *_dev pointer are device memory owned by the caller. The library
 *   allocates no device memory, keeps no pointer after the call returns, and
 *   never synchronises the device.
 * Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the null
 *   stream). MOBA_OK means "validated and enqueued"; faults inside a kernel
 *   surface at the caller's next synchronisation.
 * Errors: arguments are checked on the host before anything is enqueued; on any
 *   error nothing is enqueued and nothing is written. moba_last_error() gives a
 *   message for the calling thread's last failed call.
 * Determinism: outputs are bitwise identical for identical inputs.
 * Limits: D in {64, 128}; block_size a positive multiple of 64; topk-1 <= 16;
 *   T*Hq and T*Hq*(topk-1) below 2^31; at most 16384 blocks per sequence; every
 *   launch grid below 2^32 work-items (a batch of very many short sequences
 *   beside a long one can exceed it: MOBA_ERR_UNSUPPORTED). For bf16 inputs the
 *   selected-block partial outputs are kept in fp16, so |v| must not exceed
 *   65504 (fp16's largest finite value); larger values turn outputs into inf or
 *   NaN without an error.
 */
#ifndef MOBA_H
#define MOBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOBA_ABI_VERSION 1

typedef enum {
  MOBA_OK = 0,
  MOBA_ERR_INVALID_ARG = 1,   /* null pointer, bad count, inconsistent shapes */
  MOBA_ERR_UNSUPPORTED = 2,   /* valid request outside the supported limits */
  MOBA_ERR_WORKSPACE = 3,     /* workspace smaller than moba_workspace_bytes() */
  MOBA_ERR_HIP = 4            /* the HIP runtime refused a launch */
} moba_status_t;

typedef enum {
  MOBA_DTYPE_F32 = 0,         /* q, k, v, out in fp32; fp32 MFMA, fp32 accumulate */
  MOBA_DTYPE_BF16 = 1         /* q, k, v, out in bf16; bf16 MFMA, fp32 accumulate */
} moba_dtype_t;

typedef struct {
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* D, 64 or 128 */
  int32_t dtype;              /* a moba_dtype_t */
  float softmax_scale;        /* <= 0 selects 1/sqrt(D) */
} moba_shape_t;

/* Version of this ABI (MOBA_ABI_VERSION). */
int32_t moba_abi_version(void);

/* Message for the calling thread's last non-OK status ("" if none). The string
 * stays valid until the thread's next call into the library. */
const char* moba_last_error(void);

/* Device workspace bytes that moba_forward needs for this batch: the pooled
 * keys, the selected block ids, the routing lists and the selected-block
 * partial outputs (the self-block kernel merges them into `out`). Host-only;
 * returns 0 and sets the last error if the arguments are invalid. */
size_t moba_workspace_bytes(const int32_t* cu_seqlens_host, int32_t num_seqs,
                            const moba_shape_t* shape, int32_t block_size, int32_t topk);

/* Smallest workspace moba_forward accepts for this batch. With more than one kv
 * head this is the workspace of the kv-group mode (see moba_forward), if it is
 * smaller than moba_workspace_bytes(); a batch beyond the int32 and grid limits of
 * one pass over all heads (where moba_workspace_bytes() returns 0) may still run
 * in that mode. Host-only; 0 and the last error if neither mode can run it. */
size_t moba_workspace_bytes_min(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                const moba_shape_t* shape, int32_t block_size, int32_t topk);

/* MoBA causal prefill forward (see the top of this file for what it computes).
 *   out:     [T, Hq, D] in the input dtype, written in full.
 *   topk:    >= 1; counts the row's own block, so topk-1 past blocks are kept
 *            (all of them when a row has fewer). topk = 1 is block-diagonal
 *            causal attention.
 *   sel_out: optional (NULL to skip), int32 [T, Hq, topk-1]: the kept past
 *            blocks of every row as sequence-local block ids in ascending
 *            order, padded with -1. Ignored when topk == 1.
 *   lse_out: optional (NULL to skip), fp32 [T, Hq]: natural-log log-sum-exp of
 *            the scaled logits over each row's attended keys.
 *   workspace: 256-byte aligned. With at least moba_workspace_bytes(...) bytes
 *            every head runs in one pass. With less, but at least
 *            moba_workspace_bytes_min(...) (num_kv_heads > 1), the kv groups run
 *            one after another: each group's G = Hq/Hkv q heads and its kv head
 *            are copied into contiguous slabs inside the workspace, the same
 *            stages run on them, and out / sel_out / lse_out are copied back.
 *            Every step of the method reads only a row's own kv head, so the
 *            result is the same (bitwise); the copies cost extra HBM traffic of
 *            about twice q, k, v and out. The int32 limits below then apply to
 *            one group (T * G * (topk-1) < 2^31), so longer batches fit.
 *   When no sequence of the batch has more than topk blocks, every row keeps all
 *   of its past blocks, which makes the attended set the whole causal prefix:
 *   the call then runs the dense causal kernel (moba_dense_causal_forward's) and
 *   writes the forced selection (0 .. i-1 for a row of block i), with no pool,
 *   gate or routing; results are within rounding of the MoBA kernels' (the same
 *   attended keys, without fp16 partial outputs).
 */
moba_status_t moba_forward(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                           int32_t num_seqs, const moba_shape_t* shape, int32_t block_size,
                           int32_t topk, void* out, void* workspace, size_t workspace_bytes,
                           int32_t* sel_out, float* lse_out, void* stream);

/* moba_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and outputs as moba_forward, with the workspace
 * taken from a static scratch array inside the library instead of a caller
 * buffer. Nothing is allocated: no hipMalloc, hipFree or allocating library
 * routine is called.
 *   Limit: the batch's moba_workspace_bytes(...) must be at most
 *          MOBA_NOALLOC_SCRATCH_BYTES (256 MiB; e.g. 8192 tokens x 32 q heads at
 *          topk 3 in bf16 fit); larger batches return MOBA_ERR_WORKSPACE with
 *          nothing enqueued.
 *   Scratch: one array per GPU the library runs on, resident from the library's
 *          first use of that GPU until the process ends; its device address is
 *          looked up once per device, on the first call made with that device
 *          current. Every call on a GPU shares that GPU's array and leaves its
 *          contents behind; no call relies on them (each call writes every
 *          scratch word it reads). Calls whose work overlaps on one GPU (other
 *          streams, or other threads) race on the array: serialise them.
 *   Arguments, layouts, outputs and errors otherwise as moba_forward (all heads
 *   in one pass; the kv-group mode needs a caller workspace). */
#define MOBA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
moba_status_t moba_forward_noalloc(const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                   int32_t num_seqs, const moba_shape_t* shape,
                                   int32_t block_size, int32_t topk, void* out,
                                   int32_t* sel_out, float* lse_out, void* stream);

/* Dense causal flash attention with the same kernels (one block per sequence):
 * every row attends to keys 0..t of its own sequence. The comparison point for
 * MoBA's speed-up (README, "Seamlessly Transition between Full and Sparse
 * Attention"). Needs no workspace.
 *   out: [T, Hq, D] in the input dtype.  lse_out: optional fp32 [T, Hq]. */
moba_status_t moba_dense_causal_forward(const void* q, const void* k, const void* v,
                                        const int32_t* cu_seqlens_dev,
                                        const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        const moba_shape_t* shape, void* out, float* lse_out,
                                        void* stream);

/* Per-call switch between sparse (MoBA) and full causal attention, for hybrid
 * stacks in which some layers, or some phases of training, run full attention
 * and the rest MoBA with the same weights (README, "Seamlessly Transition
 * between Full and Sparse Attention"; MoBA是什么, "MoBA的技术原理").
 *   mode: MOBA_MODE_SPARSE is moba_forward with every argument as given;
 *         MOBA_MODE_FULL is moba_dense_causal_forward: block_size, topk,
 *         workspace, workspace_bytes and sel_out are ignored (0 / NULL allowed).
 *   Any other mode is MOBA_ERR_INVALID_ARG. */
typedef enum {
  MOBA_MODE_SPARSE = 0,
  MOBA_MODE_FULL = 1
} moba_mode_t;
moba_status_t moba_attention_forward(int32_t mode, const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens_dev,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs,
                                     const moba_shape_t* shape, int32_t block_size,
                                     int32_t topk, void* out, void* workspace,
                                     size_t workspace_bytes, int32_t* sel_out, float* lse_out,
                                     void* stream);

/* ---- Backward ---------------------------------------------------------------
 * Gradients of moba_forward's out with respect to q, k and v, given the
 * gradient dout of a loss with respect to out. The forward's selection is
 * held fixed (top-k is piecewise constant: no gradient reaches the gate;
 * README, "Trainable Block Sparse Attention"). With p the attention weights of
 * a row over its attended keys, Delta = dout . out, dS = p (dout . v - Delta):
 *   dq = scale * sum dS k,  dk = scale * sum_rows dS q,  dv = sum_rows p dout,
 * dk and dv summed over every row (all q heads of the kv group) that attends
 * the key. Deterministic (no atomics).
 *   out, lse:  the forward's out and lse_out ([T, Hq, D] input dtype; fp32
 *              [T, Hq]) for these q, k, v.
 *   dout:      [T, Hq, D] input dtype.
 *   sel:       the forward's sel_out, int32 [T, Hq, topk-1] (unused when topk == 1),
 *              for the same q, k, block_size and topk. Other contents give
 *              meaningless gradients (ids outside a row's past blocks are
 *              ignored, so nothing is accessed out of bounds).
 *   dq: [T, Hq, D]; dk, dv: [T, Hkv, D] (input dtype), written in full.
 *   workspace: at least moba_backward_workspace_bytes(...), 256-byte aligned.
 * Same shapes and limits as moba_forward. */
size_t moba_backward_workspace_bytes(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                     const moba_shape_t* shape, int32_t block_size,
                                     int32_t topk);
moba_status_t moba_backward(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, const int32_t* sel,
                            const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                            int32_t num_seqs, const moba_shape_t* shape, int32_t block_size,
                            int32_t topk, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---- Decoding against a KV cache (gated decode / chunked-prefill
 * continuation) ------------------------------------------------------------
 * README FAQ (issue #27, decoding); "Parameter-less Gating Mechanism". New
 * rows are the last tokens of their sequences: a row at position p attends its
 * own block up to p (causal) plus the top-(topk-1) complete past blocks by the
 * score of its query against their mean-pooled keys -- exactly the prefill's
 * row p. Layout: the caches are packed like prefill inputs, k_cache, v_cache
 * [Tk, Hkv, D] with sequence n at tokens [cu_k[n], cu_k[n+1]) and the new
 * tokens' K/V already appended; q_new [Tq, Hq, D] holds sequence n's new rows
 * at [cu_q[n], cu_q[n+1]), which are its last cu_q[n+1]-cu_q[n] cached tokens.
 * The pooled keys live in a caller-owned fp32 cache kbar_cache
 * [num_seqs * max_blocks, Hkv, D]: block j of sequence n at row
 * n * max_blocks + j; max_blocks must cover every cache length. */

/* Pool the blocks that became complete when each sequence grew from
 * prev_len[n] tokens to its cache length (blocks prev_len/B .. len/B - 1) into
 * kbar_cache, with the same fp32 summation order as moba_block_pool (so the
 * means equal a prefill's). prev_len: int32 [num_seqs], host and device
 * copies with the same values, 0 <= prev_len[n] <= length. Blocks not yet
 * complete are left alone. */
moba_status_t moba_kbar_append(const void* k_cache, const int32_t* cu_k_dev,
                               const int32_t* cu_k_host, const int32_t* prev_len_dev,
                               const int32_t* prev_len_host, int32_t num_seqs,
                               const moba_shape_t* shape, int32_t block_size, int32_t max_blocks,
                               float* kbar_cache, void* stream);

/* Device workspace bytes for moba_decode_forward (the kept blocks and the
 * per-segment partial outputs of every new row). Host-only; 0 and the last
 * error on invalid arguments. */
size_t moba_decode_workspace_bytes(const int32_t* cu_q_host, const int32_t* cu_k_host,
                                   int32_t num_seqs, const moba_shape_t* shape,
                                   int32_t block_size, int32_t topk, int32_t max_blocks);

/* MoBA attention for the new rows against the cache (see above).
 *   kbar_cache: must hold every complete block before each new row's block
 *               (moba_kbar_append after appending K); unused when topk == 1.
 *   out:     [Tq, Hq, D] in the input dtype.
 *   sel_out: optional int32 [Tq, Hq, topk-1], as moba_forward's.
 *   lse_out: optional fp32 [Tq, Hq].
 *   workspace: at least moba_decode_workspace_bytes(...), 256-byte aligned.
 * Limits as moba_forward's; block_size a multiple of 64. */
moba_status_t moba_decode_forward(const void* q_new, const void* k_cache, const void* v_cache,
                                  const int32_t* cu_q_dev, const int32_t* cu_q_host,
                                  const int32_t* cu_k_dev, const int32_t* cu_k_host,
                                  int32_t num_seqs, const moba_shape_t* shape,
                                  int32_t block_size, int32_t topk, const float* kbar_cache,
                                  int32_t max_blocks, void* out, void* workspace,
                                  size_t workspace_bytes, int32_t* sel_out, float* lse_out,
                                  void* stream);

/* The block mean-pool step alone (Kimi发布MoBA突破性实现无限上下文, "PyTorch实现
 * 关键要点": one mean-pooled key per block). Only k is read.
 *   kbar_out:  fp32 [NB, Hkv, D], NB = sum_n ceil(S_n / block_size), blocks
 *              numbered sequence by sequence; the last block of a sequence is
 *              averaged over its true length. Sums run in fp32 in a fixed order.
 *   workspace: at least moba_workspace_bytes(cu_seqlens_host, num_seqs, shape,
 *              block_size, 1) bytes, 256-byte aligned (holds the block table). */
moba_status_t moba_block_pool(const void* k, const int32_t* cu_seqlens_dev,
                              const int32_t* cu_seqlens_host, int32_t num_seqs,
                              const moba_shape_t* shape, int32_t block_size, float* kbar_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Number of routing lists and routed entries for a batch, for sizing the
 * buffers of moba_route. A list is a (global block, kv-head) pair, numbered
 * block-major: list = global_block * Hkv + kv_head. Host-only. Returns MOBA_OK
 * or MOBA_ERR_INVALID_ARG. */
moba_status_t moba_route_sizes(const int32_t* cu_seqlens_host, int32_t num_seqs,
                               const moba_shape_t* shape, int32_t block_size, int32_t topk,
                               int64_t* num_lists, int64_t* num_entries);

/* The routing step alone: the MoE-style inversion of a selection map (MoBA
 * README, abstract: MoE principles applied to attention; Kimi article, "PyTorch
 * 实现关键要点": the data is reorganised by selected block before attention).
 *   sel_dev:        int32 [T, Hq, topk-1] as written by moba_forward's sel_out
 *                   (valid ids first, ascending, then -1).
 *   list_offsets:   int32 [num_lists + 1] out: list L holds entries
 *                   [list_offsets[L], list_offsets[L+1]).
 *   entries:        int32 [num_entries] out: entry = row * (topk-1) + slot, where
 *                   row = token * Hq + head and sel[row][slot] names the block;
 *                   rows ascend within each list.
 *   workspace:      as for moba_forward with the same arguments.
 * Requires topk >= 2. */
moba_status_t moba_route(const int32_t* sel_dev, const int32_t* cu_seqlens_dev,
                         const int32_t* cu_seqlens_host, int32_t num_seqs,
                         const moba_shape_t* shape, int32_t block_size, int32_t topk,
                         int32_t* list_offsets, int32_t* entries, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Per-stage timing with HIP events, for benchmarks. While enabled, every call
 * records an event pair around each stage's launches on the call's stream.
 * moba_timing_read() waits for the recorded events, writes per stage the summed
 * milliseconds and the number of timed launches, then clears the record.
 * Stage ids: 0 pool, 1 gate, 2 route, 3 self-block attention (which also
 * merges the parts), 4 selected-block attention, 5 merge (no separate launch:
 * always 0 launches; the id is kept so that the others stay fixed), 6 dense
 * causal attention, 7 decode (gate, parts and merge of moba_decode_forward),
 * 8 pooled-key append, 9 backward (Delta, dq and dk/dv passes; its routing is
 * timed as stage 2), 10 the kv-group mode's slab copies. Returns the number of stages
 * written. At most 4096 event pairs are kept; later ones are not recorded. */
moba_status_t moba_timing_enable(int32_t enable);
int32_t moba_timing_read(double* stage_ms, int32_t* stage_launches, int32_t max_stages);
const char* moba_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H */

/*
 * lightning_attn.h -- C ABI of the MI355X (gfx950) lightning-attention library: prefill,
 * sequence-split prefill, backward and decode.
 *
 * The operation.  Lightning attention is causal linear attention computed block by block:
 * inside a block the left product ((Q K^T) masked) V, across blocks the right product
 * Q (K^T V) carried by a running d x d state, which avoids the slow cumulative sum
 * ("MiniMax-01 technical report digest", futurefh.com, section 1 "core innovation"; the
 * associativity (QK^T)V = Q(K^T V) is stated in the nabfollower blog, section "The Core Tech:
 * Lightning Attention").  Decode keeps only the fixed-size state and updates it per token
 * (nabfollower blog, analogy section), and prefill and decode run as separate paths (digest,
 * section 3 "efficient inference framework").  Packed variable-length batches follow the data
 * packing of the digest's section 4.  With a constant per-head decay lambda_h (the pages state
 * none; this library adopts one scalar per head, constant in time), for each packed sequence
 * and head, with local token index t:
 *
 *     S_t = lambda S_{t-1} + k_t^T v_t          (S_{-1} = initial state, or 0)
 *     o_t = q_t S_t  =  sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s  + lambda^(t+1) q_t S_{-1}
 *
 * i.e. the output uses the state that already includes token t.  There is no normaliser, no
 * feature map and no 1/sqrt(d) scaling inside the operation.
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   activations q, k, v, out : [T][H][D]     (feature index fastest), dtype per la_dtype
 *   decay                    : [H] float32, lambda_h in [0, 1]
 *   cu_seqlens               : [S+1] int32,  0 = cu[0] <= cu[1] <= ... <= cu[S] = T
 *   states                   : [S][H][D][D]  float32, state[a][b] = sum lambda^.. k[a] v[b]
 *                              (a = key feature, b = value feature)
 *
 * Supported: D in {64, 128}; dtype LA_BF16 (bf16 storage, fp32 accumulation, MFMA) or LA_F32
 * (fp32 storage and arithmetic).  Devices: gfx950 only.
 *
 * Ownership and memory.  The caller owns every buffer; the library keeps no pointer after a
 * call returns and allocates no device memory.  Every buffer a call writes (out, the states it
 * writes or updates, gradients, a workspace) must not overlap any other buffer argument of the
 * call, read or written, decay and cu_seqlens included; buffers that are only read (q, k, v,
 * decay, an initial state, ...) may share memory.  The host checks these byte ranges (from the
 * sizes given) and returns LA_ERR_INVALID_ARG on an overlap.
 *
 * Finite inputs.  q, k, v (and states) must be finite.  The definition masks future tokens out
 * by selection, so a non-finite value could never reach an earlier output; the kernels keep
 * that for q and k (future scores are selected away, the state only carries a token forward),
 * but a block's matrix products multiply the masked-out (exactly zero) weights by v on the
 * matrix cores, and 0 * inf or 0 * NaN is NaN there.  So a non-finite v at token t reaches
 * earlier outputs of its own block (within the 32-token operand group of the intra product in
 * bf16, at either block size; the 16-token tile in fp32), never those of an earlier block nor
 * anything before the sequence's start.
 *
 * Errors.  Argument checks run on the host before any HIP call and return a status; nothing
 * throws across this ABI.  Device data is not validated: non-monotone cu_seqlens or lambda
 * outside [0, 1] give undefined results (never an out-of-bounds access for cu values within
 * [0, T]).  Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream);
 * LA_ERR_HIP reports a failed HIP call or launch (including "no device").  la_last_error()
 * gives a human-readable detail for the calling thread's last failure.  Thread-safe.
 */
#ifndef LIGHTNING_ATTN_H
#define LIGHTNING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1, /* NULL required pointer, negative size, S < 1, H < 1, ...   */
  LA_ERR_UNSUPPORTED = 2, /* D not in {64,128}, unknown dtype, device not gfx950       */
  LA_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed / no device    */
} la_status;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* ABI version of this header (bumped on any incompatible change). */
#define LA_ABI_VERSION 2
int32_t la_abi_version(void);

/*
 * Prefill (the block-wise forward pass): within each block (128 tokens for bf16, 64 for fp32; see
 * la_prefill_with_block_size) the left product, across
 * blocks the right product through the running state (digest, section 1), over a packed batch
 * of sequences delimited by cu_seqlens with the state reset at every sequence start (digest,
 * section 4, data packing).
 *   q, k, v     in  [T][H][D] dtype           (may be NULL when T == 0)
 *   decay       in  [H] float32
 *   cu_seqlens  in  [S+1] int32, or NULL meaning one sequence of length T (then S must be 1)
 *   out         out [T][H][D] dtype           (may be NULL when T == 0)
 *   final_state out [S][H][D][D] float32, or NULL to skip; an empty sequence gives its
 *               initial state (or zeros)
 *   T >= 0 tokens in total, S >= 1 sequences, H >= 1 heads, D head dimension.
 */
la_status la_prefill(const void *q, const void *k, const void *v, const float *decay,
                     const int32_t *cu_seqlens, void *out, float *final_state, int64_t T,
                     int32_t S, int32_t H, int32_t D, la_dtype dtype, void *stream);

/*
 * Prefill continuing from a given state per (sequence, head) (chunked prefill; the state
 * S_{-1} above).  Linear attention carries the whole past in the fixed-size state (nabfollower
 * blog, analogy section), so a sequence prefilled in pieces, each piece starting from the state
 * the previous one left, gives the same result as one call.  initial_state: [S][H][D][D]
 * float32 or NULL (= zeros); it is read only and may not overlap final_state or out.  All other
 * arguments as la_prefill.
 */
la_status la_prefill_ex(const void *q, const void *k, const void *v, const float *decay,
                        const int32_t *cu_seqlens, const float *initial_state, void *out,
                        float *final_state, int64_t T, int32_t S, int32_t H, int32_t D,
                        la_dtype dtype, void *stream);

/*
 * Prefill with a chosen block size B (la_prefill_ex with its initial state, plus block_size).
 * The split into blocks (digest, section 1: left product inside a block, right product across
 * blocks) is exact algebra for any B, so every B gives the same result up to rounding; B only
 * trades the number of serial block steps of a scan against the size of each block's intra
 * product (4 B d + 4 d^2 FLOP per token-head).
 *   block_size  0 = the default: 128 for bf16 storage (faster on MI355X; the environment
 *               variable LA_BLOCK = 64 or 128 overrides it, read once per process; any other
 *               value makes bf16 calls fail with LA_ERR_INVALID_ARG), 64 for fp32 storage;
 *               la_prefill and la_prefill_ex use this default
 *               64 or 128 (128: bf16 storage only, else LA_ERR_UNSUPPORTED)
 * Other arguments, result and errors as la_prefill_ex, plus LA_ERR_INVALID_ARG for any other
 * block_size.  la_backward's scans take the same default; the segment scans of the split
 * prefill and of la_backward_split pick theirs by segment length (128 for segments of 4,096
 * tokens or more in whole 128-token blocks); the fp32 path uses B = 64.
 */
la_status la_prefill_with_block_size(const void *q, const void *k, const void *v,
                                     const float *decay, const int32_t *cu_seqlens,
                                     const float *initial_state, void *out, float *final_state,
                                     int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype,
                                     int32_t block_size, void *stream);

/*
 * Sequence-split prefill: the same result as la_prefill_ex, computed with every sequence cut
 * into segments of seg_blocks * 64 tokens that are scanned in parallel.  Meant for batches with
 * few (sequence, head) pairs, where the plain prefill runs one workgroup per (sequence, head,
 * 32 value columns) and leaves most of the device idle.
 *
 * The block recurrence (digest, section 1: the running state of the right product) is linear
 * in the state, so a segment of m tokens maps its incoming state S_in to lambda^m S_in + L with
 * L independent of S_in.  bf16 storage (while no sequence has more than 16 segments and a
 * segment's byte offsets fit 32 bits): two launches on `stream`, L of every segment but the
 * last of each sequence (k and v read once; computed as 2, 4 or 8 sub-segment states when
 * those segments are too few to fill the device), then the prefill of every segment, which
 * forms its incoming state from the earlier segments' states (the first from initial_state or
 * 0) and, for the last segment, writes the final state.  Otherwise four launches: a segment
 * table built from cu_seqlens on the device; L of every segment; a combine that walks each
 * sequence's segments in order (final state = what follows the last); the prefill of every
 * segment from its incoming state.  k and v are read twice in total, q once, out is written
 * once.  The result differs from la_prefill_ex only in rounding order.
 *
 *   seg_blocks       >= 1: segment length in 64-token blocks (la_prefill_split_blocks suggests
 *                    one for the current device)
 *   workspace        device memory of at least la_prefill_split_workspace_size(...) bytes,
 *                    256-byte aligned, owned by the caller; holds the segment states and the
 *                    segment table between the launches (no initial contents needed; not
 *                    read after the call's work on `stream` completes).  Calls that share a
 *                    workspace must be ordered (same stream).
 *   T < 2^31 (segment starts are int32); all other arguments as la_prefill_ex.
 * Errors: as la_prefill_ex, plus LA_ERR_INVALID_ARG for seg_blocks < 1, a NULL, misaligned or
 * too small workspace, T >= 2^31 or more than 2^31 segment workgroups.
 */
la_status la_prefill_split(const void *q, const void *k, const void *v, const float *decay,
                           const int32_t *cu_seqlens, const float *initial_state, void *out,
                           float *final_state, int64_t T, int32_t S, int32_t H, int32_t D,
                           la_dtype dtype, int32_t seg_blocks, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * la_prefill_split without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * segment states and segment table live in a static device array of
 * LA_SPLIT_STATIC_SCRATCH_BYTES that every device the library runs on holds from the library's
 * load until the process ends.  The call allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine); the caller still owns every other buffer.  Same arguments,
 * result and errors as la_prefill_split otherwise, plus LA_ERR_INVALID_ARG when these sizes
 * need more than LA_SPLIT_STATIC_SCRATCH_BYTES of workspace even with one state per segment
 * (the call keeps no sub-segment states when they would not fit; sizes with
 * la_prefill_split_workspace_size(T, S, H, D, seg_blocks) <= LA_SPLIT_STATIC_SCRATCH_BYTES
 * always fit).
 * All calls on one device share its scratch: calls that overlap in time on one device (two
 * streams, two host threads) race and give wrong results; order them on one stream.  The
 * scratch needs no initial contents.
 */
#define LA_SPLIT_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
la_status la_prefill_split_static(const void *q, const void *k, const void *v,
                                  const float *decay, const int32_t *cu_seqlens,
                                  const float *initial_state, void *out, float *final_state,
                                  int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype,
                                  int32_t seg_blocks, void *stream);

/* Workspace bytes la_prefill_split and la_backward_split need for these sizes (0 for invalid
 * sizes).  The bound holds for any valid cu_seqlens: (ceil(T / (64 seg_blocks)) + S - 1) * sub
 * states of H*D*D floats plus the segment table, where sub (1, 2, 4 or 8; a function of these
 * sizes only) is the number of sub-segment states per segment that the bf16 two-launch form may
 * keep. */
size_t la_prefill_split_workspace_size(int64_t T, int32_t S, int32_t H, int32_t D,
                                       int32_t seg_blocks);

/* Suggested seg_blocks for the current device: about one segment workgroup per compute unit,
 * at least 4 blocks per segment; 0 (use the plain scan) when splitting would not add
 * parallelism (the plain launch already has a workgroup per compute unit, or no sequence would
 * be cut), when a cost model of both paths (fitted to MI355X timings: per-block cost by dtype,
 * head size, workgroups in flight and whether q, k, v and out fit the 256 MB last-level cache;
 * the mean sequence length T / S stands in for the longest) predicts the split saves less than
 * 5% (short sequences, where its fixed cost of two or four launches dominates), or on any error. */
int32_t la_prefill_split_blocks(int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype);

/* The same suggestion for a device with compute_units compute units (no device access; 0 for
 * invalid sizes or dtype). */
int32_t la_prefill_split_blocks_for(int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype,
                                    int32_t compute_units);

/*
 * Backward of la_prefill_ex: gradients of a loss L given dL/dout (d_out) and, optionally,
 * dL/dfinal_state (d_final_state).  The pages give no backward pass (they state training at up
 * to 1M tokens of context: abstract of the MiniMax-01 report; digest, section 2); these are the
 * derivatives of the operation defined at the top of this header, per sequence and head with
 * local token indices and n tokens:
 *
 *   dq_t = sum_{s<=t} lambda^(t-s) (do_t . v_s) k_s  + lambda^(t+1) S0 do_t
 *   dk_s = sum_{t>=s} lambda^(t-s) (do_t . v_s) q_t  + lambda^(n-1-s) dSn v_s
 *   dv_s = sum_{t>=s} lambda^(t-s) (q_t . k_s) do_t  + lambda^(n-1-s) dSn^T k_s
 *   dS0  = sum_t lambda^(t+1) q_t^T do_t + lambda^n dSn
 *
 * Each is a scan of the same block form as the prefill: dq is the forward scan with
 * (query, key, value) = (do, v, k) from S0^T; dk and dv are reversed-time scans with (v, do, q)
 * from dSn^T and (k, q, do) from dSn; dS0 is lambda times the last of these scans' final
 * state.  Three launches on `stream`, no workspace, with the prefill's default block size (for
 * bf16 128 tokens, or LA_BLOCK).  lambda gets no gradient (a constant).
 *
 *   q, k, v, decay, cu_seqlens, initial_state: the forward call's inputs (initial_state may be
 *                 NULL = zeros)
 *   d_out         in  [T][H][D] dtype
 *   d_final_state in  [S][H][D][D] float32, or NULL (= zeros)
 *   dq, dk, dv    out [T][H][D] dtype, distinct, not aliasing any input
 *   d_initial_state out [S][H][D][D] float32, or NULL to skip
 * Errors: as la_prefill_ex, plus LA_ERR_INVALID_ARG for a NULL, misaligned or aliasing gradient
 * buffer.
 */
la_status la_backward(const void *q, const void *k, const void *v, const float *decay,
                      const int32_t *cu_seqlens, const float *initial_state, const void *d_out,
                      const float *d_final_state, void *dq, void *dk, void *dv,
                      float *d_initial_state, int64_t T, int32_t S, int32_t H, int32_t D,
                      la_dtype dtype, void *stream);

/*
 * la_backward with every sequence cut into segments of seg_blocks blocks that are scanned in
 * parallel, for batches with few (sequence, head) pairs (the construction of la_prefill_split,
 * applied to the three gradient scans).  dq: segment states of the forward scan, combined from
 * S0^T, then every segment from its incoming state.  dk and dv: their reversed-time states are
 * transposes of each other, so one reversed state-only pass over the segments serves both; the
 * combine walks each sequence's segments from the last to the first starting from dSn, and its
 * result times lambda is dS0; then every segment of dv and of dk from its incoming state (the
 * last segment of a sequence, met first, from dSn as the unsplit scans use it).  Eight launches
 * on `stream`.  The result differs from la_backward only in rounding order.
 *
 *   seg_blocks, workspace, workspace_bytes: as la_prefill_split; the workspace size is
 *                 la_prefill_split_workspace_size(T, S, H, D, seg_blocks) and must not overlap
 *                 any other argument
 *   T < 2^31; all other arguments as la_backward.
 * Errors: as la_backward, plus those of la_prefill_split's workspace and segment arguments.
 */
la_status la_backward_split(const void *q, const void *k, const void *v, const float *decay,
                            const int32_t *cu_seqlens, const float *initial_state,
                            const void *d_out, const float *d_final_state, void *dq, void *dk,
                            void *dv, float *d_initial_state, int64_t T, int32_t S, int32_t H,
                            int32_t D, la_dtype dtype, int32_t seg_blocks, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for Bt independent sequences (one new token each).  Decoding keeps
 * only the fixed-size state, so each token costs the same whatever the context length
 * (nabfollower blog, analogy section), and it runs as its own path beside prefill (digest,
 * section 3):
 *   S' = lambda S + k^T v ;  o = q S' ;  state <- S'   (in place)
 *   q, k, v in [Bt][H][D] dtype; decay [H] float32; state in/out [Bt][H][D][D] float32;
 *   out [Bt][H][D] dtype.  Bt >= 0 (0 is a no-op).  state and out must not overlap each other
 *   or q, k, v, decay.
 */
la_status la_decode_step(const void *q, const void *k, const void *v, const float *decay,
                         float *state, void *out, int32_t Bt, int32_t H, int32_t D,
                         la_dtype dtype, void *stream);

/*
 * m decode steps per sequence in one pass (speculative or chunked decode): for i = 0..m-1,
 *   S <- lambda S + k_i^T v_i ;  o_i = q_i S
 * with the state read and written once for all m tokens, so the step's HBM traffic per token
 * falls as 1/m.  Same result as m calls of la_decode_step (and as la_prefill_ex over sequences
 * of m tokens from the states), up to rounding order.
 *   q, k, v in [Bt][m][H][D] dtype (token i of sequence b is row b*m + i of a [Bt*m][H][D]
 *   packed tensor); out [Bt][m][H][D] dtype; state in/out [Bt][H][D][D] float32; m >= 1.
 * Errors as la_decode_step, plus LA_ERR_INVALID_ARG for m < 1.
 */
la_status la_decode_tokens(const void *q, const void *k, const void *v, const float *decay,
                           float *state, void *out, int32_t Bt, int32_t m, int32_t H, int32_t D,
                           la_dtype dtype, void *stream);

/* Static string naming a status code. */
const char *la_status_str(la_status s);

/* Detail of the calling thread's most recent failed call ("" if none). */
const char *la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_ATTN_H */

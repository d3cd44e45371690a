/*
 * cpattn.h — C ABI of libcpattn: one context-parallel rank's blockwise
 * (zigzag ring) attention over packed variable-length sequences, on one
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  "Scaling Video Training with Parallelism" (section 2,
 * Ring Attention paragraph) describes ring attention as blockwise attention:
 * each device attends its local queries to one key/value block at a time
 * while the blocks travel round the ring, and the per-block results are
 * combined.  The LongVILA article names the zigzag variant
 * (ZIGZAG-RINGATTN) that balances causal work across ranks.  "Speeding up
 * Variable-Length Training with Dynamic Context Parallelism and NVIDIA
 * Megatron Core" (section A2) fixes the input format: packed THD tensors
 * (batch folded into the token dimension) described by cu_seqlens, with the
 * context-parallel size carried per batch.  On one GPU the ring's K/V steps
 * are iterated locally at their real per-rank shapes; nothing here talks to
 * another GPU.
 *
 * Calling sequence for rank r of cp ranks:
 *     cpattn_partition (Q to rank r, K/V to every source rank)
 *     lse = -inf (out needs no initialisation)   (cpattn_fill_f32)
 *     for s in 0..cp-1:
 *         cpattn_fwd_step(step = {cp, r, s})     -> out_partial, lse_partial
 *         cpattn_merge(out, lse, out_partial, lse_partial)
 *     backward:
 *         dq, dk, dv = 0                         (cpattn_fill_f32)
 *         cpattn_bwd_preprocess(out, dout)       -> delta
 *         for s in 0..cp-1: cpattn_bwd_step(step = {cp, r, s})
 *
 * Conventions shared by every entry point
 *   Memory.   Every pointer named *_dev or held in a cpattn_tensor is device
 *             memory owned by the caller; *_host pointers are host memory.
 *             The library never allocates, frees or keeps caller memory and
 *             keeps no per-call state.  Scratch space is the caller's
 *             `workspace` (size from cpattn_workspace_size).
 *   Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *             stream).  Device calls only enqueue work on it; none
 *             synchronises, except cpattn_workspace_status which waits for
 *             the stream.  Calls are thread-safe; calls that share one
 *             workspace must be ordered on one stream.
 *   Errors.   Arguments are checked before anything is launched; on failure
 *             the call returns a non-zero status and enqueues nothing.  A
 *             failed launch returns CPATTN_ERR_HIP.  No C++ exception
 *             crosses this boundary.  cu_seqlens arrays in device memory are
 *             checked on the device (non-decreasing, cu[0] = 0, within the
 *             tensor, chunk-divisible when cp > 1); a bad array makes the
 *             call write nothing and leaves a status code in the workspace
 *             that cpattn_workspace_status returns.
 *   Layout.   THD: row t of a [tokens, heads, head_dim] tensor is token t;
 *             head_dim is contiguous; strides are in elements.  LSE and
 *             delta arrays are fp32 [heads][tokens], contiguous.  fp32
 *             accumulators (out, dq, dk, dv) are dense [tokens][heads][d].
 *   Softmax.  s_ij = scale * <q_i, k_j>, natural-log LSE; scale <= 0
 *             selects 1/sqrt(head_dim).  A query row with no allowed key in
 *             a step gets out_partial = 0 and lse_partial = -inf.
 *   GQA.      Hq must be a multiple of Hkv; q-head h reads kv-head
 *             h / (Hq/Hkv) (contiguous groups).
 *   Types.    q, k, v, dout, out_partial share one dtype: bf16 (head_dim
 *             128 or 64, MFMA path) or fp32 (head_dim 64 or 128).
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CPATTN_OK = 0,
    CPATTN_ERR_INVALID_ARG = 1,   /* bad pointer, size, stride, rank/step, cu_seqlens */
    CPATTN_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype, head_dim) */
    CPATTN_ERR_WORKSPACE = 3,     /* workspace missing or too small */
    CPATTN_ERR_HIP = 4,           /* a HIP runtime call or launch failed */
    CPATTN_ERR_INFEASIBLE = 5,    /* planner: no plan fits the memory cap */
    CPATTN_ERR_NOMEM = 6          /* host memory for a planner call ran out */
} cpattn_status;

typedef enum { CPATTN_F32 = 0, CPATTN_BF16 = 1 } cpattn_dtype;

/* Masks over in-sequence positions of the unsplit sequence.
 *   CAUSAL   key position <= query position.
 *   BIDIR    every key of the same sequence.
 *   TF_BLOCK teacher forcing ("Scaling Video Training with Parallelism",
 *            section 4): each sequence is [clean history ; noisy target],
 *            N time chunks of B tokens per stream (sequence length 2*N*B).
 *            Clean chunk c sees clean chunks <= c; noisy chunk c sees clean
 *            chunks < c plus its own noisy chunk.  With cp > 1 the local
 *            tensors follow the balanced split (cpattn_partition_tf, same
 *            page, balanced SP): N must be a multiple of cp and B >= 32. */
typedef enum { CPATTN_MASK_CAUSAL = 0, CPATTN_MASK_BIDIR = 1, CPATTN_MASK_TF_BLOCK = 2 } cpattn_mask_mode;

/* A THD tensor view.  data: device pointer, 16-byte aligned.  stride_token
 * and stride_head in elements, multiples of 8 (16 bytes for bf16, 32 for
 * fp32); the head_dim elements of one (token, head) are contiguous. */
typedef struct {
    void* data;
    cpattn_dtype dtype;
    int64_t tokens;
    int32_t heads;
    int32_t head_dim;
    int64_t stride_token;
    int64_t stride_head;
} cpattn_tensor;

/* One ring step: rank `rank` of `cp` ranks at step `step`; its K/V are the
 * share of rank (rank - step) mod cp.  tf_chunk_tokens (B) and
 * tf_num_chunks (N) are read only for CPATTN_MASK_TF_BLOCK. */
typedef struct {
    int32_t cp;
    int32_t rank;
    int32_t step;
    int32_t tf_chunk_tokens;
    int32_t tf_num_chunks;
} cpattn_step;

const char* cpattn_version(void);
const char* cpattn_status_string(cpattn_status s);

/* Text of the HIP error behind the last CPATTN_ERR_HIP returned on the
 * calling thread ("" if none).  Valid until the next call on that thread. */
const char* cpattn_last_hip_error(void);

/* Compute units and peak shader clock (kHz) of HIP device `device`: the
 * figures a dense matrix-core peak follows from (on gfx950, 4096 bf16 FLOP
 * per clock per CU).  Host call, no launch.  CPATTN_ERR_INVALID_ARG for a
 * NULL output or a negative device, CPATTN_ERR_HIP if HIP cannot query the
 * device; the outputs are written only on success. */
cpattn_status cpattn_device_info(int32_t device, int32_t* cu_count_host, int32_t* clock_khz_host);

/* ---- zigzag partition -----------------------------------------------------
 * Zigzag split (LongVILA article, ZIGZAG-RINGATTN; the chunk rule is not
 * printed there, this is the reading that balances causal work exactly):
 * sequence b of length L_b is cut into 2*cp chunks of C_b = L_b/(2*cp)
 * tokens and rank r keeps chunks r and 2*cp-1-r, in that order.  The local
 * tensor is, sequence after sequence, [chunk r ; chunk 2cp-1-r]; its
 * cu_seqlens are the prefix sums of L_b/cp.  cp = 1 is the identity (no
 * divisibility requirement).  Requires L_b % (2*cp) == 0 when cp > 1. */

/* Host-only index plan.  cu_seqlens_global_host[num_seqs+1] (int32, cu[0]=0,
 * non-decreasing).  Writes cu_seqlens_local_host[num_seqs+1] and, when not
 * NULL, local_to_global_host[cu_global[num_seqs]/cp] (global row of every
 * local row).  Bit-exact integer work; INVALID_ARG on a bad array. */
cpattn_status cpattn_partition_index(const int32_t* cu_seqlens_global_host, int32_t num_seqs,
                                     int32_t cp, int32_t rank,
                                     int32_t* cu_seqlens_local_host,
                                     int64_t* local_to_global_host);

/* Device gather of rank `rank`'s share: dst_local[t] = src_global[l2g(t)]
 * for every local row t < cu_global[num_seqs]/cp.  src and dst have equal
 * dtype, heads and head_dim; dst->tokens >= src tokens / cp.  Copies bytes
 * (bit-exact).  cu_seqlens_global_dev: device int32[num_seqs+1]. */
cpattn_status cpattn_partition(const cpattn_tensor* src_global, cpattn_tensor* dst_local,
                               const int32_t* cu_seqlens_global_dev, int32_t num_seqs,
                               int32_t cp, int32_t rank, void* stream);

/* Inverse scatter: dst_global[l2g(t)] = src_local[t].  Rows of other ranks
 * are left untouched. */
cpattn_status cpattn_unpartition(const cpattn_tensor* src_local, cpattn_tensor* dst_global,
                                 const int32_t* cu_seqlens_global_dev, int32_t num_seqs,
                                 int32_t cp, int32_t rank, void* stream);

/* ---- balanced teacher-forcing split --------------------------------------
 * "Scaling Video Training with Parallelism", section 4 (balanced SP): every
 * rank keeps the clean and the noisy chunk of the same time segments, so the
 * noisy (loss-carrying) targets spread evenly.  The page does not print the
 * assignment; the rule taken here deals time chunks c = 0..N-1 to ranks in
 * snake order over rounds of 2*cp chunks (c goes to rank u or 2cp-1-u of its
 * round, u = c mod 2cp), which gives every rank equal teacher-forcing work
 * when N is a multiple of 2*cp.  Rank r's local rows of a sequence are its
 * N/cp clean chunks in ascending time order, then its noisy chunks in the
 * same order, B rows each.  Every sequence has 2*B*N tokens
 * (B = tf_chunk_tokens, N = tf_num_chunks, N a multiple of cp); the local
 * cu_seqlens are the prefix sums of L_b/cp.  Arguments, copies and errors
 * as for the zigzag functions above. */
cpattn_status cpattn_partition_index_tf(const int32_t* cu_seqlens_global_host, int32_t num_seqs,
                                        int32_t cp, int32_t rank, int32_t tf_chunk_tokens,
                                        int32_t tf_num_chunks, int32_t* cu_seqlens_local_host,
                                        int64_t* local_to_global_host);
cpattn_status cpattn_partition_tf(const cpattn_tensor* src_global, cpattn_tensor* dst_local,
                                  const int32_t* cu_seqlens_global_dev, int32_t num_seqs,
                                  int32_t cp, int32_t rank, int32_t tf_chunk_tokens,
                                  int32_t tf_num_chunks, void* stream);
cpattn_status cpattn_unpartition_tf(const cpattn_tensor* src_local, cpattn_tensor* dst_global,
                                    const int32_t* cu_seqlens_global_dev, int32_t num_seqs,
                                    int32_t cp, int32_t rank, int32_t tf_chunk_tokens,
                                    int32_t tf_num_chunks, void* stream);

/* ---- height/width token split ----------------------------------------------
 * LongCat-Video context-parallel page (split_tensor_in_cp_2d,
 * get_optimal_split): video latent tokens are split along height, then width,
 * with the factors chosen automatically as the split closest to square.
 * Readings taken (the page gives no formula): every sample is frames x H x W
 * tokens in row-major order; cp = split_h * split_w with H % split_h == 0 and
 * W % split_w == 0, choosing the split whose per-rank tile
 * (H/split_h) x (W/split_w) is closest to square (ties: smaller split_h);
 * rank r holds grid cell (r / split_w, r mod split_w) of every frame, frame
 * by frame, cell rows top to bottom and each left to right.  Attention over
 * such shares is order-free under CPATTN_MASK_BIDIR, which the ring steps
 * accept at any cp (each local sequence is one block of rows).
 * cpattn_split_hw returns the factors (CPATTN_ERR_INVALID_ARG when no even
 * split exists); the index and gather/scatter functions follow the zigzag
 * ones above with cp = split_h * split_w and every sequence frames*H*W long. */
cpattn_status cpattn_split_hw(int32_t H, int32_t W, int32_t cp, int32_t* split_h, int32_t* split_w);
cpattn_status cpattn_partition_index_hw(const int32_t* cu_seqlens_global_host, int32_t num_seqs, int32_t frames,
                                        int32_t H, int32_t W, int32_t split_h, int32_t split_w, int32_t rank,
                                        int32_t* cu_seqlens_local_host, int64_t* local_to_global_host);
cpattn_status cpattn_partition_hw(const cpattn_tensor* src_global, cpattn_tensor* dst_local,
                                  const int32_t* cu_seqlens_global_dev, int32_t num_seqs, int32_t frames,
                                  int32_t H, int32_t W, int32_t split_h, int32_t split_w, int32_t rank,
                                  void* stream);
cpattn_status cpattn_unpartition_hw(const cpattn_tensor* src_local, cpattn_tensor* dst_global,
                                    const int32_t* cu_seqlens_global_dev, int32_t num_seqs, int32_t frames,
                                    int32_t H, int32_t W, int32_t split_h, int32_t split_w, int32_t rank,
                                    void* stream);

/* ---- Ulysses sequence <-> head exchange ------------------------------------
 * "Scaling Video Training with Parallelism", SP landscape (DeepSpeed-Ulysses;
 * USP / LoongTrain 2D-Attention): Ulysses shards the sequence and exchanges
 * all-to-all around attention, so that member g of an n-way group holds all
 * tokens of head group g (heads [g*H/n, (g+1)*H/n)); the head count must
 * divide by n.  With every shard on one device the exchange is a gather:
 *   shards        array of n_shards THD views [T_s, H, d], in rank order
 *                 (contiguous token ranges of the packed batch)
 *   gathered      [>= sum T_s, H/n_shards, d]; rows of shard s start at row
 *                 sum_{s'<s} T_s'
 *   group         head group g in [0, n_shards)
 * cpattn_seq_to_head copies the shards' head group g into `gathered`;
 * cpattn_head_to_seq writes it back (the exchange after attention), leaving
 * the shards' other heads untouched.  dtype and head_dim must match.  Bytes
 * are copied bit-exact, one strided copy per shard on `stream`.  Attention
 * on the gathered tensors is cpattn_fwd_step / cpattn_bwd_step with cp = 1. */
cpattn_status cpattn_seq_to_head(const cpattn_tensor* shards, int32_t n_shards, int32_t group,
                                 cpattn_tensor* gathered, void* stream);
cpattn_status cpattn_head_to_seq(const cpattn_tensor* gathered, int32_t n_shards, int32_t group,
                                 cpattn_tensor* shards, void* stream);

/* Exact number of allowed (query, key) pairs per head between rank `rank`'s
 * queries and the keys it holds at ring step `step` (host-only, closed form
 * per sequence).  This is the count behind FLOP accounting from real
 * sequence lengths ("Speeding up Variable-Length Training ...", section A2,
 * loss and FLOPS accounting): forward 4*d*Hq*pairs, backward 10*d*Hq*pairs.
 * Returns -1 on invalid arguments. */
int64_t cpattn_count_pairs(const int32_t* cu_seqlens_global_host, int32_t num_seqs,
                           cpattn_mask_mode mask_mode, const cpattn_step* step);

/* Source rank of a ring step: the rank whose K/V share rank step->rank holds
 * at step step->step, (rank - step) mod cp ("Scaling Video Training with
 * Parallelism", section 2, Ring Attention paragraph: the K/V blocks move one
 * rank along the ring per step, so step 0 is the rank's own share).  The
 * dK/dV accumulators cpattn_bwd_step adds into belong to this rank.  Host
 * only; returns -1 for a NULL step or cp < 1 or rank/step outside [0, cp). */
int32_t cpattn_step_source(const cpattn_step* step);

/* ---- workspace -------------------------------------------------------------
 * Bytes of device workspace any call below needs for a rank with tokens_q
 * local query rows, tokens_k local key rows and num_seqs sequences. */
size_t cpattn_workspace_size(int64_t tokens_q, int64_t tokens_k, int32_t num_seqs);

/* Waits for `stream`, then reads the device-side status the last call on
 * this workspace left (CPATTN_OK or CPATTN_ERR_INVALID_ARG for a bad
 * device cu_seqlens array). */
cpattn_status cpattn_workspace_status(const void* workspace, void* stream, cpattn_status* status_out);

/* ---- forward step ----------------------------------------------------------
 * Blockwise attention of rank step->rank's local queries against the K/V
 * share it holds at ring step step->step ("Scaling Video Training with
 * Parallelism", section 2, Ring Attention paragraph).  Masks are applied on
 * positions in the unsplit sequences, recovered from the zigzag rule (from
 * the balanced split for TF_BLOCK at cp > 1, where every tile the scheduler
 * emits is fully allowed or fully skipped).
 *   q            [Tq, Hq, d]      local queries (rank step->rank)
 *   k, v         [Tk, Hkv, d]     K/V share of rank (rank - step) mod cp
 *   cu_seqlens_q_dev, cu_seqlens_k_dev  local int32[num_seqs+1]; for cp > 1
 *                and for CAUSAL / TF_BLOCK the per-sequence lengths of q and k
 *                must match (every rank's share has the same lengths); for
 *                CAUSAL at cp > 1 they are even (two zigzag chunks).
 *   out_partial  [Tq, Hq, d]      same dtype as q; every row is overwritten
 *                                 (0 for rows with no key, including rows
 *                                 past cu_seqlens_q[num_seqs] in a padded
 *                                 buffer)
 *   lse_partial_dev  fp32 [Hq][Tq]  (-inf for rows with no key)
 * Fully masked tiles are skipped by a device-side tile scheduler. */
cpattn_status cpattn_fwd_step(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                              const int32_t* cu_seqlens_q_dev, const int32_t* cu_seqlens_k_dev,
                              int32_t num_seqs, cpattn_mask_mode mask_mode, const cpattn_step* step,
                              float softmax_scale, cpattn_tensor* out_partial, float* lse_partial_dev,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- allocation-free forward step -------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as cpattn_fwd_step, with the schedule workspace taken from a
 * device array inside the library instead of a caller buffer.  The array is
 * CPATTN_SCRATCH_BYTES per GPU, held from the library's first call on that
 * GPU until the process ends; a shape whose cpattn_workspace_size(Tq, Tk,
 * num_seqs) exceeds it returns CPATTN_ERR_WORKSPACE before anything is
 * enqueued (16 MiB covers about 1.9M local query rows with as many key rows).
 * The call allocates nothing.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * ordered by the caller.  Nothing in the array needs clearing between calls.
 * A bad device cu_seqlens array leaves out_partial / lse_partial untouched,
 * as for cpattn_fwd_step; its status stays in the array, unreported.
 * Arguments and outputs otherwise as cpattn_fwd_step. */
#define CPATTN_SCRATCH_BYTES (16 * 1024 * 1024)
cpattn_status cpattn_fwd_step_noalloc(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                      const int32_t* cu_seqlens_q_dev, const int32_t* cu_seqlens_k_dev,
                                      int32_t num_seqs, cpattn_mask_mode mask_mode, const cpattn_step* step,
                                      float softmax_scale, cpattn_tensor* out_partial, float* lse_partial_dev,
                                      void* stream);

/* ---- LSE merge -------------------------------------------------------------
 * "Scaling Video Training with Parallelism", section 2, Ring Attention
 * paragraph: each ring step yields attention over one K/V block, and the
 * blocks' results are combined into attention over all keys (the page does
 * not print the combination; this is the log-sum-exp union it implies).
 * Folds one step's partial result into the running result, in place, as the
 * softmax over the union of two disjoint key sets:
 *     lse' = log(exp(lse) + exp(lse_p))
 *     out' = exp(lse - lse') * out + exp(lse_p - lse') * out_p
 * Rows with lse_p = -inf pass through bit-exact (and are not read);
 * running rows at -inf take the partial, or 0 when lse_p is -inf too, so
 * out_dev needs no initialisation: the starting state is lse = -inf.
 *   out_dev      fp32 [T][H][d] dense, running output (in/out)
 *   lse_dev      fp32 [H][T], running LSE (in/out)
 *   out_partial  [T, H, d] bf16 or fp32 view
 *   lse_partial_dev fp32 [H][T] */
cpattn_status cpattn_merge(float* out_dev, float* lse_dev, const cpattn_tensor* out_partial,
                           const float* lse_partial_dev, void* stream);

/* Sets count fp32 values at dst_dev to `value`: the ring's starting state
 * before the first merge (running lse = -inf: a result over no keys) and the
 * zeroed gradient accumulators that cpattn_bwd_step adds into.  dst_dev 16-byte aligned; count 0 enqueues
 * nothing.  A kernel, not a memset, so it records into HIP graphs like the
 * other calls.  INVALID_ARG for a NULL or misaligned pointer or count < 0. */
cpattn_status cpattn_fill_f32(float* dst_dev, int64_t count, float value, void* stream);

/* ---- backward --------------------------------------------------------------
 * "Scaling Video Training with Parallelism", section 1: splitting a sample
 * over ranks must leave the loss (and so its gradients) unchanged; the
 * backward of the ring therefore differentiates attention over the whole
 * sequence, one K/V share at a time, from the final merged O and LSE.
 *
 * Backward preprocess: delta_dev[h][t] = <dout[t,h,:], out[t,h,:]>, with out
 * the final merged fp32 output (dense [T][H][d], all T*H rows read).
 *   dout      [T, H, d] bf16 or fp32 view (T = dout->tokens)
 *   delta_dev fp32 [H][T], written for every row
 * INVALID_ARG for NULL or misaligned out/delta when T > 0. */
cpattn_status cpattn_bwd_preprocess(const float* out_dev, const cpattn_tensor* dout,
                                    float* delta_dev, void* stream);

/* One ring step of the backward ("Scaling Video Training with Parallelism",
 * section 1: the gradient of the unsplit loss; section 2: the same blockwise
 * ring, one K/V share per step), recomputing P from the saved final LSE:
 *     P_ij = exp(scale <q_i,k_j> - lse_i),  dS_ij = P_ij (<dO_i,v_j> - delta_i)
 *     dq_accum[i]  += scale * sum_j dS_ij k_j
 *     dk_accum[j]  += scale * sum_i dS_ij q_i     (summed over a GQA group)
 *     dv_accum[j]  += sum_i P_ij dO_i             (summed over a GQA group)
 * j runs over the keys of source rank (rank - step) mod cp; dk/dv_accum are
 * that source's buffers.  Accumulators are fp32 dense, += (caller zeroes
 * them once).  lse_dev / delta_dev: fp32 [Hq][Tq] from the forward merge and
 * cpattn_bwd_preprocess. */
cpattn_status cpattn_bwd_step(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                              const cpattn_tensor* dout, const float* lse_dev, const float* delta_dev,
                              const int32_t* cu_seqlens_q_dev, const int32_t* cu_seqlens_k_dev,
                              int32_t num_seqs, cpattn_mask_mode mask_mode, const cpattn_step* step,
                              float softmax_scale, float* dq_accum_dev, float* dk_accum_dev,
                              float* dv_accum_dev, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- Dynamic-CP microbatch planner (host only) -----------------------------
 * "Speeding up Variable-Length Training with Dynamic Context Parallelism and
 * NVIDIA Megatron Core", section A2 (data scheduling model, Eq. 1-3) and
 * section A7 (zero-overhead runtime, Fig. 7): pack a global batch of
 * variable-length samples into microbatches and give each microbatch its
 * own power-of-two context-parallel size, so that short samples are not
 * split and every rank gets the same modelled work.  The page describes the
 * steps in words; the readings (constants, order, tie-breaks) are:
 *   - `gpus` ranks share the data/context-parallel work of one pipeline
 *     stage; a microbatch of cp size c occupies one slot on each rank of an
 *     aligned group of c ranks; every rank runs m slots.
 *   - workload w(S) = work_quad*S^2 + work_lin*S; a rank's share of a
 *     sample under cp size c is w(S)/c and its memory is S tokens for c = 1,
 *     else S rounded up to 2c equal chunks, over c (the zigzag split).
 *   - quota W = total workload / (gpus * m) (Eq. 1-3 with equal m).
 *   - stage 1: each sample gets the smallest power-of-two c <= max_cp with
 *     share <= W and tokens <= mem_tokens (max_cp if the quota is never
 *     met); samples with c > 1 open their own microbatch.
 *   - stage 2: those microbatches, heaviest first, take the lightest
 *     unsplit samples while quota and memory hold.
 *   - stage 3: the remaining samples, heaviest first, go to the least-loaded
 *     cp = 1 microbatch with room; there are gpus*m - sum(c) of those.
 *   - placement: split microbatches, largest c first, on the free aligned
 *     group of least load; cp = 1 microbatches on the least-loaded rank.
 *   - step time: max over ranks of V*sum(slot shares) + (p-1)*max(slot
 *     share), which is Eq. 1's W (m V + p - 1) for equal shares.
 *   - m runs over [m_min, m_max] within knee_radius of the knee of the
 *     budget curve max(total/(gpus m), max w / max_cp) (the point farthest
 *     below the chord of the normalised curve); knee_radius < 0 searches
 *     every m.  The least step time wins; ties go to the smaller m.
 * Decisions are exact integer comparisons (the knee: IEEE double); ties go
 * to the lower index, so the plan is a deterministic function of the input.
 * Host memory only, thread-safe, no GPU involved. */
typedef struct {
    int32_t gpus;         /* ranks in the pool, 1..65536, a multiple of max_cp */
    int32_t max_cp;       /* largest cp size, a power of two <= gpus */
    int32_t pp;           /* pipeline stages p, 1..4096 */
    int32_t vpp;          /* virtual stages per pipeline rank V, 1..4096 */
    int64_t mem_tokens;   /* tokens one rank holds for one microbatch, >= 1 */
    int64_t work_quad;    /* a in w(S) = a S^2 + b S, 0..2^16 */
    int64_t work_lin;     /* b, 0..2^32; a + b > 0 */
    int32_t m_min;        /* microbatches per rank searched: m_min..m_max, */
    int32_t m_max;        /*   1 <= m_min <= m_max <= 4096, gpus*m_max <= 2^22 */
    int32_t knee_radius;  /* search |m - knee| <= knee_radius; < 0: all m */
} cpattn_dcp_config;

/* Result arrays are caller-owned host memory. */
typedef struct {
    int32_t m;                /* out: chosen microbatches per rank */
    int32_t knee;             /* out: knee of the budget curve */
    int32_t num_buckets;      /* out: microbatches in the plan (<= gpus*m) */
    double step_time;         /* out: modelled step time, workload units */
    int32_t* sample_bucket;   /* [n]   microbatch of every sample */
    int32_t* bucket_cp;       /* [cap] cp size */
    int32_t* bucket_slot;     /* [cap] slot 0..m-1 */
    int32_t* bucket_rank;     /* [cap] first rank of its group (a multiple of cp) */
    int64_t* bucket_tokens;   /* [cap] tokens per rank */
    double* bucket_load;      /* [cap] sum of w(S) over its samples */
    double* times;            /* [m_max-m_min+1] step time per m; -1 infeasible,
                                 -2 outside the knee's radius */
    double* budget;           /* [m_max-m_min+1] budget curve */
    int32_t bucket_capacity;  /* entries of the bucket arrays, >= gpus*m_max */
} cpattn_dcp_plan;

/* Plans lengths[n] (1 <= n <= 2^24, 1 <= length <= 2^22).  Microbatches are
 * numbered split ones first (by workload, heaviest first), then the cp = 1
 * ones.  INVALID_ARG on a bad argument; INFEASIBLE when no m in the range
 * yields a plan: a sample over the memory cap even at max_cp, split
 * microbatches needing more cells than gpus*m, or unsplit samples that do
 * not fit the memory of the cp = 1 microbatches left over. */
cpattn_status cpattn_dcp_plan_batch(const int32_t* lengths, int32_t n, const cpattn_dcp_config* cfg,
                                    cpattn_dcp_plan* out);

/* Eq. 1-3 of the same section: per-microbatch workload quota W[i] of each of
 * n data-parallel ranks running m[i] >= 1 microbatches, with V = vpp virtual
 * stages and p = pp pipeline stages, such that every rank finishes together
 * (W_i (m_i V + p - 1) equal) and sum_i W_i m_i = total.  Double precision;
 * INVALID_ARG on a bad argument. */
cpattn_status cpattn_dcp_quotas(const int32_t* m, int32_t n, int32_t vpp, int32_t pp, double total, double* W);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_H */

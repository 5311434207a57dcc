/*
 * dpsync.h -- C ABI of libdpsync: data-parallel gradient and parameter
 * synchronisation on one MI355X, with K data-parallel ranks emulated as K
 * buffers in the GPU's HBM.
 *
 * Interface model: one call per collective taking (send buffers, receive
 * buffers, element count, data type, reduction op, stream), with every
 * operation bound to a stream that the caller synchronises (CMU 11-868
 * L14-L15 notes, sections "NCCL's five building blocks" and the ncclAllReduce
 * listing that follows "Ring AllReduce: ReduceScatter, then AllGather"). The
 * communicator is replaced by explicit host arrays of K device pointers, one
 * per emulated rank.
 *
 * Common conventions
 *   - Pointer arrays (send, recv, ...) are HOST arrays of K DEVICE pointers.
 *     They are read during the call only (copied into kernel arguments).
 *   - Every device buffer belongs to the caller; the library never allocates,
 *     frees or synchronises in these calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream of
 *     the current device) and the call returns at once. Completion is the
 *     caller's stream synchronisation or event.
 *   - Arguments are validated before anything is enqueued. On any error
 *     nothing runs and outputs are untouched. The library never aborts or
 *     prints.
 *   - Element counts are per rank. n == 0 is a no-op returning DP_OK.
 *   - Every pointer must be aligned to its element size. A faster path is
 *     taken where the K inputs and the output of a shard share their address
 *     phase modulo 16 bytes.
 *   - Shards: L = dp_shard_len(n, k) = ceil(n / k). Shard c covers elements
 *     [c*L, min((c+1)*L, n)) of every rank; the last shards are short, or
 *     empty when n < k*L, and are padded to L ("Sharding and Parallelism",
 *     section "Global arrays and device-local shards": the local shard is
 *     A[d/q] and non-divisible sizes need padding).
 *   - Reduction order: the element of shard c is the left fold of the K rank
 *     values in ring order rho_c = (c+1, c+2, ..., c+K-1, c) mod K, the order
 *     in which a unidirectional ring r -> r+1 accumulates chunk c when rank c
 *     ends up owning it (CMU notes, "Ring AllReduce: ReduceScatter, then
 *     AllGather"). Sums are accumulated in fp32 (wrapping uint32 for int32)
 *     and results are bit-identical for any s_chunks, stream or run.
 *   - s_chunks (S >= 1): each shard is cut into S contiguous sub-chunks of
 *     ceil(L/S) elements, processed in sub-chunk order, as messages are chopped
 *     into S pieces for pipelining (CMU notes, "Why a ring: chop the data so
 *     transfers pipeline"). It changes only the work decomposition.
 */
#ifndef DPSYNC_H
#define DPSYNC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DP_MAX_K 64

typedef enum {
    DP_OK = 0,
    DP_ERR_INVALID_ARG = 1,  /* null pointer, k out of [1, DP_MAX_K], s_chunks < 1,
                                misaligned pointer, size overflow, bad token counts */
    DP_ERR_UNSUPPORTED = 2,  /* dtype/op outside the enums, or AVG/weighted on DP_I32 */
    DP_ERR_ALIAS = 3,        /* buffers overlap other than in the documented in-place forms */
    DP_ERR_HIP = 4,          /* a HIP launch failed; see dp_last_hip_error() */
    DP_ERR_SCRATCH = 5       /* the call's workspaces exceed DP_STATIC_SCRATCH_BYTES
                                (dp_fsdp_layer_static only) */
} dp_status_t;

typedef enum { DP_F32 = 0, DP_BF16 = 1, DP_I32 = 2 } dp_dtype_t;

typedef enum {
    DP_SUM = 0,  /* plain sum */
    DP_AVG = 1   /* sum, then one IEEE division of the fp32 sum by K (the average
                    gradient of the data-parallel step, CMU notes section
                    "Intuition: data parallelism has only one thing to
                    synchronize", step 3) */
} dp_op_t;

/* ceil(n / k); 0 when n == 0 or k < 1. */
size_t dp_shard_len(size_t n, int k);

/* Static text for a status code (never NULL). */
const char *dp_status_string(int status);

/* hipError_t value behind the last DP_ERR_HIP returned on this thread (0 if none). */
int dp_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int dp_version(void);

/*
 * ReduceScatter ("Sharding and Parallelism", section "The cost of the
 * inserted collectives", T_RS,ring: every rank starts with a reducible buffer
 * and ends with its 1/K share; CMU notes, ring phase 1).
 *   send[r] : n elements of rank r (dtype dt).
 *   recv[c] : L = dp_shard_len(n,k) elements; receives shard c, the ring-order
 *             fold over the K ranks of elements [c*L, c*L + n_c), then op's
 *             epilogue (DP_AVG divides by K in fp32; bf16 is rounded once,
 *             to nearest even, after the fp32 sum); elements n_c..L-1 are
 *             written as zero.
 *   In place: recv[c] == send[c] + c*L (in elements) for every c is allowed
 *   when n == k*L; any other overlap of a recv range with a send or recv
 *   range returns DP_ERR_ALIAS.
 */
dp_status_t dp_reduce_scatter(const void *const *send, void *const *recv, size_t n, int k,
                              int dt, int op, int s_chunks, void *stream);

/*
 * AllGather (same page and section, T_AG,ring: each rank starts with B/X and
 * ends with all of B; CMU notes, ring phase 2).
 *   send[c] : shard c, L elements of which the first n_c are read (pads ignored).
 *   recv[r] : n elements; recv[r][c*L + j] = send[c][j] for every rank r.
 *   In place: send[c] == recv[c] + c*L for every c is allowed (shard c is then
 *   already at its place in rank c's output and is copied to the other ranks
 *   only); other overlaps return DP_ERR_ALIAS.
 */
dp_status_t dp_all_gather(const void *const *send, void *const *recv, size_t n, int k,
                          int dt, int s_chunks, void *stream);

/*
 * A ReduceScatter of one buffer set and an AllGather of another, in one launch:
 * the step of a bucketed sync in which bucket b+1 is reduced while bucket b is
 * gathered, so that the two phases of consecutive buckets pipeline the way the
 * chunks of a ring do (CMU notes, "Why a ring: chop the data so transfers
 * pipeline"). On one GPU it also balances HBM traffic: the ReduceScatter reads
 * k bytes for every byte it writes and the AllGather writes k for every byte
 * it reads.
 *   Same results as dp_reduce_scatter(rs_send, rs_recv, rs_n, k, dt, op,
 *   s_chunks) followed by dp_all_gather(ag_send, ag_recv, ag_n, k, dt,
 *   s_chunks), bit for bit; each operation follows that call's buffer and
 *   in-place rules, and no buffer of one operation may overlap a buffer of
 *   the other (DP_ERR_ALIAS). rs_n or ag_n may be 0 (then only the other
 *   operation runs; the arrays of the empty one must be non-NULL but are not
 *   read).
 *   Cache use: the ReduceScatter stores its shards with ordinary stores, so
 *   that they can stay in the caches for the AllGather that reads them next
 *   (this call's AllGather half in the next pipeline step); in the
 *   ReduceScatter-only form only when the K shards fit in 128 MiB, else with
 *   the nontemporal hint, as dp_reduce_scatter always stores them.
 */
dp_status_t dp_reduce_scatter_all_gather(const void *const *rs_send, void *const *rs_recv,
                                         size_t rs_n, const void *const *ag_send,
                                         void *const *ag_recv, size_t ag_n, int k, int dt, int op,
                                         int s_chunks, void *stream);

/*
 * AllReduce = ReduceScatter followed by AllGather (CMU notes, section "NCCL's
 * five building blocks"; T_AR,ring equation in "Sharding and Parallelism").
 *   send[r], recv[r] : n elements. Every recv[r] receives the full reduced
 *   vector, bit-identical to dp_all_gather(dp_reduce_scatter(send)).
 *   By default one pass folds each shard in ring order and writes the result
 *   to all K outputs (K*n*s bytes read and K*n*s written, against (K+1)*n*s
 *   each way for the two collectives); with DP_LAUNCH_TWO_PHASE
 *   (dp_all_reduce_ex) shard c is first reduced into recv[c] at offset c*L,
 *   then copied from there to the other ranks. No workspace either way.
 *   In place: for every r, recv[r] either equals send[r] or overlaps no send
 *   buffer; receive buffers are pairwise disjoint.
 */
dp_status_t dp_all_reduce(const void *const *send, void *const *recv, size_t n, int k,
                          int dt, int op, int s_chunks, void *stream);

/*
 * Token-weighted AllReduce for uneven per-rank token counts (the imbalance of
 * variable-length SFT batches in "Using ODC to Accelerate AMD SFT Training",
 * section "Why FSDP is Slow: ... Workload-imbalance Bubble"):
 *   recv[r][i] = (sum_r f32(t_r) * send[r][i]) / f32(sum_r t_r)
 * with the products folded in ring order without fused multiply-add and one
 * IEEE division at the end. dt is DP_F32 or DP_BF16 (fp32 accumulation).
 *   tokens : HOST array of k counts, each >= 0, with a positive int64 sum.
 *   Buffers and in-place rule as dp_all_reduce.
 */
dp_status_t dp_weighted_reduce(const void *const *send, void *const *recv,
                               const int64_t *tokens, size_t n, int k, int dt, int s_chunks,
                               void *stream);

/*
 * FSDP layer step, fp32, row-major ("Sharding and Parallelism", section "Real
 * HLO before and after partitioning", FSDP fixture: AllGather(w[64,512]) ->
 * w[512,512] then the local dot; section "FSDP and ZeRO": the forward pass
 * gathers W[D,F] before the dot and the backward pass reduce-scatters the
 * gradient).
 *   x_local[r]  : [m_local, d]   activations of rank r
 *   w_shard[c]  : [R, f], R = ceil(d/k): rows c*R .. min((c+1)R, d) of W,
 *                 pad rows ignored
 *   dy_local[r] : [m_local, f] upstream gradient of rank r, or NULL for the
 *                 forward step only
 *   w_full[r]   : [d, f] workspace, receives the gathered W
 *   y_local[r]  : [m_local, f] = x_local[r] . W   (fp32 MFMA)
 *   dw_full[r]  : [d, f] workspace, receives x_local[r]^T . dy_local[r]
 *                 (unused and may be NULL when dy_local is NULL)
 *   dw_shard[c] : [R, f] receives rows c*R.. of sum_r dw_full[r] (ring-order
 *                 fp32 ReduceScatter, DP_SUM), pad rows zero (may be NULL
 *                 when dy_local is NULL)
 *   All buffers must be pairwise disjoint (DP_ERR_ALIAS otherwise).
 */
dp_status_t dp_fsdp_layer(int k, int64_t m_local, int64_t d, int64_t f,
                          const float *const *x_local, const float *const *w_shard,
                          const float *const *dy_local, float *const *w_full,
                          float *const *y_local, float *const *dw_full, float *const *dw_shard,
                          void *stream);

/*
 * dp_fsdp_layer with the input gradient of the backward pass as well
 * ("Sharding and Parallelism", section "FSDP and ZeRO": the backward pass
 * needs the gathered weight for the gradient that flows to the previous layer
 * while the weight gradient is reduce-scattered):
 *   dx_local[r] : [m_local, d] = dy_local[r] . W^T (fp32 MFMA), or NULL (then
 *                 exactly dp_fsdp_layer). Requires dy_local; must be disjoint
 *                 from every other buffer (DP_ERR_ALIAS).
 * Where the shapes allow (K <= 8; m_local, d, f multiples of 64; shards of a
 * multiple of 64 rows; d divisible by K; 16-byte aligned buffers) the whole
 * step is one launch in which the dx dot, the forward dot and the weight
 * gradient with its ReduceScatter run side by side; other shapes run separate
 * launches. The results are the same either way up to the summation order of
 * the dots (dw_shard is always the ring-order ReduceScatter of dw_full).
 */
dp_status_t dp_fsdp_layer_ex(int k, int64_t m_local, int64_t d, int64_t f,
                             const float *const *x_local, const float *const *w_shard,
                             const float *const *dy_local, float *const *w_full,
                             float *const *y_local, float *const *dx_local,
                             float *const *dw_full, float *const *dw_shard, void *stream);

/*
 * dp_fsdp_layer_ex for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the gathered weights w_full[r] and the per-rank weight
 * gradients dw_full[r] are kept in a static device buffer of the library
 * instead of caller workspaces. Same arguments, results and validation as
 * dp_fsdp_layer_ex without w_full and dw_full (dy_local NULL: forward only,
 * dw_shard is then ignored and dx_local must be NULL; dx_local NULL: no input
 * gradient). The same kernels run, so the results are bit-identical to
 * dp_fsdp_layer_ex with caller workspaces of the same shapes.
 *   Limit: 2 * k * roundup256(d * f * 4 bytes) <= DP_STATIC_SCRATCH_BYTES
 *   (32 MiB: e.g. K = 8 ranks with d = f = 512 use 16 MiB), else
 *   DP_ERR_SCRATCH with nothing enqueued.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine). Each GPU holds one copy of the buffer, shared by every call on that
 * GPU: calls on one GPU that can run at the same time (on different streams,
 * or from different threads) race on it; serialise them. Every call
 * overwrites the parts it uses, so nothing carries over from earlier calls.
 */
#define DP_STATIC_SCRATCH_BYTES (32u << 20)

dp_status_t dp_fsdp_layer_static(int k, int64_t m_local, int64_t d, int64_t f,
                                 const float *const *x_local, const float *const *w_shard,
                                 const float *const *dy_local, float *const *y_local,
                                 float *const *dx_local, float *const *dw_shard, void *stream);

/*
 * Dense bf16 GEMM used as the compute side of concurrent computation and
 * communication (the GEMM kernel of a (GEMM, collective) pair, "Optimizing ML
 * Concurrent Computation and Communication with GPU DMA Engines", section
 * "Problem Formulation").
 *   c[m,n] = a[m,kk] . b[kk,n]: a is [m,kk], b is [kk,n], c is [m,n], all
 *   row-major bf16 device buffers; fp32 accumulation on MFMA, result rounded
 *   to nearest even bf16. dp_gemm_bf16_ex with DP_LAUNCH_B_NK takes b as
 *   [n,kk] instead (c = a . b^T, both operands k-contiguous: the linear-layer
 *   weight layout).
 *   m, n, kk in [1, 2^24] and every pointer aligned to its 2-byte element
 *   (else DP_ERR_INVALID_ARG); c must not overlap a or b (DP_ERR_ALIAS).
 *   The products are summed over k in ascending steps of 16 into fp32 (each
 *   step one matrix-core instruction, zero-padded past kk), the same order for
 *   every shape, layout and variant, so all give the same bits. Rows that are
 *   16-byte aligned (a and b 16-byte aligned, kk a multiple of 8, and n a
 *   multiple of 8 for b [kk,n]) take the staged kernels: m and n multiples of
 *   256 with kk a multiple of 128 and >= 256 (>= 384 for b [n,kk]), or a
 *   multiple of 64 and >= 1024, a 4-wave kernel (one wave per SIMD), other
 *   shapes the 8-wave kernel
 *   (guarded edge tiles where needed); other rows a slower kernel that
 *   gathers operands element by element. c may start at any element; where
 *   it is 16-byte aligned the 4-wave kernels write it in 16-byte stores.
 */
dp_status_t dp_gemm_bf16(const void *a, const void *b, void *c, int64_t m, int64_t n,
                         int64_t kk, void *stream);

/*
 * Launch options for running a collective beside other GPU work (concurrent
 * computation and communication, "Optimizing ML Concurrent Computation and
 * Communication with GPU DMA Engines", section Q2: schedule prioritisation and
 * resource partitioning decide how the collective and the GEMM share CUs).
 *   max_workgroups : 0 = the default grid (one workgroup per tile). > 0 caps
 *                    the sync kernels at that many resident workgroups
 *                    (256 threads each), which then walk the tiles
 *                    persistently; results are bit-identical either way.
 *   flags          : DP_LAUNCH_SHARE_CU selects, for dp_gemm_bf16_ex, the GEMM
 *                    variant with a smaller register footprint (8 waves,
 *                    depth-32 k stages, 198 VGPRs) so that a default sync
 *                    workgroup can be resident on the same CU as a GEMM
 *                    workgroup. DP_LAUNCH_TWO_PHASE makes
 *                    dp_all_reduce_ex / dp_weighted_reduce_ex run a
 *                    ReduceScatter then an AllGather instead of the one-pass
 *                    kernel (same results). DP_LAUNCH_LEAN selects, for the
 *                    ReduceScatter and AllReduce kernels, the variant with one
 *                    16-byte vector per lane per rank and at most 64 VGPRs
 *                    (same results), and for the GEMM the 8-wave variant with
 *                    depth-64 stages (224 VGPRs): one lean sync workgroup fits
 *                    in the registers that GEMM workgroup leaves free on a CU,
 *                    so the two kernels can be resident together. (The default
 *                    GEMM runs one wave per SIMD and uses all of its registers
 *                    where the shape allows; every GEMM variant gives the same
 *                    bits.) DP_LAUNCH_B_NK: dp_gemm_bf16_ex's b is stored
 *                    [n,kk] (c = a . b^T). Other calls ignore the flags.
 *   reserved       : must be zero.
 * A NULL opts pointer means all defaults. Invalid fields return
 * DP_ERR_INVALID_ARG.
 */
#define DP_LAUNCH_SHARE_CU 1
#define DP_LAUNCH_TWO_PHASE 2
#define DP_LAUNCH_LEAN 4
#define DP_LAUNCH_B_NK 8

typedef struct {
    int max_workgroups;
    int flags;
    int reserved[2];
} dp_launch_opts_t;

/* The same operations as dp_reduce_scatter, dp_all_gather, dp_all_reduce and
 * dp_gemm_bf16, with launch options. */
dp_status_t dp_reduce_scatter_ex(const void *const *send, void *const *recv, size_t n, int k,
                                 int dt, int op, int s_chunks, const dp_launch_opts_t *opts,
                                 void *stream);
dp_status_t dp_all_gather_ex(const void *const *send, void *const *recv, size_t n, int k,
                             int dt, int s_chunks, const dp_launch_opts_t *opts, void *stream);
dp_status_t dp_all_reduce_ex(const void *const *send, void *const *recv, size_t n, int k,
                             int dt, int op, int s_chunks, const dp_launch_opts_t *opts,
                             void *stream);
dp_status_t dp_gemm_bf16_ex(const void *a, const void *b, void *c, int64_t m, int64_t n,
                            int64_t kk, const dp_launch_opts_t *opts, void *stream);
dp_status_t dp_weighted_reduce_ex(const void *const *send, void *const *recv,
                                  const int64_t *tokens, size_t n, int k, int dt, int s_chunks,
                                  const dp_launch_opts_t *opts, void *stream);

/*
 * Backward pass with the gradient AllReduce overlapped, bucket by bucket
 * ("CMU 11-868 L14-L15 ...", section "When to sync: gradient bucketing":
 * gradients appear layer by layer from the back, parameters sit in buckets in
 * that order, and a bucket is AllReduced as soon as every gradient in it is
 * ready while backward goes on computing earlier layers).
 *
 * Each rank's gradient is one flat bf16 vector of `total` elements made of
 * n_pieces weight gradients in backward order. Piece g is an [m, n] row-major
 * matrix at element `offset` (the pieces must tile [0, total) in order):
 *   grad[r][offset + i*n + j] = sum_s dy[g*k + r][i, s] * x[g*k + r][j, s]
 * i.e. dW = dY^T X for a linear layer, with dy [m, t] and x [n, t] stored
 * token-contiguous (t tokens per rank, t a multiple of 8, 16-byte aligned), bf16
 * in, fp32 accumulation on MFMA, bf16 out (the dp_gemm_bf16 kernel).
 * Bucket b covers [b*bucket_elems, min((b+1)*bucket_elems, total)).
 *
 * Schedule: on compute_stream, for each piece in order, the k GEMMs of that
 * piece; after them, every bucket whose elements are now all computed is
 * AllReduced (op DP_SUM or DP_AVG, bf16, fp32 accumulation in ring order, the
 * dp_all_reduce kernel) from grad into out on comm_stream, in bucket order.
 * The comm stream waits for the bucket with events[b] (recorded on
 * compute_stream after the bucket's last GEMM); events is a HOST array of at
 * least ceil(total / bucket_elems) hipEvent_t created by the caller.
 * When comm_stream == compute_stream everything runs in that one stream in the
 * same order (no overlap, events unused and may be NULL).
 * opts: DP_LAUNCH_SHARE_CU selects the GEMM variant that leaves room for a
 * sync workgroup on each CU; DP_LAUNCH_LEAN the AllReduce variant and the GEMM
 * variant that fit together on a CU; max_workgroups caps the AllReduce grid;
 * DP_LAUNCH_TWO_PHASE runs each AllReduce as ReduceScatter then AllGather.
 *
 * The results do not depend on the schedule: out equals dp_all_reduce of the
 * computed grad, bit for bit. out[r] may equal grad[r] (in place); other
 * overlaps between grad, out, dy and x return DP_ERR_ALIAS. Completion: the
 * gradients are final when compute_stream completes and the outputs when
 * comm_stream completes. All arguments are validated before anything is
 * enqueued; a launch failure part way returns DP_ERR_HIP with the earlier
 * work already enqueued.
 */
typedef struct {
    int64_t offset;  /* element offset of the piece in every rank's gradient vector */
    int64_t m, n;    /* the piece is an [m, n] row-major matrix */
} dp_grad_piece_t;

dp_status_t dp_backward_allreduce_overlap(int k, int n_pieces, const dp_grad_piece_t *pieces,
                                          int64_t t, const void *const *dy, const void *const *x,
                                          void *const *grad, void *const *out, int64_t total,
                                          int64_t bucket_elems, int op,
                                          const dp_launch_opts_t *opts, void *compute_stream,
                                          void *comm_stream, void *const *events, int n_events);

/*
 * On-demand communication: scatter-accumulate push ("Using ODC to Accelerate
 * AMD SFT Training", section "From Collective Primitives to Two One-sided P2P
 * Primitives", Figure 2: after computing a gradient, a rank pushes each shard
 * of it to the rank that owns the shard, which adds it into its gradient
 * accumulator Acc).
 *   grads[i] : push i's gradient (one rank's microbatch gradient), n elements
 *              of dt (DP_F32 or DP_BF16), i < np, 1 <= np <= DP_MAX_K
 *   acc[c]   : owner c's fp32 accumulator, L = dp_shard_len(n, k) elements
 *   Effect   : for i = 0, 1, ..., np-1 in that order,
 *              acc[c][j] = acc[c][j] + f32(grads[i][c*L + j]) for j < n_c
 *              (one fp32 addition each, no FMA); pads j >= n_c untouched.
 * One call with np pushes gives the same bits as np calls with one push each,
 * in the same order: an owner applying, in arrival order, all pushes that have
 * landed. Calls on one stream apply in issue order, so any push sequence has a
 * deterministic result, the left fold of the pushed values. The accumulators
 * must be pairwise disjoint and overlap no gradient (DP_ERR_ALIAS); gradients
 * may overlap one another. dt = DP_I32 returns DP_ERR_UNSUPPORTED. The fast
 * path needs 16-byte alignment of acc[c] and of every grads[i] + c*L; any
 * element alignment works.
 */
dp_status_t dp_scatter_accumulate(const void *const *grads, int np, int dt, float *const *acc,
                                  size_t n, int k, void *stream);

/*
 * On-demand communication: the per-minibatch settle ("Using ODC to Accelerate
 * AMD SFT Training", section "From Per-iteration to Per-minibatch
 * Synchronization": gradients accumulate over the minibatch and one settle at
 * its end makes them final before the optimizer reads them).
 *   acc[c] : owner c's fp32 accumulator (L elements)
 *   out[c] : owner c's settled shard, L elements of dt (DP_F32 or DP_BF16)
 *   Effect : out[c][j] = cast(acc[c][j] / divisor) for j < n_c (one IEEE fp32
 *            division, bf16 rounded to nearest even once), out[c][j] = 0 for
 *            n_c <= j < L. divisor = 1 gives the sum; the number of
 *            contributions gives the mean. With reset != 0 the accumulator's
 *            valid elements are set to zero afterwards, ready for the next
 *            minibatch.
 * divisor must be finite and non-zero (DP_ERR_INVALID_ARG). The outputs must
 * be pairwise disjoint and must not overlap any accumulator, except that with
 * dt = DP_F32 and reset = 0 out[c] may equal acc[c] (settle in place); other
 * overlaps return DP_ERR_ALIAS.
 */
dp_status_t dp_settle(float *const *acc, void *const *out, size_t n, int k, int dt, float divisor,
                      int reset, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DPSYNC_H */

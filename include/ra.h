/*
 * ra.h -- C ABI of libra.so: one rank's blockwise ring-attention step on an
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Ring attention keeps each rank's block of queries fixed
 * and passes key/value blocks around a ring until every query block has seen
 * every key/value block it needs ("Sequence Parallelism III: Ring Attention for
 * Context That Does Not Fit"; dictionary entry "context parallelism").  Each
 * arriving block yields a partial output and its log-sum-exp (DeDLOC guide,
 * "Step 3", local attention returning output and LSE), and partials are merged
 * by log-sum-exp rescaling (DeDLOC guide, "3. Online Softmax Rescaling Across
 * Decentralized Ranks").  Under a causal mask, blocks above the diagonal are
 * skipped (DeDLOC guide, "Best Practices", row "Causal Mask Handling").
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Tensor pointers are HIP device pointers owned by the caller.  The
 *   library never allocates, frees or synchronises; work is enqueued on the
 *   caller's stream (`stream` is a hipStream_t passed as void*, NULL = the
 *   null stream).  The caller keeps buffers alive until the stream completes.
 * Layouts.  Contiguous, row-major:
 *   q  [B, Sq, Hq,  D]   element type `dtype`
 *   k  [B, Sk, Hkv, D]   element type `dtype`
 *   v  [B, Sk, Hkv, D]   element type `dtype`
 *   o  [B, Sq, Hq,  D]   float32, normalised output
 *   lse[B, Sq, Hq]       float32, natural-log log-sum-exp of the scaled scores
 *                        of each (row, head), in O's row order.
 *   Query head h reads key/value head h / (Hq / Hkv) (consecutive grouping).
 * Positions.  Rows of q and k are a rank's tokens in its local order.  Spans
 *   give their global positions: local rows [off, off + len) of span i hold
 *   global tokens [start, start + len), spans concatenated in order.  The
 *   causal mask compares global positions: key j is visible to query i iff
 *   j <= i.
 * Empty rows.  A row that sees no key has the merge identity o = 0,
 *   lse = -inf.  Merging with the identity returns the other side bit-exactly.
 * Errors.  Every call returns RA_OK (0) or a negative status.  Arguments are
 *   validated before anything is enqueued, so on error nothing was enqueued and
 *   no output was touched; ra_last_error() describes the failure (thread-local
 *   string, valid until the next call on the same thread).  RA_E_HIP reports
 *   a failed kernel launch.
 * Threading.  The library keeps no state between calls; calls are reentrant.
 *   Calls that write the same output buffers must be ordered by the caller.
 */
#ifndef RA_H
#define RA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 1

/* status codes */
#define RA_OK 0
#define RA_E_INVAL (-1)       /* bad shape, divisibility, null pointer or flag */
#define RA_E_UNSUPPORTED (-2) /* dtype or head dimension not built            */
#define RA_E_HIP (-3)         /* the HIP runtime refused a launch             */

/* element types of q, k, v */
#define RA_DTYPE_F32 0
#define RA_DTYPE_BF16 1

/* chunk-to-rank orders */
#define RA_ORDER_CONTIGUOUS 0
#define RA_ORDER_ZIGZAG 1

/* ra_step flags */
#define RA_STEP_INIT 0u  /* overwrite (o, lse) with this block's partial     */
#define RA_STEP_ACCUM 1u /* merge this block's partial into (o, lse)         */

/* ra_ulysses_relayout directions */
#define RA_SEQ2HEAD 0
#define RA_HEAD2SEQ 1

/* token grouping of ra_ulysses_pieces tensors */
#define RA_GROUP_HEADS 0 /* tensor [B, s_loc, P_u runs]: piece j = run j */
#define RA_GROUP_SEQ 1   /* tensor [B, P_u blocks of s_loc tokens]: piece u = block u */

/* classes of a (query span, key span) pair */
#define RA_CLASS_SKIP 0 /* no pair visible                               */
#define RA_CLASS_FULL 1 /* every pair visible                            */
#define RA_CLASS_DIAG 2 /* some pairs visible: the diagonal needs a mask */

typedef struct ra_span {
  int64_t start; /* global position of the span's first token */
  int64_t len;   /* number of tokens                          */
} ra_span;

/* One ring step: a rank's fixed query rows against one arrived K/V block. */
typedef struct ra_step_desc {
  int32_t dtype;    /* RA_DTYPE_F32 or RA_DTYPE_BF16                         */
  int32_t B, Hq, Hkv, D;
  int64_t Sq, Sk;   /* rows of q and of k/v; each = sum of its span lengths   */
  int32_t causal;   /* 1: key j visible to query i iff j <= i; 0: all visible */
  float scale;      /* score scale, normally 1/sqrt(D)                        */
  int32_t n_qspans, n_kspans; /* 1 or 2 each                                  */
  ra_span qspans[2], kspans[2];
} ra_step_desc;

/*
 * ra_step -- one ring step (the per-step block computation of the DeDLOC
 * guide, "Step 3", plus the merge of its section 3, fused).
 *
 * flags == RA_STEP_INIT: (o, lse) := this block's partial result; rows that
 *   see no key of the block get (0, -inf).
 * flags == RA_STEP_ACCUM: (o, lse) := merge((o, lse), partial).  Rows that see
 *   no key are left untouched.
 * Key tiles that the mask hides entirely are neither loaded nor computed.
 * Requires: dtype/D in {F32: 64, 128; BF16: 64, 128}; Hq % Hkv == 0; spans of
 * non-negative length whose lengths sum to Sq (Sk); 16-byte aligned q, k, v, o.
 * Lengths need not be multiples of the kernel tiles.
 */
int ra_step(const ra_step_desc* d, const void* q, const void* k, const void* v,
            float* o, float* lse, uint32_t flags, void* stream);

/*
 * ra_lse_merge -- merge two partial results of the same rows (DeDLOC guide,
 * "3. Online Softmax Rescaling Across Decentralized Ranks"):
 *   m = max(lse_a, lse_b), w_x = exp(lse_x - m),
 *   o = (w_a o_a + w_b o_b) / (w_a + w_b),  lse = m + ln(w_a + w_b),
 * with (0, -inf) as the exact identity.  o_* are [rows, D] float32, lse_* are
 * [rows] float32.  o_out may alias o_a or o_b and lse_out may alias lse_a or
 * lse_b (element-wise in place); other overlaps are not allowed.  rows >= 0
 * (0 enqueues nothing), 1 <= D <= 4096.
 */
int ra_lse_merge(int64_t rows, int32_t D, const float* o_a, const float* lse_a,
                 const float* o_b, const float* lse_b, float* o_out,
                 float* lse_out, void* stream);

/* One rank of a ring of P, all of whose K/V shards are resident. */
typedef struct ra_rank_desc {
  int32_t dtype;  /* RA_DTYPE_F32 or RA_DTYPE_BF16 */
  int32_t B, Hq, Hkv, D;
  int64_t S;      /* global sequence length */
  int32_t P, rank;
  int32_t order;  /* RA_ORDER_CONTIGUOUS or RA_ORDER_ZIGZAG */
  int32_t causal;
  float scale;
} ra_rank_desc;

/*
 * ra_rank_forward -- rank `rank`'s P ring steps, run in ring order on one GPU.
 * At step s the rank holds the shard of rank (rank - s) mod P (the static ring
 * 0 -> 1 -> ... -> P-1 -> 0 of the DeDLOC guide, "The Geo-Distributed
 * Long-Context Crisis").  Shards follow the chunk order: contiguous, rank r
 * owns tokens [r S/P, (r+1) S/P); zigzag, the sequence is cut into 2P chunks
 * and rank r owns chunk r then chunk 2P-1-r (ringmaster "Layout": contiguous
 * shard and head_tail balancer; "Sequence Parallelism IV ... Load-Balanced
 * Rings").
 *   q_local  [B, S/P, Hq, D]       this rank's queries in its local order
 *   k_shards [P, B, S/P, Hkv, D]   shard p in rank p's local order; v_shards same
 *   o        [B, S/P, Hq, D] float32, lse [B, S/P, Hq] float32
 * Equivalent to ra_step INIT at step 0 followed by ACCUM steps; a step whose
 * whole block is masked is not launched.  Requires S % P == 0 (contiguous) or
 * S % (2P) == 0 (zigzag), 0 <= rank < P, and ra_step's requirements.
 */
int ra_rank_forward(const ra_rank_desc* d, const void* q_local,
                    const void* k_shards, const void* v_shards, float* o,
                    float* lse, void* stream);

/* Mask variants of the tile classifier (ringmaster "Status": sliding-window
 * attention through the kernel's window; packing / varlen).  Readings: a
 * window w > 0 (with the causal mask) lets query t see keys t-w+1 .. t;
 * packed sequences with boundaries 0 = c_0 < c_1 < ... < c_n = S let a query
 * see only keys of its own sequence (under the causal rule, and the window,
 * if set). */
typedef struct ra_mask {
  int64_t window;               /* 0: no window; > 0 requires causal         */
  int32_t n_seqs;               /* packed sequences: count, or 0 (none)      */
  const int64_t* cu_seqlens;    /* host copy of the n_seqs + 1 boundaries    */
  const int64_t* cu_seqlens_dev;/* the same values in device memory          */
} ra_mask;

/*
 * ra_rank_forward_masked -- ra_rank_forward with a sliding window and/or
 * packed sequences.  Tiles the mask hides are not visited; a step whose
 * whole block is hidden is not launched; rows with no visible key in a step
 * keep the merge identity.  m == NULL is ra_rank_forward.  Both dtypes.
 * Both copies of the boundaries must stay unchanged until the work
 * completes.
 */
int ra_rank_forward_masked(const ra_rank_desc* d, const ra_mask* m,
                           const void* q_local, const void* k_shards,
                           const void* v_shards, float* o, float* lse,
                           void* stream);

/*
 * ra_allgather_forward -- the all-gather form of the same rank's attention:
 * every key/value token is resident at once, so the rank's queries attend to
 * the whole sequence in one launch with no per-step merge (ringmaster
 * "Status", Ring row: the allgather rotater, the faster option that keeps
 * all of K/V resident, beside the memory-optimal p2p ring).
 *   q_local  [B, S/P, Hq, D]       this rank's queries in its local order
 *   k_global [B, S, Hkv, D]        all keys in global token order; v_global same
 *   o        [B, S/P, Hq, D] float32, lse [B, S/P, Hq] float32 (written, INIT)
 * The result equals ra_rank_forward's (same definition; the order of the
 * floating-point sums differs).  Requirements as for ra_rank_forward.
 */
int ra_allgather_forward(const ra_rank_desc* d, const void* q_local,
                         const void* k_global, const void* v_global, float* o,
                         float* lse, void* stream);

/*
 * ra_rank_backward -- the backward pass of rank `rank`'s ring attention,
 * simulated on one GPU: the flash-style reverse ring of ringmaster's
 * description ("Status", Ring row, forward and backward; the note on the p2p
 * and allgather paths).  dQ of the rank's rows accumulates locally over the P
 * steps; the contribution to dK and dV of the block held at step s is added
 * into that block's gradient (which in a real ring travels back to its owner
 * with the block).  The arithmetic is the chain rule through the softmax:
 *   P = exp(scale q K^T - L),  dP = dO V^T,  delta = rowsum(dO * O),
 *   dS = P * (dP - delta),  dQ = scale dS K,  dK += scale dS^T Q,  dV += P^T dO,
 * with L and O the forward's final log-sum-exp and output.
 *   q_local   [B, S/P, Hq, D]        this rank's queries (local order)
 *   k_shards, v_shards [P, B, S/P, Hkv, D]  as for ra_rank_forward
 *   o         [B, S/P, Hq, D] float32, lse [B, S/P, Hq] float32 (ra_rank_forward's)
 *   dout      [B, S/P, Hq, D]        the loss gradient of o (q's dtype)
 *   dq        [B, S/P, Hq, D] float32: written
 *   dk_shards, dv_shards [P, B, S/P, Hkv, D] float32: ADDED to (the caller
 *             zeroes them; running every rank into the same buffers gives the
 *             full gradients)
 *   delta     [B, S/P, Hq] float32: caller-provided workspace, written with
 *             -rowsum(dout * o) (negated: the kernels start their dP
 *             accumulation from it)
 * bf16 inputs with D = 128 run the tuned MFMA kernels (P and dS rounded to
 * bf16 before their products); float32 inputs, or D = 64, run plain SIMT
 * kernels in float32, meant for parity-scale problems.  Other requirements
 * as for ra_rank_forward.  Work is enqueued on `stream`: per launched step
 * a dQ kernel, then the dK/dV kernels.
 */
int ra_rank_backward(const ra_rank_desc* d, const void* q_local,
                     const void* k_shards, const void* v_shards,
                     const float* o, const float* lse, const void* dout,
                     float* dq, float* dk_shards, float* dv_shards,
                     float* delta, void* stream);

/*
 * ra_rank_backward_masked -- ra_rank_backward under a sliding window and/or
 * packed sequences (the masks of ra_rank_forward_masked; lse and o must come
 * from that call with the same mask).  A query's gradient terms run over the
 * keys the mask lets it see, the same set as in the forward: hidden tiles are
 * not visited, and a step whose whole block is hidden adds nothing to dK and
 * dV.  m == NULL is ra_rank_backward.  Requirements and errors as for
 * ra_rank_backward, plus the mask checks of ra_rank_forward_masked.
 */
int ra_rank_backward_masked(const ra_rank_desc* d, const ra_mask* m,
                            const void* q_local, const void* k_shards,
                            const void* v_shards, const float* o,
                            const float* lse, const void* dout, float* dq,
                            float* dk_shards, float* dv_shards, float* delta,
                            void* stream);

/*
 * ra_rank_backward_noalloc -- ra_rank_backward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, but the
 * delta workspace is the library's own scratch array instead of an argument.
 * The scratch is a file-scope device array of RA_NOALLOC_MAX_ROWS floats
 * (16 MiB), one per device the library runs on, held until the process ends;
 * its address is resolved on the first call on each device.  The call itself
 * allocates nothing.  Requires B * S/P * Hq <= RA_NOALLOC_MAX_ROWS (else
 * RA_E_INVAL, nothing enqueued), no mask, and everything ra_rank_backward
 * requires.  The scratch is fully written by each call before it is read, so
 * nothing carries over between calls; but every call on one device shares
 * the one array, so calls that overlap on a device (different streams, or
 * threads without ordering) race and must be ordered by the caller.
 */
#define RA_NOALLOC_MAX_ROWS 4194304
int ra_rank_backward_noalloc(const ra_rank_desc* d, const void* q_local,
                             const void* k_shards, const void* v_shards,
                             const float* o, const float* lse, const void* dout,
                             float* dq, float* dk_shards, float* dv_shards,
                             void* stream);

/*
 * ra_ulysses_relayout -- the local pack/unpack around the Ulysses all-to-all
 * ("Sequence Parallelism II: DeepSpeed Ulysses and All-to-All Attention": a
 * rank goes from all heads of its tokens to all tokens of a subset of heads).
 * Destination j of P_u owns heads [j H/P_u, (j+1) H/P_u).
 *   RA_SEQ2HEAD: in [B, s_loc, H, D] -> out [P_u, B, s_loc, H/P_u, D],
 *                out[j, b, t, h', :] = in[b, t, j H/P_u + h', :]
 *   RA_HEAD2SEQ: the exact inverse.
 * A bit-exact permutation of elem_bytes-byte elements (1, 2, 4 or 8).
 * Requires H % P_u == 0, P_u >= 1; in and out must not overlap.
 */
int ra_ulysses_relayout(int32_t dir, int32_t elem_bytes, int32_t B,
                        int64_t s_loc, int32_t H, int32_t D, int32_t P_u,
                        const void* in, void* out, void* stream);

/*
 * ra_ulysses_pieces -- the messages of one Ulysses all-to-all, for up to 4
 * tensors in one launch ("Sequence Parallelism II": all heads of a rank's
 * tokens become all tokens of a head subset; ringmaster's Ulysses leg sends
 * K and V in one collective, its "Status" row 7 fuses Q, K and V).
 * A piece is the message between one pair of ranks: the n tensors' sections
 * one after another, section i being [B, s_loc, run_bytes[i]] (a run is the
 * bytes of one token that go to one destination).  pieces is [P_u, piece],
 * piece = sum_i B * s_loc * run_bytes[i] bytes.
 *   RA_GROUP_HEADS (the sender's pack, and the inverse unpack of the returned
 *     outputs): tensors[i] is [B, s_loc, P_u * run_bytes[i]], and piece j
 *     section i holds bytes [j run, (j+1) run) of every token (head block j).
 *   RA_GROUP_SEQ (the receiver's side): tensors[i] is
 *     [B, P_u * s_loc, run_bytes[i]] in global token order, and piece u
 *     section i holds tokens [u s_loc, (u+1) s_loc) (those of source u).
 * to_pieces = 1: tensors -> pieces; 0: pieces -> tensors.  A bit-exact
 * permutation.  Requires 1 <= n <= 4, P_u >= 1, run_bytes[i] >= 1, pieces
 * overlapping no tensor, and fewer than 2^31 moved units per tensor.
 */
int ra_ulysses_pieces(int32_t to_pieces, int32_t group, int32_t B, int64_t s_loc,
                      int32_t P_u, int32_t n, void* const* tensors,
                      const int64_t* run_bytes, void* pieces, void* stream);

/* Host-side plan of one ring step (integers only, no GPU work). */
typedef struct ra_plan_out {
  int32_t src;                 /* rank whose shard is held at this step    */
  int32_t n_qspans, n_kspans;
  ra_span qspans[2], kspans[2];/* global spans, local order                */
  int32_t pair_class[2][2];    /* RA_CLASS_* of (query span i, key span j) */
  int64_t tiles_full, tiles_diag, tiles_skip; /* (tile_q x tile_k) tiles   */
} ra_plan_out;

/*
 * ra_plan -- the index maps and mask classes behind ra_rank_forward, exposed
 * so they can be checked exactly: the source shard of step `step` (the static
 * ring 0 -> 1 -> ... -> P-1 -> 0 of the DeDLOC guide, "The Geo-Distributed
 * Long-Context Crisis"), both ranks' global spans (ringmaster "Layout":
 * contiguous shards and the head_tail balancer; "Sequence Parallelism IV ...
 * Load-Balanced Rings"), the class of each (query span, key span) pair (the
 * causal skip of the DeDLOC guide, "Best Practices", row "Causal Mask
 * Handling"), and the number of FULL / DIAG / SKIP tiles when query rows are
 * cut into tiles of tile_q and key rows into tiles of tile_k (tiles restart
 * at each span; the last tile of a span may be short).  Same requirements on
 * (S, P, rank) as ra_rank_forward, 0 <= step < P, tile sizes >= 1.
 */
int ra_plan(int32_t order, int64_t S, int32_t P, int32_t rank, int32_t step,
            int32_t causal, int32_t tile_q, int32_t tile_k, ra_plan_out* out);

/* Kernels a ring step may launch (reported by ra_rank_launches). */
#define RA_KERNEL_NONE 0            /* the step launches nothing               */
#define RA_KERNEL_STEP_F32 1        /* float32 inputs                          */
#define RA_KERNEL_STEP_BF16 2       /* bf16, four waves, two workgroups per CU */
#define RA_KERNEL_STEP_BF16_KSPLIT 3/* bf16 D 128, eight waves splitting each
                                       item's key tiles (few items)            */
#define RA_KERNEL_BWD_FUSED 4       /* backward bf16 D 128: dQ, fused dK/dV    */
#define RA_KERNEL_BWD_SPLIT 5       /* backward bf16 D 128: dQ, dV, dK kernels */
#define RA_KERNEL_BWD_SIMT 6        /* backward float32 or D 64                */

typedef struct ra_launch_info {
  int32_t kernel;   /* RA_KERNEL_*                                          */
  int32_t masked;   /* 1: the window / packed-sequence instantiation        */
  int32_t items;    /* work items with work: forward, query tiles x heads;
                       backward, key tiles seen by some query x kv heads    */
  int32_t grid;     /* workgroups of the (forward or dQ) launch             */
  int32_t lpt;      /* 1: each XCD walks whole heads, heaviest tile first   */
  int32_t first_heavy; /* 1: the first query tiles see the most keys        */
} ra_launch_info;

/*
 * ra_rank_launches -- which kernels ra_rank_forward(_masked) (backward == 0)
 * or ra_rank_backward(_masked) (backward == 1) would launch for each of the
 * P ring steps of `d` under mask `m` (NULL: none), in step order, into
 * out[0 .. P-1].  Host-only: nothing is enqueued.  The choice depends on the
 * number of compute units: n_cus > 0 plans for that many; n_cus == 0 uses
 * the current device's count (which needs a GPU).  The same host code builds
 * the launches themselves.  Requirements as for the matching call (shapes,
 * mask); tensor pointers are not needed.
 */
int ra_rank_launches(const ra_rank_desc* d, const ra_mask* m, int32_t backward, int32_t n_cus,
                     ra_launch_info* out);

/* Message describing the last failure on the calling thread ("" if none). */
const char* ra_last_error(void);

/* RA_ABI_VERSION of the built library. */
int ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */

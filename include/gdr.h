/*
 * gdr.h -- C ABI of libgdr.so: the channelwise gated delta rule on AMD Instinct MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * The operation.  For every batch b and value head h (key head kh = h / (HV/HK)) the
 * library carries an fp32 state S[dk][dv] and, for every token t,
 *     S   <- diag(exp(g_t)) S                              per-channel decay, g_t in R^dk
 *     S   <- S + beta_t k_t (v_t - S^T k_t)^T              rank-one delta update
 *     o_t  = S^T q_t                                       output from the updated state
 * This is the recurrence whose decode step ExecuTorch PR #21021 ("Reorder channelwise
 * gated delta rule chunked hot loops for autovectorization") restructures into two
 * state traversals (first commit summary) and whose prefill it evaluates in chunkwise
 * WY/UT form, routed by sequence length (second commit summary).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to dense row-major arrays, 16-byte aligned:
 *       q, k  [B][T][HK][dk]   (qkv_dtype)      v     [B][T][HV][dv]  (qkv_dtype)
 *       g     [B][T][HV][dk]   log-decay, fp32 (bf16 with GDR_G_BF16; [B][T][HK][dk] with
 *                              GDR_G_PER_KEY_HEAD)
 *       beta  [B][T][HV]       fp32
 *       h0,ht [B][HV][dk][dv]  fp32 state       o     [B][T][HV][dv]  fp32 (bf16 with
 *                                                                        GDR_O_BF16)
 *     value head h reads key head h / (HV/HK) (contiguous GQA groups).
 *   - h0 == NULL means a zero initial state; ht == NULL means the final state is not
 *     written.  ht may equal h0 exactly (in-place carry) but must not partially overlap
 *     it.  o must not overlap any input, h0 or ht.
 *   - The caller owns every buffer.  The library never allocates or frees device memory
 *     and keeps no per-call state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without waiting; buffers must stay valid until the stream reaches it.
 *   - Every argument check runs on the host before any HIP call: a call that returns an
 *     error has enqueued nothing and written nothing.  Launch failures return
 *     GDR_ERR_HIP.  The library never aborts or prints.  NaN/Inf inputs are not checked
 *     and propagate.
 *   - Supported: dk, dv in {32, 64, 128}; chunk in {16, 32, 64}; HV % HK == 0; B, T >= 1;
 *     q/k/v in bf16 or fp32.  One prefill launch takes a batch element of T tokens while
 *     (T + chunk)*HV*max(dk, dv)*4 < 2^31 (its g and o rows, padding rows of the last chunk
 *     included) and ceil(T/chunk) * (workspace bytes per chunk) < 2^31 (one head's chunk
 *     records): up to 131007 tokens at HV = 32, dk = dv = 128, chunk 64.  gdr_chunk_prefill
 *     (and gdr_forward) runs longer sequences as a chain of windows of W tokens, W the
 *     largest multiple of the chunk length within that limit (130944 in the same case), one
 *     batch element at a time, handing the state on through ht or a slot in the workspace
 *     (gdr_chunk_prefill_workspace_bytes sizes it); the chunk grid is that of one call.
 *     gdr_chunk_prep, gdr_chunk_carry and the packed-batch calls take only what one launch
 *     takes (GDR_ERR_SHAPE beyond).
 *     Decay values are expected to satisfy g <= 0 with the total
 *     decay over any 8 consecutive tokens below 80 in every channel (exp(g) >= ~5e-5 per
 *     token); outside that range the prefill path's intra-chunk decay factors can
 *     overflow fp32.  The decode and fused recurrent paths have no such limit.
 *   - Magnitudes.  The prefill's matrix-core products take fp16 operands, each brought into
 *     fp16's range by exact power-of-two scales: per query row (and 16-row block) for q, per
 *     column group and chunk for the state and for v, each separately.  So q, v, h0 and the
 *     state may take any magnitude within fp32's normal range, independently of each other,
 *     and results match the fp64 recurrence to the same relative accuracy at any such scale.
 *     Two limits remain: the pseudo-values U = Tb V - W S keep fp16's precision while
 *     beta >= 2^-12 (beta = 0 exactly is exact), and the segmented carry's transition
 *     matrices assume non-expansive updates (beta |k|^2 <= 2, e.g. unit-norm keys with beta
 *     in [0, 1]).  Keys are used as given (no normalisation); their entries must be
 *     representable in fp16 (|k| < 65504).
 *   - Results are bitwise reproducible for identical inputs and dims (no atomics).
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 8

typedef enum {
    GDR_OK = 0,
    GDR_ERR_NULL = 1,        /* a required pointer (dims, q, k, v, g, beta, o) is NULL     */
    GDR_ERR_SHAPE = 2,       /* B/T/HK/HV < 1, HV % HK != 0, decode step with T != 1, a
                                size past the limits below                                 */
    GDR_ERR_UNSUPPORTED = 3, /* dk/dv/chunk/dtype outside the supported set               */
    GDR_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned                   */
    GDR_ERR_ALIAS = 5,       /* o overlaps an input/h0/ht, or ht partially overlaps h0    */
    GDR_ERR_WORKSPACE = 6,   /* workspace NULL, misaligned or smaller than required       */
    GDR_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed                 */
    GDR_ERR_SCRATCH = 8      /* gdr_chunk_prefill_noalloc: the call needs more workspace than
                                GDR_NOALLOC_SCRATCH_BYTES                                   */
} gdr_status;

typedef enum { GDR_BF16 = 0, GDR_F32 = 1 } gdr_dtype;

/*
 * Input-format flags (gdr_dims.flags; 0 = the defaults above).
 *   GDR_G_BF16  g is stored as bf16 instead of fp32 -- the I/O-lean input of the
 *               follow-up work on the prefill's HBM bytes: g is the largest input (dk values
 *               per token and value head), and bf16 halves it.  The kernels widen each value
 *               exactly to fp32, so a call gives bitwise the result of the same call with an
 *               fp32 g holding the same (bf16-representable) values.  Requires bf16 q/k/v.
 */
#define GDR_G_BF16 0x1
/*
 * Fused input prologue (gdr_dims.flags), the follow-up work's I/O-lean mode on the
 * pre-processing side: the real-scale input recipe of the uzu PR #576 review feeds the
 * recurrence L2-normalised keys and a softplus decay, which a caller would otherwise
 * compute in separate passes over k and g (each a read and a write of the tensor).
 *   GDR_K_L2NORM  k holds raw keys; every kernel uses k_t / max(|k_t|_2, 1e-12), the norm
 *                 taken per token and key head over dk.
 *   GDR_G_SOFTPLUS g holds gate logits a (same layout and dtype rules as g); every kernel
 *                 uses the log-decay g = -softplus(a) = -log(1 + exp(a)).
 * Both apply to every entry point and combine freely with each other and with GDR_G_BF16.
 * Results equal those of the same call with the pre-processed k and g given explicitly, up
 * to fp32 rounding of the pre-processing.
 */
#define GDR_K_L2NORM 0x2
#define GDR_G_SOFTPLUS 0x4
/*
 * Gate shared per key head (gdr_dims.flags).
 *   GDR_G_PER_KEY_HEAD  g is [B][T][HK][dk] (dtype and prologue rules unchanged): every value
 *                 head of a GQA group decays with its key head's gate, value head h using
 *                 g row h / (HV/HK).  beta stays per value head.  Every entry point takes it.
 * With a shared gate the prefill's unscaled gram sum_c k_rc k_sc exp(gam_rc - gam_sc) is the
 * same for the G value heads of a group; only beta, a row scaling of it, differs.  The
 * uzu PR #576 review thread on the per-value-head gram weighs a gram per value head fused
 * with the rest against a gram per key head with the solve split off.  The prefill has both
 * forms of its chunk-parallel stage:
 *   fused  one workgroup per (batch, value head, chunk), as for a gate per value head;
 *   split  one workgroup per (batch, key head, chunk): the gram, causal terms and decayed
 *          operands once, then the solve and the pseudo-keys for each of the G value heads
 *          (G <= GDR_PREP_SPLIT_MAX_GROUP).
 * Both give bitwise the same results.  The library picks the split form when the call has
 * enough (batch, key head, chunk) triples to fill the GPU with it, the fused form
 * otherwise; GDR_PREP_SPLIT or GDR_PREP_FUSED forces one (the other entry points ignore
 * both).  GDR_PREP_SPLIT without GDR_G_PER_KEY_HEAD, with HV/HK above the limit, or with
 * GDR_PREP_FUSED returns GDR_ERR_UNSUPPORTED.
 * Any other bit, or GDR_G_BF16 with fp32 q/k/v, returns GDR_ERR_UNSUPPORTED.
 */
#define GDR_G_PER_KEY_HEAD 0x8
#define GDR_PREP_SPLIT 0x10
#define GDR_PREP_FUSED 0x20
#define GDR_PREP_SPLIT_MAX_GROUP 8
/*
 * Output format (gdr_dims.flags).
 *   GDR_O_BF16  o is stored as bf16: every output is computed in fp32 exactly as without the
 *               flag and rounded to the nearest bf16 (ties to even) as it is stored, so the
 *               call's o is bitwise the bf16 rounding of the same call's fp32 o; states
 *               stay fp32.  The I/O-lean output of the follow-up work on the prefill's HBM
 *               bytes: o (dv values per token and value head) is the prefill's largest
 *               output.  Every entry point takes it, with either q/k/v dtype.  The rounding
 *               alone moves each value by up to 2^-8 of it (about 1.7e-3 relative over a
 *               tensor of normally distributed values), so the fp32 path's agreement with
 *               the fp64 recurrence does not carry over to o below that level.
 */
#define GDR_O_BF16 0x40

typedef struct {
    int32_t B, T, HK, HV, dk, dv;
    int32_t chunk;      /* prefill chunk length C (ignored by the token-recurrence calls)  */
    int32_t qkv_dtype;  /* gdr_dtype of q, k and v                                         */
    int32_t flags;      /* GDR_G_BF16 | GDR_K_L2NORM | GDR_G_SOFTPLUS | GDR_G_PER_KEY_HEAD |
                           GDR_O_BF16, GDR_PREP_SPLIT or GDR_PREP_FUSED                      */
} gdr_dims;

/*
 * One autoregressive decode step (T must be 1): the two-pass token recurrence of
 * ExecuTorch PR #21021, first commit summary -- pass 1 forms the prediction S^T k with
 * the decay folded in, pass 2 applies decay and the rank-one update and accumulates the
 * output.  On the GPU each state element is read from HBM once and written once.
 * Normally called in place (ht == h0).  Uses no workspace.
 */
int gdr_decode_step(const gdr_dims* dims, const void* q, const void* k, const void* v,
                    const void* g, const float* beta, const float* h0, void* o, float* ht,
                    void* stream);

/*
 * The same two-pass token recurrence for T >= 1 tokens in one launch (chunk ignored):
 * each workgroup loads its slice of the state once, applies the T tokens in order with
 * the slice held in registers, writes o for every token and stores the state once.  The
 * pages route only T == 1 to the token recurrence (ExecuTorch PR #21021, second commit
 * summary); this is the same recurrence for short multi-token calls (a speculative chain
 * of a few tokens, a short continuation), where T decode steps would move the whole
 * state T times and the chunked path pays its fixed cost.  Arguments, layouts and
 * checks are those of gdr_decode_step with any T >= 1; T == 1 gives bitwise the result of
 * gdr_decode_step.  Uses no workspace.
 */
int gdr_fused_recurrent(const gdr_dims* dims, const void* q, const void* k, const void* v,
                        const void* g, const float* beta, const float* h0, void* o, float* ht,
                        void* stream);

/*
 * Bytes of device workspace gdr_chunk_prefill needs for these dims (0 if dims are
 * invalid).  The workspace holds per-chunk operands that the chunk-parallel kernel hands
 * to the sequential state-carry kernel -- the per-worker scratch arena of ExecuTorch PR
 * #21021 (second commit summary), carved per (batch, head, chunk).  When the carry splits
 * the sequence into segments (few heads, many chunks), it also holds, per head, each
 * segment's fp32 summary (the state it produces from zero and its dk x dk transition
 * matrix) and each segment's fp32 start state.  The size depends on the dims only.
 */
size_t gdr_chunk_prefill_workspace_bytes(const gdr_dims* dims);

/*
 * Chunkwise WY/UT prefill for any T >= 1 (ExecuTorch PR #21021, second commit summary):
 * per-channel log-decay prefixes, the beta-folded strictly-lower gram A, an exact
 * 16x16-block forward-substitution solve of (I + A), WY pseudo-keys and pseudo-values,
 * causal intra-chunk query/key terms, and the inter-chunk state carry; the ragged last
 * chunk is handled by the same code (zero-padded rows).  The block solve follows the
 * exact block forward substitution of uzu PR #576 ("Support TreeUpdateSolve kernel").
 * `workspace` must be a 256-byte-aligned device buffer of at least
 * gdr_chunk_prefill_workspace_bytes(dims) bytes; its contents on entry are ignored.
 */
int gdr_chunk_prefill(const gdr_dims* dims, const void* q, const void* k, const void* v,
                      const void* g, const float* beta, const float* h0, void* o, float* ht,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages of gdr_chunk_prefill as separate calls, with the same arguments and
 * checks.  gdr_chunk_prefill(...) is exactly gdr_chunk_prep(...) followed by
 * gdr_chunk_carry(...) on the same stream and workspace.
 *   gdr_chunk_prep  -- chunk-parallel stage (one workgroup per batch, value head, chunk):
 *                      decay prefixes, gram A and causal terms P on the matrix cores, the
 *                      16x16-block solve of (I + A), WY pseudo-keys; writes the workspace.
 *                      Reads q, k, g, beta; never touches v, h0, o or ht.
 *   gdr_chunk_carry -- sequential stage (chunks in order): pseudo-values, outputs and
 *                      the state carry, either with the value dimension split across
 *                      workgroups or one workgroup per head; with few heads and many
 *                      chunks the sequence is cut into segments that carry in parallel
 *                      (segment summaries, then their ordered combination, then every
 *                      segment from its start state).  Reads the workspace written by
 *                      gdr_chunk_prep for the same inputs, v and h0; writes o and ht (and
 *                      the carry's part of the workspace).
 * Splitting them lets a caller time or overlap the stages.
 */
int gdr_chunk_prep(const gdr_dims* dims, const void* q, const void* k, const void* v,
                   const void* g, const float* beta, const float* h0, void* o, float* ht,
                   void* workspace, size_t workspace_bytes, void* stream);
int gdr_chunk_carry(const gdr_dims* dims, const void* q, const void* k, const void* v,
                    const void* g, const float* beta, const float* h0, void* o, float* ht,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Routed call for any T >= 1, in the spirit of the length routing of ExecuTorch PR #21021
 * (second commit summary), with the threshold set by measurement on MI355X: T <=
 * GDR_RECURRENT_MAX_T runs gdr_fused_recurrent (workspace may be NULL), longer calls run
 * gdr_chunk_prefill (workspace as documented there).  Measured at B = 32, HV = 32,
 * dk = dv = 128: one fused launch beats T decode steps from T = 2 and the chunked path up
 * to T = 8; the chunked path wins from T = 16.
 */
#define GDR_RECURRENT_MAX_T 8
int gdr_forward(const gdr_dims* dims, const void* q, const void* k, const void* v,
                const void* g, const float* beta, const float* h0, void* o, float* ht,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length batches.  The pages route work by sequence length (ExecuTorch PR
 * #21021, second commit summary) and batch speculative chains of different lengths (uzu PR
 * #576 review: dispatch cost at small T); a batch of sequences of different lengths is laid
 * end to end instead of padded:
 *   dims->B     number of sequences N (1 .. GDR_VARLEN_MAX_SEQS)
 *   dims->T     rows in all, the packed length
 *   cu_seqlens  device array [N + 1] of int32, 4-byte aligned: sequence i is on rows
 *               [cu_seqlens[i], cu_seqlens[i + 1]); expected non-decreasing from 0 to T.
 *   q, k        [T][HK][dk]         v, o  [T][HV][dv]       beta  [T][HV]
 *   g           [T][HV][dk] (or [T][HK][dk] with GDR_G_PER_KEY_HEAD)
 *   h0, ht      [N][HV][dk][dv]: one state per sequence
 * i.e. the dense layouts with B = 1 for the token tensors and B = N for the states.  Every
 * sequence runs the recurrence from its own h0 (zero if h0 is NULL) and ends in its own ht;
 * a sequence with no rows passes h0 to ht.  Flags and other rules are those of the dense
 * calls.  The library reads cu_seqlens on the device only: entries are clamped to [0, T]
 * and to the running maximum of the entries before them, so no access leaves the tensors
 * whatever they hold, but results are defined only for non-decreasing entries from 0 to T
 * (rows outside [cu_seqlens[0], cu_seqlens[N]) are then not written).
 */
#define GDR_VARLEN_MAX_SEQS 4096

/*
 * Chunkwise prefill of a packed batch: each sequence chunked from its own first row (its
 * last chunk ragged), the chunk-parallel stage over every sequence's chunks at once, the
 * carry per (sequence, head).  A first small kernel turns cu_seqlens into the plan the
 * others read (kept in the workspace).  Equal to one gdr_chunk_prefill call per sequence.
 * `workspace` as for gdr_chunk_prefill, of at least
 * gdr_chunk_prefill_varlen_workspace_bytes(dims) bytes (a bound that holds for any split of
 * T rows into N sequences).
 */
size_t gdr_chunk_prefill_varlen_workspace_bytes(const gdr_dims* dims);
int gdr_chunk_prefill_varlen(const gdr_dims* dims, const int32_t* cu_seqlens, const void* q,
                             const void* k, const void* v, const void* g, const float* beta,
                             const float* h0, void* o, float* ht, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * The fused token recurrence (gdr_fused_recurrent) over a packed batch: one workgroup per
 * (sequence, value head, column block) runs that sequence's rows.  Uses no workspace.
 */
int gdr_fused_recurrent_varlen(const gdr_dims* dims, const int32_t* cu_seqlens, const void* q,
                               const void* k, const void* v, const void* g, const float* beta,
                               const float* h0, void* o, float* ht, void* stream);

/*
 * Tree-verify solve (uzu PR #576, "Support TreeUpdateSolve kernel": a gram over a
 * speculative token tree, keys times the initial state, an exact triangular solve).  Each
 * batch element holds a tree of T <= GDR_TREE_MAX_T tokens in topological order:
 * parent[b][t] is the parent node of node t, in [-1, t), -1 meaning the node continues
 * from the initial state h0 (zero if h0 is NULL); entries outside that range are read
 * as -1.  Node t's output o[b][t] is the output of the recurrence run along its root
 * path (every node continues from its parent's state).  The final states are not
 * written.  parent is a device array [B][T] of int32, 4-byte aligned; the other
 * arguments, layouts and checks are those of gdr_fused_recurrent (chunk ignored).  The
 * cumulative decay along any root path must stay above -80 in every channel.  Uses no
 * workspace.  T above GDR_TREE_MAX_T returns GDR_ERR_UNSUPPORTED.
 */
#define GDR_TREE_MAX_T 64
int gdr_tree_verify(const gdr_dims* dims, const int32_t* parent, const void* q, const void* k,
                    const void* v, const void* g, const float* beta, const float* h0, void* o,
                    void* stream);

/*
 * Allocation-free variant of gdr_chunk_prefill, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, checks and results as gdr_chunk_prefill, minus the
 * workspace: the library uses its own per-device scratch array of GDR_NOALLOC_SCRATCH_BYTES
 * (64 MiB: the chunk records of a prefill of up to 1984 tokens at HV = 32, dk = 128, chunk 64), which
 * each GPU the library runs on holds until the process ends.  Calls whose workspace
 * (gdr_chunk_prefill_workspace_bytes) exceeds it return GDR_ERR_SCRATCH before any HIP
 * call.  It calls no allocating routine (the array's device address is looked up once per
 * device, on the first call made with that device current).  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (concurrent streams or threads) race and
 * must be serialised by the caller.  The array's contents between calls are not meaningful.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gdr_chunk_prefill_noalloc(const gdr_dims* dims, const void* q, const void* k, const void* v,
                              const void* g, const float* beta, const float* h0, void* o,
                              float* ht, void* stream);

/* Static English text for a status code (never NULL). */
const char* gdr_status_str(int status);

/* GDR_ABI_VERSION of the loaded library. */
int gdr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */

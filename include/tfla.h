/*
 * tfla.h -- C ABI of libtfla: the chunkwise-parallel forward pass of gated
 * linear attention (mLSTMsig and two gate variants) on AMD gfx950.
 *
 * The operation.  Per batch b and head h, with matrix memory C in
 * R^{d_qk x d_hv} starting at C_0 = 0 (or a given state: tfla_fwd_state):
 *
 *     C_t = diag(f_t) C_{t-1} + i_t k_t v_t^T,     h_t = C_t^T q_t / sqrt(d_qk)
 *
 * mLSTMsig (the mLSTM with a sigmoid input gate and neither normaliser nor
 * max state) is defined in words in "Tiled Flash Linear Attention: More
 * Efficient Linear RNN and xLSTM Kernels" (research-map summary, sections
 * Approach and Surprising findings); the fixed per-head decay is the RetNet
 * row and the per-key-channel gate the GLA row of the flash-linear-attention
 * README's model table; the data-dependent gate is from "Gated Linear
 * Attention Transformers with Hardware-Efficient Training" (Abstract).
 *
 * The library evaluates it chunkwise (TFLA abstract: chunkwise-parallel
 * formulation with a second level of sequence tiling inside each chunk, so
 * the chunk size L is not bounded by on-chip memory): a gate prefix-sum
 * kernel, an inter-chunk state kernel that walks the state in fp32 and
 * materialises it at every chunk boundary (the "ParallelChunk" form of the
 * README) in the I/O type, the operand type of the matrix-core products that
 * read it, and an intra-chunk kernel on bf16 matrix cores.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, contiguous row-major.  The library keeps no pointer after a
 *     call returns.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream) and the call returns without waiting.  Device faults
 *     surface at the caller's next synchronisation.
 *   - Arguments are validated before any HIP call; a rejected call has no
 *     side effect.  Every call returns a tfla_status; tfla_last_error()
 *     returns a thread-local message describing the last failure.
 *   - Calls are reentrant; the only mutable global state is that message
 *     and the test overrides of tfla_dbg_set_knob (unset unless a test sets
 *     them).  The library reads no environment variable.
 */
#ifndef TFLA_H
#define TFLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `variant` = gate kind (low byte) | I/O element type flag. */
enum tfla_variant {
    TFLA_MLSTM_SIG = 0,     /* i = sigmoid(igate_pre[t]), f = sigmoid(fgate_pre[t])       */
    TFLA_SCALAR_DECAY = 1,  /* i = 1, f = sigmoid(fgate_pre[h]) fixed per head            */
    TFLA_GLA_KEY = 2,       /* i = 1, f_{t,c} = exp(logsigmoid(fgate_pre[t,c]) / 16)      */
    TFLA_MLSTM_EXP = 3,     /* mLSTMexp: i = exp(igate_pre[t]), f = sigmoid(fgate_pre[t]),
                               normaliser and max state (tfla_fwd, _ws, _ws_marked and
                               _noalloc only; see tfla_fwd)                                 */
    TFLA_IO_BF16 = 0x100,   /* q, k, v, h are bf16; without the flag they are fp32        */
    TFLA_BWD_REUSE_FWD = 0x200, /* tfla_bwd only: reuse the forward pass's gate sums and
                                   states left in the workspace (see tfla_bwd)              */
    TFLA_STATES_FP32 = 0x400    /* forward calls, bf16 I/O: materialise the chunk states in
                                   fp32 rather than bf16 (outputs are identical: the
                                   intra-chunk products round the states to bf16 either way;
                                   the state bytes double); no effect with fp32 I/O or on
                                   tfla_fwd_recurrent; TFLA_ERR_UNSUPPORTED for the
                                   backward calls                                           */
};

enum tfla_status {
    TFLA_OK = 0,
    TFLA_ERR_INVALID_ARG = 1,   /* NULL/misaligned pointer, bad size, unknown variant   */
    TFLA_ERR_UNSUPPORTED = 2,   /* valid but not built: head dims or chunk size          */
    TFLA_ERR_HIP = 3,           /* a HIP launch or runtime call failed                   */
    TFLA_ERR_OUT_OF_MEMORY = 4  /* workspace allocation failed, or the caller's is small */
};

/*
 * tfla_fwd -- the forward pass.
 *
 *   q          [B,H,T,d_qk]  bf16 or fp32 (see TFLA_IO_BF16)
 *   k          [B,H,T,d_qk]
 *   v          [B,H,T,d_hv]
 *   igate_pre  fp32 [B,H,T] input-gate pre-activations for TFLA_MLSTM_SIG and
 *              TFLA_MLSTM_EXP; must be NULL for the other variants (their
 *              input gate is 1).
 *   fgate_pre  fp32 forget-gate pre-activations:
 *                TFLA_MLSTM_SIG, TFLA_MLSTM_EXP [B,H,T]
 *                TFLA_SCALAR_DECAY [H]      (logit of the per-head decay;
 *                                            +inf means no decay)
 *                TFLA_GLA_KEY      [B,H,T,d_qk]
 *   h          [B,H,T,d_hv] output, same element type as q; fully
 *              overwritten; must not overlap any input.
 *   B, H, T    >= 1.  T need not be a multiple of L (the last chunk may be
 *              partial).
 *   d_qk       64, 128 or 256
 *   d_hv       a multiple of 64, <= 512
 *   L          chunk size: 64, 128, 256, 512 or 1024
 *
 * Gate pre-activations may be +-inf (a gate of exactly 1 or 0).  The log
 * forget gate is floored at -100 (a forget gate below e^-100 acts as
 * e^-100), which keeps log-decay differences finite.
 *
 * TFLA_MLSTM_EXP -- the mLSTM with an exponential input gate, a normaliser
 * state n and a max state m (what mLSTMsig simplifies: "Tiled Flash Linear
 * Attention ..." research-map summary, Approach):
 *     C_t = f_t C_{t-1} + i_t k_t v_t^T,   n_t = f_t n_{t-1} + i_t k_t,
 *     h_t = (C_t^T q_t / sqrt(d_qk)) / max(|n_t . q_t| / sqrt(d_qk), 1),
 * i_t = exp(igate_pre_t), f_t = sigmoid(fgate_pre_t), evaluated with the max
 * state so that exp(igate_pre) never overflows.  igate_pre must not be
 * +inf; it is floored at -100 (an input gate below e^-100 acts as e^-100).
 * Forward only: the state-I/O, step-by-step and backward entry points and
 * the test hooks return TFLA_ERR_UNSUPPORTED for it.
 *
 * Scratch: allocates its workspace (tfla_workspace_bytes) stream-ordered
 * with hipMallocAsync and frees it with hipFreeAsync on `stream`.
 */
int tfla_fwd(const void* q, const void* k, const void* v,
             const float* igate_pre, const float* fgate_pre, void* h,
             int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* stream);

/* Bytes of device workspace tfla_fwd_ws needs for these arguments (0 when
 * the arguments are invalid or unsupported). */
size_t tfla_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant);

/* tfla_fwd with a caller-owned device workspace of at least
 * tfla_workspace_bytes(...) bytes, 256-byte aligned; no allocation.  The
 * workspace must not be used by other work while this call's kernels run,
 * and must not overlap a tensor argument (checked: TFLA_ERR_INVALID_ARG). */
int tfla_fwd_ws(const void* q, const void* k, const void* v,
                const float* igate_pre, const float* fgate_pre, void* h,
                int B, int H, int T, int d_qk, int d_hv, int L, int variant,
                void* workspace, size_t workspace_bytes, void* stream);

/* tfla_fwd_ws with timing marks for profiling: `marks` points to four
 * hipEvent_t (created by the caller) that are recorded on `stream` before
 * the gate kernel, after it, after the state kernel and after the
 * intra-chunk kernel, so the caller can time each kernel on the stream it
 * runs on.  marks == NULL behaves exactly like tfla_fwd_ws. */
int tfla_fwd_ws_marked(const void* q, const void* k, const void* v,
                       const float* igate_pre, const float* fgate_pre, void* h,
                       int B, int H, int T, int d_qk, int d_hv, int L, int variant,
                       void* workspace, size_t workspace_bytes, void* const* marks, void* stream);

/*
 * tfla_fwd_noalloc -- tfla_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): it calls no hipMalloc / hipFree or other allocating
 * routine.  Its workspace is a static device array inside the library of
 * tfla_fwd_noalloc_max_workspace() bytes (64 MiB), one per GPU, held until
 * the process ends; its address is looked up once per device on the first
 * call there.  Problems whose tfla_workspace_bytes(...) exceed it return
 * TFLA_ERR_OUT_OF_MEMORY (use tfla_fwd_ws).  Every call on one GPU shares
 * that GPU's array: calls whose kernels overlap in time on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller,
 * e.g. by issuing them on one stream.  Arguments, layouts and results are
 * those of tfla_fwd.
 */
int tfla_fwd_noalloc(const void* q, const void* k, const void* v,
                     const float* igate_pre, const float* fgate_pre, void* h,
                     int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* stream);
size_t tfla_fwd_noalloc_max_workspace(void);

/*
 * tfla_fwd_state -- the forward pass from a given initial state, returning
 * the final state (chunked prefill; splitting a long sequence into calls;
 * the sequence-sharded evaluation of several devices).  The recurrence is
 * the one above with C_0 taken from c0: the carried state of the
 * step-by-step form (the "FusedRecurrent" row of the flash-linear-attention
 * README's list of computation forms) made explicit.
 *
 *   c0        fp32 [B,H,d_qk,d_hv] initial state C_0 (row c = key channel,
 *             column j = value channel), or NULL for C_0 = 0.
 *   c_final   fp32 [B,H,d_qk,d_hv] receives C_T, or NULL.  May be the same
 *             pointer as c0 (the state is then updated in place); must not
 *             otherwise overlap c0, an input or h.
 *   workspace caller-owned device workspace of at least
 *             tfla_state_workspace_bytes(...) bytes, 256-byte aligned and
 *             disjoint from every tensor argument, or NULL to let the call
 *             allocate it stream-ordered (hipMallocAsync / hipFreeAsync on
 *             `stream`).
 * Every other argument, layout and rule is that of tfla_fwd.  With c0 and
 * c_final both NULL the result equals tfla_fwd's.
 */
int tfla_fwd_state(const void* q, const void* k, const void* v,
                   const float* igate_pre, const float* fgate_pre, const float* c0,
                   void* h, float* c_final,
                   int B, int H, int T, int d_qk, int d_hv, int L, int variant,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace tfla_fwd_state needs (it includes a slot for
 * the initial state); 0 when the arguments are invalid or unsupported. */
size_t tfla_state_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant);

/*
 * tfla_fwd_recurrent -- the same recurrence evaluated step by step in one
 * fused kernel (the O(T) "FusedRecurrent" form of the
 * flash-linear-attention README): for decoding one or a few steps from a
 * carried state.  Work per call is O(T d_qk d_hv), serial in T, so long
 * sequences belong to tfla_fwd / tfla_fwd_state.
 *
 *   state     fp32 [B,H,d_qk,d_hv], read as C_0 and overwritten with C_T
 *             (the layout of tfla_fwd_state's c0 / c_final, so the two
 *             calls chain); must not overlap an input or h.
 * q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv and variant are as
 * for tfla_fwd (there is no chunk size).  No workspace; no allocation.
 */
int tfla_fwd_recurrent(const void* q, const void* k, const void* v,
                       const float* igate_pre, const float* fgate_pre, float* state, void* h,
                       int B, int H, int T, int d_qk, int d_hv, int variant, void* stream);

/*
 * tfla_bwd -- the backward pass: given dh = dL/dh for the forward pass of
 * tfla_fwd (C_0 = 0), the gradients of L with respect to every input.  The
 * pages list forward-and-backward timings for each computation form (the
 * "fwdbwd" columns of the flash-linear-attention README's timing table) and
 * TFLA's training kernels; this is the chunkwise form of the same
 * recurrence run backwards:
 *
 *     dC_t = q_t dh_t^T / sqrt(d_qk) + diag(f_{t+1}) dC_{t+1},   dC_T from dh_T only
 *     dq_t = C_t dh_t / sqrt(d_qk),   dk_t = i_t dC_t v_t,   dv_t = i_t dC_t^T k_t
 *     dL/dlog i_t = k_t . dk_t,       dL/dlog f_t = sum_{t'>=t} (q_t'.dq_t' - k_t'.dk_t')
 *
 * (for the per-key-channel gate diag(f) acts per channel and the last sum is
 * taken per channel c: q_t',c dq_t',c - k_t',c dk_t',c), and the gate
 * pre-activations through their sigmoids (a log forget gate at its floor of
 * -100 passes no gradient).  The states C_k are recomputed
 * (nothing is kept from the forward call); the gradient into the state at
 * each chunk boundary is walked backwards over the chunks in fp32 and
 * materialised like C_k; dq, dk and dv are intra-chunk matrix-core products over
 * 64-step tiles as in the forward pass.
 *
 *   q, k, v, igate_pre, fgate_pre: as for tfla_fwd.
 *   dh        [B,H,T,d_hv], the element type of q.
 *   dq, dk    [B,H,T,d_qk] outputs, the element type of q.
 *   dv        [B,H,T,d_hv] output, the element type of q.
 *   dig       fp32 [B,H,T] output for TFLA_MLSTM_SIG; NULL otherwise.
 *   dfg       fp32 output shaped like fgate_pre: [B,H,T] (TFLA_MLSTM_SIG),
 *             [H] (TFLA_SCALAR_DECAY: summed over batches and steps),
 *             [B,H,T,d_qk] (TFLA_GLA_KEY).
 *   Outputs are fully overwritten and must not overlap each other or an
 *   input.
 *   variant   any gate kind | TFLA_IO_BF16, as for tfla_fwd, optionally
 *             | TFLA_BWD_REUSE_FWD: the caller asserts that `workspace` (which
 *             must then be given) was last used by a completed tfla_fwd_ws
 *             call with the same inputs, shape, chunk size and variant (so
 *             without TFLA_STATES_FP32), and
 *             nothing has written its first tfla_workspace_bytes(...) bytes
 *             since; the gate prefix sums and the states C_k found there are
 *             used as they are, skipping their recomputation.  Results are
 *             then bitwise those without the flag.
 *   d_qk      as for tfla_fwd; d_hv 64, 128, 256 or 512, since the dq and
 *             dk products contract over it.
 *   workspace caller-owned device workspace of at least
 *             tfla_bwd_workspace_bytes(...) bytes, 256-byte aligned and
 *             disjoint from every tensor argument, or NULL to let the call
 *             allocate it stream-ordered (hipMallocAsync / hipFreeAsync on
 *             `stream`).
 */
int tfla_bwd(const void* q, const void* k, const void* v,
             const float* igate_pre, const float* fgate_pre, const void* dh,
             void* dq, void* dk, void* dv, float* dig, float* dfg,
             int B, int H, int T, int d_qk, int d_hv, int L, int variant,
             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace tfla_bwd needs; 0 when the arguments are
 * invalid or unsupported. */
size_t tfla_bwd_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant);

/*
 * tfla_bwd_state -- the backward pass of tfla_fwd_state: the forward pass
 * ran from the initial state c0 (NULL: 0), and the loss also depends on the
 * final state C_T through dc_final = dL/dC_T (NULL: it does not), so
 *
 *     dC_T = q_T dh_T^T / sqrt(d_qk) + dc_final,   dL/dC_0 = diag(f_1) dC_1.
 *
 * This is what chains the backward passes of consecutive segments of one
 * sequence (a long sequence trained in pieces, or split over devices): a
 * segment's dc0 is the dc_final of the segment before it, whose c0 chain
 * is the forward pass's.  The forget-gate gradient includes the paths
 * through C_0 and into C_T.
 *
 *   c0        fp32 [B,H,d_qk,d_hv] or NULL, as for tfla_fwd_state.
 *   dc_final  fp32 [B,H,d_qk,d_hv] or NULL.
 *   dc0       fp32 [B,H,d_qk,d_hv] output dL/dC_0, or NULL.  May be the
 *             same pointer as c0 or as dc_final (updated in place).
 *   workspace at least tfla_bwd_state_workspace_bytes(...) bytes, or NULL;
 *             TFLA_BWD_REUSE_FWD is not accepted here.
 * Every other argument and rule is that of tfla_bwd; with c0, dc_final and
 * dc0 all NULL the gradients equal tfla_bwd's.
 */
int tfla_bwd_state(const void* q, const void* k, const void* v,
                   const float* igate_pre, const float* fgate_pre, const float* c0,
                   const void* dh, const float* dc_final,
                   void* dq, void* dk, void* dv, float* dig, float* dfg, float* dc0,
                   int B, int H, int T, int d_qk, int d_hv, int L, int variant,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace tfla_bwd_state needs (whatever of c0, dc_final
 * and dc0 are given); 0 when the arguments are invalid or unsupported. */
size_t tfla_bwd_state_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant);

/*
 * Test hooks: run part of the path and copy its intermediate out.
 *
 * tfla_dbg_gates -- the gate prefix-sum kernel alone.  Outputs (device, fp32):
 *   a_out   chunk-local inclusive sums of the log forget gate:
 *           [B,H,T] (TFLA_GLA_KEY: [B,H,T,d_qk])
 *   li_out  log input gate [B,H,T]
 *   g_out   a at the last step of each chunk: [B,H,ceil(T/L)]
 *           (TFLA_GLA_KEY: [B,H,ceil(T/L),d_qk])
 * For TFLA_SCALAR_DECAY the path computes these in closed form inside the
 * other kernels; this hook evaluates the same closed form.
 *
 * tfla_dbg_states -- gates plus the inter-chunk state kernel.  states_out
 * (device, the I/O type: bf16 with TFLA_IO_BF16 unless TFLA_STATES_FP32 is
 * set, else fp32) receives the state after chunks 1..N_c-1 (N_c = ceil(T/L)),
 * each rounded to that type (RNE) and stored TRANSPOSED as [d_hv][d_qk]:
 * layout [B,H,N_c-1,d_hv,d_qk].
 * q is not needed; h is untouched.
 */
int tfla_dbg_gates(const float* igate_pre, const float* fgate_pre,
                   float* a_out, float* li_out, float* g_out,
                   int B, int H, int T, int d_qk, int L, int variant, void* stream);
int tfla_dbg_states(const void* k, const void* v,
                    const float* igate_pre, const float* fgate_pre, void* states_out,
                    int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* stream);

/*
 * tfla_dbg_stream -- measurement aid, not part of the computation: a plain
 * streaming kernel that measures the HBM rate a kernel on this device
 * reaches.  mode 0 reads `bytes` of `src` (device) and folds them into one
 * register per lane (`dst`: device scratch of at least 4 KB, written only
 * in a case that does not occur); mode 1 copies `bytes` from `src` to `dst`
 * (device, not overlapping).  `loads_per_thread` (1, 2, 4, 8 or 16)
 * independent 16-byte loads per thread per round, `workgroups` (>= 1)
 * workgroups of 256 threads striding over the buffer; both set the bytes a
 * CU keeps in flight.  `bytes` a multiple of 16, pointers 16-byte aligned.
 * Asynchronous on `stream`.  Returns TFLA_ERR_INVALID_ARG for arguments out
 * of these ranges.
 */
int tfla_dbg_stream(int mode, const void* src, void* dst, size_t bytes, int loads_per_thread, int workgroups,
                    void* stream);

/*
 * tfla_dbg_mfma -- measurement aid, not part of the computation: the rate
 * the matrix cores reach on back-to-back 32x32x16 bf16 instructions with
 * register operands.  `workgroups` (>= 1) workgroups of 256 threads, each
 * wavefront running 4 independent accumulator chains of `iters` (>= 1)
 * instructions: 4 * iters * 32768 flops per wavefront, 4 wavefronts per
 * workgroup.  `sink`: device scratch of at least 1 KB, written only in a
 * case that does not occur.  Asynchronous on `stream`.  Returns
 * TFLA_ERR_INVALID_ARG for arguments out of these ranges.
 */
int tfla_dbg_mfma(int iters, int workgroups, void* sink, void* stream);

/*
 * tfla_dbg_lds -- measurement aid, not part of the computation: the rate at
 * which a CU serves the LDS operand reads of the intra-chunk kernels, alone
 * and each feeding one 32x32x16 bf16 matrix instruction.  `workgroups` (>= 1)
 * workgroups of `waves` (4 or 8) wavefronts, each holding 96 KB of LDS (one
 * per CU); every wavefront runs `iters` (>= 1) iterations of 8 fragment reads
 * of 1 KB (64 lanes x 16 bytes): mode 0 16-byte row reads of a 64 x 264 bf16
 * tile, mode 1 transpose reads (ds_read_b64_tr_b16) of a 64 x 160 tile, modes
 * 2 and 3 the same with each fragment the A operand of one matrix
 * instruction (4 independent accumulator chains), mode 4 the 8 instructions
 * alone on a register operand.  `clocks` (device, 2 * workgroups uint64):
 * the shader clock of each workgroup before and after its loop, both after a
 * barrier.  `sink`: device scratch of at least 2 KB, written only in a case
 * that does not occur.  Asynchronous on `stream`.  Returns
 * TFLA_ERR_INVALID_ARG for arguments out of these ranges.
 */
int tfla_dbg_lds(int mode, int waves, int iters, int workgroups, void* clocks, void* sink, void* stream);

/*
 * tfla_dbg_set_knob -- test hook: process-wide overrides of choices the
 * library otherwise makes from the problem shape, for tests that must reach
 * a particular kernel at a small size and for tuning comparisons.  `value`
 * < 0 restores the default.  Results stay correct under every setting
 * (only the kernel choice or tiling changes), except TFLA_KNOB_FAULT_ALLOC,
 * which makes the library's own workspace allocations fail.  Calls that
 * run while a knob changes may see either setting.  Returns
 * TFLA_ERR_INVALID_ARG for an unknown knob.
 */
enum tfla_knob {
    TFLA_KNOB_INTRA_SWEEP = 0,     /* 0: the per-tile intra-chunk kernel where the value sweep
                                      would run                                               */
    TFLA_KNOB_INTRA_BV = 1,        /* 64: cap the per-tile kernel's value tile at 64 columns  */
    TFLA_KNOB_INTRA_ROWS = 2,      /* 64, 128 or 256: cap its query rows per workgroup        */
    TFLA_KNOB_STATE_SEGMENTS = 3,  /* n >= 1: the state walk's segment count                  */
    TFLA_KNOB_STATE_SB = 4,        /* 64 or 128: cap the state walk's block of steps          */
    TFLA_KNOB_FAULT_ALLOC = 5,     /* 1: the library's own workspace allocations fail         */
    TFLA_KNOB_STATE_REWALK = 6,    /* 1: the forward segmented state walk walks every segment
                                      again from its true start instead of fixing up the
                                      states it stored (the fixed decay always does)          */
    TFLA_KNOB_COUNT = 7
};
int tfla_dbg_set_knob(int knob, int value);

/* Static description of a status code. */
const char* tfla_error_string(int code);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* tfla_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int tfla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TFLA_H */

// kernels.hpp -- host-side launchers of the libtfla kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace tfla {

enum GateKind { kSig = 0, kScalar = 1, kGla = 2, kExp = 3 };

// mLSTMsig and mLSTMexp share the per-step exponents of the chunkwise form
// (mLSTMexp's are stabilised by its max state; see gates_exp.hip)
constexpr bool per_step_li(int gate) { return gate == kSig || gate == kExp; }

// Test and tuning overrides set through tfla_dbg_set_knob (tfla.h knob
// numbers); -1 when unset, which every reader takes as "the default".  The
// library reads no environment variable.
int knob(int which);

// Operand modes of the intra-chunk kernel (bit set) for the gradient products;
// kStateF32: the forward pass reading fp32 states with bf16 I/O.
enum IntraMode { kNatState = 1, kMirror = 2, kRowDots = 4, kEmitP = 8, kGivenP = 16, kStateF32 = 32 };

// Problem description shared by the launchers.  Sizes in elements.
struct Problem {
    int B, H, T, dqk, dhv, L;
    int nc;          // number of chunks, ceil(T / L)
    int gate;        // GateKind
    bool bf16;       // element type of q, k, v, h
    bool st32 = false;   // states materialised in fp32 (always for fp32 I/O)
    bool walk_norm = false;   // mLSTMexp: the state walk also forms the normaliser states
};

// Workspace carve-up (device pointers into one allocation).
struct Workspace {
    float* a;        // [B,H,T] (GLA: [B,H,T,dqk]) chunk-local log-forget sums; NULL for kScalar
    float* li;       // [B,H,T] log input gate; kSig only
    float* g;        // [B,H,nc] (GLA: [B,H,nc,dqk]); NULL for kScalar
    // per-channel gate: k_t o e^{g_k - a_t} in the I/O type, the forward state
    // walk's weighted keys, formed by the gate kernel (NULL: the walk weights K)
    void* kw = nullptr;
    void* states;    // [B,H,ns,dhv,dqk] I/O type (fp32 when Problem::st32),
                     // transposed states before chunks (walked in fp32; the
                     // intra-chunk kernel rounds them to the I/O type for its
                     // matrix cores anyway)
                     // 1..nc-1 (ns = nc-1), or 0..nc-1 with an initial state (ns = nc)
    // mLSTMexp (kExp): a, li and g hold its stabilised exponents (the
    // mLSTMsig kernels then form the stabilised numerator), plus
    float* lb = nullptr;      // [B,H,T] log of the lower bound of the normaliser, -(a_t + M_t)
    float* nst = nullptr;     // [B,H,nc-1,dqk] stabilised normaliser state before chunks 1..nc-1
    float* npart = nullptr;   // [B,H,nc,dqk] each chunk's own normaliser contribution
    float* mprev = nullptr;   // [B,H,nc] max state entering each chunk
    float* uk = nullptr;      // [B,H,nc] chunk maximum of igate_pre - a
    const float* c0 = nullptr;   // caller's initial state [B,H,dqk,dhv] (NULL: zero)
    float* c_final = nullptr;    // caller's final-state output [B,H,dqk,dhv] (NULL: none)
    float* seg_end = nullptr;    // segmented state walk: end states [B*H][P][dqk][dhv]
    float* seg_start = nullptr;  //                       start states [B*H][P][dqk][dhv]
    // intra-chunk gradient modes with kRowDots: per output row and value
    // tile, the dot product of the fp32 output row with the same row of
    // `dot_partner` (an I/O-typed [B,H,T,out] tensor), into dots [B,H,T][out/BV].
    // Reverse state walk: `dot_partner` = the forward states (the type and
    // layout of `states`), dots = per-wave partials of <D_m, C_m>
    // [B,H,nc-1][state_dot_parts(p)].
    const void* dot_partner = nullptr;
    float* dots = nullptr;
    // reverse walk: slots per head of the forward states in dot_partner and
    // the slot of the state after chunk 0 (1 when they begin with C_0);
    // boundaries per head in dots; factor on the end state written to c_final
    int dot_slots = 0, dot_off = 0, dot_bound = 0;
    float end_scale = 1.0f;
    // intra-chunk kEmitP: P out ([B,H,T,L], I/O type); kGivenP: P read
    void* p_out = nullptr;
    const void* p_in = nullptr;
};

// Segmented state walk (few heads, long sequences): number of segments P
// (1: unsegmented), chunks per segment, and whether 128x128 state tiles
// are used.  Functions of the problem shape only.
int state_segments(const Problem& p);
// mLSTMexp: the (unsegmented) state walk forms the normaliser states beside
// the numerator states, so the gate kernels leave them out
bool exp_walk_normaliser(const Problem& p);
int state_segments_for(const Problem& p, long heads_tiles);
int state_chunks_per_segment(const Problem& p, int P);
// Value-tile width of the intra-chunk kernel for an output width p.dhv
// contracted over p.dqk (the number of row-dot partials is p.dhv / BV).
int intra_value_tile(const Problem& p);
bool state_big_tiles(const Problem& p);
// Partials per chunk boundary of the reverse walk's state product (tiles x
// waves; per-channel gate: per key channel, value tiles x 2).
int state_dot_parts(const Problem& p);

// Lays the workspace out from `base` (NULL: sizes only); returns its byte size.
// with_c0 reserves the extra state slot an initial state needs.
size_t workspace_layout(const Problem& p, Workspace* ws, char* base, bool with_states = true,
                        bool with_c0 = false);

// k: the keys, for the per-channel gate's weighted keys (ws.kw); may be NULL
hipError_t launch_gates(const Problem& p, const void* k, const float* igate_pre, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream);
// mLSTMexp's gate work (gates_exp.hip): fills ws.a, ws.li, ws.g with its
// stabilised exponents and ws.lb, ws.nst (ws.npart, ws.mprev, ws.uk as
// scratch); k is read for the normaliser.
hipError_t launch_gates_exp(const Problem& p, const void* k, const float* igate_pre, const float* fgate_pre,
                            const Workspace& ws, hipStream_t stream);
hipError_t launch_gates_closed_form(const Problem& p, const float* fgate_pre, float* a, float* li,
                                    float* g, hipStream_t stream);
hipError_t launch_state(const Problem& p, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream);
// The reverse state walk of the backward pass: ws.states receives
// D_0..D_{nc-2} (D_j: gradient into the state from the chunks after chunk
// j, without the 1/sqrt(d_qk) factor), transposed [d_hv][d_qk], followed by
// D_{nc-1} when ws.c0 holds one (the final-state gradient, same factor,
// [d_qk][d_hv]); ws.c_final receives D_{-1} * ws.end_scale when given.
hipError_t launch_state_rev(const Problem& p, const void* q, const void* dh, const float* fgate_pre,
                            const Workspace& ws, hipStream_t stream);
hipError_t launch_recurrent(const Problem& p, const void* q, const void* k, const void* v,
                            const float* igate_pre, const float* fgate_pre, float* state, void* h,
                            hipStream_t stream);
hipError_t launch_intra(const Problem& p, const void* q, const void* k, const void* v,
                        const float* fgate_pre, const Workspace& ws, void* h, hipStream_t stream);
// The forward intra-chunk kernel that forms a chunk's P once and sweeps
// every value tile with it (launch_intra picks it where intra_sweeps holds).
bool intra_sweeps(const Problem& p);
bool intra_sweeps_dv(const Problem& p);   // the same for the dv product

// plain streaming kernels (probe.hip): mode 0 reads `bytes` of src, mode 1
// copies them to dst; `loads` 16-byte loads per thread per round (1, 2, 4, 8
// or 16), `blocks` workgroups of 256 threads
hipError_t launch_stream_probe(int mode, const void* src, void* dst, size_t bytes, int loads, int blocks,
                               hipStream_t stream);
// back-to-back bf16 matrix instructions (4 x 32768 flops per wavefront per iteration)
hipError_t launch_mfma_probe(int iters, int blocks, float* sink, hipStream_t stream);
hipError_t launch_lds_probe(int mode, int waves, int iters, int blocks, unsigned long long* out, float* sink,
                            hipStream_t stream);
hipError_t launch_intra_sweep(const Problem& p, const void* q, const void* k, const void* v,
                              const float* fgate_pre, const Workspace& ws, void* h, hipStream_t stream);
// The same kernel in the dv gradient mode (mirrored chunks; see launch_intra_dv).
hipError_t launch_intra_sweep_dv(const Problem& p, const void* q, const void* k, const void* v,
                                 const float* fgate_pre, const Workspace& ws, void* out, float scale,
                                 hipStream_t stream);
// The intra-chunk kernel in its gradient modes (dq: kNatState | kRowDots;
// dk: kNatState | kMirror | kRowDots; dv: kMirror): p.dqk is the contracted width (64..512),
// p.dhv the output width; ws.a / ws.li / ws.states as the mode reads them;
// every output row scaled by `scale`.
hipError_t launch_intra_dq(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                           const Workspace& ws, void* out, float scale, hipStream_t stream);
hipError_t launch_intra_dk(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                           const Workspace& ws, void* out, float scale, hipStream_t stream);
// The shared P of dq and dk (per-step gates): kEmitP over the dq operands,
// then dq and dk with kGivenP reading it (dk transposed, in mirrored order).
hipError_t launch_intra_p(const Problem& p, const void* q, const void* k, const float* fgate_pre,
                          const Workspace& ws, hipStream_t stream);
hipError_t launch_intra_dq_p(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                             const Workspace& ws, void* out, float scale, hipStream_t stream);
hipError_t launch_intra_dk_p(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                             const Workspace& ws, void* out, float scale, hipStream_t stream);
hipError_t launch_intra_dv(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                           const Workspace& ws, void* out, float scale, hipStream_t stream);

// Backward-pass gate work: mirrored gate exponents for the mirrored intra
// mode (mLSTMsig), and the input / forget gate gradients from the dq and dk
// kernels' row partials (q_t.dq_t and k_t.dk_t, np per step, [B,H,T][np])
// and the reverse walk's partials of <D_m, C_m> (nx per boundary,
// [B,H,nbound][nx], nbound = nc-1, or nc with a final-state gradient);
// with_states: an initial state or a final-state gradient is present;
// head_part: [B,H] double scratch of the fixed decay.
hipError_t launch_gates_mirror(const Problem& p, const Workspace& ws, float* ar, float* lr, hipStream_t stream);
hipError_t launch_gate_grads(const Problem& p, const float* xpart, int nx, int nbound, bool with_states,
                             const float* dq_dots, const float* dk_dots, int np, const float* igate_pre,
                             const float* fgate_pre, float* dig, float* dfg, double* head_part, hipStream_t stream);
// y = a x (n floats)
hipError_t launch_scale_copy(const float* x, float* y, size_t n, float a, hipStream_t stream);
// the coupling across the end of the sequence, <dC_T sqrt(d_qk), C_T>, into
// boundary nbound-1 of xpart (per key channel for the per-channel gate)
hipError_t launch_final_coupling(const Problem& p, const float* g_scaled, const float* c_final, float* xpart, int nx,
                                 int nbound, hipStream_t stream);

}  // namespace tfla

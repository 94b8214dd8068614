// tfla_api.cpp -- the C ABI declared in include/tfla.h: argument validation
// (no HIP call before it passes), workspace sizing and carve-up, and the
// launches of the forward and backward paths on the caller's stream.
#include "tfla.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};
Range range_of(const void* p, size_t bytes)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }


// Shape and variant checks shared by every entry point.  Fills *p.
int check_problem(int B, int H, int T, int d_qk, int d_hv, int L, int variant, tfla::Problem* p)
{
    const int gate = variant & 0xff;
    if ((variant & ~(0xff | TFLA_IO_BF16 | TFLA_STATES_FP32)) != 0 || gate > TFLA_MLSTM_EXP || gate < 0)
        return fail(TFLA_ERR_INVALID_ARG, "unknown variant " + std::to_string(variant));
    if (B < 1 || H < 1 || T < 1 || d_qk < 1 || d_hv < 1 || L < 1)
        return fail(TFLA_ERR_INVALID_ARG, "B, H, T, d_qk, d_hv and L must be >= 1");
    const bool bf16 = (variant & TFLA_IO_BF16) != 0;
    if (!(d_qk == 64 || d_qk == 128 || d_qk == 256))
        return fail(TFLA_ERR_UNSUPPORTED, "d_qk must be 64, 128 or 256, got " + std::to_string(d_qk));
    if (d_hv % 64 != 0 || d_hv > 512)
        return fail(TFLA_ERR_UNSUPPORTED, "d_hv must be a multiple of 64 up to 512, got " + std::to_string(d_hv));
    if (!(L == 64 || L == 128 || L == 256 || L == 512 || L == 1024))
        return fail(TFLA_ERR_UNSUPPORTED, "chunk size L must be 64, 128, 256, 512 or 1024, got " +
                                              std::to_string(L));
    const long long bh = (long long)B * H;
    if (bh > 65535) return fail(TFLA_ERR_UNSUPPORTED, "B*H must be <= 65535");
    const long long nqt = (T + 63) / 64;
    if (bh * nqt * (d_hv / 64) > 0x7fffffffLL)
        return fail(TFLA_ERR_UNSUPPORTED, "problem too large for one launch grid");
    p->B = B;
    p->H = H;
    p->T = T;
    p->dqk = d_qk;
    p->dhv = d_hv;
    p->L = L;
    p->nc = (T + L - 1) / L;
    p->gate = gate;
    p->bf16 = bf16;
    p->st32 = !bf16 || (variant & TFLA_STATES_FP32) != 0;
    return TFLA_OK;
}

int check_gates(const tfla::Problem& p, const float* igate_pre, const float* fgate_pre)
{
    if (!fgate_pre) return fail(TFLA_ERR_INVALID_ARG, "fgate_pre is NULL");
    if (!aligned(fgate_pre, 4)) return fail(TFLA_ERR_INVALID_ARG, "fgate_pre is not 4-byte aligned");
    // the per-channel gate kernel reads rows of fgate_pre in 16-byte pieces
    if (p.gate == tfla::kGla && !aligned(fgate_pre, 16))
        return fail(TFLA_ERR_INVALID_ARG, "fgate_pre (per-channel gate) is not 16-byte aligned");
    if (tfla::per_step_li(p.gate)) {
        if (!igate_pre) return fail(TFLA_ERR_INVALID_ARG, "igate_pre is NULL but the variant has an input gate");
        if (!aligned(igate_pre, 4)) return fail(TFLA_ERR_INVALID_ARG, "igate_pre is not 4-byte aligned");
    } else if (igate_pre) {
        return fail(TFLA_ERR_INVALID_ARG, "igate_pre must be NULL for this variant (input gate is 1)");
    }
    return TFLA_OK;
}

size_t gate_bytes(const tfla::Problem& p)
{
    const size_t bh = (size_t)p.B * p.H;
    if (tfla::per_step_li(p.gate)) return bh * p.T * 4;
    if (p.gate == tfla::kScalar) return (size_t)p.H * 4;
    return bh * p.T * p.dqk * 4;
}

// Byte ranges of the tensors of a forward call: q, k, v, h, fgate_pre, igate_pre.
void fwd_ranges(const tfla::Problem& p, const void* q, const void* k, const void* v, const float* igate_pre,
                const float* fgate_pre, const void* h, Range out[6])
{
    const size_t esz = p.bf16 ? 2 : 4;
    const size_t bht = (size_t)p.B * p.H * p.T;
    out[0] = range_of(q, bht * p.dqk * esz);
    out[1] = range_of(k, bht * p.dqk * esz);
    out[2] = range_of(v, bht * p.dhv * esz);
    out[3] = range_of(h, bht * p.dhv * esz);
    out[4] = range_of(fgate_pre, gate_bytes(p));
    out[5] = igate_pre ? range_of(igate_pre, bht * 4) : Range{0, 0};
}

// The caller's workspace must not share a byte with any tensor of the call.
int check_workspace_disjoint(const void* workspace, size_t bytes, const Range* tensors, size_t n)
{
    const Range w = range_of(workspace, bytes);
    for (size_t i = 0; i < n; ++i)
        if (overlaps(w, tensors[i])) return fail(TFLA_ERR_INVALID_ARG, "workspace overlaps an input or output");
    return TFLA_OK;
}

int check_fwd(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
              const void* h, int B, int H, int T, int d_qk, int d_hv, int L, int variant, tfla::Problem* p)
{
    int rc = check_problem(B, H, T, d_qk, d_hv, L, variant, p);
    if (rc) return rc;
    if (!q || !k || !v || !h) return fail(TFLA_ERR_INVALID_ARG, "q, k, v and h must not be NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(h, 16))
        return fail(TFLA_ERR_INVALID_ARG, "q, k, v and h must be 16-byte aligned");
    rc = check_gates(*p, igate_pre, fgate_pre);
    if (rc) return rc;
    const size_t esz = p->bf16 ? 2 : 4;
    const size_t bht = (size_t)B * H * T;
    const Range hr = range_of(h, bht * d_hv * esz);
    if (overlaps(hr, range_of(q, bht * d_qk * esz)) || overlaps(hr, range_of(k, bht * d_qk * esz)) ||
        overlaps(hr, range_of(v, bht * d_hv * esz)) || overlaps(hr, range_of(fgate_pre, gate_bytes(*p))) ||
        (igate_pre && overlaps(hr, range_of(igate_pre, bht * 4))))
        return fail(TFLA_ERR_INVALID_ARG, "h overlaps an input");
    return TFLA_OK;
}

// Initial / final state buffers: fp32 [B,H,d_qk,d_hv], 16-byte aligned.
// c_final may be c0 itself (in-place update); otherwise neither overlaps an
// input or h.
int check_state_io(const tfla::Problem& p, const void* q, const void* k, const void* v, const float* igate_pre,
                   const float* fgate_pre, const void* h, const float* c0, const float* c_final)
{
    if ((c0 && !aligned(c0, 16)) || (c_final && !aligned(c_final, 16)))
        return fail(TFLA_ERR_INVALID_ARG, "c0 and c_final must be 16-byte aligned");
    const size_t esz = p.bf16 ? 2 : 4;
    const size_t bht = (size_t)p.B * p.H * p.T;
    const size_t sbytes = (size_t)p.B * p.H * p.dqk * p.dhv * 4;
    const Range ins[] = {range_of(q, bht * p.dqk * esz), range_of(k, bht * p.dqk * esz),
                         range_of(v, bht * p.dhv * esz), range_of(h, bht * p.dhv * esz),
                         range_of(fgate_pre, gate_bytes(p)),
                         igate_pre ? range_of(igate_pre, bht * 4) : Range{0, 0}};
    for (const float* st : {c0, c_final}) {
        if (!st) continue;
        const Range r = range_of(st, sbytes);
        for (const Range& x : ins)
            if (overlaps(r, x)) return fail(TFLA_ERR_INVALID_ARG, "c0 / c_final overlaps q, k, v, h or a gate");
    }
    if (c0 && c_final && c0 != c_final && overlaps(range_of(c0, sbytes), range_of(c_final, sbytes)))
        return fail(TFLA_ERR_INVALID_ARG, "c_final overlaps c0 without being the same buffer");
    return TFLA_OK;
}

// ---- the allocation-free entry point's scratch ------------------------------
// tfla_fwd_noalloc keeps its workspace in this file-scope device array (one
// copy per GPU, held until the process ends).  Host code never uses the
// array's name as an address: on each device the address comes from
// hipGetSymbolAddress once, with that device current, and is cached here.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device; NULL after a failure (message
// in *err).
void* scratch_on_current_device(std::string* err)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = std::string("no usable current device: ") + hipGetErrorString(e);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *err = std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e);
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Test and tuning overrides (tfla_dbg_set_knob): -1 = unset.
std::atomic<int> g_knobs[TFLA_KNOB_COUNT] = {-1, -1, -1, -1, -1, -1, -1};

// Failure injection for tests of the error paths: the fault knob set to 1
// makes the library's own workspace allocation fail before any launch.
bool inject_alloc_fault() { return tfla::knob(TFLA_KNOB_FAULT_ALLOC) == 1; }

int hip_fail(hipError_t e, const char* what)
{
    return fail(TFLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int mark(void* const* marks, int i, hipStream_t stream)
{
    if (!marks) return TFLA_OK;
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(marks[i]), stream);
    return e == hipSuccess ? TFLA_OK : hip_fail(e, "timing mark");
}

int run_path(const tfla::Problem& p, const void* q, const void* k, const void* v, const float* igate_pre,
             const float* fgate_pre, void* h, const tfla::Workspace& ws, hipStream_t stream,
             void* const* marks = nullptr)
{
    int rc = mark(marks, 0, stream);
    if (rc) return rc;
    hipError_t e = p.gate == tfla::kExp ? tfla::launch_gates_exp(p, k, igate_pre, fgate_pre, ws, stream)
                                        : tfla::launch_gates(p, k, igate_pre, fgate_pre, ws, stream);
    if (e != hipSuccess) return hip_fail(e, "gate kernel launch");
    if ((rc = mark(marks, 1, stream))) return rc;
    e = tfla::launch_state(p, k, v, fgate_pre, ws, stream);
    if (e != hipSuccess) return hip_fail(e, "state kernel launch");
    if ((rc = mark(marks, 2, stream))) return rc;
    e = tfla::launch_intra(p, q, k, v, fgate_pre, ws, h, stream);
    if (e != hipSuccess) return hip_fail(e, "intra-chunk kernel launch");
    return mark(marks, 3, stream);
}

// Backward pass: the forward workspace, then the reverse-walk states, the
// mirrored gate exponents (mLSTMsig) and the per-step gate-gradient sums.
struct BwdWorkspace {
    tfla::Workspace fwd;
    void* dstates;    // [B,H,nc-1,d_hv,d_qk], I/O type
    float* ar;        // [B,H,T] mLSTMsig, [B,H,T,d_qk] per-channel gate
    float* lr;        // [B,H,T] mLSTMsig
    float* dq_dots;   // [B,H,T][np]: q_t . dq_t per value tile of the dq kernel
                      // (per-channel gate: np = d_qk per-element products)
    float* dk_dots;   // [B,H,T][np]: k_t . dk_t likewise
    float* xpart;     // [B,H,nc-1][nx]: partials of <D_k, C_k> across each chunk boundary
                      // (per-channel gate: [B,H,nc-1,d_qk][nx])
    double* head_part;  // [B,H]: per-(batch, head) part of the fixed decay's gradient
    void* pmat;       // per-step gates: the shared P of dq and dk [B,H,T,L], I/O type
    float* g_scaled;  // tfla_bwd_state: the final-state gradient times sqrt(d_qk) [B,H,d_qk,d_hv]
    float* c_T;       // tfla_bwd_state: the recomputed final state [B,H,d_qk,d_hv]
    int np, nx;
};

// The state arguments of tfla_bwd_state (all NULL for tfla_bwd).
struct BwdStateIO {
    const float* c0 = nullptr;         // initial state C_0
    const float* dc_final = nullptr;   // dL/dC_T
    float* dc0 = nullptr;              // receives dL/dC_0
};

// the dq and dk products: contract d_hv, emit d_qk
tfla::Problem grad_qk_problem(const tfla::Problem& p)
{
    tfla::Problem pc = p;
    pc.dqk = p.dhv;
    pc.dhv = p.dqk;
    return pc;
}

// dq and dk take a P computed once (per-step gates) where each would
// otherwise recompute S = dh V^T for several value tiles of d_qk; with one
// tile the separate P pass costs more than it saves (measured).
bool shares_p(const tfla::Problem& p)
{
    if (p.gate == tfla::kGla) return false;
    // fp32 I/O, 256- or 512-wide contraction: the P pass holds no
    // accumulators, and dq / dk given P hold no Q fragments, where forming
    // P inside them would spill hundreds of registers
    if (!p.bf16 && p.dhv >= 256) return true;
    const tfla::Problem pc = grad_qk_problem(p);
    return pc.dhv / tfla::intra_value_tile(pc) >= 2;
}

// with_states: the layout of tfla_bwd_state (a slot for C_0 among the
// forward states, one for the final-state gradient among the reverse-walk
// states, a coupling across the end of the sequence, C_T and the scaled
// final-state gradient)
size_t bwd_layout(const tfla::Problem& p, BwdWorkspace* ws, char* base, bool with_states = false)
{
    size_t off = tfla::workspace_layout(p, &ws->fwd, base, true, with_states);
    const size_t bh = (size_t)p.B * p.H;
    auto take = [&](size_t bytes) -> float* {
        float* ptr = base ? reinterpret_cast<float*>(base + off) : nullptr;
        off += align256(bytes);
        return ptr;
    };
    const size_t rslots = p.nc - 1 + (with_states ? 1 : 0);   // reverse-walk states
    ws->dstates = rslots > 0 ? take(bh * rslots * p.dhv * p.dqk * (p.bf16 ? 2 : 4)) : nullptr;
    const bool sig = p.gate == tfla::kSig, gla = p.gate == tfla::kGla;
    ws->ar = sig ? take(bh * p.T * 4) : gla ? take(bh * p.T * p.dqk * 4) : nullptr;
    ws->lr = sig ? take(bh * p.T * 4) : nullptr;
    ws->np = gla ? p.dqk : p.dqk / tfla::intra_value_tile(grad_qk_problem(p));
    ws->dq_dots = take(bh * p.T * ws->np * 4);
    ws->dk_dots = take(bh * p.T * ws->np * 4);
    ws->nx = tfla::state_dot_parts(p);
    const size_t per_boundary = (size_t)ws->nx * (p.gate == tfla::kGla ? p.dqk : 1);
    ws->xpart = rslots > 0 ? take(bh * rslots * per_boundary * 4) : nullptr;
    ws->head_part = p.gate == tfla::kScalar ? reinterpret_cast<double*>(take(bh * 8)) : nullptr;
    const size_t pbytes = shares_p(p) ? bh * p.T * p.L * (p.bf16 ? 2 : 4) : 0;
    ws->pmat = pbytes ? take(pbytes) : nullptr;
    const size_t sbytes = bh * p.dqk * p.dhv * 4;
    ws->g_scaled = with_states ? take(sbytes) : nullptr;
    ws->c_T = with_states ? take(sbytes) : nullptr;
    return off;
}

// Shapes the backward pass is built for: d_hv (the width the dq and dk
// products contract) a power of two the intra kernel is instantiated for.
int check_bwd_problem(int B, int H, int T, int d_qk, int d_hv, int L, int variant, tfla::Problem* p)
{
    if (variant & TFLA_STATES_FP32)
        return fail(TFLA_ERR_UNSUPPORTED, "TFLA_STATES_FP32 is an option of the forward calls only");
    int rc = check_problem(B, H, T, d_qk, d_hv, L, variant & ~TFLA_BWD_REUSE_FWD, p);
    if (rc) return rc;
    if (p->gate == tfla::kExp) return fail(TFLA_ERR_UNSUPPORTED, "mLSTMexp has a forward pass only (no backward)");
    if (!(d_hv == 64 || d_hv == 128 || d_hv == 256 || d_hv == 512))
        return fail(TFLA_ERR_UNSUPPORTED, "backward: d_hv must be 64, 128, 256 or 512, got " + std::to_string(d_hv));
    return TFLA_OK;
}

int run_bwd(const tfla::Problem& p, const void* q, const void* k, const void* v, const float* igate_pre,
            const float* fgate_pre, const void* dh, void* dq, void* dk, void* dv, float* dig, float* dfg,
            const BwdWorkspace& ws, bool reuse_fwd, const BwdStateIO& io, hipStream_t stream)
{
    const float scale = 1.0f / sqrtf((float)p.dqk);
    const bool has_c0 = io.c0 != nullptr, has_g = io.dc_final != nullptr;
    const int nbound = p.nc - 1 + (has_g ? 1 : 0);   // chunk boundaries with a coupling
    hipError_t e;
    if (!reuse_fwd) {
        if ((e = tfla::launch_gates(p, k, igate_pre, fgate_pre, ws.fwd, stream)) != hipSuccess)
            return hip_fail(e, "gate kernel launch");
        // forward states C_1..C_{nc-1}, [d_hv][d_qk] each (preceded by C_0 when
        // given), and C_T when a final-state gradient needs its coupling
        tfla::Workspace fw = ws.fwd;
        fw.c0 = io.c0;
        fw.c_final = has_g ? ws.c_T : nullptr;
        if ((e = tfla::launch_state(p, k, v, fgate_pre, fw, stream)) != hipSuccess)
            return hip_fail(e, "state kernel launch");
    }
    tfla::Workspace mirrored = ws.fwd;   // gate exponents of the mirrored chunks
    if (p.gate != tfla::kScalar) {
        if ((e = tfla::launch_gates_mirror(p, ws.fwd, ws.ar, ws.lr, stream)) != hipSuccess)
            return hip_fail(e, "mirrored gate kernel launch");
        mirrored.a = ws.ar;
        mirrored.li = ws.lr;
    }
    // reverse walk: D_0..D_{nc-2}, [d_hv][d_qk] each, then D_{nc-1} = dC_T sqrt(d_qk)
    // when given; dL/dC_0 = D_{-1} / sqrt(d_qk) on request
    if (has_g && (e = tfla::launch_scale_copy(io.dc_final, ws.g_scaled, (size_t)p.B * p.H * p.dqk * p.dhv,
                                              sqrtf((float)p.dqk), stream)) != hipSuccess)
        return hip_fail(e, "final-state gradient copy");
    tfla::Workspace rev = ws.fwd;
    rev.states = ws.dstates;
    rev.c0 = has_g ? ws.g_scaled : nullptr;
    rev.c_final = io.dc0;
    rev.end_scale = scale;
    rev.dot_partner = ws.fwd.states;
    rev.dots = ws.xpart;
    rev.dot_slots = p.nc - 1 + (has_c0 ? 1 : 0);
    rev.dot_off = has_c0 ? 1 : 0;
    rev.dot_bound = nbound;
    if ((e = tfla::launch_state_rev(p, q, dh, fgate_pre, rev, stream)) != hipSuccess)
        return hip_fail(e, "reverse state kernel launch");
    if (has_g && (e = tfla::launch_final_coupling(p, ws.g_scaled, ws.c_T, ws.xpart, ws.nx, nbound, stream)) !=
                     hipSuccess)
        return hip_fail(e, "final coupling kernel launch");
    mirrored.states = ws.dstates;
    mirrored.c0 = has_g ? ws.g_scaled : nullptr;   // the last chunk reads the final-state gradient
    // dq = scale (e^{a_t} C_{k-1} dh_t + sum_{s<=t} w_ts (dh_t . v_s) k_s): contract d_hv, emit d_qk
    const tfla::Problem pc = grad_qk_problem(p);
    // P_ts = w_ts (dh_t . v_s) once per chunk, shared by dq (P k) and dk (P^T q)
    const bool shared_p = shares_p(p);
    if (shared_p) {
        tfla::Workspace wp = ws.fwd;
        wp.p_out = ws.pmat;
        tfla::Problem pp = pc;
        pp.dhv = 64;   // one value tile: every query tile of the grid computes its P rows once
        if ((e = tfla::launch_intra_p(pp, dh, v, fgate_pre, wp, stream)) != hipSuccess)
            return hip_fail(e, "shared P kernel launch");
    }
    tfla::Workspace wq = ws.fwd;
    wq.c0 = io.c0;   // the first chunk reads C_0 from the states
    wq.dot_partner = q;
    wq.dots = ws.dq_dots;
    wq.p_in = ws.pmat;
    e = shared_p ? tfla::launch_intra_dq_p(pc, dh, v, k, fgate_pre, wq, dq, scale, stream)
                 : tfla::launch_intra_dq(pc, dh, v, k, fgate_pre, wq, dq, scale, stream);
    if (e != hipSuccess) return hip_fail(e, "dq kernel launch");
    // dk = scale (e^{a'_t} D_k v_t + sum_{s>=t} w_st (v_t . dh_s) q_s): mirrored, contract d_hv
    tfla::Workspace wk = mirrored;
    wk.dot_partner = k;
    wk.dots = ws.dk_dots;
    wk.p_in = ws.pmat;
    e = shared_p ? tfla::launch_intra_dk_p(pc, v, dh, q, fgate_pre, wk, dk, scale, stream)
                 : tfla::launch_intra_dk(pc, v, dh, q, fgate_pre, wk, dk, scale, stream);
    if (e != hipSuccess) return hip_fail(e, "dk kernel launch");
    // dv = scale (e^{a'_t} D_k^T k_t + sum_{s>=t} w_st (k_t . q_s) dh_s): mirrored, contract d_qk
    if ((e = tfla::launch_intra_dv(p, k, q, dh, fgate_pre, mirrored, dv, scale, stream)) != hipSuccess)
        return hip_fail(e, "dv kernel launch");
    if ((e = tfla::launch_gate_grads(p, ws.xpart, ws.nx, nbound, has_c0 || has_g, ws.dq_dots, ws.dk_dots, ws.np,
                                     igate_pre, fgate_pre, dig, dfg, ws.head_part, stream)) != hipSuccess)
        return hip_fail(e, "gate gradient kernel launch");
    return TFLA_OK;
}

int check_bwd(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
              const void* dh, const void* dq, const void* dk, const void* dv, const float* dig, const float* dfg,
              int B, int H, int T, int d_qk, int d_hv, int L, int variant, tfla::Problem* p)
{
    int rc = check_bwd_problem(B, H, T, d_qk, d_hv, L, variant, p);
    if (rc) return rc;
    if (!q || !k || !v || !dh || !dq || !dk || !dv)
        return fail(TFLA_ERR_INVALID_ARG, "q, k, v, dh, dq, dk and dv must not be NULL");
    for (const void* x : {q, k, v, dh, dq, dk, dv})
        if (!aligned(x, 16)) return fail(TFLA_ERR_INVALID_ARG, "q, k, v, dh, dq, dk and dv must be 16-byte aligned");
    if ((rc = check_gates(*p, igate_pre, fgate_pre))) return rc;
    if (!dfg || !aligned(dfg, 4)) return fail(TFLA_ERR_INVALID_ARG, "dfg must be non-NULL and 4-byte aligned");
    if (p->gate == tfla::kSig) {
        if (!dig || !aligned(dig, 4))
            return fail(TFLA_ERR_INVALID_ARG, "dig must be non-NULL and 4-byte aligned for mLSTMsig");
    } else if (dig) {
        return fail(TFLA_ERR_INVALID_ARG, "dig must be NULL for this variant (input gate is 1)");
    }
    const size_t esz = p->bf16 ? 2 : 4;
    const size_t bht = (size_t)B * H * T;
    const Range ins[] = {range_of(q, bht * d_qk * esz), range_of(k, bht * d_qk * esz),
                         range_of(v, bht * d_hv * esz), range_of(dh, bht * d_hv * esz),
                         range_of(fgate_pre, gate_bytes(*p)),
                         igate_pre ? range_of(igate_pre, bht * 4) : Range{0, 0}};
    const Range outs[] = {range_of(dq, bht * d_qk * esz), range_of(dk, bht * d_qk * esz),
                          range_of(dv, bht * d_hv * esz), range_of(dfg, gate_bytes(*p)),
                          dig ? range_of(dig, bht * 4) : Range{0, 0}};
    for (size_t i = 0; i < 5; ++i) {
        for (const Range& x : ins)
            if (overlaps(outs[i], x)) return fail(TFLA_ERR_INVALID_ARG, "a gradient output overlaps an input");
        for (size_t j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outs[j])) return fail(TFLA_ERR_INVALID_ARG, "gradient outputs overlap");
    }
    return TFLA_OK;
}

// tfla_bwd_state's state buffers: fp32 [B,H,d_qk,d_hv], 16-byte aligned,
// disjoint from every other tensor of the call; dc0 may be c0 or dc_final
// itself (updated in place).
int check_bwd_state_io(const tfla::Problem& p, const void* q, const void* k, const void* v, const float* igate_pre,
                       const float* fgate_pre, const void* dh, const void* dq, const void* dk, const void* dv,
                       const float* dig, const float* dfg, const BwdStateIO& io)
{
    for (const float* x : {io.c0, io.dc_final, (const float*)io.dc0})
        if (x && !aligned(x, 16)) return fail(TFLA_ERR_INVALID_ARG, "c0, dc_final and dc0 must be 16-byte aligned");
    const size_t esz = p.bf16 ? 2 : 4;
    const size_t bht = (size_t)p.B * p.H * p.T;
    const size_t sbytes = (size_t)p.B * p.H * p.dqk * p.dhv * 4;
    Range others[11];
    fwd_ranges(p, q, k, v, igate_pre, fgate_pre, dh, others);
    others[6] = range_of(dq, bht * p.dqk * esz);
    others[7] = range_of(dk, bht * p.dqk * esz);
    others[8] = range_of(dv, bht * p.dhv * esz);
    others[9] = range_of(dfg, gate_bytes(p));
    others[10] = dig ? range_of(dig, bht * 4) : Range{0, 0};
    const float* st[3] = {io.c0, io.dc_final, io.dc0};
    for (int i = 0; i < 3; ++i) {
        if (!st[i]) continue;
        const Range r = range_of(st[i], sbytes);
        for (const Range& o : others)
            if (overlaps(r, o)) return fail(TFLA_ERR_INVALID_ARG, "c0, dc_final or dc0 overlaps another tensor");
        for (int j = i + 1; j < 3; ++j) {
            if (!st[j] || !overlaps(r, range_of(st[j], sbytes))) continue;
            if (j == 2 && st[i] == st[j]) continue;   // dc0 in place of c0 or dc_final
            return fail(TFLA_ERR_INVALID_ARG, "c0, dc_final and dc0 overlap (dc0 may only be one of them exactly)");
        }
    }
    return TFLA_OK;
}

// tfla_bwd and tfla_bwd_state: validation, workspace, launches
int bwd_entry(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
              const void* dh, void* dq, void* dk, void* dv, float* dig, float* dfg, int B, int H, int T, int d_qk,
              int d_hv, int L, int variant, void* workspace, size_t workspace_bytes, void* stream,
              const BwdStateIO* io)
{
    tfla::Problem p;
    int rc = check_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, L, variant, &p);
    if (rc) return rc;
    const bool states = io != nullptr;
    if (states && (rc = check_bwd_state_io(p, q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, *io))) return rc;
    BwdWorkspace ws;
    const size_t need = bwd_layout(p, &ws, nullptr, states);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* base = workspace;
    const bool reuse_fwd = (variant & TFLA_BWD_REUSE_FWD) != 0;
    if (reuse_fwd && !workspace)
        return fail(TFLA_ERR_INVALID_ARG, "TFLA_BWD_REUSE_FWD needs the forward pass's workspace");
    if (reuse_fwd && states)
        return fail(TFLA_ERR_INVALID_ARG, "TFLA_BWD_REUSE_FWD is for tfla_bwd only");
    if (workspace) {
        if (!aligned(workspace, 256)) return fail(TFLA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
        if (workspace_bytes < need)
            return fail(TFLA_ERR_OUT_OF_MEMORY, "workspace of " + std::to_string(workspace_bytes) +
                                                    " bytes is smaller than the " + std::to_string(need) + " needed");
        const size_t esz = p.bf16 ? 2 : 4;
        const size_t bht = (size_t)B * H * T;
        Range tensors[14];
        fwd_ranges(p, q, k, v, igate_pre, fgate_pre, dh, tensors);   // slot 3: dh, shaped like h
        tensors[6] = range_of(dq, bht * d_qk * esz);
        tensors[7] = range_of(dk, bht * d_qk * esz);
        tensors[8] = range_of(dv, bht * d_hv * esz);
        tensors[9] = range_of(dfg, gate_bytes(p));
        tensors[10] = dig ? range_of(dig, bht * 4) : Range{0, 0};
        const size_t sbytes = (size_t)B * H * d_qk * d_hv * 4;
        tensors[11] = states && io->c0 ? range_of(io->c0, sbytes) : Range{0, 0};
        tensors[12] = states && io->dc_final ? range_of(io->dc_final, sbytes) : Range{0, 0};
        tensors[13] = states && io->dc0 ? range_of(io->dc0, sbytes) : Range{0, 0};
        if ((rc = check_workspace_disjoint(workspace, need, tensors, 14))) return rc;
    } else {
        if (inject_alloc_fault())
            return fail(TFLA_ERR_OUT_OF_MEMORY, "injected allocation failure (fault knob)");
        hipError_t e = hipMallocAsync(&base, need, s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(TFLA_ERR_OUT_OF_MEMORY, std::string("workspace allocation of ") + std::to_string(need) +
                                                    " bytes failed: " + hipGetErrorString(e));
        }
    }
    bwd_layout(p, &ws, static_cast<char*>(base), states);
    rc = run_bwd(p, q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, ws, reuse_fwd,
                 states ? *io : BwdStateIO{}, s);
    if (!workspace && base) {
        hipError_t e = hipFreeAsync(base, s);
        if (e != hipSuccess && rc == TFLA_OK) rc = hip_fail(e, "workspace free");
    }
    return rc;
}

}  // namespace

namespace tfla {

int knob(int which)
{
    if (which < 0 || which >= TFLA_KNOB_COUNT) return -1;
    return g_knobs[which].load(std::memory_order_relaxed);
}

size_t workspace_layout(const Problem& p, Workspace* ws, char* base, bool with_states, bool with_c0)
{
    const size_t bh = (size_t)p.B * p.H;
    const size_t w = p.gate == kGla ? p.dqk : 1;
    size_t off = 0;
    auto take = [&](size_t bytes) -> float* {
        float* ptr = base ? reinterpret_cast<float*>(base + off) : nullptr;
        off += align256(bytes);
        return ptr;
    };
    ws->a = p.gate == kScalar ? nullptr : take(bh * p.T * w * 4);
    ws->li = per_step_li(p.gate) ? take(bh * p.T * 4) : nullptr;
    ws->g = p.gate == kScalar ? nullptr : take(bh * p.nc * w * 4);
    ws->kw = p.gate == kGla ? take(bh * p.T * p.dqk * (p.bf16 ? 2 : 4)) : nullptr;
    if (p.gate == kExp) {
        ws->lb = take(bh * p.T * 4);
        ws->npart = take(bh * p.nc * p.dqk * 4);
        ws->nst = p.nc > 1 ? take(bh * (p.nc - 1) * p.dqk * 4) : nullptr;
        ws->mprev = take(bh * p.nc * 4);
        ws->uk = take(bh * p.nc * 4);
    }
    const size_t slots = p.nc - 1 + (with_c0 ? 1 : 0);
    ws->states = (with_states && slots > 0) ? take(bh * slots * p.dhv * p.dqk * (p.st32 ? 4 : 2)) : nullptr;
    const int P = state_segments(p);
    ws->seg_end = P > 1 ? take(bh * P * p.dhv * p.dqk * 4) : nullptr;
    ws->seg_start = P > 1 ? take(bh * P * p.dhv * p.dqk * 4) : nullptr;
    return off;
}

}  // namespace tfla

extern "C" {

size_t tfla_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant)
{
    tfla::Problem p;
    if (check_problem(B, H, T, d_qk, d_hv, L, variant, &p) != TFLA_OK) return 0;
    tfla::Workspace ws;
    return tfla::workspace_layout(p, &ws, nullptr);
}

int tfla_fwd_ws(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
                void* h, int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* workspace,
                size_t workspace_bytes, void* stream)
{
    return tfla_fwd_ws_marked(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, workspace,
                              workspace_bytes, nullptr, stream);
}

int tfla_fwd_ws_marked(const void* q, const void* k, const void* v, const float* igate_pre,
                       const float* fgate_pre, void* h, int B, int H, int T, int d_qk, int d_hv, int L,
                       int variant, void* workspace, size_t workspace_bytes, void* const* marks, void* stream)
{
    tfla::Problem p;
    int rc = check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, &p);
    if (rc) return rc;
    tfla::Workspace ws;
    const size_t need = tfla::workspace_layout(p, &ws, nullptr);
    if (need > 0 && (!workspace || !aligned(workspace, 256)))
        return fail(TFLA_ERR_INVALID_ARG, "workspace is NULL or not 256-byte aligned");
    if (workspace_bytes < need)
        return fail(TFLA_ERR_OUT_OF_MEMORY, "workspace of " + std::to_string(workspace_bytes) +
                                                " bytes is smaller than the " + std::to_string(need) + " needed");
    Range tensors[6];
    fwd_ranges(p, q, k, v, igate_pre, fgate_pre, h, tensors);
    if ((rc = check_workspace_disjoint(workspace, need, tensors, 6))) return rc;
    tfla::workspace_layout(p, &ws, static_cast<char*>(workspace));
    return run_path(p, q, k, v, igate_pre, fgate_pre, h, ws, static_cast<hipStream_t>(stream), marks);
}

int tfla_fwd(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
             void* h, int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* stream)
{
    tfla::Problem p;
    int rc = check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, &p);
    if (rc) return rc;
    tfla::Workspace ws;
    const size_t need = tfla::workspace_layout(p, &ws, nullptr);
    if (inject_alloc_fault()) return fail(TFLA_ERR_OUT_OF_MEMORY, "injected allocation failure (fault knob)");
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* base = nullptr;
    if (need > 0) {
        hipError_t e = hipMallocAsync(&base, need, s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(TFLA_ERR_OUT_OF_MEMORY, std::string("workspace allocation of ") + std::to_string(need) +
                                                    " bytes failed: " + hipGetErrorString(e));
        }
    }
    tfla::workspace_layout(p, &ws, static_cast<char*>(base));
    rc = run_path(p, q, k, v, igate_pre, fgate_pre, h, ws, s);
    if (base) {
        hipError_t e = hipFreeAsync(base, s);
        if (e != hipSuccess && rc == TFLA_OK) rc = hip_fail(e, "workspace free");
    }
    return rc;
}

int tfla_fwd_noalloc(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
                     void* h, int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* stream)
{
    tfla::Problem p;
    int rc = check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, &p);
    if (rc) return rc;
    tfla::Workspace ws;
    const size_t need = tfla::workspace_layout(p, &ws, nullptr);
    if (need > kScratchBytes)
        return fail(TFLA_ERR_OUT_OF_MEMORY, "tfla_fwd_noalloc: the problem needs " + std::to_string(need) +
                                                " bytes of workspace; its static scratch holds " +
                                                std::to_string(kScratchBytes) + " (use tfla_fwd or tfla_fwd_ws)");
    std::string err;
    void* base = scratch_on_current_device(&err);
    if (!base) return fail(TFLA_ERR_HIP, "tfla_fwd_noalloc: " + err);
    // the scratch is device memory of this library; no tensor can overlap it
    // unless a caller passed a pointer into it
    Range tensors[6];
    fwd_ranges(p, q, k, v, igate_pre, fgate_pre, h, tensors);
    if ((rc = check_workspace_disjoint(base, need, tensors, 6))) return rc;
    // every workspace byte the kernels read is written earlier in the same
    // call (gate sums, states, segment states), so nothing needs clearing
    tfla::workspace_layout(p, &ws, static_cast<char*>(base));
    return run_path(p, q, k, v, igate_pre, fgate_pre, h, ws, static_cast<hipStream_t>(stream));
}

size_t tfla_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

size_t tfla_state_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant)
{
    tfla::Problem p;
    if (check_problem(B, H, T, d_qk, d_hv, L, variant, &p) != TFLA_OK) return 0;
    if (p.gate == tfla::kExp) return 0;
    tfla::Workspace ws;
    return tfla::workspace_layout(p, &ws, nullptr, true, true);
}

int tfla_fwd_state(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
                   const float* c0, void* h, float* c_final, int B, int H, int T, int d_qk, int d_hv, int L,
                   int variant, void* workspace, size_t workspace_bytes, void* stream)
{
    tfla::Problem p;
    int rc = check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, &p);
    if (rc) return rc;
    if ((rc = check_state_io(p, q, k, v, igate_pre, fgate_pre, h, c0, c_final))) return rc;
    if (p.gate == tfla::kExp)
        return fail(TFLA_ERR_UNSUPPORTED, "mLSTMexp has no state input or output (use tfla_fwd)");
    tfla::Workspace ws;
    const bool with_c0 = c0 != nullptr;
    const size_t need = tfla::workspace_layout(p, &ws, nullptr, true, with_c0);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* base = workspace;
    if (workspace) {
        if (!aligned(workspace, 256)) return fail(TFLA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
        if (workspace_bytes < need)
            return fail(TFLA_ERR_OUT_OF_MEMORY, "workspace of " + std::to_string(workspace_bytes) +
                                                    " bytes is smaller than the " + std::to_string(need) + " needed");
        const size_t sbytes = (size_t)p.B * p.H * p.dqk * p.dhv * 4;
        Range tensors[8];
        fwd_ranges(p, q, k, v, igate_pre, fgate_pre, h, tensors);
        tensors[6] = c0 ? range_of(c0, sbytes) : Range{0, 0};
        tensors[7] = c_final ? range_of(c_final, sbytes) : Range{0, 0};
        if ((rc = check_workspace_disjoint(workspace, need, tensors, 8))) return rc;
    } else if (need > 0) {
        if (inject_alloc_fault())
            return fail(TFLA_ERR_OUT_OF_MEMORY, "injected allocation failure (fault knob)");
        hipError_t e = hipMallocAsync(&base, need, s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(TFLA_ERR_OUT_OF_MEMORY, std::string("workspace allocation of ") + std::to_string(need) +
                                                    " bytes failed: " + hipGetErrorString(e));
        }
    }
    tfla::workspace_layout(p, &ws, static_cast<char*>(base), true, with_c0);
    ws.c0 = c0;
    ws.c_final = c_final;
    rc = run_path(p, q, k, v, igate_pre, fgate_pre, h, ws, s);
    if (!workspace && base) {
        hipError_t e = hipFreeAsync(base, s);
        if (e != hipSuccess && rc == TFLA_OK) rc = hip_fail(e, "workspace free");
    }
    return rc;
}

int tfla_fwd_recurrent(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
                       float* state, void* h, int B, int H, int T, int d_qk, int d_hv, int variant, void* stream)
{
    tfla::Problem p;
    // the chunk size plays no part here; any valid one passes the shared checks
    int rc = check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, 64, variant, &p);
    if (rc) return rc;
    if (p.gate == tfla::kExp) return fail(TFLA_ERR_UNSUPPORTED, "mLSTMexp has no step-by-step form here");
    if (!state) return fail(TFLA_ERR_INVALID_ARG, "state must not be NULL");
    if ((rc = check_state_io(p, q, k, v, igate_pre, fgate_pre, h, state, nullptr))) return rc;
    hipError_t e = tfla::launch_recurrent(p, q, k, v, igate_pre, fgate_pre, state, h, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TFLA_OK : hip_fail(e, "recurrent kernel launch");
}

int tfla_dbg_gates(const float* igate_pre, const float* fgate_pre, float* a_out, float* li_out, float* g_out,
                   int B, int H, int T, int d_qk, int L, int variant, void* stream)
{
    tfla::Problem p;
    int rc = check_problem(B, H, T, d_qk, 64, L, variant, &p);
    if (rc) return rc;
    if (p.gate == tfla::kExp) return fail(TFLA_ERR_UNSUPPORTED, "tfla_dbg_gates: not for mLSTMexp");
    rc = check_gates(p, igate_pre, fgate_pre);
    if (rc) return rc;
    if (!a_out || !li_out || !g_out) return fail(TFLA_ERR_INVALID_ARG, "a_out, li_out and g_out must not be NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (p.gate == tfla::kScalar) {
        e = tfla::launch_gates_closed_form(p, fgate_pre, a_out, li_out, g_out, s);
    } else {
        tfla::Workspace ws{a_out, li_out, g_out, nullptr};
        if (p.gate == tfla::kGla) {
            e = hipMemsetAsync(li_out, 0, (size_t)B * H * T * 4, s);
            if (e != hipSuccess) return hip_fail(e, "li_out clear");
        }
        e = tfla::launch_gates(p, nullptr, igate_pre, fgate_pre, ws, s);
    }
    if (e != hipSuccess) return hip_fail(e, "gate kernel launch");
    return TFLA_OK;
}

int tfla_dbg_stream(int mode, const void* src, void* dst, size_t bytes, int loads_per_thread, int workgroups,
                    void* stream)
{
    if (mode != 0 && mode != 1) return fail(TFLA_ERR_INVALID_ARG, "tfla_dbg_stream: mode must be 0 (read) or 1 (copy)");
    if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16) || bytes % 16 != 0)
        return fail(TFLA_ERR_INVALID_ARG, "tfla_dbg_stream: 16-byte aligned buffers and a multiple of 16 bytes");
    const int l = loads_per_thread;
    if (!(l == 1 || l == 2 || l == 4 || l == 8 || l == 16) || workgroups < 1)
        return fail(TFLA_ERR_INVALID_ARG, "tfla_dbg_stream: loads_per_thread 1, 2, 4, 8 or 16; workgroups >= 1");
    const hipError_t e = tfla::launch_stream_probe(mode, src, dst, bytes, l, workgroups,
                                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TFLA_OK : hip_fail(e, "stream probe launch");
}

int tfla_dbg_mfma(int iters, int workgroups, void* sink, void* stream)
{
    if (iters < 1 || workgroups < 1 || !sink || !aligned(sink, 16))
        return fail(TFLA_ERR_INVALID_ARG, "tfla_dbg_mfma: iters >= 1, workgroups >= 1, a 16-byte aligned sink");
    const hipError_t e = tfla::launch_mfma_probe(iters, workgroups, static_cast<float*>(sink),
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TFLA_OK : hip_fail(e, "matrix-core probe launch");
}

int tfla_dbg_lds(int mode, int waves, int iters, int workgroups, void* clocks, void* sink, void* stream)
{
    if (mode < 0 || mode > 4 || (waves != 4 && waves != 8) || iters < 1 || workgroups < 1 || !clocks ||
        !aligned(clocks, 8) || !sink || !aligned(sink, 16))
        return fail(TFLA_ERR_INVALID_ARG,
                    "tfla_dbg_lds: mode 0..4, waves 4 or 8, iters >= 1, workgroups >= 1, 8-byte aligned clocks, "
                    "a 16-byte aligned sink");
    const hipError_t e = tfla::launch_lds_probe(mode, waves, iters, workgroups,
                                                static_cast<unsigned long long*>(clocks), static_cast<float*>(sink),
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TFLA_OK : hip_fail(e, "LDS probe launch");
}

int tfla_dbg_states(const void* k, const void* v, const float* igate_pre, const float* fgate_pre, void* states_out,
                    int B, int H, int T, int d_qk, int d_hv, int L, int variant, void* stream)
{
    tfla::Problem p;
    int rc = check_problem(B, H, T, d_qk, d_hv, L, variant, &p);
    if (rc) return rc;
    if (p.gate == tfla::kExp) return fail(TFLA_ERR_UNSUPPORTED, "tfla_dbg_states: not for mLSTMexp");
    rc = check_gates(p, igate_pre, fgate_pre);
    if (rc) return rc;
    if (!k || !v || !aligned(k, 16) || !aligned(v, 16))
        return fail(TFLA_ERR_INVALID_ARG, "k and v must be non-NULL and 16-byte aligned");
    if (p.nc > 1 && (!states_out || !aligned(states_out, 16)))
        return fail(TFLA_ERR_INVALID_ARG, "states_out must be non-NULL and 16-byte aligned");
    // gate sums in a private allocation; the states go straight to states_out
    tfla::Workspace ws;
    const size_t need = tfla::workspace_layout(p, &ws, nullptr, false);
    if (inject_alloc_fault()) return fail(TFLA_ERR_OUT_OF_MEMORY, "injected allocation failure (fault knob)");
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* base = nullptr;
    hipError_t e = hipSuccess;
    if (need > 0) {
        e = hipMallocAsync(&base, need, s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(TFLA_ERR_OUT_OF_MEMORY, "workspace allocation failed");
        }
    }
    tfla::workspace_layout(p, &ws, static_cast<char*>(base), false);
    ws.states = states_out;
    e = tfla::launch_gates(p, k, igate_pre, fgate_pre, ws, s);
    if (e == hipSuccess) e = tfla::launch_state(p, k, v, fgate_pre, ws, s);
    rc = e == hipSuccess ? TFLA_OK : hip_fail(e, "gate/state kernel launch");
    if (base) {
        e = hipFreeAsync(base, s);
        if (e != hipSuccess && rc == TFLA_OK) rc = hip_fail(e, "workspace free");
    }
    return rc;
}

size_t tfla_bwd_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant)
{
    tfla::Problem p;
    if (check_bwd_problem(B, H, T, d_qk, d_hv, L, variant, &p) != TFLA_OK) return 0;
    BwdWorkspace ws;
    return bwd_layout(p, &ws, nullptr);
}

int tfla_bwd(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
             const void* dh, void* dq, void* dk, void* dv, float* dig, float* dfg, int B, int H, int T, int d_qk,
             int d_hv, int L, int variant, void* workspace, size_t workspace_bytes, void* stream)
{
    return bwd_entry(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, L, variant,
                     workspace, workspace_bytes, stream, nullptr);
}

size_t tfla_bwd_state_workspace_bytes(int B, int H, int T, int d_qk, int d_hv, int L, int variant)
{
    tfla::Problem p;
    if (check_bwd_problem(B, H, T, d_qk, d_hv, L, variant, &p) != TFLA_OK) return 0;
    BwdWorkspace ws;
    return bwd_layout(p, &ws, nullptr, true);
}

int tfla_bwd_state(const void* q, const void* k, const void* v, const float* igate_pre, const float* fgate_pre,
                   const float* c0, const void* dh, const float* dc_final, void* dq, void* dk, void* dv, float* dig,
                   float* dfg, float* dc0, int B, int H, int T, int d_qk, int d_hv, int L, int variant,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    BwdStateIO io;
    io.c0 = c0;
    io.dc_final = dc_final;
    io.dc0 = dc0;
    return bwd_entry(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, L, variant,
                     workspace, workspace_bytes, stream, &io);
}

int tfla_dbg_set_knob(int which, int value)
{
    if (which < 0 || which >= TFLA_KNOB_COUNT)
        return fail(TFLA_ERR_INVALID_ARG, "unknown knob " + std::to_string(which));
    g_knobs[which].store(value < 0 ? -1 : value, std::memory_order_relaxed);
    return TFLA_OK;
}

const char* tfla_error_string(int code)
{
    switch (code) {
    case TFLA_OK: return "success";
    case TFLA_ERR_INVALID_ARG: return "invalid argument";
    case TFLA_ERR_UNSUPPORTED: return "unsupported shape or chunk size";
    case TFLA_ERR_HIP: return "HIP runtime error";
    case TFLA_ERR_OUT_OF_MEMORY: return "out of memory";
    default: return "unknown status code";
    }
}

const char* tfla_last_error(void) { return g_last_error.c_str(); }

int tfla_version(void) { return 300; }

}  // extern "C"

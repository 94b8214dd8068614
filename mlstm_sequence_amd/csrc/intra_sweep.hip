// intra_sweep.hip -- the forward pass's intra-chunk kernel for value widths
// of two or more 128-column tiles (bf16 I/O, chunks of 64, 128 or 256 steps), and
// the same computation over mirrored chunks for the dv product.
//
// Per chunk it evaluates the same sum as the per-tile kernel (intra_impl.hpp)
//   h_t = scale * ( e^{a_t} q_t^T C_{k-1} + sum_{cs <= s <= t} P_ts v_s ),
//   P_ts = e^{a_t - a_s + li_s} (q_t . k_s)       (fixed decay: f^{t-s} (q_t . k_s))
// but one workgroup owns a whole chunk of one head and every value column.
// When value tiles belong to separate workgroups, each of them reads the
// chunk's Q and K again and forms S = K Q^T again; on this chip the kernel's
// time follows the bytes its CUs pull from L2, and Q and K are most of them.
// Here:
//   1. P once: K tiles staged in LDS, S^T = K Q^T on the matrix cores with
//      the Q fragments in registers, decay and causal mask in fp32, and each
//      wave's P rows parked in LDS as matrix-core A fragments -- written and
//      read back by the lane that owns them, so no barrier guards them;
//   2. per 128-wide value tile: acc = Q C_{k-1}^T[:, tile] (C^T blocks staged
//      in LDS; rows scaled by e^{a_t}), acc += P V_tile (V tiles staged in
//      LDS, read by transpose reads), h = scale * acc out through LDS.
// Q and K cross from L2 once per chunk instead of once per value tile, and S
// is formed once.  The products, their order and every rounding are those of
// the per-tile kernel, so h is the same to the bit.  Every stage (K tile,
// C^T block, V tile) is software-pipelined across the phase boundaries: its
// global loads are issued into registers while the previous stage computes.
//
// Workgroup = NW waves (8, 4 or 2 for 256-, 128- or 64-step chunks), each owning 32
// query rows; with 8 waves the two waves of a SIMD take row blocks s and
// 7 - s, which evens out the causal work.  The per-channel gate uses the
// per-tile kernel's reference-point factorisation: for each key tile, q is
// scaled by e^{a_t - a_ref} and k by e^{a_ref - a_s} with a_ref at the
// tile's middle step, and the inter-chunk term takes q o e^{a_t}.
#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"
#include "tfla.h"

namespace tfla {
namespace {

constexpr int kSweepBV = 128;   // value tile width

template <int DQK> constexpr int sweep_cw() { return DQK >= 128 ? 128 : 64; }   // C^T channels per stage

// QI: the per-channel gate's inter-chunk Q fragments (q o e^{a_t}) are
// parked in LDS when the P phase first loads q, instead of being loaded and
// rescaled again after it (by then the chunk's q and gate rows have left L2:
// a quarter more bytes per launch); only where it fits beside the P blocks
// DB: two stage buffers, used in turn (see the kernel's stage order)
template <typename T, int DQK, int NW, bool QI, bool DB, int VS> struct SweepLds {
    static constexpr int kpad = 16 / sizeof(T);   // K / C^T rows: stride = 4 banks mod 32
    static constexpr int vpad = 64 / sizeof(T);   // V rows: stride = 16 banks mod 64 (transpose reads)
    static constexpr int CW = sweep_cw<DQK>();
    union Stage {
        T ks[64][DQK + kpad];             // K tile [step][channel]
        T vs[VS][kSweepBV + vpad];        // V tile [step][value]
        T cs[kSweepBV][CW + kpad];        // C^T block [value][channel]
        T os[NW][32][64 + kpad];          // per wave: 32 output rows x 64 columns on their way out
    };
    Stage st[DB ? 2 : 1];
    // P fragments: the wave with row block b owns the 32-key blocks m <= b
    // of its rows, two 16-key halves each, one 16-byte fragment per lane:
    // entry 2 (b(b+1)/2 + m) + half
    bf16x8 p[NW * (NW + 1)][64];
    float bcol[DB ? 2 : 1][64];           // mLSTMsig: (li_s - a_s) log2(e) per key step of the K tile
    // per wave and channel block: lane-owned Q fragments, read back by the lane that wrote them
    bf16x8 qi[QI ? NW * (DQK / 16) : 1][QI ? 64 : 1];
};

// REV: the mirrored chunks of the backward pass's dv product (logical row
// cs + r is physical step cs + len - 1 - r; the gate arrays are indexed by
// the logical row, the key-side exponent stored pre-combined in li; the
// chunk's own state is that of the chunks after it, slot kc, none for the
// last chunk unless a final-state gradient sits there)
template <typename T, int GATE, int DQK, int NW, typename S, bool REV>
__global__ __launch_bounds__(64 * NW, NW >= 8 ? 2 : 1) void intra_kernel_sweep(const T* __restrict__ q, const T* __restrict__ k,
                                                                const T* __restrict__ v,
                                                                const float* __restrict__ a,
                                                                const float* __restrict__ li,
                                                                const float* __restrict__ fg,
                                                                const S* __restrict__ states, T* __restrict__ h,
                                                                int H, int T_, int dhv, int nc, int c0, float scale,
                                                                const float* __restrict__ lbp,
                                                                const float* __restrict__ nst)
{
    constexpr int NTH = 64 * NW, BQ = 32 * NW, BV = kSweepBV, NT = BV / 32, KQ = DQK / 16;
    constexpr int CW = sweep_cw<DQK>(), NKV = BQ / 64;
    // V tiles of VS steps: 128 in the forward pass at eight waves (two V
    // stages per value tile instead of four: T = 8192 workload, L = 256,
    // intra 0.218 -> 0.215 ms), else 64 (the mirrored dv product measured
    // 3% slower with 128)
    constexpr int VS = NW == 8 && !REV ? 128 : 64, NVS = BQ / VS;
    constexpr int VEC = Elem<T>::vec, SVEC = Elem<S>::vec;
    constexpr int NK = 64 * DQK / VEC / NTH;      // K tile: 16-byte items per thread
    constexpr int NV = VS * BV / VEC / NTH;       // V tile: 16-byte items per thread
    constexpr int NC = BV * CW / 8 / NTH;         // C^T block: 8-element items per thread
    static_assert(NK >= 1 && NV >= 1 && NC >= 1, "tile too small for the workgroup");
    typedef typename Elem<T>::frag Frag;
    constexpr bool QI = GATE == kGla && NW <= 4 && std::is_same_v<T, bf16>;
    // DB (eight waves, an even number of C^T blocks): stage i is written into
    // buffer i mod 2 while the waves may still read stage i - 1 from the other,
    // so one barrier per stage (after the write) suffices.  Every stage count
    // per phase is even (K tiles, C^T blocks, V tiles), so a stage's buffer is
    // its index in its phase mod 2 and the last V tile of a value tile sits in
    // buffer 1, where the output blocks then go while the next stage is
    // written into buffer 0.  EARLY: the loads of stage i + 1 leave before that
    // barrier rather than after it (T = 8192 workload, L = 256: intra 0.228 ->
    // 0.223 ms once the inter-chunk choice was made at compile time; before,
    // it spilled registers for every gate but mLSTMexp)
    constexpr bool DB = NW == 8 && (DQK / CW) % 2 == 0;
    constexpr bool EARLY = DB;
    __shared__ SweepLds<T, DQK, NW, QI, DB, VS> sm;
    static_assert(sizeof(sm) <= 160 * 1024, "LDS");
    static_assert(!DB || (NKV % 2 == 0 && NVS % 2 == 0), "stage parity");

    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const size_t bh = blk / nc;
    // the query tile is the chunk; chunks are visited in the reverse of the
    // order the state walk wrote their states (forward: the last chunk
    // first), so the first workgroups find the states, K and V the walk
    // touched last in the last-level cache
    const int kc = REV ? blk % nc : nc - 1 - blk % nc, cs = kc * BQ;
    const int nvt = dhv / BV;
    const int clen = min(BQ, T_ - cs);            // steps in this chunk
    // physical step of logical row t (t <= T-1)
    auto row = [&](int t) { return REV ? 2 * cs + clen - 1 - t : t; };

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, hh = lane >> 5, i32 = lane & 31;
    const int wr = (NW == 8 && w >= 4) ? 11 - w : w;
    const int tlo = cs + 32 * wr;                 // first query row of this wave
    // Rows at or past T are read clamped to row T-1: a query row past the
    // end only feeds its own output row, which is never stored, and a key /
    // value row past the end only meets query rows before it through the
    // causal select (P = 0, times finite data).
    const int tqc = min(tlo + i32, T_ - 1);

    const T* qb = q + bh * (size_t)T_ * DQK;
    const T* kb = k + bh * (size_t)T_ * DQK;
    const T* vb = v + bh * (size_t)T_ * dhv;
    const float* ab = per_step_li(GATE) ? a + bh * (size_t)T_ : (GATE == kGla) ? a + bh * (size_t)T_ * DQK : nullptr;
    const float* lb = per_step_li(GATE) ? li + bh * (size_t)T_ : nullptr;
    float lg2 = 0.0f;   // log2 of the fixed decay
    if (GATE == kScalar) lg2 = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor) * kLog2e;

    // states hold C before chunks 1..nc-1, preceded by C_0 when one is given
    // (mirrored: the state of chunks kc+1.. in slot kc)
    const bool inter_rt = REV ? kc < nc - 1 + c0 : (kc > 0 || c0);
    const S* sb = inter_rt ? states + (bh * (nc - 1 + c0) + (REV ? kc : kc - 1 + c0)) * (size_t)dhv * DQK : states;

    // ---- stage loaders (global -> registers) and writers (registers -> LDS)
    Vec16<T> pk[NK], pv[NV];
    Vec16<S> pc[NC][8 / SVEC];
    float pli = 0.0f, pa = 0.0f;
    auto fetch_k = [&](int s0) {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int idx = tid + NTH * u, r = idx / (DQK / VEC), c = (idx % (DQK / VEC)) * VEC;
            pk[u].load(kb + (size_t)row(min(s0 + r, T_ - 1)) * DQK + c);
        }
        if (per_step_li(GATE) && tid < 64) {
            const int s = min(s0 + tid, T_ - 1);
            pli = lb[s];
            if (!REV) pa = ab[s];
        }
    };
    // per-channel gate: k scaled by e^{a_ref - a_s} in fp32 (factor <= 1 for
    // keys before the reference row) before its one rounding into LDS
    auto store_k = [&](int s0, int ref_row, int b) {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int idx = tid + NTH * u, r = idx / (DQK / VEC), c = (idx % (DQK / VEC)) * VEC;
            if constexpr (GATE == kGla) {
                const int s = min(s0 + r, T_ - 1);
#pragma unroll
                for (int e4 = 0; e4 < VEC / 4; ++e4) {
                    const f32x4 er = *reinterpret_cast<const f32x4*>(ab + (size_t)ref_row * DQK + c + 4 * e4);
                    const f32x4 es = *reinterpret_cast<const f32x4*>(ab + (size_t)s * DQK + c + 4 * e4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pk[u].set(4 * e4 + e, pk[u].get(4 * e4 + e) * exp2_fast((er[e] - es[e]) * kLog2e));
                }
            }
            pk[u].store(&sm.st[b].ks[r][c]);
        }
        if (per_step_li(GATE) && tid < 64) sm.bcol[b][tid] = (REV ? pli : pli - pa) * kLog2e;
    };
    auto fetch_c = [&](int v0, int cb) {
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int idx = tid + NTH * u, vr = idx / (CW / 8), c8 = (idx % (CW / 8)) * 8;
            const S* src = sb + (size_t)(v0 + vr) * DQK + cb + c8;
#pragma unroll
            for (int x = 0; x < 8 / SVEC; ++x) pc[u][x].load(src + SVEC * x);
        }
    };
    auto store_c = [&](int b) {
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int idx = tid + NTH * u, vr = idx / (CW / 8), c8 = (idx % (CW / 8)) * 8;
            if constexpr (std::is_same_v<S, T>) {
#pragma unroll
                for (int x = 0; x < 8 / VEC; ++x) pc[u][x].store(&sm.st[b].cs[vr][c8 + VEC * x]);
            } else {
                // fp32 states, bf16 operands: RNE on the way into LDS
                Vec16<T> y;
#pragma unroll
                for (int e = 0; e < 8; ++e) y.set(e, pc[u][e / SVEC].get(e % SVEC));
                y.store(&sm.st[b].cs[vr][c8]);
            }
        }
    };
    auto fetch_v = [&](int v0, int s0) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + NTH * u, r = idx / (BV / VEC), c = (idx % (BV / VEC)) * VEC;
            pv[u].load(vb + (size_t)row(min(s0 + r, T_ - 1)) * dhv + v0 + c);
        }
    };
    auto store_v = [&](int b) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + NTH * u, r = idx / (BV / VEC), c = (idx % (BV / VEC)) * VEC;
            pv[u].store(&sm.st[b].vs[r][c]);
        }
    };

    // Q fragments (lane row tqc, channels 16 kq + 8 hh ..): the B operand of
    // S^T = K Q^T and the A operand of Q C^T.  Per-channel gate: q scaled by
    // e^{a_t - a_ref} in fp32 (ref_row < 0: the chunk start, where a = 0) --
    // the reference-point factorisation of the per-tile kernel
    Frag qf[KQ];
    // park: also form q o e^{a_t} (what ref_row < 0 gives) and keep it in LDS
    auto load_q = [&](int ref_row, bool park = false) {
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
            const int c = 16 * kq + 8 * hh;
            if constexpr (GATE != kGla) {
                qf[kq] = load8(qb + (size_t)row(tqc) * DQK + c);
            } else {
                const Frag raw = load8(qb + (size_t)row(tqc) * DQK + c);
                f32x4 ex[2];
                ex[0] = *reinterpret_cast<const f32x4*>(ab + (size_t)tqc * DQK + c);
                ex[1] = *reinterpret_cast<const f32x4*>(ab + (size_t)tqc * DQK + c + 4);
                if constexpr (QI) {
                    if (park) {
                        Frag qi;
#pragma unroll
                        for (int e = 0; e < 8; ++e) frag_set(qi, e, frag_get(raw, e) * exp2_fast(ex[e >> 2][e & 3] * kLog2e));
                        sm.qi[w * KQ + kq][lane] = qi;
                    }
                }
                if (ref_row >= 0) {
                    ex[0] -= *reinterpret_cast<const f32x4*>(ab + (size_t)ref_row * DQK + c);
                    ex[1] -= *reinterpret_cast<const f32x4*>(ab + (size_t)ref_row * DQK + c + 4);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) frag_set(qf[kq], e, frag_get(raw, e) * exp2_fast(ex[e >> 2][e & 3] * kLog2e));
            }
        }
    };
    if (GATE != kGla) load_q(-1);

    // Chunks with and without an inter-chunk term run separate copies of
    // the rest: with the choice known at compile time, the loads that start
    // the next value tile go straight into the registers of their stage (a
    // run-time choice between the C^T and the V stage merged the two register
    // sets after the branch, and the copies waited for the loads at once)
    auto body = [&](auto inter_c) {
        // 0 or 1: the choice, known at compile time; 2: taken at run time
        constexpr int IM = decltype(inter_c)::value;
        const bool inter = IM == 2 ? inter_rt : IM == 1;
        // the first stage of value tile nv
        auto fetch_first = [&](int nv) {
            if constexpr (IM == 2) {
                if (inter) fetch_c(nv * BV, 0);
                else fetch_v(nv * BV, cs);
            } else if constexpr (IM == 1) {
                fetch_c(nv * BV, 0);
            } else {
                fetch_v(nv * BV, cs);
            }
        };
        bf16x8 (*const pw)[64] = &sm.p[wr * (wr + 1)];   // this wave's P blocks

        // ---------------- 1. P = decay o mask o S, once per chunk
        const float at2 = per_step_li(GATE) ? ab[tqc] * kLog2e : 0.0f;
        float rsum = 0.0f;   // mLSTMexp: this lane's part of the row sum of P (the normaliser)
        fetch_k(cs);
        for (int j = 0; j < NKV; ++j) {
            const int s0 = cs + 64 * j;
            // per-channel gate: every key tile overlaps the query tile (the
            // chunk), so its reference row is its middle step, and the Q
            // fragments are rescaled to it
            const int ref_row = (GATE == kGla) ? min(s0 + 31, T_ - 1) : -1;
            if (GATE == kGla) load_q(ref_row, QI && j == 0 && inter);
            const int b = DB ? j & 1 : 0;
            auto next = [&]() {
                if (j + 1 < NKV) fetch_k(s0 + 64);
                else fetch_first(0);
            };
            if constexpr (!DB) __syncthreads();
            store_k(s0, ref_row, b);
            if constexpr (EARLY) next();
            __syncthreads();
            if constexpr (!EARLY) next();
            // the next stage's loads leave here, before this stage's matrix
            // work: at 256 registers the compiler otherwise sinks them below it
            // (to shorten their registers' lives), and they then arrive late
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int slo = s0 + 32 * mt;
                if (slo > tlo || slo >= T_) continue;   // wholly above the diagonal, or past the end
                const bool diag = slo == tlo;
                // S^T (32 key steps x 32 query rows of this wave)
                f32x16 st;
                for (int r = 0; r < 16; ++r) st[r] = 0.0f;
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) {
                    const Frag af = load8(&sm.st[b].ks[32 * mt + i32][16 * kq + 8 * hh]);
                    st = mma32(af, qf[kq], st);
                }
                // decay and causal mask: element r is key step slo + sr, query row tlo + i32
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int sr = 8 * (r >> 2) + 4 * hh + (r & 3);
                    float p = st[r];
                    if (per_step_li(GATE)) p *= exp2_fast(at2 + sm.bcol[b][32 * mt + sr]);
                    else if (GATE == kScalar) p *= exp2_fast((float)(tlo + i32 - slo - sr) * lg2);
                    st[r] = (diag && sr > i32) ? 0.0f : p;
                }
                if constexpr (GATE == kExp) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) rsum += st[r];
                }
                // the accumulator, in its own order, is the A operand of P V
                const int m = (slo - cs) / 32;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    Frag pfr;
                    for (int e = 0; e < 8; ++e) frag_set(pfr, e, st[8 * half + e]);
                    pw[2 * m + half][lane] = pfr;
                }
            }
        }

        // per-channel gate: the inter-chunk term takes q o e^{a_t}
        if (GATE == kGla && inter) {
            if constexpr (QI) {
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) qf[kq] = sm.qi[w * KQ + kq][lane];
            } else {
                load_q(-1);
            }
        }

        // mLSTMexp: each row's factor scale / max(|scale den_t|, e^{lb_t}) with
        // den_t = sum_s P_ts + e^{a'_t} q_t . n_{k-1} (the stabilised normaliser),
        // formed in this lane (row tlo + i32) and handed to the accumulator
        // layout (row_fac) where rows run along the registers
        float fac = scale;
        if constexpr (GATE == kExp) {
            rsum += __shfl_xor(rsum, 32, 64);
            float qn = 0.0f;
            if (inter) {
                const float* nb = nst + (bh * (nc - 1) + kc - 1) * (size_t)DQK;
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) {
                    const int c = 16 * kq + 8 * hh;
                    f32x4 nv[2];
                    nv[0] = *reinterpret_cast<const f32x4*>(nb + c);
                    nv[1] = *reinterpret_cast<const f32x4*>(nb + c + 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) qn += frag_get(qf[kq], e) * nv[e >> 2][e & 3];
                }
                qn += __shfl_xor(qn, 32, 64);
            }
            const float den = rsum + exp2_fast(at2) * qn;
            fac = scale / fmaxf(fabsf(den * scale), exp2_fast(lbp[bh * (size_t)T_ + tqc] * kLog2e));
        }
        // the factor of accumulator row rr (held by lane rr in the S^T layout)
        auto row_fac = [&](int rr) { return GATE == kExp ? __shfl(fac, rr, 64) : scale; };

        // ---------------- 2. every value tile
        T* const hbase = h + bh * (size_t)T_ * dhv;
        for (int nv = 0; nv < nvt; ++nv) {
            const int v0 = nv * BV;
            f32x16 acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;
            if (inter) {
                // e^{a_t} q_t^T C_{k-1}
                for (int cb = 0; cb < DQK; cb += CW) {
                    const int b = DB ? (cb / CW) & 1 : 0;
                    auto next = [&]() {
                        if (cb + CW < DQK) fetch_c(v0, cb + CW);
                        else fetch_v(v0, cs);
                    };
                    if constexpr (!DB) __syncthreads();
                    store_c(b);
                    if constexpr (EARLY) next();
                    __syncthreads();
                    if constexpr (!EARLY) next();
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int kk = 0; kk < CW / 16; ++kk) {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            const Frag bf = load8(&sm.st[b].cs[32 * nt + i32][16 * kk + 8 * hh]);
                            acc[nt] = mma32(qf[cb / 16 + kk], bf, acc[nt]);
                        }
                    }
                }
                if (GATE != kGla) {   // per-channel gate: e^{a_t} already inside q
                    // a_t of accumulator row rr comes from lane rr, which holds
                    // it for its own row (at2), not from a load of its own: a
                    // load here would wait behind the V tile's loads in flight
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
                        const int t = min(tlo + rr, T_ - 1);
                        const float e = per_step_li(GATE) ? exp2_fast(__shfl(at2, rr, 64))
                                                       : exp2_fast((float)(t - cs + (REV ? 0 : 1)) * lg2);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= e;
                    }
                }
            }
            // + P V, key tile by key tile
            for (int j = 0; j < NVS; ++j) {
                const int s0 = cs + VS * j;
                const int b = DB ? j & 1 : 0;
                auto next = [&]() {
                    if (j + 1 < NVS) fetch_v(v0, s0 + VS);
                    else if (nv + 1 < nvt) fetch_first(nv + 1);
                };
                if constexpr (!DB) __syncthreads();
                store_v(b);
                if constexpr (EARLY) next();
                __syncthreads();
                if constexpr (!EARLY) next();
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mt = 0; mt < VS / 32; ++mt) {
                    const int slo = s0 + 32 * mt;
                    if (slo > tlo || slo >= T_) continue;   // the blocks step 1 skipped
                    const int m = (slo - cs) / 32;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const Frag pfr = pw[2 * m + half][lane];
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            const Frag vf = frag_tr(sm.st[b].vs, 32 * mt + 16 * half, 32 * nt, lane);
                            acc[nt] = mma32(pfr, vf, acc[nt]);
                        }
                    }
                }
            }
            // out through LDS, 64 columns at a time: the wave writes its
            // accumulators (lane = column) into its own 32 x 64 block, then every
            // lane stores 16-byte runs of rows
            __syncthreads();   // every wave is done with the V tile the blocks overlay
            T* const hrow = hbase + v0;
#pragma unroll
            for (int ph = 0; ph < NT / 2; ++ph) {
                auto os = sm.st[DB ? (NVS - 1) & 1 : 0].os[w];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
                    const float fr = row_fac(rr);
                    os[rr][i32] = from_float<T>(acc[2 * ph][r] * fr);
                    os[rr][32 + i32] = from_float<T>(acc[2 * ph + 1][r] * fr);
                }
                __syncthreads();
#pragma unroll
                for (int qq = 0; qq < 32 / VEC; ++qq) {
                    const int c = lane + 64 * qq;                 // 16-byte piece of the 32 x 64 block
                    const int rr = c / (64 / VEC), col = (c % (64 / VEC)) * VEC;
                    const int t = tlo + rr;
                    if (t < T_) {
                        Vec16<T> x;
                        x.load(&os[rr][col]);
                        x.store_nt(hrow + (size_t)row(t) * dhv + 64 * ph + col);   // (the library does not read h)
                    }
                }
                // this block is read before it is overwritten (the next half, or
                // the next value tile's first stage after its own barrier; with
                // two buffers that stage goes to the other one, and the stage
                // after it waits for the first one's barrier)
                if (ph + 1 < NT / 2) __syncthreads();
            }
        }
    };
    if constexpr (GATE == kGla) {
        body(std::integral_constant<int, 2>{});   // (two copies of the per-channel gate's body spill)
    } else {
        if (inter_rt) body(std::integral_constant<int, 1>{});
        else body(std::integral_constant<int, 0>{});
    }
}

template <typename S, int GATE, int DQK, int NW, bool REV>
hipError_t launch_sweep_t(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                          const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    const long blocks = (long)p.B * p.H * p.nc;
    intra_kernel_sweep<bf16, GATE, DQK, NW, S, REV><<<(unsigned)blocks, 64 * NW, 0, stream>>>(
        static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), ws.a, ws.li, fg,
        static_cast<const S*>(ws.states), static_cast<bf16*>(h), p.H, p.T, p.dhv, p.nc, ws.c0 != nullptr, scale,
        ws.lb, ws.nst);
    return hipGetLastError();
}

// one wave per 32 steps of the chunk: 8 waves at L = 256, 4 at 128, 2 at 64
// (fewer than 8 at one wave per SIMD: their larger per-thread prefetch needs
// the registers)
template <typename S, int GATE, int DQK, bool REV>
hipError_t sweep_nw(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                    const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    if (p.L == 64) return launch_sweep_t<S, GATE, DQK, 2, REV>(p, q, k, v, fg, ws, h, scale, stream);
    // (the per-channel gate's per-tile Q rescaling does not fit 4 or 8 waves at d_qk = 256)
    if constexpr (GATE != kGla || DQK <= 128) {
        if (p.L == 128) return launch_sweep_t<S, GATE, DQK, 4, REV>(p, q, k, v, fg, ws, h, scale, stream);
        return launch_sweep_t<S, GATE, DQK, 8, REV>(p, q, k, v, fg, ws, h, scale, stream);
    }
    return hipErrorInvalidValue;
}

template <typename S, int GATE, bool REV>
hipError_t sweep_dqk(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                     const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    switch (p.dqk) {
    case 64: return sweep_nw<S, GATE, 64, REV>(p, q, k, v, fg, ws, h, scale, stream);
    case 128: return sweep_nw<S, GATE, 128, REV>(p, q, k, v, fg, ws, h, scale, stream);
    case 256: return sweep_nw<S, GATE, 256, REV>(p, q, k, v, fg, ws, h, scale, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename S, bool REV>
hipError_t sweep_gate(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                      const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    if (p.gate == kSig) return sweep_dqk<S, kSig, REV>(p, q, k, v, fg, ws, h, scale, stream);
    if (p.gate == kScalar) return sweep_dqk<S, kScalar, REV>(p, q, k, v, fg, ws, h, scale, stream);
    if (p.gate == kExp) {
        if constexpr (!REV) return sweep_dqk<S, kExp, REV>(p, q, k, v, fg, ws, h, scale, stream);
        return hipErrorInvalidValue;
    }
    return sweep_dqk<S, kGla, REV>(p, q, k, v, fg, ws, h, scale, stream);
}

}  // namespace

// Applies to bf16 I/O, chunks of 64, 128 or 256 steps (one wave per 32
// steps), a contraction of 64..256 channels and two or more 128-wide value
// tiles; every gate (the per-channel gate at L >= 128 only up to d_qk = 128:
// its Q fragments, rescaled per key tile, spill at 4 or 8 waves and d_qk =
// 256), in the forward pass and in the dv product.
// The intra-sweep knob set to 0 turns it off (the per-tile kernel then runs;
// tests of bitwise agreement and tuning comparisons).
bool intra_sweeps(const Problem& p)
{
    if (knob(TFLA_KNOB_INTRA_SWEEP) == 0) return false;
    return p.bf16 && (p.L == 64 || p.L == 128 || p.L == 256) && (p.dqk == 64 || p.dqk == 128 || p.dqk == 256) &&
           p.dhv % kSweepBV == 0 && p.dhv / kSweepBV >= 2 && !(p.gate == kGla && p.L >= 128 && p.dqk == 256);
}

bool intra_sweeps_dv(const Problem& p) { return intra_sweeps(p); }

hipError_t launch_intra_sweep(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                              const Workspace& ws, void* h, hipStream_t stream)
{
    if (!intra_sweeps(p)) return hipErrorInvalidValue;
    const float scale = 1.0f / sqrtf((float)p.dqk);
    if (p.st32) return sweep_gate<float, false>(p, q, k, v, fgate_pre, ws, h, scale, stream);
    return sweep_gate<bf16, false>(p, q, k, v, fgate_pre, ws, h, scale, stream);
}

hipError_t launch_intra_sweep_dv(const Problem& p, const void* q, const void* k, const void* v,
                                 const float* fgate_pre, const Workspace& ws, void* out, float scale,
                                 hipStream_t stream)
{
    if (!intra_sweeps_dv(p) || p.st32) return hipErrorInvalidValue;
    return sweep_gate<bf16, true>(p, q, k, v, fgate_pre, ws, out, scale, stream);
}

}  // namespace tfla

// intra_impl.hpp -- intra-chunk kernel (third kernel of the path) and its
// dispatch; instantiated by intra.hip (forward) and intra_bwd_*.hip (the
// gradient modes), one translation unit each so they build in parallel.
//
// For step t of chunk k (steps [cs, cs+L)):
//   h_t = scale * ( e^{a_t} q_t^T C_{k-1}           (C_{-1}: the initial state, or 0)
//                   + sum_{cs <= s <= t} e^{a_t - a_s + li_s} (q_t . k_s) v_s )
// (GLA gate: the decay enters per key channel inside q.k, and the inter term
// is (q_t o e^{a_t}) C_{k-1}).  TFLA's second level of sequence parallelism
// (TFLA abstract; research-map summary, Approach) tiles this along the
// sequence: a workgroup owns BQ query steps x BV value columns of one chunk
// and loops over the 64-step key/value tiles up to its own rows, so the
// chunk size L is bounded by nothing on chip.
//
// Workgroup = NW wavefronts (2, 4 or 8), each owning 32 query rows (BQ =
// 32 NW, at most the chunk size; with 8 waves the two waves of a SIMD take
// row blocks s and 7 - s, which evens out the causal work);
// all products are 32x32x16 matrix-core tiles:
//   inter: acc = Q C_{k-1}[:, v-tile]; C^T is staged in LDS per CW-channel
//          block (stored in the operand type by the state walk; fp32 states
//          are rounded RNE on the way in); Q fragments stay in registers
//          (A operand here, B operand of S^T below); rows scaled by e^{a_t}.
//   intra: per key tile j: K_j and V_j staged row-major in LDS; per 32-step
//          half: S^T = K Q^T, decay and causal mask in fp32 (a select, never
//          a multiply by 0), and the S^T accumulators reused in place as the A
//          operand of acc += P V_j -- the step index is contracted in the
//          order the accumulator holds it, and V_j is read in that order with
//          LDS transpose reads.  Halves entirely above the diagonal are
//          skipped per wave.
//   out:   h = acc * scale, rounded to the I/O type, through LDS (each wave
//          stages 32 rows x 64 columns, then stores 16-byte runs of rows).
// Every stage (a block of C^T, a K/V tile) is software-pipelined: its global
// loads are issued into registers right after the previous stage reached
// LDS, with consecutive lanes on consecutive 16-byte pieces of a row.
// Per-channel gates use a reference-point factorisation: tiles wholly before
// the query tile scale q by e^{a_t - a_ref} and k by e^{a_ref - a_s} with
// a_ref at the step before the query tile (both factors <= 1); tiles that
// overlap it use the tile's middle step.
//
// The same kernel evaluates the three gradient products of the backward pass
// (the intra-chunk structure is shared; see tfla_bwd) through MODE bits:
//   kNatState: the state block is stored contraction-major ([d_c][d_out],
//              the natural layout of a state whose rows are contracted);
//              it is staged as stored and read through transpose reads.
//   kMirror:   the rows of every chunk are visited in reverse order (logical
//              row cs + r is physical step cs + len - 1 - r), which turns the
//              anti-causal sums of the backward pass into causal ones; the
//              chunk's own state is that of the chunks after it (slot kc,
//              none for the last chunk), and the gate arrays are indexed by
//              the logical row (a' = g - a + li for the query rows, and the
//              key-side exponent li_s - a'_s = a_s - g stored pre-combined).
//   kRowDots:  also the fp32 row dot products of the output with a partner
//              tensor (per-step gates), or the per-element products (the
//              per-channel gate), for the gate gradients.
//   kEmitP / kGivenP: P (the decayed, masked S of a chunk, per-step gates)
//              written once, or read instead of computed (dq reads it by
//              rows, dk transposed in mirrored order).
//   kStateF32: the forward pass reading fp32 states with bf16 I/O.
#pragma once

#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"
#include "tfla.h"

namespace tfla {
namespace {

// NATL: the state block is staged as stored, contraction-major (cst), and
// read through transpose reads; NW waves stage their outputs in os
template <typename T, int DQK, int BV, int CW, bool NATL, int NW> struct IntraLds {
    static constexpr int kpad = 16 / sizeof(T);   // K / C^T rows: stride = 4 banks mod 32
    static constexpr int vpad = 64 / sizeof(T);   // V rows: stride = 16 banks mod 64 (transpose reads)
    union {
        struct {
            T ks[64][DQK + kpad];   // K tile [step][channel]
            T vs[64][BV + vpad];    // V tile [step][value]
        } kv;
        T cs[NATL ? 1 : BV][CW + kpad];    // CW-channel block of C^T [value][channel]
        T cst[NATL ? CW : 1][BV + vpad];   // the same block as [channel][value], rows permuted (see store_c)
        T os[NW][32][64 + kpad];           // per wave: 32 output rows x 64 columns on their way out
    };
    float bcol[64];                 // mLSTMsig: (li_s - a_s) log2(e) per key step
};

// One stage's global loads, held in registers while the previous stage
// computes.  A C^T block and a K/V tile are never in flight together, so they
// share the registers.
// S: the stored state type
template <typename T, typename S, int DQK, int BV, int CW, int NTH> struct Prefetch {
    typedef typename Elem<T>::frag Frag;
    static constexpr int VEC = Elem<T>::vec;
    static constexpr int SVEC = Elem<S>::vec;
    static constexpr int NC = BV * CW / 8 / NTH;          // C^T block: 8 elements per item
    static constexpr int NK = 64 * DQK / VEC / NTH;       // K tile: 16 bytes per item
    static constexpr int NV = 64 * BV / VEC / NTH;        // V tile: 16 bytes per item
    static_assert(NC >= 1 && NK >= 1 && NV >= 1, "tile too small for the workgroup");
    union {
        Vec16<S> c[NC][8 / SVEC];
        struct {
            Vec16<T> k[NK];
            Vec16<T> v[NV];
            Frag p[2][2];   // given-P mode: this wave's P fragments of the tile
        } kv;
    };
    float li, a;
};

// 8 consecutive fp32 gate values (16-byte aligned) as two vector loads
__device__ __forceinline__ void load_gates8(const float* p, f32x4 (&x)[2])
{
    x[0] = *reinterpret_cast<const f32x4*>(p);
    x[1] = *reinterpret_cast<const f32x4*>(p + 4);
}

template <typename T, int GATE, int DQK, int BV, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, NW >= 4 && DQK <= 256 ? 2 : 1) void intra_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const float* __restrict__ a,
                                                           const float* __restrict__ li,
                                                           const float* __restrict__ fg,
                                                           const std::conditional_t<(MODE & kStateF32) != 0, float, T>* __restrict__ states,
                                                           T* __restrict__ h, int H, int T_, int dhv, int L,
                                                           int nc, int c0, float scale,
                                                           const T* __restrict__ partner,
                                                           float* __restrict__ dots, T* __restrict__ pout,
                                                           const T* __restrict__ pin,
                                                           const float* __restrict__ lbp,
                                                           const float* __restrict__ nst)
{
    constexpr bool NAT = (MODE & kNatState) != 0, REV = (MODE & kMirror) != 0, DOTS = (MODE & kRowDots) != 0;
    // forward (h): a scheduling barrier after each stage's fetch keeps its
    // loads ahead of the stage's matrix work, where the compiler would sink
    // them (T = 4096 fixed-decay workload: 0.305 -> 0.295 ms); the gradient
    // modes measured slower with it and leave the order to the compiler
    constexpr bool PIN = (MODE & ~kStateF32) == 0;
    // per-channel gate: decay inside the contraction (forward, dv), or on the
    // output columns (dq, dk: the contracted index is the value channel)
    constexpr bool OUTDECAY = GATE == kGla && NAT, INDECAY = GATE == kGla && !NAT;
    // P = the decayed, masked S of a chunk ([B*H][T][L], row = query step,
    // column = key step - chunk start): written (EMITP) or read (GIVENP;
    // mirrored: read transposed, row = the key's step, column = the query's)
    // instead of computed; per-step gates only
    constexpr bool EMITP = (MODE & kEmitP) != 0, GIVENP = (MODE & kGivenP) != 0;
    static_assert(!(EMITP || GIVENP) || GATE != kGla, "shared P covers the per-step gates only");
    constexpr int NTH = 64 * NW;
    constexpr int BQ = 32 * NW;           // query rows per workgroup
    // C^T channels per stage: 128 (two stages at d_qk = 256) when the
    // registers allow, 64 for fp32 at four or more waves; two-wave
    // workgroups and the 512-wide contraction at four waves hold a larger
    // K/V prefetch, which 128- (256-) channel blocks of bf16 states fit inside
    constexpr int CW = NW >= 4 ? ((sizeof(T) == 2 && DQK >= 128) ? (NW == 4 && DQK == 512 ? 256 : 128) : 64)
                               : (DQK >= 128 ? 128 : 64);
    constexpr int KQ = DQK / 16;          // 16-channel contraction steps
    constexpr int NT = BV / 32;           // 32-wide output column tiles
    constexpr int VEC = Elem<T>::vec;
    typedef typename Elem<T>::frag Frag;
    typedef IntraLds<T, DQK, BV, CW, NAT, NW> Lds;
    typedef std::conditional_t<(MODE & kStateF32) != 0, float, T> S;   // stored state type
    constexpr int SVEC = Elem<S>::vec;
    typedef Prefetch<T, S, DQK, BV, CW, NTH> PF;
    __shared__ Lds sm;

    const int nqt = (T_ + BQ - 1) / BQ;
    const int nvt = dhv / BV;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const size_t bh = blk / (nqt * nvt);
    const int rem = blk % (nqt * nvt);
    const int qt = rem / nvt;
    const int v0 = (rem % nvt) * BV;
    const int t0 = qt * BQ;
    const int kc = t0 / L, cs = kc * L;
    const int clen = min(L, T_ - cs);      // steps in this chunk
    // physical step of logical row t (t <= T-1)
    auto row = [&](int t) { return REV ? 2 * cs + clen - 1 - t : t; };

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, hh = lane >> 5, i32 = lane & 31;
    // this wave's 32-row block: with 8 waves, waves w and w + 4 share a SIMD,
    // and block b meets b + 1 causal key halves, so the pairs take blocks
    // {s, 7 - s} (9 halves per SIMD instead of 6..12)
    const int wr = (NW == 8 && w >= 4) ? 11 - w : w;
    const int tq = t0 + 32 * wr + i32;     // query step of this lane's fragment row
    // Rows at or past T are read clamped to row T-1 (branch-free loads): a
    // query row past the end only feeds its own output row, which is never
    // stored, and a key/value row past the end only meets query rows before
    // it through the causal select (P = 0, times finite data).
    const int tqc = min(tq, T_ - 1);

    const T* qb = q + bh * (size_t)T_ * DQK;
    const T* kb = k + bh * (size_t)T_ * DQK;
    const T* vb = v + bh * (size_t)T_ * dhv;
    const int gw = OUTDECAY ? dhv : DQK;   // per-channel gate row width
    const float* ab = (GATE == kGla) ? a + bh * (size_t)T_ * gw : a + bh * (size_t)T_;
    const float* lb = per_step_li(GATE) ? li + bh * (size_t)T_ : nullptr;
    const float at2 = per_step_li(GATE) ? ab[tqc] * kLog2e : 0.0f;   // a of this lane's row, log2 units
    float lg2 = 0.0f;   // log2 of the fixed decay
    if (GATE == kScalar) lg2 = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor) * kLog2e;

    PF pf;

    // Q fragments (lane row tq, channels 16 kq + 8 hh ..); per-channel gate:
    // q * e^{a_t - a_ref} (ref_row < 0: the chunk start, where a = 0)
    Frag qf[KQ];
    auto load_q = [&](int ref_row) {
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
            const int c = 16 * kq + 8 * hh;
            if (!INDECAY) {
                qf[kq] = load8(qb + (size_t)row(tqc) * DQK + c);
            } else {
                const Frag raw = load8(qb + (size_t)row(tqc) * DQK + c);
                // 8 consecutive channels of the gate row: two 16-byte loads
                f32x4 ex[2];
                load_gates8(ab + (size_t)tqc * DQK + c, ex);
                if (ref_row >= 0) {
                    f32x4 er[2];
                    load_gates8(ab + (size_t)ref_row * DQK + c, er);
                    ex[0] -= er[0];
                    ex[1] -= er[1];
                }
                for (int e = 0; e < 8; ++e)
                    frag_set(qf[kq], e, frag_get(raw, e) * exp2_fast(ex[e >> 2][e & 3] * kLog2e));
            }
        }
    };

    // ---- stage loaders (global -> registers) and writers (registers -> LDS)
    auto fetch_c = [&](const S* st, int cb) {
#pragma unroll
        for (int u = 0; u < PF::NC; ++u) {
            const int idx = tid + NTH * u;
            if constexpr (NAT) {
                // 8 consecutive output columns of contraction row c: the lanes
                // read each row's run of columns with 16-byte loads
                const int c = idx / (BV / 8), col8 = (idx % (BV / 8)) * 8;
                const S* src = st + (size_t)(cb + c) * dhv + col8;
#pragma unroll
                for (int x = 0; x < 8 / SVEC; ++x) pf.c[u][x].load(src + SVEC * x);
            } else {
                const int vr = idx / (CW / 8), c8 = (idx % (CW / 8)) * 8;
                const S* src = st + (size_t)vr * DQK + cb + c8;
#pragma unroll
                for (int x = 0; x < 8 / SVEC; ++x) pf.c[u][x].load(src + SVEC * x);
            }
        }
    };
    auto store_c = [&]() {
#pragma unroll
        for (int u = 0; u < PF::NC; ++u) {
            const int idx = tid + NTH * u;
            if constexpr (NAT) {
                // Transpose reads hand lane half hh the contraction rows
                // 4hh..4hh+3 and 8+4hh..8+4hh+3 of each 16-row group, where
                // the Q fragments hold channels 8hh..8hh+7 in order: storing
                // contraction row c at row c with bits 2 and 3 swapped makes
                // the two agree.
                const int c = idx / (BV / 8), col8 = (idx % (BV / 8)) * 8;
                const int r = (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1);
                static_assert(std::is_same_v<S, T>, "gradient modes store states in the I/O type");
#pragma unroll
                for (int x = 0; x < 8 / VEC; ++x) pf.c[u][x].store(&sm.cst[r][col8 + VEC * x]);
                continue;
            }
            const int vr = idx / (CW / 8);
            const int c8 = (idx % (CW / 8)) * 8;
            if constexpr (std::is_same_v<S, T>) {
#pragma unroll
                for (int x = 0; x < 8 / VEC; ++x) pf.c[u][x].store(&sm.cs[vr][c8 + VEC * x]);
            } else {
                // fp32 states, bf16 operands: RNE on the way into LDS
                Vec16<T> y;
#pragma unroll
                for (int e = 0; e < 8; ++e) y.set(e, pf.c[u][e / SVEC].get(e % SVEC));
                y.store(&sm.cs[vr][c8]);
            }
        }
    };
    auto fetch_kv = [&](int s0) {
        if constexpr (!GIVENP) {
#pragma unroll
            for (int u = 0; u < PF::NK; ++u) {
                const int idx = tid + NTH * u, r = idx / (DQK / VEC), c = (idx % (DQK / VEC)) * VEC;
                const int s = row(min(s0 + r, T_ - 1));
                pf.kv.k[u].load(kb + (size_t)s * DQK + c);
            }
        }
        if constexpr (!EMITP) {
#pragma unroll
            for (int u = 0; u < PF::NV; ++u) {
                const int idx = tid + NTH * u, r = idx / (BV / VEC), c = (idx % (BV / VEC)) * VEC;
                const int s = row(min(s0 + r, T_ - 1));
                pf.kv.v[u].load(vb + (size_t)s * dhv + v0 + c);
            }
        }
        if constexpr (GIVENP && !REV) {
            // this lane's P row, keys in the order the accumulator holds them
            const T* pr = pin + (bh * (size_t)T_ + tqc) * L + (s0 - cs) + 4 * hh;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    pf.kv.p[mt][half] = load4x2(pr + 32 * mt + 16 * half, pr + 32 * mt + 16 * half + 8);
        } else if constexpr (GIVENP) {
            // mirrored: element (logical row r, logical key c) is P[row(c)][row(r) - cs];
            // for one element index all lanes of a half read one P row
            const T* pc = pin + bh * (size_t)T_ * L + (row(tqc) - cs);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int c = min(s0 + 32 * mt + 16 * half + 8 * (e >> 2) + 4 * hh + (e & 3), T_ - 1);
                        frag_set(pf.kv.p[mt][half], e, to_float(pc[(size_t)row(c) * L]));
                    }
        }
        if (per_step_li(GATE) && !GIVENP && tid < 64) {
            const int s = min(s0 + tid, T_ - 1);
            pf.li = lb[s];
            if (!REV) pf.a = ab[s];
        }
    };
    auto store_kv = [&](int s0, int ref_row) {
#pragma unroll
        for (int u = 0; u < (GIVENP ? 0 : PF::NK); ++u) {
            const int idx = tid + NTH * u, r = idx / (DQK / VEC), c = (idx % (DQK / VEC)) * VEC;
            if (INDECAY) {
                const int s = min(s0 + r, T_ - 1);
                f32x4 er[VEC / 4], es[VEC / 4];
                for (int e4 = 0; e4 < VEC / 4; ++e4) {
                    er[e4] = *reinterpret_cast<const f32x4*>(ab + (size_t)ref_row * DQK + c + 4 * e4);
                    es[e4] = *reinterpret_cast<const f32x4*>(ab + (size_t)s * DQK + c + 4 * e4);
                }
                for (int e = 0; e < VEC; ++e)
                    pf.kv.k[u].set(e, pf.kv.k[u].get(e) * exp2_fast((er[e >> 2][e & 3] - es[e >> 2][e & 3]) * kLog2e));
            }
            pf.kv.k[u].store(&sm.kv.ks[r][c]);
        }
#pragma unroll
        for (int u = 0; u < (EMITP ? 0 : PF::NV); ++u) {
            const int idx = tid + NTH * u, r = idx / (BV / VEC), c = (idx % (BV / VEC)) * VEC;
            if (OUTDECAY) {
                // output-side decay: value row s scaled by e^{a_R - a_s} per
                // column, R the last step of its 32-step half (factor <= 1)
                const int s = min(s0 + r, T_ - 1);
                const int R = min(s0 + 32 * (r >> 5) + 31, T_ - 1);
                f32x4 er[VEC / 4], es[VEC / 4];
                for (int e4 = 0; e4 < VEC / 4; ++e4) {
                    er[e4] = *reinterpret_cast<const f32x4*>(ab + (size_t)R * gw + v0 + c + 4 * e4);
                    es[e4] = *reinterpret_cast<const f32x4*>(ab + (size_t)s * gw + v0 + c + 4 * e4);
                }
                for (int e = 0; e < VEC; ++e)
                    pf.kv.v[u].set(e, pf.kv.v[u].get(e) * exp2_fast((er[e >> 2][e & 3] - es[e >> 2][e & 3]) * kLog2e));
            }
            pf.kv.v[u].store(&sm.kv.vs[r][c]);
        }
        if (per_step_li(GATE) && !GIVENP && tid < 64) sm.bcol[tid] = (REV ? pf.li : pf.li - pf.a) * kLog2e;
    };

    f32x16 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;

    // ---------------- inter-chunk term: e^{a_t} q_t^T C_{k-1}
    // states hold C before chunks 1..nc-1, preceded by C_0 when one is given
    // (c0 = 1); mirrored: the state of chunks kc+1.. in slot kc, the last
    // chunk's (a final-state gradient) in slot nc-1 when one is given (c0 = 1)
    const bool inter = EMITP ? false : REV ? kc < nc - 1 + c0 : (kc > 0 || c0);
    if (inter) {
        const size_t slot = bh * (nc - 1 + c0) + (REV ? kc : kc - 1 + c0);
        const S* st = NAT ? states + slot * DQK * (size_t)dhv + v0
                          : states + (slot * dhv + v0) * DQK;
        fetch_c(st, 0);
        load_q(-1);
        for (int cb = 0; cb < DQK; cb += CW) {
            __syncthreads();
            store_c();
            __syncthreads();
            // the next stage's loads fly while this block is multiplied
            if (cb + CW < DQK) fetch_c(st, cb + CW);
            else fetch_kv(cs);
            if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < CW / 16; ++kk) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    Frag bf;
                    if constexpr (NAT) bf = frag_tr(sm.cst, 16 * kk, 32 * nt, lane);
                    else bf = load8(&sm.cs[32 * nt + i32][16 * kk + 8 * hh]);
                    acc[nt] = mma32(qf[cb / 16 + kk], bf, acc[nt]);
                }
            }
        }
        if (GATE != kGla) {
            // a_t of accumulator row rr from lane rr (its own row's at2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
                const int t = min(t0 + 32 * wr + rr, T_ - 1);
                const float e = per_step_li(GATE) ? exp2_fast(__shfl(at2, rr, 64))
                                                  : exp2_fast((float)(t - cs + (REV ? 0 : 1)) * lg2);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= e;
            }
        }
    } else {
        fetch_kv(cs);
    }

    // ---------------- intra-chunk term, tiled along the chunk
    if (!INDECAY && !GIVENP && !inter) load_q(-1);
    // output-side decay: acc holds its partial sums in the frame of step
    // fref (true value = acc e^{a_t - a_fref}; fref < 0: the chunk start,
    // a = 0); the frame moves forward half by half, each move a factor <= 1
    int fref = -1;
    auto move_frame = [&](int R) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = v0 + 32 * nt + i32;
            float ex = ab[(size_t)R * gw + col];
            if (fref >= 0) ex -= ab[(size_t)fref * gw + col];
            const float e = exp2_fast(ex * kLog2e);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nt][r] *= e;
        }
        fref = R;
    };
    float rsum = 0.0f;   // mLSTMexp: this lane's part of the row sum of P (the normaliser)
    const int tlo = t0 + 32 * wr;                  // first query row of this wave
    const int nkv = (t0 - cs) / 64 + BQ / 64;     // key tiles up to the end of the query tile
    int q_ref = -2;                               // reference row the Q fragments are scaled for

    for (int j = 0; j < nkv; ++j) {
        const int s0 = cs + 64 * j;
        int ref_row = -1;
        if (INDECAY) {
            ref_row = (s0 + 63 < t0) ? t0 - 1 : min(s0 + 31, T_ - 1);
            if (ref_row != q_ref) {
                load_q(ref_row);
                q_ref = ref_row;
            }
        }
        __syncthreads();
        store_kv(s0, ref_row);
        Frag pcur[2][2];   // given P: this tile's fragments, before the next fetch reuses pf
        if constexpr (GIVENP) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                for (int half = 0; half < 2; ++half) pcur[mt][half] = pf.kv.p[mt][half];
        }
        __syncthreads();
        if (j + 1 < nkv) fetch_kv(s0 + 64);
        if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int slo = s0 + 32 * mt;
            if (slo > tlo + 31 || slo >= T_) continue;   // wholly above the diagonal, or past the end
            const bool diag = slo == tlo;
            if (OUTDECAY) move_frame(min(slo + 31, T_ - 1));
            if constexpr (GIVENP) {
                // P from memory; pairs above the diagonal or past the end may
                // hold anything there and are selected to zero
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    Frag pfr = pcur[mt][half];
                    if (diag || slo + 31 >= T_) {
                        for (int e = 0; e < 8; ++e) {
                            const int key = slo + 16 * half + 8 * (e >> 2) + 4 * hh + (e & 3);
                            if (key > tlo + i32 || key >= T_) frag_set(pfr, e, 0.0f);
                        }
                    }
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const Frag vf = frag_tr(sm.kv.vs, 32 * mt + 16 * half, 32 * nt, lane);
                        acc[nt] = mma32(pfr, vf, acc[nt]);
                    }
                }
                continue;
            }
            // S^T (32 key steps x 32 query rows of this wave)
            f32x16 st;
            for (int r = 0; r < 16; ++r) st[r] = 0.0f;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                const Frag af = load8(&sm.kv.ks[32 * mt + i32][16 * kq + 8 * hh]);
                st = mma32(af, qf[kq], st);
            }
            // decay and causal mask: element r is key step slo + sr, query row tlo + i32
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int sr = 8 * (r >> 2) + 4 * hh + (r & 3);
                float p = st[r];
                if (per_step_li(GATE)) {
                    p *= exp2_fast(at2 + sm.bcol[32 * mt + sr]);
                } else if (GATE == kScalar) {
                    p *= exp2_fast((float)(tlo + i32 - slo - sr) * lg2);
                }
                st[r] = (diag && sr > i32) ? 0.0f : p;
            }
            if constexpr (GATE == kExp) {
#pragma unroll
                for (int r = 0; r < 16; ++r) rsum += st[r];
            }
            if constexpr (EMITP) {
                // P row t (this lane), keys slo + sr: four runs of 4 consecutive keys
                const int t = tlo + i32;
                if (t < T_) {
                    T* prow = pout + (bh * (size_t)T_ + t) * L + (slo - cs) + 4 * hh;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        store4(prow + 8 * g4, st[4 * g4], st[4 * g4 + 1], st[4 * g4 + 2], st[4 * g4 + 3]);
                }
                continue;
            }
            // acc += P V: 16-step halves, in accumulator order
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Frag pfr;
                for (int e = 0; e < 8; ++e) frag_set(pfr, e, st[8 * half + e]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const Frag vf = frag_tr(sm.kv.vs, 32 * mt + 16 * half, 32 * nt, lane);
                    acc[nt] = mma32(pfr, vf, acc[nt]);
                }
            }
        }
    }

    // ---------------- output
    if constexpr (EMITP) return;
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
                load_gates8(nb + c, nv);
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
    if (OUTDECAY) {
        // out of the frame: e^{a_t - a_fref}, t within 31 steps before fref
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = min(t0 + 32 * wr + 8 * (r >> 2) + 4 * hh + (r & 3), T_ - 1);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int col = v0 + 32 * nt + i32;
                float ex = ab[(size_t)t * gw + col];
                if (fref >= 0) ex -= ab[(size_t)fref * gw + col];
                acc[nt][r] *= exp2_fast(ex * kLog2e);
            }
        }
    }
    // Out through LDS, 64 columns at a time: the wave writes its accumulators
    // (lane = column) into its own 32 x 64 block, then every lane stores
    // 16-byte runs of rows -- 32/VEC wide stores per lane instead of 64
    // two-byte ones, which otherwise keep the memory pipeline busy after
    // the last tile.
    static_assert(NT % 2 == 0, "value tiles are multiples of 64 columns");
    // Row dots (per-step gates) and per-element products (per-channel gate):
    // the partner rows arrive as 16-byte pieces and reach the accumulator
    // layout through the same blocks; the products leave through an fp32 view
    // of the staging area where it fits.
    constexpr bool RDOTS = DOTS && GATE != kGla, GDOTS = DOTS && GATE == kGla;
    constexpr bool FSTAGE = GDOTS && sizeof(float) * NW * 32 * 68 <= sizeof(Lds) - sizeof(float) * 64;   // not into bcol
    Vec16<T> ppc[DOTS ? NT / 2 : 1][32 / VEC];
    float sum[16];
    if constexpr (DOTS) {
        const T* pb = partner + bh * (size_t)T_ * dhv + v0;
#pragma unroll
        for (int ph = 0; ph < NT / 2; ++ph)
#pragma unroll
            for (int qq = 0; qq < 32 / VEC; ++qq) {
                const int c = lane + 64 * qq, rr = c / (64 / VEC), col = (c % (64 / VEC)) * VEC;
                const int t = min(t0 + 32 * wr + rr, T_ - 1);
                ppc[ph][qq].load(pb + (size_t)row(t) * dhv + 64 * ph + col);
            }
#pragma unroll
        for (int r = 0; r < 16; ++r) sum[r] = 0.0f;
    }
    __syncthreads();   // every wave is done with the tiles the staging blocks overlay
    T* const hrow = h + bh * (size_t)T_ * dhv + v0;   // this workgroup's output columns
#pragma unroll
    for (int ph = 0; ph < NT / 2; ++ph) {
        auto os = sm.os[w];
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
            const int t = t0 + 32 * wr + rr;
            if (t < T_) {
                Vec16<T> x;
                x.load(&os[rr][col]);
                x.store_nt(hrow + (size_t)row(t) * dhv + 64 * ph + col);   // (not read again by the library)
            }
        }
        if constexpr (RDOTS) {
            // row dot products of the fp32 output with the partner rows, before
            // rounding: the gate gradients sum them over the sequence, where
            // rounding first would not cancel
            __syncthreads();   // the output pieces have been read
#pragma unroll
            for (int qq = 0; qq < 32 / VEC; ++qq) {
                const int c = lane + 64 * qq, rr = c / (64 / VEC), col = (c % (64 / VEC)) * VEC;
                ppc[ph][qq].store(&os[rr][col]);
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
                sum[r] += acc[2 * ph][r] * scale * to_float(os[rr][i32]);
                sum[r] += acc[2 * ph + 1][r] * scale * to_float(os[rr][32 + i32]);
            }
        }
        if constexpr (GDOTS) {
            // per-element products of the fp32 output with the partner, before
            // rounding (the per-channel gate gradient sums them per channel)
            __syncthreads();   // the output pieces have been read
#pragma unroll
            for (int qq = 0; qq < 32 / VEC; ++qq) {
                const int c = lane + 64 * qq, rr = c / (64 / VEC), col = (c % (64 / VEC)) * VEC;
                ppc[ph][qq].store(&os[rr][col]);
            }
            __syncthreads();
            float prod[2][16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
                prod[0][r] = acc[2 * ph][r] * scale * to_float(os[rr][i32]);
                prod[1][r] = acc[2 * ph + 1][r] * scale * to_float(os[rr][32 + i32]);
            }
            float* db = dots + bh * (size_t)T_ * dhv + v0 + 64 * ph;
            if constexpr (FSTAGE) {
                // this wave's 32 x 64 fp32 block (stride 68), then 16-byte runs of rows
                __syncthreads();   // every wave has read its partner values
                float (*fs)[68] = reinterpret_cast<float (*)[68]>(&sm) + 32 * w;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
                    fs[rr][i32] = prod[0][r];
                    fs[rr][32 + i32] = prod[1][r];
                }
                __syncthreads();
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int c = lane + 64 * qq, rr = c / 16, col = (c % 16) * 4;
                    const int t = t0 + 32 * wr + rr;
                    if (t < T_)
                        *reinterpret_cast<f32x4*>(db + (size_t)row(t) * dhv + col) =
                            *reinterpret_cast<const f32x4*>(&fs[rr][col]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = t0 + 32 * wr + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (t >= T_) continue;
                    db[(size_t)row(t) * dhv + i32] = prod[0][r];
                    db[(size_t)row(t) * dhv + 32 + i32] = prod[1][r];
                }
            }
        }
        if (ph + 1 < NT / 2) __syncthreads();   // this block is read before it is overwritten
    }
    if constexpr (RDOTS) {
#pragma unroll
        for (int m = 1; m < 32; m <<= 1)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] += __shfl_xor(sum[r], m, 64);
        if (i32 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = t0 + 32 * wr + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (t < T_) dots[(bh * (size_t)T_ + row(t)) * nvt + v0 / BV] = sum[r];
            }
        }
    }
}

template <typename T, int GATE, int DQK, int BV, int NW, int MODE>
hipError_t launch_intra_t(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                          const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    constexpr int BQ = 32 * NW;
    const int nqt = (p.T + BQ - 1) / BQ;
    const int blocks = p.B * p.H * nqt * (p.dhv / BV);
    intra_kernel<T, GATE, DQK, BV, NW, MODE><<<blocks, 64 * NW, 0, stream>>>(
        static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), ws.a, ws.li, fg,
        static_cast<const std::conditional_t<(MODE & kStateF32) != 0, float, T>*>(ws.states), static_cast<T*>(h), p.H, p.T, p.dhv, p.L, p.nc, ws.c0 != nullptr, scale,
        static_cast<const T*>(ws.dot_partner), ws.dots, static_cast<T*>(ws.p_out), static_cast<const T*>(ws.p_in),
        ws.lb, ws.nst);
    return hipGetLastError();
}

// Value-tile width: 128 when it divides d_hv (bf16 I/O), else 64 (fp32 I/O
// always: its doubled fragments would not fit the register budget; nor
// would a 512-wide contraction's at two waves, i.e. L = 64).
// The intra-BV knob set to 64 forces 64 (tuning sweeps).
inline int intra_bv(const Problem& p)
{
    if (knob(TFLA_KNOB_INTRA_BV) == 64) return 64;
    if (p.dqk > 256 && p.L < 128) return 64;
    return (p.bf16 && p.dhv % 128 == 0) ? 128 : 64;
}

// Query rows per workgroup (32 per wave): as many as the chunk allows, up to
// 256 (bf16) -- every staged C^T block and K/V tile then serves more rows.
// A 512-wide contraction (the dq and dk products of the backward pass)
// keeps 128: its 32 Q fragments need the whole register file, i.e. four
// waves at one wave per SIMD (measured 14% faster over the backward pass
// than eight spilling waves, and than 64-wide value tiles, which recompute
// S = K Q^T for twice as many tiles).  The intra-rows knob (64, 128 or 256)
// caps it (tuning sweeps).
inline int intra_rows(const Problem& p)
{
    int cap = p.bf16 ? (p.dqk > 256 ? 128 : 256) : 128;
    const int want = knob(TFLA_KNOB_INTRA_ROWS);
    if (want == 64 || want == 128 || want == 256) cap = want < cap ? want : cap;
    int rows = 64;
    while (rows * 2 <= cap && p.L % (rows * 2) == 0) rows *= 2;
    return rows;
}

template <typename T, int GATE, int DQK, int BV, int MODE>
hipError_t dispatch_nw(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                       const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    // a workgroup's query rows never straddle a chunk; writing P holds no
    // accumulators, so 8 waves fit a 512-wide contraction there
    const int rows = MODE == kEmitP ? intra_rows(Problem{p.B, p.H, p.T, 256, p.dhv, p.L, p.nc, p.gate, p.bf16, p.st32})
                                    : intra_rows(p);
    if constexpr (sizeof(T) == 2 && (DQK <= 256 || MODE == kEmitP)) {
        if (rows == 256) return launch_intra_t<T, GATE, DQK, BV, 8, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    }
    if (rows >= 128) return launch_intra_t<T, GATE, DQK, BV, 4, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    return launch_intra_t<T, GATE, DQK, BV, 2, MODE>(p, q, k, v, fg, ws, h, scale, stream);
}

template <typename T, int GATE, int DQK, int MODE>
hipError_t dispatch_bv(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                       const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    if constexpr (sizeof(T) == 2) {
        if (intra_bv(p) == 128) return dispatch_nw<T, GATE, DQK, 128, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    }
    return dispatch_nw<T, GATE, DQK, 64, MODE>(p, q, k, v, fg, ws, h, scale, stream);
}

// contraction widths: 64, 128, 256 (bf16) for the forward pass; the gradient
// modes also contract over d_hv, up to 512 (bf16)
template <typename T, int GATE, int MODE>
hipError_t dispatch_dqk(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                        const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    switch (p.dqk) {
    case 64: return dispatch_bv<T, GATE, 64, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    case 128: return dispatch_bv<T, GATE, 128, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    case 256:
        // (fp32 I/O: 64-wide value tiles keep the 256-channel Q fragments
        // within the registers of four waves)
        return dispatch_bv<T, GATE, 256, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    case 512:
        // (fp32 I/O: the 512 fp32 channels of the Q fragments fit four waves
        // only where P is given; the backward pass shares P there)
        if constexpr (MODE != 0 && MODE != kStateF32)
            return dispatch_bv<T, GATE, 512, MODE>(p, q, k, v, fg, ws, h, scale, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int MODE>
hipError_t dispatch_gate(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                         const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    switch (p.gate) {
    case kSig: return dispatch_dqk<T, kSig, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    case kScalar: return dispatch_dqk<T, kScalar, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    case kExp:
        // mLSTMexp has a forward pass only
        if constexpr (MODE == 0 || MODE == kStateF32) return dispatch_dqk<T, kExp, MODE>(p, q, k, v, fg, ws, h, scale, stream);
        return hipErrorInvalidValue;
    default:
        if constexpr ((MODE & (kEmitP | kGivenP)) == 0) return dispatch_dqk<T, kGla, MODE>(p, q, k, v, fg, ws, h, scale, stream);
        return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t dispatch_type(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                         const Workspace& ws, void* h, float scale, hipStream_t stream)
{
    if (p.bf16) return dispatch_gate<bf16, MODE>(p, q, k, v, fg, ws, h, scale, stream);
    return dispatch_gate<float, MODE>(p, q, k, v, fg, ws, h, scale, stream);
}

}  // namespace
}  // namespace tfla

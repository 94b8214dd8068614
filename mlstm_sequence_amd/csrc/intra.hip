// intra.hip -- intra-chunk kernel (third kernel of the path).
//
// For step t of chunk k (steps [cs, cs+L)):
//   h_t = scale * ( e^{a_t} q_t^T C_{k-1}
//                   + sum_{cs <= s <= t} e^{a_t - a_s + li_s} (q_t . k_s) v_s )
// (GLA gate: the decay enters per key channel inside q.k, and the inter term
// is (q_t o e^{a_t}) C_{k-1}).  TFLA's second level of sequence parallelism
// (TFLA abstract; research-map summary, Approach) tiles this along the
// sequence: a workgroup owns 64 query steps x BV value columns of one chunk
// and loops over the 64-step key/value tiles at or before its own, so the
// chunk size L is bounded by nothing on chip.
//
// Every stage (a block of C^T, or a K/V tile) is software-pipelined: its
// global loads are issued into registers right after the previous stage was
// written to LDS, so they are in flight while the matrix cores work.
//
// Per workgroup (4 wavefronts, wave w owns query rows 16w..16w+15):
//   inter: acc = Q C_{k-1}[:, v-tile]  (C^T staged in LDS per 32-channel
//          block, rounded fp32 -> operand type), rows scaled by e^{a_t};
//   intra: for each key tile j <= own tile: stage K_j (row-major) and V_j^T
//          in LDS; S^T = K_j Q^T on matrix cores (Q fragments stay in
//          registers, they are the B operand here and the A operand of the
//          inter product); decay and causal mask applied in fp32 (a select,
//          never a multiply by 0); the S^T accumulators are reused directly
//          as the A operand of acc += P V_j, by contracting the step index in
//          the order the accumulator layout holds it (V_j^T is read in the
//          same order);
//   out:   h = acc * scale, rounded to the I/O type.
// Per-channel gates use a reference-point factorisation: off-diagonal tiles
// scale q by e^{a_t - a_ref} and k by e^{a_ref - a_s} with a_ref at the step
// before the query tile (both factors <= 1); the diagonal tile uses the
// tile's middle step.
#include <cstdlib>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

template <typename T, int DQK, int BV> struct IntraLds {
    static constexpr int pad = 16 / sizeof(T);
    union {
        struct {
            T ks[64][DQK + pad];   // K tile, row-major [step][channel]
            T vt[BV][64 + pad];    // V tile transposed [value][step]
        } kv;
        T cs[BV][32 + pad];        // 32-channel block of C^T [value][channel]
    };
    float bcol[64];                // mLSTMsig: (li_s - a_s) log2(e) per key step
};

// Registers holding one stage's global loads while the previous stage computes.
template <typename T, int DQK, int BV> struct Prefetch {
    static constexpr int VEC = Elem<T>::vec;
    static constexpr int NC = BV / 64;                     // C^T block: 8 floats per item
    static constexpr int NK = 64 * DQK / VEC / 256;        // K tile: 16 bytes per item
    static constexpr int NV = 32 * (BV / VEC) / 256;       // V tile: two rows x 16 bytes per item
    static_assert(NC >= 1 && NK >= 1 && NV >= 1, "tile too small for 256 threads");
    f32x4 c[NC][2];
    Vec16<T> k[NK];
    Vec16<T> v[NV][2];
    float li, a;
};

template <typename T, int GATE, int DQK, int BV>
__global__ __launch_bounds__(256, (BV >= 256 ? 1 : 2)) void intra_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, const float* __restrict__ a,
                                                       const float* __restrict__ li,
                                                       const float* __restrict__ fg,
                                                       const float* __restrict__ states, T* __restrict__ h,
                                                       int H, int T_, int dhv, int L, int nc, float scale)
{
    __shared__ IntraLds<T, DQK, BV> sm;
    typedef typename Elem<T>::frag Frag;
    typedef Prefetch<T, DQK, BV> PF;
    constexpr int VEC = Elem<T>::vec;
    constexpr int KQ = DQK / 32;   // contraction steps over key channels
    constexpr int NT = BV / 16;    // 16-wide output column tiles

    const int nqt = (T_ + 63) >> 6;
    const int nvt = dhv / BV;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const size_t bh = blk / (nqt * nvt);
    const int rem = blk % (nqt * nvt);
    const int qt = rem / nvt;
    const int v0 = (rem % nvt) * BV;
    const int t0 = qt * 64;
    const int kc = t0 / L, cs = kc * L, qi = (t0 - cs) >> 6;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, l16 = lane & 15;
    const int tq = t0 + 16 * w + l16;       // query step of this lane's fragment row
    const bool tq_ok = tq < T_;

    const T* qb = q + bh * (size_t)T_ * DQK;
    const T* kb = k + bh * (size_t)T_ * DQK;
    const T* vb = v + bh * (size_t)T_ * dhv;
    const float* ab = (GATE == kGla) ? a + bh * (size_t)T_ * DQK : a + bh * (size_t)T_;
    const float* lb = (GATE == kSig) ? li + bh * (size_t)T_ : nullptr;
    float lg2 = 0.0f;   // log2 of the fixed decay
    if (GATE == kScalar) lg2 = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor) * kLog2e;

    PF pf;

    // Q fragments; per-channel gate: q * e^{a_t - a_ref} (ref_row < 0: chunk start, a = 0)
    Frag qf[KQ];
    auto load_q = [&](int ref_row) {
        for (int kq = 0; kq < KQ; ++kq) {
            const int c = 32 * kq + 8 * gq;
            if (!tq_ok) {
                for (int e = 0; e < 8; ++e) frag_set(qf[kq], e, 0.0f);
                continue;
            }
            if (GATE != kGla) {
                qf[kq] = load8(qb + (size_t)tq * DQK + c);
            } else {
                const Frag raw = load8(qb + (size_t)tq * DQK + c);
                for (int e = 0; e < 8; ++e) {
                    float ex = ab[(size_t)tq * DQK + c + e];
                    if (ref_row >= 0) ex -= ab[(size_t)ref_row * DQK + c + e];
                    frag_set(qf[kq], e, frag_get(raw, e) * exp2_fast(ex * kLog2e));
                }
            }
        }
    };

    // ---- stage loaders (global -> registers) and writers (registers -> LDS)
    auto fetch_c = [&](const float* st, int cb) {
#pragma unroll
        for (int u = 0; u < PF::NC; ++u) {
            const int idx = tid + 256 * u, vr = idx >> 2, c8 = (idx & 3) * 8;
            const float* src = st + (size_t)vr * DQK + cb + c8;
            pf.c[u][0] = *reinterpret_cast<const f32x4*>(src);
            pf.c[u][1] = *reinterpret_cast<const f32x4*>(src + 4);
        }
    };
    auto store_c = [&]() {
#pragma unroll
        for (int u = 0; u < PF::NC; ++u) {
            const int idx = tid + 256 * u, vr = idx >> 2, c8 = (idx & 3) * 8;
            if constexpr (sizeof(T) == 2) {
                Vec16<T> x;
                for (int e = 0; e < 4; ++e) {
                    x.set(e, pf.c[u][0][e]);
                    x.set(4 + e, pf.c[u][1][e]);
                }
                x.store(&sm.cs[vr][c8]);
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(&sm.cs[vr][c8])) = pf.c[u][0];
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(&sm.cs[vr][c8 + 4])) = pf.c[u][1];
            }
        }
    };
    auto fetch_kv = [&](int s0) {
#pragma unroll
        for (int u = 0; u < PF::NK; ++u) {
            const int idx = tid + 256 * u, r = idx / (DQK / VEC), c = (idx % (DQK / VEC)) * VEC;
            const int s = s0 + r;
            if (s < T_) pf.k[u].load(kb + (size_t)s * DQK + c); else pf.k[u].zero();
        }
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int idx = tid + 256 * u, sp = idx & 31, cg = (idx >> 5) * VEC;
            const int s = s0 + 2 * sp;
            if (s < T_) pf.v[u][0].load(vb + (size_t)s * dhv + v0 + cg); else pf.v[u][0].zero();
            if (s + 1 < T_) pf.v[u][1].load(vb + (size_t)(s + 1) * dhv + v0 + cg); else pf.v[u][1].zero();
        }
        if (GATE == kSig && tid < 64) {
            const int s = s0 + tid;
            pf.li = (s < T_) ? lb[s] : 0.0f;
            pf.a = (s < T_) ? ab[s] : 0.0f;
        }
    };
    auto store_kv = [&](int s0, int ref_row) {
#pragma unroll
        for (int u = 0; u < PF::NK; ++u) {
            const int idx = tid + 256 * u, r = idx / (DQK / VEC), c = (idx % (DQK / VEC)) * VEC;
            if (GATE == kGla) {
                const int s = s0 + r;
                if (s < T_) {
                    for (int e = 0; e < VEC; ++e) {
                        const float ex = ab[(size_t)ref_row * DQK + c + e] - ab[(size_t)s * DQK + c + e];
                        pf.k[u].set(e, pf.k[u].get(e) * exp2_fast(ex * kLog2e));
                    }
                }
            }
            pf.k[u].store(&sm.kv.ks[r][c]);
        }
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int idx = tid + 256 * u, sp = idx & 31, cg = (idx >> 5) * VEC;
            for (int e = 0; e < VEC; ++e)
                store2(&sm.kv.vt[cg + e][2 * sp], pf.v[u][0].get(e), pf.v[u][1].get(e));
        }
        if (GATE == kSig && tid < 64) sm.bcol[tid] = (pf.li - pf.a) * kLog2e;
    };

    f32x4 acc[NT];
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---------------- inter-chunk term: e^{a_t} q_t^T C_{k-1}
    if (kc > 0) {
        const float* st = states + ((bh * (nc - 1) + kc - 1) * (size_t)dhv + v0) * DQK;
        fetch_c(st, 0);
        load_q(-1);
        for (int kq = 0; kq < KQ; ++kq) {
            __syncthreads();
            store_c();
            __syncthreads();
            // the next stage's loads fly while this block is multiplied
            if (kq + 1 < KQ) fetch_c(st, 32 * (kq + 1));
            else fetch_kv(cs);
            for (int nt = 0; nt < NT; ++nt) {
                const Frag bf = load8(&sm.cs[16 * nt + l16][8 * gq]);
                acc[nt] = mma(qf[kq], bf, acc[nt]);
            }
        }
        if (GATE != kGla) {
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 16 * w + 4 * gq + r;
                float e = 0.0f;
                if (t < T_) {
                    e = (GATE == kSig) ? exp2_fast(ab[t] * kLog2e)
                                       : exp2_fast((float)(t - cs + 1) * lg2);
                }
                for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= e;
            }
        }
    } else {
        fetch_kv(cs);
    }

    // ---------------- intra-chunk term, tiled along the chunk
    if (GATE != kGla) {
        if (kc == 0) load_q(-1);
    }
    const float at2 = (GATE == kSig && tq_ok) ? ab[tq] * kLog2e : 0.0f;
    const int tl = 16 * w + l16;            // query row inside the tile

    for (int j = 0; j <= qi; ++j) {
        const bool diag = (j == qi);
        const int s0 = cs + 64 * j;
        int ref_row = -1;
        if (GATE == kGla) {
            ref_row = diag ? min(t0 + 31, T_ - 1) : t0 - 1;
            if (j == 0 || diag) load_q(ref_row);
        }
        __syncthreads();
        store_kv(s0, ref_row);
        __syncthreads();
        if (!diag) fetch_kv(s0 + 64);

        // S^T (64 key steps x 16 query rows of this wave)
        f32x4 st[4];
        for (int mt = 0; mt < 4; ++mt) st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kq = 0; kq < KQ; ++kq) {
            for (int mt = 0; mt < 4; ++mt) {
                const Frag af = load8(&sm.kv.ks[16 * mt + l16][32 * kq + 8 * gq]);
                st[mt] = mma(af, qf[kq], st[mt]);
            }
        }
        // decay and causal mask: element (mt, r) is key step sl = 16mt + 4gq + r, query row tl
        for (int mt = 0; mt < 4; ++mt) {
            for (int r = 0; r < 4; ++r) {
                const int sl = 16 * mt + 4 * gq + r;
                float p = st[mt][r];
                if (GATE == kSig) {
                    p *= exp2_fast(at2 + sm.bcol[sl]);
                } else if (GATE == kScalar) {
                    p *= exp2_fast((float)(64 * (qi - j) + tl - sl) * lg2);
                }
                st[mt][r] = (diag && sl > tl) ? 0.0f : p;
            }
        }
        // acc += P V_j, step index contracted in accumulator order
        for (int kk = 0; kk < 2; ++kk) {
            Frag pfr;
            for (int e = 0; e < 4; ++e) {
                frag_set(pfr, e, st[2 * kk][e]);
                frag_set(pfr, 4 + e, st[2 * kk + 1][e]);
            }
            for (int nt = 0; nt < NT; ++nt) {
                const T* row = sm.kv.vt[16 * nt + l16];
                const Frag vf = load4x2(row + 32 * kk + 4 * gq, row + 32 * kk + 16 + 4 * gq);
                acc[nt] = mma(pfr, vf, acc[nt]);
            }
        }
    }

    // ---------------- output
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * w + 4 * gq + r;
        if (t >= T_) continue;
        T* dst = h + (bh * (size_t)T_ + t) * dhv + v0 + l16;
        for (int nt = 0; nt < NT; ++nt) dst[16 * nt] = from_float<T>(acc[nt][r] * scale);
    }
}

template <typename T, int GATE, int DQK, int BV>
hipError_t launch_intra_t(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                          const Workspace& ws, void* h, hipStream_t stream)
{
    const int nqt = (p.T + 63) / 64;
    const int blocks = p.B * p.H * nqt * (p.dhv / BV);
    const float scale = 1.0f / sqrtf((float)DQK);
    intra_kernel<T, GATE, DQK, BV><<<blocks, 256, 0, stream>>>(
        static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), ws.a, ws.li, fg,
        ws.states, static_cast<T*>(h), p.H, p.T, p.dhv, p.L, p.nc, scale);
    return hipGetLastError();
}

// Value-tile width: the widest of 128 / 64 dividing d_hv.  128 keeps two
// workgroups per CU; 256 (one workgroup per CU, no recomputed S across value
// tiles) measured slower.  TFLA_INTRA_BV=64|128|256 overrides (bf16 I/O only
// for 256) for tuning sweeps.
inline int intra_bv(const Problem& p)
{
    int cap = 128;
    if (const char* e = std::getenv("TFLA_INTRA_BV")) {
        const int want = std::atoi(e);
        if (want == 64 || want == 128 || want == 256) cap = (want == 256 && !p.bf16) ? 128 : want;
    }
    for (int bv = cap; bv >= 64; bv /= 2)
        if (p.dhv % bv == 0) return bv;
    return 64;
}

template <typename T, int GATE, int DQK>
hipError_t dispatch_bv(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                       const Workspace& ws, void* h, hipStream_t stream)
{
    const int bv = intra_bv(p);
    if constexpr (sizeof(T) == 2) {
        if (bv == 256) return launch_intra_t<T, GATE, DQK, 256>(p, q, k, v, fg, ws, h, stream);
    }
    if (bv >= 128) return launch_intra_t<T, GATE, DQK, 128>(p, q, k, v, fg, ws, h, stream);
    return launch_intra_t<T, GATE, DQK, 64>(p, q, k, v, fg, ws, h, stream);
}

template <typename T, int GATE>
hipError_t dispatch_dqk(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                        const Workspace& ws, void* h, hipStream_t stream)
{
    switch (p.dqk) {
    case 64: return dispatch_bv<T, GATE, 64>(p, q, k, v, fg, ws, h, stream);
    case 128: return dispatch_bv<T, GATE, 128>(p, q, k, v, fg, ws, h, stream);
    default:
        if constexpr (sizeof(T) == 2) return dispatch_bv<T, GATE, 256>(p, q, k, v, fg, ws, h, stream);
        return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t dispatch_gate(const Problem& p, const void* q, const void* k, const void* v, const float* fg,
                         const Workspace& ws, void* h, hipStream_t stream)
{
    switch (p.gate) {
    case kSig: return dispatch_dqk<T, kSig>(p, q, k, v, fg, ws, h, stream);
    case kScalar: return dispatch_dqk<T, kScalar>(p, q, k, v, fg, ws, h, stream);
    default: return dispatch_dqk<T, kGla>(p, q, k, v, fg, ws, h, stream);
    }
}

}  // namespace

hipError_t launch_intra(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, void* h, hipStream_t stream)
{
    if (p.bf16) return dispatch_gate<bf16>(p, q, k, v, fgate_pre, ws, h, stream);
    return dispatch_gate<float>(p, q, k, v, fgate_pre, ws, h, stream);
}

}  // namespace tfla

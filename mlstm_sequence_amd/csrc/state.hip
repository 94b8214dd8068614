// state.hip -- inter-chunk state kernel (second kernel of the path).
//
// Materialises the matrix memory at every chunk boundary (the
// "ParallelChunk" form of the flash-linear-attention README: states written
// to global memory for each chunk; the TFLA abstract names this the traffic
// its larger chunks cut):
//   C_k = diag(e^{g_k}) C_{k-1} + sum_{s in chunk k} w_s k_s v_s^T,
//   w_s = e^{g_k - a_s + li_s}    (per key channel c for the GLA gate:
//                                  e^{g_{k,c} - a_{s,c}})
// with C_0 = 0.  States after chunks 1..N_c-1 are written in fp32,
// transposed ([d_hv][d_qk]) so the intra-chunk kernel reads them as
// contiguous matrix-core B operands.
//
// One workgroup (4 wavefronts) owns a 64x64 tile of C^T (64 value rows x 64
// key columns) for one head and walks the chunks serially, keeping the fp32
// tile in accumulator registers.  Per 64-step block of a chunk it stages V^T
// and (w.K)^T in LDS, transposing on the way (K is scaled in fp32 and then
// rounded, once, to the operand type).  Wave w owns value rows 16w..16w+15.
// The block loop is software-pipelined: the next block's global loads are
// issued right after the current block reaches LDS.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

constexpr int kTile = 64;   // C^T tile: 64 value rows x 64 key columns
constexpr int kSB = 64;     // steps per staged block

template <typename T> struct StateLds {
    static constexpr int pad = 16 / sizeof(T);   // keeps 16-byte row alignment
    static constexpr int row = kSB + pad;
    T vt[kTile][row];   // V^T block: [value][step]
    T kt[kTile][row];   // (w.K)^T block: [key channel][step]
};

// One 64-step block's global loads, held in registers while the previous
// block is multiplied.  Item = two consecutive steps x VEC columns.
template <typename T, int GATE> struct StatePrefetch {
    static constexpr int VEC = Elem<T>::vec;
    static constexpr int NI = (kSB / 2) * (kTile / VEC) / 256;
    static_assert(NI >= 1, "block too small for 256 threads");
    Vec16<T> v[NI][2], k[NI][2];
    float a[NI][2], li[NI][2];                 // mLSTMsig step gates
    f32x4 ga[NI][2][VEC / 4];                  // per-channel gate: a of the item's columns
    f32x4 gg[NI][VEC / 4];                     // per-channel gate: g of the item's columns
    float g;                                   // mLSTMsig: g of the block's chunk
};

template <typename T, int GATE>
__global__ __launch_bounds__(256) void state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                    const float* __restrict__ a,
                                                    const float* __restrict__ li,
                                                    const float* __restrict__ g,
                                                    const float* __restrict__ fg,
                                                    float* __restrict__ states, int H, int T_,
                                                    int dqk, int dhv, int L, int nc)
{
    __shared__ StateLds<T> sm;
    typedef StatePrefetch<T, GATE> PF;
    constexpr int VEC = Elem<T>::vec;

    const int ntv = dhv / kTile, ntk = dqk / kTile;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int tiles = ntv * ntk;
    const size_t bh = blk / tiles;
    const int tile = blk % tiles;
    const int v0 = (tile / ntk) * kTile;
    const int c0 = (tile % ntk) * kTile;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, l16 = lane & 15;

    const T* kb = k + bh * (size_t)T_ * dqk;
    const T* vb = v + bh * (size_t)T_ * dhv;
    float lg2 = 0.0f;
    if (GATE == kScalar) lg2 = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor) * kLog2e;

    const int bpc = L / kSB;                 // blocks per chunk
    const int nblocks = (nc - 1) * bpc;      // chunks 0..nc-2 are full and feed a state

    PF pf;
    auto item = [&](int u, int& sp, int& cg) {
        const int idx = tid + 256 * u;
        sp = idx % (kSB / 2);                // step pair fastest: transposed LDS writes spread over banks
        cg = (idx / (kSB / 2)) * VEC;
    };
    auto fetch = [&](int b) {
        const int kc = b / bpc;
        const int s0 = b * kSB;              // block start (chunks are full, so = kc*L + (b%bpc)*kSB)
        if (GATE == kSig) pf.g = g[bh * nc + kc];
#pragma unroll
        for (int u = 0; u < PF::NI; ++u) {
            int sp, cg;
            item(u, sp, cg);
            const int s = s0 + 2 * sp;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                pf.v[u][r].load(vb + (size_t)(s + r) * dhv + v0 + cg);
                pf.k[u][r].load(kb + (size_t)(s + r) * dqk + c0 + cg);
                if (GATE == kSig) {
                    pf.a[u][r] = a[bh * T_ + s + r];
                    pf.li[u][r] = li[bh * T_ + s + r];
                }
                if (GATE == kGla) {
                    const float* ar = a + (bh * T_ + s + r) * (size_t)dqk + c0 + cg;
                    for (int e4 = 0; e4 < VEC / 4; ++e4) pf.ga[u][r][e4] = *reinterpret_cast<const f32x4*>(ar + 4 * e4);
                }
            }
            if (GATE == kGla) {
                const float* gr = g + (bh * nc + kc) * (size_t)dqk + c0 + cg;
                for (int e4 = 0; e4 < VEC / 4; ++e4) pf.gg[u][e4] = *reinterpret_cast<const f32x4*>(gr + 4 * e4);
            }
        }
    };
    auto store = [&](int b) {
        const int kc = b / bpc;
        const int cs = kc * L;
#pragma unroll
        for (int u = 0; u < PF::NI; ++u) {
            int sp, cg;
            item(u, sp, cg);
            const int s = b * kSB + 2 * sp;
            float w0 = 1.0f, w1 = 1.0f;
            if (GATE == kSig) {
                w0 = exp2_fast((pf.g - pf.a[u][0] + pf.li[u][0]) * kLog2e);
                w1 = exp2_fast((pf.g - pf.a[u][1] + pf.li[u][1]) * kLog2e);
            } else if (GATE == kScalar) {
                const int p0 = s - cs;
                w0 = exp2_fast((float)(L - 1 - p0) * lg2);
                w1 = exp2_fast((float)(L - 2 - p0) * lg2);
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int col = cg + e;
                store2(&sm.vt[col][2 * sp], pf.v[u][0].get(e), pf.v[u][1].get(e));
                float kw0, kw1;
                if (GATE == kGla) {
                    const float gc = pf.gg[u][e / 4][e % 4];
                    kw0 = pf.k[u][0].get(e) * exp2_fast((gc - pf.ga[u][0][e / 4][e % 4]) * kLog2e);
                    kw1 = pf.k[u][1].get(e) * exp2_fast((gc - pf.ga[u][1][e / 4][e % 4]) * kLog2e);
                } else {
                    kw0 = pf.k[u][0].get(e) * w0;
                    kw1 = pf.k[u][1].get(e) * w1;
                }
                store2(&sm.kt[col][2 * sp], kw0, kw1);
            }
        }
    };

    f32x4 acc[4];
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nblocks > 0) fetch(0);
    for (int b = 0; b < nblocks; ++b) {
        const int kc = b / bpc;
        const bool first = (b % bpc) == 0, last = (b % bpc) == bpc - 1;
        __syncthreads();
        store(b);
        __syncthreads();
        if (b + 1 < nblocks) fetch(b + 1);
        if (first) {
            // decay of the carried state across chunk kc
            if (GATE == kSig) {
                const float e = exp2_fast(g[bh * nc + kc] * kLog2e);
                for (int nt = 0; nt < 4; ++nt) acc[nt] *= e;
            } else if (GATE == kScalar) {
                const float e = exp2_fast((float)L * lg2);
                for (int nt = 0; nt < 4; ++nt) acc[nt] *= e;
            } else {
                for (int nt = 0; nt < 4; ++nt) {
                    const int c = c0 + nt * 16 + l16;
                    acc[nt] *= exp2_fast(g[(bh * nc + kc) * dqk + c] * kLog2e);
                }
            }
        }
        // acc[nt] (value rows 16w.., key cols 16nt..) += V^T (w.K)
        for (int ks = 0; ks < kSB; ks += 32) {
            const auto af = load8(&sm.vt[16 * w + l16][ks + 8 * gq]);
            for (int nt = 0; nt < 4; ++nt) {
                const auto bf = load8(&sm.kt[16 * nt + l16][ks + 8 * gq]);
                acc[nt] = mma(af, bf, acc[nt]);
            }
        }
        if (last) {
            // C^T tile of the state after chunk kc
            float* dst = states + ((bh * (nc - 1) + kc) * (size_t)dhv + v0 + 16 * w + 4 * gq) * dqk + c0 + l16;
            for (int nt = 0; nt < 4; ++nt)
                for (int r = 0; r < 4; ++r) dst[(size_t)r * dqk + 16 * nt] = acc[nt][r];
        }
    }
}

template <typename T>
hipError_t launch_state_t(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                          hipStream_t stream)
{
    if (p.nc < 2) return hipSuccess;
    const int blocks = p.B * p.H * (p.dhv / kTile) * (p.dqk / kTile);
    switch (p.gate) {
    case kSig:
        state_kernel<T, kSig><<<blocks, 256, 0, stream>>>(k, v, ws.a, ws.li, ws.g, fg, ws.states, p.H, p.T,
                                                           p.dqk, p.dhv, p.L, p.nc);
        break;
    case kScalar:
        state_kernel<T, kScalar><<<blocks, 256, 0, stream>>>(k, v, ws.a, ws.li, ws.g, fg, ws.states, p.H,
                                                              p.T, p.dqk, p.dhv, p.L, p.nc);
        break;
    default:
        state_kernel<T, kGla><<<blocks, 256, 0, stream>>>(k, v, ws.a, ws.li, ws.g, fg, ws.states, p.H, p.T,
                                                           p.dqk, p.dhv, p.L, p.nc);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state(const Problem& p, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream)
{
    if (p.bf16)
        return launch_state_t<bf16>(p, static_cast<const bf16*>(k), static_cast<const bf16*>(v), fgate_pre, ws,
                                    stream);
    return launch_state_t<float>(p, static_cast<const float*>(k), static_cast<const float*>(v), fgate_pre, ws,
                                 stream);
}

}  // namespace tfla

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
    constexpr int VEC = Elem<T>::vec;

    const int ntv = dhv / kTile, ntk = dqk / kTile;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int tiles = ntv * ntk;
    const size_t bh = blk / tiles;
    const int tile = blk % tiles;
    const int v0 = (tile / ntk) * kTile;
    const int c0 = (tile % ntk) * kTile;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, gq = lane >> 4, li16 = lane & 15;

    const T* kb = k + bh * (size_t)T_ * dqk;
    const T* vb = v + bh * (size_t)T_ * dhv;
    float lgam = 0.0f;
    if (GATE == kScalar) lgam = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor);

    f32x4 acc[4];
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = 0; kc + 1 < nc; ++kc) {
        const int cs = kc * L;
        // decay of the carried state across chunk kc
        if (GATE == kSig) {
            const float e = exp2_fast(g[bh * nc + kc] * kLog2e);
            for (int nt = 0; nt < 4; ++nt) acc[nt] *= e;
        } else if (GATE == kScalar) {
            const float e = exp2_fast((float)L * lgam * kLog2e);
            for (int nt = 0; nt < 4; ++nt) acc[nt] *= e;
        } else {
            for (int nt = 0; nt < 4; ++nt) {
                const int c = c0 + nt * 16 + li16;
                acc[nt] *= exp2_fast(g[(bh * nc + kc) * dqk + c] * kLog2e);
            }
        }
        const float gk = (GATE == kSig) ? g[bh * nc + kc] : 0.0f;

        for (int sb = 0; sb < L; sb += kSB) {
            __syncthreads();
            // stage: items = (kSB/2 step pairs) x (kTile/VEC column groups),
            // step pair fastest so the transposed LDS writes spread over banks
            constexpr int CG = kTile / VEC;
            for (int it = tid; it < (kSB / 2) * CG; it += 256) {
                const int sp = it % (kSB / 2), cg = it / (kSB / 2);
                const int s = cs + sb + 2 * sp;        // always < T: chunk kc is full
                Vec16<T> v0r, v1r, k0r, k1r;
                v0r.load(vb + (size_t)s * dhv + v0 + cg * VEC);
                v1r.load(vb + (size_t)(s + 1) * dhv + v0 + cg * VEC);
                k0r.load(kb + (size_t)s * dqk + c0 + cg * VEC);
                k1r.load(kb + (size_t)(s + 1) * dqk + c0 + cg * VEC);
                float w0 = 1.0f, w1 = 1.0f;
                if (GATE == kSig) {
                    w0 = exp2_fast((gk - a[bh * T_ + s] + li[bh * T_ + s]) * kLog2e);
                    w1 = exp2_fast((gk - a[bh * T_ + s + 1] + li[bh * T_ + s + 1]) * kLog2e);
                } else if (GATE == kScalar) {
                    const int p0 = s - cs;
                    w0 = exp2_fast((float)(L - 1 - p0) * lgam * kLog2e);
                    w1 = exp2_fast((float)(L - 2 - p0) * lgam * kLog2e);
                }
                for (int e = 0; e < VEC; ++e) {
                    const int col = cg * VEC + e;
                    store2(&sm.vt[col][2 * sp], v0r.get(e), v1r.get(e));
                    float kw0 = k0r.get(e) * w0, kw1 = k1r.get(e) * w1;
                    if (GATE == kGla) {
                        const size_t gi = (bh * nc + kc) * dqk + c0 + col;
                        const float gc = g[gi];
                        kw0 = k0r.get(e) * exp2_fast((gc - a[(bh * T_ + s) * dqk + c0 + col]) * kLog2e);
                        kw1 = k1r.get(e) * exp2_fast((gc - a[(bh * T_ + s + 1) * dqk + c0 + col]) * kLog2e);
                    }
                    store2(&sm.kt[col][2 * sp], kw0, kw1);
                }
            }
            __syncthreads();
            // acc[nt] (value rows 16w.., key cols 16nt..) += V^T (w.K)
            for (int ks = 0; ks < kSB; ks += 32) {
                const auto af = load8(&sm.vt[16 * w + li16][ks + 8 * gq]);
                for (int nt = 0; nt < 4; ++nt) {
                    const auto bf = load8(&sm.kt[16 * nt + li16][ks + 8 * gq]);
                    acc[nt] = mma(af, bf, acc[nt]);
                }
            }
        }
        // write C^T tile of the state after chunk kc
        float* dst = states + ((bh * (nc - 1) + kc) * (size_t)dhv + v0 + 16 * w + 4 * gq) * dqk + c0 + li16;
        for (int nt = 0; nt < 4; ++nt)
            for (int r = 0; r < 4; ++r) dst[(size_t)r * dqk + 16 * nt] = acc[nt][r];
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

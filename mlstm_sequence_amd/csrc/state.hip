// state.hip -- inter-chunk state kernel (second kernel of the path).
//
// Materialises the matrix memory at every chunk boundary (the
// "ParallelChunk" form of the flash-linear-attention README: states written
// to global memory for each chunk; the TFLA abstract names this the traffic
// its larger chunks cut):
//   C_k = diag(e^{g_k}) C_{k-1} + sum_{s in chunk k} w_s k_s v_s^T,
//   w_s = e^{g_k - a_s + li_s}    (per key channel c for the GLA gate:
//                                  e^{g_{k,c} - a_{s,c}})
// from C_0 = 0 or a given initial state.  The state before chunk k (k >= 1,
// and k = 0 when an initial state is given) is written in fp32, transposed
// ([d_hv][d_qk]) so the intra-chunk kernel reads it as contiguous
// matrix-core B operands.  On request the walk continues through the last
// (possibly partial) chunk and writes the final state C_T in the caller's
// [d_qk][d_hv] layout.
//
// One workgroup owns a TV x TC tile of C^T (value rows x key columns; 128x128
// with 8 wavefronts when the problem is large enough to give every CU one,
// else 64x64 with 4) for one head and walks the chunks serially, keeping the
// fp32 tile in accumulator registers spread over its waves.  Per block
// it stages V and w.K row-major in LDS (K scaled in fp32, rounded once to the
// operand type) -- consecutive lanes load consecutive 16-byte pieces of a
// row -- and reads both operands of acc += V^T (w.K) with LDS transpose
// reads.  The block loop is software-pipelined: the next block's loads are
// issued into registers right after the current block reached LDS.  Blocks
// are as long as the chunk allows (up to 256 steps on 128x128 tiles).
// States leave as 128-byte rows.
#include <cstdlib>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

// Tile of C^T per workgroup: TV value rows x TC key columns; NWS wavefronts
// in a 2 x (NWS/2) grid, each owning a (TV/2) x (2 TC/NWS) piece as 32x32
// accumulators.
template <typename T, int SB, int TV, int TC> struct StateLds {
    static constexpr int pad = 32 / sizeof(T);   // row stride = 8 banks mod 32 (transpose reads)
    T vs[SB][TV + pad];   // V block [step][value]
    T ks[SB][TC + pad];   // w.K block [step][key channel]
};

// One block's global loads, held in registers while earlier blocks are
// multiplied.  V item u: step row r, VEC value columns; K item u likewise.
template <typename T, int SB, int TV, int TC, int NTH> struct StatePrefetch {
    static constexpr int VEC = Elem<T>::vec;
    static constexpr int NV = SB * (TV / VEC) / NTH;
    static constexpr int NK = SB * (TC / VEC) / NTH;
    static_assert(NV >= 1 && NK >= 1, "block too small for the workgroup");
    Vec16<T> v[NV], k[NK];
    float a[NK], li[NK];          // mLSTMsig step gates of each K item's row
    f32x4 ga[NK][VEC / 4];        // per-channel gate: a of the K item's columns
    f32x4 gg[NK][VEC / 4];        // per-channel gate: g of the K item's columns
    float g;                      // mLSTMsig: g of the block's chunk
};

template <typename T, int GATE, int SB, int TV, int TC, int NWS>
__global__ __launch_bounds__(64 * NWS) void state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                    const float* __restrict__ a,
                                                    const float* __restrict__ li,
                                                    const float* __restrict__ g,
                                                    const float* __restrict__ fg,
                                                    float* __restrict__ states,
                                                    const float* __restrict__ c_init,
                                                    float* __restrict__ c_final, int H, int T_,
                                                    int dqk, int dhv, int L, int nc)
{
    constexpr int NTH = 64 * NWS;
    typedef StatePrefetch<T, SB, TV, TC, NTH> PF;
    __shared__ StateLds<T, SB, TV, TC> sm;
    constexpr int VEC = Elem<T>::vec;
    constexpr int WC = NWS / 2;                        // waves along the key columns
    constexpr int MV = TV / 64, MC = TC / WC / 32;     // 32x32 accumulators per wave along value / key
    static_assert(MC >= 1, "tile too narrow for the waves");

    const int ntv = dhv / TV, ntk = dqk / TC;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int tiles = ntv * ntk;
    const size_t bh = blk / tiles;
    const int tile = blk % tiles;
    const int v0 = (tile / ntk) * TV;
    const int c0 = (tile % ntk) * TC;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, hh = lane >> 5, i32 = lane & 31;
    const int vw = (TV / 2) * (w / WC), cw = (TC / WC) * (w % WC);   // this wave's piece

    const T* kb = k + bh * (size_t)T_ * dqk;
    const T* vb = v + bh * (size_t)T_ * dhv;
    float lg2 = 0.0f;
    if (GATE == kScalar) lg2 = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor) * kLog2e;

    const int bpc = L / SB;                  // blocks per chunk
    // chunks 0..nc-2 are full and feed a state; the last one (steps
    // [(nc-1)L, T)) only feeds the final state
    const int ns = nc - 1 + (c_init != nullptr);   // stored states per head
    const int soff = c_init != nullptr;            // slot of the state after chunk kc: kc + soff
    const int nblocks = (nc - 1) * bpc + (c_final ? (T_ - (nc - 1) * L + SB - 1) / SB : 0);

    auto fetch = [&](PF& pf, int b) {
        const int kc = b / bpc;
        const int s0 = b * SB;               // = kc*L + (b%bpc)*SB
        if (GATE == kSig) pf.g = g[bh * nc + kc];
        // rows past the end (partial last chunk) are read clamped and weighted 0
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int idx = tid + NTH * u, r = idx / (TV / VEC), c = (idx % (TV / VEC)) * VEC;
            pf.v[u].load(vb + (size_t)min(s0 + r, T_ - 1) * dhv + v0 + c);
        }
#pragma unroll
        for (int u = 0; u < PF::NK; ++u) {
            const int idx = tid + NTH * u, r = idx / (TC / VEC), c = (idx % (TC / VEC)) * VEC;
            const int s = min(s0 + r, T_ - 1);
            pf.k[u].load(kb + (size_t)s * dqk + c0 + c);
            if (GATE == kSig) {
                pf.a[u] = a[bh * T_ + s];
                pf.li[u] = li[bh * T_ + s];
            }
            if (GATE == kGla) {
                const float* ar = a + (bh * T_ + s) * (size_t)dqk + c0 + c;
                const float* gr = g + (bh * nc + kc) * (size_t)dqk + c0 + c;
                for (int e4 = 0; e4 < VEC / 4; ++e4) {
                    pf.ga[u][e4] = *reinterpret_cast<const f32x4*>(ar + 4 * e4);
                    pf.gg[u][e4] = *reinterpret_cast<const f32x4*>(gr + 4 * e4);
                }
            }
        }
    };
    auto store = [&](PF& pf, int b) {
        const int cs = (b / bpc) * L;
        const int len = min(L, T_ - cs);     // steps in this chunk
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int idx = tid + NTH * u, r = idx / (TV / VEC), c = (idx % (TV / VEC)) * VEC;
            pf.v[u].store(&sm.vs[r][c]);
        }
#pragma unroll
        for (int u = 0; u < PF::NK; ++u) {
            const int idx = tid + NTH * u, r = idx / (TC / VEC), c = (idx % (TC / VEC)) * VEC;
            const int s = b * SB + r;
            const bool live = s < T_;
            float ws = 1.0f;
            if (GATE == kSig) ws = exp2_fast((pf.g - pf.a[u] + pf.li[u]) * kLog2e);
            else if (GATE == kScalar) ws = exp2_fast((float)(len - 1 - (s - cs)) * lg2);
            Vec16<T> kw;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float x = pf.k[u].get(e);
                if (GATE == kGla) x *= exp2_fast((pf.gg[u][e / 4][e % 4] - pf.ga[u][e / 4][e % 4]) * kLog2e);
                else x *= ws;
                kw.set(e, live ? x : 0.0f);
            }
            kw.store(&sm.ks[r][c]);
        }
    };

    // accumulator element r of lane (hh, i32) in tile (mv, mc): value row
    // vw + 32 mv + arow(r), key column cw + 32 mc + i32
    auto arow = [&](int r) { return 8 * (r >> 2) + 4 * hh + (r & 3); };
    auto put_state = [&](const f32x16 (&acc)[MV][MC], int slot) {
#pragma unroll
        for (int mv = 0; mv < MV; ++mv) {
            float* dst = states + ((bh * ns + slot) * (size_t)dhv + v0 + vw + 32 * mv) * dqk + c0 + cw + i32;
#pragma unroll
            for (int mc = 0; mc < MC; ++mc)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[(size_t)arow(r) * dqk + 32 * mc] = acc[mv][mc][r];
        }
    };

    f32x16 acc[MV][MC];
    if (c_init) {
        // C_0 in [d_qk][d_hv]: read once, and stored transposed as the state
        // before chunk 0
        const float* src = c_init + bh * (size_t)dqk * dhv;
#pragma unroll
        for (int mv = 0; mv < MV; ++mv)
            for (int mc = 0; mc < MC; ++mc)
                for (int r = 0; r < 16; ++r)
                    acc[mv][mc][r] = src[(size_t)(c0 + cw + 32 * mc + i32) * dhv + v0 + vw + 32 * mv + arow(r)];
        put_state(acc, 0);
    } else {
#pragma unroll
        for (int mv = 0; mv < MV; ++mv)
            for (int mc = 0; mc < MC; ++mc)
                for (int r = 0; r < 16; ++r) acc[mv][mc][r] = 0.0f;
    }

    // one block: stage it, launch the next block's loads into the freed
    // registers, multiply, and write the state at a chunk end
    PF pf;
    if (nblocks > 0) fetch(pf, 0);
    for (int b = 0; b < nblocks; ++b) {
        const int kc = b / bpc;
        const bool first = (b % bpc) == 0, last = (b % bpc) == bpc - 1 || b == nblocks - 1;
        __syncthreads();
        store(pf, b);
        const float gk = pf.g;                // g of this block's chunk, before the next fetch overwrites it
        __syncthreads();
        if (b + 1 < nblocks) fetch(pf, b + 1);
        if (first) {
            // decay of the carried state across chunk kc (column c of C^T = row c of C)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                float e;
                if (GATE == kSig) e = exp2_fast(gk * kLog2e);
                else if (GATE == kScalar) e = exp2_fast((float)min(L, T_ - kc * L) * lg2);
                else e = exp2_fast(g[(bh * nc + kc) * dqk + c0 + cw + 32 * mc + i32] * kLog2e);
#pragma unroll
                for (int mv = 0; mv < MV; ++mv) acc[mv][mc] *= e;
            }
        }
        // acc (value rows vw.., key columns cw..) += V^T (w.K) over this block
#pragma unroll
        for (int kb16 = 0; kb16 < SB; kb16 += 16) {
            typename Elem<T>::frag af[MV], bf[MC];
#pragma unroll
            for (int mv = 0; mv < MV; ++mv) af[mv] = frag_tr(sm.vs, kb16, vw + 32 * mv, lane);
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) bf[mc] = frag_tr(sm.ks, kb16, cw + 32 * mc, lane);
#pragma unroll
            for (int mv = 0; mv < MV; ++mv)
#pragma unroll
                for (int mc = 0; mc < MC; ++mc) acc[mv][mc] = mma32(af[mv], bf[mc], acc[mv][mc]);
        }
        if (last) {
            if (kc < nc - 1) {
                put_state(acc, kc + soff);
            } else {
                // C_T in [d_qk][d_hv]; each workgroup writes only the tile it read
                // from C_0, so the two may be the same buffer
                float* dst = c_final + bh * (size_t)dqk * dhv;
#pragma unroll
                for (int mv = 0; mv < MV; ++mv)
                    for (int mc = 0; mc < MC; ++mc)
                        for (int r = 0; r < 16; ++r)
                            dst[(size_t)(c0 + cw + 32 * mc + i32) * dhv + v0 + vw + 32 * mv + arow(r)] = acc[mv][mc][r];
            }
        }
    }
}

template <typename T, int SB, int TV, int TC, int NWS>
hipError_t launch_state_cfg(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                            hipStream_t stream)
{
    const int blocks = p.B * p.H * (p.dhv / TV) * (p.dqk / TC);
    const int threads = 64 * NWS;
    switch (p.gate) {
    case kSig:
        state_kernel<T, kSig, SB, TV, TC, NWS><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, ws.states, ws.c0, ws.c_final, p.H, p.T, p.dqk, p.dhv, p.L, p.nc);
        break;
    case kScalar:
        state_kernel<T, kScalar, SB, TV, TC, NWS><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, ws.states, ws.c0, ws.c_final, p.H, p.T, p.dqk, p.dhv, p.L, p.nc);
        break;
    default:
        state_kernel<T, kGla, SB, TV, TC, NWS><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, ws.states, ws.c0, ws.c_final, p.H, p.T, p.dqk, p.dhv, p.L, p.nc);
        break;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_state_t(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                          hipStream_t stream)
{
    if (p.nc < 2 && !ws.c0 && !ws.c_final) return hipSuccess;
    // 128x128 tiles halve the LDS bytes per flop and the L2 re-reads of K and
    // V; use them when they still give every CU a workgroup (bf16 I/O only:
    // fp32 blocks would not fit LDS), else 64x64 tiles for parallelism.  The
    // big tiles run 8 waves over blocks of up to 256 steps (128 KB of loads in
    // flight per workgroup).
    const long big = (long)p.B * p.H * (p.dhv / 128) * (p.dqk / 128);
    int sb_cap = 256;   // TFLA_STATE_SB=64|128 caps the block (tuning sweeps)
    if (const char* e = std::getenv("TFLA_STATE_SB")) sb_cap = std::atoi(e);
    if constexpr (sizeof(T) == 2) {
        if (p.dhv % 128 == 0 && p.dqk % 128 == 0 && big >= 256) {
            if (p.L >= 256 && sb_cap >= 256) return launch_state_cfg<T, 256, 128, 128, 8>(p, k, v, fg, ws, stream);
            if (p.L >= 128 && sb_cap >= 128) return launch_state_cfg<T, 128, 128, 128, 8>(p, k, v, fg, ws, stream);
            return launch_state_cfg<T, 64, 128, 128, 8>(p, k, v, fg, ws, stream);
        }
    }
    if (p.L >= 128) return launch_state_cfg<T, 128, 64, 64, 4>(p, k, v, fg, ws, stream);
    return launch_state_cfg<T, 64, 64, 64, 4>(p, k, v, fg, ws, stream);
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

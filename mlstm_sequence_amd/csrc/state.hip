// state.hip -- inter-chunk state kernel (second kernel of the path).
//
// Materialises the matrix memory at every chunk boundary (the
// "ParallelChunk" form of the flash-linear-attention README: states written
// to global memory for each chunk; the TFLA abstract names this the traffic
// its larger chunks cut):
//   C_k = diag(e^{g_k}) C_{k-1} + sum_{s in chunk k} w_s k_s v_s^T,
//   w_s = e^{g_k - a_s + li_s}    (per key channel c for the GLA gate:
//                                  e^{g_{k,c} - a_{s,c}})
// from C_0 = 0 or a given initial state, in fp32.  The state before chunk k
// (k >= 1, and k = 0 when an initial state is given) is written in the I/O
// type (the intra-chunk kernel's matrix-core operand type, to which it would
// round an fp32 copy anyway: half the bytes for bf16; fp32 on request),
// transposed
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
//
// Few heads and long sequences leave most CUs idle on that serial walk.
// Then the chunk chain is cut into P segments (sequence parallelism on one
// device, the same decomposition that shards a sequence over devices):
//   pass 1: every segment but the last walks its chunks from zero and
//           writes its end state E_p;
//   combine: S_0 = C_0, S_{p+1} = diag(e^{G_p}) S_p + E_p, G_p the segment's
//           summed log forget gate (per key channel for the GLA gate);
//   pass 2: every segment walks its chunks again from its true start S_p
//           and writes the states (and C_T).
// It costs one more read of k and v; the serial part left is P steps of a
// d_qk x d_hv elementwise update.
//
// Reverse walk (REV, for the backward pass): the gradient that flows into
// the state from the chunks after chunk j,
//   D_{j-1} = diag(e^{g_j}) D_j + sum_{t in chunk j} e^{a_t} q_t dh_t^T,
// D_{nc-1} = 0, is the same walk over the chunks in reverse order with
// k := q, v := dh and weights e^{a_t}; D_{j-1} is stored in slot j-1 (the
// intra-chunk kernel's mirrored mode reads slot kc for chunk kc).  Logical
// chunk kl of the walk is chunk nc-1-kl; the partial last chunk comes first.
// Where it stores D_m it also forms the Frobenius product with the forward
// state C_m of the same slot (the gate gradients' boundary coupling), as one
// partial per wavefront: [B*H][nc-1][tiles][waves]; for the per-channel gate
// one per key channel (the row dot of D_m and C_m in that channel),
// [B*H][nc-1][d_qk][value tiles x 2].
#include <algorithm>
#include <cstdlib>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

// What one launch of the state kernel walks and writes.  Grid =
// tiles x heads x nseg, segment slowest.
struct StateWalk {
    const float* init;   // initial states [B*H][nseg_buf][d_qk][d_hv]; NULL: zero
    float* end;          // end states: [B*H][nseg_buf][d_qk][d_hv] (end_all), else
                         // [B*H][d_qk][d_hv] written by the last segment; NULL: none
    int nseg_buf;        // segments per head in the init / end buffers
    int nseg;            // segments in the grid
    int cps;             // chunks per segment
    int nwalk;           // chunks walked in all (nc-1, or nc to reach C_T)
    int put_c0;          // segment 0 stores its initial state as the state before chunk 0
    int end_all;         // every segment writes its end state
    int write_states;    // store the state after every chunk kc < nc-1
    int soff;            // 1 when the stored states start with C_0
    // reverse walk: the forward states its couplings read (slots per head,
    // slot of the state after chunk 0), boundaries per head in xpart, and
    // the factor on the end state it writes
    int cp_slots = 0, cp_off = 0, nbound = 0;
    float end_scale = 1.0f;
};

// Tile of C^T per workgroup: TV value rows x TC key columns; NWS wavefronts
// in a 2 x (NWS/2) grid, each owning a (TV/2) x (2 TC/NWS) piece as 32x32
// accumulators.
template <typename T, int SB, int TV, int TC> struct StateLds {
    // row stride = 16 banks mod 64: the 32 lanes of one transpose-read phase
    // (4 rows x 64 B) land on distinct banks (LDS bank conflicts 37.5% -> 0%
    // by counter; 256-step blocks then fill the 160 KB exactly)
    static constexpr int pad = 64 / sizeof(T);
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

// S: the stored state type (T, or fp32 on request)
template <typename T, int GATE, int SB, int TV, int TC, int NWS, bool REV, typename S>
__global__ __launch_bounds__(64 * NWS) void state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                    const float* __restrict__ a,
                                                    const float* __restrict__ li,
                                                    const float* __restrict__ g,
                                                    const float* __restrict__ fg,
                                                    S* __restrict__ states, StateWalk wk, int H,
                                                    int T_, int dqk, int dhv, int L, int nc,
                                                    const S* __restrict__ cstates,
                                                    float* __restrict__ xpart)
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
    const int nbh = gridDim.x / (tiles * wk.nseg);
    const int tile = blk % tiles;
    const size_t bh = (blk / tiles) % nbh;
    const int seg = blk / (tiles * nbh);
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
    // [(nc-1)L, T)) only feeds the final state.  This workgroup walks the
    // chunks [kbeg, kend) of its segment: blocks [b0, bend).
    const int ns = nc - 1 + wk.soff;                // stored states per head
    // (the buffer's last segment also takes any chunks past P * cps)
    const int kbeg = seg * wk.cps;
    const int kend = seg == wk.nseg_buf - 1 ? wk.nwalk : min(kbeg + wk.cps, wk.nwalk);
    const int b0 = kbeg * bpc;
    const int bend = (REV || kend <= nc - 1) ? kend * bpc
                                             : (nc - 1) * bpc + (T_ - (nc - 1) * L + SB - 1) / SB;
    // chunk of walk position kc
    auto chunk = [&](int kc) { return REV ? nc - 1 - kc : kc; };

    auto fetch = [&](PF& pf, int b) {
        const int kc = chunk(b / bpc);
        const int s0 = kc * L + (b % bpc) * SB;
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
                if (!REV) pf.li[u] = li[bh * T_ + s];
            }
            if (GATE == kGla) {
                const float* ar = a + (bh * T_ + s) * (size_t)dqk + c0 + c;
                const float* gr = g + (bh * nc + kc) * (size_t)dqk + c0 + c;
                for (int e4 = 0; e4 < VEC / 4; ++e4) {
                    pf.ga[u][e4] = *reinterpret_cast<const f32x4*>(ar + 4 * e4);
                    if (!REV) pf.gg[u][e4] = *reinterpret_cast<const f32x4*>(gr + 4 * e4);
                }
            }
        }
    };
    auto store = [&](PF& pf, int b) {
        const int cs = chunk(b / bpc) * L;
        const int len = min(L, T_ - cs);     // steps in this chunk
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int idx = tid + NTH * u, r = idx / (TV / VEC), c = (idx % (TV / VEC)) * VEC;
            pf.v[u].store(&sm.vs[r][c]);
        }
#pragma unroll
        for (int u = 0; u < PF::NK; ++u) {
            const int idx = tid + NTH * u, r = idx / (TC / VEC), c = (idx % (TC / VEC)) * VEC;
            const int s = cs + (b % bpc) * SB + r;
            const bool live = s < T_;
            float ws = 1.0f;
            if (REV) {
                ws = GATE == kSig ? exp2_fast(pf.a[u] * kLog2e) : exp2_fast((float)(s - cs + 1) * lg2);
            } else if (GATE == kSig) {
                ws = exp2_fast((pf.g - pf.a[u] + pf.li[u]) * kLog2e);
            } else if (GATE == kScalar) {
                ws = exp2_fast((float)(len - 1 - (s - cs)) * lg2);
            }
            Vec16<T> kw;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float x = pf.k[u].get(e);
                if (GATE == kGla && REV) x *= exp2_fast(pf.ga[u][e / 4][e % 4] * kLog2e);
                else if (GATE == kGla) x *= exp2_fast((pf.gg[u][e / 4][e % 4] - pf.ga[u][e / 4][e % 4]) * kLog2e);
                else x *= ws;
                kw.set(e, live ? x : 0.0f);
            }
            kw.store(&sm.ks[r][c]);
        }
    };

    // accumulator element r of lane (hh, i32) in tile (mv, mc): value row
    // vw + 32 mv + arow(r), key column cw + 32 mc + i32
    auto arow = [&](int r) { return 8 * (r >> 2) + 4 * hh + (r & 3); };
    // The tile leaves through LDS (the block tiles' space, free between
    // blocks): the waves write their accumulators (lane = key column), then
    // every thread stores 16-byte runs of rows -- a few wide stores per lane
    // instead of MV*MC*16 element stores.  Called by every thread.
    constexpr int SP = 16 / sizeof(S);                 // row pad: 16 bytes
    constexpr bool STAGE = sizeof(S) * TV * (TC + SP) <= sizeof(StateLds<T, SB, TV, TC>);
    static_assert(STAGE || !REV, "the reverse walk's couplings go through the staging area");
    // reverse walk: the forward state's tile in 16-byte pieces, CPN per thread
    constexpr int CEV = 16 / sizeof(S), CPR = TC / CEV, CPN = TV * CPR / NTH;
    static_assert(TV * CPR % NTH == 0, "tile pieces spread evenly over the threads");
    auto put_state = [&](const f32x16 (&acc)[MV][MC], int slot) {
        if constexpr (STAGE) {
            S (*stg)[TC + SP] = reinterpret_cast<S (*)[TC + SP]>(&sm);
            __syncthreads();   // every wave is done reading the block's tiles
#pragma unroll
            for (int mv = 0; mv < MV; ++mv)
#pragma unroll
                for (int mc = 0; mc < MC; ++mc)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        stg[vw + 32 * mv + arow(r)][cw + 32 * mc + i32] = from_float<S>(acc[mv][mc][r]);
            __syncthreads();
            constexpr int EV = 16 / sizeof(S), PR = TC / EV;   // elements per piece, pieces per row
            S* dst = states + ((bh * ns + slot) * (size_t)dhv + v0) * dqk + c0;
#pragma unroll
            for (int c = tid; c < TV * PR; c += NTH) {
                const int rr = c / PR, col = (c % PR) * EV;
                Vec16<S> x;
                x.load(&stg[rr][col]);
                x.store(dst + (size_t)rr * dqk + col);
            }
            // the next block's first barrier orders these reads before LDS is refilled
        } else {
#pragma unroll
            for (int mv = 0; mv < MV; ++mv) {
                S* dst = states + ((bh * ns + slot) * (size_t)dhv + v0 + vw + 32 * mv) * dqk + c0 + cw + i32;
#pragma unroll
                for (int mc = 0; mc < MC; ++mc)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[(size_t)arow(r) * dqk + 32 * mc] = from_float<S>(acc[mv][mc][r]);
            }
        }
    };

    // tile element (acc layout) <-> index in a [d_qk][d_hv] state
    auto nat = [&](int mv, int mc, int r) {
        return (size_t)(c0 + cw + 32 * mc + i32) * dhv + v0 + vw + 32 * mv + arow(r);
    };
    f32x16 acc[MV][MC];
    if (wk.init) {
        // the segment's initial state in [d_qk][d_hv]: read once; segment 0
        // stores the caller's C_0 transposed as the state before chunk 0
        const float* src = wk.init + (bh * wk.nseg_buf + seg) * (size_t)dqk * dhv;
#pragma unroll
        for (int mv = 0; mv < MV; ++mv)
            for (int mc = 0; mc < MC; ++mc)
                for (int r = 0; r < 16; ++r) acc[mv][mc][r] = src[nat(mv, mc, r)];
        // (reverse walk: the final-state gradient, the state of the chunks
        // after the last one, in slot nc-1)
        if (seg == 0 && wk.put_c0) put_state(acc, REV ? nc - 1 : 0);
    } else {
#pragma unroll
        for (int mv = 0; mv < MV; ++mv)
            for (int mc = 0; mc < MC; ++mc)
                for (int r = 0; r < 16; ++r) acc[mv][mc][r] = 0.0f;
    }

    // one block: stage it, launch the next block's loads into the freed
    // registers, multiply, and write the state at a chunk end
    PF pf;
    if (b0 < bend) fetch(pf, b0);
    for (int b = b0; b < bend; ++b) {
        const int kc = b / bpc;               // walk position; chunk(kc) is the chunk
        const bool first = (b % bpc) == 0, last = (b % bpc) == bpc - 1 || b == bend - 1;
        __syncthreads();
        store(pf, b);
        const float gk = pf.g;                // g of this block's chunk, before the next fetch overwrites it
        __syncthreads();
        if (b + 1 < bend) fetch(pf, b + 1);
        if (first) {
            // decay of the carried state across chunk kc (column c of C^T = row c of C)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                float e;
                if (GATE == kSig) e = exp2_fast(gk * kLog2e);
                else if (GATE == kScalar) e = exp2_fast((float)min(L, T_ - chunk(kc) * L) * lg2);
                else e = exp2_fast(g[(bh * nc + chunk(kc)) * dqk + c0 + cw + 32 * mc + i32] * kLog2e);
#pragma unroll
                for (int mv = 0; mv < MV; ++mv) acc[mv][mc] *= e;
            }
        }
        // the forward state of the boundary this block ends (reverse walk):
        // loaded now, used after the block's products
        // (16-byte pieces of rows, as put_state stores them; they reach the
        // accumulator layout through the staging area at the chunk end)
        const bool dot_now = REV && xpart && last && wk.write_states && kc < nc - 1;
        Vec16<S> cvec[CPN];
        if (dot_now) {
            const S* src = cstates + ((bh * wk.cp_slots + (nc - 2 - kc) + wk.cp_off) * (size_t)dhv + v0) * dqk + c0;
#pragma unroll
            for (int j = 0; j < CPN; ++j) {
                const int c = tid + NTH * j, rr = c / CPR, col = (c % CPR) * CEV;
                cvec[j].load(src + (size_t)rr * dqk + col);
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
        if (last && wk.write_states && kc < nc - 1) {
            put_state(acc, REV ? nc - 2 - kc : kc + wk.soff);
            float cpre[MV][MC][16];
            if (dot_now) {
                if constexpr (REV) {
                    S (*stg)[TC + SP] = reinterpret_cast<S (*)[TC + SP]>(&sm);
                    __syncthreads();   // the state's pieces have been read out of the staging area
#pragma unroll
                    for (int j = 0; j < CPN; ++j) {
                        const int c = tid + NTH * j, rr = c / CPR, col = (c % CPR) * CEV;
                        cvec[j].store(&stg[rr][col]);
                    }
                    __syncthreads();
#pragma unroll
                    for (int mv = 0; mv < MV; ++mv)
#pragma unroll
                        for (int mc = 0; mc < MC; ++mc)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                cpre[mv][mc][r] = to_float(stg[vw + 32 * mv + arow(r)][cw + 32 * mc + i32]);
                }
                // the coupling <D_m, C_m> across this chunk boundary: this
                // wave's share, against the forward state stored in the
                // same slot and layout
                const int slot = nc - 2 - kc;
                if constexpr (GATE == kGla) {
                    // per key channel: [B*H][nc-1][d_qk][value tiles x 2 row groups]
                    const int nvp = (dhv / TV) * 2, part = (tile / ntk) * 2 + w / WC;
#pragma unroll
                    for (int mc = 0; mc < MC; ++mc) {
                        float x = 0.0f;
#pragma unroll
                        for (int mv = 0; mv < MV; ++mv)
#pragma unroll
                            for (int r = 0; r < 16; ++r) x += acc[mv][mc][r] * cpre[mv][mc][r];
                        x += __shfl_xor(x, 32, 64);
                        if (hh == 0)
                            xpart[((bh * wk.nbound + slot) * dqk + c0 + cw + 32 * mc + i32) * nvp + part] = x;
                    }
                } else {
                    float x = 0.0f;
#pragma unroll
                    for (int mv = 0; mv < MV; ++mv)
#pragma unroll
                        for (int mc = 0; mc < MC; ++mc)
#pragma unroll
                            for (int r = 0; r < 16; ++r) x += acc[mv][mc][r] * cpre[mv][mc][r];
#pragma unroll
                    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
                    if (lane == 0) xpart[((bh * wk.nbound + slot) * tiles + tile) * NWS + w] = x;
                }
            }
        }
        if (b == bend - 1 && wk.end && (wk.end_all || seg == wk.nseg - 1)) {
            // the state after the walk, in [d_qk][d_hv]; each workgroup writes
            // only the tile it read from its initial state, so the caller's C_0
            // and C_T may be the same buffer
            float* dst = wk.end + (bh * (wk.end_all ? wk.nseg_buf : 1) + (wk.end_all ? seg : 0)) * (size_t)dqk * dhv;
#pragma unroll
            for (int mv = 0; mv < MV; ++mv)
                for (int mc = 0; mc < MC; ++mc)
                    for (int r = 0; r < 16; ++r) dst[nat(mv, mc, r)] = acc[mv][mc][r] * wk.end_scale;
        }
    }
}

// combine pass: start states of the segments from their end states
template <int GATE, bool REV>
__global__ __launch_bounds__(256) void state_combine_kernel(const float* __restrict__ E, float* __restrict__ S,
                                                            const float* __restrict__ c0,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ fg, int H, int T_, int dqk,
                                                            int dhv, int L, int nc, int P, int cps)
{
    const size_t n = (size_t)dqk * dhv;
    const size_t bh = blockIdx.y;
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const int c = (int)(e / dhv);
    float lgam = 0.0f;
    if (GATE == kScalar) lgam = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor);
    float st = c0 ? c0[bh * n + e] : 0.0f;
    S[(bh * P) * n + e] = st;
    constexpr int U = 8;   // segments whose loads are issued together
    for (int p0 = 0; p0 + 1 < P; p0 += U) {
        float ev[U], gv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            ev[u] = 0.0f;
            gv[u] = 0.0f;
            if (p + 1 < P) {
                ev[u] = E[(bh * P + p) * n + e];
                if (GATE == kScalar) {
                    // the reverse walk's first segment holds the partial last chunk
                    const int steps = REV && p == 0 ? (cps - 1) * L + (T_ - (nc - 1) * L) : cps * L;
                    gv[u] = (float)steps * lgam;
                } else {
                    for (int kw = p * cps; kw < (p + 1) * cps; ++kw) {
                        const int kc = REV ? nc - 1 - kw : kw;
                        gv[u] += GATE == kSig ? g[bh * nc + kc] : g[(bh * nc + kc) * dqk + c];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            if (p + 1 < P) {
                st = exp2_fast(gv[u] * kLog2e) * st + ev[u];
                S[(bh * P + p + 1) * n + e] = st;
            }
        }
    }
}

template <typename T, int SB, int TV, int TC, int NWS, bool REV, typename S>
hipError_t launch_walk_s(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                         const StateWalk& wk, hipStream_t stream)
{
    const int blocks = p.B * p.H * (p.dhv / TV) * (p.dqk / TC) * wk.nseg;
    const int threads = 64 * NWS;
    S* st = static_cast<S*>(ws.states);
    const S* cst = static_cast<const S*>(ws.dot_partner);
    switch (p.gate) {
    case kSig:
        state_kernel<T, kSig, SB, TV, TC, NWS, REV, S><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L, p.nc, cst, ws.dots);
        break;
    case kScalar:
        state_kernel<T, kScalar, SB, TV, TC, NWS, REV, S><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L, p.nc, cst, ws.dots);
        break;
    default:
        state_kernel<T, kGla, SB, TV, TC, NWS, REV, S><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L, p.nc, cst, ws.dots);
        break;
    }
    return hipGetLastError();
}

// states in the I/O type, or fp32 on request (forward walk, bf16 I/O)
template <typename T, int SB, int TV, int TC, int NWS, bool REV>
hipError_t launch_walk(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                       const StateWalk& wk, hipStream_t stream)
{
    if constexpr (!REV && sizeof(T) == 2) {
        if (p.st32) return launch_walk_s<T, SB, TV, TC, NWS, REV, float>(p, k, v, fg, ws, wk, stream);
    }
    return launch_walk_s<T, SB, TV, TC, NWS, REV, T>(p, k, v, fg, ws, wk, stream);
}

template <bool REV>
hipError_t launch_combine(const Problem& p, const float* fg, const Workspace& ws, int P, int cps,
                          hipStream_t stream)
{
    const dim3 cgrid((unsigned)((p.dqk * p.dhv + 255) / 256), (unsigned)(p.B * p.H));
    switch (p.gate) {
    case kSig:
        state_combine_kernel<kSig, REV><<<cgrid, 256, 0, stream>>>(ws.seg_end, ws.seg_start, ws.c0, ws.g, fg, p.H,
                                                                   p.T, p.dqk, p.dhv, p.L, p.nc, P, cps);
        break;
    case kScalar:
        state_combine_kernel<kScalar, REV><<<cgrid, 256, 0, stream>>>(ws.seg_end, ws.seg_start, ws.c0, ws.g, fg,
                                                                      p.H, p.T, p.dqk, p.dhv, p.L, p.nc, P, cps);
        break;
    default:
        state_combine_kernel<kGla, REV><<<cgrid, 256, 0, stream>>>(ws.seg_end, ws.seg_start, ws.c0, ws.g, fg,
                                                                     p.H, p.T, p.dqk, p.dhv, p.L, p.nc, P, cps);
        break;
    }
    return hipGetLastError();
}

// the reverse walk's coupling partner and end-state factor, from the workspace
inline void set_rev_fields(StateWalk& wk, const Workspace& ws)
{
    wk.cp_slots = ws.dot_slots;
    wk.cp_off = ws.dot_off;
    wk.nbound = ws.dot_bound;
    wk.end_scale = ws.end_scale;
}

// One configuration: unsegmented walk, or pass 1 + combine + pass 2.
template <typename T, int SB, int TV, int TC, int NWS, bool REV>
hipError_t launch_state_cfg(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                            hipStream_t stream)
{
    const int P = state_segments(p);
    const int soff = ws.c0 != nullptr;
    const int nwalk = p.nc - 1 + (ws.c_final != nullptr);
    if (P <= 1) {
        StateWalk wk{ws.c0, ws.c_final, 1, 1, nwalk > 0 ? nwalk : 1, nwalk, soff, 0, 1, soff};
        set_rev_fields(wk, ws);
        return launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, wk, stream);
    }
    const int cps = state_chunks_per_segment(p, P);
    const StateWalk pass1{nullptr, ws.seg_end, P, P - 1, cps, p.nc - 1, 0, 1, 0, soff};
    hipError_t e = launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, pass1, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_combine<REV>(p, fg, ws, P, cps, stream)) != hipSuccess) return e;
    StateWalk pass2{ws.seg_start, ws.c_final, P, P, cps, nwalk, soff, 0, 1, soff};
    set_rev_fields(pass2, ws);
    return launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, pass2, stream);
}

template <typename T, bool REV>
hipError_t launch_state_t(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                          hipStream_t stream)
{
    if (p.nc < 2 && !ws.c0 && !ws.c_final) return hipSuccess;
    int sb_cap = 256;   // TFLA_STATE_SB=64|128 caps the block (tuning sweeps)
    if (const char* e = std::getenv("TFLA_STATE_SB")) sb_cap = std::atoi(e);
    if constexpr (sizeof(T) == 2) {
        if (state_big_tiles(p)) {
            // 256-step blocks fill the 160 KB of LDS (one workgroup per CU): only
            // when the walk has no more workgroups than the device has CUs;
            // otherwise 128-step blocks let two share a CU
            const long wgs = (long)p.B * p.H * (p.dhv / 128) * (p.dqk / 128) * state_segments(p);
            if (p.L >= 256 && sb_cap >= 256 && wgs <= 256)
                return launch_state_cfg<T, 256, 128, 128, 8, REV>(p, k, v, fg, ws, stream);
            if (p.L >= 128 && sb_cap >= 128)
                return launch_state_cfg<T, 128, 128, 128, 8, REV>(p, k, v, fg, ws, stream);
            return launch_state_cfg<T, 64, 128, 128, 8, REV>(p, k, v, fg, ws, stream);
        }
    }
    if (p.L >= 128) return launch_state_cfg<T, 128, 64, 64, 4, REV>(p, k, v, fg, ws, stream);
    return launch_state_cfg<T, 64, 64, 64, 4, REV>(p, k, v, fg, ws, stream);
}

}  // namespace

// 128x128 tiles halve the LDS bytes per flop and the L2 re-reads of k and v;
// they are used (bf16 I/O only: fp32 blocks would not fit LDS) when they give
// every CU a workgroup -- counting the segments of a segmented walk -- else
// 64x64 tiles.  The big tiles run 8 waves over blocks of up to 256 steps.
bool state_big_tiles(const Problem& p)
{
    if (!p.bf16 || p.dhv % 128 != 0 || p.dqk % 128 != 0) return false;
    const long heads_tiles = (long)p.B * p.H * (p.dhv / 128) * (p.dqk / 128);
    return heads_tiles >= 256 || state_segments_for(p, heads_tiles) > 1;
}

// Segments of the chunk chain: enough workgroups for about two per CU of
// a 256-CU device (512), each segment at least two chunks long; 1 when the
// heads and tiles alone fill the device.  TFLA_STATE_SEGMENTS=n overrides
// (tuning).
int state_segments_for(const Problem& p, long heads_tiles)
{
    const int nfeed = p.nc - 1;   // chunks that feed a stored state
    if (nfeed < 4) return 1;
    long P = 1;
    if (const char* e = std::getenv("TFLA_STATE_SEGMENTS")) P = std::atol(e);
    else if (heads_tiles < 256) P = (512 + heads_tiles - 1) / heads_tiles;
    P = std::min<long>(P, nfeed / 2);
    if (P < 2) return 1;
    const int cps = (int)((nfeed + P - 1) / P);
    return (nfeed + cps - 1) / cps;   // no empty segment
}

int state_dot_parts(const Problem& p)
{
    const bool big = p.bf16 && state_big_tiles(p);
    if (p.gate == kGla) return (p.dhv / (big ? 128 : 64)) * 2;
    if (big) return (p.dhv / 128) * (p.dqk / 128) * 8;
    return (p.dhv / 64) * (p.dqk / 64) * 4;
}

int state_segments(const Problem& p)
{
    const bool big128 = p.bf16 && p.dhv % 128 == 0 && p.dqk % 128 == 0;
    long tiles128 = (long)p.B * p.H * (p.dhv / 128) * (p.dqk / 128);
    if (big128 && (tiles128 >= 256 || state_segments_for(p, tiles128) > 1)) return state_segments_for(p, tiles128);
    return state_segments_for(p, (long)p.B * p.H * (p.dhv / 64) * (p.dqk / 64));
}

int state_chunks_per_segment(const Problem& p, int P)
{
    const int nfeed = p.nc - 1;
    return (nfeed + P - 1) / P;
}

hipError_t launch_state(const Problem& p, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream)
{
    if (p.bf16)
        return launch_state_t<bf16, false>(p, static_cast<const bf16*>(k), static_cast<const bf16*>(v), fgate_pre,
                                           ws, stream);
    return launch_state_t<float, false>(p, static_cast<const float*>(k), static_cast<const float*>(v), fgate_pre,
                                        ws, stream);
}

hipError_t launch_state_rev(const Problem& p, const void* q, const void* dh, const float* fgate_pre,
                            const Workspace& ws, hipStream_t stream)
{
    if (p.bf16)
        return launch_state_t<bf16, true>(p, static_cast<const bf16*>(q), static_cast<const bf16*>(dh), fgate_pre,
                                          ws, stream);
    return launch_state_t<float, true>(p, static_cast<const float*>(q), static_cast<const float*>(dh), fgate_pre,
                                       ws, stream);
}

}  // namespace tfla

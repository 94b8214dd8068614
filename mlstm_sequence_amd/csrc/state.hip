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
// States leave as 128-byte rows.  For the per-channel gate the forward walk
// reads keys the gate kernel has already weighted (the same fp32 expression
// and rounding it would apply), not K and the fp32 gate rows; for mLSTMexp
// it also sums w.K per key channel into the normaliser states.
//
// Few heads and long sequences leave most CUs idle on that serial walk.
// Then the chunk chain is cut into P segments (sequence parallelism on one
// device, the same decomposition that shards a sequence over devices).
// Forward:
//   walk:    every segment walks its chunks once, from zero (segment 0 from
//            C_0), stores the states it reaches and its end state E_p;
//   combine: S_0 = 0, S_{p+1} = diag(e^{G_p}) S_p + E_p, G_p the segment's
//            summed log forget gate (per key channel for the per-channel
//            gate): the true start state of every segment;
//   fix-up:  the state a segment p >= 1 stored after its chunk k becomes
//            state + diag(e^{G_{p,k}}) S_p, G_{p,k} the log forget gate
//            summed from the segment's start through chunk k (and C_T
//            likewise from the last segment's end state).
// K and V cross from memory once; the fix-up reads and writes the stored
// states once more, which for bf16 states is a quarter of the bytes of K and
// V per chunk at d_qk = d_hv.  The serial part left is P steps of a
// d_qk x d_hv elementwise update.  (The stored states are rounded to the
// state type before the fix-up adds the start state: one more rounding than
// a walk from the true start.  The gate gradient of the fixed decay, one
// number per head summed over the couplings of every chunk boundary, feels
// it -- about 2.5x its error at two segments -- so that gate keeps the
// two-pass form below; the per-step and per-channel gate gradients do not
// change.  The forward walk and the backward pass's recomputation of it
// take the same form, so reusing a forward workspace stays bitwise.)
// Reverse (the backward pass's walk), and the forward walk of the fixed
// decay: pass 1 walks every segment but the last from zero for its end
// state, the combine as above (from C_0, or from the final state gradient),
// and pass 2 walks every segment again from its true start and stores the
// states (and couplings).

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
#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"
#include "tfla.h"

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
    // init holds one state per head, read by segment 0 only (the others
    // start from zero)
    int init_first = 0;
    // mLSTMexp, forward walk: the stabilised normaliser state after each
    // chunk k < nc-1, [B*H][nc-1][d_qk], formed beside C (NULL: not)
    float* nst = nullptr;
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
    float gd[4];                  // per-channel gate: g of the block's chunk at the lane's key columns
};

// S: the stored state type (T, or fp32 on request); NORM: mLSTMexp's
// forward walk, which also forms the normaliser states (wk.nst); PREW: the
// per-channel gate's forward walk reading keys the gate kernel has already
// weighted (k points at them; no gate rows are read)
template <typename T, int GATE, int SB, int TV, int TC, int NWS, bool REV, typename S, bool NORM = false,
          bool PREW = false>
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
    static_assert(MC >= 1 && MC <= 4, "tile too narrow for the waves");

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
        if (GATE == kGla) {
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) pf.gd[mc] = g[(bh * nc + kc) * dqk + c0 + cw + 32 * mc + i32];
        }
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
            if (GATE == kGla && !PREW) {
                const float* ar = a + (bh * T_ + s) * (size_t)dqk + c0 + c;
                const float* gr = g + (bh * nc + kc) * (size_t)dqk + c0 + c;
                for (int e4 = 0; e4 < VEC / 4; ++e4) {
                    pf.ga[u][e4] = *reinterpret_cast<const f32x4*>(ar + 4 * e4);
                    if (!REV) pf.gg[u][e4] = *reinterpret_cast<const f32x4*>(gr + 4 * e4);
                }
            }
        }
    };
    // mLSTMexp: n_k = e^{g_k} n_{k-1} + sum_{s in k} w_s k_s with the walk's
    // weights, from the fp32 products w.K before their rounding into LDS:
    // each thread of a first-value-tile workgroup sums its K items (one
    // group of VEC key channels, every NTH-th item) per chunk, decayed like
    // the state; the chunk end adds the threads' sums up per key column.
    static_assert(!NORM || (!REV && GATE == kSig), "the normaliser rides on the forward mLSTMsig walk");
    static_assert(!PREW || (!REV && GATE == kGla), "weighted keys: the per-channel gate's forward walk");
    static_assert(64 % (TC / VEC) == 0, "a thread's K items share one channel group, the lane's");
    static_assert(NTH * VEC * sizeof(float) <= sizeof(StateLds<T, SB, TV, TC>), "the sums fit the staging area");
    const bool norm = NORM && v0 == 0;
    float nrm[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) nrm[e] = 0.0f;
    auto store = [&](PF& pf, int b) {
        const int cs = chunk(b / bpc) * L;
        const int len = min(L, T_ - cs);     // steps in this chunk
        if (norm && b % bpc == 0) {
            const float d = exp2_fast(pf.g * kLog2e);   // the state's decay across this chunk
#pragma unroll
            for (int e = 0; e < VEC; ++e) nrm[e] *= d;
        }
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
                else if (GATE == kGla && !PREW) x *= exp2_fast((pf.gg[u][e / 4][e % 4] - pf.ga[u][e / 4][e % 4]) * kLog2e);
                else if (GATE != kGla) x *= ws;
                kw.set(e, live ? x : 0.0f);
                if (norm) nrm[e] += live ? x : 0.0f;
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
    // An unsegmented walk's states are read again only by the intra kernels,
    // after the walk: they leave with non-temporal stores, so the caches do
    // not hold them dirty into those kernels (T = 8192 workload, L = 256:
    // forward step 0.434 -> 0.431 ms, backward 1.500 -> 1.491 ms; per-channel
    // gate forward 0.253 -> 0.250 ms).  A segmented walk's fix-up reads its
    // states back at once and keeps the plain stores.  The empty asm
    // statements keep the compiler from merging the two stores into one,
    // which would drop the non-temporal hint.
    const bool nt_states = wk.nseg == 1;
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
                if (nt_states) {
                    x.store_nt(dst + (size_t)rr * dqk + col);
                } else {
                    __asm__ volatile("" ::: "memory");
                    x.store(dst + (size_t)rr * dqk + col);
                    __asm__ volatile("" ::: "memory");
                }
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
    if (wk.init && (!wk.init_first || seg == 0)) {
        // the segment's initial state in [d_qk][d_hv]: read once; segment 0
        // stores the caller's C_0 transposed as the state before chunk 0
        const float* src = wk.init_first ? wk.init + bh * (size_t)dqk * dhv
                                         : wk.init + (bh * wk.nseg_buf + seg) * (size_t)dqk * dhv;
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

    // one block: stage it, launch the loads of the block DEPTH places on
    // into the freed registers, multiply, and write the state at a chunk end.
    // The forward walk keeps two blocks' loads in flight (two register sets,
    // used in turn): the loads of block b+1 are still arriving while block b
    // is staged and the loads of b+2 go out, so the CU's memory requests do
    // not drain at every block boundary.  For 128-step blocks: the 256-step
    // ones and the reverse walk's couplings need those registers, and the
    // 64-step blocks ran slower with it (T = 8192 workload, L = 64: state
    // walk 0.316 against 0.303 ms; L = 128: 0.228 against 0.240 ms) --
    // except the per-channel gate's walk over pre-weighted keys, whose
    // 64-step blocks are whole chunks (below).
    // ahead (std::true_type): the block DEPTH places on exists, so its
    // fetch and the walk's last-block work need no run-time test.
    constexpr int DEPTH = !REV && (SB == 128 || PREW) ? 2 : 1;
    auto block = [&](PF& pf, int b, auto ahead) {
        const int kc = b / bpc;               // walk position; chunk(kc) is the chunk
        const bool first = (b % bpc) == 0, last = (b % bpc) == bpc - 1 || b == bend - 1;
        __syncthreads();
        store(pf, b);
        const float gk = pf.g;                // g of this block's chunk, before the next fetch overwrites it
        float gdk[MC];                        // likewise the per-channel gate's g at this lane's key columns
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) gdk[mc] = pf.gd[mc];
        __syncthreads();
        if constexpr (decltype(ahead)::value) fetch(pf, b + DEPTH);
        else if (b + DEPTH < bend) fetch(pf, b + DEPTH);
        if (first) {
            // decay of the carried state across chunk kc (column c of C^T = row c of C)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                float e;
                if (GATE == kSig) e = exp2_fast(gk * kLog2e);
                else if (GATE == kScalar) e = exp2_fast((float)min(L, T_ - chunk(kc) * L) * lg2);
                else e = exp2_fast(gdk[mc] * kLog2e);
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
        // acc (value rows vw.., key columns cw..) += V^T (w.K) over this block.
        // The operands of the next 16 steps are read from LDS (into the other
        // of two fragment sets) before this step's products are issued, so
        // the reads' latency overlaps the matrix work instead of preceding it
        // (T = 8192 workload, L = 256: walk 0.205 -> 0.199 ms)
        {
            typename Elem<T>::frag af[2][MV], bf[2][MC];
            auto frags = [&](int set, int kb16) {
#pragma unroll
                for (int mv = 0; mv < MV; ++mv) af[set][mv] = frag_tr(sm.vs, kb16, vw + 32 * mv, lane);
#pragma unroll
                for (int mc = 0; mc < MC; ++mc) bf[set][mc] = frag_tr(sm.ks, kb16, cw + 32 * mc, lane);
            };
            frags(0, 0);
#pragma unroll
            for (int kb16 = 0; kb16 < SB; kb16 += 16) {
                const int cur = (kb16 / 16) & 1;
                if (kb16 + 16 < SB) frags(cur ^ 1, kb16 + 16);
#pragma unroll
                for (int mv = 0; mv < MV; ++mv)
#pragma unroll
                    for (int mc = 0; mc < MC; ++mc) acc[mv][mc] = mma32(af[cur][mv], bf[cur][mc], acc[mv][mc]);
            }
        }
        if (last && wk.write_states && kc < nc - 1) {
            put_state(acc, REV ? nc - 2 - kc : kc + wk.soff);
            if (norm) {
                // n after this chunk: the threads' partial sums of each key
                // column, added within each wavefront (lanes l, l + NG, ...
                // hold channel group l % NG) and then over the wavefronts
                // through LDS (the staging area is free once every thread
                // has stored its state pieces)
                constexpr int NG = TC / VEC;
                float part[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float x = nrm[e];
#pragma unroll
                    for (int off = NG; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
                    part[e] = x;
                }
                float* red = reinterpret_cast<float*>(&sm);
                __syncthreads();
                if (lane < NG) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) red[(w * NG + lane) * VEC + e] = part[e];
                }
                __syncthreads();
                if (tid < TC) {
                    float sum = 0.0f;
#pragma unroll
                    for (int j = 0; j < NWS; ++j) sum += red[(j * NG + tid / VEC) * VEC + tid % VEC];
                    wk.nst[(bh * (nc - 1) + kc) * (size_t)dqk + c0 + tid] = sum;
                }
                // the next block's first barrier orders these reads before LDS is refilled
            }
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
        if (!decltype(ahead)::value && b == bend - 1 && wk.end && (wk.end_all || seg == wk.nseg - 1)) {
            // the state after the walk, in [d_qk][d_hv]; each workgroup writes
            // only the tile it read from its initial state, so the caller's C_0
            // and C_T may be the same buffer
            float* dst = wk.end + (bh * (wk.end_all ? wk.nseg_buf : 1) + (wk.end_all ? seg : 0)) * (size_t)dqk * dhv;
#pragma unroll
            for (int mv = 0; mv < MV; ++mv)
                for (int mc = 0; mc < MC; ++mc)
                    for (int r = 0; r < 16; ++r) dst[nat(mv, mc, r)] = acc[mv][mc][r] * wk.end_scale;
        }
    };
    const std::true_type ahead;
    const std::false_type check;
    // The memory-counter waits the compiler places before a block's staging
    // follow every path into it: a path on which the other register set was
    // not fetched (a conditional fetch, a skipped block) makes it wait for
    // every load in flight, the other set's too.  The per-channel gate's walk
    // (a state store after every 64-step block) therefore runs a steady loop
    // in which both sets are always fetched, and the last blocks after it;
    // its decay reads g from the prefetched set, not with a load of its own
    // whose wait would drain the other set's loads and the state stores
    // (T = 2048 per-channel workload: walk 0.101 -> 0.075 ms).  On the
    // mLSTMsig walk the same steady loop measured slower (T = 8192, L = 256:
    // 0.202 -> 0.211 ms), so it keeps the plain loop.
    if constexpr (DEPTH == 1) {
        PF pf;
        if (b0 < bend) fetch(pf, b0);
        for (int b = b0; b < bend; ++b) block(pf, b, check);
    } else if constexpr (!PREW) {
        PF pfa, pfb;
        if (b0 < bend) fetch(pfa, b0);
        if (b0 + 1 < bend) fetch(pfb, b0 + 1);
        for (int b = b0; b < bend; b += 2) {
            block(pfa, b, check);
            if (b + 1 < bend) block(pfb, b + 1, check);
        }
    } else {
        PF pfa, pfb;
        if (b0 < bend) {
            fetch(pfa, b0);
            fetch(pfb, min(b0 + 1, bend - 1));
        }
        int b = b0;
        for (; b + 3 < bend; b += 2) {
            block(pfa, b, ahead);
            block(pfb, b + 1, ahead);
        }
        if (b < bend) block(pfa, b, check);
        if (b + 1 < bend) block(pfb, b + 1, check);
        if (b + 2 < bend) block(pfa, b + 2, check);
    }
}

// combine pass: start states of the segments from their end states.  A
// thread owns VE consecutive elements of one row (4-, 8- or 16-byte pieces;
// one key channel, so one gate for the per-channel gate too) and walks the
// segments in order; the end states of 16 segments are loaded together, and
// the gates summed over a segment's chunks are the same for the whole head
// (scalar loads) except for the per-channel gate.  VE is as large as keeps
// 512 or more workgroups: the pass moves few bytes per head and is bound by
// the rate each CU loads at, so it wants every CU busy.
template <int VE>
struct CombineVec {
    float x[VE];
    __device__ __forceinline__ void load(const float* p)
    {
        if constexpr (VE == 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(p);
            for (int j = 0; j < 4; ++j) x[j] = t[j];
        } else if constexpr (VE == 2) {
            const float2 t = *reinterpret_cast<const float2*>(p);
            x[0] = t.x;
            x[1] = t.y;
        } else {
            x[0] = *p;
        }
    }
    __device__ __forceinline__ void store(float* p) const
    {
        if constexpr (VE == 4) *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
        else if constexpr (VE == 2) *reinterpret_cast<float2*>(p) = float2{x[0], x[1]};
        else *p = x[0];
    }
};

template <int GATE, bool REV, int VE>
__global__ __launch_bounds__(256) void state_combine_kernel(const float* __restrict__ E, float* __restrict__ S,
                                                            const float* __restrict__ c0,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ fg, int H, int T_, int dqk,
                                                            int dhv, int L, int nc, int P, int cps)
{
    // segments whose loads are issued together (U x the workgroup's key
    // channels <= 256: up to 5 channels at 4-byte pieces, 16 at 16-byte ones)
    constexpr int U = VE == 1 ? 32 : 16;
    // a batch's segment gate sums, per key channel of the workgroup for the
    // per-channel gate: [segment of the batch][channel]; formed by one thread
    // each (its chunks' loads go out together) instead of by every thread
    // one dependent load at a time
    __shared__ float gs[256];
    const size_t n = (size_t)dqk * dhv;
    const size_t bh = blockIdx.y;
    const size_t eb = (size_t)blockIdx.x * 256 * VE;   // the workgroup's first element
    const size_t e = eb + (size_t)threadIdx.x * VE;
    const bool live = e < n;
    const int c = (int)(min(e, n - 1) / dhv);
    const int clo = (int)(eb / dhv);
    const int nch = GATE == kGla ? (int)((min(eb + 256 * VE, n) - 1) / dhv) - clo + 1 : 1;   // <= 16
    float lgam = 0.0f;
    if (GATE == kScalar) lgam = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor);
    CombineVec<VE> st;
    if (c0 && live) st.load(c0 + bh * n + e);
    else
        for (int j = 0; j < VE; ++j) st.x[j] = 0.0f;
    if (live) st.store(S + (bh * P) * n + e);
    for (int p0 = 0; p0 + 1 < P; p0 += U) {
        // the batch's end states first: their loads are in flight while the
        // gate sums are formed
        CombineVec<VE> ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            for (int j = 0; j < VE; ++j) ev[u].x[j] = 0.0f;
            if (p0 + u + 1 < P && live) ev[u].load(E + (bh * P + p0 + u) * n + e);
        }
        if (GATE != kScalar) {
            const int t = threadIdx.x, p = p0 + t / nch;
            if (t < U * nch && p + 1 < P) {
                // summed from the segment's first chunk on (the fix-up sums
                // the same terms in the same order)
                float sum = 0.0f;
#pragma unroll 8
                for (int kw = p * cps; kw < (p + 1) * cps; ++kw) {
                    const int kc = REV ? nc - 1 - kw : kw;
                    sum += GATE == kSig ? g[bh * nc + kc] : g[(bh * nc + kc) * dqk + clo + t % nch];
                }
                gs[t] = sum;
            }
            __syncthreads();
        }
        float gv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            gv[u] = 0.0f;
            if (p + 1 < P) {
                if (GATE == kScalar) {
                    // the reverse walk's first segment holds the partial last chunk
                    const int steps = REV && p == 0 ? (cps - 1) * L + (T_ - (nc - 1) * L) : cps * L;
                    gv[u] = (float)steps * lgam;
                } else {
                    gv[u] = gs[u * nch + (GATE == kGla ? c - clo : 0)];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            if (p + 1 < P) {
                const float d = exp2_fast(gv[u] * kLog2e);
#pragma unroll
                for (int j = 0; j < VE; ++j) st.x[j] = d * st.x[j] + ev[u].x[j];
                if (live) st.store(S + (bh * P + p + 1) * n + e);
            }
        }
        if (GATE != kScalar) __syncthreads();   // gs is read before the next batch refills it
    }
}

// Fix-up of the forward segmented walk: one workgroup per 64 x 64 tile of
// the state ([d_qk] x [d_hv]), head and segment p >= 1.  The segment's start
// state tile S_p (fp32 [d_qk][d_hv]) is staged in LDS; for each chunk k of
// the segment the stored state (transposed, [d_hv][d_qk], type S) gains
// e^{G_{p,k}} S_p, G_{p,k} the gate summed from the segment's first chunk
// through k in the order the combine kernel sums it; the last segment's end
// state gives C_T the same way.  Thread (v, 16-channel run) for the stored
// states, (c, 16-value run) for C_T.
template <int GATE, typename S>
__global__ __launch_bounds__(256) void state_fixup_kernel(S* __restrict__ states, const float* __restrict__ segs,
                                                          const float* __restrict__ ends, float* __restrict__ cT,
                                                          const float* __restrict__ g, const float* __restrict__ fg,
                                                          int H, int T_, int dqk, int dhv, int L, int nc, int P,
                                                          int cps, int nwalk, int soff)
{
    __shared__ float ss[64][65];                 // S_p tile [channel][value]
    const int ntv = dhv / 64;
    const int c0 = (blockIdx.x / ntv) * 64, v0 = (blockIdx.x % ntv) * 64;
    const size_t bh = blockIdx.y;
    const int p = blockIdx.z + 1;
    const int tid = threadIdx.x;
    const size_t n = (size_t)dqk * dhv;
    const float* sp = segs + (bh * P + p) * n;
    for (int i = tid; i < 64 * 16; i += 256) {   // 16-byte pieces of the tile's rows
        const f32x4 x = *reinterpret_cast<const f32x4*>(sp + (size_t)(c0 + i / 16) * dhv + v0 + 4 * (i % 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) ss[i / 16][4 * (i % 16) + j] = x[j];
    }
    __syncthreads();
    float lgam = 0.0f;
    if (GATE == kScalar) lgam = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor);
    // log forget gate of chunk kc (per head, or per key channel c)
    auto gate = [&](int kc, int c) {
        if (GATE == kSig) return g[bh * nc + kc];
        if (GATE == kScalar) return (float)min(L, T_ - kc * L) * lgam;
        return g[(bh * nc + kc) * (size_t)dqk + c];
    };
    const int kbeg = p * cps, kend = p == P - 1 ? nwalk : min(kbeg + cps, nwalk);
    const int ns = nc - 1 + soff;                // stored states per head
    {
        // stored states: row v of the tile, channels cr .. cr+15; the rows of
        // CG chunks are loaded together
        constexpr int VEC = Elem<S>::vec, NQ = 16 / VEC, CG = 4;
        const int v = tid / 4, cr = (tid % 4) * 16;
        float G[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) G[j] = 0.0f;
        const int klast = min(kend, nc - 1);     // chunks with a stored state
        for (int k0 = kbeg; k0 < klast; k0 += CG) {
            Vec16<S> x[CG][NQ];
#pragma unroll
            for (int u = 0; u < CG; ++u) {
                const int kc = min(k0 + u, klast - 1);
                const S* row = states + ((bh * ns + kc + soff) * (size_t)dhv + v0 + v) * dqk + c0 + cr;
#pragma unroll
                for (int q = 0; q < NQ; ++q) x[u][q].load(row + VEC * q);
            }
#pragma unroll
            for (int u = 0; u < CG; ++u) {
                const int kc = k0 + u;
                if (kc >= klast) break;
                float d[16];
                if (GATE == kGla) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        G[j] += gate(kc, c0 + cr + j);
                        d[j] = exp2_fast(G[j] * kLog2e);
                    }
                } else {
                    G[0] += gate(kc, 0);
                    const float dd = exp2_fast(G[0] * kLog2e);
#pragma unroll
                    for (int j = 0; j < 16; ++j) d[j] = dd;
                }
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    x[u][j / VEC].set(j % VEC, x[u][j / VEC].get(j % VEC) + d[j] * ss[cr + j][v]);
                S* row = states + ((bh * ns + kc + soff) * (size_t)dhv + v0 + v) * dqk + c0 + cr;
#pragma unroll
                for (int q = 0; q < NQ; ++q) x[u][q].store(row + VEC * q);
            }
        }
    }
    if (cT && p == P - 1) {
        // C_T = E_{P-1} + e^{G} S_{P-1}: row c of the tile, values vr .. vr+15
        const int c = tid / 4, vr = (tid % 4) * 16;
        float G = 0.0f;
        for (int kc = kbeg; kc < kend; ++kc) G += gate(kc, c0 + c);
        const float d = exp2_fast(G * kLog2e);
        const float* e = ends + (bh * P + p) * n + (size_t)(c0 + c) * dhv + v0 + vr;
        float* o = cT + bh * n + (size_t)(c0 + c) * dhv + v0 + vr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 x = *reinterpret_cast<const f32x4*>(e + 4 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] += d * ss[c][vr + 4 * q + j];
            *reinterpret_cast<f32x4*>(o + 4 * q) = x;
        }
    }
}

template <int GATE, typename S>
hipError_t launch_fixup_s(const Problem& p, const Workspace& ws, const float* fg, int P, int cps, int nwalk, int soff,
                          hipStream_t stream)
{
    const dim3 grid((unsigned)((p.dqk / 64) * (p.dhv / 64)), (unsigned)(p.B * p.H), (unsigned)(P - 1));
    state_fixup_kernel<GATE, S><<<grid, 256, 0, stream>>>(static_cast<S*>(ws.states), ws.seg_start, ws.seg_end,
                                                          ws.c_final, ws.g, fg, p.H, p.T, p.dqk, p.dhv, p.L, p.nc,
                                                          P, cps, nwalk, soff);
    return hipGetLastError();
}

template <typename S>
hipError_t launch_fixup(const Problem& p, const Workspace& ws, const float* fg, int P, int cps, int nwalk, int soff,
                        hipStream_t stream)
{
    switch (p.gate) {
    case kSig: return launch_fixup_s<kSig, S>(p, ws, fg, P, cps, nwalk, soff, stream);
    case kScalar: return launch_fixup_s<kScalar, S>(p, ws, fg, P, cps, nwalk, soff, stream);
    default: return launch_fixup_s<kGla, S>(p, ws, fg, P, cps, nwalk, soff, stream);
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
        if constexpr (!REV) {
            if (wk.nst) {
                state_kernel<T, kSig, SB, TV, TC, NWS, REV, S, true><<<blocks, threads, 0, stream>>>(
                    k, v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L, p.nc, cst, ws.dots);
                break;
            }
        }
        state_kernel<T, kSig, SB, TV, TC, NWS, REV, S><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L, p.nc, cst, ws.dots);
        break;
    case kScalar:
        state_kernel<T, kScalar, SB, TV, TC, NWS, REV, S><<<blocks, threads, 0, stream>>>(
            k, v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L, p.nc, cst, ws.dots);
        break;
    default:
        if constexpr (!REV) {
            if (ws.kw) {   // keys weighted by the gate kernel
                state_kernel<T, kGla, SB, TV, TC, NWS, REV, S, false, true><<<blocks, threads, 0, stream>>>(
                    static_cast<const T*>(ws.kw), v, ws.a, ws.li, ws.g, fg, st, wk, p.H, p.T, p.dqk, p.dhv, p.L,
                    p.nc, cst, ws.dots);
                break;
            }
        }
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

template <int GATE, bool REV, int VE>
hipError_t launch_combine_ve(const Problem& p, const float* fg, const Workspace& ws, const float* c0, int P, int cps,
                             hipStream_t stream)
{
    const dim3 cgrid((unsigned)((p.dqk * p.dhv / VE + 255) / 256), (unsigned)(p.B * p.H));
    state_combine_kernel<GATE, REV, VE><<<cgrid, 256, 0, stream>>>(ws.seg_end, ws.seg_start, c0, ws.g, fg, p.H, p.T,
                                                                   p.dqk, p.dhv, p.L, p.nc, P, cps);
    return hipGetLastError();
}

template <int GATE, bool REV>
hipError_t launch_combine_g(const Problem& p, const float* fg, const Workspace& ws, const float* c0, int P, int cps,
                            hipStream_t stream)
{
    // d_qk d_hv is a multiple of 4096 (both multiples of 64)
    const long per_head4 = (long)p.dqk * p.dhv / 4 / 256;
    const long heads = (long)p.B * p.H;
    if (per_head4 * heads >= 512) return launch_combine_ve<GATE, REV, 4>(p, fg, ws, c0, P, cps, stream);
    if (2 * per_head4 * heads >= 512) return launch_combine_ve<GATE, REV, 2>(p, fg, ws, c0, P, cps, stream);
    return launch_combine_ve<GATE, REV, 1>(p, fg, ws, c0, P, cps, stream);
}

template <bool REV>
hipError_t launch_combine(const Problem& p, const float* fg, const Workspace& ws, const float* c0, int P, int cps,
                          hipStream_t stream)
{
    switch (p.gate) {
    case kSig: return launch_combine_g<kSig, REV>(p, fg, ws, c0, P, cps, stream);
    case kScalar: return launch_combine_g<kScalar, REV>(p, fg, ws, c0, P, cps, stream);
    default: return launch_combine_g<kGla, REV>(p, fg, ws, c0, P, cps, stream);
    }
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
        if (!REV && p.walk_norm) wk.nst = ws.nst;
        return launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, wk, stream);
    }
    const int cps = state_chunks_per_segment(p, P);
    // (the fixed decay walks twice: its gate gradient, one number per head,
    // sums the couplings of every boundary and feels the fix-up's rounding)
    if (!REV && p.gate != kScalar && knob(TFLA_KNOB_STATE_REWALK) != 1) {
        // one walk of every segment (segment 0 from C_0) storing the states
        // it reaches and every end state, the combine from S_0 = 0, the fix-up
        StateWalk walk{ws.c0, ws.seg_end, P, P, cps, nwalk, soff, 1, 1, soff};
        walk.init_first = 1;
        hipError_t e = launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, walk, stream);
        if (e != hipSuccess) return e;
        if ((e = launch_combine<REV>(p, fg, ws, nullptr, P, cps, stream)) != hipSuccess) return e;
        if (sizeof(T) == 2 && p.st32) return launch_fixup<float>(p, ws, fg, P, cps, nwalk, soff, stream);
        return launch_fixup<T>(p, ws, fg, P, cps, nwalk, soff, stream);
    }
    const StateWalk pass1{nullptr, ws.seg_end, P, P - 1, cps, p.nc - 1, 0, 1, 0, soff};
    hipError_t e = launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, pass1, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_combine<REV>(p, fg, ws, ws.c0, P, cps, stream)) != hipSuccess) return e;
    StateWalk pass2{ws.seg_start, ws.c_final, P, P, cps, nwalk, soff, 0, 1, soff};
    set_rev_fields(pass2, ws);
    return launch_walk<T, SB, TV, TC, NWS, REV>(p, k, v, fg, ws, pass2, stream);
}

template <typename T, bool REV>
hipError_t launch_state_t(const Problem& p, const T* k, const T* v, const float* fg, const Workspace& ws,
                          hipStream_t stream)
{
    if (p.nc < 2 && !ws.c0 && !ws.c_final) return hipSuccess;
    int sb_cap = 256;   // the state-block knob (64 or 128) caps the block (tuning sweeps)
    if (knob(TFLA_KNOB_STATE_SB) > 0) sb_cap = knob(TFLA_KNOB_STATE_SB);
    if constexpr (sizeof(T) == 2) {
        if (state_big_tiles(p)) {
            // reverse walk: 256-step blocks fill the 160 KB of LDS (one
            // workgroup per CU), only when the walk has no more workgroups than
            // the device has CUs; otherwise 128-step blocks let two share a CU.
            // The forward walk takes 128-step blocks with two blocks' loads in
            // flight (T = 8192, L = 256: 0.190-0.203 against 0.199-0.207 ms
            // with 256-step blocks and one, on two devices)
            const long wgs = (long)p.B * p.H * (p.dhv / 128) * (p.dqk / 128) * state_segments(p);
            if constexpr (REV) {
                if (p.L >= 256 && sb_cap >= 256 && wgs <= 256)
                    return launch_state_cfg<T, 256, 128, 128, 8, REV>(p, k, v, fg, ws, stream);
            }
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

// Segments of the chunk chain: enough workgroups for about one per CU of a
// 256-CU device, each segment at least two chunks long; 1 when the heads
// and tiles alone fill the device.  (One per CU rather than two: the
// combine and the fix-up move half the bytes -- 0.261 ms against 0.273 ms
// per forward at 64 segments on the T = 65536, 8-head workload.)  The state-segments knob overrides it (tests
// reach the segmented walk at small sizes with it; tuning).
int state_segments_for(const Problem& p, long heads_tiles)
{
    const int nfeed = p.nc - 1;   // chunks that feed a stored state
    if (nfeed < 4) return 1;
    long P = 1;
    if (knob(TFLA_KNOB_STATE_SEGMENTS) > 0) P = knob(TFLA_KNOB_STATE_SEGMENTS);
    else if (heads_tiles < 256) P = (256 + heads_tiles - 1) / heads_tiles;
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

bool exp_walk_normaliser(const Problem& p) { return p.gate == kExp && state_segments(p) <= 1; }

int state_chunks_per_segment(const Problem& p, int P)
{
    const int nfeed = p.nc - 1;
    return (nfeed + P - 1) / P;
}

hipError_t launch_state(const Problem& pin, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream)
{
    // mLSTMexp: the mLSTMsig walk over its stabilised exponents (gates_exp.hip)
    Problem p = pin;
    if (p.gate == kExp) {
        p.gate = kSig;
        p.walk_norm = exp_walk_normaliser(pin);
    }
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

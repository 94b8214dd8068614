// gates_exp.hip -- the gate work of mLSTMexp: exponential input gate with a
// normaliser state and a max state (the variant mLSTMsig simplifies, TFLA
// research-map summary, Approach), in the chunkwise form of the other
// variants.
//
// With chunk-local sums a_t of log f (as for mLSTMsig) and u_s = igate_pre_s
// - a_s, the log weight of the pair (t, s <= t) inside a chunk is a_t + u_s,
// and that of the carried state C_{k-1} (stabilised by its max state m_{k-1})
// is a_t + m_{k-1}.  Every term of row t is taken relative to
//   mu_t = a_t + M_t,  M_t = max(m_{k-1}, max_{cs <= s <= t} u_s),
// and the states relative to m_k = g_k + max(m_{k-1}, U_k), U_k the chunk's
// largest u (m before the first chunk: U_0, which any later term at least
// equals).  In the exponents the mLSTMsig kernels use, that is
//   a'_t  = m_{k-1} - M_t         (row exponent: inter-chunk term e^{a'_t})
//   li'_s = u_s - M_s             (so the pair exponent a'_t - a'_s + li'_s = u_s - M_t)
//   g'_k  = m_{k-1} - max(m_{k-1}, U_k)   (decay of the carried state)
// all <= 0 where they are used: the state walk and the intra-chunk kernels
// then form the stabilised numerator unchanged.  Added for mLSTMexp:
//   lb_t  = -(a_t + M_t)          (h_t = num_t / max(|den_t|, e^{lb_t}))
//   n_k   = e^{g'_k} n_{k-1} + sum_{s in k} e^{g'_k - a'_s + li'_s} k_s
// the stabilised normaliser before each chunk (the state walk's weights,
// same fp32 expression).  Launches: chunk-local sums and maxima, the
// max-state chain over chunks (one wavefront per head, runs of chunks per
// lane joined by a scan), the per-step exponents.  The normaliser states
// come from the state walk itself when it is not segmented (it forms
// sum_s w_s k_s from the w.K it stages); a segmented walk takes them from
// here: each chunk's normaliser contribution (k read once) and the
// normaliser chain (runs per wavefront).
//
// The input-gate pre-activation is floored at -100 (an input gate below
// e^-100 acts as e^-100), which keeps every maximum finite; the log forget
// gate is floored at -100 as for mLSTMsig.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

constexpr float kLogInputFloor = -100.0f;

// One wavefront per (chunk, head).  Lane j owns E = L/64 consecutive steps:
// serial prefix sum and prefix maximum over its steps, then scans of the lane
// totals across the wavefront.  Writes a (chunk-local sums of log f) to a,
// the prefix maxima of u = igate_pre - a to li, g to g and the chunk maximum
// U to uk.
__global__ __launch_bounds__(64) void gates_exp_local_kernel(const float* __restrict__ ig,
                                                             const float* __restrict__ fg, float* __restrict__ a,
                                                             float* __restrict__ pm, float* __restrict__ g,
                                                             float* __restrict__ uk, int T, int L, int nc)
{
    const int kc = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int lane = threadIdx.x;
    const int t0 = kc * L;
    const int n = min(L, T - t0);
    const int E = L >> 6;
    const size_t base = bh * (size_t)T + t0;
    const float ninf = -__builtin_inff();

    float av[16], uv[16];
    for (int e = 0; e < E; ++e) {
        const int p = min(lane * E + e, n - 1);
        av[e] = fg[base + p];
        uv[e] = ig[base + p];
    }
    float run = 0.0f;
    for (int e = 0; e < E; ++e) {
        float lf = 0.0f;
        if (lane * E + e < n) lf = fmaxf(log_sigmoid(av[e]), kLogForgetFloor);
        run += lf;
        av[e] = run;
    }
    float incl = run;
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    const float excl = incl - run;
    float mx = ninf;
    for (int e = 0; e < E; ++e) {
        av[e] += excl;
        const float u = lane * E + e < n ? fmaxf(uv[e], kLogInputFloor) - av[e] : ninf;
        mx = fmaxf(mx, u);
        uv[e] = mx;
    }
    float mincl = mx;
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(mincl, off, 64);
        if (lane >= off) mincl = fmaxf(mincl, o);
    }
    float mexcl = __shfl_up(mincl, 1, 64);
    if (lane == 0) mexcl = ninf;
    for (int e = 0; e < E; ++e) {
        const int p = lane * E + e;
        if (p < n) {
            a[base + p] = av[e];
            pm[base + p] = fmaxf(uv[e], mexcl);
        }
    }
    const float total = __shfl(incl, 63, 64);
    const float umax = __shfl(mincl, 63, 64);
    if (lane == 0) {
        g[bh * nc + kc] = total;
        uk[bh * nc + kc] = umax;
    }
}

__device__ __forceinline__ float readlane_f(float x, int j)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

// The max-state chain, one wavefront per head: m_k = g_k + max(m_{k-1}, U_k)
// with m before chunk 0 taken as U_0; writes the state entering each chunk.
// Each step is the map x -> max(x + A, B) with A = g_k, B = g_k + U_k, and
// two such maps compose into one of the same form (A_i + A_j,
// max(B_i + A_j, B_j)), so lane j composes the maps of its run of
// consecutive chunks, a shuffle scan over the lanes gives the state
// entering each run, and each lane then steps through its run writing the
// states.  Inside a run each link is the fp32 recurrence the state walk
// implies (its decay g' is formed from the stored m); where a run starts,
// the entering m comes from the composed maps, whose sums of g are
// associated differently: it can differ from a serial walk's by a few ulp,
// which scales the carried state by e^delta against the stabiliser the
// next chunk assumes, |delta| of that size (the normaliser and numerator
// carry the same factor).
__global__ __launch_bounds__(64) void gates_exp_chain_kernel(const float* __restrict__ g,
                                                             const float* __restrict__ uk,
                                                             float* __restrict__ mprev, int nc)
{
    const size_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const int run = (nc + 63) / 64;
    const int k0 = min(lane * run, nc), k1 = min(k0 + run, nc);
    const float* gb = g + bh * nc;
    const float* ub = uk + bh * nc;
    const float ninf = -__builtin_inff();
    // this lane's composed map (identity: A = 0, B = -inf)
    float A = 0.0f, B = ninf;
    for (int k = k0; k < k1; ++k) {
        const float gk = gb[k];
        B = fmaxf(B + gk, ub[k] + gk);
        A += gk;
    }
    // exclusive scan of the maps over the lanes (earlier runs first)
    float eA = A, eB = B;
    for (int off = 1; off < 64; off <<= 1) {
        const float pA = __shfl_up(eA, off, 64), pB = __shfl_up(eB, off, 64);
        if (lane >= off) {
            eB = fmaxf(pB + eA, eB);
            eA = pA + eA;
        }
    }
    // inclusive -> exclusive: the maps of the runs before this lane's
    float xA = __shfl_up(eA, 1, 64), xB = __shfl_up(eB, 1, 64);
    if (lane == 0) {
        xA = 0.0f;
        xB = ninf;
    }
    const float m0 = ub[0];
    float m = fmaxf(m0 + xA, xB);
    for (int k = k0; k < k1; ++k) {
        mprev[bh * nc + k] = m;
        m = gb[k] + fmaxf(m, ub[k]);
    }
}

// Per (chunk, head), 256 threads: the stabilised exponents a', li', lb, g'
// (a and li overwritten in place: each step is read and written by one
// thread), then (npart not NULL: a segmented state walk) the chunk's
// normaliser contribution sum_s w_s k_s with the state walk's weight
// w_s = e^{g' - a'_s + li'_s}: threads own 16-byte column groups of K at
// interleaved steps, summed over the steps through LDS.
template <typename T>
__global__ __launch_bounds__(256) void gates_exp_final_kernel(const float* __restrict__ ig,
                                                              const T* __restrict__ k, float* __restrict__ a,
                                                              float* __restrict__ li, float* __restrict__ lb,
                                                              float* __restrict__ g,
                                                              const float* __restrict__ mprev,
                                                              const float* __restrict__ uk,
                                                              float* __restrict__ npart, int T_, int dqk, int L,
                                                              int nc)
{
    constexpr int NTH = 256, VEC = Elem<T>::vec;
    __shared__ float wsh[1024];
    __shared__ float red[NTH * 8];
    const int kc = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int t0 = kc * L;
    const int n = min(L, T_ - t0);
    const size_t base = bh * (size_t)T_ + t0;
    const float mp = mprev[bh * nc + kc];
    const float Mk = fmaxf(mp, uk[bh * nc + kc]);
    const float gp = mp - Mk;
    for (int p = tid; p < n; p += NTH) {
        const float araw = a[base + p];
        const float M = fmaxf(mp, li[base + p]);
        const float u = fmaxf(ig[base + p], kLogInputFloor) - araw;
        const float ar = mp - M, lip = u - M;
        a[base + p] = ar;
        li[base + p] = lip;
        lb[base + p] = -(araw + M);
        if (npart) wsh[p] = exp2_fast((gp - ar + lip) * kLog2e);
    }
    if (tid == 0) g[bh * nc + kc] = gp;
    if (!npart) return;   // the state walk forms the normaliser states itself
    __syncthreads();
    const int NG = dqk / VEC, NP = NTH / NG;   // column groups, step phases
    const int cg = tid % NG, sp = tid / NG;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    const T* kb = k + base * dqk + cg * VEC;
    for (int p = sp; p < n; p += NP) {
        Vec16<T> x;
        x.load(kb + (size_t)p * dqk);
        const float w = wsh[p];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += w * x.get(e);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[sp * dqk + cg * VEC + e] = acc[e];
    __syncthreads();
    for (int c = tid; c < dqk; c += NTH) {
        float sum = 0.0f;
        for (int j = 0; j < NP; ++j) sum += red[j * dqk + c];
        npart[(bh * nc + kc) * dqk + c] = sum;
    }
}

// The normaliser chain n_k = e^{g'_k} n_{k-1} + npart_k, stored for chunks
// 0..nc-2 (the state before chunk k+1).  A workgroup owns 64 key channels
// of one head (a lane each) and cuts the chain into 16 runs (a wave each):
// every wave composes its run's maps x -> d x + p from zero, the carry into
// each run comes from composing the earlier runs' maps through LDS, and each
// wave then steps through its run from that carry in the state walk's order
// of operations (the first run exactly as a serial walk).
__global__ __launch_bounds__(1024) void gates_exp_norm_kernel(const float* __restrict__ g,
                                                              const float* __restrict__ npart,
                                                              float* __restrict__ nst, int dqk, int nc)
{
    constexpr int W = 16;
    __shared__ float sd[W][64], sp[W][64];
    const size_t bh = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const bool live = c < dqk;
    const int nch = nc - 1;                      // states stored
    const int run = (nch + W - 1) / W;
    const int k0 = min(w * run, nch), k1 = min(k0 + run, nch);
    const float* gb = g + bh * nc;
    const float* pb = npart + bh * nc * (size_t)dqk + (live ? c : 0);
    float D = 1.0f, P = 0.0f;
    for (int k = k0; k < k1; ++k) {
        const float d = exp2_fast(gb[k] * kLog2e);
        P = d * P + pb[(size_t)k * dqk];
        D *= d;
    }
    sd[w][lane] = D;
    sp[w][lane] = P;
    __syncthreads();
    float nv = 0.0f;
    for (int j = 0; j < w; ++j) nv = sd[j][lane] * nv + sp[j][lane];
    if (!live) return;
    float* ob = nst + bh * (size_t)nch * dqk + c;
    for (int k = k0; k < k1; ++k) {
        nv = exp2_fast(gb[k] * kLog2e) * nv + pb[(size_t)k * dqk];
        ob[(size_t)k * dqk] = nv;
    }
}

}  // namespace

hipError_t launch_gates_exp(const Problem& p, const void* k, const float* igate_pre, const float* fgate_pre,
                            const Workspace& ws, hipStream_t stream)
{
    const dim3 grid(p.nc, p.B * p.H);
    // an unsegmented state walk forms the normaliser states beside the
    // numerator states (from the w.K it stages), so k is not read here
    const bool walk_n = exp_walk_normaliser(p);
    float* npart = walk_n ? nullptr : ws.npart;
    gates_exp_local_kernel<<<grid, 64, 0, stream>>>(igate_pre, fgate_pre, ws.a, ws.li, ws.g, ws.uk, p.T, p.L, p.nc);
    gates_exp_chain_kernel<<<p.B * p.H, 64, 0, stream>>>(ws.g, ws.uk, ws.mprev, p.nc);
    if (p.bf16)
        gates_exp_final_kernel<bf16><<<grid, 256, 0, stream>>>(igate_pre, static_cast<const bf16*>(k), ws.a, ws.li,
                                                               ws.lb, ws.g, ws.mprev, ws.uk, npart, p.T, p.dqk,
                                                               p.L, p.nc);
    else
        gates_exp_final_kernel<float><<<grid, 256, 0, stream>>>(igate_pre, static_cast<const float*>(k), ws.a,
                                                                ws.li, ws.lb, ws.g, ws.mprev, ws.uk, npart, p.T,
                                                                p.dqk, p.L, p.nc);
    if (p.nc > 1 && !walk_n) {
        const dim3 ngrid((unsigned)((p.dqk + 63) / 64), (unsigned)(p.B * p.H));
        gates_exp_norm_kernel<<<ngrid, 1024, 0, stream>>>(ws.g, ws.npart, ws.nst, p.dqk, p.nc);
    }
    return hipGetLastError();
}

}  // namespace tfla

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
// same fp32 expression).  Four launches: chunk-local sums and maxima, the
// max-state chain over chunks (one wavefront per head, serial in the
// chunks), the per-step exponents with each chunk's normaliser
// contribution, and the normaliser chain.
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
// Serial in the chunks (a few instructions each); the loads of 64 chunks go
// out together.
__global__ __launch_bounds__(64) void gates_exp_chain_kernel(const float* __restrict__ g,
                                                             const float* __restrict__ uk,
                                                             float* __restrict__ mprev, int nc)
{
    const size_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    float m = 0.0f;
    for (int k0 = 0; k0 < nc; k0 += 64) {
        const int k = k0 + lane;
        const float gk = k < nc ? g[bh * nc + k] : 0.0f;
        const float uv = k < nc ? uk[bh * nc + k] : 0.0f;
        const int cnt = min(64, nc - k0);
        float mine = 0.0f;
        for (int j = 0; j < cnt; ++j) {
            const float gj = readlane_f(gk, j), uj = readlane_f(uv, j);
            if (k0 + j == 0) m = uj;
            if (lane == j) mine = m;
            m = gj + fmaxf(m, uj);
        }
        if (k < nc) mprev[bh * nc + k] = mine;
    }
}

// Per (chunk, head), 256 threads: the stabilised exponents a', li', lb, g'
// (a and li overwritten in place: each step is read and written by one
// thread), then the chunk's normaliser contribution sum_s w_s k_s with the
// state walk's weight w_s = e^{g' - a'_s + li'_s}: threads own 16-byte
// column groups of K at interleaved steps, summed over the steps through LDS.
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
        wsh[p] = exp2_fast((gp - ar + lip) * kLog2e);
    }
    if (tid == 0) g[bh * nc + kc] = gp;
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

// The normaliser chain, one thread per (head, key channel):
// n_k = e^{g'_k} n_{k-1} + npart_k, stored for chunks 0..nc-2 (the state
// before chunk k+1), in the state walk's order of operations.
__global__ __launch_bounds__(256) void gates_exp_norm_kernel(const float* __restrict__ g,
                                                             const float* __restrict__ npart,
                                                             float* __restrict__ nst, int dqk, int nc, long nthreads)
{
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nthreads) return;
    const size_t bh = idx / dqk;
    const int c = (int)(idx % dqk);
    constexpr int U = 8;   // chunks whose loads go out together
    float nv = 0.0f;
    for (int k0 = 0; k0 < nc - 1; k0 += U) {
        float gv[U], pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = min(k0 + u, nc - 2);
            gv[u] = g[bh * nc + kk];
            pv[u] = npart[(bh * nc + kk) * dqk + c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k0 + u < nc - 1) {
                nv = exp2_fast(gv[u] * kLog2e) * nv + pv[u];
                nst[(bh * (nc - 1) + k0 + u) * dqk + c] = nv;
            }
        }
    }
}

}  // namespace

hipError_t launch_gates_exp(const Problem& p, const void* k, const float* igate_pre, const float* fgate_pre,
                            const Workspace& ws, hipStream_t stream)
{
    const dim3 grid(p.nc, p.B * p.H);
    gates_exp_local_kernel<<<grid, 64, 0, stream>>>(igate_pre, fgate_pre, ws.a, ws.li, ws.g, ws.uk, p.T, p.L, p.nc);
    gates_exp_chain_kernel<<<p.B * p.H, 64, 0, stream>>>(ws.g, ws.uk, ws.mprev, p.nc);
    if (p.bf16)
        gates_exp_final_kernel<bf16><<<grid, 256, 0, stream>>>(igate_pre, static_cast<const bf16*>(k), ws.a, ws.li,
                                                               ws.lb, ws.g, ws.mprev, ws.uk, ws.npart, p.T, p.dqk,
                                                               p.L, p.nc);
    else
        gates_exp_final_kernel<float><<<grid, 256, 0, stream>>>(igate_pre, static_cast<const float*>(k), ws.a,
                                                                ws.li, ws.lb, ws.g, ws.mprev, ws.uk, ws.npart, p.T,
                                                                p.dqk, p.L, p.nc);
    if (p.nc > 1) {
        const long n = (long)p.B * p.H * p.dqk;
        gates_exp_norm_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(ws.g, ws.npart, ws.nst, p.dqk, p.nc,
                                                                             n);
    }
    return hipGetLastError();
}

}  // namespace tfla

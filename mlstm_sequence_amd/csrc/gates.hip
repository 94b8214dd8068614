// gates.hip -- log-sigmoid gate prefix sums (first kernel of the path).
//
// For step t of chunk [t0, t0+L) the chunkwise form needs the log of the
// forget-gate product since the chunk start and the log input gate:
//   a_t  = sum_{r=t0..t} log f_r,   li_t = log i_t,   g = a at the chunk end
// (for the per-key-channel gate, a and g are vectors over key channels).
// Sums are chunk-local: the decay between two steps of one chunk is
// exp(a_t - a_s), and exponent arguments stay small even for long sequences.
// The mLSTMsig gates are sigmoids of the pre-activations (TFLA research-map
// summary, Approach); the per-channel gate is logsigmoid(x)/16.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

// One wavefront per (chunk, head).  Lane j owns E = L/64 consecutive steps:
// a serial prefix over its steps, then an exclusive scan of the lane totals
// across the wavefront.
__global__ __launch_bounds__(64) void gates_sig_kernel(const float* __restrict__ ig,
                                                       const float* __restrict__ fg,
                                                       float* __restrict__ a, float* __restrict__ li,
                                                       float* __restrict__ g, int T, int L, int nc)
{
    const int kc = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int lane = threadIdx.x;
    const int t0 = kc * L;
    const int n = min(L, T - t0);
    const int E = L >> 6;                     // L is a multiple of 64, <= 1024
    const size_t base = bh * (size_t)T + t0;

    // both gates' loads go out together (one memory round trip)
    float vals[16], livals[16];
    float run = 0.0f;
    for (int e = 0; e < E; ++e) {
        const int p = min(lane * E + e, n - 1);
        vals[e] = fg[base + p];
        livals[e] = ig[base + p];
    }
    for (int e = 0; e < E; ++e) {
        float lf = 0.0f;
        if (lane * E + e < n) lf = fmaxf(log_sigmoid(vals[e]), kLogForgetFloor);
        run += lf;
        vals[e] = run;
    }
    // exclusive scan of lane totals
    float incl = run;
    for (int off = 1; off < 64; off <<= 1) {
        float o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    const float excl = incl - run;
    for (int e = 0; e < E; ++e) {
        const int p = lane * E + e;
        if (p < n) {
            a[base + p] = vals[e] + excl;
            li[base + p] = log_sigmoid(livals[e]);
        }
    }
    const float total = __shfl(incl, 63, 64);
    if (lane == 0) g[bh * nc + kc] = total;
}

// Per-key-channel gate, one 256-thread workgroup per (chunk, head, run of
// CW key channels).  A thread owns 4 consecutive channels (one 16-byte piece
// of a step's row) and E consecutive steps: its E loads go out together (a
// wavefront's lanes cover whole rows of the workgroup's channels), it forms
// log f for its 4E values and their running sums over its steps, and the
// segment totals of the threads before it on the same channels (through
// LDS) give the chunk-local prefix.  256 threads cover 1024 E / CW steps per
// pass (64 at d_qk = 256 with 128-channel runs and E = 8; 128 at 128, 256 at
// 64 with E = 16); longer chunks take several passes, carrying the running
// total per channel.  log f on the transcendental unit (log_sigmoid_fast):
// with the library calls the evaluations per thread, not the loads, set the
// kernel's time.  Two workgroups per chunk at d_qk = 256 (half the loads in
// flight per thread, twice the workgroups) measured faster than one.
// With kw: the forward state walk's weighted keys k_t o e^{g_k - a_t} as
// well, in the I/O type (the walk's own fp32 expression from the stored a
// and g, and its rounding, so the walk reads them instead of K and the gate
// rows and its states do not change).  A chunk of one pass forms them in
// the pass, once the segment totals give the chunk's total; longer chunks
// read their gate rows back after the passes (each thread the ones it
// wrote).
__device__ __forceinline__ f32x4 load4(const bf16* p)
{
    const bf16x4 t = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <int E, typename T>
__global__ __launch_bounds__(256) void gates_gla_kernel(const float* __restrict__ x,
                                                        float* __restrict__ a, float* __restrict__ g,
                                                        const T* __restrict__ k, T* __restrict__ kw,
                                                        int T_, int dqk, int cw, int L, int nc)
{
    __shared__ f32x4 tot[256];                   // [segment][channel group] totals of a pass
    __shared__ f32x4 carry[64];                  // running total per channel group
    const int runs = dqk / cw;
    const int kc = blockIdx.x / runs, c0 = (blockIdx.x % runs) * cw;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int ncg = cw / 4;                      // channel groups (16-byte pieces per row)
    const int nseg = 256 / ncg;                  // step segments per pass
    const int cg = tid % ncg, seg = tid / ncg;
    const int t0 = kc * L;
    const int n = min(L, T_ - t0);
    const size_t rs = dqk / 4;                   // row stride in 16-byte pieces
    const f32x4* xb = reinterpret_cast<const f32x4*>(x + (bh * (size_t)T_ + t0) * dqk + c0) + cg;
    f32x4* ab = reinterpret_cast<f32x4*>(a + (bh * (size_t)T_ + t0) * dqk + c0) + cg;
    if (tid < ncg) carry[tid] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const size_t rb = (bh * (size_t)T_ + t0) * dqk + c0 + 4 * cg;   // this thread's keys in row 0
    // a chunk of one pass forms the weighted keys in the pass (its total is
    // known once the segment totals are in), longer ones after the passes
    const bool one = kw && n <= nseg * E;
    for (int p0 = 0; p0 < n; p0 += nseg * E) {
        const int s0 = p0 + seg * E;             // this thread's first step
        f32x4 v[E], kv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = xb[(size_t)min(s0 + e, n - 1) * rs];
        if (one) {
#pragma unroll
            for (int e = 0; e < E; ++e) kv[e] = load4(k + rb + (size_t)min(s0 + e, n - 1) * dqk);
        }
        f32x4 run = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < E; ++e) {
            f32x4 lf;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                lf[c] = s0 + e < n ? fmaxf(log_sigmoid_fast(v[e][c]) * (1.0f / 16.0f), kLogForgetFloor) : 0.0f;
            run += lf;
            v[e] = run;
        }
        tot[tid] = run;
        __syncthreads();
        // the totals of the earlier segments of this pass, and the carry
        f32x4 off = carry[cg];
        for (int j = 0; j < seg; ++j) off += tot[j * ncg + cg];
        if (one) {
            // the chunk's total, summed as the last segment's thread forms it
            f32x4 gc = carry[cg];
            for (int j = 0; j < nseg - 1; ++j) gc += tot[j * ncg + cg];
            gc += tot[(nseg - 1) * ncg + cg];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (s0 + e >= n) break;
                const f32x4 av = v[e] + off;
                ab[(size_t)(s0 + e) * rs] = av;
                f32x4 o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = kv[e][c] * exp2_fast((gc[c] - av[c]) * kLog2e);
                store4(kw + rb + (size_t)(s0 + e) * dqk, o[0], o[1], o[2], o[3]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (s0 + e < n) ab[(size_t)(s0 + e) * rs] = v[e] + off;
        }
        __syncthreads();                         // every thread has read carry and tot
        if (seg == nseg - 1) carry[cg] = off + run;
        __syncthreads();
    }
    if (tid < ncg) reinterpret_cast<f32x4*>(g + (bh * nc + kc) * (size_t)dqk + c0)[tid] = carry[tid];
    if (kw && !one) {
        const f32x4 gc = carry[cg];              // the chunk's total, this thread's channels
        for (int p0 = 0; p0 < n; p0 += nseg * E) {
            const int s0 = p0 + seg * E;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (s0 + e >= n) break;
                const f32x4 av = ab[(size_t)(s0 + e) * rs];
                const f32x4 kv = load4(k + rb + (size_t)(s0 + e) * dqk);
                f32x4 o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = kv[c] * exp2_fast((gc[c] - av[c]) * kLog2e);
                store4(kw + rb + (size_t)(s0 + e) * dqk, o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// Fixed per-head decay: a_t = (t - t0 + 1) log(gamma_h) in closed form.
// Only the test hook materialises it; the other kernels evaluate the same
// expression inline.
__global__ void gates_scalar_kernel(const float* __restrict__ fg, float* __restrict__ a,
                                    float* __restrict__ li, float* __restrict__ g, int H, int T,
                                    int L, int nc)
{
    const size_t bh = blockIdx.y;
    const float lgam = fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor);
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        const int p = t % L;
        a[bh * T + t] = (float)(p + 1) * lgam;
        li[bh * T + t] = 0.0f;
        if (p == L - 1 || t == T - 1) g[bh * nc + t / L] = (float)(p + 1) * lgam;
    }
}

}  // namespace

template <typename T>
void launch_gla(const Problem& p, const T* k, const float* fgate_pre, const Workspace& ws, hipStream_t stream)
{
    T* kw = k ? static_cast<T*>(ws.kw) : nullptr;
    if (p.dqk == 256) {
        const dim3 g2(p.nc * 2, p.B * p.H);
        gates_gla_kernel<8, T><<<g2, 256, 0, stream>>>(fgate_pre, ws.a, ws.g, k, kw, p.T, p.dqk, 128, p.L, p.nc);
    } else {
        const dim3 grid(p.nc, p.B * p.H);
        gates_gla_kernel<16, T><<<grid, 256, 0, stream>>>(fgate_pre, ws.a, ws.g, k, kw, p.T, p.dqk, p.dqk, p.L,
                                                          p.nc);
    }
}

hipError_t launch_gates(const Problem& p, const void* k, const float* igate_pre, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream)
{
    const dim3 grid(p.nc, p.B * p.H);
    if (p.gate == kSig) {
        gates_sig_kernel<<<grid, 64, 0, stream>>>(igate_pre, fgate_pre, ws.a, ws.li, ws.g, p.T, p.L, p.nc);
    } else if (p.gate == kGla) {
        if (p.bf16) launch_gla<bf16>(p, static_cast<const bf16*>(k), fgate_pre, ws, stream);
        else launch_gla<float>(p, static_cast<const float*>(k), fgate_pre, ws, stream);
    } else {
        return hipSuccess;   // closed form, evaluated inside the consumers
    }
    return hipGetLastError();
}

hipError_t launch_gates_closed_form(const Problem& p, const float* fgate_pre, float* a, float* li,
                                    float* g, hipStream_t stream)
{
    const dim3 grid((p.T + 255) / 256, p.B * p.H);
    gates_scalar_kernel<<<grid, 256, 0, stream>>>(fgate_pre, a, li, g, p.H, p.T, p.L, p.nc);
    return hipGetLastError();
}

}  // namespace tfla

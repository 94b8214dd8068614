// grad.hip -- the gate work of the backward pass.
//
// Gradients of the loss L through h_t = C_t^T q_t / sqrt(d_qk) with
// C_t = f_t C_{t-1} + i_t k_t v_t^T (the recurrence of the mLSTMsig and
// scalar-decay variants).  The matrix products (dq, dk, dv) run in the
// intra-chunk kernel's gradient modes; this file holds what is left:
//
//   mirrored gates:  for chunk rows visited in reverse (logical row cs + r
//                    is step p = cs + len - 1 - r), the query-side exponent
//                    a'_t = g - a_p + li_p and the key-side exponent
//                    li'_t - a'_t = a_p - g (stored pre-combined, so an input
//                    gate of 0 never meets -inf - -inf).
//   gate gradients:  log f_t enters every state from C_t on, and a direct
//                    calculation gives
//                       dL/dlog f_t = sum_{t' >= t} (q_t' . dq_t' - k_t' . dk_t'),
//                       dL/dlog i_t = k_t . dk_t.
//                    r_t = q_t.dq_t - k_t.dk_t and k_t.dk_t come from the dq
//                    and dk kernels' fp32 row partials (one per value tile).
//                    The suffix sum is split at the chunk end: the part of it
//                    past chunk k's last step equals the coupling carried
//                    across that boundary,
//                       X_k = <D_k, C_k> / sqrt(d_qk)   (X_{nc-1} = 0),
//                    the Frobenius product of the two fp32 states the path
//                    materialises (every pair s <= end of chunk k < t
//                    contributes once to it; the reverse state walk forms it
//                    in partials where it stores D_k), so
//                       dL/dlog f_t = sum_{t <= t' in chunk k} r_t' + X_k
//                    and no error accumulates over the sequence.  The fixed
//                    per-head decay shares one log f over every step; with
//                    sum_t r_t = 0 (scaling q by e^e and k by e^-e leaves h
//                    unchanged) the same split gives
//                       dL/dlog f = sum_t (t - cs_t - (L-1)/2) r_t + L sum_k X_k
//                    summed over batches: chunk-centred weights of at most L/2
//                    instead of weights up to T on two sums that nearly
//                    cancel.  Through the sigmoids: dig = (k.dk)(1 - i),
//                    dfg = dL/dlog f (1 - f), 0 where the log forget gate
//                    sits at its floor.
//                    Per-channel gate: every quantity above per key channel c,
//                    r_{t,c} = q_{t,c} dq_{t,c} - k_{t,c} dk_{t,c} (from the dq and dk
//                    kernels' fp32 per-element products), X_{k,c} the row dot
//                    of D_k and C_k in channel c, and d log f / dx = (1 - sigmoid(x))/16.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

constexpr int kScanThreads = 256;

__global__ __launch_bounds__(256) void gates_mirror_kernel(const float* __restrict__ a, const float* __restrict__ li,
                                                          const float* __restrict__ g, float* __restrict__ ar,
                                                          float* __restrict__ lr, int T_, int L, int nc)
{
    const size_t bh = blockIdx.y;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T_) return;
    const int kc = t / L, cs = kc * L, len = min(L, T_ - cs);
    const int p = 2 * cs + len - 1 - t;
    const float gk = g[bh * nc + kc];
    const float ap = a[bh * T_ + p];
    ar[bh * T_ + t] = gk - ap + li[bh * T_ + p];
    lr[bh * T_ + t] = ap - gk;
}

// per-channel gate, mirrored chunks: a'_{t,c} = g_{k,c} - a_{p,c}
__global__ __launch_bounds__(256) void gates_mirror_gla_kernel(const float* __restrict__ a,
                                                              const float* __restrict__ g, float* __restrict__ ar,
                                                              int T_, int L, int nc, int dqk)
{
    // four consecutive channels per thread (d_qk is a multiple of 64)
    const size_t bh = blockIdx.y;
    const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int t = (int)(idx / dqk), c = (int)(idx % dqk);
    if (t >= T_) return;
    const int kc = t / L, cs = kc * L, len = min(L, T_ - cs);
    const int p = 2 * cs + len - 1 - t;
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + (bh * nc + kc) * dqk + c);
    const f32x4 av = *reinterpret_cast<const f32x4*>(a + (bh * T_ + p) * dqk + c);
    *reinterpret_cast<f32x4*>(ar + (bh * T_ + t) * dqk + c) = gv - av;
}

// r_t and k_t.dk_t from the per-tile partial dots of step t
__device__ __forceinline__ void step_dots(const float* dq_dots, const float* dk_dots, size_t t, int np, double& r,
                                          double& kd)
{
    double a = 0.0, b = 0.0;
    for (int j = 0; j < np; ++j) {
        a += dq_dots[t * np + j];
        b += dk_dots[t * np + j];
    }
    r = a - b;
    kd = b;
}

// X_k = scale <D_k, C_k> from the reverse walk's nx partials of boundary k
__device__ __forceinline__ double coupling(const float* xpart, size_t k, int nx, float scale)
{
    double x = 0.0;
    for (int j = 0; j < nx; ++j) x += xpart[k * nx + j];
    return x * scale;
}

// mLSTMsig: one workgroup per (batch-head, chunk); thread i owns steps
// [cs + i n, cs + (i+1) n) of the chunk.  Sums are kept in double.
__global__ __launch_bounds__(kScanThreads) void grad_scan_sig_kernel(const float* __restrict__ dq_dots,
                                                                    const float* __restrict__ dk_dots, int np,
                                                                    const float* __restrict__ xpart, int nx,
                                                                    float scale, const float* __restrict__ ig,
                                                                    const float* __restrict__ fg,
                                                                    float* __restrict__ dig, float* __restrict__ dfg,
                                                                    int T_, int L, int nc, int nbound)
{
    __shared__ double part[2][kScanThreads];
    const int kc = blockIdx.x % nc;
    const size_t bh = blockIdx.x / nc;
    const size_t base = bh * T_;
    const int cs = kc * L, ce = min(cs + L, T_);
    const int tid = threadIdx.x;
    const int n = (L + kScanThreads - 1) / kScanThreads;
    const int t0 = min(cs + tid * n, ce), t1 = min(t0 + n, ce);
    double s = 0.0, r, kd;
    for (int t = t0; t < t1; ++t) {
        step_dots(dq_dots, dk_dots, base + t, np, r, kd);
        s += r;
    }
    // suffix sums over the threads after this one (Hillis-Steele, reversed)
    int cur = 0;
    part[cur][tid] = s;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
        const double x = part[cur][tid] + (tid + d < kScanThreads ? part[cur][tid + d] : 0.0);
        part[cur ^ 1][tid] = x;
        cur ^= 1;
        __syncthreads();
    }
    // sum over the steps of the chunk after t1, plus the coupling past it
    double acc = part[cur][tid] - s + (kc < nbound ? coupling(xpart, bh * nbound + kc, nx, scale) : 0.0);
    for (int t = t1 - 1; t >= t0; --t) {
        step_dots(dq_dots, dk_dots, base + t, np, r, kd);
        acc += r;
        const float x = fg[base + t];
        const bool floored = log_sigmoid(x) < kLogForgetFloor;
        dfg[base + t] = floored ? 0.0f : (float)(acc / (1.0 + exp((double)x)));
        dig[base + t] = (float)(kd / (1.0 + exp((double)ig[base + t])));
    }
}

// Per-channel gate: one workgroup per (batch-head, chunk), one thread per key
// channel walking the chunk backwards from its boundary coupling.
__global__ __launch_bounds__(256) void grad_gla_kernel(const float* __restrict__ dq_prod,
                                                      const float* __restrict__ dk_prod,
                                                      const float* __restrict__ xpart, int nx, float scale,
                                                      const float* __restrict__ fg, float* __restrict__ dfg,
                                                      int T_, int L, int nc, int dqk, int nbound)
{
    const int kc = blockIdx.x % nc;
    const size_t bh = blockIdx.x / nc;
    const int c = threadIdx.x;
    if (c >= dqk) return;
    const int cs = kc * L, ce = min(cs + L, T_);
    double acc = 0.0;
    if (kc < nbound) {
        const float* xp = xpart + ((bh * nbound + kc) * dqk + c) * nx;
        for (int j = 0; j < nx; ++j) acc += xp[j];
        acc *= scale;
    }
    // the running sum in double; the factor d log f / dx = sigmoid(-x) / 16
    // in fp32 (full relative precision); loads of U steps issued together
    constexpr int U = 8;
    for (int t1 = ce; t1 > cs; t1 -= U) {
        float dqv[U], dkv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t o = (bh * T_ + max(t1 - 1 - u, cs)) * dqk + c;
            dqv[u] = dq_prod[o];
            dkv[u] = dk_prod[o];
            xv[u] = fg[o];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t1 - 1 - u;
            if (t < cs) break;
            acc += (double)dqv[u] - (double)dkv[u];
            const float x = xv[u];
            const bool floored = log_sigmoid(x) * (1.0f / 16.0f) < kLogForgetFloor;
            const float f = 1.0f / (16.0f * (1.0f + expf(x)));
            dfg[(bh * T_ + t) * dqk + c] = floored ? 0.0f : (float)(acc * (double)f);
        }
    }
}

// Fixed per-head decay: one workgroup per (batch, head) sums its part of
// dL/dlog gamma in double; a second kernel adds the batches of each head in
// a fixed order.  Every step of chunk k adds sum_{t <= t' in k} r_t' + X_k,
// i.e. sum_t (t - cs_t + 1) r_t + sum_k len_k X_k; without an initial state
// or a final-state gradient sum_t r_t = 0 and the weights are centred on
// the chunk (centred = 1).
__global__ __launch_bounds__(kScanThreads) void grad_scalar_kernel(const float* __restrict__ dq_dots,
                                                                  const float* __restrict__ dk_dots, int np,
                                                                  const float* __restrict__ xpart, int nx,
                                                                  float scale, double* __restrict__ part_out,
                                                                  int T_, int L, int nc, int nbound, int centred)
{
    __shared__ double part[kScanThreads];
    const size_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const double centre = centred ? 0.5 * (L - 1) : -1.0;
    double s = 0.0, r, kd;
    for (int t = tid; t < T_; t += kScanThreads) {
        step_dots(dq_dots, dk_dots, bh * T_ + t, np, r, kd);
        s += ((double)(t % L) - centre) * r;
    }
    for (int k = tid; k < nbound; k += kScanThreads)
        s += (double)min(L, T_ - k * L) * coupling(xpart, bh * nbound + k, nx, scale);
    part[tid] = s;
    __syncthreads();
    for (int d = kScanThreads / 2; d >= 1; d >>= 1) {
        if (tid < d) part[tid] += part[tid + d];
        __syncthreads();
    }
    if (tid == 0) part_out[bh] = part[0];
}

__global__ __launch_bounds__(64) void grad_scalar_final_kernel(const double* __restrict__ part,
                                                              const float* __restrict__ fg,
                                                              float* __restrict__ dfg, int B, int H)
{
    const int h = blockIdx.x * 64 + threadIdx.x;
    if (h >= H) return;
    double s = 0.0;
    for (int b = 0; b < B; ++b) s += part[(size_t)b * H + h];
    const float x = fg[h];
    const bool floored = log_sigmoid(x) < kLogForgetFloor;
    dfg[h] = floored ? 0.0f : (float)(s / (1.0 + exp((double)x)));
}

// y = a x over n floats
__global__ __launch_bounds__(256) void scale_copy_kernel(const float* __restrict__ x, float* __restrict__ y, size_t n,
                                                         float a)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = a * x[i];
}

// Coupling across the end of the sequence: the Frobenius product of the
// final-state gradient (given as dC_T sqrt(d_qk), the reverse walk's
// scaling) and C_T, both [d_qk][d_hv], over the whole state (per head) or
// over one key channel's row (per-channel gate: one workgroup per row).  It
// is stored as partial 0 of boundary nbound-1, the other partials zero.
__global__ __launch_bounds__(256) void final_coupling_kernel(const float* __restrict__ g, const float* __restrict__ c,
                                                            float* __restrict__ xpart, int nx, int nbound, int dqk,
                                                            int dhv, int per_channel)
{
    __shared__ double part[256];
    const int rows = per_channel ? 1 : dqk;   // rows of the state per workgroup
    const size_t bh = per_channel ? blockIdx.x / dqk : blockIdx.x;
    const int ch = per_channel ? blockIdx.x % dqk : 0;
    const size_t base = (bh * dqk + ch) * (size_t)dhv;
    const size_t n = (size_t)rows * dhv;
    double s = 0.0;
    for (size_t i = threadIdx.x; i < n; i += 256) s += (double)g[base + i] * c[base + i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int d = 128; d >= 1; d >>= 1) {
        if (threadIdx.x < d) part[threadIdx.x] += part[threadIdx.x + d];
        __syncthreads();
    }
    float* dst = per_channel ? xpart + ((bh * nbound + nbound - 1) * dqk + ch) * nx
                             : xpart + (bh * nbound + nbound - 1) * nx;
    for (int j = threadIdx.x; j < nx; j += 256) dst[j] = j == 0 ? (float)part[0] : 0.0f;
}

}  // namespace

hipError_t launch_gates_mirror(const Problem& p, const Workspace& ws, float* ar, float* lr, hipStream_t stream)
{
    if (p.gate == kGla) {
        const dim3 grid((unsigned)(((size_t)p.T * p.dqk / 4 + 255) / 256), (unsigned)(p.B * p.H));
        gates_mirror_gla_kernel<<<grid, 256, 0, stream>>>(ws.a, ws.g, ar, p.T, p.L, p.nc, p.dqk);
    } else {
        const dim3 grid((unsigned)((p.T + 255) / 256), (unsigned)(p.B * p.H));
        gates_mirror_kernel<<<grid, 256, 0, stream>>>(ws.a, ws.li, ws.g, ar, lr, p.T, p.L, p.nc);
    }
    return hipGetLastError();
}

hipError_t launch_scale_copy(const float* x, float* y, size_t n, float a, hipStream_t stream)
{
    scale_copy_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(x, y, n, a);
    return hipGetLastError();
}

hipError_t launch_final_coupling(const Problem& p, const float* g_scaled, const float* c_final, float* xpart, int nx,
                                 int nbound, hipStream_t stream)
{
    const bool per_channel = p.gate == kGla;
    const unsigned blocks = (unsigned)(p.B * p.H * (per_channel ? p.dqk : 1));
    final_coupling_kernel<<<blocks, 256, 0, stream>>>(g_scaled, c_final, xpart, nx, nbound, p.dqk, p.dhv, per_channel);
    return hipGetLastError();
}

hipError_t launch_gate_grads(const Problem& p, const float* xpart, int nx, int nbound, bool with_states,
                             const float* dq_dots, const float* dk_dots, int np, const float* igate_pre,
                             const float* fgate_pre, float* dig, float* dfg, double* head_part, hipStream_t stream)
{
    const float scale = 1.0f / sqrtf((float)p.dqk);
    if (p.gate == kGla)
        grad_gla_kernel<<<p.B * p.H * p.nc, 256, 0, stream>>>(dq_dots, dk_dots, xpart, nx, scale, fgate_pre, dfg, p.T,
                                                              p.L, p.nc, p.dqk, nbound);
    else if (p.gate == kSig)
        grad_scan_sig_kernel<<<p.B * p.H * p.nc, kScanThreads, 0, stream>>>(
            dq_dots, dk_dots, np, xpart, nx, scale, igate_pre, fgate_pre, dig, dfg, p.T, p.L, p.nc, nbound);
    else {
        grad_scalar_kernel<<<p.B * p.H, kScanThreads, 0, stream>>>(dq_dots, dk_dots, np, xpart, nx, scale,
                                                                   head_part, p.T, p.L, p.nc, nbound, !with_states);
        grad_scalar_final_kernel<<<(p.H + 63) / 64, 64, 0, stream>>>(head_part, fgate_pre, dfg, p.B, p.H);
    }
    return hipGetLastError();
}

}  // namespace tfla

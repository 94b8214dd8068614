// recurrent.hip -- fused recurrent kernel: the step-by-step form of the
// recurrence (the O(T) "FusedRecurrent" form in the flash-linear-attention
// README's list of computation forms), for decoding and short continuations
// from a carried state.
//
//   C_t = diag(f_t) C_{t-1} + i_t k_t v_t^T,   h_t = C_t^T q_t / sqrt(d_qk)
//
// One workgroup (4 wavefronts) owns all d_qk rows x 32 value columns of one
// head's state and keeps them in fp32 registers for the whole call: lane j
// holds value column v0 + (j mod 32), and the half-wave j / 32 of wave w
// holds key rows p R .. p R + R - 1 with p = 2 w + j / 32 (R = d_qk / 8).
// Each half-wave reads and writes 128 contiguous bytes of a state row, and
// the 32-column split gives twice the workgroups of a 64-column one (the
// step is bound by moving the state, and more workgroups keep more of it in
// flight).  Steps run in batches of kSteps: the batch's q and k (as fp32),
// gates and v columns are staged in LDS once, every step updates the
// thread's state rows and forms its partial dot product with q, and the
// eight row parts meet in LDS and are summed in a fixed order, so results
// are deterministic.  The state is read once at the start and written back
// once at the end, by the same thread, so it is updated in place.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

constexpr int kSteps = 16;   // steps staged per batch

template <typename T, int GATE, int DQK>
__global__ __launch_bounds__(256) void recurrent_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, const float* __restrict__ ig,
                                                        const float* __restrict__ fg, float* __restrict__ state,
                                                        T* __restrict__ h, int H, int T_, int dhv, float scale)
{
    constexpr int S = kSteps, R = DQK / 8;
    constexpr int GW = GATE == kGla ? DQK : 1;
    __shared__ float qs[S][DQK], ks[S][DQK];
    __shared__ float fs[S][GW];          // per-channel forget gates (GLA)
    __shared__ float vs[S][32];
    __shared__ float gi[S], gf[S];       // mLSTMsig input / forget gate of each step
    __shared__ float part[S][8][32];     // partial outputs of the eight row parts

    const int nvt = dhv / 32;
    const size_t bh = blockIdx.x / nvt;
    const int v0 = (blockIdx.x % nvt) * 32;
    const int tid = threadIdx.x, col = tid & 31, part_id = tid >> 5;   // part_id = 2 w + half-wave

    float* cb = state + bh * (size_t)DQK * dhv + v0 + col;   // column v0 + col of C [d_qk][d_hv]
    float c[R];
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] = cb[(size_t)(part_id * R + r) * dhv];

    float gam = 1.0f;   // fixed decay
    if (GATE == kScalar) gam = exp2_fast(fmaxf(log_sigmoid(fg[bh % H]), kLogForgetFloor) * kLog2e);

    for (int t0 = 0; t0 < T_; t0 += S) {
        const int n = min(S, T_ - t0);
        __syncthreads();   // the previous batch is done with LDS
        for (int idx = tid; idx < S * DQK; idx += 256) {
            const int s = idx / DQK, cc = idx % DQK;
            const size_t row = bh * T_ + min(t0 + s, T_ - 1);
            qs[s][cc] = to_float(q[row * DQK + cc]);
            ks[s][cc] = to_float(k[row * DQK + cc]);
            if (GATE == kGla)
                fs[s][cc % GW] =
                    exp2_fast(fmaxf(log_sigmoid(fg[row * DQK + cc]) * (1.0f / 16.0f), kLogForgetFloor) * kLog2e);
        }
        for (int idx = tid; idx < S * 32; idx += 256) {
            const int s = idx / 32, j = idx % 32;
            const size_t row = bh * T_ + min(t0 + s, T_ - 1);
            vs[s][j] = to_float(v[row * dhv + v0 + j]);
        }
        if (GATE == kSig && tid < S) {
            const size_t row = bh * T_ + min(t0 + tid, T_ - 1);
            gi[tid] = exp2_fast(log_sigmoid(ig[row]) * kLog2e);
            gf[tid] = exp2_fast(fmaxf(log_sigmoid(fg[row]), kLogForgetFloor) * kLog2e);
        }
        __syncthreads();
        for (int s = 0; s < n; ++s) {
            float f = gam, iv = vs[s][col];
            if (GATE == kSig) {
                f = gf[s];
                iv *= gi[s];
            }
            float o = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int cc = part_id * R + r;
                const float fc = GATE == kGla ? fs[s][cc % GW] : f;
                c[r] = fc * c[r] + ks[s][cc] * iv;
                o += c[r] * qs[s][cc];
            }
            part[s][part_id][col] = o;
        }
        __syncthreads();
        for (int idx = tid; idx < n * 32; idx += 256) {
            const int s = idx / 32, j = idx % 32;
            const float o = ((part[s][0][j] + part[s][1][j]) + (part[s][2][j] + part[s][3][j])) +
                            ((part[s][4][j] + part[s][5][j]) + (part[s][6][j] + part[s][7][j]));
            h[(bh * T_ + t0 + s) * dhv + v0 + j] = from_float<T>(o * scale);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) cb[(size_t)(part_id * R + r) * dhv] = c[r];
}

template <typename T, int GATE>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v, const float* ig,
                    const float* fg, float* state, void* h, hipStream_t stream)
{
    const int blocks = p.B * p.H * (p.dhv / 32);
    const float scale = 1.0f / sqrtf((float)p.dqk);
    const T* qt = static_cast<const T*>(q);
    const T* kt = static_cast<const T*>(k);
    const T* vt = static_cast<const T*>(v);
    T* ht = static_cast<T*>(h);
    switch (p.dqk) {
    case 64:
        recurrent_kernel<T, GATE, 64><<<blocks, 256, 0, stream>>>(qt, kt, vt, ig, fg, state, ht, p.H, p.T, p.dhv, scale);
        break;
    case 128:
        recurrent_kernel<T, GATE, 128><<<blocks, 256, 0, stream>>>(qt, kt, vt, ig, fg, state, ht, p.H, p.T, p.dhv, scale);
        break;
    default:
        recurrent_kernel<T, GATE, 256><<<blocks, 256, 0, stream>>>(qt, kt, vt, ig, fg, state, ht, p.H, p.T, p.dhv, scale);
        break;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gate(const Problem& p, const void* q, const void* k, const void* v, const float* ig,
                       const float* fg, float* state, void* h, hipStream_t stream)
{
    switch (p.gate) {
    case kSig: return launch_t<T, kSig>(p, q, k, v, ig, fg, state, h, stream);
    case kScalar: return launch_t<T, kScalar>(p, q, k, v, ig, fg, state, h, stream);
    default: return launch_t<T, kGla>(p, q, k, v, ig, fg, state, h, stream);
    }
}

}  // namespace

hipError_t launch_recurrent(const Problem& p, const void* q, const void* k, const void* v, const float* igate_pre,
                            const float* fgate_pre, float* state, void* h, hipStream_t stream)
{
    if (p.bf16) return launch_gate<bf16>(p, q, k, v, igate_pre, fgate_pre, state, h, stream);
    return launch_gate<float>(p, q, k, v, igate_pre, fgate_pre, state, h, stream);
}

}  // namespace tfla

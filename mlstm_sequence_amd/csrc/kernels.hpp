// kernels.hpp -- host-side launchers of the libtfla kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace tfla {

enum GateKind { kSig = 0, kScalar = 1, kGla = 2 };

// Problem description shared by the launchers.  Sizes in elements.
struct Problem {
    int B, H, T, dqk, dhv, L;
    int nc;          // number of chunks, ceil(T / L)
    int gate;        // GateKind
    bool bf16;       // element type of q, k, v, h
};

// Workspace carve-up (device pointers into one allocation).
struct Workspace {
    float* a;        // [B,H,T] (GLA: [B,H,T,dqk]) chunk-local log-forget sums; NULL for kScalar
    float* li;       // [B,H,T] log input gate; kSig only
    float* g;        // [B,H,nc] (GLA: [B,H,nc,dqk]); NULL for kScalar
    float* states;   // [B,H,ns,dhv,dqk] fp32, transposed states before chunks
                     // 1..nc-1 (ns = nc-1), or 0..nc-1 with an initial state (ns = nc)
    const float* c0 = nullptr;   // caller's initial state [B,H,dqk,dhv] (NULL: zero)
    float* c_final = nullptr;    // caller's final-state output [B,H,dqk,dhv] (NULL: none)
    float* seg_end = nullptr;    // segmented state walk: end states [B*H][P][dqk][dhv]
    float* seg_start = nullptr;  //                       start states [B*H][P][dqk][dhv]
};

// Segmented state walk (few heads, long sequences): number of segments P
// (1: unsegmented), chunks per segment, and whether 128x128 state tiles
// are used.  Functions of the problem shape only.
int state_segments(const Problem& p);
int state_segments_for(const Problem& p, long heads_tiles);
int state_chunks_per_segment(const Problem& p, int P);
bool state_big_tiles(const Problem& p);

// Lays the workspace out from `base` (NULL: sizes only); returns its byte size.
// with_c0 reserves the extra state slot an initial state needs.
size_t workspace_layout(const Problem& p, Workspace* ws, char* base, bool with_states = true,
                        bool with_c0 = false);

hipError_t launch_gates(const Problem& p, const float* igate_pre, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream);
hipError_t launch_gates_closed_form(const Problem& p, const float* fgate_pre, float* a, float* li,
                                    float* g, hipStream_t stream);
hipError_t launch_state(const Problem& p, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, hipStream_t stream);
hipError_t launch_recurrent(const Problem& p, const void* q, const void* k, const void* v,
                            const float* igate_pre, const float* fgate_pre, float* state, void* h,
                            hipStream_t stream);
hipError_t launch_intra(const Problem& p, const void* q, const void* k, const void* v,
                        const float* fgate_pre, const Workspace& ws, void* h, hipStream_t stream);

}  // namespace tfla

// Host-side interface of the dense GEMV kernels (used by the step and MoE).
#pragma once

#include "gemv_core.hpp"

namespace ocrdec {

enum { EPI_F32 = 0, EPI_F16 = 1, EPI_RESID = 2, EPI_GLU = 3, EPI_ARGMAX = 4 };

struct GemvParams {
    const uint8_t* w;
    int n, k;
    int64_t nchunks;
    XDirect xs;
    void* y;          // output (EPI_RESID: the fp32 residual, updated in place)
    int64_t ldy;
    int half_tiles;   // EPI_GLU: tiles in the gate half (= d_ff / 16)
    float* part;      // EPI_ARGMAX: [grid][rows][3] (best, index bits, second)
    int* counter;     // EPI_ARGMAX, and EPI_RESID with norm_w: zero on entry; the last
                      // workgroup to finish does the follow-up work and resets it
    const uint16_t* norm_w;  // EPI_RESID: RMSNorm gain applied to the updated residual, or NULL
    float eps;
    uint16_t* norm_out;      // fp16 [rows][n] normalised residual
    int32_t* tok_out; // EPI_ARGMAX outputs
    float* top2;
    int32_t* gen_index;
    int n_groups;
};

struct GemvPlan {
    int nt, ks, xt, groups, grid;
};

GemvPlan plan_gemv(int fmt, int n, int k, int rows, int epi);
void launch_gemv(int fmt, int epi, const GemvPlan& pl, GemvParams p, hipStream_t s);
// Argmax workspace: partials, then the arrival counter (must be zero before
// the first use; every launch leaves it zero).
size_t argmax_ws_bytes(int grid, int rows);

// Merge of two (best, index, second) argmax states; ties go to the lower index.
OCR_DEV void argmax_merge(float& b, int& bi, float& s, float ob, int oi, float os) {
    if (ob > b || (ob == b && oi < bi)) {
        s = fmaxf(fmaxf(s, os), b);
        b = ob;
        bi = oi;
    } else {
        s = fmaxf(fmaxf(s, os), ob);
    }
}

}  // namespace ocrdec

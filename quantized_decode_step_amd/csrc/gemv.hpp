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
    void* y;          // output (EPI_RESID: the fixed-point residual, updated in place)
    int64_t ldy;
    int half_tiles;   // EPI_GLU: tiles in the gate half (= d_ff / 16)
    float* part;      // EPI_ARGMAX: [grid][rows][4] (best, index bits, second, flag bits)
    int n_groups;
    // LDS-staged kernels: with hn non-NULL the activations are formed in the
    // staging step, x = fp16(RMSNorm(hn[tok]) * gamma) from the fixed-point
    // rows hn [rows][k] (the decode step's residual), instead of read from xs.
    const fix_t* hn;
    const uint16_t* gamma;
    float eps;
    uint32_t* status;  // status word (kStat* bits) or NULL
    // With er.table non-NULL as well (one 16-token pass): the rows are the
    // fp16 embedding rows er.table[er.tok[r]] instead of hn, and workgroup 0
    // also stores them as the residual eh [rows][k] (fixed point) and opens
    // the status words (the embedding step of the decode step, folded into
    // the first consumer).
    EmbedRows er;
    fix_t* eh;
};

struct GemvPlan {
    int nt, ks, xt, groups, grid;
    bool lds;  // activations staged in LDS
};

GemvPlan plan_gemv(int fmt, int n, int k, int rows, int epi);
void launch_gemv(int fmt, int epi, const GemvPlan& pl, GemvParams p, hipStream_t s);
size_t argmax_ws_bytes(int grid, int rows);

// LM head with fused argmax: the CU-balanced kernel for up to 16 rows, or
// the general GEMV; grid = number of partials for launch_argmax_final.
struct LmPlan {
    bool dyn;
    int grid;
};
LmPlan plan_lm(int fmt, int n, int k, int rows);
void launch_lm_argmax(int fmt, const LmPlan& lp, GemvParams p, hipStream_t s);
void launch_argmax_final(const float* part, int n_wg, int rows, int32_t* tok_out, float* top2, int32_t* gen_index,
                         uint32_t* status, hipStream_t s);

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

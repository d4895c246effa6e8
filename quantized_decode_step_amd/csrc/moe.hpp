// Host-side interface of the MoE kernels (used by ocrdec_moe_layer and the step).
#pragma once

#include <algorithm>

#include "gemv.hpp"

namespace ocrdec {

inline int pack_cb(int fmt) {
    PackGeom g;
    pack_geom(fmt, &g);
    return g.cb;
}

struct MoeParams {
    int rows, n_experts, top_k, n_shared;
    const float* logits;
    const float* bias;
    const int32_t* forced;
    int32_t* idx;
    float* w;
    int32_t* rank;
    int32_t* hist;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv;
    int32_t* vrows;    // [rows * top_k + n_shared * rows] row of every grouped slot
    int32_t* n_virt;
    int4* virt;        // [n_experts + n_shared] (expert, first slot, count, -)
    int32_t* cap_idx;
    float* cap_w;
    int32_t* cap_counts;
    int32_t* cap_offsets;
    int32_t* cap_perm;
    int lslices;     // router logits as lslices partial sums, lslice floats apart (0/1: one)
    int64_t lslice;
    float* sw;          // non-NULL (decode-sized grouping): the combine weight of every grouped slot
};

struct GroupedParams {
    const uint8_t* w_routed;
    const uint8_t* w_shared;
    int n_experts;
    int k;
    int64_t nchunks;
    int64_t expert_bytes;
    int half_tiles;
    int groups_per_expert;
    int max_virt;
    const int32_t* n_virt;
    const int4* virt;
    const int32_t* vrows;
    int np;
    const uint16_t* x;
    int64_t ldx;
    void* y;
    int64_t ldy;
    int out_tiles;   // expert GEMM: output tiles per expert (SwiGLU: tiles of each half)
    int dense_rows;  // expert GEMM: > 0 means one implicit expert over rows [0, dense_rows) (router)
    int kslices;     // expert GEMM: k range split over this many workgroups (0/1: none), partial
    int64_t ly_slice;  //   products of slice z written ly_slice elements after slice 0's
    // Grouped down projection adding into the fixed-point residual h
    // [rows][ldh] itself (sw non-NULL): every output of slot s goes to
    // h[vrows[s]] with weight sw[s] by an atomic integer add (no expert-output
    // buffer, no combine; the sum does not depend on the order).
    fix_t* h;
    int64_t ldh;
    const float* sw;
    uint32_t* status;
    int one_row;       // one token row in all (decode of one row): every slot's row is 0
    int entries16;     // every work entry holds at most 16 tokens (decode-sized grouping)
    // Expert-indexed decode MoE (no grouping pass, pidx non-NULL): a
    // workgroup finds its entry's expert and tokens in pidx [rows][top_k] (the
    // chosen experts, row-major: pair i = r * top_k + j) itself: shared
    // experts' 16-token blocks first, then the routed experts holding tokens
    // (expert_entry).  A routed pair's slot of a is its pair index, shared
    // expert s's slot of row r is rows*top_k + s*rows + r; the combine weight
    // is pw[pair] (shared: 1).  max_virt = (n_experts + n_shared) * nb16.
    const int32_t* pidx;
    const float* pw;
    int rows, top_k, nb16, n_shared;
};

struct CombineParams {
    int rows, hidden, top_k, n_shared, np;
    const float* w;
    const int32_t* inv;
    const float* y;
    void* h;          // the residual: fp16, fp32 or fixed point (h_mode)
    int h_mode;
    int64_t ldh;
    int add_residual;
    const uint16_t* norm_w;  // RMSNorm gain of the next block, or NULL
    float eps;
    uint16_t* x_out;
    int64_t ldx;
    uint32_t* status;
};

struct MoeWs {
    float* logits;
    int32_t* idx;
    float* w;
    int32_t* rank;
    int32_t* hist;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv;
    int32_t* vrows;
    int32_t* n_virt;
    int4* virt;
    uint16_t* a;
    float* y;
    float* sw;
    size_t bytes;
};

// Dense GEMM over many rows on the expert GEMM (one implicit expert):
// y[rows][n] = x[rows][k] W^T as fp32, or with glu, W = [gate; up] of n rows
// each and y[rows][n] = fp16(silu(x G^T) * (x U^T)).  dense_gemm_ok says
// whether the format and shape have that kernel (else use the GEMV).
bool dense_gemm_ok(int fmt, int n, int k, int rows, int64_t ldx);
void launch_dense_gemm(int fmt, bool glu, const uint8_t* w, int n, int k, int rows, const uint16_t* x, int64_t ldx,
                       void* y, int64_t ldy, hipStream_t s);

MoeWs carve_moe(void* ws, int rows, const ocrdec_moe_weights* w);
ocrdec_status check_moe(const ocrdec_moe_weights* w, int rows);
// Residual representations of launch_moe's h.
enum { RESID_F16 = 0, RESID_F32 = 1, RESID_FIX = 2 };

// h: the residual in representation h_mode.  h_norm (fixed point, the decode
// step's residual) with norm_in: the MoE input x is formed as
// fp16(RMSNorm(h_norm) * norm_in) first.  fuse_combine (with RESID_FIX and a
// decode-sized batch): the down projection adds into h itself.
void launch_moe(const ocrdec_moe_weights* w, int rows, const uint16_t* x, int64_t ldx, void* h, int h_mode, int64_t ldh,
                int add_residual, const int32_t* forced, const ocrdec_moe_capture* cap, int32_t* cap_idx,
                float* cap_w, const MoeWs& m, const uint16_t* norm_w, float eps, uint16_t* x_out, int64_t ldxo,
                hipStream_t s, const fix_t* h_norm = nullptr, const uint16_t* norm_in = nullptr, float eps_in = 0.f,
                bool fuse_combine = false, uint32_t* status = nullptr);

}  // namespace ocrdec

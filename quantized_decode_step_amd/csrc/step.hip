// The decode step ("Eseguire Unlimited-OCR su Apple Silicon con C e Metal",
// section "Il decoder e il Mixture of Experts"): embedding lookup, the layer
// stack (pre-norm attention over the prefix + ring cache, then the dense
// SwiGLU or the MoE), the final RMSNorm and the language-head argmax, all
// enqueued on the caller's stream with no host synchronisation, so the token
// of one step can feed the next on the device ("How it is meant to be run",
// Falcon-OCR card: rows of a round share one read of the weights).
#include <mutex>

#include "attn.hpp"
#include "moe.hpp"

// Scratch of ocrdec_decode_step_noalloc: the step's workspace for callers that
// cannot allocate, in device memory that every GPU the library runs on holds
// until the process ends.  Host code never passes this name to a kernel or a
// copy (on the host it is only a stand-in for the symbol): it uses the device
// address that hipGetSymbolAddress returns for the current device.
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace ocrdec {

namespace {

constexpr int kMaxRows = 32;

// h[r] = embed[tok[r]] (fp16 table) or src[r] (fp32); x[r] = norm(h[r]),
// formed from the values as stored.  One wavefront per row (H <= 4096).  HT:
// the residual's representation (the decode step's fixed point, or fp32 for
// the prompt pass).
template <class HT>
__global__ __launch_bounds__(64) void embed_norm_kernel(const int32_t* tok, const uint16_t* embed, int vocab,
                                                        const float* src, HT* h, const uint16_t* gamma, int H,
                                                        float eps, uint16_t* x, const uint16_t* rows16,
                                                        uint32_t* status, int rows) {
    const int r = blockIdx.x, lane = threadIdx.x;
    HT* hr = h + (int64_t)r * H;
    const int n4 = H / 4;
    bool tok_bad = false, bad = false;
    float4 v[16];
    if (tok || rows16) {
        // a row of the fp16 table, or row r of fp16 input features
        int t = tok ? tok[r] : 0;
        tok_bad = t < 0 || t >= vocab;
        t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
        const uint2* from = (const uint2*)(tok ? embed + (int64_t)t * H : rows16 + (int64_t)r * H);
        uint2 e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = from[min(lane + 64 * i, n4 - 1)];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = make_float4(h2f((uint16_t)(e[i].x & 0xFFFF)), h2f((uint16_t)(e[i].x >> 16)),
                               h2f((uint16_t)(e[i].y & 0xFFFF)), h2f((uint16_t)(e[i].y >> 16)));
    } else {
        const float4* from = (const float4*)(src + (int64_t)r * H);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = from[min(lane + 64 * i, n4 - 1)];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c4 = lane + 64 * i;
        v[i] = c4 < n4 ? st_resid4(hr, c4, v[i], bad) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    status_begin(status, r, rows, tok_bad, bad);
    rmsnorm_regs<16>(v, gamma, H, eps, x + (int64_t)r * H, nullptr);
}

// h[r] = row tok[r] of a packed quantised table, dequantised; x[r] = norm(h[r]).
// One wavefront per row.  In the packed layout row t sits in 16-row tile
// t / 16 at position t % 16: for chunk c and k-group g, "lane" t%16 + 16g of
// the chunk holds the codes of columns c*KC + 32j + 8g + i (block j < SB,
// i < 8) and the row's block scales.  Lane l of the wavefront takes the
// (chunk, group) pairs p = l, l+64, ...; each product d*q is exact in fp32
// (q and (q-8) are integers of at most 8 bits, d has 11).
template <int FMT, class HT, int NV>
__global__ __launch_bounds__(64) void embed_q_norm_kernel(const int32_t* tok, const uint8_t* table, int vocab,
                                                          int64_t nchunks, HT* h, const uint16_t* gamma, int H,
                                                          float eps, uint16_t* x, uint32_t* status, int rows) {
    constexpr int SB = Geom<FMT>::SB, CB = Geom<FMT>::CB, KC = 32 * SB;
    const int r = blockIdx.x, lane = threadIdx.x;
    HT* hr = h + (int64_t)r * H;
    int t = tok[r];
    const bool tok_bad = t < 0 || t >= vocab;
    bool bad = false;
    t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
    const uint8_t* tile = table + (int64_t)(t >> 4) * nchunks * CB;
    const int np = (int)nchunks * 4;
    for (int p = lane; p < np; p += 64) {
        const int c = p >> 2, g = p & 3;
        WRegs w;
        load_wchunk<FMT>(tile + (int64_t)c * CB, (t & 15) + 16 * g, w);
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const half8v q = wfrag<FMT>(w, j);
            const float d = wscale<FMT>(w, j);
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (FMT == OCRDEC_U8A_G32) v[i] = d * ((float)q[i] - wzero_u8a(w, j));
                else if constexpr (FMT == OCRDEC_F16) v[i] = (float)q[i];
                else v[i] = d * (float)q[i];
            }
            const int k0 = c * KC + 32 * j + 8 * g;
            if (k0 < H) {
                st_resid4(hr, k0 / 4, make_float4(v[0], v[1], v[2], v[3]), bad);
                st_resid4(hr, k0 / 4 + 1, make_float4(v[4], v[5], v[6], v[7]), bad);
            }
        }
    }
    status_begin(status, r, rows, tok_bad, bad);
    __threadfence_block();
    wave_rmsnorm_row<NV>(hr, gamma, H, eps, x + (int64_t)r * H);
}

// h[r] += y[r]; x[r] = fp16(RMSNorm(h[r]) * gamma): one wavefront per row.
__global__ __launch_bounds__(64) void resid_norm_kernel(float* h, const float* y, const uint16_t* gamma, int H,
                                                        float eps, uint16_t* x) {
    const int r = blockIdx.x, lane = threadIdx.x;
    float4* hr = (float4*)(h + (int64_t)r * H);
    const float4* yr = (const float4*)(y + (int64_t)r * H);
    const int n4 = H / 4;
    float4 a[16], b[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c4 = lane + 64 * i;
        a[i] = c4 < n4 ? hr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        b[i] = c4 < n4 ? yr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < n4) hr[c4] = make_float4(a[i].x + b[i].x, a[i].y + b[i].y, a[i].z + b[i].z, a[i].w + b[i].w);
    }
    __threadfence_block();
    wave_rmsnorm_row(h + (int64_t)r * H, gamma, H, eps, x + (int64_t)r * H);
}

// dst[i] = src[idx[i]]: rows of H halves (H % 8 == 0), one workgroup per row.
struct RowList {
    int idx[PREFILL_MAX_SEQ];
};
__global__ __launch_bounds__(64) void gather_rows_kernel(const uint16_t* src, uint16_t* dst, int H, RowList rl) {
    const uint4* s = (const uint4*)(src + (int64_t)rl.idx[blockIdx.x] * H);
    uint4* d = (uint4*)(dst + (int64_t)blockIdx.x * H);
    for (int c = threadIdx.x; c < H / 8; c += blockDim.x) d[c] = s[c];
}

// x[r] = fp16(RMSNorm(h[r]) * gamma) of the fixed-point residual: one
// wavefront per row (H <= 256 * NV).
template <int NV>
__global__ __launch_bounds__(64) void norm_kernel(const fix_t* h, const uint16_t* gamma, int H, float eps,
                                                  uint16_t* x) {
    const int r = blockIdx.x;
    wave_rmsnorm_row<NV>(h + (int64_t)r * H, gamma, H, eps, x + (int64_t)r * H);
}

// norm_kernel with the register count its row size needs
void launch_norm(const fix_t* h, const uint16_t* gamma, int H, float eps, uint16_t* x, int rows, hipStream_t s) {
    if (H <= 1280) hipLaunchKernelGGL(norm_kernel<5>, dim3(rows), dim3(64), 0, s, h, gamma, H, eps, x);
    else if (H <= 2048) hipLaunchKernelGGL(norm_kernel<8>, dim3(rows), dim3(64), 0, s, h, gamma, H, eps, x);
    else hipLaunchKernelGGL(norm_kernel<16>, dim3(rows), dim3(64), 0, s, h, gamma, H, eps, x);
}

__global__ void copy_rows_kernel(const float* src, float* dst, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

// The fixed-point residual as fp32.
__global__ void fix_rows_kernel(const fix_t* src, float* dst, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = fix_to(src[i]);
}

__global__ void bump_kernel(int32_t* gen_index, int rows) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r < rows) gen_index[r] += 1;
}

struct StepWs {
    uint32_t* status;  // [1 + kStatusRows] (first in the workspace)
    fix_t* h;
    uint16_t* x;
    float* qkv;
    float* attn_part;
    uint16_t* o;
    uint16_t* a;
    float* lm_part;
    MoeWs moe;
    size_t bytes;
};

int lm_grid(const ocrdec_model* m, int rows) {
    if (!m->lm_head.data) return 0;
    return plan_lm(m->lm_head.fmt, m->lm_head.n, m->lm_head.k, rows).grid;
}

StepWs carve_step(void* ws, const ocrdec_model* m, int rows, int cache_cap) {
    Carve cv(ws);
    StepWs w;
    const int H = m->hidden, HD = m->n_heads * m->head_dim;
    int dense_ff = 0;
    const ocrdec_moe_weights* moe = nullptr;
    for (int l = 0; l < m->n_layers; ++l) {
        if (m->layers[l].is_moe) moe = &m->layers[l].moe;
        else dense_ff = std::max(dense_ff, m->layers[l].dense_ff);
    }
    w.status = cv.take<uint32_t>(1 + kStatusRows);
    w.h = cv.take<fix_t>((size_t)rows * H);
    w.x = cv.take<uint16_t>((size_t)rows * H);
    w.qkv = cv.take<float>((size_t)rows * 3 * HD);
    w.attn_part = cv.take<float>(attn_ws_bytes(rows, m->n_heads, m->head_dim, cache_cap) / sizeof(float));
    w.o = cv.take<uint16_t>((size_t)rows * HD);
    w.a = cv.take<uint16_t>((size_t)rows * std::max(dense_ff, 1));
    w.lm_part = cv.take<float>(argmax_ws_bytes(std::max(lm_grid(m, rows), 1), rows) / sizeof(float));
    if (moe) {
        MoeWs probe = carve_moe(nullptr, rows, moe);
        char* base = (char*)cv.take<char>(probe.bytes);
        w.moe = carve_moe(ws ? base : nullptr, rows, moe);
    } else {
        w.moe = MoeWs{};
    }
    w.bytes = cv.off;
    return w;
}

struct PrefillWs {
    float* h;
    uint16_t* x;
    float* qkv;
    uint16_t* q;
    uint16_t* o;
    float* y;
    uint16_t* a;
    float* lm_part;
    float* attn_part;
    uint16_t* x_last;  // [n_seq][H] the last position of every sequence (LM-head input)
    MoeWs moe;
    size_t bytes;
};

// P: packed positions of all sequences; n_seq sequences, the longest max_len
PrefillWs carve_prefill(void* ws, const ocrdec_model* m, int P, int n_seq, int max_len) {
    Carve cv(ws);
    PrefillWs w;
    const int H = m->hidden, HD = m->n_heads * m->head_dim;
    int dense_ff = 0;
    const ocrdec_moe_weights* moe = nullptr;
    for (int l = 0; l < m->n_layers; ++l) {
        if (m->layers[l].is_moe) moe = &m->layers[l].moe;
        else dense_ff = std::max(dense_ff, m->layers[l].dense_ff);
    }
    w.h = cv.take<float>((size_t)P * H);
    w.x = cv.take<uint16_t>((size_t)P * H);
    w.qkv = cv.take<float>((size_t)P * 3 * HD);
    w.q = cv.take<uint16_t>((size_t)P * HD);
    w.o = cv.take<uint16_t>((size_t)P * HD);
    w.y = cv.take<float>((size_t)P * H);
    w.a = cv.take<uint16_t>((size_t)P * std::max(dense_ff, 1));
    w.lm_part = cv.take<float>(argmax_ws_bytes(std::max(lm_grid(m, n_seq), 1), n_seq) / sizeof(float));
    w.attn_part = cv.take<float>(prefill_attn_part_bytes(n_seq, max_len, m->n_heads) / sizeof(float));
    w.x_last = cv.take<uint16_t>((size_t)n_seq * H);
    if (moe) {
        MoeWs probe = carve_moe(nullptr, P, moe);
        char* base = (char*)cv.take<char>(probe.bytes);
        w.moe = carve_moe(ws ? base : nullptr, P, moe);
    } else {
        w.moe = MoeWs{};
    }
    w.bytes = cv.off;
    return w;
}

// y[rows][...] = x W^T: the expert GEMM where it has the format and shape,
// else the GEMV kernel in 16/32-token passes
void prefill_gemm(const ocrdec_qmat& W, bool glu, int rows, const uint16_t* x, int64_t ldx, void* y, int64_t ldy,
                  hipStream_t s) {
    const int n_out = glu ? W.n / 2 : W.n;
    if (dense_gemm_ok(W.fmt, n_out, W.k, rows, ldx)) {
        launch_dense_gemm(W.fmt, glu, (const uint8_t*)W.data, n_out, W.k, rows, x, ldx, y, ldy, s);
        return;
    }
    const int epi = glu ? EPI_GLU : EPI_F32;
    GemvPlan pl = plan_gemv(W.fmt, W.n, W.k, rows, epi);
    GemvParams gp{};
    gp.w = (const uint8_t*)W.data;
    gp.n = W.n;
    gp.k = W.k;
    gp.nchunks = n_chunks(W.fmt, W.k);
    gp.xs = XDirect{x, ldx, rows};
    gp.y = y;
    gp.ldy = ldy;
    if (glu) gp.half_tiles = n_out / 16;
    launch_gemv(W.fmt, epi, pl, gp, s);
}

ocrdec_status check_step(const ocrdec_model* m, const ocrdec_state* st, int moe_rows = -1) {
    OCR_CHECK_ARG(m && st, "model and state must be non-NULL");
    if (moe_rows < 0) moe_rows = st->rows;
    OCR_CHECK_ARG(st->rows >= 1 && st->rows <= kMaxRows, "rows must be in [1, 32]");
    OCR_CHECK_ARG(st->ring_cap >= 1 && st->prefix_cap >= 0, "ring_cap must be >= 1 and prefix_cap >= 0");
    OCR_CHECK_ARG(st->prefix_len && st->gen_index, "state arrays must be non-NULL");
    OCR_CHECK_ARG(m->n_layers >= 1 && m->layers, "model needs at least one layer");
    OCR_CHECK_ARG(m->hidden > 0 && m->hidden % 32 == 0 && m->hidden <= 4096,
                  "hidden must be a positive multiple of 32, at most 4096");
    if (m->head_dim != 64 && m->head_dim != 128) return fail(OCRDEC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    OCR_CHECK_ARG(m->n_heads >= 1, "n_heads must be >= 1");
    OCR_CHECK_ARG((m->n_heads * m->head_dim) % 32 == 0, "n_heads*head_dim must be a multiple of 32");
    const int H = m->hidden, HD = m->n_heads * m->head_dim;
    ocrdec_status s;
    const ocrdec_moe_weights* moe0 = nullptr;
    for (int l = 0; l < m->n_layers; ++l) {
        const ocrdec_layer& L = m->layers[l];
        const std::string tag = "layer " + std::to_string(l) + ": ";
        OCR_CHECK_ARG(L.attn_norm && L.ffn_norm, tag + "norm gains must be non-NULL");
        OCR_CHECK_ARG(L.k_cache && L.v_cache, tag + "caches must be non-NULL");
        OCR_CHECK_ARG((L.k_scale == nullptr) == (L.v_scale == nullptr),
                      tag + "k_scale and v_scale must both be given (int8 cache) or both be NULL");
        if ((s = check_qmat(&L.wqkv, "wqkv")) != OCRDEC_OK) return s;
        if ((s = check_qmat(&L.wo, "wo")) != OCRDEC_OK) return s;
        OCR_CHECK_ARG(L.wqkv.n == 3 * HD && L.wqkv.k == H, tag + "wqkv must be [3*n_heads*head_dim][hidden]");
        OCR_CHECK_ARG(L.wo.n == H && L.wo.k == HD, tag + "wo must be [hidden][n_heads*head_dim]");
        if (L.is_moe) {
            if ((s = check_moe(&L.moe, moe_rows)) != OCRDEC_OK) return s;
            OCR_CHECK_ARG(L.moe.hidden == H, tag + "moe.hidden must equal hidden");
            if (moe0) {
                OCR_CHECK_ARG(L.moe.n_experts == moe0->n_experts && L.moe.top_k == moe0->top_k &&
                                  L.moe.n_shared == moe0->n_shared && L.moe.d_ff == moe0->d_ff,
                              tag + "all MoE layers must share n_experts, top_k, n_shared and d_ff");
            }
            moe0 = &L.moe;
        } else {
            if ((s = check_qmat(&L.dense_gate_up, "dense_gate_up")) != OCRDEC_OK) return s;
            if ((s = check_qmat(&L.dense_down, "dense_down")) != OCRDEC_OK) return s;
            OCR_CHECK_ARG(L.dense_ff > 0 && L.dense_ff % 32 == 0, tag + "dense_ff must be a positive multiple of 32");
            OCR_CHECK_ARG(L.dense_gate_up.n == 2 * L.dense_ff && L.dense_gate_up.k == H,
                          tag + "dense_gate_up must be [2*dense_ff][hidden]");
            OCR_CHECK_ARG(L.dense_down.n == H && L.dense_down.k == L.dense_ff,
                          tag + "dense_down must be [hidden][dense_ff]");
        }
    }
    if (!m->embed && m->embed_q.data) {
        if ((s = check_qmat(&m->embed_q, "embed_q")) != OCRDEC_OK) return s;
        OCR_CHECK_ARG(m->embed_q.k == H && m->embed_q.n == m->vocab, "embed_q must be [vocab][hidden]");
    }
    if (m->lm_head.data) {
        if ((s = check_qmat(&m->lm_head, "lm_head")) != OCRDEC_OK) return s;
        OCR_CHECK_ARG(m->lm_head.k == H && m->lm_head.n == m->vocab, "lm_head must be [vocab][hidden]");
        OCR_CHECK_ARG(m->final_norm, "final_norm must be non-NULL with an LM head");
    }
    return OCRDEC_OK;
}

}  // namespace

}  // namespace ocrdec

using namespace ocrdec;

extern "C" ocrdec_status ocrdec_step_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st,
                                                     size_t* bytes) {
    ocrdec_status s0 = check_step(m, st);
    if (s0 != OCRDEC_OK) return s0;
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    OCR_CHECK_ARG(st->prefix_cap + st->ring_cap <= (1 << 16), "prefix_cap + ring_cap must be <= 65536");
    *bytes = carve_step(nullptr, m, st->rows, st->prefix_cap + st->ring_cap).bytes;
    return OCRDEC_OK;
}

namespace {

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; NULL if the lookup fails.
void* scratch_ptr(std::string* err) {
    static std::mutex mu;
    static void* ptrs[64] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        *err = std::string("hipGetDevice: ") + (e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
            return nullptr;
        }
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

}  // namespace

extern "C" ocrdec_status ocrdec_decode_step_noalloc(const ocrdec_model* m, const ocrdec_state* st,
                                                    const int32_t* tok_in, float* hidden, int32_t* tok_out,
                                                    const int32_t* forced_topk, const ocrdec_step_capture* cap,
                                                    void* stream) {
    ocrdec_status s0 = check_step(m, st);
    if (s0 != OCRDEC_OK) return s0;
    OCR_CHECK_ARG(st->prefix_cap + st->ring_cap <= (1 << 16), "prefix_cap + ring_cap must be <= 65536");
    const size_t need = carve_step(nullptr, m, st->rows, st->prefix_cap + st->ring_cap).bytes;
    if (need > kScratchBytes)
        return fail(OCRDEC_ERR_WORKSPACE, "ocrdec_decode_step_noalloc: this model and state need a " +
                                              std::to_string(need) + "-byte workspace; the static scratch holds " +
                                              std::to_string(kScratchBytes) + " bytes (use ocrdec_decode_step)");
    std::string err;
    void* ws = scratch_ptr(&err);
    if (!ws) return fail(OCRDEC_ERR_DEVICE, err);
    return ocrdec_decode_step(m, st, tok_in, hidden, tok_out, forced_topk, cap, ws, kScratchBytes, stream);
}

extern "C" ocrdec_status ocrdec_device_status(const void* ws, size_t ws_bytes, void* stream, uint32_t* flags) {
    OCR_CHECK_ARG(ws && flags, "ws and flags must be non-NULL");
    const size_t need = sizeof(uint32_t) * (1 + kStatusRows);
    if (ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "status: a step workspace holds at least " + std::to_string(need) +
                                              " bytes, got " + std::to_string(ws_bytes));
    OCR_HIP(hipStreamSynchronize((hipStream_t)stream));
    uint32_t words[1 + kStatusRows];
    OCR_HIP(hipMemcpy(words, ws, sizeof(words), hipMemcpyDeviceToHost));
    uint32_t f = 0;
    for (uint32_t w : words) f |= w;
    *flags = f & (OCRDEC_DEV_TOKEN_RANGE | OCRDEC_DEV_RESIDUAL | OCRDEC_DEV_LOGIT | OCRDEC_DEV_NO_TOKEN);
    return OCRDEC_OK;
}

extern "C" ocrdec_status ocrdec_decode_step(const ocrdec_model* m, const ocrdec_state* st, const int32_t* tok_in,
                                            float* hidden, int32_t* tok_out, const int32_t* forced_topk,
                                            const ocrdec_step_capture* cap, void* ws, size_t ws_bytes, void* stream) {
    ocrdec_status s0 = check_step(m, st);
    if (s0 != OCRDEC_OK) return s0;
    OCR_CHECK_ARG(tok_in || hidden, "either tok_in or hidden must be given");
    OCR_CHECK_ARG(!tok_in || m->embed || m->embed_q.data, "tok_in needs an embedding table");
    const int R = st->rows, H = m->hidden, HD = m->n_heads * m->head_dim;
    const int cache_cap = st->prefix_cap + st->ring_cap;
    OCR_CHECK_ARG(cache_cap <= (1 << 16), "prefix_cap + ring_cap must be <= 65536");
    const size_t need = carve_step(nullptr, m, R, cache_cap).bytes;
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "step workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    hipStream_t s = (hipStream_t)stream;
    StepWs w = carve_step(ws, m, R, cache_cap);

    // Up to 16 rows: the kernels that consume a normalised residual (QKV,
    // the dense MLP, the language head) form RMSNorm(h) in their LDS staging
    // and the MoE down projection adds its weighted outputs into the residual,
    // so no separate norm or combine kernel runs.  (With more rows the
    // per-consumer norms cost more than the kernels they replace.)  Up to 24
    // rows the attention merge runs inside the O projection.  With an fp16
    // embedding table the first QKV projection also reads the embedding rows
    // itself and stores the residual (no embedding kernel).
    const bool prolog = R <= 16 && lds_x_bytes(H, 1) <= 65536;
    const bool fold_embed = prolog && tok_in && m->embed;
    if (!fold_embed) prof_mark(s, OCRDEC_K_EMBED);
    if (fold_embed) {
        // (in the first QKV projection below)
    } else if (tok_in && !m->embed) {
        const uint8_t* tq = (const uint8_t*)m->embed_q.data;
        const int64_t nch = n_chunks(m->embed_q.fmt, H);
#define OCR_EQ(F_)                                                                                                 \
    case F_:                                                                                                       \
        if (H <= 1280)                                                                                             \
            hipLaunchKernelGGL((embed_q_norm_kernel<F_, fix_t, 5>), dim3(R), dim3(64), 0, s, tok_in, tq, m->vocab, \
                               nch, w.h, m->layers[0].attn_norm, H, m->norm_eps, w.x, w.status, R);                \
        else                                                                                                       \
            hipLaunchKernelGGL((embed_q_norm_kernel<F_, fix_t, 16>), dim3(R), dim3(64), 0, s, tok_in, tq, m->vocab,\
                               nch, w.h, m->layers[0].attn_norm, H, m->norm_eps, w.x, w.status, R);                \
        break;
        switch (m->embed_q.fmt) {
            OCR_EQ(OCRDEC_F16)
            OCR_EQ(OCRDEC_Q8_0)
            OCR_EQ(OCRDEC_Q4_0)
            OCR_EQ(OCRDEC_U8A_G32)
        }
#undef OCR_EQ
    } else {
        hipLaunchKernelGGL(embed_norm_kernel<fix_t>, dim3(R), dim3(64), 0, s, tok_in, m->embed, m->vocab, hidden,
                           w.h, m->layers[0].attn_norm, H, m->norm_eps, w.x, (const uint16_t*)nullptr, w.status, R);
    }
    // attention arguments shared by every layer (RoPE frequencies once per call)
    AttnParams ap0{};
    ap0.rows = R;
    ap0.n_heads = m->n_heads;
    ap0.head_dim = m->head_dim;
    ap0.qkv = w.qkv;
    ap0.ld_qkv = 3 * HD;
    ap0.prefix_cap = st->prefix_cap;
    ap0.ring_cap = st->ring_cap;
    ap0.cache_cap = cache_cap;
    ap0.prefix_len = st->prefix_len;
    ap0.gen_index = st->gen_index;
    ap0.sink = nullptr;
    ap0.scale = 1.0f / sqrtf((float)m->head_dim);
    ap0.out = w.o;
    ap0.ld_out = HD;
    ap0.n_split = attn_n_split(cache_cap);
    ap0.part = w.attn_part;
    attn_set_rope(ap0, m->rope_theta);
    int moe_l = 0;
    for (int l = 0; l < m->n_layers; ++l) {
        const ocrdec_layer& L = m->layers[l];
        const uint16_t* next_norm = (l + 1 < m->n_layers) ? m->layers[l + 1].attn_norm : m->final_norm;
        // QKV
        {
            GemvPlan pl = plan_gemv(L.wqkv.fmt, L.wqkv.n, H, R, EPI_F32);
            GemvParams gp{};
            gp.w = (const uint8_t*)L.wqkv.data;
            gp.n = L.wqkv.n;
            gp.k = H;
            gp.nchunks = n_chunks(L.wqkv.fmt, H);
            gp.xs = XDirect{w.x, H, R};
            gp.y = w.qkv;
            gp.ldy = 3 * HD;
            if (prolog) {
                gp.hn = w.h;
                gp.gamma = L.attn_norm;
                gp.eps = m->norm_eps;
            }
            if (l == 0 && fold_embed) {
                gp.er = EmbedRows{m->embed, tok_in, m->vocab};
                gp.eh = w.h;
                gp.status = w.status;
            }
            prof_mark(s, OCRDEC_K_QKV);
            launch_gemv(L.wqkv.fmt, EPI_F32, pl, gp, s);
        }
        // attention, and the O projection + residual (up to 24 rows: the
        // merge of the splits and the projection are one launch)
        AttnParams ap = ap0;
        ap.k_cache = L.k_cache;
        ap.v_cache = L.v_cache;
        ap.k_scale = L.k_scale;
        ap.v_scale = L.v_scale;
        if (attn_merge_o_ok(ap, L.wo.fmt, H)) {
            launch_attn_merge_o(ap, L.wo.fmt, (const uint8_t*)L.wo.data, H, w.h, H, w.status, s);
        } else {
            launch_attn(ap, s);
            GemvPlan pl = plan_gemv(L.wo.fmt, H, HD, R, EPI_RESID);
            GemvParams gp{};
            gp.w = (const uint8_t*)L.wo.data;
            gp.n = H;
            gp.k = HD;
            gp.nchunks = n_chunks(L.wo.fmt, HD);
            gp.xs = XDirect{w.o, HD, R};
            gp.y = w.h;
            gp.ldy = H;
            gp.status = w.status;
            prof_mark(s, OCRDEC_K_O_PROJ);
            launch_gemv(L.wo.fmt, EPI_RESID, pl, gp, s);
        }
        if (L.is_moe) {
            const int K = L.moe.top_k;
            int32_t* ci = cap && cap->topk_idx ? cap->topk_idx + (int64_t)moe_l * R * K : nullptr;
            float* cw = cap && cap->topk_w ? cap->topk_w + (int64_t)moe_l * R * K : nullptr;
            const int32_t* fo = forced_topk ? forced_topk + (int64_t)moe_l * R * K : nullptr;
            // the routing kernel forms x = RMSNorm(h) itself
            launch_moe(&L.moe, R, w.x, H, w.h, RESID_FIX, H, 1, fo, nullptr, ci, cw, w.moe,
                       prolog ? nullptr : next_norm, m->norm_eps, w.x, H, s, w.h, L.ffn_norm, m->norm_eps, true,
                       w.status);
            ++moe_l;
        } else {
            if (!prolog) {
                prof_mark(s, OCRDEC_K_NORM);
                launch_norm(w.h, L.ffn_norm, H, m->norm_eps, w.x, R, s);
            }
            const int F = L.dense_ff;
            {
                GemvPlan pl = plan_gemv(L.dense_gate_up.fmt, 2 * F, H, R, EPI_GLU);
                GemvParams gp{};
                gp.w = (const uint8_t*)L.dense_gate_up.data;
                gp.n = 2 * F;
                gp.k = H;
                gp.nchunks = n_chunks(L.dense_gate_up.fmt, H);
                gp.xs = XDirect{w.x, H, R};
                gp.y = w.a;
                gp.ldy = F;
                gp.half_tiles = F / 16;
                if (prolog) {
                    gp.hn = w.h;
                    gp.gamma = L.ffn_norm;
                    gp.eps = m->norm_eps;
                }
                prof_mark(s, OCRDEC_K_DENSE_GLU);
                launch_gemv(L.dense_gate_up.fmt, EPI_GLU, pl, gp, s);
            }
            {
                GemvPlan pl = plan_gemv(L.dense_down.fmt, H, F, R, EPI_RESID);
                GemvParams gp{};
                gp.w = (const uint8_t*)L.dense_down.data;
                gp.n = H;
                gp.k = F;
                gp.nchunks = n_chunks(L.dense_down.fmt, F);
                gp.xs = XDirect{w.a, F, R};
                gp.y = w.h;
                gp.ldy = H;
                gp.status = w.status;
                prof_mark(s, OCRDEC_K_DENSE_DOWN);
                launch_gemv(L.dense_down.fmt, EPI_RESID, pl, gp, s);
            }
            if (next_norm && !prolog) {
                prof_mark(s, OCRDEC_K_NORM);
                launch_norm(w.h, next_norm, H, m->norm_eps, w.x, R, s);
            }
        }
    }
    if (hidden) {
        const int64_t n = (int64_t)R * H;
        prof_mark(s, OCRDEC_K_OTHER);
        hipLaunchKernelGGL(fix_rows_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 1024)), dim3(256), 0, s,
                           w.h, hidden, n);
    }
    if (m->lm_head.data && tok_out) {
        const LmPlan lp = plan_lm(m->lm_head.fmt, m->vocab, H, R);
        GemvParams gp{};
        gp.w = (const uint8_t*)m->lm_head.data;
        gp.n = m->vocab;
        gp.k = H;
        gp.nchunks = n_chunks(m->lm_head.fmt, H);
        gp.xs = XDirect{w.x, H, R};
        gp.part = w.lm_part;
        if (prolog) {
            gp.hn = w.h;
            gp.gamma = m->final_norm;
            gp.eps = m->norm_eps;
        }
        prof_mark(s, OCRDEC_K_LM_HEAD);
        launch_lm_argmax(m->lm_head.fmt, lp, gp, s);
        prof_mark(s, OCRDEC_K_ARGMAX);
        launch_argmax_final(w.lm_part, lp.grid, R, tok_out, cap ? cap->lm_top2 : nullptr, st->gen_index, w.status, s);
    } else {
        prof_mark(s, OCRDEC_K_OTHER);
        hipLaunchKernelGGL(bump_kernel, dim3(1), dim3(64), 0, s, st->gen_index, R);
    }
    return launch_status("ocrdec_decode_step");
}

namespace {

// Validation of a batch of prompt passes; fills the packed offsets.
ocrdec_status check_prefill(const ocrdec_model* m, const ocrdec_state* st, int n, const int32_t* rows,
                            const int32_t* P, int* total, int* max_len) {
    OCR_CHECK_ARG(n >= 1 && n <= PREFILL_MAX_SEQ, "n must be in [1, 32]");
    OCR_CHECK_ARG(rows && P, "rows and P must be non-NULL");
    OCR_CHECK_ARG(m && st, "model and state must be non-NULL");
    int64_t T = 0;
    *max_len = 1;
    for (int i = 0; i < n; ++i) {
        const std::string tag = "sequence " + std::to_string(i) + ": ";
        OCR_CHECK_ARG(P[i] >= 1 && P[i] <= st->prefix_cap, tag + "P must be in [1, prefix_cap] (the prompt fills the prefix region)");
        OCR_CHECK_ARG(rows[i] >= 0 && rows[i] < st->rows, tag + "row must be in [0, rows)");
        for (int j = 0; j < i; ++j) OCR_CHECK_ARG(rows[j] != rows[i], tag + "rows must be distinct");
        T += P[i];
        *max_len = std::max(*max_len, (int)P[i]);
    }
    OCR_CHECK_ARG(T <= 65536, "the positions of all sequences must total at most 65536");
    *total = (int)T;
    ocrdec_status s0 = check_step(m, st, *total);
    if (s0 != OCRDEC_OK) return s0;
    OCR_CHECK_ARG(st->prefix_cap + st->ring_cap <= (1 << 16), "prefix_cap + ring_cap must be <= 65536");
    return OCRDEC_OK;
}

}  // namespace

extern "C" ocrdec_status ocrdec_prefill_batch_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st,
                                                              int32_t n, const int32_t* rows, const int32_t* P,
                                                              size_t* bytes) {
    int T = 0, max_len = 1;
    ocrdec_status s0 = check_prefill(m, st, n, rows, P, &T, &max_len);
    if (s0 != OCRDEC_OK) return s0;
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    *bytes = carve_prefill(nullptr, m, T, n, max_len).bytes;
    return OCRDEC_OK;
}

extern "C" ocrdec_status ocrdec_prefill_batch(const ocrdec_model* m, const ocrdec_state* st, int32_t n,
                                              const int32_t* rows, const int32_t* P, const int32_t* tok,
                                              const uint16_t* emb, const int32_t* forced_topk, int32_t* tok_out,
                                              float* hidden, const ocrdec_step_capture* cap, void* ws,
                                              size_t ws_bytes, void* stream) {
    int T = 0, max_len = 1;
    ocrdec_status s0 = check_prefill(m, st, n, rows, P, &T, &max_len);
    if (s0 != OCRDEC_OK) return s0;
    OCR_CHECK_ARG(tok || emb, "either tok or emb must be given");
    OCR_CHECK_ARG(!tok || m->embed || m->embed_q.data, "tok needs an embedding table");
    OCR_CHECK_ARG(!emb || ((uintptr_t)emb & 7) == 0, "emb must be 8-byte aligned");
    const int H = m->hidden, HD = m->n_heads * m->head_dim, D = m->head_dim;
    const int cache_cap = st->prefix_cap + st->ring_cap;
    const size_t need = carve_prefill(nullptr, m, T, n, max_len).bytes;
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "prefill workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    hipStream_t s = (hipStream_t)stream;
    PrefillWs w = carve_prefill(ws, m, T, n, max_len);
    prof_mark(s, OCRDEC_K_EMBED);
    // h = the input rows, x = fp16(RMSNorm(h) * attn_norm of layer 0)
    if (tok && !m->embed) {
        const uint8_t* tq = (const uint8_t*)m->embed_q.data;
        const int64_t nch = n_chunks(m->embed_q.fmt, H);
#define OCR_EQ(F_)                                                                                                 \
    case F_:                                                                                                       \
        hipLaunchKernelGGL((embed_q_norm_kernel<F_, float, 16>), dim3(T), dim3(64), 0, s, tok, tq, m->vocab, nch,  \
                           w.h, m->layers[0].attn_norm, H, m->norm_eps, w.x, (uint32_t*)nullptr, T);               \
        break;
        switch (m->embed_q.fmt) {
            OCR_EQ(OCRDEC_F16)
            OCR_EQ(OCRDEC_Q8_0)
            OCR_EQ(OCRDEC_Q4_0)
            OCR_EQ(OCRDEC_U8A_G32)
        }
#undef OCR_EQ
    } else {
        hipLaunchKernelGGL(embed_norm_kernel<float>, dim3(T), dim3(64), 0, s, tok, m->embed, m->vocab, nullptr, w.h,
                           m->layers[0].attn_norm, H, m->norm_eps, w.x, tok ? (const uint16_t*)nullptr : emb,
                           (uint32_t*)nullptr, T);
    }
    PrefillAttnParams ap{};
    ap.P = T;
    ap.n_heads = m->n_heads;
    ap.head_dim = D;
    ap.qkv = w.qkv;
    ap.ld_qkv = 3 * HD;
    ap.q = w.q;
    ap.cache_cap = cache_cap;
    ap.scale = 1.0f / sqrtf((float)D);
    ap.out = w.o;
    ap.ld_out = HD;
    ap.part = w.attn_part;
    ap.n_seq = n;
    RowList last{};
    for (int i = 0, off = 0; i < n; off += P[i], ++i) {
        ap.seq_off[i] = off;
        ap.seq_len[i] = P[i];
        ap.seq_row[i] = rows[i];
        last.idx[i] = off + P[i] - 1;
    }
    prefill_set_rope(ap, m->rope_theta);
    int moe_l = 0;
    for (int l = 0; l < m->n_layers; ++l) {
        const ocrdec_layer& L = m->layers[l];
        const uint16_t* next_norm = (l + 1 < m->n_layers) ? m->layers[l + 1].attn_norm : m->final_norm;
        if (!next_norm) next_norm = L.attn_norm;  // no LM head: the last norm is not used
        prof_mark(s, OCRDEC_K_QKV);
        prefill_gemm(L.wqkv, false, T, w.x, H, w.qkv, 3 * HD, s);
        ap.k_cache = L.k_cache;
        ap.v_cache = L.v_cache;
        ap.k_scale = L.k_scale;
        ap.v_scale = L.v_scale;
        launch_attn_prefill(ap, s);
        prof_mark(s, OCRDEC_K_O_PROJ);
        prefill_gemm(L.wo, false, T, w.o, HD, w.y, H, s);
        prof_mark(s, OCRDEC_K_NORM);
        hipLaunchKernelGGL(resid_norm_kernel, dim3(T), dim3(64), 0, s, w.h, w.y, L.ffn_norm, H, m->norm_eps, w.x);
        if (L.is_moe) {
            const int K = L.moe.top_k;
            int32_t* ci = cap && cap->topk_idx ? cap->topk_idx + (int64_t)moe_l * T * K : nullptr;
            float* cw = cap && cap->topk_w ? cap->topk_w + (int64_t)moe_l * T * K : nullptr;
            const int32_t* fo = forced_topk ? forced_topk + (int64_t)moe_l * T * K : nullptr;
            // the combine adds into h and forms the next block's normalised input
            launch_moe(&L.moe, T, w.x, H, w.h, RESID_F32, H, 1, fo, nullptr, ci, cw, w.moe, next_norm, m->norm_eps, w.x, H,
                       s);
            ++moe_l;
        } else {
            const int F = L.dense_ff;
            prof_mark(s, OCRDEC_K_DENSE_GLU);
            prefill_gemm(L.dense_gate_up, true, T, w.x, H, w.a, F, s);
            prof_mark(s, OCRDEC_K_DENSE_DOWN);
            prefill_gemm(L.dense_down, false, T, w.a, F, w.y, H, s);
            prof_mark(s, OCRDEC_K_NORM);
            hipLaunchKernelGGL(resid_norm_kernel, dim3(T), dim3(64), 0, s, w.h, w.y, next_norm, H, m->norm_eps, w.x);
        }
    }
    if (hidden) {
        const int64_t cnt = (int64_t)T * H;
        prof_mark(s, OCRDEC_K_OTHER);
        hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)std::min<int64_t>((cnt + 255) / 256, 1024)), dim3(256), 0,
                           s, w.h, hidden, cnt);
    }
    if (m->lm_head.data && tok_out) {
        // the last position of every sequence, normalised with final_norm by the last layer
        prof_mark(s, OCRDEC_K_OTHER);
        hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(64), 0, s, w.x, w.x_last, H, last);
        const LmPlan lp = plan_lm(m->lm_head.fmt, m->vocab, H, n);
        GemvParams gp{};
        gp.w = (const uint8_t*)m->lm_head.data;
        gp.n = m->vocab;
        gp.k = H;
        gp.nchunks = n_chunks(m->lm_head.fmt, H);
        gp.xs = XDirect{w.x_last, H, n};
        gp.part = w.lm_part;
        prof_mark(s, OCRDEC_K_LM_HEAD);
        launch_lm_argmax(m->lm_head.fmt, lp, gp, s);
        prof_mark(s, OCRDEC_K_ARGMAX);
        launch_argmax_final(w.lm_part, lp.grid, n, tok_out, cap ? cap->lm_top2 : nullptr, nullptr, nullptr, s);
    }
    return launch_status("ocrdec_prefill_batch");
}

extern "C" ocrdec_status ocrdec_prefill_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, int32_t P,
                                                        size_t* bytes) {
    const int32_t row = 0;
    return ocrdec_prefill_batch_workspace_bytes(m, st, 1, &row, &P, bytes);
}

extern "C" ocrdec_status ocrdec_prefill(const ocrdec_model* m, const ocrdec_state* st, int32_t row, int32_t P,
                                        const int32_t* tok, const uint16_t* emb, const int32_t* forced_topk,
                                        int32_t* tok_out, float* hidden, const ocrdec_step_capture* cap, void* ws,
                                        size_t ws_bytes, void* stream) {
    return ocrdec_prefill_batch(m, st, 1, &row, &P, tok, emb, forced_topk, tok_out, hidden, cap, ws, ws_bytes,
                                stream);
}

/*
 * libocrdec — decode step of an OCR vision-language decoder on AMD Instinct
 * MI355X (gfx950), as a C ABI.
 *
 * The decoder is the one described in "Eseguire Unlimited-OCR su Apple
 * Silicon con C e Metal" (section "Il decoder e il Mixture of Experts"):
 * a DeepSeek-V2-style stack, hidden 1280, 10 heads of 128, layer 0 with a
 * dense SwiGLU MLP and the other layers with a Mixture of Experts (64 routed
 * experts, top-6, 2 shared experts), activations in fp16, generated tokens
 * kept in a 128-slot ring cache after a fixed image+prompt prefix, and an
 * argmax over the language head at the end of every step.  Weights are
 * block-quantised (same page, section "Quantizzazione: Q8 prima, Q4 dove
 * conviene": Q8_0, Q4_0; and "Nicolassuez/Falcon-OCR-int8-openvino",
 * paragraph on NNCF INT8_ASYM: int8 asymmetric) and dequantised inside the
 * kernels.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the argument says "host".  The
 *    caller owns every buffer; the library allocates and frees nothing and
 *    keeps no device state between calls ("The KV cache is an INPUT, not
 *    model state", Falcon-OCR card).
 *  - fp16 is IEEE binary16 passed as uint16_t; fp32 is float.  Matrices are
 *    row-major.
 *  - Compute calls are asynchronous on `stream` (a hipStream_t, NULL = the
 *    null stream).  The returned status covers argument validation, which is
 *    done on the host before anything is enqueued, and launch errors.  A
 *    non-OK status leaves all outputs untouched.
 *  - Errors: a status code, and a per-thread message from ocrdec_last_error()
 *    naming the bad argument (and, for workspaces, the needed and given bytes;
 *    Unlimited-OCR page, "Memoria": requests that do not fit are rejected with
 *    a detailed error).
 *  - Calls are reentrant.  Concurrent calls need distinct outputs, workspaces
 *    and caches (one lane per instance, Unlimited-OCR page, "Dall'ABI C
 *    all'API Python").
 *  - Rounding: fp16 stores are round-to-nearest-even from fp32; accumulation
 *    is fp32.
 */
#ifndef OCRDEC_H
#define OCRDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OCRDEC_OK = 0,
    OCRDEC_ERR_INVALID_ARG = 1, /* a pointer, size or shape is out of range */
    OCRDEC_ERR_UNSUPPORTED = 2, /* valid but not implemented (format, shape) */
    OCRDEC_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    OCRDEC_ERR_DEVICE = 4       /* a HIP call failed */
} ocrdec_status;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ocrdec_last_error(void);

/* Library version string. */
const char* ocrdec_version(void);

/* ------------------------------------------------------------------------ */
/* Kernel timing                                                             */
/* ------------------------------------------------------------------------ */

/* Profiling of the kernels the library enqueues (Unlimited-OCR page, "Dall'ABI
 * C all'API Python": the C interface reports memory and profiling).  While a
 * profile is set on the calling thread, every kernel a call of this thread
 * enqueues is preceded by a HIP event recorded on the call's stream, and the
 * kind of that kernel is noted; ocrdec_profile_mark adds a final event.  The
 * time between events i and i+1 (hipEventElapsedTime) is then kernel i's
 * duration plus the gap before it.  Recording also works under stream
 * capture (the events become graph nodes).  When `capacity` events have been
 * recorded, later ones are dropped and `count` stays at capacity. */
typedef enum {
    OCRDEC_K_EMBED = 0,       /* embedding lookup + first norm (up to 16 rows with an fp16 table it runs
                                 inside the first QKV projection and has no event of its own) */
    OCRDEC_K_QKV = 1,         /* QKV projection (norm staged in it up to 16 rows) */
    OCRDEC_K_ATTN = 2,        /* attention partials over 64-key splits (RoPE, cache write) */
    OCRDEC_K_ATTN_MERGE = 3,  /* merge of the splits */
    OCRDEC_K_ATTN_MERGE_O = 4,/* merge of the splits + O projection into the residual */
    OCRDEC_K_O_PROJ = 5,      /* O projection into the residual */
    OCRDEC_K_NORM = 6,        /* RMSNorm of the residual */
    OCRDEC_K_ROUTE = 7,       /* router, top-k, grouping */
    OCRDEC_K_EXPERT_GLU = 8,  /* grouped expert gate/up + SwiGLU */
    OCRDEC_K_EXPERT_DOWN = 9, /* grouped expert down projection */
    OCRDEC_K_COMBINE = 10,    /* weighted recombine */
    OCRDEC_K_DENSE_GLU = 11,  /* dense gate/up + SwiGLU */
    OCRDEC_K_DENSE_DOWN = 12, /* dense down projection into the residual */
    OCRDEC_K_LM_HEAD = 13,    /* language head with fused argmax (partials) */
    OCRDEC_K_ARGMAX = 14,     /* merge of the argmax partials */
    OCRDEC_K_OTHER = 15       /* anything else (copies, generation index, prompt pass) */
} ocrdec_kernel;

typedef struct {
    void** events;     /* host array [capacity] of hipEvent_t, created by the caller with timing enabled */
    int32_t* kernels;  /* host array [capacity]: kernels[i] is the ocrdec_kernel enqueued after events[i]
                          (-1 after the final mark) */
    int32_t capacity;
    int32_t count;     /* events recorded so far (the library advances it) */
} ocrdec_profile;

/* Sets the calling thread's profile (NULL: stop recording).  The struct and
 * its arrays must stay valid while set.  Errors: INVALID_ARG for a non-NULL
 * profile with NULL arrays or a negative capacity or count. */
ocrdec_status ocrdec_profile_set(ocrdec_profile* prof);
/* Records the final event of the profile on `stream` (no-op without one).
 * Errors: DEVICE if the event cannot be recorded. */
ocrdec_status ocrdec_profile_mark(void* stream);

/* ------------------------------------------------------------------------ */
/* Weight formats                                                            */
/* ------------------------------------------------------------------------ */

/* Canonical (interchange) layouts, host memory, for W[n][k] (k % 32 == 0 for
 * block formats).  Blocks run along k within a row; rows follow each other.
 *   OCRDEC_F16      n*k fp16
 *   OCRDEC_Q8_0     34-byte blocks: fp16 d, int8 q[32];            w = d*q
 *   OCRDEC_Q4_0     18-byte blocks: fp16 d, uint8 b[16]; byte j holds element
 *                   j in its low nibble and element j+16 in its high nibble;
 *                   w = d*(q-8)
 *   OCRDEC_U8A_G32  36-byte blocks: fp16 s, fp16 z, uint8 q[32];    w = s*(q-z)
 * The Unlimited-OCR page names Q8_0/Q4_0 and the Falcon-OCR card INT8_ASYM
 * with u8 weights; block size 32, the fp16 scale, (q-8)*d and the nibble
 * order are this library's definition of those formats. */
typedef enum { OCRDEC_F16 = 0, OCRDEC_Q8_0 = 1, OCRDEC_Q4_0 = 2, OCRDEC_U8A_G32 = 3 } ocrdec_qfmt;

/* A packed weight matrix on the device (see ocrdec_pack). */
typedef struct {
    int32_t fmt;       /* ocrdec_qfmt */
    int32_t n, k;      /* y[n] = sum_k W[n][k] x[k] */
    const void* data;  /* packed bytes, 256-byte aligned, ocrdec_packed_bytes() long */
} ocrdec_qmat;

/* Host-only.  Size in bytes of the packed form of W[n][k].
 * Errors: INVALID_ARG if n <= 0, k <= 0, k % 32 != 0, or bytes is NULL;
 * UNSUPPORTED for an unknown fmt. */
ocrdec_status ocrdec_packed_bytes(int32_t fmt, int32_t n, int32_t k, size_t* bytes);

/* Host-only.  Canonical -> packed (both host memory; `packed` must hold
 * ocrdec_packed_bytes()).  The packed form groups 16 output rows into a tile
 * and cuts k into chunks (128 weights for Q4_0, 64 for Q8_0 and U8A_G32, 32 for
 * F16); each (tile, chunk) is 1 KiB of codes laid out so that one 64-lane
 * wavefront reads it with one 16-byte load per lane, followed by that chunk's
 * scales.  Rows past n and columns past k are zero-filled.  The layout is an
 * internal contract between ocrdec_pack and the kernels; only
 * unpack(pack(w)) == w is promised.  Same errors as ocrdec_packed_bytes, plus
 * INVALID_ARG for NULL buffers. */
ocrdec_status ocrdec_pack(int32_t fmt, int32_t n, int32_t k, const void* canonical, void* packed);

/* Host-only.  Packed -> canonical (inverse of ocrdec_pack, bit for bit). */
ocrdec_status ocrdec_unpack(int32_t fmt, int32_t n, int32_t k, const void* packed, void* canonical);

/* ------------------------------------------------------------------------ */
/* ocrdec_gemv_q: weight-streaming GEMV / skinny GEMM                         */
/* ------------------------------------------------------------------------ */

typedef enum { OCRDEC_OUT_F32 = 0, OCRDEC_OUT_F16 = 1 } ocrdec_otype;

/* y[r][j] = sum_k W[j][k] * x[r][k] for r < rows, j < W->n, with W dequantised
 * in registers (Unlimited-OCR page, "Quantizzazione": dequantisation fused into
 * the GEMV, no fp16 copy of the weights) and fp32 accumulation.
 *   W     host pointer to the descriptor; W->data on the device.
 *   x     fp16 [rows][ldx], ldx >= W->k, 16-byte aligned rows (ldx % 8 == 0).
 *   y     [rows][ldy] fp32 (y_type OUT_F32) or fp16 (OUT_F16), ldy >= W->n.
 *   rows  1 .. 4096 (all rows share one read of W).
 * Errors: INVALID_ARG for NULL pointers, bad sizes or misalignment;
 * UNSUPPORTED for an unknown format; DEVICE if the launch fails. */
ocrdec_status ocrdec_gemv_q(const ocrdec_qmat* W, int32_t rows, const uint16_t* x, int64_t ldx,
                            void* y, int32_t y_type, int64_t ldy, void* stream);

/* Language-head argmax (Unlimited-OCR page, "Il decoder e il Mixture of
 * Experts": the decode loop ends with an argmax over the language head; the
 * "Quantizzazione" section fuses it with the dequantising GEMV):
 *   tok_out[r] = argmax_v sum_k W[v][k] x[r][k], ties to the lowest v,
 * with the logits kept on chip (never written to memory).
 *   x        fp16 [rows][W->k], already normalised
 *   tok_out  int32 [rows]
 *   top2     fp32 [rows][2] (best and second-best logit) or NULL
 *   rows     1 .. 32
 * Workspace: ocrdec_lm_argmax_workspace_bytes (per-workgroup partial
 * results, merged by a second short kernel).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE. */
ocrdec_status ocrdec_lm_argmax_workspace_bytes(const ocrdec_qmat* W, int32_t rows, size_t* bytes);
ocrdec_status ocrdec_lm_argmax(const ocrdec_qmat* W, int32_t rows, const uint16_t* x, int32_t* tok_out,
                               float* top2, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* ocrdec_attn_decode: single-query attention over a prefix + ring KV cache  */
/* ------------------------------------------------------------------------ */

/* One decode step of attention for `rows` independent sequences.
 *
 * Inputs are the raw (un-rotated) projections of the new token, fp32
 * [rows][ld_qkv] with q at column 0, k at n_heads*head_dim, v at
 * 2*n_heads*head_dim.  The call rotates q and k (RoPE, rotate-half, theta
 * rope_theta, over the whole head), rounds q, k, v to fp16, writes k and v
 * into the row's cache slot, and attends:
 *   o_h = sum_j softmax_j(scale * q_h . k_hj) v_hj   (fp32 softmax)
 * and stores o as fp16 [rows][ld_out] (head h at column h*head_dim).
 *
 * Caches: k_cache, v_cache fp16 [rows][n_heads][cache_cap][head_dim],
 * caller-owned ("The KV cache is an INPUT", Falcon-OCR card); the call writes
 * only the new token's slot.
 *
 * Ring mode (ring_cap > 0), cache_cap = prefix_cap + ring_cap: row r has a
 * fixed prefix of prefix_len[r] keys at [0, prefix_len[r]) and generated
 * tokens in ring slots [prefix_cap, prefix_cap + ring_cap) (Unlimited-OCR
 * page: a 128-token ring keeps decode memory bounded).  With t = gen_index[r],
 * the new token goes to slot prefix_cap + t % ring_cap and the attended
 * window is the prefix plus ring slots [0, min(t+1, ring_cap)) — the ring's
 * capacity counts the new token.  RoPE position: prefix_len[r] + t.
 *
 * Linear mode (ring_cap == 0), cache_cap = prefix_cap: row r holds
 * prefix_len[r] cached keys; the new token is written at index prefix_len[r]
 * (< prefix_cap) and keys [0, prefix_len[r]] are attended.  RoPE position:
 * prefix_len[r] - (sink ? 1 : 0).
 *
 * Sink (Falcon-OCR card, attention sink paragraph): if `sink` is non-NULL,
 * sink[h] is added to the score of cache index 0, where the host has seeded
 * a zero key and a zero value; this is the page's extra key with logit =
 * sink and value 0 (its constant-1 query lane folded into a logit).
 *
 * INT8 KV cache (k_scale and v_scale non-NULL): k_cache and v_cache hold
 * int8 codes [rows][n_heads][cache_cap][head_dim] and the cached value of a
 * (row, head, slot) row is scale * code.  The new token's key and value
 * rows are stored as s = fp16(max|x| / 127) and code = round-half-away(x / s)
 * clamped to [-127, 127] (both divisions in fp32, correctly rounded; s = 0
 * gives code 0), and the attention reads them as stored.  The pages say only
 * that an INT8 KV cache exists (Falcon-OCR card, "How it is meant to be
 * run"); this one-scale-per-row form is this library's.  Caches 16-byte
 * aligned.
 *
 * gen_index and prefix_len are read, never written.
 * head_dim: 64 or 128.  rows >= 1.  Workspace: ocrdec_attn_workspace_bytes.
 * Errors: INVALID_ARG (NULL pointers, head_dim, ld_* too small, caps),
 * WORKSPACE (too small), DEVICE. */
typedef struct {
    int32_t rows, n_heads, head_dim;
    const float* qkv;          /* [rows][ld_qkv] fp32 */
    int64_t ld_qkv;
    uint16_t* k_cache;         /* [rows][n_heads][cache_cap][head_dim] fp16 */
    uint16_t* v_cache;
    int32_t prefix_cap, ring_cap;
    const int32_t* prefix_len; /* [rows] */
    const int32_t* gen_index;  /* [rows] (ring mode) */
    const float* sink;         /* [n_heads] or NULL */
    float rope_theta;
    float scale;               /* score scale, normally 1/sqrt(head_dim) */
    uint16_t* out;             /* [rows][ld_out] fp16 */
    int64_t ld_out;
    uint16_t* k_scale;         /* INT8 KV cache: fp16 [rows][n_heads][cache_cap], see below; NULL: fp16 cache */
    uint16_t* v_scale;
} ocrdec_attn_args;

ocrdec_status ocrdec_attn_workspace_bytes(const ocrdec_attn_args* a, size_t* bytes);
ocrdec_status ocrdec_attn_decode(const ocrdec_attn_args* a, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* ocrdec_moe_layer: DeepSeek-V2-style MoE                                   */
/* ------------------------------------------------------------------------ */

/* Weights of one MoE layer (Unlimited-OCR page, "Il decoder e il Mixture of
 * Experts": 64 routed experts, top-6, 2 shared experts).  Each expert is a
 * SwiGLU: a = fp16(silu(G x) * (U x)), y = D a.  The routed experts are stacked:
 *   gate_up  [n_experts * 2 * d_ff][hidden]: expert e owns rows
 *            [e*2*d_ff, e*2*d_ff + d_ff) (gate) and the next d_ff rows (up);
 *   down     [n_experts * hidden][d_ff]: expert e owns rows [e*hidden, (e+1)*hidden);
 *   sh_gate_up, sh_down: the same for the n_shared shared experts.
 * hidden and d_ff must be multiples of 16 (a packed tile never straddles two
 * experts).  router: [n_experts][hidden]; router_bias: fp32 [n_experts] added
 * to the router logits before the softmax, or NULL. */
typedef struct {
    int32_t hidden, n_experts, top_k, n_shared, d_ff;
    ocrdec_qmat router;
    const float* router_bias;
    ocrdec_qmat gate_up, down;
    ocrdec_qmat sh_gate_up, sh_down;
} ocrdec_moe_weights;

/* Optional outputs (any pointer may be NULL):
 *   topk_idx  int32 [rows][top_k]  chosen experts, by probability descending,
 *                                  ties to the lower index
 *   topk_w    fp32  [rows][top_k]  renormalised weights
 *   counts    int32 [n_experts]    tokens per expert
 *   offsets   int32 [n_experts+1]  exclusive scan of counts
 *   perm      int32 [rows*top_k]   grouped position -> pair index r*top_k + j,
 *                                  grouped by expert, then row, then rank */
typedef struct {
    int32_t* topk_idx;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
} ocrdec_moe_capture;

/* out[r] = [h[r] +] sum_s shared_s(x[r]) + sum_j w_rj expert_{idx_rj}(x[r]),
 * summed in fp32 (shared first, then ranks in order), rounded once to fp16.
 * Routing: logits = router . x (+ bias); p = softmax(logits); the top_k
 * experts by p (ties: lower index); w = p / sum of the chosen p.  Tokens are
 * grouped per expert on the device (counting sort, stable by row then rank)
 * before the expert projections, and recombined with their weights.
 *   x            fp16 [rows][hidden] (the MoE input, already normalised)
 *   h            fp16 [rows][hidden]: if add_residual, h += moe; else h = moe
 *   forced_topk  int32 [rows][top_k] or NULL: use these experts (a row whose
 *                first entry is < 0 routes itself); weights still come from
 *                this call's probabilities
 *   rows         1 .. 65536
 * Errors: INVALID_ARG, UNSUPPORTED (top_k > 8, n_experts > 256), WORKSPACE, DEVICE. */
ocrdec_status ocrdec_moe_workspace_bytes(const ocrdec_moe_weights* w, int32_t rows, size_t* bytes);
ocrdec_status ocrdec_moe_layer(const ocrdec_moe_weights* w, int32_t rows, const uint16_t* x, uint16_t* h,
                               int32_t add_residual, const int32_t* forced_topk,
                               const ocrdec_moe_capture* capture, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------ */
/* ocrdec_decode_step: one token for every row through the whole decoder     */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t* attn_norm;   /* fp16 [hidden] RMSNorm gain before attention */
    ocrdec_qmat wqkv;            /* [3*n_heads*head_dim][hidden]: q rows, k rows, v rows */
    ocrdec_qmat wo;              /* [hidden][n_heads*head_dim] */
    const uint16_t* ffn_norm;    /* fp16 [hidden] RMSNorm gain before the MLP/MoE */
    int32_t is_moe;
    int32_t dense_ff;            /* dense layers: SwiGLU width */
    ocrdec_qmat dense_gate_up;   /* [2*dense_ff][hidden]: gate rows then up rows */
    ocrdec_qmat dense_down;      /* [hidden][dense_ff] */
    ocrdec_moe_weights moe;      /* MoE layers */
    uint16_t* k_cache;           /* fp16 [rows][n_heads][prefix_cap+ring_cap][head_dim], or int8 codes */
    uint16_t* v_cache;
    uint16_t* k_scale;           /* INT8 KV cache (as in ocrdec_attn_args): fp16 [rows][n_heads][cap]; */
    uint16_t* v_scale;           /* NULL for fp16 caches */
} ocrdec_layer;

typedef struct {
    int32_t n_layers, hidden, n_heads, head_dim, vocab;
    float rope_theta, norm_eps;
    const uint16_t* embed;       /* fp16 [vocab][hidden] or NULL (input from `hidden`) */
    const uint16_t* final_norm;  /* fp16 [hidden] (needed with an LM head) */
    ocrdec_qmat lm_head;         /* [vocab][hidden]; lm_head.data NULL = no LM head */
    const ocrdec_layer* layers;  /* HOST array [n_layers] */
    ocrdec_qmat embed_q;         /* [vocab][hidden] embedding in any storage format, used when embed is
                                    NULL and embed_q.data is not: row tok dequantised (w = d*q, d*(q-8),
                                    s*(q-z) or the fp16 value) into the fp32 residual */
} ocrdec_model;

typedef struct {
    int32_t rows, prefix_cap, ring_cap;   /* ring_cap > 0 */
    const int32_t* prefix_len;            /* [rows] */
    int32_t* gen_index;                   /* [rows]; the step adds 1 to each */
} ocrdec_state;

/* Optional per-step outputs (any pointer may be NULL):
 *   topk_idx, topk_w  [n_moe_layers][rows][top_k] routing of every MoE layer
 *   lm_top2           fp32 [rows][2]: the best and second-best logits */
typedef struct {
    int32_t* topk_idx;
    float* topk_w;
    float* lm_top2;
} ocrdec_step_capture;

/* One decode step (Unlimited-OCR page, "Il decoder e il Mixture of Experts"):
 * h = embed[tok_in] (or row tok_in of embed_q dequantised; or `hidden` if
 * tok_in is NULL); for each layer:
 *   x = fp16(RMSNorm(h) * attn_norm); qkv = Wqkv x; attention as in
 *   ocrdec_attn_decode (ring mode, scale 1/sqrt(head_dim)); h += Wo o;
 *   x = fp16(RMSNorm(h) * ffn_norm); h += MLP(x) with MLP the dense SwiGLU or
 *   the MoE of ocrdec_moe_layer;
 * then `hidden` (if non-NULL) receives h, and if the model has an LM head and
 * tok_out is non-NULL: tok_out[r] = argmax_v (W_lm . fp16(RMSNorm(h) *
 * final_norm))[v], ties to the lowest v, logits never leave the chip.
 * Finally gen_index[r] += 1.  The residual h is kept in fp32 between blocks
 * (the fp16 activations are the projection inputs, the cache and the SwiGLU
 * intermediate; the HunyuanOCR ncnn page, section 3.1, keeps an FP32 residual
 * between blocks for the same reason: no accumulation of low-precision round
 * trips).  tok_out may alias tok_in (the step reads tok_in before it writes
 * tok_out), so a caller can feed tokens back on the device.
 * The residual is accumulated exactly: every addend (an fp32 projection or
 * expert output) is rounded once to a multiple of 2^-32 and the sums are
 * 64-bit integer sums, so the result does not depend on the order in which
 * the GPU adds the parts, and two runs on the same inputs give the same bits
 * (tokens, routing, hidden state).  Readers take it as fp32.  Its range is
 * |h| < 2^30; see ocrdec_device_status for values beyond it.
 *   hidden       fp32 [rows][hidden]: input if tok_in is NULL; output if non-NULL
 *   forced_topk  int32 [n_moe_layers][rows][top_k] or NULL (see ocrdec_moe_layer)
 *   rows         1 .. 32; prefix_cap + ring_cap <= 65536
 * Workspace: ocrdec_step_workspace_bytes(m, st) bytes (it depends on rows and
 * the cache capacity of the state).  Its first bytes hold the step's device
 * status word (ocrdec_device_status).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE. */
ocrdec_status ocrdec_step_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, size_t* bytes);
ocrdec_status ocrdec_decode_step(const ocrdec_model* m, const ocrdec_state* st, const int32_t* tok_in,
                                 float* hidden, int32_t* tok_out, const int32_t* forced_topk,
                                 const ocrdec_step_capture* capture, void* ws, size_t ws_bytes,
                                 void* stream);

/* ocrdec_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of 16 MiB that the library holds on every GPU it runs on until the process
 * ends (enough for 32 rows with a cache of 4096 + 128 positions in the
 * 12-layer decoder); the call allocates nothing.  All calls on one GPU share
 * that array, so calls that overlap in time on one GPU (other streams, other
 * threads) race and must not be made; consecutive calls on one stream are
 * fine (nothing in it needs to start at zero).  Arguments and results as
 * ocrdec_decode_step.  ocrdec_device_status cannot be used with it.
 * Errors: as ocrdec_decode_step; WORKSPACE if the step needs more than the
 * static array; DEVICE if the array's address cannot be obtained. */
ocrdec_status ocrdec_decode_step_noalloc(const ocrdec_model* m, const ocrdec_state* st, const int32_t* tok_in,
                                         float* hidden, int32_t* tok_out, const int32_t* forced_topk,
                                         const ocrdec_step_capture* capture, void* stream);

/* Device-side conditions of the most recent ocrdec_decode_step that used the
 * workspace `ws` (the Falcon-OCR card, "Two traps the host must avoid": a
 * wrong cache length or position does not fail, it yields fluent but
 * degenerate text; the Unlimited-OCR page, "Memoria": what cannot be served
 * is rejected with a detailed error).  The step cannot return these through
 * its status (it is asynchronous), so it records them on the device: each
 * step clears the bits in its first kernel and sets them as it runs.
 *   OCRDEC_DEV_TOKEN_RANGE  a tok_in id outside [0, vocab) was clamped
 *   OCRDEC_DEV_RESIDUAL     a non-finite value, or one of magnitude >= 2^30,
 *                           was to enter the residual (it was replaced by 0)
 *   OCRDEC_DEV_LOGIT        a language-head logit was NaN or infinite (a NaN
 *                           never wins the argmax)
 *   OCRDEC_DEV_NO_TOKEN     a row had no finite best logit; its token was set
 *                           to 0
 * The call synchronises `stream` (the stream the step ran on), then reads the
 * bits into *flags (0: nothing to report).  It does not clear them.
 *   ws, ws_bytes  the step's workspace (device) and its size
 * Errors: INVALID_ARG (NULL pointers), WORKSPACE (ws_bytes smaller than the
 * status area), DEVICE (synchronisation or copy failed). */
typedef enum {
    OCRDEC_DEV_TOKEN_RANGE = 1,
    OCRDEC_DEV_RESIDUAL = 2,
    OCRDEC_DEV_LOGIT = 4,
    OCRDEC_DEV_NO_TOKEN = 8
} ocrdec_device_flag;
ocrdec_status ocrdec_device_status(const void* ws, size_t ws_bytes, void* stream, uint32_t* flags);

/* ------------------------------------------------------------------------ */
/* ocrdec_prefill: the prompt pass of one row                                */
/* ------------------------------------------------------------------------ */

/* The prompt pass before token-by-token decoding (HunyuanOCR ncnn page,
 * section 3.2: prefill and incremental decoding use causal masks of
 * different shapes, and decoding reuses every layer's cache; Unlimited-OCR
 * page: the model runs a prefill, then generates token by token).  P prompt
 * positions of row `row` go through every layer at once: h = embed[tok[i]]
 * (or embed_q's row dequantised), or h = emb[i] when tok is NULL; per layer
 * x = fp16(RMSNorm(h) * attn_norm), q/k/v = Wqkv x, RoPE at the linear
 * positions i = 0..P-1, k and v written to cache indices 0..P-1 of the row
 * (fp16; or, where the layer's k_scale and v_scale are set, int8 codes and
 * fp16 scales quantised as the decode step quantises a new token), causal
 * attention (query i attends keys 0..i, scale 1/sqrt(head_dim)) over the
 * values as stored (scale x code for an INT8 cache), h += Wo o, then
 * h += MLP(fp16(RMSNorm(h) * ffn_norm))
 * (dense SwiGLU, or the MoE of ocrdec_moe_layer over the P positions).  If
 * the model has an LM head and tok_out is non-NULL, tok_out[0] = the argmax
 * at position P-1 (the first generated token), as in ocrdec_decode_step.
 * The call does not change prefix_len or gen_index: to decode after it, the
 * caller sets prefix_len[row] = P and gen_index[row] = 0; the first decode
 * step then places its token at RoPE position P.
 *   st           the decode state the caches belong to (rows, prefix_cap,
 *                ring_cap); only row `row` of every layer's cache is written
 *   P            1 .. prefix_cap
 *   tok          int32 [P] token ids, or NULL
 *   emb          fp16 [P][hidden] input features (used when tok is NULL)
 *   forced_topk  int32 [n_moe_layers][P][top_k] or NULL (see ocrdec_moe_layer)
 *   hidden       fp32 [P][hidden] or NULL: the residual after the last layer
 *   capture      topk_idx / topk_w [n_moe_layers][P][top_k], lm_top2 [1][2]
 *                (any pointer may be NULL)
 * Workspace: ocrdec_prefill_workspace_bytes(m, st, P) bytes.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE. */
ocrdec_status ocrdec_prefill_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, int32_t P,
                                             size_t* bytes);
ocrdec_status ocrdec_prefill(const ocrdec_model* m, const ocrdec_state* st, int32_t row, int32_t P,
                             const int32_t* tok, const uint16_t* emb, const int32_t* forced_topk,
                             int32_t* tok_out, float* hidden, const ocrdec_step_capture* capture, void* ws,
                             size_t ws_bytes, void* stream);

/* The prompt passes of n rows at once (the same computation as ocrdec_prefill
 * for each; batching lets the projections and experts of all the prompts
 * share each weight read).  Sequence i has P[i] positions and goes to row
 * rows[i] (distinct rows); the inputs are packed one sequence after
 * another: tok int32 [sum P] or emb fp16 [sum P][hidden].
 *   n            1 .. 32; sum of P at most 65536
 *   rows, P      HOST int32 [n]
 *   forced_topk  int32 [n_moe_layers][sum P][top_k] or NULL (packed positions)
 *   tok_out      int32 [n]: the argmax at each sequence's last position
 *   hidden       fp32 [sum P][hidden] or NULL
 *   capture      topk_idx / topk_w [n_moe_layers][sum P][top_k], lm_top2 [n][2]
 * Workspace: ocrdec_prefill_batch_workspace_bytes(m, st, n, rows, P).
 * Errors: as ocrdec_prefill. */
ocrdec_status ocrdec_prefill_batch_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, int32_t n,
                                                   const int32_t* rows, const int32_t* P, size_t* bytes);
ocrdec_status ocrdec_prefill_batch(const ocrdec_model* m, const ocrdec_state* st, int32_t n, const int32_t* rows,
                                   const int32_t* P, const int32_t* tok, const uint16_t* emb,
                                   const int32_t* forced_topk, int32_t* tok_out, float* hidden,
                                   const ocrdec_step_capture* capture, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* ocrdec_run_round: a queue of requests decoded together                    */
/* ------------------------------------------------------------------------ */

/* One request of a round.  The prompt is `tokens` (device int32 [P]) or, when
 * tokens is NULL, `features` (device fp16 [P][hidden]); out is a HOST buffer
 * of max_new tokens.  n_out and stop are set by ocrdec_run_round: stop = 1
 * (an EOS token was produced) or 2 (max_new tokens). */
typedef struct {
    const int32_t* tokens;
    const uint16_t* features;
    int32_t P;
    int32_t max_new;
    int32_t* out;
    int32_t n_out;
    int32_t stop;
} ocrdec_request;

/* Serves the requests with the rows of `st` (Falcon-OCR card, "How it is
 * meant to be run": rows of one round share each decode step's read of the
 * weights, and merging requests into a round is what makes a queue
 * affordable).  Requests are taken in order; each gets the lowest free row.
 * The prompt passes of the requests admitted together run as one
 * ocrdec_prefill_batch (token requests and feature requests separately, the
 * inputs packed into the workspace), which fills the rows' cache prefixes
 * and gives their first tokens; then decode steps (ocrdec_decode_step,
 * tokens fed back on the device) advance every occupied row together.  After each step the new
 * tokens are read on the host: a request stops at a token of the EOS set
 * (HunyuanOCR ncnn page, section 3.5: the end token is not handed out; with
 * keep_eos it is appended, for comparisons) or after max_new tokens, and
 * its row takes the next request.  The call returns when every request has
 * stopped; it synchronises the stream once per step.  It sets prefix_len and
 * gen_index of the rows it admits and overwrites the rows' caches.
 *   st       rows = the round's row slots (1..32); prefix_cap >= every P
 *   eos      HOST int32 [n_eos] (may be empty)
 * Workspace: ocrdec_round_workspace_bytes(m, st, max P) bytes.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE (a failed step ends
 * the round; the requests keep what they had). */
ocrdec_status ocrdec_round_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, int32_t max_P,
                                           size_t* bytes);
ocrdec_status ocrdec_run_round(const ocrdec_model* m, const ocrdec_state* st, ocrdec_request* reqs, int32_t n_reqs,
                               const int32_t* eos, int32_t n_eos, int32_t keep_eos, void* ws, size_t ws_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif
#endif /* OCRDEC_H */
